// Per-step blockwise causal attention on bf16 matrix cores (gfx950).
//
// Work: one workgroup per (row tile, ring step, head group) entry of the
// host plan. Ring step s of rank r attends the rank's rows to the keys of
// source rank j = (r - s) mod P (Ring Attention, Liu et al., ICLR 2024);
// the context-parallel multimodal page (xuesongtap.github.io/2026/03/22/
// context-parallel-multimodal, sections 1.1 and 4.1) fixes which rows and
// keys those are. The plan gives each entry its key spans, already clipped
// to the keys its rows can see, so a key tile is either fully visible
// (no mask work) or crosses the causal diagonal / a span end (masked);
// tiles no row can see were never emitted.
//
// Per wave: 32 query rows of one head. Scores are computed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: each lane then owns one query
// row (lane % 32) and 16 keys per 32-key block, so the softmax max and sum
// are in-lane plus one swap with lane ^ 32. The accumulator layout of S^T is
// directly the B operand layout of O^T = V^T P^T, so probabilities go from
// registers to the second MFMA without an LDS round trip. V stays in its
// natural [key][d] layout in LDS; ds_read_b64_tr_b16 produces the V^T
// operand. K and V tiles of 64 keys are double-buffered in LDS; the next
// tile's global loads are in flight while the current tile is computed.
// Several waves of a workgroup share each K/V tile: 4 row blocks of one
// head (MHA) or one row block of 2 or 4 heads that read the same KV head
// (GQA).
//
// Global K/V loads go through a buffer resource whose size ends at the
// span end: rows past it read as zeros in hardware, so the loads need no
// branches and their per-lane offsets never change.
//
// Online softmax with a lazy reference max: probabilities are
// exp2((s - m_ref) * log2(e)/sqrt(D)); m_ref moves (and the output and sum
// are rescaled) only when a row's running max exceeds it by more than
// kRescaleLog2 in the exp2 domain, so probabilities stay below
// 2^kRescaleLog2 and most tiles skip the rescale. The output and the sum
// always share the same m_ref, so the normalised result is unchanged.
//
// Output per entry: O_s normalised by its own softmax sum (fp32) and
// lse_s = m_ref/sqrt(D) + ln(sum) (fp32), combined across steps by the LSE
// merge.
#include "kernels.h"

namespace cpattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBufferWord3 = 0x00020000;  // raw buffer access, gfx9 family
constexpr float kRescaleLog2 = 8.0f;      // lazy-rescale threshold (exp2 domain)
constexpr int kWaitVmcnt0 = 0x0F70;       // s_waitcnt vmcnt(0), expcnt and lgkmcnt untouched
// __builtin_amdgcn_sched_group_barrier instruction classes
constexpr int kSchedValu = 0x0002;
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;

// Our value combined with that of lane ^ 32: the swap puts lanes 0-31 of
// one copy next to lanes 32-63 of the other.
__device__ inline float max_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferWord3);
}

template <int D, int NW, int G>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_step_bf16_kernel(const AttnArgs a) {
  constexpr int BN = kBlockN;               // keys per tile
  constexpr int KS = D + 8;                 // K row stride in LDS (bf16): b128 reads conflict-free
  constexpr int VS = D + 32;                // V row stride: transposed b64 reads conflict-free
  constexpr int NT = NW * 64;
  constexpr int PIECES = BN * D / 8;        // 16-byte pieces per K (or V) tile
  constexpr int PPT = PIECES / NT;          // pieces per thread
  constexpr int RPIECES = D / 8;            // pieces per key row
  constexpr int KBUF = BN * KS, VBUF = BN * VS, STAGE = KBUF + VBUF;
  constexpr int ND = D / 32;                // 32-wide blocks of head_dim
  constexpr int NQ = D / 16;                // MFMAs per 32x32 score block
  static_assert(PIECES % NT == 0, "tile pieces must split evenly over threads");
  static_assert(NW % G == 0, "waves must cover whole heads");
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hg = blockIdx.x % a.n_hg;
  const EntryRec ent = a.entries[blockIdx.x / a.n_hg];
  const TileRec tile = a.tiles[ent.tile];
  const int h = hg * G + (wave % G);
  const int rsub = wave / G;
  const int kvh = (hg * G) / a.group;
  const int ql = lane & 31, hh = lane >> 5;
  const int rin = rsub * 32 + ql;
  const bool row_ok = rin < tile.nrows;
  const int lrow = tile.local0 + rin;
  const int grow = tile.g0 + rin;
  const int wave_lo = tile.g0 + rsub * 32;                 // first row of this wave
  const int wave_rows = min(32, tile.nrows - rsub * 32);   // <= 0: wave has no rows
  const int wave_hi = wave_lo + wave_rows - 1;             // last row of this wave

  // Q as the B operand of S^T = K Q^T: lane holds q[row][16*jj + 8*hh + 0..7].
  bf16x8 qf[NQ];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.qr) + (int64_t(lrow) * a.H + h) * D + 8 * hh;
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) {
      if (row_ok) {
        qf[jj] = *reinterpret_cast<const bf16x8*>(qp + 16 * jj);
      } else {
        s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        qf[jj] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }

  // K/V tile loads: per-lane byte offsets inside a tile never change; the
  // tile's base and its valid size go into the buffer resource.
  const int tok_bytes = a.Hkv * D * 2;  // bytes between consecutive tokens
  const char* kbase = static_cast<const char*>(a.k) + int64_t(kvh) * D * 2;
  const char* vbase = static_cast<const char*>(a.v) + int64_t(kvh) * D * 2;
  int goff[PPT], loff[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = tid + i * NT;
    const int row = p / RPIECES, col = p % RPIECES;
    goff[i] = row * tok_bytes + col * 16;
    loff[i] = row * KS + col * 8;  // K; V adds row * (VS - KS)
  }
  u32x4 kreg[PPT], vreg[PPT];
  auto load_tile = [&](int kt, int k1) {
    const int valid = min(k1 - kt, BN) * tok_bytes;
    const int64_t off = int64_t(kt) * tok_bytes;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + off, valid);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + off, valid);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, goff[i], 0, 0);
      vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, goff[i], 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* ks = smem + buf * STAGE;
    __bf16* vs = ks + KBUF;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int row = (tid + i * NT) / RPIECES;
      *reinterpret_cast<u32x4*>(ks + loff[i]) = kreg[i];
      *reinterpret_cast<u32x4*>(vs + loff[i] + row * (VS - KS)) = vreg[i];
    }
  };

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int t = 0; t < 16; ++t) o[db][t] = 0.f;
  float m_ref = -INFINITY;  // reference max (raw score units) for this lane's row
  float l = 0.f;            // sum over this lane's keys (other half in lane ^ 32)
  const float c2 = a.scale_log2;
  const float thr = kRescaleLog2 / c2;

  auto compute = [&](int buf, int kt, int k1) {
    const __bf16* ks = smem + buf * STAGE;
    const __bf16* vs = ks + KBUF;
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 16; ++t) s[kb][t] = 0.f;
      const __bf16* kr = ks + (32 * kb + ql) * KS + 8 * hh;
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kr + 16 * jj);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[jj], s[kb], 0, 0, 0);
      }
    }
    // lane owns row grow; register t of block kb holds key
    // kt + 32*kb + 8*(t/4) + 4*hh + t%4
    if (kt + BN > k1 || kt + BN - 1 > wave_lo) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int key = kt + 32 * kb + 8 * (t >> 2) + 4 * hh + (t & 3);
          if (key >= k1 || key > grow) s[kb][t] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 16; ++t) mx = fmaxf(mx, s[kb][t]);
    mx = max_with_partner(mx);
    const bool grow_ref = mx > m_ref + thr;  // also true on a row's first visible key
    if (__builtin_amdgcn_ballot_w64(grow_ref) != 0) {
      const float m_new = grow_ref ? mx : m_ref;
      const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * c2);  // 0 when m_ref = -inf
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t) o[db][t] *= alpha;
      m_ref = m_new;
    }
    const float ms = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
    bf16x8 pb[2][2];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][t], c2, -ms));
        rs += p;
        pb[kb][t >> 3][t & 7] = (__bf16)p;
      }
    l += rs;
    // O^T += V^T P^T. A operand (V^T): lane holds V[key][32*db + lane%32]
    // for the 8 keys whose probabilities sit in its B operand; built from
    // two transposed 4-key reads per MFMA.
    const int trow = (lane & 15) >> 2;                         // key offset inside a 4-key read
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // d offset inside a 32-block
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int key0 = 32 * kb + 16 * sub + 4 * hh + trow;
          const __bf16* p0 = vs + key0 * VS + 32 * db + tcol;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * VS));
          const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both),
                                                          pb[kb][sub], o[db], 0, 0, 0);
        }
  };

  int sp = ent.span_begin;
  SpanRec span = a.spans[sp];
  int kt = span.k0, k1 = span.k1;
  load_tile(kt, k1);
  store_tile(0);
  __syncthreads();
  int buf = 0;
  while (true) {
    int nkt = kt + BN, nk1 = k1, nsp = sp;
    if (nkt >= k1) {
      ++nsp;
      if (nsp < ent.span_end) {
        const SpanRec ns = a.spans[nsp];
        nkt = ns.k0;
        nk1 = ns.k1;
      }
    }
    const bool has_next = nsp < ent.span_end;
    if (has_next) load_tile(nkt, nk1);
    if (wave_rows > 0 && kt <= wave_hi) compute(buf, kt, k1);
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    if (!has_next) break;
    kt = nkt;
    k1 = nk1;
    sp = nsp;
    buf ^= 1;
  }

  const float lt = sum_with_partner(l);
  if (!row_ok) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  float* po = a.part_o + ((int64_t(ent.step) * a.R + lrow) * a.H + h) * D + 4 * hh;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int tq = 0; tq < 4; ++tq) {
      const float4 val = make_float4(o[db][4 * tq] * inv, o[db][4 * tq + 1] * inv,
                                     o[db][4 * tq + 2] * inv, o[db][4 * tq + 3] * inv);
      *reinterpret_cast<float4*>(po + 32 * db + 8 * tq) = val;
    }
  if (hh == 0)
    a.part_lse[(int64_t(ent.step) * a.H + h) * a.R + lrow] =
        lt > 0.f ? m_ref * a.scale + logf(lt) : -INFINITY;
}

// ---------------------------------------------------------------------------
// head_dim 128: software-pipelined variant.
//
// Differences from the kernel above:
//  * V is read from a V^T copy made once per call, blocked by 8 keys
//    (vt[g][key/8][d][key%8]), so the PV operand needs no transposing
//    read: each lane's 8 keys at one d are 16 contiguous bytes, read with
//    ds_read_b128 like K, and a 64-key tile is one contiguous 16 KiB run.
//  * Lane ql of the QK^T operand reads K row sigma(ql), sigma swapping bits
//    2 and 3 of the row index. The S^T accumulator register t of lane half
//    hh then holds key 16*(t/8) + 8*hh + t%8: eight consecutive keys per
//    MFMA operand, exactly the keys of the lane's contiguous V^T read.
//  * K and V^T tiles go from HBM straight into LDS (buffer_load ... lds),
//    no staging registers. One wave instruction fills 1 KiB of LDS (lane l
//    at byte 16*l), so rows are unpadded and bank conflicts are avoided by
//    XOR-swizzling 16-byte granules: K granule g of row r sits at
//    g ^ (r & 15) (16 rows read together land on 16 granule slots); V^T
//    granule g of row d sits at g ^ ((d >> 1) & 7) (128-byte rows, two per
//    bank sweep, 16 rows read together land on 16 slots). All LDS read
//    addresses are per-lane constants plus immediates.
//  * Key tiles start at multiples of 8 keys so V^T rows load 16-byte
//    aligned; keys below the span start are masked like those past its end.
//  * K runs one tile ahead of V: while the softmax of tile t runs on VALU,
//    the QK^T MFMAs of tile t+1 are already issued, so matrix and vector
//    work overlap inside one wave. K is double-buffered and V
//    triple-buffered, so each tile needs a single barrier.
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_step_bf16_d128_kernel(const AttnArgs a) {
  constexpr int D = 128, BN = kBlockN, NW = 4;
  constexpr int TILE = BN * D * 2;           // bytes of one K (or V^T) tile
  constexpr int CH = TILE / 1024 / NW;       // LDS-DMA instructions per wave per tensor
  constexpr int ND = D / 32, NQ = D / 16;
  static_assert(BN == 64, "tile walk assumes 64-key tiles");
  // Separate arrays per buffer, each chosen at compile time in the unrolled
  // loop, so the compiler can tell an in-flight LDS-DMA target from the
  // buffers being read and waits only where they alias.
  __shared__ __attribute__((aligned(1024))) char k0s[TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[TILE];
  __shared__ __attribute__((aligned(1024))) char v2s[TILE];
  typedef __attribute__((address_space(3))) void lds_void;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hg = blockIdx.x % a.n_hg;
  const EntryRec ent = a.entries[blockIdx.x / a.n_hg];
  const TileRec tile = a.tiles[ent.tile];
  const int h = hg * G + (wave % G);
  const int rsub = wave / G;
  const int kvh = (hg * G) / a.group;
  const int ql = lane & 31, hh = lane >> 5;
  const int rin = rsub * 32 + ql;
  const bool row_ok = rin < tile.nrows;
  const int lrow = tile.local0 + rin;
  const int grow = tile.g0 + rin;
  const int wave_lo = tile.g0 + rsub * 32;

  // Key spans (at most 3: image prefix and two text chunks), walked in
  // 64-key tiles starting at the span start rounded down to 8 keys.
  int sk0[3] = {0, 0, 0}, sk1[3] = {0, 0, 0}, snt[3] = {0, 0, 0};
  int n_tiles = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (ent.span_begin + i < ent.span_end) {
      const SpanRec sp = a.spans[ent.span_begin + i];
      sk0[i] = sp.k0;
      sk1[i] = sp.k1;
      snt[i] = (sp.k1 - (sp.k0 & ~7) + BN - 1) / BN;
      n_tiles += snt[i];
    }
  }
  auto tile_at = [&](int t, int& kt, int& k0, int& k1) {
    if (t < snt[0]) { k0 = sk0[0]; k1 = sk1[0]; kt = (k0 & ~7) + t * BN; return; }
    t -= snt[0];
    if (t < snt[1]) { k0 = sk0[1]; k1 = sk1[1]; kt = (k0 & ~7) + t * BN; return; }
    t -= snt[1];
    k0 = sk0[2];
    k1 = sk1[2];
    kt = (k0 & ~7) + t * BN;
  };

  bf16x8 qf[NQ];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.qr) + (int64_t(lrow) * a.H + h) * D + 8 * hh;
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) {
      if (row_ok) {
        qf[jj] = *reinterpret_cast<const bf16x8*>(qp + 16 * jj);
      } else {
        s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        qf[jj] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }

  // LDS-DMA source offsets. K: instruction i of this wave fills rows 4c..4c+3
  // (c = wave*CH + i) of 256 bytes; lane l fills physical granule l%16 of row
  // 4c + l/16. V^T in LDS: rows are 128 bytes (64 keys of one d);
  // instruction i fills rows 8c..8c+7, lane l physical granule l%8 of row
  // 8c + l/8, reading the 16 bytes of key block l%8 at that d.
  const int tok_bytes = a.Hkv * D * 2;
  const char* kbase = static_cast<const char*>(a.k) + int64_t(kvh) * D * 2;
  // V^T: 8-key blocks of 128 d-rows (16 bytes each); a tile at kt is the
  // contiguous 16 KiB starting at key block kt / 8
  const char* vtbase = static_cast<const char*>(a.vt) + int64_t(kvh) * a.tpad * D * 2;
  int kgo[CH], vgo[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = wave * CH + i;
    const int krow = 4 * c + (lane >> 4), kp = lane & 15;
    kgo[i] = krow * tok_bytes + 16 * (kp ^ (krow & 15));
    const int d = 8 * c + (lane >> 3), vp = lane & 7;
    vgo[i] = (vp ^ ((d >> 1) & 7)) * (D * 16) + d * 16;
  }
  auto issue = [&](int t, char* kdst, char* vdst) {
    int kt, k0, k1;
    tile_at(t, kt, k0, k1);
    const int valid = min(k1 - kt, BN) * tok_bytes;  // K rows past the span end read as 0
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + int64_t(kt) * tok_bytes, valid);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vtbase + int64_t(kt) * D * 2, (a.tpad - kt) * D * 2);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kdst + (wave * CH + i) * 1024), 16,
                                               kgo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vdst + (wave * CH + i) * 1024), 16,
                                               vgo[i], 0, 0, 0);
    }
  };

  // K operand: lane reads row 32*kb + sigma(ql), logical granule 2*jj + hh.
  const int srow = (ql & ~12) | ((ql & 4) << 1) | ((ql & 8) >> 1);  // sigma: swap bits 2, 3
  int kro[NQ];
#pragma unroll
  for (int jj = 0; jj < NQ; ++jj) kro[jj] = srow * 256 + 16 * ((2 * jj + hh) ^ (srow & 15));
  // V^T operand: lane reads row d = 32*db + ql, keys 32*kb + 16*sub + 8*hh
  // .. +7 = logical granule 4*kb + 2*sub + hh.
  const int vx = (ql >> 1) & 7;
  int vro[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) vro[kb][sub] = ql * 128 + 16 * ((4 * kb + 2 * sub + hh) ^ vx);

  auto qk = [&](const char* kb0, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb0 + kb * 32 * 256 + kro[jj]);
        if (jj == 0) {
          f32x16 z;
#pragma unroll
          for (int t = 0; t < 16; ++t) z[t] = 0.f;
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[jj], z, 0, 0, 0);
        } else {
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[jj], s[kb], 0, 0, 0);
        }
      }
    }
  };

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int t = 0; t < 16; ++t) o[db][t] = 0.f;
  float m_ref = -INFINITY, l = 0.f;
  const float c2 = a.scale_log2;
  const float thr = kRescaleLog2 / c2;

  // Softmax, first half: mask (diagonal and span-edge tiles only), row max,
  // lazy rescale. Branches live here, before the interleaved region.
  auto softmax_max = [&](int t, f32x16 (&s)[2]) {
    int kt, k0, k1;
    tile_at(t, kt, k0, k1);
    // register r of block kb holds key kt + 32*kb + 16*(r/8) + 8*hh + r%8
    if (kt < k0 || kt + BN > k1 || kt + BN - 1 > wave_lo) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
          if (key < k0 || key >= k1 || key > grow) s[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_with_partner(mx);
    const bool grow_ref = mx > m_ref + thr;
    if (__builtin_amdgcn_ballot_w64(grow_ref) != 0) {
      const float m_new = grow_ref ? mx : m_ref;
      const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * c2);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_ref = m_new;
    }
  };

  // One branch-free scheduling region: QK^T of the next tile (independent
  // MFMAs) interleaved with the probabilities of this tile (VALU), then PV
  // of this tile. The group barriers ask the scheduler for that order and
  // keep each K operand read two MFMAs ahead of its use.
  auto interleaved = [&](const char* kread, f32x16 (&sn)[2], const char* vb0, f32x16 (&s)[2]) {
    qk(kread, sn);
    const float ms = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
    bf16x8 pb[2][2];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c2, -ms));
        rs += p;
        pb[kb][r >> 3][r & 7] = (__bf16)p;
      }
    l += rs;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vb0 + db * 32 * 128 + vro[kb][sub]);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kb][sub], o[db], 0, 0, 0);
        }
    // requested order: 2 K reads; 16 x {MFMA, K read, 7 VALU}; then PV with
    // its V^T reads two ahead
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (i < 14) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 7, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (i < 14) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
  };

  // Pipeline (see the comment above the kernel). Step t: wait for tile
  // t+1's K/V^T, barrier, start loading tile t+2 (K slot t%2, V slot
  // (t+2)%3), then QK^T of tile t+1 (K slot (t+1)%2) interleaved with the
  // softmax and PV of tile t (V slot t%3). On the last tile the QK^T reads
  // a stale K slot and its result is unused. Unrolled by six so every slot
  // is a compile-time choice and the two score register sets alternate.
  f32x16 sa[2], sb[2];
  auto step = [&](int t, const char* kread, char* kdst, char* vdst, const char* vread,
                  f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 2 < n_tiles) issue(t + 2, kdst, vdst);
    softmax_max(t, sc);
    interleaved(kread, sn, vread, sc);
    return t + 1 < n_tiles;
  };
  issue(0, k0s, v0s);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (n_tiles > 1) issue(1, k1s, v1s);
  qk(k0s, sa);
  for (int t = 0; t < n_tiles; t += 6) {
    if (!step(t, k1s, k0s, v2s, v0s, sa, sb)) break;
    if (!step(t + 1, k0s, k1s, v0s, v1s, sb, sa)) break;
    if (!step(t + 2, k1s, k0s, v1s, v2s, sa, sb)) break;
    if (!step(t + 3, k0s, k1s, v2s, v0s, sb, sa)) break;
    if (!step(t + 4, k1s, k0s, v0s, v1s, sa, sb)) break;
    if (!step(t + 5, k0s, k1s, v1s, v2s, sb, sa)) break;
  }

  const float lt = sum_with_partner(l);
  if (!row_ok) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // O^T register r of block db holds d = 32*db + 8*(r/4) + 4*hh + r%4
  float* po = a.part_o + ((int64_t(ent.step) * a.R + lrow) * a.H + h) * D + 4 * hh;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int tq = 0; tq < 4; ++tq) {
      const float4 val = make_float4(o[db][4 * tq] * inv, o[db][4 * tq + 1] * inv,
                                     o[db][4 * tq + 2] * inv, o[db][4 * tq + 3] * inv);
      *reinterpret_cast<float4*>(po + 32 * db + 8 * tq) = val;
    }
  if (hh == 0)
    a.part_lse[(int64_t(ent.step) * a.H + h) * a.R + lrow] =
        lt > 0.f ? m_ref * a.scale + logf(lt) : -INFINITY;
}

template <int G>
hipError_t launch_d128(const AttnArgs& a, int n_entries, hipStream_t stream) {
  const int64_t blocks = int64_t(n_entries) * a.n_hg;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_step_bf16_d128_kernel<G>), dim3(uint32_t(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_g(const AttnArgs& a, int n_entries, hipStream_t stream) {
  const int64_t blocks = int64_t(n_entries) * a.n_hg;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_step_bf16_kernel<D, kBf16Waves, G>), dim3(uint32_t(blocks)),
                     dim3(kBf16Waves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, int heads_per_wg, int n_entries,
                            hipStream_t stream) {
  if (n_entries == 0) return hipSuccess;
  if (head_dim == 128) {
    if (heads_per_wg == 4) return launch_d128<4>(a, n_entries, stream);
    if (heads_per_wg == 2) return launch_d128<2>(a, n_entries, stream);
    return launch_d128<1>(a, n_entries, stream);
  }
  if (head_dim == 64) {
    if (heads_per_wg == 4) return launch_g<64, 4>(a, n_entries, stream);
    if (heads_per_wg == 2) return launch_g<64, 2>(a, n_entries, stream);
    return launch_g<64, 1>(a, n_entries, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace cpattn
