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
#include "device_util.h"
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
constexpr int kLdsAhead = 4;             // LDS operand reads issued ahead of their MFMA
constexpr int kWaitVmcnt0 = 0x0F70;       // s_waitcnt vmcnt(0), expcnt and lgkmcnt untouched
// __builtin_amdgcn_sched_group_barrier instruction classes
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedVmemRead = 0x0020;
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
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (int64_t(grow) * a.H + h) * D + 8 * hh;
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
// head_dim 128: ping-pong variant.
//
// Work: one workgroup of 8 waves per (unit, head group), a unit being one
// row tile over the union of its ring steps' key ranges, in key order (or,
// for small grids, one (row tile, step) entry). All of the unit's key tiles
// run through one online softmax: the running output, sum and reference
// carry over span boundaries, so the blocks of every step are merged by the
// log-sum-exp update as they come and no per-step partial leaves the
// registers. Waves w and w+4 share a SIMD; waves 0-3 form group 0 and waves
// 4-7 group 1. Each wave owns 32 query rows of one head; with G query heads
// per KV head (G = 4, 2, 1) a group covers 4/G row blocks of G heads, so the
// workgroup's 8 waves share every K/V tile.
//
// Differences from the kernel above:
//  * V stays in its [T, Hkv, D] layout. The PV product O^T = V^T P^T needs,
//    per lane, 8 consecutive keys at one d; gfx950's transposing LDS read
//    (ds_read_b64_tr_b16) gives exactly that from a row-major V tile: in a
//    16-lane group, lane j receives element j % 4 of the 4-element rows that
//    lanes 4e + j / 4 address (e = 0..3). Two such reads (keys +0..3 and
//    +4..7) form one 8-key operand.
//  * Lane ql of the QK^T operand reads K row sigma(ql), sigma swapping bits
//    2 and 3 of the row index. The S^T accumulator register r of lane half
//    hh then holds key 16*(r/8) + 8*hh + r%8: eight consecutive keys per
//    MFMA operand, exactly the keys of the lane's PV operand.
//  * K and V tiles go from HBM straight into LDS (buffer_load ... lds), no
//    staging registers. One wave instruction fills 1 KiB of LDS (lane l at
//    byte 16*l), so rows are unpadded and bank conflicts are avoided by
//    XOR-swizzling 16-byte granules: K granule g of row r sits at
//    g ^ (r & 15) (16 rows read together land on 16 granule slots); V
//    granule g of row r sits at g ^ f(r), f(r) = ((r & 3) << 2) | ((r >> 2) & 3),
//    so the 4 rows x 4 granules a half-wave's transposing read touches land
//    on 16 distinct slots. All LDS read addresses are per-lane constants
//    plus immediates.
//  * Key tiles start at multiples of 8 keys (keys below the span start are
//    masked like those past its end).
//  * Ping-pong: each wave alternates a softmax phase (VALU: exp, sum,
//    convert) and a matrix phase (MFMA: PV of tile t, QK^T of tile t+1).
//    Group 1 runs one phase behind group 0 and every phase ends at a
//    workgroup barrier, so on each SIMD one wave keeps the matrix core busy
//    while its partner does the vector work.
//  * Matrix phases read each MFMA operand from LDS kLdsAhead MFMAs ahead,
//    which hides LDS latency under load; group 0 spreads the next tile's
//    LDS-DMA loads over the QK^T half of its matrix phase, one every other
//    MFMA, so the memory queue never stalls the matrix work.
//  * Masks of diagonal and span-edge tiles are built as a 64-bit lane mask
//    and applied with bitfield selects, keeping scalar registers free.
// Scalar walk over a unit's 64-key tiles, span after span, each span
// walked from its start rounded down to 8 keys. Holds the current tile
// start kt and its span's [k0, k1).
struct TileCursor {
  int kt, k0, k1, span;
};

template <int G>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_rank_bf16_d128_kernel(const AttnArgs a) {
  constexpr int D = 128, BN = kBlockN;
  constexpr int TILE = BN * D * 2;           // bytes of one K (or V) tile
  constexpr int CH = TILE / 1024 / 4;        // LDS-DMA instructions per loading wave per tensor
  constexpr int ND = D / 32, NQ = D / 16;
  constexpr int RB = 4 / G;                  // row blocks per wave group
  static_assert(BN == 64, "tile walk assumes 64-key tiles");
  __shared__ __attribute__((aligned(1024))) char k0s[TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[TILE];
  typedef __attribute__((address_space(3))) void lds_void;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int grp = wave >> 2, wg = wave & 3;  // waves w and w+4 share a SIMD
  // Workgroup order: unit-major (unit b / n_hg, head group b % n_hg), or
  // XCD-major: workgroups go to the XCDs round-robin (b % 8), and XCD x runs
  // head groups x, x + 8, ... one after another, each over all units.
  int hg, unit_id;
  if (a.xcd_major) {
    const int x = blockIdx.x % 8, slot = blockIdx.x / 8;
    hg = x + 8 * (slot / a.n_units);
    unit_id = slot % a.n_units;
  } else {
    hg = blockIdx.x % a.n_hg;
    unit_id = blockIdx.x / a.n_hg;
  }
  // plan records through scalar views: their loads are scalar, so a wait
  // for one never waits for the K/V loads in flight
  const UnitRec unit = scalar_load(a.units, unit_id);
  const TileRec tile = scalar_load(a.tiles, unit.tile);
  const const_ptr<EntryRec> steps = scalar_view(a.tile_entries) + unit.e0;
  const int n_steps = unit.e1 - unit.e0;
  const int h = hg * G + (wg % G);
  const int rsub = grp * RB + wg / G;
  const int kvh = (hg * G) / a.group;
  const int ql = lane & 31, hh = lane >> 5;
  const int rin = rsub * 32 + ql;
  const bool row_ok = rin < tile.nrows;
  const int lrow = tile.local0 + rin;
  const int grow = tile.g0 + rin;
  const int wave_lo = tile.g0 + rsub * 32;
  // The unit's key spans, contiguous in the span list: the union of its
  // steps' spans in key order (row-tile schedule) or one step's spans.
  const const_ptr<SpanRec> spans = scalar_view(a.spans) + steps[0].span_begin;
  const int n_spans = steps[n_steps - 1].span_end - steps[0].span_begin;
  const int n_tiles = unit.n_tiles;  // the planner counted the unit's 64-key tiles
  auto start = [&](TileCursor& c) {
    c.span = 0;
    c.k0 = spans[0].k0;
    c.k1 = spans[0].k1;
    c.kt = c.k0 & ~7;
  };
  auto advance = [&](TileCursor& c) {
    c.kt += BN;
    if (c.kt >= c.k1 && c.span + 1 < n_spans) {
      ++c.span;
      c.k0 = spans[c.span].k0;
      c.k1 = spans[c.span].k1;
      c.kt = c.k0 & ~7;
    }
  };

  bf16x8 qf[NQ];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (int64_t(grow) * a.H + h) * D + 8 * hh;
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

  // K/V loads are issued by the four waves of group 0 only, in their matrix
  // phases. Wave wg fills 1-KiB pieces wg*CH..+CH-1 of each tile.
  const int tok_bytes = a.Hkv * D * 2;
  const char* kbase = static_cast<const char*>(a.k) + int64_t(kvh) * D * 2;
  const char* vbase = static_cast<const char*>(a.v) + int64_t(kvh) * D * 2;
  // V granule swizzle of tile row r (see the kernel notes)
  auto vswz = [](int r) { return ((r & 3) << 2) | ((r >> 2) & 3); };
  int kgo[CH], vgo[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = wg * CH + i;
    const int krow = 4 * c + (lane >> 4), kp = lane & 15;
    kgo[i] = krow * tok_bytes + 16 * (kp ^ (krow & 15));
    vgo[i] = krow * tok_bytes + 16 * (kp ^ vswz(krow));
  }

  const int srow = (ql & ~12) | ((ql & 4) << 1) | ((ql & 8) >> 1);
  int kro[NQ];
#pragma unroll
  for (int jj = 0; jj < NQ; ++jj) kro[jj] = srow * 256 + 16 * ((2 * jj + hh) ^ (srow & 15));
  // PV operand reads: for d block db and key half tb (keys +4 tb .. +4 tb + 3
  // of the lane's 8), this lane addresses tile row 8 (g >> 1) + 4 tb + s / 4
  // (plus the 16-key step's row offset, an immediate) at d
  // 32 db + 16 (g & 1) + 4 (s % 4), where g = lane / 16 and s = lane % 16.
  int vtr[ND][2];
  {
    const int g16 = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int r = 8 * (g16 >> 1) + 4 * tb + (s16 >> 2);
        const int gran = 4 * db + 2 * (g16 & 1) + ((s16 & 3) >> 1);
        vtr[db][tb] = r * 256 + 16 * (gran ^ vswz(r)) + 8 * (s16 & 1);
      }
  }

  f32x16 sc[2];     // scores of the tile whose softmax is next
  bf16x8 pb[2][2];  // probabilities of the tile whose PV is next
  f32x16 o[ND];     // output of the current ring step, not yet normalised
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int t = 0; t < 16; ++t) o[db][t] = 0.f;
  float m_ref = -INFINITY, l = 0.f;
  const float c2 = a.scale_log2;

  auto qk = [&](const char* kb0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb0 + kb * 32 * 256 + kro[jj]);
        if (jj == 0) {
          f32x16 z;
#pragma unroll
          for (int t = 0; t < 16; ++t) z[t] = 0.f;
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[jj], z, 0, 0, 0);
        } else {
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[jj], sc[kb], 0, 0, 0);
        }
      }
    }
  };
  auto pv = [&](const char* vb0) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const char* const rb = vb0 + (32 * kb + 16 * sub) * 256;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rb + vtr[db][0]));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rb + vtr[db][1]));
          const s16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pb[kb][sub], o[db], 0, 0, 0);
        }
  };
  // Register fences: an empty asm that "reads and writes" the values forces
  // the work producing them to stay before it (barriers order memory only,
  // so arithmetic could otherwise drift into the next phase).
  auto fence_p = [&]() {
    asm volatile("" : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]), "+v"(l), "+v"(m_ref));
  };
  auto fence_s = [&]() {
    asm volatile("" : "+v"(sc[0]), "+v"(sc[1]));
    asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
  };
  // Softmax phase. Probabilities are exp2((s - m_ref) * c2): any reference
  // works while the values stay finite, since the output and the sum share
  // it. The common path computes them against the current reference; only
  // if a row's partial sum exceeds 2^64 (or the row has no reference yet)
  // does the slow path compute the row max, move the reference there,
  // rescale the output and the sum, and recompute.
  auto probs = [&](float& rs) {
    const float ms = (m_ref == -INFINITY) ? 0.f : m_ref * c2;
    rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], c2, -ms));
        rs += p;
        pb[kb][r >> 3][r & 7] = (__bf16)p;
      }
  };
  auto softmax = [&](const TileCursor& c) {
    if (c.kt < c.k0 || c.kt + BN > c.k1 || c.kt + BN - 1 > wave_lo) {
      // Keys of this lane sit at offsets 32kb + 16(r>>3) + (r&7) from
      // kt + 8hh; the visible ones form the range [lo, hi). Build that range
      // as a 64-bit lane mask and select with bitfield ops, so no per-key
      // compare results occupy scalar registers.
      const int base = c.kt + 8 * hh;
      const int lo = min(max(c.k0 - base, 0), 64);
      const int hi = min(max(min(c.k1, grow + 1) - base, 0), 64);
      const uint64_t below_hi = hi >= 64 ? ~0ull : (1ull << hi) - 1;
      const uint64_t below_lo = lo >= 64 ? ~0ull : (1ull << lo) - 1;
      const uint64_t vis = below_hi & ~below_lo;
      const int w0 = int(uint32_t(vis)), w1 = int(uint32_t(vis >> 32));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = __builtin_amdgcn_sbfe(kb ? w1 : w0, 16 * (r >> 3) + (r & 7), 1);
          float y;
          asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(y) : "v"(m), "v"(sc[kb][r]), "v"(-INFINITY));
          sc[kb][r] = y;
        }
    }
    float rs;
    probs(rs);
    const bool redo = (m_ref == -INFINITY) || !(rs <= 0x1p64f);  // also catches NaN
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = max_with_partner(mx);
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * c2);  // 0 if m_ref = -inf
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_ref = m_new;
      probs(rs);
    }
    l += rs;
  };

  // Ping-pong schedule. Each wave runs QK(0), then per tile t a softmax
  // phase S(t) and a matrix phase M(t) = PV(t) + QK(t+1). Group 1 runs one
  // phase behind group 0, so on every SIMD one wave is in a matrix phase
  // while its partner is in a softmax phase; phases end at a workgroup
  // barrier. Load group j = {K(j+1), V(j)} lives in LDS slot j%2. Group 0
  // issues group j inside its matrix phase M(j-1) (phase 2j), spread
  // between the MFMAs, waits for it at the end of its softmax phase S(j)
  // (phase 2j+1), and both groups read it in M(j) (phases 2j+2, 2j+3).
  // The two groups run separate copies of the loop, so neither carries a
  // branch on its group inside a phase. Tiles run through all ring steps of
  // the unit without a break: a step boundary is just the next tile.
  TileCursor cs, ck, cv;   // softmax tile; K and V tiles of the last load group
  start(cs);
  start(ck);
  start(cv);
  // Buffer resources of a load group; past the last tile they cover no
  // bytes (the loads then write zeros into a slot nobody reads again).
  // (readfirstlane: the values are wave-uniform; this keeps them scalar)
  auto krsrc = [&](const TileCursor& c) {
    const int kt = __builtin_amdgcn_readfirstlane(c.kt);
    const int valid = __builtin_amdgcn_readfirstlane(max(min(c.k1 - kt, BN), 0) * tok_bytes);
    return make_rsrc(kbase + int64_t(kt) * tok_bytes, valid);
  };
  auto vrsrc = [&](const TileCursor& c) {
    const int kt = __builtin_amdgcn_readfirstlane(c.kt);
    const int valid = __builtin_amdgcn_readfirstlane(max(min(c.k1 - kt, BN), 0) * tok_bytes);
    return make_rsrc(vbase + int64_t(kt) * tok_bytes, valid);
  };
  // Phase barrier: a bare s_barrier. __syncthreads() would add a release
  // fence, i.e. wait for every outstanding memory operation of the wave --
  // including the LDS-DMA loads group 0 has just issued for a later tile.
  // LDS ordering is explicit here instead: a slot's DMA is waited for
  // (vmcnt) by its issuing waves before the barrier that publishes it, and
  // every LDS read completes inside its phase (its MFMA consumes it). The
  // "memory" clobber keeps the compiler from moving memory accesses across.
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_group = [&](__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, char* kdst, char* vdst) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kdst + (wg * CH + i) * 1024), 16,
                                               kgo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vdst + (wg * CH + i) * 1024), 16,
                                               vgo[i], 0, 0, 0);
    }
  };
  // Matrix phase: PV of tile t and QK^T of tile t+1, 32 MFMAs fed by LDS
  // reads issued kLdsAhead MFMAs ahead. With loads, one
  // LDS-DMA instruction goes out beside every other QK^T MFMA, so the memory
  // queue never holds up the matrix work. On the last tile the QK^T reads a stale K
  // slot; those scores are never used.
  auto matrix = [&](const char* vb, const char* kb, bool loads, char* kdst, char* vdst) {
    pv(vb);
    qk(kb);
    // LDS reads per MFMA: two for the 16 PV MFMAs (transposing reads), one
    // for the 16 QK^T MFMAs; each MFMA's reads go out kLdsAhead MFMAs ahead
    static_assert(kLdsAhead <= 16, "the first kLdsAhead MFMAs are PV MFMAs");
    if (loads) load_group(krsrc(ck), vrsrc(cv), kdst, vdst);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kLdsAhead, 0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      // the 2 CH loads go out in the QK^T half, beside every other MFMA (the PV
      // half's transposing reads keep the LDS busier)
      static_assert(2 * CH == 8, "eight loads per matrix phase");
      if (loads && i >= 16 && i % 2 == 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (i + kLdsAhead < 16)
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      else if (i + kLdsAhead < 32)
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    fence_s();
  };

  // A wave with no rows (in a row tile's tail) runs only the phase
  // barriers, and in group 0 its share of the K/V loads: no matrix or
  // softmax work. The kernel is power-bound, so work skipped on some waves
  // raises the clock of all.
  const bool idle = tile.nrows <= rsub * 32;
  // The walk visits keys in increasing order, and no span reaches past the
  // tile's last row, so the key tiles that lie wholly past this wave's last
  // row (none of its rows can see them) are the last ones of the walk, all
  // in the last span: on a tile that ends on the causal diagonal, up to
  // three of the four diagonal tiles for the first waves. The wave does its
  // matrix and softmax work up to its last visible tile, rounded up to a
  // whole loop iteration (two tiles), and only the barriers (and its loads)
  // after that. The skipped tiles would add exact zeros.
  int t_work = 0;
  if (!idle) {
    const int last_k0 = spans[n_spans - 1].k0, last_k1 = spans[n_spans - 1].k1;
    const int first_kt = last_k0 & ~7;
    const int wave_hi = tile.g0 + min(rsub * 32 + 32, tile.nrows);  // keys >= wave_hi: unseen
    const int in_last = (last_k1 - first_kt + BN - 1) / BN;
    const int seen_last = max(wave_hi - first_kt + BN - 1, 0) / BN;
    const int skip = max(in_last - seen_last, 0);
    t_work = min(n_tiles, (n_tiles - skip + 1) & ~1);
  }

  if (grp == 0) {
    // prologue: K(0) into the slot of group -1 (k1s), group 0 into slot 0
    load_group(krsrc(ck), vrsrc(cv), k1s, v0s);  // V(0) and, harmlessly, K(0) twice
    advance(ck);
    {
      const __amdgpu_buffer_rsrc_t kr = krsrc(ck);
#pragma unroll
      for (int i = 0; i < CH; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(k0s + (wg * CH + i) * 1024), 16,
                                                 kgo[i], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    sync();
    if (!idle) qk(k1s);  // phase 0
    fence_s();
    sync();
    for (int t = 0; t < t_work; t += 2) {
      // phase 2t+1: S(t); prepare load group t+1
      advance(ck);
      advance(cv);
      softmax(cs);
      advance(cs);
      fence_p();
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // group t has landed
      sync();
      matrix(v0s, k0s, true, k1s, v1s);  // phase 2t+2: M(t), loads group t+1
      sync();
      if (t + 1 >= n_tiles) break;
      advance(ck);
      advance(cv);
      softmax(cs);
      advance(cs);
      fence_p();
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      sync();
      matrix(v1s, k1s, true, k0s, v0s);
      sync();
    }
    for (int t = t_work; t < n_tiles; t += 2) {  // (nothing left to see: loads only)
      advance(ck);
      advance(cv);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      sync();
      load_group(krsrc(ck), vrsrc(cv), k1s, v1s);
      sync();
      if (t + 1 >= n_tiles) break;
      advance(ck);
      advance(cv);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      sync();
      load_group(krsrc(ck), vrsrc(cv), k0s, v0s);
      sync();
    }
    // The last matrix phase's loads (past the end of the keys) still write
    // their slots; they land before the barrier, as the epilogue reuses the
    // slots.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    sync();  // group 1's last matrix phase
  } else {
    sync();  // prologue loads
    sync();  // phase 0
    if (!idle) qk(k1s);  // phase 1
    fence_s();
    sync();
    for (int t = 0; t < t_work; t += 2) {
      softmax(cs);
      advance(cs);
      fence_p();
      sync();
      matrix(v0s, k0s, false, nullptr, nullptr);
      sync();
      if (t + 1 >= n_tiles) break;
      softmax(cs);
      advance(cs);
      fence_p();
      sync();
      matrix(v1s, k1s, false, nullptr, nullptr);
      sync();
    }
    for (int t = t_work; t < n_tiles; t += 2) {  // (nothing left to see: barriers only)
      sync();
      sync();
      if (t + 1 >= n_tiles) break;
      sync();
      sync();
    }
  }

  const float lt = sum_with_partner(l);
  if (a.per_step) {
    // One step per unit (small grids): this step's partial goes out in the
    // [P, R, H, D] / [P, H, R] layout for the separate LSE merge pass.
    if (!row_ok) return;
    const int step = steps[0].step;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* const po = a.part_o + ((int64_t(step) * a.R + lrow) * a.H + h) * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int tq = 0; tq < 4; ++tq)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * tq) =
            make_float4(o[db][4 * tq] * inv, o[db][4 * tq + 1] * inv, o[db][4 * tq + 2] * inv,
                        o[db][4 * tq + 3] * inv);
    if (hh == 0)
      a.part_lse[(int64_t(step) * a.H + h) * a.R + lrow] =
          lt > 0.f ? m_ref * a.scale + logf(lt) : -INFINITY;
    return;
  }
  // The online softmax ran across every ring step of the unit, so the
  // running output, sum and reference already merge all steps' blocks.
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (row_ok && hh == 0) a.lse[int64_t(h) * a.R + lrow] = lt > 0.f ? m_ref * a.scale + logf(lt) : -INFINITY;
  // The output goes out through LDS: a lane holds 4 consecutive d of one
  // row per (db, tq), so a direct store writes 16 bytes into each of 32 rows
  // 8 KiB apart. Each wave writes its 32 rows x 256 bytes into its own 8 KiB
  // of the K/V slots (16-byte granules XOR-swizzled by row), reads them
  // back as whole rows and stores 256-byte rows, 16 lanes each, four rows
  // per instruction. After the last barrier no LDS read of a matrix phase
  // and no LDS-DMA load is outstanding, so the slots are free.
  char* const stg = (wave < 2 ? k0s : wave < 4 ? k1s : wave < 6 ? v0s : v1s) + (wave & 1) * 8192;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int tq = 0; tq < 4; ++tq) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 val = {(__bf16)(o[db][4 * tq] * inv), (__bf16)(o[db][4 * tq + 1] * inv),
                          (__bf16)(o[db][4 * tq + 2] * inv), (__bf16)(o[db][4 * tq + 3] * inv)};
      *reinterpret_cast<bf16x4*>(stg + ql * 256 + 16 * ((4 * db + tq) ^ (ql & 15)) + 8 * hh) = val;
    }
  const int gran = lane & 15;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = 4 * k + (lane >> 4);  // row of the wave's 32
    const uint4 val = *reinterpret_cast<const uint4*>(stg + r * 256 + 16 * (gran ^ (r & 15)));
    if (rsub * 32 + r < tile.nrows) {
      char* const dst = static_cast<char*>(a.out) + ((int64_t(tile.local0 + rsub * 32 + r) * a.H + h) * D) * 2;
      *reinterpret_cast<uint4*>(dst + 16 * gran) = val;
    }
  }
}

template <int G>
hipError_t launch_units(const AttnArgs& a, int n_units, hipStream_t stream) {
  const int64_t blocks = int64_t(n_units) * a.n_hg;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_rank_bf16_d128_kernel<G>), dim3(uint32_t(blocks)), dim3(512), 0, stream, a);
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
  if (head_dim == 64) {
    if (heads_per_wg == 4) return launch_g<64, 4>(a, n_entries, stream);
    if (heads_per_wg == 2) return launch_g<64, 2>(a, n_entries, stream);
    return launch_g<64, 1>(a, n_entries, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bf16_units(const AttnArgs& a, int heads_per_wg, int n_units,
                                  hipStream_t stream) {
  if (n_units == 0) return hipSuccess;
  if (heads_per_wg == 4) return launch_units<4>(a, n_units, stream);
  if (heads_per_wg == 2) return launch_units<2>(a, n_units, stream);
  return launch_units<1>(a, n_units, stream);
}

}  // namespace cpattn
