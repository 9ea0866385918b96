// Gradients of one CP rank's attention share, bf16 inputs, head_dim 128.
//
// The forward gives each rank's rows out = softmax(S) V with S = Q K^T / sqrt(D)
// over the keys its ring steps expose (causal, within a sample). For a loss
// gradient dO on those rows, with P = exp(S - lse) (the forward's merged
// log-sum-exp) and Delta = rowsum(dO * O):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),
//   dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D).
// Ring Attention runs the same blockwise steps in reverse for the backward;
// on one GPU every step's K/V is in HBM, so the ring steps only decide which
// keys each row sees (the forward's spans), and the gradients of a key sum
// over the rank's rows and the query heads that read its KV head.
//
// Three kernels, no atomics (results are deterministic):
//  * prep: Delta[h][r] = sum_d dO[r][h][d] * O[r][h][d], and per 32-row block
//    and head a record of lse * log2(e), Delta and each row's visible key
//    range that the dK/dV kernel stages through LDS with its operands;
//  * dQ: one workgroup of 4 waves per (row tile, head group), two
//    workgroups per compute unit; each wave owns 32 rows of one head and
//    walks the tile's key spans over all ring steps, 32 keys at a time,
//    recomputing S^T = K Q^T and dP^T = V dO^T (K and V rows from LDS, Q and
//    dO in registers) and accumulating dQ^T += K^T dS^T, the K^T operand
//    read from the same row-major K tile with transposing LDS reads. The
//    steps are software-pipelined: the scores of tile t + 1 go to the matrix
//    cores while the vector units turn tile t's scores into dS, then tile
//    t's dQ product follows. K and V tiles stream through a four-slot LDS
//    ring (64 KiB), two tiles ahead of the scores;
//  * dK/dV: one workgroup of 8 waves per (128-key tile, KV head); waves w
//    and w + 4 share a SIMD and 32 keys, and walk the rank's 32-row blocks
//    that see the tile, for every query head of the KV head. Wave w keeps
//    the keys' K rows in registers and computes S = Q K^T, P and
//    dV += P^T dO; wave w + 4 keeps V, computes dP = dO V^T, takes P
//    through LDS, and computes dS = P (dP - Delta) and dK += dS^T Q, one
//    step behind. The two waves of a SIMD alternate matrix and vector
//    phases (ping-pong, two barriers per step). The dO and Q operands of
//    the products are read from the
//    same row-major tiles with transposing LDS reads. The accumulator
//    layout of S (keys in lanes, rows in registers) is directly the A
//    operand of those products once the rows are read in the order sigma
//    (bits 2 and 3 of the row swapped). The row blocks stream through a
//    four-slot LDS ring, two blocks ahead, so no wave waits on memory
//    inside a step.
#include "device_util.h"
#include "kernels.h"

namespace cpattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBufferWord3 = 0x00020000;  // raw buffer access, gfx9 family

// s_waitcnt immediate for vmcnt(n) alone (n < 64: low four bits in [3:0],
// high two in [15:14]; expcnt 7 and lgkmcnt 15 mean "no wait").
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Granule swizzle of row r of a row-major LDS tile (16-byte granule g of row
// r sits at slot g ^ tile_swizzle(r)). It is a bijection of r & 15, so 16
// rows read at one granule land on 16 slots, and the 4 rows x 4 granules
// that a half-wave's transposing read touches land on 16 slots too.
__device__ inline int tile_swizzle(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Transposing LDS read (ds_read_b64_tr_b16): in a 16-lane group, lane j
// receives element j % 4 of the 4-element rows that lanes 4e + j / 4
// address (e = 0..3). tr_offsets gives, for an operand of 8 consecutive tile
// rows R0 + 8 (lane / 32) + 0..7 at column c0 + lane % 32 (R0 a multiple of
// 16, c0 of 32; the row offset R0 * 256 is added by the caller), the two
// per-lane byte offsets of its halves (rows +0..3 and +4..7); the tile has
// 256-byte rows swizzled by tile_swizzle.
__device__ inline void tr_offsets(int lane, int c0, int (&off)[2]) {
  const int g = lane >> 4, s = lane & 15;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int r = 8 * (g >> 1) + 4 * tb + (s >> 2);
    const int gran = c0 / 8 + 2 * (g & 1) + ((s & 3) >> 1);
    off[tb] = r * 256 + 16 * (gran ^ tile_swizzle(r)) + 8 * (s & 1);
  }
}
__device__ inline bf16x8 tr_read8(const char* base, const int (&off)[2]) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off[0]));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off[1]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferWord3);
}

__device__ inline float sum_with_partner16(float x) {
  // sum over the 16 lanes of a quarter-wave (xor butterflies)
  x += __shfl_xor(x, 8, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 1, 16);
  return x;
}

// ---------------------------------------------------------------- prep
// 16 lanes per (row, head) pair, D/16 elements each; 16 pairs per 256
// threads; rows up to 32 nrb (rows >= R get pad records). Any input dtype
// (bf16 or fp32) and head_dim (64 or 128).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const T* __restrict__ out, const T* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      const int32_t* __restrict__ index,
                                                      const int32_t* __restrict__ row_lo,
                                                      float* __restrict__ delta, int32_t* __restrict__ rec,
                                                      int32_t R, int32_t H, int32_t nrb) {
  constexpr int E = D / 16;
  const int64_t pair = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool ok = pair < int64_t(nrb) * kBwdRowBlock * H;
  const int64_t pc = ok ? pair : 0;  // inactive groups read pair 0 and store nothing
  const int r = int(pc / H), h = int(pc % H);
  const bool in = r < R;
  float s = 0.f;
  if (in) {
    const int64_t off = (int64_t(r) * H + h) * D + sub * E;  // [R, H, D]
#pragma unroll
    for (int i = 0; i < E; ++i) s = __builtin_fmaf(float(out[off + i]), float(dout[off + i]), s);
  }
  s = sum_with_partner16(s);
  if (!ok || sub != 0) return;
  if (in) delta[int64_t(h) * R + r] = s;
  const int gid = in ? index[r] : -1;
  const bool real = gid >= 0;
  int32_t* const w = rec + (int64_t(h) * nrb + r / kBwdRowBlock) * (4 * kBwdRowBlock) + r % kBwdRowBlock;
  w[0] = __float_as_int(real ? lse[int64_t(h) * R + r] * kLog2e : INFINITY);
  w[kBwdRowBlock] = __float_as_int(real ? s : 0.f);
  w[2 * kBwdRowBlock] = real ? row_lo[r] : 0;
  w[3 * kBwdRowBlock] = real ? gid - row_lo[r] : -1;
}

// Scalar walk over a unit's 64-key tiles (as in the forward).
struct Cursor {
  int kt, k0, k1, span;
};

// ---------------------------------------------------------------- dQ
// __builtin_amdgcn_sched_group_barrier instruction classes
constexpr int kSchedValu = 0x0002;
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;
// One pipelined dQ step: the 16 score MFMAs of the next tile, each with its
// LDS read issued kDqAhead MFMAs ahead and a share of this tile's dS vector
// work beside it, then the 8 dQ MFMAs (two transposing reads each).
constexpr int kDqAhead = 2;
constexpr int kDqValuPerMfma = 7;
__device__ inline void schedule_dq_step() {
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kDqAhead, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, kDqValuPerMfma, 0);
    if (i + kDqAhead < 16) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (i + 2 < 8) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
  }
}

template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(const BwdArgs a) {
  constexpr int D = 128, BN = 32, NQ = 8, ND = 4, RB = 4 / G;
  constexpr int TILE = BN * D * 2;     // bytes of a K or V tile
  constexpr int CH = TILE / 1024 / 4;  // LDS-DMA instructions per wave per tensor
  constexpr int PER_STAGE = 2 * CH;    // LDS-DMA instructions per wave per tile
  // ring slots: K tile, then V tile
  __shared__ __attribute__((aligned(1024))) char sl0[2 * TILE], sl1[2 * TILE], sl2[2 * TILE], sl3[2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // unit-major (unit b / n_hg, head group b % n_hg) or XCD-major order
  int hg, unit_id;
  if (a.q_xcd_major) {
    const int x = blockIdx.x % 8, slot = blockIdx.x / 8;
    hg = x + 8 * (slot / a.n_units);
    unit_id = slot % a.n_units;
  } else {
    hg = blockIdx.x % a.n_hg;
    unit_id = blockIdx.x / a.n_hg;
  }
  const UnitRec unit = scalar_load(a.units, unit_id);
  const TileRec tile = scalar_load(a.tiles, unit.tile);
  const const_ptr<EntryRec> steps = scalar_view(a.tile_entries) + unit.e0;
  const int n_steps = unit.e1 - unit.e0;
  const int h = hg * G + (wave % G);
  const int rsub = wave / G;
  const int kvh = (hg * G) / a.group;
  const int ql = lane & 31, hh = lane >> 5;
  const int rin = rsub * 32 + ql;
  const bool row_ok = rin < tile.nrows;
  const int lrow = tile.local0 + rin;
  const int grow = tile.g0 + rin;
  static_assert(RB * G == 4, "4 waves");
  const const_ptr<SpanRec> spans = scalar_view(a.spans) + steps[0].span_begin;
  const int n_spans = steps[n_steps - 1].span_end - steps[0].span_begin;
  static_assert(BN == kDqBlockN, "the backward plan counts dQ key tiles");
  const int n_tiles = unit.n_tiles;  // the planner counted the unit's BN-key tiles
  auto start = [&](Cursor& c) {
    c.span = 0;
    c.k0 = spans[0].k0;
    c.k1 = spans[0].k1;
    c.kt = c.k0 & ~7;
  };
  auto advance = [&](Cursor& c) {
    c.kt += BN;
    if (c.kt >= c.k1 && c.span + 1 < n_spans) {
      ++c.span;
      c.k0 = spans[c.span].k0;
      c.k1 = spans[c.span].k1;
      c.kt = c.k0 & ~7;
    }
  };

  // Q and dO as B operands: lane holds row ql, d = 16 jj + 8 hh + 0..7.
  bf16x8 qf[NQ], df[NQ];
  {
    const int64_t roff = (int64_t(lrow) * a.H + h) * D + 8 * hh;
    const __bf16* qp = static_cast<const __bf16*>(a.qr) + roff;
    const __bf16* dp = static_cast<const __bf16*>(a.dout) + roff;
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) {
      if (row_ok) {
        qf[jj] = *reinterpret_cast<const bf16x8*>(qp + 16 * jj);
        df[jj] = *reinterpret_cast<const bf16x8*>(dp + 16 * jj);
      } else {
        const s16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        qf[jj] = __builtin_bit_cast(bf16x8, z);
        df[jj] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }
  // exp2 offset of this row: P = exp2(S * c2 - lse * log2 e); rows outside
  // the tile get +inf (P = 0)
  const float lse2 = row_ok ? a.lse[int64_t(h) * a.R + lrow] * kLog2e : INFINITY;
  const float dl = row_ok ? a.delta[int64_t(h) * a.R + lrow] : 0.f;
  const float c2 = a.scale_log2;

  // LDS-DMA offsets: K and V rows are 256-byte tile rows swizzled by
  // tile_swizzle; every wave loads a quarter of each tile.
  const int tok_bytes = a.Hkv * D * 2;
  const char* kbase = static_cast<const char*>(a.k) + int64_t(kvh) * D * 2;
  const char* vbase = static_cast<const char*>(a.v) + int64_t(kvh) * D * 2;
  int kgo[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = wave * CH + i;
    const int krow = 4 * c + (lane >> 4), kp = lane & 15;
    kgo[i] = krow * tok_bytes + 16 * (kp ^ tile_swizzle(krow));
  }
  auto issue = [&](const Cursor& c, char* kd, char* vd) {
    const int kt = __builtin_amdgcn_readfirstlane(c.kt);
    const int valid = __builtin_amdgcn_readfirstlane(max(min(c.k1 - kt, BN), 0) * tok_bytes);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + int64_t(kt) * tok_bytes, valid);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + int64_t(kt) * tok_bytes, valid);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kd + (wave * CH + i) * 1024), 16, kgo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vd + (wave * CH + i) * 1024), 16, kgo[i], 0, 0, 0);
    }
  };

  const int srow = (ql & ~12) | ((ql & 4) << 1) | ((ql & 8) >> 1);
  int kro[NQ];
#pragma unroll
  for (int jj = 0; jj < NQ; ++jj) kro[jj] = srow * 256 + 16 * ((2 * jj + hh) ^ tile_swizzle(srow));
  // K^T operands of dQ^T += K^T dS^T: transposing reads of the K tile
  int ktr[ND][2];
#pragma unroll
  for (int db = 0; db < ND; ++db) tr_offsets(lane, 32 * db, ktr[db]);

  f32x16 acc[ND];  // dQ^T: d = 32 db + 8 (t/4) + 4 hh + t%4 ... (rows in lanes)
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[db][t] = 0.f;

  // Scores of a tile: S^T = K Q^T and dP^T = V dO^T (register r of lane
  // half hh holds key kt + 16 (r / 8) + 8 hh + r % 8 of row ql).
  auto scores = [&](const char* ks, const char* vs, f32x16& s, f32x16& dp) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      s[t] = 0.f;
      dp[t] = 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + kro[jj]);
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs + kro[jj]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[jj], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[jj], dp, 0, 0, 0);
    }
  };
  // dS = P (dP - Delta) of a tile, as the bf16 B operands of dQ^T += K^T dS^T
  auto dscores = [&](const Cursor& c, const f32x16& s, const f32x16& dp, bf16x8 (&dsb)[2]) {
    // visible keys of this lane's row, as bits relative to kt + 8 hh (in a
    // tile inside the span and below the wave's first row this is all ones
    // on the bits the lane uses)
    const int base = c.kt + 8 * hh;
    const int lo = min(max(c.k0 - base, 0), 32);
    const int hi = min(max(min(c.k1, grow + 1) - base, 0), 32);
    const uint32_t below_hi = hi >= 32 ? ~0u : (1u << hi) - 1;
    const uint32_t below_lo = lo >= 32 ? ~0u : (1u << lo) - 1;
    const int w0 = int(below_hi & ~below_lo);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = __builtin_amdgcn_sbfe(w0, 16 * (r >> 3) + (r & 7), 1);
      float arg;
      asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(arg) : "v"(m), "v"(__builtin_fmaf(s[r], c2, -lse2)), "v"(-INFINITY));
      const float p = __builtin_amdgcn_exp2f(arg);
      dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dl));
    }
  };
  auto dq_update = [&](const char* ks, const bf16x8 (&dsb)[2]) {
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const bf16x8 tf = tr_read8(ks + 16 * sub * 256, ktr[db]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf, dsb[sub], acc[db], 0, 0, 0);
      }
  };

  // Software pipeline over a ring of four LDS slots (tile t in slot t % 4):
  // step t computes the scores of tile t + 1 while the vector units turn the
  // scores of tile t into dS, then adds tile t's dQ product. Tiles t + 2 and
  // t + 3 are in flight meanwhile; tile t + 3 goes into the slot tile t - 1
  // left (every wave finished it before this step's barrier). Every step
  // issues a tile -- past the last one the loads cover no bytes and write
  // zeros into a slot nobody reads again -- so every step waits for the same
  // count. On the last step the scores read a slot holding no tile; they are
  // never used. The main loop runs whole groups of four steps with no
  // condition inside: where paths with different loads in flight merge, the
  // compiler's own LDS-DMA tracking falls back to waiting for every load.
  Cursor cs, cl;
  start(cs);
  start(cl);
  issue(cl, sl0, (sl0 + TILE));
  advance(cl);
  issue(cl, sl1, (sl1 + TILE));
  advance(cl);
  issue(cl, sl2, (sl2 + TILE));
  f32x16 s0, d0, s1, d1;
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * PER_STAGE));
  asm volatile("s_barrier" ::: "memory");
  scores(sl0, (sl0 + TILE), s0, d0);
#define DQ_STEP(T, KC, KN, VN, KL, VL, SC, DC, SN, DN)                \
  {                                                                   \
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(PER_STAGE));                \
    asm volatile("s_barrier" ::: "memory");                           \
    advance(cl);                                                      \
    issue(cl, KL, VL);                                                \
    scores(KN, VN, SN, DN);                                           \
    bf16x8 dsb[2];                                                    \
    dscores(cs, SC, DC, dsb);                                         \
    dq_update(KC, dsb);                                               \
    schedule_dq_step();                                               \
    advance(cs);                                                      \
  }
  int t = 0;
  for (; t + 4 <= n_tiles; t += 4) {
    DQ_STEP(t, sl0, sl1, (sl1 + TILE), sl3, (sl3 + TILE), s0, d0, s1, d1);
    DQ_STEP(t + 1, sl1, sl2, (sl2 + TILE), sl0, (sl0 + TILE), s1, d1, s0, d0);
    DQ_STEP(t + 2, sl2, sl3, (sl3 + TILE), sl1, (sl1 + TILE), s0, d0, s1, d1);
    DQ_STEP(t + 3, sl3, sl0, (sl0 + TILE), sl2, (sl2 + TILE), s1, d1, s0, d0);
  }
  if (t < n_tiles) {
    DQ_STEP(t, sl0, sl1, (sl1 + TILE), sl3, (sl3 + TILE), s0, d0, s1, d1);
    if (t + 1 < n_tiles) DQ_STEP(t + 1, sl1, sl2, (sl2 + TILE), sl0, (sl0 + TILE), s1, d1, s0, d0);
    if (t + 2 < n_tiles) DQ_STEP(t + 2, sl2, sl3, (sl3 + TILE), sl1, (sl1 + TILE), s0, d0, s1, d1);
  }
#undef DQ_STEP

  if (!row_ok) return;
  float* const dq = a.dq + (int64_t(lrow) * a.H + h) * D + 4 * hh;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int tq = 0; tq < 4; ++tq)
      *reinterpret_cast<float4*>(dq + 32 * db + 8 * tq) =
          make_float4(acc[db][4 * tq] * a.scale, acc[db][4 * tq + 1] * a.scale,
                      acc[db][4 * tq + 2] * a.scale, acc[db][4 * tq + 3] * a.scale);
}

// ---------------------------------------------------------------- dK / dV
// s_waitcnt immediate for vmcnt(n) and lgkmcnt(0) together.
constexpr int wait_vmcnt_lgkm0(int n) { return (wait_vmcnt(n) & ~0x0F00); }
// A matrix phase of the dK/dV kernel: 8 product MFMAs (two transposing LDS
// reads each), then 8 score MFMAs (one LDS read each); every MFMA's reads go
// out kPhaseAhead MFMAs before it.
constexpr int kPhaseAhead = 4;
__device__ inline void schedule_matrix_phase() {
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPhaseAhead, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (i + kPhaseAhead < 8)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    else if (i + kPhaseAhead < 16)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
}

// A matrix phase of two steps: 16 product MFMAs (two transposing LDS reads
// each), then 16 score MFMAs (one LDS read each); reads kPhaseAhead MFMAs
// ahead.
__device__ inline void schedule_matrix_phase2() {
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPhaseAhead, 0);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (i + kPhaseAhead < 16)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    else if (i + kPhaseAhead < 32)
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkdv_kernel(const BwdArgs a) {
  constexpr int D = 128, NQ = 8, ND = 4, RBK = kBwdRowBlock;
  constexpr int ROWT = RBK * D * 2;    // bytes of a 32-row Q or dO tile
  constexpr int CH = ROWT / 1024 / 8;  // 16-byte LDS-DMA instructions per wave per tile (1)
  static_assert(kBwdKeyTile == 128 && RBK == 32 && CH == 1, "4 wave pairs of 32 keys, 32-row blocks");
  // One ring slot: Q | dO | row records (every wave loads 256 B of records;
  // the first 512 B are the record, the rest reads as zeros).
  constexpr int OQ = 0, OD = ROWT, OREC = 2 * ROWT;
  constexpr int STAGE = 2 * ROWT + 2048;
  constexpr int REC_BYTES = 4 * RBK * 4;
  // LDS-DMA instructions per partner wave per slot: the four partner waves
  // issue every load (two 1-KiB pieces of Q and of dO, and a record piece);
  // the P waves, whose matrix phase starts right after the barrier, issue none
  constexpr int PER_STAGE = 4 * CH + 1;
  // P of one step, from the P wave of each pair to its partner: bf16, in the
  // register order of the P wave (two 16-byte pieces per lane)
  constexpr int PBUF = 4 * 2 * 1024;
  // Each loop iteration takes two consecutive steps (a double step), so a
  // matrix phase holds 32 MFMAs: a ring of four slot pairs (two steps
  // each), and one P buffer with a half per step of the pair -- the P waves
  // write it in phase B, the partners read it in the next phase A, and the
  // barrier between the two phases orders the next write after those reads.
  // 8 x 18 KiB + 16 KiB = the 160 KiB of LDS of a compute unit.
  __shared__ __attribute__((aligned(1024))) char s0[STAGE], s1[STAGE], s2[STAGE], s3[STAGE];
  __shared__ __attribute__((aligned(1024))) char s4[STAGE], s5[STAGE], s6[STAGE], s7[STAGE];
  __shared__ __attribute__((aligned(1024))) char pbf[2 * PBUF];
  static_assert(8 * STAGE + 2 * PBUF <= 160 * 1024, "LDS of one compute unit");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;           // waves w and w + 4 share a SIMD and 32 keys
  const bool pwave = wave < 4;         // S, P, dV; its partner: dP, dS, dK
  // tile-major (key tile b / Hkv, KV head b % Hkv) or XCD-major order
  int g, kt_id;
  if (a.kv_xcd_major) {
    const int x = blockIdx.x % 8, slot = blockIdx.x / 8;
    g = x + 8 * (slot / a.n_ktiles);
    kt_id = slot % a.n_ktiles;
  } else {
    g = blockIdx.x % a.Hkv;
    kt_id = blockIdx.x / a.Hkv;
  }
  const KeyTileRec kt = scalar_load(a.ktiles, kt_id);
  const const_ptr<int32_t> blk = scalar_view(a.blk);
  const int kl = lane & 31, hh = lane >> 5;
  const int kw0 = kt.k0 + 32 * pair;  // the pair's first key
  const int key = kw0 + kl;           // this lane's key (column of S)

  // K (P wave) or V (partner) rows of the pair's 32 keys as B operands:
  // lane holds key kl, d = 16 jj + 8 hh + 0..7. Keys >= k1 read as zeros.
  bf16x8 kv[NQ];
  {
    const int tok_bytes = a.Hkv * D * 2;
    const int valid = __builtin_amdgcn_readfirstlane(max(min(kt.k1 - kw0, 32), 0) * tok_bytes);
    const int64_t base = (int64_t(kw0) * a.Hkv + g) * D * 2;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(static_cast<const char*>(pwave ? a.k : a.v) + base, valid);
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) {
      const int off = kl * tok_bytes + (16 * jj + 8 * hh) * 2;
      kv[jj] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
  }

  // LDS-DMA offsets. Q and dO row tiles are 32 rows x 256 B, swizzled by
  // tile_swizzle: wave w fills rows 4w..4w+3 of each.
  const int row_bytes = a.H * D * 2;
  int ngo[2];  // partner wave of pair p: rows 4 (p + 4 i) .. + 3, i = 0, 1
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * (pair + 4 * i) + (lane >> 4), p = lane & 15;
    ngo[i] = r * row_bytes + 16 * (p ^ tile_swizzle(r));
  }
  // the (row block, head) steps: rb in [rb0, rb1) outer, the query heads of
  // KV head g (a.group of them) inner
  const int group = a.group;
  const int n_blocks = (kt.rb1 - kt.rb0) * group;
  // Position of a block step j = (rb - rb0) * group + hq: its row block and
  // query head within the group, advanced one step at a time (no division
  // in the loop); past the last step it stays there.
  struct StepPos {
    int rb, hq, j;
  };
  const int last = n_blocks - 1;
  auto next = [&](StepPos& p) {
    if (p.j < last) {
      ++p.j;
      if (++p.hq == group) {
        p.hq = 0;
        ++p.rb;
      }
    }
  };
  auto issue = [&](const StepPos& p, char* st) {
    const int rb = p.rb, h = g * group + p.hq;
    const int r0 = rb * RBK;
    const int valid = __builtin_amdgcn_readfirstlane(max(min(a.R - r0, RBK), 0) * row_bytes);
    const int64_t noff = (int64_t(r0) * a.H + h) * D * 2;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(static_cast<const char*>(a.qr) + noff, valid);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(static_cast<const char*>(a.dout) + noff, valid);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.rec + (int64_t(h) * a.nrb + rb) * (4 * RBK), REC_BYTES);
    if (pwave) return;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void*)(st + OQ + (pair + 4 * i) * 1024), 16, ngo[i], 0, 0,
                                               0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void*)(st + OD + (pair + 4 * i) * 1024), 16, ngo[i], 0, 0,
                                               0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void*)(st + OREC + pair * 256), 4, pair * 256 + 4 * lane,
                                             0, 0, 0);
  };
  // A operands of S (Q) and dP (dO): lane reads row sigma(kl) of the tile
  const int srow = (kl & ~12) | ((kl & 4) << 1) | ((kl & 8) >> 1);
  int nro[NQ];
#pragma unroll
  for (int jj = 0; jj < NQ; ++jj) nro[jj] = srow * 256 + 16 * ((2 * jj + hh) ^ tile_swizzle(srow));
  // B operands of dV (dO) and dK (Q) -- rows 16 kk + 8 hh + 0..7 at
  // d = 32 db + kl -- by transposing reads of the same tiles
  int ttr[ND][2];
#pragma unroll
  for (int db = 0; db < ND; ++db) tr_offsets(lane, 32 * db, ttr[db]);

  f32x16 acc[ND];  // dV (P wave) or dK (partner): key 32 pair + (t/4)*8 + 4 hh + t%4, d = 32 db + kl
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[db][t] = 0.f;
  const float c2 = a.scale_log2;

  // scores: S = Q K^T (P wave) or dP = dO V^T (partner) of a slot. Register
  // t of lane half hh holds row 32 rb + 16 (t / 8) + 8 hh + t % 8.
  auto scores = [&](const char* tile, f32x16& s) {
#pragma unroll
    for (int t = 0; t < 16; ++t) s[t] = 0.f;
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(tile + nro[jj]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, kv[jj], s, 0, 0, 0);
    }
  };
  // the product acc += A^T B for A in the P wave's register order (pa) and
  // B the tile read transposed (dO for dV, Q for dK)
  auto product = [&](const bf16x8 (&pa)[2], const char* tile) {
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk], tr_read8(tile + 16 * kk * 256, ttr[db]), acc[db],
                                                          0, 0, 0);
  };
  // P wave, step j in slot st: the mask on S, P = exp2(S c2 - lse log2 e)
  // (0 for pad rows, whose record holds +inf), P to the partner
  // The softmax inputs that do not depend on S: the row block's bounds (an
  // 8-byte scalar load) and the rows' lse log2 e from the slot's record,
  // loaded at the end of the P wave's matrix phase so that their latency
  // passes under the phase barrier.
  struct SoftIn {
    int64_t bounds;
    f32x4 l2[2][2];
  };
  auto p_softmax_in = [&](int rb, const char* st, SoftIn& in) {
    const int* const rec = reinterpret_cast<const int*>(st + OREC);
    in.bounds = *(const_ptr<int64_t>)(blk + 2 * rb);
#pragma unroll
    for (int run = 0; run < 2; ++run)
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4)
        in.l2[run][q4] = *reinterpret_cast<const f32x4*>(rec + 16 * run + 8 * hh + 4 * q4);
  };
  auto p_softmax = [&](const SoftIn& in, const char* st, f32x16& s, bf16x8 (&pa)[2], char* pbuf, bool valid) {
    const int* const rec = reinterpret_cast<const int*>(st + OREC);
    // every row of the block sees every key of the pair unless the block
    // holds a causal edge or a sample boundary; then S = -inf where the key
    // is outside [sample start, row's global id]
    const int64_t bounds = in.bounds;
    if (!((int(bounds) <= kw0) & (kw0 + 31 <= int(bounds >> 32)))) {
#pragma unroll
      for (int run = 0; run < 2; ++run)
#pragma unroll
        for (int q4 = 0; q4 < 2; ++q4) {
          const int row = 16 * run + 8 * hh + 4 * q4;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(rec + 2 * RBK + row);
          const i32x4 sp = *reinterpret_cast<const i32x4*>(rec + 3 * RBK + row);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 8 * run + 4 * q4 + e;
            const bool vis = uint32_t(key - lo[e]) <= uint32_t(sp[e]);
            s[t] = vis ? s[t] : -INFINITY;
          }
        }
    }
#pragma unroll
    for (int run = 0; run < 2; ++run)
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        const f32x4 l2 = in.l2[run][q4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pa[run][4 * q4 + e] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * run + 4 * q4 + e], c2, -l2[e]));
      }
    if (!valid) {  // the step past the end of an odd count: it adds nothing
#pragma unroll
      for (int run = 0; run < 2; ++run)
#pragma unroll
        for (int e = 0; e < 8; ++e) pa[run][e] = (__bf16)0.f;
    }
    bf16x8* const pw = reinterpret_cast<bf16x8*>(pbuf + pair * 2048) + lane;
    pw[0] = pa[0];
    pw[64] = pa[1];
  };
  // partner, the step in slot st: dS = P (dP - Delta) with P from its P wave
  auto p_ds = [&](const char* st, const char* pbuf, const f32x16& dp, bf16x8 (&dsa)[2]) {
    const bf16x8* const pr = reinterpret_cast<const bf16x8*>(pbuf + pair * 2048) + lane;
    const bf16x8 pa[2] = {pr[0], pr[64]};
    const int* const rec = reinterpret_cast<const int*>(st + OREC);
#pragma unroll
    for (int run = 0; run < 2; ++run)
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        const f32x4 dl = *reinterpret_cast<const f32x4*>(rec + RBK + 16 * run + 8 * hh + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q4 + e;
          dsa[run][i] = (__bf16)(float(pa[run][i]) * (dp[8 * run + i] - dl[e]));
        }
      }
  };

  // Double steps J = 0 .. n_pairs - 1 take steps 2J and 2J + 1 (the second
  // past the end when n_blocks is odd). Double step J sits in slot pair
  // J % 4; pairs J + 1 and J + 2 are in flight while J is consumed.
  // Iteration J has two phases, each ending at a workgroup barrier, and in
  // each phase one wave of a pair works on the matrix cores while its
  // partner does vector work:
  //   phase A: P wave   dV += P(J-1)^T dO(J-1), then S(J) = Q(J) K^T  (MFMA)
  //            partner  dS(J-1) = P(J-1) (dP(J-1) - Delta)           (VALU)
  //   phase B: P wave   mask, P(J) = exp2(...), P(J) to LDS          (VALU)
  //            partner  dK += dS(J-1)^T Q(J-1), then dP(J) = dO(J) V^T (MFMA)
  // (each for both steps of the pair). Pair J + 2 is issued at the start of
  // iteration J into the slots of pair J - 2, which both waves finished in
  // iteration J - 1. Every iteration issues one pair (past the end, the last
  // step again), so the count of loads in flight after pair J's is always
  // one pair's.
  const int n_pairs = (n_blocks + 1) / 2;
  StepPos ip = {kt.rb0, 0, 0};  // the next step to issue
  StepPos cp = {kt.rb0, 0, 0};  // the step the P waves compute
  if (n_blocks > 0) {
    issue(ip, s0);
    next(ip);
    issue(ip, s1);
    next(ip);
    issue(ip, s2);
    next(ip);
    issue(ip, s3);
    next(ip);
  }
  // The slots of pair -1 (s6, s7) and the P buffer hold zeros, so the first
  // iteration's products of pair -1 add nothing and the phases need no
  // branch on the step.
  {
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint4* const zs = reinterpret_cast<uint4*>(t == 0 ? s6 : s7);
#pragma unroll
      for (int i = 0; i < STAGE / 16 / 512; ++i) zs[i * 512 + tid] = z;
      if (tid < (STAGE / 16) % 512) zs[(STAGE / 16 / 512) * 512 + tid] = z;
    }
    uint4* const zp = reinterpret_cast<uint4*>(pbf);
#pragma unroll
    for (int i = 0; i < 2 * PBUF / 16 / 512; ++i) zp[i * 512 + tid] = z;
  }
  f32x16 sdp[2];    // S (P wave) or dP (partner) of the two steps
  bf16x8 pd[2][2];  // P (P wave) or dS (partner) of the two steps
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int t = 0; t < 16; ++t) sdp[h][t] = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) pd[h][i][e] = (__bf16)0.f;
  }
  int j2 = 0;  // first step of the current double step
  SoftIn sin[2];  // the P wave's softmax inputs of the two steps

  // Each role runs its own copy of the loop: with one loop and a branch on
  // the role inside every phase, the two roles' accumulators met at every
  // phase end and the compiler copied them between registers there. The
  // barrier sequence is the same in both loops: two per iteration, the
  // same iteration count.
#define DKDV_HEAD(NA, NB, VM)                                 \
  __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(VM));           \
  asm volatile("s_barrier" ::: "memory");                     \
  issue(ip, NA);                                              \
  next(ip);                                                   \
  issue(ip, NB);                                              \
  next(ip);
#define DKDV_MID                                              \
  __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(63));           \
  asm volatile("s_barrier" ::: "memory");
  // P wave: phase A products of pair J-1 and scores of pair J (MFMA),
  // phase B the softmax of pair J (VALU)
#define DKDV_STEP_P(CA, CB, PA, PB, NA, NB)                   \
  {                                                           \
    DKDV_HEAD(NA, NB, 0)                                      \
    __builtin_amdgcn_s_setprio(1);                            \
    product(pd[0], PA + OD);                                  \
    product(pd[1], PB + OD);                                  \
    scores(CA + OQ, sdp[0]);                                  \
    scores(CB + OQ, sdp[1]);                                  \
    schedule_matrix_phase2();                                 \
    __builtin_amdgcn_sched_barrier(0);                        \
    p_softmax_in(cp.rb, CA, sin[0]);                          \
    next(cp);                                                 \
    p_softmax_in(cp.rb, CB, sin[1]);                          \
    next(cp);                                                 \
    __builtin_amdgcn_s_setprio(0);                            \
    DKDV_MID                                                  \
    p_softmax(sin[0], CA, sdp[0], pd[0], pbf, true);          \
    p_softmax(sin[1], CB, sdp[1], pd[1], pbf + PBUF, j2 + 1 < n_blocks); \
    j2 += 2;                                                  \
  }
  // partner: phase A dS of pair J-1 (VALU), phase B its products and the
  // dP scores of pair J (MFMA)
#define DKDV_STEP_D(CA, CB, PA, PB, NA, NB)                   \
  {                                                           \
    DKDV_HEAD(NA, NB, 2 * PER_STAGE)                          \
    p_ds(PA, pbf, sdp[0], pd[0]);                             \
    p_ds(PB, pbf + PBUF, sdp[1], pd[1]);                      \
    DKDV_MID                                                  \
    __builtin_amdgcn_s_setprio(1);                            \
    product(pd[0], PA + OQ);                                  \
    product(pd[1], PB + OQ);                                  \
    scores(CA + OD, sdp[0]);                                  \
    scores(CB + OD, sdp[1]);                                  \
    schedule_matrix_phase2();                                 \
    __builtin_amdgcn_s_setprio(0);                            \
  }
  // (guarded steps rather than early exits: one loop exit keeps the
  // accumulators in place instead of copying them at every exit)
#define DKDV_LOOP(STEP)                                       \
  {                                                           \
    int jj = 0;                                               \
    for (; jj + 4 <= n_pairs; jj += 4) {                      \
      STEP(s0, s1, s6, s7, s4, s5);                           \
      STEP(s2, s3, s0, s1, s6, s7);                           \
      STEP(s4, s5, s2, s3, s0, s1);                           \
      STEP(s6, s7, s4, s5, s2, s3);                           \
    }                                                         \
    if (jj < n_pairs) STEP(s0, s1, s6, s7, s4, s5);           \
    if (jj + 1 < n_pairs) STEP(s2, s3, s0, s1, s6, s7);       \
    if (jj + 2 < n_pairs) STEP(s4, s5, s2, s3, s0, s1);       \
    __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(0));          \
    asm volatile("s_barrier" ::: "memory");                   \
  }
  // the last pair's remaining work: dV (P wave) and dS then dK (partner) of
  // pair n_pairs - 1 (slot pair (n_pairs - 1) % 4); the loads issued past
  // the end land before the kernel exits
  const int lp = (n_pairs - 1) & 3;
  const char* const la = lp == 0 ? s0 : lp == 1 ? s2 : lp == 2 ? s4 : s6;
  const char* const lb = lp == 0 ? s1 : lp == 1 ? s3 : lp == 2 ? s5 : s7;
  if (pwave) {
    DKDV_LOOP(DKDV_STEP_P)
    if (n_blocks > 0) {
      product(pd[0], la + OD);
      product(pd[1], lb + OD);
    }
  } else {
    DKDV_LOOP(DKDV_STEP_D)
    if (n_blocks > 0) {
      p_ds(la, pbf, sdp[0], pd[0]);
      p_ds(lb, pbf + PBUF, sdp[1], pd[1]);
      product(pd[0], la + OQ);
      product(pd[1], lb + OQ);
    }
  }
#undef DKDV_LOOP
#undef DKDV_STEP_D
#undef DKDV_STEP_P
#undef DKDV_MID
#undef DKDV_HEAD

  // accumulator register t of lane half hh: key 32 pair + (t/4)*8 + 4 hh + t%4,
  // d = 32 db + kl
  float* const outp = pwave ? a.dv : a.dk;
  const float sc = pwave ? 1.f : a.scale;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int k = kw0 + (t >> 2) * 8 + 4 * hh + (t & 3);
    if (k >= kt.k1) continue;
    float* const op = outp + (int64_t(k) * a.Hkv + g) * D + kl;
#pragma unroll
    for (int db = 0; db < ND; ++db) op[32 * db] = acc[db][t] * sc;
  }
}

template <int G>
hipError_t launch_bwd_g(const BwdArgs& a, int n_units, int n_ktiles, hipStream_t stream) {
  if (n_units > 0) {
    const int64_t blocks = int64_t(n_units) * a.n_hg;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dq_kernel<G>), dim3(uint32_t(blocks)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_ktiles > 0) {
    const int64_t blocks = int64_t(n_ktiles) * a.Hkv;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dkdv_kernel, dim3(uint32_t(blocks)), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, const int32_t* index,
                           const int32_t* row_lo, float* delta, int32_t* rec, int32_t R, int32_t H,
                           int32_t nrb, int32_t dtype, int32_t head_dim, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int64_t blocks = (int64_t(nrb) * kBwdRowBlock * H + 15) / 16;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const dim3 grid = dim3(uint32_t(blocks)), block = dim3(256);
#define PREP(T, DD)                                                                                          \
  hipLaunchKernelGGL((bwd_prep_kernel<T, DD>), grid, block, 0, stream, static_cast<const T*>(out),            \
                     static_cast<const T*>(dout), lse, index, row_lo, delta, rec, R, H, nrb)
  if (dtype == 1 && head_dim == 128)
    PREP(__bf16, 128);
  else if (dtype == 1 && head_dim == 64)
    PREP(__bf16, 64);
  else if (dtype == 0 && head_dim == 128)
    PREP(float, 128);
  else if (dtype == 0 && head_dim == 64)
    PREP(float, 64);
  else
    return hipErrorInvalidValue;
#undef PREP
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int heads_per_wg, int n_units, int n_ktiles,
                      hipStream_t stream) {
  if (heads_per_wg == 4) return launch_bwd_g<4>(a, n_units, n_ktiles, stream);
  if (heads_per_wg == 2) return launch_bwd_g<2>(a, n_units, n_ktiles, stream);
  return launch_bwd_g<1>(a, n_units, n_ktiles, stream);
}

}  // namespace cpattn
