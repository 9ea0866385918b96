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
//  * delta: Delta[h][r] = sum_d dO[r][h][d] * O[r][h][d];
//  * dQ: one workgroup of 4 waves per (row tile, head group); each wave owns
//    32 rows of one head and walks the tile's key spans over all ring steps,
//    recomputing S^T = K Q^T and dP^T = V dO^T (K and V rows from LDS, Q and
//    dO in registers) and accumulating dQ^T += K^T dS^T (K^T from a blocked
//    copy, as the forward reads V^T);
//  * dK/dV: one workgroup of 4 waves per (128-key tile, KV head); each wave
//    owns 32 keys, keeps its K and V rows in registers, and walks the
//    rank's 32-row blocks that see the tile, for every query head of the KV
//    head: S = Q K^T and dP = dO V^T (Q, dO rows from LDS), then
//    dV += P^T dO and dK += dS^T Q with Q^T and dO^T read from blocked
//    copies. The accumulator layout of S (keys in lanes, rows in
//    registers) is directly the A operand of those products once the rows
//    are read in the order sigma (bits 2 and 3 of the row swapped).
#include "kernels.h"

namespace cpattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBufferWord3 = 0x00020000;  // raw buffer access, gfx9 family
constexpr int kWaitVmcnt0 = 0x0F70;       // s_waitcnt vmcnt(0), expcnt and lgkmcnt untouched
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

// ---------------------------------------------------------------- delta
// 16 lanes per (row, head) pair, 8 elements each; 16 pairs per 256 threads.
__global__ __launch_bounds__(256) void delta_kernel(const __bf16* __restrict__ out,
                                                   const __bf16* __restrict__ dout,
                                                   float* __restrict__ delta, int32_t R, int32_t H) {
  const int64_t pair = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool ok = pair < int64_t(R) * H;
  const int64_t pc = ok ? pair : 0;  // inactive groups read pair 0 and store nothing
  const int r = int(pc / H), h = int(pc % H);
  const int64_t off = pc * 128 + sub * 8;  // [R, H, 128]: pair (r, h) starts at (r H + h) 128
  const bf16x8 o = *reinterpret_cast<const bf16x8*>(out + off);
  const bf16x8 d = *reinterpret_cast<const bf16x8*>(dout + off);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = __builtin_fmaf(float(o[i]), float(d[i]), s);
  s = sum_with_partner16(s);
  if (ok && sub == 0) delta[int64_t(h) * R + r] = s;
}

// Scalar walk over a unit's 64-key tiles (as in the forward).
struct Cursor {
  int kt, k0, k1, span;
};

// ---------------------------------------------------------------- dQ
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dq_kernel(const BwdArgs a) {
  constexpr int D = 128, BN = 64, NQ = 8, ND = 4, RB = 4 / G;
  constexpr int TILE = BN * D * 2;     // bytes of a K, V or K^T tile
  constexpr int CH = TILE / 1024 / 4;  // LDS-DMA instructions per wave per tensor
  __shared__ __attribute__((aligned(1024))) char k0s[TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[TILE];
  __shared__ __attribute__((aligned(1024))) char t0s[TILE];
  __shared__ __attribute__((aligned(1024))) char t1s[TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = blockIdx.x % a.n_hg;
  const UnitRec unit = a.units[blockIdx.x / a.n_hg];
  const TileRec tile = a.tiles[unit.tile];
  const EntryRec* const steps = a.tile_entries + unit.e0;
  const int n_steps = unit.e1 - unit.e0;
  const int h = hg * G + (wave % G);
  const int rsub = wave / G;
  const int kvh = (hg * G) / a.group;
  const int ql = lane & 31, hh = lane >> 5;
  const int rin = rsub * 32 + ql;
  const bool row_ok = rin < tile.nrows;
  const int lrow = tile.local0 + rin;
  const int grow = tile.g0 + rin;
  const int wave_lo = tile.g0 + rsub * 32;
  static_assert(RB * G == 4, "4 waves");
  const SpanRec* spans = a.spans + steps[0].span_begin;
  const int n_spans = steps[n_steps - 1].span_end - steps[0].span_begin;
  int n_tiles = 0;
  for (int i = 0; i < n_spans; ++i) n_tiles += (spans[i].k1 - (spans[i].k0 & ~7) + BN - 1) / BN;
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

  // LDS-DMA offsets (as in the forward: K rows swizzled g ^ (r & 15), K^T
  // rows g ^ ((d >> 1) & 7)); every wave loads a quarter of each tile.
  const int tok_bytes = a.Hkv * D * 2;
  const char* kbase = static_cast<const char*>(a.k) + int64_t(kvh) * D * 2;
  const char* vbase = static_cast<const char*>(a.v) + int64_t(kvh) * D * 2;
  const char* tbase = static_cast<const char*>(a.kt) + int64_t(kvh) * a.tpad * D * 2;
  int kgo[CH], tgo[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = wave * CH + i;
    const int krow = 4 * c + (lane >> 4), kp = lane & 15;
    kgo[i] = krow * tok_bytes + 16 * (kp ^ (krow & 15));
    const int d = 8 * c + (lane >> 3), vp = lane & 7;
    tgo[i] = (vp ^ ((d >> 1) & 7)) * (D * 16) + d * 16;
  }
  auto issue = [&](const Cursor& c, char* kd, char* vd, char* td) {
    const int kt = __builtin_amdgcn_readfirstlane(c.kt);
    const int valid = __builtin_amdgcn_readfirstlane(max(min(c.k1 - kt, BN), 0) * tok_bytes);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + int64_t(kt) * tok_bytes, valid);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + int64_t(kt) * tok_bytes, valid);
    const int tvalid = __builtin_amdgcn_readfirstlane(max(a.tpad - kt, 0) * D * 2);
    const __amdgpu_buffer_rsrc_t tr = make_rsrc(tbase + int64_t(kt) * D * 2, tvalid);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kd + (wave * CH + i) * 1024), 16, kgo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vd + (wave * CH + i) * 1024), 16, kgo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(tr, (lds_void*)(td + (wave * CH + i) * 1024), 16, tgo[i], 0, 0, 0);
    }
  };

  const int srow = (ql & ~12) | ((ql & 4) << 1) | ((ql & 8) >> 1);
  int kro[NQ];
#pragma unroll
  for (int jj = 0; jj < NQ; ++jj) kro[jj] = srow * 256 + 16 * ((2 * jj + hh) ^ (srow & 15));
  const int vx = (ql >> 1) & 7;
  int tro[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) tro[kb][sub] = ql * 128 + 16 * ((4 * kb + 2 * sub + hh) ^ vx);

  f32x16 acc[ND];  // dQ^T: d = 32 db + 8 (t/4) + 4 hh + t%4 ... (rows in lanes)
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[db][t] = 0.f;

  auto tile_step = [&](const Cursor& c, const char* ks, const char* vs, const char* ts) {
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        s[kb][t] = 0.f;
        dp[kb][t] = 0.f;
      }
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + kb * 32 * 256 + kro[jj]);
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs + kb * 32 * 256 + kro[jj]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[jj], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[jj], dp[kb], 0, 0, 0);
      }
    }
    // register r of lane half hh holds key kt + 32 kb + 16 (r / 8) + 8 hh + r % 8
    const bool edge = c.kt < c.k0 || c.kt + BN > c.k1 || c.kt + BN - 1 > wave_lo;
    const int base = c.kt + 8 * hh;
    const int lo = min(max(c.k0 - base, 0), 64);
    const int hi = min(max(min(c.k1, grow + 1) - base, 0), 64);
    const uint64_t below_hi = hi >= 64 ? ~0ull : (1ull << hi) - 1;
    const uint64_t below_lo = lo >= 64 ? ~0ull : (1ull << lo) - 1;
    const uint64_t vis = edge ? (below_hi & ~below_lo) : ~0ull;
    const int w0 = int(uint32_t(vis)), w1 = int(uint32_t(vis >> 32));
    bf16x8 dsb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = __builtin_amdgcn_sbfe(kb ? w1 : w0, 16 * (r >> 3) + (r & 7), 1);
        float arg;
        asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(arg) : "v"(m), "v"(__builtin_fmaf(s[kb][r], c2, -lse2)),
            "v"(-INFINITY));
        const float p = __builtin_amdgcn_exp2f(arg);
        dsb[kb][r >> 3][r & 7] = (__bf16)(p * (dp[kb][r] - dl));
      }
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const bf16x8 tf = *reinterpret_cast<const bf16x8*>(ts + db * 32 * 128 + tro[kb][sub]);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf, dsb[kb][sub], acc[db], 0, 0, 0);
        }
  };

  Cursor cs, cl;
  start(cs);
  start(cl);
  issue(cl, k0s, v0s, t0s);
  for (int t = 0; t < n_tiles; t += 2) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    advance(cl);
    if (t + 1 < n_tiles) issue(cl, k1s, v1s, t1s);
    tile_step(cs, k0s, v0s, t0s);
    advance(cs);
    if (t + 1 >= n_tiles) break;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    advance(cl);
    if (t + 2 < n_tiles) issue(cl, k0s, v0s, t0s);
    tile_step(cs, k1s, v1s, t1s);
    advance(cs);
  }

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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dkdv_kernel(const BwdArgs a) {
  constexpr int D = 128, NQ = 8, ND = 4, RBK = kBwdRowBlock;
  constexpr int ROWT = RBK * D * 2;    // bytes of a 32-row Q, dO, Q^T or dO^T tile
  constexpr int CH = ROWT / 1024 / 4;  // LDS-DMA instructions per wave per tensor (2)
  static_assert(kBwdKeyTile == 128 && RBK == 32, "4 waves of 32 keys, 32-row blocks");
  __shared__ __attribute__((aligned(1024))) char q0s[ROWT], q1s[ROWT];
  __shared__ __attribute__((aligned(1024))) char d0s[ROWT], d1s[ROWT];
  __shared__ __attribute__((aligned(1024))) char qt0s[ROWT], qt1s[ROWT];
  __shared__ __attribute__((aligned(1024))) char dt0s[ROWT], dt1s[ROWT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x % a.Hkv;
  const KeyTileRec kt = a.ktiles[blockIdx.x / a.Hkv];
  const int kl = lane & 31, hh = lane >> 5;
  const int key = kt.k0 + 32 * wave + kl;  // this lane's key (column of S)

  // K and V rows of the wave's 32 keys as B operands: lane holds key kl,
  // d = 16 jj + 8 hh + 0..7. Keys >= k1 read as zeros.
  bf16x8 kf[NQ], vf[NQ];
  {
    const int tok_bytes = a.Hkv * D * 2;
    const int k0w = kt.k0 + 32 * wave;
    const int valid = max(min(kt.k1 - k0w, 32), 0) * tok_bytes;
    const __amdgpu_buffer_rsrc_t kr =
        make_rsrc(static_cast<const char*>(a.k) + (int64_t(k0w) * a.Hkv + g) * D * 2, valid);
    const __amdgpu_buffer_rsrc_t vr =
        make_rsrc(static_cast<const char*>(a.v) + (int64_t(k0w) * a.Hkv + g) * D * 2, valid);
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) {
      const int off = kl * tok_bytes + (16 * jj + 8 * hh) * 2;
      kf[jj] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
      vf[jj] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
    }
  }

  // LDS-DMA offsets. Q and dO row tiles (32 rows x 256 B, granule
  // g ^ (row & 15)): instruction i of this wave fills rows 4c..4c+3,
  // c = 2 wave + i. Q^T and dO^T tiles (128 d-rows x 64 B of 32 rows,
  // granule g ^ ((d >> 2) & 3)): instruction i fills d-rows 16c..16c+15; the
  // blocked source holds 8 rows x 128 d per 2 KiB.
  const int row_bytes = a.H * D * 2;
  int ngo[CH], tgo[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = wave * CH + i;
    const int r = 4 * c + (lane >> 4), p = lane & 15;
    ngo[i] = r * row_bytes + 16 * (p ^ (r & 15));
    const int d = 16 * c + (lane >> 2), s = lane & 3;
    tgo[i] = (s ^ ((d >> 2) & 3)) * (D * 16) + d * 16;
  }
  auto issue = [&](int rb, int h, char* qd, char* dd, char* qtd, char* dtd) {
    const int r0 = rb * RBK;
    const int valid = __builtin_amdgcn_readfirstlane(max(min(a.R - r0, RBK), 0) * row_bytes);
    const int64_t noff = (int64_t(r0) * a.H + h) * D * 2;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(static_cast<const char*>(a.qr) + noff, valid);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(static_cast<const char*>(a.dout) + noff, valid);
    const int64_t toff = (int64_t(h) * a.rpad + r0) * D * 2;
    const __amdgpu_buffer_rsrc_t qtr = make_rsrc(static_cast<const char*>(a.qt) + toff, ROWT);
    const __amdgpu_buffer_rsrc_t dtr = make_rsrc(static_cast<const char*>(a.dot) + toff, ROWT);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int slot = (wave * CH + i) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void*)(qd + slot), 16, ngo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void*)(dd + slot), 16, ngo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qtr, (lds_void*)(qtd + slot), 16, tgo[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(dtr, (lds_void*)(dtd + slot), 16, tgo[i], 0, 0, 0);
    }
  };
  // A operands of S and dP: lane reads row sigma(kl) of the Q / dO tile
  const int srow = (kl & ~12) | ((kl & 4) << 1) | ((kl & 8) >> 1);
  int nro[NQ];
#pragma unroll
  for (int jj = 0; jj < NQ; ++jj) nro[jj] = srow * 256 + 16 * ((2 * jj + hh) ^ (srow & 15));
  // B operands of dV and dK: lane reads d-row 32 db + kl, rows 16 kk + 8 hh + 0..7
  int tro[ND][2];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int d = 32 * db + kl;
      tro[db][kk] = d * 64 + 16 * ((2 * kk + hh) ^ ((d >> 2) & 3));
    }

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      dk[db][t] = 0.f;
      dv[db][t] = 0.f;
    }
  const float c2 = a.scale_log2;

  // one (row block, query head) step. Register t of lane half hh holds row
  // 32 rb + rr(t): rr = 8 hh + t (t < 8), 16 + 8 hh + t - 8 (t >= 8).
  auto block_step = [&](int rb, int h, const char* qs, const char* ds, const char* qts, const char* dts) {
    f32x16 s, dp;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      s[t] = 0.f;
      dp[t] = 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) {
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qs + nro[jj]);
      const bf16x8 da = *reinterpret_cast<const bf16x8*>(ds + nro[jj]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[jj], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[jj], dp, 0, 0, 0);
    }
    // per-row lse, delta and global id: two runs of 8 rows per lane half
    const int r0 = rb * RBK;
    const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.lse + int64_t(h) * a.R, a.R * 4);
    const __amdgpu_buffer_rsrc_t er = make_rsrc(a.delta + int64_t(h) * a.R, a.R * 4);
    const __amdgpu_buffer_rsrc_t ir = make_rsrc(a.index, a.R * 4);
    float lse_r[16], dl_r[16];
    int gid_r[16];
#pragma unroll
    for (int run = 0; run < 2; ++run)
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        const int row = r0 + 16 * run + 8 * hh + 4 * q4;
        const f32x4 l4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(lr, row * 4, 0, 0));
        const f32x4 d4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(er, row * 4, 0, 0));
        const i32x4 g4 = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ir, row * 4, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 8 * run + 4 * q4 + e;
          const bool in = row + e < a.R;
          lse_r[t] = l4[e];
          dl_r[t] = d4[e];
          gid_r[t] = in ? g4[e] : -1;
        }
      }
    bf16x8 pa[2], dsa[2];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int gid = gid_r[t];
      const bool vis = gid >= 0 && key <= gid && gid < kt.s1 && key < kt.k1;
      const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[t], c2, -lse_r[t] * kLog2e)) : 0.f;
      pa[t >> 3][t & 7] = (__bf16)p;
      dsa[t >> 3][t & 7] = (__bf16)(p * (dp[t] - dl_r[t]));
    }
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 dob = *reinterpret_cast<const bf16x8*>(dts + tro[db][kk]);
        const bf16x8 qb = *reinterpret_cast<const bf16x8*>(qts + tro[db][kk]);
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk], dob, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsa[kk], qb, dk[db], 0, 0, 0);
      }
  };

  // the (row block, head) steps: rb in [rb0, rb1) outer, the query heads
  // of KV head g (a.group of them) inner
  const int group = a.group;
  const int n_blocks = (kt.rb1 - kt.rb0) * group;
  auto step_at = [&](int i, int& rb, int& h) {
    rb = kt.rb0 + i / group;
    h = g * group + i % group;
  };
  if (n_blocks > 0) {
    int rb, h;
    step_at(0, rb, h);
    issue(rb, h, q0s, d0s, qt0s, dt0s);
  }
  for (int i = 0; i < n_blocks; i += 2) {
    int rb, h, rbn, hn;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (i + 1 < n_blocks) {
      step_at(i + 1, rbn, hn);
      issue(rbn, hn, q1s, d1s, qt1s, dt1s);
    }
    step_at(i, rb, h);
    block_step(rb, h, q0s, d0s, qt0s, dt0s);
    if (i + 1 >= n_blocks) break;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (i + 2 < n_blocks) {
      step_at(i + 2, rbn, hn);
      issue(rbn, hn, q0s, d0s, qt0s, dt0s);
    }
    step_at(i + 1, rb, h);
    block_step(rb, h, q1s, d1s, qt1s, dt1s);
  }

  // accumulator register t of lane half hh: key 32 wave + (t/4)*8 + 4 hh + t%4,
  // d = 32 db + kl
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int k = kt.k0 + 32 * wave + (t >> 2) * 8 + 4 * hh + (t & 3);
    if (k >= kt.k1) continue;
    float* const dkp = a.dk + (int64_t(k) * a.Hkv + g) * D + kl;
    float* const dvp = a.dv + (int64_t(k) * a.Hkv + g) * D + kl;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      dkp[32 * db] = dk[db][t] * a.scale;
      dvp[32 * db] = dv[db][t];
    }
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
    hipLaunchKernelGGL(dkdv_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_delta(const void* out, const void* dout, float* delta, int32_t R, int32_t H,
                            hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int64_t blocks = (int64_t(R) * H + 15) / 16;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(delta_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream,
                     static_cast<const __bf16*>(out), static_cast<const __bf16*>(dout), delta, R, H);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int heads_per_wg, int n_units, int n_ktiles,
                      hipStream_t stream) {
  if (heads_per_wg == 4) return launch_bwd_g<4>(a, n_units, n_ktiles, stream);
  if (heads_per_wg == 2) return launch_bwd_g<2>(a, n_units, n_ktiles, stream);
  return launch_bwd_g<1>(a, n_units, n_ktiles, stream);
}

}  // namespace cpattn
