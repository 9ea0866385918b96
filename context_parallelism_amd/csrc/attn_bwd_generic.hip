// Gradients of one CP rank's attention share for fp32 inputs and for
// head_dim 64 (bf16 or fp32): the same chain rule as the bf16 head_dim-128
// kernels -- P = exp(S - lse), Delta = rowsum(dO * O), dS = P (dP - Delta),
// dQ = dS K / sqrt(D), dK = dS^T Q / sqrt(D), dV = P^T dO -- over the same
// plan (row tiles with their ring-step key spans; key tiles with the 32-row
// blocks that see them), computed with plain fp32 FMAs: values are
// converted to fp32 as they are staged, P and dS stay fp32, accumulation is
// fp32. No atomics.
//
// L = D / 32 lanes share one row (dQ) or one key (dK/dV), each lane owning
// 32 consecutive elements of head_dim; dot products are summed over the L
// lanes with xor shuffles. The staged LDS rows are skewed by one float per
// 32 so that the L lanes of a group read different banks.
#include "kernels.h"

namespace cpattn {

namespace {

constexpr float kLog2eG = 1.4426950408889634f;
constexpr int kKeyChunk = 32;  // keys staged per LDS round in dQ
constexpr int kRowsG = kBwdRowBlock;

template <int L>
__device__ inline float group_sum(float x) {
  if (L >= 2) x += __shfl_xor(x, 1, 64);
  if (L >= 4) x += __shfl_xor(x, 2, 64);
  return x;
}

// LDS column of element d in a skewed row (33 floats per 32 elements)
__device__ inline int skew(int d) { return 33 * (d >> 5) + (d & 31); }

// ---------------------------------------------------------------- dQ
// One workgroup of 256 threads per (row tile, head): 256 / L rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void dq_generic_kernel(const BwdArgs a) {
  constexpr int L = D / 32;
  constexpr int W = 33 * L;  // skewed row width in floats
  __shared__ float ks[kKeyChunk * W], vs[kKeyChunk * W];
  const int h = blockIdx.x % a.H;
  const UnitRec unit = a.units[blockIdx.x / a.H];
  const TileRec tile = a.tiles[unit.tile];
  const EntryRec* const steps = a.tile_entries + unit.e0;
  const int n_steps = unit.e1 - unit.e0;
  const int kvh = h / a.group;
  const int t = threadIdx.x, ri = t / L, part = t % L;
  const bool row_ok = ri < tile.nrows;
  const int lrow = tile.local0 + ri, grow = tile.g0 + ri;

  float q[32], dout[32], dq[32];
  {
    const int64_t off = (int64_t(row_ok ? lrow : 0) * a.H + h) * D + 32 * part;
    const T* const qp = static_cast<const T*>(a.qr) + off;
    const T* const dp = static_cast<const T*>(a.dout) + off;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      q[i] = row_ok ? float(qp[i]) : 0.f;
      dout[i] = row_ok ? float(dp[i]) : 0.f;
      dq[i] = 0.f;
    }
  }
  const float lse2 = row_ok ? a.lse[int64_t(h) * a.R + lrow] * kLog2eG : INFINITY;
  const float dl = row_ok ? a.delta[int64_t(h) * a.R + lrow] : 0.f;
  const float c2 = a.scale_log2;
  const SpanRec* const spans = a.spans + steps[0].span_begin;
  const int n_spans = steps[n_steps - 1].span_end - steps[0].span_begin;
  const T* const kg = static_cast<const T*>(a.k);
  const T* const vg = static_cast<const T*>(a.v);

  for (int si = 0; si < n_spans; ++si) {
    const int k0 = spans[si].k0, k1 = spans[si].k1;
    for (int kc = k0; kc < k1; kc += kKeyChunk) {
      const int nk = min(kKeyChunk, k1 - kc);
      __syncthreads();
      for (int e = t; e < kKeyChunk * D; e += 256) {
        const int kr = e / D, d = e % D;
        const int64_t src = (int64_t(kc + kr) * a.Hkv + kvh) * D + d;
        ks[kr * W + skew(d)] = kr < nk ? float(kg[src]) : 0.f;
        vs[kr * W + skew(d)] = kr < nk ? float(vg[src]) : 0.f;
      }
      __syncthreads();
      for (int kr = 0; kr < nk; ++kr) {
        const float* const kr_row = ks + kr * W + 33 * part;
        const float* const vr_row = vs + kr * W + 33 * part;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          s = __builtin_fmaf(q[i], kr_row[i], s);
          dp = __builtin_fmaf(dout[i], vr_row[i], dp);
        }
        s = group_sum<L>(s);
        dp = group_sum<L>(dp);
        const bool vis = row_ok && kc + kr <= grow;
        const float p = vis ? exp2f(__builtin_fmaf(s, c2, -lse2)) : 0.f;
        const float ds = p * (dp - dl);
#pragma unroll
        for (int i = 0; i < 32; ++i) dq[i] = __builtin_fmaf(ds, kr_row[i], dq[i]);
      }
    }
  }
  if (!row_ok) return;
  float* const o = a.dq + (int64_t(lrow) * a.H + h) * D + 32 * part;
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = dq[i] * a.scale;
}

// ---------------------------------------------------------------- dK / dV
// One workgroup of kBwdKeyTile * L threads per (key tile, KV head): L lanes
// per key; the rank's 32-row blocks that see the tile are staged in LDS one
// (block, query head) at a time.
template <typename T, int D>
__global__ __launch_bounds__(512) void dkdv_generic_kernel(const BwdArgs a) {
  constexpr int L = D / 32;
  constexpr int W = 33 * L;
  constexpr int NT = kBwdKeyTile * L;
  __shared__ float qs[kRowsG * W], ds_[kRowsG * W];
  __shared__ float rl2[kRowsG], rdl[kRowsG];
  __shared__ int rlo[kRowsG], rsp[kRowsG];
  const int g = blockIdx.x % a.Hkv;
  const KeyTileRec kt = a.ktiles[blockIdx.x / a.Hkv];
  const int t = threadIdx.x, ki = t / L, part = t % L;
  const int key = kt.k0 + ki;
  const bool key_ok = key < kt.k1;

  float k[32], v[32], dk[32], dv[32];
  {
    const int64_t off = (int64_t(key_ok ? key : 0) * a.Hkv + g) * D + 32 * part;
    const T* const kp = static_cast<const T*>(a.k) + off;
    const T* const vp = static_cast<const T*>(a.v) + off;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      k[i] = key_ok ? float(kp[i]) : 0.f;
      v[i] = key_ok ? float(vp[i]) : 0.f;
      dk[i] = 0.f;
      dv[i] = 0.f;
    }
  }
  const float c2 = a.scale_log2;
  const T* const qg = static_cast<const T*>(a.qr);
  const T* const dg = static_cast<const T*>(a.dout);
  for (int rb = kt.rb0; rb < kt.rb1; ++rb) {
    for (int hq = 0; hq < a.group; ++hq) {
      const int h = g * a.group + hq;
      const int r0 = rb * kRowsG;
      __syncthreads();
      for (int e = t; e < kRowsG * D; e += NT) {
        const int r = e / D, d = e % D;
        const bool ok = r0 + r < a.R;
        const int64_t src = (int64_t(ok ? r0 + r : 0) * a.H + h) * D + d;
        qs[r * W + skew(d)] = ok ? float(qg[src]) : 0.f;
        ds_[r * W + skew(d)] = ok ? float(dg[src]) : 0.f;
      }
      if (t < kRowsG) {
        const int32_t* const rec = a.rec + (int64_t(h) * a.nrb + rb) * (4 * kRowsG);
        rl2[t] = __int_as_float(rec[t]);
        rdl[t] = __int_as_float(rec[kRowsG + t]);
        rlo[t] = rec[2 * kRowsG + t];
        rsp[t] = rec[3 * kRowsG + t];
      }
      __syncthreads();
      for (int r = 0; r < kRowsG; ++r) {
        const float* const q_row = qs + r * W + 33 * part;
        const float* const d_row = ds_ + r * W + 33 * part;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          s = __builtin_fmaf(q_row[i], k[i], s);
          dp = __builtin_fmaf(d_row[i], v[i], dp);
        }
        s = group_sum<L>(s);
        dp = group_sum<L>(dp);
        // visible: sample start <= key <= the row's global id (pad rows'
        // records hold lse +inf, so their P is 0)
        const bool vis = key_ok && uint32_t(key - rlo[r]) <= uint32_t(rsp[r]);
        const float p = vis ? exp2f(__builtin_fmaf(s, c2, -rl2[r])) : 0.f;
        const float dsv = p * (dp - rdl[r]);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          dv[i] = __builtin_fmaf(p, d_row[i], dv[i]);
          dk[i] = __builtin_fmaf(dsv, q_row[i], dk[i]);
        }
      }
    }
  }
  if (!key_ok) return;
  float* const dkp = a.dk + (int64_t(key) * a.Hkv + g) * D + 32 * part;
  float* const dvp = a.dv + (int64_t(key) * a.Hkv + g) * D + 32 * part;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    dkp[i] = dk[i] * a.scale;
    dvp[i] = dv[i];
  }
}

template <typename T, int D>
hipError_t launch_generic(const BwdArgs& a, int n_units, int n_ktiles, hipStream_t stream) {
  if (n_units > 0) {
    const int64_t blocks = int64_t(n_units) * a.H;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dq_generic_kernel<T, D>), dim3(uint32_t(blocks)), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_ktiles > 0) {
    const int64_t blocks = int64_t(n_ktiles) * a.Hkv;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dkdv_generic_kernel<T, D>), dim3(uint32_t(blocks)), dim3(kBwdKeyTile * (D / 32)), 0,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_generic(const BwdArgs& a, int32_t dtype, int32_t head_dim, int n_units, int n_ktiles,
                              hipStream_t stream) {
  if (dtype == 0 && head_dim == 128) return launch_generic<float, 128>(a, n_units, n_ktiles, stream);
  if (dtype == 0 && head_dim == 64) return launch_generic<float, 64>(a, n_units, n_ktiles, stream);
  if (dtype == 1 && head_dim == 64) return launch_generic<__bf16, 64>(a, n_units, n_ktiles, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn
