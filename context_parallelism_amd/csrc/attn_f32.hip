// Per-step blockwise causal attention, fp32 path (exact fp32 products, no
// MFMA): used for fp32 inputs, where results must match the fp64 oracle to
// about 1e-5. Same work list as the bf16 kernel: one workgroup per
// (row tile, ring step, head); two lanes per query row, each owning half of
// head_dim; keys stream through LDS 32 at a time and each tile updates an
// online softmax (running max, rescaled sum and output). The step's output
// is normalised by its own sum and written with its log-sum-exp, to be
// combined across steps by the LSE merge (Ring Attention, Liu et al.,
// ICLR 2024).
#include "kernels.h"

namespace cpattn {

namespace {

constexpr int kKeysPerTile = 32;
constexpr int kThreads = 2 * kF32RowsPerTile;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_step_f32_kernel(AttnArgs a) {
  constexpr int HALF = D / 2;
  __shared__ float ks[kKeysPerTile][D];
  __shared__ float vs[kKeysPerTile][D];

  const int h = blockIdx.x % a.H;
  const EntryRec ent = a.entries[blockIdx.x / a.H];
  const TileRec tile = a.tiles[ent.tile];
  const int t = threadIdx.x;
  const int rin = t >> 1, half = t & 1;
  const bool row_ok = rin < tile.nrows;
  const int lrow = tile.local0 + rin;
  const int grow = tile.g0 + rin;
  const int kvh = h / a.group;
  const float* qp = static_cast<const float*>(a.q) + (int64_t(grow) * a.H + h) * D + half * HALF;
  const float* kg = static_cast<const float*>(a.k);
  const float* vg = static_cast<const float*>(a.v);
  const int64_t tok_stride = int64_t(a.Hkv) * D;

  float q[HALF], acc[HALF];
#pragma unroll
  for (int d = 0; d < HALF; ++d) {
    q[d] = row_ok ? qp[d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int sp = ent.span_begin; sp < ent.span_end; ++sp) {
    const SpanRec span = a.spans[sp];
    for (int kt = span.k0; kt < span.k1; kt += kKeysPerTile) {
      __syncthreads();  // previous tile fully consumed
      for (int i = t; i < kKeysPerTile * D; i += kThreads) {
        const int key = i / D, d = i % D;
        const int g = kt + key;
        const bool in = g < span.k1;
        const int64_t off = int64_t(g) * tok_stride + int64_t(kvh) * D + d;
        ks[key][d] = in ? kg[off] : 0.f;
        vs[key][d] = in ? vg[off] : 0.f;
      }
      __syncthreads();
      if (!row_ok) continue;
      float s[kKeysPerTile];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < kKeysPerTile; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < HALF; ++d) dot = fmaf(q[d], ks[j][half * HALF + d], dot);
        dot += __shfl_xor(dot, 1);
        const int g = kt + j;
        s[j] = (g < span.k1 && g <= grow) ? dot * a.scale : -INFINITY;
        tmax = fmaxf(tmax, s[j]);
      }
      const float m_new = fmaxf(m, tmax);
      if (m_new == -INFINITY) continue;  // nothing visible yet
      const float alpha = expf(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < HALF; ++d) acc[d] *= alpha;
#pragma unroll
      for (int j = 0; j < kKeysPerTile; ++j) {
        const float p = (s[j] == -INFINITY) ? 0.f : expf(s[j] - m_new);
        l += p;
#pragma unroll
        for (int d = 0; d < HALF; ++d) acc[d] = fmaf(p, vs[j][half * HALF + d], acc[d]);
      }
      m = m_new;
    }
  }
  if (!row_ok) return;
  float* po = a.part_o + ((int64_t(ent.step) * a.R + lrow) * a.H + h) * D + half * HALF;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int d = 0; d < HALF; ++d) po[d] = acc[d] * inv;
  if (half == 0)
    a.part_lse[(int64_t(ent.step) * a.H + h) * a.R + lrow] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, int n_entries, hipStream_t stream) {
  if (n_entries == 0) return hipSuccess;
  const int64_t blocks = int64_t(n_entries) * a.H;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_step_f32_kernel<128>, dim3(uint32_t(blocks)), dim3(kThreads), 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(attn_step_f32_kernel<64>, dim3(uint32_t(blocks)), dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn
