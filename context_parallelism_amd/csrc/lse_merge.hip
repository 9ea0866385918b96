// Log-sum-exp merge of per-step partial attention results (Ring
// Attention, Liu et al., ICLR 2024: blockwise partial outputs combine
// exactly by their log-sum-exp). One wavefront covers one rank-local row
// and 256/D heads; each lane owns four consecutive head_dim elements of
// one head, loaded as float4, so a wavefront reads contiguous 1 KiB runs
// of every step's partial. Up to 8 steps, every step's loads are issued
// before the reduction. The reduction over steps runs in increasing step
// order, the same for every lane, so results are deterministic.
#include "kernels.h"

namespace cpattn {

namespace {

constexpr int kMergeThreads = 256;

__device__ inline void store_out(float* out, int64_t i4, float4 v) {
  reinterpret_cast<float4*>(out)[i4] = v;
}

__device__ inline void store_out(__bf16* out, int64_t i4, float4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 b = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
  reinterpret_cast<bf16x4*>(out)[i4] = b;
}

// NS > 0: at most NS steps (unrolled: every step's lse and partial load is
// in flight before the reduction); NS = 0: any count up to 32, one step at
// a time.
template <int D, int NS, typename OutT>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const uint32_t* __restrict__ mask, uint32_t valid_bits, int32_t n_rows, int32_t H,
    int32_t head_groups,
    OutT* __restrict__ out, float* __restrict__ lse) {
  constexpr int kLanesPerHead = D / 4;
  constexpr int kHeadsPerWave = 64 / kLanesPerHead;
  const int64_t wave = (int64_t(blockIdx.x) * kMergeThreads + threadIdx.x) / 64;
  const int lane = threadIdx.x % 64;
  const int64_t row = wave / head_groups;
  if (row >= n_rows) return;
  const int h = int(wave % head_groups) * kHeadsPerWave + lane / kLanesPerHead;
  if (h >= H) return;
  const int d4 = lane % kLanesPerHead;
  const int64_t out4 = (row * H + h) * kLanesPerHead + d4;
  const uint32_t bits = mask[row] & valid_bits;
  auto empty_row = [&]() {
    store_out(out, out4, make_float4(0.f, 0.f, 0.f, 0.f));
    if (d4 == 0) lse[int64_t(h) * n_rows + row] = -INFINITY;
  };
  if (bits == 0) {
    empty_row();
    return;
  }
  const float4* const po = reinterpret_cast<const float4*>(part_o);
  const int64_t step_stride4 = int64_t(n_rows) * H * kLanesPerHead;
  const int64_t row4 = (row * H + h) * kLanesPerHead + d4;
  float m = -INFINITY, wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (NS > 0) {
    float ls[NS];
    float4 o[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bool on = (bits >> s) & 1u;
      ls[s] = on ? part_lse[(int64_t(s) * H + h) * n_rows + row] : -INFINITY;
      o[s] = on ? po[int64_t(s) * step_stride4 + row4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) m = fmaxf(m, ls[s]);
    // steps in increasing order, empty partials (lse -inf) skipped
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (ls[s] == -INFINITY) continue;
      const float w = expf(ls[s] - m);
      wsum += w;
      acc.x += w * o[s].x;
      acc.y += w * o[s].y;
      acc.z += w * o[s].z;
      acc.w += w * o[s].w;
    }
  } else {
    for (uint32_t b = bits; b; b &= b - 1) {
      const int s = __builtin_ctz(b);
      m = fmaxf(m, part_lse[(int64_t(s) * H + h) * n_rows + row]);
    }
    for (uint32_t b = bits; b; b &= b - 1) {
      const int s = __builtin_ctz(b);
      const float ls = part_lse[(int64_t(s) * H + h) * n_rows + row];
      if (ls == -INFINITY) continue;  // an empty partial: its output is not read
      const float w = expf(ls - m);
      const float4 o = po[int64_t(s) * step_stride4 + row4];
      wsum += w;
      acc.x += w * o.x;
      acc.y += w * o.y;
      acc.z += w * o.z;
      acc.w += w * o.w;
    }
  }
  if (!(wsum > 0.f)) {  // every partial empty
    empty_row();
    return;
  }
  const float inv = 1.f / wsum;
  store_out(out, out4, make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv));
  if (d4 == 0) lse[int64_t(h) * n_rows + row] = m + logf(wsum);
}

template <int D>
hipError_t launch_merge_d(const float* part_o, const float* part_lse, const uint32_t* mask,
                          int32_t n_steps, int64_t n_rows, int32_t heads, int32_t dtype, void* out,
                          float* lse, hipStream_t stream) {
  const uint32_t valid = n_steps >= 32 ? 0xffffffffu : ((1u << n_steps) - 1u);
  constexpr int kHeadsPerWave = 64 / (D / 4);
  const int head_groups = (heads + kHeadsPerWave - 1) / kHeadsPerWave;
  const int64_t waves = n_rows * head_groups;
  const int64_t blocks = (waves * 64 + kMergeThreads - 1) / kMergeThreads;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
#define MERGE(NSV)                                                                                       \
  {                                                                                                      \
    if (dtype == 1)                                                                                      \
      hipLaunchKernelGGL((lse_merge_kernel<D, NSV, __bf16>), dim3(uint32_t(blocks)), dim3(kMergeThreads), 0, \
                         stream, part_o, part_lse, mask, valid, int32_t(n_rows), heads, head_groups,     \
                         static_cast<__bf16*>(out), lse);                                                \
    else                                                                                                 \
      hipLaunchKernelGGL((lse_merge_kernel<D, NSV, float>), dim3(uint32_t(blocks)), dim3(kMergeThreads), 0,  \
                         stream, part_o, part_lse, mask, valid, int32_t(n_rows), heads, head_groups,     \
                         static_cast<float*>(out), lse);                                                 \
  }
  if (n_steps <= 2)
    MERGE(2)
  else if (n_steps <= 4)
    MERGE(4)
  else if (n_steps <= 8)
    MERGE(8)
  else
    MERGE(0)
#undef MERGE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const float* part_o, const float* part_lse, const uint32_t* mask,
                            int32_t n_steps, int64_t n_rows, int32_t heads, int32_t head_dim, int32_t dtype,
                            void* out, float* lse, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  if (head_dim == 128)
    return launch_merge_d<128>(part_o, part_lse, mask, n_steps, n_rows, heads, dtype, out, lse, stream);
  if (head_dim == 64)
    return launch_merge_d<64>(part_o, part_lse, mask, n_steps, n_rows, heads, dtype, out, lse, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn
