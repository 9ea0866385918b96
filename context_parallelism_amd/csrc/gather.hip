// Chunk-index gather: the rank-local query rows, dst[i] = src[index[i]]
// (zero for pad rows, index -1). This is the index_select of the
// context-parallel multimodal page, section 1.1, done as one HBM-bound
// copy with 16-byte accesses: consecutive lanes move consecutive 16-byte
// pieces of a row, so every wavefront reads and writes whole contiguous
// runs of a row.
#include "kernels.h"

namespace cpattn {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;  // 16-byte pieces in flight per thread

__global__ __launch_bounds__(kGatherThreads) void gather_rows_kernel(
    const uint4* __restrict__ src, const int32_t* __restrict__ index, uint4* __restrict__ dst,
    uint32_t row_vec, uint32_t total_vec) {
  const uint32_t base = blockIdx.x * (kGatherThreads * kGatherUnroll) + threadIdx.x;
  uint4 val[kGatherUnroll];
  uint32_t pos[kGatherUnroll];
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u) {
    pos[u] = base + u * kGatherThreads;
    val[u] = make_uint4(0, 0, 0, 0);
    if (pos[u] < total_vec) {
      const uint32_t row = pos[u] / row_vec;
      const uint32_t col = pos[u] - row * row_vec;
      const int32_t g = index[row];
      if (g >= 0) val[u] = src[uint64_t(g) * row_vec + col];
    }
  }
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u)
    if (pos[u] < total_vec) dst[pos[u]] = val[u];
}

// Pad rows (index -1) of the outputs: zero output row, lse -inf (if lse is set). One thread
// per (row, 16-byte piece of a row); piece 0 also writes the row's lse.
__global__ __launch_bounds__(kGatherThreads) void fill_pad_rows_kernel(
    const int32_t* __restrict__ index, uint4* __restrict__ out, float* __restrict__ lse,
    uint32_t row_vec, uint32_t n_rows, uint32_t heads) {
  const uint32_t i = blockIdx.x * kGatherThreads + threadIdx.x;
  if (i >= row_vec * n_rows) return;
  const uint32_t row = i / row_vec, piece = i % row_vec;
  if (index[row] >= 0) return;
  out[i] = make_uint4(0, 0, 0, 0);
  if (lse != nullptr && piece < heads) lse[uint64_t(piece) * n_rows + row] = -INFINITY;
}

}  // namespace

hipError_t launch_fill_pad_rows(const int32_t* index, int64_t n_rows, int32_t heads,
                                int32_t head_dim, int32_t dtype, void* out, float* lse,
                                hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const int64_t row_bytes = int64_t(heads) * head_dim * (dtype == 1 ? 2 : 4);  // bf16 or fp32
  const uint64_t row_vec = uint64_t(row_bytes) / 16;
  const uint64_t total = row_vec * uint64_t(n_rows);
  // piece h < heads writes head h's lse: needs at least `heads` pieces per row
  if (row_bytes % 16 != 0 || row_vec < uint64_t(heads) || total >= (uint64_t(1) << 32))
    return hipErrorInvalidValue;
  const uint32_t blocks = uint32_t((total + kGatherThreads - 1) / kGatherThreads);
  hipLaunchKernelGGL(fill_pad_rows_kernel, dim3(blocks), dim3(kGatherThreads), 0, stream, index,
                     static_cast<uint4*>(out), lse, uint32_t(row_vec), uint32_t(n_rows),
                     uint32_t(heads));
  return hipGetLastError();
}

hipError_t launch_gather(const void* src, const int32_t* index, void* dst, int64_t n_rows,
                         int64_t row_bytes, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const uint64_t row_vec = uint64_t(row_bytes) / 16;
  const uint64_t total = row_vec * uint64_t(n_rows);
  if (row_bytes % 16 != 0 || total >= (uint64_t(1) << 32)) return hipErrorInvalidValue;
  const uint64_t per_block = kGatherThreads * kGatherUnroll;
  const uint32_t blocks = uint32_t((total + per_block - 1) / per_block);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(kGatherThreads), 0, stream,
                     static_cast<const uint4*>(src), index, static_cast<uint4*>(dst),
                     uint32_t(row_vec), uint32_t(total));
  return hipGetLastError();
}

}  // namespace cpattn
