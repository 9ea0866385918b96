// V -> V^T relayout for the bf16 head_dim-128 attention kernel.
//
// The attention kernel contracts P against V over keys. A matrix-core
// operand needs its reduction index (here: keys) contiguous in each lane, so
// the kernel reads V^T. Layout, per KV head g: blocks of 8 keys, each block
// holding all 128 d-rows of its 8 keys: vt[g][key / 8][d][key % 8], padded
// to tpad keys with zeros past seq_len. Any 64-key window starting at a
// multiple of 8 keys is then one contiguous 16 KiB run, which the attention
// kernel copies into LDS with long sequential reads. One workgroup moves a
// 64-key x 128-d block of one KV head: it reads 64 rows of 256 contiguous
// bytes, turns the block around in LDS and writes 16 KiB contiguously.
// HBM-bound; runs once per call, before the attention kernel.
#include "kernels.h"

namespace cpattn {

namespace {

constexpr int kKeys = 64;     // keys per block
constexpr int kD = 128;       // head_dim
constexpr int kStride = kD + 2;  // LDS row stride (bf16): odd word stride spreads the column reads

__global__ __launch_bounds__(256) void transpose_v_kernel(const unsigned short* __restrict__ v,
                                                          unsigned short* __restrict__ vt, int T,
                                                          int Hkv, int tpad) {
  __shared__ __attribute__((aligned(16))) unsigned short tile[kKeys * kStride];
  const int g = blockIdx.y;
  const int t0 = blockIdx.x * kKeys;
  const int tid = threadIdx.x;
  // 64 keys x 16 pieces of 8 d-values
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
    const int key = p >> 4, dc = p & 15;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (t0 + key < T)
      val = *reinterpret_cast<const uint4*>(v + (int64_t(t0 + key) * Hkv + g) * kD + dc * 8);
    unsigned* dst = reinterpret_cast<unsigned*>(tile + key * kStride + dc * 8);  // 4-byte aligned
    dst[0] = val.x;
    dst[1] = val.y;
    dst[2] = val.z;
    dst[3] = val.w;
  }
  __syncthreads();
  // 8 key groups x 128 d-rows of 8 keys; consecutive lanes take
  // consecutive d, so each wavefront writes 1 KiB contiguously
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    const int d = q & (kD - 1), kc = q >> 7;
    unsigned w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned lo = tile[(8 * kc + 2 * e) * kStride + d];
      const unsigned hi = tile[(8 * kc + 2 * e + 1) * kStride + d];
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(vt + ((int64_t(g) * (tpad / 8) + t0 / 8 + kc) * kD + d) * 8) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_transpose_v(const void* v, void* vt, int32_t T, int32_t Hkv, int32_t tpad,
                              hipStream_t stream) {
  if (tpad % kKeys != 0 || tpad < T) return hipErrorInvalidValue;
  const dim3 grid(uint32_t(tpad / kKeys), uint32_t(Hkv));
  hipLaunchKernelGGL(transpose_v_kernel, grid, dim3(256), 0, stream,
                     static_cast<const unsigned short*>(v), static_cast<unsigned short*>(vt), T, Hkv,
                     tpad);
  return hipGetLastError();
}

}  // namespace cpattn
