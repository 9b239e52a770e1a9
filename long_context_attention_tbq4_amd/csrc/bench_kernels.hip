// Measured-achievable denominators for the rooflines of the attention
// kernels (declared in include/tbq4_bench.h): a read-only streaming kernel
// (what HBM delivers to a plain 16-byte-per-lane read on this part) and an
// MFMA-only loop (what the matrix cores sustain on independent fp16
// 32x32x16 products).  They compute nothing of the attention itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tbq4_bench.h"
#include "tbq4_device.h"

namespace tbq4 {

// Grid-stride 16-byte loads over [buf, buf + n16 * 16); every workgroup
// folds what it read into one word so that no load can be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *buf, uint64_t n16,
                                                          uint32_t *sink) {
  __shared__ uint32_t red[4];
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t x = 0;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {   // four loads in flight per lane
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^
         d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = buf[i];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Eight independent accumulators per wavefront, each taking `iters`
// v_mfma_f32_32x32x16_f16 products of register operands.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int32_t iters, float *sink) {
  const int lane = threadIdx.x & 63;
  half8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(0.001f * (float)((lane + e) & 7));
    b[e] = (_Float16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  float16v acc[8];
  for (int k = 0; k < 8; ++k)
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.0f;
  for (int k = 0; k < 8; ++k)
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace tbq4

extern "C" {

int32_t tbq4_bench_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t n_blocks,
                               void *hip_stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15)) return -1;
  if (n_blocks < 1 || n_blocks > 65536) return -1;
  hipLaunchKernelGGL(tbq4::stream_read_kernel, dim3(n_blocks), dim3(256), 0,
                     (hipStream_t)hip_stream, (const tbq4::u32x4 *)buf, (uint64_t)(bytes / 16),
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int32_t tbq4_bench_mfma_f16(int32_t iters, float *sink, int32_t n_blocks, void *hip_stream) {
  if (!sink || iters < 1 || n_blocks < 1 || n_blocks > 65536) return -1;
  hipLaunchKernelGGL(tbq4::mfma_loop_kernel, dim3(n_blocks), dim3(256), 0,
                     (hipStream_t)hip_stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
