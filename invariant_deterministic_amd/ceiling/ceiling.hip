// Measurement probes for gfx950 (libbi_ceiling.so): a streaming read and a dense bf16
// matrix-core loop.  They carry none of the method's arithmetic; a benchmark runs them
// beside the batch-invariant kernels to show what a plain kernel sustains on the same
// device (read bandwidth; MFMA rate and shader clock with data-dependent operands).
#include <cstdint>

#include <hip/hip_runtime.h>

#include "bi_ceiling.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;

// work-group g reads span g of `grid` equal spans of n16 16-byte words, kUnroll loads in
// flight per thread, and writes the XOR of its span's 32-bit words.  The loads are
// non-temporal (global_load_dwordx4 ... nt): 7.1-7.2 TB/s on a 4 GiB buffer, against
// 6.2-6.4 TB/s for the same loop with ordinary loads.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ x, int64_t n16,
                                                               uint32_t* __restrict__ out) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = int64_t(blockIdx.x) * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += int64_t(kThreads) * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + int64_t(kThreads) * u;
      v[u] = j < hi ? make_uint4(__builtin_nontemporal_load(&x[j].x), __builtin_nontemporal_load(&x[j].y),
                                 __builtin_nontemporal_load(&x[j].z), __builtin_nontemporal_load(&x[j].w))
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__global__ __launch_bounds__(kThreads) void mfma_bf16_kernel(const bf16x8* __restrict__ src, int iters,
                                                             float* __restrict__ out, uint64_t* __restrict__ clk) {
  const int t = threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = src[(t * 8 + i) & 4095];
    b[i] = src[(t * 8 + 4 + i) & 4095];
  }
  f32x16 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const bool timer = blockIdx.x == 0 && t == 0;
  uint64_t c0 = 0, r0 = 0;
  if (timer) {
    c0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[j >> 2], acc[j], 0, 0, 0);
  }
  if (timer) {
    const uint64_t c1 = __builtin_readcyclecounter();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    clk[0] = c1 - c0;
    clk[1] = r1 - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[int64_t(blockIdx.x) * kThreads + t] = s;
}

}  // namespace

extern "C" int bic_stream_read(const void* x, int64_t bytes, uint32_t* out, int grid, hipStream_t stream) {
  if (!x || !out || (reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(out) & 3)) return 1;
  if (bytes <= 0 || bytes % 16 || grid < 1 || grid > 65536) return 2;
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(x), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int bic_mfma_bf16(const uint16_t* src, int grid, int iters, float* out, uint64_t* clk,
                             hipStream_t stream) {
  if (!src || !out || !clk || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(out) & 3) ||
      (reinterpret_cast<uintptr_t>(clk) & 7))
    return 1;
  if (grid < 1 || grid > 65536 || iters < 1) return 2;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const bf16x8*>(src), iters, out, clk);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
