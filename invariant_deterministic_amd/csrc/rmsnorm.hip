// Batch-invariant RMSNorm for gfx950.
//
// RMSNorm is one of the three operations the M-0002 record ("Deterministic and
// bit-exact inference", field `technical`, Invariance route) makes
// batch-invariant.  Here one 64-lane wave owns one row; four rows share a
// 256-thread workgroup only to amortise the launch, never a reduction.
//
// Reduction order of a row (a function of `hidden` alone):
//   lane l owns the 16-byte chunks c = l, l + 64, l + 128, ... of the row;
//   it accumulates x^2 with fmaf over its chunks in ascending c, and within a
//   chunk over its 8 elements in ascending order; the 64 lane partials are
//   then combined by a fixed xor butterfly (32, 16, 8, 4, 2, 1).
// The row is read from HBM once and kept in registers for the scaling pass;
// loads and stores stream past the caches (each byte is touched once).
#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {

constexpr int kNormRowsPerBlock = 4;

template <int NCH>  // 16-byte chunks held per lane: hidden <= NCH * 512
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint4* __restrict__ x,
                                                      const uint4* __restrict__ gamma,
                                                      uint4* __restrict__ y, int64_t rows,
                                                      int hchunks, float hidden_f, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * kNormRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4* xr = x + row * hchunks;
  uint4 v[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < hchunks ? ld_stream16(xr + c) : make_uint4(0, 0, 0, 0);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    float f[8];
    unpack8(v[i], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float r = 1.0f / __builtin_sqrtf(ss / hidden_f + eps);
  uint4* yr = y + row * hchunks;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < hchunks) {
      float f[8], g[8];
      unpack8(v[i], f);
      unpack8(gamma[c], g);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (f[e] * r) * g[e];
      const uint4 r4 = pack8(f);
      const u32x4 rv = {r4.x, r4.y, r4.z, r4.w};
      __builtin_nontemporal_store(rv, reinterpret_cast<u32x4*>(yr + c));
    }
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, uint16_t* y, int64_t rows,
                          int64_t hidden, float eps, hipStream_t s) {
  const int hchunks = int(hidden / 8);
  const int nch = (hchunks + 63) / 64;
  const dim3 grid(unsigned((rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock));
  const dim3 block(256);
  auto xp = reinterpret_cast<const uint4*>(x);
  auto gp = reinterpret_cast<const uint4*>(gamma);
  auto yp = reinterpret_cast<uint4*>(y);
  const float hf = float(hidden);
#define BI_NORM_CASE(N)                                                                   \
  if (nch <= N) {                                                                         \
    hipLaunchKernelGGL(rmsnorm_kernel<N>, grid, block, 0, s, xp, gp, yp, rows, hchunks, hf, eps); \
    return hipGetLastError();                                                             \
  }
  BI_NORM_CASE(1)
  BI_NORM_CASE(2)
  BI_NORM_CASE(4)
  BI_NORM_CASE(8)
  BI_NORM_CASE(16)
  BI_NORM_CASE(32)
#undef BI_NORM_CASE
  return hipErrorInvalidValue;
}

}  // namespace bi
