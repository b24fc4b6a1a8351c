// Quantised KV cache for gfx950: int8 keys and values with one float32 scale
// per (token, kv head), in 64-token pages.
//
// The "Receipts" page ("What a receipt proves") names a quantised cache among
// the load settings that decide the bits.  Quantisation is per token and per
// head, so a token's cache entry depends only on that token: a request's bits
// stay independent of the batch and of where its pages live.  For each
// (row, head): a = max |x_d| (exact), scale = a / 127 (IEEE fp32 division),
// q_d = clamp(rint(x_d / scale), -127, 127), ties to even; a = 0 stores zeros
// and scale 0.  Attention kernels read bf16(float(q_d) * scale).
#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

// one wave per (row, head, K or V); lane holds D / 64 values
template <int D>
__global__ __launch_bounds__(64) void kv_quant_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                      const int64_t* __restrict__ dst_row, int Hkv,
                                                      int8_t* __restrict__ kq, int8_t* __restrict__ vq,
                                                      float* __restrict__ ks, float* __restrict__ vs) {
  constexpr int PL = D / 64;
  const int64_t r = blockIdx.x;
  const int g = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const int lane = threadIdx.x;
  const uint16_t* src = (is_v ? v : k) + (r * Hkv + g) * D + lane * PL;
  float x[PL];
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    x[i] = bf2f(src[i]);
    a = fmaxf(a, fabsf(x[i]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
  const float scale = a / 127.0f;
  const int64_t dr = dst_row[r];
  int8_t* dq = (is_v ? vq : kq) + (dr * Hkv + g) * D + lane * PL;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    float qf = scale > 0.f ? rintf(x[i] / scale) : 0.f;
    qf = fminf(fmaxf(qf, -127.f), 127.f);
    dq[i] = int8_t(int(qf));
  }
  if (lane == 0) (is_v ? vs : ks)[dr * Hkv + g] = scale;
}

}  // namespace

hipError_t launch_kv_quant(const uint16_t* k, const uint16_t* v, const int64_t* dst_row, int64_t rows, int Hkv,
                           int D, int8_t* kq, int8_t* vq, float* ks, float* vs, hipStream_t s) {
  const dim3 grid(unsigned(rows), unsigned(Hkv), 2);
  if (D == 64)
    hipLaunchKernelGGL(kv_quant_kernel<64>, grid, dim3(64), 0, s, k, v, dst_row, Hkv, kq, vq, ks, vs);
  else if (D == 128)
    hipLaunchKernelGGL(kv_quant_kernel<128>, grid, dim3(64), 0, s, k, v, dst_row, Hkv, kq, vq, ks, vs);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bi
