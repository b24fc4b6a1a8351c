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

// one wave per (row, head, K or V); lane holds D / 64 values.  Destination: pool row
// dst_row[r]; or, PAGED, the row of position p = pos[r] of a sequence whose page-table
// entries start at e0 = dst_row[r] - p: pages[e0 + p / 64] * 64 + p % 64 (a page index
// outside 0 .. n_pages - 1 writes nothing).
template <int D, bool PAGED>
__global__ __launch_bounds__(64) void kv_quant_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                      const int64_t* __restrict__ dst_row,
                                                      const int32_t* __restrict__ pos,
                                                      const int32_t* __restrict__ pages, int64_t n_pages, int Hkv,
                                                      int8_t* __restrict__ kq, int8_t* __restrict__ vq,
                                                      float* __restrict__ ks, float* __restrict__ vs) {
  constexpr int PL = D / 64;
  const int64_t r = blockIdx.x;
  const int g = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const int lane = threadIdx.x;
  int64_t dr = dst_row[r];
  if constexpr (PAGED) {
    const int p = pos[r];
    const int64_t page = pages[dr - p + p / kPrefillKeyBlock];
    if (page < 0 || page >= n_pages) return;  // the whole wave: nothing written
    dr = page * kPrefillKeyBlock + p % kPrefillKeyBlock;
  }
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
    hipLaunchKernelGGL((kv_quant_kernel<64, false>), grid, dim3(64), 0, s, k, v, dst_row, nullptr, nullptr, 0, Hkv, kq,
                       vq, ks, vs);
  else if (D == 128)
    hipLaunchKernelGGL((kv_quant_kernel<128, false>), grid, dim3(64), 0, s, k, v, dst_row, nullptr, nullptr, 0, Hkv,
                       kq, vq, ks, vs);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_kv_quant_paged(const uint16_t* k, const uint16_t* v, const int64_t* entry_plus_pos,
                                 const int32_t* pos, const int32_t* pages, int64_t n_pages, int64_t rows, int Hkv,
                                 int D, int8_t* kq, int8_t* vq, float* ks, float* vs, hipStream_t s) {
  const dim3 grid(unsigned(rows), unsigned(Hkv), 2);
  if (D == 64)
    hipLaunchKernelGGL((kv_quant_kernel<64, true>), grid, dim3(64), 0, s, k, v, entry_plus_pos, pos, pages, n_pages,
                       Hkv, kq, vq, ks, vs);
  else if (D == 128)
    hipLaunchKernelGGL((kv_quant_kernel<128, true>), grid, dim3(64), 0, s, k, v, entry_plus_pos, pos, pages, n_pages,
                       Hkv, kq, vq, ks, vs);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bi
