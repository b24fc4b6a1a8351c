// Elementwise steps of the decoder block for gfx950: residual add, SwiGLU,
// and RoPE with key/value append.  None of them reduces anything; each output
// element is a fixed expression of its own inputs (and, for RoPE, of its
// absolute position), so they are batch-invariant by construction.  Each
// thread moves whole 16-byte chunks (8 bf16).
#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

// h may alias x or o (each thread reads its chunk of both before writing it): no __restrict__
__global__ __launch_bounds__(256) void add_kernel(const uint4* x, const uint4* o, uint4* h, int64_t chunks) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < chunks;
       i += int64_t(gridDim.x) * 256) {
    float a[8], b[8];
    unpack8(x[i], a);
    unpack8(o[i], b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = resid1(a[e], b[e]);
    h[i] = pack8(a);
  }
}

// act = bf16(silu(g) * u), silu(g) = g / (1 + exp(-g)), fp32 inside.
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ gu,
                                                     uint16_t* __restrict__ act, int64_t rows,
                                                     int64_t F) {
  const int64_t fch = F / 8;
  const int64_t total = rows * fch;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / fch;
    const int64_t c = i % fch;
    float g[8], u[8];
    unpack8(*reinterpret_cast<const uint4*>(gu + r * 2 * F + c * 8), g);
    unpack8(*reinterpret_cast<const uint4*>(gu + r * 2 * F + F + c * 8), u);
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = swiglu1(g[e], u[e]);
    *reinterpret_cast<uint4*>(act + r * F + c * 8) = pack8(g);
  }
}

// One work-group per token row.  The D/2 rotation angles of the row are
// computed once in fp64 from the absolute position (pos * theta^(-2i/D),
// then sin/cos in fp64, rounded to fp32) and shared through LDS by all heads.
// Thread work item = (head, 8 consecutive pair indices): rotates the chunks
// [i0, i0+8) and [i0 + D/2, i0 + D/2 + 8) of one q or k head, or copies one
// 16-byte chunk of a v head.
template <int D>
__global__ __launch_bounds__(256) void rope_kv_kernel(const uint16_t* __restrict__ qkv,
                                                      const int32_t* __restrict__ pos,
                                                      const int64_t* __restrict__ kv_row,
                                                      uint16_t* __restrict__ q_out,
                                                      uint16_t* __restrict__ k_pool,
                                                      uint16_t* __restrict__ v_pool, int Hq,
                                                      int Hkv, double theta) {
  constexpr int HALF = D / 2;
  constexpr int PCH = HALF / 8;  // work items per rotated head
  constexpr int VCH = D / 8;     // work items per value head
  __shared__ float s_cos[HALF];
  __shared__ float s_sin[HALF];
  const int64_t r = blockIdx.x;
  const int p = pos[r];
  const bool rotate = theta != 0.0;
  if (threadIdx.x < HALF) {
    float c = 1.f, s = 0.f;
    if (rotate) {
      const double inv_freq = pow(theta, -2.0 * double(threadIdx.x) / double(D));
      double sd, cd;
      sincos(double(p) * inv_freq, &sd, &cd);
      c = float(cd);
      s = float(sd);
    }
    s_cos[threadIdx.x] = c;
    s_sin[threadIdx.x] = s;
  }
  __syncthreads();
  const int64_t kvr = kv_row ? kv_row[r] : r;  // no row list: k and v go to rows r of the pools
  const uint16_t* src = qkv + r * int64_t(Hq + 2 * Hkv) * D;
  const int n_rot = (Hq + Hkv) * PCH;
  const int n_items = n_rot + Hkv * VCH;
  for (int it = threadIdx.x; it < n_items; it += 256) {
    if (it < n_rot && !rotate) {
      // no rotary embedding: q and k heads are copied bit for bit
      const int head = it / PCH;
      const int i0 = (it % PCH) * 8;
      uint16_t* dst = head < Hq ? q_out + r * int64_t(Hq) * D + head * D
                                : k_pool + (kvr * Hkv + (head - Hq)) * D;
      *reinterpret_cast<uint4*>(dst + i0) = *reinterpret_cast<const uint4*>(src + head * D + i0);
      *reinterpret_cast<uint4*>(dst + HALF + i0) =
          *reinterpret_cast<const uint4*>(src + head * D + HALF + i0);
    } else if (it < n_rot) {
      const int head = it / PCH;          // 0..Hq-1 query heads, then Hq..Hq+Hkv-1 key heads
      const int i0 = (it % PCH) * 8;
      float a[8], b[8];
      unpack8(*reinterpret_cast<const uint4*>(src + head * D + i0), a);
      unpack8(*reinterpret_cast<const uint4*>(src + head * D + HALF + i0), b);
      float ya[8], yb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = s_cos[i0 + e], s = s_sin[i0 + e];
        ya[e] = a[e] * c - b[e] * s;
        yb[e] = b[e] * c + a[e] * s;
      }
      uint16_t* dst = head < Hq ? q_out + r * int64_t(Hq) * D + head * D
                                : k_pool + (kvr * Hkv + (head - Hq)) * D;
      *reinterpret_cast<uint4*>(dst + i0) = pack8(ya);
      *reinterpret_cast<uint4*>(dst + HALF + i0) = pack8(yb);
    } else {
      const int j = it - n_rot;
      const int g = j / VCH;
      const int c = j % VCH;
      *reinterpret_cast<uint4*>(v_pool + (kvr * Hkv + g) * D + c * 8) =
          *reinterpret_cast<const uint4*>(src + (Hq + Hkv + g) * D + c * 8);
    }
  }
}

unsigned grid_for(int64_t items) {
  int64_t blocks = (items + 255) / 256;
  const int64_t cap = 256 * 64;  // grid-stride beyond ~16K work-groups
  return unsigned(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace

hipError_t launch_add(const uint16_t* x, const uint16_t* o, uint16_t* h, int64_t n, hipStream_t s) {
  const int64_t chunks = n / 8;
  hipLaunchKernelGGL(add_kernel, dim3(grid_for(chunks)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(x), reinterpret_cast<const uint4*>(o),
                     reinterpret_cast<uint4*>(h), chunks);
  return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t* gu, uint16_t* act, int64_t rows, int64_t F, hipStream_t s) {
  hipLaunchKernelGGL(swiglu_kernel, dim3(grid_for(rows * (F / 8))), dim3(256), 0, s, gu, act, rows, F);
  return hipGetLastError();
}

hipError_t launch_rope_kv(const uint16_t* qkv, const int32_t* pos, const int64_t* kv_row,
                          uint16_t* q_out, uint16_t* k_pool, uint16_t* v_pool, int64_t rows,
                          int Hq, int Hkv, int D, double theta, hipStream_t s) {
  if (D == 64)
    hipLaunchKernelGGL(rope_kv_kernel<64>, dim3(unsigned(rows)), dim3(256), 0, s, qkv, pos, kv_row,
                       q_out, k_pool, v_pool, Hq, Hkv, theta);
  else if (D == 128)
    hipLaunchKernelGGL(rope_kv_kernel<128>, dim3(unsigned(rows)), dim3(256), 0, s, qkv, pos, kv_row,
                       q_out, k_pool, v_pool, Hq, Hkv, theta);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bi
