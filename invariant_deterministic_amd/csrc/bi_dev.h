// Device-side helpers shared by the gfx950 kernels of the library.
//
// Every kernel in this library follows one rule: the floating-point
// operations that produce an output element, and their order, are a function
// of the problem's fixed dimensions (hidden size, N, K, head_dim, heads) and
// of the element's own absolute coordinates -- never of the number of rows,
// the batch, a row's position in the batch or a chunk boundary.  No kernel
// uses atomics.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kWave = 64;

// 16-byte load that streams past the caches (data read exactly once).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf2f_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf2f_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two values in one v_cvt_pk_bf16_f32 (the same rounding as f2bf on each).
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Unpack 8 bf16 (one 16-byte chunk) into fp32.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf2f_lo(v.x); f[1] = bf2f_hi(v.x);
  f[2] = bf2f_lo(v.y); f[3] = bf2f_hi(v.y);
  f[4] = bf2f_lo(v.z); f[5] = bf2f_hi(v.z);
  f[6] = bf2f_lo(v.w); f[7] = bf2f_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 r;
  r.x = pack2bf(f[0], f[1]);
  r.y = pack2bf(f[2], f[3]);
  r.z = pack2bf(f[4], f[5]);
  r.w = pack2bf(f[6], f[7]);
  return r;
}

// SwiGLU of one element from bf16 inputs (as floats): silu(g) * u, silu(g) = g / (1 + e^-g).
// One definition for the standalone kernel and the fused GEMM epilogue, so both round alike.
__device__ __forceinline__ float swiglu1(float g, float u) { return (g / (1.0f + __expf(-g))) * u; }
// Residual add of one element from bf16 inputs (as floats): x + o.
__device__ __forceinline__ float resid1(float x, float o) { return x + o; }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// Butterfly sum over `width` lanes (a power of two <= 64) that differ only in
// the low log2(width) bits of the lane id.  Every lane ends with the same
// bits: at each stage the two partners add the same two values.
template <int WIDTH>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int off = WIDTH / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int WIDTH>
__device__ __forceinline__ float xor_max(float v) {
#pragma unroll
  for (int off = WIDTH / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Lane-pair exchanges without LDS (v_permlane16_swap / v_permlane32_swap).
// pswap16(a, b): within each 32-lane half, the odd 16-lane row of a trades
// places with the even row of b; pswap32(a, b): the upper 32 lanes of a trade
// places with the lower 32 lanes of b.  With a == b, a op b afterwards combines
// lanes l and l ^ 16 (l ^ 32) -- for a commutative op every lane of the pair
// gets the same bits.
__device__ __forceinline__ void pswap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pswap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x16(float x) { float y = x; pswap16(x, y); return x + y; }
__device__ __forceinline__ float sum_x32(float x) { float y = x; pswap32(x, y); return x + y; }
__device__ __forceinline__ float max_x16(float x) { float y = x; pswap16(x, y); return fmaxf(x, y); }
__device__ __forceinline__ float max_x32(float x) { float y = x; pswap32(x, y); return fmaxf(x, y); }

// Raw buffer resource over `bytes` bytes at p.  Loads through it at byte
// offsets >= bytes return zero and touch no memory, so a tile's ragged edge
// needs no branch (a branch around a load can cost a full-latency wait).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, int(bytes), 0x00020000);
}
// NDW (4 or 2) dwords at byte offset off, streamed past the caches.
template <int NDW>
__device__ __forceinline__ void buf_ld_stream(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* out) {
  if constexpr (NDW == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 2);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, 2);
    out[0] = v.x; out[1] = v.y;
  }
}

// A value the caller knows is the same in every lane of the wave, moved to a
// scalar register (buffer resources must be scalar).
__device__ __forceinline__ const uint16_t* wave_uniform(const uint16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const uint16_t*>((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ uint32_t wave_uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace bi
