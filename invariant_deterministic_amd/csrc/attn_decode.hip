// Decode attention with a fixed key/value split size for gfx950.
//
// The M-0002 record ("Deterministic and bit-exact inference", field
// `technical`) makes attention batch-invariant by splitting the key/value
// axis into pieces of a fixed *size* rather than into a fixed *number* of
// pieces.  Here the piece is 256 keys: request b with L_b keys has
// ceil(L_b / 256) units, unit s covering keys [256 s, min(256 s + 256, L_b)).
// How a unit is reduced depends only on its keys, and the units of a request
// are merged in ascending s by a second kernel, so a request's bits never
// depend on the batch, the other requests' lengths or the grid.
//
// Split kernel: one 256-thread work-group per (unit s, kv head g, request b).
// Each wave streams 64 of the unit's keys; lane l takes the 16-byte chunk
// l % (D/8) of key l / (D/8) of each wave-wide load, so one load instruction
// covers D/8 * 16 bytes of each of 64/(D/8) keys.  For the G query heads that
// share kv head g:
//   score = (q_scaled . k) by an fmaf chain over the lane's 8 dims, then an xor
//           butterfly over the D/8 lanes of the key (fixed tree);
//   m     = exact maximum over the unit (order-free);
//   p     = exp2(score - m); l = sum of p; o = sum of p * v, each summed per
//           lane in ascending key order, then by xor butterflies across the
//           key groups of the wave, then across the 4 waves in ascending
//           order through LDS.
// Partials (m, l, o[D]) go to the workspace in fp32.  Scores are in log2
// units (q is pre-multiplied by scale * log2(e)), so exp2 is the native
// instruction.  Keys past L_b are neither loaded nor counted (p = 0).
//
// Combine kernel: one thread per (request, head, dim) walks s = 0 .. S_b - 1
// in ascending order: M = max m_s; w_s = exp2(m_s - M); O = sum w_s o_s,
// Lsum = sum w_s l_s; output bf16(O / Lsum).
#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

constexpr int kSplit = kKvSplit;      // 256 keys per unit
constexpr int kWavesPerUnit = 4;      // 64 keys per wave
constexpr int kKeysPerWave = kSplit / kWavesPerUnit;

template <int D, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_all,
    const uint16_t* __restrict__ v_all, const DecodeSeq* __restrict__ seqs, int Hkv,
    int64_t max_len, int max_splits, float qscale, float* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  constexpr int CH = D / 8;      // lanes per key row
  constexpr int KPL = 64 / CH;   // keys per wave-wide load
  constexpr int NIT = kKeysPerWave / KPL;
  __shared__ float s_m[kWavesPerUnit][G];
  __shared__ float s_l[kWavesPerUnit][G];
  __shared__ float s_o[kWavesPerUnit][G][D];

  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const DecodeSeq sq = seqs[b];
  const int64_t L = sq.kv_len;
  if (L < 1 || L > max_len) return;  // the combine kernel reports the request as NaN
  const int64_t nsplit = (L + kSplit - 1) / kSplit;
  if (s >= nsplit) return;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int dc = lane % CH;
  const int kl = lane / CH;
  const int Hq = Hkv * G;

  // queries of the G heads of group g, dims dc*8 .. dc*8+7, times scale*log2(e)
  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 raw = *reinterpret_cast<const uint4*>(q + sq.q_row * q_stride + (g * G + h) * D + dc * 8);
    unpack8(raw, qf[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[h][e] *= qscale;
  }

  const int64_t row_stride = int64_t(Hkv) * D;
  const uint16_t* kb = k_all + sq.kv_offset * row_stride + g * D + dc * 8;
  const uint16_t* vb = v_all + sq.kv_offset * row_stride + g * D + dc * 8;
  const int64_t key0 = int64_t(s) * kSplit + w * kKeysPerWave + kl;

  // ---- scores
  uint4 kr[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int64_t key = key0 + it * KPL;
    kr[it] = key < L ? ld_stream16(kb + key * row_stride)
                     : make_uint4(0, 0, 0, 0);
  }
  float sc[NIT][G];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float kf[8];
    unpack8(kr[it], kf);
    const bool valid = key0 + it * KPL < L;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = __builtin_fmaf(qf[h][e], kf[e], d);
#pragma unroll
      for (int off = CH / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off, 64);
      sc[it][h] = valid ? d : -INFINITY;
    }
  }

  // ---- exact maximum of the unit
  float m[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = sc[0][h];
#pragma unroll
    for (int it = 1; it < NIT; ++it) mx = fmaxf(mx, sc[it][h]);
#pragma unroll
    for (int off = CH; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if (lane == 0) s_m[w][h] = mx;
  }

  // issue the value loads before waiting on the other waves
  uint4 vr[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int64_t key = key0 + it * KPL;
    vr[it] = key < L ? ld_stream16(vb + key * row_stride)
                     : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h)
    m[h] = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));

  // ---- weights and their sum (ascending key order within the lane)
  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lsum[h] = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = __builtin_amdgcn_exp2f(sc[it][h] - m[h]);
      sc[it][h] = p;
      lsum[h] += p;
    }

  // ---- weighted values
  float oacc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[h][e] = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float vf[8];
    unpack8(vr[it], vf);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) oacc[h][e] = __builtin_fmaf(sc[it][h], vf[e], oacc[h][e]);
  }

  // ---- across the key groups of the wave (lanes with equal dc), fixed tree
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = CH; off < 64; off <<= 1) lsum[h] += __shfl_xor(lsum[h], off, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int off = CH; off < 64; off <<= 1) oacc[h][e] += __shfl_xor(oacc[h][e], off, 64);
  }
  if (kl == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[w][h][dc * 8 + e] = oacc[h][e];
      if (dc == 0) s_l[w][h] = lsum[h];
    }
  }
  __syncthreads();

  // ---- across the 4 waves in ascending order; write the unit's partials
  for (int i = threadIdx.x; i < G * D; i += 256) {
    const int h = i / D;
    const int d = i % D;
    const float o = ((s_o[0][h][d] + s_o[1][h][d]) + s_o[2][h][d]) + s_o[3][h][d];
    const int64_t slot = (int64_t(b) * Hq + g * G + h) * max_splits + s;
    ws_o[slot * D + d] = o;
    if (d == 0) {
      ws_ml[slot * 2 + 0] = m[h];
      ws_ml[slot * 2 + 1] = ((s_l[0][h] + s_l[1][h]) + s_l[2][h]) + s_l[3][h];
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    const DecodeSeq* __restrict__ seqs, int Hq, int max_splits, int64_t max_len,
    uint16_t* __restrict__ o, int64_t o_stride) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const DecodeSeq sq = seqs[b];
  const int64_t L = sq.kv_len;
  uint16_t* dst = o + sq.q_row * o_stride + h * D + d;
  if (L < 1 || L > max_len) {
    *dst = 0x7FC0;  // NaN: the request's length is outside what the grid covered
    return;
  }
  const int S = int((L + kSplit - 1) / kSplit);
  const int64_t base = (int64_t(b) * Hq + h) * max_splits;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ws_ml[(base + s) * 2]);
  float Lsum = 0.f, O = 0.f;
  for (int s = 0; s < S; ++s) {
    const float w = __builtin_amdgcn_exp2f(ws_ml[(base + s) * 2] - M);
    Lsum = __builtin_fmaf(w, ws_ml[(base + s) * 2 + 1], Lsum);
    O = __builtin_fmaf(w, ws_o[(base + s) * D + d], O);
  }
  *dst = f2bf(O / Lsum);
}

// Packs the standalone entry point's offset / length arrays into DecodeSeq.
__global__ void decode_pack_kernel(const int64_t* __restrict__ kv_offset,
                                   const int32_t* __restrict__ kv_len, int B,
                                   DecodeSeq* __restrict__ out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    DecodeSeq sq;
    sq.q_row = b;
    sq.kv_offset = kv_offset[b];
    sq.kv_len = kv_len[b];
    sq.pad = 0;
    out[b] = sq;
  }
}

template <int D, int G>
hipError_t launch_split(const uint16_t* q, int64_t q_stride, const uint16_t* k_all,
                        const uint16_t* v_all, const DecodeSeq* seqs, int B, int64_t max_len,
                        int max_splits, int Hkv, float qscale, float* ws_o, float* ws_ml,
                        hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<D, G>), dim3(max_splits, Hkv, B), dim3(256), 0, s, q,
                     q_stride, k_all, v_all, seqs, Hkv, max_len, max_splits, qscale, ws_o, ws_ml);
  return hipGetLastError();
}

}  // namespace

// Workspace: ws_o [B][Hq][S][D] fp32, ws_ml [B][Hq][S][2] fp32, then the
// packed DecodeSeq array of the standalone entry point; 256-byte aligned parts.
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t decode_workspace_bytes(int B, int64_t max_kv_len, int Hq, int D) {
  const int64_t S = (max_kv_len + kSplit - 1) / kSplit;
  const size_t slots = size_t(B) * Hq * S;
  return align256(slots * D * 4) + align256(slots * 2 * 4) + align256(size_t(B) * sizeof(DecodeSeq));
}

hipError_t launch_attn_decode(const uint16_t* q, int64_t q_row_stride, const uint16_t* k_all,
                              const uint16_t* v_all, const DecodeSeq* d_seqs, int B,
                              int64_t max_kv_len, int Hq, int Hkv, int D, float scale, void* ws,
                              uint16_t* o, int64_t o_row_stride, hipStream_t s) {
  const int max_splits = int((max_kv_len + kSplit - 1) / kSplit);
  const size_t slots = size_t(B) * Hq * max_splits;
  float* ws_o = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(slots * D * 4));
  const float qscale = scale * 1.4426950408889634f;  // scores in log2 units
  const int G = Hq / Hkv;
  hipError_t e = hipErrorInvalidValue;
#define BI_DEC(DD, GG)                                                                          \
  if (D == DD && G == GG)                                                                     \
    e = launch_split<DD, GG>(q, q_row_stride, k_all, v_all, d_seqs, B, max_kv_len, max_splits, \
                             Hkv, qscale, ws_o, ws_ml, s);
  BI_DEC(64, 1) BI_DEC(64, 2) BI_DEC(64, 4) BI_DEC(64, 8)
  BI_DEC(128, 1) BI_DEC(128, 2) BI_DEC(128, 4) BI_DEC(128, 8)
#undef BI_DEC
  if (e != hipSuccess) return e;
  if (D == 64)
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(Hq, B), dim3(64), 0, s, ws_o, ws_ml, d_seqs,
                       Hq, max_splits, max_kv_len, o, o_row_stride);
  else
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(Hq, B), dim3(128), 0, s, ws_o, ws_ml,
                       d_seqs, Hq, max_splits, max_kv_len, o, o_row_stride);
  return hipGetLastError();
}

hipError_t launch_attn_decode_arrays(const uint16_t* q, const uint16_t* k_all,
                                     const uint16_t* v_all, const int64_t* kv_offset,
                                     const int32_t* kv_len, int B, int64_t max_kv_len, int Hq,
                                     int Hkv, int D, float scale, void* ws, uint16_t* o,
                                     hipStream_t s) {
  const int max_splits = int((max_kv_len + kSplit - 1) / kSplit);
  const size_t slots = size_t(B) * Hq * max_splits;
  DecodeSeq* seqs = reinterpret_cast<DecodeSeq*>(static_cast<char*>(ws) + align256(slots * D * 4) +
                                                 align256(slots * 2 * 4));
  hipLaunchKernelGGL(decode_pack_kernel, dim3((B + 255) / 256), dim3(256), 0, s, kv_offset, kv_len,
                     B, seqs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_decode(q, int64_t(Hq) * D, k_all, v_all, seqs, B, max_kv_len, Hq, Hkv, D,
                            scale, ws, o, int64_t(Hq) * D, s);
}

}  // namespace bi
