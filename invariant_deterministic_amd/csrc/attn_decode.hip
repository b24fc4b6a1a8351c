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
// Split kernel: one 512-thread work-group per (kv head g, unit s, request b)
// (the block entry point passes a host-built list of the step's real units,
// the standalone one launches the max-units grid and idle groups exit);
// For the G query heads sharing kv head g (8 waves, each owning 32 of the
// unit's keys):
//   scores  S^T = K Q^T on v_mfma_f32_16x16x32_bf16, the keys streamed from
//           HBM straight into the MFMA operand layout (16 keys x 32 dims per
//           operand, D/32 steps in ascending order), times scale * log2(e);
//   m       exact maximum over the unit (order-free);
//   p       exp2(score - m), staged in LDS; l = sum of p (fixed in-lane order,
//           xor lanes 16 and 32, then waves 0..7);
//   o       sum of p * v on the VALU: lane (key group kl, dims 8 dc..) walks
//           its keys in ascending order with fmaf; the key groups of a wave
//           are added by a fixed xor tree, the 8 waves in ascending order
//           through LDS.
// Partials (m, l, o[D]) go to the workspace in fp32.  Keys past L_b are
// neither loaded nor counted (score -inf, p = 0, value 0).
//
// Combine kernel: one thread per (request, head, dim) walks s = 0 .. S_b - 1
// in ascending order: M = max m_s; w_s = exp2(m_s - M); O = sum w_s o_s,
// Lsum = sum w_s l_s; output bf16(O / Lsum).
#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

constexpr int kSplit = kKvSplit;      // 256 keys per unit
constexpr int kWavesPerUnit = 8;      // 32 keys per wave
constexpr int kKeysPerWave = kSplit / kWavesPerUnit;

constexpr int kSplitThreads = 64 * kWavesPerUnit;
constexpr int kKeyBlocks = kKeysPerWave / 16;  // 16-key MFMA blocks per wave

template <int D, int G>
__global__ __launch_bounds__(kSplitThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_all,
    const uint16_t* __restrict__ v_all, const DecodeSeq* __restrict__ seqs,
    const int2* __restrict__ units, int Hkv, int64_t max_len, int max_splits, float qscale,
    float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  constexpr int KS = D / 32;     // MFMA k-steps over the head dimension
  constexpr int CH = D / 8;      // lanes per key row in the value pass
  constexpr int KPL = 64 / CH;   // keys per wave-wide value load
  constexpr int NIT = kKeysPerWave / KPL;
  static_assert(G <= 16, "one 16-wide MFMA column block holds the group's heads");
  __shared__ float s_m[kWavesPerUnit][G];
  __shared__ float s_l[kWavesPerUnit][G];
  __shared__ __attribute__((aligned(16))) float s_p[kWavesPerUnit][kKeysPerWave][G];
  __shared__ float s_o[kWavesPerUnit][G][D];

  const int g = blockIdx.x;   // kv heads of one key block are dispatched together
  // (request, unit) from a host-built list of real units, or the full grid
  const int b = units ? units[blockIdx.y].x : int(blockIdx.z);
  const int s = units ? units[blockIdx.y].y : int(blockIdx.y);
  const DecodeSeq sq = seqs[b];
  const int64_t L = sq.kv_len;
  if (L < 1 || L > max_len) return;  // the combine kernel reports the request as NaN
  const int64_t nsplit = (L + kSplit - 1) / kSplit;
  if (s >= nsplit) return;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int Hq = Hkv * G;
  const int64_t row_stride = int64_t(Hkv) * D;
  const int64_t key_base = int64_t(s) * kSplit + w * kKeysPerWave;

  // ---- S^T = K Q^T with v_mfma_f32_16x16x32_bf16, straight from HBM.
  // A operand (keys): lane holds K[key_base + 16 kb + l16][32 ks + 8 grp .. + 8]
  // B operand (heads): lane holds Q[head l16][32 ks + 8 grp .. + 8] (0 past G)
  const uint16_t* kb_ptr = k_all + (sq.kv_offset + key_base + l16) * row_stride + g * D + grp * 8;
  uint4 kr[kKeyBlocks][KS];
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb) {
    const bool valid = key_base + 16 * kb + l16 < L;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kr[kb][ks] = valid ? ld_stream16(kb_ptr + int64_t(16 * kb) * row_stride + 32 * ks)
                         : make_uint4(0, 0, 0, 0);
  }
  bf16x8 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (l16 < G) v = *reinterpret_cast<const uint4*>(q + sq.q_row * q_stride + (g * G + l16) * D + 32 * ks + grp * 8);
    qb[ks] = as_bf16x8(v);
  }
  f32x4 sacc[kKeyBlocks];
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb) {
    sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[kb][ks]), qb[ks], sacc[kb], 0, 0, 0);
  }

  // value loads go out now; their latency overlaps the softmax
  const int dc = lane % CH;
  const int kl = lane / CH;
  const uint16_t* vb_ptr = v_all + (sq.kv_offset + key_base + kl) * row_stride + g * D + dc * 8;
  uint4 vr[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it)
    vr[it] = key_base + it * KPL + kl < L ? ld_stream16(vb_ptr + int64_t(it * KPL) * row_stride)
                                          : make_uint4(0, 0, 0, 0);

  // ---- scores: lane holds head l16, keys key_base + 16 kb + 4 grp + r
  float sc[kKeyBlocks][4];
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = key_base + 16 * kb + 4 * grp + r < L;
      const float v = valid ? sacc[kb][r] * qscale : -INFINITY;
      sc[kb][r] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (grp == 0 && l16 < G) s_m[w][l16] = mx;
  __syncthreads();
  const int hh = l16 < G ? l16 : 0;
  float m = s_m[0][hh];
#pragma unroll
  for (int ww = 1; ww < kWavesPerUnit; ++ww) m = fmaxf(m, s_m[ww][hh]);
  float ls = 0.f;
#pragma unroll
  for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(sc[kb][r] - m);
      ls += p;
      if (l16 < G) s_p[w][16 * kb + 4 * grp + r][l16] = p;
    }
  ls += __shfl_xor(ls, 16, 64);
  ls += __shfl_xor(ls, 32, 64);
  if (grp == 0 && l16 < G) s_l[w][l16] = ls;
  __syncthreads();

  // ---- weighted values: lane takes dims 8 dc .. + 8 of keys kl, kl + KPL, ...
  float oacc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[h][e] = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float vf[8];
    unpack8(vr[it], vf);
    const float* pp = s_p[w][it * KPL + kl];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = pp[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) oacc[h][e] = __builtin_fmaf(p, vf[e], oacc[h][e]);
    }
  }
  // key groups of the wave (lanes with equal dc) by a fixed xor tree, then
  // one partial per wave through LDS
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = oacc[h][e];
#pragma unroll
      for (int off = CH; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
      oacc[h][e] = v;
    }
  if (kl == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[w][h][dc * 8 + e] = oacc[h][e];
  }
  __syncthreads();

  // ---- fixed-order sum over the waves; write the unit's partials
  for (int i = threadIdx.x; i < G * D; i += kSplitThreads) {
    const int h = i / D;
    const int d = i % D;
    float o = s_o[0][h][d];
#pragma unroll
    for (int ww = 1; ww < kWavesPerUnit; ++ww) o += s_o[ww][h][d];
    const int64_t slot = (int64_t(b) * Hq + g * G + h) * max_splits + s;
    ws_o[slot * D + d] = o;
    if (d == 0) {
      float mm = s_m[0][h], ll = s_l[0][h];
#pragma unroll
      for (int ww = 1; ww < kWavesPerUnit; ++ww) {
        mm = fmaxf(mm, s_m[ww][h]);
        ll += s_l[ww][h];
      }
      ws_ml[slot * 2 + 0] = mm;
      ws_ml[slot * 2 + 1] = ll;
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
                        const uint16_t* v_all, const DecodeSeq* seqs, const int2* units,
                        int n_units, int B, int64_t max_len, int max_splits, int Hkv, float qscale,
                        float* ws_o, float* ws_ml, hipStream_t s) {
  const dim3 grid = units ? dim3(Hkv, n_units, 1) : dim3(Hkv, max_splits, B);
  hipLaunchKernelGGL((decode_split_kernel<D, G>), grid, dim3(kSplitThreads), 0, s, q, q_stride, k_all,
                     v_all, seqs, units, Hkv, max_len, max_splits, qscale, ws_o, ws_ml);
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
                              const uint16_t* v_all, const DecodeSeq* d_seqs, const int2* d_units,
                              int n_units, int B, int64_t max_kv_len, int Hq, int Hkv, int D,
                              float scale, void* ws, uint16_t* o, int64_t o_row_stride,
                              hipStream_t s) {
  const int max_splits = int((max_kv_len + kSplit - 1) / kSplit);
  const size_t slots = size_t(B) * Hq * max_splits;
  float* ws_o = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(slots * D * 4));
  const float qscale = scale * 1.4426950408889634f;  // scores in log2 units
  const int G = Hq / Hkv;
  hipError_t e = hipErrorInvalidValue;
#define BI_DEC(DD, GG)                                                                          \
  if (D == DD && G == GG)                                                                     \
    e = launch_split<DD, GG>(q, q_row_stride, k_all, v_all, d_seqs, d_units, n_units, B, \
                             max_kv_len, max_splits, Hkv, qscale, ws_o, ws_ml, s);
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
  return launch_attn_decode(q, int64_t(Hq) * D, k_all, v_all, seqs, nullptr, 0, B, max_kv_len,
                            Hq, Hkv, D, scale, ws, o, int64_t(Hq) * D, s);
}

}  // namespace bi
