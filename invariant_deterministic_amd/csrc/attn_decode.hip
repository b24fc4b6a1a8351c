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
// the standalone one launches the max-units grid and idle groups exit), for
// the G query heads sharing kv head g; 8 waves, each owning 32 of the keys.
//   loads   token-major: a lane takes 16 bytes (D/16 dims) of one key row, so
//           each load instruction covers four whole head rows; raw buffer
//           loads bounded at the request's last key read zero past it, with no
//           branch.  The query rows go once through LDS.
//   scores  S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (D/32 k-steps in ascending
//           order), K passed through a per-wave LDS block of 16 keys to reach
//           the operand layout, times scale * log2(e).  The block's row order
//           is chosen so that each lane ends up holding the scores of the very
//           keys whose values it loaded.
//   m       exact maximum over the unit (order-free);
//   p       exp2(score - m); l = sum of p (fixed in-lane order, lane pairs
//           16 and 32 apart, then waves 0..7);
//   o       P V on v_mfma_f32_16x16x32_bf16: the value operand is the lane's own
//           token-major registers regrouped by byte permutes (eight keys of one
//           dim), P enters as a bf16 high part plus a bf16 remainder; the 8
//           waves' partials are added in ascending order through LDS.
// Partials (m, l, o[D]) go to the workspace in fp32.  Keys past L_b contribute
// score -inf, p = 0 and value 0.
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

template <int D, int G>
__global__ __launch_bounds__(kSplitThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_all,
    const uint16_t* __restrict__ v_all, const DecodeSeq* __restrict__ seqs,
    const int2* __restrict__ units, int Hkv, int64_t max_len, int max_splits, float qscale,
    float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  constexpr int LD = D / 16;              // dims per lane in the token-major loads
  constexpr int NDW = LD / 2;             // their dwords
  constexpr int KS = D / 32;              // MFMA k-steps over the head dimension
  constexpr int NG = D / 8;               // 16-byte granules per key row
  constexpr int NIT = kKeysPerWave / 4;   // lane keys: 4 it + grp
  constexpr int NKB = kKeysPerWave / 16;  // 16-key score blocks
  constexpr int NKS = kKeysPerWave / 32;  // 32-key value steps
  static_assert(kKeysPerWave % 32 == 0 && G <= 8, "whole value steps; a wave's partial fits its key buffer");
  // per wave: one 16-key block of K (row-major, 16-byte granules xor-swizzled
  // by the row), later the wave's partial o[G][D] in fp32
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kWavesPerUnit][16 * D];
  __shared__ float s_m[kWavesPerUnit][G];
  __shared__ float s_l[kWavesPerUnit][G];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G * D];  // the G query heads

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

  // ---- loads.  Query: the G rows of this kv head, 16 bytes per thread.
  const bool q_thread = threadIdx.x < G * D / 8;
  uint32_t qv[4];
  buf_ld_stream<4>(buf_rsrc(q + sq.q_row * q_stride + g * G * D, G * D * 2), threadIdx.x * 16, qv);
  // Keys and values: lane (grp, l16) takes dims LD l16 .. + LD of keys
  // key_base + 4 it + grp; the buffers end at the unit's last valid key.
  const int64_t left = L - int64_t(s) * kSplit;
  const uint32_t nv = uint32_t(left < kSplit ? left : kSplit);
  const uint32_t row_bytes = uint32_t(row_stride) * 2;
  const int64_t unit_row = sq.kv_offset + int64_t(s) * kSplit;
  const __amdgpu_buffer_rsrc_t krs = buf_rsrc(k_all + unit_row * row_stride + g * D, nv * row_bytes);
  const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(v_all + unit_row * row_stride + g * D, nv * row_bytes);
  const uint32_t lane_off = uint32_t(w * kKeysPerWave + grp) * row_bytes + uint32_t(l16) * LD * 2;
  uint32_t kw[NIT][NDW], vw[NIT][NDW];
#pragma unroll
  for (int it = 0; it < NIT; ++it) buf_ld_stream<NDW>(krs, lane_off + uint32_t(4 * it) * row_bytes, kw[it]);
#pragma unroll
  for (int it = 0; it < NIT; ++it) buf_ld_stream<NDW>(vrs, lane_off + uint32_t(4 * it) * row_bytes, vw[it]);
  if (q_thread) *reinterpret_cast<uint4*>(s_q + threadIdx.x * 8) = make_uint4(qv[0], qv[1], qv[2], qv[3]);
  __syncthreads();

  // ---- S^T = K Q^T, one 16-key block kb at a time through the wave's LDS
  // buffer.  Block row i holds wave key 16 kb + 4 (i & 3) + (i >> 2), so output
  // register r of lane (head l16, grp) is the score of key 4 (4 kb + r) + grp:
  // the keys of the lane's own value registers.
  uint16_t* sk = s_k[w];
  f32x4 sacc[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kr = 4 * j + grp;  // key row within the block
      const uint32_t* src = kw[4 * kb + j];
      if constexpr (NDW == 4) {
        const int phys = l16 ^ (kr & (NG - 1));
        *reinterpret_cast<uint4*>(sk + kr * D + phys * 8) = make_uint4(src[0], src[1], src[2], src[3]);
      } else {
        const int phys = (l16 >> 1) ^ (kr & (NG - 1));
        *reinterpret_cast<uint2*>(sk + kr * D + phys * 8 + (l16 & 1) * 4) = make_uint2(src[0], src[1]);
      }
    }
    const int rr = 4 * (l16 & 3) + (l16 >> 2);
    sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // A operand: K[row rr][32 ks + 8 grp .. + 8]; B operand: Q[head l16][same dims] (0 past G)
      const int phys = (4 * ks + grp) ^ (rr & (NG - 1));
      const uint4 a = *reinterpret_cast<const uint4*>(sk + rr * D + phys * 8);
      const uint4 qq = l16 < G ? *reinterpret_cast<const uint4*>(s_q + l16 * D + 32 * ks + 8 * grp)
                               : make_uint4(0, 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qq), sacc[kb], 0, 0, 0);
    }
  }

  // ---- softmax over the unit: lane holds head l16, keys key_base + 4 it + grp
  float sc[NIT];
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int it = 4 * kb + r;
      const bool valid = key_base + 4 * it + grp < L;
      const float v = valid ? sacc[kb][r] * qscale : -INFINITY;
      sc[it] = v;
      mx = fmaxf(mx, v);
    }
  mx = max_x32(max_x16(mx));
  if (grp == 0 && l16 < G) s_m[w][l16] = mx;
  __syncthreads();
  const int hh = l16 < G ? l16 : 0;
  float m = s_m[0][hh];
#pragma unroll
  for (int ww = 1; ww < kWavesPerUnit; ++ww) m = fmaxf(m, s_m[ww][hh]);
  float p[NIT];
  float ls = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    p[it] = l16 < G ? __builtin_amdgcn_exp2f(sc[it] - m) : 0.f;
    ls += p[it];
  }
  ls = sum_x32(sum_x16(ls));
  if (grp == 0 && l16 < G) s_l[w][l16] = ls;
  // P as a bf16 high part plus a bf16 remainder (A operand: row head l16,
  // k = it of the lane's key group)
  uint4 ph[NKS], pl[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    uint32_t h4[4], l4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p0 = p[8 * kk + 2 * j], p1 = p[8 * kk + 2 * j + 1];
      const uint16_t a = f2bf(p0), c = f2bf(p1);
      h4[j] = uint32_t(a) | (uint32_t(c) << 16);
      l4[j] = pack2bf(p0 - bf2f(a), p1 - bf2f(c));
    }
    ph[kk] = make_uint4(h4[0], h4[1], h4[2], h4[3]);
    pl[kk] = make_uint4(l4[0], l4[1], l4[2], l4[3]);
  }

  // ---- O = P V, one MFMA block per lane dim e: B operand lane (col l16, grp)
  // holds V[key 4 it + grp][dim LD l16 + e], it = 8 kk .. 8 kk + 7, regrouped
  // from the token-major registers by byte permutes.  Lane (l16, grp) gets
  // heads 4 grp + r of dim LD l16 + e; the wave's partial goes into its own
  // (now free) key buffer.
  float* so = reinterpret_cast<float*>(sk);
#pragma unroll
  for (int e = 0; e < LD; ++e) {
    f32x4 oacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      uint32_t vt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vt[j] = __builtin_amdgcn_perm(vw[8 * kk + 2 * j + 1][e >> 1], vw[8 * kk + 2 * j][e >> 1],
                                      (e & 1) ? 0x07060302u : 0x05040100u);
      const bf16x8 vb = as_bf16x8(make_uint4(vt[0], vt[1], vt[2], vt[3]));
      oacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ph[kk]), vb, oacc, 0, 0, 0);
      oacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pl[kk]), vb, oacc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * grp + r < G) so[(4 * grp + r) * D + LD * l16 + e] = oacc[r];
  }
  __syncthreads();

  // ---- fixed-order sum over the waves; write the unit's partials
  for (int i = threadIdx.x; i < G * D; i += kSplitThreads) {
    const int h = i / D;
    const int d = i % D;
    float o = reinterpret_cast<const float*>(s_k[0])[h * D + d];
#pragma unroll
    for (int ww = 1; ww < kWavesPerUnit; ++ww) o += reinterpret_cast<const float*>(s_k[ww])[h * D + d];
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
  // (unrolled so several units' loads are in flight; the sums stay in
  // ascending s)
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < S; ++s) M = fmaxf(M, ws_ml[(base + s) * 2]);
  float Lsum = 0.f, O = 0.f;
#pragma unroll 8
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
