// Causal prefill attention (GQA) for gfx950, invariant under chunked prefill.
//
// The "Receipts" page (opening paragraph) asks that a request's output not
// depend on the prompt cache or on a prompt run ahead while it was typed: the
// same prompt prefilled in one pass or in chunks over an existing cache must
// give the same bits.  The M-0002 record ("Deterministic and bit-exact
// inference", field `technical`) lists attention among the operations made
// batch-invariant.  Both follow from one rule here: everything a query at
// absolute position t computes is a function of t and of the keys 0..t.
//  * Keys are processed in blocks of 64 aligned to absolute position 0,
//    block j = keys [64 j, 64 j + 64), in ascending j, with an online softmax.
//  * Queries are processed in wave tiles of 32 positions, also aligned to
//    absolute position 0.  A wave tile at position 32 i visits key blocks
//    0..floor(32 i / 64), so query t visits blocks 0..floor(t / 64) whatever
//    the chunk it arrived in; keys after t inside that block are masked.
//  * Rows of a tile outside the chunk (before its first position or after its
//    last) are computed with zero queries and never stored; keys at or after
//    the end of the chunk are not read (zero in LDS) and are always masked.
//
// Per wave and key block (D = head_dim, G = query heads per kv head):
//   S^T[key][q] = K Q^T   with v_mfma_f32_32x32x16_bf16 (A = K from LDS,
//                         B = Q held in registers), D/16 steps ascending;
//   m_new = max(m, rowmax S), alpha = exp2(m - m_new), P = exp2(S - m_new)
//   in fp32, l = l * alpha + rowsum(P) (fixed in-lane order plus one lane
//   exchange), O^T = O^T * alpha + V^T P^T with the same MFMA (A = V^T from a
//   transposed LDS copy, B = P split into two bf16 terms, see below).
// Scores are in log2 units (scale * log2(e) applied to S in fp32).  The final
// output is bf16(O / l).
//
// Work-group = 8 waves = (kv head g, tile of P = 256 / G positions): wave w
// takes query head g*G + w % G and the 32 positions tile + 32 (w / G).  The
// waves share the K / V^T blocks in LDS (double-buffered through registers;
// half the threads move K, the other half move V and transpose it 2 or 4 keys
// at a time).  Tiles run longest first.
#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

constexpr int KB = kPrefillKeyBlock;  // 64 keys per block
constexpr int QW = 32;                // query positions per wave
constexpr int NW = 8;                 // waves per work-group
constexpr int NTH = NW * 64;

// K block in LDS: [64 keys][D], 16-byte chunks xor-swizzled by key.
template <int D>
__device__ __forceinline__ int k_off(int key, int chunk) {
  return key * D + ((chunk ^ (key & 7)) << 3);
}
// V^T block in LDS: [D][64 keys], 8-byte granules (4 keys) xor-swizzled by row.
__device__ __forceinline__ int vt_off(int d, int key) {
  return d * KB + ((((key >> 2) ^ (d & 15)) << 2) | (key & 3));
}

template <int D, int G>
__global__ __launch_bounds__(NTH, 1) void prefill_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, uint16_t* __restrict__ o, int64_t o_stride,
    const PrefillSeq* __restrict__ seqs, PrefillSeq single, int Hkv, float sscale) {
  constexpr int P = QW * NW / G;      // positions per work-group tile
  constexpr int DCH = D / 8;          // 16-byte chunks per row
  constexpr int KK = D / 16;          // MFMA k-steps for S
  constexpr int BD = D / 32;          // output blocks along D
  constexpr int HT = NTH / 2;         // threads moving K (first half) or V (second half)
  constexpr int KPT = KB * DCH / HT;  // K chunks / V keys per thread
  static_assert(KPT == 2 || KPT == 4 || KPT == 8, "value transpose handles 2, 4 or 8 keys per thread");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][KB * D];

  // a device descriptor per sequence, or one sequence passed by value
  const PrefillSeq sq = seqs ? seqs[blockIdx.z] : single;
  const int g = blockIdx.y;
  const int first_tile = sq.q_start / P;
  const int last_pos = sq.q_start + sq.q_len - 1;
  const int n_tiles = last_pos / P - first_tile + 1;
  if (int(blockIdx.x) >= n_tiles) return;
  // longest tiles first
  const int tile_pos = (first_tile + n_tiles - 1 - int(blockIdx.x)) * P;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int h = g * G + (w % G);
  const int wpos = tile_pos + QW * (w / G);        // first position of this wave's queries
  const bool wave_active = wpos <= last_pos && wpos + QW - 1 >= sq.q_start;
  const int wave_last_blk = wpos / KB;             // diagonal block of the wave
  const int n_blk = min(tile_pos + P - 1, last_pos) / KB + 1;  // blocks the work-group loads
  const int kv_valid = last_pos + 1;               // keys 0 .. last_pos are in the cache

  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int64_t kv_stride = int64_t(Hkv) * D;

  // ---- queries of this wave: B operand of S^T = K Q^T, lane holds
  // Q[pos = wpos + l32][dims (2 kk + hf) * 8 .. + 8]
  bf16x8 qf[KK];
  {
    const int pos = wpos + l32;
    const bool in = pos >= sq.q_start && pos <= last_pos;
    const uint16_t* src = q + (sq.q_row + (pos - sq.q_start)) * q_stride + h * D + hf * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (in) v = *reinterpret_cast<const uint4*>(src + kk * 16);
      qf[kk] = as_bf16x8(v);
    }
  }

  // ---- block loads.  The first half of the work-group moves K: thread u
  // takes chunk u % DCH of keys u / DCH + (HT / DCH) i.  The second half moves
  // V: thread u takes chunk u % DCH of the KPT consecutive keys KPT (u / DCH)
  // .., which it transposes in registers into KPT-key rows of V^T.
  const bool is_k = t < HT;
  const int u = t % HT;
  const int uc = u % DCH;
  const int ur = u / DCH;
  const uint16_t* kbase = k_cache + sq.kv_base * kv_stride + int64_t(g) * D + uc * 8;
  const uint16_t* vbase = v_cache + sq.kv_base * kv_stride + int64_t(g) * D + uc * 8;
  uint4 rr[KPT];
  auto load_block = [&](int blk) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = blk * KB + (is_k ? ur + (HT / DCH) * i : KPT * ur + i);
      rr[i] = make_uint4(0, 0, 0, 0);
      if (key < kv_valid)
        rr[i] = *reinterpret_cast<const uint4*>((is_k ? kbase : vbase) + int64_t(key) * kv_stride);
    }
  };
  auto store_block = [&](int stage) {
    if (is_k) {
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        *reinterpret_cast<uint4*>(&sK[stage][k_off<D>(ur + (HT / DCH) * i, uc)]) = rr[i];
    } else {
      // rr[i] holds dims 8 uc .. + 8 of key KPT ur + i; row d of V^T gets the
      // KPT keys' values of dim d (2 bytes each, ascending key), written as
      // 8-byte granules of 4 keys.
      const uint32_t* w32 = reinterpret_cast<const uint32_t*>(rr);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = uc * 8 + e;
        // 16-bit element e of key i sits in word 4 i + e / 2, half e % 2
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        if constexpr (KPT == 2) {
          *reinterpret_cast<uint32_t*>(&sV[stage][vt_off(d, KPT * ur)]) =
              __builtin_amdgcn_perm(w32[4 + e / 2], w32[0 + e / 2], sel);
        } else {
#pragma unroll
          for (int q4 = 0; q4 < KPT / 4; ++q4) {
            uint2 v;
            v.x = __builtin_amdgcn_perm(w32[16 * q4 + 4 + e / 2], w32[16 * q4 + 0 + e / 2], sel);
            v.y = __builtin_amdgcn_perm(w32[16 * q4 + 12 + e / 2], w32[16 * q4 + 8 + e / 2], sel);
            *reinterpret_cast<uint2*>(&sV[stage][vt_off(d, KPT * ur + 4 * q4)]) = v;
          }
        }
      }
    }
  };

  f32x16 acc_o[BD];
#pragma unroll
  for (int bd = 0; bd < BD; ++bd)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[bd][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  load_block(0);
  store_block(0);
  __syncthreads();

  for (int blk = 0; blk < n_blk; ++blk) {
    const int cur = blk & 1;
    if (blk + 1 < n_blk) load_block(blk + 1);
    if (wave_active && blk <= wave_last_blk) {
      const uint16_t* cK = sK[cur];
      const uint16_t* cV = sV[cur];
      // S^T blocks [bk]: keys 32 bk .. of the block, queries of the wave
      f32x16 s[2];
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[bk][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(cK + k_off<D>(32 * bk + l32, 2 * kk + hf));
          s[bk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[bk], 0, 0, 0);
        }
      // scale, mask, online softmax.  Lane holds query wpos + l32 and keys
      // blk*64 + 32 bk + 8 (r / 4) + 4 hf + r % 4.
      const bool diag = blk == wave_last_blk;
      const int qpos = wpos + l32;
      float mx = -INFINITY;
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = blk * KB + 32 * bk + 8 * (r >> 2) + 4 * hf + (r & 3);
          float v = s[bk][r] * sscale;
          if (diag && (key > qpos || key >= kv_valid)) v = -INFINITY;
          s[bk][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(s[bk][r] - m_new);
          s[bk][r] = pv;
          rs += pv;
        }
      rs += __shfl_xor(rs, 32, 64);
      l_run = l_run * alpha + rs;
      // multiplying by exactly 1 changes nothing: skip when no lane's max moved
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int bd = 0; bd < BD; ++bd)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[bd][r] *= alpha;
      }
      // O^T[d][q] += V^T[d][key] P^T[key][q].  P (fp32) enters the bf16 MFMA as
      // two bf16 terms, P = hi + lo with hi = bf16(P), lo = bf16(P - hi), so
      // the weights carry ~16 significant bits; each k-step adds V hi, then
      // V lo.  MFMA k-slot hf*8 + e of step (bk, half) is key
      // 32 bk + 16 half + 8 (e / 4) + 4 hf + e % 4, which is register
      // 8 half + e of the S^T block; the V^T operand reads the same keys.
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int key_a = 32 * bk + 16 * half + 4 * hf;
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = s[bk][8 * half + 2 * e];
            const float b = s[bk][8 * half + 2 * e + 1];
            const uint32_t hp = pack2bf(a, b);
            hw[e] = hp;
            lw[e] = pack2bf(a - bf2f_lo(hp), b - bf2f_hi(hp));
          }
          const bf16x8 p_hi = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
          const bf16x8 p_lo = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
          for (int bd = 0; bd < BD; ++bd) {
            const int d = 32 * bd + l32;
            const uint2 lo = *reinterpret_cast<const uint2*>(cV + vt_off(d, key_a));
            const uint2 hi = *reinterpret_cast<const uint2*>(cV + vt_off(d, key_a + 8));
            const bf16x8 vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
            acc_o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p_hi, acc_o[bd], 0, 0, 0);
            acc_o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p_lo, acc_o[bd], 0, 0, 0);
          }
        }
    }
    if (blk + 1 < n_blk) store_block(cur ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
  // ---- normalise and store: lane holds query wpos + l32 and dims
  // 32 bd + 8 (r / 4) + 4 hf + r % 4 (4 consecutive dims per register group).
  const int pos = wpos + l32;
  if (pos < sq.q_start || pos > last_pos) return;
  const float inv = 1.0f / l_run;
  uint16_t* dst = o + (sq.q_row + (pos - sq.q_start)) * o_stride + h * D;
#pragma unroll
  for (int bd = 0; bd < BD; ++bd)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = 32 * bd + 8 * rg + 4 * hf;
      uint2 v;
      v.x = pack2bf(acc_o[bd][4 * rg + 0] * inv, acc_o[bd][4 * rg + 1] * inv);
      v.y = pack2bf(acc_o[bd][4 * rg + 2] * inv, acc_o[bd][4 * rg + 3] * inv);
      *reinterpret_cast<uint2*>(dst + d) = v;
    }
}

template <int D, int G>
hipError_t launch_t(const uint16_t* q, int64_t q_stride, const uint16_t* k, const uint16_t* v,
                    uint16_t* o, int64_t o_stride, const PrefillSeq* seqs, PrefillSeq single,
                    int n_seqs, int max_tiles, int Hkv, float sscale, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<D, G>), dim3(max_tiles, Hkv, n_seqs), dim3(NTH), 0, s, q,
                     q_stride, k, v, o, o_stride, seqs, single, Hkv, sscale);
  return hipGetLastError();
}

}  // namespace

int prefill_positions_per_tile(int group) { return QW * NW / group; }

hipError_t launch_attn_prefill(const uint16_t* q, int64_t q_row_stride, const uint16_t* k_cache,
                               const uint16_t* v_cache, uint16_t* o, int64_t o_row_stride,
                               const PrefillSeq* d_seqs, const PrefillSeq* h_single, int n_seqs,
                               int max_tiles, int Hq, int Hkv, int D, float scale, hipStream_t s) {
  PrefillSeq single{};
  if (h_single) single = *h_single;
  const int G = Hq / Hkv;
  const float sscale = scale * 1.4426950408889634f;
#define BI_PF(DD, GG)                                                                          \
  if (D == DD && G == GG)                                                                    \
    return launch_t<DD, GG>(q, q_row_stride, k_cache, v_cache, o, o_row_stride, d_seqs, single, \
                            n_seqs, max_tiles, Hkv, sscale, s);
  BI_PF(64, 1) BI_PF(64, 2) BI_PF(64, 4)
  BI_PF(128, 1) BI_PF(128, 2) BI_PF(128, 4)
#undef BI_PF
  return hipErrorInvalidValue;
}

}  // namespace bi
