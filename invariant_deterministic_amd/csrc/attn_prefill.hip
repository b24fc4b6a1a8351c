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
//    block j = keys [64 j, 64 j + 64), in ascending j.  Each block is cut in
//    two halves, keys [64 j, 64 j + 32) and [64 j + 32, 64 j + 64); every query
//    keeps one online softmax per half over the blocks 0..floor(t / 64), and
//    the two are merged once at the end, half 0 first.
//  * Queries are processed in wave tiles of 32 positions, also aligned to
//    absolute position 0, so query t sees the same halves in the same order
//    whatever the chunk it arrived in; keys after t are masked (a half that
//    lies wholly after the wave's queries is skipped).
//  * Rows of a tile outside the chunk (before its first position or after its
//    last) are computed with zero queries and never stored; keys at or after
//    the end of the chunk read as zero (bounded buffer loads, no branch) and
//    are always masked.
//
// Per wave and block (D = head_dim, G = query heads per kv head), for the
// wave's 32 keys.  Within a half, key 4 j + c (j = 0..7) is "class" c = 0..3;
// every sum below groups the keys by class, in a layout a one-query decode
// kernel can reproduce operation for operation (so a token's bits do not
// depend on whether it was prefilled or decoded):
//   S^T[key][q] = K Q^T   with v_mfma_f32_32x32x16_bf16 (A = K from LDS, its
//                         rows permuted so that output register r of lane
//                         half hf holds class 2 (r / 8) + hf, j = r % 8;
//                         B = Q held in registers), D/16 steps ascending;
//   the row's reference maximum m moves to rowmax(S) * scale only when that
//   exceeds m by more than 8 (log2 units), so weights stay <= 2^8 and O is
//   rescaled rarely: alpha = exp2(m - m_new), P = exp2(fma(S, scale, -m_new))
//   in fp32 (one rounding of the scaled, shifted score),
//   rowsum(P) = ((sum c0 + sum c2) + (sum c1 + sum c3)), each class summed in
//   ascending j, l = fma(l, alpha, rowsum);
//   O^T = O^T * alpha + V^T P^T with the same MFMA (A = V^T from a transposed
//   LDS copy whose keys are stored class by class, B = P split into two bf16
//   terms, see below), four instructions per 32 dims: P_hi of classes 0 and
//   1, P_hi of 2 and 3, P_lo of 0 and 1, P_lo of 2 and 3 (each instruction
//   adds two 8-key groups in order).  Each decision is the row's own, so it
//   depends on nothing outside the query's keys.
// Scores are in log2 units (scale = softmax scale * log2(e), applied in fp32).  Merge:
// M = max(m0, m1), a_i = exp2(m_i - M), output
// bf16(fma(O0, a0, O1 a1) / fma(l0, a0, l1 a1)).
//
// Work-group = 8 waves = (kv head g, tile of P = 128 / G positions): wave w
// takes query head g*G + w % G, key half (w / G) % 2 and the 32 positions
// tile + 32 (w / 2G).  The waves share the K / V^T blocks in LDS (four
// stages filled through registers; half the threads move K, the other half
// move V and transpose it 2 or 4 keys at a time).  The two waves of a SIMD
// alternate, one phase apart: a block's score and value MFMAs in one phase,
// its softmax in the next (see the block loop).  Tiles run longest
// first; when a chunk has more tiles than the GPU has compute units, the grid
// is folded so that work-group x runs tile n - 1 - x and then tile x, which
// evens out the causal triangle.  Which work-group runs a tile never changes
// what the tile computes.
#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

constexpr int KB = kPrefillKeyBlock;  // 64 keys per block
constexpr int QW = 32;                // query positions per wave
constexpr int NW = 8;                 // waves per work-group
constexpr int NTH = NW * 64;

// K block in LDS: [64 keys][D], 16-byte chunks xor-swizzled by key so that
// the 16 keys one 16-lane cycle of a fragment read touches sit on 16 distinct
// 16-byte bank groups (64 four-byte banks = 256 bytes: one D = 128 row, two
// D = 64 rows).
template <int D>
__device__ __forceinline__ int k_off(int key, int chunk) {
  if constexpr (D == 128) return key * D + ((chunk ^ (key & 15)) << 3);
  else return key * D + ((chunk ^ ((key >> 1) & 7)) << 3);
}
// K block row of key k (0..63): within each 32-key half, MFMA row i holds key
// 4 j + c with c = 2 (i / 16) + (i / 4) % 2 and j = 4 ((i / 8) % 2) + i % 4,
// which puts class c = 2 (r / 8) + hf, j = r % 8 into output register r of
// lane half hf.
__device__ __forceinline__ int k_row(int k) {
  const int c = k & 3, j = (k >> 2) & 7;
  return (k & 32) | ((c >> 1) << 4) | ((j >> 2) << 3) | ((c & 1) << 2) | (j & 3);
}
// V^T block in LDS: [D][64 positions], position 32 h + 8 c + j holding key
// 32 h + 4 j + c (the keys of a half stored class by class), in 8-byte
// granules (4 positions) xor-swizzled by ((d / 2) ^ (d / 8)) % 16: a 32-lane
// cycle of the PV fragment read (rows d .. d + 31, one granule) and of the
// transposing stores (rows 8 u + e) then spread over all 64 banks.
__device__ __forceinline__ int vt_off(int d, int pos) {
  return d * KB + ((((pos >> 2) ^ (((d >> 1) ^ (d >> 3)) & 15)) << 2) | (pos & 3));
}
__device__ __forceinline__ int key_at_pos(int pos) {
  return (pos & 32) | ((pos & 7) << 2) | ((pos >> 3) & 3);
}

template <int D, int G, bool Q8>
__global__ __launch_bounds__(NTH, 1) void prefill_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int32_t* __restrict__ pages, int64_t n_pages, uint16_t* __restrict__ o, int64_t o_stride,
    const PrefillSeq* __restrict__ seqs, PrefillSeq single, int Hkv, float sscale, int fold) {
  constexpr int R = NW / (2 * G);     // 32-position groups per tile
  constexpr int P = QW * R;           // positions per tile
  constexpr int DCH = D / 8;          // 16-byte chunks per row
  constexpr int KK = D / 16;          // MFMA k-steps for S
  constexpr int BD = D / 32;          // output blocks along D
  constexpr int HT = NTH / 2;         // threads moving K (first half) or V (second half)
  constexpr int KPT = KB * DCH / HT;  // K chunks / V keys per thread
  static_assert(KPT == 2 || KPT == 4 || KPT == 8, "value transpose handles 2, 4 or 8 keys per thread");
  constexpr int NS = 4;               // LDS stages: block b in stage b % 4
  static_assert(G * R * BD * 16 * 64 <= 2 * NS * KB * D / 2, "the half-merge fits the block buffers");
  // [0][stage] = K block, [1][stage] = V^T block; after a tile, the merge buffer
  __shared__ __attribute__((aligned(16))) uint16_t sKV[2][NS][KB * D];
  __shared__ float s_ml[G * R][2][QW];

  const PrefillSeq sq = seqs ? seqs[blockIdx.z] : single;
  const int g = blockIdx.y;
  const int first_tile = sq.q_start / P;
  const int last_pos = sq.q_start + sq.q_len - 1;
  const int n_tiles = last_pos / P - first_tile + 1;
  const int x = int(blockIdx.x);
  if (x >= (fold ? (n_tiles + 1) / 2 : n_tiles)) return;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int hs = w % G;               // query head within the kv head's group
  const int kh = (w / G) & 1;         // key half: keys 32 kh .. 32 kh + 31 of every block
  const int pg = w / (2 * G);         // 32-position group within the tile
  const int h = g * G + hs;
  const int kv_valid = last_pos + 1;  // keys 0 .. last_pos are in the cache
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int64_t kv_stride = int64_t(Hkv) * D;

  const bool is_k = t < HT;
  const int u = t % HT;
  const int uc = u % DCH;
  const int ur = u / DCH;
  // head g's slice of the sequence's cache rows; the lane's 16-byte chunk uc
  // goes into the per-lane buffer offset
  const uint16_t* kbase = static_cast<const uint16_t*>(k_cache) + sq.kv_base * kv_stride + int64_t(g) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(v_cache) + sq.kv_base * kv_stride + int64_t(g) * D;
  uint4 rr[KPT];
  uint2 rq[KPT];   // int8 cache: 8 codes of the chunk, and the key's scale
  float rsc[KPT];
  // block blk as a buffer over its valid keys (keys >= kv_valid read as zero)
  auto load_block = [&](int blk) {
    const int nvalid = min(KB, max(0, kv_valid - blk * KB));
    if constexpr (!Q8) {
      // K or V is chosen per wave (the first HT threads move K)
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(wave_uniform((is_k ? kbase : vbase) + int64_t(blk) * KB * kv_stride),
                                                 wave_uniform(uint32_t(nvalid) * uint32_t(kv_stride) * 2));
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int key = is_k ? ur + (HT / DCH) * i : key_at_pos(KPT * ur + i);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
            rs, int(uint32_t(key) * uint32_t(kv_stride) * 2 + uint32_t(uc) * 16), 0, 0);
        rr[i] = make_uint4(v.x, v.y, v.z, v.w);
      }
    } else {
      // block blk is page pages[kv_base + blk] (the sequence's entries of the table, kv_base
      // the first): rows page * 64 .. + 63 of the int8 pool; an index outside the pool is
      // clamped into it (memory stays in bounds; such a table gives meaningless output)
      int64_t page = pages[sq.kv_base + blk];
      page = page < 0 ? 0 : (page >= n_pages ? n_pages - 1 : page);
      const int64_t prow = page * KB;
      const int8_t* qb = static_cast<const int8_t*>(is_k ? k_cache : v_cache) + prow * kv_stride + int64_t(g) * D;
      const float* sb = (is_k ? k_scale : v_scale) + prow * Hkv + g;
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(wave_uniform(reinterpret_cast<const uint16_t*>(qb)),
                                                 wave_uniform(uint32_t(nvalid) * uint32_t(kv_stride)));
      const __amdgpu_buffer_rsrc_t ss = buf_rsrc(wave_uniform(reinterpret_cast<const uint16_t*>(sb)),
                                                 wave_uniform(uint32_t(nvalid) * uint32_t(Hkv) * 4));
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int key = is_k ? ur + (HT / DCH) * i : key_at_pos(KPT * ur + i);
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, int(uint32_t(key) * uint32_t(kv_stride) + uint32_t(uc) * 8), 0, 0);
        rq[i] = make_uint2(v[0], v[1]);
        rsc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ss, int(uint32_t(key) * uint32_t(Hkv) * 4), 0, 0));
      }
    }
  };
  // int8 codes of a chunk -> bf16(float(q) * scale), 8 values
  auto dequant = [&](int i) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = e < 4 ? rq[i].x : rq[i].y;
      f[e] = float(int8_t(w >> (8 * (e & 3)))) * rsc[i];
    }
    rr[i] = pack8(f);
  };
  auto store_block = [&](int stage) {
    if constexpr (Q8) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) dequant(i);
    }
    if (is_k) {
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        *reinterpret_cast<uint4*>(&sKV[0][stage][k_off<D>(k_row(ur + (HT / DCH) * i), uc)]) = rr[i];
    } else {
      const uint32_t* w32 = reinterpret_cast<const uint32_t*>(rr);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = uc * 8 + e;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        if constexpr (KPT == 2) {
          *reinterpret_cast<uint32_t*>(&sKV[1][stage][vt_off(d, KPT * ur)]) =
              __builtin_amdgcn_perm(w32[4 + e / 2], w32[0 + e / 2], sel);
        } else {
#pragma unroll
          for (int q4 = 0; q4 < KPT / 4; ++q4) {
            uint2 v;
            v.x = __builtin_amdgcn_perm(w32[16 * q4 + 4 + e / 2], w32[16 * q4 + 0 + e / 2], sel);
            v.y = __builtin_amdgcn_perm(w32[16 * q4 + 12 + e / 2], w32[16 * q4 + 8 + e / 2], sel);
            *reinterpret_cast<uint2*>(&sKV[1][stage][vt_off(d, KPT * ur + 4 * q4)]) = v;
          }
        }
      }
    }
  };

  auto do_tile = [&](int tile) {
    const int tile_pos = tile * P;
    const int wpos = tile_pos + QW * pg;               // first position of this wave's queries
    const bool wave_active = wpos <= last_pos && wpos + QW - 1 >= sq.q_start;
    // (wave-uniform values, made scalar so the branches below are uniform)
    const int wave_last_blk = __builtin_amdgcn_readfirstlane(wpos / KB);  // diagonal block of the wave
    // on the diagonal block the wave's key half may lie wholly after its queries
    const int wave_end_blk =
        __builtin_amdgcn_readfirstlane(wave_last_blk + (kh * 32 > (wpos % KB) + QW - 1 ? 0 : 1));
    const int n_blk = min(tile_pos + P - 1, last_pos) / KB + 1;  // blocks the work-group loads

    // queries: B operand of S^T = K Q^T, lane holds Q[pos = wpos + l32][dims (2 kk + hf) * 8 .. + 8]
    bf16x8 qf[KK];
    {
      // rows of the chunk as a buffer: positions outside it read as zero
      const int pos = wpos + l32;
      const int r0 = wpos - sq.q_start;  // chunk row of the wave's first position (may be negative)
      const int lo = max(r0, 0), hi = min(r0 + QW, sq.q_len);
      const uint32_t nrows = hi > lo ? uint32_t(hi - lo) : 0u;
      const __amdgpu_buffer_rsrc_t rs =
          buf_rsrc(wave_uniform(q + (sq.q_row + lo) * q_stride + h * D), wave_uniform(nrows * uint32_t(q_stride) * 2));
      // lanes before the chunk get an offset past the buffer's end
      const uint32_t row_off = pos - sq.q_start >= lo ? uint32_t(pos - sq.q_start - lo) : nrows;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
            rs, int(row_off * uint32_t(q_stride) * 2 + uint32_t(hf * 8 + kk * 16) * 2), 0, 0);
        qf[kk] = as_bf16x8(make_uint4(v.x, v.y, v.z, v.w));
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qf[kk]));  // complete before the block loop
    }
    f32x16 acc_o[BD];
#pragma unroll
    for (int bd = 0; bd < BD; ++bd)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[bd][r] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;

    // Schedule: waves w and w + 4 share a SIMD; group w / 4 = 1 runs one phase (barrier)
    // behind group 0.  Iteration b = [MFMA phase: S(b), then O += V(b - 1) P(b - 1), block
    // b + 2 stored into LDS] | [VALU phase: softmax of S(b) (mask, reference maximum,
    // alpha, O *= alpha, P), loads of block b + 3 issued], so while one wave of a SIMD
    // issues MFMAs the other runs its softmax.  Each row's operations and their order are
    // those of the plain loop (O: ..., + V(b-1) P(b-1), * alpha(b), + V(b) P(b), ...).
    // Block b lives in stage b % 4: written in the MFMA phase of iteration b - 2, read until
    // group 1's MFMA phase of iteration b + 1.
    const int grp = w >> 2;
    const int nb_w = wave_active ? wave_end_blk : 0;  // blocks whose scores this wave computes
    load_block(0);
    store_block(0);
    if (n_blk > 1) {
      load_block(1);
      store_block(1);
    }
    if (n_blk > 2) load_block(2);
    __syncthreads();
    if (grp == 1) __syncthreads();
    f32x16 s;
    bf16x8 p_hi[2], p_lo[2];
    for (int blk = 0; blk <= n_blk; ++blk) {
      // ---- MFMA phase, at raised wave priority: the SIMD's other wave is in its VALU
      // phase, and this wave's MFMAs and fragment reads go first
      __builtin_amdgcn_s_setprio(1);
      if (blk < nb_w) {
        // S^T: keys 32 kh .. 32 kh + 31 of the block, queries of the wave
        const uint16_t* cK = sKV[0][blk % NS];
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        // every K fragment is read before the chain of MFMAs starts
        bf16x8 kf[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          kf[kk] = *reinterpret_cast<const bf16x8*>(cK + k_off<D>(32 * kh + l32, 2 * kk + hf));
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
      }
      if (blk >= 1 && blk - 1 < nb_w) {
        // O^T[d][q] += V^T[d][key] P^T[key][q] for block blk - 1, P = hi + lo in bf16.  MFMA
        // k-slot e of lane half hf in instruction `half` is register 8 half + e of S^T: key
        // 4 e + c of class c = 2 half + hf, V^T positions 32 kh + 8 c + e.  Order: hi(0),
        // hi(1), lo(0), lo(1).
        const uint16_t* cV = sKV[1][(blk - 1) % NS];
#pragma unroll
        for (int bd = 0; bd < BD; ++bd) {
          const int d = 32 * bd + l32;
          bf16x8 vf[2];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int pos = 32 * kh + 8 * (2 * half + hf);
            const uint2 lo = *reinterpret_cast<const uint2*>(cV + vt_off(d, pos));
            const uint2 hi = *reinterpret_cast<const uint2*>(cV + vt_off(d, pos + 4));
            vf[half] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          }
          acc_o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[0], p_hi[0], acc_o[bd], 0, 0, 0);
          acc_o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[1], p_hi[1], acc_o[bd], 0, 0, 0);
          acc_o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[0], p_lo[0], acc_o[bd], 0, 0, 0);
          acc_o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[1], p_lo[1], acc_o[bd], 0, 0, 0);
        }
      }
      if (blk + 2 < n_blk) store_block((blk + 2) % NS);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      // ---- VALU phase
      if (blk + 3 < n_blk) load_block(blk + 3);
      if (blk < nb_w) {
        // lane holds query wpos + l32; register r the key of class 2 (r / 8) + hf, j = r % 8
        const bool diag = blk == wave_last_blk;
        const int qpos = wpos + l32;
        float mx = -INFINITY;
        if (diag) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = blk * KB + 32 * kh + 4 * (r & 7) + 2 * (r >> 3) + hf;
            if (key > qpos || key >= kv_valid) s[r] = -INFINITY;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        // the largest scaled score: scaling by a positive constant keeps the order
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sscale;
        // the row's reference maximum moves only when the block's maximum
        // exceeds it by more than 8 (log2 units): weights stay <= 2^8
        const bool lift = mx > m_run + 8.0f;
        const float m_new = lift ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sscale, -m_new));
        // per class in ascending j, then (c0 + c2) + (c1 + c3)
        float sa = s[0], sb = s[8];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
          sa += s[j];
          sb += s[8 + j];
        }
        const float tc = sa + sb;
        const float rs = tc + __shfl_xor(tc, 32, 64);
        l_run = __builtin_fmaf(l_run, alpha, rs);
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int bd = 0; bd < BD; ++bd)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[bd][r] *= alpha;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = s[8 * half + 2 * e];
            const float b = s[8 * half + 2 * e + 1];
            const uint32_t hp = pack2bf(a, b);
            hw[e] = hp;
            lw[e] = pack2bf(a - bf2f_lo(hp), b - bf2f_hi(hp));
          }
          p_hi[half] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
          p_lo[half] = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
        }
      }
      __syncthreads();
    }
    if (grp == 0) __syncthreads();

    // ---- merge the key halves in a fixed order (half 0, half 1) and store.
    // Lane holds query wpos + l32 and dims 32 bd + 8 (r / 4) + 4 hf + r % 4.
    const int slot = hs + G * pg;
    float* sm = reinterpret_cast<float*>(&sKV[0][0][0]);
    if (kh == 1 && wave_active) {
#pragma unroll
      for (int bd = 0; bd < BD; ++bd)
#pragma unroll
        for (int r = 0; r < 16; ++r) sm[((slot * BD + bd) * 16 + r) * 64 + lane] = acc_o[bd][r];
      if (hf == 0) {
        s_ml[slot][0][l32] = m_run;
        s_ml[slot][1][l32] = l_run;
      }
    }
    __syncthreads();
    if (kh == 0 && wave_active) {
      const int pos = wpos + l32;
      if (pos >= sq.q_start && pos <= last_pos) {
        const float m1 = s_ml[slot][0][l32];
        const float l1 = s_ml[slot][1][l32];
        const float mm = fmaxf(m_run, m1);
        const float a0 = __builtin_amdgcn_exp2f(m_run - mm);
        const float a1 = __builtin_amdgcn_exp2f(m1 - mm);
        const float inv = 1.0f / __builtin_fmaf(l_run, a0, l1 * a1);
        uint16_t* dst = o + (sq.q_row + (pos - sq.q_start)) * o_stride + h * D;
#pragma unroll
        for (int bd = 0; bd < BD; ++bd)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            float ov[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 4 * rg + j;
              ov[j] = __builtin_fmaf(acc_o[bd][r], a0, sm[((slot * BD + bd) * 16 + r) * 64 + lane] * a1) * inv;
            }
            const int d = 32 * bd + 8 * rg + 4 * hf;
            uint2 v;
            v.x = pack2bf(ov[0], ov[1]);
            v.y = pack2bf(ov[2], ov[3]);
            *reinterpret_cast<uint2*>(dst + d) = v;
          }
      }
    }
    __syncthreads();  // the buffers are reused by the next tile
  };

  // longest tile first; a folded grid (more tiles than the GPU holds at once)
  // also gives work-group x tile x, so each work-group has about equal work
  const int ta = n_tiles - 1 - x;
  do_tile(first_tile + ta);
  if (fold && x < ta) do_tile(first_tile + x);
}

template <int D, int G, bool Q8>
hipError_t launch_t(const uint16_t* q, int64_t q_stride, const void* k, const void* v, const float* ks,
                    const float* vs, const int32_t* pages, int64_t n_pages, uint16_t* o, int64_t o_stride,
                    const PrefillSeq* seqs, PrefillSeq single, int n_seqs, int max_tiles, int Hkv, float sscale,
                    hipStream_t s) {
  // compute units of the device, read once (a thread-safe constant): it only decides
  // whether the grid is folded, never what a tile computes
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  const int fold = int64_t(max_tiles) * Hkv * n_seqs > cus ? 1 : 0;
  const int gx = fold ? (max_tiles + 1) / 2 : max_tiles;
  hipLaunchKernelGGL((prefill_kernel<D, G, Q8>), dim3(gx, Hkv, n_seqs), dim3(NTH), 0, s, q, q_stride, k, v, ks, vs,
                     pages, n_pages, o, o_stride, seqs, single, Hkv, sscale, fold);
  return hipGetLastError();
}

}  // namespace

int prefill_positions_per_tile(int group) { return QW * NW / (2 * group); }

hipError_t launch_attn_prefill(const uint16_t* q, int64_t q_row_stride, const uint16_t* k_cache,
                               const uint16_t* v_cache, uint16_t* o, int64_t o_row_stride,
                               const PrefillSeq* d_seqs, const PrefillSeq* h_single, int n_seqs,
                               int max_tiles, int Hq, int Hkv, int D, float scale, hipStream_t s) {
  PrefillSeq single{};
  if (h_single) single = *h_single;
  const int G = Hq / Hkv;
  const float sscale = scale * 1.4426950408889634f;
#define BI_PF(DD, GG)                                                                                    \
  if (D == DD && G == GG)                                                                              \
    return launch_t<DD, GG, false>(q, q_row_stride, k_cache, v_cache, nullptr, nullptr, nullptr, 0, o,          \
                                   o_row_stride, d_seqs, single, n_seqs, max_tiles, Hkv, sscale, s);
  BI_PF(64, 1) BI_PF(64, 2) BI_PF(64, 4)
  BI_PF(128, 1) BI_PF(128, 2) BI_PF(128, 4)
#undef BI_PF
  return hipErrorInvalidValue;
}

hipError_t launch_attn_prefill_q8(const uint16_t* q, int64_t q_row_stride, const int8_t* k_pool, const int8_t* v_pool,
                                  const float* k_scale, const float* v_scale, const int32_t* pages, int64_t n_pages,
                                  uint16_t* o, int64_t o_row_stride, const PrefillSeq* d_seqs,
                                  const PrefillSeq* h_single, int n_seqs, int max_tiles, int Hq, int Hkv, int D,
                                  float scale, hipStream_t s) {
  PrefillSeq single{};
  if (h_single) single = *h_single;
  const int G = Hq / Hkv;
  const float sscale = scale * 1.4426950408889634f;
#define BI_PF(DD, GG)                                                                                    \
  if (D == DD && G == GG)                                                                              \
    return launch_t<DD, GG, true>(q, q_row_stride, k_pool, v_pool, k_scale, v_scale, pages, n_pages, o,        \
                                  o_row_stride, d_seqs, single, n_seqs, max_tiles, Hkv, sscale, s);
  BI_PF(64, 1) BI_PF(64, 2) BI_PF(64, 4)
  BI_PF(128, 1) BI_PF(128, 2) BI_PF(128, 4)
#undef BI_PF
  return hipErrorInvalidValue;
}

}  // namespace bi




