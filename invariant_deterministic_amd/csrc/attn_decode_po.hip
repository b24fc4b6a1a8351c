// Decode attention in the prefill kernel's key order for gfx950: a token
// decoded alone gets the bits it gets when prefilled (or verified inside a
// drafted chunk).
//
// The "Receipts" page (opening paragraph) lists run-ahead drafting among the
// things a request's output must not depend on, and the M-0002 record
// ("Deterministic and bit-exact inference", "Limitations") names speculative
// decoding as open work for batch-invariant serving.  Prefill computes a
// query at absolute position t over keys 0..t in a fixed order; this kernel
// repeats exactly those operations for one query per request (t = L - 1):
//  * keys in blocks of 64 aligned to position 0, ascending; each block cut
//    into halves of 32 keys with one online softmax per half, merged at the
//    end; half 1 of the diagonal block is skipped when t % 64 < 32 (prefill's
//    wave for positions 64 j .. 64 j + 31 skips it);
//  * per key, the D-long score S as MFMA steps of 8 dims in ascending order
//    (v_mfma_f32_16x16x32_bf16 here, keys as rows and the G heads as columns;
//    prefill's v_mfma_f32_32x32x16_bf16 chains the same steps), keys after t
//    set to -inf;
//  * within a half, key 4 j + c is of class c: the block maximum of S times
//    scale = softmax scale * log2(e), the lazy rescale (the reference maximum
//    m moves only when the block maximum exceeds it by more than 8),
//    alpha = exp2(m - m_new), P = exp2(fma(S, scale, -m_new)),
//    rowsum = (sum c0 + sum c2) + (sum c1 + sum c3) with
//    each class summed in ascending j, l = fma(l, alpha, rowsum), O *= alpha;
//  * P V with P = hi + lo in bf16, the 8-key groups added in the order
//    hi c0, hi c1, hi c2, hi c3, lo c0, lo c1, lo c2, lo c3;
//  * merge: M = max(m0, m1), a_i = exp2(m_i - M),
//    o = bf16(fma(O0, a0, O1 a1) / fma(l0, a0, l1 a1)).
// The lane layout makes these sums fall out directly: lane (head column l16,
// lane group grp) loads 8 keys 4 j + grp of its wave's half token-major, so
// it holds class grp; the class sums are in-lane, the tree is two lane
// exchanges, and the class-grp keys are one MFMA step of the value product.
//
// Work-group = 2 waves (key halves 0 and 1) per (request, kv head); the
// waves share nothing inside the key loop.  K and V go HBM -> registers
// (double-buffered across blocks, bounded buffer loads read zero past the
// request's last key); K reaches the MFMA operand layout through a per-wave
// LDS buffer.  An optional order array lets the caller start the longest
// requests first; the order never changes what a request computes.
#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

constexpr int KB = kPrefillKeyBlock;  // 64 keys per block
constexpr int NT = 128;               // two waves

template <int D, int G, bool Q8>
__device__ __forceinline__ void decode_po_body(
    const uint16_t* __restrict__ q, int64_t q_stride, const void* __restrict__ k_all,
    const void* __restrict__ v_all, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int32_t* __restrict__ block_tables, int max_pages, int64_t n_pages, const DecodeSeq* __restrict__ seqs,
    const int64_t* __restrict__ kv_offset, const int32_t* __restrict__ kv_len,
    const int32_t* __restrict__ order, int B, int Hkv, int64_t max_len, float sscale,
    uint16_t* __restrict__ o, int64_t o_stride) {
  constexpr int LD = D / 16;  // dims per lane in the token-major loads
  constexpr int NDW = LD / 2;
  constexpr int KS = D / 32;  // MFMA k-steps over the head dimension
  constexpr int NG = D / 8;   // 16-byte granules per key row
  static_assert(G <= 8, "heads 4 grp + r of the value product cover at most 16");
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][16 * D];  // per-wave K tile
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G * D];
  __shared__ float s_o[G * D];    // half 1's O
  __shared__ float s_ml[2][2][G];  // [half][m, l][head]

  // int8: grid (8 Hkv, ceil(B / 8)): work-group w = x + 8 Hkv y runs on XCD w % 8 = x % 8,
  // and takes kv head x / 8 of request slot 8 y + x % 8, so the kv heads of one request run
  // together on one XCD and share its L2 (the per-token scales of all heads sit in one
  // 32-byte sector).  bf16: grid (Hkv, B), the heads of a request dispatched one after
  // another (across the XCDs), which measured faster for this form.  Slots past B do nothing.
  int g, slot;
  if constexpr (Q8) {
    g = int(blockIdx.x) >> 3;
    slot = int(blockIdx.y) * 8 + (int(blockIdx.x) & 7);
  } else {
    g = int(blockIdx.x);
    slot = int(blockIdx.y);
  }
  if (slot >= B) return;
  const int b = order ? order[slot] : slot;
  // koff: cache row of key 0 (bf16); pt: first page-table entry of the request (int8 cache,
  // addressed through page tables: the sequence's kv_offset in one flat table, or row b of
  // per-request tables [B, max_pages])
  int64_t qrow, koff, L, pt;
  if (seqs) {
    const DecodeSeq sq = seqs[b];
    qrow = sq.q_row;
    koff = Q8 ? 0 : sq.kv_offset;
    pt = Q8 ? sq.kv_offset : 0;
    L = sq.kv_len;
  } else {
    qrow = b;
    koff = Q8 ? 0 : kv_offset[b];
    pt = int64_t(b) * max_pages;
    L = kv_len[b];
  }
  const int lane = threadIdx.x & 63;
  const int kh = int(wave_uniform(threadIdx.x >> 6));  // key half of every block (scalar: uniform loops)
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  uint16_t* dst = o + qrow * o_stride + int64_t(g) * G * D;
  if (L < 1 || L > max_len) {  // outside what the caller sized: NaN, as the device cannot return an error
    for (int i = threadIdx.x; i < G * D; i += NT) dst[i] = 0x7FC0;
    return;
  }
  const int t = int(L - 1);            // the query's position
  const int nblk = t / KB + 1;         // blocks 0 .. t / 64
  const int nb = (kh == 1 && t % KB < 32) ? nblk - 1 : nblk;  // blocks this half visits

  const int64_t row_stride = int64_t(Hkv) * D;
  const uint32_t row_bytes = uint32_t(row_stride) * 2;
  const uint16_t* kbase = static_cast<const uint16_t*>(k_all) + koff * row_stride + g * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(v_all) + koff * row_stride + g * D;
  const uint32_t lane_off = uint32_t(grp) * row_bytes + uint32_t(l16) * LD * 2;

  // ---- query: the G heads of kv head g, through LDS
  {
    uint32_t qv[4];
    buf_ld_stream<4>(buf_rsrc(q + qrow * q_stride + g * G * D, G * D * 2), threadIdx.x * 16, qv);
    if (threadIdx.x < G * D / 8) *reinterpret_cast<uint4*>(s_q + threadIdx.x * 8) = make_uint4(qv[0], qv[1], qv[2], qv[3]);
  }
  __syncthreads();

  // lane's keys of block blk: 64 blk + 32 kh + 4 it + grp, it = 0..7, dims LD l16 .. + LD
  uint32_t kw[8][NDW], vw[8][NDW], nkw[8][NDW], nvw[8][NDW];
  auto load = [&](uint32_t (&kd)[8][NDW], uint32_t (&vd)[8][NDW], int blk) {
    const int64_t first = int64_t(blk) * KB + 32 * kh;
    const int64_t left = L - first;
    const uint32_t nv = uint32_t(left <= 0 ? 0 : (left < 32 ? left : 32));
    const __amdgpu_buffer_rsrc_t krs = buf_rsrc(wave_uniform(kbase + first * row_stride), wave_uniform(nv * row_bytes));
    const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(wave_uniform(vbase + first * row_stride), wave_uniform(nv * row_bytes));
#pragma unroll
    for (int it = 0; it < 8; ++it) buf_ld_stream<NDW>(krs, lane_off + uint32_t(4 * it) * row_bytes, kd[it]);
#pragma unroll
    for (int it = 0; it < 8; ++it) buf_ld_stream<NDW>(vrs, lane_off + uint32_t(4 * it) * row_bytes, vd[it]);
  };
  // int8 paged cache: LD codes per key (NQ dwords) and the key's scale; block blk is page
  // block_tables[b][blk], rows page * 64 .. + 63 of the pool
  constexpr int NQ = LD / 4;
  const int32_t* bt = block_tables + pt;
  const uint32_t qlane_off = uint32_t(grp) * uint32_t(row_stride) + uint32_t(l16) * LD;
  auto load_q = [&](uint32_t (&kd)[8][NQ], float& ks, uint32_t (&vd)[8][NQ], float& vs, int blk) {
    const int64_t first = int64_t(blk) * KB + 32 * kh;
    const int64_t left = L - first;
    const uint32_t nv = uint32_t(left <= 0 ? 0 : (left < 32 ? left : 32));
    // past the keys: any real page, nothing read; an index outside the pool is clamped into it
    int64_t page = bt[min(blk, nblk - 1)];
    page = page < 0 ? 0 : (page >= n_pages ? n_pages - 1 : page);
    const int64_t prow = page * KB + 32 * kh;
    const int8_t* kb8 = static_cast<const int8_t*>(k_all) + prow * row_stride + g * D;
    const int8_t* vb8 = static_cast<const int8_t*>(v_all) + prow * row_stride + g * D;
    const __amdgpu_buffer_rsrc_t krs = buf_rsrc(wave_uniform(reinterpret_cast<const uint16_t*>(kb8)),
                                                wave_uniform(nv * uint32_t(row_stride)));
    const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(wave_uniform(reinterpret_cast<const uint16_t*>(vb8)),
                                                wave_uniform(nv * uint32_t(row_stride)));
    const __amdgpu_buffer_rsrc_t kss = buf_rsrc(wave_uniform(reinterpret_cast<const uint16_t*>(k_scale + prow * Hkv + g)),
                                                wave_uniform(nv * uint32_t(Hkv) * 4));
    const __amdgpu_buffer_rsrc_t vss = buf_rsrc(wave_uniform(reinterpret_cast<const uint16_t*>(v_scale + prow * Hkv + g)),
                                                wave_uniform(nv * uint32_t(Hkv) * 4));
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const uint32_t off = qlane_off + uint32_t(4 * it) * uint32_t(row_stride);
      if constexpr (NQ == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(krs, int(off), 0, 2);
        kd[it][0] = v[0];
        kd[it][1] = v[1];
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(vrs, int(off), 0, 2);
        vd[it][0] = w[0];
        vd[it][1] = w[1];
      } else {
        kd[it][0] = __builtin_amdgcn_raw_buffer_load_b32(krs, int(off), 0, 2);
        vd[it][0] = __builtin_amdgcn_raw_buffer_load_b32(vrs, int(off), 0, 2);
      }
    }
    // lane holds the scale of key (lane mod 32) of the half; the lanes that need it read it by a shuffle
    const uint32_t soff = uint32_t(lane & 31) * uint32_t(Hkv) * 4;
    ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kss, int(soff), 0, 0));
    vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vss, int(soff), 0, 0));
  };
  // bf16(float(code) * scale): code b of a dword
  auto dq = [](uint32_t w, int b, float sc) { return float(int8_t(w >> (8 * b))) * sc; };

  f32x4 oacc[LD];
#pragma unroll
  for (int e = 0; e < LD; ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  uint16_t* sk = s_k[kh];
  const int rr = 4 * (l16 & 3) + (l16 >> 2);  // K tile row read as MFMA row l16

  // per block, in two stages: scores (K tile through LDS, S = K Q^T on MFMA), then the
  // online softmax and value product of this wave's half.  The int8 loop runs the scores
  // of block j + 1 beside the softmax and P V of block j (independent work the scheduler
  // can interleave), with three register sets in rotation so block j + 2's loads are in
  // flight meanwhile.  Every block's operations and their order are the same either way.
  // kword(it, c): dword c (two bf16) of key it's K slice; vpair(jj, e): dim e of keys 2 jj, 2 jj + 1
  auto scores = [&](auto&& kword, f32x4 (&sacc)[2]) {
      // ---- scores: two 16-key tiles; tile row 4 j + grp holds key 4 (4 kb + j) + grp, so
      // output register r of lane (head l16, grp) is key 4 (4 kb + r) + grp
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 4 * j + grp;
          const int it = 4 * kb + j;
          if constexpr (NDW == 4) {
            const int phys = l16 ^ (kr & (NG - 1));
            *reinterpret_cast<uint4*>(sk + kr * D + phys * 8) =
                make_uint4(kword(it, 0), kword(it, 1), kword(it, 2), kword(it, 3));
          } else {
            const int phys = (l16 >> 1) ^ (kr & (NG - 1));
            *reinterpret_cast<uint2*>(sk + kr * D + phys * 8 + (l16 & 1) * 4) = make_uint2(kword(it, 0), kword(it, 1));
          }
        }
        sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int phys = (4 * ks + grp) ^ (rr & (NG - 1));
          const uint4 a = *reinterpret_cast<const uint4*>(sk + rr * D + phys * 8);
          const uint4 qq = l16 < G ? *reinterpret_cast<const uint4*>(s_q + l16 * D + 32 * ks + 8 * grp)
                                   : make_uint4(0, 0, 0, 0);
          sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qq), sacc[kb], 0, 0, 0);
        }
      }
  };
  auto soft_pv = [&](const f32x4 (&sacc)[2], auto&& vpair, int blk) {
      // ---- online softmax of this half (lane: head l16, class grp, j = 4 kb + r)
      const bool diag = blk == nblk - 1;
      const int key0 = blk * KB + 32 * kh + grp;
      float p[8];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = sacc[j >> 2][j & 3];
        if (diag && key0 + 4 * j > t) v = -INFINITY;
        p[j] = v;
        mx = fmaxf(mx, v);
      }
      // the largest scaled score: scaling by a positive constant keeps the order
      mx = max_x32(max_x16(mx)) * sscale;
      const bool lift = mx > m_run + 8.0f;
      const float m_new = lift ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(p[j], sscale, -m_new));
      float cs = p[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) cs += p[j];
      const float tc = cs + __shfl_xor(cs, 32, 64);      // c0 + c2, c1 + c3
      const float rs = tc + __shfl_xor(tc, 16, 64);      // (c0 + c2) + (c1 + c3)
      l_run = __builtin_fmaf(l_run, alpha, rs);
      // O's rows are heads 4 grp + r: each takes its own head's alpha (held by lane 4 grp + r).
      // Skipped, exactly, when every alpha of the wave is 1 (no reference maximum moved).
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(alpha, 4 * grp + r, 64);
#pragma unroll
          for (int e = 0; e < LD; ++e) oacc[e][r] *= ar;
        }
      }
      // ---- O += P V: A = P (row head l16, k-slots 8 grp + j = class grp), B = V (col dim
      // LD l16 + e, same keys from the lane's own token-major registers)
      uint32_t h4[4], w4[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t hp = pack2bf(p[2 * jj], p[2 * jj + 1]);
        h4[jj] = hp;
        w4[jj] = pack2bf(p[2 * jj] - bf2f_lo(hp), p[2 * jj + 1] - bf2f_hi(hp));
      }
      const bf16x8 ph = as_bf16x8(make_uint4(h4[0], h4[1], h4[2], h4[3]));
      const bf16x8 pl = as_bf16x8(make_uint4(w4[0], w4[1], w4[2], w4[3]));
#pragma unroll
      for (int e = 0; e < LD; ++e) {
        const bf16x8 vb = as_bf16x8(make_uint4(vpair(0, e), vpair(1, e), vpair(2, e), vpair(3, e)));
        oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, oacc[e], 0, 0, 0);
        oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, oacc[e], 0, 0, 0);
      }
  };

  // past the request's keys the loads read zeros (bf16) or nothing (int8); the int8 loop
  // computes the scores of the block after the last and never uses them
  if constexpr (!Q8) {
    // bf16: two register sets, alternating, each block's scores then its softmax and P V
    uint32_t kw[8][NDW], vw[8][NDW], nkw[8][NDW], nvw[8][NDW];
    auto run = [&](const uint32_t (&kd)[8][NDW], const uint32_t (&vd)[8][NDW], int blk) {
      f32x4 sa[2];
      scores([&](int it, int c) { return kd[it][c]; }, sa);
      soft_pv(sa,
              [&](int jj, int e) {
                return __builtin_amdgcn_perm(vd[2 * jj + 1][e >> 1], vd[2 * jj][e >> 1],
                                             (e & 1) ? 0x07060302u : 0x05040100u);
              },
              blk);
    };
    if (nb > 0) load(kw, vw, 0);
    for (int blk = 0; blk < nb; blk += 2) {
      load(nkw, nvw, blk + 1);
      run(kw, vw, blk);
      if (blk + 1 >= nb) break;
      load(kw, vw, blk + 2);
      run(nkw, nvw, blk + 1);
    }
  } else {
    // int8 codes dequantised where they are consumed: K while the K tile is written, V while
    // the value operand is built (the same bf16(float(code) * scale) values throughout)
    uint32_t k0[8][NQ], v0[8][NQ], k1[8][NQ], v1[8][NQ], k2[8][NQ], v2[8][NQ];
    float ks0 = 0.f, vs0 = 0.f, ks1 = 0.f, vs1 = 0.f, ks2 = 0.f, vs2 = 0.f;
    f32x4 s0[2], s1[2], s2[2];
    auto sc = [&](const uint32_t (&kd)[8][NQ], float ksr, f32x4 (&sa)[2]) {
      float ks[8];
#pragma unroll
      for (int it = 0; it < 8; ++it) ks[it] = __shfl(ksr, 4 * it + grp, 64);
      scores([&](int it, int c) {
               const uint32_t w = kd[it][c >> 1];
               const int b0 = 2 * (c & 1);
               return pack2bf(dq(w, b0, ks[it]), dq(w, b0 + 1, ks[it]));
             },
             sa);
    };
    auto sp = [&](const f32x4 (&sa)[2], const uint32_t (&vd)[8][NQ], float vsr, int blk) {
      float vs[8];
#pragma unroll
      for (int it = 0; it < 8; ++it) vs[it] = __shfl(vsr, 4 * it + grp, 64);
      soft_pv(sa,
              [&](int jj, int e) {
                return pack2bf(dq(vd[2 * jj][e >> 2], e & 3, vs[2 * jj]),
                               dq(vd[2 * jj + 1][e >> 2], e & 3, vs[2 * jj + 1]));
              },
              blk);
    };
    if (nb > 0) {
      load_q(k0, ks0, v0, vs0, 0);
      load_q(k1, ks1, v1, vs1, 1);
      sc(k0, ks0, s0);
      for (int blk = 0;; blk += 3) {
        load_q(k2, ks2, v2, vs2, blk + 2);
        sc(k1, ks1, s1);
        sp(s0, v0, vs0, blk);
        if (blk + 1 >= nb) break;
        load_q(k0, ks0, v0, vs0, blk + 3);
        sc(k2, ks2, s2);
        sp(s1, v1, vs1, blk + 1);
        if (blk + 2 >= nb) break;
        load_q(k1, ks1, v1, vs1, blk + 4);
        sc(k0, ks0, s0);
        sp(s2, v2, vs2, blk + 2);
        if (blk + 3 >= nb) break;
      }
    }
  }

  // ---- merge the halves (half 0, then half 1).  Lane (l16, grp) holds O of heads
  // 4 grp + r, dims LD l16 + e; its own softmax state is head l16's.
  if (grp == 0 && l16 < G) {
    s_ml[kh][0][l16] = m_run;
    s_ml[kh][1][l16] = l_run;
  }
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * grp + r < G)
#pragma unroll
        for (int e = 0; e < LD; ++e) s_o[(4 * grp + r) * D + LD * l16 + e] = oacc[e][r];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * grp + r;
      if (h < G) {
        const float m0 = s_ml[0][0][h], l0 = s_ml[0][1][h];
        const float m1 = s_ml[1][0][h], l1 = s_ml[1][1][h];
        const float mm = fmaxf(m0, m1);
        const float a0 = __builtin_amdgcn_exp2f(m0 - mm);
        const float a1 = __builtin_amdgcn_exp2f(m1 - mm);
        const float inv = 1.0f / __builtin_fmaf(l0, a0, l1 * a1);
        float ov[LD];
#pragma unroll
        for (int e = 0; e < LD; ++e) ov[e] = __builtin_fmaf(oacc[e][r], a0, s_o[h * D + LD * l16 + e] * a1) * inv;
        uint16_t* dh = dst + h * D + LD * l16;
        if constexpr (LD == 8)
          *reinterpret_cast<uint4*>(dh) = make_uint4(pack2bf(ov[0], ov[1]), pack2bf(ov[2], ov[3]),
                                                     pack2bf(ov[4], ov[5]), pack2bf(ov[6], ov[7]));
        else
          *reinterpret_cast<uint2*>(dh) = make_uint2(pack2bf(ov[0], ov[1]), pack2bf(ov[2], ov[3]));
      }
    }
  }
}

#define BI_DPO_PARAMS                                                                                     \
  const uint16_t *__restrict__ q, int64_t q_stride, const void *__restrict__ k_all,                         \
      const void *__restrict__ v_all, const float *__restrict__ k_scale, const float *__restrict__ v_scale,  \
      const int32_t *__restrict__ block_tables, int max_pages, int64_t n_pages,                             \
      const DecodeSeq *__restrict__ seqs, const int64_t *__restrict__ kv_offset,                            \
      const int32_t *__restrict__ kv_len, const int32_t *__restrict__ order, int B, int Hkv,                \
      int64_t max_len, float sscale, uint16_t *__restrict__ o, int64_t o_stride
#define BI_DPO_ARGS                                                                                       \
  q, q_stride, k_all, v_all, k_scale, v_scale, block_tables, max_pages, n_pages, seqs, kv_offset, kv_len,   \
      order, B, Hkv, max_len, sscale, o, o_stride

template <int D, int G>
__global__ __launch_bounds__(NT) void decode_po_kernel(BI_DPO_PARAMS) {
  decode_po_body<D, G, false>(BI_DPO_ARGS);
}

// The int8 kernel is held to two waves per SIMD (at most 256 registers): left free, the
// compiler takes over 300 for the three rotating register sets and runs one wave per SIMD,
// about a quarter slower; at two waves it needs no spills.
template <int D, int G>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_po_q8_kernel(
    BI_DPO_PARAMS) {
  decode_po_body<D, G, true>(BI_DPO_ARGS);
}
#undef BI_DPO_PARAMS
#undef BI_DPO_ARGS

template <int D, int G, bool Q8>
hipError_t launch_t(const uint16_t* q, int64_t q_stride, const void* k_all, const void* v_all, const float* ks,
                    const float* vs, const int32_t* bt, int max_pages, int64_t n_pages, const DecodeSeq* seqs,
                    const int64_t* kv_offset, const int32_t* kv_len, const int32_t* order, int B, int64_t max_len,
                    int Hkv, float sscale, uint16_t* o, int64_t o_stride, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if constexpr (Q8)
    hipLaunchKernelGGL((decode_po_q8_kernel<D, G>), dim3(8 * Hkv, (B + 7) / 8), dim3(NT), 0, s, q, q_stride, k_all,
                       v_all, ks, vs, bt, max_pages, n_pages, seqs, kv_offset, kv_len, order, B, Hkv, max_len, sscale,
                       o, o_stride);
  else
    hipLaunchKernelGGL((decode_po_kernel<D, G>), dim3(Hkv, B), dim3(NT), 0, s, q, q_stride, k_all, v_all, ks, vs, bt,
                       max_pages, n_pages, seqs, kv_offset, kv_len, order, B, Hkv, max_len, sscale, o, o_stride);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_decode_po(const uint16_t* q, int64_t q_row_stride, const uint16_t* k_all,
                                 const uint16_t* v_all, const DecodeSeq* d_seqs, const int64_t* kv_offset,
                                 const int32_t* kv_len, const int32_t* d_order, int B, int64_t max_kv_len,
                                 int Hq, int Hkv, int D, float scale, uint16_t* o, int64_t o_row_stride,
                                 hipStream_t s) {
  const float sscale = scale * 1.4426950408889634f;  // scores in log2 units, as prefill
  const int G = Hq / Hkv;
#define BI_DPO(DD, GG)                                                                                         \
  if (D == DD && G == GG)                                                                                    \
    return launch_t<DD, GG, false>(q, q_row_stride, k_all, v_all, nullptr, nullptr, nullptr, 0, 0, d_seqs,      \
                                   kv_offset, kv_len, d_order, B, max_kv_len, Hkv, sscale, o, o_row_stride, s);
  BI_DPO(64, 1) BI_DPO(64, 2) BI_DPO(64, 4) BI_DPO(64, 8)
  BI_DPO(128, 1) BI_DPO(128, 2) BI_DPO(128, 4) BI_DPO(128, 8)
#undef BI_DPO
  return hipErrorInvalidValue;
}

hipError_t launch_attn_decode_po_q8(const uint16_t* q, int64_t q_row_stride, const int8_t* k_pool,
                                    const int8_t* v_pool, const float* k_scale, const float* v_scale,
                                    const int32_t* block_tables, int max_pages, int64_t n_pages,
                                    const DecodeSeq* d_seqs, const int32_t* kv_len, const int32_t* d_order, int B,
                                    int64_t max_kv_len, int Hq, int Hkv, int D, float scale, uint16_t* o,
                                    int64_t o_row_stride, hipStream_t s) {
  const float sscale = scale * 1.4426950408889634f;
  const int G = Hq / Hkv;
#define BI_DPO(DD, GG)                                                                                          \
  if (D == DD && G == GG)                                                                                     \
    return launch_t<DD, GG, true>(q, q_row_stride, k_pool, v_pool, k_scale, v_scale, block_tables, max_pages,     \
                                  n_pages, d_seqs, nullptr, kv_len, d_order, B, max_kv_len, Hkv, sscale, o,      \
                                  o_row_stride, s);
  BI_DPO(64, 1) BI_DPO(64, 2) BI_DPO(64, 4) BI_DPO(64, 8)
  BI_DPO(128, 1) BI_DPO(128, 2) BI_DPO(128, 4) BI_DPO(128, 8)
#undef BI_DPO
  return hipErrorInvalidValue;
}

}  // namespace bi
