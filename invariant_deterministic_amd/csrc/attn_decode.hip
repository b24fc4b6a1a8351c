// Decode attention with a fixed key/value split size for gfx950.
//
// The M-0002 record ("Deterministic and bit-exact inference", field
// `technical`) makes attention batch-invariant by splitting the key/value
// axis into pieces of a fixed *size* rather than into a fixed *number* of
// pieces.  Here the piece is 256 keys: request b with L_b keys has
// ceil(L_b / 256) units, unit s covering keys [256 s, min(256 s + 256, L_b)).
// The pieces are reduced and merged in a tree whose shape depends only on
// L_b: each unit on its own, then runs of 8 consecutive units (units
// 8 r .. 8 r + 7 form run r) merged in ascending unit order, then the runs
// merged in ascending order.  A request's bits therefore never depend on the
// batch, the other requests' lengths, the launch order or the grid.
//
// Unit kernel: one 2-wave work-group per (run r of request b, kv head g), for
// the G query heads sharing kv head g (the block entry point passes a
// host-built list of the step's runs, those with the most units first; the
// standalone one builds the same list on the device).  A unit is 4 blocks of
// 64 keys; wave kh takes keys 32 kh .. 32 kh + 31 of every block.
//   loads   token-major: a lane takes 16 bytes (D/16 dims) of one key row, so
//           each load instruction covers four whole head rows; raw buffer
//           loads bounded at the request's last key read zero past it, with no
//           branch.  Two register sets alternate, so the next block (also
//           across a unit's end) is in flight while one is reduced.
//   scores  S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (D/32 k-steps in ascending
//           order), K passed through a per-wave LDS tile of 16 keys to reach
//           the operand layout, times scale * log2(e); keys past L_b -inf.
//   softmax online per wave over its 32-key halves, from a fresh state at each
//           unit: the reference maximum m moves only when a block's maximum
//           exceeds it by more than 8; alpha = exp2(m - m_new), p = exp2(score
//           - m_new), l = fma(l, alpha, rowsum) with the rowsum in a fixed
//           in-lane and lane-pair order, O *= alpha (each output row by its
//           own head's alpha);
//   o       P V on v_mfma_f32_16x16x32_bf16: the value operand is the lane's
//           own token-major registers regrouped by byte permutes (eight keys
//           of one dim), P enters as a bf16 high part plus a bf16 remainder.
//   unit    the halves merge through LDS: m = max(m0, m1), a_i = exp2(m_i -
//           m), l = fma(l0, a0, l1 a1), o = fma(O0, a0, O1 a1); the unit's
//           (m, l, o) stays in LDS.
//   run     at the run's end its units merge in ascending order with the
//           formula below; the run's (m, l, o[D]) goes to the workspace in
//           fp32 (one record per 2048 keys and head: partial sums are a small
//           fraction of the bytes moved, which keeps HBM on the key/value
//           stream).
// Merge of pieces 0 .. S - 1 (units of a run, then runs of a request):
// M = max m_s; w_s = exp2(m_s - M); O = sum w_s o_s and Lsum = sum w_s l_s
// as fmas in ascending s.  The combine kernel, one thread per (request, head,
// dim), merges the runs and writes bf16(O / Lsum).
#include <mutex>

#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

constexpr int kSplit = kKvSplit;      // 256 keys per unit
constexpr int KB = 64;                // keys per block; a unit is 4 blocks
constexpr int kUnitBlocks = kSplit / KB;
constexpr int NT = 128;               // two waves: key halves

// One work-group per (run list entry blockIdx.x = (request b, first unit u0), kv head
// blockIdx.y); entries at or past *n_runs (when given) have nothing to do.
template <int D, int G>
__global__ __launch_bounds__(NT) void decode_unit_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_all,
    const uint16_t* __restrict__ v_all, const DecodeSeq* __restrict__ seqs,
    const int2* __restrict__ runs, const int* __restrict__ n_runs, int Hkv, int64_t max_len,
    int max_runs, float sscale, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  constexpr int LD = D / 16;  // dims per lane in the token-major loads
  constexpr int NDW = LD / 2;
  constexpr int KS = D / 32;  // MFMA k-steps over the head dimension
  constexpr int NG = D / 8;   // 16-byte granules per key row
  static_assert(G <= 8, "heads 4 grp + r of the value product cover at most 16");
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][16 * D];  // per-wave K tile
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G * D];
  __shared__ float s_o[2][G * D];      // half 1's O at a unit's end (two units alternate)
  __shared__ float s_ml[2][2][2][G];   // [unit parity][half][m, l][head]
  // the run's unit partials, merged at its end: head h, unit i of the run at
  // s_part[(h * kDecodeRun + i) * D ...], (m, l) at s_pml[(h * kDecodeRun + i) * 2 ...]
  __shared__ __attribute__((aligned(16))) float s_part[G * kDecodeRun * D];
  __shared__ float s_pml[G * kDecodeRun * 2];

  if (n_runs && int(blockIdx.x) >= *n_runs) return;
  const int2 run = runs[blockIdx.x];
  const int b = run.x;
  const int u0 = run.y;
  const int g = blockIdx.y;
  const DecodeSeq sq = seqs[b];
  const int64_t L = sq.kv_len;
  if (L < 1 || L > max_len) return;  // the combine kernel reports the request as NaN
  const int n_units = int((L + kSplit - 1) / kSplit);
  if (u0 < 0 || u0 >= n_units) return;
  const int nu = min(kDecodeRun, n_units - u0);
  const int lane = threadIdx.x & 63;
  const int kh = int(wave_uniform(threadIdx.x >> 6));  // key half of every block (scalar: uniform loops)
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int nblk = int((L + KB - 1) / KB);
  // blocks of this run for this half: half 1 has no key in a last block holding <= 32 keys
  const int blk0 = u0 * kUnitBlocks;
  const int blk_end = min((u0 + nu) * kUnitBlocks, nblk) - (kh == 1 && L - int64_t(nblk - 1) * KB <= 32 && (u0 + nu) * kUnitBlocks >= nblk ? 1 : 0);

  const int64_t row_stride = int64_t(Hkv) * D;
  const uint32_t row_bytes = uint32_t(row_stride) * 2;
  const uint16_t* kbase = k_all + sq.kv_offset * row_stride + g * D;
  const uint16_t* vbase = v_all + sq.kv_offset * row_stride + g * D;
  const uint32_t lane_off = uint32_t(grp) * row_bytes + uint32_t(l16) * LD * 2;

  {
    uint32_t qv[4];
    buf_ld_stream<4>(buf_rsrc(q + sq.q_row * q_stride + g * G * D, G * D * 2), threadIdx.x * 16, qv);
    if (threadIdx.x < G * D / 8) *reinterpret_cast<uint4*>(s_q + threadIdx.x * 8) = make_uint4(qv[0], qv[1], qv[2], qv[3]);
  }
  __syncthreads();

  // lane's keys of block blk: 64 blk + 32 kh + 4 it + grp, it = 0..7, dims LD l16 .. + LD
  uint32_t kw[8][NDW], vw[8][NDW], nkw[8][NDW], nvw[8][NDW];
  auto load = [&](uint32_t (&kd)[8][NDW], uint32_t (&vd)[8][NDW], int blk) {
    const int64_t first = int64_t(blk) * KB + 32 * kh;
    const int64_t left = (blk < blk_end ? L : 0) - first;  // nothing is read past the run
    const uint32_t nv = uint32_t(left <= 0 ? 0 : (left < 32 ? left : 32));
    const __amdgpu_buffer_rsrc_t krs = buf_rsrc(wave_uniform(kbase + first * row_stride), wave_uniform(nv * row_bytes));
    const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(wave_uniform(vbase + first * row_stride), wave_uniform(nv * row_bytes));
#pragma unroll
    for (int it = 0; it < 8; ++it) buf_ld_stream<NDW>(krs, lane_off + uint32_t(4 * it) * row_bytes, kd[it]);
#pragma unroll
    for (int it = 0; it < 8; ++it) buf_ld_stream<NDW>(vrs, lane_off + uint32_t(4 * it) * row_bytes, vd[it]);
  };

  f32x4 oacc[LD];
  float m_run, l_run;
  auto reset = [&] {
#pragma unroll
    for (int e = 0; e < LD; ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  };
  reset();
  uint16_t* sk = s_k[kh];
  const int rr = 4 * (l16 & 3) + (l16 >> 2);  // K tile row read as MFMA row l16

  // one block: scores, online softmax (reference maximum moves when the block maximum
  // exceeds it by more than 8) and value product of this wave's 32 keys
  auto process = [&](const uint32_t (&kd)[8][NDW], const uint32_t (&vd)[8][NDW], int blk) {
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kr = 4 * j + grp;
        const uint32_t* src = kd[4 * kb + j];
        if constexpr (NDW == 4) {
          const int phys = l16 ^ (kr & (NG - 1));
          *reinterpret_cast<uint4*>(sk + kr * D + phys * 8) = make_uint4(src[0], src[1], src[2], src[3]);
        } else {
          const int phys = (l16 >> 1) ^ (kr & (NG - 1));
          *reinterpret_cast<uint2*>(sk + kr * D + phys * 8 + (l16 & 1) * 4) = make_uint2(src[0], src[1]);
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
    const bool last = blk == nblk - 1;
    const int64_t key0 = int64_t(blk) * KB + 32 * kh + grp;
    float p[8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = sacc[j >> 2][j & 3] * sscale;
      if (last && key0 + 4 * j >= L) v = -INFINITY;
      p[j] = v;
      mx = fmaxf(mx, v);
    }
    mx = max_x32(max_x16(mx));
    const bool lift = mx > m_run + 8.0f;
    const float m_new = lift ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(p[j] - m_new);
    float cs = p[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) cs += p[j];
    const float tc = cs + __shfl_xor(cs, 32, 64);
    const float rs = tc + __shfl_xor(tc, 16, 64);
    l_run = __builtin_fmaf(l_run, alpha, rs);
    // O's rows are heads 4 grp + r, each scaled by its own head's alpha; skipped, exactly,
    // when every alpha of the wave is 1 (no reference maximum moved)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * grp + r, 64);
#pragma unroll
        for (int e = 0; e < LD; ++e) oacc[e][r] *= ar;
      }
    }
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
      uint32_t vt[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        vt[jj] = __builtin_amdgcn_perm(vd[2 * jj + 1][e >> 1], vd[2 * jj][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
      const bf16x8 vb = as_bf16x8(make_uint4(vt[0], vt[1], vt[2], vt[3]));
      oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, oacc[e], 0, 0, 0);
      oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, oacc[e], 0, 0, 0);
    }
  };

  // end of unit i of the run: merge the halves (half 0 first) into the unit's partial in
  // LDS, then reset.  Lane (l16, grp) holds O of heads 4 grp + r, dims LD l16 + e.  Half 1's
  // state alternates between two buffers, so one barrier per unit suffices: half 1 writes
  // buffer i & 1 again only after the next unit's barrier, which half 0 passes after reading it.
  auto finish_unit = [&](int i) {
    const int pb = i & 1;
    if (grp == 0 && l16 < G) {
      s_ml[pb][kh][0][l16] = m_run;
      s_ml[pb][kh][1][l16] = l_run;
    }
    if (kh == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * grp + r < G)
#pragma unroll
          for (int e = 0; e < LD; ++e) s_o[pb][(4 * grp + r) * D + LD * l16 + e] = oacc[e][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * grp + r;
        if (h < G) {
          const float m0 = s_ml[pb][0][0][h], l0 = s_ml[pb][0][1][h];
          const float m1 = s_ml[pb][1][0][h], l1 = s_ml[pb][1][1][h];
          const float mm = fmaxf(m0, m1);
          const float a0 = __builtin_amdgcn_exp2f(m0 - mm);
          const float a1 = __builtin_amdgcn_exp2f(m1 - mm);
          float ov[LD];
#pragma unroll
          for (int e = 0; e < LD; ++e) ov[e] = __builtin_fmaf(oacc[e][r], a0, s_o[pb][h * D + LD * l16 + e] * a1);
          float* dst = s_part + (h * kDecodeRun + i) * D + LD * l16;
#pragma unroll
          for (int e = 0; e < LD; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(ov[e], ov[e + 1], ov[e + 2], ov[e + 3]);
          if (l16 == 0) {
            s_pml[(h * kDecodeRun + i) * 2 + 0] = mm;
            s_pml[(h * kDecodeRun + i) * 2 + 1] = __builtin_fmaf(l0, a0, l1 * a1);
          }
        }
      }
    }
    reset();
  };

  // the run's units in order; within a unit its (at most 4) blocks, two register sets
  // alternating so the next block is in flight while one is processed.  A full unit has an
  // even number of blocks, so every unit starts in the first set and the last load of a unit
  // already brings the next unit's first block.  Both waves finish every unit (a half with no
  // block in the run's last unit finishes it with an empty state).
  if (blk0 < blk_end) load(kw, vw, blk0);
  for (int i = 0; i < nu; ++i) {
    const int ub = blk0 + kUnitBlocks * i;
    const int ue = min(ub + kUnitBlocks, blk_end);
    for (int blk = ub; blk < ue; blk += 2) {
      load(nkw, nvw, blk + 1);  // past the run's blocks this reads nothing
      process(kw, vw, blk);
      if (blk + 1 >= ue) break;
      load(kw, vw, blk + 2);
      process(nkw, nvw, blk + 1);
    }
    finish_unit(i);
  }
  // the run's record: its units merged in ascending order (thread x: head x / D, dim x % D)
  __syncthreads();
  const int Hq = Hkv * G;
  const int r = u0 / kDecodeRun;
  for (int x = threadIdx.x; x < G * D; x += NT) {
    const int h = x / D, d = x % D;
    const float* pml = s_pml + h * kDecodeRun * 2;
    const float* po = s_part + h * kDecodeRun * D + d;
    float M = -INFINITY;
    for (int i = 0; i < nu; ++i) M = fmaxf(M, pml[2 * i]);
    float Lsum = 0.f, O = 0.f;
    for (int i = 0; i < nu; ++i) {
      const float w = __builtin_amdgcn_exp2f(pml[2 * i] - M);
      Lsum = __builtin_fmaf(w, pml[2 * i + 1], Lsum);
      O = __builtin_fmaf(w, po[i * D], O);
    }
    const int64_t slot = (int64_t(b) * Hq + g * G + h) * max_runs + r;
    ws_o[slot * D + d] = O;
    if (d == 0) {
      ws_ml[slot * 2 + 0] = M;
      ws_ml[slot * 2 + 1] = Lsum;
    }
  }
}

// number of runs of a request with L keys
__device__ __host__ inline int runs_of(int64_t L) {
  const int64_t units = (L + kSplit - 1) / kSplit;
  return int((units + kDecodeRun - 1) / kDecodeRun);
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    const DecodeSeq* __restrict__ seqs, int Hq, int max_runs, int64_t max_len,
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
  const int S = runs_of(L);
  const int64_t base = (int64_t(b) * Hq + h) * max_runs;
  float M = -INFINITY;
#pragma unroll 4
  for (int s = 0; s < S; ++s) M = fmaxf(M, ws_ml[(base + s) * 2]);
  float Lsum = 0.f, O = 0.f;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float w = __builtin_amdgcn_exp2f(ws_ml[(base + s) * 2] - M);
    Lsum = __builtin_fmaf(w, ws_ml[(base + s) * 2 + 1], Lsum);
    O = __builtin_fmaf(w, ws_o[(base + s) * D + d], O);
  }
  *dst = f2bf(O / Lsum);
}

// Exclusive prefix sum over a 1024-thread work-group; `total` receives the sum.
// Exclusive prefix sum over a 1024-thread work-group (16 waves) of a 64-bit value; the
// work-group's total in `total`.  Packed fields add independently as long as no field's
// total overflows.
__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t v, uint64_t* s_w, uint64_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint64_t t = s_w[i];
    before += i < w ? t : 0;
    all += t;
  }
  __syncthreads();  // s_w is reused by the next scan
  total = all;
  return before + x - v;
}

// Standalone entry point's set-up, one 1024-thread work-group: packs the offset / length
// arrays into DecodeSeq and lists the runs (request, first unit) with the most units first
// (every full run in request order, then the last runs of 7, 6, .., 1 units, each in
// request order; the order the block entry point's host list has).  A request whose length
// is outside 1 .. max_len gets no run (the combine kernel writes NaN for it).  Counts of the
// seven partial-run classes travel packed in 16-bit fields of two 64-bit words (classes
// 1..4 and 5..7; no class holds more than B <= 65535 runs), full runs in a third word, so
// each pass takes three work-group scans; every thread keeps the class bases itself.
__global__ __launch_bounds__(1024) void decode_prep_kernel(const int64_t* __restrict__ kv_offset,
                                                           const int32_t* __restrict__ kv_len, int B,
                                                           int64_t max_len, DecodeSeq* __restrict__ seqs,
                                                           int2* __restrict__ runs, int* __restrict__ n_runs) {
  constexpr int R = kDecodeRun;
  static_assert(R == 8, "seven partial-run classes, packed four and three per word");
  __shared__ uint64_t s_w[16];
  auto units = [&](int b) -> int {
    const int64_t L = kv_len[b];
    return (L >= 1 && L <= max_len) ? int((L + kSplit - 1) / kSplit) : 0;
  };
  auto field = [](int p) -> uint64_t { return uint64_t(1) << (16 * ((p - 1) & 3)); };
  auto count = [](uint64_t lo, uint64_t hi, int k) -> int {  // class k = 1 .. 7
    return int(((k <= 4 ? lo : hi) >> (16 * ((k - 1) & 3))) & 0xFFFF);
  };
  // pass 1: runs per class
  uint64_t lo = 0, hi = 0, full = 0;
  for (int b = threadIdx.x; b < B; b += 1024) {
    const int U = units(b);
    full += uint64_t(U / R);
    const int p = U % R;
    if (p) (p <= 4 ? lo : hi) += field(p);
  }
  uint64_t t_lo, t_hi, t_full;
  block_exclusive_scan(lo, s_w, t_lo);
  block_exclusive_scan(hi, s_w, t_hi);
  block_exclusive_scan(full, s_w, t_full);
  // bases: full runs first, then the classes 7, 6, .., 1
  int base[R + 1];
  base[R] = 0;
  int at = int(t_full);
#pragma unroll
  for (int k = R - 1; k >= 1; --k) {
    base[k] = at;
    at += count(t_lo, t_hi, k);
  }
  if (threadIdx.x == 0) *n_runs = at;
  // pass 2: positions, 1024 requests at a time in request order
  for (int c = 0; c < B; c += 1024) {
    const int b = c + int(threadIdx.x);
    int U = 0;
    if (b < B) {
      DecodeSeq sq;
      sq.q_row = b;
      sq.kv_offset = kv_offset[b];
      sq.kv_len = kv_len[b];
      sq.pad = 0;
      seqs[b] = sq;
      U = units(b);
    }
    const int f = U / R, p = U % R;
    uint64_t c_lo, c_hi, c_full;
    const uint64_t x_lo = block_exclusive_scan(p >= 1 && p <= 4 ? field(p) : 0, s_w, c_lo);
    const uint64_t x_hi = block_exclusive_scan(p >= 5 ? field(p) : 0, s_w, c_hi);
    const uint64_t x_full = block_exclusive_scan(uint64_t(f), s_w, c_full);
    for (int i = 0; i < f; ++i) runs[base[R] + int(x_full) + i] = make_int2(b, i * R);
    int bp = 0;  // base of class p (a select chain: no runtime index into base[])
#pragma unroll
    for (int k = 1; k < R; ++k) bp = p == k ? base[k] : bp;
    if (p) runs[bp + count(x_lo, x_hi, p)] = make_int2(b, f * R);
    base[R] += int(c_full);
#pragma unroll
    for (int k = 1; k < R; ++k) base[k] += count(c_lo, c_hi, k);
  }
}

template <int D, int G>
hipError_t launch_units(const uint16_t* q, int64_t q_stride, const uint16_t* k_all, const uint16_t* v_all,
                        const DecodeSeq* seqs, const int2* runs, const int* n_runs, int grid_runs, int64_t max_len,
                        int max_runs, int Hkv, float sscale, float* ws_o, float* ws_ml, hipStream_t s) {
  if (grid_runs <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_unit_kernel<D, G>), dim3(grid_runs, Hkv), dim3(NT), 0, s, q, q_stride, k_all, v_all,
                     seqs, runs, n_runs, Hkv, max_len, max_runs, sscale, ws_o, ws_ml);
  return hipGetLastError();
}

struct WsParts {
  float* o;
  float* ml;
  DecodeSeq* seqs;
  int2* runs;
  int* n_runs;
};

}  // namespace

// Workspace: ws_o [B][Hq][R][D] fp32 and ws_ml [B][Hq][R][2] fp32 (R = runs of the
// longest request), then for the standalone entry point the packed DecodeSeq array,
// the run list (B R pairs at most) and its length; 256-byte aligned parts.
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static int max_runs_of(int64_t max_kv_len) { return runs_of(max_kv_len); }

static WsParts ws_parts(void* ws, int B, int64_t max_kv_len, int Hq, int D, size_t* total) {
  const size_t R = size_t(max_runs_of(max_kv_len));
  const size_t slots = size_t(B) * Hq * R;
  char* p = static_cast<char*>(ws);
  size_t off = 0;
  WsParts w;
  w.o = reinterpret_cast<float*>(p + off);
  off += align256(slots * D * 4);
  w.ml = reinterpret_cast<float*>(p + off);
  off += align256(slots * 2 * 4);
  w.seqs = reinterpret_cast<DecodeSeq*>(p + off);
  off += align256(size_t(B) * sizeof(DecodeSeq));
  w.runs = reinterpret_cast<int2*>(p + off);
  off += align256(size_t(B) * R * sizeof(int2));
  w.n_runs = reinterpret_cast<int*>(p + off);
  off += 256;
  if (total) *total = off;
  return w;
}

size_t decode_workspace_bytes(int B, int64_t max_kv_len, int Hq, int D) {
  size_t total = 0;
  ws_parts(nullptr, B, max_kv_len, Hq, D, &total);
  return total;
}

static hipError_t run_decode(const uint16_t* q, int64_t q_row_stride, const uint16_t* k_all, const uint16_t* v_all,
                             const DecodeSeq* d_seqs, const int2* d_runs, const int* d_n_runs, int grid_runs, int B,
                             int64_t max_kv_len, int Hq, int Hkv, int D, float scale, const WsParts& w, uint16_t* o,
                             int64_t o_row_stride, hipStream_t s) {
  const int max_runs = max_runs_of(max_kv_len);
  const float qscale = scale * 1.4426950408889634f;  // scores in log2 units (as prefill)
  const int G = Hq / Hkv;
  hipError_t e = hipErrorInvalidValue;
#define BI_DEC(DD, GG)                                                                                 \
  if (D == DD && G == GG)                                                                            \
    e = launch_units<DD, GG>(q, q_row_stride, k_all, v_all, d_seqs, d_runs, d_n_runs, grid_runs, max_kv_len, \
                             max_runs, Hkv, qscale, w.o, w.ml, s);
  BI_DEC(64, 1) BI_DEC(64, 2) BI_DEC(64, 4) BI_DEC(64, 8)
  BI_DEC(128, 1) BI_DEC(128, 2) BI_DEC(128, 4) BI_DEC(128, 8)
#undef BI_DEC
  if (e != hipSuccess) return e;
  if (D == 64)
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(Hq, B), dim3(64), 0, s, w.o, w.ml, d_seqs, Hq, max_runs,
                       max_kv_len, o, o_row_stride);
  else
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(Hq, B), dim3(128), 0, s, w.o, w.ml, d_seqs, Hq, max_runs,
                       max_kv_len, o, o_row_stride);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const uint16_t* q, int64_t q_row_stride, const uint16_t* k_all,
                              const uint16_t* v_all, const DecodeSeq* d_seqs, const int2* d_runs,
                              int n_runs, int B, int64_t max_kv_len, int Hq, int Hkv, int D,
                              float scale, void* ws, uint16_t* o, int64_t o_row_stride,
                              hipStream_t s) {
  if (!d_runs) return hipErrorInvalidValue;
  const WsParts w = ws_parts(ws, B, max_kv_len, Hq, D, nullptr);
  return run_decode(q, q_row_stride, k_all, v_all, d_seqs, d_runs, nullptr, n_runs, B, max_kv_len, Hq, Hkv, D,
                    scale, w, o, o_row_stride, s);
}

// Scratch of the allocation-free decode entry point: a file-scope device array, one copy
// per GPU, held until the process ends.  In host code its name stands for no device
// address: kernels get the address hipGetSymbolAddress returns for the current device,
// looked up once per device and kept in scratch_dev.  Every call on a GPU shares that
// GPU's copy (calls that overlap on one GPU race on it).  Nothing in it has to start at
// zero: the list kernel writes the run count and list, the unit kernel every partial the
// combine kernel reads, all within the call.
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};
}  // namespace

static hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_attn_decode_noalloc(const uint16_t* q, const uint16_t* k_all, const uint16_t* v_all,
                                      const int64_t* kv_offset, const int32_t* kv_len, int B, int64_t max_kv_len,
                                      int Hq, int Hkv, int D, float scale, uint16_t* o, hipStream_t s) {
  if (decode_workspace_bytes(B, max_kv_len, Hq, D) > kDecodeScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_attn_decode_arrays(q, k_all, v_all, kv_offset, kv_len, B, max_kv_len, Hq, Hkv, D, scale, ws, o, s);
}

hipError_t launch_attn_decode_arrays(const uint16_t* q, const uint16_t* k_all,
                                     const uint16_t* v_all, const int64_t* kv_offset,
                                     const int32_t* kv_len, int B, int64_t max_kv_len, int Hq,
                                     int Hkv, int D, float scale, void* ws, uint16_t* o,
                                     hipStream_t s) {
  const WsParts w = ws_parts(ws, B, max_kv_len, Hq, D, nullptr);
  hipLaunchKernelGGL(decode_prep_kernel, dim3(1), dim3(1024), 0, s, kv_offset, kv_len, B, max_kv_len, w.seqs,
                     w.runs, w.n_runs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t grid = int64_t(B) * max_runs_of(max_kv_len);  // bound on the list's length
  if (grid > (int64_t(1) << 24)) return hipErrorInvalidValue;  // grid x stays far below 2^32 threads
  return run_decode(q, int64_t(Hq) * D, k_all, v_all, w.seqs, w.runs, w.n_runs, int(grid), B, max_kv_len, Hq, Hkv,
                    D, scale, w, o, int64_t(Hq) * D, s);
}

}  // namespace bi
