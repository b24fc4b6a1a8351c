// The step after the block for gfx950: seeded sampling of the next token and
// BLAKE3 hashes of token ids.
//
// The "Receipts" page ("Making a receipt") records a request's sampler
// settings (temperature, top-k, top-p, min-p, repeat / presence / frequency
// penalties, seed) and its prompt and output token ids with their BLAKE3 over
// the ids as little-endian 32-bit integers; "What a receipt proves" promises
// the same output tokens for the same inputs within one device class and
// build.  Everything here is per row: a row's token depends only on its
// logits, its history, its seed and its position, never on the batch.
//
// Sampler (one 512-thread work-group per row):
//  1. penalties in fp32 for each distinct history token (repeat: l > 0 ->
//     l / r else l * r; then l - (presence + count * frequency)), written with
//     contraction off so no fused multiply-add changes a rounding;
//  2. candidates: the K' = top_k + (distinct history tokens) largest
//     unpenalised bf16 logits, ordered by (logit desc, id asc), found by a
//     16-way search over the 16-bit order keys (four counting passes with
//     integer sums, no atomics) and a compaction in id order (waves own
//     contiguous ranges; lane prefix sums place each hit, so equal keys are
//     taken lowest id first); the union with every history token at its
//     penalised value holds the top_k penalised logits;
//  3. bitonic sort of the union by (logit desc, id asc); temperature 0 takes
//     the first (greedy);
//  4. otherwise, in fp64 for the first top_k: w = exp((l - l_0) / T), min-p
//     keeps w >= min_p, top-p keeps the shortest prefix whose running sum
//     reaches top_p times the total, and the token is the first whose running
//     sum exceeds u times the kept total, u from Philox4x64-10 with key
//     (seed, 0) and counter (position, 0, 0, 0) (Salmon et al., SC 2011).
//
// Token hash (one wave per sequence): BLAKE3 in hash mode.  Lanes compress
// the 1024-byte chunks in parallel (each chunk's 64-byte blocks in order);
// lane 0 then merges the chunk chaining values with the usual stack of
// subtree roots and finishes with the ROOT compression.
#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

// ------------------------------------------------------------------ sampler
constexpr int ST = 512;          // threads per row (8 waves)
constexpr int NWV = ST / 64;
constexpr int MAXC = 2048;       // candidate slots (top_k <= 1024, history <= 256 twice)

__device__ __forceinline__ uint32_t order_key(uint16_t bf) {
  if ((bf & 0x7FFFu) == 0) bf = 0;              // -0 sorts with +0
  return (bf & 0x8000u) ? uint32_t(uint16_t(~bf)) : uint32_t(bf | 0x8000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  const uint16_t bf = (k & 0x8000u) ? uint16_t(k & 0x7FFFu) : uint16_t(~k);
  return bf2f(bf);
}
// (a before b) when a's logit is larger, or equal with a smaller id
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ float penalised(float v, float r, float pr, float fr, float cnt) {
#pragma clang fp contract(off)
  v = v > 0.f ? v / r : v * r;
  const float sub = pr + cnt * fr;
  return v - sub;
}

__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
    const uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += 0x9E3779B97F4A7C15ull;
    k1 += 0xBB67AE8584CAA73Bull;
  }
}

__global__ __launch_bounds__(ST) void sample_kernel(const uint16_t* __restrict__ logits, int64_t vocab,
                                                    BiSampling prm, const uint64_t* __restrict__ seeds,
                                                    const int64_t* __restrict__ positions,
                                                    const int32_t* __restrict__ history, int n_hist,
                                                    int32_t* __restrict__ out) {
  __shared__ int s_htok[256];
  __shared__ float s_hval[256];
  __shared__ int s_hfirst[256];
  __shared__ int s_cnt[NWV][16];
  __shared__ int s_tot[16];
  __shared__ float s_ckey[MAXC];
  __shared__ int s_cidx[MAXC];
  __shared__ int s_scan[NWV];
  __shared__ int s_scan2[NWV];
  __shared__ double s_w[1024];
  __shared__ int s_nd;

  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const uint16_t* lr = logits + int64_t(row) * vocab;
  const int V = int(vocab);

  // ---- 1. history: distinct tokens and their penalised values
  if (t < n_hist) {
    int tok = history[int64_t(row) * n_hist + t];
    if (tok < 0 || tok >= V) tok = -1;  // ids outside the vocabulary are ignored
    s_htok[t] = tok;
  }
  __syncthreads();
  if (t < n_hist) {
    const int tok = s_htok[t];
    int first = tok >= 0 ? 1 : 0, cnt = 0;
    for (int j = 0; j < n_hist; ++j) {
      if (s_htok[j] == tok) {
        ++cnt;
        if (j < t) first = 0;
      }
    }
    s_hfirst[t] = first;
    s_hval[t] = first ? penalised(bf2f(lr[tok]), prm.repeat, prm.presence, prm.frequency, float(cnt)) : 0.f;
  }
  __syncthreads();
  if (t == 0) {
    int nd = 0;
    for (int j = 0; j < n_hist; ++j) nd += s_hfirst[j];
    s_nd = nd;
  }
  __syncthreads();
  const int nd = s_nd;
  const int kq = prm.temperature == 0.f ? 1 : prm.top_k;
  const int K = min(V, kq + nd);  // unpenalised candidates to collect

  // ---- 2a. threshold: the K-th largest order key, 4 bits per pass (16-byte loads, 8 keys each)
  const uint4* lr4 = reinterpret_cast<const uint4*>(lr);  // vocab % 8 == 0
  const int V8 = V / 8;
  const int w = t >> 6, lane = t & 63;
  uint32_t prefix = 0;
  int above = 0;
  for (int s = 12; s >= 0; s -= 4) {
    int c[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) c[d] = 0;
    for (int i0 = t; i0 < V8; i0 += 4 * ST) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = lr4[min(i0 + u * ST, V8 - 1)];  // clamped: no branch around a load
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = i0 + u * ST < V8;
        const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t k = order_key(uint16_t(wd[e >> 1] >> (16 * (e & 1))));
          if (ok && (k >> (s + 4)) == prefix) {
            const uint32_t dg = (k >> s) & 15u;
#pragma unroll
            for (int d = 0; d < 16; ++d) c[d] += dg == uint32_t(d) ? 1 : 0;
          }
        }
      }
    }
#pragma unroll
    for (int d = 0; d < 16; ++d) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) c[d] += __shfl_xor(c[d], o, 64);
    }
    if (lane == 0) {
#pragma unroll
      for (int d = 0; d < 16; ++d) s_cnt[w][d] = c[d];
    }
    __syncthreads();
    if (t < 16) {
      int sum = 0;
      for (int j = 0; j < NWV; ++j) sum += s_cnt[j][t];
      s_tot[t] = sum;
    }
    __syncthreads();
    int d = 15, acc = above;
    for (; d > 0; --d) {
      if (acc + s_tot[d] >= K) break;
      acc += s_tot[d];
    }
    above = acc;
    prefix = (prefix << 4) | uint32_t(d);
    __syncthreads();
  }
  const uint32_t thr = prefix;
  const int need_eq = K - above;

  // ---- 2b. compaction in id order: keys > thr, then the first need_eq keys == thr.  Wave w
  // takes a contiguous range of 16-byte groups; within a pass over 64 groups, lane order is
  // id order, and lane prefix sums give the slots.
  const int per_wave = ((V8 + NWV - 1) / NWV + 63) / 64 * 64;
  const int g0 = min(V8, w * per_wave), g1 = min(V8, g0 + per_wave);
  {
    int cg = 0, ce = 0;
    for (int gb = g0 + lane; gb < g1; gb += 4 * 64) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = lr4[min(gb + 64 * u, V8 - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = gb + 64 * u < g1;
        const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t k = order_key(uint16_t(wd[e >> 1] >> (16 * (e & 1))));
          cg += ok && k > thr ? 1 : 0;
          ce += ok && k == thr ? 1 : 0;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      cg += __shfl_xor(cg, o, 64);
      ce += __shfl_xor(ce, o, 64);
    }
    if (lane == 0) {
      s_scan[w] = cg;
      s_scan2[w] = ce;
    }
  }
  __syncthreads();
  {
    int base_g = 0, base_e = 0;
    for (int j = 0; j < w; ++j) {
      base_g += s_scan[j];
      base_e += s_scan2[j];
    }
    for (int g = g0 + lane; g - lane < g1; g += 64) {
      const bool valid = g < g1;
      const uint4 v = lr4[min(g, V8 - 1)];
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
      uint32_t kk[8];
      int hg = 0, he = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kk[e] = order_key(uint16_t(wd[e >> 1] >> (16 * (e & 1))));
        hg += valid && kk[e] > thr ? 1 : 0;
        he += valid && kk[e] == thr ? 1 : 0;
      }
      int ig = hg, ie = he;  // inclusive lane prefix sums
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int yg = __shfl_up(ig, o, 64), ye = __shfl_up(ie, o, 64);
        if (lane >= o) {
          ig += yg;
          ie += ye;
        }
      }
      int pg = base_g + ig - hg, pe = base_e + ie - he;
      if (valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (kk[e] > thr) {
            s_ckey[pg] = key_value(kk[e]);
            s_cidx[pg] = 8 * g + e;
            ++pg;
          } else if (kk[e] == thr) {
            if (pe < need_eq) {
              s_ckey[above + pe] = key_value(kk[e]);
              s_cidx[above + pe] = 8 * g + e;
            }
            ++pe;
          }
        }
      }
      base_g += __shfl(ig, 63, 64);
      base_e += __shfl(ie, 63, 64);
    }
  }
  __syncthreads();
  // history tokens: drop their unpenalised entries, add them at their penalised values
  for (int j = t; j < K; j += ST) {
    const int idx = s_cidx[j];
    bool hit = false;
    for (int h = 0; h < n_hist; ++h) hit |= s_hfirst[h] && s_htok[h] == idx;
    if (hit) s_ckey[j] = -INFINITY, s_cidx[j] = 0x7FFFFFFF;
  }
  int n = K;
  if (t < n_hist) {
    // slot of this distinct token among the distinct ones
    int slot = 0;
    for (int h = 0; h < t; ++h) slot += s_hfirst[h];
    if (s_hfirst[t]) {
      s_ckey[K + slot] = s_hval[t];
      s_cidx[K + slot] = s_htok[t];
    }
  }
  n = K + nd;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  for (int j = n + t; j < np2; j += ST) {
    s_ckey[j] = -INFINITY;
    s_cidx[j] = 0x7FFFFFFF;
  }
  __syncthreads();

  // ---- 3. bitonic sort by (value desc, id asc)
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < np2 / 2; i += ST) {
        const int a = 2 * stride * (i / stride) + (i % stride);
        const int b = a + stride;
        const bool asc = ((a & size) == 0);  // "asc" = (before) order in this subsequence
        const float va = s_ckey[a], vb = s_ckey[b];
        const int ia = s_cidx[a], ib = s_cidx[b];
        const bool swap = asc ? before(vb, ib, va, ia) : before(va, ia, vb, ib);
        if (swap) {
          s_ckey[a] = vb;
          s_ckey[b] = va;
          s_cidx[a] = ib;
          s_cidx[b] = ia;
        }
      }
      __syncthreads();
    }
  }

  if (prm.temperature == 0.f) {
    if (t == 0) out[row] = s_cidx[0];
    return;
  }
  // ---- 4. weights in fp64, min-p, top-p, the draw
  const int k = min(prm.top_k, V);  // the first min(top_k, V) sorted entries are all real tokens
  const double T = double(prm.temperature);
  const double z0 = double(s_ckey[0]);
  for (int j = t; j < k; j += ST) s_w[j] = exp((double(s_ckey[j]) - z0) / T);
  __syncthreads();
  if (t == 0) {
    const double mp = double(prm.min_p);
    int m = 0;
    while (m < k && s_w[m] >= mp) ++m;
    double csum = 0.0;
    const double tot = [&] {
      double s = 0.0;
      for (int j = 0; j < m; ++j) s += s_w[j];
      return s;
    }();
    const double tp = double(prm.top_p) * tot;
    int cut = m;
    for (int j = 0; j < m; ++j) {
      csum += s_w[j];
      if (csum >= tp) {
        cut = j + 1;
        break;
      }
    }
    uint64_t c[4] = {uint64_t(positions[row]), 0, 0, 0};
    philox4x64_10(c, seeds[row], 0);
    const double u = double(c[0] >> 11) * 0x1.0p-53;
    double kept = 0.0;
    for (int j = 0; j < cut; ++j) kept += s_w[j];
    const double target = u * kept;
    double run = 0.0;
    int pick = cut - 1;
    for (int j = 0; j < cut; ++j) {
      run += s_w[j];
      if (run > target) {
        pick = j;
        break;
      }
    }
    out[row] = s_cidx[pick];
  }
}

// ------------------------------------------------------------------- BLAKE3
constexpr uint32_t CHUNK_START = 1, CHUNK_END = 2, PARENT = 4, ROOT = 8;

__device__ __forceinline__ constexpr uint32_t iv(int i) {
  constexpr uint32_t v[8] = {0x6A09E667u, 0xBB67AE85u, 0x3C6EF372u, 0xA54FF53Au,
                             0x510E527Fu, 0x9B05688Cu, 0x1F83D9ABu, 0x5BE0CD19u};
  return v[i];
}
// message word used at position i of round r: the permutation applied r times
__device__ __forceinline__ constexpr int msg(int r, int i) {
  constexpr int P[16] = {2, 6, 3, 10, 7, 0, 4, 13, 1, 11, 12, 5, 9, 14, 15, 8};
  for (; r > 0; --r) i = P[i];
  return i;
}
__device__ __forceinline__ uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }
__device__ __forceinline__ void gmix(uint32_t* v, int a, int b, int c, int d, uint32_t x, uint32_t y) {
  v[a] = v[a] + v[b] + x;
  v[d] = rotr(v[d] ^ v[a], 16);
  v[c] = v[c] + v[d];
  v[b] = rotr(v[b] ^ v[c], 12);
  v[a] = v[a] + v[b] + y;
  v[d] = rotr(v[d] ^ v[a], 8);
  v[c] = v[c] + v[d];
  v[b] = rotr(v[b] ^ v[c], 7);
}

// cv[8] <- first 8 words of compress(cv, m, counter, len, flags)
__device__ __forceinline__ void compress(uint32_t cv[8], const uint32_t m[16], uint64_t counter, uint32_t len,
                                         uint32_t flags) {
  uint32_t v[16] = {cv[0], cv[1], cv[2], cv[3], cv[4], cv[5], cv[6], cv[7], iv(0), iv(1), iv(2), iv(3),
                    uint32_t(counter), uint32_t(counter >> 32), len, flags};
#pragma unroll
  for (int r = 0; r < 7; ++r) {
    gmix(v, 0, 4, 8, 12, m[msg(r, 0)], m[msg(r, 1)]);
    gmix(v, 1, 5, 9, 13, m[msg(r, 2)], m[msg(r, 3)]);
    gmix(v, 2, 6, 10, 14, m[msg(r, 4)], m[msg(r, 5)]);
    gmix(v, 3, 7, 11, 15, m[msg(r, 6)], m[msg(r, 7)]);
    gmix(v, 0, 5, 10, 15, m[msg(r, 8)], m[msg(r, 9)]);
    gmix(v, 1, 6, 11, 12, m[msg(r, 10)], m[msg(r, 11)]);
    gmix(v, 2, 7, 8, 13, m[msg(r, 12)], m[msg(r, 13)]);
    gmix(v, 3, 4, 9, 14, m[msg(r, 14)], m[msg(r, 15)]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) cv[i] = v[i] ^ v[i + 8];
}

constexpr int kMaxChunks = 256;  // 65536 ids

// chaining value of chunk c of ids[0..count) (words = ids); ROOT on its last block when root
__device__ void chunk_cv(const int32_t* ids, int64_t count, int c, bool root, uint32_t cv[8]) {
  const int64_t bytes = 4 * count - int64_t(c) * 1024;
  const int nbytes = int(bytes < 1024 ? bytes : 1024);
  const int nblocks = nbytes == 0 ? 1 : (nbytes + 63) / 64;
#pragma unroll
  for (int i = 0; i < 8; ++i) cv[i] = iv(i);
  for (int b = 0; b < nblocks; ++b) {
    uint32_t m[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t w = int64_t(c) * 256 + 16 * b + j;
      m[j] = w < count ? uint32_t(ids[w]) : 0u;
    }
    const int len = b == nblocks - 1 ? nbytes - 64 * b : 64;
    uint32_t fl = (b == 0 ? CHUNK_START : 0) | (b == nblocks - 1 ? CHUNK_END : 0);
    if (root && b == nblocks - 1) fl |= ROOT;
    compress(cv, m, uint64_t(c), uint32_t(len), fl);
  }
}

__device__ __forceinline__ void parent(const uint32_t l[8], const uint32_t r[8], uint32_t flags, uint32_t out[8]) {
  uint32_t m[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m[i] = l[i];
    m[8 + i] = r[i];
    out[i] = iv(i);
  }
  compress(out, m, 0, 64, PARENT | flags);
}

__global__ __launch_bounds__(64) void token_hash_kernel(const int32_t* __restrict__ ids,
                                                        const int64_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ counts,
                                                        uint8_t* __restrict__ out) {
  __shared__ uint32_t s_cv[kMaxChunks][8];
  __shared__ uint32_t s_stack[9][8];  // roots of complete subtrees (lane 0)
  const int sq = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t count = counts[sq];
  const int32_t* p = ids + offsets[sq];
  uint32_t* dst = reinterpret_cast<uint32_t*>(out + int64_t(sq) * 32);
  const int n = count == 0 ? 1 : int((4 * count + 1023) / 1024);
  if (count < 0 || n > kMaxChunks) {  // outside what the host checked: all-ones digest
    if (lane < 8) dst[lane] = 0xFFFFFFFFu;
    return;
  }
  if (n == 1) {
    if (lane == 0) {
      uint32_t cv[8];
      chunk_cv(p, count, 0, true, cv);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = cv[i];
    }
    return;
  }
  for (int c = lane; c < n; c += 64) {
    uint32_t cv[8];
    chunk_cv(p, count, c, false, cv);
#pragma unroll
    for (int i = 0; i < 8; ++i) s_cv[c][i] = cv[i];
  }
  __syncthreads();
  if (lane == 0) {
    uint32_t(*stack)[8] = s_stack;
    int depth = 0;
    for (int c = 0; c + 1 < n; ++c) {  // every chunk but the last, merging complete subtrees
      uint32_t cv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) cv[i] = s_cv[c][i];
      for (int total = c + 1; (total & 1) == 0; total >>= 1) {
        uint32_t pcv[8];
        parent(stack[--depth], cv, 0, pcv);
#pragma unroll
        for (int i = 0; i < 8; ++i) cv[i] = pcv[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) stack[depth][i] = cv[i];
      ++depth;
    }
    uint32_t cv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) cv[i] = s_cv[n - 1][i];
    while (depth > 0) {
      --depth;
      uint32_t pcv[8];
      parent(stack[depth], cv, depth == 0 ? ROOT : 0, pcv);
#pragma unroll
      for (int i = 0; i < 8; ++i) cv[i] = pcv[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = cv[i];
  }
}

}  // namespace

hipError_t launch_sample(const uint16_t* logits, int64_t rows, int64_t vocab, const BiSampling& prm,
                         const uint64_t* seeds, const int64_t* positions, const int32_t* history, int n_hist,
                         int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(sample_kernel, dim3(unsigned(rows)), dim3(ST), 0, s, logits, vocab, prm, seeds, positions,
                     history, n_hist, out);
  return hipGetLastError();
}

hipError_t launch_token_hash(const int32_t* ids, const int64_t* offsets, const int32_t* counts, int n_seqs,
                             uint8_t* out, hipStream_t s) {
  hipLaunchKernelGGL(token_hash_kernel, dim3(n_seqs), dim3(64), 0, s, ids, offsets, counts, out);
  return hipGetLastError();
}

int token_hash_max_ids() { return kMaxChunks * 256; }

}  // namespace bi
