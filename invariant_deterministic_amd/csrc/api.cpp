// The C-ABI of the library: argument checks, then kernel launches on the
// caller's stream.  Every check runs before anything is enqueued, so an error
// return leaves every output untouched.  The block entry point composes the
// kernels in a fixed order; nothing here depends on the batch composition
// except how many work-groups are launched.
#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <utility>
#include <vector>

#include <hip/hip_vector_types.h>

#include "../../include/bi.h"
#include "bi_internal.h"

#ifndef BI_BUILD_ID
#define BI_BUILD_ID "unversioned0000"
#endif

namespace {

using bi::DecodeSeq;
using bi::PrefillSeq;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bi_status from_hip(hipError_t e) { return e == hipSuccess ? BI_OK : BI_ERR_HIP; }

// Launch-grid limits: a grid dimension times its work-group size stays below 2^32
// work-items, and the y / z dimensions below 65536.
constexpr int64_t kMaxNormRows = (int64_t(1) << 26) - 1024;  // 64 work-items per row
constexpr int64_t kMaxRopeRows = (int64_t(1) << 24) - 1;     // one 256-thread work-group per row
constexpr int64_t kMaxQuantRows = (int64_t(1) << 26) - 1;    // one 64-thread work-group per (row, head, K|V)
constexpr int64_t kMaxPrefillTiles = (int64_t(1) << 23) - 1; // 512-thread work-groups along x
constexpr int64_t kMaxGridYZ = 65535;                        // decode requests, prefill sequences
constexpr int64_t kMaxDecodeLen = int64_t(1) << 30;
constexpr int64_t kMaxDecodeRuns = int64_t(1) << 24;         // split decode: one work-group per run and head
constexpr int64_t kMaxGemmTiles = (int64_t(1) << 23) - 1;    // 512-thread work-groups along x

bi_status check_rmsnorm(const void* x, const void* g, const void* y, int64_t rows, int64_t hidden,
                        float eps) {
  if (!x || !g || !y) return BI_ERR_NULL;
  if (rows < 1 || hidden < 1) return BI_ERR_SHAPE;
  if (hidden % 8 || hidden > 16384 || rows > kMaxNormRows) return BI_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || eps > 3.0e38f) return BI_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(g) || !aligned16(y)) return BI_ERR_ALIGN;
  return BI_OK;
}

// Shape limits of the GEMM kernels (operand offsets, tile counts and the 1-D grid).
bi_status gemm_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return BI_ERR_SHAPE;
  if (N % 8 || K % bi::kGemmBK) return BI_ERR_UNSUPPORTED;
  if (M > INT32_MAX || N > INT32_MAX || K > bi::kGemmMaxK || M * K > (int64_t(1) << 40) ||
      M * N > (int64_t(1) << 40))
    return BI_ERR_UNSUPPORTED;
  const int64_t tiles = ((M + bi::kGemmBM - 1) / bi::kGemmBM) * ((N + bi::kGemmBNNarrow - 1) / bi::kGemmBNNarrow);
  if (tiles > kMaxGemmTiles) return BI_ERR_UNSUPPORTED;
  return BI_OK;
}

bi_status check_gemm(const void* A, const void* W, const void* C, int64_t M, int64_t N, int64_t K) {
  if (!A || !W || !C) return BI_ERR_NULL;
  const bi_status st = gemm_shape(M, N, K);
  if (st != BI_OK) return st;
  if (!aligned16(A) || !aligned16(W) || !aligned16(C)) return BI_ERR_ALIGN;
  return BI_OK;
}

// Query tiles of a prefill chunk of T queries starting at q_start.
int64_t prefill_tiles(int64_t q_start, int64_t T, int group) {
  const int P = bi::prefill_positions_per_tile(group);
  return (q_start + T - 1) / P - q_start / P + 1;
}

bool head_shape_ok(int Hq, int Hkv, int D, int max_group) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (G > max_group) return false;
  // a 256-key unit of one kv head is addressed with 32-bit buffer offsets
  if (int64_t(Hkv) * D > 65536) return false;
  return D == 64 || D == 128;
}

bool scale_ok(float s) { return s > 0.f && s < 3.0e38f; }

// ---- step metadata layout (host bytes uploaded by the caller)
struct MetaLayout {
  size_t prefill, decode, pos, kv, runs, order, total;
};
// Layout of the packed step description: header, prefill descriptors, decode
// descriptors, per-row positions, per-row KV rows, the split decode's run list
// (one (request, first unit) int32 pair per run of up to kDecodeRun 256-key
// units, longest runs first), then the decode requests ordered longest first
// (int32 indices).
MetaLayout meta_layout(int n_seqs, int64_t n_tokens, int64_t n_runs) {
  MetaLayout L;
  L.prefill = 256;
  L.decode = L.prefill + align256(size_t(n_seqs) * sizeof(PrefillSeq));
  L.pos = L.decode + align256(size_t(n_seqs) * sizeof(DecodeSeq));
  L.kv = L.pos + align256(size_t(n_tokens) * sizeof(int32_t));
  L.runs = L.kv + align256(size_t(n_tokens) * sizeof(int64_t));
  L.order = L.runs + align256(size_t(n_runs) * 8);
  L.total = L.order + align256(size_t(n_seqs) * sizeof(int32_t));
  return L;
}
int64_t units_of(int64_t kv_len) { return (kv_len + bi::kKvSplit - 1) / bi::kKvSplit; }
int64_t decode_runs(const bi_seq* seqs, int n_seqs) {
  int64_t r = 0;
  for (int i = 0; i < n_seqs; ++i)
    if (seqs[i].q_len == 1) r += (units_of(int64_t(seqs[i].ctx_len) + 1) + bi::kDecodeRun - 1) / bi::kDecodeRun;
  return r;
}

struct StepSummary {
  int64_t M = 0;
  int n_prefill = 0, n_decode = 0;
  int64_t max_prefill_last = 0;  // unused by sizing; kept for clarity
  int64_t max_decode_len = 0;
};

bi_status summarize(const bi_seq* seqs, int n_seqs, StepSummary* out) {
  if (!seqs) return BI_ERR_NULL;
  if (n_seqs < 1) return BI_ERR_SHAPE;
  StepSummary s;
  for (int i = 0; i < n_seqs; ++i) {
    const bi_seq& q = seqs[i];
    if (q.q_len < 1 || q.ctx_len < 0 || q.kv_base < 0) return BI_ERR_SHAPE;
    if (int64_t(q.ctx_len) + q.q_len > INT32_MAX) return BI_ERR_UNSUPPORTED;
    s.M += q.q_len;
    if (q.q_len == 1) {
      ++s.n_decode;
      s.max_decode_len = std::max<int64_t>(s.max_decode_len, int64_t(q.ctx_len) + 1);
    } else {
      ++s.n_prefill;
    }
  }
  if (s.M > INT32_MAX) return BI_ERR_UNSUPPORTED;
  *out = s;
  return BI_OK;
}

bi_status check_cfg(const bi_block_cfg* c) {
  if (!c) return BI_ERR_NULL;
  if (c->hidden < 8 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 || c->ffn < 0)
    return BI_ERR_SHAPE;
  if (c->hidden % 64 || c->hidden > 16384) return BI_ERR_UNSUPPORTED;
  if (!head_shape_ok(c->n_q_heads, c->n_kv_heads, c->head_dim, 4)) return BI_ERR_UNSUPPORTED;
  if ((c->n_q_heads * c->head_dim) % 64) return BI_ERR_UNSUPPORTED;
  if (c->ffn % 64) return BI_ERR_UNSUPPORTED;
  if (!(c->eps >= 0.f) || c->eps > 3.0e38f) return BI_ERR_SHAPE;
  if (!(c->rope_theta >= 0.0) || c->rope_theta > 1e300) return BI_ERR_SHAPE;
  if (c->weight_format != BI_WEIGHTS_BF16 && c->weight_format != BI_WEIGHTS_INT4_G32)
    return BI_ERR_UNSUPPORTED;
  if (c->decode_order != BI_DECODE_SPLIT && c->decode_order != BI_DECODE_PREFILL_ORDER)
    return BI_ERR_UNSUPPORTED;
  if (c->kv_format != BI_KV_BF16 && c->kv_format != BI_KV_INT8_PAGED) return BI_ERR_UNSUPPORTED;
  // the paged int8 cache is read in the prefill kernel's key order only
  if (c->kv_format == BI_KV_INT8_PAGED && c->decode_order != BI_DECODE_PREFILL_ORDER) return BI_ERR_UNSUPPORTED;
  return BI_OK;
}

bool paged(const bi_block_cfg& c) { return c.kv_format == BI_KV_INT8_PAGED; }

bi_status check_weight(const bi_weight& w, int fmt) {
  if (!w.w) return BI_ERR_NULL;
  if (!aligned16(w.w)) return BI_ERR_ALIGN;
  if (fmt == BI_WEIGHTS_INT4_G32) {
    if (!w.scale) return BI_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(w.scale) & 1u) != 0) return BI_ERR_ALIGN;
  }
  return BI_OK;
}

// the gate/up GEMM carries SwiGLU in its epilogue when its tile can pair the columns
// The gated gate/up GEMM (SwiGLU in its epilogue) needs F % 128 == 0; with bf16 weights its
// operand offsets, 32-bit from the tile's first gate row, reach (F + 128) rows of W.
bool gated_ok(int64_t F, int64_t K, bool bf16_weights) {
  return F % 128 == 0 && (!bf16_weights || (F + 128) * K * 2 < (int64_t(1) << 32));
}
bool ffn_fused(const bi_block_cfg& c) { return gated_ok(c.ffn, c.hidden, c.weight_format == BI_WEIGHTS_BF16); }

struct WsLayout {
  bi_block_ws_layout pub;
};

WsLayout ws_layout(const bi_block_cfg& c, const StepSummary& s) {
  const size_t M = size_t(s.M);
  const size_t H = size_t(c.hidden);
  const size_t qd = size_t(c.n_q_heads) * c.head_dim;
  const size_t qkv = size_t(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const size_t F = size_t(c.ffn);
  const size_t none = SIZE_MAX;
  WsLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.pub.n1 = take(M * H * 2);
  L.pub.qkv = take(M * qkv * 2);
  L.pub.q = take(M * qd * 2);
  L.pub.attn = take(M * qd * 2);
  // o and d go straight into the residual sums h and y (fused epilogues); gu only when the
  // gate/up GEMM cannot carry SwiGLU
  L.pub.o = none;
  L.pub.h = F ? take(M * H * 2) : none;
  L.pub.n2 = F ? take(M * H * 2) : none;
  L.pub.gu = F && !ffn_fused(c) ? take(M * 2 * F * 2) : none;
  L.pub.act = F ? take(M * F * 2) : none;
  L.pub.d = none;
  L.pub.kv_new = paged(c) ? take(2 * M * size_t(c.n_kv_heads) * c.head_dim * 2) : none;
  L.pub.decode_partials =
      s.n_decode && c.decode_order == BI_DECODE_SPLIT
          ? take(bi::decode_workspace_bytes(s.n_decode, s.max_decode_len, c.n_q_heads, c.head_dim))
          : none;
  L.pub.total = off;
  return L;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}
template <class T>
const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

hipError_t run_gemm(const bi_block_cfg& c, const bi_weight& w, const uint16_t* A, uint16_t* C,
                    int64_t M, int64_t N, int64_t K, hipStream_t s, int epi = bi::kEpiPlain,
                    const uint16_t* R = nullptr) {
  if (c.weight_format == BI_WEIGHTS_INT4_G32)
    return bi::launch_gemm_w4_ex(static_cast<const uint8_t*>(w.w), w.scale, A, R, C, M, N, K, epi, s);
  return bi::launch_gemm_ex(A, static_cast<const uint16_t*>(w.w), R, C, M, N, K, epi, s);
}


}  // namespace

extern "C" {

const char* bi_status_str(bi_status st) {
  switch (st) {
    case BI_OK: return "BI_OK";
    case BI_ERR_NULL: return "BI_ERR_NULL: a required pointer is NULL";
    case BI_ERR_SHAPE: return "BI_ERR_SHAPE: a size is zero, negative or inconsistent";
    case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED: size outside what the kernels implement";
    case BI_ERR_ALIGN: return "BI_ERR_ALIGN: pointer not 16-byte aligned";
    case BI_ERR_WORKSPACE: return "BI_ERR_WORKSPACE: workspace missing or too small";
    case BI_ERR_HIP: return "BI_ERR_HIP: HIP launch error";
  }
  return "bi_status: unknown code";
}

const char* bi_build_id(void) { return BI_BUILD_ID; }

int bi_kv_split_size(void) { return bi::kKvSplit; }

void bi_gemm_tile(int out[3]) {
  if (!out) return;
  out[0] = bi::kGemmBM;
  out[1] = bi::kGemmBN;
  out[2] = bi::kGemmBK;
}

int bi_gemm_tile_cols(int64_t N, int weight_format) {
  if (N < 1) return 0;
  return weight_format == BI_WEIGHTS_BF16 ? bi::gemm_tile_n(N, bi::kEpiPlain) : bi::gemm_w4_tile_n(N, bi::kEpiPlain);
}

bi_status bi_rmsnorm(const bi_bf16* x, const bi_bf16* gamma, bi_bf16* y, int64_t rows,
                     int64_t hidden, float eps, hipStream_t stream) {
  const bi_status st = check_rmsnorm(x, gamma, y, rows, hidden, eps);
  if (st != BI_OK) return st;
  if (x == y) return BI_ERR_SHAPE;
  return from_hip(bi::launch_rmsnorm(x, gamma, y, rows, hidden, eps, stream));
}

bi_status bi_gemm(const bi_bf16* A, const bi_bf16* W, bi_bf16* C, int64_t M, int64_t N, int64_t K,
                  hipStream_t stream) {
  const bi_status st = check_gemm(A, W, C, M, N, K);
  if (st != BI_OK) return st;
  return from_hip(bi::launch_gemm(A, W, C, M, N, K, stream));
}

bi_status bi_gemm_w4(const bi_bf16* A, const uint8_t* Wq, const bi_f16* Ws, bi_bf16* C, int64_t M,
                     int64_t N, int64_t K, hipStream_t stream) {
  if (!Ws) return BI_ERR_NULL;
  const bi_status st = check_gemm(A, Wq, C, M, N, K);
  if (st != BI_OK) return st;
  if ((reinterpret_cast<uintptr_t>(Ws) & 1u) != 0) return BI_ERR_ALIGN;
  return from_hip(bi::launch_gemm_w4(A, Wq, Ws, C, M, N, K, stream));
}

bi_status bi_gemm_residual(const bi_bf16* A, const bi_bf16* W, const bi_bf16* R, bi_bf16* C, int64_t M, int64_t N,
                           int64_t K, hipStream_t stream) {
  if (!R) return BI_ERR_NULL;
  const bi_status st = check_gemm(A, W, C, M, N, K);
  if (st != BI_OK) return st;
  if (!aligned16(R)) return BI_ERR_ALIGN;
  return from_hip(bi::launch_gemm_ex(A, W, R, C, M, N, K, bi::kEpiResid, stream));
}

bi_status bi_gemm_swiglu(const bi_bf16* A, const bi_bf16* W, bi_bf16* act, int64_t M, int64_t F, int64_t K,
                         hipStream_t stream) {
  if (F < 1) return BI_ERR_SHAPE;
  const bi_status st = check_gemm(A, W, act, M, 2 * F, K);
  if (st != BI_OK) return st;
  if (!gated_ok(F, K, true)) return BI_ERR_UNSUPPORTED;
  return from_hip(bi::launch_gemm_ex(A, W, nullptr, act, M, F, K, bi::kEpiGated, stream));
}

bi_status bi_gemm_w4_residual(const bi_bf16* A, const uint8_t* Wq, const bi_f16* Ws, const bi_bf16* R, bi_bf16* C,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (!Ws || !R) return BI_ERR_NULL;
  const bi_status st = check_gemm(A, Wq, C, M, N, K);
  if (st != BI_OK) return st;
  if ((reinterpret_cast<uintptr_t>(Ws) & 1u) != 0 || !aligned16(R)) return BI_ERR_ALIGN;
  return from_hip(bi::launch_gemm_w4_ex(Wq, Ws, A, R, C, M, N, K, bi::kEpiResid, stream));
}

bi_status bi_gemm_w4_swiglu(const bi_bf16* A, const uint8_t* Wq, const bi_f16* Ws, bi_bf16* act, int64_t M,
                            int64_t F, int64_t K, hipStream_t stream) {
  if (!Ws) return BI_ERR_NULL;
  if (F < 1) return BI_ERR_SHAPE;
  const bi_status st = check_gemm(A, Wq, act, M, 2 * F, K);
  if (st != BI_OK) return st;
  if (F % 128) return BI_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(Ws) & 1u) != 0) return BI_ERR_ALIGN;
  return from_hip(bi::launch_gemm_w4_ex(Wq, Ws, A, nullptr, act, M, F, K, bi::kEpiGated, stream));
}

bi_status bi_add(const bi_bf16* x, const bi_bf16* o, bi_bf16* h, int64_t n, hipStream_t stream) {
  if (!x || !o || !h) return BI_ERR_NULL;
  if (n < 1) return BI_ERR_SHAPE;
  if (n % 8) return BI_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(o) || !aligned16(h)) return BI_ERR_ALIGN;
  return from_hip(bi::launch_add(x, o, h, n, stream));
}

bi_status bi_swiglu(const bi_bf16* gu, bi_bf16* act, int64_t rows, int64_t F, hipStream_t stream) {
  if (!gu || !act) return BI_ERR_NULL;
  if (rows < 1 || F < 1) return BI_ERR_SHAPE;
  if (F % 8) return BI_ERR_UNSUPPORTED;
  if (!aligned16(gu) || !aligned16(act)) return BI_ERR_ALIGN;
  return from_hip(bi::launch_swiglu(gu, act, rows, F, stream));
}

bi_status bi_rope_kv(const bi_bf16* qkv, const int32_t* pos, const int64_t* kv_row, bi_bf16* q_out,
                     bi_bf16* k_pool, bi_bf16* v_pool, int64_t rows, int Hq, int Hkv, int D,
                     double theta, hipStream_t stream) {
  if (!qkv || !pos || !kv_row || !q_out || !k_pool || !v_pool) return BI_ERR_NULL;
  if (rows < 1) return BI_ERR_SHAPE;
  if (rows > kMaxRopeRows) return BI_ERR_UNSUPPORTED;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return BI_ERR_SHAPE;
  if (D != 64 && D != 128) return BI_ERR_UNSUPPORTED;
  if (!(theta >= 0.0) || theta > 1e300) return BI_ERR_SHAPE;
  if (!aligned16(qkv) || !aligned16(q_out) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned8(kv_row) || (reinterpret_cast<uintptr_t>(pos) & 3u))
    return BI_ERR_ALIGN;
  return from_hip(bi::launch_rope_kv(qkv, pos, kv_row, q_out, k_pool, v_pool, rows, Hq, Hkv, D,
                                     theta, stream));
}

bi_status bi_attn_prefill(const bi_bf16* q, const bi_bf16* k_cache, const bi_bf16* v_cache,
                          bi_bf16* o, int64_t q_start, int64_t T, int Hq, int Hkv, int D,
                          float scale, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !o) return BI_ERR_NULL;
  if (T < 1 || q_start < 0) return BI_ERR_SHAPE;
  if (q_start + T > INT32_MAX) return BI_ERR_UNSUPPORTED;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return BI_ERR_SHAPE;
  if (!head_shape_ok(Hq, Hkv, D, 4)) return BI_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return BI_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return BI_ERR_ALIGN;
  const int64_t tiles = prefill_tiles(q_start, T, Hq / Hkv);
  if (tiles > kMaxPrefillTiles || Hkv > kMaxGridYZ) return BI_ERR_UNSUPPORTED;
  PrefillSeq one;
  one.q_row = 0;
  one.kv_base = 0;
  one.q_start = int32_t(q_start);
  one.q_len = int32_t(T);
  return from_hip(bi::launch_attn_prefill(q, int64_t(Hq) * D, k_cache, v_cache, o, int64_t(Hq) * D,
                                          nullptr, &one, 1, int(tiles), Hq, Hkv, D, scale, stream));
}

size_t bi_attn_decode_workspace(int B, int64_t max_kv_len, int Hq, int D) {
  if (B < 1 || max_kv_len < 1 || Hq < 1 || D < 1) return 0;
  return bi::decode_workspace_bytes(B, max_kv_len, Hq, D);
}

bi_status bi_attn_decode(const bi_bf16* q, const bi_bf16* k_all, const bi_bf16* v_all,
                         const int64_t* kv_offset, const int32_t* kv_len, int B,
                         int64_t max_kv_len, int Hq, int Hkv, int D, float scale, void* ws,
                         size_t ws_bytes, bi_bf16* o, hipStream_t stream) {
  if (!q || !k_all || !v_all || !kv_offset || !kv_len || !o) return BI_ERR_NULL;
  if (B < 1 || max_kv_len < 1) return BI_ERR_SHAPE;
  if (B > kMaxGridYZ || max_kv_len > kMaxDecodeLen || Hkv > kMaxGridYZ) return BI_ERR_UNSUPPORTED;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return BI_ERR_SHAPE;
  if (!head_shape_ok(Hq, Hkv, D, 8)) return BI_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return BI_ERR_SHAPE;
  const int64_t run_keys = int64_t(bi::kKvSplit) * bi::kDecodeRun;
  if (int64_t(B) * ((max_kv_len + run_keys - 1) / run_keys) > kMaxDecodeRuns) return BI_ERR_UNSUPPORTED;
  if (!ws) return BI_ERR_WORKSPACE;
  if (ws_bytes < bi::decode_workspace_bytes(B, max_kv_len, Hq, D)) return BI_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_all) || !aligned16(v_all) || !aligned16(o) || !aligned16(ws) ||
      !aligned8(kv_offset) || (reinterpret_cast<uintptr_t>(kv_len) & 3u))
    return BI_ERR_ALIGN;
  return from_hip(bi::launch_attn_decode_arrays(q, k_all, v_all, kv_offset, kv_len, B, max_kv_len,
                                                Hq, Hkv, D, scale, ws, o, stream));
}

bi_status bi_attn_decode_noalloc(const bi_bf16* q, const bi_bf16* k_all, const bi_bf16* v_all,
                                 const int64_t* kv_offset, const int32_t* kv_len, int B, int64_t max_kv_len, int Hq,
                                 int Hkv, int D, float scale, bi_bf16* o, hipStream_t stream) {
  if (!q || !k_all || !v_all || !kv_offset || !kv_len || !o) return BI_ERR_NULL;
  if (B < 1 || max_kv_len < 1) return BI_ERR_SHAPE;
  if (B > kMaxGridYZ || max_kv_len > kMaxDecodeLen || Hkv > kMaxGridYZ) return BI_ERR_UNSUPPORTED;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return BI_ERR_SHAPE;
  if (!head_shape_ok(Hq, Hkv, D, 8)) return BI_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return BI_ERR_SHAPE;
  const int64_t run_keys = int64_t(bi::kKvSplit) * bi::kDecodeRun;
  if (int64_t(B) * ((max_kv_len + run_keys - 1) / run_keys) > kMaxDecodeRuns) return BI_ERR_UNSUPPORTED;
  // the partials must fit the library's fixed scratch
  if (bi::decode_workspace_bytes(B, max_kv_len, Hq, D) > bi::kDecodeScratchBytes) return BI_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_all) || !aligned16(v_all) || !aligned16(o) || !aligned8(kv_offset) ||
      (reinterpret_cast<uintptr_t>(kv_len) & 3u))
    return BI_ERR_ALIGN;
  return from_hip(bi::launch_attn_decode_noalloc(q, k_all, v_all, kv_offset, kv_len, B, max_kv_len, Hq, Hkv, D,
                                                 scale, o, stream));
}

bi_status bi_attn_decode_prefill_order(const bi_bf16* q, const bi_bf16* k_all, const bi_bf16* v_all,
                                       const int64_t* kv_offset, const int32_t* kv_len,
                                       const int32_t* order, int B, int64_t max_kv_len, int Hq,
                                       int Hkv, int D, float scale, bi_bf16* o, hipStream_t stream) {
  if (!q || !k_all || !v_all || !kv_offset || !kv_len || !o) return BI_ERR_NULL;
  if (B < 1 || max_kv_len < 1) return BI_ERR_SHAPE;
  if (B > kMaxGridYZ || max_kv_len > kMaxDecodeLen || Hkv > kMaxGridYZ) return BI_ERR_UNSUPPORTED;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return BI_ERR_SHAPE;
  if (!head_shape_ok(Hq, Hkv, D, 8)) return BI_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return BI_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_all) || !aligned16(v_all) || !aligned16(o) || !aligned8(kv_offset) ||
      (reinterpret_cast<uintptr_t>(kv_len) & 3u) || (reinterpret_cast<uintptr_t>(order) & 3u))
    return BI_ERR_ALIGN;
  return from_hip(bi::launch_attn_decode_po(q, int64_t(Hq) * D, k_all, v_all, nullptr, kv_offset, kv_len,
                                            order, B, max_kv_len, Hq, Hkv, D, scale, o, int64_t(Hq) * D,
                                            stream));
}

bi_status bi_kv_append_q8(const bi_bf16* k, const bi_bf16* v, const int64_t* dst_row, int64_t rows, int Hkv,
                          int D, int8_t* k_pool, int8_t* v_pool, float* k_scale, float* v_scale,
                          hipStream_t stream) {
  if (!k || !v || !dst_row || !k_pool || !v_pool || !k_scale || !v_scale) return BI_ERR_NULL;
  if (rows < 1 || Hkv < 1) return BI_ERR_SHAPE;
  if (rows > kMaxQuantRows || Hkv > kMaxGridYZ || (D != 64 && D != 128)) return BI_ERR_UNSUPPORTED;
  if (!aligned16(k) || !aligned16(v) || !aligned8(dst_row) || !aligned16(k_pool) || !aligned16(v_pool) ||
      (reinterpret_cast<uintptr_t>(k_scale) & 3u) || (reinterpret_cast<uintptr_t>(v_scale) & 3u))
    return BI_ERR_ALIGN;
  return from_hip(bi::launch_kv_quant(k, v, dst_row, rows, Hkv, D, k_pool, v_pool, k_scale, v_scale, stream));
}

bi_status bi_attn_prefill_paged_q8(const bi_bf16* q, const int8_t* k_pool, const int8_t* v_pool,
                                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                                   bi_bf16* o, int64_t q_start, int64_t T, int Hq, int Hkv, int D, float scale,
                                   hipStream_t stream) {
  if (!q || !k_pool || !v_pool || !k_scale || !v_scale || !block_table || !o) return BI_ERR_NULL;
  if (T < 1 || q_start < 0) return BI_ERR_SHAPE;
  if (q_start + T > INT32_MAX) return BI_ERR_UNSUPPORTED;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return BI_ERR_SHAPE;
  if (!head_shape_ok(Hq, Hkv, D, 4)) return BI_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return BI_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(k_scale) & 3u) || (reinterpret_cast<uintptr_t>(v_scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return BI_ERR_ALIGN;
  const int64_t tiles = prefill_tiles(q_start, T, Hq / Hkv);
  if (tiles > kMaxPrefillTiles || Hkv > kMaxGridYZ) return BI_ERR_UNSUPPORTED;
  PrefillSeq one;
  one.q_row = 0;
  one.kv_base = 0;
  one.q_start = int32_t(q_start);
  one.q_len = int32_t(T);
  return from_hip(bi::launch_attn_prefill_q8(q, int64_t(Hq) * D, k_pool, v_pool, k_scale, v_scale, block_table,
                                             INT64_MAX, o, int64_t(Hq) * D, nullptr, &one, 1, int(tiles), Hq, Hkv, D,
                                             scale, stream));
}

bi_status bi_attn_decode_paged_q8(const bi_bf16* q, const int8_t* k_pool, const int8_t* v_pool,
                                  const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                  int max_pages, const int32_t* kv_len, const int32_t* order, int B,
                                  int64_t max_kv_len, int Hq, int Hkv, int D, float scale, bi_bf16* o,
                                  hipStream_t stream) {
  if (!q || !k_pool || !v_pool || !k_scale || !v_scale || !block_tables || !kv_len || !o) return BI_ERR_NULL;
  if (B < 1 || max_kv_len < 1 || max_pages < 1) return BI_ERR_SHAPE;
  if (B > kMaxGridYZ || max_kv_len > kMaxDecodeLen || Hkv > kMaxGridYZ) return BI_ERR_UNSUPPORTED;
  if (int64_t(max_pages) * bi::kPrefillKeyBlock < max_kv_len) return BI_ERR_SHAPE;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return BI_ERR_SHAPE;
  if (!head_shape_ok(Hq, Hkv, D, 8)) return BI_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return BI_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(k_scale) & 3u) || (reinterpret_cast<uintptr_t>(v_scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(kv_len) & 3u) ||
      (reinterpret_cast<uintptr_t>(order) & 3u))
    return BI_ERR_ALIGN;
  return from_hip(bi::launch_attn_decode_po_q8(q, int64_t(Hq) * D, k_pool, v_pool, k_scale, v_scale, block_tables,
                                               max_pages, INT64_MAX, nullptr, kv_len, order, B, max_kv_len, Hq, Hkv,
                                               D, scale, o, int64_t(Hq) * D, stream));
}

bi_status bi_sample(const bi_bf16* logits, int64_t rows, int64_t vocab, const bi_sampling* params,
                    const uint64_t* seeds, const int64_t* positions, const int32_t* history, int n_hist,
                    int32_t* out_ids, hipStream_t stream) {
  if (!logits || !params || !seeds || !positions || !out_ids) return BI_ERR_NULL;
  if (n_hist > 0 && !history) return BI_ERR_NULL;
  if (rows < 1 || vocab < 1 || n_hist < 0) return BI_ERR_SHAPE;
  if (rows > INT32_MAX || vocab > (int64_t(1) << 24) || vocab % 8 || n_hist > 256) return BI_ERR_UNSUPPORTED;
  const bi_sampling& p = *params;
  auto finite = [](float x) { return x == x && x < 3.0e38f && x > -3.0e38f; };
  if (!finite(p.temperature) || p.temperature < 0.f) return BI_ERR_SHAPE;
  if (p.temperature > 0.f) {
    if (p.top_k < 1) return BI_ERR_SHAPE;
    if (p.top_k > 1024) return BI_ERR_UNSUPPORTED;
    if (!(p.top_p > 0.f && p.top_p <= 1.f) || !(p.min_p >= 0.f && p.min_p < 1.f)) return BI_ERR_SHAPE;
  }
  if (!finite(p.repeat_penalty) || !(p.repeat_penalty > 0.f) || !finite(p.presence_penalty) ||
      !finite(p.frequency_penalty))
    return BI_ERR_SHAPE;
  if (!aligned16(logits) || !aligned8(seeds) || !aligned8(positions) ||
      (reinterpret_cast<uintptr_t>(history) & 3u) || (reinterpret_cast<uintptr_t>(out_ids) & 3u))
    return BI_ERR_ALIGN;
  bi::BiSampling q;
  q.temperature = p.temperature;
  q.top_k = p.top_k;
  q.top_p = p.top_p;
  q.min_p = p.min_p;
  q.repeat = p.repeat_penalty;
  q.presence = p.presence_penalty;
  q.frequency = p.frequency_penalty;
  return from_hip(bi::launch_sample(logits, rows, vocab, q, seeds, positions, history, n_hist, out_ids, stream));
}

bi_status bi_token_hash(const int32_t* ids, const int64_t* offsets, const int32_t* counts, int n_seqs,
                        uint8_t* out, hipStream_t stream) {
  if (!ids || !offsets || !counts || !out) return BI_ERR_NULL;
  if (n_seqs < 1) return BI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(ids) & 3u) || !aligned8(offsets) || (reinterpret_cast<uintptr_t>(counts) & 3u) ||
      (reinterpret_cast<uintptr_t>(out) & 3u))
    return BI_ERR_ALIGN;
  return from_hip(bi::launch_token_hash(ids, offsets, counts, n_seqs, out, stream));
}

size_t bi_step_meta_bytes(const bi_seq* seqs, int n_seqs) {
  StepSummary s;
  if (summarize(seqs, n_seqs, &s) != BI_OK) return 0;
  return meta_layout(n_seqs, s.M, decode_runs(seqs, n_seqs)).total;
}

bi_status bi_step_pack(const bi_seq* seqs, int n_seqs, void* host_meta, size_t bytes) {
  StepSummary s;
  bi_status st = summarize(seqs, n_seqs, &s);
  if (st != BI_OK) return st;
  if (!host_meta) return BI_ERR_NULL;
  const int64_t n_runs = decode_runs(seqs, n_seqs);
  if (n_runs > INT32_MAX) return BI_ERR_UNSUPPORTED;
  const MetaLayout L = meta_layout(n_seqs, s.M, n_runs);
  if (bytes < L.total) return BI_ERR_WORKSPACE;
  // scratch for sorting the run list, allocated before the output is touched (no exception
  // leaves this function)
  std::vector<std::pair<int32_t, int32_t>> rl;
  try {
    rl.resize(static_cast<size_t>(n_runs));
  } catch (...) {
    return BI_ERR_UNSUPPORTED;
  }
  memset(host_meta, 0, L.total);
  int64_t* hdr = at<int64_t>(host_meta, 0);
  hdr[0] = n_seqs;
  hdr[1] = s.M;
  hdr[2] = s.n_prefill;
  hdr[3] = s.n_decode;
  hdr[4] = n_runs;
  int32_t* runs = at<int32_t>(host_meta, L.runs);
  int64_t u = 0;
  PrefillSeq* pf = at<PrefillSeq>(host_meta, L.prefill);
  DecodeSeq* dc = at<DecodeSeq>(host_meta, L.decode);
  int32_t* pos = at<int32_t>(host_meta, L.pos);
  int64_t* kvr = at<int64_t>(host_meta, L.kv);
  int64_t row = 0;
  int np = 0, nd = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const bi_seq& q = seqs[i];
    if (q.q_len == 1) {
      DecodeSeq d;
      d.q_row = row;
      d.kv_offset = q.kv_base;
      d.kv_len = q.ctx_len + 1;
      d.pad = 0;
      const int64_t nu = units_of(d.kv_len);
      for (int64_t k = 0; k < nu; k += bi::kDecodeRun, ++u) {
        runs[2 * u] = nd;
        runs[2 * u + 1] = int32_t(k);
      }
      dc[nd++] = d;
    } else {
      PrefillSeq p;
      p.q_row = row;
      p.kv_base = q.kv_base;
      p.q_start = q.ctx_len;
      p.q_len = q.q_len;
      pf[np++] = p;
    }
    for (int j = 0; j < q.q_len; ++j) {
      pos[row + j] = q.ctx_len + j;
      kvr[row + j] = q.kv_base + q.ctx_len + j;
    }
    row += q.q_len;
  }
  // runs with the most units first (ties in list order): only the launch order
  {
    for (int64_t i = 0; i < n_runs; ++i) rl[size_t(i)] = {runs[2 * i], runs[2 * i + 1]};
    auto run_units = [&](const std::pair<int32_t, int32_t>& r) {
      return std::min<int64_t>(bi::kDecodeRun, units_of(dc[r.first].kv_len) - r.second);
    };
    std::stable_sort(rl.begin(), rl.end(), [&](const auto& a, const auto& b) { return run_units(a) > run_units(b); });
    for (int64_t i = 0; i < n_runs; ++i) {
      runs[2 * i] = rl[size_t(i)].first;
      runs[2 * i + 1] = rl[size_t(i)].second;
    }
  }
  // decode requests longest first (ties by index): only the launch order
  int32_t* order = at<int32_t>(host_meta, L.order);
  for (int i = 0; i < nd; ++i) order[i] = i;
  std::stable_sort(order, order + nd, [&](int32_t a, int32_t b) { return dc[a].kv_len > dc[b].kv_len; });
  return BI_OK;
}

bi_status bi_block_workspace(const bi_block_cfg* cfg, const bi_seq* seqs, int n_seqs,
                             bi_block_ws_layout* layout) {
  bi_status st = check_cfg(cfg);
  if (st != BI_OK) return st;
  StepSummary s;
  st = summarize(seqs, n_seqs, &s);
  if (st != BI_OK) return st;
  if (!layout) return BI_ERR_NULL;
  *layout = ws_layout(*cfg, s).pub;
  return BI_OK;
}

bi_status bi_block_forward(const bi_block_cfg* cfg, const bi_block_weights* w, const bi_seq* seqs,
                           int n_seqs, const void* d_meta, const bi_kv_pool* kv, const bi_bf16* x,
                           bi_bf16* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  bi_status st = check_cfg(cfg);
  if (st != BI_OK) return st;
  if (!w || !kv || !x || !y || !d_meta) return BI_ERR_NULL;
  StepSummary s;
  st = summarize(seqs, n_seqs, &s);
  if (st != BI_OK) return st;
  const bi_block_cfg& c = *cfg;
  const int fmt = c.weight_format;
  if (!w->gamma1) return BI_ERR_NULL;
  if ((st = check_weight(w->qkv, fmt)) != BI_OK) return st;
  if ((st = check_weight(w->o, fmt)) != BI_OK) return st;
  if (c.ffn) {
    if (!w->gamma2) return BI_ERR_NULL;
    if ((st = check_weight(w->gate_up, fmt)) != BI_OK) return st;
    if ((st = check_weight(w->down, fmt)) != BI_OK) return st;
    if (!aligned16(w->gamma2)) return BI_ERR_ALIGN;
  }
  if (!kv->k || !kv->v) return BI_ERR_NULL;
  if (kv->rows < 1) return BI_ERR_SHAPE;
  const int64_t kb = bi::kPrefillKeyBlock;  // page size of the paged cache
  if (paged(c)) {
    if (!kv->k_scale || !kv->v_scale || !kv->page_table) return BI_ERR_NULL;
    if (kv->rows % kb || kv->page_entries < 1) return BI_ERR_SHAPE;
    for (int i = 0; i < n_seqs; ++i)
      if (seqs[i].kv_base + (int64_t(seqs[i].ctx_len) + seqs[i].q_len + kb - 1) / kb > kv->page_entries)
        return BI_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(kv->k_scale) & 3u) || (reinterpret_cast<uintptr_t>(kv->v_scale) & 3u) ||
        (reinterpret_cast<uintptr_t>(kv->page_table) & 3u))
      return BI_ERR_ALIGN;
  } else {
    for (int i = 0; i < n_seqs; ++i)
      if (seqs[i].kv_base + int64_t(seqs[i].ctx_len) + seqs[i].q_len > kv->rows) return BI_ERR_SHAPE;
  }
  if (x == y) return BI_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y) || !aligned16(w->gamma1) || !aligned16(kv->k) ||
      !aligned16(kv->v) || !aligned16(d_meta) || !aligned16(ws))
    return BI_ERR_ALIGN;
  const WsLayout L = ws_layout(c, s);
  if (!ws || ws_bytes < L.pub.total) return BI_ERR_WORKSPACE;

  const int64_t M = s.M;
  const int H = c.hidden, Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim, F = c.ffn;
  const int qkv_n = (Hq + 2 * Hkv) * D;
  const int64_t n_runs = decode_runs(seqs, n_seqs);
  // every launch below must fit its grid: checked here, before the first one is enqueued
  if (M > kMaxRopeRows || M > kMaxNormRows) return BI_ERR_UNSUPPORTED;
  if (s.n_decode > kMaxGridYZ || s.n_prefill > kMaxGridYZ || Hkv > kMaxGridYZ) return BI_ERR_UNSUPPORTED;
  if (s.max_decode_len > kMaxDecodeLen || n_runs > kMaxDecodeRuns) return BI_ERR_UNSUPPORTED;
  int64_t max_tiles = 0;
  for (int i = 0; i < n_seqs; ++i)
    if (seqs[i].q_len > 1)
      max_tiles = std::max(max_tiles, prefill_tiles(seqs[i].ctx_len, seqs[i].q_len, Hq / Hkv));
  if (max_tiles > kMaxPrefillTiles) return BI_ERR_UNSUPPORTED;
  if ((st = gemm_shape(M, qkv_n, H)) != BI_OK || (st = gemm_shape(M, H, int64_t(Hq) * D)) != BI_OK) return st;
  if (F && ((st = gemm_shape(M, 2 * int64_t(F), H)) != BI_OK || (st = gemm_shape(M, H, F)) != BI_OK)) return st;
  const MetaLayout ML = meta_layout(n_seqs, M, n_runs);
  uint16_t* n1 = at<uint16_t>(ws, L.pub.n1);
  uint16_t* qkv = at<uint16_t>(ws, L.pub.qkv);
  uint16_t* q = at<uint16_t>(ws, L.pub.q);
  uint16_t* attn = at<uint16_t>(ws, L.pub.attn);
  uint16_t* h = F ? at<uint16_t>(ws, L.pub.h) : y;

  hipError_t e;
#define BI_TRY(expr)                   \
  do {                                 \
    e = (expr);                        \
    if (e != hipSuccess) return BI_ERR_HIP; \
  } while (0)
  BI_TRY(bi::launch_rmsnorm(x, w->gamma1, n1, M, H, c.eps, stream));
  BI_TRY(run_gemm(c, w->qkv, n1, qkv, M, qkv_n, H, stream));
  const float scale = float(1.0 / __builtin_sqrt(double(D)));
  if (paged(c)) {
    // rotated keys and the values go to the workspace (rows of the step), then into the
    // sequences' pages as int8 codes and scales; attention reads the pages
    uint16_t* k_new = at<uint16_t>(ws, L.pub.kv_new);
    uint16_t* v_new = k_new + M * Hkv * D;
    int8_t* kq = static_cast<int8_t*>(kv->k);
    int8_t* vq = static_cast<int8_t*>(kv->v);
    const int64_t n_pages = kv->rows / kb;
    BI_TRY(bi::launch_rope_kv(qkv, at<int32_t>(d_meta, ML.pos), nullptr, q, k_new, v_new, M, Hq, Hkv, D,
                              c.rope_theta, stream));
    BI_TRY(bi::launch_kv_quant_paged(k_new, v_new, at<int64_t>(d_meta, ML.kv), at<int32_t>(d_meta, ML.pos),
                                     kv->page_table, n_pages, M, Hkv, D, kq, vq, kv->k_scale, kv->v_scale, stream));
    if (s.n_prefill)
      BI_TRY(bi::launch_attn_prefill_q8(q, int64_t(Hq) * D, kq, vq, kv->k_scale, kv->v_scale, kv->page_table, n_pages,
                                        attn, int64_t(Hq) * D, at<PrefillSeq>(d_meta, ML.prefill), nullptr,
                                        s.n_prefill, int(max_tiles), Hq, Hkv, D, scale, stream));
    if (s.n_decode)
      BI_TRY(bi::launch_attn_decode_po_q8(q, int64_t(Hq) * D, kq, vq, kv->k_scale, kv->v_scale, kv->page_table, 0,
                                          n_pages, at<DecodeSeq>(d_meta, ML.decode), nullptr,
                                          at<int32_t>(d_meta, ML.order), s.n_decode, s.max_decode_len, Hq, Hkv, D,
                                          scale, attn, int64_t(Hq) * D, stream));
  } else {
    uint16_t* kc = static_cast<uint16_t*>(kv->k);
    uint16_t* vc = static_cast<uint16_t*>(kv->v);
    BI_TRY(bi::launch_rope_kv(qkv, at<int32_t>(d_meta, ML.pos), at<int64_t>(d_meta, ML.kv), q, kc,
                              vc, M, Hq, Hkv, D, c.rope_theta, stream));
    if (s.n_prefill) {
      BI_TRY(bi::launch_attn_prefill(q, int64_t(Hq) * D, kc, vc, attn, int64_t(Hq) * D,
                                     at<PrefillSeq>(d_meta, ML.prefill), nullptr, s.n_prefill,
                                     int(max_tiles), Hq, Hkv, D, scale, stream));
    }
    if (s.n_decode && c.decode_order == BI_DECODE_PREFILL_ORDER) {
      BI_TRY(bi::launch_attn_decode_po(q, int64_t(Hq) * D, kc, vc, at<DecodeSeq>(d_meta, ML.decode),
                                       nullptr, nullptr, at<int32_t>(d_meta, ML.order), s.n_decode,
                                       s.max_decode_len, Hq, Hkv, D, scale, attn, int64_t(Hq) * D, stream));
    } else if (s.n_decode) {
      BI_TRY(bi::launch_attn_decode(q, int64_t(Hq) * D, kc, vc, at<DecodeSeq>(d_meta, ML.decode),
                                    at<int2>(d_meta, ML.runs), int(n_runs), s.n_decode,
                                    s.max_decode_len, Hq, Hkv, D, scale,
                                    at<void>(ws, L.pub.decode_partials), attn, int64_t(Hq) * D,
                                    stream));
    }
  }
  BI_TRY(run_gemm(c, w->o, attn, h, M, H, int64_t(Hq) * D, stream, bi::kEpiResid, x));  // h = x + o
  if (F) {
    uint16_t* n2 = at<uint16_t>(ws, L.pub.n2);
    uint16_t* act = at<uint16_t>(ws, L.pub.act);
    BI_TRY(bi::launch_rmsnorm(h, w->gamma2, n2, M, H, c.eps, stream));
    if (ffn_fused(c)) {
      BI_TRY(run_gemm(c, w->gate_up, n2, act, M, F, H, stream, bi::kEpiGated));
    } else {
      uint16_t* gu = at<uint16_t>(ws, L.pub.gu);
      BI_TRY(run_gemm(c, w->gate_up, n2, gu, M, 2 * int64_t(F), H, stream));
      BI_TRY(bi::launch_swiglu(gu, act, M, F, stream));
    }
    BI_TRY(run_gemm(c, w->down, act, y, M, H, F, stream, bi::kEpiResid, h));  // y = h + d
  }
#undef BI_TRY
  return BI_OK;
}

}  // extern "C"
