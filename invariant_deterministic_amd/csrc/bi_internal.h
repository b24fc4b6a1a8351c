// Internal launchers of the library (host side).  Arguments are assumed to
// have passed the checks of api.cpp; each launcher only enqueues kernels on
// the given stream and returns the launch status.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace bi {

// GEMM tile shape: one shape for every M (no split-K).  bf16 weights of at most
// kGemmNarrowN rows (outside the gated form) use kGemmBNNarrow-wide column tiles.
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;
constexpr int kGemmBK = 64;
constexpr int kGemmBNNarrow = 192;
constexpr int64_t kGemmNarrowN = 3072;
// operand offsets of the bf16 schedule are 32-bit from the tile's first rows
constexpr int64_t kGemmMaxK = int64_t(1) << 22;
// column-tile width of the bf16 GEMM for a weight of N rows (epi: kEpi*)
int gemm_tile_n(int64_t N, int epi);
// int4 weights of at most kGemmW4NarrowN rows use kGemmBNNarrow-wide column tiles
constexpr int64_t kGemmW4NarrowN = 4096;
int gemm_w4_tile_n(int64_t N, int epi);

// Decode attention: fixed key/value split size.
constexpr int kKvSplit = 256;
// split decode: units 8 r .. 8 r + 7 of a request form run r; a run's units are
// merged first (ascending), then the runs (ascending)
constexpr int kDecodeRun = 8;

// Prefill attention: key block size (blocks are aligned to absolute position 0).
constexpr int kPrefillKeyBlock = 64;

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, uint16_t* y, int64_t rows,
                          int64_t hidden, float eps, hipStream_t s);

// GEMM epilogues (see gemm.hip): plain C = A W^T; residual C = R + A W^T (R [M, N]); gated
// C = swiglu(A W_gate^T, A W_up^T) with W = [gate; up] of 2N rows and N % 128 == 0
enum : int { kEpiPlain = 0, kEpiResid = 1, kEpiGated = 2 };
hipError_t launch_gemm_ex(const uint16_t* A, const uint16_t* W, const uint16_t* R, uint16_t* C, int64_t M,
                          int64_t N, int64_t K, int epi, hipStream_t s);
hipError_t launch_gemm_w4_ex(const uint8_t* Wq, const uint16_t* Ws, const uint16_t* A, const uint16_t* R,
                             uint16_t* C, int64_t M, int64_t N, int64_t K, int epi, hipStream_t s);
hipError_t launch_gemm(const uint16_t* A, const uint16_t* W, uint16_t* C, int64_t M, int64_t N,
                       int64_t K, hipStream_t s);
hipError_t launch_gemm_w4(const uint16_t* A, const uint8_t* Wq, const uint16_t* Ws, uint16_t* C,
                          int64_t M, int64_t N, int64_t K, hipStream_t s);

hipError_t launch_add(const uint16_t* x, const uint16_t* o, uint16_t* h, int64_t n, hipStream_t s);
hipError_t launch_swiglu(const uint16_t* gu, uint16_t* act, int64_t rows, int64_t F, hipStream_t s);

hipError_t launch_rope_kv(const uint16_t* qkv, const int32_t* pos, const int64_t* kv_row,
                          uint16_t* q_out, uint16_t* k_pool, uint16_t* v_pool, int64_t rows,
                          int Hq, int Hkv, int D, double theta, hipStream_t s);

// Multi-sequence prefill attention.  Sequence descriptors live in device
// memory (PrefillSeq array d_seqs), or, for one sequence, are passed by value
// (d_seqs == nullptr, h_single != nullptr).  The host passes the largest
// number of query tiles any sequence needs, for the grid only.
struct PrefillSeq {
  int64_t q_row;     // first row of the sequence's queries in q / o
  int64_t kv_base;   // cache row of the sequence's position 0
  int32_t q_start;   // absolute position of its first query
  int32_t q_len;     // number of queries (>= 1)
};
int prefill_positions_per_tile(int group);
hipError_t launch_attn_prefill(const uint16_t* q, int64_t q_row_stride, const uint16_t* k_cache,
                               const uint16_t* v_cache, uint16_t* o, int64_t o_row_stride,
                               const PrefillSeq* d_seqs, const PrefillSeq* h_single, int n_seqs,
                               int max_tiles, int Hq, int Hkv, int D, float scale, hipStream_t s);

// Decode attention.  Per request: query row, cache offset and length in
// device memory.
struct DecodeSeq {
  int64_t q_row;      // row of the request's query in q / o
  int64_t kv_offset;  // cache row of the request's key 0
  int32_t kv_len;     // number of keys (>= 1)
  int32_t pad;
};
size_t decode_workspace_bytes(int B, int64_t max_kv_len, int Hq, int D);
// d_runs: device list of (request, first unit) pairs, one per run of up to
// kDecodeRun units (n_runs of them, each run of each request exactly once).
hipError_t launch_attn_decode(const uint16_t* q, int64_t q_row_stride, const uint16_t* k_all,
                              const uint16_t* v_all, const DecodeSeq* d_seqs, const int2* d_runs,
                              int n_runs, int B, int64_t max_kv_len, int Hq, int Hkv, int D,
                              float scale, void* ws, uint16_t* o, int64_t o_row_stride,
                              hipStream_t s);
// Variant for the standalone entry point: separate offset / length arrays.
hipError_t launch_attn_decode_arrays(const uint16_t* q, const uint16_t* k_all,
                                     const uint16_t* v_all, const int64_t* kv_offset,
                                     const int32_t* kv_len, int B, int64_t max_kv_len, int Hq,
                                     int Hkv, int D, float scale, void* ws, uint16_t* o,
                                     hipStream_t s);
// The same with the library's own per-device scratch (kDecodeScratchBytes) as workspace:
// allocates nothing.  Fails with hipErrorInvalidValue when the workspace would not fit.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t launch_attn_decode_noalloc(const uint16_t* q, const uint16_t* k_all, const uint16_t* v_all,
                                      const int64_t* kv_offset, const int32_t* kv_len, int B, int64_t max_kv_len,
                                      int Hq, int Hkv, int D, float scale, uint16_t* o, hipStream_t s);

// Decode attention in the prefill kernel's key order (bitwise equal to prefill
// for the same query).  Request descriptors come from d_seqs, or, when d_seqs
// is nullptr, from the offset / length arrays with q_row = b.  d_order
// (optional) is a permutation of 0..B-1: the launch order of the requests.
hipError_t launch_attn_decode_po(const uint16_t* q, int64_t q_row_stride, const uint16_t* k_all,
                                 const uint16_t* v_all, const DecodeSeq* d_seqs, const int64_t* kv_offset,
                                 const int32_t* kv_len, const int32_t* d_order, int B, int64_t max_kv_len,
                                 int Hq, int Hkv, int D, float scale, uint16_t* o, int64_t o_row_stride,
                                 hipStream_t s);

// Quantised, paged KV cache: int8 codes [rows, Hkv, D] with float32 scales
// [rows, Hkv]; pages of 64 rows; page tables are int32.
hipError_t launch_kv_quant(const uint16_t* k, const uint16_t* v, const int64_t* dst_row, int64_t rows, int Hkv,
                           int D, int8_t* kq, int8_t* vq, float* ks, float* vs, hipStream_t s);
// Paged int8 attention.  pages: page indices; a sequence's entries start at its
// PrefillSeq / DecodeSeq kv_base / kv_offset (d_seqs given), else at 0 (prefill, one
// sequence by value) or b * max_pages (decode, per-request tables).  Page indices outside
// 0 .. n_pages - 1 are clamped into the pool.
hipError_t launch_attn_prefill_q8(const uint16_t* q, int64_t q_row_stride, const int8_t* k_pool, const int8_t* v_pool,
                                  const float* k_scale, const float* v_scale, const int32_t* pages, int64_t n_pages,
                                  uint16_t* o, int64_t o_row_stride, const PrefillSeq* d_seqs,
                                  const PrefillSeq* h_single, int n_seqs, int max_tiles, int Hq, int Hkv, int D,
                                  float scale, hipStream_t s);
hipError_t launch_attn_decode_po_q8(const uint16_t* q, int64_t q_row_stride, const int8_t* k_pool,
                                    const int8_t* v_pool, const float* k_scale, const float* v_scale,
                                    const int32_t* block_tables, int max_pages, int64_t n_pages,
                                    const DecodeSeq* d_seqs, const int32_t* kv_len, const int32_t* d_order, int B,
                                    int64_t max_kv_len, int Hq, int Hkv, int D, float scale, uint16_t* o,
                                    int64_t o_row_stride, hipStream_t s);
// Paged int8 append: token r (bf16 k, v rows r of [rows, Hkv, D]) at position pos[r] of a
// sequence whose table entries start at entry_plus_pos[r] - pos[r].  A page index outside
// the pool writes nothing.
hipError_t launch_kv_quant_paged(const uint16_t* k, const uint16_t* v, const int64_t* entry_plus_pos,
                                 const int32_t* pos, const int32_t* pages, int64_t n_pages, int64_t rows, int Hkv,
                                 int D, int8_t* kq, int8_t* vq, float* ks, float* vs, hipStream_t s);

// Sampler settings (mirrors bi_sampling of the public header).
struct BiSampling {
  float temperature;
  int top_k;
  float top_p, min_p, repeat, presence, frequency;
};
hipError_t launch_sample(const uint16_t* logits, int64_t rows, int64_t vocab, const BiSampling& prm,
                         const uint64_t* seeds, const int64_t* positions, const int32_t* history, int n_hist,
                         int32_t* out, hipStream_t s);
hipError_t launch_token_hash(const int32_t* ids, const int64_t* offsets, const int32_t* counts, int n_seqs,
                             uint8_t* out, hipStream_t s);
int token_hash_max_ids();

}  // namespace bi
