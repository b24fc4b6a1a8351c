/*
 * bi.h -- batch-invariant transformer forward kernels for AMD MI355X (gfx950).
 *
 * What the library computes.  "Deterministic and bit-exact inference" (M-0002
 * record, field `technical`, the Invariance route, and its body section "How
 * it works") describes kernels that fix the reduction order of every output
 * element whatever the batch size, for RMSNorm, matrix multiplication and
 * attention -- the last with a fixed split *size* along the key/value axis
 * instead of a fixed number of splits.  The "Receipts" page (opening
 * paragraph) asks for outputs that do not depend on other requests in the
 * batch, on the prompt cache or on run-ahead, i.e. on chunked prefill; its
 * section "What a receipt proves" adds that bits are promised within one
 * device class and one build, and that parallel workers split rows, never
 * sums.  The M-0002 threat model ("No atomic functions") and its
 * "Residual nondeterminism" limitation rule out atomics, including in integer
 * de-quantisation.
 *
 * Contract of every entry point below.  With one build of this library on
 * gfx950, output row r depends only on row r's own inputs (for attention: on
 * the request's own keys/values and absolute positions).  It never depends on
 * the number of rows M, the batch size B, the row's position in the batch,
 * chunk boundaries of a prefill, KV-cache capacity, other requests, or on the
 * run.  No kernel uses atomic instructions, split-K or stream-K.
 *
 * Conventions.
 *  - bf16 / fp16 tensors are passed as raw 16-bit patterns (bi_bf16, bi_f16).
 *  - All tensors are row-major and dense (last index contiguous) in device
 *    memory, except where an argument is marked "host".
 *  - Device pointers must be 16-byte aligned; row lengths that are given in
 *    elements must keep every row 16-byte aligned where stated.
 *  - Accumulation is fp32; every bf16 output is rounded to nearest even.
 *  - Ownership: the caller allocates and owns every buffer (inputs, outputs,
 *    KV pools, workspaces).  The library allocates nothing and keeps no
 *    mutable global state; calls are reentrant and asynchronous on the given
 *    stream (0 = the null stream).  No call synchronises the device.
 *  - Errors: every argument check runs before anything is launched.  On an
 *    error the call returns a non-BI_OK status, launches nothing and leaves
 *    every output untouched.  A failed launch returns BI_ERR_HIP.  No C++
 *    exception crosses this interface.
 */
#ifndef BI_H_
#define BI_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t bi_bf16; /* raw bfloat16 bits */
typedef uint16_t bi_f16;  /* raw IEEE binary16 bits */

typedef enum {
  BI_OK = 0,
  BI_ERR_NULL = 1,        /* a required pointer is NULL */
  BI_ERR_SHAPE = 2,       /* a size is zero, negative or inconsistent */
  BI_ERR_UNSUPPORTED = 3, /* a size outside what the kernels implement */
  BI_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  BI_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  BI_ERR_HIP = 6          /* the HIP runtime reported a launch error */
} bi_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* bi_status_str(bi_status status);

/* Identifier of this build: 16 hex digits hashing the kernel sources and the
 * compiler flags.  Bits are promised only between calls of the same build on
 * the same device class ("Receipts", "What a receipt proves"). */
const char* bi_build_id(void);

/* The fixed key/value split size of decode attention: 256 keys. */
int bi_kv_split_size(void);

/* Compile-time tile shape of bi_gemm / bi_gemm_w4 (the same for every M):
 * writes BM, BN, BK into out[0..2] (256, 256, 64). */
void bi_gemm_tile(int out[3]);

/* Column-tile width the GEMMs use for a weight of N rows: 256, or 192 for
 * bf16 weights (weight_format BI_WEIGHTS_BF16) of at most 3072 rows and int4
 * weights of at most 4096 rows, where 256-wide tiles would leave many compute
 * units idle.  A function of the weight alone, never of M; the SwiGLU forms
 * always pair 128 gate and 128 up rows per tile.  Returns 0 for N < 1.  (No
 * element's bits depend on it.)                                             */
int bi_gemm_tile_cols(int64_t N, int weight_format);

/* ------------------------------------------------------------------ RMSNorm
 * y[r, j] = bf16( x[r, j] * rsqrt(sum_j x[r, j]^2 / hidden + eps) * gamma[j] )
 * (the RMSNorm of M-0002 `technical`).  One fixed fp32 reduction tree per row,
 * chosen from `hidden` alone.
 *   x     [rows, hidden] bf16      y [rows, hidden] bf16 (may not alias x)
 *   gamma [hidden] bf16
 *   1 <= rows <= 2^26 - 1024; hidden % 8 == 0, 8 <= hidden <= 16384;
 *   eps finite, >= 0.                                                        */
bi_status bi_rmsnorm(const bi_bf16* x, const bi_bf16* gamma, bi_bf16* y,
                     int64_t rows, int64_t hidden, float eps, hipStream_t stream);

/* --------------------------------------------------------------------- GEMM
 * C = A * W^T, fp32 accumulation, bf16 output (M-0002 `technical`: matrix
 * multiplication).  One tile shape for every M (see bi_gemm_tile and
 * bi_gemm_tile_cols), no split-K: each C[i, j] is accumulated over
 * k = 0..K-1 in the same order for every M and every position of row i.
 *   A [M, K] bf16   W [N, K] bf16   C [M, N] bf16 (must not alias A or W)
 *   M >= 1; N >= 8, N % 8 == 0; K >= 64, K % 64 == 0, K <= 2^22;
 *   M K and M N at most 2^40; fewer than 2^23 tiles of 256 x 192.           */
bi_status bi_gemm(const bi_bf16* A, const bi_bf16* W, bi_bf16* C,
                  int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* C = A * Wd^T with Wd de-quantised inside the kernel from symmetric int4:
 * Wd[j, k] = bf16(code[j, k] * Ws[j, k / 32]) where code[j, k] is the
 * two's-complement nibble (range -8..7) of byte Wq[j, k / 2], low nibble for
 * even k, high nibble for odd k.  De-quantisation is elementwise with no
 * atomics ("Residual nondeterminism" in the M-0002 limitations).  The result
 * is bit-identical to bi_gemm on the de-quantised weight.
 *   A [M, K] bf16   Wq [N, K/2] u8   Ws [N, K/32] fp16   C [M, N] bf16
 *   same size rules as bi_gemm.                                              */
bi_status bi_gemm_w4(const bi_bf16* A, const uint8_t* Wq, const bi_f16* Ws, bi_bf16* C,
                     int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* GEMMs with the block's elementwise step fused into their epilogue.  Each
 * element's reduction is the GEMM's (same MFMA chain, same tile for every M),
 * so the bits equal the GEMM followed by bi_add or bi_swiglu:
 *   bi_gemm_residual:  C = bf16(R + bf16(A W^T)), R and C [M, N] bf16 (C may
 *                      alias R); the residual connection of the block;
 *   bi_gemm_swiglu:    act[m, j] = bf16(silu(g) u), g = bf16((A W^T)[m, j]),
 *                      u = bf16((A W^T)[m, F + j]) for W [2F, K] (gate rows,
 *                      then up rows); act [M, F] bf16, F % 128 == 0 (the
 *                      tile pairs gate and up columns of the same outputs)
 *                      and (F + 128) K 2 < 2^32 (bf16 weights);
 *   _w4 forms: W given as int4 codes and fp16 scales as for bi_gemm_w4.
 * Other size rules as bi_gemm (for bi_gemm_swiglu with N = 2F).              */
bi_status bi_gemm_residual(const bi_bf16* A, const bi_bf16* W, const bi_bf16* R, bi_bf16* C,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream);
bi_status bi_gemm_swiglu(const bi_bf16* A, const bi_bf16* W, bi_bf16* act, int64_t M, int64_t F,
                         int64_t K, hipStream_t stream);
bi_status bi_gemm_w4_residual(const bi_bf16* A, const uint8_t* Wq, const bi_f16* Ws, const bi_bf16* R,
                              bi_bf16* C, int64_t M, int64_t N, int64_t K, hipStream_t stream);
bi_status bi_gemm_w4_swiglu(const bi_bf16* A, const uint8_t* Wq, const bi_f16* Ws, bi_bf16* act,
                            int64_t M, int64_t F, int64_t K, hipStream_t stream);

/* --------------------------------------------------------- elementwise steps
 * h[i] = bf16(x[i] + o[i]) for i < n (the residual connection).  n % 8 == 0.
 * h may alias x or o.                                                        */
bi_status bi_add(const bi_bf16* x, const bi_bf16* o, bi_bf16* h, int64_t n, hipStream_t stream);

/* act[r, j] = bf16(silu(g) * u), g = gu[r, j], u = gu[r, F + j], silu(g) =
 * g / (1 + exp(-g)).  gu [rows, 2F] bf16 (gate columns then up columns),
 * act [rows, F] bf16.  rows >= 1, F % 8 == 0.                               */
bi_status bi_swiglu(const bi_bf16* gu, bi_bf16* act, int64_t rows, int64_t F, hipStream_t stream);

/* --------------------------------------------------------- RoPE + KV append
 * For each token row r of qkv [rows, (Hq + 2 Hkv) * D] (query heads, then key
 * heads, then value heads, D contiguous per head):
 *   q_out[r, h, :] = RoPE(q[r, h, :], pos[r])            (h < Hq)
 *   k_pool[kv_row[r], g, :] = RoPE(k[r, g, :], pos[r])   (g < Hkv)
 *   v_pool[kv_row[r], g, :] = v[r, g, :]
 * RoPE rotates the pair (i, i + D/2), i < D/2, by pos * theta^(-2 i / D),
 * computed from the absolute position (so a prompt's keys do not depend on
 * how it was chunked: "Receipts", opening paragraph).  theta == 0 disables
 * the rotation (plain copy).
 *   1 <= rows < 2^24;  pos [rows] int32 device, >= 0;  kv_row [rows] int64 device, row index
 *   into the pools k_pool, v_pool [*, Hkv, D] bf16.  D in {64, 128};
 *   Hq % Hkv == 0.  The pools' sizes are not passed: every kv_row[r] must
 *   name a row of the pools (bi_block_forward checks its rows against
 *   bi_kv_pool.rows before any launch).                                     */
bi_status bi_rope_kv(const bi_bf16* qkv, const int32_t* pos, const int64_t* kv_row,
                     bi_bf16* q_out, bi_bf16* k_pool, bi_bf16* v_pool,
                     int64_t rows, int Hq, int Hkv, int D, double theta, hipStream_t stream);

/* ------------------------------------------------------- prefill attention
 * Causal attention of one sequence's chunk of T queries at absolute
 * positions q_start .. q_start + T - 1 over that sequence's cache:
 *   o[t, h, :] = bf16( sum_{s <= q_start + t} softmax_s(scale q[t,h,:].k[s,g,:]) v[s,g,:] )
 * with g = h / (Hq / Hkv).  Key blocks and query tiles are aligned to
 * absolute position 0, so every query visits the same key blocks in the same
 * order whatever the chunking ("Receipts", opening paragraph: independent of
 * the prompt cache and run-ahead).
 *   q [T, Hq * D] bf16; k_cache, v_cache [>= q_start + T, Hkv, D] bf16 with
 *   keys 0 .. q_start + T - 1 valid; o [T, Hq * D] bf16.
 *   T >= 1, q_start >= 0, q_start + T < 2^31, fewer than 2^23 query tiles
 *   (a tile is 128 / (Hq / Hkv) positions); D in {64, 128};
 *   Hq / Hkv in {1, 2, 4}; Hkv <= 65535.                                     */
bi_status bi_attn_prefill(const bi_bf16* q, const bi_bf16* k_cache, const bi_bf16* v_cache,
                          bi_bf16* o, int64_t q_start, int64_t T,
                          int Hq, int Hkv, int D, float scale, hipStream_t stream);

/* -------------------------------------------------------- decode attention
 * One query per request b over its L_b cached keys (the newest at position
 * L_b - 1), split into fixed 256-key units (M-0002 `technical`: a fixed split
 * size, not a fixed number of splits).  Unit s covers keys [256 s,
 * min(256 s + 256, L_b)) and is reduced on its own; units 8 r .. 8 r + 7 form
 * run r and are merged in ascending order (max, sum, weighted values in
 * fp32, one record per run and head in the workspace), and a second kernel
 * merges the runs of each request in ascending r.  The merge tree depends
 * only on L_b.
 *   q [B, Hq * D] bf16; k_all, v_all [sum L, Hkv, D] bf16 packed;
 *   kv_offset [B] int64 device: first row of request b in k_all / v_all;
 *   kv_len [B] int32 device: L_b, 1 <= L_b <= max_kv_len (a request outside
 *   that range gets NaN output, as the device cannot return an error);
 *   B >= 1 and max_kv_len >= 1 are host values used only to size the grid
 *   (B * ceil(max_kv_len / 2048) <= 2^24);
 *   D in {64, 128}; Hq / Hkv in {1, 2, 4, 8}; o [B, Hq * D] bf16.
 *   ws: device workspace of at least bi_attn_decode_workspace() bytes.       */
size_t bi_attn_decode_workspace(int B, int64_t max_kv_len, int Hq, int D);
bi_status bi_attn_decode(const bi_bf16* q, const bi_bf16* k_all, const bi_bf16* v_all,
                         const int64_t* kv_offset, const int32_t* kv_len,
                         int B, int64_t max_kv_len, int Hq, int Hkv, int D, float scale,
                         void* ws, size_t ws_bytes, bi_bf16* o, hipStream_t stream);

/* bi_attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and the same bits, with the workspace taken from a fixed
 * scratch array the library holds on each GPU (32 MiB, kept until the process
 * ends; its device address is looked up once per device, on the first call
 * with that device current).  Calls nothing that allocates.  Sizes whose
 * workspace (bi_attn_decode_workspace) exceeds 32 MiB return
 * BI_ERR_WORKSPACE -- e.g. 256 requests of up to 8192 keys (21 MB) and 64 of
 * up to 32768 keys (17 MB) fit.  All calls on one GPU share its scratch, so
 * calls that overlap in time on one GPU (other streams or threads) race and
 * must be ordered by the caller.  Other arguments and errors as
 * bi_attn_decode.                                                            */
bi_status bi_attn_decode_noalloc(const bi_bf16* q, const bi_bf16* k_all, const bi_bf16* v_all,
                                 const int64_t* kv_offset, const int32_t* kv_len,
                                 int B, int64_t max_kv_len, int Hq, int Hkv, int D, float scale,
                                 bi_bf16* o, hipStream_t stream);

/* ------------------------------------- decode attention in prefill key order
 * The same result as bi_attn_decode, computed with exactly the operations
 * bi_attn_prefill performs for a query at position L_b - 1 (its 64-key blocks
 * from position 0, two 32-key halves per block with an online softmax each,
 * the same sums in the same order), so a token decoded alone gets the bits
 * it gets when prefilled or verified inside a drafted chunk ("Receipts",
 * opening paragraph: independent of run-ahead drafting; M-0002 "Limitations":
 * speculative decoding is open work).  No workspace.
 *   q, k_all, v_all, kv_offset, kv_len, B, max_kv_len, o: as bi_attn_decode
 *   (a request whose length is outside 1..max_kv_len gets NaN output);
 *   order: optional device int32 [B], a permutation of 0..B-1 giving the
 *   order in which requests start (longest first shortens the step); NULL =
 *   ascending.  It never changes any request's result.
 *   D in {64, 128}; Hq / Hkv in {1, 2, 4, 8}.                                 */
bi_status bi_attn_decode_prefill_order(const bi_bf16* q, const bi_bf16* k_all, const bi_bf16* v_all,
                                       const int64_t* kv_offset, const int32_t* kv_len,
                                       const int32_t* order, int B, int64_t max_kv_len,
                                       int Hq, int Hkv, int D, float scale, bi_bf16* o,
                                       hipStream_t stream);

/* --------------------------------------------- quantised, paged KV cache
 * The "Receipts" page ("What a receipt proves") lists a quantised cache among
 * the load settings that decide the bits; the pages give no format.  Here:
 * int8 codes, symmetric, one float32 scale per (token, kv head): with
 * a = max |x_d| over the head, scale = a / 127, q_d = clamp(rint(x_d /
 * scale), -127, 127) (IEEE fp32 division, ties to even; a = 0 stores zeros);
 * attention reads bf16(float(q_d) * scale).  Pools are [rows, Hkv, D] int8
 * codes and [rows, Hkv] float32 scales, in pages of 64 rows; a sequence's
 * logical position p lives in row table[p / 64] * 64 + p % 64.  Everything a
 * query computes is the bf16 kernels' arithmetic on the dequantised values,
 * so results do not depend on page placement, batch or chunking.
 * Page indices are not range-checked on the device: every index in a table
 * must name a page of the pools.  D in {64, 128}.                            */

/* Quantise rows of bf16 keys and values [rows, Hkv, D] into pool rows
 * dst_row[r] (device int64 [rows]); 1 <= rows < 2^26, Hkv <= 65535.          */
bi_status bi_kv_append_q8(const bi_bf16* k, const bi_bf16* v, const int64_t* dst_row, int64_t rows,
                          int Hkv, int D, int8_t* k_pool, int8_t* v_pool, float* k_scale, float* v_scale,
                          hipStream_t stream);

/* bi_attn_prefill over a paged int8 cache: block_table (device int32) holds
 * at least ceil((q_start + T) / 64) page indices of the sequence.           */
bi_status bi_attn_prefill_paged_q8(const bi_bf16* q, const int8_t* k_pool, const int8_t* v_pool,
                                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                                   bi_bf16* o, int64_t q_start, int64_t T, int Hq, int Hkv, int D,
                                   float scale, hipStream_t stream);

/* bi_attn_decode_prefill_order over a paged int8 cache (bitwise equal to
 * bi_attn_prefill_paged_q8 for the same query): block_tables [B, max_pages]
 * int32 device with max_pages >= ceil(max_kv_len / 64); kv_len, order, B,
 * max_kv_len, o as there.                                                    */
bi_status bi_attn_decode_paged_q8(const bi_bf16* q, const int8_t* k_pool, const int8_t* v_pool,
                                  const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                  int max_pages, const int32_t* kv_len, const int32_t* order, int B,
                                  int64_t max_kv_len, int Hq, int Hkv, int D, float scale, bi_bf16* o,
                                  hipStream_t stream);

/* ------------------------------------------------- the step after the block
 * Seeded sampling of the next token for each row of logits (after the final
 * RMSNorm, bi_rmsnorm, and the LM head, bi_gemm with N = vocabulary), and
 * BLAKE3 hashes of token ids as a receipt records them ("Receipts", "Making a
 * receipt": prompt and output ids with their BLAKE3 over little-endian
 * 32-bit integers; the sampler settings and the seed).  A row's token depends
 * only on its logits, history, seed and position, never on the batch.
 * Sampler, per row:
 *   1. penalties (fp32) for each distinct history token: repeat
 *      (l > 0 ? l / r : l * r), then l - (presence + count * frequency);
 *   2. temperature 0: the largest logit, lowest id on ties;
 *   3. otherwise the top_k logits ordered by (logit desc, id asc); in fp64
 *      w = exp((l - l_max) / T); min-p keeps w >= min_p; top-p keeps the
 *      shortest prefix whose running sum reaches top_p of the total; the
 *      token is the first whose running sum exceeds u times the kept total,
 *      u = (first word of Philox4x64-10, key (seed, 0), counter
 *      (position, 0, 0, 0)) >> 11, times 2^-53.                              */
typedef struct {
  float temperature;       /* >= 0; 0 = greedy */
  int   top_k;             /* 1..1024 when temperature > 0 */
  float top_p;             /* (0, 1] */
  float min_p;             /* [0, 1) */
  float repeat_penalty;    /* > 0; 1 = off */
  float presence_penalty;  /* 0 = off */
  float frequency_penalty; /* 0 = off */
} bi_sampling;

/*   logits [rows, vocab] bf16, 16-byte aligned, vocab % 8 == 0, vocab <= 2^24
 *   (the LM head GEMM needs N % 8 == 0 as well);
 *   params: host; seeds [rows] uint64 and positions [rows] int64 (device);
 *   history [rows, n_hist] int32 device, 0 <= n_hist <= 256 (ids outside
 *   0..vocab-1 are ignored; may be NULL when n_hist == 0);
 *   out_ids [rows] int32 device.                                             */
bi_status bi_sample(const bi_bf16* logits, int64_t rows, int64_t vocab, const bi_sampling* params,
                    const uint64_t* seeds, const int64_t* positions, const int32_t* history,
                    int n_hist, int32_t* out_ids, hipStream_t stream);

/* BLAKE3 (hash mode, 32 bytes) of each sequence's ids as little-endian
 * 32-bit integers.  ids: device int32; offsets [n_seqs] int64 and counts
 * [n_seqs] int32 (device): sequence s is ids[offsets[s] .. + counts[s]).
 * out [n_seqs, 32] bytes (device).  A count outside 0..65536 (which the host
 * cannot see) gives an all-ones digest for that sequence.                    */
bi_status bi_token_hash(const int32_t* ids, const int64_t* offsets, const int32_t* counts, int n_seqs,
                        uint8_t* out, hipStream_t stream);

/* ------------------------------------------------------------ decoder block
 * One forward step of a pre-norm decoder block over a batch of sequences:
 *   n1 = RMSNorm(x, gamma1); qkv = n1 Wqkv^T; q, k = RoPE(q, k); append k, v;
 *   a = Attn(q, cache); o = a Wo^T; h = x + o;
 *   [FFN] n2 = RMSNorm(h, gamma2); gu = n2 Wgu^T; act = silu(g) u;
 *         d = act Wdown^T; y = h + d      (without FFN, y = h)
 * with a bf16 rounding at every arrow.  Sequences with q_len == 1 use decode
 * attention (bi_attn_decode, or bi_attn_decode_prefill_order when
 * decode_order is BI_DECODE_PREFILL_ORDER); longer ones use prefill
 * attention.                                                                */
typedef enum { BI_WEIGHTS_BF16 = 0, BI_WEIGHTS_INT4_G32 = 1 } bi_weight_format;
typedef enum { BI_DECODE_SPLIT = 0, BI_DECODE_PREFILL_ORDER = 1 } bi_decode_order;
/* KV cache of the block: contiguous bf16 rows per sequence, or the quantised,
 * paged int8 cache of bi_kv_append_q8 ("Receipts", "What a receipt proves":
 * a quantised cache is one of the load settings that decide the bits). */
typedef enum { BI_KV_BF16 = 0, BI_KV_INT8_PAGED = 1 } bi_kv_format;

typedef struct {
  int hidden;        /* H, % 8 == 0 */
  int n_q_heads;     /* Hq */
  int n_kv_heads;    /* Hkv, Hq / Hkv in {1, 2, 4} */
  int head_dim;      /* D in {64, 128} */
  int ffn;           /* F (% 64 == 0), or 0 for a block without FFN */
  float eps;         /* RMSNorm epsilon */
  double rope_theta; /* 0 = no rotary embedding */
  int weight_format; /* bi_weight_format */
  int decode_order;  /* bi_decode_order: fixed 256-key split (default), or the
                        prefill kernel's key order (decoded bits = prefilled) */
  int kv_format;     /* bi_kv_format; BI_KV_INT8_PAGED needs
                        decode_order == BI_DECODE_PREFILL_ORDER */
} bi_block_cfg;

typedef struct {
  const void* w;       /* bf16 [N, K], or int4 packed u8 [N, K/2] */
  const bi_f16* scale; /* int4 only: fp16 [N, K/32]; NULL for bf16 */
} bi_weight;

typedef struct {
  const bi_bf16* gamma1; /* [H] */
  const bi_bf16* gamma2; /* [H] (FFN only) */
  bi_weight qkv;         /* N = (Hq + 2 Hkv) D, K = H; rows: q heads, k heads, v heads */
  bi_weight o;           /* N = H, K = Hq D */
  bi_weight gate_up;     /* N = 2F, K = H; rows 0..F-1 gate, F..2F-1 up (FFN only) */
  bi_weight down;        /* N = H, K = F (FFN only) */
} bi_block_weights;

typedef struct {
  int32_t q_len;   /* new tokens of this sequence in the step (>= 1) */
  int32_t ctx_len; /* tokens already in its cache (>= 0) */
  int64_t kv_base; /* bf16 pools: pool row holding its position 0; paged int8
                      pools: first entry of the sequence's pages in
                      bi_kv_pool.page_table (position p lives in pool row
                      page_table[kv_base + p / 64] * 64 + p % 64) */
} bi_seq;

typedef struct {
  void* k;                   /* bf16 [rows, Hkv, D]; paged int8: codes [rows, Hkv, D] */
  void* v;                   /* as k */
  int64_t rows;              /* capacity of the pools in token rows (paged: pages * 64) */
  float* k_scale;            /* paged int8 only: fp32 [rows, Hkv]; NULL for bf16 */
  float* v_scale;            /* paged int8 only: fp32 [rows, Hkv]; NULL for bf16 */
  const int32_t* page_table; /* paged int8 only: device int32 page indices, every one
                                in 0 .. rows / 64 - 1 (an index outside is clamped
                                into the pool when read and skipped when written:
                                memory stays in bounds, results are then undefined) */
  int64_t page_entries;      /* paged int8 only: entries in page_table */
} bi_kv_pool;

/* Step metadata.  The kernels read a packed device copy of the step
 * description; bi_step_pack writes it into caller host memory, and the caller
 * uploads those bytes to device memory (e.g. through pinned memory) and
 * passes the device address to bi_block_forward together with the same host
 * bi_seq array.  This keeps every call free of hidden synchronisation.      */
size_t bi_step_meta_bytes(const bi_seq* seqs, int n_seqs); /* 0 if the step is invalid */
bi_status bi_step_pack(const bi_seq* seqs, int n_seqs, void* host_meta, size_t bytes);

/* Offsets (bytes into the block workspace) of every intermediate stage, for
 * inspection after a call: each is bf16 row-major [M, width].  Entries of a
 * stage the block does not store are SIZE_MAX: the FFN stages without an FFN,
 * and o, d (always) and gu (when F % 128 == 0), which exist only inside the
 * fused GEMM epilogues (bi_gemm[_w4]_residual / _swiglu).                   */
typedef struct {
  size_t n1, qkv, q, attn, o, h, n2, gu, act, d;
  size_t kv_new;  /* paged int8 pools: the step's rotated keys, then its values,
                     bf16 [2, M, Hkv, D] before quantisation; else SIZE_MAX */
  size_t decode_partials;
  size_t total;
} bi_block_ws_layout;

bi_status bi_block_workspace(const bi_block_cfg* cfg, const bi_seq* seqs, int n_seqs,
                             bi_block_ws_layout* layout);

/*   seqs / n_seqs: host description of the step (>= 1 sequence); rows of x
 *     and y are the sequences' new tokens concatenated in order (M = sum of
 *     q_len).  d_meta: device copy of bi_step_pack(seqs) output.
 *   kv: pools updated in place at rows kv_base + ctx_len .. + q_len - 1;
 *     rows kv_base .. kv_base + ctx_len - 1 must hold the cached keys/values.
 *     Paged int8 pools (cfg.kv_format): the step's keys and values are
 *     quantised (bi_kv_append_q8) into positions ctx_len .. + q_len - 1 of
 *     each sequence's pages, and attention reads bf16(code * scale) through
 *     the page table (bi_attn_prefill_paged_q8, bi_attn_decode_paged_q8):
 *     kv_base + ceil((ctx_len + q_len) / 64) <= page_entries.
 *   x, y [M, H] bf16 (y may not alias x).  ws: >= layout.total bytes.
 *   Limits (BI_ERR_UNSUPPORTED, checked before the first launch): M < 2^24;
 *   at most 65535 decode and 65535 prefill sequences; decode lengths up to
 *   2^30 keys; every GEMM within bi_gemm's limits.                          */
bi_status bi_block_forward(const bi_block_cfg* cfg, const bi_block_weights* w,
                           const bi_seq* seqs, int n_seqs, const void* d_meta,
                           const bi_kv_pool* kv, const bi_bf16* x, bi_bf16* y,
                           void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_H_ */
