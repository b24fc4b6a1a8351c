// Host-only stand-ins for the library's kernel launchers, for a sanitizer build of the
// C-ABI's argument checks (api.cpp) without a GPU.  Each stub records its name in a
// log and returns hipSuccess; no stub touches the pointers it is given.  The three
// size helpers return self-consistent values: the checks under test compare sizes
// against them, never the kernels' real layouts.
#include <string>
#include <vector>

#include "bi_internal.h"

std::vector<std::string> g_launches;

namespace bi {

static hipError_t logged(const char* name) {
  g_launches.emplace_back(name);
  return hipSuccess;
}

int gemm_tile_n(int64_t N, int epi) { return (epi != kEpiGated && N <= kGemmNarrowN) ? kGemmBNNarrow : kGemmBN; }
int gemm_w4_tile_n(int64_t N, int epi) { return (epi != kEpiGated && N <= kGemmW4NarrowN) ? kGemmBNNarrow : kGemmBN; }
int prefill_positions_per_tile(int group) { return 128 / group; }
size_t decode_workspace_bytes(int B, int64_t max_kv_len, int Hq, int D) {
  const int64_t runs = (max_kv_len + kKvSplit * kDecodeRun - 1) / (kKvSplit * kDecodeRun);
  return size_t(B) * Hq * runs * (D + 2) * 4 + size_t(B) * 32 + 4096;
}

hipError_t launch_rmsnorm(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int64_t, float, hipStream_t) {
  return logged("rmsnorm");
}
hipError_t launch_gemm_ex(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int64_t, int64_t, int64_t,
                          int epi, hipStream_t) {
  return logged(epi == kEpiResid ? "gemm_resid" : epi == kEpiGated ? "gemm_gated" : "gemm");
}
hipError_t launch_gemm_w4_ex(const uint8_t*, const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int64_t,
                             int64_t, int64_t, int epi, hipStream_t) {
  return logged(epi == kEpiResid ? "gemm_w4_resid" : epi == kEpiGated ? "gemm_w4_gated" : "gemm_w4");
}
hipError_t launch_gemm(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int64_t, int64_t, hipStream_t) {
  return logged("gemm");
}
hipError_t launch_gemm_w4(const uint16_t*, const uint8_t*, const uint16_t*, uint16_t*, int64_t, int64_t, int64_t,
                          hipStream_t) {
  return logged("gemm_w4");
}
hipError_t launch_add(const uint16_t*, const uint16_t*, uint16_t*, int64_t, hipStream_t) { return logged("add"); }
hipError_t launch_swiglu(const uint16_t*, uint16_t*, int64_t, int64_t, hipStream_t) { return logged("swiglu"); }
hipError_t launch_rope_kv(const uint16_t*, const int32_t*, const int64_t*, uint16_t*, uint16_t*, uint16_t*, int64_t,
                          int, int, int, double, hipStream_t) {
  return logged("rope_kv");
}
hipError_t launch_attn_prefill(const uint16_t*, int64_t, const uint16_t*, const uint16_t*, uint16_t*, int64_t,
                               const PrefillSeq*, const PrefillSeq*, int, int, int, int, int, float, hipStream_t) {
  return logged("prefill");
}
hipError_t launch_attn_decode(const uint16_t*, int64_t, const uint16_t*, const uint16_t*, const DecodeSeq*,
                              const int2*, int, int, int64_t, int, int, int, float, void*, uint16_t*, int64_t,
                              hipStream_t) {
  return logged("decode_split");
}
hipError_t launch_attn_decode_arrays(const uint16_t*, const uint16_t*, const uint16_t*, const int64_t*,
                                     const int32_t*, int, int64_t, int, int, int, float, void*, uint16_t*,
                                     hipStream_t) {
  return logged("decode_split");
}
hipError_t launch_attn_decode_noalloc(const uint16_t*, const uint16_t*, const uint16_t*, const int64_t*,
                                      const int32_t*, int, int64_t, int, int, int, float, uint16_t*, hipStream_t) {
  return logged("decode_noalloc");
}
hipError_t launch_attn_decode_po(const uint16_t*, int64_t, const uint16_t*, const uint16_t*, const DecodeSeq*,
                                 const int64_t*, const int32_t*, const int32_t*, int, int64_t, int, int, int, float,
                                 uint16_t*, int64_t, hipStream_t) {
  return logged("decode_po");
}
hipError_t launch_kv_quant(const uint16_t*, const uint16_t*, const int64_t*, int64_t, int, int, int8_t*, int8_t*,
                           float*, float*, hipStream_t) {
  return logged("kv_quant");
}
hipError_t launch_attn_prefill_q8(const uint16_t*, int64_t, const int8_t*, const int8_t*, const float*, const float*,
                                  const int32_t*, int64_t, uint16_t*, int64_t, const PrefillSeq*, const PrefillSeq*,
                                  int, int, int, int, int, float, hipStream_t) {
  return logged("prefill_q8");
}
hipError_t launch_attn_decode_po_q8(const uint16_t*, int64_t, const int8_t*, const int8_t*, const float*,
                                    const float*, const int32_t*, int, int64_t, const DecodeSeq*, const int32_t*,
                                    const int32_t*, int, int64_t, int, int, int, float, uint16_t*, int64_t,
                                    hipStream_t) {
  return logged("decode_po_q8");
}
hipError_t launch_kv_quant_paged(const uint16_t*, const uint16_t*, const int64_t*, const int32_t*, const int32_t*,
                                 int64_t, int64_t, int, int, int8_t*, int8_t*, float*, float*, hipStream_t) {
  return logged("kv_quant_paged");
}
hipError_t launch_sample(const uint16_t*, int64_t, int64_t, const BiSampling&, const uint64_t*, const int64_t*,
                         const int32_t*, int, int32_t*, hipStream_t) {
  return logged("sample");
}
hipError_t launch_token_hash(const int32_t*, const int64_t*, const int32_t*, int, uint8_t*, hipStream_t) {
  return logged("token_hash");
}
int token_hash_max_ids() { return 65536; }

}  // namespace bi
