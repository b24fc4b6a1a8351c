// Host-only exercise of the C-ABI's argument checks, step packing and block sequencing,
// built with the address and undefined-behaviour sanitizers together with api.cpp and
// the launcher stand-ins of launch_stubs.cpp.  Fake device addresses are never
// dereferenced (the stubs ignore them); host buffers are sized exactly, so an overrun
// is reported by the sanitizer.  Prints one line per section and "api_check ok".
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <string>
#include <vector>

#include "../../include/bi.h"

extern std::vector<std::string> g_launches;

static int g_checks = 0;
#define CHECK(cond)                                                            \
  do {                                                                         \
    ++g_checks;                                                                \
    if (!(cond)) {                                                             \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

template <class T>
static T* fake(uintptr_t a) { return reinterpret_cast<T*>(a); }

static bi_block_weights fake_weights(bool int4) {
  bi_block_weights w{};
  w.gamma1 = fake<bi_bf16>(0x10000);
  w.gamma2 = fake<bi_bf16>(0x20000);
  const bi_f16* sc = int4 ? fake<bi_f16>(0x30000) : nullptr;
  w.qkv = {fake<void>(0x40000), sc};
  w.o = {fake<void>(0x50000), sc};
  w.gate_up = {fake<void>(0x60000), sc};
  w.down = {fake<void>(0x70000), sc};
  return w;
}

static void checks_of_single_calls() {
  void* a = fake<void>(0x100000);
  void* b = fake<void>(0x200000);
  void* c = fake<void>(0x300000);
  bi_bf16* A = static_cast<bi_bf16*>(a);
  bi_bf16* B = static_cast<bi_bf16*>(b);
  bi_bf16* C = static_cast<bi_bf16*>(c);
  g_launches.clear();
  CHECK(bi_rmsnorm(nullptr, B, C, 4, 256, 1e-6f, 0) == BI_ERR_NULL);
  CHECK(bi_rmsnorm(A, B, C, 0, 256, 1e-6f, 0) == BI_ERR_SHAPE);
  CHECK(bi_rmsnorm(A, B, C, int64_t(1) << 26, 256, 1e-6f, 0) == BI_ERR_UNSUPPORTED);
  CHECK(bi_rmsnorm(A + 1, B, C, 4, 256, 1e-6f, 0) == BI_ERR_ALIGN);
  CHECK(bi_gemm(A, B, C, 7, 12, 64, 0) == BI_ERR_UNSUPPORTED);
  CHECK(bi_gemm(A, B, C, 7, 16, 65, 0) == BI_ERR_UNSUPPORTED);
  CHECK(bi_gemm(A, B, C, 7, 16, int64_t(1) << 23, 0) == BI_ERR_UNSUPPORTED);
  CHECK(bi_gemm_w4(A, fake<uint8_t>(0x200000), nullptr, C, 7, 16, 64, 0) == BI_ERR_NULL);
  CHECK(bi_gemm_swiglu(A, B, C, 7, 100, 64, 0) == BI_ERR_UNSUPPORTED);  // F % 128
  CHECK(bi_attn_prefill(A, B, C, A, 0, 0, 32, 8, 128, 0.1f, 0) == BI_ERR_SHAPE);
  CHECK(bi_attn_prefill(A, B, C, A, int64_t(1) << 31, 4, 32, 8, 128, 0.1f, 0) == BI_ERR_UNSUPPORTED);
  CHECK(bi_attn_decode(A, B, C, fake<int64_t>(0x400000), fake<int32_t>(0x500000), 70000, 100, 32, 8, 128, 0.1f, a,
                       size_t(1) << 40, C, 0) == BI_ERR_UNSUPPORTED);
  CHECK(bi_rope_kv(A, fake<int32_t>(0x400000), fake<int64_t>(0x500000), A, B, C, 1 << 24, 32, 8, 128, 1e6, 0) ==
        BI_ERR_UNSUPPORTED);
  bi_sampling sp{0.8f, 50, 0.95f, 0.05f, 1.f, 0.f, 0.f};
  CHECK(bi_sample(A, 4, 100, &sp, fake<uint64_t>(0x400000), fake<int64_t>(0x500000), nullptr, 0,
                  fake<int32_t>(0x600000), 0) == BI_ERR_UNSUPPORTED);  // vocab % 8
  sp.top_k = 2000;
  CHECK(bi_sample(A, 4, 128, &sp, fake<uint64_t>(0x400000), fake<int64_t>(0x500000), nullptr, 0,
                  fake<int32_t>(0x600000), 0) == BI_ERR_UNSUPPORTED);
  CHECK(g_launches.empty());
  // valid calls reach their launcher exactly once
  CHECK(bi_rmsnorm(A, B, C, 4, 256, 1e-6f, 0) == BI_OK);
  CHECK(bi_gemm(A, B, C, 7, 16, 64, 0) == BI_OK);
  CHECK(bi_gemm_residual(A, B, A, C, 7, 16, 64, 0) == BI_OK);
  CHECK(g_launches.size() == 3 && g_launches[0] == "rmsnorm" && g_launches[1] == "gemm" &&
        g_launches[2] == "gemm_resid");
  printf("single calls: %zu launches after the valid calls only\n", g_launches.size());
}

// Random steps: pack into exactly sized host buffers and check the packed header and run list.
static void step_pack_fuzz() {
  std::mt19937_64 rng(12345);
  int steps = 0;
  for (int it = 0; it < 3000; ++it) {
    const int n = 1 + int(rng() % (it % 10 == 0 ? 2000 : 40));
    std::vector<bi_seq> seqs(n);
    int64_t M = 0, n_dec = 0, n_pre = 0, runs = 0, base = 0;
    for (auto& s : seqs) {
      const bool dec = rng() % 3 != 0;
      s.q_len = dec ? 1 : 2 + int(rng() % 700);
      s.ctx_len = int(rng() % (rng() % 5 == 0 ? 40000 : 3000));
      s.kv_base = base;
      base += s.ctx_len + s.q_len + int64_t(rng() % 50);
      M += s.q_len;
      if (dec) {
        ++n_dec;
        const int64_t units = (int64_t(s.ctx_len) + 1 + 255) / 256;
        runs += (units + 7) / 8;
      } else {
        ++n_pre;
      }
    }
    const size_t bytes = bi_step_meta_bytes(seqs.data(), n);
    CHECK(bytes > 0);
    std::vector<unsigned char> buf(bytes);
    CHECK(bi_step_pack(seqs.data(), n, buf.data(), bytes - 1) == BI_ERR_WORKSPACE);
    CHECK(bi_step_pack(seqs.data(), n, buf.data(), bytes) == BI_OK);
    int64_t hdr[5];
    memcpy(hdr, buf.data(), sizeof hdr);
    CHECK(hdr[0] == n && hdr[1] == M && hdr[2] == n_pre && hdr[3] == n_dec && hdr[4] == runs);
    ++steps;
  }
  // invalid steps are rejected, never packed
  bi_seq bad[2] = {{1, 5, 0}, {0, 0, 100}};
  CHECK(bi_step_meta_bytes(bad, 2) == 0);
  unsigned char tmp[4096];
  CHECK(bi_step_pack(bad, 2, tmp, sizeof tmp) == BI_ERR_SHAPE);
  printf("step pack: %d random steps packed into exact buffers\n", steps);
}

static std::vector<std::string> block_launches(const bi_block_cfg& cfg, const std::vector<bi_seq>& seqs,
                                               int64_t rows, bi_status* st, int64_t page_entries = 0) {
  g_launches.clear();
  bi_block_ws_layout lay{};
  *st = bi_block_workspace(&cfg, seqs.data(), int(seqs.size()), &lay);
  if (*st != BI_OK) return g_launches;
  const bi_block_weights w = fake_weights(cfg.weight_format == BI_WEIGHTS_INT4_G32);
  bi_kv_pool pool{fake<void>(0x1000000), fake<void>(0x2000000), rows, nullptr, nullptr, nullptr, 0};
  if (page_entries) {
    pool.k_scale = fake<float>(0x7000000);
    pool.v_scale = fake<float>(0x7100000);
    pool.page_table = fake<int32_t>(0x7200000);
    pool.page_entries = page_entries;
  }
  *st = bi_block_forward(&cfg, &w, seqs.data(), int(seqs.size()), fake<void>(0x3000000), &pool,
                         fake<bi_bf16>(0x4000000), fake<bi_bf16>(0x5000000), fake<void>(0x6000000), lay.total, 0);
  return g_launches;
}

static std::string join(const std::vector<std::string>& v) {
  std::string s;
  for (const auto& x : v) s += (s.empty() ? "" : " ") + x;
  return s;
}

static void block_sequencing() {
  bi_block_cfg dense{2560, 32, 8, 128, 9728, 1e-6f, 1e6, BI_WEIGHTS_BF16, BI_DECODE_SPLIT, BI_KV_BF16};
  const std::vector<bi_seq> mixed = {{1, 700, 0}, {250, 250, 1000}, {1, 0, 5000}};
  bi_status st;
  auto l = block_launches(dense, mixed, 6000, &st);
  CHECK(st == BI_OK);
  CHECK(join(l) == "rmsnorm gemm rope_kv prefill decode_split gemm_resid rmsnorm gemm_gated gemm_resid");
  bi_block_cfg po = dense;
  po.decode_order = BI_DECODE_PREFILL_ORDER;
  CHECK(join(block_launches(po, mixed, 6000, &st)) ==
        "rmsnorm gemm rope_kv prefill decode_po gemm_resid rmsnorm gemm_gated gemm_resid");
  bi_block_cfg unfused = dense;
  unfused.ffn = 9664;  // not a multiple of 128: gate/up stored, SwiGLU separate
  CHECK(join(block_launches(unfused, mixed, 6000, &st)) ==
        "rmsnorm gemm rope_kv prefill decode_split gemm_resid rmsnorm gemm swiglu gemm_resid");
  bi_block_cfg int4 = dense;
  int4.hidden = 4096;
  int4.ffn = 12288;
  int4.weight_format = BI_WEIGHTS_INT4_G32;
  CHECK(join(block_launches(int4, mixed, 6000, &st)) ==
        "rmsnorm gemm_w4 rope_kv prefill decode_split gemm_w4_resid rmsnorm gemm_w4_gated gemm_w4_resid");
  bi_block_cfg tiny{256, 4, 4, 64, 0, 1e-6f, 0.0, BI_WEIGHTS_BF16, BI_DECODE_SPLIT, BI_KV_BF16};
  CHECK(join(block_launches(tiny, {{128, 0, 0}, {128, 0, 128}}, 256, &st)) == "rmsnorm gemm rope_kv prefill gemm_resid");
  // paged int8 cache: keys and values quantised into the pages, attention through them;
  // it pairs with the prefill-order decode only
  bi_block_cfg q8 = int4;
  q8.kv_format = BI_KV_INT8_PAGED;
  CHECK(block_launches(q8, mixed, 64 * 200, &st, 200).empty() && st == BI_ERR_UNSUPPORTED);
  q8.decode_order = BI_DECODE_PREFILL_ORDER;
  // entries: seq 0 from 0 (701 keys: 11 pages), seq 1 from 1000 (500: 8), seq 2 from 5000 (1: 1)
  CHECK(join(block_launches(q8, mixed, 64 * 200, &st, 5001)) ==
        "rmsnorm gemm_w4 rope_kv kv_quant_paged prefill_q8 decode_po_q8 gemm_w4_resid rmsnorm gemm_w4_gated "
        "gemm_w4_resid");
  CHECK(block_launches(q8, mixed, 64 * 200, &st, 5000).empty() && st == BI_ERR_SHAPE);  // seq 2's page missing
  CHECK(block_launches(q8, mixed, 64 * 200 + 1, &st, 5001).empty() && st == BI_ERR_SHAPE);  // rows not pages
  // rejected steps launch nothing
  std::vector<bi_seq> many(65536, bi_seq{1, 3, 0});
  for (size_t i = 0; i < many.size(); ++i) many[i].kv_base = int64_t(i) * 4;
  CHECK(block_launches(tiny, many, 1 << 20, &st).empty() && st == BI_ERR_UNSUPPORTED);
  CHECK(block_launches(dense, mixed, 5000, &st).empty() && st == BI_ERR_SHAPE);
  CHECK(block_launches(dense, {{1, 1 << 30, 0}}, int64_t(1) << 31, &st).empty() && st == BI_ERR_UNSUPPORTED);
  printf("block: launch order for split / prefill-order decode, fused / unfused FFN, int4, paged int8, no FFN\n");
}

int main() {
  checks_of_single_calls();
  step_pack_fuzz();
  block_sequencing();
  printf("api_check ok: %d checks\n", g_checks);
  return 0;
}
