// Batch-invariant GEMM C = A * W^T for gfx950 (bf16 weights, and int4 weights
// de-quantised inside the kernel).
//
// Matrix multiplication is one of the operations the M-0002 record
// ("Deterministic and bit-exact inference", field `technical`) makes
// batch-invariant.  The invariance argument here:
//  * one tile shape and one instruction stream for every M: 256 x 256 x 64, or
//    256 x 192 x 64 for bf16 weights of at most 3072 rows and int4 weights of at
//    most 4096 rows (the width is a function of the weight alone); there is no M-dependent
//    dispatch, no split-K and no stream-K, and rows past M are handled by
//    clamping their loads and masking their stores in the same instruction
//    stream (a wave whose 128 rows all lie past M skips its MFMAs: padding
//    work only);
//  * each C[i, j] is accumulated by one lane of one MFMA chain: K is walked in
//    64-wide steps in ascending order, each step as four 16-deep
//    v_mfma_f32_32x32x16_bf16 instructions in ascending order;
//  * the MFMA unit treats every (row, column) slot of its 32 x 32 block the
//    same way, so the bits of C[i, :] do not depend on which tile row or
//    which slot row i lands in, nor on the column-tile width.
// The tests check the last point empirically (every row at every position, and
// the 256-wide int4 GEMM against the 192-wide bf16 GEMM on the same weight).
//
// Int4 weights ("Residual nondeterminism" in the M-0002 limitations warns of
// de-quantisation kernels with atomic additions): each thread expands the two
// 32-element groups of one weight tile row per K step -- code * fp16 scale, exact
// in fp32, one rounding to bf16 -- with plain stores into the same LDS tile layout
// the bf16 path uses, so the int4 GEMM is
// bit-identical to the bf16 GEMM on the de-quantised weight.  The expansion
// takes ~2.4 VALU instructions per element (two codes per bit operation as fp16
// pairs, one mixed-precision fma each, one packed bf16 conversion per pair).
//
// Schedule (both kernels).  Four waves, one per SIMD, each owning a 128 x BNT/2
// block of the tile (256 accumulator registers): 0.5 LDS fragment reads per MFMA
// against 0.75 for eight 64-row waves.  Operand tiles sit in LDS in two stages
// (16-byte chunks xor-swizzled by row pair, so ds_read_b128 is conflict-free),
// each stage a separate array so the compiler can tell the loads in flight from
// the reads; one barrier per 64-deep K step.  The activation tile (and the bf16
// weight tile) goes from global memory straight into LDS (global_load_lds_dwordx4,
// no staging registers), a stage ahead.  Int4 weights: each thread owns one weight
// tile row, loads its codes and scales into registers two stages ahead and
// de-quantises them into the free LDS stage one stage ahead.  The wave issues,
// between the MFMAs of each 16-deep substep, the next substep's fragment reads and
// the next stages' loads and de-quantisation in a fixed interleaved order: issued
// in one burst, the loads held up the in-order MFMA stream behind them.  MFMA
// operand A is the weight tile, operand B the activation tile, so each lane ends
// with 4 consecutive output columns of one output row and stores them as one
// 8-byte write.  Operand offsets are 32-bit and relative to the tile's first rows,
// so one schedule serves every operand size.
#include <type_traits>
#include <utility>

#include "bi_dev.h"
#include "bi_internal.h"

namespace bi {
namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int NT4 = 256;                // 4 waves, 2 along N x 2 along M (128 rows each), one per SIMD
constexpr int TILE = BM * BK;           // bf16 elements of one operand tile (BM == BN)
static_assert(BM == BN, "square tile assumed by the LDS layout");

// Work-group -> tile.  Work-groups are dealt round-robin to the 8 XCDs (work-group
// wg runs on XCD wg % 8), each XCD has its own L2.  Tiles are put in a grouped
// order -- kTileGroup tile rows at a time, column by column inside the group -- and
// each XCD takes a contiguous run of that order, so the ~32 tiles an XCD runs at
// once span a few tile rows and a few tile columns and share both their A and their
// W slices in that L2.  Only whole tiles move between work-groups: no element's
// arithmetic depends on this.
constexpr int kTileGroup = 4;
__device__ __forceinline__ int tile_of(int wg, int n_tiles, int tiles_n) {
  const int q = n_tiles / 8, r = n_tiles % 8, x = wg % 8;
  const int i = x * q + min(x, r) + wg / 8;  // XCD x holds q (+1 if x < r) consecutive positions
  const int tiles_m = n_tiles / tiles_n;
  const int g = i / (kTileGroup * tiles_n), rem = i % (kTileGroup * tiles_n);
  const int rows = min(kTileGroup, tiles_m - g * kTileGroup);
  return (g * kTileGroup + rem % rows) * tiles_n + rem / rows;
}

// Element offset of 16-byte chunk `chunk` (0..7) of tile row `row`.  LDS
// serves 16 lanes of a 16-byte access per cycle from 64 four-byte banks, i.e.
// two 128-byte rows; keying the xor on row / 2 puts the 16 rows a fragment
// read touches per cycle (and the two rows a tile store touches) on 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// De-quantise 8 int4 codes (one little-endian word; nibble e is element e) with the
// group's scale s: w_e = bf16(code_e * s), code_e the two's-complement nibble.  Each
// code becomes the fp16 value 1024 + 8 + code (the exponent field of 1024, the nibble with
// its top bit flipped in the low mantissa bits: two codes per word op, no conversion
// instruction), then fma(1024 + 8 + code, s, -1032 s) = code * s exactly in fp32 (the
// product has at most 15 significant bits, -1032 s at most 19; one rounding of an exact
// value), rounded once to bf16: the bits of bf16(float(code) * s).
// sc = s as fp32, nb = -1032 * sc (exact).
__device__ __forceinline__ uint4 dequant8(uint32_t word, float sc, float nb) {
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // the fp16 pair (1024 + 8 + code_j, 1024 + 8 + code_{j+4})
    const f16x2 p = __builtin_bit_cast(f16x2, ((word >> (4 * j)) & 0x000F000Fu) ^ 0x64086408u);
    f[j] = __builtin_fmaf(float(p[0]), sc, nb);
    f[j + 4] = __builtin_fmaf(float(p[1]), sc, nb);
  }
  return make_uint4(pack2bf(f[0], f[1]), pack2bf(f[2], f[3]), pack2bf(f[4], f[5]), pack2bf(f[6], f[7]));
}

// Epilogues.  kEpiPlain: C = bf16(acc).  kEpiResid: C = bf16(R + bf16(acc)), the residual
// add of the block fused into its GEMM (same roundings as the GEMM then the add).
// kEpiGated: C[m][j] = bf16(swiglu(bf16(gate acc), bf16(up acc))) for the gate/up GEMM with
// W = [gate rows 0 .. F - 1; up rows F .. 2F - 1]: a column tile covers outputs
// 128 tn .. 128 tn + 127 and holds, in the blocks 0, 1 of the wave owning tile rows
// 128 wn .. 128 wn + 127, the gate columns 64 wn + 32 b + i and in its blocks 2, 3 the up
// columns of the same outputs, so a lane has both inputs of each of its outputs.  Every
// element's MFMA chain is the same as in the plain GEMM: the bits of the fused forms equal
// the GEMM followed by the elementwise kernel.
// W row behind tile row t of column tile tn (F: the gated GEMM's output width)
template <int EPI, int BNT = BN>
__device__ __forceinline__ int w_row(int tn, int t, int F) {
  if constexpr (EPI == kEpiGated) return ((t >> 6) & 1) * F + tn * 128 + ((t >> 7) << 6) + (t & 63);
  else return tn * BNT + t;
}

// acc[bn][bm][r] is C element (row row0 + bm*32 + (lane & 31), column tn*BNT + wn*(BNT/2) +
// bn*32 + 8*(r/4) + 4*(lane/32) + r%4) of a wave's NBR 32-row blocks of a BM x BNT tile; C has
// N columns (the gated form: N = F outputs, BNT = 256)
template <int EPI, int BNT, int NBR>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[BNT / 64][NBR], uint16_t* C,
                                           const uint16_t* R, int M, int N, int row0, int tn,
                                           int wn, int lane) {
  static_assert(EPI != kEpiGated || BNT == 256, "the gated epilogue pairs 128-column halves of a 256 tile");
#pragma unroll
  for (int bm = 0; bm < NBR; ++bm) {
    const int m = row0 + bm * 32 + (lane & 31);
    if (m >= M) continue;
    uint16_t* crow = C + int64_t(m) * N;
    if constexpr (EPI == kEpiGated) {
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = tn * 128 + wn * 64 + bn * 32 + 8 * q + 4 * (lane >> 5);
          const uint32_t g01 = pack2bf(acc[bn][bm][4 * q + 0], acc[bn][bm][4 * q + 1]);
          const uint32_t g23 = pack2bf(acc[bn][bm][4 * q + 2], acc[bn][bm][4 * q + 3]);
          const uint32_t u01 = pack2bf(acc[bn + 2][bm][4 * q + 0], acc[bn + 2][bm][4 * q + 1]);
          const uint32_t u23 = pack2bf(acc[bn + 2][bm][4 * q + 2], acc[bn + 2][bm][4 * q + 3]);
          uint2 v;
          v.x = pack2bf(swiglu1(bf2f_lo(g01), bf2f_lo(u01)), swiglu1(bf2f_hi(g01), bf2f_hi(u01)));
          v.y = pack2bf(swiglu1(bf2f_lo(g23), bf2f_lo(u23)), swiglu1(bf2f_hi(g23), bf2f_hi(u23)));
          *reinterpret_cast<uint2*>(crow + j) = v;
        }
      }
    } else {
#pragma unroll
      for (int bn = 0; bn < BNT / 64; ++bn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = tn * BNT + wn * (BNT / 2) + bn * 32 + 8 * q + 4 * (lane >> 5);
          if (n < N) {
            uint2 v;
            v.x = pack2bf(acc[bn][bm][4 * q + 0], acc[bn][bm][4 * q + 1]);
            v.y = pack2bf(acc[bn][bm][4 * q + 2], acc[bn][bm][4 * q + 3]);
            if constexpr (EPI == kEpiResid) {
              const uint2 x = *reinterpret_cast<const uint2*>(R + int64_t(m) * N + n);
              v.x = pack2bf(resid1(bf2f_lo(x.x), bf2f_lo(v.x)), resid1(bf2f_hi(x.x), bf2f_hi(v.x)));
              v.y = pack2bf(resid1(bf2f_lo(x.y), bf2f_lo(v.y)), resid1(bf2f_hi(x.y), bf2f_hi(v.y)));
            }
            *reinterpret_cast<uint2*>(crow + n) = v;
          }
        }
      }
    }
  }
}

// s_waitcnt immediate (gfx9 layout: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr unsigned kWaitVm0 = 0x0F70;  // vmcnt(0)

// One 16-byte-per-lane direct load into LDS: lane l's 16 bytes from src land at dst + 16 l
// bytes (dst wave-uniform).  A plain function, so that calls from templates whose
// arguments depend on template parameters are checked once, for the device only.
__device__ __forceinline__ void load_lds_b128(const char* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// The extra instructions issued after MFMA i of a 16-deep substep: the substep's list of
// nr fragment reads (for the next substep) and nd direct loads (of the next stage), merged
// read, load, read, load, ... (the longer list's rest at the end), is spread evenly over its
// nm MFMAs: MFMA i is followed by list entries first(i) .. first(i + 1) - 1.
constexpr int issue_first(int i, int nops, int nm) { return i * nops / nm; }
// entry q of the merged list: kind (0 read, 1 load) and index within its own list
constexpr int issue_kind(int q, int nr, int nd) { return q < 2 * (nr < nd ? nr : nd) ? (q & 1) : (nr > nd ? 0 : 1); }
constexpr int issue_index(int q, int nr, int nd) {
  return q < 2 * (nr < nd ? nr : nd) ? (q >> 1) : q - (nr < nd ? nr : nd);
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), in order
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// bf16 GEMM (see the file comment), BM x BNT x BK tiles, four waves of 128 x BNT/2.  Operand
// offsets are 32-bit byte offsets from the tile's first row of A and of W (the caller checks
// (BM + 1) K 2 < 2^32, and for the gated form (F + 256) K 2 < 2^32).
template <int EPI, int BNT>
__global__ __launch_bounds__(NT4, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ W,
                                                           const uint16_t* R,  // may alias C (resid)
                                                           uint16_t* C, int M, int N, int K,
                                                           int tiles_n, int n_tiles) {
  static_assert(BNT == 256 || (BNT == 192 && EPI != kEpiGated), "tile width");
  constexpr int NB = BNT / 64;   // 32-column blocks per wave (two waves along N)
  constexpr int WB = BNT / 32;   // 1 KB blocks of the W tile each wave loads
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sW0[BNT * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[BNT * BK];

  const int tile = tile_of(blockIdx.x, n_tiles, tiles_n);
  const int tm = tile / tiles_n;
  const int tn = tile % tiles_n;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = int(__builtin_amdgcn_readfirstlane(t >> 6));
  const int wn = wave & 1;   // BNT / 2 output columns
  const int wm = wave >> 1;  // 128 output rows

  // Direct loads: wave w fills 1 KB blocks 8w .. 8w + 7 of the A tile (rows 64w .. 64w +
  // 63) and blocks WB w .. WB w + WB - 1 of the W tile; lane l writes bytes 16 l of its
  // block: tile row 8 b + l / 8, stored chunk l % 8, which holds logical chunk
  // (l % 8) ^ ((row / 2) % 8) (the layout lds_off describes).  Rows past M (past N) are
  // clamped: computed, never stored.
  const uint16_t* At = A + int64_t(tm) * BM * K;
  const int w_first = EPI == kEpiGated ? tn * 128 : tn * BNT;
  const uint16_t* Wt = W + int64_t(w_first) * K;
  const int a_rows = min(BM, M - tm * BM);
  const int w_last = (EPI == kEpiGated ? 2 * N : N) - 1;
  uint32_t a_vo[8], w_vo[WB];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 64 * wave + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    a_vo[j] = uint32_t(min(row, a_rows - 1)) * uint32_t(K) * 2u + uint32_t(chunk) * 16u;
  }
#pragma unroll
  for (int j = 0; j < WB; ++j) {
    const int row = 8 * WB * wave + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    w_vo[j] = uint32_t(min(w_row<EPI, BNT>(tn, row, N), w_last) - w_first) * uint32_t(K) * 2u + uint32_t(chunk) * 16u;
  }
  auto load_a = [&](int kt, uint16_t* dA, int j) {
    load_lds_b128(reinterpret_cast<const char*>(At + kt * BK) + a_vo[j], dA + (8 * wave + j) * 512);
  };
  auto load_w = [&](int kt, uint16_t* dW, int j) {
    load_lds_b128(reinterpret_cast<const char*>(Wt + kt * BK) + w_vo[j], dW + (WB * wave + j) * 512);
  };

  f32x16 acc[NB][4];
#pragma unroll
  for (int bn = 0; bn < NB; ++bn)
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bn][bm][r] = 0.f;

  // fragment rows base + (lane & 31), base a multiple of 32, share the swizzle key
  // ((lane & 31) / 2) % 8: a fragment's LDS offset is (row base) * BK + a lane offset
  const int fr = lane & 31, fc = lane >> 5;
  const int fkey = (fr >> 1) & 7;
  const int a_base = (wm * 128) * BK, w_base = (wn * (BNT / 2)) * BK;
  const int wave_row0 = tm * BM + wm * 128;

  // One K step from stage (sA, sW): four 16-deep substeps of NB NBM MFMAs.  The fragments of
  // substep kk + 1 are read, and stage kn's direct loads issued (A during substep 0, W
  // during substep 1; kn < 0: none), between the MFMAs of substep kk in a fixed order, each
  // MFMA and what follows it fenced from the scheduler.  A wave with at most 32 valid rows
  // computes its first 32-row block only (NBM = 1), one whose 128 rows all lie past M only
  // issues its loads (NBM = 0): that removes padding work alone.
  auto step = [&](const uint16_t* sA, const uint16_t* sW, int kn, uint16_t* nA, uint16_t* nW, auto nbm_c) {
    constexpr int NBM = decltype(nbm_c)::value;  // 32-row blocks computed (4, or 1 when <= 32 rows are valid)
    constexpr int NMB = NB * NBM;                // MFMAs per substep
    if constexpr (NBM == 0) {
      if (kn >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) load_a(kn, nA, j);
#pragma unroll
        for (int j = 0; j < WB; ++j) load_w(kn, nW, j);
      }
    } else {
      bf16x8 wf[2][NB], af[2][NBM];
      {
        const int lo = fr * BK + ((fc ^ fkey) << 3);
#pragma unroll
        for (int bm = 0; bm < NBM; ++bm) af[0][bm] = *reinterpret_cast<const bf16x8*>(sA + a_base + lo + bm * 32 * BK);
#pragma unroll
        for (int bn = 0; bn < NB; ++bn) wf[0][bn] = *reinterpret_cast<const bf16x8*>(sW + w_base + lo + bn * 32 * BK);
      }
      static_for<BK / 16>([&](auto kk_c) {
        constexpr int kk = decltype(kk_c)::value;
        constexpr int cb = kk & 1;
        constexpr int nr = kk + 1 < BK / 16 ? NBM + NB : 0;
        constexpr int nd = kk == 0 ? 8 : (kk == 1 ? WB : 0);
        const int lo_n = fr * BK + (((2 * (kk + 1) + fc) ^ fkey) << 3);
        static_for<NMB>([&](auto i_c) {
          constexpr int i = decltype(i_c)::value;
          constexpr int bn = i / NBM, bm = i % NBM;
          acc[bn][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb][bn], af[cb][bm], acc[bn][bm], 0, 0, 0);
          constexpr int q0 = issue_first(i, nr + nd, NMB);
          static_for<issue_first(i + 1, nr + nd, NMB) - q0>([&](auto d_c) {
            constexpr int q = q0 + decltype(d_c)::value;
            constexpr int x = issue_index(q, nr, nd);
            if constexpr (issue_kind(q, nr, nd) == 0) {
              if constexpr (x < NBM) af[cb ^ 1][x] = *reinterpret_cast<const bf16x8*>(sA + a_base + lo_n + x * 32 * BK);
              else wf[cb ^ 1][x - NBM] = *reinterpret_cast<const bf16x8*>(sW + w_base + lo_n + (x - NBM) * 32 * BK);
            } else {
              if (kn >= 0) {
                if constexpr (kk == 0) load_a(kn, nA, x);
                else load_w(kn, nW, x);
              }
            }
          });
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    }
  };

  // Stage k lives in LDS buffer k % 2.  Step k: wait for this wave's stage-k loads, barrier
  // (every wave's stage-k loads have landed and every wave is done reading stage k - 1, whose
  // buffer stage k + 1 takes), then the step, issuing stage k + 1's loads.  The loop takes
  // two steps at a time, so the buffers stay compile-time distinct (the compiler can then
  // tell the loads in flight from the reads); an odd last step follows it.
  const int KT = K / BK;
  auto run = [&](auto nbm_c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) load_a(0, sA0, j);
#pragma unroll
    for (int j = 0; j < WB; ++j) load_w(0, sW0, j);
    int k = 0;
    for (; k + 1 < KT; k += 2) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      step(sA0, sW0, k + 1, sA1, sW1, nbm_c);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      step(sA1, sW1, k + 2 < KT ? k + 2 : -1, sA0, sW0, nbm_c);
    }
    if (k < KT) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      step(sA0, sW0, -1, sA1, sW1, nbm_c);
    }
  };
  if (wave_row0 + 32 < M) run(std::integral_constant<int, 4>{});
  else if (wave_row0 < M) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});

  store_rows<EPI, BNT, 4>(acc, C, R, M, N, wave_row0, tn, wn, lane);
}

// int4-weight GEMM, four waves of 128 x BNT/2 like the bf16 kernel.  A goes global -> LDS
// directly; each thread owns one W tile row: its 64 codes and two group scales of stage
// k + 2 are loaded into registers during step k (substep 1), and those of stage k + 1
// (loaded during step k - 1) are de-quantised into the free LDS stage during substeps 2
// and 3, interleaved with the MFMAs.
template <int EPI, int BNT>
__global__ __launch_bounds__(NT4, 1) void gemm_w4_kernel(const uint16_t* __restrict__ A,
                                                          const uint8_t* __restrict__ Wq,
                                                          const uint16_t* __restrict__ Ws,
                                                          const uint16_t* R,  // may alias C (resid)
                                                          uint16_t* C, int M, int N, int K,
                                                          int tiles_n, int n_tiles) {
  static_assert(BNT == 256 || (BNT == 192 && EPI != kEpiGated), "tile width");
  constexpr int NB = BNT / 64;
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sW0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[TILE];

  const int tile = tile_of(blockIdx.x, n_tiles, tiles_n);
  const int tm = tile / tiles_n;
  const int tn = tile % tiles_n;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = int(__builtin_amdgcn_readfirstlane(t >> 6));
  const int wn = wave & 1;
  const int wm = wave >> 1;

  const uint16_t* At = A + int64_t(tm) * BM * K;
  const int a_rows = min(BM, M - tm * BM);
  uint32_t a_vo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 64 * wave + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    a_vo[j] = uint32_t(min(row, a_rows - 1)) * uint32_t(K) * 2u + uint32_t(chunk) * 16u;
  }
  auto load_a = [&](int kt, uint16_t* dA, int j) {
    load_lds_b128(reinterpret_cast<const char*>(At + kt * BK) + a_vo[j], dA + (8 * wave + j) * 512);
  };
  // W tile row of thread t: each 8-lane group takes rows 16 a + p + 0, 2, .., 14, whose
  // swizzle keys (row / 2) % 8 are 0 .. 7, so the group's 16-byte writes of one chunk index
  // land on 8 distinct chunk positions.  A 192-wide tile uses rows 0 .. 191; the threads of
  // rows 192 .. 255 expand a clamped row into the unused rest.
  const int q_row = 16 * (t >> 4) + 2 * (t & 7) + ((t >> 3) & 1);
  const int w_last = (EPI == kEpiGated ? 2 * N : N) - 1;
  const int q_r = min(w_row<EPI, BNT>(tn, q_row, N), w_last);
  const uint8_t* q_src = Wq + int64_t(q_r) * (K / 2);
  const uint16_t* s_src = Ws + int64_t(q_r) * (K / 32);
  uint4 wc[2][2];      // [register set][half]: 64 codes of one stage
  uint32_t wsc[2];     // [register set]: the two group scales (fp16 pair)
  auto load_w = [&](int kt, int set, int x) {
    if (x < 2) wc[set][x] = *reinterpret_cast<const uint4*>(q_src + int64_t(kt) * (BK / 2) + 16 * x);
    else wsc[set] = *reinterpret_cast<const uint32_t*>(s_src + int64_t(kt) * (BK / 32));
  };
  auto dequant_w = [&](int set, uint16_t* dW, int j) {  // chunk j (codes 8 j .. 8 j + 7)
    const uint32_t sc2 = wsc[set];
    const float s = float(__builtin_bit_cast(_Float16, uint16_t(j < 4 ? sc2 & 0xFFFFu : sc2 >> 16)));
    const uint4 h = wc[set][j >> 2];
    const uint32_t w = (j & 3) == 0 ? h.x : (j & 3) == 1 ? h.y : (j & 3) == 2 ? h.z : h.w;
    *reinterpret_cast<uint4*>(dW + lds_off(q_row, j)) = dequant8(w, s, -1032.0f * s);
  };

  f32x16 acc[NB][4];
#pragma unroll
  for (int bn = 0; bn < NB; ++bn)
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bn][bm][r] = 0.f;

  const int fr = lane & 31, fc = lane >> 5;
  const int fkey = (fr >> 1) & 7;
  const int a_base = (wm * 128) * BK, w_base = (wn * (BNT / 2)) * BK;
  const int wave_row0 = tm * BM + wm * 128;

  // one K step from stage (sA, sW); ka: stage whose A loads and W de-quantisation (from
  // register set DQ into nW) go into (nA, nW), kw: stage whose W codes are loaded into
  // register set 1 - DQ (-1: none)
  auto step = [&](const uint16_t* sA, const uint16_t* sW, int ka, int kw, uint16_t* nA, uint16_t* nW,
                  auto dq_c, auto nbm_c) {
    constexpr int DQ = decltype(dq_c)::value;
    constexpr int NBM = decltype(nbm_c)::value;  // 32-row blocks computed (4, or 1 when <= 32 rows are valid)
    constexpr int NMB = NB * NBM;                // MFMAs per substep
    if constexpr (NBM == 0) {
      if (ka >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) load_a(ka, nA, j);
      }
      if (kw >= 0) {
#pragma unroll
        for (int x = 0; x < 3; ++x) load_w(kw, 1 - DQ, x);
      }
      if (ka >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) dequant_w(DQ, nW, j);
      }
    } else {
      bf16x8 wf[2][NB], af[2][NBM];
      {
        const int lo = fr * BK + ((fc ^ fkey) << 3);
#pragma unroll
        for (int bm = 0; bm < NBM; ++bm) af[0][bm] = *reinterpret_cast<const bf16x8*>(sA + a_base + lo + bm * 32 * BK);
#pragma unroll
        for (int bn = 0; bn < NB; ++bn) wf[0][bn] = *reinterpret_cast<const bf16x8*>(sW + w_base + lo + bn * 32 * BK);
      }
      static_for<BK / 16>([&](auto kk_c) {
        constexpr int kk = decltype(kk_c)::value;
        constexpr int cb = kk & 1;
        constexpr int nr = kk + 1 < BK / 16 ? NBM + NB : 0;
        constexpr int nd = kk == 0 ? 8 : (kk == 1 ? 3 : 4);
        const int lo_n = fr * BK + (((2 * (kk + 1) + fc) ^ fkey) << 3);
        static_for<NMB>([&](auto i_c) {
          constexpr int i = decltype(i_c)::value;
          constexpr int bn = i / NBM, bm = i % NBM;
          acc[bn][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb][bn], af[cb][bm], acc[bn][bm], 0, 0, 0);
          constexpr int q0 = issue_first(i, nr + nd, NMB);
          static_for<issue_first(i + 1, nr + nd, NMB) - q0>([&](auto d_c) {
            constexpr int q = q0 + decltype(d_c)::value;
            constexpr int x = issue_index(q, nr, nd);
            if constexpr (issue_kind(q, nr, nd) == 0) {
              if constexpr (x < NBM) af[cb ^ 1][x] = *reinterpret_cast<const bf16x8*>(sA + a_base + lo_n + x * 32 * BK);
              else wf[cb ^ 1][x - NBM] = *reinterpret_cast<const bf16x8*>(sW + w_base + lo_n + (x - NBM) * 32 * BK);
            } else if constexpr (kk == 0) {
              if (ka >= 0) load_a(ka, nA, x);
            } else if constexpr (kk == 1) {
              if (kw >= 0) load_w(kw, 1 - DQ, x);
            } else {
              if (ka >= 0) dequant_w(DQ, nW, 4 * (kk - 2) + x);
            }
          });
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    }
  };

  // prologue: stage 0 (A direct, W codes of stages 0 and 1 into register sets 0 and 1,
  // stage 0 de-quantised into sW0)
  const int KT = K / BK;
  auto run = [&](auto nbm_c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) load_a(0, sA0, j);
#pragma unroll
    for (int x = 0; x < 3; ++x) load_w(0, 0, x);
    if (KT > 1) {
#pragma unroll
      for (int x = 0; x < 3; ++x) load_w(1, 1, x);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
    for (int j = 0; j < 8; ++j) dequant_w(0, sW0, j);
    int k = 0;
    for (; k + 1 < KT; k += 2) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      step(sA0, sW0, k + 1, k + 2 < KT ? k + 2 : -1, sA1, sW1, std::integral_constant<int, 1>{}, nbm_c);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      step(sA1, sW1, k + 2 < KT ? k + 2 : -1, k + 3 < KT ? k + 3 : -1, sA0, sW0, std::integral_constant<int, 0>{},
           nbm_c);
    }
    if (k < KT) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      step(sA0, sW0, -1, -1, sA1, sW1, std::integral_constant<int, 1>{}, nbm_c);
    }
  };
  if (wave_row0 + 32 < M) run(std::integral_constant<int, 4>{});
  else if (wave_row0 < M) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});

  store_rows<EPI, BNT, 4>(acc, C, R, M, N, wave_row0, tn, wn, lane);
}

}  // namespace

// Column-tile width of the bf16 GEMM for a weight of N rows: 256, or 192 for weights of at
// most kGemmNarrowN rows (not the gated form).  It depends on the weight alone, never on M.
int gemm_tile_n(int64_t N, int epi) { return (epi != kEpiGated && N <= kGemmNarrowN) ? kGemmBNNarrow : BN; }
// The same for int4 weights: 192-wide tiles up to kGemmW4NarrowN rows.
int gemm_w4_tile_n(int64_t N, int epi) { return (epi != kEpiGated && N <= kGemmW4NarrowN) ? kGemmBNNarrow : BN; }

// epi: kEpiPlain / kEpiResid (R [M, N]) / kEpiGated (N = F outputs, W [2F, K], F % 128 == 0)
hipError_t launch_gemm_ex(const uint16_t* A, const uint16_t* W, const uint16_t* R, uint16_t* C, int64_t M,
                          int64_t N, int64_t K, int epi, hipStream_t s) {
  const int bnt = gemm_tile_n(N, epi);
  const int tiles_m = int((M + BM - 1) / BM);
  const int tiles_n = epi == kEpiGated ? int(N / 128) : int((N + bnt - 1) / bnt);
  const int n_tiles = tiles_m * tiles_n;
#define BI_GEMM(E, T)                                                                                          \
  if (epi == E && bnt == T) {                                                                                  \
    hipLaunchKernelGGL((gemm_bf16_kernel<E, T>), dim3(n_tiles), dim3(NT4), 0, s, A, W, R, C, int(M), int(N), int(K), \
                       tiles_n, n_tiles);                                                                      \
    return hipGetLastError();                                                                                  \
  }
  BI_GEMM(kEpiPlain, BN) BI_GEMM(kEpiResid, BN) BI_GEMM(kEpiGated, BN)
  BI_GEMM(kEpiPlain, kGemmBNNarrow) BI_GEMM(kEpiResid, kGemmBNNarrow)
#undef BI_GEMM
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_w4_ex(const uint8_t* Wq, const uint16_t* Ws, const uint16_t* A, const uint16_t* R,
                             uint16_t* C, int64_t M, int64_t N, int64_t K, int epi, hipStream_t s) {
  const int bnt = gemm_w4_tile_n(N, epi);
  const int tiles_m = int((M + BM - 1) / BM);
  const int tiles_n = epi == kEpiGated ? int(N / 128) : int((N + bnt - 1) / bnt);
  const int n_tiles = tiles_m * tiles_n;
#define BI_GEMM(E, T)                                                                                          \
  if (epi == E && bnt == T) {                                                                                  \
    hipLaunchKernelGGL((gemm_w4_kernel<E, T>), dim3(n_tiles), dim3(NT4), 0, s, A, Wq, Ws, R, C, int(M), int(N),  \
                       int(K), tiles_n, n_tiles);                                                              \
    return hipGetLastError();                                                                                  \
  }
  BI_GEMM(kEpiPlain, BN) BI_GEMM(kEpiResid, BN) BI_GEMM(kEpiGated, BN)
  BI_GEMM(kEpiPlain, kGemmBNNarrow) BI_GEMM(kEpiResid, kGemmBNNarrow)
#undef BI_GEMM
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const uint16_t* A, const uint16_t* W, uint16_t* C, int64_t M, int64_t N,
                       int64_t K, hipStream_t s) {
  return launch_gemm_ex(A, W, nullptr, C, M, N, K, kEpiPlain, s);
}

hipError_t launch_gemm_w4(const uint16_t* A, const uint8_t* Wq, const uint16_t* Ws, uint16_t* C,
                          int64_t M, int64_t N, int64_t K, hipStream_t s) {
  return launch_gemm_w4_ex(Wq, Ws, A, nullptr, C, M, N, K, kEpiPlain, s);
}

}  // namespace bi


