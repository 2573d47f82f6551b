// Expert-grouped MXFP8 GEMM on gfx950:
//   C[m][j] = sum over c of A[m][c] * B[e(m)][j][c]
// with E4M3 elements and one E8M0 scale per 32 contraction elements on both
// operands, f32 accumulation, bf16 output.  Token
// rows m are bucketed by expert through the offsets (the tinygrad page's
// expert_off; e(m) is the Slang page's expert_for_row), and each expert has
// its own MXFP8 weight matrix B[e] with scales along the contraction (the
// vLLM page's mfma_f8f8: fp8 weights with one E8M0 scale per 32 of k).  With
// A = x and B[e] = W_e this is the MoE forward y = x W_e^T; with A = g
// (quantised along its features) and B[e] = W_e^T (quantised along N by the
// transposing quantiser) it is an MXFP8 data gradient g W_e.
//
// Design (gfx950), sharing the weight gradient's core (mx_gemm_core.hpp):
//  * Persistent grid, one 512-thread workgroup per CU; output tiles of up to
//    256 token rows x 256 columns, every tile inside one expert: expert e's
//    rows split into ceil(n_e / 256) row tiles, so each tile is one pass of
//    K/128 steps.  A scan of the offsets in LDS at kernel start gives each
//    expert's rows (offsets clamped to [0, M] and made nondecreasing) and its
//    first row tile; rows of no expert form extra tiles that store +0.0.
//  * Tile order: expert, column tile, row tile, so the workgroups sharing a
//    weight tile run together; workgroup b walks tiles lb, lb + G, ... with
//    the workgroups of one XCD (b mod 8) on consecutive tiles.
//  * Roles in the core: the weight tile B[e][j0..j0+255][c..c+127] is the
//    x-role (MFMA A operand; output rows j), the token tile A[m0..][c..] the
//    g-role (MFMA B operand; output columns m), so the epilogue writes
//    C[m][j] as whole 128-byte row pieces.
//  * Exact form (default entry points): each 32-element block of both tiles
//    is converted with its scale to bf16 in registers and multiplied on the
//    bf16 MFMA, the weight gradient's exact step (no token masking: the
//    contraction here is the feature axis).  The block-scaled fp8 MFMA
//    truncates each 8-element run's products, which loses small products
//    where an outlier of one operand meets an outlier of the other; the fast
//    entry points make that one pass.
//  * Each 128-element contraction step stages both tiles (32 KB each) and
//    their scale dwords in LDS with buffer loads that write LDS directly,
//    double-buffered; the workgroup walks the steps of all its tiles as one
//    stream, and waves 4-7 issue all stage loads.  A partial row tile still
//    runs all its MFMAs (on zeros past its last row): letting those waves skip
//    them desynchronised the workgroups that share a weight tile and raised
//    the L2 misses by a third for a 1.5% gain.
//  * Rows past M read as zero (buffer-descriptor range) and their stores are
//    dropped the same way, so M needs no padding.
//  * a8w4 (the decode page's mfma_f4f8: fp4 weights times MXFP8 activations):
//    B[e] may hold E2M1 codes, two per byte along the contraction, with the
//    same E8M0 scales; the weight tile is then 16 KB per step (MFMA format 4
//    for the x-role), loaded by four stage loads per loading wave instead of
//    eight.
#include "common.hpp"
#include "mx_gemm_core.hpp"
#include "../../include/moe_gg.h"

namespace moe_gg {
namespace {

using namespace mxgemm;

constexpr int NWAVE = 8;
constexpr int NTHREAD = NWAVE * 64;

constexpr int MAX_E = 2048;                   // experts (LDS tables of E + 1 entries)
constexpr int SCAN_PER = (MAX_E + 1 + NTHREAD - 1) / NTHREAD;   // table entries per thread in the scans

// Inclusive scan over the workgroup's 512 threads (Hillis-Steele through LDS).
template <bool MAX>
__device__ __forceinline__ int block_scan(int x, int *red, int tid) {
#pragma unroll 1
  for (int d = 1; d < NTHREAD; d <<= 1) {
    red[tid] = x;
    barrier();
    if (tid >= d) x = MAX ? max(x, red[tid - d]) : x + red[tid - d];
    barrier();
  }
  return x;
}

// An output tile: 256 columns jt of up to 256 token rows [m0, m0 + rows)
// that all belong to expert e (kind 1), or rows of no expert (kind 2).
struct Tile {
  int kind, e, jt, m0, rows;
};

// EXACT: operands converted exactly to bf16 and multiplied on the bf16 MFMA;
// otherwise one block-scaled fp8 MFMA pass.
template <bool EXACT, bool XFP4>
__global__ __launch_bounds__(NTHREAD, 1) void grouped_mxfp8_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, uint16_t *__restrict__ C,
    const uint8_t *__restrict__ SA, const uint8_t *__restrict__ SB,
    const int32_t *__restrict__ off, int M, int N, int K, int E) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE_BYTES];
  __shared__ int s_row[MAX_E + 1];    // expert e owns token rows [s_row[e], s_row[e + 1])
  __shared__ int s_pre[MAX_E + 1];    // row tiles of the experts before e

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tilesJ = N / TA;
  const int nk = K / TT;                   // contraction steps per tile
  const int G = gridDim.x;

  // ---- expert row ranges and row-tile prefix (one pass over the offsets) ----
  // Rows: offsets clamped to [0, M] and made nondecreasing by a running
  // maximum, so the experts' row ranges are disjoint; for well-formed offsets
  // this is off itself.  Each expert splits into ceil(rows / 256) row tiles.
  {
    int *red = reinterpret_cast<int *>(smem);
    const int e0 = tid * SCAN_PER;
    int v[SCAN_PER];
    int run = 0;
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) {
      const int e = e0 + j;
      if (e <= E) run = max(run, clampi(off[e], 0, M));
      v[j] = run;
    }
    int incl = block_scan<true>(run, red, tid);
    red[tid] = incl;
    barrier();
    const int before = tid ? red[tid - 1] : 0;
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j)
      if (e0 + j <= E) s_row[e0 + j] = max(before, v[j]);
    barrier();
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) {
      const int e = e0 + j;
      v[j] = e < E ? (s_row[e + 1] - s_row[e] + TB - 1) / TB : 0;
      cnt += v[j];
    }
    incl = block_scan<false>(cnt, red, tid);
    int pre = incl - cnt;
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) {
      if (e0 + j <= E) s_pre[e0 + j] = pre;
      pre += v[j];
    }
    barrier();
  }
  const int R = s_pre[E];                                  // expert row tiles
  const int row_first = s_row[0], row_end = s_row[E];
  const int Zh = (row_first + TB - 1) / TB;                // row tiles of no expert before / after
  const int Zt = (M - row_end + TB - 1) / TB;
  const int expert_tiles = R * tilesJ;
  const int total = (R + Zh + Zt) * tilesJ;

  // Tile order o: expert-major, then the column tile, then the expert's row
  // tile, so the workgroups that share a weight tile B[e][j0..] run together;
  // the rows of no expert come last.  Workgroup b runs o = lb, lb + G, ...
  // with lb chosen so that the workgroups of one XCD (b mod 8, the dispatch
  // order) hold consecutive o and share that XCD's L2.
  auto tile_of = [&](int o) __attribute__((always_inline)) {
    Tile t;
    t.kind = 0; t.e = 0; t.jt = 0; t.m0 = 0; t.rows = 0;
    if (o >= total) return t;
    if (o < expert_tiles) {
      int lo = 0, hi = E;                                  // s_pre[lo] * tilesJ <= o < s_pre[hi] * tilesJ
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pre[mid] * tilesJ <= o) lo = mid; else hi = mid;
      }
      const int ce = s_pre[lo + 1] - s_pre[lo];
      const int r = o - s_pre[lo] * tilesJ;
      const int jt = r / ce, i = r - jt * ce;
      t.kind = 1; t.e = lo; t.jt = jt;
      t.m0 = s_row[lo] + i * TB;
      t.rows = min(TB, s_row[lo + 1] - t.m0);
    } else {
      const int z = o - expert_tiles;
      const int zr = z / tilesJ;
      t.kind = 2; t.jt = z - zr * tilesJ;
      if (zr < Zh) { t.m0 = zr * TB; t.rows = min(TB, row_first - t.m0); }
      else { t.m0 = row_end + (zr - Zh) * TB; t.rows = min(TB, M - t.m0); }
    }
    return t;
  };
  const int b = blockIdx.x;
  const int lb = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;

  // ---- per-lane constants -------------------------------------------------
  const uint32_t smem_base = lds_addr(smem);
  const uint32_t Kb = static_cast<uint32_t>(K);
  const uint32_t Kx = XFP4 ? Kb / 2 : Kb;  // bytes per weight row
  const uint32_t scale_row = Kb / 32;      // bytes per scale row
  // stage loads a loading wave issues per step: 8 (E4M3) or 4 (fp4) for the
  // weight tile, 8 for the token tile, 2 scale loads
  constexpr int LOADS_PER_STEP = (XFP4 ? 4 : 8) + 8 + 2;
  // Stage loads by waves 4-7: wave 4 + w4 fills blocks 8w4..8w4+7 of both
  // operand tiles (block 8G + q holds rows 64G + 8j + q at slot j; lane L ->
  // slot L/8, bytes 16(L%8)..16(L%8)+15 of the row's step) and the scale
  // dwords of rows 64w4..64w4+63 of both operands.
  const bool loader = wave >= 4;
  const int w4 = wave & 3;
  uint32_t voff_t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 64 * w4 + 8 * (lane >> 3) + i;
    voff_t[i] = static_cast<uint32_t>(r) * Kb + static_cast<uint32_t>(lane & 7) * 16u;
  }
  const uint32_t voff_s = static_cast<uint32_t>(w4 * 64 + lane) * scale_row;
  // fp4 weight tile: wave 4 + w4 fills blocks 4w4..4w4+3 (block 4G + q holds
  // rows 64G + 4j + q at slot j; lane L -> slot L/4, bytes 16(L%4)..+15)
  uint32_t voff_x4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    voff_x4[i] = static_cast<uint32_t>(64 * w4 + 4 * (lane >> 2) + i) * Kx + static_cast<uint32_t>(lane & 3) * 16u;

  // MFMA operand addressing
  const int wk = wave >> 2, wn = wave & 3;
  const int g = lane >> 5, l32 = lane & 31;
  uint32_t xrow[4], grow[2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
    xrow[a] = ST_A + (XFP4 ? tile_row4(wk * 128 + a * 32 + l32) : tile_row(wk * 128 + a * 32 + l32));
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) grow[bb] = ST_B + tile_row(wn * 64 + bb * 32 + l32);
  const uint32_t growh[2] = {ST_B + tile_row(wn * 32 + l32), 0u};   // the half layout's rows
  uint32_t chunk_off[2][2];   // [half][piece] -> 16-byte chunk offset within the row
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    chunk_off[h][0] = (4 * h + g) * 16;
    chunk_off[h][1] = (4 * h + 2 + g) * 16;
  }

  // the load cursor: the workgroup's k-th tile, step s (expert tiles only;
  // they precede every tile of no expert in the order)
  int ld_k = 0, ld_s = 0;
  Tile ld_t = tile_of(lb);
  auto advance = [&]() __attribute__((always_inline)) {
    if (++ld_s < nk) return;
    ld_s = 0;
    ++ld_k;
    ld_t = tile_of(lb + ld_k * G);
  };

  int ops = 0;               // vector-memory instructions this wave has issued (uniform)
  int mark[2] = {0, 0};      // value of ops right after the loads of the step in buffer 0 / 1

  auto issue_stage = [&](uint32_t buf) __attribute__((always_inline)) {
    if (!loader) return;
    const uint32_t cpos = static_cast<uint32_t>(ld_s * TT);
    const size_t wrow = static_cast<size_t>(ld_t.e) * N + static_cast<size_t>(ld_t.jt) * TA;   // first weight row
    const uint32_t rows = static_cast<uint32_t>(ld_t.rows);
    const v4i srd_x = make_srd(B + wrow * Kx, TA * Kx);
    const v4i srd_g = make_srd(A + static_cast<size_t>(ld_t.m0) * K, rows * Kb);
    const uint32_t base = smem_base + buf * STAGE_BYTES;
    if constexpr (XFP4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dma_b128(srd_x, voff_x4[i], cpos / 2, __builtin_amdgcn_readfirstlane(base + ST_A + (w4 * 4 + i) * BLK4));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma_b128(srd_x, voff_t[i], cpos, __builtin_amdgcn_readfirstlane(base + ST_A + (w4 * 8 + i) * BLK));
    }
    // a half tile (exact form, at most 128 token rows) reads token rows 0..127
    // only: loaders 2 and 3 leave rows 128..255 and their scales unloaded
    const bool token_rows = !(EXACT && rows <= 128u && w4 >= 2);
    if (token_rows) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma_b128(srd_g, voff_t[i], cpos, __builtin_amdgcn_readfirstlane(base + ST_B + (w4 * 8 + i) * BLK));
    }
    const v4i srd_sx = make_srd(SB + wrow * scale_row, 256u * scale_row);
    const v4i srd_sg = make_srd(SA + static_cast<size_t>(ld_t.m0) * scale_row, rows * scale_row);
    dma_b32(srd_sx, voff_s, cpos / 32, __builtin_amdgcn_readfirstlane(base + ST_SA + w4 * 256));
    if (token_rows) dma_b32(srd_sg, voff_s, cpos / 32, __builtin_amdgcn_readfirstlane(base + ST_SB + w4 * 256));
    ops += token_rows ? LOADS_PER_STEP : LOADS_PER_STEP - 9;
  };
  // wait until the loads of the step in buffer b have landed: every vector
  // memory instruction issued after them may still be in flight
  // (the counts that occur: a step's loads, a tile's stores, both, and a
  // zero tile's stores on top; any smaller count is also correct)
  auto wait_step = [&](int bf) __attribute__((always_inline)) {
    constexpr int L = LOADS_PER_STEP, S = STORES_PER_TILE;
    const int younger = ops - mark[bf];
    if (younger >= L + 2 * S) wait_vmcnt<L + 2 * S>();
    else if (younger >= L + S) wait_vmcnt<L + S>();
    else if (younger >= (L > S ? L : S)) wait_vmcnt<(L > S ? L : S)>();
    else if (younger >= (L > S ? S : L)) wait_vmcnt<(L > S ? S : L)>();
    else if (younger >= 8) wait_vmcnt<8>();
    else wait_vmcnt<0>();
  };

  // ---- prologue: first step in flight ----
  if (ld_t.kind == 1 && nk > 0) {
    issue_stage(0);
    mark[0] = ops;
    advance();
  }

  uint32_t buf = 0;                    // buffer of the step being computed
  v16f acc[4][2];
  const uint32_t Nu = static_cast<uint32_t>(N);
#pragma unroll 1
  for (int k = 0;; ++k) {
    const Tile cur = tile_of(lb + k * G);
    if (cur.kind == 0) break;
    const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
        C + static_cast<size_t>(cur.m0) * N + static_cast<size_t>(cur.jt) * TA, static_cast<short>(0),
        static_cast<int>((static_cast<uint32_t>(cur.rows - 1) * Nu + TA) * 2u), 0x00020000);
    if (cur.kind == 2) {                                  // rows of no expert: +0.0
      store_zero_tile(crsrc, Nu, tid);
      ops += STORES_PER_TILE;
      continue;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][bb][i] = 0.f;
    // the tile's steps; NB = 1: the half layout (all eight waves on token
    // rows 0..127, 32 each), NB = 2: the full one
    auto run = [&](auto nb) __attribute__((always_inline)) {
      constexpr int NB = decltype(nb)::value;
#pragma unroll 1
      for (int s = 0; s < nk; ++s) {
        wait_step(buf);
        barrier();
        if (ld_t.kind == 1) {
          issue_stage(buf ^ 1);
          mark[buf ^ 1] = ops;
          advance();
        }
        const uint8_t *st = smem + buf * STAGE_BYTES;
        if constexpr (EXACT)
          compute_step_bf16<XFP4, NB>(st, acc, xrow, NB == 2 ? grow : growh, wk, wn, l32, g);
        else
          compute_step<XFP4>(st, acc, xrow, grow, chunk_off, wk, wn, l32, g);
        buf ^= 1;
      }
      // ---- epilogue: C[m0 + m][j0 + j] for the tile's rows; the descriptor
      // drops the rest
      store_tile<NB>(acc, smem + (buf ^ 1) * STAGE_BYTES, crsrc, Nu, wk, wn, tid);
      ops += STORES_PER_TILE * NB / 2;
    };
    if (EXACT && cur.rows <= 128)
      run(std::integral_constant<int, 1>());
    else
      run(std::integral_constant<int, 2>());
  }
  wait_vmcnt<0>();
}

int launch_grouped(bool exact, bool xfp4, const uint8_t *A, const uint8_t *B, uint16_t *C, const uint8_t *scale_A,
                   const uint8_t *scale_B, const int32_t *expert_off, int M, int N, int K, int E,
                   hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || E <= 0 || !expert_off) return MOE_GG_EINVAL;
  if (M == 0 || N == 0) return MOE_GG_OK;                 // no output element
  // an empty contraction (K = 0) writes zeros; the operands, then of zero
  // size, are never read and may be null
  if (!C || (K > 0 && (!A || !B || !scale_A || !scale_B))) return MOE_GG_EINVAL;
  if (K % 32) return MOE_GG_EINVAL;
  if (N % TA || K % TT || E > MAX_E) return MOE_GG_EUNSUPPORTED;
  // 32-bit byte offsets inside one 256-row panel and inside a tile of C
  if (static_cast<uint64_t>(TB) * static_cast<uint64_t>(K) > 0xFFFFFFFFull) return MOE_GG_EUNSUPPORTED;
  if (static_cast<uint64_t>(TB) * static_cast<uint64_t>(N) * 2u > 0x7FFFFFFFull) return MOE_GG_EUNSUPPORTED;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_GG_ELAUNCH;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_GG_ELAUNCH;
  // row tiles: at most one partial tile per expert beyond ceil(M / 256), plus
  // the rows of no expert before and after
  const int64_t total = (static_cast<int64_t>((M + TB - 1) / TB) + E + 2) * (N / TA);
  if (total > 0x7FFFFFFF) return MOE_GG_EUNSUPPORTED;
  if (const int st = check_offsets_if_asked(expert_off, E, M, stream)) return st;
  const int grid = static_cast<int>(total < cus ? total : cus);
#define MOE_GG_LAUNCH(S, X)                                                                              \
  hipLaunchKernelGGL((grouped_mxfp8_kernel<S, X>), dim3(grid), dim3(NTHREAD), 0, stream, A, B, C, scale_A, \
                     scale_B, expert_off, M, N, K, E)
  if (exact && xfp4) MOE_GG_LAUNCH(true, true);
  else if (exact) MOE_GG_LAUNCH(true, false);
  else if (xfp4) MOE_GG_LAUNCH(false, true);
  else MOE_GG_LAUNCH(false, false);
#undef MOE_GG_LAUNCH
  return hipGetLastError() == hipSuccess ? MOE_GG_OK : MOE_GG_ELAUNCH;
}

}  // namespace
}  // namespace moe_gg

extern "C" MOE_GG_API int moe_gg_grouped_mxfp8(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                               const uint8_t *scale_A, const uint8_t *scale_B,
                                               const int32_t *expert_off, int M, int N, int K, int E,
                                               hipStream_t stream) {
  return moe_gg::launch_grouped(true, false, A, B, C, scale_A, scale_B, expert_off, M, N, K, E, stream);
}

extern "C" MOE_GG_API int moe_gg_grouped_mxfp8_fast(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                                    const uint8_t *scale_A, const uint8_t *scale_B,
                                                    const int32_t *expert_off, int M, int N, int K, int E,
                                                    hipStream_t stream) {
  return moe_gg::launch_grouped(false, false, A, B, C, scale_A, scale_B, expert_off, M, N, K, E, stream);
}

extern "C" MOE_GG_API int moe_gg_grouped_a8w4(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                              const uint8_t *scale_A, const uint8_t *scale_B,
                                              const int32_t *expert_off, int M, int N, int K, int E,
                                              hipStream_t stream) {
  return moe_gg::launch_grouped(true, true, A, B, C, scale_A, scale_B, expert_off, M, N, K, E, stream);
}

extern "C" MOE_GG_API int moe_gg_grouped_a8w4_fast(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                                   const uint8_t *scale_A, const uint8_t *scale_B,
                                                   const int32_t *expert_off, int M, int N, int K, int E,
                                                   hipStream_t stream) {
  return moe_gg::launch_grouped(false, true, A, B, C, scale_A, scale_B, expert_off, M, N, K, E, stream);
}
