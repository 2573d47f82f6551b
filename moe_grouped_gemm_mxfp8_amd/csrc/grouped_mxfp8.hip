// Expert-grouped MXFP8 GEMM on gfx950:
//   C[m][j] = sum over c of A[m][c] * B[e(m)][j][c]
// with E4M3 elements and one E8M0 scale per 32 contraction elements on both
// operands, f32 accumulation in the block-scaled MFMA, bf16 output.  Token
// rows m are bucketed by expert through the offsets (the tinygrad page's
// expert_off; e(m) is the Slang page's expert_for_row), and each expert has
// its own MXFP8 weight matrix B[e] with scales along the contraction (the
// vLLM page's mfma_f8f8: fp8 weights with one E8M0 scale per 32 of k).  With
// A = x and B[e] = W_e this is the MoE forward y = x W_e^T; with A = g
// (quantised along its features) and B[e] = W_e^T (quantised along N by the
// transposing quantiser) it is an MXFP8 data gradient g W_e.
//
// Design (gfx950), sharing the weight gradient's core (mx_gemm_core.hpp):
//  * Persistent grid, one 512-thread workgroup per CU; output tiles of 256
//    token rows x 256 columns.  A tile's rows may belong to several experts:
//    it then makes one contraction pass per expert present (B[e] changes),
//    with the rows of the other experts zeroed in the g-role fragments, into
//    the same accumulators.
//  * Roles in the core: the weight tile B[e][j0..j0+255][c..c+127] is the
//    x-role (MFMA A operand; output rows j), the token tile A[m0..][c..] the
//    g-role (MFMA B operand; output columns m), so the epilogue writes
//    C[m][j] rows with whole 512-byte row segments.  The two-pass form splits
//    the token operand's codes (activations and gradients carry the
//    outliers).
//  * Each 128-element contraction step stages both tiles (32 KB each) and
//    their scale dwords in LDS with buffer loads that write LDS directly,
//    double-buffered; the workgroup walks the steps of all its tiles and
//    expert passes as one stream, and waves 4-7 issue all stage loads.
//  * Rows past M read as zero (buffer-descriptor range) and their stores are
//    dropped the same way, so M needs no padding.
#include "common.hpp"
#include "mx_gemm_core.hpp"
#include "../../include/moe_gg.h"

namespace moe_gg {
namespace {

using namespace mxgemm;

constexpr int NWAVE = 8;
constexpr int NTHREAD = NWAVE * 64;
constexpr int LOADS_PER_STEP = 18;            // stage loads a loading wave issues per step

// One pass of an output tile: token-row tile mt, column tile jt, expert e,
// whose rows [rlo, rhi) of the tile (relative to m0 = 256 mt) count.
struct Pass {
  int valid, t, e, rlo, rhi;
};

// The expert pass of tile t at or after expert e (the next one with rows in
// the tile), or none.
__device__ __forceinline__ Pass pass_from(int t, int e, int total, int tilesJ, const int32_t *__restrict__ off,
                                          int M, int E) {
  Pass p;
  p.valid = 0; p.t = t; p.e = e; p.rlo = 0; p.rhi = 0;
  if (t >= total) return p;
  const int m0 = (t / tilesJ) * TN;
  const int m1 = min(m0 + TN, M);
  const int e_last = expert_of_row(off, E, m1 - 1);
  e = max(e, expert_of_row(off, E, m0));      // experts before the one owning m0 hold no rows here
  for (; e <= e_last; ++e) {
    const int o0 = clampi(off[e], 0, M);
    const int o1 = clampi(off[e + 1], o0, M);
    const int lo = max(o0, m0), hi = min(o1, m1);
    if (hi > lo) {
      p.valid = 1; p.e = e; p.rlo = lo - m0; p.rhi = hi - m0;
      return p;
    }
  }
  return p;
}

template <bool SPLIT>
__global__ __launch_bounds__(NTHREAD, 1) void grouped_mxfp8_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, uint16_t *__restrict__ C,
    const uint8_t *__restrict__ SA, const uint8_t *__restrict__ SB,
    const int32_t *__restrict__ off, int M, int N, int K, int E) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tilesM = (M + TN - 1) / TN, tilesJ = N / TK;
  const int total = tilesM * tilesJ;
  const int nk = K / TT;                   // contraction steps per pass
  const int G = gridDim.x;

  // ---- per-lane constants -------------------------------------------------
  const uint32_t smem_base = lds_addr(smem);
  const uint32_t Kb = static_cast<uint32_t>(K);
  const uint32_t scale_row = Kb / 32;      // bytes per scale row
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

  // MFMA operand addressing
  const int wk = wave >> 2, wn = wave & 3;
  const int g = lane >> 5, l32 = lane & 31;
  uint32_t xrow[4], grow[2];
#pragma unroll
  for (int a = 0; a < 4; ++a) xrow[a] = ST_X + tile_row(wk * 128 + a * 32 + l32);
#pragma unroll
  for (int b = 0; b < 2; ++b) grow[b] = ST_G + tile_row(wn * 64 + b * 32 + l32);
  uint32_t chunk_off[2][2];   // [half][piece] -> 16-byte chunk offset within the row
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    chunk_off[h][0] = (4 * h + g) * 16;
    chunk_off[h][1] = (4 * h + 2 + g) * 16;
  }

  // the load cursor: pass p, step s; after a tile's last pass, the first pass
  // of the workgroup's next tile that has one
  struct Cursor {
    Pass p;
    int s;
  };
  auto seek = [&](int t) __attribute__((always_inline)) {
    Pass p = pass_from(t, 0, total, tilesJ, off, M, E);
    while (t < total && !p.valid) { t += G; p = pass_from(t, 0, total, tilesJ, off, M, E); }
    return p;
  };
  auto advance = [&](Cursor &c) __attribute__((always_inline)) {
    if (c.s + 1 < nk) { ++c.s; return; }
    c.s = 0;
    Pass q = pass_from(c.p.t, c.p.e + 1, total, tilesJ, off, M, E);
    c.p = q.valid ? q : seek(c.p.t + G);
  };

  int ops = 0;               // vector-memory instructions this wave has issued (uniform)
  int mark[2] = {0, 0};      // value of ops right after the loads of the step in buffer 0 / 1

  auto issue_stage = [&](const Cursor &c, uint32_t buf) __attribute__((always_inline)) {
    if (!loader) return;
    const int t = c.p.t;
    const int mt = t / tilesJ, jt = t - mt * tilesJ;
    const int m0 = mt * TN;
    const uint32_t rows = static_cast<uint32_t>(min(TN, M - m0));
    const uint32_t cpos = static_cast<uint32_t>(c.s * TT);
    const size_t wrow = static_cast<size_t>(c.p.e) * N + static_cast<size_t>(jt) * TK;   // first weight row
    const v4i srd_x = make_srd(B + wrow * K, TK * Kb);
    const v4i srd_g = make_srd(A + static_cast<size_t>(m0) * K, rows * Kb);
    const uint32_t base = smem_base + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma_b128(srd_x, voff_t[i], cpos, __builtin_amdgcn_readfirstlane(base + ST_X + (w4 * 8 + i) * BLK));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma_b128(srd_g, voff_t[i], cpos, __builtin_amdgcn_readfirstlane(base + ST_G + (w4 * 8 + i) * BLK));
    const v4i srd_sx = make_srd(SB + wrow * scale_row, 256u * scale_row);
    const v4i srd_sg = make_srd(SA + static_cast<size_t>(m0) * scale_row, rows * scale_row);
    dma_b32(srd_sx, voff_s, cpos / 32, __builtin_amdgcn_readfirstlane(base + ST_SX + w4 * 256));
    dma_b32(srd_sg, voff_s, cpos / 32, __builtin_amdgcn_readfirstlane(base + ST_SG + w4 * 256));
    ops += LOADS_PER_STEP;
  };
  // wait until the loads of the step in buffer b have landed: every vector
  // memory instruction issued after them may still be in flight
  auto wait_step = [&](int b) __attribute__((always_inline)) {
    const int younger = ops - mark[b];
    if (younger >= 50) wait_vmcnt<50>();
    else if (younger >= 34) wait_vmcnt<34>();
    else if (younger >= 18) wait_vmcnt<18>();
    else if (younger >= 16) wait_vmcnt<16>();
    else if (younger >= 8) wait_vmcnt<8>();
    else wait_vmcnt<0>();
  };

  // ---- prologue: first step in flight ----
  Cursor ld;
  ld.p = seek(blockIdx.x);
  ld.s = 0;
  if (ld.p.valid) {
    issue_stage(ld, 0);
    mark[0] = ops;
    advance(ld);
  }

  uint32_t buf = 0;                    // buffer of the step being computed
  v16f acc[4][2];
  for (int t = blockIdx.x; t < total; t += G) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    Pass cur = pass_from(t, 0, total, tilesJ, off, M, E);
    const bool any = cur.valid;
#pragma unroll 1
    while (cur.valid) {
#pragma unroll 1
      for (int s = 0; s < nk; ++s) {
        wait_step(buf);
        barrier();
        if (ld.p.valid) {
          issue_stage(ld, buf ^ 1);
          mark[buf ^ 1] = ops;
          advance(ld);
        }
        const uint8_t *st = smem + buf * STAGE_BYTES;
        compute_step<SPLIT>(st, acc, xrow, grow, chunk_off, wk, wn, l32, g, 0, TT, cur.rlo, cur.rhi);
        buf ^= 1;
      }
      cur = pass_from(t, cur.e + 1, total, tilesJ, off, M, E);
    }

    // ---- epilogue: C[m0 + m][j0 + j], rows past M dropped by the descriptor
    const int mt = t / tilesJ, jt = t - mt * tilesJ;
    const int m0 = mt * TN;
    const uint32_t Nu = static_cast<uint32_t>(N);
    const uint32_t rows = static_cast<uint32_t>(min(TN, M - m0));
    const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
        C + static_cast<size_t>(m0) * N + static_cast<size_t>(jt) * TK, static_cast<short>(0),
        static_cast<int>(((rows - 1u) * Nu + TK) * 2u), 0x00020000);
    if (!any) store_zero_tile(crsrc, Nu, tid);            // rows of no expert: +0.0
    else store_tile(acc, smem + (buf ^ 1) * STAGE_BYTES, crsrc, Nu, wk, wn, tid);
    ops += STORES_PER_TILE;
  }
  wait_vmcnt<0>();
}

int launch_grouped(bool split, const uint8_t *A, const uint8_t *B, uint16_t *C, const uint8_t *scale_A,
                   const uint8_t *scale_B, const int32_t *expert_off, int M, int N, int K, int E,
                   hipStream_t stream) {
  if (!A || !B || !C || !scale_A || !scale_B || !expert_off) return MOE_GG_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || E <= 0) return MOE_GG_EINVAL;
  if (K % 32) return MOE_GG_EINVAL;
  if (N % TK || K % TT) return MOE_GG_EUNSUPPORTED;
  // 32-bit byte offsets inside one 256-row panel and inside a tile of C
  if (static_cast<uint64_t>(TN) * static_cast<uint64_t>(K) > 0xFFFFFFFFull) return MOE_GG_EUNSUPPORTED;
  if (static_cast<uint64_t>(TN) * static_cast<uint64_t>(N) * 2u > 0x7FFFFFFFull) return MOE_GG_EUNSUPPORTED;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_GG_ELAUNCH;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_GG_ELAUNCH;
  const int64_t total = static_cast<int64_t>((M + TN - 1) / TN) * (N / TK);
  if (total > 0x7FFFFFFF) return MOE_GG_EUNSUPPORTED;
  const int grid = static_cast<int>(total < cus ? total : cus);
  if (split)
    hipLaunchKernelGGL(grouped_mxfp8_kernel<true>, dim3(grid), dim3(NTHREAD), 0, stream, A, B, C, scale_A,
                       scale_B, expert_off, M, N, K, E);
  else
    hipLaunchKernelGGL(grouped_mxfp8_kernel<false>, dim3(grid), dim3(NTHREAD), 0, stream, A, B, C, scale_A,
                       scale_B, expert_off, M, N, K, E);
  return hipGetLastError() == hipSuccess ? MOE_GG_OK : MOE_GG_ELAUNCH;
}

}  // namespace
}  // namespace moe_gg

extern "C" MOE_GG_API int moe_gg_grouped_mxfp8(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                               const uint8_t *scale_A, const uint8_t *scale_B,
                                               const int32_t *expert_off, int M, int N, int K, int E,
                                               hipStream_t stream) {
  return moe_gg::launch_grouped(true, A, B, C, scale_A, scale_B, expert_off, M, N, K, E, stream);
}

extern "C" MOE_GG_API int moe_gg_grouped_mxfp8_fast(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                                    const uint8_t *scale_A, const uint8_t *scale_B,
                                                    const int32_t *expert_off, int M, int N, int K, int E,
                                                    hipStream_t stream) {
  return moe_gg::launch_grouped(false, A, B, C, scale_A, scale_B, expert_off, M, N, K, E, stream);
}
