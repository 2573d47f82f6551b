// Grouped MXFP8 weight gradient on gfx950:
//   grad_w[e*N + n][k] = sum over tokens m of expert e of  g^T[n][m] x^T[k][m]
// with E4M3 elements and one E8M0 scale per 32 tokens, f32 accumulation,
// bf16 output (the tinygrad page "grouped_mxfp8_wgrad.cpp":
// its global layouts, the per-expert 128-token k-loop and the epilogue).
//
// Design (gfx950):
//  * Persistent grid, one 512-thread workgroup per CU.  Output tiles are
//    256 (k) x 256 (n) of one expert; every expert owns (K/256)(N/256) tiles.
//    Tiles are ordered expert by expert, the experts with the most 128-token
//    steps first (ranked once per workgroup from the offsets), and dealt
//    round-robin to the workgroups, so the long tiles start first (each XCD
//    starting at a different expert of that ranking).  Inside an
//    expert the tile order keeps the tiles that run at the same time on one
//    XCD (blockIdx mod 8) in one 4 x 8 patch, so they share operand rows in
//    that XCD's L2.
//  * Each 128-token step stages x^T[256 x 128] and g^T[256 x 128] fp8 (32 KB
//    each) plus their 256 scale dwords in LDS, with buffer loads that write
//    LDS directly (no VGPR round trip), double-buffered.  A workgroup walks
//    the steps of all its tiles as one stream: the load of the next step
//    (possibly the next tile's first) is issued right after the step's
//    barrier.  (Warming L2 a few steps ahead with one load per line was
//    measured slower: the extra lines evict operands still in use.)
//    One barrier per step: it both publishes the step's data and frees the
//    other buffer.  An operand tile in LDS is 32 blocks of 8 rows x 128
//    bytes, each block padded by 16 bytes; a load instruction fills one
//    block, eight lanes per row reading the row's 128 bytes in order (whole
//    lines, no permuted lanes), and rows are placed so that the 16 rows an
//    MFMA operand read touches at once fall on 16 distinct bank groups.
//    An expert whose bounds are not multiples of 128 has a partial first and
//    last step: before those steps' MFMAs all 512 threads zero the staged
//    g^T codes of the tokens outside the expert (one pass over the tile and
//    one more barrier), so the step code itself never masks.
//  * 8 waves as 2 (k) x 4 (n); each wave owns a 128 (k) x 64 (n) output
//    patch as 4 x 2 accumulators of 32 x 32 MFMA results.  x^T is the MFMA A
//    operand (rows = k) and g^T the B operand (columns = n).
//  * Exact form (the default entry point): the block-scaled fp8 MFMA
//    truncates the products of every run of 8 tokens to 2^(largest exponent
//    sum - 13), so where an outlier of g meets an outlier of x at one token
//    the run's other products are lost (errors of ~1 against a bound of ~0.3
//    on the 8192^3 workload, whichever codes are split into separate passes:
//    several outliers of one row can share a run).  The default entry point
//    therefore converts the staged E4M3 codes, times their E8M0 scales, to
//    bf16 (exact) and multiplies on the bf16 MFMA, whose sums carry no such
//    truncation (compute_step_bf16 in mx_gemm_core.hpp).  The single fp8
//    pass (v_mfma_scale_f32_32x32x64_f8f6f4) stays available as the fast
//    entry point, whose results follow the hardware's rounding.
//  * Operand lane layout of the scaled MFMA (measured on gfx950, the decode
//    page's lds_b8 note says the same for 16x16x128): lane l holds row l%32;
//    lane group g = l/32 holds tokens 16g..16g+15 and 32+16g..32+16g+15 of the
//    64-token half; the scale of lane l covers row l%32, 32-token block g of
//    the half.  The four scale bytes of a row for one 128-token step are one
//    dword (scales are row-major [rows][M/32]); shifted right by 8g it serves
//    both halves through op_sel = 0 and 2.
//  * Epilogue: the bf16 tile goes through LDS (the buffer the tile's last
//    step has freed) so that each store instruction writes whole 128-byte row
//    pieces; partial-line non-temporal stores measured several times slower.
//    The stores drain while the next tile's steps run.
#include "common.hpp"
#include "mx_gemm_core.hpp"
#include "../../include/moe_gg.h"

namespace moe_gg {
namespace {

using namespace mxgemm;
constexpr int NWAVE = 8;
constexpr int NTHREAD = NWAVE * 64;
constexpr int MAX_EXPERTS = 1024;

constexpr int LOADS_PER_STEP = 18;            // stage loads a loading wave issues per step

// One output tile: expert e, n-tile nt, k-tile kt.  The expert's tokens
// [o0, o1) are covered by nk 128-token steps from tok0 = 128 floor(o0/128);
// lo = o0 - tok0 and hi = o1 - tok0 bound the tokens that count.
struct Tile {
  int valid, e, nk, tok0, lo, hi, nt, kt;
};

__device__ __forceinline__ Tile tile_info(int t, int total, int T, int tilesK, const int *s_order,
                                          const int32_t *__restrict__ off, int M) {
  Tile ti;
  ti.valid = t < total;
  if (!ti.valid) { ti.e = ti.nk = ti.tok0 = ti.lo = ti.hi = ti.nt = ti.kt = 0; return ti; }
  const int rank0 = t / T;
  int u = t - rank0 * T;
  // Each XCD walks the ranked experts from its own starting point: tile t of
  // rank r takes the expert of rank (r + rot) mod E with rot = (t mod 8) E / 8.
  // With T a multiple of 8, t mod 8 = u mod 8, so for each u this is a
  // rotation of the ranks (every tile still done once), and the workgroups of
  // one XCD (t mod 8 fixed) keep sharing an expert.  The XCDs then reach
  // their tile ends at different times instead of all storing at once
  // (measured: 6-8% faster on 64 small experts, neutral at E=8).
  const int E = total / T;
  const int rank = (T & 7) == 0 ? (rank0 + (((t & 7) * E) >> 3)) % E : rank0;
  ti.e = __builtin_amdgcn_readfirstlane(s_order[rank]);
  const int o0 = clampi(off[ti.e], 0, M);
  const int o1 = clampi(off[ti.e + 1], o0, M);
  ti.tok0 = o0 / TT * TT;
  ti.nk = o1 > o0 ? (o1 + TT - 1) / TT - o0 / TT : 0;
  ti.lo = o0 - ti.tok0;
  ti.hi = o1 - ti.tok0;
  // XCD-aware order: with T a multiple of 8, the tiles a workgroup on XCD x
  // gets (u = x mod 8) become a contiguous run of T/8 in the grouped order.
  if ((T & 7) == 0) u = (u & 7) * (T >> 3) + (u >> 3);
  const int tilesN = T / tilesK;
  constexpr int GROUP = 4;            // n-tiles per group
  const int per_group = GROUP * tilesK;
  const int grp = u / per_group;
  const int first_n = grp * GROUP;
  const int gsz = min(tilesN - first_n, GROUP);
  const int w = u - grp * per_group;
  ti.nt = first_n + w % gsz;
  ti.kt = w / gsz;
  return ti;
}

// Position in a workgroup's stream of 128-token steps (tiles t = blockIdx.x,
// blockIdx.x + gridDim.x, ...; tiles of empty experts have no steps).
struct Cursor {
  int t, s;
  Tile ti;
};

template <bool EXACT>
__global__ __launch_bounds__(NTHREAD, 1) void wgrad_mxfp8_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, uint16_t *__restrict__ C,
    const uint8_t *__restrict__ SA, const uint8_t *__restrict__ SB,
    const int32_t *__restrict__ off, int M, int N, int K, int E) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE_BYTES];
  __shared__ int s_order[MAX_EXPERTS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tilesN = N / TB, tilesK = K / TA;     // x^T rows are the A operand, g^T rows the B operand
  const int T = tilesN * tilesK;
  const int total = E * T;
  const int G = gridDim.x;

  // ---- expert ranking: most 128-token steps first, ties by index --------
  {
    int *s_cnt = reinterpret_cast<int *>(smem);
    for (int e = tid; e < E; e += NTHREAD) {
      const int o0 = clampi(off[e], 0, M);
      const int o1 = clampi(off[e + 1], o0, M);
      s_cnt[e] = o1 > o0 ? (o1 + TT - 1) / TT - o0 / TT : 0;
    }
    __syncthreads();
    for (int e = tid; e < E; e += NTHREAD) {
      const int c = s_cnt[e];
      int rank = 0;
      for (int j = 0; j < E; ++j) {
        const int cj = s_cnt[j];
        rank += (cj > c) | ((cj == c) & (j < e));
      }
      s_order[rank] = e;
    }
    __syncthreads();
  }

  // ---- per-lane constants -------------------------------------------------
  const uint32_t smem_base = lds_addr(smem);
  const uint32_t Mb = static_cast<uint32_t>(M);
  const uint32_t scale_row = Mb / 32;      // bytes per scale row
  // Stage loads are issued by waves 4-7 only: a wave blocks while the
  // address FIFO is full, and so the other wave on each SIMD (0-3) starts
  // its MFMAs right after the barrier instead of waiting behind its loads.
  // Wave 4 + w4 fills blocks 8w4..8w4+7 of both operand tiles; block 8G + q
  // holds rows 64G + 8j + q (slot j), lane L -> slot L/8, bytes
  // 16(L%8)..16(L%8)+15 of the row's 128-token step; and the scale dwords of
  // rows 64w4..64w4+63 of both operands.
  const bool loader = wave >= 4;
  const int w4 = wave & 3;
  uint32_t voff_t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 64 * w4 + 8 * (lane >> 3) + i;
    voff_t[i] = static_cast<uint32_t>(r) * Mb + static_cast<uint32_t>(lane & 7) * 16u;
  }
  const uint32_t voff_s = static_cast<uint32_t>(w4 * 64 + lane) * scale_row;

  // MFMA operand addressing: wave (wk, wn) owns grad_w columns wk*128 .. +127
  // (k, A operand) and rows wn*64 .. +63 (n, B operand) of the tile
  const int wk = wave >> 2, wn = wave & 3;
  const int g = lane >> 5, l32 = lane & 31;
  uint32_t xrow[4], grow[2];
#pragma unroll
  for (int a = 0; a < 4; ++a) xrow[a] = ST_A + tile_row(wk * 128 + a * 32 + l32);
#pragma unroll
  for (int b = 0; b < 2; ++b) grow[b] = ST_B + tile_row(wn * 64 + b * 32 + l32);
  uint32_t chunk_off[2][2];   // [half][piece] -> 16-byte chunk offset within the row
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    chunk_off[h][0] = (4 * h + g) * 16;
    chunk_off[h][1] = (4 * h + 2 + g) * 16;
  }

  auto info = [&](int t) { return tile_info(t, total, T, tilesK, s_order, off, M); };
  // next position with a step, or t >= total when the stream is done
  auto advance = [&](Cursor &c) {
    if (c.s + 1 < c.ti.nk) { ++c.s; return; }
    c.s = 0;
    c.t += G;
    c.ti = info(c.t);
    while (c.ti.valid && c.ti.nk == 0) { c.t += G; c.ti = info(c.t); }
  };
  auto first = [&](int t) {
    Cursor c;
    c.t = t; c.s = 0; c.ti = info(t);
    while (c.ti.valid && c.ti.nk == 0) { c.t += G; c.ti = info(c.t); }
    return c;
  };

  int ops = 0;               // vector-memory instructions this wave has issued (uniform)
  int mark[2] = {0, 0};      // value of ops right after the loads of the step in buffer 0 / 1

  auto issue_stage = [&](const Cursor &c, uint32_t buf) {
    if (!loader) return;
    const Tile &ti = c.ti;
    const uint32_t tok = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ti.tok0 + c.s * TT));
    const v4i srd_x = make_srd(B + static_cast<size_t>(ti.kt) * TA * M, TA * Mb);
    const v4i srd_g = make_srd(A + static_cast<size_t>(ti.nt) * TB * M, TB * Mb);
    const uint32_t base = smem_base + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma_b128(srd_x, voff_t[i], tok, __builtin_amdgcn_readfirstlane(base + ST_A + (w4 * 8 + i) * BLK));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma_b128(srd_g, voff_t[i], tok, __builtin_amdgcn_readfirstlane(base + ST_B + (w4 * 8 + i) * BLK));
    const v4i srd_sx = make_srd(SB + static_cast<size_t>(ti.kt) * TA * scale_row, 256u * scale_row);
    const v4i srd_sg = make_srd(SA + static_cast<size_t>(ti.nt) * TB * scale_row, 256u * scale_row);
    dma_b32(srd_sx, voff_s, tok / 32, __builtin_amdgcn_readfirstlane(base + ST_SA + w4 * 256));
    dma_b32(srd_sg, voff_s, tok / 32, __builtin_amdgcn_readfirstlane(base + ST_SB + w4 * 256));
    ops += LOADS_PER_STEP;
  };
  // wait until the loads of the step in buffer b have landed: every vector
  // memory instruction issued after them may still be in flight
  auto wait_step = [&](int b) {
    const int younger = ops - mark[b];
    if (younger >= 50) wait_vmcnt<50>();
    else if (younger >= 34) wait_vmcnt<34>();
    else if (younger >= 18) wait_vmcnt<18>();
    else if (younger >= 16) wait_vmcnt<16>();
    else if (younger >= 8) wait_vmcnt<8>();
    else wait_vmcnt<0>();
  };

  // ---- prologue: first step in flight ----
  Cursor ld = first(blockIdx.x);        // next step to load into LDS
  uint32_t ld_buf = 0;
  if (ld.ti.valid) {
    issue_stage(ld, 0);
    mark[0] = ops;
    advance(ld);
  }

  uint32_t buf = 0;                    // buffer of the step being computed
  v16f acc[4][2];
  for (int t = blockIdx.x; t < total; t += G) {
    const Tile cur = info(t);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

#pragma unroll 1
    for (int s = 0; s < cur.nk; ++s) {
      wait_step(buf);
      barrier();
      ld_buf = buf ^ 1;
      if (ld.ti.valid) {
        issue_stage(ld, ld_buf);
        mark[ld_buf] = ops;
        advance(ld);
      }

      uint8_t *st = smem + buf * STAGE_BYTES;
      const int rlo = cur.lo - s * TT, rhi = cur.hi - s * TT;
      if (rlo > 0 || rhi < TT) {               // an expert's partial first or last step
        mask_stage_elements(st, tid, rlo, rhi);
        barrier();
      }
      if constexpr (EXACT)
        compute_step_bf16(st, acc, xrow, grow, wk, wn, l32, g);
      else
        compute_step(st, acc, xrow, grow, chunk_off, wk, wn, l32, g);
      buf ^= 1;
    }

    // ---- epilogue from registers -------------------------------------------
    // the output tile: 256 rows of K bf16 from (e*N + nt*256, kt*256), written
    // through a buffer descriptor with 32-bit byte offsets (non-temporal)
    const uint32_t Ku = static_cast<uint32_t>(K);
    const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
        C + (static_cast<size_t>(cur.e) * N + static_cast<size_t>(cur.nt) * TB) * K + static_cast<size_t>(cur.kt) * TA,
        static_cast<short>(0), static_cast<int>(TB * Ku * 2u), 0x00020000);
    if (cur.nk == 0) store_zero_tile(crsrc, Ku, tid);     // empty expert: +0.0 everywhere
    else store_tile(acc, smem + (buf ^ 1) * STAGE_BYTES, crsrc, Ku, wk, wn, tid);
    ops += STORES_PER_TILE;
  }
  wait_vmcnt<0>();
}

}  // namespace
}  // namespace moe_gg

namespace moe_gg {
namespace {
int launch_wgrad(bool exact, const uint8_t *A, const uint8_t *B, uint16_t *C, const uint8_t *scale_A,
                 const uint8_t *scale_B, const int32_t *expert_off, int M, int N, int K, int E,
                 hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || E <= 0 || !expert_off) return MOE_GG_EINVAL;
  if (N == 0 || K == 0) return MOE_GG_OK;                 // no output element
  // no tokens (M = 0): every expert is empty and its rows are written +0.0;
  // the operands, then of zero size, are never read and may be null
  if (!C || (M > 0 && (!A || !B || !scale_A || !scale_B))) return MOE_GG_EINVAL;
  if (M % 32) return MOE_GG_EINVAL;                       // whole 32-token scale blocks
  // the kernel steps through the tokens 128 at a time, with scale dwords of
  // four blocks (rows of M/32 scale bytes stay 4-byte aligned)
  if (M % TT || N % TB || K % TA || E > MAX_EXPERTS) return MOE_GG_EUNSUPPORTED;
  // the buffer descriptors address one 256-row operand panel with 32-bit offsets
  if (static_cast<uint64_t>(TA) * static_cast<uint64_t>(M) > 0xFFFFFFFFull) return MOE_GG_EUNSUPPORTED;
  // and one 256-row tile of the bf16 output (a signed 32-bit size)
  if (static_cast<uint64_t>(TB) * static_cast<uint64_t>(K) * 2u > 0x7FFFFFFFull) return MOE_GG_EUNSUPPORTED;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_GG_ELAUNCH;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_GG_ELAUNCH;
  const int64_t total = static_cast<int64_t>(E) * (N / TB) * (K / TA);
  if (total > 0x7FFFFFFF) return MOE_GG_EUNSUPPORTED;
  if (const int st = check_offsets_if_asked(expert_off, E, M, stream)) return st;
  const int grid = static_cast<int>(total < cus ? total : cus);
  if (exact)
    hipLaunchKernelGGL(wgrad_mxfp8_kernel<true>, dim3(grid), dim3(NTHREAD), 0, stream, A, B, C, scale_A,
                       scale_B, expert_off, M, N, K, E);
  else
    hipLaunchKernelGGL(wgrad_mxfp8_kernel<false>, dim3(grid), dim3(NTHREAD), 0, stream, A, B, C, scale_A,
                       scale_B, expert_off, M, N, K, E);
  return hipGetLastError() == hipSuccess ? MOE_GG_OK : MOE_GG_ELAUNCH;
}
}  // namespace
}  // namespace moe_gg

extern "C" MOE_GG_API int moe_gg_wgrad_mxfp8(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                             const uint8_t *scale_A, const uint8_t *scale_B,
                                             const int32_t *expert_off, int M, int N, int K, int E,
                                             hipStream_t stream) {
  return moe_gg::launch_wgrad(true, A, B, C, scale_A, scale_B, expert_off, M, N, K, E, stream);
}

extern "C" MOE_GG_API int moe_gg_wgrad_mxfp8_fast(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                                  const uint8_t *scale_A, const uint8_t *scale_B,
                                                  const int32_t *expert_off, int M, int N, int K, int E,
                                                  hipStream_t stream) {
  return moe_gg::launch_wgrad(false, A, B, C, scale_A, scale_B, expert_off, M, N, K, E, stream);
}
