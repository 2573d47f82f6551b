// Grouped f32 data gradient on gfx950 and its row -> expert map:
//   dx[r][k] = sum_n g[r][n] W[e(r)][n][k],   e(r): off[e] <= r < off[e+1]
// (the oarust page "grouped_gemm_m_data_backward.slang": push constants,
// expert_for_row, the per-row-expert path of tiles whose rows span several
// experts, the overwriting store).
//
// Design (gfx950):
//  * Output tiles of 128 rows x 128 columns, 256 threads = 4 waves, wave w
//    the 32-column strip 32w..32w+31 of the tile as up to four 32 x 32
//    v_mfma_f32_32x32x2_f32 accumulators, one per 32-row block (f32 products,
//    f32 accumulation: the f32 matrix-core rate).
//  * The tile's first and last row give its expert range with a wave-uniform
//    binary search over the offsets.  A tile inside one expert runs one pass
//    over n with that expert's W.  A tile whose rows straddle experts runs one
//    pass per expert present; a pass multiplies only the 32-row blocks that
//    hold its expert's rows and stores only those rows at its end, so every
//    row is written once, with exactly its own expert's products (another
//    expert's rows inside those blocks give accumulator rows that are never
//    stored), and a pass over r rows costs ceil(r/32)/4 of a full
//    one (two passes of a straddling tile together cost 1.25-1.5 passes
//    instead of 2).
//  * When the tile's 128 columns lie inside K and N is a nonzero multiple of
//    32 (the common case), a pass is dgrad_pass_dma: chunks of 16 n whose g
//    and W go by LDS-DMA into a ring of four LDS stages, three chunks ahead,
//    with no bounds tests in the loop (the global latency is what one chunk
//    ahead left exposed).
//  * Otherwise dgrad_pass: the contraction in chunks of 32 n, g[128 x 32]
//    and W_e[32 x 128] read with 16-byte coalesced loads (g rows and W rows
//    are contiguous along n and k) into registers, one chunk ahead (two for
//    a pass over fewer than four row blocks), then written to a
//    double-buffered LDS stage while the previous chunk is multiplied.
//  * One-dimensional grid in an XCD-aware order: the tiles one XCD runs at
//    once form a patch of row tiles x 8 column tiles sharing g rows and W
//    columns in that XCD's L2.
//  * In dgrad_pass's chunk the MFMA k index s = 0..15 of lane group h = l/32
//    is n = 16h + s, so each lane reads its 16 g values with 4 ds_read_b128.  g
//    rows in LDS are 128 bytes with their 16-byte groups XOR-swizzled by
//    (row/2) mod 8; W rows for n >= 16 have column bit 5 flipped, so the two
//    half-waves of a W operand read land in different bank halves.
#include "common.hpp"
#include "../../include/moe_gg.h"

namespace moe_gg {
namespace {

constexpr int BM = 128;      // rows per tile
constexpr int BK = 128;      // output columns (k) per tile
constexpr int BC = 32;       // contraction (n) per chunk
constexpr int NTHREAD = 256;
constexpr int XGROUP = 8;    // column tiles per group of the XCD-aware tile order

constexpr int LG = 0;                    // g chunk   [128][32] f32 = 16 KB
constexpr int LW = BM * BC * 4;          // W chunk   [32][128] f32 = 16 KB
constexpr int STAGE = LW + BC * BK * 4;  // 32 KB

__device__ __forceinline__ uint32_t g_lds_off(int row, int q /*16B group 0..7*/) {
  return LG + row * (BC * 4) + ((q ^ ((row >> 1) & 7)) << 4);
}
__device__ __forceinline__ uint32_t w_lds_off(int n, int col /*float index*/) {
  return LW + n * (BK * 4) + ((col ^ ((n >> 4) << 5)) << 2);
}

// One expert pass over a tile: rows [lo, hi) of expert e (W_e = We), which lie
// in the NRB 32-row blocks ib0 .. ib0 + NRB - 1 of the tile; the whole
// contraction in chunks of 32 n, loaded ahead into registers and
// double-buffered through LDS, then the pass's rows stored.  Every wave runs
// it (it contains the workgroup's barriers).
template <int NRB>
__device__ __forceinline__ void dgrad_pass(const float *__restrict__ G, const float *__restrict__ We,
                                           float *__restrict__ DX, uint8_t *smem, int M, int N, int K, int r0,
                                           int k0, int lo, int hi, int ib0, int tid, int wave) {
  // the per-lane offsets below are formed here, not hoisted to the kernel's
  // start where they would stay live across every pass (and spill)
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  // global -> register loader coordinates (NRB float4 of g and 4 of W per
  // thread; only the pass's row blocks are loaded and staged, the MFMAs read
  // no other rows)
  const int g_row = tid >> 3, g_q = tid & 7;      // rows g_row + 32(ib0 + j), group g_q
  const int w_n = tid >> 5, w_q = tid & 31;       // n rows w_n + 8i, float4 column w_q
  const int nchunks = (N + BC - 1) / BC;

  v16f acc[NRB];
#pragma unroll
  for (int i = 0; i < NRB; ++i)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[i][x] = 0.f;

  // Chunks are loaded DEPTH ahead into registers.  A pass with fewer than four
  // row blocks (little MFMA work per chunk) keeps two register sets: chunk
  // c + 2 is loaded while chunk c multiplies and chunk c + 1 waits in the
  // other set, so the global load latency has two chunks of MFMA time to hide
  // behind.  A full pass loads one chunk ahead (a second set would not fit
  // beside its accumulators in 256 VGPRs).
  constexpr int DEPTH = NRB < 4 ? 2 : 1;
  v4f greg[DEPTH][NRB], wreg[DEPTH][4];
  auto load_chunk = [&](int c, int set) __attribute__((always_inline)) {
    const int n0 = c * BC;
#pragma unroll
    for (int j = 0; j < NRB; ++j) {
      const int r = r0 + g_row + 32 * (ib0 + j);
      const int n = n0 + 4 * g_q;
      if (r >= lo && r < hi && n < N)
        greg[set][j] = *reinterpret_cast<const v4f *>(G + static_cast<size_t>(r) * N + n);
      else
        greg[set][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + w_n + 8 * i;
      const int k = k0 + 4 * w_q;
      if (n < N && k < K)
        wreg[set][i] = *reinterpret_cast<const v4f *>(We + static_cast<size_t>(n) * K + k);
      else
        wreg[set][i] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store_chunk = [&](int set, int buf) __attribute__((always_inline)) {
    uint8_t *st = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < NRB; ++j)
      *reinterpret_cast<v4f *>(st + g_lds_off(g_row + 32 * (ib0 + j), g_q)) = greg[set][j];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<v4f *>(st + w_lds_off(w_n + 8 * i, 4 * w_q)) = wreg[set][i];
  };

  // chunk c (c % 2 = P) multiplies from LDS buffer P
  auto chunk = [&](int c, auto parity) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    constexpr int LOAD_SET = DEPTH == 2 ? P : 0, NEXT_SET = DEPTH == 2 ? (P ^ 1) : 0;
    if (c + DEPTH < nchunks) load_chunk(c + DEPTH, LOAD_SET);
    const uint8_t *st = smem + P * STAGE;
    // this lane's 16 n values n = 16h .. 16h+15 in four groups of four: group
    // q's g values (one 16-byte read per row block) and W values are read
    // while group q - 1 multiplies, into a second register set
    v4f ga[2][NRB];
    float wv[2][4];
    auto read_group = [&](int q, v4f (&gq)[NRB], float (&wq)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NRB; ++i) gq[i] = *reinterpret_cast<const v4f *>(st + g_lds_off((ib0 + i) * 32 + l32, 4 * h + q));
#pragma unroll
      for (int t = 0; t < 4; ++t)
        wq[t] = *reinterpret_cast<const float *>(st + w_lds_off(16 * h + 4 * q + t, wave * 32 + l32));
    };
    read_group(0, ga[0], wv[0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < 3) read_group(q + 1, ga[(q + 1) & 1], wv[(q + 1) & 1]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < NRB; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(ga[q & 1][i][t], wv[q & 1][t], acc[i], 0, 0, 0);
      // the next group's reads ahead of this group's MFMAs, and no later
      // group's reads hoisted above them
      if (q < 3) {
        __builtin_amdgcn_sched_group_barrier(0x100, NRB + 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * NRB, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c + 1 < nchunks) store_chunk(NEXT_SET, P ^ 1);
    barrier();
  };

  load_chunk(0, 0);
  if (DEPTH == 2 && nchunks > 1) load_chunk(1, DEPTH - 1);
  store_chunk(0, 0);
  barrier();
#pragma unroll 1
  for (int c = 0; c < nchunks; c += 2) {
    chunk(c, std::integral_constant<int, 0>());
    if (c + 1 < nchunks) chunk(c + 1, std::integral_constant<int, 1>());
  }

  // this pass's rows: register x of acc[i] is row (ib0 + i)*32 + 8(x/4) + 4h +
  // x%4 of the tile, column 32 wave + l32
  const int col = k0 + wave * 32 + l32;
  if (col < K) {
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int row = r0 + (ib0 + i) * 32 + 8 * (x >> 2) + 4 * h + (x & 3);
        if (row >= lo && row < hi) DX[static_cast<size_t>(row) * K + col] = acc[i][x];
      }
  }
}

// The same pass, for a tile whose 128 columns lie inside K, with N a nonzero
// multiple of 32 (the common case), with a deeper pipeline than dgrad_pass's
// and no bounds tests in its loop.  The contraction runs in chunks of 16 n;
// both operands of a chunk go by LDS-DMA (no staging registers) into a ring
// of four LDS stages, chunk c + 3 issued while chunk c multiplies, so the
// global latency has three chunks of MFMA time to hide behind (one and a half
// of dgrad_pass's 32-n chunks, against one there).  Past the end
// the last chunk is fetched again into the ring's next stage, which no chunk
// reads any more, so every chunk issues the same four DMAs per wave and waits
// on one count.  All 128 g rows of the tile are fetched: rows of other
// experts are either outside the pass's blocks (not multiplied) or give
// accumulator rows that are not stored; rows past M fall outside the g
// descriptor, which reads them as zeros without touching memory.
constexpr int FC = 16;                       // n per chunk
constexpr int FG = BM * FC * 4;              // g [128][16] f32 = 8 KB, then W [16][128] = 8 KB
constexpr int FSTAGE = FG + FC * BK * 4;     // 16 KB
constexpr int FNS = 4;                       // stages in the ring (64 KB)

// g rows are 64 bytes, their 16-byte groups XOR-swizzled by (row/4) mod 4, so
// the 16 rows one ds_read_b128 phase touches (16 lanes, 64 banks of 4 bytes)
// fall on 16 distinct 16-byte bank groups;
// W rows for n mod 16 >= 8 have column bit 5 flipped, so the two half-waves
// of a W read land in different bank halves.
__device__ __forceinline__ uint32_t fg_off(int row, int q /*16B group 0..3*/) {
  return row * (FC * 4) + ((q ^ ((row >> 2) & 3)) << 4);
}
__device__ __forceinline__ uint32_t fw_off(int n, int col /*float index*/) {
  return FG + n * (BK * 4) + ((col ^ (((n >> 3) & 1) << 5)) << 2);
}

template <int NRB, bool ALLROWS>
__device__ __forceinline__ void dgrad_pass_dma(const float *__restrict__ G, const float *__restrict__ We,
                                               float *__restrict__ DX, uint8_t *smem, int M, int N, int K, int r0,
                                               int k0, int lo, int hi, int ib0, int tid, int wave) {
  asm volatile("" : "+v"(tid));   // as in dgrad_pass
  // vmcnt(0) in a form the compiler sees (an asm wait is opaque to it): a
  // previous pass's stores and loads are complete, so the compiler places no
  // wait of its own in the loop below (it would otherwise drain the ring's
  // DMAs to protect their registers).  Immediate: vmcnt 0 (bits 3:0, 15:14),
  // expcnt 7 (bits 6:4) and lgkmcnt 15 (bits 11:8), i.e. no wait on those.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  const int lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int nch = N / FC;
  const uint32_t smem_base = lds_addr(smem);

  // DMA instruction j of wave w: g rows (2w + j) * 16 + lane/4, 16-byte slot
  // lane % 4; W rows n = (2w + j) * 2 + lane/32, columns 4 (lane % 32) .. +3.
  // Each lane fetches the global element that the swizzle puts in its slot.
  const v4i srd_g = make_srd(G + static_cast<size_t>(r0) * N, static_cast<uint32_t>(min(M - r0, BM)) * N * 4u);
  const v4i srd_w = make_srd(We + k0, 0xFFFFFFFFu);
  uint32_t vg[2], vw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (2 * wave + j) * 16 + (lane >> 2);
    vg[j] = static_cast<uint32_t>(row) * N * 4u + 16u * static_cast<uint32_t>((lane & 3) ^ ((row >> 2) & 3));
    const int n = (2 * wave + j) * 2 + (lane >> 5);
    vw[j] = static_cast<uint32_t>(n) * K * 4u + 4u * static_cast<uint32_t>((4 * (lane & 31)) ^ (((n >> 3) & 1) << 5));
  }
  // chunk c's operands into stage `stage`
  auto issue = [&](int c, int stage) __attribute__((always_inline)) {
    const uint32_t st = __builtin_amdgcn_readfirstlane(smem_base + stage * FSTAGE + 2 * wave * 1024);
    const uint32_t sg = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(c) * FC * 4u);
    const uint32_t sw = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(c) * FC * K * 4u);
    dma_b128(srd_g, vg[0], sg, st);
    dma_b128(srd_g, vg[1], sg, st + 1024);
    dma_b128(srd_w, vw[0], sw, st + FG);
    dma_b128(srd_w, vw[1], sw, st + FG + 1024);
  };

  v16f acc[NRB];
#pragma unroll
  for (int i = 0; i < NRB; ++i)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[i][x] = 0.f;

  // lane (h, l32) takes contraction slots n = 8h + s, s = 0..7: g row
  // 32(ib0 + i) + l32 groups 2h and 2h + 1, W rows 8h + s at column 32 wave + l32
  // (the swizzle of row 32 b + l32 does not depend on b)
  const uint32_t blk = ib0 * 32 * FC * 4;
  const uint32_t ga_off0 = blk + fg_off(l32, 2 * h), ga_off1 = blk + fg_off(l32, 2 * h + 1);
  const uint32_t w_col = 32 * wave + l32;

#pragma unroll
  for (int c = 0; c < FNS - 1; ++c) issue(min(c, nch - 1), c);
  wait_vmcnt<8>();      // chunk 0 landed (younger: chunks 1 and 2, 4 DMAs each)
  barrier();
#pragma unroll 1
  for (int c = 0; c < nch; ++c) {
    issue(min(c + FNS - 1, nch - 1), (c + FNS - 1) % FNS);   // stage (c - 1) % 4, freed by the last barrier
    const uint8_t *st = smem + (c % FNS) * FSTAGE;
    v4f ga[2][NRB];
    float wv[8];
#pragma unroll
    for (int i = 0; i < NRB; ++i) ga[0][i] = *reinterpret_cast<const v4f *>(st + ga_off0 + i * 32 * FC * 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) wv[t] = *reinterpret_cast<const float *>(st + fw_off(8 * h + t, w_col));
#pragma unroll
    for (int i = 0; i < NRB; ++i) ga[1][i] = *reinterpret_cast<const v4f *>(st + ga_off1 + i * 32 * FC * 4);
#pragma unroll
    for (int t = 4; t < 8; ++t) wv[t] = *reinterpret_cast<const float *>(st + fw_off(8 * h + t, w_col));
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < NRB; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(ga[g2][i][t], wv[4 * g2 + t], acc[i], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);   // the chunk's MFMAs stay ahead of the wait and the barrier
    wait_vmcnt<8>();    // chunk c + 1 landed (younger: chunks c + 2 and c + 3)
    barrier();
  }
  wait_vmcnt<0>();      // the repeated DMAs past the end land before the workgroup ends

  // register x of acc[i] is row (ib0 + i)*32 + 8(x/4) + 4h + x%4 of the tile;
  // the pass stores the rows in [lo, hi) (ALLROWS: all 128).  The base is made opaque here so
  // that the store addresses are formed after the loop instead of being
  // hoisted (and spilled) ahead of it.
  const int row0 = r0 + ib0 * 32 + 4 * h;
  float *dst = DX + static_cast<size_t>(row0) * K + k0 + wave * 32 + l32;
  asm volatile("" : "+v"(dst));
#pragma unroll
  for (int i = 0; i < NRB; ++i)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int dr = i * 32 + 8 * (x >> 2) + (x & 3);
      if (ALLROWS || (row0 + dr >= lo && row0 + dr < hi)) dst[static_cast<size_t>(dr) * K] = acc[i][x];
    }
}

__global__ __launch_bounds__(NTHREAD, 2) void dgrad_f32_kernel(
    const float *__restrict__ G, const float *__restrict__ W, float *__restrict__ DX,
    const int32_t *__restrict__ off, int M, int N, int K, int E) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE > FNS * FSTAGE ? 2 * STAGE : FNS * FSTAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // column strip 32 wave .. +31
  // Tile of this workgroup.  Workgroup b runs on XCD b mod 8, so with the
  // tile count T a multiple of 8 the workgroups of one XCD take the
  // contiguous range u = (b mod 8) T/8 + b/8 of a grouped order: groups of
  // XGROUP column tiles, row-major inside a group.  The tiles one XCD runs
  // at once then form a patch of about 64/XGROUP row tiles x XGROUP column
  // tiles, which share g rows and W columns in that XCD's L2 (column tiles
  // alone would give each XCD every g row).
  const int tilesR = (M + BM - 1) / BM, tilesC = (K + BK - 1) / BK;
  const int T = tilesR * tilesC;
  const int b = blockIdx.x;
  const int u = (T & 7) == 0 ? (b & 7) * (T >> 3) + (b >> 3) : b;
  const int grp = u / (tilesR * XGROUP);
  const int gw = min(XGROUP, tilesC - grp * XGROUP);
  const int w = u - grp * tilesR * XGROUP;
  const int r0 = (w / gw) * BM;
  const int k0 = (grp * XGROUP + w % gw) * BK;
  const int r_last = min(r0 + BM, M) - 1;
  const int e_first = __builtin_amdgcn_readfirstlane(expert_of_row(off, E, r0));
  const int e_last = __builtin_amdgcn_readfirstlane(expert_of_row(off, E, r_last));

  // the LDS-DMA passes: full columns, N a nonzero multiple of 32, and offsets
  // that fit the 32-bit buffer addressing (g: 128 rows, W_e: one expert)
  const bool dma = k0 + BK <= K && N >= BC && N % BC == 0 && N <= (1 << 22) &&
                   static_cast<int64_t>(N) * K < (1 << 29);
  for (int e = e_first; e <= e_last; ++e) {
    const int lo = max(clampi(off[e], 0, M), r0);
    const int hi = min(clampi(off[e + 1], 0, M), r0 + BM);
    if (hi <= lo) continue;
    const float *We = W + static_cast<size_t>(e) * N * K;
    // the 32-row blocks [ib0, ib1) of the tile that hold this expert's rows
    const int ib0 = __builtin_amdgcn_readfirstlane((lo - r0) >> 5);
    const int ib1 = __builtin_amdgcn_readfirstlane((hi - r0 + 31) >> 5);
    if (dma) {
      switch (ib1 - ib0) {
        case 1: dgrad_pass_dma<1, false>(G, We, DX, smem, M, N, K, r0, k0, lo, hi, ib0, tid, wave); break;
        case 2: dgrad_pass_dma<2, false>(G, We, DX, smem, M, N, K, r0, k0, lo, hi, ib0, tid, wave); break;
        case 3: dgrad_pass_dma<3, false>(G, We, DX, smem, M, N, K, r0, k0, lo, hi, ib0, tid, wave); break;
        default:
          if (lo == r0 && hi == r0 + BM)
            dgrad_pass_dma<4, true>(G, We, DX, smem, M, N, K, r0, k0, lo, hi, ib0, tid, wave);
          else
            dgrad_pass_dma<4, false>(G, We, DX, smem, M, N, K, r0, k0, lo, hi, ib0, tid, wave);
          break;
      }
    } else {
      switch (ib1 - ib0) {
        case 1: dgrad_pass<1>(G, We, DX, smem, M, N, K, r0, k0, lo, hi, ib0, tid, wave); break;
        case 2: dgrad_pass<2>(G, We, DX, smem, M, N, K, r0, k0, lo, hi, ib0, tid, wave); break;
        case 3: dgrad_pass<3>(G, We, DX, smem, M, N, K, r0, k0, lo, hi, ib0, tid, wave); break;
        default: dgrad_pass<4>(G, We, DX, smem, M, N, K, r0, k0, lo, hi, ib0, tid, wave); break;
      }
    }
  }
  // rows before off[0] or from off[E] on belong to no expert: +0.0
  const int c0 = clampi(off[0], 0, M), c1 = max(c0, clampi(off[E], 0, M));
  if (r0 < c0 || r_last >= c1) {
    const int lane = tid & 63;
    const int col = k0 + wave * 32 + (lane & 31);
    if (col < K)
      for (int rr = lane >> 5; rr < BM; rr += 2) {
        const int row = r0 + rr;
        if (row < M && (row < c0 || row >= c1)) DX[static_cast<size_t>(row) * K + col] = 0.f;
      }
  }
}

__global__ void row_experts_kernel(const int32_t *__restrict__ off, int E, int M, int32_t *__restrict__ out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < M) out[r] = expert_of_row(off, E, r);
}

}  // namespace
}  // namespace moe_gg

extern "C" MOE_GG_API int moe_gg_dgrad_f32(const float *A, const float *B, float *C,
                                           const int32_t *expert_off, int M, int N, int K, int E,
                                           hipStream_t stream) {
  using namespace moe_gg;
  if (M < 0 || N < 0 || K < 0 || E <= 0 || !expert_off) return MOE_GG_EINVAL;
  if (M == 0 || K == 0) return MOE_GG_OK;                 // no output element
  // an empty contraction (N = 0) writes zeros; g and W, then of zero size,
  // are never read and may be null
  if (!C || (N > 0 && (!A || !B))) return MOE_GG_EINVAL;
  if (K % 4 || N % 4) return MOE_GG_EUNSUPPORTED;
  if (const int st = check_offsets_if_asked(expert_off, E, M, stream)) return st;
  const int64_t tiles = static_cast<int64_t>((K + BK - 1) / BK) * ((M + BM - 1) / BM);
  if (tiles > 0x7FFFFFFF) return MOE_GG_EUNSUPPORTED;
  hipLaunchKernelGGL(dgrad_f32_kernel, dim3(static_cast<uint32_t>(tiles)), dim3(NTHREAD), 0, stream, A, B, C,
                     expert_off, M, N, K, E);
  return hipGetLastError() == hipSuccess ? MOE_GG_OK : MOE_GG_ELAUNCH;
}

extern "C" MOE_GG_API int moe_gg_row_experts(const int32_t *expert_off, int E, int M, int32_t *out,
                                             hipStream_t stream) {
  using namespace moe_gg;
  if (!expert_off || M < 0 || E <= 0) return MOE_GG_EINVAL;
  if (M == 0) return MOE_GG_OK;
  if (!out) return MOE_GG_EINVAL;
  const int threads = 256;
  hipLaunchKernelGGL(row_experts_kernel, dim3((M + threads - 1) / threads), dim3(threads), 0, stream,
                     expert_off, E, M, out);
  return hipGetLastError() == hipSuccess ? MOE_GG_OK : MOE_GG_ELAUNCH;
}
