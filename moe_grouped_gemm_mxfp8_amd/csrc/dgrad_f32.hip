// Grouped f32 data gradient on gfx950 and its row -> expert map:
//   dx[r][k] = sum_n g[r][n] W[e(r)][n][k],   e(r): off[e] <= r < off[e+1]
// (the oarust page "grouped_gemm_m_data_backward.slang": push constants,
// expert_for_row, the per-row-expert path of tiles whose rows span several
// experts, the overwriting store).
//
// Design (gfx950):
//  * Output tiles of 128 rows x 128 columns, 256 threads = 4 waves as 2 x 2,
//    each wave a 64 x 64 patch of 2 x 2 v_mfma_f32_32x32x2_f32 accumulators
//    (f32 products, f32 accumulation: the f32 matrix-core rate).
//  * The tile's first and last row give its expert range with a wave-uniform
//    binary search over the offsets.  A tile inside one expert runs one pass
//    over n with that expert's W.  A tile whose rows straddle experts runs one
//    pass per expert present, each pass with the g rows of the other experts
//    masked to zero, into the same accumulators: every row ends with exactly
//    its own expert's products.
//  * The contraction runs in chunks of 32 n.  g[128 x 32] and W_e[32 x 128]
//    are read with 16-byte coalesced loads (g rows and W rows are contiguous
//    along n and k) into registers, then written to a double-buffered LDS
//    stage while the previous chunk is multiplied.
//  * Inside a chunk the MFMA k index s = 0..15 of lane group h = l/32 is
//    n = 16h + s, so each lane reads its 16 g values with 4 ds_read_b128.  g
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

constexpr int LG = 0;                    // g chunk   [128][32] f32 = 16 KB
constexpr int LW = BM * BC * 4;          // W chunk   [32][128] f32 = 16 KB
constexpr int STAGE = LW + BC * BK * 4;  // 32 KB

__device__ __forceinline__ uint32_t g_lds_off(int row, int q /*16B group 0..7*/) {
  return LG + row * (BC * 4) + ((q ^ ((row >> 1) & 7)) << 4);
}
__device__ __forceinline__ uint32_t w_lds_off(int n, int col /*float index*/) {
  return LW + n * (BK * 4) + ((col ^ ((n >> 4) << 5)) << 2);
}

__global__ __launch_bounds__(NTHREAD, 2) void dgrad_f32_kernel(
    const float *__restrict__ G, const float *__restrict__ W, float *__restrict__ DX,
    const int32_t *__restrict__ off, int M, int N, int K, int E) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;

  const int r0 = blockIdx.y * BM;
  const int k0 = blockIdx.x * BK;
  const int r_last = min(r0 + BM, M) - 1;
  const int e_first = __builtin_amdgcn_readfirstlane(expert_of_row(off, E, r0));
  const int e_last = __builtin_amdgcn_readfirstlane(expert_of_row(off, E, r_last));

  // global -> register loader coordinates (4 float4 of g and 4 of W per thread)
  const int g_row = tid >> 3, g_q = tid & 7;      // rows g_row + 32i, group g_q
  const int w_n = tid >> 5, w_q = tid & 31;       // n rows w_n + 8i, float4 column w_q

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[i][j][x] = 0.f;

  const int nchunks = (N + BC - 1) / BC;

  for (int e = e_first; e <= e_last; ++e) {
    const int lo = max(clampi(off[e], 0, M), r0);
    const int hi = min(clampi(off[e + 1], 0, M), r0 + BM);
    if (hi <= lo) continue;
    const float *We = W + static_cast<size_t>(e) * N * K;

    v4f greg[4], wreg[4];
    auto load_chunk = [&](int c) {
      const int n0 = c * BC;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + g_row + 32 * i;
        const int n = n0 + 4 * g_q;
        if (r >= lo && r < hi && n < N)
          greg[i] = *reinterpret_cast<const v4f *>(G + static_cast<size_t>(r) * N + n);
        else
          greg[i] = (v4f){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + w_n + 8 * i;
        const int k = k0 + 4 * w_q;
        if (n < N && k < K)
          wreg[i] = *reinterpret_cast<const v4f *>(We + static_cast<size_t>(n) * K + k);
        else
          wreg[i] = (v4f){0.f, 0.f, 0.f, 0.f};
      }
    };
    auto store_chunk = [&](int buf) {
      uint8_t *st = smem + buf * STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<v4f *>(st + g_lds_off(g_row + 32 * i, g_q)) = greg[i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<v4f *>(st + w_lds_off(w_n + 8 * i, 4 * w_q)) = wreg[i];
    };

    load_chunk(0);
    store_chunk(0);
    barrier();
    for (int c = 0; c < nchunks; ++c) {
      const int buf = c & 1;
      if (c + 1 < nchunks) load_chunk(c + 1);
      const uint8_t *st = smem + buf * STAGE;
      // this lane's 16 g values per row block: n = 16h .. 16h+15
      v4f ga[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wr * 64 + i * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ga[i][q] = *reinterpret_cast<const v4f *>(st + g_lds_off(row, 4 * h + q));
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        float wb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          wb[j] = *reinterpret_cast<const float *>(st + w_lds_off(16 * h + s, wc * 64 + j * 32 + l32));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(ga[i][s >> 2][s & 3], wb[j], acc[i][j], 0, 0, 0);
      }
      if (c + 1 < nchunks) {
        store_chunk(buf ^ 1);
      }
      barrier();
    }
  }

  // store: register x of acc[i][j] is row wr*64 + i*32 + 8(x/4) + 4h + x%4, column wc*64 + j*32 + l32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = k0 + wc * 64 + j * 32 + l32;
      if (col >= K) continue;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int row = r0 + wr * 64 + i * 32 + 8 * (x >> 2) + 4 * h + (x & 3);
        if (row < M) DX[static_cast<size_t>(row) * K + col] = acc[i][j][x];
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
  if (!A || !B || !C || !expert_off) return MOE_GG_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || E <= 0) return MOE_GG_EINVAL;
  if (K % 4 || N % 4) return MOE_GG_EUNSUPPORTED;
  const dim3 grid((K + BK - 1) / BK, (M + BM - 1) / BM);
  if (grid.y > 65535u) return MOE_GG_EUNSUPPORTED;
  hipLaunchKernelGGL(dgrad_f32_kernel, grid, dim3(NTHREAD), 0, stream, A, B, C, expert_off, M, N, K, E);
  return hipGetLastError() == hipSuccess ? MOE_GG_OK : MOE_GG_ELAUNCH;
}

extern "C" MOE_GG_API int moe_gg_row_experts(const int32_t *expert_off, int E, int M, int32_t *out,
                                             hipStream_t stream) {
  using namespace moe_gg;
  if (!expert_off || !out || M <= 0 || E <= 0) return MOE_GG_EINVAL;
  const int threads = 256;
  hipLaunchKernelGGL(row_experts_kernel, dim3((M + threads - 1) / threads), dim3(threads), 0, stream,
                     expert_off, E, M, out);
  return hipGetLastError() == hipSuccess ? MOE_GG_OK : MOE_GG_ELAUNCH;
}
