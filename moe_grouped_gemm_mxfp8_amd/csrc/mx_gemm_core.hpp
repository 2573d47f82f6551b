// Shared core of the block-scaled MXFP8 GEMM kernels on gfx950: the LDS
// stage layout, the step of 128 contraction elements for one wave's
// 128 x 64 patch, and the two-pass split of the g-role codes.
//
// A stage holds two operand tiles of 256 rows x 128 contraction bytes (E4M3)
// and their scale dwords: the x-role tile (MFMA A operand, whose rows become
// the MFMA output rows) and the g-role tile (MFMA B operand).  An operand tile
// in LDS is 32 blocks of 8 rows x 128 bytes, each block padded by 16 bytes;
// one stage-load instruction fills a block, eight lanes per row reading the
// row's 128 bytes in order, and the padding puts the 16 rows an MFMA operand
// read touches at once on 16 distinct bank groups.
//
// The x-role tile may instead hold E2M1 (fp4) codes, two per byte (MFMA
// format 4): 256 rows x 64 bytes per step, 16 blocks of 16 rows x 64 bytes,
// each padded by 16 bytes.  Row r sits in block 4(r/64) + r%4 at slot
// (r%64)/4, so a stage load fills a block with four lanes per row reading
// its 64 bytes in order, and the 16 rows an operand read touches at once
// (r%4 and (r/4)%4 all different) fall on 16 distinct bank groups.  A lane's
// fp4 operand of a 64-deep half is 16 bytes: the 32 codes of its 32-element
// block (lane group g = block g of the half), low nibble first.
#pragma once

#include "common.hpp"

namespace moe_gg {
namespace mxgemm {

constexpr int TK = 256;             // rows of the x-role tile (MFMA A operand)
constexpr int TN = 256;             // rows of the g-role tile (MFMA B operand)
constexpr int TT = 128;             // contraction elements per pipeline step
// Row r of a 64-row group G = r/64 sits in block 8G + r%8 at slot (r%64)/8.
constexpr int BLK = 8 * TT + 16;              // 1040: 8 rows of 128 bytes + padding
constexpr int TILE_BYTES = 32 * BLK;          // 33280: a 256-row operand tile
constexpr int ST_X = 0;                       // x-role tile
constexpr int ST_G = ST_X + TILE_BYTES;       // g-role tile
constexpr int ST_SX = ST_G + TILE_BYTES;      // x-role scale dwords [256]
constexpr int ST_SG = ST_SX + TK * 4;         // g-role scale dwords [256]
constexpr int STAGE_BYTES = ST_SG + TN * 4;   // 68608
static_assert(8 * 8192 <= STAGE_BYTES, "the epilogue stages eight 8 KB wave regions in one buffer");

// LDS byte offset of row r (0..255) inside an operand tile.
__device__ __forceinline__ uint32_t tile_row(int r) {
  return static_cast<uint32_t>(((r >> 6) * 8 + (r & 7)) * BLK + ((r & 63) >> 3) * TT);
}

// The same for an fp4 x-role tile (64 bytes per row and step).
constexpr int TT4 = TT / 2;                   // bytes of an fp4 row per step
constexpr int BLK4 = 16 * TT4 + 16;           // 1040: 16 rows of 64 bytes + padding
static_assert(16 * BLK4 <= TILE_BYTES, "an fp4 x-role tile fits the x-role area");
__device__ __forceinline__ uint32_t tile_row4(int r) {
  return static_cast<uint32_t>(((r >> 6) * 4 + (r & 3)) * BLK4 + ((r & 63) >> 2) * TT4);
}

// Byte mask of the E4M3 codes in a dword whose magnitude is >= 128
// (exponent field >= 14): 0xFF in those bytes, 0x00 elsewhere.  Bit 7 of
// each byte of y flags such a code; v_perm_b32 selectors 8-11 broadcast the
// top bit of bytes 1 and 3 of each source, so y supplies bytes 1 and 3 and
// y << 8 bytes 0 and 2.
__device__ __forceinline__ uint32_t big_code_mask(uint32_t x) {
  const uint32_t y = (x & 0x70707070u) + 0x10101010u;
  return __builtin_amdgcn_perm(y << 8, y, 0x090B080Au);
}

// Zeroes the codes of the tokens outside [rlo, rhi) (step-relative) in a g^T
// fragment of 64-token half h: dword i of lane group g holds tokens
// 64h + 16g + 4i .. +3 (i < 4) and 64h + 32 + 16g + 4(i-4) .. +3 (i >= 4).  A
// zero code makes the product zero, so the step then sums the expert's
// tokens only.  Used on the first and last step of an expert whose bounds
// are not multiples of 128.
__device__ __forceinline__ uint32_t keep_bytes(int first, int end) {
  // bytes j of a dword with first <= j < end, for first, end clamped to [0, 4]
  const int a = clampi(first, 0, 4), b = clampi(end, 0, 4);
  const uint32_t below_b = b >= 4 ? 0xFFFFFFFFu : ((1u << (8 * b)) - 1u);
  const uint32_t below_a = a >= 4 ? 0xFFFFFFFFu : ((1u << (8 * a)) - 1u);
  return b > a ? (below_b & ~below_a) : 0u;
}
__device__ __forceinline__ void mask_tokens(v8i &frag, int h, int g, int rlo, int rhi) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = 64 * h + (i < 4 ? 16 * g + 4 * i : 32 + 16 * g + 4 * (i - 4));
    frag[i] = static_cast<int>(static_cast<uint32_t>(frag[i]) & keep_bytes(rlo - t, rhi - t));
  }
}

// One 128-step of the contraction for a wave's 128 x 64 patch: 16
// block-scaled MFMAs (32 in the two-pass form).  The x-role tile (MFMA A
// operand, rows = output rows of the MFMA) and the g-role tile (MFMA B
// operand) sit at ST_X and ST_G of stage st.  Contraction elements outside
// [rlo, rhi) and g-role rows outside [row_lo, row_hi) are zeroed in the
// g-role fragments first (both bounds step- and tile-relative).  The fragments of both 64-token halves are
// read from LDS up front and the MFMAs of the first half are interleaved
// with the reads of the second, so only the first reads' latency is exposed.
template <bool SPLIT, bool XFP4 = false>
__device__ __forceinline__ void compute_step(const uint8_t *st, v16f (&acc)[4][2], const uint32_t (&xrow)[4],
                                             const uint32_t (&grow)[2], const uint32_t (&chunk_off)[2][2],
                                             int wk, int wn, int l32, int g, int rlo, int rhi, int row_lo,
                                             int row_hi) {
  uint32_t sx[4], sg[2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
    sx[a] = *reinterpret_cast<const uint32_t *>(st + ST_SX + 4 * (wk * 128 + a * 32 + l32)) >> (8 * g);
#pragma unroll
  for (int b = 0; b < 2; ++b)
    sg[b] = *reinterpret_cast<const uint32_t *>(st + ST_SG + 4 * (wn * 64 + b * 32 + l32)) >> (8 * g);
  auto frag = [&](uint32_t row, int h) {
    const v4i lo = *reinterpret_cast<const v4i *>(st + row + chunk_off[h][0]);
    const v4i hi = *reinterpret_cast<const v4i *>(st + row + chunk_off[h][1]);
    return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // x-role fragment of half h: E4M3 as above, or the 16 bytes of fp4 codes of
  // this lane's 32-element block (the MFMA reads the low four dwords)
  auto xfrag = [&](uint32_t row, int h) {
    if constexpr (XFP4) {
      const v4i v = *reinterpret_cast<const v4i *>(st + row + (2 * h + g) * 16);
      return (v8i){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    } else {
      return frag(row, h);
    }
  };
  constexpr int XFMT = XFP4 ? 4 : 0;           // MFMA A-operand format: E2M1 or E4M3
  auto mm = [&](int a, int b, const v8i &x, const v8i &gop, int h) {
    if (h == 0)
      acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          x, gop, acc[a][b], XFMT, 0, 0, static_cast<int>(sx[a]), 0, static_cast<int>(sg[b]));
    else
      acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          x, gop, acc[a][b], XFMT, 0, 2, static_cast<int>(sx[a]), 2, static_cast<int>(sg[b]));
  };
  // first half: g fragments and x fragments; second half: g fragments early,
  // each x fragment as soon as the first half's fragment of the same rows is done
  v8i g0[2], g1[2], x[4];
#pragma unroll
  for (int b = 0; b < 2; ++b) g0[b] = frag(grow[b], 0);
#pragma unroll
  for (int a = 0; a < 4; ++a) x[a] = xfrag(xrow[a], 0);
#pragma unroll
  for (int b = 0; b < 2; ++b) g1[b] = frag(grow[b], 1);
  if (rlo > 0 || rhi < TT) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      mask_tokens(g0[b], 0, g, rlo, rhi);
      mask_tokens(g1[b], 1, g, rlo, rhi);
    }
  }
  if (row_lo > 0 || row_hi < TN) {
    // g-role rows outside [row_lo, row_hi) take no part (rows of another expert)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int row = wn * 64 + b * 32 + l32;
      const bool in = row >= row_lo && row < row_hi;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        g0[b][i] = in ? g0[b][i] : 0;
        g1[b][i] = in ? g1[b][i] : 0;
      }
    }
  }
  if constexpr (SPLIT) {
    // two passes: the g^T codes of magnitude >= 128, then the rest, so that no
    // 8-token run of the MFMA mixes a block's largest codes with its small ones.
    // The passes over one accumulator are 8 MFMAs apart (no result-latency stall).
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8i gh[2], gl[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t v = static_cast<uint32_t>(h == 0 ? g0[b][i] : g1[b][i]);
          const uint32_t m = big_code_mask(v);
          gh[b][i] = static_cast<int>(v & m);
          gl[b][i] = static_cast<int>(v & ~m);
        }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        mm(a, 0, x[a], gh[0], h);
        mm(a, 1, x[a], gh[1], h);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        mm(a, 0, x[a], gl[0], h);
        mm(a, 1, x[a], gl[1], h);
        if (h == 0) x[a] = xfrag(xrow[a], 1);
      }
    }
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      mm(a, 0, x[a], g0[0], 0);
      mm(a, 1, x[a], g0[1], 0);
      x[a] = xfrag(xrow[a], 1);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      mm(a, 0, x[a], g1[0], 1);
      mm(a, 1, x[a], g1[1], 1);
    }
    // scales and first-half reads, then MFMAs with the second half's x reads between
    // (an fp4 x fragment is one 16-byte read instead of two)
    __builtin_amdgcn_sched_group_barrier(0x100, XFP4 ? 18 : 22, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, XFP4 ? 1 : 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  }
}

constexpr int STORES_PER_TILE = 16;           // 16-byte stores per lane per output tile

// Epilogue of a 512-thread workgroup's 256 x 256 f32 tile (eight waves as
// 2 (k) x 4 (n) patches of 128 x 64, MFMA output rows k, columns n): bf16
// (round to nearest even) into C[n][k] through a buffer descriptor whose
// byte offset 0 is the tile's element (0, 0) and whose row stride is ld
// elements; stores past the descriptor's size are dropped.  Each wave stages
// its own patch in a private 8 KB region of stg (free: its last step has been
// read), 64 columns at a time as 64 rows of 128 bytes with the 16-byte pieces
// XOR-swizzled by (row mod 8), and reads it back as whole rows, so every
// store instruction writes eight 128-byte row pieces (whole lines;
// partial-line non-temporal stores measured several times slower).  One
// workgroup barrier in all: a wave's LDS writes and reads of its own region
// execute in order.  (Staging the tile in two halves shared by all waves,
// with four barriers, measured 2-3% slower end to end.)
__device__ __forceinline__ void store_tile(const v16f (&acc)[4][2], uint8_t *stg, __amdgpu_buffer_rsrc_t crsrc,
                                           uint32_t ld, int wk, int wn, int tid) {
  // recompute the lane coordinates here rather than keep them live across
  // the step loop (spilled addresses would be reloaded with a vmcnt wait
  // that drains the next step's loads)
  int etid = tid;
  asm volatile("" : "+v"(etid));
  const int lane = etid & 63, el32 = lane & 31, eg = lane >> 5;
  uint8_t *reg = stg + (wk * 4 + wn) * 8192;
  barrier();                                   // all waves are done reading that buffer
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    // columns wk*128 + 64c .. +63: accumulators a = 2c, 2c + 1
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int rl = b * 32 + el32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int a = 2 * c + a2, q = a2 * 4 + j;          // 16-byte piece of the 128-byte row
          const uint32_t lo = pack_bf16x2(acc[a][b][4 * j + 0], acc[a][b][4 * j + 1]);
          const uint32_t hi = pack_bf16x2(acc[a][b][4 * j + 2], acc[a][b][4 * j + 3]);
          typedef uint32_t u2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<u2 *>(reg + rl * 128 + ((q ^ (rl & 7)) << 4) + 8 * eg) = (u2){lo, hi};
        }
      }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int row = p * 8 + (lane >> 3), q = lane & 7;
      const v4u v = *reinterpret_cast<const v4u *>(reg + row * 128 + ((q ^ (row & 7)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(
          v, crsrc,
          static_cast<int>((static_cast<uint32_t>(wn * 64 + row) * ld + wk * 128 + c * 64 + q * 8) * 2u), 0, 2);
    }
    // the next chunk overwrites the region only after these reads (in order)
    asm volatile("" ::: "memory");
  }
  // the next step's barrier (which waits for LDS) precedes any load into stg
}

// +0.0 into the same 256 x 256 bf16 tile, whole 512-byte row segments.
__device__ __forceinline__ void store_zero_tile(__amdgpu_buffer_rsrc_t crsrc, uint32_t ld, int tid) {
  int etid = tid;
  asm volatile("" : "+v"(etid));
  const v4u z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int p = 0; p < STORES_PER_TILE; ++p) {
    const uint32_t row = static_cast<uint32_t>(p * 16 + (etid >> 5));
    __builtin_amdgcn_raw_buffer_store_b128(z, crsrc, static_cast<int>((row * ld + (etid & 31) * 8) * 2u), 0, 2);
  }
}

}  // namespace mxgemm
}  // namespace moe_gg
