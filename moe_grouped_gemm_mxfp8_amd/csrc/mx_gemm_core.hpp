// Shared core of the block-scaled MXFP8 GEMM kernels on gfx950: the LDS
// stage layout, the step of 128 contraction elements for one wave's
// 128 x 64 patch (block-scaled fp8 MFMA, or exact on the bf16 MFMA) and the
// epilogues.
//
// A stage holds two operand tiles of 256 rows x 128 contraction bytes (E4M3)
// and their scale dwords: the A-operand tile (whose rows become the MFMA output
// rows) and the B-operand tile (whose rows become the output columns).  An operand tile
// in LDS is 32 blocks of 8 rows x 128 bytes, each block padded by 16 bytes;
// one stage-load instruction fills a block, eight lanes per row reading the
// row's 128 bytes in order, and the padding puts the 16 rows an MFMA operand
// read touches at once on 16 distinct bank groups.
//
// The A-operand tile may instead hold E2M1 (fp4) codes, two per byte (MFMA
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

constexpr int TA = 256;             // rows of the A-operand tile
constexpr int TB = 256;             // rows of the B-operand tile
constexpr int TT = 128;             // contraction elements per pipeline step
// Row r of a 64-row group G = r/64 sits in block 8G + r%8 at slot (r%64)/8.
constexpr int BLK = 8 * TT + 16;              // 1040: 8 rows of 128 bytes + padding
constexpr int TILE_BYTES = 32 * BLK;          // 33280: a 256-row operand tile
constexpr int ST_A = 0;                       // A-operand tile
constexpr int ST_B = ST_A + TILE_BYTES;       // B-operand tile
constexpr int ST_SA = ST_B + TILE_BYTES;      // A-operand scale dwords [256]
constexpr int ST_SB = ST_SA + TA * 4;         // B-operand scale dwords [256]
constexpr int STAGE_BYTES = ST_SB + TB * 4;   // 68608
static_assert(8 * 8192 <= STAGE_BYTES, "the epilogue stages eight 8 KB wave regions in one buffer");

// LDS byte offset of row r (0..255) inside an operand tile.
__device__ __forceinline__ uint32_t tile_row(int r) {
  return static_cast<uint32_t>(((r >> 6) * 8 + (r & 7)) * BLK + ((r & 63) >> 3) * TT);
}

// The same for an fp4 A-operand tile (64 bytes per row and step).
constexpr int TT4 = TT / 2;                   // bytes of an fp4 row per step
constexpr int BLK4 = 16 * TT4 + 16;           // 1040: 16 rows of 64 bytes + padding
static_assert(16 * BLK4 <= TILE_BYTES, "an fp4 A-operand tile fits the A-operand area");
__device__ __forceinline__ uint32_t tile_row4(int r) {
  return static_cast<uint32_t>(((r >> 6) * 4 + (r & 3)) * BLK4 + ((r & 63) >> 2) * TT4);
}

// Byte mask of a dword of codes keeping bytes j with first <= j < end (the
// elements of an expert, relative to the dword's first element).
__device__ __forceinline__ uint32_t keep_bytes(int first, int end) {
  // bytes j of a dword with first <= j < end, for first, end clamped to [0, 4]
  const int a = clampi(first, 0, 4), b = clampi(end, 0, 4);
  const uint32_t below_b = b >= 4 ? 0xFFFFFFFFu : ((1u << (8 * b)) - 1u);
  const uint32_t below_a = a >= 4 ? 0xFFFFFFFFu : ((1u << (8 * a)) - 1u);
  return b > a ? (below_b & ~below_a) : 0u;
}

// One 128-step of the contraction for a wave's 128 x 64 patch: 16
// block-scaled MFMAs.  The A-operand tile (rows =
// output rows of the MFMA) and the B-operand tile (rows = output columns) sit
// at ST_A and ST_B of stage st (elements outside an expert already zeroed
// by mask_stage_elements).  The fragments of
// both 64-element halves are read from LDS up front and the MFMAs of the
// first half are interleaved with the reads of the second, so only the first
// reads' latency is exposed.
template <bool XFP4 = false>
__device__ __forceinline__ void compute_step(const uint8_t *st, v16f (&acc)[4][2], const uint32_t (&xrow)[4],
                                             const uint32_t (&grow)[2], const uint32_t (&chunk_off)[2][2],
                                             int wk, int wn, int l32, int g) {
  uint32_t sx[4], sg[2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
    sx[a] = *reinterpret_cast<const uint32_t *>(st + ST_SA + 4 * (wk * 128 + a * 32 + l32)) >> (8 * g);
#pragma unroll
  for (int b = 0; b < 2; ++b)
    sg[b] = *reinterpret_cast<const uint32_t *>(st + ST_SB + 4 * (wn * 64 + b * 32 + l32)) >> (8 * g);
  auto frag = [&](uint32_t row, int h) {
    const v4i lo = *reinterpret_cast<const v4i *>(st + row + chunk_off[h][0]);
    const v4i hi = *reinterpret_cast<const v4i *>(st + row + chunk_off[h][1]);
    return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // A-operand fragment of half h: E4M3 as above, or the 16 bytes of fp4 codes of
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

// The exact form of a 128-element step.  The scaled fp8 MFMA truncates the
// products of every run of 8 contraction elements to 2^(largest exponent sum
// of the run - 13) (measured; the products of one run are not added exactly),
// so where an outlier of one operand meets an outlier of the other at the
// same token, the run's other products are lost.  The bf16 MFMA adds its 16
// products to within 2^-22 of the largest (measured: 2^20 + 15 ones come out
// exact, and products spanning 2^14 give the exact sum rounded once), the
// error of an f32 accumulation.  An E4M3 code times its E8M0
// scale is exactly a bf16 (3 mantissa bits of 7, the scale inside bf16's
// exponent range), so this step converts the fragments with
// v_cvt_scalef32_pk_bf16_fp8 (two codes per instruction, the block's scale
// 2^(s - 127) as the f32 multiplier) and multiplies them on
// v_mfma_f32_32x32x16_bf16: 8 chunks of 16 elements, lane l holding row l%32
// and 8 elements of the chunk (lane group l/32 the other 8).  The
// accumulators have the fp8 MFMA's 32 x 32 layout, so the epilogues serve both.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// f32 bits of the E8M0 scale byte j of a row's scale dword: 2^(s - 127); byte 0
// (2^-127) is the f32 denormal 0x00400000.
__device__ __forceinline__ float e8m0_f32(uint32_t dw, int j) {
  const uint32_t s = (dw >> (8 * j)) & 0xFFu;
  return __builtin_bit_cast(float, max(s << 23, 0x00400000u));
}
__device__ __forceinline__ bf16x8 cvt8(uint32_t w0, uint32_t w1, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
  return (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
// The same for eight E2M1 codes (one dword, element 2i in the low nibble of
// byte i): an E2M1 value times its E8M0 scale is exactly a bf16 as well.
__device__ __forceinline__ bf16x8 cvt8_fp4(uint32_t w, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Zeroes the codes of the step's contraction elements outside [rlo, rhi)
// (step-relative) in the B-operand tile of a stage, in LDS: thread t of the
// 512 rewrites bytes 64(t%2) .. +63 of row t/2.  A zero code makes the product
// zero, so the step then sums the expert's tokens only (the weight gradient's
// first and last step of an expert whose bounds are not multiples of 128).
// The caller separates it from the stage's readers by barriers.
__device__ __forceinline__ void mask_stage_elements(uint8_t *st, int tid, int rlo, int rhi) {
  const int row = tid >> 1, h = tid & 1;
  uint8_t *p = st + ST_B + tile_row(row) + 64 * h;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v4u v = *reinterpret_cast<const v4u *>(p + 16 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 64 * h + 16 * c + 4 * i;      // step-relative element of byte 0 of dword i
      v[i] &= keep_bytes(rlo - t, rhi - t);
    }
    *reinterpret_cast<v4u *>(p + 16 * c) = v;
  }
}

// One 128-element step of a wave's 128 x 64 patch in the exact form (64
// bf16 MFMAs).  Elements are taken 32 at a time (one scale block j): lane
// group g reads the 16 bytes of elements 32j + 16g .. +15 of its row with one
// 16-byte LDS read (8-byte reads measured at half the LDS throughput) and
// feeds bytes 0-7 to chunk 2j and bytes 8-15 to chunk 2j + 1, the same
// mapping for both operands, so every chunk's products pair the same tokens.
// The step masks no element (mask_stage_elements zeroes them in the stage
// beforehand): a run-time mask test inside the block loop split it into basic
// blocks, at whose edges every read of the next block waited for its data
// before the current block's MFMAs (measured in the generated code).  The
// next block's bytes are read while the current block's MFMAs run; a
// scheduling fence per block keeps later blocks' reads from being hoisted
// (their registers would spill).  An fp4 A-operand tile (XFP4) holds the
// same 16 elements of a lane in 8 bytes (dword 0 for chunk 2j, dword 1 for
// chunk 2j + 1).
//
// NB = 2: the wave's B-operand rows are wn*64 .. +63 (grow[0..1]); NB = 1:
// only wn*32 .. +31 (grow[0]; accumulators acc[a][0]), the layout of a tile
// whose B-operand rows past 128 are all empty.
template <bool XFP4 = false, int NB = 2>
__device__ __forceinline__ void compute_step_bf16(const uint8_t *st, v16f (&acc)[4][2], const uint32_t (&xrow)[4],
                                                  const uint32_t (&grow)[2], int wk, int wn, int l32, int g) {
  uint32_t sx[4], sg[NB];
#pragma unroll
  for (int a = 0; a < 4; ++a) sx[a] = *reinterpret_cast<const uint32_t *>(st + ST_SA + 4 * (wk * 128 + a * 32 + l32));
#pragma unroll
  for (int b = 0; b < NB; ++b)
    sg[b] = *reinterpret_cast<const uint32_t *>(st + ST_SB + 4 * (wn * 32 * NB + b * 32 + l32));
  auto read = [&](int j, v4u (&xr)[4], v4u (&gr)[NB]) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if constexpr (XFP4) {
        const v2u w = *reinterpret_cast<const v2u *>(st + xrow[a] + 16 * j + 8 * g);
        xr[a] = (v4u){w[0], w[1], 0u, 0u};
      } else {
        xr[a] = *reinterpret_cast<const v4u *>(st + xrow[a] + 32 * j + 16 * g);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) gr[b] = *reinterpret_cast<const v4u *>(st + grow[b] + 32 * j + 16 * g);
  };
  v4u xr[4], gr[NB];
  read(0, xr, gr);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v4u xn[4], gn[NB];
    if (j < 3) read(j + 1, xn, gn);
    float fx[4], fg[NB];
#pragma unroll
    for (int a = 0; a < 4; ++a) fx[a] = e8m0_f32(sx[a], j);
#pragma unroll
    for (int b = 0; b < NB; ++b) fg[b] = e8m0_f32(sg[b], j);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      bf16x8 xa[4], gb[NB];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        xa[a] = XFP4 ? cvt8_fp4(xr[a][q], fx[a]) : cvt8(xr[a][2 * q], xr[a][2 * q + 1], fx[a]);
#pragma unroll
      for (int b = 0; b < NB; ++b) gb[b] = cvt8(gr[b][2 * q], gr[b][2 * q + 1], fg[b]);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[a], gb[b], acc[a][b], 0, 0, 0);
    }
    if (j < 3) {
#pragma unroll
      for (int a = 0; a < 4; ++a) xr[a] = xn[a];
#pragma unroll
      for (int b = 0; b < NB; ++b) gr[b] = gn[b];
    }
    // keep the scheduler from hoisting later blocks' reads (register pressure)
    __builtin_amdgcn_sched_barrier(0);
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
// NB = 1: the half layout of compute_step_bf16 (the wave's output rows
// wn*32 .. +31, accumulators acc[a][0]; eight stores per lane).
template <int NB = 2>
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
      for (int b = 0; b < NB; ++b) {
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
    // all eight row pieces first, then the stores: one LDS round trip per
    // chunk instead of one per store
    constexpr int NP = 4 * NB;                 // eight rows per piece, 32 NB rows
    v4u v[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = p * 8 + (lane >> 3), q = lane & 7;
      v[p] = *reinterpret_cast<const v4u *>(reg + row * 128 + ((q ^ (row & 7)) << 4));
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = p * 8 + (lane >> 3), q = lane & 7;
      __builtin_amdgcn_raw_buffer_store_b128(
          v[p], crsrc,
          static_cast<int>((static_cast<uint32_t>(wn * 32 * NB + row) * ld + wk * 128 + c * 64 + q * 8) * 2u), 0, 2);
    }
    // the next chunk overwrites the region only after these reads (in order)
    asm volatile("" ::: "memory");
  }
  // the next step's barrier (which waits for LDS) precedes any load into stg
}

// Epilogue of the same tile written as the MFMA produces it: C[row][column]
// with rows = A-operand rows (wave (wk, wn): rows wk*128 .. +127, accumulator
// a = rows 32a ..) and columns = B-operand rows (wn*64 .. +63, accumulator b).
// In the 32 x 32 result layout lane l holds column l%32 and, in register j,
// row 8(j/4) + 4(l/32) + j%4, so lanes 0..31 of one register hold 32
// consecutive columns of one row.  Each wave converts to bf16 (round to
// nearest even, two rows per pack) and stages its patch in its private 8 KB
// LDS region, 64 rows at a time as 64 rows of 128 bytes (its 64 columns), the
// 16-byte pieces XOR-swizzled by (row mod 8), then reads whole rows back so
// that every store instruction writes eight 128-byte row pieces.
__device__ __forceinline__ void store_tile_rows(const v16f (&acc)[4][2], uint8_t *stg, __amdgpu_buffer_rsrc_t crsrc,
                                                uint32_t ld, int wk, int wn, int tid) {
  int etid = tid;
  asm volatile("" : "+v"(etid));
  const int lane = etid & 63, el32 = lane & 31, eg = lane >> 5;
  uint8_t *reg = stg + (wk * 4 + wn) * 8192;
  barrier();                                   // all waves are done reading that buffer
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    // rows 64c .. 64c+63 of the wave's patch: accumulators a = 2c, 2c + 1
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int col = b * 32 + el32;                        // 0..63: byte 2*col of the staged row
        const uint32_t cpos = static_cast<uint32_t>(col * 2);
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          // registers j and j+1 are rows r and r+1 of the same column
          const int r = a2 * 32 + 8 * (j >> 2) + 4 * eg + (j & 3);
          const uint32_t pk = pack_bf16x2(acc[2 * c + a2][b][j], acc[2 * c + a2][b][j + 1]);
          const uint32_t o0 = static_cast<uint32_t>(r * 128) + ((((cpos >> 4) ^ r) & 7) << 4) + (cpos & 15);
          const uint32_t o1 = static_cast<uint32_t>((r + 1) * 128) + ((((cpos >> 4) ^ (r + 1)) & 7) << 4) + (cpos & 15);
          *reinterpret_cast<uint16_t *>(reg + o0) = static_cast<uint16_t>(pk);
          *reinterpret_cast<uint16_t *>(reg + o1) = static_cast<uint16_t>(pk >> 16);
        }
      }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int row = p * 8 + (lane >> 3), q = lane & 7;
      const v4u v = *reinterpret_cast<const v4u *>(reg + row * 128 + ((q ^ (row & 7)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(
          v, crsrc,
          static_cast<int>((static_cast<uint32_t>(wk * 128 + 64 * c + row) * ld + wn * 64 + q * 8) * 2u), 0, 2);
    }
    // the next chunk overwrites the region only after these reads (in order)
    asm volatile("" ::: "memory");
  }
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
