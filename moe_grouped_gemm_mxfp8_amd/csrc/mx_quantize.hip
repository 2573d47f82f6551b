// MX quantiser on gfx950: f32 -> E4M3 codes with one E8M0 scale per 32
// consecutive elements along the contiguous axis.
//
// Scale rule: 2^(floor(log2(block max)) - 8), so the block max lands in
// [256, 512) (the 8192^3 workload's statement), the byte clamped to [1, 254]
// and 1 for an all-zero block (the decode page's mx8_scale clamps its byte
// to that range); elements are divided by the scale and rounded to nearest
// E4M3, ties to even, saturating at +-448 (the decode page's mx8_q clamps to
// +-FP8_MAX before its conversion), sign of zero kept.
//
// The rounding is done on the integer fields of the f32 input: the division
// by a power of two only moves the exponent, so the E4M3 code follows from
// the 24-bit significand shifted to the target quantum with a round-to-
// nearest-even on the dropped bits.  That is exact for every finite input,
// including f32 subnormals and scaled values below E4M3's subnormal range,
// and independent of the hardware's denormal mode.
//
// HBM-bound streaming kernel: rows never split a block (L % 32 == 0), so the
// [R][L] input is a flat sequence of blocks.  A wave handles 512 elements per
// step as two coalesced 1 KB float4 sweeps; the 8 lanes that share a block
// reduce its max with xor shuffles; each lane writes its 4 codes as one dword
// and the first lane of each block the scale byte.
#include "common.hpp"
#include "../../include/moe_gg.h"

namespace moe_gg {
namespace {

__device__ __forceinline__ int floor_log2_bits(uint32_t a /* |x| bits, nonzero */) {
  const int fe = static_cast<int>(a >> 23);
  if (fe != 0) return fe - 127;
  return (31 - __clz(a)) - 149;          // f32 subnormal: value = a * 2^-149
}

__device__ __forceinline__ uint32_t scale_byte(uint32_t amax_bits) {
  if (amax_bits == 0) return 1u;
  const int s = floor_log2_bits(amax_bits) - 8 + 127;
  return static_cast<uint32_t>(s < 1 ? 1 : (s > 254 ? 254 : s));
}

// E4M3 code of x * 2^(127 - sb), round to nearest even, saturating.
__device__ __forceinline__ uint32_t e4m3_code(float x, int sb) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7FFFFFFFu;
  if (a == 0) return sign;
  uint32_t sig;
  int ex;                                 // |x| = sig * 2^ex
  if ((a >> 23) != 0) { sig = (a & 0x7FFFFFu) | 0x800000u; ex = static_cast<int>(a >> 23) - 150; }
  else { sig = a; ex = -149; }
  const int t = ex + 127 - sb;            // scaled value = sig * 2^t
  const int p = (31 - __clz(sig)) + t;    // floor(log2(scaled value))
  int q = p - 3;                          // quantum exponent: 3 mantissa bits ...
  if (q < -9) q = -9;                     // ... down to the subnormal step 2^-9
  const int sh = q - t;                   // >= 0 for every finite input and sb >= 1
  uint32_t n;
  if (sh >= 25) {
    n = 0;                                // below half the quantum
  } else if (sh == 0) {
    n = sig;
  } else {
    n = sig >> sh;
    const uint32_t rem = sig & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (n & 1u))) ++n;
  }
  if (n == 0) return sign;
  if (n >= 16) { n >>= 1; ++q; }          // rounding carried into the next binade
  if (n < 8) return sign | n;             // subnormal (q == -9)
  const int e = q + 10;                   // value = (n/8) 2^(q+3) = (1 + m/8) 2^(e-7)
  const uint32_t m = n - 8;
  if (e > 15 || (e == 15 && m == 7)) return sign | 0x7Eu;   // saturate to 448
  return sign | (static_cast<uint32_t>(e) << 3) | m;
}

__global__ __launch_bounds__(256) void mx_quantize_kernel(const float *__restrict__ X, uint8_t *__restrict__ Q,
                                                          uint8_t *__restrict__ S, int64_t total) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_global = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  for (int64_t base = wave_global * 512; base < total; base += nwaves * 512) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t i0 = base + half * 256 + 4 * lane;   // this lane's 4 elements
      const bool live = i0 < total;                       // whole 32-blocks are live or not
      v4f v = live ? __builtin_nontemporal_load(reinterpret_cast<const v4f *>(X + i0)) : (v4f){0.f, 0.f, 0.f, 0.f};
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
      m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 1)));
      m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 2)));
      m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 4)));
      const uint32_t sb = scale_byte(m);
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) word |= e4m3_code(v[i], static_cast<int>(sb)) << (8 * i);
      if (live) {
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(Q + i0));
        if ((lane & 7) == 0) S[i0 >> 5] = static_cast<uint8_t>(sb);
      }
    }
  }
}

}  // namespace
}  // namespace moe_gg

extern "C" MOE_GG_API int moe_gg_mx_quantize(const float *X, uint8_t *Q, uint8_t *S, int R, int L,
                                             hipStream_t stream) {
  using namespace moe_gg;
  if (!X || !Q || !S || R <= 0 || L < 32 || L % 32) return MOE_GG_EINVAL;
  const int64_t total = static_cast<int64_t>(R) * L;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_GG_ELAUNCH;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_GG_ELAUNCH;
  const int64_t waves_needed = (total + 511) / 512;
  int64_t blocks = (waves_needed + 3) / 4;
  const int64_t cap = static_cast<int64_t>(cus) * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, X, Q, S, total);
  return hipGetLastError() == hipSuccess ? MOE_GG_OK : MOE_GG_ELAUNCH;
}
