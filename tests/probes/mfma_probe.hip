// Single-instruction probes of gfx950's block-scaled fp8 MFMAs, and of the
// bf16 MFMA the exact GEMM entry points run on.
//
// Each case is one wave: 64 lanes x 8 dwords of A operand, 64 x 8 of B,
// one scale dword per lane for A and for B.  The wave runs
// v_mfma_scale_f32_16x16x128_f8f6f4 and v_mfma_scale_f32_32x32x64_f8f6f4
// (fp8 E4M3 A and B) once for each op_sel value 0..3 (the same value for the
// A and the B scale) and writes the raw accumulator registers out.  The test
// that drives it derives the operand, scale and result lane layouts from
// one-hot and small-integer inputs.  bf16_probe_run does the same for
// v_mfma_f32_32x32x16_bf16 (64 lanes x 4 dwords of A and of B, zero C), so a
// test can check how it adds its products.  Test infrastructure only.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int S>
__device__ inline void run_one(v8i a, v8i b, int sa, int sb, float* o16, float* o32) {
  v4f c = {0.f, 0.f, 0.f, 0.f};
  c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, S, sa, S, sb);
  v16f d = {};
  d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, d, 0, 0, S, sa, S, sb);
  for (int i = 0; i < 4; ++i) o16[i] = c[i];
  for (int i = 0; i < 16; ++i) o32[i] = d[i];
}

__global__ __launch_bounds__(64) void probe_kernel(const int* __restrict__ A, const int* __restrict__ B,
                                                   const int* __restrict__ SA, const int* __restrict__ SB,
                                                   float* __restrict__ out16, float* __restrict__ out32) {
  const int cs = blockIdx.x, l = threadIdx.x;
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = A[(cs * 64 + l) * 8 + i];
    b[i] = B[(cs * 64 + l) * 8 + i];
  }
  const int sa = SA[cs * 64 + l], sb = SB[cs * 64 + l];
  float* o16 = out16 + (size_t)cs * 4 * 64 * 4 + l * 4;
  float* o32 = out32 + (size_t)cs * 4 * 64 * 16 + l * 16;
  run_one<0>(a, b, sa, sb, o16 + 0 * 256, o32 + 0 * 1024);
  run_one<1>(a, b, sa, sb, o16 + 1 * 256, o32 + 1 * 1024);
  run_one<2>(a, b, sa, sb, o16 + 2 * 256, o32 + 2 * 1024);
  run_one<3>(a, b, sa, sb, o16 + 3 * 256, o32 + 3 * 1024);
}

// out16: [ncases][4 opsel][64 lanes][4]; out32: [ncases][4 opsel][64 lanes][16]
extern "C" __attribute__((visibility("default"))) int mfma_probe_run(
    const int* A, const int* B, const int* SA, const int* SB, float* out16, float* out32,
    int ncases, hipStream_t stream) {
  if (!A || !B || !SA || !SB || !out16 || !out32 || ncases <= 0) return -1;
  hipLaunchKernelGGL(probe_kernel, dim3(ncases), dim3(64), 0, stream, A, B, SA, SB, out16, out32);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

__global__ __launch_bounds__(64) void bf16_probe_kernel(const int* __restrict__ A, const int* __restrict__ B,
                                                        float* __restrict__ out) {
  const int cs = blockIdx.x, l = threadIdx.x;
  v4i a, b;
  for (int i = 0; i < 4; ++i) {
    a[i] = A[(cs * 64 + l) * 4 + i];
    b[i] = B[(cs * 64 + l) * 4 + i];
  }
  v16f d = {};
  d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), d, 0, 0, 0);
  for (int i = 0; i < 16; ++i) out[((size_t)cs * 64 + l) * 16 + i] = d[i];
}

// A, B: [ncases][64 lanes][8] bf16 bit patterns (as 4 dwords); out: [ncases][64][16]
extern "C" __attribute__((visibility("default"))) int bf16_probe_run(const int* A, const int* B, float* out,
                                                                     int ncases, hipStream_t stream) {
  if (!A || !B || !out || ncases <= 0) return -1;
  hipLaunchKernelGGL(bf16_probe_kernel, dim3(ncases), dim3(64), 0, stream, A, B, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
