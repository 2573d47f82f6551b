// Device helpers shared by the gfx950 kernels of the MoE grouped-GEMM backward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_gg {

// Host: with MOE_GG_VALIDATE=1, copy the offsets to the host (synchronising
// the stream) and return MOE_GG_EINVAL unless off[0] = 0, off[e] <= off[e+1]
// and off[E] = M; otherwise MOE_GG_OK without touching them (status.cpp).
int check_offsets_if_asked(const int32_t *off, int E, int M, hipStream_t stream);

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Buffer resource descriptor of a raw (stride 0) byte buffer.  Loads at byte
// offsets >= num_bytes return zeros instead of touching memory.
__device__ __forceinline__ v4i make_srd(const void *base, uint32_t num_bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = static_cast<int>(static_cast<uint32_t>(b));
  r[1] = static_cast<int>(static_cast<uint32_t>(b >> 32) & 0xFFFFu);
  r[2] = static_cast<int>(num_bytes);
  r[3] = 0x00020000;  // 32-bit data format, no swizzle, no add-tid
  r[0] = __builtin_amdgcn_readfirstlane(r[0]);
  r[1] = __builtin_amdgcn_readfirstlane(r[1]);
  r[2] = __builtin_amdgcn_readfirstlane(r[2]);
  r[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return r;
}

// Global -> LDS without a trip through VGPRs: lane i's 16 (or 4) bytes at
// srd.base + voff + soff land at LDS byte lds_base + 16*i (or 4*i).  Issued as
// inline asm so that the compiler's conservative LDS-DMA alias waits do not
// serialise the double buffer; completion is tracked with vmcnt by the caller.
// The LDS address comes from m0, a register the compiler reserves for itself:
// the statement saves m0, sets it, waits the one wait state an m0 write needs
// before an LDS-DMA load reads it, issues the load and puts m0 back, so no
// value the compiler keeps in m0 is disturbed.
__device__ __forceinline__ void dma_b128(v4i srd, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(srd), "s"(soff), "s"(lds_base) : "memory");
}
__device__ __forceinline__ void dma_b32(v4i srd, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(srd), "s"(soff), "s"(lds_base) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Workgroup barrier that also orders this wave's LDS traffic: its LDS reads
// and writes have completed before any wave passes.  (A fence-based
// __syncthreads would also wait for every outstanding global load, which
// would drain the in-flight next pipeline stage.)
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Expert of token row r: the number of e in [1, E-1] with off[e] <= r.  For a
// nondecreasing offset array this is the e with off[e] <= r < off[e+1] (empty
// experts skipped); for any array it lies in [0, E-1].
__device__ __forceinline__ int expert_of_row(const int32_t *__restrict__ off, int E, int r) {
  int lo = 1, hi = E;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= r) lo = mid + 1; else hi = mid;
  }
  return lo - 1;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Two f32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

}  // namespace moe_gg
