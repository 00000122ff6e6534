// Internal declarations shared by the HIP translation units of libwq.
// Not part of the public ABI (that is include/wq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "wq.h"

namespace wq {

// ---------------------------------------------------------------- vectors
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef unsigned int uint4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------- 16-bit <-> fp32 helpers
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// An fp32 value held in a register as is.  Narrowing a product to 16 bits
// right after it lets the compiler fuse both into one mixed-precision
// multiply (v_fma_mixlo_f16) that rounds the exact product once; where the
// definition is "the fp32 product, then a 16-bit rounding" and the product
// is not exact in fp32, pass it through here first.  The empty asm emits
// nothing.
__device__ __forceinline__ float as_f32(float v) {
  asm("" : "+v"(v));
  return v;
}
// fp32 -> fp16, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  _Float16 h = (_Float16)v;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}
// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
template <int DT>
__device__ __forceinline__ float load16(const uint16_t* p) {
  return DT == WQ_BF16 ? bf16_bits_to_f32(*p) : f16_bits_to_f32(*p);
}

// ------------------------------------------- direct loads and waits
typedef __attribute__((address_space(3))) void lds_void_t;

// One direct global->LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds + 16*l (lds is wave-uniform, passed in M0).
// Issued from inline asm on purpose: the compiler's wait-count bookkeeping
// treats these loads as completing out of order with ordinary loads and then
// falls back to waiting for every outstanding load.  Hidden from it, its
// automatic waits for ordinary loads count only ordinary loads, which can
// only make them stricter (each direct load it does not see is one more
// outstanding load that must finish first); the kernels wait for their
// direct loads themselves (vm_wait with counts that include them) before any
// LDS read of the data.  No output register, so nothing is left in flight
// behind the compiler's back but LDS bytes the explicit waits cover.  The
// s_nop is the one wait state an LDS-DMA instruction needs after a scalar
// write of M0, which the compiler pads for its own such loads but cannot
// see here.
__device__ __forceinline__ void lds_dma16(const void* gaddr, lds_void_t* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "{m0}"(l) : "memory");
}

// The same with the non-temporal cache policy: for streamed data that no
// other load of the kernel reads again (the decode kernels' codes at M = 1).
__device__ __forceinline__ void lds_dma16_nt(const void* gaddr, lds_void_t* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gaddr), "{m0}"(l) : "memory");
}

// The 4-byte form (global_load_lds_dword): lane l's 4 bytes land at
// lds + 4*l, 256 bytes per wave.
__device__ __forceinline__ void lds_dma4(const void* gaddr, lds_void_t* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gaddr), "{m0}"(l) : "memory");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima, i.e. no wait).
template <int N>
__device__ __forceinline__ void vm_wait() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maxima): this wave's
// LDS writes are done
__device__ __forceinline__ void lgkm_wait0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would make every wave wait for all of its outstanding global loads (the
// direct-to-LDS loads are counted with them), which serializes the weight
// stream behind the first phase.  Callers wait for exactly the loads that
// must have landed (vm_wait) before calling it; the empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; shapes were validated by the
// ABI layer.
hipError_t launch_quant_int4(const void* w, int wdt, int64_t n, int64_t k, int group,
                             uint32_t* codes, uint16_t* scales, uint8_t* zeros,
                             hipStream_t s);
hipError_t launch_quant_int8_rows(const void* w, int wdt, int64_t n, int64_t k,
                                  int8_t* codes, float* scales, hipStream_t s);
hipError_t launch_pack_nf4(const void* w, int wdt, int64_t numel, int double_quant,
                           const float* thresholds15, uint8_t* codes, void* absmax,
                           float* absmax_scale, hipStream_t s, bool fp4 = false);

struct W4Plan {
  int path;      // 1 = gemm (m > 16), 3 = streaming decode (m <= 16)
  int tpg;       // decode: row tiles of 16 per workgroup
  int gpw;       // decode: groups of 128 per wave and phase
  int mp;        // decode: activation rows staged in LDS: 1, 4 or 16
  int cfg;       // decode configuration id (see plan_w4a16)
  int phases;    // decode: phases over K
  int grid;      // decode: workgroups
  bool szl;      // decode: scales and zero points staged in LDS
};
W4Plan plan_w4a16(int64_t m, const wq_weight* w);
hipError_t launch_w4a16(const void* x, int xdt, int64_t m, const wq_weight* w,
                        const float* levels16, void* y, int ydt, const W4Plan& plan,
                        hipStream_t s);
// gate/up pair sharing x (same format, n and k; FP4 weights come as the NF4
// kernel view with levels16 the FP4 table); act 1: yg = silu(gate) * up
W4Plan plan_w4a16_pair(int64_t m, const wq_weight* wg, const wq_weight* wu);
hipError_t launch_w4a16_pair(const void* x, int xdt, int64_t m, const wq_weight* wg,
                             const wq_weight* wu, const float* levels16, int act, void* yg,
                             void* yu, int ydt, const W4Plan& plan, hipStream_t s);

hipError_t launch_int8_prepare(const uint16_t* x, int64_t m, int64_t k, float thr,
                               uint8_t* mask, int32_t* idx, int32_t* count, int8_t* qx,
                               float* sx, hipStream_t s);
hipError_t launch_int8_gemm(const uint16_t* x, int64_t m, const wq_weight* w,
                            const int8_t* qx, const float* sx, const int32_t* idx,
                            const int32_t* count, void* y, int ydt, int32_t* acc_out,
                            hipStream_t s);

// dst[r][j] = src[r][perm[j]] for a 16-bit [rows][k] matrix (k % 8 == 0)
hipError_t launch_permute_cols(const uint16_t* src, int64_t rows, int64_t k,
                               const int32_t* perm, uint16_t* dst, hipStream_t s);

// dst[r][c] = round16(src[r][c] * scale[c]) (in place allowed; k % 8 == 0)
hipError_t launch_scale_cols(const uint16_t* src, int dt, int64_t rows, int64_t k,
                             const float* scale, uint16_t* dst, hipStream_t s);

hipError_t launch_dequantize(const wq_weight* w, const float* levels16, void* out, int odt,
                             hipStream_t s);

// Host-side NF4 codebook (levels) and decision midpoints (thresholds).
const float* nf4_levels();
const float* nf4_thresholds();
// FP4 (E2M1): 16 levels indexed by code, and the 7 magnitude midpoints
// (padded to 15 with zeros)
const float* fp4_levels();
const float* fp4_thresholds();

}  // namespace wq
