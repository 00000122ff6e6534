// NF4 blockwise encoder with optional double quantization.
//
// NF4 ("LLM quantization selection: five mainstream schemes compared",
// sections 6.1-6.3): each block of 64 consecutive weights is scaled by its
// absolute maximum and every weight is replaced by the nearest of 16 levels
// placed at normal quantiles.  Double quantization (section 6.2 there)
// quantizes the absmax values again: here to int8 per block of 256 absmax
// values with one fp32 second-level scale (max/127).
//
// FP4 (same section 6.3 there; the E2M1 layout in "Inference & deployment
// 05: quantized deployment compared", section 7.2) shares everything but the
// codes: the sign of w/a goes to bit 3 and the magnitude code (bits 0-2, the
// E2M1 exponent and mantissa) counts the 7 magnitude midpoints |w/a|
// exceeds; an all-zero block gives code 0.
//
// One workgroup encodes one superblock of 256 blocks (16384 weights), so the
// second-level scale needs no second pass: the 256 absmax values stay in LDS.
// Eight lanes cover one 64-weight block (8 weights each, one 16-byte load,
// one 4-byte store of 8 packed codes).
#include "internal.h"

namespace wq {
namespace {

struct Thresholds {
  float t[15];
};

template <int DT, bool FP4>
__global__ __launch_bounds__(256) void pack_nf4_kernel(
    const uint16_t* __restrict__ w, int64_t nblocks, int double_quant, Thresholds th,
    uint32_t* __restrict__ codes, void* __restrict__ absmax, float* __restrict__ absmax_scale) {
  __shared__ float amax_s[256];
  const int64_t sb = blockIdx.x;
  const int64_t b0 = sb * 256;
  const int nb = (int)min<int64_t>(256, nblocks - b0);
  const int lane8 = threadIdx.x & 7;
  for (int it = 0; it < 8; ++it) {
    const int lb = it * 32 + (threadIdx.x >> 3);   // local block index
    const bool valid = lb < nb;
    const int64_t e0 = (b0 + lb) * 64 + lane8 * 8; // first element of this lane
    float v[8];
    if (valid) {
      uint4_t raw = *reinterpret_cast<const uint4_t*>(w + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t u = raw[i];
        v[2 * i] = DT == WQ_BF16 ? bf16_bits_to_f32(u & 0xFFFFu) : f16_bits_to_f32(u & 0xFFFFu);
        v[2 * i + 1] = DT == WQ_BF16 ? bf16_bits_to_f32(u >> 16) : f16_bits_to_f32(u >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t c = FP4 ? 0 : 7;
      if (a != 0.0f) {
        const float nv = __fdiv_rn(v[i], a);
        c = 0;
        if constexpr (FP4) {
          const float mag = fabsf(nv);
#pragma unroll
          for (int t = 0; t < 7; ++t) c += mag > th.t[t] ? 1u : 0u;
          c |= nv < 0.0f ? 8u : 0u;
        } else {
#pragma unroll
          for (int t = 0; t < 15; ++t) c += nv > th.t[t] ? 1u : 0u;
        }
      }
      word |= c << (4 * i);
    }
    if (valid) {
      codes[e0 / 8] = word;
      if (lane8 == 0) amax_s[lb] = a;
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (!double_quant) {
    if (t < nb) static_cast<float*>(absmax)[b0 + t] = amax_s[t];
    return;
  }
  __shared__ float red[4];
  float m = t < nb ? amax_s[t] : 0.0f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float c2 = __fdiv_rn(m, 127.0f);
  if (c2 == 0.0f) c2 = 1.0f;
  if (t < nb) {
    float q = fminf(fmaxf(rintf(__fdiv_rn(amax_s[t], c2)), 0.0f), 127.0f);
    static_cast<int8_t*>(absmax)[b0 + t] = (int8_t)(int)q;
  }
  if (t == 0) absmax_scale[sb] = c2;
}

}  // namespace

hipError_t launch_pack_nf4(const void* w, int wdt, int64_t numel, int double_quant,
                           const float* thresholds15, uint8_t* codes, void* absmax,
                           float* absmax_scale, hipStream_t s, bool fp4) {
  Thresholds th;
  for (int i = 0; i < 15; ++i) th.t[i] = thresholds15[i];
  const int64_t nblocks = numel / 64;
  const dim3 grid((unsigned)((nblocks + 255) / 256));
  const uint16_t* wp = static_cast<const uint16_t*>(w);
  uint32_t* cw = reinterpret_cast<uint32_t*>(codes);
#define WQ_PACK(DT, F) \
  pack_nf4_kernel<DT, F><<<grid, 256, 0, s>>>(wp, nblocks, double_quant, th, cw, absmax, absmax_scale)
  if (wdt == WQ_BF16) {
    if (fp4) WQ_PACK(WQ_BF16, true); else WQ_PACK(WQ_BF16, false);
  } else {
    if (fp4) WQ_PACK(WQ_F16, true); else WQ_PACK(WQ_F16, false);
  }
#undef WQ_PACK
  return hipGetLastError();
}

}  // namespace wq
