// Weight quantization kernels: asymmetric INT4 per group, symmetric INT8 per
// row.
//
// INT4 follows the asymmetric formula of "Inference & deployment 05:
// quantized deployment compared" section 2.3 (scale = (max - min)/(2^b - 1),
// zero = round(-min/scale)) with b = 4, per group of `group` weights along k
// (section 2.2 there; group 128 in "LLM quantization selection" section 3.2).
// The range is widened to contain 0 so that the zero point is a code that
// represents float 0 (the concepts article, section 一).  The stored fp16
// scale is what the codes are computed with.
//
// INT8 is the symmetric formula of the same section 2.3 (scale = max|w|/127,
// range [-127, 127]) with one scale per output feature ("LLM quantization
// selection" section 2.1, vector-wise quantization).
//
// Both kernels are HBM-bound one-pass encoders: each lane reads 16 bytes of
// weights with one vector load and writes its codes with one store.
#include "internal.h"

namespace wq {
namespace {

template <int DT>
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  uint4_t raw = *reinterpret_cast<const uint4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t u = raw[i];
    uint16_t lo = (uint16_t)(u & 0xFFFFu), hi = (uint16_t)(u >> 16);
    v[2 * i] = DT == WQ_BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
    v[2 * i + 1] = DT == WQ_BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
  }
}

// One unit = two adjacent groups of one row (they share a zero-point byte);
// GROUP/8 lanes per group, 8 weights per lane.
template <int DT, int GROUP>
__global__ __launch_bounds__(256) void quant_int4_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, uint32_t* __restrict__ codes,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros) {
  constexpr int LPG = GROUP / 8;        // lanes per group
  constexpr int LPU = 2 * LPG;          // lanes per unit (pair of groups)
  const int64_t G = k / GROUP;
  const int64_t npairs = (G + 1) / 2;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t unit = gtid / LPU;
  const int li = (int)(gtid % LPU);
  const int gp = li / LPG, lg = li % LPG;
  const int64_t row = unit / npairs;
  const int64_t g = 2 * (unit % npairs) + gp;
  const bool valid = row < n && g < G;

  float v[8];
  if (valid) {
    load8<DT>(w + row * k + g * GROUP + lg * 8, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float lo = 0.0f, hi = 0.0f;           // the range always holds 0
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo = fminf(lo, v[i]);
    hi = fmaxf(hi, v[i]);
  }
#pragma unroll
  for (int off = 1; off < LPG; off <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, off));
    hi = fmaxf(hi, __shfl_xor(hi, off));
  }
  const float s32 = __fdiv_rn(hi - lo, 15.0f);
  uint16_t sbits = f32_to_f16_bits(s32);
  if ((sbits & 0x7FFFu) == 0) sbits = 0x3C00u;       // 0 -> 1.0
  const float s = f16_bits_to_f32(sbits);
  const float z = fminf(fmaxf(rintf(__fdiv_rn(-lo, s)), 0.0f), 15.0f);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = fminf(fmaxf(rintf(__fdiv_rn(v[i], s)) + z, 0.0f), 15.0f);
    word |= ((uint32_t)q) << (4 * i);
  }
  const uint32_t zi = (uint32_t)z;
  const uint32_t zpartner = __shfl_down(zi, LPG);
  if (valid) {
    codes[row * (k / 8) + g * LPG + lg] = word;
    if (lg == 0) scales[row * G + g] = sbits;
    if (lg == 0 && gp == 0) {
      uint32_t zb = zi | (g + 1 < G ? (zpartner << 4) : 0u);
      zeros[row * npairs + g / 2] = (uint8_t)zb;
    }
  }
}

// One workgroup per row: absmax reduction, then encode.
template <int DT>
__global__ __launch_bounds__(256) void quant_int8_rows_kernel(
    const uint16_t* __restrict__ w, int64_t k, int8_t* __restrict__ codes,
    float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* wr = w + row * k;
  const int64_t chunks = k / 8;
  float amax = 0.0f;
  for (int64_t c = threadIdx.x; c < chunks; c += 256) {
    float v[8];
    load8<DT>(wr + c * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = __fdiv_rn(amax, 127.0f);
  if (s == 0.0f) s = 1.0f;
  if (threadIdx.x == 0) scales[row] = s;
  for (int64_t c = threadIdx.x; c < chunks; c += 256) {
    float v[8];
    load8<DT>(wr + c * 8, v);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = fminf(fmaxf(rintf(__fdiv_rn(v[i], s)), -127.0f), 127.0f);
      uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)q;
      if (i < 4) lo |= b << (8 * i);
      else hi |= b << (8 * (i - 4));
    }
    uint2 out;
    out.x = lo;
    out.y = hi;
    *reinterpret_cast<uint2*>(codes + row * k + c * 8) = out;
  }
}

template <int DT>
hipError_t quant_int4_dt(const void* w, int64_t n, int64_t k, int group, uint32_t* codes,
                         uint16_t* scales, uint8_t* zeros, hipStream_t s) {
  const int64_t G = k / group;
  const int64_t units = n * ((G + 1) / 2);
  const int64_t lanes = units * (group / 4);
  const dim3 grid((unsigned)((lanes + 255) / 256));
  const uint16_t* wp = static_cast<const uint16_t*>(w);
  switch (group) {
    case 32: quant_int4_kernel<DT, 32><<<grid, 256, 0, s>>>(wp, n, k, codes, scales, zeros); break;
    case 64: quant_int4_kernel<DT, 64><<<grid, 256, 0, s>>>(wp, n, k, codes, scales, zeros); break;
    default: quant_int4_kernel<DT, 128><<<grid, 256, 0, s>>>(wp, n, k, codes, scales, zeros); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_int4(const void* w, int wdt, int64_t n, int64_t k, int group,
                             uint32_t* codes, uint16_t* scales, uint8_t* zeros,
                             hipStream_t s) {
  if (wdt == WQ_BF16) return quant_int4_dt<WQ_BF16>(w, n, k, group, codes, scales, zeros, s);
  return quant_int4_dt<WQ_F16>(w, n, k, group, codes, scales, zeros, s);
}

hipError_t launch_quant_int8_rows(const void* w, int wdt, int64_t n, int64_t k,
                                  int8_t* codes, float* scales, hipStream_t s) {
  const uint16_t* wp = static_cast<const uint16_t*>(w);
  if (wdt == WQ_BF16)
    quant_int8_rows_kernel<WQ_BF16><<<dim3((unsigned)n), 256, 0, s>>>(wp, k, codes, scales);
  else
    quant_int8_rows_kernel<WQ_F16><<<dim3((unsigned)n), 256, 0, s>>>(wp, k, codes, scales);
  return hipGetLastError();
}

}  // namespace wq
