// Whole-matrix dequantization into 16-bit values (test / debugging hook).
//
// INT4: w_hat = round16((q - z) * s)      (the product is exact in fp32)
// NF4 : w_hat = round16(L[code] * a_hat)  (a_hat = q8 * c2 with double quant)
// INT8: w_hat = round16(fp32(q) * s)
// These are the dequantizations the linear kernels apply in registers
// ("LLM quantization selection", section 5 opening: weights go back to FP16
// before the multiply-add; section 6.2: NF4 goes back to the compute dtype).
#include "internal.h"

namespace wq {
namespace {

struct Levels {
  float v[16];
};

template <int FMT, int ODT>
__global__ __launch_bounds__(256) void dequant_kernel(wq_weight w, Levels lv,
                                                      uint16_t* __restrict__ out) {
  const int64_t chunk = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8 elements each
  const int64_t total = w.n * w.k / 8;
  if (chunk >= total) return;
  const int64_t e0 = chunk * 8;
  const int64_t r = e0 / w.k, c0 = e0 % w.k;
  float v[8];
  if constexpr (FMT == WQ_FMT_INT4_ASYM) {
    const uint32_t word = static_cast<const uint32_t*>(w.codes)[chunk];
    const int64_t G = w.k / w.group;
    const int64_t g = c0 / w.group;
    const float s = f16_bits_to_f32(static_cast<const uint16_t*>(w.scales)[r * G + g]);
    const uint8_t zb = w.zeros[r * ((G + 1) / 2) + g / 2];
    const float z = (float)((g & 1) ? (zb >> 4) : (zb & 15));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ((float)((word >> (4 * i)) & 15u) - z) * s;
  } else if constexpr (FMT == WQ_FMT_NF4) {
    const uint32_t word = static_cast<const uint32_t*>(w.codes)[chunk];
    const int64_t blk = e0 / w.group;
    float ah;
    if (w.scales2 != nullptr)
      ah = (float)static_cast<const int8_t*>(w.scales)[blk] * w.scales2[blk / w.group2];
    else
      ah = static_cast<const float*>(w.scales)[blk];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = as_f32(lv.v[(word >> (4 * i)) & 15u] * ah);
  } else {
    const int8_t* q = static_cast<const int8_t*>(w.codes) + e0;
    const float s = static_cast<const float*>(w.scales)[r];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = as_f32((float)q[i] * s);
  }
  uint4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t lo = ODT == WQ_BF16 ? f32_to_bf16_bits(v[2 * i]) : f32_to_f16_bits(v[2 * i]);
    const uint16_t hi =
        ODT == WQ_BF16 ? f32_to_bf16_bits(v[2 * i + 1]) : f32_to_f16_bits(v[2 * i + 1]);
    o[i] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
  *reinterpret_cast<uint4_t*>(out + e0) = o;
}

template <int ODT>
hipError_t dequant_odt(const wq_weight* w, const float* levels, uint16_t* out, hipStream_t s) {
  Levels lv;
  for (int i = 0; i < 16; ++i) lv.v[i] = levels[i];
  const int64_t chunks = w->n * w->k / 8;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  switch (w->fmt) {
    case WQ_FMT_INT4_ASYM: dequant_kernel<WQ_FMT_INT4_ASYM, ODT><<<grid, 256, 0, s>>>(*w, lv, out); break;
    case WQ_FMT_NF4: dequant_kernel<WQ_FMT_NF4, ODT><<<grid, 256, 0, s>>>(*w, lv, out); break;
    default: dequant_kernel<WQ_FMT_INT8_SYM_ROW, ODT><<<grid, 256, 0, s>>>(*w, lv, out); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(const wq_weight* w, const float* levels16, void* out, int odt,
                             hipStream_t s) {
  uint16_t* o = static_cast<uint16_t*>(out);
  if (odt == WQ_BF16) return dequant_odt<WQ_BF16>(w, levels16, o, s);
  return dequant_odt<WQ_F16>(w, levels16, o, s);
}

}  // namespace wq
