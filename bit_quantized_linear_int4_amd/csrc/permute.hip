// Column transforms of a 16-bit row-major matrix.
//
// Gather: dst[r][j] = src[r][perm[j]].
// Act-order ("LLM quantization selection: five mainstream schemes
// compared", section 3.2; "Open-source model quantization guide", section
// 3.2) quantizes the input channels in an importance order, so inference has
// to reorder: the weights are stored with their columns in that order (this
// gather, once, before quantizing) and the activations of every call are
// gathered the same way before the linear.
//
// One lane writes 8 consecutive outputs of a row (one 16-byte store) from
// 8 gathered 2-byte loads; indices outside [0, k) are clamped, so a bad
// permutation gives wrong values but no out-of-bounds access.
//
// Scaling: dst[r][c] = round16(src[r][c] * scale[c]), the fp32 product
// rounded once.  SmoothQuant ("LLM quantization selection: five mainstream
// schemes compared", section 5) moves activation range into the weights with
// a per-channel s: weights times s (offline, before INT8 quantization),
// activations divided by s (upstream of the W8A8 product).  One lane
// scales 8 consecutive elements (16-byte load and store).
#include "internal.h"

namespace wq {
namespace {

__global__ __launch_bounds__(256) void permute_cols_kernel(const uint16_t* __restrict__ src,
                                                           int64_t rows, int64_t k,
                                                           const int32_t* __restrict__ perm,
                                                           uint16_t* __restrict__ dst) {
  const int64_t chunk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = k / 8;
  if (chunk >= rows * per_row) return;
  const int64_t r = chunk / per_row, j0 = (chunk % per_row) * 8;
  const uint16_t* s = src + r * k;
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p0 = min((uint32_t)perm[j0 + 2 * i], (uint32_t)(k - 1));
    const uint32_t p1 = min((uint32_t)perm[j0 + 2 * i + 1], (uint32_t)(k - 1));
    o[i] = (uint32_t)s[p0] | ((uint32_t)s[p1] << 16);
  }
  *reinterpret_cast<uint4_t*>(dst + r * k + j0) = uint4_t{o[0], o[1], o[2], o[3]};
}

template <int DT>
__global__ __launch_bounds__(256) void scale_cols_kernel(const uint16_t* src,   // may be dst
                                                         int64_t rows, int64_t k,
                                                         const float* __restrict__ scale,
                                                         uint16_t* dst) {
  const int64_t chunk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = k / 8;
  if (chunk >= rows * per_row) return;
  const int64_t e0 = chunk * 8, c0 = (chunk % per_row) * 8;
  const uint4_t v = *reinterpret_cast<const uint4_t*>(src + e0);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = v[i];
    const float a0 = DT == WQ_BF16 ? bf16_bits_to_f32(u & 0xFFFFu) : f16_bits_to_f32(u & 0xFFFFu);
    const float a1 = DT == WQ_BF16 ? bf16_bits_to_f32(u >> 16) : f16_bits_to_f32(u >> 16);
    const float p0 = as_f32(a0 * scale[c0 + 2 * i]), p1 = as_f32(a1 * scale[c0 + 2 * i + 1]);
    o[i] = DT == WQ_BF16 ? ((uint32_t)f32_to_bf16_bits(p0) | ((uint32_t)f32_to_bf16_bits(p1) << 16))
                         : ((uint32_t)f32_to_f16_bits(p0) | ((uint32_t)f32_to_f16_bits(p1) << 16));
  }
  *reinterpret_cast<uint4_t*>(dst + e0) = uint4_t{o[0], o[1], o[2], o[3]};
}

}  // namespace

hipError_t launch_scale_cols(const uint16_t* src, int dt, int64_t rows, int64_t k,
                             const float* scale, uint16_t* dst, hipStream_t s) {
  const int64_t chunks = rows * (k / 8);
  const dim3 grid((unsigned)((chunks + 255) / 256));
  if (dt == WQ_BF16)
    scale_cols_kernel<WQ_BF16><<<grid, 256, 0, s>>>(src, rows, k, scale, dst);
  else
    scale_cols_kernel<WQ_F16><<<grid, 256, 0, s>>>(src, rows, k, scale, dst);
  return hipGetLastError();
}

hipError_t launch_permute_cols(const uint16_t* src, int64_t rows, int64_t k,
                               const int32_t* perm, uint16_t* dst, hipStream_t s) {
  const int64_t chunks = rows * (k / 8);
  permute_cols_kernel<<<dim3((unsigned)((chunks + 255) / 256)), 256, 0, s>>>(src, rows, k, perm,
                                                                             dst);
  return hipGetLastError();
}

}  // namespace wq
