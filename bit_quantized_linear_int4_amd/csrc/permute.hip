// Column gather of a 16-bit row-major matrix: dst[r][j] = src[r][perm[j]].
//
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

}  // namespace

hipError_t launch_permute_cols(const uint16_t* src, int64_t rows, int64_t k,
                               const int32_t* perm, uint16_t* dst, hipStream_t s) {
  const int64_t chunks = rows * (k / 8);
  permute_cols_kernel<<<dim3((unsigned)((chunks + 255) / 256)), 256, 0, s>>>(src, rows, k, perm,
                                                                             dst);
  return hipGetLastError();
}

}  // namespace wq
