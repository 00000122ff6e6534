// LLM.int8() mixed-precision decomposition ("LLM quantization selection: five
// mainstream schemes compared", section 2.1):
//   * feature columns whose activations exceed the threshold (6.0,
//     llm_int8_threshold in "Inference & deployment 05", section 6.1) in
//     absolute value for any token are outliers and stay in fp16;
//   * the rest is quantized to int8 (activations per token, weights per
//     output feature) and multiplied in int8 with int32 accumulation;
//   * the two products are summed.
//
// Kernels, in launch order:
//   int8_colflags   per (64-row chunk, column): any |x| > threshold
//   int8_compact    one workgroup: OR over row chunks -> mask, ascending
//                   outlier list, count (no host round trip; the count stays
//                   on the device)
//   int8_quant_act  one workgroup per token: absmax over the non-outlier
//                   columns -> sx, codes (0 in outlier columns)
//   int8_gemm       256 x BN output tiles: v_mfma_i32_16x16x64_i8 over K, then
//                   y = acc * sx * sw, then the outlier columns through
//                   v_mfma_f32_16x16x32_f16 on fp16 activations and the int8
//                   weights dequantized to fp16, accumulated into the same
//                   registers.
#include <algorithm>

#include "internal.h"

namespace wq {
namespace {

constexpr int kRowChunk = 64;

__global__ __launch_bounds__(256) void int8_colflags_kernel(const uint16_t* __restrict__ x,
                                                            int64_t m, int64_t k, float thr,
                                                            uint8_t* __restrict__ flags) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= k) return;
  const int64_t r0 = (int64_t)blockIdx.y * kRowChunk;
  const int64_t r1 = std::min<int64_t>(m, r0 + kRowChunk);
  bool any = false;
  for (int64_t r = r0; r < r1; ++r) any |= fabsf(f16_bits_to_f32(x[r * k + c])) > thr;
  flags[(int64_t)blockIdx.y * k + c] = any ? 1 : 0;
}

__global__ __launch_bounds__(1024) void int8_compact_kernel(const uint8_t* __restrict__ flags,
                                                            int64_t k, int chunks,
                                                            uint8_t* __restrict__ mask,
                                                            int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ count) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = (k + 1023) / 1024;
  const int64_t c0 = std::min<int64_t>(k, t * per), c1 = std::min<int64_t>(k, c0 + per);
  int32_t n = 0;
  for (int64_t c = c0; c < c1; ++c) {
    uint8_t f = 0;
    for (int j = 0; j < chunks; ++j) f |= flags[(int64_t)j * k + c];
    mask[c] = f;
    n += f;
  }
  part[t] = n;
  __syncthreads();
  // inclusive scan (Hillis-Steele) over 1024 partial counts
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t pos = part[t] - n;
  for (int64_t c = c0; c < c1; ++c)
    if (mask[c]) idx[pos++] = (int32_t)c;
  if (t == 1023) *count = part[1023];
}

__global__ __launch_bounds__(256) void int8_quant_act_kernel(const uint16_t* __restrict__ x,
                                                             int64_t k,
                                                             const uint8_t* __restrict__ mask,
                                                             int8_t* __restrict__ qx,
                                                             float* __restrict__ sx) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * k;
  const int64_t chunks = k / 8;
  float amax = 0.0f;
  for (int64_t c = threadIdx.x; c < chunks; c += 256) {
    const uint4_t raw = *reinterpret_cast<const uint4_t*>(xr + c * 8);
    const uint2 mk = *reinterpret_cast<const uint2*>(mask + c * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = (raw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const uint32_t mb = ((i < 4 ? mk.x : mk.y) >> (8 * (i & 3))) & 0xFFu;
      if (!mb) amax = fmaxf(amax, fabsf(f16_bits_to_f32((uint16_t)h)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = __fdiv_rn(amax, 127.0f);
  if (s == 0.0f) s = 1.0f;
  if (threadIdx.x == 0) sx[row] = s;
  for (int64_t c = threadIdx.x; c < chunks; c += 256) {
    const uint4_t raw = *reinterpret_cast<const uint4_t*>(xr + c * 8);
    const uint2 mk = *reinterpret_cast<const uint2*>(mask + c * 8);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = (raw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const uint32_t mb = ((i < 4 ? mk.x : mk.y) >> (8 * (i & 3))) & 0xFFu;
      float q = fminf(fmaxf(rintf(__fdiv_rn(f16_bits_to_f32((uint16_t)h), s)), -127.0f), 127.0f);
      if (mb) q = 0.0f;
      const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)q;
      if (i < 4) lo |= b << (8 * i);
      else hi |= b << (8 * (i - 4));
    }
    uint2 o;
    o.x = lo;
    o.y = hi;
    *reinterpret_cast<uint2*>(qx + row * k + c * 8) = o;
  }
}

// ---------------------------------------------------------------- GEMM
constexpr int IBM = 256, IBK = 128, ILD = IBK + 16;   // bytes per LDS row

template <int NT>
struct Int8Tile {
  static constexpr int BN = NT * 16;
};

__device__ __forceinline__ int4_t mfma_i8(uint4_t a, uint4_t b, int4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(int4_t, a),
                                               __builtin_bit_cast(int4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma_f16(uint4_t a, uint4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

struct Int8GemmArgs {
  const uint16_t* x;     // fp16 [m][k]
  const int8_t* qx;      // [m][k]
  const float* sx;       // [m]
  const int8_t* qw;      // [n][k]
  const float* sw;       // [n]
  const int32_t* idx;
  const int32_t* count;
  int m, n, k;
  void* y;
  int32_t* acc_out;
};

template <int NT, int YDT>
__global__ __launch_bounds__(256) void int8_gemm_kernel(Int8GemmArgs a) {
  constexpr int BN = NT * 16;
  __shared__ __attribute__((aligned(16))) uint8_t smem[IBM * ILD + BN * ILD];
  uint8_t* As = smem;
  uint8_t* Bs = smem + IBM * ILD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * IBM, n0 = blockIdx.x * BN;

  constexpr int AV = IBM * IBK / 16 / 256;   // uint4 per thread for the x tile (8)
  constexpr int BV = BN * IBK / 16;          // uint4 for the weight tile
  constexpr int BVT = (BV + 255) / 256;
  uint4_t ra[AV], rb[BVT];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int r = 0; r < AV; ++r) {
      const int i = tid + 256 * r;
      const int row = i >> 3, col = (i & 7) * 16;
      if (m0 + row < a.m)
        ra[r] = *reinterpret_cast<const uint4_t*>(a.qx + (int64_t)(m0 + row) * a.k + k0 + col);
      else
        ra[r] = uint4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < BVT; ++r) {
      const int i = tid + 256 * r;
      if (i < BV) {
        const int row = i >> 3, col = (i & 7) * 16;
        const int rg = min(n0 + row, a.n - 1);
        rb[r] = *reinterpret_cast<const uint4_t*>(a.qw + (int64_t)rg * a.k + k0 + col);
      }
    }
  };

  int4_t acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = int4_t{0, 0, 0, 0};

  const int nk = a.k / IBK;
  load_tile(0);
  for (int ks = 0; ks < nk; ++ks) {
#pragma unroll
    for (int r = 0; r < AV; ++r) {
      const int i = tid + 256 * r;
      *reinterpret_cast<uint4_t*>(&As[(i >> 3) * ILD + (i & 7) * 16]) = ra[r];
    }
#pragma unroll
    for (int r = 0; r < BVT; ++r) {
      const int i = tid + 256 * r;
      if (i < BV) *reinterpret_cast<uint4_t*>(&Bs[(i >> 3) * ILD + (i & 7) * 16]) = rb[r];
    }
    __syncthreads();
    if (ks + 1 < nk) load_tile((ks + 1) * IBK);
#pragma unroll
    for (int kk = 0; kk < IBK / 64; ++kk) {
      uint4_t af[4], bf[NT];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const uint4_t*>(
            &As[(wave * 64 + i * 16 + (lane & 15)) * ILD + kk * 64 + (lane >> 4) * 16]);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bf[j] = *reinterpret_cast<const uint4_t*>(
            &Bs[(j * 16 + (lane & 15)) * ILD + kk * 64 + (lane >> 4) * 16]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma_i8(af[i], bf[j], acc[i][j]);
    }
    __syncthreads();
  }

  // ---- epilogue: raw accumulators (optional), rescale, outlier slice
  float4_t yf[4][NT];
  float swv[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int nn = n0 + j * 16 + (lane & 15);
    swv[j] = nn < a.n ? a.sw[nn] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int mm = m0 + wave * 64 + i * 16 + (lane >> 4) * 4 + e;
      const float sxv = mm < a.m ? a.sx[mm] : 0.0f;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int nn = n0 + j * 16 + (lane & 15);
        if (a.acc_out != nullptr && mm < a.m && nn < a.n)
          a.acc_out[(int64_t)mm * a.n + nn] = acc[i][j][e];
        yf[i][j][e] = ((float)acc[i][j][e] * sxv) * swv[j];
      }
    }
  }

  const int cnt = *a.count;
  uint16_t* Xo = reinterpret_cast<uint16_t*>(smem);              // [IBM][40] fp16
  uint16_t* Wo = reinterpret_cast<uint16_t*>(smem) + IBM * 40;   // [BN][40] fp16
  for (int c0 = 0; c0 < cnt; c0 += 32) {
    for (int e = tid; e < IBM * 32; e += 256) {
      const int r = e >> 5, j = e & 31;
      uint16_t v = 0;
      if (c0 + j < cnt && m0 + r < a.m) v = a.x[(int64_t)(m0 + r) * a.k + a.idx[c0 + j]];
      Xo[r * 40 + j] = v;
    }
    for (int e = tid; e < BN * 32; e += 256) {
      const int r = e >> 5, j = e & 31;
      uint16_t v = 0;
      if (c0 + j < cnt && n0 + r < a.n) {
        const float wq = (float)a.qw[(int64_t)(n0 + r) * a.k + a.idx[c0 + j]];
        v = f32_to_f16_bits(as_f32(wq * a.sw[n0 + r]));
      }
      Wo[r * 40 + j] = v;
    }
    __syncthreads();
    uint4_t af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const uint4_t*>(
          &Xo[(wave * 64 + i * 16 + (lane & 15)) * 40 + (lane >> 4) * 8]);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint4_t bf =
          *reinterpret_cast<const uint4_t*>(&Wo[(j * 16 + (lane & 15)) * 40 + (lane >> 4) * 8]);
#pragma unroll
      for (int i = 0; i < 4; ++i) yf[i][j] = mfma_f16(af[i], bf, yf[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int mm = m0 + wave * 64 + i * 16 + (lane >> 4) * 4 + e;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int nn = n0 + j * 16 + (lane & 15);
        if (mm < a.m && nn < a.n) {
          if constexpr (YDT == WQ_F32)
            static_cast<float*>(a.y)[(int64_t)mm * a.n + nn] = yf[i][j][e];
          else
            static_cast<uint16_t*>(a.y)[(int64_t)mm * a.n + nn] = f32_to_f16_bits(yf[i][j][e]);
        }
      }
    }
}

}  // namespace

hipError_t launch_int8_prepare(const uint16_t* x, int64_t m, int64_t k, float thr,
                               uint8_t* mask, int32_t* idx, int32_t* count, int8_t* qx,
                               float* sx, hipStream_t s) {
  // The per-row-chunk column flags (chunks * k bytes) are staged in qx, which
  // holds m * k >= chunks * k bytes and is overwritten by int8_quant_act after
  // int8_compact has consumed them (same stream, in order).
  const int chunks = (int)((m + kRowChunk - 1) / kRowChunk);
  uint8_t* flags = reinterpret_cast<uint8_t*>(qx);
  int8_colflags_kernel<<<dim3((unsigned)((k + 255) / 256), (unsigned)chunks), 256, 0, s>>>(
      x, m, k, thr, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int8_compact_kernel<<<1, 1024, 0, s>>>(flags, k, chunks, mask, idx, count);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int8_quant_act_kernel<<<dim3((unsigned)m), 256, 0, s>>>(x, k, mask, qx, sx);
  return hipGetLastError();
}

hipError_t launch_int8_gemm(const uint16_t* x, int64_t m, const wq_weight* w, const int8_t* qx,
                            const float* sx, const int32_t* idx, const int32_t* count, void* y,
                            int ydt, int32_t* acc_out, hipStream_t s) {
  Int8GemmArgs a;
  a.x = x;
  a.qx = qx;
  a.sx = sx;
  a.qw = static_cast<const int8_t*>(w->codes);
  a.sw = static_cast<const float*>(w->scales);
  a.idx = idx;
  a.count = count;
  a.m = (int)m;
  a.n = (int)w->n;
  a.k = (int)w->k;
  a.y = y;
  a.acc_out = acc_out;
  constexpr int NT = 8;
  const dim3 grid((unsigned)((w->n + NT * 16 - 1) / (NT * 16)), (unsigned)((m + IBM - 1) / IBM));
  if (ydt == WQ_F32)
    int8_gemm_kernel<NT, WQ_F32><<<grid, 256, 0, s>>>(a);
  else
    int8_gemm_kernel<NT, WQ_F16><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace wq
