// W4A16 linear: y = x . w_hat^T with 4-bit weights dequantized to 16 bits
// inside the kernel ("LLM quantization selection: five mainstream schemes
// compared", section 5 opening: W4A16 dequantizes the weights back to FP16 and
// multiplies in FP16; section 4.3: a GEMV version for single requests and a
// GEMM version for batches).
//
// Two kernel families:
//
//  * skinny (m <= 16, decode).  HBM-bound: the packed weights are streamed
//    once with 16-byte loads.  Each wave owns 16*RT weight rows and a range
//    of 128-wide groups; every lane loads one 16-byte chunk (32 codes of one
//    row) per row tile and group.  The multiply runs on the matrix cores
//    (v_mfma_f32_16x16x32_{f16,bf16}) with the activations (m padded to 16)
//    as the A operand and the codes as the B operand, so no cross-lane
//    reduction is needed inside a wave.
//
//    INT4 codes become 16-bit values with the exponent-bias trick: OR-ing a
//    nibble into the mantissa of 1024.0 (fp16) or 128.0 (bf16) gives exactly
//    1024 + q (or 128 + q).  The MFMA accumulates sum_k x_k (B + q_k) over a
//    group, and the zero point and bias are removed afterwards with the
//    group's activation sum X = sum_k x_k (itself an MFMA against a ones
//    operand):  sum_k x_k (q_k - z) s = s * (acc - (B + z) X).
//    The nibble extraction yields (q0,q4),(q1,q5),(q2,q6),(q3,q7) pairs;
//    the activations are permuted the same way (the dot product does not
//    care about the order of k inside one MFMA).
//
//    NF4 codes are looked up in the 16-level table (LDS), multiplied by the
//    block's absmax and rounded to the activation type, exactly as the
//    dequantization defines them.
//
//    The four waves of a workgroup split the workgroup's group range and
//    their results are summed in LDS in a fixed order.  When the schedule
//    also splits K across workgroups, each workgroup writes fp32 partial
//    sums to the workspace and a second kernel adds them in a fixed order,
//    so results are deterministic.
//
//  * gemm (m > 16, prefill).  MFMA-bound: 128x128 output tiles, the weight
//    tile is dequantized once into LDS in the activation type and both
//    operands are read from LDS by four waves (64x64 each).
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "internal.h"

namespace wq {
namespace {

constexpr int kWave = 64;

template <int XDT>
using mfma_in_t = typename std::conditional<XDT == WQ_BF16, bf16x8_t, half8_t>::type;

template <int XDT>
__device__ __forceinline__ float4_t mfma16(uint4_t a, uint4_t b, float4_t c) {
  if constexpr (XDT == WQ_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
}

// (x0..x7) -> (x0,x4),(x1,x5),(x2,x6),(x3,x7): the order the INT4 unpack
// produces for the codes.
__device__ __forceinline__ uint4_t perm_x(uint4_t d) {
  uint4_t r;
  r[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
  return r;
}

template <int XDT>
__device__ __forceinline__ uint16_t f32_to_x(float v) {
  return XDT == WQ_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
}

template <int YDT>
__device__ __forceinline__ void store_y(void* y, int64_t idx, float v) {
  if constexpr (YDT == WQ_F32) {
    static_cast<float*>(y)[idx] = v;
  } else if constexpr (YDT == WQ_BF16) {
    static_cast<uint16_t*>(y)[idx] = f32_to_bf16_bits(v);
  } else {
    static_cast<uint16_t*>(y)[idx] = f32_to_f16_bits(v);
  }
}

struct SkinnyArgs {
  const uint16_t* x;
  const uint32_t* codes;     // INT4: [n][k/8]; NF4: bytes [n*k/2] viewed as words
  const void* scales;        // INT4: fp16 [n][G]; NF4: int8 or fp32 absmax
  const uint8_t* zeros;      // INT4 only
  const float* scales2;      // NF4 double-quant second level, or nullptr
  int m, n, k, G, zb;        // zb = bytes per row of zeros
  float* partial;            // [splits][m][n] when the K range is split
  void* y;
};

struct Levels {
  float v[16];
};

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// One 32-bit word of 8 codes -> 8 biased fp16 values 1024 + q, ordered
// (q0,q4),(q1,q5),(q2,q6),(q3,q7) (v_and_or_b32 per pair).
__device__ __forceinline__ uint4_t unpack_biased_f16(uint32_t w) {
  const uint32_t kM = 0x000F000Fu, kB = 0x64006400u;
  uint4_t r;
  r[0] = and_or(w, kM, kB);
  r[1] = and_or(w >> 4, kM, kB);
  r[2] = and_or(w >> 8, kM, kB);
  r[3] = and_or(w >> 12, kM, kB);
  return r;
}

// Decoders for one 32-bit word of 8 codes in natural order -> 8 dequantized
// 16-bit weights, rounded once into the activation type.
template <int XDT>
__device__ __forceinline__ uint4_t dequant_int4_word(uint32_t w, float z, float s) {
  uint4_t b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float q0 = (float)((w >> (8 * e)) & 15u);
    const float q1 = (float)((w >> (8 * e + 4)) & 15u);
    b[e] = (uint32_t)f32_to_x<XDT>((q0 - z) * s) | ((uint32_t)f32_to_x<XDT>((q1 - z) * s) << 16);
  }
  return b;
}
template <int XDT>
__device__ __forceinline__ uint4_t dequant_nf4_word(uint32_t w, const float* lut, float ah) {
  uint4_t b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v0 = lut[(w >> (8 * e)) & 15u] * ah;
    const float v1 = lut[(w >> (8 * e + 4)) & 15u] * ah;
    b[e] = (uint32_t)f32_to_x<XDT>(v0) | ((uint32_t)f32_to_x<XDT>(v1) << 16);
  }
  return b;
}

// Decode-shaped kernel.  A workgroup owns TPG row tiles (16 rows each) and a
// chunk of KCG = 4*GPW groups of 128 along K; its four waves take GPW groups
// each, for all TPG tiles.  Every wave issues all of its weight loads up
// front (one load round), after the loads that stage the activation chunk
// (MP rows, zero-padded) into LDS; the multiply consumes the weights in
// arrival order.  The waves' partial sums are added in LDS in a fixed order.
// FAST (INT4 weights, fp16 activations) uses the exponent-bias unpack with
// the per-group correction; the other decoders build exactly rounded
// dequantized weights.
template <int XDT, int YDT, int FMT, int TPG, int GPW, int MP>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs a, Levels lv) {
  constexpr int KCG = 4 * GPW;
  constexpr bool FAST = (FMT == WQ_FMT_INT4_ASYM) && (XDT == WQ_F16);
  constexpr int XTOT = KCG * 16 * MP;            // staged 16-byte chunks
  constexpr int XU = (XTOT + 255) / 256;
  constexpr int RED = 4 * TPG * 4 * kWave;       // floats for the wave reduction
  constexpr int SMEM16 = XTOT > RED / 4 ? XTOT : RED / 4;
  __shared__ uint4_t xs[SMEM16];                  // activations, then the reduction
  __shared__ float lut[16];
  float* red = reinterpret_cast<float*>(xs);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, kq = lane >> 4;
  const int g0 = blockIdx.y * KCG;
  const int ntiles = (a.n + 15) / 16;
  const int tile0 = blockIdx.x * TPG;

  // 1. activation chunk loads (first, so that waiting for them does not wait
  //    for the weight loads issued after them)
  uint4_t xv[XU];
#pragma unroll
  for (int r = 0; r < XU; ++r) {
    const int i = tid + 256 * r;
    const int g = i / (16 * MP), q = i % (16 * MP), m = q / 16, c16 = q % 16;
    const int gg = min(g0 + g, a.G - 1), mm = min(m, a.m - 1);
    const uint4_t v = *reinterpret_cast<const uint4_t*>(a.x + (int64_t)mm * a.k + gg * 128 + c16 * 8);
    xv[r] = (i < XTOT && m < a.m && g0 + g < a.G) ? v : uint4_t{0u, 0u, 0u, 0u};
  }
  // 2. all weight loads of this wave
  const uint4_t* q4 = reinterpret_cast<const uint4_t*>(a.codes);
  const int k32 = a.k / 32;
  uint4_t wv[TPG][GPW];
  float sv[TPG][GPW];
  uint32_t zv[TPG][GPW];
#pragma unroll
  for (int t = 0; t < TPG; ++t) {
    const int row = min(min(tile0 + t, ntiles - 1) * 16 + nl, a.n - 1);
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      const int g = min(g0 + wave * GPW + u, a.G - 1);
      wv[t][u] = q4[(int64_t)row * k32 + g * 4 + kq];
      if constexpr (FMT == WQ_FMT_INT4_ASYM) {
        sv[t][u] = f16_bits_to_f32(static_cast<const uint16_t*>(a.scales)[(int64_t)row * a.G + g]);
        zv[t][u] = a.zeros[(int64_t)row * a.zb + (g >> 1)];
      } else {
        const int64_t blk = (int64_t)row * (a.k / 64) + 2 * g + (kq >> 1);
        if (a.scales2 != nullptr)
          sv[t][u] = (float)static_cast<const int8_t*>(a.scales)[blk] * a.scales2[blk >> 8];
        else
          sv[t][u] = static_cast<const float*>(a.scales)[blk];
        zv[t][u] = 0;
      }
    }
  }
  // 3. stage the activations; layout [group][16-byte chunk c16][row m]
#pragma unroll
  for (int r = 0; r < XU; ++r) {
    const int i = tid + 256 * r;
    if (i < XTOT) {
      const int g = i / (16 * MP), q = i % (16 * MP), m = q / 16, c16 = q % 16;
      xs[(g * 16 + c16) * MP + m] = FAST ? perm_x(xv[r]) : xv[r];
    }
  }
  if (FMT == WQ_FMT_NF4 && tid < 16) lut[tid] = lv.v[tid];
  __syncthreads();

  // 4. multiply
  constexpr uint32_t kOne = 0x3C003C00u;
  const uint4_t ones = {kOne, kOne, kOne, kOne};
  float4_t acc[TPG];
#pragma unroll
  for (int t = 0; t < TPG; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  const int mrow = min(nl, MP - 1);
#pragma unroll
  for (int u = 0; u < GPW; ++u) {
    const int gl = wave * GPW + u;
    const int gabs = g0 + gl;
    uint4_t A[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      A[j] = nl < a.m ? xs[(gl * 16 + kq * 4 + j) * MP + mrow] : uint4_t{0u, 0u, 0u, 0u};
    if constexpr (FAST) {
      float4_t X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) X = mfma16<XDT>(A[j], ones, X);
#pragma unroll
      for (int t = 0; t < TPG; ++t) {
        float4_t tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) tmp = mfma16<XDT>(A[j], unpack_biased_f16(wv[t][u][j]), tmp);
        const uint32_t z = (gabs & 1) ? (zv[t][u] >> 4) : (zv[t][u] & 15u);
        const float zb = 1024.0f + (float)z;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(fmaf(-zb, X[e], tmp[e]), sv[t][u], acc[t][e]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < TPG; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint4_t b;
          if constexpr (FMT == WQ_FMT_INT4_ASYM) {
            const float z = (float)((gabs & 1) ? (zv[t][u] >> 4) : (zv[t][u] & 15u));
            b = dequant_int4_word<XDT>(wv[t][u][j], z, sv[t][u]);
          } else {
            b = dequant_nf4_word<XDT>(wv[t][u][j], lut, sv[t][u]);
          }
          acc[t] = mfma16<XDT>(A[j], b, acc[t]);
        }
      }
    }
  }
  // 5. add the four waves' sums in a fixed order, then store
  __syncthreads();  // every wave is done reading the activations
#pragma unroll
  for (int t = 0; t < TPG; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * TPG + t) * 4 + e) * kWave + lane] = acc[t][e];
  __syncthreads();
  constexpr int NV = TPG * 4 * kWave;
  const bool splitting = gridDim.y > 1;
  for (int i = tid; i < NV; i += 256) {
    const int te = i / kWave, l = i % kWave, t = te / 4, e = te % 4;
    const int mm = (l >> 4) * 4 + e;
    const int nn = (tile0 + t) * 16 + (l & 15);
    if (mm < a.m && nn < a.n) {
      float v = red[i];
      v += red[i + NV];
      v += red[i + 2 * NV];
      v += red[i + 3 * NV];
      if (splitting)
        a.partial[((int64_t)blockIdx.y * a.m + mm) * a.n + nn] = v;
      else
        store_y<YDT>(a.y, (int64_t)mm * a.n + nn, v);
    }
  }
}

template <int YDT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int64_t mn, void* y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn) return;
  float v = part[i];
  for (int s = 1; s < splits; ++s) v += part[(int64_t)s * mn + i];
  store_y<YDT>(y, i, v);
}

// ------------------------------------------------------------------ GEMM
constexpr int GBM = 128, GBN = 128, GBK = 64, GLD = GBK + 8;  // LDS row stride (halfs)

struct GemmArgs {
  const uint16_t* x;
  const uint32_t* codes;
  const void* scales;
  const uint8_t* zeros;
  const float* scales2;
  int m, n, k, G, zb;
  void* y;
};

// Dequantize 32 consecutive weights (one 16-byte chunk of codes) of row r,
// starting at column c0, into 32 16-bit values in natural order.
template <int FMT, int XDT>
__device__ __forceinline__ void dequant32(const GemmArgs& a, const float* lut, int r, int c0,
                                          uint4_t wv, uint32_t (&out)[16]) {
  if constexpr (FMT == WQ_FMT_INT4_ASYM) {
    const int g = c0 >> 7;
    const float s = f16_bits_to_f32(static_cast<const uint16_t*>(a.scales)[(int64_t)r * a.G + g]);
    const uint8_t zbyte = a.zeros[(int64_t)r * a.zb + (g >> 1)];
    const float z = (float)((g & 1) ? (zbyte >> 4) : (zbyte & 15));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = wv[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float q0 = (float)((w >> (8 * e)) & 15u);
        const float q1 = (float)((w >> (8 * e + 4)) & 15u);
        // (q - z) * s is exact in fp32; one rounding into the activation type
        out[j * 4 + e] = (uint32_t)f32_to_x<XDT>((q0 - z) * s) |
                         ((uint32_t)f32_to_x<XDT>((q1 - z) * s) << 16);
      }
    }
  } else {
    const int64_t blk = ((int64_t)r * a.k + c0) >> 6;
    float ah;
    if (a.scales2 != nullptr)
      ah = (float)static_cast<const int8_t*>(a.scales)[blk] * a.scales2[blk >> 8];
    else
      ah = static_cast<const float*>(a.scales)[blk];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = wv[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = lut[(w >> (8 * e)) & 15u] * ah;
        const float v1 = lut[(w >> (8 * e + 4)) & 15u] * ah;
        out[j * 4 + e] = (uint32_t)f32_to_x<XDT>(v0) | ((uint32_t)f32_to_x<XDT>(v1) << 16);
      }
    }
  }
}

template <int FMT, int XDT, int YDT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a, Levels lv) {
  __shared__ uint16_t As[GBM * GLD];
  __shared__ uint16_t Bs[GBN * GLD];
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = lv.v[threadIdx.x];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;          // 2 x 2 waves of 64 x 64
  const int m0 = blockIdx.y * GBM, n0 = blockIdx.x * GBN;

  // global -> register loaders
  uint4_t xa[4];
  uint4_t wb;
  const int brow = tid >> 1, bhalf = tid & 1;        // weight tile: 128 rows x 2 chunks
  const int brow_g = min(n0 + brow, a.n - 1);
  const uint4_t* q4 = reinterpret_cast<const uint4_t*>(a.codes);
  const int k32 = a.k / 32;

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = tid + 256 * r;
      const int row = i >> 3, col = (i & 7) * 8;
      if (m0 + row < a.m)
        xa[r] = *reinterpret_cast<const uint4_t*>(a.x + (int64_t)(m0 + row) * a.k + k0 + col);
      else
        xa[r] = uint4_t{0u, 0u, 0u, 0u};
    }
    wb = q4[(int64_t)brow_g * k32 + (k0 >> 5) + bhalf];
  };

  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = a.k / GBK;
  load_tile(0);
  __syncthreads();  // lut visible
  for (int ks = 0; ks < nk; ++ks) {
    const int k0 = ks * GBK;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = tid + 256 * r;
      const int row = i >> 3, col = (i & 7) * 8;
      *reinterpret_cast<uint4_t*>(&As[row * GLD + col]) = xa[r];
    }
    {
      uint32_t dq[16];
      dequant32<FMT, XDT>(a, lut, brow_g, k0 + bhalf * 32, wb, dq);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint4_t*>(&Bs[brow * GLD + bhalf * 32 + c * 8]) =
            uint4_t{dq[4 * c], dq[4 * c + 1], dq[4 * c + 2], dq[4 * c + 3]};
    }
    __syncthreads();
    if (ks + 1 < nk) load_tile(k0 + GBK);
#pragma unroll
    for (int kk = 0; kk < GBK / 32; ++kk) {
      uint4_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const uint4_t*>(&As[row * GLD + kk * 32 + (lane >> 4) * 8]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 64 + j * 16 + (lane & 15);
        bf[j] = *reinterpret_cast<const uint4_t*>(&Bs[row * GLD + kk * 32 + (lane >> 4) * 8]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<XDT>(af[i], bf[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int mm = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        const int nn = n0 + wn * 64 + j * 16 + (lane & 15);
        if (mm < a.m && nn < a.n) store_y<YDT>(a.y, (int64_t)mm * a.n + nn, acc[i][j][e]);
      }
}

// ---------------------------------------------------------------- launch
template <int XDT, int YDT, int FMT, int TPG, int GPW, int MP>
void launch_skinny_t(const SkinnyArgs& a, const Levels& lv, dim3 grid, hipStream_t s) {
  skinny_kernel<XDT, YDT, FMT, TPG, GPW, MP><<<grid, 256, 0, s>>>(a, lv);
}

// Schedules compiled for the decode kernel: (TPG, GPW, MP).
template <int XDT, int YDT, int FMT>
bool launch_skinny(const SkinnyArgs& a, const Levels& lv, const W4Plan& p, dim3 grid,
                   hipStream_t s) {
#define WQ_CASE(T, W, M)                                                       \
  if (p.tpg == T && p.gpw == W && p.mp == M) {                                 \
    launch_skinny_t<XDT, YDT, FMT, T, W, M>(a, lv, grid, s);                   \
    return true;                                                               \
  }
  WQ_CASE(1, 8, 1) WQ_CASE(2, 8, 1) WQ_CASE(1, 8, 4) WQ_CASE(2, 8, 4)
  WQ_CASE(1, 4, 1) WQ_CASE(1, 4, 4)
  WQ_CASE(1, 4, 16) WQ_CASE(2, 4, 16) WQ_CASE(3, 4, 16) WQ_CASE(4, 4, 16)
  WQ_CASE(1, 2, 16) WQ_CASE(2, 2, 16)
#undef WQ_CASE
  return false;
}

template <int XDT, int YDT>
hipError_t launch_typed(const void* x, int64_t m, const wq_weight* w, const float* levels,
                        void* y, void* ws, const W4Plan& p, hipStream_t s) {
  Levels lv;
  for (int i = 0; i < 16; ++i) lv.v[i] = levels[i];
  if (p.path == 1) {
    GemmArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.codes = static_cast<const uint32_t*>(w->codes);
    a.scales = w->scales;
    a.zeros = w->zeros;
    a.scales2 = w->scales2;
    a.m = (int)m;
    a.n = (int)w->n;
    a.k = (int)w->k;
    a.G = (int)(w->k / 128);
    a.zb = (a.G + 1) / 2;
    a.y = y;
    const dim3 grid((unsigned)((w->n + GBN - 1) / GBN), (unsigned)((m + GBM - 1) / GBM));
    if (w->fmt == WQ_FMT_NF4)
      gemm_kernel<WQ_FMT_NF4, XDT, YDT><<<grid, 256, 0, s>>>(a, lv);
    else
      gemm_kernel<WQ_FMT_INT4_ASYM, XDT, YDT><<<grid, 256, 0, s>>>(a, lv);
    return hipGetLastError();
  }
  SkinnyArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.codes = static_cast<const uint32_t*>(w->codes);
  a.scales = w->scales;
  a.zeros = w->zeros;
  a.scales2 = w->scales2;
  a.m = (int)m;
  a.n = (int)w->n;
  a.k = (int)w->k;
  a.G = (int)(w->k / 128);
  a.zb = (a.G + 1) / 2;
  a.partial = static_cast<float*>(ws);
  a.y = y;
  const int ntiles = (int)((w->n + 15) / 16);
  const dim3 grid((unsigned)((ntiles + p.tpg - 1) / p.tpg), (unsigned)p.splits);
  const bool ok = w->fmt == WQ_FMT_NF4 ? launch_skinny<XDT, YDT, WQ_FMT_NF4>(a, lv, p, grid, s)
                                       : launch_skinny<XDT, YDT, WQ_FMT_INT4_ASYM>(a, lv, p, grid, s);
  if (!ok) return hipErrorInvalidConfiguration;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t mn = m * w->n;
  splitk_reduce_kernel<YDT><<<dim3((unsigned)((mn + 255) / 256)), 256, 0, s>>>(
      static_cast<const float*>(ws), p.splits, mn, y);
  return hipGetLastError();
}

template <int XDT>
hipError_t launch_x(const void* x, int64_t m, const wq_weight* w, const float* levels, void* y,
                    int ydt, void* ws, const W4Plan& p, hipStream_t s) {
  switch (ydt) {
    case WQ_F32: return launch_typed<XDT, WQ_F32>(x, m, w, levels, y, ws, p, s);
    case WQ_BF16: return launch_typed<XDT, WQ_BF16>(x, m, w, levels, y, ws, p, s);
    default: return launch_typed<XDT, WQ_F16>(x, m, w, levels, y, ws, p, s);
  }
}

}  // namespace

W4Plan plan_w4a16(int64_t m, const wq_weight* w) {
  W4Plan p;
  p.path = m > 16 ? 1 : 0;
  p.tpg = 1;
  p.gpw = 8;
  p.mp = 1;
  p.splits = 1;
  p.ws = 0;
  if (p.path == 1) return p;
  const int64_t G = w->k / 128;
  const int64_t ntiles = (w->n + 15) / 16;
  p.mp = m <= 1 ? 1 : (m <= 4 ? 4 : 16);
  if (p.mp <= 4) {
    // the activation chunk is small: one workgroup covers up to 32 groups of
    // its tile, so K <= 4096 needs no split
    p.gpw = G >= 32 ? 8 : (G > 16 ? 8 : 4);
    p.splits = (int)((G + 4 * p.gpw - 1) / (4 * p.gpw));
    p.tpg = ntiles * p.splits >= 2048 ? 2 : 1;
  } else {
    // 16 staged rows: 16 groups (64 KB of activations) per workgroup, two
    // workgroups per CU, and enough tiles per workgroup that the grid is
    // resident in one scheduling round (<= 512 workgroups)
    p.gpw = 4;
    p.splits = (int)((G + 15) / 16);
    int64_t tpg = (ntiles * p.splits + 511) / 512;
    p.tpg = (int)std::max<int64_t>(1, std::min<int64_t>(4, tpg));
  }
#ifdef WQ_TUNE_ENV
  if (const char* e = getenv("WQ_SKINNY")) sscanf(e, "%d,%d,%d", &p.tpg, &p.gpw, &p.mp);
  p.splits = (int)((G + 4 * p.gpw - 1) / (4 * p.gpw));
#endif
  if (p.splits > 1) p.ws = (size_t)p.splits * (size_t)m * (size_t)w->n * sizeof(float);
  return p;
}

hipError_t launch_w4a16(const void* x, int xdt, int64_t m, const wq_weight* w,
                        const float* levels16, void* y, int ydt, void* ws, const W4Plan& plan,
                        hipStream_t s) {
  if (xdt == WQ_BF16) return launch_x<WQ_BF16>(x, m, w, levels16, y, ydt, ws, plan, s);
  return launch_x<WQ_F16>(x, m, w, levels16, y, ydt, ws, plan, s);
}

}  // namespace wq
