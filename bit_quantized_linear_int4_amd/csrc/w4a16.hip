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

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima, i.e. no wait).
template <int N>
__device__ __forceinline__ void vm_wait() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Full-K decode kernel.  Workgroup b owns row tiles b, b + gridDim.x, ...
// (TPG of them) over the whole K range, so no partial sums leave the
// workgroup.  The activations (MP rows, m padded) stream into LDS by direct
// global->LDS loads in phases of CG = NW*GPP groups (NBUF buffers); in each
// phase every wave multiplies GPP groups of each of its tiles.  All weight
// loads are issued up front (one round), after the first activation phases,
// so the weights stream from HBM while the multiply consumes them in order.
// The NW waves' sums are added in LDS in a fixed order at the end.
template <int XDT, int YDT, int FMT, int NW, int TPG, int GPP, int MP, int PMAX, int NBUF>
__global__ __launch_bounds__(NW * 64) void decode_kernel(SkinnyArgs a, Levels lv, int phases) {
  constexpr int NT = NW * 64;
  constexpr int CG = NW * GPP;                   // groups per phase
  constexpr int PCH = CG * 16 * MP;              // 16-byte chunks per phase buffer
  constexpr int XL = (PCH + NT - 1) / NT;        // direct loads per thread per phase
  constexpr bool FAST = (FMT == WQ_FMT_INT4_ASYM) && (XDT == WQ_F16);
  constexpr int RED = NW * TPG * 4 * kWave;      // floats for the final reduction
  constexpr int SM16 = (NBUF * PCH > RED / 4) ? NBUF * PCH : RED / 4;
  static_assert(PCH % NT == 0, "every wave issues the same number of direct loads");
  __shared__ uint4_t xs[SM16];
  __shared__ float lut[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, kq = lane >> 4;
  const int ntiles = (a.n + 15) / 16;

  // direct loads of phase p's activation chunk into buffer p % NBUF; layout
  // [group in phase][16-byte chunk c16][row m]; chunks outside x are loaded
  // from a clamped address and masked when read
  auto issue_x = [&](int p) {
    uint4_t* buf = xs + (p % NBUF) * PCH;
#pragma unroll
    for (int r = 0; r < XL; ++r) {
      const int base = r * NT + wave * 64;       // wave-uniform
      if (base < PCH) {
        const int c = base + lane;
        const int gi = c / (16 * MP), c16 = (c / MP) % 16, m = c % MP;
        const int g = min(p * CG + gi, a.G - 1), mm = min(m, a.m - 1);
        const uint16_t* src = a.x + (int64_t)mm * a.k + g * 128 + c16 * 8;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(buf + base), 16, 0, 0);
      }
    }
  };
  issue_x(0);
  if (NBUF > 1 && phases > 1) issue_x(1);

  // all weight loads of this wave: PMAX*TPG*GPP units, three loads each,
  // unconditional (clamped addresses) so the count is known at compile time
  const uint4_t* q4 = reinterpret_cast<const uint4_t*>(a.codes);
  const int k32 = a.k / 32;
  const bool dq = a.scales2 != nullptr;
  const float* s2p = dq ? a.scales2 : static_cast<const float*>(a.scales);
  uint4_t wv[PMAX][TPG][GPP];
  float sv[PMAX][TPG][GPP];
  uint32_t zv[PMAX][TPG][GPP];
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
#pragma unroll
    for (int t = 0; t < TPG; ++t) {
      const int tile = min((int)blockIdx.x + t * (int)gridDim.x, ntiles - 1);
      const int row = min(tile * 16 + nl, a.n - 1);
#pragma unroll
      for (int u = 0; u < GPP; ++u) {
        const int g = min(p * CG + wave * GPP + u, a.G - 1);
        wv[p][t][u] = q4[(int64_t)row * k32 + g * 4 + kq];
        if constexpr (FMT == WQ_FMT_INT4_ASYM) {
          sv[p][t][u] = f16_bits_to_f32(static_cast<const uint16_t*>(a.scales)[(int64_t)row * a.G + g]);
          zv[p][t][u] = a.zeros[(int64_t)row * a.zb + (g >> 1)];
        } else {
          // exactly two loads on either path: the first-level absmax (int8
          // code or fp32) and the second-level scale (unused without double
          // quantization)
          const int64_t blk = (int64_t)row * (a.k / 64) + 2 * g + (kq >> 1);
          const float l2 = s2p[dq ? (blk >> 8) : 0];
          const float l1 = dq ? (float)static_cast<const int8_t*>(a.scales)[blk]
                              : static_cast<const float*>(a.scales)[blk];
          sv[p][t][u] = dq ? l1 * l2 : l1;
          zv[p][t][u] = 0;
        }
      }
    }
  }
  if (FMT == WQ_FMT_NF4 && tid < 16) lut[tid] = lv.v[tid];

  constexpr uint32_t kOne = 0x3C003C00u;
  const uint4_t ones = {kOne, kOne, kOne, kOne};
  const int mrow = min(nl, MP - 1);
  float4_t acc[TPG];
#pragma unroll
  for (int t = 0; t < TPG; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
    if (p < phases) {
      // this wave's direct loads for phase p have landed: everything issued
      // after them may still be in flight (the next phase's activation
      // loads and, for the first phases, the weight loads)
      constexpr int WLOADS = PMAX * TPG * GPP * 3;
      if (p == 0) {
        if (NBUF > 1 && phases > 1) vm_wait<XL + WLOADS>(); else vm_wait<WLOADS>();
      } else if (p == 1 && NBUF > 1) {
        vm_wait<WLOADS>();
      } else {
        if (NBUF > 1 && p + 1 < phases) vm_wait<XL>(); else vm_wait<0>();
      }
      __syncthreads();  // ... and so have every other wave's
      const uint4_t* buf = xs + (p % NBUF) * PCH;
#pragma unroll
      for (int u = 0; u < GPP; ++u) {
        const int gi = wave * GPP + u;
        const int g = p * CG + gi;
        const bool live = nl < a.m && g < a.G;
        uint4_t A[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4_t v = buf[(gi * 16 + kq * 4 + j) * MP + mrow];
          A[j] = live ? (FAST ? perm_x(v) : v) : uint4_t{0u, 0u, 0u, 0u};
        }
        if constexpr (FAST) {
          float4_t X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) X = mfma16<XDT>(A[j], ones, X);
#pragma unroll
          for (int t = 0; t < TPG; ++t) {
            float4_t tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) tmp = mfma16<XDT>(A[j], unpack_biased_f16(wv[p][t][u][j]), tmp);
            const uint32_t z = (g & 1) ? (zv[p][t][u] >> 4) : (zv[p][t][u] & 15u);
            const float zb = 1024.0f + (float)z;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(fmaf(-zb, X[e], tmp[e]), sv[p][t][u], acc[t][e]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < TPG; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              uint4_t b;
              if constexpr (FMT == WQ_FMT_INT4_ASYM) {
                const float z = (float)((g & 1) ? (zv[p][t][u] >> 4) : (zv[p][t][u] & 15u));
                b = dequant_int4_word<XDT>(wv[p][t][u][j], z, sv[p][t][u]);
              } else {
                b = dequant_nf4_word<XDT>(wv[p][t][u][j], lut, sv[p][t][u]);
              }
              acc[t] = mfma16<XDT>(A[j], b, acc[t]);
            }
          }
        }
      }
      if (p + NBUF < phases) {
        __syncthreads();  // everyone is done with this buffer
        issue_x(p + NBUF);
      }
    }
  }
  // fixed-order sum of the NW waves' partial results
  __syncthreads();
  float* red = reinterpret_cast<float*>(xs);
#pragma unroll
  for (int t = 0; t < TPG; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * TPG + t) * 4 + e) * kWave + lane] = acc[t][e];
  __syncthreads();
  constexpr int NV = TPG * 4 * kWave;
  for (int i = tid; i < NV; i += NT) {
    const int te = i / kWave, l = i % kWave, t = te / 4, e = te % 4;
    const int mm = (l >> 4) * 4 + e;
    const int tile = (int)blockIdx.x + t * (int)gridDim.x;
    const int nn = tile * 16 + (l & 15);
    if (mm < a.m && tile < ntiles && nn < a.n) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[i + w * NV];
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

// Full-K decode configurations: NW, TPG, GPP, MP, PMAX, NBUF.
//  cfg 0..2   m == 1,  K <= 4096:  4 waves, 8 groups/wave, 1 phase, TPG 1/2
//  cfg 3..4   m <= 4,  K <= 4096
//  cfg 5..7   m <= 16, K <= 4096:  8 waves, 4 groups/wave, x fully in LDS
//  cfg 8      m <= 16, K <= 12288: 8 waves, 2 groups/wave, 6 double-buffered phases
//  cfg 9..10  m <= 4,  K <= 12288: 4 waves, 8 groups/wave, 3 phases
template <int XDT, int YDT, int FMT>
bool launch_decode(const SkinnyArgs& a, const Levels& lv, const W4Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.grid);
#define WQ_DEC(C, NW, TPG, GPP, MP, PMAX, NBUF)                                            \
  case C:                                                                                  \
    decode_kernel<XDT, YDT, FMT, NW, TPG, GPP, MP, PMAX, NBUF><<<grid, NW * 64, 0, s>>>(  \
        a, lv, p.phases);                                                                  \
    return true;
  switch (p.cfg) {
    WQ_DEC(0, 4, 1, 8, 1, 1, 1)
    WQ_DEC(1, 4, 2, 8, 1, 1, 1)
    WQ_DEC(2, 4, 4, 4, 1, 2, 1)
    WQ_DEC(3, 4, 1, 8, 4, 1, 1)
    WQ_DEC(4, 4, 2, 8, 4, 1, 1)
    WQ_DEC(5, 8, 1, 4, 16, 1, 1)
    WQ_DEC(6, 8, 2, 4, 16, 1, 1)
    WQ_DEC(7, 8, 3, 4, 16, 1, 1)
    WQ_DEC(8, 8, 1, 2, 16, 6, 2)
    WQ_DEC(9, 4, 1, 8, 1, 3, 1)
    WQ_DEC(10, 4, 1, 8, 4, 3, 1)
    default: return false;
  }
#undef WQ_DEC
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
  if (p.path == 2) {
    const bool ok = w->fmt == WQ_FMT_NF4 ? launch_decode<XDT, YDT, WQ_FMT_NF4>(a, lv, p, s)
                                         : launch_decode<XDT, YDT, WQ_FMT_INT4_ASYM>(a, lv, p, s);
    return ok ? hipGetLastError() : hipErrorInvalidConfiguration;
  }
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
  p.path = m > 16 ? 1 : 2;
  p.tpg = 1;
  p.gpw = 8;
  p.mp = 1;
  p.splits = 1;
  p.cfg = 0;
  p.phases = 1;
  p.grid = 0;
  p.ws = 0;
  if (p.path == 1) return p;
  const int64_t G = w->k / 128;
  const int64_t ntiles = (w->n + 15) / 16;
  p.mp = m <= 1 ? 1 : (m <= 4 ? 4 : 16);
  // full-K kernel: one workgroup per CU-share of row tiles, no partial sums
  struct Cfg { int id, tpg, cg, mp, pmax; };
  static const Cfg cfgs[] = {
      {0, 1, 32, 1, 1}, {1, 2, 32, 1, 1}, {2, 4, 16, 1, 2}, {3, 1, 32, 4, 1}, {4, 2, 32, 4, 1},
      {5, 1, 32, 16, 1}, {6, 2, 32, 16, 1}, {7, 3, 32, 16, 1}, {8, 1, 16, 16, 6},
      {9, 1, 32, 1, 3}, {10, 1, 32, 4, 3}};
  int best = -1;
  int64_t best_grid = 0;
  for (const Cfg& c : cfgs) {
    if (c.mp != p.mp) continue;
    const int64_t phases = (G + c.cg - 1) / c.cg;
    if (phases > c.pmax) continue;
    const int64_t grid = (ntiles + c.tpg - 1) / c.tpg;
    // prefer the fewest phases slots that fit, then about one workgroup per
    // CU for the 16-row configurations (128 KB of LDS each)
    const bool fits_round = c.mp == 16 ? grid <= 256 : grid <= 1024;
    if (best < 0 || (fits_round && !(best_grid <= (p.mp == 16 ? 256 : 1024))) ||
        (fits_round == (best_grid <= (p.mp == 16 ? 256 : 1024)) && c.pmax < cfgs[best].pmax)) {
      best = (int)(&c - cfgs);
      best_grid = grid;
    }
  }
  auto split_k = [&]() {
    p.path = 0;
    p.gpw = 4;
    p.splits = (int)((G + 15) / 16);
    const int64_t tpg = (ntiles * p.splits + 511) / 512;
    p.tpg = (int)std::max<int64_t>(1, std::min<int64_t>(4, tpg));
    if (p.mp <= 4) p.tpg = 1;
  };
  if (best >= 0) {
    const Cfg& c = cfgs[best];
    p.cfg = c.id;
    p.tpg = c.tpg;
    p.phases = (int)((G + c.cg - 1) / c.cg);
    p.grid = (int)((ntiles + c.tpg - 1) / c.tpg);
  } else {
    split_k();  // K beyond the full-K configurations
  }
#ifdef WQ_TUNE_ENV
  if (const char* e = getenv("WQ_DECODE")) {
    int cfg = -2;
    if (sscanf(e, "%d", &cfg) == 1 && cfg == -1) split_k();
    if (cfg >= 0) {
      for (const Cfg& c : cfgs)
        if (c.id == cfg) {
          p.path = 2;
          p.cfg = c.id;
          p.tpg = c.tpg;
          p.phases = (int)((G + c.cg - 1) / c.cg);
          p.grid = (int)((ntiles + c.tpg - 1) / c.tpg);
        }
    }
  }
#endif
  if (p.path == 0 && p.splits > 1)
    p.ws = (size_t)p.splits * (size_t)m * (size_t)w->n * sizeof(float);
  return p;
}

hipError_t launch_w4a16(const void* x, int xdt, int64_t m, const wq_weight* w,
                        const float* levels16, void* y, int ydt, void* ws, const W4Plan& plan,
                        hipStream_t s) {
  if (xdt == WQ_BF16) return launch_x<WQ_BF16>(x, m, w, levels16, y, ydt, ws, plan, s);
  return launch_x<WQ_F16>(x, m, w, levels16, y, ydt, ws, plan, s);
}

}  // namespace wq
