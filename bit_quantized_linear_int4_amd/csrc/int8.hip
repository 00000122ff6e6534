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
//   int8_colmask    per column: any |x| > threshold over the rows -> mask
//   int8_quant_act  one workgroup per token: absmax over the non-outlier
//                   columns -> sx, codes (0 in outlier columns); one more
//                   workgroup compacts the mask into the ascending outlier
//                   list and its count (no host round trip; the count stays
//                   on the device)
//   int8_gemm       256 x BN output tiles: v_mfma_i32_16x16x64_i8 over K, then
//                   y = acc * sx * sw, then the outlier columns through
//                   v_mfma_f32_16x16x32_f16 on fp16 activations and the int8
//                   weights dequantized to fp16, accumulated into the same
//                   registers.
#include <algorithm>

#include "internal.h"

namespace wq {
namespace {

// Column mask: workgroup b covers columns 64b .. 64b+63 over every row; a
// thread reads 8 columns (16 bytes) of rows tid/8, tid/8 + 32, ..., and the
// 32 row groups' flags are OR-ed in LDS before the mask bytes are written.
__global__ __launch_bounds__(256) void int8_colmask_kernel(const uint16_t* __restrict__ x,
                                                           int64_t m, int64_t k, float thr,
                                                           uint8_t* __restrict__ mask) {
  __shared__ uint32_t part[32][8];
  const int t = threadIdx.x, cc = t & 7, rg = t >> 3;
  const int64_t c0 = (int64_t)blockIdx.x * 64 + cc * 8;
  uint32_t f = 0;   // bit i: column c0 + i
  if (c0 < k) {
#pragma unroll 8
    for (int64_t r = rg; r < m; r += 32) {
      const uint4_t v = *reinterpret_cast<const uint4_t*>(x + r * k + c0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t h = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
        if (fabsf(f16_bits_to_f32(h)) > thr) f |= 1u << i;
      }
    }
  }
  part[rg][cc] = f;
  __syncthreads();
  if (t < 64 && (int64_t)blockIdx.x * 64 + t < k) {
    uint32_t o = 0;
#pragma unroll
    for (int g = 0; g < 32; ++g) o |= part[g][t >> 3];
    mask[(int64_t)blockIdx.x * 64 + t] = (uint8_t)((o >> (t & 7)) & 1u);
  }
}

// Ascending list of the flagged columns and their count, by one workgroup
// of 256 threads (no host round trip; the count stays on the device).  The
// mask bytes are 0 or 1; each thread reads a contiguous run of 16-byte
// chunks (k % 16 == 0, mask 16-byte aligned), counts them with popcounts,
// and an exclusive scan of the counts gives its first output position.
__device__ void compact_mask(const uint8_t* __restrict__ mask, int64_t k,
                             int32_t* __restrict__ idx, int32_t* __restrict__ count,
                             int32_t* part) {
  const int t = threadIdx.x;
  const int64_t chunks = k / 16, per = (chunks + 255) / 256;
  const int64_t c0 = std::min<int64_t>(chunks, t * per), c1 = std::min<int64_t>(chunks, c0 + per);
  const uint4_t* m16 = reinterpret_cast<const uint4_t*>(mask);
  int32_t n = 0;
  for (int64_t c = c0; c < c1; ++c) {
    const uint4_t v = m16[c];
    n += __popc(v[0]) + __popc(v[1]) + __popc(v[2]) + __popc(v[3]);
  }
  part[t] = n;
  __syncthreads();
  // inclusive scan (Hillis-Steele) over 256 partial counts
  for (int off = 1; off < 256; off <<= 1) {
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t pos = part[t] - n;
  for (int64_t c = c0; c < c1; ++c) {
    const uint4_t v = m16[c];
    if ((v[0] | v[1] | v[2] | v[3]) == 0u) continue;
#pragma unroll
    for (int b = 0; b < 16; ++b)
      if ((v[b >> 2] >> (8 * (b & 3))) & 1u) idx[pos++] = (int32_t)(c * 16 + b);
  }
  if (t == 255) *count = part[255];
}

// One workgroup per token row; one more workgroup (the last) compacts the
// mask meanwhile.
__global__ __launch_bounds__(256) void int8_quant_act_kernel(const uint16_t* __restrict__ x,
                                                             int64_t k,
                                                             const uint8_t* __restrict__ mask,
                                                             int8_t* __restrict__ qx,
                                                             float* __restrict__ sx,
                                                             int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ count) {
  __shared__ float red[4];
  __shared__ int32_t part[256];
  if (blockIdx.x == gridDim.x - 1) {
    compact_mask(mask, k, idx, count, part);
    return;
  }
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
// Workgroup tile 256 (m) x BN = 16*NT (n) with NT = 7 or 8; four waves, wave
// w owning rows 64w .. 64w+63 of the tile and all BN columns (4 x NT MFMA
// tiles of 16x16).  K advances 128 bytes per step (two K extents of
// v_mfma_i32_16x16x64_i8).  Weight rows are in exactly one tile for m <= 256,
// so the int8 weights stream from HBM once; the activation codes (at most a
// few MB) are re-read from L2 by every tile.
//
//  * Every load lands in registers (global_load_dwordx4), so the compiler
//    counts every load in its own waits.  (The direct global->LDS version
//    of this kernel took 125 us on the 70B layer, this one 94-108 us.)
//  * A wave's activation rows are its own: they are loaded straight into
//    the MFMA A-operand registers, two steps ahead (RA = 2 register stages).
//  * The weight slice of a step is shared by the four waves: each thread
//    loads 4 x 16 bytes of it RB = 4 steps ahead, writes them into one of two
//    LDS buffers a step before they are multiplied, and one barrier per step
//    publishes that buffer and proves the other one free.
//  * 16-byte chunk c of weight row r sits at slot c ^ swz(r) of the row's
//    eight, so the 16 rows an operand read touches fall in distinct LDS banks
//    (for both 128- and 256-byte bank rows).
//  * Epilogue: y = acc * sx[m] * sw[n] in fp32, then the outlier columns in
//    chunks of 32 through v_mfma_f32_16x16x32_f16 on the fp16 activations and
//    the int8 weights dequantized to fp16, added into the same registers.
constexpr int kI8BM = 256, kI8BK = 128;
constexpr int kI8WS = 128 * kI8BK / 16;      // 16-byte slots per weight buffer (up to 128 rows)

__device__ __forceinline__ int i8_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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
  constexpr int RA = 2, RB = 4;                 // register stages: activations, weights
  static_assert(NT == 7 || NT == 8, "tile widths 112 and 128");
  __shared__ uint4_t wsl[2 * kI8WS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, kc = lane >> 4;
  const int m0 = (int)blockIdx.y * kI8BM, n0 = (int)blockIdx.x * BN;
  const int nk = a.k / kI8BK;

  // activation rows of this lane's A operands (rows past m read row m - 1,
  // never stored): operand (kk, i) = 16 bytes of row wave*64 + i*16 + nl at
  // byte kk*64 + kc*16 of the step
  const int8_t* xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    xrow[i] = a.qx + (int64_t)min(m0 + wave * 64 + i * 16 + nl, a.m - 1) * a.k + kc * 16;
  // weight slots of this thread: slot tid + 256u = row r, chunk c; rows past
  // BN (NT = 7: waves 2 and 3 for u = 3) are not loaded, rows past n read the
  // tile's last valid row
  const int8_t* wsrc[4];
  int wdst[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int sl = tid + 256 * u, r = sl >> 3, c = sl & 7;
    wsrc[u] = a.qw + (int64_t)(n0 + min(r, a.n - 1 - n0)) * a.k + c * 16;
    wdst[u] = r * 8 + (c ^ i8_swz(r));
  }
  // K order: every workgroup starts at its own step and wraps around, so at
  // any moment the workgroups of an XCD (every 8th one) read lines at many
  // different K offsets, spread over the L2 channels, instead of the same
  // offset of rows a power of two apart (int32 sums do not depend on the
  // order)
  const unsigned bid = blockIdx.x;
  const int kstart = (int)(((bid >> 3) * 5u + (bid & 7u) * 3u + blockIdx.y * 7u) % (unsigned)nk);
  auto koff = [&](int g) {
    int gk = min(g, nk - 1) + kstart;
    gk -= gk >= nk ? nk : 0;
    return gk * kI8BK;
  };
  auto wload = [&](uint4_t (&wr)[4], int g) {
    const int off = koff(g);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < 3 || BN == 128 || wave < (BN * 8 - 768) / 64)
        wr[u] = *reinterpret_cast<const uint4_t*>(wsrc[u] + off);
  };
  auto wstore = [&](const uint4_t (&wr)[4], int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < 3 || BN == 128 || wave < (BN * 8 - 768) / 64) wsl[buf * kI8WS + wdst[u]] = wr[u];
  };
  auto aload = [&](uint4_t (&ar)[2][4], int g) {
    const int off = koff(g);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ar[kk][i] = *reinterpret_cast<const uint4_t*>(xrow[i] + off + kk * 64);
  };

  int4_t acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = int4_t{0, 0, 0, 0};

  uint4_t wr[RB][4];
  uint4_t ar[RA][2][4];
#pragma unroll
  for (int b = 0; b < RB; ++b) wload(wr[b], b);
#pragma unroll
  for (int b = 0; b < RA; ++b) aload(ar[b], b);
  wstore(wr[0], 0);
  wload(wr[0], RB);
  lgkm_wait0();
  wg_barrier();

  // step g (U = g % 4): weights of step g are in LDS buffer g & 1, those of
  // step g + 1 in registers wr[(g + 1) % RB], activations in ar[g % RA]
  auto step = [&](int g, auto uc) {
    constexpr int U = decltype(uc)::value;
    constexpr int WB = (U + 1) % RB;
    wstore(wr[WB], (U + 1) & 1);   // step g + 1 (past the end: never read)
    wload(wr[WB], g + 1 + RB);
    const uint4_t* wc = wsl + (U & 1) * kI8WS;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + kc;
      uint4_t bf[NT];   // all reads first: one LDS latency per half step
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int r = j * 16 + nl;
        bf[j] = wc[r * 8 + (c ^ i8_swz(r))];
      }
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mfma_i8(ar[U % RA][kk][i], bf[j], acc[i][j]);
    }
    aload(ar[U % RA], g + RA);
    lgkm_wait0();   // this wave's LDS writes of step g + 1 ...
    wg_barrier();   // ... and every wave's; every wave is done with buffer g & 1
  };
  // groups of four steps with no branch between them, so the compiler's
  // load counting stays exact across the loop; then the last 0-3 steps
  int g0 = 0;
  for (; g0 + 4 <= nk; g0 += 4) {
    step(g0, std::integral_constant<int, 0>{});
    step(g0 + 1, std::integral_constant<int, 1>{});
    step(g0 + 2, std::integral_constant<int, 2>{});
    step(g0 + 3, std::integral_constant<int, 3>{});
  }
  if (g0 < nk) step(g0, std::integral_constant<int, 0>{});
  if (g0 + 1 < nk) step(g0 + 1, std::integral_constant<int, 1>{});
  if (g0 + 2 < nk) step(g0 + 2, std::integral_constant<int, 2>{});

  // ---- epilogue: raw accumulators (optional), rescale, outlier slice
  float4_t yf[4][NT];
  float swv[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int nn = n0 + j * 16 + nl;
    swv[j] = nn < a.n ? a.sw[nn] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int mm = m0 + wave * 64 + i * 16 + kc * 4 + e;
      const float sxv = mm < a.m ? a.sx[mm] : 0.0f;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int nn = n0 + j * 16 + nl;
        if (a.acc_out != nullptr && mm < a.m && nn < a.n)
          a.acc_out[(int64_t)mm * a.n + nn] = acc[i][j][e];
        yf[i][j][e] = ((float)acc[i][j][e] * sxv) * swv[j];
      }
    }
  }

  const int cnt = *a.count;
  static_assert((kI8BM + 128) * 40 * 2 <= 2 * kI8WS * 16, "outlier staging fits");
  uint16_t* Xo = reinterpret_cast<uint16_t*>(wsl);              // [256][40] fp16
  uint16_t* Wo = reinterpret_cast<uint16_t*>(wsl) + kI8BM * 40;  // [BN][40] fp16
  __shared__ int32_t sidx[32];
  for (int c0 = 0; c0 < cnt; c0 += 32) {
    // the chunk's column indices once (-1 past the count); then every gather
    // load of a thread is issued before any is used, so the chunk costs one
    // memory latency rather than one per element
    if (tid < 32) sidx[tid] = c0 + tid < cnt ? a.idx[c0 + tid] : -1;
    __syncthreads();
    {
      // activations: thread t gathers row t of the tile, 32 columns
      const bool rv = m0 + tid < a.m;
      const uint16_t* xr = a.x + (int64_t)min(m0 + tid, a.m - 1) * a.k;
      uint32_t v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int c = sidx[j];
        v[j] = (rv && c >= 0) ? (uint32_t)xr[c] : 0u;
      }
#pragma unroll
      for (int j = 0; j < 32; j += 2)
        *reinterpret_cast<uint32_t*>(&Xo[tid * 40 + j]) = v[j] | (v[j + 1] << 16);
    }
    if (tid < 2 * BN) {
      // weights: thread t gathers 16 columns (half t & 1) of row t >> 1,
      // dequantized to fp16 as fp16(fp32(q) * sw)
      const int r = tid >> 1, h = (tid & 1) * 16;
      const bool rv = n0 + r < a.n;
      const int nr = min(n0 + r, a.n - 1);
      const int8_t* wrow = a.qw + (int64_t)nr * a.k;
      const float sc = a.sw[nr];
      float q[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = sidx[h + j];
        q[j] = (rv && c >= 0) ? (float)wrow[c] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const uint32_t lo = f32_to_f16_bits(as_f32(q[j] * sc));
        const uint32_t hi = f32_to_f16_bits(as_f32(q[j + 1] * sc));
        *reinterpret_cast<uint32_t*>(&Wo[r * 40 + h + j]) = lo | (hi << 16);
      }
    }
    __syncthreads();
    uint4_t ao[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ao[i] = *reinterpret_cast<const uint4_t*>(&Xo[(wave * 64 + i * 16 + nl) * 40 + kc * 8]);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint4_t bo = *reinterpret_cast<const uint4_t*>(&Wo[(j * 16 + nl) * 40 + kc * 8]);
#pragma unroll
      for (int i = 0; i < 4; ++i) yf[i][j] = mfma_f16(ao[i], bo, yf[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int mm = m0 + wave * 64 + i * 16 + kc * 4 + e;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int nn = n0 + j * 16 + nl;
        if (mm < a.m && nn < a.n) {
          const int64_t o = (int64_t)mm * a.n + nn;
          if constexpr (YDT == WQ_F32)
            static_cast<float*>(a.y)[o] = yf[i][j][e];
          else if constexpr (YDT == WQ_BF16)
            static_cast<uint16_t*>(a.y)[o] = f32_to_bf16_bits(yf[i][j][e]);
          else
            static_cast<uint16_t*>(a.y)[o] = f32_to_f16_bits(yf[i][j][e]);
        }
      }
    }
}

template <int NT>
hipError_t launch_int8_gemm_nt(const Int8GemmArgs& a, int ydt, hipStream_t s) {
  const dim3 grid((unsigned)((a.n + NT * 16 - 1) / (NT * 16)), (unsigned)((a.m + kI8BM - 1) / kI8BM));
  if (ydt == WQ_F32)
    int8_gemm_kernel<NT, WQ_F32><<<grid, 256, 0, s>>>(a);
  else if (ydt == WQ_BF16)
    int8_gemm_kernel<NT, WQ_BF16><<<grid, 256, 0, s>>>(a);
  else
    int8_gemm_kernel<NT, WQ_F16><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_int8_prepare(const uint16_t* x, int64_t m, int64_t k, float thr,
                               uint8_t* mask, int32_t* idx, int32_t* count, int8_t* qx,
                               float* sx, hipStream_t s) {
  int8_colmask_kernel<<<dim3((unsigned)((k + 63) / 64)), 256, 0, s>>>(x, m, k, thr, mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int8_quant_act_kernel<<<dim3((unsigned)(m + 1)), 256, 0, s>>>(x, k, mask, qx, sx, idx, count);
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
  // tile width 112 or 128: the one with less work per CU over the rounds of
  // 256 workgroups (one per CU) the grid takes; ties go to 112 (more CUs)
  const int64_t ntm = (m + kI8BM - 1) / kI8BM;
  auto rounds = [&](int64_t bn) { return ((w->n + bn - 1) / bn * ntm + 255) / 256; };
  if (rounds(112) * 7 <= rounds(128) * 8) return launch_int8_gemm_nt<7>(a, ydt, s);
  return launch_int8_gemm_nt<8>(a, ydt, s);
}

}  // namespace wq
