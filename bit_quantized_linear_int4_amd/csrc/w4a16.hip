// W4A16 linear: y = x . w_hat^T with 4-bit weights dequantized to 16 bits
// inside the kernel ("LLM quantization selection: five mainstream schemes
// compared", section 5 opening: W4A16 dequantizes the weights back to FP16 and
// multiplies in FP16; section 4.3: a GEMV version for single requests and a
// GEMM version for batches).
//
// Two kernel families:
//
//  * stream (m <= 16, decode).  HBM-bound: the packed codes are streamed
//    once with 16-byte loads, 16 rows x 64 bytes per wave instruction (8
//    rows x 128 bytes, whole lines, where a wave takes groups in pairs).  The
//    multiply runs on the matrix cores (v_mfma_f32_16x16x32_{f16,bf16}) with
//    the activations (m padded to 1, 4 or 16 staged rows) as the A operand
//    and the codes as the B operand, so no cross-lane reduction is needed
//    inside a wave.  Each wave walks K in phases and keeps several phases of
//    loads in flight (a software pipeline per wave, no barriers), so the
//    multiply of a phase overlaps the loads of the next ones.  The waves'
//    partial sums are added in LDS in a fixed order: results are
//    deterministic and no partial sums leave the workgroup.
//
//    INT4 codes become 16-bit values with the exponent-bias trick: OR-ing a
//    nibble into the mantissa of 1024.0 (fp16) gives exactly 1024 + q.  The
//    MFMA accumulates sum_k x_k (1024 + q_k) over a group, and the zero
//    point and bias are removed afterwards with the group's activation sum
//    X = sum_k x_k (itself an MFMA against a ones operand):
//    sum_k x_k (q_k - z) s = s * (acc - (1024 + z) X).  The nibble
//    extraction yields (q0,q4),(q1,q5),(q2,q6),(q3,q7) pairs; the
//    activations are permuted the same way (the dot product does not care
//    about the order of k inside one MFMA).  With bf16 activations the codes
//    are dequantized exactly, (q - z) * s rounded once to bf16.
//
//    With INT4 groups of 64 or 32 a unit of 128 holds several groups, which
//    one MFMA would mix; those weights are dequantized exactly in the B
//    operand instead ((1024 + q) - (1024 + z), times s, one fp16 rounding).
//
//    NF4 and FP4 codes are looked up in the 16-level table (LDS), multiplied
//    by the block's absmax and rounded to the activation type, exactly as
//    the dequantization defines them.
//
//    A gate/up pair sharing x runs as one launch whose workgroups hold the
//    row tiles of both matrices (the activations are staged once).
//
//  * gemm (m > 16, prefill).  MFMA-bound.  gemm_i4_kernel (INT4, fp16
//    activations, at most 64 groups per row): 128 x 256 workgroup tiles,
//    8 waves of 128 x 32, activations and codes reach LDS by direct loads
//    a step or two ahead, every code is dequantized exactly in registers by
//    the wave that multiplies it, tiles ordered per XCD.  gemm_kernel
//    (everything else): 128 x 128 tiles, the weight tile dequantized once
//    into LDS in the activation type, four waves of 64 x 64.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

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

// Two fp32 values -> two 16-bit values of the activation type in one word
// (low half = v0), each rounded to nearest even once (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32).
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <int XDT>
__device__ __forceinline__ uint32_t pack2_x(float v0, float v1) {
  const float2_t v = {v0, v1};
  uint32_t u;
  if constexpr (XDT == WQ_BF16) {
    const bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
    __builtin_memcpy(&u, &b, 4);
  } else {
    const half2_t h = __builtin_convertvector(v, half2_t);
    __builtin_memcpy(&u, &h, 4);
  }
  return u;
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
  int m, n, k, G, zb;        // G = k/128 units of 128; zb = bytes per row of zeros
  int GS, sub;               // INT4: groups per row (k/group), groups per unit (1, 2, 4)
  void* y;
  // second matrix of a gate/up pair (same format, n, k; same x), its
  // output, and the epilogue: 0 = both outputs, 1 = y = silu(gate) * up only
  const uint32_t* codes_b;
  const void* scales_b;
  const uint8_t* zeros_b;
  const float* scales2_b;
  void* y_b;
  int act;
};

struct Levels {
  float v[16];
};

// Per-tile metadata staged in LDS by the decode kernel (SZL), in bytes.
// INT4: the 16 rows' fp16 scales (a) and zero-point bytes (b), each rounded
// up to the 1 KB direct loads that bring them in.  NF4 with double-quantized
// absmax: the int8 absmax codes of the 16 rows' blocks (a: 16 * k/64
// contiguous bytes, 1 KB loads) and the fp32 second-level scales that cover
// them (b: at most 16 * k/64 / 256 + 2 values, plain loads).
__host__ __device__ inline int staged_a_bytes(int fmt, int GS, int k) {
  return fmt == WQ_FMT_NF4 ? (16 * (k / 64) + 1023) / 1024 * 1024 : (32 * GS + 1023) / 1024 * 1024;
}
__host__ __device__ inline int staged_c2_count(int k) { return 16 * (k / 64) / 256 + 2; }
__host__ __device__ inline int staged_b_bytes(int fmt, int zb, int k) {
  return fmt == WQ_FMT_NF4 ? (staged_c2_count(k) * 4 + 15) / 16 * 16 : (16 * zb + 1023) / 1024 * 1024;
}

// c in a VGPR, opaque to the optimizer (the empty asm emits nothing).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t c) {
  asm("" : "+v"(c));
  return c;
}

// (a & m) | o as one v_and_or_b32 / v_bitop3_b32: with m and o opaque VGPR
// values the compiler cannot split it into two literal-operand instructions.
// Plain C rather than inline asm on purpose: an MFMA that reads a VGPR needs
// two wait states after the VALU instruction that wrote it, and the compiler
// inserts them only for instructions it emitted itself, so an asm def
// feeding an MFMA operand can be read stale.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  return (a & in_vgpr(m)) | in_vgpr(o);
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
// Each pair of weights is rounded into the activation type by one
// v_cvt_pk_{bf16,f16}_f32.
template <int XDT>
__device__ __forceinline__ uint4_t dequant_int4_word(uint32_t w, float z, float s) {
  uint4_t b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float q0 = (float)((w >> (8 * e)) & 15u);
    const float q1 = (float)((w >> (8 * e + 4)) & 15u);
    // (q - z) * s is exact in fp32
    b[e] = pack2_x<XDT>((q0 - z) * s, (q1 - z) * s);
  }
  return b;
}
// lut2[b] = (level of code b & 15, level of code b >> 4): one 8-byte LDS
// read per byte of codes
template <int XDT>
__device__ __forceinline__ uint4_t dequant_nf4_word(uint32_t w, const float2_t* lut2, float ah) {
  uint4_t b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float2_t l = lut2[(w >> (8 * e)) & 255u];
    b[e] = pack2_x<XDT>(as_f32(l.x * ah), as_f32(l.y * ah));
  }
  return b;
}

// s_waitcnt vmcnt(n) for a wave-uniform count known only at run time, by
// binary search over the immediates (counts above the hardware maximum wait
// for that maximum, which waits for more loads than asked: safe).
template <int LO, int HI>
__device__ __forceinline__ void vm_wait_range(int n) {
  if constexpr (LO == HI) {
    vm_wait<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) vm_wait_range<LO, MID>(n); else vm_wait_range<MID + 1, HI>(n);
  }
}
__device__ __forceinline__ void vm_wait_n(int n) { vm_wait_range<0, 63>(n); }

// Streaming decode kernel.  Workgroup b owns row tiles b, b + gridDim.x, ...
// (TPG of them) over the whole K range.  K is walked in phases of
// CG = NW*GPP groups; in phase p wave w owns groups p*CG + w*GPP + [0, GPP)
// for all TPG tiles, so no data is shared between the waves until the final
// sum.  Each wave stages the activations of its own groups (MP rows, padded)
// into a private LDS ring of NBUF phase buffers with direct global->LDS
// loads; the codes of NBUF phases are held in registers (or, with SZL, in a
// second per-wave LDS ring filled the same way).  Loads are issued
// phase by phase (codes, then activations), NBUF phases ahead of the
// multiply, so the multiply of a phase starts as soon as that phase's own
// loads have landed and the loads of later phases keep streaming meanwhile.
//
// SZL (INT4): the workgroup's scales and zero points -- 16 consecutive rows
// of each, contiguous in HBM -- are staged into LDS up front with a few
// 1 KB direct loads instead of two small loads per code load.  It needs
// 16-byte aligned scale and zero buffers whose sizes are multiples of 16.
//
// The 16-byte chunk c16 of activation row m sits in slot c16 ^ (m & 15) of
// the row, so the 16 rows an MFMA operand read touches fall in different LDS
// banks.  LDS is sized at launch (stream_lds_bytes).
// SG (INT4, fp16 activations): groups of 64 or 32, dequantized exactly in the
// B operand; a separate instantiation, so the g128 kernels carry none of its
// registers.
template <int XDT, int YDT, int FMT, int NW, int TPG, int GPP, int MP, int NBUF, bool SZL,
          bool DUAL, bool SG>
__global__ __launch_bounds__(NW * 64) void stream_kernel(SkinnyArgs a, Levels lv, int phases) {
  // DUAL: TPG counts the tiles of both matrices; tile t < TH is row tile t
  // of the first (gate) matrix, tile TH + t the same rows of the second (up)
  constexpr int TH = DUAL ? TPG / 2 : TPG;                 // row tiles per workgroup
  static_assert(!DUAL || TPG % 2 == 0, "a pair holds the same tiles of both matrices");
  // codes through a per-wave LDS ring (with staged scales), else in
  // registers; pairs with 16 staged rows keep them in registers (15.2
  // against 15.8 us through LDS for the 11008-row pair at M = 16, while at
  // M = 1 the ring is faster, 13.1 against 14.1 us; A/B in one run)
  constexpr bool CRING = SZL && (!DUAL || MP == 1);
  // whole-line code loads (codes through the LDS ring, groups taken in
  // pairs): a load covers 8 rows x 128 bytes, two adjacent groups, instead
  // of 16 rows x 64 bytes, so no 128-byte line is split between two loads;
  // lane l of load v
  // of a pair brings chunk (l & 7) ^ lsw(r) of row r = 8 v + (l >> 3), which
  // keeps the 16 rows an operand read gathers in different LDS banks
  // (4096 x 11008 at M = 1: 8.06-8.18 against 8.41-8.46 us, the same bits;
  // at M = 16 with four waves 11.59-11.62 against 11.91-11.94 us for eight
  // waves and one group per phase; A/B in one run, twice each)
  constexpr bool PAIRLD = CRING && GPP % 2 == 0;
  constexpr int CG = NW * GPP;                             // groups per phase
  constexpr int XS = (MP * GPP * 16 + 63) / 64 * 64;       // slots per wave buffer
  // direct activation loads per phase: 1 KB each, or with one staged row
  // (MP = 1) one 256-byte load per group (lane l: 4 bytes at 4 l), so a
  // phase moves the row's 256 bytes instead of a KB of duplicates
  constexpr int XI = MP == 1 ? GPP : XS / 64;
  constexpr int LPU = SZL ? 1 : 3;                         // loads per code unit
  constexpr int WU = TPG * GPP * LPU;                      // code-side loads per phase
  constexpr bool FAST = (FMT == WQ_FMT_INT4_ASYM) && (XDT == WQ_F16);
  extern __shared__ uint4_t dsm[];
  __shared__ float2_t lut2[FMT == WQ_FMT_NF4 ? 256 : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, kq = lane >> 4;
  auto lsw = [](int r) { return (r >> 1) & 7; };   // chunk swizzle of row r (PAIRLD)
  // INT4 group of this lane's codes: lane kq holds quarter kq (32 codes) of
  // each unit of 128, i.e. group unit * sub + lq
  const int lq = (kq * a.sub) >> 2;
  const int ntiles = (a.n + 15) / 16;
  // every workgroup covers the whole K range, units [0, G); units past G
  // (the last phase's padding) load a clamped address and are skipped
  const int nun = a.G;
  auto unit = [&](int g) { return min(g, nun - 1); };
  uint4_t* const ring = dsm + wave * NBUF * XS;
  // staged metadata per tile: SCB and ZCB bytes (INT4 scales and zero
  // points; NF4 absmax codes and second-level scales)
  const int SCB = staged_a_bytes(FMT, a.GS, a.k);
  const int ZCB = staged_b_bytes(FMT, a.zb, a.k);
  const int bpr = a.k / 64;                  // NF4 blocks per row
  const int NC2 = staged_c2_count(a.k);      // NF4 second-level scales per tile
  uint8_t* const scl = reinterpret_cast<uint8_t*>(dsm + NW * NBUF * XS);
  uint8_t* const zcl = scl + TPG * SCB;
  // CRING: the codes also arrive through LDS (per-wave ring, 1 KB per unit:
  // lane l's 16 bytes at slot l), so no load inside the loop lands in a
  // register and the compiler adds no waits of its own
  uint4_t* const wring = reinterpret_cast<uint4_t*>(zcl + TPG * ZCB) + wave * NBUF * TPG * GPP * 64;
  // row tile and matrix of tile t
  auto tile_of = [&](int t) {
    return min((int)blockIdx.x + (t % TH) * (int)gridDim.x, ntiles - 1);
  };
  auto second = [&](int t) { return DUAL && t >= TH; };

  if constexpr (FMT == WQ_FMT_NF4) {
    static_assert(NW * 64 >= 256, "one thread per pair-table entry");
    if (tid < 256) lut2[tid] = float2_t{lv.v[tid & 15], lv.v[tid >> 4]};
    if constexpr (SZL) {
      // the second-level scales of each tile's blocks (indices clamped to
      // the last one), with plain loads before any direct load is issued
      const int64_t n2 = ((int64_t)a.n * bpr + 255) >> 8;
      float* c2l = reinterpret_cast<float*>(zcl);
      for (int i = tid; i < TPG * NC2; i += NW * 64) {
        const int t = i / NC2, j = i % NC2;
        const int64_t c0 = ((int64_t)tile_of(t) * 16 * bpr) >> 8;
        c2l[t * (ZCB / 4) + j] = (second(t) ? a.scales2_b : a.scales2)[min(c0 + j, n2 - 1)];
      }
    }
    __syncthreads();   // before any direct load is in flight: costs no wait
  }
  if constexpr (SZL) {
    // 1 KB direct loads of the tiles' scale and zero rows (NF4: absmax
    // codes), spread over the waves; chunks past the end of a buffer reload
    // its last 16 bytes
    constexpr bool NF = FMT == WQ_FMT_NF4;
    const int nsc = SCB / 1024, nzc = NF ? 0 : ZCB / 1024, per = nsc + nzc;
    const int64_t sbytes = NF ? (int64_t)a.n * bpr : (int64_t)a.n * a.GS * 2;
    const int64_t zbytes = (int64_t)a.n * a.zb;
    for (int i = wave; i < TPG * per; i += NW) {
      const int t = i / per, j = i % per;
      const int tile = tile_of(t);
      const bool isz = j >= nsc;
      const int jj = isz ? j - nsc : j;
      const int64_t off = (int64_t)tile * 16 * (isz ? a.zb : (NF ? bpr : 2 * a.GS)) + jj * 1024 + lane * 16;
      const int64_t lim = (isz ? zbytes : sbytes) - 16;
      const uint8_t* zsrc = second(t) ? a.zeros_b : a.zeros;
      const uint8_t* ssrc = static_cast<const uint8_t*>(second(t) ? a.scales_b : a.scales);
      const uint8_t* src = (isz ? zsrc : ssrc) + min(off, lim);
      uint8_t* dst = (isz ? zcl + t * ZCB : scl + t * SCB) + jj * 1024;
      lds_dma16(src, (lds_void_t*)dst);
    }
    asm volatile("" ::: "memory");
  }

  // activation loads of phase p into ring buffer p % NBUF: lane l of load i
  // fills slot 64*i + l, i.e. row m = slot / (16*GPP), group gl, chunk c16
  // (swizzled); slots past the wave's rows, groups past K and rows past m
  // read clamped addresses and are never used
  auto issue_x = [&](int p) {
    uint4_t* buf = ring + (p % NBUF) * XS;
    if constexpr (MP == 1) {
#pragma unroll
      for (int gl = 0; gl < GPP; ++gl) {
        const int g = unit(p * CG + wave * GPP + gl);
        lds_dma4(a.x + g * 128 + lane * 2, (lds_void_t*)(buf + gl * 16));
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int sl = i * 64 + lane;
      const int m = min(sl / (16 * GPP), MP - 1);
      const int gl = (sl / 16) % GPP;
      const int c16 = (sl % 16) ^ (m & 15);
      const int g = unit(p * CG + wave * GPP + gl);
      const int mm = min(m, a.m - 1);
      lds_dma16(a.x + (int64_t)mm * a.k + g * 128 + c16 * 8, (lds_void_t*)(buf + i * 64));
    }
  };

  const uint4_t* q4a = reinterpret_cast<const uint4_t*>(a.codes);
  const uint4_t* q4b = reinterpret_cast<const uint4_t*>(DUAL ? a.codes_b : a.codes);
  const int k32 = a.k / 32;
  const bool dq = a.scales2 != nullptr;   // both matrices of a pair alike
  uint4_t wv[NBUF][TPG][GPP];
  float sv[NBUF][TPG][GPP];
  uint32_t zv[NBUF][TPG][GPP];
  // code loads of phase p into register slot b (plus, without staged
  // scales, the unit's scale and zero point or NF4 absmax levels)
  auto issue_w = [&](int p, auto bc) {
    constexpr int b = decltype(bc)::value;
#pragma unroll
    for (int t = 0; t < TPG; ++t) {
      const int row = min(tile_of(t) * 16 + nl, a.n - 1);
      const uint4_t* q4 = second(t) ? q4b : q4a;
#pragma unroll
      for (int u = 0; u < GPP; ++u) {
        const int g = unit(p * CG + wave * GPP + u);
        if constexpr (PAIRLD) {
          // groups u and u + 1 (u even): rows 8 v .. 8 v + 7 of the tile, 128
          // bytes each; chunks past the row end reload its last one
          if (u % 2 == 0) {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
              const int r = 8 * v + (lane >> 3);
              const int rw = min(tile_of(t) * 16 + r, a.n - 1);
              const int c = min(g * 4 + ((lane & 7) ^ lsw(r)), k32 - 1);
              lds_void_t* dst = (lds_void_t*)(wring + ((b * TPG + t) * GPP + u + v) * 64);
              if constexpr (MP == 1) lds_dma16_nt(q4 + (int64_t)rw * k32 + c, dst);
              else lds_dma16(q4 + (int64_t)rw * k32 + c, dst);
            }
          }
        } else if constexpr (CRING) {
          // one staged activation row (M = 1): the non-temporal policy for
          // the codes (1.5-2.5% faster on the M = 1 layers, A/B in one run;
          // with 16 rows, where the activations are re-read from L2 far
          // more, 4% slower)
          const uint4_t* src = q4 + (int64_t)row * k32 + g * 4 + kq;
          lds_void_t* dst = (lds_void_t*)(wring + ((b * TPG + t) * GPP + u) * 64);
          if constexpr (MP == 1) lds_dma16_nt(src, dst); else lds_dma16(src, dst);
        } else {
          wv[b][t][u] = q4[(int64_t)row * k32 + g * 4 + kq];
        }
        if constexpr (SZL) {
        } else if constexpr (FMT == WQ_FMT_INT4_ASYM) {
          const uint16_t* sp = static_cast<const uint16_t*>(second(t) ? a.scales_b : a.scales);
          const int gq = g * a.sub + lq;
          sv[b][t][u] = f16_bits_to_f32(sp[(int64_t)row * a.GS + gq]);
          zv[b][t][u] = (second(t) ? a.zeros_b : a.zeros)[(int64_t)row * a.zb + (gq >> 1)];
        } else {
          // the first-level absmax (int8 code or fp32) and the second-level
          // scale (a harmless reload of element 0 without double quantization)
          const int64_t blk = (int64_t)row * (a.k / 64) + 2 * g + (kq >> 1);
          const void* s1p = second(t) ? a.scales_b : a.scales;
          const float* s2p = dq ? (second(t) ? a.scales2_b : a.scales2)
                                : static_cast<const float*>(s1p);
          const float l2 = s2p[dq ? (blk >> 8) : 0];
          const float l1 = dq ? (float)static_cast<const int8_t*>(s1p)[blk]
                              : static_cast<const float*>(s1p)[blk];
          sv[b][t][u] = dq ? l1 * l2 : l1;
          zv[b][t][u] = 0;
        }
      }
    }
  };

  // the loads of one phase.  With codes in registers the activation loads
  // go first: the compiler's own wait before the first use of a phase's
  // code registers counts only register loads, so the loads it forces to
  // complete beyond the explicit wait are the next phase's activation
  // loads (L2 hits), not its code loads.
  auto issue_phase = [&](int p, auto bc) {
    if constexpr (CRING) {
      issue_w(p, bc);
      issue_x(p);
    } else {
      issue_x(p);
      issue_w(p, bc);
    }
  };

  // prologue: phases 0 .. NBUF-1 (always issued; phases past the end load
  // clamped addresses, which keeps the load count fixed)
  [&]<int... B>(std::integer_sequence<int, B...>) {
    (issue_phase(B, std::integral_constant<int, B>{}), ...);
  }(std::make_integer_sequence<int, NBUF>{});
  asm volatile("" ::: "memory");

  constexpr uint32_t kOne = 0x3C003C00u;
  const uint4_t ones = {kOne, kOne, kOne, kOne};
  const int mrow = min(nl, MP - 1);     // rows past m duplicate a staged row; not stored
  float4_t acc[TPG];
#pragma unroll
  for (int t = 0; t < TPG; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  const int issued_max = max(phases, NBUF) - 1;   // last phase whose loads get issued

  auto step = [&](int p, auto bc) {
    constexpr int b = decltype(bc)::value;
    // loads issued after this phase's: those of every later phase issued so
    // far
    const int later = min(p + NBUF - 1, issued_max) - p;
    if (SZL && p == 0) {
      // the staged scale/zero loads precede every phase's loads: once no
      // more than the NBUF phases' loads are outstanding they have landed,
      // and the barrier publishes every wave's share without waiting for
      // any other wave's codes
      vm_wait<NBUF * (XI + WU)>();
      wg_barrier();
    }
    vm_wait_n(later * (XI + WU));
    asm volatile("" ::: "memory");
    const uint4_t* buf = ring + b * XS + mrow * (16 * GPP);
#pragma unroll
    for (int u = 0; u < GPP; ++u) {
      const int gl = p * CG + wave * GPP + u;   // logical unit
      const int gq = unit(gl) * a.sub + lq;     // this lane's INT4 group
      if (gl < nun) {
        if constexpr (SZL) {
#pragma unroll
          for (int t = 0; t < TPG; ++t) {
            if constexpr (PAIRLD) {
              const int cc = (u & 1) * 4 + kq;          // chunk within the pair's 128 bytes
              wv[b][t][u] = wring[((b * TPG + t) * GPP + (u & ~1) + (nl >> 3)) * 64 + (nl & 7) * 8 +
                                  (cc ^ lsw(nl))];
            } else if constexpr (CRING) {
              wv[b][t][u] = wring[((b * TPG + t) * GPP + u) * 64 + lane];
            }
            if constexpr (FMT == WQ_FMT_NF4) {
              // absmax of this lane's block, fp32(q8) * c2 as the double
              // quantization defines it
              const int rb = nl * bpr + 2 * unit(gl) + (kq >> 1);   // block within the tile
              const int64_t tb = (int64_t)tile_of(t) * 16 * bpr;
              const float c2 = reinterpret_cast<const float*>(zcl + t * ZCB)[((tb + rb) >> 8) - (tb >> 8)];
              sv[b][t][u] = (float)reinterpret_cast<const int8_t*>(scl + t * SCB)[rb] * c2;
            } else {
              const uint16_t sc = *reinterpret_cast<const uint16_t*>(scl + t * SCB + (nl * a.GS + gq) * 2);
              sv[b][t][u] = f16_bits_to_f32(sc);
              zv[b][t][u] = zcl[t * ZCB + nl * a.zb + (gq >> 1)];
            }
          }
        }
        uint4_t A[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4_t v = buf[u * 16 + ((kq * 4 + j) ^ (mrow & 15))];
          A[j] = FAST ? perm_x(v) : v;
        }
        if constexpr (FAST) {
          if constexpr (!SG) {
            // one group per unit: the MFMA sums x (1024 + q) over the unit,
            // then s (acc - (1024 + z) X) removes bias and zero point
            float4_t X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) X = mfma16<XDT>(A[j], ones, X);
#pragma unroll
            for (int t = 0; t < TPG; ++t) {
              float4_t tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int j = 0; j < 4; ++j) tmp = mfma16<XDT>(A[j], unpack_biased_f16(wv[b][t][u][j]), tmp);
              const uint32_t z = (gq & 1) ? (zv[b][t][u] >> 4) : (zv[b][t][u] & 15u);
              const float zb = 1024.0f + (float)z;
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(fmaf(-zb, X[e], tmp[e]), sv[b][t][u], acc[t][e]);
            }
          } else {
            // groups of 64 or 32: an MFMA sums over every quarter of the unit,
            // so each lane dequantizes exactly with its own group's scale and
            // zero point: (1024 + q) - (1024 + z) = q - z, times s, rounded
            // once to fp16 -- the weight the method defines
#pragma unroll
            for (int t = 0; t < TPG; ++t) {
              const uint32_t z = (gq & 1) ? (zv[b][t][u] >> 4) : (zv[b][t][u] & 15u);
              const _Float16 nz = (_Float16)(-(1024.0f + (float)z));
              const _Float16 sc = (_Float16)sv[b][t][u];
              const half2_t nz2 = {nz, nz}, s2 = {sc, sc};
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint4_t bq = unpack_biased_f16(wv[b][t][u][j]);
                uint4_t bw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  half2_t h;
                  const uint32_t ue = bq[e];
                  __builtin_memcpy(&h, &ue, 4);
                  h = (h + nz2) * s2;
                  uint32_t o;
                  __builtin_memcpy(&o, &h, 4);
                  bw[e] = o;
                }
                acc[t] = mfma16<XDT>(A[j], bw, acc[t]);
              }
            }
          }
        } else {
#pragma unroll
          for (int t = 0; t < TPG; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              uint4_t bw;
              if constexpr (FMT == WQ_FMT_INT4_ASYM) {
                const float z = (float)((gq & 1) ? (zv[b][t][u] >> 4) : (zv[b][t][u] & 15u));
                bw = dequant_int4_word<XDT>(wv[b][t][u][j], z, sv[b][t][u]);
              } else {
                bw = dequant_nf4_word<XDT>(wv[b][t][u][j], lut2, sv[b][t][u]);
              }
              acc[t] = mfma16<XDT>(A[j], bw, acc[t]);
            }
          }
        }
      }
    }
    // refill this ring slot with phase p + NBUF (this wave's reads of it are
    // complete: their values fed the MFMAs above)
    if (p + NBUF < phases) {
      asm volatile("" ::: "memory");
      issue_phase(p + NBUF, bc);
      asm volatile("" ::: "memory");
    }
  };
  for (int p0 = 0; p0 < phases; p0 += NBUF) {
    [&]<int... B>(std::integer_sequence<int, B...>) {
      ((p0 + B < phases ? step(p0 + B, std::integral_constant<int, B>{}) : void()), ...);
    }(std::make_integer_sequence<int, NBUF>{});
  }
  vm_wait<0>();   // clamped loads of unused prologue phases

  // fixed-order sum of the NW waves' partial results.  Lane l holds rows
  // (l >> 4) * 4 + e of its 16 x 16 tile; with MP staged rows only the
  // entries of rows below MP can be stored (MP <= 4: lanes 0-15 and e < MP),
  // so only those go through LDS and get summed.
  constexpr int EV = MP < 4 ? MP : 4;                // entries e that can be stored
  constexpr int LV = MP <= 4 ? 16 : kWave;           // lanes that can
  __syncthreads();
  float* red = reinterpret_cast<float*>(dsm);
  if (LV == kWave || lane < LV) {
#pragma unroll
    for (int t = 0; t < TPG; ++t)
#pragma unroll
      for (int e = 0; e < EV; ++e) red[((wave * TPG + t) * EV + e) * LV + lane] = acc[t][e];
  }
  __syncthreads();
  constexpr int NV = TPG * EV * LV;
  constexpr int NH = TH * EV * LV;                   // the second matrix's sums start here
  // the sum of entry i of the NV results over the waves, in a fixed order
  auto total = [&](int i) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[i + w * NV];
    return v;
  };
  for (int i = tid; i < NH; i += NW * 64) {
    const int te = i / LV, l = i % LV, t = te / EV, e = te % EV;
    const int mm = (l >> 4) * 4 + e;
    const int tile = (int)blockIdx.x + t * (int)gridDim.x;
    const int nn = tile * 16 + (l & 15);
    if (mm < a.m && tile < ntiles && nn < a.n) {
      const float v = total(i);
      if constexpr (DUAL) {
        const float v2 = total(i + NH);
        const int64_t o = (int64_t)mm * a.n + nn;
        if (a.act) {
          store_y<YDT>(a.y, o, v / (1.0f + expf(-v)) * v2);   // silu(gate) * up
        } else {
          store_y<YDT>(a.y, o, v);
          store_y<YDT>(a.y_b, o, v2);
        }
        continue;
      }
      store_y<YDT>(a.y, (int64_t)mm * a.n + nn, v);
    }
  }
}

// Dynamic LDS bytes of one stream_kernel workgroup.
inline size_t stream_lds_bytes(int nw, int tpg, int gpp, int mp, int nbuf, bool szl, bool dual,
                               int fmt, int GS, int zb, int k) {
  const size_t xs = (size_t)((mp * gpp * 16 + 63) / 64 * 64) * 16;
  size_t b = (size_t)nw * nbuf * xs;
  if (szl)
    b += (size_t)tpg * (staged_a_bytes(fmt, GS, k) + staged_b_bytes(fmt, zb, k)) +
         (dual && mp > 1 ? 0 : (size_t)nw * nbuf * tpg * gpp * 1024);
  const size_t red = (size_t)nw * tpg * 4 * 64 * 4;   // an upper bound of the sums' LDS
  return b > red ? b : red;
}

// ------------------------------------------------------------------ GEMM
constexpr int GBM = 128, GBN = 128, GBK = 64, GLD = GBK + 8;  // LDS row stride (halfs)

struct GemmArgs {
  const uint16_t* x;
  const uint32_t* codes;
  const void* scales;
  const uint8_t* zeros;
  const float* scales2;
  int m, n, k, G, zb;        // G = k/128 units of 128; zb = bytes per row of zeros
  int GS, sub;               // INT4: groups per row (k/group), groups per unit (1, 2, 4)
  void* y;
};

// Dequantize 32 consecutive weights (one 16-byte chunk of codes) of row r,
// starting at column c0, into 32 16-bit values in natural order.
template <int FMT, int XDT>
__device__ __forceinline__ void dequant32(const GemmArgs& a, const float* lut, int r, int c0,
                                          uint4_t wv, uint32_t (&out)[16]) {
  if constexpr (FMT == WQ_FMT_INT4_ASYM) {
    const int g = c0 / (128 / a.sub);               // a 32-chunk lies in one group
    const float s = f16_bits_to_f32(static_cast<const uint16_t*>(a.scales)[(int64_t)r * a.GS + g]);
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
        const float v0 = as_f32(lut[(w >> (8 * e)) & 15u] * ah);
        const float v1 = as_f32(lut[(w >> (8 * e + 4)) & 15u] * ah);
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

// INT4 weights x fp16 activations GEMM (m > 16, prefill).  Workgroup tile
// 128 (m) x 32 NWG (n), NWG waves side by side along n (8: each 128 x 32 =
// 8 x 2 MFMA tiles of 16x16, two waves per SIMD); K advances one group (128)
// per step.  Every code is
// dequantized in registers by the wave that uses it, so the vector work per
// MFMA falls with the rows a wave covers; 128-row waves keep it under the
// matrix-core time on gfx950 (a wave64 vector instruction issues in about 4
// cycles, a 16x16x32 MFMA in 16).
//
//  * Both operands reach LDS by direct global->LDS loads, issued ahead of
//    use: the activation slice of group g+1 (2 buffers) and the codes of
//    group g+2 (3 buffers) during step g.  One barrier per step publishes
//    group g's buffers and proves every wave is done with the ones being
//    refilled.  No load lands in a register inside the loop, so the
//    compiler adds no waits of its own; the explicit wait before the barrier
//    counts exactly the loads issued after the ones it needs.
//    Activation chunk c16 of row r sits at slot c16 ^ (r & 15), code chunk c
//    (of 4) of row r at slot c ^ ((r >> 2) & 3): conflict-free operand reads.
//  * Codes are dequantized exactly in the natural k order: byte e of a word
//    is copied into bytes 0 and 2 (v_perm_b32), its low nibble OR'ed into
//    1024.0 (giving 1024 + q) and its high nibble, now at bits 4-7 of the
//    upper half, into 64.0 (where the mantissa step is 1/16, giving 64 + q);
//    a packed fp16 add of -(bias + z) gives q - z exactly and a packed fp16
//    multiply by the scale gives (q - z) * s rounded once -- the 16-bit
//    weight the dequantization defines.
//  * The workgroup's scales and zero points (contiguous for its 256 rows)
//    are staged into LDS once.
// Staged scale / zero-point capacity: 256 rows x up to kGemmMaxGroups groups.
constexpr int kGemmMaxGroups = 64;
constexpr int kGemmWaves = 8;   // 128 x 32 per wave, two waves per SIMD
constexpr int kGemmScaleBytes = 256 * kGemmMaxGroups * 2;
constexpr int kGemmZeroBytes = 256 * kGemmMaxGroups / 2;

// FMT/XDT: INT4 with fp16 activations takes the exponent-bias dequant above;
// INT4 with bf16 activations and NF4/FP4 (double-quantized absmax) take the
// exact general one: each weight is formed in fp32 ((q - z) * s, exact; or
// level * absmax, rounded once) and rounded once into the activation type
// (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32), as the dequantization defines.
template <int FMT, int XDT, int YDT, int NWG, int SUB>   // SUB: INT4 groups per unit of 128 (1, 2, 4)
__global__ __launch_bounds__(NWG * 64) void gemm_i4_kernel(GemmArgs a, Levels lv) {
  constexpr bool FAST = FMT == WQ_FMT_INT4_ASYM && XDT == WQ_F16;
  static_assert(FMT == WQ_FMT_INT4_ASYM || SUB == 1, "NF4 blocks: one unit of 128 = two blocks");
  constexpr int NW = NWG, BM = 128, BN = 32 * NWG;   // 32 code rows per wave
  constexpr int NF = BN / 16 / NW;               // 16-row code tiles per wave (n)
  constexpr int MI = BM / 16;                    // 16-row activation tiles per wave (m): all
  constexpr int XBUF = BM * 16;                  // 16-byte chunks per activation buffer
  constexpr int WBUF = BN * 4;                   // 16-byte chunks per code buffer
  constexpr int XL = XBUF / 64;                  // activation loads per group
  constexpr int XI = (XL + NW - 1) / NW;         // ... per wave, at most (fewer for some if NW does not divide XL)
  constexpr int WI = WBUF / 64 / NW;             // code loads per wave and group
  __shared__ uint4_t xr[2 * XBUF];
  __shared__ uint4_t wr[3 * WBUF];
  __shared__ __attribute__((aligned(16))) uint8_t scl[kGemmScaleBytes];
  __shared__ __attribute__((aligned(16))) uint8_t zcl[kGemmZeroBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave;                           // the wave's rows: wn * 16 * NF + [0, 16 * NF)
  const int nl = lane & 15, kq = lane >> 4;
  // Tile of this workgroup.  Workgroups are dispatched to the 8 XCDs round
  // robin (workgroup i to XCD i % 8), each XCD with its own L2: tile t
  // goes to workgroup (t % (T/8)) * 8 + t / (T/8) (T rounded down to a
  // multiple of 8; the rest keep their index), so every XCD runs a
  // contiguous run of T/8 tiles.  Tiles are numbered in groups of GM m-tiles
  // by all n-tiles, so such a run is a block of about GM x (T/8/GM) tiles:
  // each activation row block and each code column block is fetched from
  // HBM by few XCDs.
  constexpr int GM = 4;
  const int ntn = (a.n + BN - 1) / BN, ntm = (a.m + BM - 1) / BM;
  const int full = (ntn * ntm) & ~7;
  const int bid = blockIdx.x;
  const int tile = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
  const int grp = tile / (GM * ntn), gm = min(ntm - grp * GM, GM);
  const int tr = tile - grp * GM * ntn;
  const int m0 = (grp * GM + tr % gm) * BM, n0 = (tr / gm) * BN;
  const int G = a.G, GS = a.GS;                  // units of 128; groups per row
  const int SCB = (BN * GS * 2 + 1023) / 1024 * 1024;
  const int ZCB = (BN * a.zb + 1023) / 1024 * 1024;
  const int lq = (kq * SUB) >> 2;                // this lane's group within a unit

  // NF4: the 16 levels, and the second-level scales of the tile's blocks
  // (rows n0 .. n0+255 hold blocks n0*k/64 .. (n0+256)*k/64 - 1; their
  // scales2 indices start at c2b), written before any direct load is issued
  // so the compiler's wait for these loads waits for nothing else
  // lut2[b] = (level of code b & 15, level of code b >> 4): one 8-byte
  // read per byte of codes
  __shared__ float2_t lut2[FMT != WQ_FMT_INT4_ASYM ? 256 : 1];
  const int bpr = a.k / 64;                      // NF4 blocks per row
  const int64_t c2b = ((int64_t)n0 * bpr) >> 8;
  if constexpr (FMT != WQ_FMT_INT4_ASYM) {
    float* c2s = reinterpret_cast<float*>(zcl);
    const int nc2 = (int)((((int64_t)min(n0 + BN, a.n) * bpr - 1) >> 8) - c2b + 1);
    if (tid < 256) lut2[tid] = float2_t{lv.v[tid & 15], lv.v[tid >> 4]};
    for (int i = tid; i < nc2; i += NW * 64) c2s[i] = a.scales2[c2b + i];
    lgkm_wait0();
  }
  // staged scales and zero points of rows n0 .. n0+255 (NF4: the int8
  // absmax codes of their blocks), clamped at the end of the buffers; rows
  // past n are never stored
  if constexpr (FMT != WQ_FMT_INT4_ASYM) {
    const int nab = (BN * bpr + 1023) / 1024;
    const int64_t abytes = (int64_t)a.n * bpr;
    for (int i = wave; i < nab; i += NW) {
      const int64_t off = (int64_t)n0 * bpr + i * 1024 + lane * 16;
      lds_dma16(static_cast<const uint8_t*>(a.scales) + min(off, abytes - 16),
                (lds_void_t*)(scl + i * 1024));
    }
  } else {
    const int nsc = SCB / 1024, nzc = ZCB / 1024;
    const int64_t sbytes = (int64_t)a.n * GS * 2, zbytes = (int64_t)a.n * a.zb;
    for (int i = wave; i < nsc + nzc; i += NW) {
      const bool isz = i >= nsc;
      const int j = isz ? i - nsc : i;
      const int64_t off = (int64_t)n0 * (isz ? a.zb : 2 * GS) + j * 1024 + lane * 16;
      const uint8_t* src = (isz ? a.zeros : static_cast<const uint8_t*>(a.scales)) +
                           min(off, (isz ? zbytes : sbytes) - 16);
      lds_dma16(src, (lds_void_t*)((isz ? zcl : scl) + j * 1024));
    }
  }

  // per-lane source offsets of the direct loads, relative to the tile's
  // first activation row and first code row (a group adds a uniform one);
  // 32 bits hold them for k up to 2^23
  const char* const xb = reinterpret_cast<const char*>(a.x) + (int64_t)m0 * a.k * 2;
  const char* const cb = reinterpret_cast<const char*>(a.codes) + (int64_t)n0 * (a.k / 2);
  uint32_t xoff[XI], woff[WI];
#pragma unroll
  for (int t = 0; t < XI; ++t) {
    const int i = min(t * NW + wave, XL - 1);    // load i fills slots 64 i .. 64 i + 63
    const int r = i * 4 + (lane >> 4);
    const int c16 = (lane & 15) ^ (r & 15);
    xoff[t] = (uint32_t)min(r, a.m - 1 - m0) * (uint32_t)(a.k * 2) + c16 * 16;
  }
#pragma unroll
  for (int t = 0; t < WI; ++t) {
    const int i = t * NW + wave;
    const int row = i * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);   // chunk c of a row sits at slot c ^ ((row >> 2) & 3)
    woff[t] = (uint32_t)min(row, a.n - 1 - n0) * (uint32_t)(a.k / 2) + c * 16;
  }
  // direct loads of group g (clamped: groups past the end reload the last
  // one, so every step issues the same loads)
  auto issue_x = [&](int gi) {
    const char* base = xb + (int64_t)min(gi, G - 1) * 256;
    uint4_t* buf = xr + (gi & 1) * XBUF;
#pragma unroll
    for (int t = 0; t < XI; ++t)
      if (XL % NW == 0 || t * NW + wave < XL)
        lds_dma16(base + xoff[t], (lds_void_t*)(buf + (t * NW + wave) * 64));
  };
  auto issue_w = [&](int gi) {
    const char* base = cb + (int64_t)min(gi, G - 1) * 64;
    uint4_t* buf = wr + (gi % 3) * WBUF;
#pragma unroll
    for (int t = 0; t < WI; ++t) lds_dma16(base + woff[t], (lds_void_t*)(buf + (t * NW + wave) * 64));
  };

  float4_t acc[MI][NF];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  issue_w(0);
  issue_x(0);
  issue_w(1);

  constexpr uint32_t kMask = 0x00F0000Fu, kBias = 0x54006400u;   // 64.0 (hi), 1024.0 (lo)
  for (int g = 0; g < G; ++g) {
    // this wave's loads of group g's activations (and, issued earlier, its
    // codes and the staged scales) have landed: only the codes of group g+1
    // were issued after them
    vm_wait<WI>();
    wg_barrier();   // ... and every wave's; the buffers refilled below are free
    issue_x(g + 1);
    issue_w(g + 2);
    const uint4_t* xcur = xr + (g & 1) * XBUF;
    const uint4_t* wcur = wr + (g % 3) * WBUF;
    // codes, scales and zero points (NF4: absmax) of this wave's row tiles
    // for group g
    uint4_t wv[NF];
    half2_t s2[NF], nz2[NF];
    float sf[NF], zf[NF];   // INT4: s and -z * s (exact); NF4: absmax, unused
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int r = wn * 16 * NF + j * 16 + nl;
      wv[j] = wcur[r * 4 + (kq ^ ((r >> 2) & 3))];
      if constexpr (FMT == WQ_FMT_INT4_ASYM) {
        const int gq = g * SUB + lq;
        _Float16 sc16;
        __builtin_memcpy(&sc16, scl + (r * GS + gq) * 2, 2);
        const uint32_t zb = zcl[r * a.zb + (gq >> 1)];
        const float z = (float)((gq & 1) ? (zb >> 4) : (zb & 15u));
        s2[j] = half2_t{sc16, sc16};
        nz2[j] = half2_t{(_Float16)(-(1024.0f + z)), (_Float16)(-(64.0f + z))};
        sf[j] = (float)sc16;
        zf[j] = -z * sf[j];
      } else {
        // absmax of this lane's block (quarter kq of the unit lies in block
        // 2g + kq/2 of the row): fp32(q8) * c2, as the double quantization
        // defines it
        const int bl = r * bpr + 2 * g + (kq >> 1);
        const float c2 = reinterpret_cast<const float*>(zcl)[(((int64_t)n0 * bpr + bl) >> 8) - c2b];
        sf[j] = (float)reinterpret_cast<const int8_t*>(scl)[bl] * c2;
        zf[j] = 0.0f;
      }
    }
    // activation fragments of chunk s; with the INT4 fp16 decoder those of
    // chunk s + 1 are read while chunk s multiplies (66.98 against 68.75 us
    // on 2048 x 4096 x 4096; the NF4 decoder, whose table reads share the
    // LDS, measured 3.6% slower with it), A/B in one run
    constexpr int AB = FAST ? 2 : 1;
    uint4_t AA[AB][MI];
    auto read_a = [&](uint4_t (&dst)[MI], int s) {
#pragma unroll
      for (int i = 0; i < MI; ++i) dst[i] = xcur[(i * 16 + nl) * 16 + ((kq * 4 + s) ^ nl)];
    };
    if constexpr (AB == 2) read_a(AA[0], 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (AB == 2) {
        if (s + 1 < 4) read_a(AA[(s + 1) & 1], s + 1);
      } else {
        read_a(AA[0], s);
      }
      const uint4_t(&A)[MI] = AA[AB == 2 ? (s & 1) : 0];
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const uint32_t w = wv[j][s];
        uint4_t B;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (FAST) {
            const uint32_t u = and_or(__builtin_amdgcn_perm(w, w, 0x01010101u * e), kMask, kBias);
            // through scalar copies: a bit_cast straight from a vector element
            // produced wrong code here
            half2_t h;
            __builtin_memcpy(&h, &u, 4);
            h = (h + nz2[j]) * s2[j];
            uint32_t be;
            __builtin_memcpy(&be, &h, 4);
            B[e] = be;
          } else {
            float v0, v1;
            if constexpr (FMT == WQ_FMT_INT4_ASYM) {
              // q * s - z * s in one fma: (q - z) * s is exact in fp32, so
              // the single rounding of the fma changes nothing
              const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
              v0 = fmaf((float)((lo >> (8 * e)) & 255u), sf[j], zf[j]);
              v1 = fmaf((float)((hi >> (8 * e)) & 255u), sf[j], zf[j]);
            } else {
              const float2_t l = lut2[(w >> (8 * e)) & 255u];
              v0 = as_f32(l.x * sf[j]);
              v1 = as_f32(l.y * sf[j]);
            }
            B[e] = pack2_x<XDT>(v0, v1);
          }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) acc[i][j] = mfma16<XDT>(A[i], B, acc[i][j]);
      }
    }
  }
  vm_wait<0>();   // the clamped loads past the last group

#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int mm = m0 + i * 16 + kq * 4 + e;
        const int nn = n0 + wn * 16 * NF + j * 16 + nl;
        if (mm < a.m && nn < a.n) store_y<YDT>(a.y, (int64_t)mm * a.n + nn, acc[i][j][e]);
      }
}

template <int FMT, int XDT, int YDT, int NWG>
hipError_t launch_gemm_i4_w(const GemmArgs& a, const Levels& lv, hipStream_t s) {
  // one launch per slice of rows keeps the 1-D grid within 2^22 workgroups
  constexpr int BN = 32 * NWG;
  const int64_t ntn = (a.n + BN - 1) / BN, ysz = YDT == WQ_F32 ? 4 : 2;
  const int64_t rows = 128 * std::max<int64_t>(1, (int64_t(1) << 22) / ntn);
  for (int64_t r0 = 0; r0 < a.m; r0 += rows) {
    GemmArgs b = a;
    b.m = (int)std::min<int64_t>(a.m - r0, rows);
    b.x = a.x + r0 * a.k;
    b.y = static_cast<char*>(a.y) + r0 * a.n * ysz;
    const dim3 grid((unsigned)(ntn * ((b.m + 127) / 128)));
    if constexpr (FMT != WQ_FMT_INT4_ASYM) {
      gemm_i4_kernel<FMT, XDT, YDT, NWG, 1><<<grid, NWG * 64, 0, s>>>(b, lv);
    } else {
      if (a.sub == 4)
        gemm_i4_kernel<FMT, XDT, YDT, NWG, 4><<<grid, NWG * 64, 0, s>>>(b, lv);
      else if (a.sub == 2)
        gemm_i4_kernel<FMT, XDT, YDT, NWG, 2><<<grid, NWG * 64, 0, s>>>(b, lv);
      else
        gemm_i4_kernel<FMT, XDT, YDT, NWG, 1><<<grid, NWG * 64, 0, s>>>(b, lv);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Eight waves (tiles 128 x 256) or seven (128 x 224): seven where the
// narrower tiles need no more rounds of 256 workgroups, which shortens each
// round by an eighth (the NF4 8B layer at m = 512: 256 tiles of 224 columns
// in one round instead of 224 tiles of 256 on 224 CUs, 77.7 against
// 96.0 us, the same bits, A/B in one run, twice).
template <int FMT, int XDT, int YDT>
hipError_t launch_gemm_i4(const GemmArgs& a, const Levels& lv, hipStream_t s) {
  const int64_t ntm = (a.m + 127) / 128;
  const int64_t r8 = ((a.n + 255) / 256 * ntm + 255) / 256;
  const int64_t r7 = ((a.n + 223) / 224 * ntm + 255) / 256;
  if (r7 * 224 < r8 * 256) return launch_gemm_i4_w<FMT, XDT, YDT, 7>(a, lv, s);
  return launch_gemm_i4_w<FMT, XDT, YDT, kGemmWaves>(a, lv, s);
}

// INT4 groups per row (k / group); other formats: the units of 128.
inline int int4_groups(const wq_weight* w) {
  return (int)(w->fmt == WQ_FMT_INT4_ASYM ? w->k / w->group : w->k / 128);
}

// ---------------------------------------------------------------- launch
// Streaming decode configurations: NW, TPG, GPP, MP, NBUF.
template <int XDT, int YDT, int FMT, int NW, int TPG, int GPP, int MP, int NBUF, bool SZL,
          bool DUAL, bool SG>
hipError_t launch_stream_t(const SkinnyArgs& a, const Levels& lv, const W4Plan& p, hipStream_t s) {
  auto kern = stream_kernel<XDT, YDT, FMT, NW, TPG, GPP, MP, NBUF, SZL, DUAL, SG>;
  const size_t lds = stream_lds_bytes(NW, TPG, GPP, MP, NBUF, SZL, DUAL, FMT, a.GS, a.zb, a.k);
  if (a.m > MP) return hipErrorInvalidValue;   // rows past MP are never staged
  if (lds > 160 * 1024 - 256) return hipErrorInvalidConfiguration;
  // raise the dynamic LDS limit of this instantiation when a launch needs
  // more than the default (the static NF4 table shares the 160 KB)
  static std::atomic<size_t> allowed{64 * 1024};
  if (lds > allowed.load(std::memory_order_relaxed)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    size_t cur = allowed.load(std::memory_order_relaxed);
    while (lds > cur && !allowed.compare_exchange_weak(cur, lds)) {
    }
  }
  kern<<<dim3((unsigned)p.grid), NW * 64, lds, s>>>(a, lv, p.phases);
  return hipGetLastError();
}

template <int XDT, int YDT, int FMT>
hipError_t launch_stream(const SkinnyArgs& a, const Levels& lv, const W4Plan& p, hipStream_t s) {
#define WQ_STR(C, NW, TPG, GPP, MP, NBUF)                                                     \
  case C:                                                                                     \
    if constexpr (FMT == WQ_FMT_INT4_ASYM) {                                                  \
      if constexpr (XDT == WQ_F16) {                                                          \
        if (a.sub > 1) {                                                                      \
          if (p.szl)                                                                          \
            return launch_stream_t<XDT, YDT, FMT, NW, TPG, GPP, MP, NBUF, true, false, true>(  \
                a, lv, p, s);                                                                 \
          return launch_stream_t<XDT, YDT, FMT, NW, TPG, GPP, MP, NBUF, false, false, true>(   \
              a, lv, p, s);                                                                   \
        }                                                                                     \
      }                                                                                       \
    }                                                                                         \
    if (p.szl)                                                                                \
      return launch_stream_t<XDT, YDT, FMT, NW, TPG, GPP, MP, NBUF, true, false, false>(      \
          a, lv, p, s);                                                                       \
    return launch_stream_t<XDT, YDT, FMT, NW, TPG, GPP, MP, NBUF, false, false, false>(a, lv, p, s);
  switch (p.cfg) {
    WQ_STR(40, 8, 1, 1, 1, 2)
    WQ_STR(42, 8, 1, 1, 4, 2)
    WQ_STR(43, 8, 3, 1, 16, 2)
    WQ_STR(45, 8, 1, 1, 16, 2)
    WQ_STR(47, 8, 1, 2, 1, 2)
    WQ_STR(50, 8, 2, 1, 16, 2)
    WQ_STR(51, 8, 4, 1, 16, 2)
    WQ_STR(54, 4, 1, 2, 16, 2)
    WQ_STR(74, 16, 1, 1, 1, 2)
    default: return hipErrorInvalidConfiguration;
  }
#undef WQ_STR
}

// Gate/up pair configurations: NW, TPG (tiles of both matrices), GPP, MP, NBUF.
template <int FMT, int XDT, int YDT>
hipError_t launch_stream_pair(const SkinnyArgs& a, const Levels& lv, const W4Plan& p,
                              hipStream_t s) {
#define WQ_PAIR_T(NW, TPG, GPP, MP, NBUF, SG)                                                  \
  if (p.szl)                                                                                  \
    return launch_stream_t<XDT, YDT, FMT, NW, TPG, GPP, MP, NBUF, true, true, SG>(a, lv, p, s); \
  /* NF4 absmax loaded per unit with eight tiles would spill: never planned */                \
  if constexpr (FMT == WQ_FMT_NF4 && TPG >= 8) return hipErrorInvalidConfiguration;           \
  else                                                                                        \
    return launch_stream_t<XDT, YDT, FMT, NW, TPG, GPP, MP, NBUF, false, true, SG>(a, lv, p, s);
#define WQ_PAIR(C, NW, TPG, GPP, MP, NBUF)                                                    \
  case C:                                                                                     \
    if constexpr (FMT == WQ_FMT_INT4_ASYM && XDT == WQ_F16) {                                 \
      if (a.sub > 1) {                                                                        \
        WQ_PAIR_T(NW, TPG, GPP, MP, NBUF, true)                                               \
      }                                                                                       \
    }                                                                                         \
    WQ_PAIR_T(NW, TPG, GPP, MP, NBUF, false)
  switch (p.cfg) {
    WQ_PAIR(60, 8, 2, 1, 1, 2)
    WQ_PAIR(61, 8, 2, 1, 4, 2)
    WQ_PAIR(62, 8, 2, 1, 16, 2)
    WQ_PAIR(63, 8, 4, 1, 16, 2)
    WQ_PAIR(65, 8, 8, 1, 16, 2)
    WQ_PAIR(67, 8, 6, 1, 16, 1)
    default: return hipErrorInvalidConfiguration;
  }
#undef WQ_PAIR
#undef WQ_PAIR_T
}

template <int XDT, int YDT>
hipError_t launch_typed(const void* x, int64_t m, const wq_weight* w, const float* levels,
                        void* y, const W4Plan& p, hipStream_t s) {
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
    a.GS = int4_groups(w);
    a.sub = a.GS / a.G;
    a.zb = (a.GS + 1) / 2;
    a.y = y;
    if (w->fmt == WQ_FMT_INT4_ASYM && p.szl && a.GS <= kGemmMaxGroups)
      return launch_gemm_i4<WQ_FMT_INT4_ASYM, XDT, YDT>(a, lv, s);
    // NF4/FP4 with double-quantized absmax: the int8 codes of a tile's 256
    // rows (256 * k/64 bytes) are staged in the scale buffer, so k <= 8192,
    // staged by 16-byte direct loads (aligned buffer, size a multiple of 16)
    if (w->fmt == WQ_FMT_NF4 && w->scales2 != nullptr && w->k <= 64 * kGemmMaxGroups * 2 &&
        ((uintptr_t)w->scales % 16) == 0 && (w->n * (w->k / 64)) % 16 == 0)
      return launch_gemm_i4<WQ_FMT_NF4, XDT, YDT>(a, lv, s);
    const dim3 grid((unsigned)((w->n + GBN - 1) / GBN), (unsigned)((m + GBM - 1) / GBM));
    if (w->fmt == WQ_FMT_NF4)
      gemm_kernel<WQ_FMT_NF4, XDT, YDT><<<grid, 256, 0, s>>>(a, lv);
    else
      gemm_kernel<WQ_FMT_INT4_ASYM, XDT, YDT><<<grid, 256, 0, s>>>(a, lv);
    return hipGetLastError();
  }
  SkinnyArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.codes = static_cast<const uint32_t*>(w->codes);
  a.scales = w->scales;
  a.zeros = w->zeros;
  a.scales2 = w->scales2;
  a.m = (int)m;
  a.n = (int)w->n;
  a.k = (int)w->k;
  a.G = (int)(w->k / 128);
  a.GS = int4_groups(w);
  a.sub = a.GS / a.G;
  a.zb = (a.GS + 1) / 2;
  a.y = y;
  return w->fmt == WQ_FMT_NF4 ? launch_stream<XDT, YDT, WQ_FMT_NF4>(a, lv, p, s)
                              : launch_stream<XDT, YDT, WQ_FMT_INT4_ASYM>(a, lv, p, s);
}

template <int XDT, int YDT>
hipError_t launch_pair_typed(const void* x, int64_t m, const wq_weight* wg, const wq_weight* wu,
                             const float* levels, int act, void* yg, void* yu, const W4Plan& p,
                             hipStream_t s) {
  Levels lv{};
  for (int i = 0; i < 16; ++i) lv.v[i] = levels[i];
  SkinnyArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.codes = static_cast<const uint32_t*>(wg->codes);
  a.scales = wg->scales;
  a.zeros = wg->zeros;
  a.scales2 = wg->scales2;
  a.m = (int)m;
  a.n = (int)wg->n;
  a.k = (int)wg->k;
  a.G = (int)(wg->k / 128);
  a.GS = int4_groups(wg);
  a.sub = a.GS / a.G;
  a.zb = (a.GS + 1) / 2;
  a.y = yg;
  a.codes_b = static_cast<const uint32_t*>(wu->codes);
  a.scales_b = wu->scales;
  a.zeros_b = wu->zeros;
  a.scales2_b = wu->scales2;
  a.y_b = yu;
  a.act = act;
  if (wg->fmt == WQ_FMT_NF4) return launch_stream_pair<WQ_FMT_NF4, XDT, YDT>(a, lv, p, s);
  return launch_stream_pair<WQ_FMT_INT4_ASYM, XDT, YDT>(a, lv, p, s);
}

template <int XDT>
hipError_t launch_x(const void* x, int64_t m, const wq_weight* w, const float* levels, void* y,
                    int ydt, const W4Plan& p, hipStream_t s) {
  switch (ydt) {
    case WQ_F32: return launch_typed<XDT, WQ_F32>(x, m, w, levels, y, p, s);
    case WQ_BF16: return launch_typed<XDT, WQ_BF16>(x, m, w, levels, y, p, s);
    default: return launch_typed<XDT, WQ_F16>(x, m, w, levels, y, p, s);
  }
}

}  // namespace

W4Plan plan_w4a16(int64_t m, const wq_weight* w) {
  // Streaming decode configurations (NW waves, TPG row tiles, GPP groups per
  // wave and phase, MP staged activation rows, NBUF phases in flight).
  struct SCfg { int id, nw, tpg, gpp, mp, nbuf; };
  static const SCfg scfgs[] = {{40, 8, 1, 1, 1, 2},  {42, 8, 1, 1, 4, 2},  {43, 8, 3, 1, 16, 2},
                               {45, 8, 1, 1, 16, 2}, {47, 8, 1, 2, 1, 2},  {50, 8, 2, 1, 16, 2},
                               {51, 8, 4, 1, 16, 2}, {54, 4, 1, 2, 16, 2}, {74, 16, 1, 1, 1, 2}};
  W4Plan p;
  p.path = m > 16 ? 1 : 3;
  p.tpg = 1;
  p.gpw = 1;
  p.mp = 1;
  p.cfg = 0;
  p.phases = 1;
  p.grid = 0;
  const int64_t GS = int4_groups(w);
  p.szl = w->fmt == WQ_FMT_INT4_ASYM && ((uintptr_t)w->scales % 16) == 0 &&
          ((uintptr_t)w->zeros % 16) == 0 && (w->n * GS * 2) % 16 == 0 &&
          (w->n * ((GS + 1) / 2)) % 16 == 0;
  if (p.path == 1) return p;
  // NF4/FP4 decode: the int8 absmax codes of a tile's blocks staged by 1 KB
  // direct loads (16-byte aligned buffer, a multiple of 16 bytes long)
  if (w->fmt == WQ_FMT_NF4)
    p.szl = w->scales2 != nullptr && ((uintptr_t)w->scales % 16) == 0 &&
            (w->n * (w->k / 64)) % 16 == 0;
  const int64_t G = w->k / 128;
  const int64_t ntiles = (w->n + 15) / 16;
  // measured on MI355X (graph-replayed calls of the 7B/8B decode shapes);
  // two phases in flight per wave beat deeper pipelines: with every load in
  // flight at once the memory system returns the phases out of order, and a
  // wave's loads complete in issue order, so its multiply waits for all of
  // them.
  //  m = 1: eight waves, one group per wave and phase (two for long K);
  //         sixteen waves for INT4 with at most one workgroup per CU and
  //         K below 64 groups (4096x4096: 5.02 against 5.19 us per call,
  //         A/B on one box, twice; NF4 and larger grids measured slower);
  //  m <= 4: eight waves, one tile;
  //  m <= 16: one workgroup per CU, as many tiles per workgroup as that
  //           takes (at most 4; more tiles take several rounds); INT4 with
  //           one tile and K of 64 groups or more: four waves taking their
  //           groups in pairs (whole-line code loads: 4096x11008 at m = 16
  //           11.6 against 11.9 us; at K = 4096 6.1 against 5.9, so not
  //           there).
  int cfg;
  if (m <= 1) {
    cfg = G >= 64 ? 47 : (w->fmt == WQ_FMT_INT4_ASYM && ntiles <= 256 ? 74 : 40);
  } else if (m <= 4) {
    cfg = 42;
  } else {
    const int64_t tpg = (ntiles + 255) / 256;
    cfg = tpg >= 4 ? 51 : tpg == 3 ? 43 : (tpg == 2 ? 50 : (G >= 64 && w->fmt == WQ_FMT_INT4_ASYM ? 54 : 45));
  }
  for (const SCfg& sc : scfgs)
    if (sc.id == cfg) {
      p.cfg = sc.id;
      p.tpg = sc.tpg;
      p.gpw = sc.gpp;
      p.mp = sc.mp;
      p.phases = (int)((G + sc.nw * sc.gpp - 1) / (sc.nw * sc.gpp));
      p.grid = (int)((ntiles + sc.tpg - 1) / sc.tpg);
      // staged scales must fit beside the activation ring
      if (p.szl) {
        const size_t lds = stream_lds_bytes(sc.nw, sc.tpg, sc.gpp, sc.mp, sc.nbuf, true, false,
                                            w->fmt, (int)GS, (int)((GS + 1) / 2), (int)w->k);
        if (lds > 160 * 1024 - 256) p.szl = false;
      }
    }
  return p;
}

hipError_t launch_w4a16(const void* x, int xdt, int64_t m, const wq_weight* w,
                        const float* levels16, void* y, int ydt, const W4Plan& plan,
                        hipStream_t s) {
  if (xdt == WQ_BF16) return launch_x<WQ_BF16>(x, m, w, levels16, y, ydt, plan, s);
  return launch_x<WQ_F16>(x, m, w, levels16, y, ydt, plan, s);
}

W4Plan plan_w4a16_pair(int64_t m, const wq_weight* wg, const wq_weight* wu) {
  // Gate/up pairs (m <= 16): the single-matrix schedules with the tiles of
  // both matrices in one workgroup (codes in registers, scales staged), so
  // the activations are staged once for both.
  struct PCfg { int id, nw, tpg, gpp, mp, nbuf; };
  static const PCfg pcfgs[] = {{60, 8, 2, 1, 1, 2},  {61, 8, 2, 1, 4, 2}, {62, 8, 2, 1, 16, 2},
                               {63, 8, 4, 1, 16, 2}, {65, 8, 8, 1, 16, 2}, {67, 8, 6, 1, 16, 1}};
  W4Plan p = plan_w4a16(m, wg);
  p.szl = p.szl && plan_w4a16(m, wu).szl;
  if (p.path == 1) return p;
  const int64_t G = wg->k / 128;
  const int64_t ntiles = (wg->n + 15) / 16;
  int cfg;
  if (m <= 1) {
    cfg = 60;
  } else if (m <= 4) {
    cfg = 61;
  } else {
    // three row tiles of each matrix (the 11008-row gate/up shape): one
    // phase in flight per wave measured faster than two (15.2-15.6 against
    // 16.3-16.8 us for the pair at m = 16, A/B on one box, twice); the
    // twelve code loads of a phase already keep the CU busy
    const int64_t th = (ntiles + 255) / 256;
    cfg = th >= 4 ? 65 : th == 3 ? 67 : (th == 2 ? 63 : 62);
  }
  const bool szl0 = p.szl;
  auto apply = [&](int id) {
    p.szl = szl0;
    for (const PCfg& pc : pcfgs)
      if (pc.id == id) {
        p.cfg = pc.id;
        p.tpg = pc.tpg;
        p.gpw = pc.gpp;
        p.mp = pc.mp;
        p.phases = (int)((G + pc.nw * pc.gpp - 1) / (pc.nw * pc.gpp));
        p.grid = (int)((ntiles + pc.tpg / 2 - 1) / (pc.tpg / 2));
        const int64_t GSp = int4_groups(wg);
        if (p.szl && stream_lds_bytes(pc.nw, pc.tpg, pc.gpp, pc.mp, pc.nbuf, true, true,
                                      wg->fmt, (int)GSp, (int)((GSp + 1) / 2),
                                      (int)wg->k) > 160 * 1024 - 256)
          p.szl = false;
      }
  };
  apply(cfg);
  // NF4/FP4 whose absmax is not staged: four tiles of each matrix would hold
  // too many registers (their absmax is loaded per unit); two instead
  if (p.cfg == 65 && wg->fmt == WQ_FMT_NF4 && !p.szl) apply(63);
  return p;
}

namespace {

// yg = silu(yg) * yu elementwise, in fp32 on the stored values (the SiLU
// product after the two prefill GEMMs); a workgroup takes 2048 consecutive
// elements, lane l the elements l, l + 256, ... of them, so every load and
// store of a wave covers consecutive elements.
template <int YDT>
__global__ __launch_bounds__(256) void silu_mul_kernel(void* __restrict__ yg,
                                                       const void* __restrict__ yu,
                                                       int64_t count) {
  const int64_t i0 = (int64_t)blockIdx.x * 2048 + threadIdx.x;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t i = i0 + j * 256;
    if (i >= count) return;
    float g, u;
    if constexpr (YDT == WQ_F32) {
      g = static_cast<const float*>(yg)[i];
      u = static_cast<const float*>(yu)[i];
    } else {
      g = load16<YDT>(static_cast<const uint16_t*>(yg) + i);
      u = load16<YDT>(static_cast<const uint16_t*>(yu) + i);
    }
    store_y<YDT>(yg, i, g / (1.0f + expf(-g)) * u);
  }
}

hipError_t launch_silu_mul(void* yg, const void* yu, int64_t count, int ydt, hipStream_t s) {
  const dim3 grid((unsigned)((count + 2047) / 2048));
  if (ydt == WQ_F32)
    silu_mul_kernel<WQ_F32><<<grid, 256, 0, s>>>(yg, yu, count);
  else if (ydt == WQ_BF16)
    silu_mul_kernel<WQ_BF16><<<grid, 256, 0, s>>>(yg, yu, count);
  else
    silu_mul_kernel<WQ_F16><<<grid, 256, 0, s>>>(yg, yu, count);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a16_pair(const void* x, int xdt, int64_t m, const wq_weight* wg,
                             const wq_weight* wu, const float* levels16, int act, void* yg,
                             void* yu, int ydt, const W4Plan& plan, hipStream_t s) {
  if (plan.path == 1) {
    // prefill: two GEMMs (the pair gains nothing once the weights are reused
    // across many rows); act 1 then forms silu(gate) * up from the two
    // stored outputs, the up projection held in yu
    hipError_t e = launch_w4a16(x, xdt, m, wg, levels16, yg, ydt, plan, s);
    if (e != hipSuccess) return e;
    e = launch_w4a16(x, xdt, m, wu, levels16, yu, ydt, plan_w4a16(m, wu), s);
    if (e != hipSuccess || act == 0) return e;
    return launch_silu_mul(yg, yu, m * wg->n, ydt, s);
  }
#define WQ_PAIR_Y(XDT)                                                                      \
  switch (ydt) {                                                                            \
    case WQ_F32:                                                                            \
      return launch_pair_typed<XDT, WQ_F32>(x, m, wg, wu, levels16, act, yg, yu, plan, s);  \
    case WQ_BF16:                                                                           \
      return launch_pair_typed<XDT, WQ_BF16>(x, m, wg, wu, levels16, act, yg, yu, plan, s); \
    default:                                                                                \
      return launch_pair_typed<XDT, WQ_F16>(x, m, wg, wu, levels16, act, yg, yu, plan, s);  \
  }
  if (xdt == WQ_BF16) {
    WQ_PAIR_Y(WQ_BF16)
  }
  WQ_PAIR_Y(WQ_F16)
#undef WQ_PAIR_Y
}

}  // namespace wq
