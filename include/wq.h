/*
 * wq.h -- C ABI of the group-wise low-bit weight-quantized linear layer
 * library for AMD Instinct MI355X (gfx950).
 *
 * Pages the operations follow (titles translated):
 *   [P1] "LLM quantization selection: five mainstream schemes compared"
 *        (www.0539edu.com/news/5934728)
 *   [P2] the quantization-concepts article "many people's understanding of
 *        quantization stops at making the model smaller"
 *        (aicoding.csdn.net/6a6874d110ee7a33f2936327.html)
 *   [P3] "LLM quantization hands-on manual" (devpress.csdn.net/awstech/...)
 *   [P5] "Inference & deployment 05: quantized deployment compared (GPTQ,
 *        AWQ, GGUF, FP8)" (devpress.csdn.net/amd/6a55d4ea662f9a54cb8f2c4c.html)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - W is [n][k] row-major: n output features, k input features.  x is
 *    [m][k] row-major, y is [m][n] row-major, y = x . w_hat^T.
 *  - Every data pointer is a DEVICE pointer owned by the caller, except
 *    the wq_weight descriptor itself and wq_nf4_codebook's output, which
 *    are host memory read/written during the call.  The library allocates
 *    nothing on the device and frees nothing; scratch space, where an
 *    operation needs it, is the caller's `workspace`, sized by the matching
 *    *_workspace() query.
 *  - `stream` is a hipStream_t passed as an opaque pointer (NULL = the
 *    null stream).  Calls only enqueue work on `stream` and never
 *    synchronize; outputs are valid once `stream` reaches them.  Calls on
 *    different streams that write distinct buffers may overlap.
 *  - Argument checks happen before any HIP call, so a call that returns an
 *    error other than WQ_ERR_HIP has enqueued nothing.  WQ_ERR_HIP reports
 *    a failed kernel launch.  NaN/Inf inputs are not checked and give
 *    unspecified (but memory-safe) results.
 *  - Sizes: every dimension (m, n, k) is below 2^23 and every matrix
 *    (n x k weights, m x k activations, m x n outputs) holds at most 2^34
 *    elements; larger sizes return WQ_ERR_SHAPE.
 *  - Rounding: every "round" is round-half-to-even; every division is an
 *    IEEE fp32 division; 16-bit conversions round to nearest even.
 *  - The library's only mutable global state is the per-kernel LDS limit it
 *    raises once (atomically) on first use and, per GPU, the address of the
 *    no-allocation scratch array (looked up once, under a lock); calls are
 *    thread-safe, except that wq_linear_int8_decomp_noalloc calls sharing a
 *    GPU's scratch must not overlap.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WQ_OK = 0,
  WQ_ERR_NULL = 1,        /* a required pointer is NULL                       */
  WQ_ERR_SHAPE = 2,       /* sizes are negative, zero where not allowed, or   */
                          /* not multiples of what the format needs           */
  WQ_ERR_ALIGN = 3,       /* a pointer misses its documented alignment        */
  WQ_ERR_UNSUPPORTED = 4, /* a valid but unimplemented combination            */
  WQ_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the query says    */
  WQ_ERR_HIP = 6          /* a kernel launch failed                           */
} wq_status;

typedef enum { WQ_F16 = 0, WQ_BF16 = 1, WQ_F32 = 2 } wq_dtype;

typedef enum {
  WQ_FMT_INT4_ASYM = 0,   /* wq_quantize_groupwise(bits=4, symmetric=0)       */
  WQ_FMT_NF4 = 1,         /* wq_pack_nf4                                      */
  WQ_FMT_INT8_SYM_ROW = 2,/* wq_quantize_groupwise(bits=8, symmetric=1, k)    */
  WQ_FMT_FP4 = 3          /* wq_pack_fp4                                      */
} wq_format;

/*
 * A quantized weight matrix, as produced by the quantize/pack calls.
 *
 *  fmt = WQ_FMT_INT4_ASYM:
 *    codes   uint32 [n][k/8]; element (r, c) in bits 4*(c%8)..+3 of word
 *            (r, c/8).  16-byte aligned.
 *    scales  fp16 [n][G], G = k/group.  2-byte aligned.
 *    zeros   uint8 [n][ceil(G/2)]; zero point of group g in byte g/2, low
 *            nibble when g is even.
 *    group   the group size along k (128 is the workload value).
 *  fmt = WQ_FMT_NF4:
 *    codes   uint8 [n*k/2]; element 2j is the low nibble of byte j (the
 *            same order as INT4 inside a little-endian word).  16-byte
 *            aligned.
 *    scales  int8 [n*k/group] double-quantized absmax when scales2 != NULL,
 *            else fp32 [n*k/group] absmax.
 *    scales2 fp32 [ceil(n*k/group / group2)] second-level scales, or NULL.
 *    group   NF4 block size (64); group2 the double-quant block (256).
 *  fmt = WQ_FMT_FP4: the NF4 layout with E2M1 codes (see wq_pack_fp4).
 *  perm (INT4 only, optional): act-order.  The input channels were
 *    quantized in the order perm[0], perm[1], ... ([P1] 3.2, [P4] 3.2), so
 *    the groups run along that order: codes, scales and zeros hold the
 *    columns in that order (column j is input channel perm[j]; quantize
 *    W[:, perm], made by wq_permute_columns).  wq_linear_w4a16 then gathers
 *    x[:, perm] into its workspace before the multiply.  NULL: plain order.
 *  fmt = WQ_FMT_INT8_SYM_ROW:
 *    codes   int8 [n][k], 16-byte aligned; scales fp32 [n]; group = k.
 */
typedef struct {
  int32_t fmt;            /* wq_format                                        */
  int32_t group;
  int64_t n, k;
  const void* codes;
  const void* scales;
  const uint8_t* zeros;   /* INT4 only, else NULL                             */
  const float* scales2;   /* NF4 double quantization only, else NULL          */
  int32_t group2;
  int32_t reserved;
  const int32_t* perm;    /* INT4 act-order: device int32 [k], else NULL      */
} wq_weight;

/*
 * Group-wise weight quantization (one launch).
 *
 * bits = 4, symmetric = 0 (asymmetric INT4, [P5] section 2.3 with b = 4;
 * per-group granularity [P5] 2.2, group 128 [P1] 3.2):
 *   for each row r and group g of `group` consecutive k:
 *     lo = min(min w, 0), hi = max(max w, 0)     (the range holds float 0,
 *                                                 which the zero point encodes)
 *     s  = fp16((hi - lo) / 15)   (1.0 if that rounds to 0)
 *     z  = clamp(round(-lo / s), 0, 15)
 *     q  = clamp(round(w / s) + z, 0, 15)
 *   outputs: codes uint32 [n][k/8], scales fp16 [n][k/group],
 *   zeros uint8 [n][ceil((k/group)/2)] (layout as in wq_weight).
 *   group in {32, 64, 128}; k % group == 0.
 *
 * bits = 8, symmetric = 1, group = k (vector-wise INT8, one scale per output
 * feature, [P1] 2.1; symmetric formula [P5] 2.3):
 *     s = max|w[r,:]| / 127 (1.0 for an all-zero row),
 *     q = clamp(round(w / s), -127, 127)
 *   outputs: codes int8 [n][k], scales fp32 [n]; zeros must be NULL.
 *
 * w: fp16 or bf16 [n][k] (wdt), 16-byte aligned, k % 8 == 0.
 * Other (bits, symmetric, group) combinations return WQ_ERR_UNSUPPORTED.
 */
wq_status wq_quantize_groupwise(const void* w, int32_t wdt, int64_t n, int64_t k,
                                int32_t bits, int32_t group, int32_t symmetric,
                                void* codes, void* scales, uint8_t* zeros,
                                void* stream);

/*
 * NF4 blockwise quantization ([P1] sections 6.1-6.3, [P5] 6.1-6.2).
 *
 *   Blocks of `block` (64) consecutive elements of the row-major W:
 *     a = max|w| (fp32); code = number of the 15 level midpoints that w/a
 *     exceeds (nearest NF4 level, ties to the lower); a == 0 gives code 7.
 *   double_quant != 0: blocks of `block2` (256) consecutive absmax values,
 *     c2 = max(a)/127 (1.0 if 0), q8 = clamp(round(a/c2), 0, 127);
 *     absmax receives int8 q8 [nblocks], absmax_scale fp32 c2
 *     [ceil(nblocks/block2)].
 *   double_quant == 0: absmax receives fp32 a [nblocks]; absmax_scale must
 *     be NULL.
 *   codes: uint8 [n*k/2], two codes per byte, element 2j low nibble.
 *
 * w: fp16 or bf16, 16-byte aligned; n*k % block == 0; block == 64;
 * block2 == 256 when double_quant.
 */
wq_status wq_pack_nf4(const void* w, int32_t wdt, int64_t n, int64_t k,
                      int32_t block, int32_t double_quant, int32_t block2,
                      uint8_t* codes, void* absmax, float* absmax_scale,
                      void* stream);

/*
 * FP4 blockwise quantization, the FP4 variant of the NF4 path ([P1] 6.3
 * names bitsandbytes' NF4 and FP4 formats; the E2M1 layout, sign bit,
 * 2-bit exponent, 1-bit mantissa, is [P5] 7.2).  Arguments, blocks, absmax
 * and double quantization exactly as wq_pack_nf4; only the codes differ:
 *   code bit 3 = (w/a < 0); bits 0-2 = number of the 7 midpoints between
 *   adjacent E2M1 magnitudes {0, 1/2, 1, 3/2, 2, 3, 4, 6}/6 that |w/a|
 *   exceeds (nearest magnitude, ties to the lower); a == 0 gives code 0.
 * Code c decodes to wq_fp4_codebook()[c] * absmax (code 8 is -0).
 */
wq_status wq_pack_fp4(const void* w, int32_t wdt, int64_t n, int64_t k,
                      int32_t block, int32_t double_quant, int32_t block2,
                      uint8_t* codes, void* absmax, float* absmax_scale,
                      void* stream);

/*
 * The FP4 codebook (host call, no GPU): out[c] = E2M1 value of code c / 6
 * in fp32, exponent bias 1 (out[7] = 1, out[15] = -1, out[8] = -0).
 */
wq_status wq_fp4_codebook(float* out);

/*
 * The NF4 codebook the library uses (host call, no GPU): 16 fp32 levels,
 * ascending, out[0] = -1, out[7] = 0, out[15] = 1.  Level i > 7 is
 * PhiInv(p_i)/PhiInv(31/32) for p_i = 1/2 + (31/32 - 1/2) (i-7)/8, level
 * i < 7 is -PhiInv(q_i)/PhiInv(31/32) for q_i = 1/2 + (31/32 - 1/2)(7-i)/7
 * (quantiles at evenly spaced probabilities, [P1] 6.1).  `out` is host
 * memory of 16 floats.
 */
wq_status wq_nf4_codebook(float* out);

/*
 * Scratch bytes wq_linear_w4a16 needs for this (m, weight) pair: an
 * act-order weight needs m * k * 2 bytes (rounded up to 256) for the
 * gathered activations; every other weight needs none (0).  Returns 0 for
 * invalid arguments as well (the call itself then reports the error).
 */
size_t wq_linear_w4a16_workspace(int64_t m, const wq_weight* w);

/*
 * Fused dequantize-and-multiply (W4A16: 4-bit weights, 16-bit activations;
 * the weights are dequantized back to 16 bits and multiplied in 16-bit
 * with fp32 accumulation, [P1] section 5 opening, [P1] 6.2, [P2] 十一).
 *
 *   y[i][j] = sum_c x[i][c] * w_hat[j][c]
 *     INT4: w_hat = (q - z) * s, NF4 and FP4: w_hat = L[code] * a_hat
 *     (L the format's codebook), with fp32 accumulation.
 *
 * Decode-shaped calls (m <= 16) run a bandwidth-bound dequant-GEMV; larger
 * m runs an MFMA dequant-GEMM (the GEMV / GEMM kernel versions of [P1] 4.3).
 *
 * x: xdt in {WQ_F16, WQ_BF16}, [m][k], 16-byte aligned.  w: fmt INT4_ASYM
 * (group 128, 64 or 32: the group-size knob of [P5] 2.2 and [P1] 3.2), NF4
 * or FP4 (block 64).  y: ydt in {F16, BF16, F32}, [m][n].
 * workspace: at least wq_linear_w4a16_workspace(m, w) bytes, 256-byte
 * aligned (may be NULL when that is 0).  m >= 1; k % 128 == 0.  With
 * w->perm set (INT4 act-order) the activations are gathered into the
 * workspace first; NF4/FP4 with perm give WQ_ERR_UNSUPPORTED.
 */
wq_status wq_linear_w4a16(const void* x, int32_t xdt, int64_t m,
                          const wq_weight* w, void* y, int32_t ydt,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * The gate and up projections of a gated MLP block ([P3] step 4 lists the
 * gate, up and down projections of each block) as one call sharing x:
 *
 *   act = 0:  y_gate = x * W_gate_hat^T,  y_up = x * W_up_hat^T
 *             (each exactly what wq_linear_w4a16 computes for it);
 *   act = 1:  y_gate = silu(g) * u with silu(v) = v / (1 + exp(-v)), for
 *             m <= 16 with g, u those two products in fp32 (y_up is not
 *             written and may be NULL); for m > 16 with g, u the two GEMM
 *             outputs as stored in ydt (y_up is required: it receives u).
 *
 * For m <= 16 one pass streams both matrices with the activations staged
 * once; larger m runs the two GEMMs.
 *
 * x: xdt in {WQ_F16, WQ_BF16}, [m][k], 16-byte aligned.  w_gate, w_up: one
 * format for both -- INT4_ASYM (group 128, 64 or 32), NF4 or FP4 (block 64,
 * both with or both without double quantization) -- with equal n and k.
 * y_gate, y_up: ydt in {F16, BF16, F32}, [m][n] each (y_up may be NULL when
 * act = 1 and m <= 16).
 * Errors: WQ_ERR_SHAPE when n, k or the group size differ; WQ_ERR_NULL when
 * y_up is NULL for act = 0 or for act = 1 with m > 16; WQ_ERR_UNSUPPORTED
 * for mixed formats, INT8 weights, NF4/FP4 with double quantization on one
 * matrix only, act-order weights or act outside {0, 1}.  No workspace.
 */
wq_status wq_linear_w4a16_gate_up(const void* x, int32_t xdt, int64_t m,
                                  const wq_weight* w_gate, const wq_weight* w_up,
                                  int32_t act, void* y_gate, void* y_up, int32_t ydt,
                                  void* stream);

/*
 * LLM.int8() activation side ([P1] 2.1; threshold 6.0 in [P5] 6.1):
 *   outlier columns O = { c : |x[i][c]| > threshold for some row i }
 *     (strict); mask[c] = 1 for c in O else 0; idx = ascending list of O,
 *     *count = |O| (device int32).
 *   per row i: sx[i] = max_{c not in O} |x[i][c]| / 127 (1.0 if 0),
 *     qx[i][c] = clamp(round(x[i][c] / sx[i]), -127, 127), 0 for c in O.
 * x: fp16 [m][k], 16-byte aligned, k % 16 == 0.  mask uint8 [k] (16-byte
 * aligned), idx int32 [k], count int32 [1], qx int8 [m][k] (16-byte
 * aligned), sx fp32 [m].  threshold >= 0 (use +inf for no outliers).
 */
wq_status wq_int8_prepare_activations(const void* x, int64_t m, int64_t k,
                                      float threshold, uint8_t* mask,
                                      int32_t* idx, int32_t* count, int8_t* qx,
                                      float* sx, void* stream);

/* Scratch bytes of wq_linear_int8_decomp (mask, idx, count, qx, sx). */
size_t wq_linear_int8_decomp_workspace(int64_t m, int64_t k);

/*
 * LLM.int8() mixed-precision decomposition ([P1] 2.1):
 *   y = acc * sx[i] * sw[j] + sum_{c in O} x[i][c] * w16[j][c]
 *   acc[i][j] = sum_c qx[i][c] * qw[j][c]   (exact int32)
 *   w16 = fp16(fp32(qw) * sw)               (the int8 weights dequantized;
 *                                            no fp16 copy of W is kept)
 * x: fp16 [m][k], 16-byte aligned; w: fmt INT8_SYM_ROW with k % 128 == 0 and
 * k <= 133,143 (so that 127 * 127 * k, the largest possible |acc|, fits in
 * int32; larger k returns WQ_ERR_SHAPE); y: ydt in {F16, BF16, F32}
 * (acc * sx * sw plus the outlier sum in fp32, rounded once to ydt).
 * workspace: at least
 * wq_linear_int8_decomp_workspace(m, k) bytes, 256-byte aligned.
 * outlier_count (device int32, nullable) receives |O|; acc_out (device int32
 * [m][n], nullable) receives acc.
 */
wq_status wq_linear_int8_decomp(const void* x, int64_t m, const wq_weight* w,
                                float threshold, void* y, int32_t ydt,
                                void* workspace, size_t ws_bytes,
                                int32_t* outlier_count, int32_t* acc_out,
                                void* stream);

/*
 * wq_linear_int8_decomp for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops and harnesses that forbid
 * allocation): the same computation and kernels, with no workspace
 * argument.  The scratch (outlier mask and list, count, int8 activations,
 * row scales) is a device array of WQ_INT8_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; the call allocates and
 * frees nothing.  Arguments, results and errors as wq_linear_int8_decomp;
 * calls whose wq_linear_int8_decomp_workspace(m, k) exceeds the array return
 * WQ_ERR_WORKSPACE, and WQ_ERR_HIP also reports a failure to find the
 * array on the current device.  Every call on one GPU uses that GPU's
 * array and leaves its contents behind (no byte of it needs to start at
 * zero): calls that overlap on one GPU -- on different streams or from
 * different host threads -- race, and the caller must order them.
 */
#define WQ_INT8_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
wq_status wq_linear_int8_decomp_noalloc(const void* x, int64_t m, const wq_weight* w,
                                        float threshold, void* y, int32_t ydt,
                                        int32_t* outlier_count, int32_t* acc_out,
                                        void* stream);

/*
 * Column gather (act-order reordering, [P1] 3.2, [P4] 3.2):
 *   dst[r][j] = src[r][perm[j]],  r < rows, j < k.
 * src, dst: dt in {F16, BF16} [rows][k], distinct buffers, dst 16-byte
 * aligned; perm: device int32 [k], a permutation of 0..k-1 (entries outside
 * [0, k) are clamped: wrong values, no out-of-bounds access); k % 8 == 0.
 */
wq_status wq_permute_columns(const void* src, int32_t dt, int64_t rows, int64_t k,
                             const int32_t* perm, void* dst, void* stream);

/*
 * Column scaling for SmoothQuant-style W8A8 ([P1] section 5: the
 * activation range is moved into the weights by a per-channel s, folded
 * offline; then the INT8 product runs with no outlier columns, i.e.
 * wq_linear_int8_decomp with threshold = +inf):
 *   dst[r][c] = round16(src[r][c] * scale[c])  (fp32 product, one rounding)
 * Use scale = s on the weights before wq_quantize_groupwise(bits = 8) and
 * scale = 1/s on the activations.  src, dst: dt in {F16, BF16} [rows][k],
 * 16-byte aligned, may be the same buffer; scale: device fp32 [k];
 * k % 8 == 0.
 */
wq_status wq_scale_columns(const void* src, int32_t dt, int64_t rows, int64_t k,
                           const float* scale, void* dst, void* stream);

/*
 * Dequantize a whole weight into 16-bit values (a test and debugging hook;
 * an act-order weight comes out in its stored column order):
 * INT4: fp(q - z) * s rounded to odt; NF4, FP4: L[code] * a_hat rounded to odt;
 * INT8: fp32(q) * s rounded to odt.  out: odt in {F16, BF16} [n][k].
 */
wq_status wq_dequantize(const wq_weight* w, void* out, int32_t odt, void* stream);

/* Static, human-readable name of a status code. */
const char* wq_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
