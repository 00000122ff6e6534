// C ABI of libwq: argument validation, schedule choice, launch.
//
// Every check runs before the first HIP call, so an error other than
// WQ_ERR_HIP means nothing was enqueued.  No C++ exception crosses the ABI.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "internal.h"

using namespace wq;

namespace {

// Size limits: every dimension below 2^23 and every matrix at most 2^34
// elements, so every launch's grid stays within 32-bit work-item counts.
constexpr int64_t kMaxDim = int64_t(1) << 23;
constexpr int64_t kMaxElems = int64_t(1) << 34;
// LLM.int8: the int32 accumulator holds 127 * 127 * k exactly for k up to
// this bound (k multiples of 128: 133,120 at most).
constexpr int64_t kMaxInt8K = ((int64_t(1) << 31) - 1) / (127 * 127);

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool is16(int32_t dt) { return dt == WQ_F16 || dt == WQ_BF16; }
bool is_out(int32_t dt) { return dt == WQ_F16 || dt == WQ_BF16 || dt == WQ_F32; }
uintptr_t dt_bytes(int32_t dt) { return dt == WQ_F32 ? 4 : 2; }

wq_status hip_status(hipError_t e) { return e == hipSuccess ? WQ_OK : WQ_ERR_HIP; }

bool sizes_ok(int64_t n, int64_t k) {
  return n >= 1 && k >= 1 && n < kMaxDim && k < kMaxDim && n <= kMaxElems / k;
}

// Validates a weight descriptor for the given use.  `linear_w4` restricts to
// the formats and group sizes wq_linear_w4a16 runs.
wq_status check_weight(const wq_weight* w, bool linear_w4) {
  if (w == nullptr || w->codes == nullptr || w->scales == nullptr) return WQ_ERR_NULL;
  if (!sizes_ok(w->n, w->k)) return WQ_ERR_SHAPE;
  if (!aligned(w->codes, 16)) return WQ_ERR_ALIGN;
  if (w->perm != nullptr) {
    if (w->fmt != WQ_FMT_INT4_ASYM) return WQ_ERR_UNSUPPORTED;   // act-order is INT4 only
    if (!aligned(w->perm, 4)) return WQ_ERR_ALIGN;
  }
  switch (w->fmt) {
    case WQ_FMT_INT4_ASYM:
      if (w->zeros == nullptr) return WQ_ERR_NULL;
      if (w->group != 32 && w->group != 64 && w->group != 128) return WQ_ERR_UNSUPPORTED;
      if (w->k % w->group != 0 || w->k % 8 != 0) return WQ_ERR_SHAPE;
      if (!aligned(w->scales, 2)) return WQ_ERR_ALIGN;
      return WQ_OK;
    case WQ_FMT_NF4:
    case WQ_FMT_FP4:
      if (w->group != 64) return WQ_ERR_UNSUPPORTED;
      if (w->scales2 != nullptr && w->group2 != 256) return WQ_ERR_UNSUPPORTED;
      if ((w->n * w->k) % 64 != 0 || w->k % 8 != 0) return WQ_ERR_SHAPE;
      if (w->scales2 == nullptr && !aligned(w->scales, 4)) return WQ_ERR_ALIGN;
      if (w->scales2 != nullptr && !aligned(w->scales2, 4)) return WQ_ERR_ALIGN;
      return WQ_OK;
    case WQ_FMT_INT8_SYM_ROW:
      if (linear_w4) return WQ_ERR_UNSUPPORTED;
      if (w->group != w->k || w->k % 16 != 0) return WQ_ERR_SHAPE;
      if (!aligned(w->scales, 4)) return WQ_ERR_ALIGN;
      return WQ_OK;
    default:
      return WQ_ERR_UNSUPPORTED;
  }
}

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// Workspace of wq_linear_w4a16: the activations gathered into the order of
// an act-order weight (m x k 16-bit values); none for any other weight.
size_t linear_ws_bytes(int64_t m, const wq_weight* w) {
  if (w->perm == nullptr) return 0;
  return round256((size_t)m * (size_t)w->k * 2);
}

// FP4 weights run the NF4 kernels with the FP4 level table.
const float* levels_for(const wq_weight* w) {
  return w->fmt == WQ_FMT_FP4 ? fp4_levels() : nf4_levels();
}
wq_weight kernel_view(const wq_weight* w) {
  wq_weight c = *w;
  if (c.fmt == WQ_FMT_FP4) c.fmt = WQ_FMT_NF4;
  return c;
}

}  // namespace

extern "C" {

const char* wq_status_string(int32_t status) {
  switch (status) {
    case WQ_OK: return "WQ_OK";
    case WQ_ERR_NULL: return "WQ_ERR_NULL: a required pointer is NULL";
    case WQ_ERR_SHAPE: return "WQ_ERR_SHAPE: sizes do not fit the format";
    case WQ_ERR_ALIGN: return "WQ_ERR_ALIGN: a pointer misses its alignment";
    case WQ_ERR_UNSUPPORTED: return "WQ_ERR_UNSUPPORTED: combination not implemented";
    case WQ_ERR_WORKSPACE: return "WQ_ERR_WORKSPACE: workspace missing or too small";
    case WQ_ERR_HIP: return "WQ_ERR_HIP: kernel launch failed";
    default: return "unknown wq_status";
  }
}

wq_status wq_fp4_codebook(float* out) {
  if (out == nullptr) return WQ_ERR_NULL;
  const float* l = fp4_levels();
  for (int i = 0; i < 16; ++i) out[i] = l[i];
  return WQ_OK;
}

wq_status wq_nf4_codebook(float* out) {
  if (out == nullptr) return WQ_ERR_NULL;
  const float* l = nf4_levels();
  for (int i = 0; i < 16; ++i) out[i] = l[i];
  return WQ_OK;
}

wq_status wq_quantize_groupwise(const void* w, int32_t wdt, int64_t n, int64_t k, int32_t bits,
                                int32_t group, int32_t symmetric, void* codes, void* scales,
                                uint8_t* zeros, void* stream) {
  if (w == nullptr || codes == nullptr || scales == nullptr) return WQ_ERR_NULL;
  if (!is16(wdt)) return WQ_ERR_UNSUPPORTED;
  if (!sizes_ok(n, k) || k % 8 != 0) return WQ_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(codes, 16)) return WQ_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bits == 4 && symmetric == 0) {
    if (zeros == nullptr) return WQ_ERR_NULL;
    if (group != 32 && group != 64 && group != 128) return WQ_ERR_UNSUPPORTED;
    if (k % group != 0) return WQ_ERR_SHAPE;
    if (!aligned(scales, 2)) return WQ_ERR_ALIGN;
    return hip_status(launch_quant_int4(w, wdt, n, k, group, static_cast<uint32_t*>(codes),
                                        static_cast<uint16_t*>(scales), zeros, s));
  }
  if (bits == 8 && symmetric == 1) {
    if (group != k) return WQ_ERR_UNSUPPORTED;
    if (zeros != nullptr) return WQ_ERR_UNSUPPORTED;
    if (!aligned(scales, 4)) return WQ_ERR_ALIGN;
    return hip_status(launch_quant_int8_rows(w, wdt, n, k, static_cast<int8_t*>(codes),
                                             static_cast<float*>(scales), s));
  }
  return WQ_ERR_UNSUPPORTED;
}

static wq_status pack_blockwise(const void* w, int32_t wdt, int64_t n, int64_t k, int32_t block,
                                int32_t double_quant, int32_t block2, uint8_t* codes,
                                void* absmax, float* absmax_scale, void* stream, bool fp4) {
  if (w == nullptr || codes == nullptr || absmax == nullptr) return WQ_ERR_NULL;
  if (!is16(wdt)) return WQ_ERR_UNSUPPORTED;
  if (block != 64) return WQ_ERR_UNSUPPORTED;
  if (double_quant) {
    if (absmax_scale == nullptr) return WQ_ERR_NULL;
    if (block2 != 256) return WQ_ERR_UNSUPPORTED;
    if (!aligned(absmax_scale, 4)) return WQ_ERR_ALIGN;
  } else {
    if (absmax_scale != nullptr) return WQ_ERR_UNSUPPORTED;
    if (!aligned(absmax, 4)) return WQ_ERR_ALIGN;
  }
  if (!sizes_ok(n, k) || (n * k) % 64 != 0) return WQ_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(codes, 16)) return WQ_ERR_ALIGN;
  return hip_status(launch_pack_nf4(w, wdt, n * k, double_quant ? 1 : 0,
                                    fp4 ? fp4_thresholds() : nf4_thresholds(), codes, absmax,
                                    absmax_scale, static_cast<hipStream_t>(stream), fp4));
}

wq_status wq_pack_nf4(const void* w, int32_t wdt, int64_t n, int64_t k, int32_t block,
                      int32_t double_quant, int32_t block2, uint8_t* codes, void* absmax,
                      float* absmax_scale, void* stream) {
  return pack_blockwise(w, wdt, n, k, block, double_quant, block2, codes, absmax, absmax_scale,
                        stream, false);
}

wq_status wq_pack_fp4(const void* w, int32_t wdt, int64_t n, int64_t k, int32_t block,
                      int32_t double_quant, int32_t block2, uint8_t* codes, void* absmax,
                      float* absmax_scale, void* stream) {
  return pack_blockwise(w, wdt, n, k, block, double_quant, block2, codes, absmax, absmax_scale,
                        stream, true);
}

size_t wq_linear_w4a16_workspace(int64_t m, const wq_weight* w) {
  if (m < 1 || m >= kMaxDim || check_weight(w, true) != WQ_OK) return 0;
  return linear_ws_bytes(m, w);
}

wq_status wq_linear_w4a16(const void* x, int32_t xdt, int64_t m, const wq_weight* w, void* y,
                          int32_t ydt, void* workspace, size_t ws_bytes, void* stream) {
  if (x == nullptr || y == nullptr) return WQ_ERR_NULL;
  const wq_status ws = check_weight(w, true);
  if (ws != WQ_OK) return ws;
  if (!is16(xdt) || !is_out(ydt)) return WQ_ERR_UNSUPPORTED;
  if (m < 1 || m >= kMaxDim || m > kMaxElems / w->k || m > kMaxElems / w->n)
    return WQ_ERR_SHAPE;
  if (w->k % 128 != 0) return WQ_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, dt_bytes(ydt))) return WQ_ERR_ALIGN;
  const wq_weight kv = kernel_view(w);
  const W4Plan plan = plan_w4a16(m, &kv);
  const size_t need = linear_ws_bytes(m, w);
  if (need > 0) {
    if (workspace == nullptr || ws_bytes < need) return WQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return WQ_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w->perm != nullptr) {
    // act-order: x[:, perm] into the workspace, then the plain linear on it
    void* xp = workspace;
    const hipError_t e = launch_permute_cols(static_cast<const uint16_t*>(x), m, w->k, w->perm,
                                             static_cast<uint16_t*>(xp), s);
    if (e != hipSuccess) return WQ_ERR_HIP;
    x = xp;
  }
  return hip_status(launch_w4a16(x, xdt, m, &kv, levels_for(w), y, ydt, plan, s));
}

wq_status wq_linear_w4a16_gate_up(const void* x, int32_t xdt, int64_t m,
                                  const wq_weight* w_gate, const wq_weight* w_up, int32_t act,
                                  void* y_gate, void* y_up, int32_t ydt, void* stream) {
  if (x == nullptr || y_gate == nullptr) return WQ_ERR_NULL;
  if (act != 0 && act != 1) return WQ_ERR_UNSUPPORTED;
  if (act == 0 && y_up == nullptr) return WQ_ERR_NULL;
  wq_status st = check_weight(w_gate, true);
  if (st != WQ_OK) return st;
  st = check_weight(w_up, true);
  if (st != WQ_OK) return st;
  // both matrices in one format (INT4, NF4 or FP4), NF4/FP4 both with or both
  // without double quantization
  if (w_gate->fmt != w_up->fmt || w_gate->fmt == WQ_FMT_INT8_SYM_ROW) return WQ_ERR_UNSUPPORTED;
  if ((w_gate->scales2 == nullptr) != (w_up->scales2 == nullptr) ||
      (w_gate->scales2 != nullptr && w_gate->group2 != w_up->group2))
    return WQ_ERR_UNSUPPORTED;
  if (w_gate->perm != nullptr || w_up->perm != nullptr) return WQ_ERR_UNSUPPORTED;
  if (!is16(xdt) || !is_out(ydt)) return WQ_ERR_UNSUPPORTED;
  if (w_gate->n != w_up->n || w_gate->k != w_up->k || w_gate->group != w_up->group ||
      w_gate->k % 128 != 0)
    return WQ_ERR_SHAPE;
  if (m < 1 || m >= kMaxDim || m > kMaxElems / w_gate->k || m > kMaxElems / w_gate->n)
    return WQ_ERR_SHAPE;
  // act 1 with m > 16 runs two GEMMs and needs y_up to hold the up projection
  const bool up_out = act == 0 || m > 16;
  if (act == 1 && m > 16 && y_up == nullptr) return WQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y_gate, dt_bytes(ydt)) ||
      (up_out && !aligned(y_up, dt_bytes(ydt))))
    return WQ_ERR_ALIGN;
  const wq_weight kg = kernel_view(w_gate), ku = kernel_view(w_up);
  const W4Plan plan = plan_w4a16_pair(m, &kg, &ku);
  return hip_status(launch_w4a16_pair(x, xdt, m, &kg, &ku, levels_for(w_gate), act, y_gate,
                                      up_out ? y_up : nullptr, ydt, plan,
                                      static_cast<hipStream_t>(stream)));
}

size_t wq_linear_int8_decomp_workspace(int64_t m, int64_t k) {
  if (m < 1 || k < 16 || k % 16 != 0 || !sizes_ok(m, k)) return 0;
  // mask u8[k] | idx i32[k] | count i32 | qx i8[m][k] | sx f32[m], each 256-aligned
  auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
  return up((size_t)k) + up(4 * (size_t)k) + up(4) + up((size_t)m * (size_t)k) + up(4 * (size_t)m);
}

wq_status wq_int8_prepare_activations(const void* x, int64_t m, int64_t k, float threshold,
                                      uint8_t* mask, int32_t* idx, int32_t* count, int8_t* qx,
                                      float* sx, void* stream) {
  if (x == nullptr || mask == nullptr || idx == nullptr || count == nullptr || qx == nullptr ||
      sx == nullptr)
    return WQ_ERR_NULL;
  if (!sizes_ok(m, k) || k % 16 != 0) return WQ_ERR_SHAPE;
  if (!(threshold >= 0.0f)) return WQ_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(qx, 16) || !aligned(mask, 16) || !aligned(idx, 4) ||
      !aligned(count, 4) || !aligned(sx, 4))
    return WQ_ERR_ALIGN;
  return hip_status(launch_int8_prepare(static_cast<const uint16_t*>(x), m, k, threshold, mask,
                                        idx, count, qx, sx, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Argument checks shared by the two LLM.int8 entry points (everything but
// the workspace).
wq_status check_int8_decomp(const void* x, int64_t m, const wq_weight* w, float threshold,
                            const void* y, int32_t ydt, const int32_t* outlier_count,
                            const int32_t* acc_out) {
  if (x == nullptr || y == nullptr) return WQ_ERR_NULL;
  const wq_status st = check_weight(w, false);
  if (st != WQ_OK) return st;
  if (w->fmt != WQ_FMT_INT8_SYM_ROW) return WQ_ERR_UNSUPPORTED;
  if (!is_out(ydt)) return WQ_ERR_UNSUPPORTED;
  if (!sizes_ok(m, w->k) || m > kMaxElems / w->n || w->k % 128 != 0 || w->k > kMaxInt8K)
    return WQ_ERR_SHAPE;
  if (!(threshold >= 0.0f)) return WQ_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, dt_bytes(ydt))) return WQ_ERR_ALIGN;
  if (outlier_count != nullptr && !aligned(outlier_count, 4)) return WQ_ERR_ALIGN;
  if (acc_out != nullptr && !aligned(acc_out, 4)) return WQ_ERR_ALIGN;
  return WQ_OK;
}

// The two launches of the decomposition with the scratch at `base`
// (256-byte aligned, at least wq_linear_int8_decomp_workspace(m, k) bytes).
// Every scratch byte a kernel reads was written earlier in the same call, so
// the scratch needs no clearing.
wq_status run_int8_decomp(const void* x, int64_t m, const wq_weight* w, float threshold, void* y,
                          int32_t ydt, char* base, int32_t* outlier_count, int32_t* acc_out,
                          hipStream_t s) {
  auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t k = (size_t)w->k;
  uint8_t* mask = reinterpret_cast<uint8_t*>(base);
  int32_t* idx = reinterpret_cast<int32_t*>(base + up(k));
  int32_t* count = reinterpret_cast<int32_t*>(base + up(k) + up(4 * k));
  int8_t* qx = reinterpret_cast<int8_t*>(base + up(k) + up(4 * k) + up(4));
  float* sx = reinterpret_cast<float*>(base + up(k) + up(4 * k) + up(4) + up((size_t)m * k));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  hipError_t e = launch_int8_prepare(xp, m, w->k, threshold, mask, idx, count, qx, sx, s);
  if (e != hipSuccess) return WQ_ERR_HIP;
  e = launch_int8_gemm(xp, m, w, qx, sx, idx, count, y, ydt, acc_out, s);
  if (e != hipSuccess) return WQ_ERR_HIP;
  if (outlier_count != nullptr) {
    e = hipMemcpyAsync(outlier_count, count, sizeof(int32_t), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return WQ_ERR_HIP;
  }
  return WQ_OK;
}

// Scratch of wq_linear_int8_decomp_noalloc: a device array of fixed size,
// one copy per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: kernels get the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in `g_scratch`.
constexpr size_t kNoAllocScratchBytes = WQ_INT8_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address, or nullptr if it cannot be had.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

wq_status wq_linear_int8_decomp(const void* x, int64_t m, const wq_weight* w, float threshold,
                                void* y, int32_t ydt, void* workspace, size_t ws_bytes,
                                int32_t* outlier_count, int32_t* acc_out, void* stream) {
  const wq_status st = check_int8_decomp(x, m, w, threshold, y, ydt, outlier_count, acc_out);
  if (st != WQ_OK) return st;
  const size_t need = wq_linear_int8_decomp_workspace(m, w->k);
  if (workspace == nullptr || ws_bytes < need) return WQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return WQ_ERR_ALIGN;
  return run_int8_decomp(x, m, w, threshold, y, ydt, static_cast<char*>(workspace),
                         outlier_count, acc_out, static_cast<hipStream_t>(stream));
}

wq_status wq_linear_int8_decomp_noalloc(const void* x, int64_t m, const wq_weight* w,
                                        float threshold, void* y, int32_t ydt,
                                        int32_t* outlier_count, int32_t* acc_out,
                                        void* stream) {
  const wq_status st = check_int8_decomp(x, m, w, threshold, y, ydt, outlier_count, acc_out);
  if (st != WQ_OK) return st;
  if (wq_linear_int8_decomp_workspace(m, w->k) > kNoAllocScratchBytes) return WQ_ERR_WORKSPACE;
  void* base = device_scratch();
  if (base == nullptr) return WQ_ERR_HIP;
  return run_int8_decomp(x, m, w, threshold, y, ydt, static_cast<char*>(base), outlier_count,
                         acc_out, static_cast<hipStream_t>(stream));
}

wq_status wq_permute_columns(const void* src, int32_t dt, int64_t rows, int64_t k,
                             const int32_t* perm, void* dst, void* stream) {
  if (src == nullptr || perm == nullptr || dst == nullptr) return WQ_ERR_NULL;
  if (!is16(dt)) return WQ_ERR_UNSUPPORTED;
  if (src == dst) return WQ_ERR_UNSUPPORTED;                 // not in place
  if (!sizes_ok(rows, k) || k % 8 != 0) return WQ_ERR_SHAPE;
  if (!aligned(src, 2) || !aligned(dst, 16) || !aligned(perm, 4)) return WQ_ERR_ALIGN;
  return hip_status(launch_permute_cols(static_cast<const uint16_t*>(src), rows, k, perm,
                                        static_cast<uint16_t*>(dst),
                                        static_cast<hipStream_t>(stream)));
}

wq_status wq_scale_columns(const void* src, int32_t dt, int64_t rows, int64_t k,
                           const float* scale, void* dst, void* stream) {
  if (src == nullptr || scale == nullptr || dst == nullptr) return WQ_ERR_NULL;
  if (!is16(dt)) return WQ_ERR_UNSUPPORTED;
  if (!sizes_ok(rows, k) || k % 8 != 0) return WQ_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(scale, 4)) return WQ_ERR_ALIGN;
  return hip_status(launch_scale_cols(static_cast<const uint16_t*>(src), dt, rows, k, scale,
                                      static_cast<uint16_t*>(dst),
                                      static_cast<hipStream_t>(stream)));
}

wq_status wq_dequantize(const wq_weight* w, void* out, int32_t odt, void* stream) {
  if (out == nullptr) return WQ_ERR_NULL;
  const wq_status st = check_weight(w, false);
  if (st != WQ_OK) return st;
  if (!is16(odt)) return WQ_ERR_UNSUPPORTED;
  if (!aligned(out, 16)) return WQ_ERR_ALIGN;
  const wq_weight kv = kernel_view(w);
  return hip_status(
      launch_dequantize(&kv, levels_for(w), out, odt, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
