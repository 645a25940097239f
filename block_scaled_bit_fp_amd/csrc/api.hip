// api.hip -- the C ABI of libbsfp (declared in include/bsfp.h).
//
// Every entry point validates its arguments on the host before anything is
// enqueued, never throws, and reports failures as a status plus a
// thread-local message (a C++ exception crossing a language bridge
// terminates the process, and an unsupported group size that throws ends a
// whole test binary: "feat(quant): backend quantization capability table and
// load-time convert-or-reject policy", Gate impact).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "bsfp_device.hpp"
#include "bsfp_internal.hpp"

namespace bsfp {

namespace {

thread_local char g_err[512] = "";

bsfp_status fail(bsfp_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bsfp_status ok() {
  g_err[0] = '\0';
  return BSFP_OK;
}

bsfp_status device_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSFP_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const char* mode_name(int mode) {
  switch (mode) {
    case BSFP_AFFINE: return "affine";
    case BSFP_MXFP4: return "mxfp4";
    case BSFP_NVFP4: return "nvfp4";
    case BSFP_MXFP8: return "mxfp8";
    default: return "unknown";
  }
}

// A format variant (MXFP8, or affine other than 4-bit group 64).
bool is_variant(const bsfp_qtensor* q) {
  return format_id(q->mode, q->bits, q->group_size) >= FMT_MXFP8;
}

// Checks the descriptor of a quantized tensor; need_data: its code/scale
// buffers must be present (non-empty tensors).
bsfp_status check_qtensor(const bsfp_qtensor* q, const char* fn) {
  if (!q) return fail(BSFP_ERR_ARG, "%s: null tensor descriptor", fn);
  if (format_id(q->mode, q->bits, q->group_size) < 0)
    return fail(BSFP_ERR_UNSUPPORTED,
                "%s: unsupported format (mode %d, bits %d, group %d); supported: "
                "(affine, 4 or 8, 32/64/128), (mxfp4, 4, 32), (nvfp4, 4, 16), (mxfp8, 8, 32)",
                fn, (int)q->mode, (int)q->bits, (int)q->group_size);
  if (q->rows < 0 || q->cols < 0)
    return fail(BSFP_ERR_ARG, "%s: negative shape [%lld, %lld]", fn, (long long)q->rows,
                (long long)q->cols);
  if (q->cols % q->group_size)
    return fail(BSFP_ERR_ARG, "%s: cols %lld is not a multiple of the %s group size %d", fn,
                (long long)q->cols, mode_name(q->mode), (int)q->group_size);
  // element counts (rows * cols) are formed in int64 from here on
  if (q->rows > 0 && q->cols > 0 && q->rows > (int64_t(1) << 40) / q->cols)
    return fail(BSFP_ERR_UNSUPPORTED, "%s: [%lld, %lld] holds more than 2^40 elements", fn,
                (long long)q->rows, (long long)q->cols);
  if (q->rows > 0 && q->cols > 0) {
    if (!q->codes || !q->scales)
      return fail(BSFP_ERR_ARG, "%s: null codes or scales", fn);
    if (!aligned16(q->codes))
      return fail(BSFP_ERR_ARG, "%s: codes pointer is not 16-byte aligned", fn);
    if (q->mode == BSFP_AFFINE && !q->biases)
      return fail(BSFP_ERR_ARG, "%s: affine tensor without biases", fn);
  }
  return ok();
}

std::mutex g_cu_mutex;
int g_cu_count[64] = {0};
int g_max_lds[64] = {0};

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

thread_local LaunchEvents g_launch_events = {nullptr, nullptr};

LaunchEvents take_launch_events() {
  const LaunchEvents e = g_launch_events;
  g_launch_events = {nullptr, nullptr};
  return e;
}

int device_max_lds() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_max_lds[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        n <= 0)
      n = 64 * 1024;
    g_max_lds[dev] = n;
  }
  return g_max_lds[dev];
}

}  // namespace bsfp

// ---------------------------------------------------------------------------
// bsfp_qmm_noalloc: bsfp_qmm with the workspace in the library's own device
// memory, for callers that cannot allocate.  `scratch` is a file-scope device
// array (one copy per GPU, held until the process ends).  In host code its
// name is only a stand-in: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch_ptr, and
// only that pointer is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[BSFP_NOALLOC_WORKSPACE_BYTES];

namespace bsfp {
namespace {
std::mutex g_scratch_mutex;
void* g_scratch_ptr[64] = {nullptr};

// The device address of `scratch` on the current device (nullptr and a
// message on failure).
void* scratch_ptr(const char* fn, bsfp_status* st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = fail(BSFP_ERR_DEVICE, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= 64) {
    *st = fail(BSFP_ERR_UNSUPPORTED, "%s: device %d beyond the 64 the library tracks", fn, dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *st = fail(BSFP_ERR_DEVICE, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                 hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  *st = BSFP_OK;
  return g_scratch_ptr[dev];
}
}  // namespace
}  // namespace bsfp

using namespace bsfp;

extern "C" {

const char* bsfp_last_error(void) { return g_err; }

bsfp_status bsfp_time_next_launch(void* start_event, void* stop_event) {
  g_launch_events = {(hipEvent_t)start_event, (hipEvent_t)stop_event};
  return BSFP_OK;
}

const char* bsfp_version(void) { return "bsfp 0.1.0 (gfx950)"; }

bsfp_status bsfp_amax(const uint16_t* x, int64_t n, float* amax_out, bsfp_stream stream) {
  if (n < 0) return fail(BSFP_ERR_ARG, "bsfp_amax: negative n");
  if (!amax_out) return fail(BSFP_ERR_ARG, "bsfp_amax: null output");
  if (n > 0 && (!x || !aligned16(x)))
    return fail(BSFP_ERR_ARG, "bsfp_amax: x is null or not 16-byte aligned");
  return device_status(launch_amax(x, n, amax_out, (hipStream_t)stream), "bsfp_amax");
}

static_assert(BSFP_QUANTIZE_WS_BYTES == kAmaxParts * sizeof(float),
              "the quantize workspace holds one partial maximum per amax workgroup");

// bsfp_quantize, bsfp_quantize_sr (rbits != nullptr: stochastic rounding) and
// bsfp_quantize_ws (parts != nullptr: NVFP4 GS_COMPUTE reduces the amax from
// partial maxima there; checked by the caller).
static bsfp_status quantize_impl(const uint16_t* x, const bsfp_qtensor* q, int32_t gs,
                                 const uint32_t* rbits, bsfp_stream stream, const char* fn,
                                 float* parts = nullptr) {
  bsfp_status st = check_qtensor(q, fn);
  if (st != BSFP_OK) return st;
  const int64_t n = q->rows * q->cols;
  hipStream_t s = (hipStream_t)stream;
  if (q->mode == BSFP_NVFP4) {
    if (gs < BSFP_GS_NONE || gs > BSFP_GS_GIVEN)
      return fail(BSFP_ERR_ARG, "%s: bad global-scale flag %d", fn, (int)gs);
    if (gs != BSFP_GS_NONE && !q->global_scale)
      return fail(BSFP_ERR_ARG, "%s: nvfp4 global scale requested but global_scale is null", fn);
    if (gs == BSFP_GS_COMPUTE && !q->amax)
      return fail(BSFP_ERR_ARG, "%s: BSFP_GS_COMPUTE needs an amax buffer", fn);
  }
  if (n > 0 && (!x || !aligned16(x)))
    return fail(BSFP_ERR_ARG, "%s: x is null or not 16-byte aligned", fn);
  const int64_t n_words = n / 8;
  hipError_t e = hipSuccess;
  switch (q->mode) {
    case BSFP_NVFP4:
      if (gs == BSFP_GS_COMPUTE && parts && n > 0) {
        e = launch_amax_quantize_nvfp4(x, n, q->codes, (uint8_t*)q->scales, parts, q->amax,
                                       q->global_scale, s, rbits);
      } else if (gs == BSFP_GS_COMPUTE) {
        e = launch_amax(x, n, q->amax, s);
        if (e == hipSuccess)
          e = launch_quantize_nvfp4(x, n_words, q->codes, (uint8_t*)q->scales, q->amax, 1,
                                    q->global_scale, s, rbits);
      } else if (n_words > 0) {
        e = launch_quantize_nvfp4(x, n_words, q->codes, (uint8_t*)q->scales,
                                  gs == BSFP_GS_GIVEN ? q->global_scale : nullptr, 0, nullptr, s,
                                  rbits);
      }
      break;
    case BSFP_MXFP4:
      if (n_words > 0)
        e = launch_quantize_mxfp4(x, n_words, q->codes, (uint8_t*)q->scales, s, rbits);
      break;
    default:
      if (is_variant(q))
        e = launch_quantize_variant(x, *q, s);
      else if (n_words > 0)
        e = launch_quantize_affine(x, n_words, q->codes, (uint16_t*)q->scales, q->biases, s);
      break;
  }
  return device_status(e, fn);
}

bsfp_status bsfp_quantize(const uint16_t* x, const bsfp_qtensor* q, int32_t gs,
                          bsfp_stream stream) {
  return quantize_impl(x, q, gs, nullptr, stream, "bsfp_quantize");
}

bsfp_status bsfp_quantize_sr(const uint16_t* x, const bsfp_qtensor* q, int32_t gs,
                             const uint32_t* rbits, bsfp_stream stream) {
  if (q && q->mode != BSFP_NVFP4 && q->mode != BSFP_MXFP4)
    return fail(BSFP_ERR_UNSUPPORTED,
                "bsfp_quantize_sr: stochastic rounding applies to nvfp4 and mxfp4 only");
  if (q && q->rows * q->cols > 0 && (!rbits || !aligned16(rbits)))
    return fail(BSFP_ERR_ARG, "bsfp_quantize_sr: rbits is null or not 16-byte aligned");
  return quantize_impl(x, q, gs, rbits, stream, "bsfp_quantize_sr");
}

bsfp_status bsfp_quantize_ws(const uint16_t* x, const bsfp_qtensor* q, int32_t gs,
                             const uint32_t* rbits, void* workspace, int64_t workspace_bytes,
                             bsfp_stream stream) {
  const char* fn = "bsfp_quantize_ws";
  bsfp_status st = check_qtensor(q, fn);  // also bounds rows * cols
  if (st != BSFP_OK) return st;
  const bool nonempty = q->rows * q->cols > 0;
  if (rbits) {  // the checks of bsfp_quantize_sr
    if (q->mode != BSFP_NVFP4 && q->mode != BSFP_MXFP4)
      return fail(BSFP_ERR_UNSUPPORTED,
                  "%s: stochastic rounding applies to nvfp4 and mxfp4 only", fn);
    if (nonempty && !aligned16(rbits))
      return fail(BSFP_ERR_ARG, "%s: rbits is not 16-byte aligned", fn);
  }
  const bool uses_ws = q->mode == BSFP_NVFP4 && gs == BSFP_GS_COMPUTE;
  if (uses_ws) {
    if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 4 != 0)
      return fail(BSFP_ERR_ARG, "%s: workspace is null or not 4-byte aligned", fn);
    if (workspace_bytes < BSFP_QUANTIZE_WS_BYTES)
      return fail(BSFP_ERR_ARG, "%s: workspace of %lld bytes, %d needed", fn,
                  (long long)workspace_bytes, (int)BSFP_QUANTIZE_WS_BYTES);
  }
  return quantize_impl(x, q, gs, rbits, stream, fn,
                       uses_ws ? static_cast<float*>(workspace) : nullptr);
}

bsfp_status bsfp_dequantize(const bsfp_qtensor* q, uint16_t* out, bsfp_stream stream) {
  bsfp_status st = check_qtensor(q, "bsfp_dequantize");
  if (st != BSFP_OK) return st;
  if (q->rows * q->cols > 0 && (!out || !aligned16(out)))
    return fail(BSFP_ERR_ARG, "bsfp_dequantize: out is null or not 16-byte aligned");
  return device_status(launch_dequantize(*q, out, (hipStream_t)stream), "bsfp_dequantize");
}

bsfp_status bsfp_qmv(const uint16_t* x, int64_t M, const bsfp_qtensor* w, uint16_t* y,
                     bsfp_stream stream) {
  bsfp_status st = check_qtensor(w, "bsfp_qmv");
  if (st != BSFP_OK) return st;
  if (M < 1 || M > 8) return fail(BSFP_ERR_ARG, "bsfp_qmv: M = %lld outside 1..8", (long long)M);
  if (w->cols == 0) return fail(BSFP_ERR_ARG, "bsfp_qmv: K must be positive");
  if (!x || !aligned16(x)) return fail(BSFP_ERR_ARG, "bsfp_qmv: x is null or not 16-byte aligned");
  if (w->rows > 0 && !y) return fail(BSFP_ERR_ARG, "bsfp_qmv: null y");
  if (is_variant(w) && !qmv_variant_supported((int)M, *w))
    return fail(BSFP_ERR_UNSUPPORTED,
                "bsfp_qmv: %s %d-bit group %d needs x of at most 64 KB and K < 2^28 "
                "(M = %lld, K = %lld)", mode_name(w->mode), (int)w->bits, (int)w->group_size,
                (long long)M, (long long)w->cols);
  return device_status(launch_qmv(x, (int)M, *w, y, (hipStream_t)stream), "bsfp_qmv");
}

bsfp_status bsfp_qmv_batch(const uint16_t* x, int64_t M, const bsfp_qtensor* const* w,
                           int32_t count, uint16_t* const* y, bsfp_stream stream) {
  if (count < 1 || count > BSFP_QMV_BATCH_MAX)
    return fail(BSFP_ERR_ARG, "bsfp_qmv_batch: count = %d outside 1..%d", (int)count,
                BSFP_QMV_BATCH_MAX);
  if (!w || !y) return fail(BSFP_ERR_ARG, "bsfp_qmv_batch: null descriptor or output array");
  for (int i = 0; i < count; ++i)
    if (!w[i]) return fail(BSFP_ERR_ARG, "bsfp_qmv_batch: descriptor %d is null", i);
  for (int i = 0; i < count; ++i) {
    bsfp_status st = check_qtensor(w[i], "bsfp_qmv_batch");
    if (st != BSFP_OK) return st;
    if (w[i]->mode != w[0]->mode || w[i]->bits != w[0]->bits ||
        w[i]->group_size != w[0]->group_size || w[i]->cols != w[0]->cols)
      return fail(BSFP_ERR_ARG,
                  "bsfp_qmv_batch: matrix %d differs from matrix 0 in format or K", i);
    if (w[i]->rows > 0 && (!y[i] || !aligned16(y[i])))
      return fail(BSFP_ERR_ARG, "bsfp_qmv_batch: output %d is null or not 16-byte aligned", i);
  }
  if (M < 1 || M > 8)
    return fail(BSFP_ERR_ARG, "bsfp_qmv_batch: M = %lld outside 1..8", (long long)M);
  if (w[0]->cols == 0) return fail(BSFP_ERR_ARG, "bsfp_qmv_batch: K must be positive");
  if (!x || !aligned16(x))
    return fail(BSFP_ERR_ARG, "bsfp_qmv_batch: x is null or not 16-byte aligned");
  if (is_variant(w[0]) && !qmv_variant_supported((int)M, *w[0]))
    return fail(BSFP_ERR_UNSUPPORTED,
                "bsfp_qmv_batch: %s %d-bit group %d needs x of at most 64 KB and K < 2^28 "
                "(M = %lld, K = %lld)", mode_name(w[0]->mode), (int)w[0]->bits,
                (int)w[0]->group_size, (long long)M, (long long)w[0]->cols);
  return device_status(launch_qmv_batch(x, (int)M, w, y, count, (hipStream_t)stream),
                       "bsfp_qmv_batch");
}

size_t bsfp_qmm_workspace_bytes(int32_t mode, int64_t M, int64_t K, int32_t act) {
  if (mode < BSFP_AFFINE || mode > BSFP_NVFP4 || M < 0 || K < 0) return 0;
  if (act != BSFP_ACT_BF16 && act != BSFP_ACT_SAME) return 0;
  return qmm_workspace_bytes(mode, M, K, act);
}

// Argument checks of bsfp_qmm and bsfp_qmm_noalloc (everything but the
// workspace).  *done is set when the call has nothing to compute.
static bsfp_status check_qmm(const uint16_t* x, int64_t M, const bsfp_qtensor* w, int32_t act,
                             const uint16_t* y, const char* fn, bool* done) {
  *done = false;
  bsfp_status st = check_qtensor(w, fn);
  if (st != BSFP_OK) return st;
  if (is_variant(w))
    return fail(BSFP_ERR_UNSUPPORTED,
                "%s: %s %d-bit group %d runs on the dense path (bsfp_qmm_dense)", fn,
                mode_name(w->mode), (int)w->bits, (int)w->group_size);
  if (M < 0) return fail(BSFP_ERR_ARG, "%s: negative M", fn);
  if (act != BSFP_ACT_BF16 && act != BSFP_ACT_SAME)
    return fail(BSFP_ERR_ARG, "%s: bad activation mode %d", fn, (int)act);
  if (M == 0 || w->rows == 0) {
    *done = true;
    return ok();
  }
  if (w->cols == 0) return fail(BSFP_ERR_ARG, "%s: K must be positive", fn);
  if (!x || !aligned16(x)) return fail(BSFP_ERR_ARG, "%s: x is null or not 16-byte aligned", fn);
  if (!y || !aligned16(y)) return fail(BSFP_ERR_ARG, "%s: y is null or not 16-byte aligned", fn);
  if (w->cols % 64)
    return fail(BSFP_ERR_UNSUPPORTED, "%s: K = %lld is not a multiple of 64", fn,
                (long long)w->cols);
  if ((reinterpret_cast<uintptr_t>(w->scales) & 3) ||
      (w->biases && (reinterpret_cast<uintptr_t>(w->biases) & 3)))
    return fail(BSFP_ERR_ARG, "%s: scales and biases must be 4-byte aligned", fn);
  if (act == BSFP_ACT_SAME && w->mode == BSFP_AFFINE)
    return fail(BSFP_ERR_UNSUPPORTED,
                "%s: BSFP_ACT_SAME is supported for nvfp4 and mxfp4 weights only", fn);
  if (M > (1 << 30) || w->rows > (1 << 30))
    return fail(BSFP_ERR_UNSUPPORTED, "%s: M or N beyond 2^30", fn);
  // every launch shape keeps its grid under 2^32 threads up to 2^33 outputs
  if ((uint64_t)M * (uint64_t)w->rows > (1ULL << 33))
    return fail(BSFP_ERR_UNSUPPORTED, "%s: M * N = %llu beyond 2^33", fn,
                (unsigned long long)M * (unsigned long long)w->rows);
  // the GEMM addresses a 256-row activation tile with 32-bit byte offsets
  if (w->cols > (1 << 22))
    return fail(BSFP_ERR_UNSUPPORTED, "%s: K = %lld beyond 2^22", fn, (long long)w->cols);
  return ok();
}

bsfp_status bsfp_qmm(const uint16_t* x, int64_t M, const bsfp_qtensor* w, int32_t act,
                     void* workspace, size_t workspace_bytes, uint16_t* y, bsfp_stream stream) {
  bool done = false;
  const bsfp_status st = check_qmm(x, M, w, act, y, "bsfp_qmm", &done);
  if (st != BSFP_OK || done) return st;
  const size_t need = qmm_workspace_bytes(w->mode, M, w->cols, act);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(BSFP_ERR_ARG, "bsfp_qmm: workspace needs %zu bytes (16-byte aligned), got %zu",
                need, workspace_bytes);
  return device_status(launch_qmm(x, M, *w, act, workspace, y, (hipStream_t)stream), "bsfp_qmm");
}

bsfp_status bsfp_qmm_noalloc(const uint16_t* x, int64_t M, const bsfp_qtensor* w, int32_t act,
                             uint16_t* y, bsfp_stream stream) {
  bool done = false;
  bsfp_status st = check_qmm(x, M, w, act, y, "bsfp_qmm_noalloc", &done);
  if (st != BSFP_OK || done) return st;
  const size_t need = qmm_workspace_bytes(w->mode, M, w->cols, act);
  if (need > (size_t)BSFP_NOALLOC_WORKSPACE_BYTES)
    return fail(BSFP_ERR_UNSUPPORTED,
                "bsfp_qmm_noalloc: this product needs a %zu-byte workspace, beyond the %zu "
                "bytes of the library's static one (M = %lld, K = %lld); use bsfp_qmm with a "
                "caller workspace", need, (size_t)BSFP_NOALLOC_WORKSPACE_BYTES, (long long)M,
                (long long)w->cols);
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_ptr("bsfp_qmm_noalloc", &st);
    if (!ws) return st;
  }
  return device_status(launch_qmm(x, M, *w, act, ws, y, (hipStream_t)stream),
                       "bsfp_qmm_noalloc");
}

size_t bsfp_qmm_dense_scratch_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return (size_t)rows * (size_t)cols * 2;
}

bsfp_status bsfp_qmm_dense(const uint16_t* x, int64_t M, const bsfp_qtensor* w, void* scratch,
                           size_t scratch_bytes, uint16_t* y, bsfp_stream stream) {
  bsfp_status st = check_qtensor(w, "bsfp_qmm_dense");
  if (st != BSFP_OK) return st;
  if (M < 0) return fail(BSFP_ERR_ARG, "bsfp_qmm_dense: negative M");
  if (M == 0 || w->rows == 0) return ok();
  if (w->cols == 0) return fail(BSFP_ERR_ARG, "bsfp_qmm_dense: K must be positive");
  if (!x || !aligned16(x))
    return fail(BSFP_ERR_ARG, "bsfp_qmm_dense: x is null or not 16-byte aligned");
  if (!y || !aligned16(y))
    return fail(BSFP_ERR_ARG, "bsfp_qmm_dense: y is null or not 16-byte aligned");
  if (w->cols % 64)
    return fail(BSFP_ERR_UNSUPPORTED, "bsfp_qmm_dense: K = %lld is not a multiple of 64",
                (long long)w->cols);
  if (M > (1 << 30) || w->rows > (1 << 30))
    return fail(BSFP_ERR_UNSUPPORTED, "bsfp_qmm_dense: M or N beyond 2^30");
  if ((uint64_t)M * (uint64_t)w->rows > (1ULL << 33))
    return fail(BSFP_ERR_UNSUPPORTED, "bsfp_qmm_dense: M * N = %llu beyond 2^33",
                (unsigned long long)M * (unsigned long long)w->rows);
  if (w->cols > (1 << 22))
    return fail(BSFP_ERR_UNSUPPORTED, "bsfp_qmm_dense: K = %lld beyond 2^22",
                (long long)w->cols);
  const size_t need = bsfp_qmm_dense_scratch_bytes(w->rows, w->cols);
  if (!scratch || scratch_bytes < need || !aligned16(scratch))
    return fail(BSFP_ERR_ARG,
                "bsfp_qmm_dense: scratch needs %zu bytes (16-byte aligned), got %zu", need,
                scratch_bytes);
  return device_status(launch_qmm_dense(x, M, *w, scratch, y, (hipStream_t)stream),
                       "bsfp_qmm_dense");
}

}  // extern "C"
