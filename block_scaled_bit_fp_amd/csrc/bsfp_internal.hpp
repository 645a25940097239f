// bsfp_internal.hpp -- launchers shared between the translation units of
// libbsfp.  Every launcher enqueues on `s`, assumes its arguments were
// validated by the C-ABI layer (api.hip) and returns hipGetLastError().
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bsfp.h"

namespace bsfp {

// The event pair set by bsfp_time_next_launch (cleared when taken).
struct LaunchEvents {
  hipEvent_t start, stop;
};
LaunchEvents take_launch_events();

// Launch of a main kernel: with the pending event pair when one is set.
template <typename F, typename... Args>
void launch_main(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, Args... args) {
  const LaunchEvents ev = take_launch_events();
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, ev.start, ev.stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

// Number of compute units of the current device (cached per device).
int device_cu_count();
// Largest LDS allocation one workgroup may make on the current device.
int device_max_lds();

// ---- amax / quantize / dequantize (quantize.hip)
hipError_t launch_amax(const uint16_t* x, int64_t n, float* amax_out, hipStream_t s);

// NVFP4 quantize.  g_src: NULL (no global scale, g = 1), or a device fp32
// holding g (g_src_is_amax == 0) or the tensor amax (g_src_is_amax == 1, g =
// amax/2688).  g_out (may be NULL) receives the g used.
// rbits: stochastic rounding with 8 random words per packed word (element
// order), or nullptr for round-to-nearest.
hipError_t launch_quantize_nvfp4(const uint16_t* x, int64_t n_words, uint32_t* codes,
                                 uint8_t* scales, const float* g_src, int g_src_is_amax,
                                 float* g_out, hipStream_t s, const uint32_t* rbits = nullptr);
// NVFP4 quantize + dequantize without the global scale into fp16 xhat
// [n_words * 8] (the qq GEMM's activation operand).
hipError_t launch_quantize_dequant_nvfp4_f16(const uint16_t* x, int64_t n_words, void* xhat,
                                             const float* g_src, int g_src_is_amax,
                                             float* g_out, hipStream_t s);
// As above with bf16 output (the x of the qq decode GEMV).
hipError_t launch_quantize_dequant_nvfp4_bf16(const uint16_t* x, int64_t n_words, void* xhat,
                                              const float* g_src, int g_src_is_amax,
                                              float* g_out, hipStream_t s);
// amax of x (as per-workgroup partial maxima in parts[kAmaxParts]) and the
// fp16 quantize-dequantize (launch_quantize_dequant_nvfp4_f16) with g = amax/2688 taken from the partials:
// two launches, no initialised memory, no atomics.  *amax_out and *g_out
// receive the tensor amax and g.  n % 8 == 0.
constexpr int kAmaxParts = 256;
hipError_t launch_amax_qdq_nvfp4_f16(const uint16_t* x, int64_t n, void* xhat, float* parts,
                                     float* amax_out, float* g_out, hipStream_t s);
// NVFP4 quantize with g = amax/2688, the amax taken as for
// launch_amax_qdq_nvfp4_f16 (partials in parts[kAmaxParts]; two launches, no
// initialised memory, no atomics).  *amax_out and *g_out receive the tensor
// amax and g.  n > 0, n % 16 == 0.
hipError_t launch_amax_quantize_nvfp4(const uint16_t* x, int64_t n, uint32_t* codes,
                                      uint8_t* scales, float* parts, float* amax_out,
                                      float* g_out, hipStream_t s,
                                      const uint32_t* rbits = nullptr);
// MXFP4 quantize, then exact dequantization to bf16.
hipError_t launch_quantize_dequant_mxfp4_bf16(const uint16_t* x, int64_t n_words, void* xhat,
                                              hipStream_t s);
hipError_t launch_quantize_mxfp4(const uint16_t* x, int64_t n_words, uint32_t* codes,
                                 uint8_t* scales, hipStream_t s, const uint32_t* rbits = nullptr);
// Quantize of the format variants (MXFP8, affine other than 4-bit group 64).
hipError_t launch_quantize_variant(const uint16_t* x, const bsfp_qtensor& q, hipStream_t s);
hipError_t launch_quantize_affine(const uint16_t* x, int64_t n_words, uint32_t* codes,
                                  uint16_t* scales, uint16_t* biases, hipStream_t s);

hipError_t launch_dequantize(const bsfp_qtensor& q, uint16_t* out, hipStream_t s);

// ---- qmv (qmv.hip)
// g2: optional second device scale multiplied into the output (the qq decode
// path passes g_x there).
hipError_t launch_qmv(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y,
                      hipStream_t s, const float* g2 = nullptr);
// The GEMV of `count` (<= 4) matrices that share x, K and the format, in one
// launch where the kernels allow (one row of x, base formats), else one
// launch per matrix.
hipError_t launch_qmv_batch(const uint16_t* x, int M, const bsfp_qtensor* const* ws,
                            uint16_t* const* ys, int count, hipStream_t s);
// qq decode GEMV: x is quantized with w's format (NVFP4: global scale from
// x's amax when w has one) while the GEMV stages it, and the products run on
// its exact dequantization, with alpha = g_x * g_w on the output.  Applies
// when qmv_qx_fusable(M, w) (x fits the GEMV's LDS copy, 1 <= M <= 8).
// The format variants' GEMV needs x in one LDS copy (M * K * 2 <= 64 KB).
bool qmv_variant_supported(int M, const bsfp_qtensor& w);
bool qmv_qx_fusable(int M, const bsfp_qtensor& w);
hipError_t launch_qmv_qx(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y,
                         hipStream_t s);

// ---- qmm (qmm.hip)
size_t qmm_workspace_bytes(int mode, int64_t M, int64_t K, int act);
hipError_t launch_qmm(const uint16_t* x, int64_t M, const bsfp_qtensor& w, int act,
                      void* ws, uint16_t* y, hipStream_t s);
hipError_t launch_qmm_dense(const uint16_t* x, int64_t M, const bsfp_qtensor& w, void* scratch,
                            uint16_t* y, hipStream_t s);

}  // namespace bsfp
