/*
 * bsfp.h -- C ABI of libbsfp: block-scaled 4-bit (and 8-bit) quantization
 * and quantized matmul on AMD Instinct MI355X (gfx950).
 *
 * Formats (the contract; with b = bits, element k of a row sits at bit
 * b*(k % (32/b)) of uint32 word k/(32/b): for 4 bits nibble k%8 of word k/8,
 * low nibble first, for 8 bits byte k%4 of word k/4; every tensor row-major
 * and contiguous):
 *
 *   BSFP_NVFP4  bits 4, group 16.  codes: E2M1 (FP4) packed 8 per uint32.
 *               scales: uint8 E4M3 (OCP E4M3FN) per 16-element group.
 *               global_scale: optional fp32 g = amax/(448*6) per tensor.
 *               Value = E2M1(c) * E4M3(S) * g.
 *               (native NVFP4 is group 16 / bits 4: "feat(quant): backend
 *               quantization capability table ...", Gate impact; 448 and 6
 *               are F8E4M3_MAX and F4E2M1_MAX in "mlx 0.30.7.3 -> 0.30.7.6",
 *               qqmm_utils.cu.)
 *   BSFP_MXFP4  bits 4, group 32.  codes: E2M1.  scales: uint8 E8M0
 *               (2^(S-127)).  Value = E2M1(c) * 2^(S-127).
 *               (MX scale arm of the bits == 4 quantizer: "perf(cuda): enable
 *               hardware NVFP4/MXFP4 conversion on Blackwell builds",
 *               Current Behavior.)
 *   BSFP_AFFINE bits 4, group 64.  codes: unsigned 0..15.  scales, biases:
 *               bf16 per group.  Value = s*q + b.
 *               (affine 4-bit / group 64: "epic: NVIDIA Volta (sm_70)
 *               inference acceleration program", Baseline.)
 * Format variants ("feat(quant): backend quantization capability table
 * ...", Context: the affine 4/8-bit and mxfp8 modes a ROCm backend runs;
 * Gate impact: its GEMV groups 32, 64, 128):
 *   BSFP_AFFINE bits 4 or 8, group 32, 64 or 128.  codes unsigned
 *               0..2^bits-1.  Value = s*q + b.
 *   BSFP_MXFP8  bits 8, group 32.  codes: E4M3 (OCP E4M3FN) bytes.  scales:
 *               uint8 E8M0.  Value = E4M3(c) * 2^(S-127).
 *   Entry points: bsfp_quantize, bsfp_dequantize, bsfp_qmv (x of at most
 *   64 KB, M * K * 2 bytes) and bsfp_qmm_dense take every format;
 *   bsfp_qmm takes the three base formats, bsfp_quantize_sr NVFP4 and
 *   MXFP4.  Elsewhere a variant returns BSFP_ERR_UNSUPPORTED.
 *
 *   Codes and scales are uint32 [rows, cols*bits/32] and [rows, cols/group]; the
 *   packed shape follows quantize_input in "mlx 0.30.7.3 -> 0.30.7.6"
 *   (qqmm.cpp): last dim = cols*bits/32.  Scales are linear (not the tiled
 *   layout that file builds for cuBLASLt).
 *
 * Quantization rounds to nearest even and saturates (cvt.rn.satfinite.
 * e2m1x2.f32 in "perf(cuda): enable hardware NVFP4/MXFP4 conversion on
 * Blackwell builds", Problem / Background).  Block scales:
 *   NVFP4  S = E4M3(bamax / (6*g)), codes = E2M1(x * (1 / (E4M3(S)*g)))
 *   MXFP4  e = floor(log2 bamax) - 2, codes = E2M1(x * 2^-e), S = e + 127
 *   AFFINE s = bf16((max-min)/15), b = bf16(min), q = rint((x-b)/s) in 0..15
 *          (b bits: 2^b - 1 in place of 15)
 *   MXFP8  e = floor(log2 bamax) - 8, codes = E4M3(x * 2^-e) (saturating at
 *          448, sign bit kept), S = e + 127 (OCP MX v1.0 for E4M3 elements)
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers of the current HIP device, 16-byte
 *     aligned; bf16 travels as uint16 bit patterns.  The caller owns and
 *     allocates every buffer (the library allocates no device memory, never
 *     frees, and never writes its inputs; the one exception is the static
 *     workspace of bsfp_qmm_noalloc, which lives in the library's code
 *     object on each GPU).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     with no host synchronization.
 *   - Functions never throw and never abort.  Argument errors are detected on
 *     the host before anything is enqueued and return BSFP_ERR_ARG; a
 *     format outside the ones above returns BSFP_ERR_UNSUPPORTED; a failed
 *     launch returns BSFP_ERR_DEVICE.  bsfp_last_error() then describes it.
 *     (A C++ exception crossing a language bridge terminates the process, and
 *     an unsupported group size that throws aborts a whole test binary:
 *     "feat(quant): backend quantization capability table ...", Gate impact.)
 */
#ifndef BSFP_H
#define BSFP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BSFP_AFFINE = 0, BSFP_MXFP4 = 1, BSFP_NVFP4 = 2, BSFP_MXFP8 = 3 } bsfp_mode;

typedef enum {
    BSFP_OK = 0,
    BSFP_ERR_ARG = 1,          /* bad pointer, size, alignment or shape */
    BSFP_ERR_UNSUPPORTED = 2,  /* (mode, bits, group) outside the contract */
    BSFP_ERR_DEVICE = 3        /* launch failure reported by the runtime */
} bsfp_status;

/* Activation handling of bsfp_qmm. */
typedef enum {
    BSFP_ACT_BF16 = 0,  /* weight-only: y = x . dq(W)^T, x stays bf16 */
    BSFP_ACT_SAME = 1   /* qq: x is quantized with W's mode first, then
                           y = alpha * dq0(q(x)) . dq0(W)^T */
} bsfp_act;

/* NVFP4 global-scale handling of bsfp_quantize. */
typedef enum {
    BSFP_GS_NONE = 0,     /* no global scale: g = 1 */
    BSFP_GS_COMPUTE = 1,  /* amax over the tensor -> *amax, g = amax/2688 ->
                             *global_scale (both must be non-NULL) */
    BSFP_GS_GIVEN = 2     /* use the device fp32 *global_scale as g */
} bsfp_gs;

typedef void* bsfp_stream; /* hipStream_t */

/* A quantized tensor: logical bf16 shape [rows, cols]. */
typedef struct {
    int32_t mode;          /* bsfp_mode */
    int32_t bits;          /* 4 */
    int32_t group_size;    /* 16 NVFP4, 32 MXFP4, 64 AFFINE */
    int64_t rows, cols;    /* cols % group_size == 0; rows * cols <= 2^40 */
    uint32_t* codes;       /* [rows, cols/8] */
    void* scales;          /* NVFP4/MXFP4 uint8, AFFINE bf16: [rows, cols/group] */
    uint16_t* biases;      /* AFFINE bf16 [rows, cols/group]; NULL otherwise */
    float* global_scale;   /* NVFP4 g (device fp32) or NULL for none */
    float* amax;           /* NVFP4 tensor amax (device fp32), written by
                              BSFP_GS_COMPUTE; may be NULL otherwise */
} bsfp_qtensor;

/*
 * bsfp_amax: *amax_out = max |x_i| over the n bf16 values at x (device
 * fp32).  The source of the NVFP4 global scale (alpha = amax_x*amax_w /
 * (448*6)^2: "mlx 0.30.7.3 -> 0.30.7.6", qqmm_utils.cu,
 * compute_qqmm_pointers).  n >= 0 (n == 0 gives 0).  Exact and independent
 * of reduction order.
 */
bsfp_status bsfp_amax(const uint16_t* x, int64_t n, float* amax_out,
                      bsfp_stream stream);

/*
 * bsfp_quantize: bf16 x [q->rows, q->cols] -> q->codes, q->scales (and
 * q->biases for AFFINE; g and amax for NVFP4 per gs).  fp_quantize /
 * affine_quantize of "mlx 0.30.7.3 -> 0.30.7.6" (quantized.h, quantized.cpp
 * fast::Quantize::eval_gpu).  gs is a bsfp_gs value and is ignored unless
 * mode is NVFP4.  Codes and scales are bit-exact to the documented rules.
 */
bsfp_status bsfp_quantize(const uint16_t* x, const bsfp_qtensor* q, int32_t gs,
                          bsfp_stream stream);

/*
 * bsfp_quantize_sr: bsfp_quantize with stochastic rounding of the E2M1
 * codes, for NVFP4 and MXFP4 (the USE_SR variant of the 4-bit quantizer,
 * "perf(cuda): enable hardware NVFP4/MXFP4 conversion on Blackwell builds",
 * Current Behavior).  Scales, global scale and amax are exactly those of
 * bsfp_quantize.  Element k (row-major over [rows, cols]) takes the random
 * word rbits[k]: with its scaled value v between E2M1 grid magnitudes
 * lo < hi, the code is hi when (rbits[k] >> 8) * 2^-24 < (|v| - lo) /
 * (hi - lo), else lo (both sides exact in fp32); grid values stay, |v| >= 6
 * saturates, the sign bit follows v.  The rounding is unbiased up to 2^-24
 * of the grid spacing.  rbits: device pointer to q->rows * q->cols uint32,
 * 16-byte aligned, owned by the caller, read only; the caller chooses how
 * it is drawn.  AFFINE returns BSFP_ERR_UNSUPPORTED; other errors as for
 * bsfp_quantize.
 */
bsfp_status bsfp_quantize_sr(const uint16_t* x, const bsfp_qtensor* q, int32_t gs,
                             const uint32_t* rbits, bsfp_stream stream);

/*
 * bsfp_quantize_ws: bsfp_quantize (rbits == NULL) or bsfp_quantize_sr
 * (rbits != NULL, with its requirements) with a caller workspace.  For
 * NVFP4 with BSFP_GS_COMPUTE (the per-tensor global scale from the tensor
 * amax: fp_quantize with a global scale, "mlx 0.30.7.3 -> 0.30.7.6",
 * quantized.cpp and qqmm_utils.cu) the amax is reduced from per-workgroup
 * partial maxima kept in the workspace instead of an atomic maximum whose
 * accumulator a separate launch must zero first: two kernel launches
 * instead of three, and the same bits (a maximum is exact in any order).
 * Every other mode and gs ignores the workspace and behaves as
 * bsfp_quantize / bsfp_quantize_sr.
 *   workspace: device memory of at least BSFP_QUANTIZE_WS_BYTES bytes,
 *   4-byte aligned, owned by the caller; its contents on entry are ignored
 *   and undefined on return, and calls in flight at the same time need
 *   separate workspaces.  May be NULL where it is ignored.
 * Errors: those of bsfp_quantize / bsfp_quantize_sr, and BSFP_ERR_ARG for a
 * needed workspace that is NULL, misaligned or smaller than
 * BSFP_QUANTIZE_WS_BYTES.  Nothing is launched on an error.
 */
#define BSFP_QUANTIZE_WS_BYTES 1024
bsfp_status bsfp_quantize_ws(const uint16_t* x, const bsfp_qtensor* q, int32_t gs,
                             const uint32_t* rbits, void* workspace,
                             int64_t workspace_bytes, bsfp_stream stream);

/*
 * bsfp_dequantize: q -> bf16 out [q->rows, q->cols].  fp_dequantize /
 * affine_dequantize of "mlx 0.30.7.3 -> 0.30.7.6" (quantized.cpp).
 *   NVFP4  bf16((E2M1 * E4M3) * g)  (g = 1 when q->global_scale is NULL)
 *   MXFP4  bf16(E2M1 * 2^(S-127))
 *   AFFINE bf16(fma(s, q, b))
 */
bsfp_status bsfp_dequantize(const bsfp_qtensor* q, uint16_t* out,
                            bsfp_stream stream);

/*
 * bsfp_qmv: decode GEMV, y[m, n] = sum_k x[m, k] * dq(W)[n, k] for
 * m < M <= 8, with W = w [N = w->rows, K = w->cols] and x bf16 [M, K].
 * Weights are dequantized in registers and accumulated in fp32; y is bf16
 * [M, N] (round to nearest even).  NVFP4 includes W's global scale when
 * present.  ("epic: NVIDIA Volta (sm_70) inference acceleration program",
 * Diagnosis item 3: qmv must accumulate in float; fp_qmv(w, scales, x, out,
 * bits, group_size, M, N, K) in "mlx 0.30.7.3 -> 0.30.7.6", qqmm.cpp.)
 */
bsfp_status bsfp_qmv(const uint16_t* x, int64_t M, const bsfp_qtensor* w,
                     uint16_t* y, bsfp_stream stream);

/*
 * bsfp_qmv_batch: the decode GEMV of bsfp_qmv for `count` weight matrices
 * that share x, y_i[m, n] = sum_k x[m, k] * dq(W_i)[n, k] for i < count,
 * 1 <= count <= BSFP_QMV_BATCH_MAX.  A decoder's projections that read the
 * same activations (gate and up of an MLP) are such a set; the decode
 * weight stream the call serves is that of "epic: NVIDIA Volta (sm_70)
 * inference acceleration program", Baseline (measured), qmv per layer.
 * w[i] (host array of count descriptors) must share mode, bits, group size
 * and K (cols); rows may differ.  y[i] (host array of count device pointers)
 * is bf16 [M, w[i]->rows], 16-byte aligned.  With one row of x and a base
 * format the matrices run as one launch (their rows dealt over the CUs
 * together, so the launch's fixed start-up and drain are paid once); each
 * output row is computed exactly as bsfp_qmv computes it.  Otherwise the
 * matrices run one launch each.  Errors: BSFP_ERR_ARG for a count outside
 * 1..BSFP_QMV_BATCH_MAX, null arrays or entries, descriptors that differ in
 * mode, bits, group size or K, and everything bsfp_qmv rejects;
 * BSFP_ERR_UNSUPPORTED as bsfp_qmv.  Nothing is launched on an error.
 */
#define BSFP_QMV_BATCH_MAX 4
bsfp_status bsfp_qmv_batch(const uint16_t* x, int64_t M, const bsfp_qtensor* const* w,
                           int32_t count, uint16_t* const* y, bsfp_stream stream);

/*
 * bsfp_qmm_workspace_bytes: device scratch bytes that bsfp_qmm needs for
 * (mode, M, K, act): for BSFP_ACT_SAME, x's codes, scales and (NVFP4) amax
 * and g; 0 for BSFP_ACT_BF16.  Returns 0 for unsupported arguments.  The
 * quantized x is the intermediate that QQMatmul::eval_gpu allocates itself
 * before the GEMM (quantize_input with x's packed codes and scales, and the
 * NVFP4 scalars of create_nvfp4_scalars: "mlx 0.30.7.3 -> 0.30.7.6",
 * qqmm.cpp and qqmm_utils.cu); here the caller owns it, so that the library
 * allocates nothing.
 */
size_t bsfp_qmm_workspace_bytes(int32_t mode, int64_t M, int64_t K, int32_t act);

/*
 * bsfp_qmm: prefill GEMM on MFMA, y bf16 [M, N] with N = w->rows,
 * K = w->cols, x bf16 [M, K] row-major, W in the "transposed" MLX layout
 * [N, K] (QQMatmul::eval_gpu, w_transposed = true, lda = ldb = K:
 * "mlx 0.30.7.3 -> 0.30.7.6", qqmm.cpp).
 *   act == BSFP_ACT_BF16: y = x . dq(W)^T (bf16 MFMA; W's codes are staged
 *     in LDS and dequantized in registers, the global scale of NVFP4 applied
 *     to the fp32 sums).
 *   act == BSFP_ACT_SAME: x is quantized into `workspace` with W's mode
 *     (quantize_input in the same file), then y = alpha * dq0(q(x)) .
 *     dq0(W)^T, dq0 = dequantization without the global scale, alpha =
 *     g_x * g_w for NVFP4 with a global scale on W (g_x = amax_x/2688,
 *     computed here), else 1.  The pages' alpha = amax_x*amax_w/(448*6)^2
 *     (create_nvfp4_scalars) is the same quantity up to fp32 rounding.
 *     MXFP4 runs on the gfx950 scaled f8f6f4 MFMA; NVFP4 on fp16 MFMA with
 *     both operands dequantized exactly (E2M1 * E4M3 has at most 6
 *     significant bits, so fp16 holds it).  For M <= 8 (decode) the
 *     same product runs as the GEMV of bsfp_qmv on q(x) dequantized exactly
 *     to bf16, with alpha applied the same way (the M = 1 branch of
 *     QQMatmul, qqmm.cpp, with the global scale of w kept); when x is at
 *     most 64 KB the GEMV quantizes x itself, in one launch.
 * fp32 accumulation, bf16 (RNE) output.  `workspace` must hold
 * bsfp_qmm_workspace_bytes(...) bytes (16-byte aligned) and is overwritten.
 * x and y must be 16-byte aligned, w's scales and biases 4-byte aligned.
 * K must be a multiple of 64 and at most
 * 2^22, M and N at most 2^30 and M * N at most 2^33; BSFP_ACT_SAME needs
 * NVFP4 or MXFP4 weights.
 * Outside these limits the call returns BSFP_ERR_UNSUPPORTED and launches
 * nothing.
 */
bsfp_status bsfp_qmm(const uint16_t* x, int64_t M, const bsfp_qtensor* w,
                     int32_t act, void* workspace, size_t workspace_bytes,
                     uint16_t* y, bsfp_stream stream);

/*
 * Size of the workspace that bsfp_qmm_noalloc keeps in the library's own
 * device memory: 32 MiB per GPU.  It holds the qq workspace of
 * bsfp_qmm_workspace_bytes(...) up to that size, e.g. NVFP4 activations of
 * up to 2^24 elements (M = 3276 at K = 5120) or MXFP4 ones of up to about
 * 6.3 * 10^7.
 */
#define BSFP_NOALLOC_WORKSPACE_BYTES (32u << 20)

/*
 * bsfp_qmm_noalloc: bsfp_qmm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, semantics, limits and errors as bsfp_qmm,
 * except that the workspace is not passed: the call uses a static device
 * array of BSFP_NOALLOC_WORKSPACE_BYTES inside the library, one per GPU,
 * held until the process ends (its address on a device is looked up on the
 * first call there).  The call allocates and frees nothing; the caller still
 * owns x, w and y.  A product whose workspace would exceed that size returns
 * BSFP_ERR_UNSUPPORTED and launches nothing.  Every call on one GPU shares
 * that GPU's array, and it keeps what the last call left there (every byte
 * a call reads it first writes, so nothing needs to start at zero): calls
 * that overlap on one GPU (other streams, other threads) race and must be
 * serialized by the caller.
 */
bsfp_status bsfp_qmm_noalloc(const uint16_t* x, int64_t M, const bsfp_qtensor* w,
                             int32_t act, uint16_t* y, bsfp_stream stream);

/*
 * bsfp_qmm_dense_scratch_bytes: bytes of the bf16 copy of a [rows, cols]
 * weight that bsfp_qmm_dense dequantizes into (rows * cols * 2); 0 for
 * negative arguments.
 */
size_t bsfp_qmm_dense_scratch_bytes(int64_t rows, int64_t cols);

/*
 * bsfp_qmm_dense: the dense prefill path of "mlx: opt-in dense GEMM for
 * nvfp4 prefill (dequantise to bf16 above a row threshold)": W is
 * dequantized to bf16 exactly as bsfp_dequantize does (NVFP4 with its global
 * scale, rounded once to bf16) into `scratch`, then y = x . scratch^T with
 * a dense bf16 GEMM (bf16 MFMA, fp32 accumulation, bf16 RNE output).  x bf16
 * [M, K], y bf16 [M, N], N = w->rows, K = w->cols, every mode.
 * `scratch` is caller-owned device memory of at least
 * bsfp_qmm_dense_scratch_bytes(N, K) bytes, 16-byte aligned, not
 * overlapping x or y; it is overwritten and may be reused for the next
 * layer once the call's stream has passed it, so the transient is bounded
 * by one layer's bf16 copy.  Picking this path above a row threshold is the
 * caller's policy (the binding's qmm(dense_rows=...)).  Same limits and
 * alignment rules as bsfp_qmm with BSFP_ACT_BF16; outside them the call
 * returns BSFP_ERR_UNSUPPORTED (or BSFP_ERR_ARG for bad pointers or a small
 * scratch) and launches nothing.
 */
bsfp_status bsfp_qmm_dense(const uint16_t* x, int64_t M, const bsfp_qtensor* w,
                           void* scratch, size_t scratch_bytes, uint16_t* y,
                           bsfp_stream stream);

/*
 * bsfp_time_next_launch: measurement hook.  The main kernel of this
 * thread's next bsfp_qmv, bsfp_qmm or bsfp_qmm_dense call (the GEMV, or the
 * GEMM) is launched with hipExtLaunchKernelGGL, whose start and stop
 * events then carry that kernel's own begin and end times, with no extra
 * commands queued between kernels.  start_event and stop_event are hipEvent_t
 * handles the caller created (timing enabled) and still owns; either may be
 * NULL.  One-shot: the pair is cleared by the launch that uses it, and
 * passing two NULLs clears a pending pair.  Always returns BSFP_OK.
 */
bsfp_status bsfp_time_next_launch(void* start_event, void* stop_event);

/* Thread-local description of the last non-OK status ("" if none). */
const char* bsfp_last_error(void);

/* Library version and the GPU architecture it was compiled for. */
const char* bsfp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSFP_H */
