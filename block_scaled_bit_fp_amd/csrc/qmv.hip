// qmv.hip -- decode GEMV y[m, n] = sum_k x[m, k] * dq(W)[n, k] for M <= 8.
//
// The decode step streams every packed weight once ("epic: NVIDIA Volta
// (sm_70) inference acceleration program", Baseline: ~15 GB per step, qmv
// reaching only 7.7 % of the memory roofline); the kernel is built to be
// HBM-bound on MI355X:
//
//   - a team of T lanes (16 or 64) owns one weight row; each lane streams
//     16-byte chunks (32 codes) of that row with 128-bit loads, issuing U
//     chunk loads before consuming any, so each wave keeps ~10 KB in flight;
//   - weights are dequantized in registers and multiplied with v_dot2 on bf16
//     pairs into fp32 accumulators (the page's diagnosis: bf16 accumulation
//     at bits < 8 made the kernel ALU-bound; here accumulation is always
//     fp32), per-group scales are applied to per-group partial sums;
//   - the activations are staged once per workgroup in LDS (for affine in a
//     pair-interleaved order that matches the nibble extraction below,
//     together with per-32-element sums of x), then team partial sums are
//     reduced with a lane butterfly;
//   - workgroups are persistent over row blocks, sized to balance the rows.
//
// Affine nibble decode: an OCP E4M3 byte holding 0..15 is a subnormal (or
// the first normal binade) whose value is exactly code * 2^-9, so the gfx950
// converter v_cvt_scalef32_pk_bf16_fp8 with scale 2^9 turns bytes holding one
// nibble each into the exact integers q as bf16.  With t = w & 0x0F0F0F0F and
// u = (w >> 4) & 0x0F0F0F0F the four converted pairs are (q0,q2), (q4,q6),
// (q1,q3), (q5,q7); x is staged in LDS in that pair order.  FP4 decode uses
// v_cvt_scalef32_pk_bf16_fp4 (exact, unit scale).
#include "bsfp_device.hpp"
#include "bsfp_internal.hpp"

namespace bsfp {

namespace {

constexpr int kThreads = 256;
constexpr int kLdsBytes = 64 * 1024;

// Stage x[:, k0 : k0 + ks] into LDS as bf16 pairs.  For affine the pairs of
// each 8-element block are reordered to (x0,x2),(x4,x6),(x1,x3),(x5,x7) and
// the per-32 sums of x are stored after the pairs.
template <bool AFFINE>
__device__ void stage_x(const uint16_t* __restrict__ x, int64_t K, int M, int64_t k0, int ks,
                        uint32_t* __restrict__ xp, float* __restrict__ xs) {
  const int blocks_per_row = ks / 8;
  const int nb = M * blocks_per_row;  // multiple of 4 (ks % 32 == 0)
  for (int b = threadIdx.x; b < nb; b += kThreads) {
    const int m = b / blocks_per_row;
    const int j = b - m * blocks_per_row;
    const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + k0 + 8 * j);
    uint4 o;
    if constexpr (AFFINE) {
      o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // (x0, x2)
      o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // (x4, x6)
      o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (x1, x3)
      o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // (x5, x7)
      float s = bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) +
                bf16_lo(v.z) + bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
      s = team_sum<4>(s);  // the 4 blocks of one 32-element chunk
      if ((j & 3) == 0) xs[m * (ks / 32) + (j >> 2)] = s;
    } else {
      o = v;
    }
    reinterpret_cast<uint4*>(xp)[m * blocks_per_row + j] = o;
  }
}

// MODE: BSFP_AFFINE, BSFP_MXFP4, BSFP_NVFP4.  MAXM: compile-time bound on M.
template <int MODE, int T, int U, int MAXM>
__global__ __launch_bounds__(kThreads) void qmv_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, int64_t N,
    const uint4* __restrict__ codes, const void* __restrict__ scales,
    const uint16_t* __restrict__ biases, const float* __restrict__ gptr,
    uint16_t* __restrict__ y, int ks, int nslices, int64_t row_blocks) {
  extern __shared__ uint32_t smem[];
  constexpr bool AFF = (MODE == BSFP_AFFINE);
  constexpr int ROWS = kThreads / T;
  uint32_t* xp = smem;
  float* xs = reinterpret_cast<float*>(smem + MAXM * (ks / 2));

  const int team = threadIdx.x / T;
  const int lt = threadIdx.x % T;
  const int64_t cpr = K / 32;  // 16-byte chunks per row
  const int nch = ks / 32;     // chunks per slice
  const float g = (MODE == BSFP_NVFP4 && gptr) ? *gptr : 1.0f;

  if (nslices == 1) {
    stage_x<AFF>(x, K, M, 0, ks, xp, xs);
    __syncthreads();
  }
  for (int64_t rb = blockIdx.x; rb < row_blocks; rb += gridDim.x) {
    const int64_t row = rb * ROWS + team;
    float acc[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;

    for (int sl = 0; sl < nslices; ++sl) {
      if (nslices > 1) {
        __syncthreads();
        stage_x<AFF>(x, K, M, (int64_t)sl * ks, ks, xp, xs);
        __syncthreads();
      }
      if (row < N) {
        const int64_t cbase = row * cpr + (int64_t)sl * nch;
        const uint4* crow = codes + cbase;
        for (int base = 0; base < nch; base += T * U) {
          uint4 w[U];
          uint32_t sraw[U];
          uint32_t braw[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int c = base + u * T + lt;
            if (c < nch) {
              w[u] = crow[c];
              if constexpr (AFF) {
                const int64_t gi = (cbase + c) >> 1;  // 64-element group
                sraw[u] = reinterpret_cast<const uint16_t*>(scales)[gi];
                braw[u] = biases[gi];
              } else if constexpr (MODE == BSFP_MXFP4) {
                sraw[u] = reinterpret_cast<const uint8_t*>(scales)[cbase + c];
              } else {  // two 16-element groups per chunk
                sraw[u] = reinterpret_cast<const uint16_t*>(scales)[cbase + c];
              }
            }
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int c = base + u * T + lt;
            if (c < nch) {
              const uint4 wv = w[u];
              const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
              for (int m = 0; m < MAXM; ++m) {
                if (MAXM > 1 && m >= M) break;
                const uint4* xq = reinterpret_cast<const uint4*>(xp) + m * (ks / 8) + c * 4;
                if constexpr (AFF) {
                  float D = 0.0f;
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    const uint4 xv = xq[j];
                    const uint32_t t = ww[j] & 0x0F0F0F0Fu;
                    const uint32_t h = (ww[j] >> 4) & 0x0F0F0F0Fu;
                    D = dot2_bf16(xv.x, nibbles_to_bf16x2<false>(t), D);  // q0, q2
                    D = dot2_bf16(xv.y, nibbles_to_bf16x2<true>(t), D);   // q4, q6
                    D = dot2_bf16(xv.z, nibbles_to_bf16x2<false>(h), D);  // q1, q3
                    D = dot2_bf16(xv.w, nibbles_to_bf16x2<true>(h), D);   // q5, q7
                  }
                  const float sx = xs[m * nch + c];  // sum x over the chunk
                  acc[m] = __builtin_fmaf(__uint_as_float(sraw[u] << 16), D, acc[m]);
                  acc[m] = __builtin_fmaf(__uint_as_float(braw[u] << 16), sx, acc[m]);
                } else {
                  float D0 = 0.0f, D1 = 0.0f;
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    const uint4 xv = xq[j];
                    const uint32_t q = ww[j];
                    float D = (j < 2) ? D0 : D1;
                    D = dot2_bf16(xv.x, e2m1x2_to_bf16x2<0>(q), D);
                    D = dot2_bf16(xv.y, e2m1x2_to_bf16x2<1>(q), D);
                    D = dot2_bf16(xv.z, e2m1x2_to_bf16x2<2>(q), D);
                    D = dot2_bf16(xv.w, e2m1x2_to_bf16x2<3>(q), D);
                    if (j < 2) D0 = D; else D1 = D;
                  }
                  if constexpr (MODE == BSFP_MXFP4) {
                    acc[m] = __builtin_fmaf(D0 + D1, e8m0_decode(sraw[u]), acc[m]);
                  } else {
                    acc[m] = __builtin_fmaf(D0, e4m3_decode(sraw[u] & 0xFFu), acc[m]);
                    acc[m] = __builtin_fmaf(D1, e4m3_decode(sraw[u] >> 8), acc[m]);
                  }
                }
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      if (MAXM > 1 && m >= M) break;
      const float r = team_sum<T>(acc[m]);
      if (lt == 0 && row < N) y[(int64_t)m * N + row] = (uint16_t)f32_to_bf16(r * g);
    }
  }
}

// Word-granular fallback for NVFP4 rows whose length is not a multiple of 32
// (K % 32 == 16): one wave per row, one 32-bit code word (8 codes) per step.
template <int MAXM>
__global__ __launch_bounds__(kThreads) void qmv_nvfp4_words_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, int64_t N,
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ gptr, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= N) return;
  const float g = gptr ? *gptr : 1.0f;
  const int64_t wpr = K / 8;
  float acc[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;
  for (int64_t wi = lane; wi < wpr; wi += 64) {
    const uint32_t q = codes[row * wpr + wi];
    const float S = e4m3_decode(scales[row * (K / 16) + (wi >> 1)]);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      if (m >= M) break;
      const uint4 xv = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + wi * 8);
      float D = 0.0f;
      D = dot2_bf16(xv.x, e2m1x2_to_bf16x2<0>(q), D);
      D = dot2_bf16(xv.y, e2m1x2_to_bf16x2<1>(q), D);
      D = dot2_bf16(xv.z, e2m1x2_to_bf16x2<2>(q), D);
      D = dot2_bf16(xv.w, e2m1x2_to_bf16x2<3>(q), D);
      acc[m] = __builtin_fmaf(D, S, acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    if (m >= M) break;
    const float r = team_sum<64>(acc[m]);
    if (lane == 0) y[(int64_t)m * N + row] = (uint16_t)f32_to_bf16(r * g);
  }
}

template <int MODE, int T, int U, int MAXM>
hipError_t run(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y, hipStream_t s) {
  const int64_t N = w.rows, K = w.cols;
  // slice K so that MAXM rows of x (and, for affine, their per-32 sums) fit
  // the LDS budget: 2*MAXM + MAXM/8 bytes per element column.
  constexpr int64_t gran = (MODE == BSFP_AFFINE) ? 64 : 32;
  const int64_t bytes_per_col8 = 17 * MAXM;  // per 8 columns: 16*MAXM + MAXM
  int64_t ks = K;
  if (K / 8 * bytes_per_col8 > kLdsBytes) {
    ks = (kLdsBytes / bytes_per_col8 * 8) / gran * gran;
    while (K % ks) ks -= gran;  // K % gran == 0, so this stops at gran at worst
  }
  const int nslices = (int)(K / ks);
  const size_t lds = (size_t)ks * 2 * MAXM + (size_t)(ks / 32) * 4 * MAXM;
  constexpr int ROWS = kThreads / T;
  const int64_t row_blocks = (N + ROWS - 1) / ROWS;
  const int64_t max_grid = (int64_t)device_cu_count() * 4;
  const int64_t per_wg = (row_blocks + max_grid - 1) / max_grid;
  const int64_t grid = (row_blocks + per_wg - 1) / per_wg;
  hipLaunchKernelGGL((qmv_kernel<MODE, T, U, MAXM>), dim3((unsigned)grid), dim3(kThreads), lds,
                     s, x, M, K, N, reinterpret_cast<const uint4*>(w.codes), w.scales,
                     w.biases, w.global_scale, y, (int)ks, nslices, row_blocks);
  return hipGetLastError();
}

template <int MODE, int MAXM>
hipError_t pick_tiling(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y,
                       hipStream_t s) {
  const int64_t nch = w.cols / 32;
  if (nch <= 64) return run<MODE, 16, 4, MAXM>(x, M, w, y, s);
  if (nch <= 160) return run<MODE, 16, 10, MAXM>(x, M, w, y, s);
  return run<MODE, 64, 13, MAXM>(x, M, w, y, s);
}

template <int MODE>
hipError_t by_m(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y, hipStream_t s) {
  if (M == 1) return pick_tiling<MODE, 1>(x, M, w, y, s);
  if (M == 2) return pick_tiling<MODE, 2>(x, M, w, y, s);
  if (M <= 4) return pick_tiling<MODE, 4>(x, M, w, y, s);
  return pick_tiling<MODE, 8>(x, M, w, y, s);
}

}  // namespace

hipError_t launch_qmv(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y,
                      hipStream_t s) {
  if (w.rows == 0) return hipGetLastError();
  if (w.cols % 32 != 0) {  // NVFP4 with K % 32 == 16
    const dim3 grid((unsigned)((w.rows + 3) / 4));
    const uint16_t* xx = x;
    if (M == 1)
      hipLaunchKernelGGL(qmv_nvfp4_words_kernel<1>, grid, dim3(kThreads), 0, s, xx, M, w.cols,
                         w.rows, w.codes, (const uint8_t*)w.scales, w.global_scale, y);
    else
      hipLaunchKernelGGL(qmv_nvfp4_words_kernel<8>, grid, dim3(kThreads), 0, s, xx, M, w.cols,
                         w.rows, w.codes, (const uint8_t*)w.scales, w.global_scale, y);
    return hipGetLastError();
  }
  switch (w.mode) {
    case BSFP_AFFINE: return by_m<BSFP_AFFINE>(x, M, w, y, s);
    case BSFP_MXFP4: return by_m<BSFP_MXFP4>(x, M, w, y, s);
    default: return by_m<BSFP_NVFP4>(x, M, w, y, s);
  }
}

}  // namespace bsfp
