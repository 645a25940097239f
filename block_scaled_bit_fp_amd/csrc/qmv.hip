// qmv.hip -- decode GEMV y[m, n] = sum_k x[m, k] * dq(W)[n, k] for M <= 8.
//
// The decode step streams every packed weight once ("epic: NVIDIA Volta
// (sm_70) inference acceleration program", Baseline: ~15 GB per step, qmv
// reaching only 7.7 % of the memory roofline); this kernel is built to be
// HBM-bound on MI355X:
//
//   - a team of 32 lanes owns one weight row at a time; each lane streams
//     16-byte chunks (32 codes) of the row with 128-bit loads.  Rows are
//     dealt to teams round-robin across the whole grid;
//   - the (row, chunk) items of a team form one flat stream that is software
//     pipelined across row boundaries: kPrefetch chunk loads are always in
//     flight per lane, so a row's tail never drains the memory pipe;
//   - weights are dequantized in registers and multiplied with v_dot2 on bf16
//     pairs into fp32 accumulators (the page's diagnosis: bf16 accumulation
//     at bits < 8 made its kernel ALU-bound; here accumulation is always
//     fp32); per-group scales are applied to per-group partial sums;
//   - the activations are staged once per workgroup in LDS, laid out so that
//     the 32 lanes of a team read 32 consecutive 16-byte units (no bank
//     conflicts) and the two teams of a wave read the same addresses
//     (broadcast); the per-64-group sums of x that the affine bias term needs
//     are staged with them; team partial sums are reduced with a butterfly.
//
// Affine nibble decode: an OCP E4M3 byte holding 0..15 decodes to code * 2^-9
// (subnormals and the first normal binade), so the gfx950 converter
// v_cvt_scalef32_pk_bf16_fp8 with the exponent scale 2^9 turns bytes holding
// one nibble each into the exact integers q as bf16.  With t = w & 0x0F0F0F0F
// and u = (w >> 4) & 0x0F0F0F0F the four converted pairs are (q0,q2),
// (q4,q6), (q1,q3), (q5,q7); x is staged in that pair order.  FP4 decode uses
// v_cvt_scalef32_pk_bf16_fp4 (exact, unit scale) with x in natural order.
#include "bsfp_device.hpp"
#include "bsfp_internal.hpp"

namespace bsfp {

namespace {

constexpr int kThreads = 256;
constexpr int kTeam = 32;                 // lanes per weight row
constexpr int kTeams = kThreads / kTeam;  // rows in flight per workgroup
constexpr int kPrefetch = 4;              // chunk loads in flight per lane
constexpr int kLdsBudget = 53 * 1024;     // three workgroups per CU (160 KB LDS)

// LDS layout for one K slice of ks elements (nch = ks / 32 chunks):
//   xp: uint4 [MAXM][4][nch]: unit (m, j, c) = x[m, 32c + 8j .. 32c + 8j + 7]
//       (affine: pairs reordered (x0,x2),(x4,x6),(x1,x3),(x5,x7))
//   xs: float [MAXM][ks / 64]: per-64-group sums of x (affine only)
template <bool AFFINE>
__device__ void stage_x(const uint16_t* __restrict__ x, int64_t K, int M, int64_t k0, int ks,
                        uint4* __restrict__ xp, float* __restrict__ xs) {
  const int bpr = ks / 8;  // 8-element units per row
  const int nch = ks / 32;
  const int nb = M * bpr;  // multiple of 8 for affine (ks % 64 == 0)
  for (int b = threadIdx.x; b < nb; b += kThreads) {
    const int m = b / bpr;
    const int u = b - m * bpr;
    const int c = u >> 2, j = u & 3;
    const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + k0 + 8 * u);
    uint4 o;
    if constexpr (AFFINE) {
      o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // (x0, x2)
      o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // (x4, x6)
      o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (x1, x3)
      o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // (x5, x7)
      float s = bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) +
                bf16_lo(v.z) + bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
      s = team_sum<8>(s);  // the 8 units of one 64-element group
      if ((u & 7) == 0) xs[m * (ks / 64) + (u >> 3)] = s;
    } else {
      o = v;
    }
    xp[(m * 4 + j) * nch + c] = o;
  }
}

struct Item {
  uint4 w;     // 32 codes
  uint32_t s;  // scale bits
  uint32_t b;  // affine bias bits
};

// MAXM: compile-time bound on M.  When nslices > 1 (large M * K only) the K
// range is walked in slices that fit the LDS budget and every team owns at
// most one row, whose partial sums stay in registers across the slices.
template <int MODE, int MAXM>
__global__ __launch_bounds__(kThreads) void qmv_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, int64_t N,
    const uint4* __restrict__ codes, const void* __restrict__ scales,
    const uint16_t* __restrict__ biases, const float* __restrict__ gptr,
    uint16_t* __restrict__ y, int ks, int nslices) {
  extern __shared__ uint4 smem[];
  constexpr bool AFF = (MODE == BSFP_AFFINE);
  const int nch = ks / 32;
  uint4* xp = smem;
  float* xs = reinterpret_cast<float*>(smem + MAXM * 4 * nch);

  const int team = threadIdx.x / kTeam;
  const int lt = threadIdx.x % kTeam;
  const int64_t cpr = K / 32;                 // chunks per row
  const int ipr = (nch + kTeam - 1) / kTeam;  // items per lane per row and slice
  const float g = (MODE == BSFP_NVFP4 && gptr) ? *gptr : 1.0f;

  // rows of this team: gt, gt + T, gt + 2T, ... (T = teams in the grid)
  const int64_t gt = (int64_t)blockIdx.x * kTeams + team;
  const int64_t T = (int64_t)gridDim.x * kTeams;
  const int64_t my_rows = gt < N ? (N - 1 - gt) / T + 1 : 0;
  // uniform across the workgroup: the most rows any of its teams owns
  const int64_t wg_rows = (N - 1 - (int64_t)blockIdx.x * kTeams) / T + 1;
  const int64_t total = wg_rows * ipr;

  float acc[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;

  auto consume = [&](const Item& it, int c) {
    const uint32_t ww[4] = {it.w.x, it.w.y, it.w.z, it.w.w};
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      if (MAXM > 1 && m >= M) break;
      const uint4* xq = xp + (m * 4) * nch + c;
      if constexpr (AFF) {
        float D = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 xv = xq[j * nch];
          const uint32_t t = ww[j] & 0x0F0F0F0Fu;
          const uint32_t h = (ww[j] >> 4) & 0x0F0F0F0Fu;
          D = dot2_bf16(xv.x, nibbles_to_bf16x2<false>(t), D);  // q0, q2
          D = dot2_bf16(xv.y, nibbles_to_bf16x2<true>(t), D);   // q4, q6
          D = dot2_bf16(xv.z, nibbles_to_bf16x2<false>(h), D);  // q1, q3
          D = dot2_bf16(xv.w, nibbles_to_bf16x2<true>(h), D);   // q5, q7
        }
        acc[m] = __builtin_fmaf(__uint_as_float(it.s << 16), D, acc[m]);
        // the bias term of a 64-group, added once (with its even chunk)
        if ((c & 1) == 0)
          acc[m] = __builtin_fmaf(__uint_as_float(it.b << 16), xs[m * (nch / 2) + (c >> 1)],
                                  acc[m]);
      } else {
        float D0 = 0.0f, D1 = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 xv = xq[j * nch];
          const uint32_t q = ww[j];
          float D = (j < 2) ? D0 : D1;
          D = dot2_bf16(xv.x, e2m1x2_to_bf16x2<0>(q), D);
          D = dot2_bf16(xv.y, e2m1x2_to_bf16x2<1>(q), D);
          D = dot2_bf16(xv.z, e2m1x2_to_bf16x2<2>(q), D);
          D = dot2_bf16(xv.w, e2m1x2_to_bf16x2<3>(q), D);
          if (j < 2) D0 = D; else D1 = D;
        }
        if constexpr (MODE == BSFP_MXFP4) {
          acc[m] = __builtin_fmaf(D0 + D1, e8m0_decode(it.s), acc[m]);
        } else {
          // both E4M3 block scales with the hardware converter (exact)
          const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(it.s, 1.0f, false);
          acc[m] = __builtin_fmaf(D0, sc.x, acc[m]);
          acc[m] = __builtin_fmaf(D1, sc.y, acc[m]);
        }
      }
    }
  };

  auto finish_row = [&](int64_t row) {
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      if (MAXM > 1 && m >= M) break;
      const float r = team_sum<kTeam>(acc[m]);
      if (lt == 0 && row < N) y[(int64_t)m * N + row] = (uint16_t)f32_to_bf16(r * g);
      acc[m] = 0.0f;
    }
  };

  // Items beyond the team's rows or the row's chunks are padding: their
  // loads read a valid address (the start of the tensor) and their data are
  // zeroed, so loads and math stay branch-free and the compiler can keep
  // kPrefetch loads in flight without conservative waits.
  const int64_t total_p = (total + kPrefetch - 1) / kPrefetch * kPrefetch;
  for (int sl = 0; sl < nslices; ++sl) {
    if (sl > 0) __syncthreads();  // the previous slice is fully consumed
    stage_x<AFF>(x, K, M, (int64_t)sl * ks, ks, xp, xs);
    __syncthreads();
    const int64_t cslice = (int64_t)sl * nch;
    auto fetch = [&](int64_t r, int i, Item& it, bool& ok) {
      const int c = i * kTeam + lt;
      ok = (r < my_rows) && (c < nch);
      const int64_t ci = ok ? (gt + r * T) * cpr + cslice + c : 0;
      it.w = codes[ci];
      if constexpr (AFF) {
        it.s = reinterpret_cast<const uint16_t*>(scales)[ci >> 1];
        it.b = biases[ci >> 1];
      } else if constexpr (MODE == BSFP_MXFP4) {
        it.s = reinterpret_cast<const uint8_t*>(scales)[ci];
      } else {  // two E4M3 bytes: the chunk's two 16-element groups
        it.s = reinterpret_cast<const uint16_t*>(scales)[ci];
      }
    };
    auto advance = [&](int64_t& r, int& i) {
      if (++i == ipr) { i = 0; ++r; }
    };
    Item ring[kPrefetch];
    bool okr[kPrefetch];
    int64_t rf = 0, rc = 0;
    int i_f = 0, i_c = 0;
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) {
      fetch(rf, i_f, ring[u], okr[u]);
      advance(rf, i_f);
    }
    for (int64_t t0 = 0; t0 < total_p; t0 += kPrefetch) {
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u) {
        Item it = ring[u];
        const bool ok = okr[u];
        const int c = ok ? i_c * kTeam + lt : 0;
        it.w.x = ok ? it.w.x : 0u;
        it.w.y = ok ? it.w.y : 0u;
        it.w.z = ok ? it.w.z : 0u;
        it.w.w = ok ? it.w.w : 0u;
        it.s = ok ? it.s : 0u;
        it.b = ok ? it.b : 0u;
        consume(it, c);
        if (i_c == ipr - 1 && nslices == 1) finish_row(gt + rc * T);  // uniform
        advance(rc, i_c);
        fetch(rf, i_f, ring[u], okr[u]);
        advance(rf, i_f);
      }
    }
  }
  if (nslices > 1) finish_row(gt);
}

// Word-granular GEMV for NVFP4 rows whose length is not a multiple of 32
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

template <int MODE, int MAXM>
size_t lds_bytes(int64_t k) {
  return (size_t)k * 2 * MAXM + (MODE == BSFP_AFFINE ? (size_t)(k / 64) * 4 * MAXM : 0);
}

template <int MODE, int MAXM>
hipError_t run(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y, hipStream_t s) {
  const int64_t N = w.rows, K = w.cols;
  constexpr int64_t gran = (MODE == BSFP_AFFINE) ? 64 : 32;  // whole groups per slice
  int64_t ks = K;
  if (lds_bytes<MODE, MAXM>(K) > (size_t)kLdsBudget) {
    ks = (int64_t)(kLdsBudget / lds_bytes<MODE, MAXM>(gran)) * gran;
    while (ks > gran && K % ks) ks -= gran;  // K % gran == 0: stops at gran at worst
  }
  const int nslices = (int)(K / ks);
  const size_t lds = lds_bytes<MODE, MAXM>(ks);
  // All workgroups resident at once (3 per CU when LDS-heavy, else 4), no
  // more teams than rows; multi-slice walks use one row per team.
  const int64_t by_rows = (N + kTeams - 1) / kTeams;
  int64_t grid = (int64_t)device_cu_count() * (lds > 40 * 1024 ? 3 : 4);
  if (nslices > 1 || grid > by_rows) grid = by_rows;
  hipLaunchKernelGGL((qmv_kernel<MODE, MAXM>), dim3((unsigned)grid), dim3(kThreads), lds, s, x,
                     M, K, N, reinterpret_cast<const uint4*>(w.codes), w.scales, w.biases,
                     w.global_scale, y, (int)ks, nslices);
  return hipGetLastError();
}

template <int MODE>
hipError_t by_m(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y, hipStream_t s) {
  if (M == 1) return run<MODE, 1>(x, M, w, y, s);
  if (M == 2) return run<MODE, 2>(x, M, w, y, s);
  if (M <= 4) return run<MODE, 4>(x, M, w, y, s);
  return run<MODE, 8>(x, M, w, y, s);
}

}  // namespace

hipError_t launch_qmv(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y,
                      hipStream_t s) {
  if (w.rows == 0) return hipGetLastError();
  if (w.cols % 32 != 0) {  // only NVFP4 rows can have K % 32 == 16
    const dim3 grid((unsigned)((w.rows + 3) / 4));
    if (M == 1)
      hipLaunchKernelGGL(qmv_nvfp4_words_kernel<1>, grid, dim3(kThreads), 0, s, x, M, w.cols,
                         w.rows, w.codes, (const uint8_t*)w.scales, w.global_scale, y);
    else
      hipLaunchKernelGGL(qmv_nvfp4_words_kernel<8>, grid, dim3(kThreads), 0, s, x, M, w.cols,
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
