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
#include <algorithm>
#include <atomic>

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
    const uint16_t* __restrict__ biases, const float* __restrict__ gptr, const float* __restrict__ g2ptr,
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
  float g = ((MODE == BSFP_NVFP4 && gptr) ? *gptr : 1.0f) * (g2ptr ? *g2ptr : 1.0f);

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
    const float* __restrict__ gptr, const float* __restrict__ g2ptr, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= N) return;
  const float g = (gptr ? *gptr : 1.0f) * (g2ptr ? *g2ptr : 1.0f);
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

// ------------------------------------------------------------------ fast path
//
// Chunk c of a row (32 codes, 16 bytes) always goes to lane c % 32 of the
// row's team, so a lane works on the same x chunks for every row it visits.
// A wave owns blocks of 2R consecutive rows (team h takes rows 2r + h of the
// block) and walks them chunk step by chunk step: step j loads chunk
// 32 j + lt of each of its R rows, so the x values of one step are read from
// LDS once and used for R rows.  All addresses are per-lane constants plus
// wave-uniform offsets (raw buffer loads: descriptor at the block's first row,
// 32-bit lane offset, scalar step offset); rows past N fall outside the
// descriptor and read as zeros.  A few steps of chunk loads per lane stay in
// flight (steps_in_flight), and the pipeline runs across row blocks.
//
// Steps in flight per wave: 3 with one row per team, 2 with more (4 and 8
// chunk loads per lane).  Deeper rings measured slower: on the affine
// [5120, 25600] decode shape (one row per team) 20.3 us with 8 loads per lane
// and 22.3 us with 16, against 18.9 us with 3; on [25600, 5120] (two rows per
// team) 16.8 us with 8 against 16.2 us with 4.  Later interleaved A/B runs:
// one row per team with 2 or 4 steps, 19.7 and 19.4 us against 19.2 with 3;
// the gate+up batch at four rows per team with 1 or 3 steps, 29.8 us against
// 28.8 with 2.  The whole chip already keeps
// every row of such a matrix in flight at once.
template <int R>
constexpr int steps_in_flight() {
  return R == 1 ? 3 : 2;
}

struct Chunk {
  uint4 w;     // 32 codes (4-bit), or the first 16 of them (8-bit)
  uint4 w2;    // 8-bit: codes 16..31
  uint32_t s;  // scale bits
  uint32_t b;  // affine bias bits
};

// LDS bytes of the staged activations: x units [M][NJ][4][32] of 16 bytes,
// plus (affine) the per-chunk sums of x [M][NJ][32] for the bias term.
template <int MODE>
size_t fast_lds_bytes(int M, int NJ) {
  return (size_t)M * NJ * (2048 + (fmt_affine(MODE) ? 128 : 0));
}

// Staging of x for the fast kernel, split in two so that the x loads can go
// out before the first weight loads and the LDS writes wait only for them.
// Unit (m, c, u) holds x[m, 32c + 8u .. + 7] (affine: pairs reordered as the
// nibble decode produces them); chunks past the row end are zero, so they
// contribute nothing.  Each thread owns units tid + i * blockDim, i < XU
// (kXU, or 8 for the 512-thread variants below).
constexpr int kXU = 4;

// Rows of x per launch above 2 (above 1 with 8-bit codes) need more
// registers per lane: those variants run 512-thread workgroups (256 VGPRs),
// two per CU, staging 8 units of x per thread (the same 64 KB of x at most).
template <int FMT, int MAXM> constexpr bool fast_wide() {
  return MAXM > 2 || (fmt_bits(FMT) == 8 && MAXM > 1);  // 8-bit codes hold twice the registers
}
template <int FMT, int MAXM> constexpr int fast_threads() { return fast_wide<FMT, MAXM>() ? 512 : 1024; }
template <int FMT, int MAXM> constexpr int fast_xu() { return fast_wide<FMT, MAXM>() ? 8 : kXU; }

template <int XU>
__device__ __forceinline__ void stage_x_load(const uint16_t* __restrict__ x, int M, int K,
                                             int NJ, uint4 (&xr)[XU]) {
  const int cpr = K / 32;
  const int units = M * NJ * 128;
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int b = threadIdx.x + i * blockDim.x;
    xr[i] = make_uint4(0u, 0u, 0u, 0u);
    if (b < units) {
      const int m = b / (NJ * 128);
      const int rem = b - m * NJ * 128;
      const int c = rem >> 2, u = rem & 3;
      if (c < cpr) xr[i] = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + 32 * c + 8 * u);
    }
  }
}

// SUMS: also store the per-chunk sums of x (affine bias term); REORDER:
// store the pairs in the order the 4-bit nibble decode produces them.
template <bool SUMS, bool REORDER, int XU, int QXMODE>
__device__ __forceinline__ void stage_x_store(int M, int NJ, const uint4 (&xr)[XU],
                                              uint4* __restrict__ xp, float* __restrict__ xs,
                                              float gq) {
  const int units = M * NJ * 128;
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int b = threadIdx.x + i * blockDim.x;
    if (b < units) {  // units % 4 == 0: the 4 threads of a chunk agree
      const int m = b / (NJ * 128);
      const int rem = b - m * NJ * 128;
      const int c = rem >> 2, u = rem & 3;
      uint4 v = xr[i];
      // qq: x quantized with the weights' format and dequantized exactly
      if constexpr (QXMODE == BSFP_NVFP4) v = qdq_nvfp4_half_bf16(v, gq);
      if constexpr (QXMODE == BSFP_MXFP4) v = qdq_mxfp4_quarter_bf16(v);
      uint4 o = v;
      if constexpr (REORDER) {
        o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // (x0, x2)
        o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // (x4, x6)
        o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (x1, x3)
        o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // (x5, x7)
      }
      if constexpr (SUMS) {
        float t = bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) +
                  bf16_lo(v.z) + bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
        t = team_sum<4>(t);  // the 4 units of chunk c are 4 adjacent threads
        if (u == 0) xs[(m * NJ + (c >> 5)) * 32 + (c & 31)] = t;
      }
      xp[((m * NJ + (c >> 5)) * 4 + u) * 32 + (c & 31)] = o;
    }
  }
}

// Scale bytes of one block of 2R rows (the affine biases are as many again).
template <int MODE>
int block_scale_bytes(int R, int K) {
  return 2 * R * (K / fmt_group(MODE)) * fmt_sbytes(MODE);
}

// LDS bytes of one wave's scale staging: two block buffers (alternate
// blocks), each of whole 1 KB load windows of scales, then as many of biases.
template <int MODE>
int slds_wave_bytes(int R, int K) {
  const int win = (block_scale_bytes<MODE>(R, K) + 1023) >> 10;
  return 2 * win * 1024 * (fmt_affine(MODE) ? 2 : 1);
}

// The weight matrices of one launch of the fast kernel.  Several matrices
// that share x, K and the format (a decoder's gate and up projections) run
// as one launch: their blocks of 2R rows are numbered one matrix after the
// other (matrix i owns blocks bstart[i] ..), each block reads its own
// matrix and writes its own y, scaled by its own global scale.  A single
// matrix is count = 1.  NM slots; the kernel arguments stay as small as
// a single matrix's for NM = 1.
constexpr int kQmvMats = 4;
template <int NM>
struct QmvMats {
  const uint8_t* codes[NM];
  const uint8_t* scales[NM];
  const uint8_t* biases[NM];
  const float* gscale[NM];  // NVFP4 global scale (NULL: 1)
  uint16_t* y[NM];
  int rows[NM];
  int bstart[NM];
  int count;
};

// a[i] for a wave-uniform i < NM, by selects over constant indices (a
// dynamic index into a kernel-argument array would copy it to scratch
// memory); NM = 1 reads a[0] alone
template <int NM, class T, int L>
__device__ __forceinline__ T pick(const T (&a)[L], int i) {
  T v = a[0];
#pragma unroll
  for (int j = 1; j < NM; ++j) v = (i == j) ? a[j] : v;
  return v;
}

// MAXM: compile-time bound on M.  R: rows per team per block.
// RAGGED: the row length in chunks is not a multiple of 32, so some lanes
//   have no chunk in the last step; their scale and bias are forced to zero
//   (x is zero there already) so a NaN or Inf scale of the next row cannot
//   leak in.
// SLDS: the block's scales (2R rows, contiguous) go straight from memory
//   into one of the wave's two LDS block buffers (16 bytes per lane and
//   load, issued just before the codes of the block's first step) and are
//   read from there per chunk -- instead of one 1- or 2-byte load per chunk.
//   Consecutive blocks of a wave alternate buffers, so a block's scales land
//   while the previous block still reads its own.  The loads are not tracked
//   by the compiler: the first step of a block waits for them explicitly.
//   Memory operations complete in issue order and that step's codes were
//   issued after them, so the wait (at most PJ steps of loads in flight) is
//   one the step's own code loads need anyway; output stores issued since
//   only make it slightly stricter.  Needs a whole number of 16-byte pieces
//   per row, at most SL loads per lane (4 for NVFP4, 2 otherwise), and
//   PJ <= NJ.
// QX (qq decode): x is quantized with the weights' format while it is
// staged and the products run on its exact dequantization; for NVFP4 with
// qx_amax set, every workgroup takes the global activation scale
// g_x = amax(x) / 2688 over the whole x it stages and folds it into the
// output scale (without it, g_x = 1).
// NM: matrix slots of the launch (1 for one matrix; the code for the
// matrix list is compiled only where it is used).
template <int MODE, int MAXM, int R, bool RAGGED, bool SLDS, bool QX, int NM = 1>
__global__ __launch_bounds__((fast_threads<MODE, MAXM>())) void qmv_fast_kernel(
    const uint16_t* __restrict__ x, int M, int K, const QmvMats<NM> mats,
    const float* __restrict__ g2ptr, int NJ, int nblocks, int qx_amax) {
  static_assert(!QX || MODE == FMT_MXFP4 || MODE == FMT_NVFP4,
                "qq needs a 4-bit float format");
  static_assert(!(SLDS && RAGGED), "staged scales need whole 32-chunk steps");
  // MODE is a format id: the three base formats, MXFP8 or an affine variant
  constexpr bool AFF = fmt_affine(MODE);
  constexpr bool MX = (MODE == FMT_MXFP4 || MODE == FMT_MXFP8);  // one E8M0 byte per chunk
  constexpr int BITS = fmt_bits(MODE);
  constexpr int CB = 4 * BITS;   // code bytes of a 32-element chunk
  constexpr int PJ = steps_in_flight<R>();
  constexpr int LPS = R * (BITS == 8 ? 2 : 1);  // code loads per step
  constexpr int gs = fmt_group(MODE);
  constexpr int sbytes = fmt_sbytes(MODE);
  constexpr int sstep = 32 * 32 / gs * sbytes;  // scale bytes of one step (32 chunks)
  extern __shared__ uint4 smem[];
  uint4* xp = smem;
  float* xs = reinterpret_cast<float*>(smem + M * NJ * 128);

  const int lane = threadIdx.x & 63, h = lane >> 5, lt = lane & 31;
  const int wpg = blockDim.x >> 6;
  const int wave_in_wg = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int G = gridDim.x, wg = blockIdx.x;
  const int cpr = K >> 5;
  const int rb = K / 8 * BITS;        // code bytes per row
  const int srb = (K / gs) * sbytes;  // scale bytes per row
  // Blocks are dealt round-robin over the workgroups (one per CU), then over
  // the waves of a workgroup: pass p of this wave takes block
  // (p * wpg + wave_in_wg) * G + wg, so no CU has more than one extra block.
  const int nb_wg = nblocks > wg ? (nblocks - wg + G - 1) / G : 0;
  const int passes = wave_in_wg < nb_wg ? (nb_wg - wave_in_wg + wpg - 1) / wpg : 0;
  const int steps = passes * NJ;
  // output scale factors: a block's is ((its matrix's NVFP4 global scale)
  // * g2) * gq, in this order (gq: the qq decode's activation scale)
  const float g2v = g2ptr ? *g2ptr : 1.0f;
  // one matrix: its global scale, read once; a matrix list reads its
  // block's matrix's at the block's end
  const float gw0 = (MODE == BSFP_NVFP4 && mats.gscale[0]) ? *mats.gscale[0] : 1.0f;

  // this wave's scale areas (SLDS): two block buffers, each nsl KB of
  // [2R rows][srb] scales, then nsl KB of biases
  const int sarea = 2 * R * srb;
  const int nsl = (sarea + 1023) >> 10;  // 16-byte scale loads per lane and array
  const int sbuf = nsl * 1024;           // bytes of one array in one buffer
  const int spar = (AFF ? 2 : 1) * sbuf;  // bytes of one block buffer
  uint8_t* sl = reinterpret_cast<uint8_t*>(smem + (M * NJ * (AFF ? 136 : 128))) +
                wave_in_wg * 2 * spar;

  int vc[R], vs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    vc[r] = (2 * r + h) * rb + CB * lt;
    // the chunk's scale: its group's (affine bf16, MX one byte), NVFP4 the
    // chunk's two E4M3 bytes
    vs[r] = (2 * r + h) * srb + (AFF ? 2 * (lt * 32 / gs) : MX ? lt : 2 * lt);
  }

  rsrc_t rc, rs, rbs;
  // pass p's block: its matrix and first row there
  auto block_of = [&](int p, int& mi, int64_t& row0) {
    const int gb = (p * wpg + wave_in_wg) * G + wg;
    mi = 0;
#pragma unroll
    for (int j = 1; j < NM; ++j)
      if (j < mats.count && gb >= mats.bstart[j]) mi = j;
    row0 = (int64_t)(gb - pick<NM>(mats.bstart, mi)) * (2 * R);
  };
  auto set_block = [&](int p) {
    int mi;
    int64_t row0;
    block_of(p, mi, row0);
    const int64_t rows = min((int64_t)pick<NM>(mats.rows, mi) - row0, (int64_t)(2 * R));
    rc = make_rsrc(pick<NM>(mats.codes, mi) + row0 * rb, rows * rb);
    rs = make_rsrc(pick<NM>(mats.scales, mi) + row0 * srb, rows * srb);
    if constexpr (AFF) rbs = make_rsrc(pick<NM>(mats.biases, mi) + row0 * srb, rows * srb);
  };
  constexpr int SL = (MODE == BSFP_NVFP4) ? 4 : 2;
  // 4-bit codes and their scales are read once, each load over whole cache
  // lines: non-temporal loads (cache policy 2).  Decode sweep, interleaved
  // A/B: the codes alone 46.0-46.2 against 48.1-48.5 us per layer (down
  // 17.3 against 19.1, gate+up 28.0 against 29.0; the sc0 policy instead
  // 47.2-47.9); the scales as well, one [25600, 5120] launch: NVFP4 15.3
  // against 15.7, affine 15.6 against 16.1 us.  8-bit codes keep the
  // default policy: a lane's 32 bytes come in two loads that split each
  // cache line, and with nt the second fetches it again (MXFP8 [25600,
  // 5120] fell from 5413 to 4657 GB/s).
  constexpr bool kNt = BITS == 4;
  constexpr int kPolicy = kNt ? 2 : 0;
  // fetch step j of the current block; `real` is false for the refills past
  // the wave's last step, `par` is the block's buffer
  auto fetch = [&](Chunk (&dst)[R], int j, bool real, int par) {
    if constexpr (SLDS) {
      if (j == 0 && real) {  // the block's scales, straight into its LDS buffer
        uint8_t* b = sl + par * spar;
#pragma unroll
        for (int i = 0; i < SL; ++i) {
          if (i < nsl) {
            if constexpr (kNt) {
              buffer_load_lds16_nt(rs, reinterpret_cast<uint4*>(b + i * 1024), 16 * lane + i * 1024, 0);
              if constexpr (AFF)
                buffer_load_lds16_nt(rbs, reinterpret_cast<uint4*>(b + sbuf + i * 1024),
                                     16 * lane + i * 1024, 0);
            } else {
              buffer_load_lds16(rs, reinterpret_cast<uint4*>(b + i * 1024), 16 * lane + i * 1024, 0);
              if constexpr (AFF)
                buffer_load_lds16(rbs, reinterpret_cast<uint4*>(b + sbuf + i * 1024),
                                  16 * lane + i * 1024, 0);
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if constexpr (kNt) {
        dst[r].w = buffer_load_u128_nt(rc, vc[r], j * 32 * CB);
      } else {
        dst[r].w = buffer_load_u128(rc, vc[r], j * 32 * CB);
        if constexpr (BITS == 8) dst[r].w2 = buffer_load_u128(rc, vc[r] + 16, j * 32 * CB);
      }
      if constexpr (!SLDS) {
        if constexpr (AFF) {
          dst[r].s = __builtin_amdgcn_raw_buffer_load_b16(rs, vs[r], j * sstep, kPolicy);
          dst[r].b = __builtin_amdgcn_raw_buffer_load_b16(rbs, vs[r], j * sstep, kPolicy);
        } else if constexpr (MX) {
          dst[r].s = __builtin_amdgcn_raw_buffer_load_b8(rs, vs[r], j * sstep, kPolicy);
        } else {
          dst[r].s = __builtin_amdgcn_raw_buffer_load_b16(rs, vs[r], j * sstep, kPolicy);
        }
      }
    }
  };

  float acc[R][MAXM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[r][m] = 0.0f;

  // x loads first, then the first PJ steps of weights; staging x into LDS
  // then waits only for the x loads (loads complete in issue order).
  uint4 xr[fast_xu<MODE, MAXM>()];
  stage_x_load(x, M, K, NJ, xr);
  Chunk ring[PJ][R];
  int pf = 0, jf = 0;  // next step to fetch
  // The first PJ steps are fetched by every wave (a wave with no rows reads
  // through empty descriptors, which returns zeros without touching memory),
  // so the compiler sees a fixed number of loads after the x loads and the
  // x staging below waits for the x loads alone.
  if (steps > 0) {
    set_block(0);
  } else {
    rc = make_rsrc(mats.codes[0], 0);
    rs = make_rsrc(mats.scales[0], 0);
    if constexpr (AFF) rbs = make_rsrc(mats.biases[0], 0);
  }
#pragma unroll
  for (int u = 0; u < PJ; ++u) {
    fetch(ring[u], pf < passes ? jf : NJ - 1, pf < passes, pf & 1);
    if (pf < passes && ++jf == NJ) {
      jf = 0;
      if (++pf < passes) set_block(pf);
    }
  }
  float gq = 1.0f;
  if constexpr (QX && MODE == BSFP_NVFP4) {
    if (qx_amax) {
      // max |x| over the staged x: per wave, then over the waves through the
      // (not yet written) x area of LDS
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < fast_xu<MODE, MAXM>(); ++i) {
        float f[8];
        unpack8(xr[i], f);  // units past the end were loaded as zeros
#pragma unroll
        for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
      }
      a = team_max<64>(a);
      float* red = reinterpret_cast<float*>(xp);
      if (lane == 0) red[wave_in_wg] = a;
      __syncthreads();
      a = red[0];
      for (int w2 = 1; w2 < wpg; ++w2) a = fmaxf(a, red[w2]);
      __syncthreads();
      gq = a / 2688.0f;
    }
  }
  stage_x_store<AFF, AFF && BITS == 4, fast_xu<MODE, MAXM>(), QX ? MODE : -1>(M, NJ, xr, xp, xs, gq);
  __syncthreads();
  if (steps == 0) {
    wait_vmem();  // the empty refills have returned
    return;
  }

  int pc = 0, jc = 0;  // next step to consume
  for (int s0 = 0; s0 < steps; s0 += PJ) {
#pragma unroll
    for (int u = 0; u < PJ; ++u) {
      if (s0 + u < steps) {
        if constexpr (SLDS) {
          // this block's scales were issued before the codes of this step:
          // once at most PJ steps of code loads are in flight, they are in LDS
          if (jc == 0) wait_vmem_le<PJ * LPS>();
        }
        const bool valid = !RAGGED || (32 * jc + lt < cpr);
        uint32_t sv[R], bv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if constexpr (SLDS) {
            const uint8_t* sp = sl + (pc & 1) * spar + vs[r] + jc * sstep;
            if constexpr (AFF) {
              sv[r] = *reinterpret_cast<const uint16_t*>(sp);
              bv[r] = *reinterpret_cast<const uint16_t*>(sp + sbuf);
            } else if constexpr (MX) {
              sv[r] = *sp;
            } else {
              sv[r] = *reinterpret_cast<const uint16_t*>(sp);
            }
          } else {
            sv[r] = valid ? ring[u][r].s : 0u;
            bv[r] = valid ? ring[u][r].b : 0u;
          }
        }
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
          if (MAXM > 1 && m >= M) break;
          const uint4* xq = xp + (m * NJ + jc) * 128 + lt;
          const uint4 x0 = xq[0], x1 = xq[32], x2 = xq[64], x3 = xq[96];
          const float xsum = AFF ? xs[(m * NJ + jc) * 32 + lt] : 0.0f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            // a lane past the row's last chunk (RAGGED) loaded the next row's
            // codes: zero them, so that a NaN code there (an E4M3 byte
            // 0x7F / 0xFF) cannot reach this row's sum through 0 * NaN
            const uint4 w = valid ? ring[u][r].w : make_uint4(0u, 0u, 0u, 0u);
            if constexpr (AFF && BITS == 8) {
              // 8-bit affine: q = lo + 16 hi over the two nibble planes of
              // each byte, each converted exactly (E4M3 byte trick); x in
              // natural order, element k of a word in byte k % 4
              const uint4 w2 = valid ? ring[u][r].w2 : make_uint4(0u, 0u, 0u, 0u);
              const uint32_t ww[8] = {w.x, w.y, w.z, w.w, w2.x, w2.y, w2.z, w2.w};
              const uint32_t xx[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                       x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
              float Dl = 0.0f, Dh = 0.0f;
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const uint32_t lo = ww[q] & 0x0F0F0F0Fu, hi = (ww[q] >> 4) & 0x0F0F0F0Fu;
                Dl = dot2_bf16(xx[2 * q], nibbles_to_bf16x2<false>(lo), Dl);
                Dl = dot2_bf16(xx[2 * q + 1], nibbles_to_bf16x2<true>(lo), Dl);
                Dh = dot2_bf16(xx[2 * q], nibbles_to_bf16x2<false>(hi), Dh);
                Dh = dot2_bf16(xx[2 * q + 1], nibbles_to_bf16x2<true>(hi), Dh);
              }
              acc[r][m] = __builtin_fmaf(__uint_as_float(sv[r] << 16),
                                         __builtin_fmaf(16.0f, Dh, Dl), acc[r][m]);
              acc[r][m] = __builtin_fmaf(__uint_as_float(bv[r] << 16), xsum, acc[r][m]);
            } else if constexpr (MODE == FMT_MXFP8) {
              // E4M3 bytes -> bf16 pairs (exact), one E8M0 scale per chunk
              const uint4 w2 = valid ? ring[u][r].w2 : make_uint4(0u, 0u, 0u, 0u);
              const uint32_t ww[8] = {w.x, w.y, w.z, w.w, w2.x, w2.y, w2.z, w2.w};
              const uint32_t xx[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                       x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
              float D = 0.0f;
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                D = dot2_bf16(xx[2 * q], e4m3x2_to_bf16x2<false>(ww[q]), D);
                D = dot2_bf16(xx[2 * q + 1], e4m3x2_to_bf16x2<true>(ww[q]), D);
              }
              acc[r][m] = __builtin_fmaf(D, e8m0_decode(sv[r]), acc[r][m]);
            } else if constexpr (AFF) {
              float D0 = 0.0f, D1 = 0.0f;
              const uint64_t h01 = (((uint64_t)w.y << 32) | w.x) >> 4;
              const uint64_t h23 = (((uint64_t)w.w << 32) | w.z) >> 4;
              uint32_t t = w.x & 0x0F0F0F0Fu, q = (uint32_t)h01 & 0x0F0F0F0Fu;
              D0 = dot2_bf16(x0.x, nibbles_to_bf16x2<false>(t), D0);
              D0 = dot2_bf16(x0.y, nibbles_to_bf16x2<true>(t), D0);
              D0 = dot2_bf16(x0.z, nibbles_to_bf16x2<false>(q), D0);
              D0 = dot2_bf16(x0.w, nibbles_to_bf16x2<true>(q), D0);
              t = w.y & 0x0F0F0F0Fu, q = (uint32_t)(h01 >> 32) & 0x0F0F0F0Fu;
              D1 = dot2_bf16(x1.x, nibbles_to_bf16x2<false>(t), D1);
              D1 = dot2_bf16(x1.y, nibbles_to_bf16x2<true>(t), D1);
              D1 = dot2_bf16(x1.z, nibbles_to_bf16x2<false>(q), D1);
              D1 = dot2_bf16(x1.w, nibbles_to_bf16x2<true>(q), D1);
              t = w.z & 0x0F0F0F0Fu, q = (uint32_t)h23 & 0x0F0F0F0Fu;
              D0 = dot2_bf16(x2.x, nibbles_to_bf16x2<false>(t), D0);
              D0 = dot2_bf16(x2.y, nibbles_to_bf16x2<true>(t), D0);
              D0 = dot2_bf16(x2.z, nibbles_to_bf16x2<false>(q), D0);
              D0 = dot2_bf16(x2.w, nibbles_to_bf16x2<true>(q), D0);
              t = w.w & 0x0F0F0F0Fu, q = (uint32_t)(h23 >> 32) & 0x0F0F0F0Fu;
              D1 = dot2_bf16(x3.x, nibbles_to_bf16x2<false>(t), D1);
              D1 = dot2_bf16(x3.y, nibbles_to_bf16x2<true>(t), D1);
              D1 = dot2_bf16(x3.z, nibbles_to_bf16x2<false>(q), D1);
              D1 = dot2_bf16(x3.w, nibbles_to_bf16x2<true>(q), D1);
              acc[r][m] = __builtin_fmaf(__uint_as_float(sv[r] << 16), D0 + D1, acc[r][m]);
              acc[r][m] = __builtin_fmaf(__uint_as_float(bv[r] << 16), xsum, acc[r][m]);
            } else {
              float D0 = 0.0f, D1 = 0.0f;
              D0 = dot2_bf16(x0.x, e2m1x2_to_bf16x2<0>(w.x), D0);
              D0 = dot2_bf16(x0.y, e2m1x2_to_bf16x2<1>(w.x), D0);
              D0 = dot2_bf16(x0.z, e2m1x2_to_bf16x2<2>(w.x), D0);
              D0 = dot2_bf16(x0.w, e2m1x2_to_bf16x2<3>(w.x), D0);
              D0 = dot2_bf16(x1.x, e2m1x2_to_bf16x2<0>(w.y), D0);
              D0 = dot2_bf16(x1.y, e2m1x2_to_bf16x2<1>(w.y), D0);
              D0 = dot2_bf16(x1.z, e2m1x2_to_bf16x2<2>(w.y), D0);
              D0 = dot2_bf16(x1.w, e2m1x2_to_bf16x2<3>(w.y), D0);
              D1 = dot2_bf16(x2.x, e2m1x2_to_bf16x2<0>(w.z), D1);
              D1 = dot2_bf16(x2.y, e2m1x2_to_bf16x2<1>(w.z), D1);
              D1 = dot2_bf16(x2.z, e2m1x2_to_bf16x2<2>(w.z), D1);
              D1 = dot2_bf16(x2.w, e2m1x2_to_bf16x2<3>(w.z), D1);
              D1 = dot2_bf16(x3.x, e2m1x2_to_bf16x2<0>(w.w), D1);
              D1 = dot2_bf16(x3.y, e2m1x2_to_bf16x2<1>(w.w), D1);
              D1 = dot2_bf16(x3.z, e2m1x2_to_bf16x2<2>(w.w), D1);
              D1 = dot2_bf16(x3.w, e2m1x2_to_bf16x2<3>(w.w), D1);
              if constexpr (MODE == FMT_MXFP4) {
                acc[r][m] = __builtin_fmaf(D0 + D1, e8m0_decode(sv[r]), acc[r][m]);
              } else {
                // both E4M3 block scales with the hardware converter (exact)
                const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sv[r], 1.0f, false);
                acc[r][m] = __builtin_fmaf(D0, sc.x, acc[r][m]);
                acc[r][m] = __builtin_fmaf(D1, sc.y, acc[r][m]);
              }
            }
          }
        }
        if (jc == NJ - 1) {  // the block's rows are complete
          int mi;
          int64_t row0;
          block_of(pc, mi, row0);
          const int64_t N = pick<NM>(mats.rows, mi);
          uint16_t* const y = pick<NM>(mats.y, mi);
          float gwi = gw0;
          if constexpr (NM > 1) {
            const float* const gs_i = pick<NM>(mats.gscale, mi);
            gwi = (MODE == BSFP_NVFP4 && gs_i) ? *gs_i : 1.0f;
          }
          const float gb = (gwi * g2v) * gq;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int64_t row = row0 + 2 * r + h;
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
              if (MAXM > 1 && m >= M) break;
              const float v = dpp_sum32(acc[r][m]);
              if (lt == 0 && row < N) y[(int64_t)m * N + row] = (uint16_t)f32_to_bf16(v * gb);
              acc[r][m] = 0.0f;
            }
          }
        }
        if (++jc == NJ) {
          jc = 0;
          ++pc;
        }
      }
      // refill this slot with step s0 + u + PJ (past the end: reload the last
      // step, whose data is never consumed)
      fetch(ring[u], pf < passes ? jf : NJ - 1, pf < passes, pf & 1);
      if (pf < passes && ++jf == NJ) {
        jf = 0;
        if (++pf < passes) set_block(pf);
      }
    }
  }
}

template <int MODE, int MAXM>
size_t lds_bytes(int64_t k) {
  return (size_t)k * 2 * MAXM + (MODE == BSFP_AFFINE ? (size_t)(k / 64) * 4 * MAXM : 0);
}

template <int MODE, int MAXM>
hipError_t run(const uint16_t* x, int M, const bsfp_qtensor& w, const float* g2, uint16_t* y,
               hipStream_t s) {
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
  launch_main(&qmv_kernel<MODE, MAXM>, dim3((unsigned)grid), dim3(kThreads), lds, s, x,
                     M, K, N, reinterpret_cast<const uint4*>(w.codes), w.scales, w.biases,
                     w.global_scale, g2, y, (int)ks, nslices);
  return hipGetLastError();
}

// Launch shape of the fast kernel: one workgroup per CU (its LDS request is
// raised above half of the CU's LDS when needed, so two never share a CU),
// with as many waves (at most 16) as it takes to hold every block in one
// pass, or in as few passes as possible; at least enough waves to stage x.
struct FastShape {
  int grid, wpg;
  size_t lds;
};

// nblocks: the launch's blocks of 2R rows (a matrix list's, summed over its
// matrices), or -1 for one matrix of N rows.
template <int MODE, int MAXM, int R, bool SLDS>
FastShape fast_shape(int M, int K, int NJ, int64_t N, int64_t nblocks = -1) {
  constexpr int kMaxW = fast_threads<MODE, MAXM>() / 64, kXu = fast_xu<MODE, MAXM>();
  constexpr int kPerCu = 1024 / fast_threads<MODE, MAXM>();  // workgroups per CU
  const int cus = device_cu_count();
  if (nblocks < 0) nblocks = (N + 2 * R - 1) / (2 * R);
  const int units = M * NJ * 128;
  const int min_wpg = std::max(1, (units + kXu * 64 - 1) / (kXu * 64));
  const int64_t grid = std::min<int64_t>((int64_t)kPerCu * cus, nblocks);
  const int64_t passes = std::max<int64_t>(1, (nblocks + grid * kMaxW - 1) / (grid * kMaxW));
  // One pass: every workgroup takes the most waves (the ones without a block
  // only share the staging of x).  On the [5120, 25600] decode shape (10
  // blocks and 51 KB of x per CU) 16 waves leave no room for the per-wave
  // scale buffers next to x, so that launch reads its scales per chunk; by
  // interleaved A/B (affine, us): staged scales on 13 waves 19.3, per-chunk
  // scales on 13 waves 19.1, on 16 waves 18.9 (and 19.3-19.4 against
  // 19.9-20.1 on two more boxes).  Several passes: the fewest waves that
  // keep that many passes.
  const int wpg = passes == 1 ? kMaxW : (int)std::min<int64_t>(
      kMaxW, std::max<int64_t>(min_wpg, (nblocks + grid * passes - 1) / (grid * passes)));
  size_t lds = fast_lds_bytes<MODE>(M, NJ) +
               (SLDS ? (size_t)wpg * slds_wave_bytes<MODE>(R, K) : 0);
  const size_t half = (size_t)device_max_lds() / 2 + 16;
  if (kPerCu == 1 && grid == cus && wpg <= 8 && lds < half) lds = half;
  return FastShape{(int)grid, wpg, lds};
}

// A matrix list of `count` matrices that share x, K and the format; returns
// its number of blocks of 2R rows.
template <int NM>
int64_t fill_mats(QmvMats<NM>& m, const bsfp_qtensor* const* ws, uint16_t* const* ys,
                  int count, int R) {
  m = QmvMats<NM>{};
  int64_t nb = 0;
  for (int i = 0; i < count; ++i) {
    m.codes[i] = reinterpret_cast<const uint8_t*>(ws[i]->codes);
    m.scales[i] = reinterpret_cast<const uint8_t*>(ws[i]->scales);
    m.biases[i] = reinterpret_cast<const uint8_t*>(ws[i]->biases);
    m.gscale[i] = ws[i]->global_scale;
    m.y[i] = ys[i];
    m.rows[i] = (int)ws[i]->rows;
    m.bstart[i] = (int)nb;
    nb += (ws[i]->rows + 2 * R - 1) / (2 * R);
  }
  m.count = count;
  return nb;
}

template <int MODE, int MAXM, int R, bool RAGGED, bool SLDS, bool QX, int NM = 1>
hipError_t launch_fast_mats(const uint16_t* x, int M, const bsfp_qtensor* const* ws,
                            uint16_t* const* ys, int count, const float* g2, int NJ,
                            hipStream_t s, int qx_amax) {
  const int K = (int)ws[0]->cols;
  QmvMats<NM> mats;
  const int64_t nblocks = fill_mats(mats, ws, ys, count, R);
  int64_t N = 0;
  for (int i = 0; i < count; ++i) N += ws[i]->rows;
  const FastShape sh = fast_shape<MODE, MAXM, R, SLDS>(M, K, NJ, N, nblocks);
  // opt in to the large LDS allocation (160 KB on gfx950), once per device
  // and size
  static std::atomic<size_t> lds_granted[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (sh.lds > 64 * 1024 && sh.lds > lds_granted[dev].load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&qmv_fast_kernel<MODE, MAXM, R, RAGGED, SLDS, QX, NM>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh.lds);
    if (e != hipSuccess) return e;
    lds_granted[dev].store(sh.lds, std::memory_order_relaxed);
  }
  launch_main(&qmv_fast_kernel<MODE, MAXM, R, RAGGED, SLDS, QX, NM>, dim3((unsigned)sh.grid),
                     dim3(64 * sh.wpg), sh.lds, s, x, M, K, mats, g2, NJ, (int)nblocks,
                     qx_amax);
  return hipGetLastError();
}

template <int MODE, int MAXM, int R, bool RAGGED, bool SLDS, bool QX>
hipError_t launch_fast(const uint16_t* x, int M, const bsfp_qtensor& w, const float* g2,
                       uint16_t* y, int NJ, hipStream_t s, int qx_amax) {
  const bsfp_qtensor* ws[1] = {&w};
  uint16_t* ys[1] = {y};
  return launch_fast_mats<MODE, MAXM, R, RAGGED, SLDS, QX>(x, M, ws, ys, 1, g2, NJ, s, qx_amax);
}

// The staged x (XU units per thread) is limited to 64 KB; the per-wave
// scale areas come on top, up to the device's per-workgroup LDS limit.
constexpr size_t kFastXLdsMax = 64 * 1024;

template <int MODE>
bool fast_ok(int M, int NJ) {
  return (size_t)M * NJ * 2048 <= kFastXLdsMax &&
         fast_lds_bytes<MODE>(M, NJ) <= (size_t)device_max_lds();
}

// Staged scales apply when every row holds whole 32-chunk steps and whole
// 16-byte scale pieces, the block's scales fit the scale loads per lane,
// at most NJ steps are in flight, and the LDS fits.
template <int MODE, int R>
bool slds_ok(int K, int NJ, int M, int64_t N, int64_t nblocks = -1) {
  const int cpr = K / 32;
  const int sarea = block_scale_bytes<MODE>(R, K);
  const int srb = sarea / (2 * R);
  if (cpr % 32 || srb % 16 || sarea > (MODE == BSFP_NVFP4 ? 4 : 2) * 1024 || steps_in_flight<R>() > NJ) return false;
  return fast_shape<MODE, 1, R, true>(M, K, NJ, N, nblocks).lds <= (size_t)device_max_lds();
}

// The format variants: the same kernel with fewer launch shapes (2-row
// teams with staged scales for tall M = 1 matrices, else single rows), and
// x always in one LDS copy (callers check qmv_variant_supported).
template <int FMT>
hipError_t by_m_variant(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y,
                        hipStream_t s) {
  const int K = (int)w.cols;
  const int NJ = (int)((w.cols / 32 + 31) / 32);
  const bool ragged = (w.cols / 32) % 32 != 0;
  if (!fast_ok<FMT>(M, NJ)) return hipErrorNotSupported;
  const int64_t N = w.rows;
  if (M == 1) {
    if (N >= 32LL * device_cu_count() && slds_ok<FMT, 2>(K, NJ, M, N))
      return launch_fast<FMT, 1, 2, false, true, false>(x, M, w, nullptr, y, NJ, s, 0);
    if (slds_ok<FMT, 1>(K, NJ, M, N))
      return launch_fast<FMT, 1, 1, false, true, false>(x, M, w, nullptr, y, NJ, s, 0);
    if (ragged) return launch_fast<FMT, 1, 1, true, false, false>(x, M, w, nullptr, y, NJ, s, 0);
    return launch_fast<FMT, 1, 1, false, false, false>(x, M, w, nullptr, y, NJ, s, 0);
  }
  if (ragged) {
    if (M == 2) return launch_fast<FMT, 2, 1, true, false, false>(x, M, w, nullptr, y, NJ, s, 0);
    if (M <= 4) return launch_fast<FMT, 4, 1, true, false, false>(x, M, w, nullptr, y, NJ, s, 0);
    return launch_fast<FMT, 8, 1, true, false, false>(x, M, w, nullptr, y, NJ, s, 0);
  }
  if (M == 2) return launch_fast<FMT, 2, 1, false, false, false>(x, M, w, nullptr, y, NJ, s, 0);
  if (M <= 4) return launch_fast<FMT, 4, 1, false, false, false>(x, M, w, nullptr, y, NJ, s, 0);
  return launch_fast<FMT, 8, 1, false, false, false>(x, M, w, nullptr, y, NJ, s, 0);
}

// ---------------------------------------------------------------------------
// Several rows of x (2 <= M <= 8) on MFMA: v_mfma_f32_16x16x32_bf16 with x as
// the A operand (rows M..15 zero) and 16 weight rows, dequantized to bf16 in
// registers, as the B operand.  The per-row dot products of the GEMV above
// read every x value from LDS once per weight chunk and row of x, which makes
// M = 8 LDS-bound (and x beyond 64 KB takes the sliced fallback); here each
// wave reads an x fragment once for RBW blocks of 16 weight rows.
//   Contraction order: lane group g = lane / 16 of both operands holds the
//   32 elements k = 128 kb + 32 g + 0..31 of its row (A lane (m, g), B lane
//   (n, g); m, n = lane % 16), and MFMA i of block kb takes their elements
//   8 i .. 8 i + 7.  So a lane's weights are one 16-byte load, and each
//   lane's 32 elements are one MXFP4 group, two NVFP4 blocks, or half an
//   affine group of 64 (lane groups 0, 1 and 2, 3 hold its two groups).
//   MXFP4: the E8M0 scale goes into the E2M1 -> bf16 converter (exact).
//   NVFP4: E2M1 * E4M3 formed in fp32 and packed to bf16 (exact: at most 6
//     significant bits); the global scale multiplies the fp32 sums.
//   affine: the MFMAs run on the exact integer codes q, once with the x of
//     lane groups 0, 1 and once with those of 2, 3 (the others zeroed), and
//     on a block of ones for the sums of x in the output layout; each group
//     adds s * sum(x q) + b * sum(x) in fp32, the numerics of the GEMV above.
// Grid: one workgroup per group of 16 * RBW weight rows; its S waves split
// the K blocks (wave w takes blocks [w * kbw, (w + 1) * kbw)) and add their
// partial tiles through LDS in wave order.  Loads are raw buffer loads whose
// descriptors end with x and with the group's rows, so rows past N and
// rows of x past M read as zeros.
template <int MODE, int RBW, bool ODD>
__global__ __launch_bounds__(512) void qmv_mma_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint32_t* __restrict__ codes,
    const void* __restrict__ scales, const uint16_t* __restrict__ biases,
    const float* __restrict__ gptr, const float* __restrict__ g2ptr, uint16_t* __restrict__ y,
    int kbw) {
  static_assert(MODE == FMT_AFF4_G64 || MODE == FMT_MXFP4 || MODE == FMT_NVFP4,
                "4-bit base formats");
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr bool AFF = MODE == FMT_AFF4_G64;
  constexpr int D = 2;  // K blocks per register stage
  constexpr int P = 2;  // register stages: P - 1 of them load while one computes
  extern __shared__ f32x4_t red[];  // [S][RBW][64] partial tiles
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int S = blockDim.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * RBW;
  const int rows = (int)min((int64_t)N - n0, (int64_t)16 * RBW);
  const int rb = K / 2;                       // code bytes per row
  const int nkb = (K + 127) / 128;            // 128-element blocks
  const int kb0 = w * kbw, kb1 = min(nkb, kb0 + kbw);
  const rsrc_t rx = make_rsrc(x, (int64_t)M * K * 2);
  const rsrc_t rc = make_rsrc(reinterpret_cast<const uint8_t*>(codes) + n0 * rb,
                              (int64_t)rows * rb);
  const int srb = AFF ? (K / 64) * 2 : (MODE == FMT_MXFP4 ? K / 32 : K / 16);  // scale bytes per row
  const rsrc_t rs = make_rsrc(reinterpret_cast<const uint8_t*>(scales) + n0 * srb,
                              (int64_t)rows * srb);
  rsrc_t rbs = rs;
  if constexpr (AFF)
    rbs = make_rsrc(reinterpret_cast<const uint8_t*>(biases) + n0 * srb, (int64_t)rows * srb);

  f32x4_t acc[RBW];
#pragma unroll
  for (int r = 0; r < RBW; ++r) acc[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // bf16 ones: the B operand that turns an MFMA into sums of x
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
  // in the last block (K % 128 != 0) a lane's elements may end early: it
  // keeps its first vw 8-element words (K is a multiple of 16 for NVFP4, of
  // 32 otherwise); the words past the row end read the next row's codes or
  // zeros and are replaced by zeros below, and so are the scales that go
  // with them, so that no such value reaches the sums (not even a NaN)

  // a ring of P register stages of D blocks each: the loads of the next
  // P - 1 stages are in flight while one stage is computed
  struct Stage {
    uint4 xa[D][4];
    uint4 wc[D][RBW];
    uint32_t sc[D][RBW], bc[D][RBW];
  };
  // the loads of blocks kbr .. kbr + D - 1.  Every load is issued, with no
  // branch around it, so that the compiler's wait counts stay exact and the
  // compute of one stage waits for that stage's loads alone (a load skipped
  // on some path makes it wait for all of them).  Blocks past kb1 take an
  // offset past every descriptor's end: zeros, no memory traffic.
  constexpr int kDead = 0x7FFFFF00;
  auto load = [&](Stage& st, int kbr) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kb = kbr + d;
      const bool live = kb < kb1;
      // x[m, 128 kb + 32 g + 8 i ..]: 64 contiguous bytes per lane
      const int xo = live ? c * K * 2 + (128 * kb + 32 * g) * 2 : kDead;
#pragma unroll
      for (int i = 0; i < 4; ++i) st.xa[d][i] = buffer_load_u128(rx, xo + 16 * i, 0);
#pragma unroll
      for (int r = 0; r < RBW; ++r) {
        const int row = 16 * r + c;
        st.wc[d][r] = buffer_load_u128(rc, live ? row * rb + 64 * kb + 16 * g : kDead, 0);
        if constexpr (AFF) {  // both groups of the block: scales, then biases
          const int so = live ? row * srb + 4 * kb : kDead;
          if constexpr (!ODD) {  // 4-byte aligned: one load per array
            st.sc[d][r] = __builtin_amdgcn_raw_buffer_load_b32(rs, so, 0, 0);
            st.bc[d][r] = __builtin_amdgcn_raw_buffer_load_b32(rbs, so, 0, 0);
          } else {  // an odd number of groups per row (K % 128 == 64)
            st.sc[d][r] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0) |
                          (__builtin_amdgcn_raw_buffer_load_b16(rs, so + 2, 0, 0) << 16);
            st.bc[d][r] = __builtin_amdgcn_raw_buffer_load_b16(rbs, so, 0, 0) |
                          (__builtin_amdgcn_raw_buffer_load_b16(rbs, so + 2, 0, 0) << 16);
          }
        } else if constexpr (MODE == FMT_MXFP4) {  // the E8M0 byte of chunk 4 kb + g
          st.sc[d][r] =
              __builtin_amdgcn_raw_buffer_load_b8(rs, live ? row * srb + 4 * kb + g : kDead, 0, 0);
        } else if constexpr (!ODD) {  // the E4M3 bytes of blocks 8 kb + 2 g, 8 kb + 2 g + 1
          st.sc[d][r] = __builtin_amdgcn_raw_buffer_load_b16(
              rs, live ? row * srb + 8 * kb + 2 * g : kDead, 0, 0);
        } else {  // odd bytes per row (K % 32 == 16): the pair may be unaligned
          const int o = live ? row * srb + 8 * kb + 2 * g : kDead;
          st.sc[d][r] = __builtin_amdgcn_raw_buffer_load_b8(rs, o, 0, 0) |
                        (__builtin_amdgcn_raw_buffer_load_b8(rs, o + 1, 0, 0) << 8);
        }
      }
    }
  };
  auto compute = [&](const Stage& st, int kbr) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kb = kbr + d;
      if (kb >= kb1) break;
      const int vw = min(4, max(0, (K - 128 * kb - 32 * g) >> 3));
      float sf[RBW][2];
#pragma unroll
      for (int r = 0; r < RBW; ++r) {
        if constexpr (MODE == FMT_MXFP4) {
          // the converter reads the exponent of this float
          sf[r][0] = vw > 0 ? __uint_as_float((st.sc[d][r] & 0xFFu) << 23) : 1.0f;
        } else if constexpr (MODE == FMT_NVFP4) {
          const f32x2_t sp = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(st.sc[d][r], 1.0f, false);
          sf[r][0] = vw > 0 ? sp[0] : 0.0f;
          sf[r][1] = vw > 2 ? sp[1] : 0.0f;
        }
      }
      f32x4_t xs0 = {0.0f, 0.0f, 0.0f, 0.0f}, xs1 = xs0;
      f32x4_t dq0[RBW], dq1[RBW];
      if constexpr (AFF) {
#pragma unroll
        for (int r = 0; r < RBW; ++r) dq0[r] = dq1[r] = xs0;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 xv = i < vw ? st.xa[d][i] : zero4;
        if constexpr (AFF) {
          // groups 2 kb (lane groups 0, 1) and 2 kb + 1 (lane groups 2, 3)
          const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, g < 2 ? xv : zero4);
          const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, g < 2 ? zero4 : xv);
          xs0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8_t, ones), xs0,
                                                        0, 0, 0);
          xs1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8_t, ones), xs1,
                                                        0, 0, 0);
#pragma unroll
          for (int r = 0; r < RBW; ++r) {
            const uint4 wv = st.wc[d][r];
            const uint32_t wd =
                i >= vw ? 0u : i == 0 ? wv.x : i == 1 ? wv.y : i == 2 ? wv.z : wv.w;
            // exact integer codes q (E4M3 byte trick)
            const uint32_t t = wd & 0x0F0F0F0Fu, u = (wd >> 4) & 0x0F0F0F0Fu;
            const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(t, 512.0f, false);  // q0, q2
            const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(t, 512.0f, true);   // q4, q6
            const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u, 512.0f, false);  // q1, q3
            const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u, 512.0f, true);   // q5, q7
            uint4 bv;
            bv.x = pack_bf16x2(p0.x, p2.x);
            bv.y = pack_bf16x2(p0.y, p2.y);
            bv.z = pack_bf16x2(p1.x, p3.x);
            bv.w = pack_bf16x2(p1.y, p3.y);
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv);
            dq0[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, dq0[r], 0, 0, 0);
            dq1[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, dq1[r], 0, 0, 0);
          }
        } else {
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xv);
#pragma unroll
          for (int r = 0; r < RBW; ++r) {
            const uint4 wv = st.wc[d][r];
            const uint32_t wd =
                i >= vw ? 0u : i == 0 ? wv.x : i == 1 ? wv.y : i == 2 ? wv.z : wv.w;
            uint4 bv;
            if constexpr (MODE == FMT_MXFP4) {
              const float sce = sf[r][0];
              bv.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sce, 0));
              bv.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sce, 1));
              bv.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sce, 2));
              bv.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sce, 3));
            } else {
              // words 0, 1 lie in the lane's first NVFP4 block, 2, 3 in its second
              const float f = sf[r][i >> 1];
              const f32x2_t q0 = e2m1x2_to_f32x2<0>(wd), q1 = e2m1x2_to_f32x2<1>(wd);
              const f32x2_t q2 = e2m1x2_to_f32x2<2>(wd), q3 = e2m1x2_to_f32x2<3>(wd);
              bv.x = pack_bf16x2(q0.x * f, q0.y * f);
              bv.y = pack_bf16x2(q1.x * f, q1.y * f);
              bv.z = pack_bf16x2(q2.x * f, q2.y * f);
              bv.w = pack_bf16x2(q3.x * f, q3.y * f);
            }
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bv),
                                                             acc[r], 0, 0, 0);
          }
        }
      }
      if constexpr (AFF) {
        // per group: s * sum(x q) + b * sum(x), in fp32 (the output lane's
        // column n = c is this lane's weight row)
#pragma unroll
        for (int r = 0; r < RBW; ++r) {
          // group 2 kb + 1 is past the row end when K - 128 kb <= 64
          const bool two = K - 128 * kb > 64;
          const float s0 = __uint_as_float(st.sc[d][r] << 16);
          const float s1 = two ? __uint_as_float(st.sc[d][r] & 0xFFFF0000u) : 0.0f;
          const float b0 = __uint_as_float(st.bc[d][r] << 16);
          const float b1 = two ? __uint_as_float(st.bc[d][r] & 0xFFFF0000u) : 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float a = acc[r][j];
            a = __builtin_fmaf(s0, dq0[r][j], a);
            a = __builtin_fmaf(b0, xs0[j], a);
            a = __builtin_fmaf(s1, dq1[r][j], a);
            a = __builtin_fmaf(b1, xs1[j], a);
            acc[r][j] = a;
          }
        }
      }
    }
  };
  Stage ring[P];
#pragma unroll
  for (int u = 0; u < P - 1; ++u) load(ring[u], kb0 + u * D);
  for (int kbr = kb0; kbr < kb1; kbr += P * D) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      load(ring[(u + P - 1) % P], kbr + (u + P - 1) * D);
      compute(ring[u], kbr + u * D);
    }
  }

  // the S partial tiles of each 16-row block r, added in wave order by wave
  // r % S (S may be smaller than RBW)
#pragma unroll
  for (int r = 0; r < RBW; ++r) red[(w * RBW + r) * 64 + lane] = acc[r];
  __syncthreads();
  const float gs = ((MODE == FMT_NVFP4 && gptr) ? *gptr : 1.0f) * (g2ptr ? *g2ptr : 1.0f);
  for (int r = w; r < RBW; r += S) {
    f32x4_t v = red[r * 64 + lane];
    for (int q = 1; q < S; ++q) {
      const f32x4_t o = red[(q * RBW + r) * 64 + lane];
      v[0] += o[0];
      v[1] += o[1];
      v[2] += o[2];
      v[3] += o[3];
    }
    // output layout: lane (n = lane % 16, g) holds rows m = 4 g .. 4 g + 3
    const int64_t n = n0 + 16 * r + c;
    if (n < N) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 4 * g + j;
        if (m < M) y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16(v[j] * gs);
      }
    }
  }
}

// Launch shape of qmv_mma_kernel: RBW blocks of 16 rows per workgroup and S
// <= 8 waves per workgroup splitting K, about 4 / RBW waves per CU.  Fewer,
// longer waves keep more of each wave's K blocks behind the load ring.
// The kernel is throughput-bound per CU, so a small matrix takes the RBW
// that puts the fewest rows on the busiest CU (ceil(groups / CUs) * 16 RBW);
// ties, and matrices of 2^25 weights or more, take RBW = 2 (x read once per
// 32 rows).  By measurement at M = 8 ((RBW, S) -> us, MXFP4 unless noted):
//   N = 4096 (256 groups of 16 rows: one per CU): (1, 4) 7.4, (2, 3) 8.8;
//   N = 4224 (264 groups: 8 CUs take two): (1, 4) 11.1, (2, 3) 9.0;
//   [5760, 2880]: (2, 3) 6.4, (1, 8) 8.3;  N = 8192: (2, 2) 9.2, (1, 4) 11.5;
//   [5120, 25600] NVFP4: (2, 4) 40.6, (1, 8) 56.9, affine 52.0 / 71.6;
//   [25600, 5120] NVFP4: (2, 1) 35.6, (2, 3) 36.8, (1, 1) 38.7.
// NVFP4 and affine follow the same pattern on these shapes.
template <int MODE>
hipError_t launch_mma(const uint16_t* x, int M, const bsfp_qtensor& w, const float* g2,
                      uint16_t* y, hipStream_t s) {
  const int64_t N = w.rows;
  const int K = (int)w.cols;
  const int nkb = (K + 127) / 128;
  auto go = [&](auto rbw_c, auto odd_c) {
    constexpr int RBW = decltype(rbw_c)::value;
    constexpr bool ODD = decltype(odd_c)::value;
    const int want = (RBW == 2 ? 2 : 4) * device_cu_count();
    const int64_t groups = (N + 16 * RBW - 1) / (16 * RBW);
    int S = (int)std::min<int64_t>(8, std::max<int64_t>(1, (want + groups - 1) / groups));
    S = std::min(S, nkb);
    const int kbw = (nkb + S - 1) / S;
    S = (nkb + kbw - 1) / kbw;
    const size_t lds = (size_t)S * RBW * 64 * 16;
    launch_main(&qmv_mma_kernel<MODE, RBW, ODD>, dim3((unsigned)groups), dim3(64 * S), (uint32_t)lds, s,
                x, M, K, (int)N, w.codes, w.scales, w.biases, w.global_scale, g2, y, kbw);
    return hipGetLastError();
  };
  using one = std::integral_constant<int, 1>;
  using two = std::integral_constant<int, 2>;
  using odd = std::integral_constant<bool, true>;
  using even = std::integral_constant<bool, false>;
  const int64_t cus = device_cu_count();
  const int64_t rows1 = ((N + 15) / 16 + cus - 1) / cus * 16;   // busiest CU, RBW = 1
  const int64_t rows2 = ((N + 31) / 32 + cus - 1) / cus * 32;   // RBW = 2
  const bool rbw2 = N * K >= (int64_t(1) << 25) || rows2 <= rows1;
  // rows whose scale pairs are not aligned for one wider load: NVFP4 with
  // K % 32 == 16 (an odd number of scale bytes), affine with K % 128 == 64
  // (an odd number of groups)
  if constexpr (MODE == FMT_NVFP4 || MODE == FMT_AFF4_G64) {
    const bool odd_row = MODE == FMT_NVFP4 ? (K / 16) % 2 != 0 : (K / 64) % 2 != 0;
    if (odd_row) return rbw2 ? go(two{}, odd{}) : go(one{}, odd{});
  }
  return rbw2 ? go(two{}, even{}) : go(one{}, even{});
}

// When the GEMV runs on MFMA (qmv_mma_kernel), by measurement on the
// [25600, 5120], [5120, 25600], [5760, 2880] and [4096, 4096] shapes:
// - x too large for the one LDS copy of the kernels below (which then walk
//   K in slices): from 4 rows of x on, 1.1-3x faster;
// - x in LDS: from 4 rows on, for matrices under 2^26 weights (MXFP4
//   [5760, 2880] at M = 4: 6.7 against 8.8 us); on larger ones the LDS
//   kernels stream the weights faster up to the 64 KB limit of x (their
//   loads touch fewer cache lines per instruction than the MFMA operand
//   layout allows; [25600, 5120] at M = 2..6: 1.1-1.7x).
constexpr int kMmaMinRows = 4;
constexpr int64_t kMmaLargeWeights = int64_t(1) << 26;

template <int MODE, bool QX = false>
hipError_t by_m(const uint16_t* x, int M, const bsfp_qtensor& w, const float* g2, uint16_t* y,
                hipStream_t s, int qx_amax = 0) {
  const int K = (int)w.cols;
  const int NJ = (int)((w.cols / 32 + 31) / 32);
  const bool ragged = (w.cols / 32) % 32 != 0;
  if constexpr (!QX && (MODE == FMT_AFF4_G64 || MODE == FMT_MXFP4 || MODE == FMT_NVFP4)) {
    const bool x_lds = fast_ok<MODE>(M, NJ);
    const bool mma = x_lds ? (M >= kMmaMinRows && w.rows * w.cols < kMmaLargeWeights)
                           : M >= kMmaMinRows;
    if (mma && w.cols < (1 << 26) && w.rows < (1 << 30)) return launch_mma<MODE>(x, M, w, g2, y, s);
  }
  if (fast_ok<MODE>(M, NJ) && w.cols < (1 << 28) && w.rows < (1 << 30)) {
    if (M == 1) {
      // two rows per team once that still gives every CU 8 waves (measured
      // faster than four rows per team on the [25600, 5120] shape, where
      // both fill the CUs)
      const int64_t want = 8LL * device_cu_count();
      const int64_t N = w.rows;
      if (N >= 4 * want && slds_ok<MODE, 2>(K, NJ, M, N))
        return launch_fast<MODE, 1, 2, false, true, QX>(x, M, w, g2, y, NJ, s, qx_amax);
      if (slds_ok<MODE, 1>(K, NJ, M, N)) return launch_fast<MODE, 1, 1, false, true, QX>(x, M, w, g2, y, NJ, s, qx_amax);
      if (slds_ok<MODE, 2>(K, NJ, M, N)) return launch_fast<MODE, 1, 2, false, true, QX>(x, M, w, g2, y, NJ, s, qx_amax);
      if (slds_ok<MODE, 4>(K, NJ, M, N)) return launch_fast<MODE, 1, 4, false, true, QX>(x, M, w, g2, y, NJ, s, qx_amax);
      if (ragged) return launch_fast<MODE, 1, 1, true, false, QX>(x, M, w, g2, y, NJ, s, qx_amax);
      return launch_fast<MODE, 1, 1, false, false, QX>(x, M, w, g2, y, NJ, s, qx_amax);
    }
    if (ragged) {
      if (M == 2) return launch_fast<MODE, 2, 1, true, false, QX>(x, M, w, g2, y, NJ, s, qx_amax);
      if (M <= 4) return launch_fast<MODE, 4, 1, true, false, QX>(x, M, w, g2, y, NJ, s, qx_amax);
      return launch_fast<MODE, 8, 1, true, false, QX>(x, M, w, g2, y, NJ, s, qx_amax);
    }
    if (M == 2) return launch_fast<MODE, 2, 1, false, false, QX>(x, M, w, g2, y, NJ, s, qx_amax);
    if (M <= 4) return launch_fast<MODE, 4, 1, false, false, QX>(x, M, w, g2, y, NJ, s, qx_amax);
    return launch_fast<MODE, 8, 1, false, false, QX>(x, M, w, g2, y, NJ, s, qx_amax);
  }
  // x too large for one LDS copy: walk K in slices (plain x only; callers
  // check qmv_qx_fusable first)
  if constexpr (QX) return hipErrorInvalidValue;
  if (M == 1) return run<MODE, 1>(x, M, w, g2, y, s);
  if (M == 2) return run<MODE, 2>(x, M, w, g2, y, s);
  if (M <= 4) return run<MODE, 4>(x, M, w, g2, y, s);
  return run<MODE, 8>(x, M, w, g2, y, s);
}

// Several matrices that share x, K and the format, one row of x: one launch
// of the fast kernel with staged scales, chosen on their total rows as by_m
// chooses on one matrix's rows; when that kernel does not take them, one
// launch per matrix.
template <int MODE>
hipError_t by_m_batch(const uint16_t* x, const bsfp_qtensor* const* ws, uint16_t* const* ys,
                      int count, hipStream_t s) {
  const int K = (int)ws[0]->cols;
  const int NJ = (int)((K / 32 + 31) / 32);
  int64_t N = 0;
  for (int i = 0; i < count; ++i) N += ws[i]->rows;
  auto blocks = [&](int R) {
    int64_t nb = 0;
    for (int i = 0; i < count; ++i) nb += (ws[i]->rows + 2 * R - 1) / (2 * R);
    return nb;
  };
  // two slots for two matrices (the kernel arguments grow with the slots,
  // and a larger argument block measured slower per launch)
  auto go = [&](auto r_c, auto nm_c) {
    constexpr int R = decltype(r_c)::value, NM = decltype(nm_c)::value;
    return launch_fast_mats<MODE, 1, R, false, true, false, NM>(x, 1, ws, ys, count, nullptr,
                                                               NJ, s, 0);
  };
  using r1 = std::integral_constant<int, 1>;
  using r2 = std::integral_constant<int, 2>;
  using r4 = std::integral_constant<int, 4>;
  using nm2 = std::integral_constant<int, 2>;
  using nm4 = std::integral_constant<int, kQmvMats>;
  if (fast_ok<MODE>(1, NJ) && K < (1 << 28) && N < (1 << 30)) {
    const int64_t want = 8LL * device_cu_count();
    // four rows per team once every CU gets 16 or more blocks of 8 rows: the
    // gate+up pair of [25600, 5120] (51200 rows, 25 blocks per CU) measured
    // 29.1 against 30.2 us (interleaved A/B, two boxes); one such matrix
    // alone (12.5 blocks per CU) is faster with two rows per team
    if (N >= 16 * want && slds_ok<MODE, 4>(K, NJ, 1, N, blocks(4)))
      return count == 2 ? go(r4{}, nm2{}) : go(r4{}, nm4{});
    if (N >= 4 * want && slds_ok<MODE, 2>(K, NJ, 1, N, blocks(2)))
      return count == 2 ? go(r2{}, nm2{}) : go(r2{}, nm4{});
    if (slds_ok<MODE, 1>(K, NJ, 1, N, blocks(1)))
      return count == 2 ? go(r1{}, nm2{}) : go(r1{}, nm4{});
  }
  for (int i = 0; i < count; ++i) {
    const hipError_t e = by_m<MODE>(x, 1, *ws[i], nullptr, ys[i], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_qmv_batch(const uint16_t* x, int M, const bsfp_qtensor* const* ws,
                            uint16_t* const* ys, int count, hipStream_t s) {
  const bsfp_qtensor* w2[kQmvMats];
  uint16_t* y2[kQmvMats];
  int n = 0;
  for (int i = 0; i < count && i < kQmvMats; ++i) {
    if (ws[i]->rows == 0) continue;  // nothing to compute
    w2[n] = ws[i];
    y2[n] = ys[i];
    ++n;
  }
  if (n == 0) return hipGetLastError();
  if (M == 1 && n > 1 && w2[0]->cols % 32 == 0) {
    switch (format_id(w2[0]->mode, w2[0]->bits, w2[0]->group_size)) {
      case FMT_AFF4_G64: return by_m_batch<FMT_AFF4_G64>(x, w2, y2, n, s);
      case FMT_MXFP4: return by_m_batch<FMT_MXFP4>(x, w2, y2, n, s);
      case FMT_NVFP4: return by_m_batch<FMT_NVFP4>(x, w2, y2, n, s);
      default: break;
    }
  }
  for (int i = 0; i < n; ++i) {
    const hipError_t e = launch_qmv(x, M, *w2[i], y2[i], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

bool qmv_variant_supported(int M, const bsfp_qtensor& w) {
  if (w.cols % 32 != 0 || w.cols >= (1 << 28) || w.rows >= (1 << 30) || M < 1 || M > 8)
    return false;
  const int NJ = (int)((w.cols / 32 + 31) / 32);
  return fast_ok<FMT_MXFP8>(M, NJ) && fast_ok<FMT_AFF8_G64>(M, NJ);
}

bool qmv_qx_fusable(int M, const bsfp_qtensor& w) {
  if (w.cols % 32 != 0 || w.cols >= (1 << 28) || w.rows >= (1 << 30) || M < 1 || M > 8)
    return false;
  const int NJ = (int)((w.cols / 32 + 31) / 32);
  if (w.mode == BSFP_NVFP4) return fast_ok<BSFP_NVFP4>(M, NJ);
  if (w.mode == BSFP_MXFP4) return fast_ok<BSFP_MXFP4>(M, NJ);
  return false;
}

hipError_t launch_qmv_qx(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y,
                         hipStream_t s) {
  if (w.rows == 0) return hipGetLastError();
  if (w.mode == BSFP_NVFP4)
    return by_m<BSFP_NVFP4, true>(x, M, w, nullptr, y, s, w.global_scale ? 1 : 0);
  return by_m<BSFP_MXFP4, true>(x, M, w, nullptr, y, s, 0);
}

hipError_t launch_qmv(const uint16_t* x, int M, const bsfp_qtensor& w, uint16_t* y,
                      hipStream_t s, const float* g2) {
  if (w.rows == 0) return hipGetLastError();
  if (w.cols % 32 != 0) {  // only NVFP4 rows can have K % 32 == 16
    const dim3 grid((unsigned)((w.rows + 3) / 4));
    if (M == 1)
      launch_main(&qmv_nvfp4_words_kernel<1>, grid, dim3(kThreads), 0, s, x, M, w.cols,
                         w.rows, w.codes, (const uint8_t*)w.scales, w.global_scale, g2, y);
    else
      launch_main(&qmv_nvfp4_words_kernel<8>, grid, dim3(kThreads), 0, s, x, M, w.cols,
                         w.rows, w.codes, (const uint8_t*)w.scales, w.global_scale, g2, y);
    return hipGetLastError();
  }
  switch (format_id(w.mode, w.bits, w.group_size)) {
    case FMT_AFF4_G64: return by_m<FMT_AFF4_G64>(x, M, w, g2, y, s);
    case FMT_MXFP4: return by_m<FMT_MXFP4>(x, M, w, g2, y, s);
    case FMT_NVFP4: return by_m<FMT_NVFP4>(x, M, w, g2, y, s);
    case FMT_MXFP8: return by_m_variant<FMT_MXFP8>(x, M, w, y, s);
    case FMT_AFF4_G32: return by_m_variant<FMT_AFF4_G32>(x, M, w, y, s);
    case FMT_AFF4_G128: return by_m_variant<FMT_AFF4_G128>(x, M, w, y, s);
    case FMT_AFF8_G32: return by_m_variant<FMT_AFF8_G32>(x, M, w, y, s);
    case FMT_AFF8_G64: return by_m_variant<FMT_AFF8_G64>(x, M, w, y, s);
    case FMT_AFF8_G128: return by_m_variant<FMT_AFF8_G128>(x, M, w, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bsfp
