// qmm.hip -- prefill GEMM y[M, N] = x[M, K] . W[N, K]^T on MFMA for gfx950.
//
// gemm_dq_kernel -- 16-bit MFMA (v_mfma_f32_32x32x16_{bf16,f16}) with the
//   weights dequantized in registers.  Prefill tiles are 256 x 256 on 8 waves
//   (each 128 x 64); small M uses narrower M tiles.  Per K step of 64, the
//   16-bit A tile (bf16 x, or the fp16 dequantized NVFP4 activations of the
//   qq path), the packed weight codes and their scales all go from global
//   memory straight into LDS (buffer_load ... lds, issued as inline assembly
//   so that the compiler adds no conservative waits of its own), three
//   stages deep: the loads of step s + 2 are in flight while step s runs,
//   and one explicit vmcnt per step waits for exactly the previous ones.  A
//   tiles are XOR-swizzled in LDS so ds_read_b128 is conflict-free.  Each
//   lane reads the 16-byte code chunk (32 k-values) of its weight row from
//   LDS and expands it right before the MFMA.  The contraction order inside
//   a 64-wide K step is permuted consistently for both operands: at MFMA
//   step kk, lane half h covers k = 32h + 8kk .. 32h + 8kk + 7, so that each
//   lane reads whole code words.
//     NVFP4 qq (fp16): E2M1 * E4M3 is exact in fp16, so the weight expands
//       with one v_cvt_scalef32_pk_f16_fp4 and one v_pk_mul_f16 per pair.
//     NVFP4 weight-only (bf16): E2M1 -> fp32 pair, times the block scale,
//       packed to bf16 (exact).
//     MXFP4 weight-only (bf16): v_cvt_scalef32_pk_bf16_fp4 with the E8M0
//       block scale as the converter's exponent scale (exact).
//     affine weight-only (bf16): s * q + b rounded once to bf16 (the
//       "dequantize to bf16, then a bf16 GEMM" numerics of "mlx: opt-in dense
//       GEMM for nvfp4 prefill"); q comes from the exact fp8-byte decode.
//   The per-tensor scale (g_w, or alpha = g_x * g_w for qq) is applied in the
//   epilogue ("mlx 0.30.7.3 -> 0.30.7.6", qqmm_utils.cu: alpha =
//   amax_x * amax_w / (448*6)^2, read on the device).  When 256 x 256 tiles
//   would leave a small last round on the CUs, the output columns of that
//   round go to a second launch with 128 x 64 tiles.
//
// gemm_mxl_kernel -- MXFP4 x MXFP4 on the CDNA4 block-scaled MFMA
//   v_mfma_scale_f32_32x32x64_f8f6f4: both operands stay 4-bit, and each
//   lane hands the MFMA the E8M0 scale of the 32 k-values it holds, which is
//   exactly one MXFP4 group.  No dequantization at all.  Operand rows are
//   staged through LDS in 256-K units with coalesced buffer-to-LDS copies.
//
// fp32 accumulation, bf16 round-to-nearest-even output, rows and columns
// beyond M / N clamped on load and masked on store.
#include <algorithm>
#include <atomic>

#include "bsfp_device.hpp"
#include "bsfp_internal.hpp"

namespace bsfp {

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

enum { DEC_AFFINE = 0, DEC_MXFP4 = 1, DEC_NVFP4 = 2, DEC_NVFP4_F16 = 3, DEC_DENSE = 4 };

// Expanded B operand of one MFMA (8 consecutive k of one weight row).
struct Op8 {
  uint32_t v[4];
};

// Per-lane per-K-step weight data of one 32-column subtile.
struct BFrag {
  uint4 codes;   // 32 codes: k = k0 + 32h + 0..31
  uint32_t s0;   // scale bits (mode specific)
  uint32_t s1;   // affine bias bits
};

template <int DEC>
__device__ __forceinline__ void load_bfrag(BFrag& f, const uint32_t* __restrict__ codes,
                                           const void* __restrict__ scales,
                                           const uint16_t* __restrict__ biases, int64_t n,
                                           int K, int k0, int h) {
  f.codes = *reinterpret_cast<const uint4*>(codes + n * (K / 8) + (k0 / 8) + 4 * h);
  if constexpr (DEC == DEC_AFFINE) {
    const int64_t gi = n * (K / 64) + k0 / 64;
    f.s0 = reinterpret_cast<const uint16_t*>(scales)[gi];
    f.s1 = biases[gi];
  } else if constexpr (DEC == DEC_MXFP4) {
    f.s0 = reinterpret_cast<const uint8_t*>(scales)[n * (K / 32) + k0 / 32 + h];
  } else {  // two E4M3 bytes: blocks 2h and 2h + 1 of this 64-wide step
    f.s0 = reinterpret_cast<const uint16_t*>(scales)[n * (K / 32) + k0 / 32 + h];
  }
}

// Expand word kk of the fragment (k = 32h + 8kk + 0..7).
template <int DEC>
__device__ __forceinline__ Op8 expand(const BFrag& f, int kk) {
  const uint32_t w = kk == 0 ? f.codes.x : kk == 1 ? f.codes.y : kk == 2 ? f.codes.z : f.codes.w;
  Op8 o;
  if constexpr (DEC == DEC_NVFP4_F16) {
    // both E4M3 block scales -> fp16 with the hardware converter (exact)
    const f16x2_t sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s0, 1.0f, false);
    const _Float16 sh = (kk < 2) ? sp.x : sp.y;
    const f16x2_t s2 = {sh, sh};
    o.v[0] = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<0>(w) * s2);
    o.v[1] = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<1>(w) * s2);
    o.v[2] = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<2>(w) * s2);
    o.v[3] = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<3>(w) * s2);
  } else if constexpr (DEC == DEC_NVFP4) {
    const f32x2_t sp = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(f.s0, 1.0f, false);
    const float sc = (kk < 2) ? sp.x : sp.y;
    f32x2_t p0 = e2m1x2_to_f32x2<0>(w), p1 = e2m1x2_to_f32x2<1>(w);
    f32x2_t p2 = e2m1x2_to_f32x2<2>(w), p3 = e2m1x2_to_f32x2<3>(w);
    o.v[0] = pack_bf16x2(p0.x * sc, p0.y * sc);
    o.v[1] = pack_bf16x2(p1.x * sc, p1.y * sc);
    o.v[2] = pack_bf16x2(p2.x * sc, p2.y * sc);
    o.v[3] = pack_bf16x2(p3.x * sc, p3.y * sc);
  } else if constexpr (DEC == DEC_MXFP4) {
    const float sc = __uint_as_float(f.s0 << 23);  // the converter reads its exponent only
    o.v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    o.v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    o.v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    o.v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  } else {  // affine: s * q + b, one rounding to bf16
    const float s = __uint_as_float(f.s0 << 16), b = __uint_as_float(f.s1 << 16);
    const uint32_t t = w & 0x0F0F0F0Fu, u = (w >> 4) & 0x0F0F0F0Fu;
    // t holds q0, q2, q4, q6 in its bytes; u holds q1, q3, q5, q7
    const f32x2_t a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(t, 512.0f, false);  // q0, q2
    const f32x2_t a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(t, 512.0f, true);   // q4, q6
    const f32x2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u, 512.0f, false);  // q1, q3
    const f32x2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u, 512.0f, true);   // q5, q7
    o.v[0] = pack_bf16x2(__builtin_fmaf(s, a0.x, b), __builtin_fmaf(s, b0.x, b));
    o.v[1] = pack_bf16x2(__builtin_fmaf(s, a0.y, b), __builtin_fmaf(s, b0.y, b));
    o.v[2] = pack_bf16x2(__builtin_fmaf(s, a1.x, b), __builtin_fmaf(s, b1.x, b));
    o.v[3] = pack_bf16x2(__builtin_fmaf(s, a1.y, b), __builtin_fmaf(s, b1.y, b));
  }
  return o;
}

template <int DEC>
__device__ __forceinline__ f32x16_t mfma16(const uint4& a, const Op8& b, const f32x16_t& c) {
  const uint4 bv = {b.v[0], b.v[1], b.v[2], b.v[3]};
  if constexpr (DEC == DEC_NVFP4_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, bv), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, bv), c, 0, 0, 0);
  }
}

// XCD-aware tile order.  Workgroup b runs on XCD b % 8, so XCD x gets the
// count_x = ceil((T - x) / 8) workgroups b = x, x + 8, ...; they are given
// one contiguous range of logical tiles, [start_x, start_x + count_x), so
// tiles that share operands share that XCD's L2.  m_major: consecutive
// logical tiles share an activation row block (the weight column blocks
// stream past it); otherwise they share a weight column block across the M
// tiles, in groups of 4 M tiles when the M tiles come in multiples of 4: an
// XCD's 32 concurrent tiles are then 4 row blocks x 8 column blocks instead
// of 8 x 4, and it streams half the activation rows (at M = 2048 the qq GEMM
// fetches 30 % fewer bytes at the same speed, the dense GEMM runs 3 %
// faster; at M = 1134, 5 row blocks, the ungrouped order was faster).
// m_major = 1 from 16 row blocks up (the 16-bit GEMM at M = 4096 read 3 %
// faster that way; at M = 1134 the weight-column order was faster).
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int m_major, int& tm,
                                        int& tn) {
  const int b = blockIdx.x, T = tiles_m * tiles_n;
  const int x = b & 7, q = T >> 3, r = T & 7;
  const int L = x * q + min(x, r) + (b >> 3);
  if (m_major) {
    tm = L / tiles_n;
    tn = L % tiles_n;
  } else if (tiles_m % 4 == 0) {
    const int grp = L / (4 * tiles_n), within = L - grp * 4 * tiles_n;
    tm = grp * 4 + (within & 3);
    tn = within >> 2;
  } else {
    tm = L % tiles_m;
    tn = L / tiles_m;
  }
}

// Physical 16-byte chunk of logical chunk c in tile row r.  The XOR with r & 7
// spreads 8 consecutive rows over the 8 chunks of a 128-byte row; the extra
// bit for rows 8..15 moves them to the other half of the 256-byte bank space,
// so the 16 rows one ds_read_b128 pass touches hit 16 different bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// Per-lane weight data of one 32-column subtile, loaded through buffer
// descriptors based at the tile's first weight row.
template <int DEC>
__device__ __forceinline__ void load_bfrag_buf(BFrag& f, const rsrc_t& rc, const rsrc_t& rs,
                                               const rsrc_t& rb, int nl, int K, int k0, int h) {
  const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rc, nl * (K / 2) + 16 * h, k0 / 2, 0);
  f.codes = make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
  if constexpr (DEC == DEC_AFFINE) {
    f.s0 = __builtin_amdgcn_raw_buffer_load_b16(rs, nl * (K / 64) * 2, k0 / 32, 0);
    f.s1 = __builtin_amdgcn_raw_buffer_load_b16(rb, nl * (K / 64) * 2, k0 / 32, 0);
  } else if constexpr (DEC == DEC_MXFP4) {
    f.s0 = __builtin_amdgcn_raw_buffer_load_b8(rs, nl * (K / 32) + h, k0 / 32, 0);
  } else {  // two E4M3 bytes: blocks 2h and 2h + 1 of this 64-wide step
    f.s0 = __builtin_amdgcn_raw_buffer_load_b16(rs, nl * (K / 16) + 2 * h, k0 / 16, 0);
  }
}

// WGM x WGN waves per workgroup, each owning WMT x WNT MFMA tiles of 32 x 32.
// PP: the ping-pong schedule described at the K loop (8 waves, WGM = 2).
// NS: LDS stages (3; 2 for the dense 256 x 256 tile, whose stage is 64 KB).
template <int DEC, int WGM, int WGN, int WMT, int WNT, bool PP = false, int NS = 3>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_dq_kernel(
    const uint16_t* __restrict__ A, const uint32_t* __restrict__ codes,
    const void* __restrict__ scales, const uint16_t* __restrict__ biases,
    const float* __restrict__ g1, const float* __restrict__ g2, int M, int N, int K,
    uint16_t* __restrict__ Y, int ldy, int tiles_m, int tiles_n) {
  constexpr int NW = WGM * WGN;
  constexpr int BM = 32 * WMT * WGM, BN = 32 * WNT * WGN;
  constexpr int WROWS = BM / NW;  // A rows each wave brings into LDS per K step
  static_assert(WROWS % 8 == 0, "each wave loads whole 8-row LDS blocks");
  // Three LDS stages, each [A tile | B codes | B scales | B biases]; K steps
  // rotate through them and the loads of step s + 2 go out while step s is
  // computed.  Every global load of the loop goes straight to LDS through
  // buffer_load_lds16/4, which the compiler does not track: the only wait
  // for them is the explicit vmcnt before each step's barrier, so two steps
  // of loads stay in flight.  Every wave issues the same number of loads per
  // step, which makes that count exact for each wave.
  // DEC_DENSE: B is a plain bf16 [N, K] matrix, staged like A ([BN][8]
  // swizzled chunks), with no scales.
  constexpr bool DENSE = DEC == DEC_DENSE;
  constexpr int A_U4 = BM * 8;          // [BM][8] 16-byte chunks, swizzled
  constexpr int BC_U4 = DENSE ? BN * 8 : BN * 2;  // [BN][2] 16-byte code chunks
  constexpr int BS_U4 = DENSE ? 0 : BN / 4;       // [BN] scale dwords
  constexpr int BB_U4 = (DEC == DEC_AFFINE) ? BN / 4 : 0;  // [BN] bias dwords
  constexpr int STAGE_U4 = A_U4 + BC_U4 + BS_U4 + BB_U4;
  static_assert(NS == 2 || NS == 3, "two or three LDS stages");
  static_assert(!PP || NS == 3, "the ping-pong schedule keeps two steps of loads in flight");
  __shared__ uint4 smem[NS * STAGE_U4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int h = lane >> 5, l32 = lane & 31;
  int tm, tn;
  tile_of(tiles_m, tiles_n, tiles_m >= 16, tm, tn);
  const int m_base = tm * BM, n_base = tn * BN;
  const int rows_m = min(BM, M - m_base), rows_n = min(BN, N - n_base);

  // A: an instruction fills 8 consecutive tile rows (lane i -> row i / 8,
  // physical chunk i % 8), so the swizzle is applied to the source offsets.
  const rsrc_t ra = make_rsrc(A + (int64_t)m_base * K, (int64_t)rows_m * K * 2);
  int a_off[WROWS / 8];
#pragma unroll
  for (int s = 0; s < WROWS / 8; ++s) {
    const int r = wave * WROWS + s * 8 + (lane >> 3);
    a_off[s] = r * K * 2 + swz(r, lane & 7) * 16;
  }

  // B codes: LDS slot p of the tile's step holds row r = p / 2, half
  // (p % 2) ^ ((r >> 3) & 1): rows 8..15 of every 16 swap their halves, so
  // the 16 lanes of a phase of ds_read_b128 (16 consecutive rows, one half)
  // fall on distinct banks (with the plain order rows r and r + 8 shared
  // them: a 2-way conflict on every B read, 0.4 conflict cycles per LDS
  // instruction of the qq main loop).  Each wave loads PPW consecutive
  // slots.  Dense B: BROWS rows per wave, like A.
  constexpr int PPW = 2 * BN / NW;
  constexpr int BC_LOADS = (PPW + 63) / 64;
  static_assert(DENSE || (PPW * NW == 2 * BN && (PPW >= 64 ? PPW % 64 == 0 : 64 % PPW == 0)),
                "code pieces split evenly over the waves");
  constexpr int BROWS = BN / NW;
  static_assert(!DENSE || BROWS % 8 == 0, "each wave loads whole 8-row LDS blocks of B");
  const rsrc_t rc = DENSE ? make_rsrc(reinterpret_cast<const uint16_t*>(codes) + (int64_t)n_base * K,
                                      (int64_t)rows_n * K * 2)
                          : make_rsrc(codes + (int64_t)n_base * (K / 8), (int64_t)rows_n * (K / 2));
  int b_off[DENSE ? BROWS / 8 : 1];
  if constexpr (DENSE) {
#pragma unroll
    for (int s = 0; s < BROWS / 8; ++s) {
      const int r = wave * BROWS + s * 8 + (lane >> 3);
      b_off[s] = r * K * 2 + swz(r, lane & 7) * 16;
    }
  }
  // B scales (and affine biases): one dword per tile row and step, read by
  // BN / NW lanes of each wave.  NVFP4 needs 4 bytes per row and step (four
  // E4M3 blocks of 16); MXFP4 and affine need 2, taken from the aligned dword
  // that holds them.
  constexpr int gsz = (DEC == DEC_AFFINE) ? 64 : (DEC == DEC_MXFP4) ? 32 : 16;
  constexpr int sbytes = (DEC == DEC_AFFINE) ? 2 : 1;
  constexpr int SROWS = BN / NW;  // scale rows per wave
  static_assert(SROWS <= 64, "one scale load per wave and array");
  const int srb = (K / gsz) * sbytes;  // scale bytes per weight row
  const rsrc_t rs = DENSE ? make_rsrc(nullptr, 0)
                          : make_rsrc(reinterpret_cast<const uint8_t*>(scales) + (int64_t)n_base * srb,
                                      (int64_t)rows_n * srb);
  const rsrc_t rb = make_rsrc(biases ? biases + (int64_t)n_base * (K / 64) : nullptr,
                              biases ? (int64_t)rows_n * srb : 0);
  const int srow = wave * SROWS + lane;  // the tile row whose scales this lane loads

  auto stage = [&](int i) { return smem + i * STAGE_U4; };
  auto load_step = [&](int st, uint4* sb) {
    const int k0 = st * 64;
#pragma unroll
    for (int s = 0; s < WROWS / 8; ++s)
      buffer_load_lds16(ra, sb + (wave * WROWS + s * 8) * 8, a_off[s], k0 * 2);
    uint4* bc = sb + A_U4;
    if constexpr (DENSE) {
#pragma unroll
      for (int s = 0; s < BROWS / 8; ++s)
        buffer_load_lds16(rc, bc + (wave * BROWS + s * 8) * 8, b_off[s], k0 * 2);
      return;
    }
#pragma unroll
    for (int c = 0; c < BC_LOADS; ++c) {
      const int p0 = wave * PPW + c * 64;
      const int p = p0 + lane;
      const int r = p >> 1;
      if (PPW >= 64 || lane < PPW)
        buffer_load_lds16(rc, bc + p0, r * (K / 2) + ((p & 1) ^ ((r >> 3) & 1)) * 16, k0 / 2);
    }
    if (lane < SROWS) {
      const int so = (DEC == DEC_NVFP4 || DEC == DEC_NVFP4_F16) ? srow * srb + 4 * st
                                                                 : (srow * srb + 2 * st) & ~3;
      buffer_load_lds4(rs, sb + A_U4 + BC_U4 + wave * SROWS / 4, so, 0);
      if constexpr (DEC == DEC_AFFINE)
        buffer_load_lds4(rb, sb + A_U4 + BC_U4 + BS_U4 + wave * SROWS / 4, so, 0);
    }
  };
  // vector-memory loads one step issues per wave
  constexpr int kStepLoads =
      WROWS / 8 + (DENSE ? BROWS / 8 : BC_LOADS + ((DEC == DEC_AFFINE) ? 2 : 1));

  // this lane's weight rows within the tile
  int nl[WNT];
#pragma unroll
  for (int j = 0; j < WNT; ++j) nl[j] = wn * 32 * WNT + 32 * j + l32;
  auto read_b = [&](const uint4* sb, int st, BFrag (&dst)[WNT]) {
    const uint4* bc = sb + A_U4;
    const uint8_t* bs = reinterpret_cast<const uint8_t*>(sb + A_U4 + BC_U4);
#pragma unroll
    for (int j = 0; j < WNT; ++j) {
      dst[j].codes = bc[nl[j] * 2 + (h ^ ((nl[j] >> 3) & 1))];
      if constexpr (DEC == DEC_NVFP4 || DEC == DEC_NVFP4_F16) {
        // two E4M3 bytes: blocks 2h and 2h + 1 of this 64-wide step
        dst[j].s0 = *reinterpret_cast<const uint16_t*>(bs + nl[j] * 4 + 2 * h);
      } else {
        const int hw = ((nl[j] + n_base) * srb + 2 * st) & 2;  // byte offset in the dword
        if constexpr (DEC == DEC_MXFP4) {
          dst[j].s0 = bs[nl[j] * 4 + hw + h];
        } else {
          dst[j].s0 = *reinterpret_cast<const uint16_t*>(bs + nl[j] * 4 + hw);
          dst[j].s1 = *reinterpret_cast<const uint16_t*>(bs + BS_U4 * 16 + nl[j] * 4 + hw);
        }
      }
    }
  };

  f32x16_t acc[WMT][WNT];
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // One K step: wait for this step's loads (those of the next step stay in
  // flight), make every wave's loads visible, read the first operands, issue
  // the loads of the step after next into the stage the previous step used,
  // then run the MFMAs.
  // Past the last step the loads repeat the last step into a stage nobody
  // reads, so every step has the same loads in flight.
  const int nsteps = K / 64;
  auto step = [&](int st, int si, int pi) {
    wait_vmem_le<(NS - 2) * kStepLoads>();  // this step's loads have landed
    __syncthreads();
    const uint4* cur = stage(si);
    BFrag b[WNT];
    if constexpr (!DENSE) read_b(cur, st, b);
    // A fragments of sub-step kk + 1 are read while kk's MFMAs run
    auto read_a = [&](int kk, uint4 (&a)[WMT]) {
#pragma unroll
      for (int i = 0; i < WMT; ++i) {
        const int r = wm * 32 * WMT + 32 * i + l32;
        a[i] = cur[r * 8 + swz(r, 4 * h + kk)];
      }
    };
    auto mma = [&](int kk, const uint4 (&a)[WMT]) {
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        Op8 bo;
        if constexpr (DENSE) {
          const uint4 v = cur[A_U4 + nl[j] * 8 + swz(nl[j], 4 * h + kk)];
          bo.v[0] = v.x, bo.v[1] = v.y, bo.v[2] = v.z, bo.v[3] = v.w;
        } else {
          bo = expand<DEC>(b[j], kk);
        }
#pragma unroll
        for (int i = 0; i < WMT; ++i) acc[i][j] = mfma16<DEC>(a[i], bo, acc[i][j]);
      }
    };
    uint4 a0[WMT], a1[WMT];
    read_a(0, a0);
    read_a(1, a1);
    // the step's first LDS reads go out before the loads of step st + NS - 1,
    // so their latency overlaps the load issue
    load_step(min(st + NS - 1, nsteps - 1), stage(pi));
    mma(0, a0);
    read_a(2, a0);
    mma(1, a1);
    read_a(3, a1);
    mma(2, a0);
    mma(3, a1);
  };

  if constexpr (PP) {
    // Ping-pong.  The two waves that share a SIMD (w and w + 4: waves are
    // dealt to the 4 SIMDs round-robin) belong to different groups, g = w / 4
    // (= wm), and group 1 runs one phase behind group 0.  Each K step is four
    // phases separated by workgroup barriers: M (read the A fragments of two
    // sub-steps from LDS and expand the matching weight words in registers;
    // the first M of a step also reads the step's codes and scales and issues
    // the loads of the step after next) and C (the 16 MFMAs of those two
    // sub-steps), twice.  Between two barriers one wave of every SIMD issues
    // MFMAs while the other waits on LDS and runs the expansion, so the MFMA
    // pipe is not left idle while both waves of a SIMD sit in the same
    // read-and-expand phase.  Data hazards: step s + 1's loads are waited for
    // (vmcnt) at the end of every wave's second M of step s, before the
    // barrier that precedes group 0's first read of step s + 1; the loads of
    // step s + 2 overwrite the stage of step s - 1, whose last reads (group
    // 1's second M of step s - 1) end before that barrier.
    static_assert(NW == 8 && WGM == 2 && !DENSE, "ping-pong needs 8 waves in two rows");
    auto bar = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto pp_step = [&](int st, int si, int pi) {
      const uint4* cur = stage(si);
      BFrag b[WNT];
      uint4 a0[WMT], a1[WMT];
      Op8 e0[WNT], e1[WNT];
      auto read_a = [&](int kk, uint4 (&a)[WMT]) {
#pragma unroll
        for (int i = 0; i < WMT; ++i) {
          const int r = wm * 32 * WMT + 32 * i + l32;
          a[i] = cur[r * 8 + swz(r, 4 * h + kk)];
        }
      };
      auto expand_kk = [&](int kk, Op8 (&e)[WNT]) {
#pragma unroll
        for (int j = 0; j < WNT; ++j) e[j] = expand<DEC>(b[j], kk);
      };
      auto mma = [&](const uint4 (&a)[WMT], const Op8 (&e)[WNT]) {
#pragma unroll
        for (int j = 0; j < WNT; ++j)
#pragma unroll
          for (int i = 0; i < WMT; ++i) acc[i][j] = mfma16<DEC>(a[i], e[j], acc[i][j]);
      };
      read_b(cur, st, b);  // M: sub-steps 0 and 1
      read_a(0, a0);
      read_a(1, a1);
      load_step(min(st + 2, nsteps - 1), stage(pi));
      expand_kk(0, e0);
      expand_kk(1, e1);
      bar();
      mma(a0, e0);  // C
      mma(a1, e1);
      bar();
      read_a(2, a0);  // M: sub-steps 2 and 3
      read_a(3, a1);
      expand_kk(2, e0);
      expand_kk(3, e1);
      wait_vmem_le<kStepLoads>();  // step st + 1 has landed
      bar();
      mma(a0, e0);  // C
      mma(a1, e1);
      bar();
    };
    load_step(0, stage(0));
    load_step(min(1, nsteps - 1), stage(1));
    wait_vmem_le<kStepLoads>();
    bar();
    if (wm == 1) bar();  // group 1 starts one phase behind
    int st = 0;
    for (; st + 3 <= nsteps; st += 3) {
      pp_step(st, 0, 2);
      pp_step(st + 1, 1, 0);
      pp_step(st + 2, 2, 1);
    }
    if (st < nsteps) pp_step(st, 0, 2);
    if (st + 1 < nsteps) pp_step(st + 1, 1, 0);
    if (wm == 0) bar();  // the same number of barriers in both groups
    wait_vmem();  // the surplus loads land before the LDS is released
  } else if constexpr (NS == 3) {
    load_step(0, stage(0));
    load_step(min(1, nsteps - 1), stage(1));
    int st = 0;
    for (; st + 3 <= nsteps; st += 3) {
      step(st, 0, 2);
      step(st + 1, 1, 0);
      step(st + 2, 2, 1);
    }
    if (st < nsteps) step(st, 0, 2);
    if (st + 1 < nsteps) step(st + 1, 1, 0);
    wait_vmem();  // the surplus loads land before the LDS is released
  } else {
    // two stages: the loads of step st + 1 go out right after the barrier of
    // step st, into the stage step st - 1 used
    load_step(0, stage(0));
    int st = 0;
    for (; st + 2 <= nsteps; st += 2) {
      step(st, 0, 1);
      step(st + 1, 1, 0);
    }
    if (st < nsteps) step(st, 0, 1);
    wait_vmem();  // the surplus loads land before the LDS is released
  }

  const float sc = (g1 ? *g1 : 1.0f) * (g2 ? *g2 : 1.0f);
  const bool full = (rows_m == BM) && (rows_n == BN);
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNT; ++j) {
      const int n = n_base + wn * 32 * WNT + 32 * j + l32;
      const int m0 = m_base + wm * 32 * WMT + 32 * i + 4 * h;
      uint16_t* yp = Y + (int64_t)m0 * ldy + n;
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          yp[(int64_t)(8 * (r >> 2) + (r & 3)) * ldy] = (uint16_t)f32_to_bf16(acc[i][j][r] * sc);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 8 * (r >> 2) + (r & 3);
          if (m < M && n < N)
            yp[(int64_t)(8 * (r >> 2) + (r & 3)) * ldy] = (uint16_t)f32_to_bf16(acc[i][j][r] * sc);
        }
      }
    }
}

template <int DEC, int WGM, int WGN, int WMT, int WNT, bool PP = false, int NS = 3>
void launch_dq(const uint16_t* A, int M, const bsfp_qtensor& w, int64_t n0, int n,
               const float* g1, const float* g2, uint16_t* y, hipStream_t s, hipEvent_t ev0,
               hipEvent_t ev1) {
  constexpr int BM = 32 * WMT * WGM, BN = 32 * WNT * WGN;
  const int N = (int)w.rows, K = (int)w.cols;
  const int gsz = (DEC == DEC_AFFINE) ? 64 : (DEC == DEC_MXFP4) ? 32 : 16;
  const int sbytes = (DEC == DEC_AFFINE) ? 2 : 1;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (n + BN - 1) / BN;
  const uint32_t* codes = w.codes + n0 * (K / 8);
  const void* scales = reinterpret_cast<const uint8_t*>(w.scales) + n0 * (K / gsz) * sbytes;
  const uint16_t* biases = w.biases ? w.biases + n0 * (K / 64) : nullptr;
  auto kern = &gemm_dq_kernel<DEC, WGM, WGN, WMT, WNT, PP, NS>;
  const dim3 grid(tiles_m * tiles_n), block(64 * WGM * WGN);
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(kern, grid, block, 0u, s, ev0, ev1, 0u, A, codes, scales, biases, g1,
                          g2, M, n, K, y + n0, N, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(kern, grid, block, 0, s, A, codes, scales, biases, g1, g2, M, n, K,
                       y + n0, N, tiles_m, tiles_n);
}

template <int DEC, int WGM, int WGN, int WMT, int WNT>
hipError_t run_dq(const uint16_t* A, int M, const bsfp_qtensor& w, const float* g1,
                  const float* g2, uint16_t* y, hipStream_t s) {
  const LaunchEvents ev = take_launch_events();
  launch_dq<DEC, WGM, WGN, WMT, WNT>(A, M, w, 0, (int)w.rows, g1, g2, y, s, ev.start, ev.stop);
  return hipGetLastError();
}

// The dense GEMM on columns [n0, n0 + n) of B (bf16 [N, K]) and y.
template <int WGM, int WGN, int WMT, int WNT, bool PP, int NS>
void launch_dense(const uint16_t* A, int M, const uint16_t* B, int N, int K, int n0, int n,
                  uint16_t* y, hipStream_t s) {
  constexpr int BM = 32 * WMT * WGM, BN = 32 * WNT * WGN;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
  launch_main(&gemm_dq_kernel<DEC_DENSE, WGM, WGN, WMT, WNT, PP, NS>, dim3(tiles_m * tiles_n),
              dim3(64 * WGM * WGN), 0u, s, A,
              reinterpret_cast<const uint32_t*>(B + (int64_t)n0 * K), (const void*)nullptr,
              (const uint16_t*)nullptr, (const float*)nullptr, (const float*)nullptr, M, n, K,
              y + n0, N, tiles_m, tiles_n);
}

// Dense bf16 GEMM y[M, N] = x . B^T on the same kernel (B bf16 [N, K]):
// 256 x 256 tiles on 8 waves (128 x 64 per wave) with two 64 KB LDS stages
// from kDenseBigRows rows of x up, else 256 x 128 tiles (128 x 32 per wave)
// with three 48 KB stages.  As for the quantized GEMM, when the tiles fill
// the CUs for some whole rounds plus a small last round, the columns of the
// whole rounds run on the big tiles and the rest as 128 x 64 tiles spread
// over all CUs.  Whole dense call on W[25600, 5120] (interleaved A/B, us):
// the column split took M = 2048 from 602 to 569 and M = 4096 from 1049 to
// 989; with it, the 256 x 256 tile beats 256 x 128 at every M measured from
// 768 up (M = 768: 275 / 292, 1134: 358 / 394, 2048: 543 / 586, 2560: 628 /
// 746).
constexpr int kDenseBigRows = 768;

hipError_t run_dense(const uint16_t* A, int M, const uint16_t* B, int N, int K, uint16_t* y,
                     hipStream_t s) {
  const bool big = M >= kDenseBigRows;
  const int BN = big ? 256 : 128;
  const int cus = device_cu_count();
  const int tiles_m = (M + 255) / 256, tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  const int64_t rounds = tiles / cus;
  const int64_t rest = tiles - rounds * cus;
  int n_main = (int)std::min<int64_t>(tiles_n, rounds * cus / tiles_m) * BN;
  if (rounds == 0 || rest * 2 > cus || n_main <= 0 || n_main >= N) n_main = N;
  if (big)
    launch_dense<2, 4, 4, 2, false, 2>(A, M, B, N, K, 0, n_main, y, s);
  else
    launch_dense<2, 4, 4, 1, false, 3>(A, M, B, N, K, 0, n_main, y, s);
  if (n_main < N) launch_dense<2, 2, 2, 1, false, 3>(A, M, B, N, K, n_main, N - n_main, y, s);
  return hipGetLastError();
}

// Big tiles (256 x 256, 8 waves) for prefill row counts.  When the tiles
// fill the CUs for some whole rounds plus a small last round (800 tiles on
// 256 CUs: 3 rounds and an eighth), most CUs would idle through that last
// round; instead the weight rows of the whole rounds run with big tiles and
// the remaining rows in a second launch of 128 x 64 tiles, which spreads
// them over all CUs.
// The 256 x 256 prefill tiles run the ping-pong schedule.
constexpr bool kPingPong = true;

template <int DEC>
hipError_t run_dq_big(const uint16_t* A, int M, const bsfp_qtensor& w, const float* g1,
                      const float* g2, uint16_t* y, hipStream_t s) {
  const int N = (int)w.rows;
  const int cus = device_cu_count();
  const int tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  const int64_t rounds = tiles / cus;
  const int64_t rest = tiles - rounds * cus;
  const int n_main = (int)std::min<int64_t>(tiles_n, rounds * cus / tiles_m) * 256;
  const LaunchEvents ev = take_launch_events();
  if (rounds == 0 || rest * 2 > cus || n_main <= 0 || n_main >= N) {
    launch_dq<DEC, 2, 4, 4, 2, kPingPong>(A, M, w, 0, N, g1, g2, y, s, ev.start, ev.stop);
    return hipGetLastError();
  }
  launch_dq<DEC, 2, 4, 4, 2, kPingPong>(A, M, w, 0, n_main, g1, g2, y, s, ev.start, nullptr);
  launch_dq<DEC, 2, 2, 2, 1>(A, M, w, n_main, N - n_main, g1, g2, y, s, nullptr, ev.stop);
  return hipGetLastError();
}

// Tile shapes by the rows of x: 256 x 256 with 8 waves (each 128 x 64, the
// ping-pong schedule) from 257 rows; below, tiles 128 columns wide, so that
// a [25600, K] weight gives 200 workgroups rather than 100 for 256 CUs:
// 64 x 128 up to 64 rows, 128 x 128 up to 128, 256 x 128 up to 256.  By
// interleaved A/B on W[25600, 5120] (us, 256-wide tiles before): qq M = 64
// 53.6 -> 42.0, M = 128 68.9 -> 49.0, M = 256 103.2 -> 76.0; weight-only
// NVFP4 M = 128 68.4 -> 47.8, affine 83.3 -> 56.3.  At M = 320..512 the
// 256 x 256 tiles stay ahead (qq M = 512: 115.5 against 142.9 on 256 x 128).
template <int DEC>
hipError_t run_dq_m(const uint16_t* A, int M, const bsfp_qtensor& w, const float* g1,
                    const float* g2, uint16_t* y, hipStream_t s) {
  if (M <= 64) return run_dq<DEC, 1, 4, 2, 1>(A, M, w, g1, g2, y, s);
  if (M <= 128) return run_dq<DEC, 2, 4, 2, 1>(A, M, w, g1, g2, y, s);
  if (M <= 256) return run_dq<DEC, 2, 4, 4, 1>(A, M, w, g1, g2, y, s);
  return run_dq_big<DEC>(A, M, w, g1, g2, y, s);
}

// MXFP4 x MXFP4 staged through LDS.  A workgroup of WM x WN x KS waves owns
// a BM x BN output tile (BM = 32 WMT WM, BN = 32 WNT WN); each of its KS
// k-groups walks its own share of the 256-K units and the partial tiles are
// summed through LDS at the end in a fixed order.
//
// A stage holds one unit of the group's BM + BN operand rows: 128 code bytes
// and 8 scale bytes per row.  Every stage load is a 1 KB buffer-to-LDS copy of
// 8 whole rows (16 bytes per lane) or a 256-byte copy of 32 rows' scales, so
// global reads are contiguous 128-byte row segments; the MFMA layout (lane
// = row, one 16-byte block pair per lane) is then read from LDS.  The 16-byte
// slot of piece p in row r is p ^ ((r >> 1) & 7), which keeps every 16 lanes
// of a ds_read_b128 on distinct banks.  Same unit K order as the register
// kernel above: half h takes pieces 4h .. 4h+3, op_sel picks the scale byte.
// The last, partial unit loads only its 2J pieces (the rest come back as
// zeros) and takes its scales, masked to the valid blocks, straight from
// memory.  NS stages rotate with one barrier per unit, the loads of NS - 1
// units in flight.
template <int WM, int WN, int KS, int WMT, int WNT, int NS>
struct MxlCfg {
  static constexpr int GW = WM * WN;  // waves per k-group
  static constexpr int NW = GW * KS;
  static constexpr int BM = 32 * WMT * WM, BN = 32 * WNT * WN, R = BM + BN;
  // scale rows padded to whole 32-row loads per wave (the padding loads out
  // of range and is never read)
  static constexpr int RS = (R + 32 * GW - 1) / (32 * GW) * (32 * GW);
  static constexpr int CODE_B = R * 128, GROUP_B = R * 128 + RS * 8;
  static constexpr int STAGE_B = KS * GROUP_B;
  static constexpr int CIW = R / 8 / GW, SIW = RS / 32 / GW;  // loads per wave per stage
  static constexpr int LDS = NS * STAGE_B;
  static_assert(R % (8 * GW) == 0, "whole 8-row code loads per wave");
  static_assert(NS >= 3 && NS <= 5, "stage ring");
  static_assert((KS - 1) * GW * WMT * WNT * 4096 <= LDS, "reduction fits the ring");
};

template <int WM, int WN, int KS, int WMT, int WNT, int NS>
__global__ __launch_bounds__(64 * WM * WN * KS) void gemm_mxl_kernel(
    const uint32_t* __restrict__ xc, const uint8_t* __restrict__ xs,
    const uint32_t* __restrict__ wc, const uint8_t* __restrict__ wsc, int M, int N, int K,
    uint16_t* __restrict__ Y, int tiles_m, int tiles_n, int units_per_split) {
  using C = MxlCfg<WM, WN, KS, WMT, WNT, NS>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int kOff = 0x40000000;  // beyond every window: loads return 0
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int ks = wave / C::GW, wg = wave % C::GW;
  const int wm = wg / WN, wn = wg % WN;
  const int h = lane >> 5, l32 = lane & 31;
  int tm, tn;
  tile_of(tiles_m, tiles_n, 0, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int rows_m = min(C::BM, M - m0), rows_n = min(C::BN, N - n0);
  const int cb = K / 2, sb = K / 32;
  const rsrc_t rxc = make_rsrc(reinterpret_cast<const uint8_t*>(xc) + (int64_t)m0 * cb,
                               (int64_t)rows_m * cb);
  const rsrc_t rxs = make_rsrc(xs + (int64_t)m0 * sb, (int64_t)rows_m * sb);
  const rsrc_t rwc = make_rsrc(reinterpret_cast<const uint8_t*>(wc) + (int64_t)n0 * cb,
                               (int64_t)rows_n * cb);
  const rsrc_t rws = make_rsrc(wsc + (int64_t)n0 * sb, (int64_t)rows_n * sb);

  const int nfull = K / 256, tailJ = (K % 256) / 64;
  const int nunits = nfull + (tailJ ? 1 : 0);
  const int u0 = ks * units_per_split;
  const int u_end = min(nunits, u0 + units_per_split);

  // this wave's share of a stage: code loads s (rows 8 sg .. 8 sg + 7 of the
  // group's A-then-B rows, sg = wg CIW + s) and scale loads (32 rows each)
  int c_off[C::CIW], c_piece[C::CIW];
#pragma unroll
  for (int s = 0; s < C::CIW; ++s) {
    const int row = 8 * (wg * C::CIW + s) + (lane >> 3);
    const int piece = (lane & 7) ^ ((row >> 1) & 7);
    const int r = row < C::BM ? row : row - C::BM;
    c_off[s] = r * cb + 16 * piece;
    c_piece[s] = piece;
  }
  int s_off[C::SIW];
#pragma unroll
  for (int s = 0; s < C::SIW; ++s) {
    const int row = 32 * (wg * C::SIW + s) + (lane >> 1);
    const int r = row < C::BM ? row : row - C::BM;
    s_off[s] = row < C::R ? r * sb + 4 * (lane & 1) : kOff;  // padding rows: out of range
  }
  auto group_base = [&](int slot) { return lds + slot * C::STAGE_B + ks * C::GROUP_B; };

  auto load_stage = [&](int t, int slot) {
    const int u = u0 + t;
    const bool valid = u < u_end, tail = u == nfull;
    uint8_t* base = group_base(slot);
    const int uo = valid ? u * 128 : kOff;
#pragma unroll
    for (int s = 0; s < C::CIW; ++s) {
      const bool isA = 8 * (wg * C::CIW + s) < C::BM;  // wave-uniform
      const int off = c_off[s] + uo + ((tail && c_piece[s] >= 2 * tailJ) ? kOff : 0);
      buffer_load_lds16(isA ? rxc : rwc, reinterpret_cast<uint4*>(base) + (wg * C::CIW + s) * 64,
                        off, 0);
    }
    const int so = valid ? u * 8 : kOff;
#pragma unroll
    for (int s = 0; s < C::SIW; ++s) {
      const bool isA = 32 * (wg * C::SIW + s) < C::BM;  // padding rows sit past B
      buffer_load_lds4(isA ? rxs : rws, base + C::CODE_B + (wg * C::SIW + s) * 256,
                       s_off[s] + so, 0);
    }
  };

  f32x16_t acc[WMT][WNT];
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  constexpr bool kSplitAcc = WMT * WNT == 1;
  f32x16_t acc2;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc2[r] = 0.0f;

  int arow[WMT], brow[WNT];
#pragma unroll
  for (int i = 0; i < WMT; ++i) arow[i] = wm * 32 * WMT + 32 * i + l32;
#pragma unroll
  for (int j = 0; j < WNT; ++j) brow[j] = C::BM + wn * 32 * WNT + 32 * j + l32;

  // Scales of the last, partial unit (pieces 4h + q < 2J; the others load
  // out of range as 0, their codes being zero, or stale and then scaled below
  // fp32's range): a few bytes per lane, fetched in the first stage step so
  // their latency is long hidden when the unit comes up (fetched in the loop:
  // a value loaded before it would make the compiler wait for every load in
  // flight at the loop's entry).
  uint32_t ta[WMT][4], tb[WNT][4];
  auto load_tail_scales = [&]() {
    const bool mine = tailJ && u0 < u_end && u_end == nunits;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool v = mine && 4 * h + q < 2 * tailJ;
#pragma unroll
      for (int i = 0; i < WMT; ++i) {
        const int r = min(arow[i], rows_m - 1);
        ta[i][q] = __builtin_amdgcn_raw_buffer_load_b8(
            rxs, v ? r * sb + nfull * 8 + 4 * h + q : kOff, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        const int r = min(brow[j] - C::BM, rows_n - 1);
        tb[j][q] = __builtin_amdgcn_raw_buffer_load_b8(
            rws, v ? r * sb + nfull * 8 + 4 * h + q : kOff, 0, 0);
      }
    }
  };

  auto compute = [&](int t, int slot) {
    const int u = u0 + t;
    if (u >= u_end) return;
    const uint8_t* base = group_base(slot);
    uint32_t sa[WMT], sw[WNT];
    if (u != nfull) {
#pragma unroll
      for (int i = 0; i < WMT; ++i)
        sa[i] = *reinterpret_cast<const uint32_t*>(base + C::CODE_B + arow[i] * 8 + 4 * h);
#pragma unroll
      for (int j = 0; j < WNT; ++j)
        sw[j] = *reinterpret_cast<const uint32_t*>(base + C::CODE_B + brow[j] * 8 + 4 * h);
    } else {
      // partial unit: the scale bytes fetched at the start (the empty asm
      // keeps the combine, and so the wait for them, here rather than
      // hoisted in front of the stage loop)
#pragma unroll
      for (int i = 0; i < WMT; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(ta[i][q]));
        sa[i] = ta[i][0] | (ta[i][1] << 8) | (ta[i][2] << 16) | (ta[i][3] << 24);
      }
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(tb[j][q]));
        sw[j] = tb[j][0] | (tb[j][1] << 8) | (tb[j][2] << 16) | (tb[j][3] << 24);
      }
    }
    // all of the unit's LDS reads first, then its MFMAs back to back; a wave
    // with a single tile alternates two accumulators (even / odd sub-steps)
    // so consecutive MFMAs do not wait on each other
    uint4 a[4][WMT], b[4][WNT];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < WMT; ++i)
        a[q][i] = *reinterpret_cast<const uint4*>(
            base + arow[i] * 128 + 16 * ((4 * h + q) ^ ((arow[i] >> 1) & 7)));
#pragma unroll
      for (int j = 0; j < WNT; ++j)
        b[q][j] = *reinterpret_cast<const uint4*>(
            base + brow[j] * 128 + 16 * ((4 * h + q) ^ ((brow[j] >> 1) & 7)));
    }
    __builtin_amdgcn_sched_barrier(0);
    auto sub = [&](auto qc) {
      constexpr int Q = decltype(qc)::value;
#pragma unroll
      for (int i = 0; i < WMT; ++i) {
        const i32x8_t av = {(int)a[Q][i].x, (int)a[Q][i].y, (int)a[Q][i].z, (int)a[Q][i].w,
                            0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < WNT; ++j) {
          const i32x8_t bv = {(int)b[Q][j].x, (int)b[Q][j].y, (int)b[Q][j].z, (int)b[Q][j].w,
                              0, 0, 0, 0};
          f32x16_t& c = (kSplitAcc && (Q & 1)) ? acc2 : acc[i][j];
          // formats 4/4: FP4 E2M1 for both operands; op_sel picks the E8M0 byte
          c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, Q, (int)sa[i], Q,
                                                              (int)sw[j]);
        }
      }
    };
    sub(std::integral_constant<int, 0>{});
    sub(std::integral_constant<int, 1>{});
    sub(std::integral_constant<int, 2>{});
    sub(std::integral_constant<int, 3>{});
  };

  // every wave runs the same number of stages (units_per_split); a k-group
  // past its last unit loads out of range and skips the MFMAs
  const int nst = units_per_split;
  constexpr int L = C::CIW + C::SIW;  // loads per stage and wave
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < nst) load_stage(p, p);
  for (int t = 0; t < nst; ++t) {
    // stage t must have landed; the min(NS - 2, nst - 1 - t) stages after it
    // may stay in flight
    const int ahead = min(NS - 2, nst - 1 - t);
    if (ahead >= NS - 2) wait_vmem_le<(NS - 2) * L>();
    else if (ahead >= 2) wait_vmem_le<2 * L>();
    else if (ahead == 1) wait_vmem_le<L>();
    else wait_vmem();
    __syncthreads();
    if (t + NS - 1 < nst) load_stage(t + NS - 1, (t + NS - 1) % NS);
    if (t == 0) load_tail_scales();
    compute(t, t % NS);
  }

  if (kSplitAcc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][0][r] += acc2[r];
  }

  if (KS > 1) {
    __syncthreads();  // every wave is done reading the ring
    if (ks > 0) {
      float* dst = reinterpret_cast<float*>(lds) + (size_t)((ks - 1) * C::GW + wg) * WMT * WNT * 1024;
#pragma unroll
      for (int i = 0; i < WMT; ++i)
#pragma unroll
        for (int j = 0; j < WNT; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[((i * WNT + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (ks > 0) return;
    for (int q = 1; q < KS; ++q) {
      const float* src = reinterpret_cast<const float*>(lds) + (size_t)((q - 1) * C::GW + wg) * WMT * WNT * 1024;
#pragma unroll
      for (int i = 0; i < WMT; ++i)
#pragma unroll
        for (int j = 0; j < WNT; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += src[((i * WNT + j) * 16 + r) * 64 + lane];
    }
  }

#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNT; ++j) {
      const int n = n0 + wn * 32 * WNT + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 32 * WMT + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M && n < N) Y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16(acc[i][j][r]);
      }
    }
}

template <int WM, int WN, int KS, int WMT, int WNT, int NS>
hipError_t launch_mxl(const uint32_t* xc, const uint8_t* xs, int M, const bsfp_qtensor& w,
                      uint16_t* y, hipStream_t s) {
  using C = MxlCfg<WM, WN, KS, WMT, WNT, NS>;
  const int N = (int)w.rows, K = (int)w.cols;
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  const int nunits = (K + 255) / 256;
  const int ups = (nunits + KS - 1) / KS;
  if ((size_t)C::LDS > (size_t)device_max_lds()) return hipErrorInvalidConfiguration;
  if (C::LDS > 64 * 1024) {
    // opt in to the large LDS allocation, once per device
    static std::atomic<bool> granted[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!granted[dev].load(std::memory_order_relaxed)) {
      const hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&gemm_mxl_kernel<WM, WN, KS, WMT, WNT, NS>),
          hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
      if (e != hipSuccess) return e;
      granted[dev].store(true, std::memory_order_relaxed);
    }
  }
  launch_main(&gemm_mxl_kernel<WM, WN, KS, WMT, WNT, NS>, dim3(tiles_m * tiles_n), dim3(64 * C::NW),
              (uint32_t)C::LDS, s, xc, xs, w.codes, (const uint8_t*)w.scales, M, N, K, y, tiles_m,
              tiles_n, ups);
  return hipGetLastError();
}

hipError_t run_mx(const uint32_t* xc, const uint8_t* xs, int M, const bsfp_qtensor& w,
                  uint16_t* y, hipStream_t s) {
  // few rows: one 32 x 32 tile per workgroup with K split over 4 waves, so
  // the N / 32 workgroups still carry 4 waves each; up to 256 rows 64 x 128
  // tiles on 8 waves (32 x 32 per wave) with four stages, twice the
  // workgroups of the large tile and a deeper ring (1.2x faster at 128 and
  // 256 rows of the [5760, 2880] weights); otherwise 128 x 128 tiles on 8
  // waves (64 x 32 per wave)
  if (M <= 64) return launch_mxl<1, 1, 4, 1, 1, 3>(xc, xs, M, w, y, s);
  if (M <= 256) return launch_mxl<2, 4, 1, 1, 1, 4>(xc, xs, M, w, y, s);
  return launch_mxl<2, 4, 1, 2, 1, 3>(xc, xs, M, w, y, s);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

// Workspace for the qq paths:
//   NVFP4: [amax f32, g_x f32] (256 B), the partial maxima of |x|
//          (kAmaxParts floats), then xhat fp16 [M, K] (GEMM path); the
//          decode path puts xhat bf16 [M, K] at byte 256 instead
//   MXFP4: x codes uint32 [M, K/8] + x scales uint8 [M, K/32]
// Rows of x up to which the qq product runs as a GEMV on the exactly
// dequantized x (the decode path) instead of a GEMM.
constexpr int64_t kQqDecodeRows = 8;
constexpr size_t kNvWsHead = 256 + kAmaxParts * sizeof(float);

size_t qmm_workspace_bytes(int mode, int64_t M, int64_t K, int act) {
  if (act != BSFP_ACT_SAME) return 0;
  if (mode == BSFP_NVFP4) return kNvWsHead + align256((size_t)M * K * 2);
  if (mode == BSFP_MXFP4) {
    if (M <= kQqDecodeRows) return align256((size_t)M * K * 2);
    return align256((size_t)M * K / 2) + align256((size_t)M * K / 32);
  }
  return 0;
}

// Dense prefill path: W dequantized to bf16 (global scale included) into the
// caller's scratch, then the dense bf16 GEMM.
hipError_t launch_qmm_dense(const uint16_t* x, int64_t M, const bsfp_qtensor& w, void* scratch,
                            uint16_t* y, hipStream_t s) {
  // (a pending bsfp_time_next_launch pair stays for the GEMM: the dequantize
  // kernel launches without it)
  uint16_t* wd = reinterpret_cast<uint16_t*>(scratch);
  const hipError_t e = launch_dequantize(w, wd, s);
  if (e != hipSuccess) return e;
  return run_dense(x, (int)M, wd, (int)w.rows, (int)w.cols, y, s);
}

hipError_t launch_qmm(const uint16_t* x, int64_t M64, const bsfp_qtensor& w, int act, void* ws,
                      uint16_t* y, hipStream_t s) {
  const int M = (int)M64;
  if (act == BSFP_ACT_BF16) {
    switch (w.mode) {
      case BSFP_AFFINE: return run_dq_m<DEC_AFFINE>(x, M, w, nullptr, nullptr, y, s);
      case BSFP_MXFP4: return run_dq_m<DEC_MXFP4>(x, M, w, nullptr, nullptr, y, s);
      default: return run_dq_m<DEC_NVFP4>(x, M, w, w.global_scale, nullptr, y, s);
    }
  }
  const int64_t n = M64 * w.cols;
  if (M64 <= kQqDecodeRows) {
    // qq decode: x is quantized with w's mode and dequantized exactly to bf16
    // (E2M1 * E4M3 and E2M1 * 2^e fit bf16), then the GEMV runs on it with
    // the output scaled by alpha = g_x * g_w (NVFP4 with a global scale on w)
    // -- the same product as the GEMM path, at every M.  When x fits the
    // GEMV's LDS copy, the GEMV does all of it in one launch; otherwise the
    // quantize-dequantize runs first into the workspace.
    if (qmv_qx_fusable(M, w)) return launch_qmv_qx(x, M, w, y, s);
    if (w.mode == BSFP_NVFP4) {
      float* amax = reinterpret_cast<float*>(ws);
      float* gx = amax + 1;
      uint16_t* xhat = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + 256);
      hipError_t e = hipSuccess;
      if (w.global_scale) {
        e = launch_amax(x, n, amax, s);
        if (e == hipSuccess) e = launch_quantize_dequant_nvfp4_bf16(x, n / 8, xhat, amax, 1, gx, s);
        if (e != hipSuccess) return e;
        return launch_qmv(xhat, M, w, y, s, gx);
      }
      e = launch_quantize_dequant_nvfp4_bf16(x, n / 8, xhat, nullptr, 0, nullptr, s);
      if (e != hipSuccess) return e;
      return launch_qmv(xhat, M, w, y, s);
    }
    uint16_t* xhat = reinterpret_cast<uint16_t*>(ws);
    const hipError_t e = launch_quantize_dequant_mxfp4_bf16(x, n / 8, xhat, s);
    if (e != hipSuccess) return e;
    return launch_qmv(xhat, M, w, y, s);
  }
  if (w.mode == BSFP_NVFP4) {
    float* amax = reinterpret_cast<float*>(ws);
    float* gx = amax + 1;
    float* parts = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + 256);
    uint16_t* xhat = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + kNvWsHead);
    hipError_t e = hipSuccess;
    if (w.global_scale) {  // alpha = g_x * g_w with g_x = amax_x / 2688
      e = launch_amax_qdq_nvfp4_f16(x, n, xhat, parts, amax, gx, s);
      if (e != hipSuccess) return e;
      return run_dq_m<DEC_NVFP4_F16>(xhat, M, w, gx, w.global_scale, y, s);
    }
    e = launch_quantize_dequant_nvfp4_f16(x, n / 8, xhat, nullptr, 0, nullptr, s);
    if (e != hipSuccess) return e;
    return run_dq_m<DEC_NVFP4_F16>(xhat, M, w, nullptr, nullptr, y, s);
  }
  // MXFP4
  uint32_t* xc = reinterpret_cast<uint32_t*>(ws);
  uint8_t* xs = reinterpret_cast<uint8_t*>(ws) + align256((size_t)n / 2);
  hipError_t e = launch_quantize_mxfp4(x, n / 8, xc, xs, s);
  if (e != hipSuccess) return e;
  return run_mx(xc, xs, M, w, y, s);
}

}  // namespace bsfp
