// bsfp_device.hpp -- device-side building blocks shared by the gfx950 kernels:
// bf16 / E4M3 / E2M1 codecs, wave reductions, vector types.
//
// Format rules implemented here (the library's contract, include/bsfp.h):
//   E2M1: round to nearest even with saturation at 6, sign kept.  The gfx950
//         converter v_cvt_scalef32_pk_fp4_f32 with a unit scale implements
//         exactly this (checked over every non-NaN fp32 input); it is the
//         hardware form of the cvt.rn.satfinite.e2m1x2.f32 conversion named
//         in "perf(cuda): enable hardware NVFP4/MXFP4 conversion on Blackwell
//         builds" (Problem / Background).
//   E4M3: OCP E4M3FN, nearest even, values above 448 saturate to 448
//         (F8E4M3_MAX, "mlx 0.30.7.3 -> 0.30.7.6", qqmm_utils.cu).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsfp {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- formats
// Kernel-side format ids: the three base formats keep their bsfp mode
// values; the variants (MXFP8, affine 4-bit with groups 32 / 128, affine
// 8-bit with groups 32 / 64 / 128) follow.  8-bit codes pack 4 per word,
// element k in byte k mod 4.
enum : int {
  FMT_AFF4_G64 = 0, FMT_MXFP4 = 1, FMT_NVFP4 = 2, FMT_MXFP8 = 3,
  FMT_AFF4_G32 = 4, FMT_AFF4_G128 = 5, FMT_AFF8_G32 = 6, FMT_AFF8_G64 = 7, FMT_AFF8_G128 = 8
};
__host__ __device__ constexpr bool fmt_affine(int f) { return f == FMT_AFF4_G64 || f >= FMT_AFF4_G32; }
__host__ __device__ constexpr int fmt_bits(int f) { return (f == FMT_MXFP8 || f >= FMT_AFF8_G32) ? 8 : 4; }
__host__ __device__ constexpr int fmt_group(int f) {
  return f == FMT_NVFP4 ? 16
       : (f == FMT_MXFP4 || f == FMT_MXFP8 || f == FMT_AFF4_G32 || f == FMT_AFF8_G32) ? 32
       : (f == FMT_AFF4_G128 || f == FMT_AFF8_G128) ? 128 : 64;
}
__host__ __device__ constexpr int fmt_sbytes(int f) { return fmt_affine(f) ? 2 : 1; }
// Format id of (mode, bits, group), -1 if the library has none.
__host__ __device__ constexpr int format_id(int mode, int bits, int group) {
  return mode == 1 ? (bits == 4 && group == 32 ? FMT_MXFP4 : -1)
       : mode == 2 ? (bits == 4 && group == 16 ? FMT_NVFP4 : -1)
       : mode == 3 ? (bits == 8 && group == 32 ? FMT_MXFP8 : -1)
       : mode != 0 ? -1
       : bits == 4 ? (group == 64 ? FMT_AFF4_G64 : group == 32 ? FMT_AFF4_G32
                      : group == 128 ? FMT_AFF4_G128 : -1)
       : bits == 8 ? (group == 32 ? FMT_AFF8_G32 : group == 64 ? FMT_AFF8_G64
                      : group == 128 ? FMT_AFF8_G128 : -1)
       : -1;
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (the
// conversion of a float vector to bf16), one instruction per pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// ---------------------------------------------------------------- E4M3

// Non-negative fp32 -> E4M3 code, nearest even, > 448 -> 0x7E.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  if (!(s <= 448.0f)) return 0x7Eu;
  if (s < 0.015625f) {  // below 2^-6: subnormal grid m * 2^-9 (m = 8 is 2^-6)
    return (uint32_t)__builtin_rintf(s * 512.0f);
  }
  uint32_t u = __float_as_uint(s);
  uint32_t e = (u >> 23) - 120u;  // E4M3 biased exponent (bias 7)
  uint32_t m = u & 0x7FFFFFu;
  uint32_t r = m + 0x7FFFFu + ((m >> 20) & 1u);  // round 23 -> 3 mantissa bits
  return (e << 3) + (r >> 20);  // a mantissa carry moves into the exponent
}

// E4M3 code (sign bit ignored, never NaN here) -> fp32, exact.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;   // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E8M0 code -> 2^(c-127) as fp32 (c = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_decode(uint32_t c) {
  return c ? __uint_as_float(c << 23) : __uint_as_float(0x00400000u);
}

// ---------------------------------------------------------------- E2M1

// Two fp32 -> two E2M1 codes written into byte `SEL` of `old` (a -> low
// nibble, b -> high nibble).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Eight fp32 -> one packed word (element i -> nibble i).
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&v)[8]) {
  uint32_t w = 0;
  w = e2m1_pack2<0>(w, v[0], v[1]);
  w = e2m1_pack2<1>(w, v[2], v[3]);
  w = e2m1_pack2<2>(w, v[4], v[5]);
  w = e2m1_pack2<3>(w, v[6], v[7]);
  return w;
}

// Bytes 2 HI and 2 HI + 1 of w (two E4M3 codes) -> two bf16 values, exact
// (E4M3 has 4 significant bits).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Stochastic rounding of v to an E2M1 code with the random word r: between
// grid magnitudes lo < hi, hi when (r >> 8) * 2^-24 < (|v| - lo) / (hi - lo)
// (both exact in fp32), else lo; grid values stay, |v| >= 6 (or NaN)
// saturates, the sign bit follows v.
__device__ __forceinline__ uint32_t e2m1_encode_sr(float v, uint32_t r) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 3;
  const float a = fabsf(v);
  if (!(a < 6.0f)) return 7u | sign;
  uint32_t lo;
  float flo, inv_step;
  if (a < 2.0f) {  // grid 0, 0.5, 1, 1.5: code = floor(2a)
    lo = (uint32_t)(a * 2.0f);
    flo = (float)lo * 0.5f;
    inv_step = 2.0f;
  } else if (a < 4.0f) {  // grid 2, 3: codes 4, 5
    const uint32_t t = (uint32_t)a;
    lo = t + 2u;
    flo = (float)t;
    inv_step = 1.0f;
  } else {  // grid 4 (code 6), next 6
    lo = 6u;
    flo = 4.0f;
    inv_step = 0.5f;
  }
  const float p = (a - flo) * inv_step;  // exact: Sterbenz, power-of-two step
  const float u = (float)(r >> 8) * 5.9604644775390625e-08f;  // 2^-24, exact
  return (lo + (u < p ? 1u : 0u)) | sign;
}

// Eight fp32 -> one packed word with stochastic rounding; word i of (r0, r1)
// (r0.x .. r1.w) belongs to element i.
__device__ __forceinline__ uint32_t e2m1_pack8_sr(const float (&v)[8], const uint4& r0,
                                                  const uint4& r1) {
  const uint32_t r[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= e2m1_encode_sr(v[i], r[i]) << (4 * i);
  return w;
}

// Byte `SEL` of w (two codes) -> two bf16 values (low nibble -> .x), exact.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

// Byte `SEL` of w (two codes) -> two fp16 values (low nibble -> .x), exact.
template <int SEL>
__device__ __forceinline__ f16x2_t e2m1x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// Byte `SEL` of w -> two fp32 values, exact.
template <int SEL>
__device__ __forceinline__ f32x2_t e2m1x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Bytes (2*HI, 2*HI+1) of w, each holding a value 0..15, -> the two integers
// as bf16 (exact).  An OCP E4M3 byte 0..15 decodes to code * 2^-9 (subnormals
// and the first normal binade), and the converter's unit-exponent scale 2^9
// restores the integer.
template <bool HI>
__device__ __forceinline__ uint32_t nibbles_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------- dot

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------- reductions

// Butterfly over lanes differing in the bits of MASK..1 (power-of-two team).
template <int WIDTH>
__device__ __forceinline__ float team_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float team_min(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float team_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the 32 lanes of each half-wave, result in every lane: two
// quad_perm exchanges, row_half_mirror and row_mirror on the DPP path (no
// LDS), then one ds_swizzle xor 16 between the two 16-lane rows.
__device__ __forceinline__ float dpp_sum32(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  return v;
}

// ------------------------------------------- activation quantize-dequantize

// Byte SEL of w (two E2M1 codes) times the fp32 scale s, as a bf16 pair.
// The products are exact in fp32 and, for E4M3 or power-of-two scales, in
// bf16 as well, so the rounding in the pack never changes a value.
template <int SEL>
__device__ __forceinline__ uint32_t dq_pair_bf16(uint32_t w, float s) {
  const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return pack_bf16x2(v.x * s, v.y * s);
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// NVFP4 quantize of 8 bf16 values followed by exact dequantization without
// the global scale g: E2M1(code) * E4M3(S) as bf16.  The 8 values are half of
// a 16-value group whose other half sits in lane ^ 1 (both lanes call this).
// Codes and S are those of the NVFP4 quantizer with global scale g.
__device__ __forceinline__ uint4 qdq_nvfp4_half_bf16(const uint4 xv, float g) {
#pragma clang fp contract(off)
  float f[8];
  unpack8(xv, f);
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
  a = team_max<2>(a);
  uint32_t S = 0;
  float d = 0.0f;
  if (g != 0.0f) {
    S = e4m3_encode(a / (6.0f * g));
    d = e4m3_decode(S) * g;
  }
  uint4 o = {0u, 0u, 0u, 0u};
  if (d != 0.0f) {
    const float inv = 1.0f / d;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = f[k] * inv;
    const uint32_t w = e2m1_pack8(v);
    const float sf = e4m3_decode(S);
    o.x = dq_pair_bf16<0>(w, sf);
    o.y = dq_pair_bf16<1>(w, sf);
    o.z = dq_pair_bf16<2>(w, sf);
    o.w = dq_pair_bf16<3>(w, sf);
  }
  return o;
}

// MXFP4 quantize of 8 bf16 values followed by exact dequantization:
// E2M1(code) * 2^e as bf16 (exact for the exponents a bf16 input can
// produce).  The 8 values are a quarter of a 32-value group spread over 4
// adjacent lanes (all four call this).
__device__ __forceinline__ uint4 qdq_mxfp4_quarter_bf16(const uint4 xv) {
#pragma clang fp contract(off)
  float f[8];
  unpack8(xv, f);
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
  a = team_max<4>(a);
  // floor(log2 a) = biased exponent - 127 for normal a; subnormal or zero a
  // gives an exponent below -128, which the clamp maps to -127
  const int be = (int)(__float_as_uint(a) >> 23);
  const int e = max(be - 129, -127);
  const float p = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = f[k] * p;
  const uint32_t w = e2m1_pack8(v);
  const float sc = ldexpf(1.0f, e);  // 2^e, subnormal for e = -127
  uint4 o;
  o.x = dq_pair_bf16<0>(w, sc);
  o.y = dq_pair_bf16<1>(w, sc);
  o.z = dq_pair_bf16<2>(w, sc);
  o.w = dq_pair_bf16<3>(w, sc);
  return o;
}

// ---------------------------------------------------------------- buffers

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [base, base + bytes), bytes < 2^32: 32-bit
// offsets, and a load whose per-lane offset lies past the end returns 0.
constexpr int kRawBufferFlags = 0x00020000;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)(uint32_t)bytes, kRawBufferFlags);
}

__device__ __forceinline__ uint4 buffer_load_u128(rsrc_t r, int voff, int soff) {
  const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// The same load with the non-temporal cache policy (the `nt` bit, cache
// policy 2 on gfx950), for data read once: a decode GEMV's weights.
__device__ __forceinline__ uint4 buffer_load_u128_nt(rsrc_t r, int voff, int soff) {
  const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// s_waitcnt vmcnt(0): every vector-memory load of this wave has landed,
// including the direct-to-LDS ones the compiler does not track.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from a buffer straight into LDS: M0 holds the
// wave-uniform LDS byte offset and lane i lands at M0 + 16 i.  Written as
// inline assembly on purpose: the compiler does not track it, so it adds no
// waits of its own before LDS reads of other buffers (it cannot tell the
// buffers apart and would otherwise hold every read behind every such load);
// the kernel waits for these loads itself, with an explicit vmcnt before it
// reads the buffer (and a barrier when other waves read it).
__device__ __forceinline__ void buffer_load_lds16(rsrc_t r, uint4* lds, int voff, int soff) {
  typedef __attribute__((address_space(3))) uint4 lds_u4;
  const uint32_t base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u4*)lds);
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(r), "s"(soff), "{m0}"(base)
               : "memory");
}

// The same with the non-temporal cache policy, for data read once.
__device__ __forceinline__ void buffer_load_lds16_nt(rsrc_t r, uint4* lds, int voff, int soff) {
  typedef __attribute__((address_space(3))) uint4 lds_u4;
  const uint32_t base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u4*)lds);
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds"
               :
               : "v"(voff), "s"(r), "s"(soff), "{m0}"(base)
               : "memory");
}

// s_waitcnt vmcnt(N): at most N vector-memory loads of this wave still in
// flight (loads complete in issue order), the direct-to-LDS ones included.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 4 bytes per lane from a buffer straight into LDS (lane i lands at M0 + 4 i),
// untracked by the compiler like buffer_load_lds16.
__device__ __forceinline__ void buffer_load_lds4(rsrc_t r, void* lds, int voff, int soff) {
  typedef __attribute__((address_space(3))) uint32_t lds_u32;
  const uint32_t base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u32*)lds);
  asm volatile("buffer_load_dword %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(r), "s"(soff), "{m0}"(base)
               : "memory");
}

}  // namespace bsfp
