// quantize.hip -- tensor amax, quantize (NVFP4 / MXFP4 / affine 4-bit) and
// dequantize kernels for gfx950.
//
// All three quantizers are HBM-bound streaming kernels over the flattened
// tensor: one lane owns 8 consecutive elements (one 16-byte load, one packed
// output word), a group is a power-of-two team of adjacent lanes (NVFP4 16
// elements = 2 lanes, MXFP4 32 = 4, affine 64 = 8), and the group statistic
// is a butterfly over the team.  Because cols is a multiple of the group
// size, groups never straddle rows, so the flat word index maps directly to
// the row-major code, scale and bias arrays.
//
// This file is compiled with -ffp-contract=off: every fp32 operation below is
// one correctly rounded IEEE operation, which keeps codes and scales
// bit-identical to the documented rules.
//
// Rules (the pages give the interfaces, not the arithmetic; the steps below
// are the library's contract, include/bsfp.h):
//   NVFP4  g = amax/2688 (448*6; "mlx 0.30.7.3 -> 0.30.7.6", qqmm_utils.cu);
//          S = E4M3(bamax / (6g)); d = E4M3(S)*g; code = E2M1(x * (1/d)),
//          d == 0 -> scale 0 and codes 0.
//   MXFP4  e = floor(log2 bamax) - 2 clamped to [-127, 127] (OCP MX shared
//          exponent); S = e + 127; code = E2M1(x * 2^-e).
//   AFFINE s = bf16((max - min)/15), b = bf16(min) = min,
//          q = clamp(rint((x - b) * (1/s)), 0, 15), s == 0 -> q = 0.
#include <algorithm>

#include "bsfp_device.hpp"
#include "bsfp_internal.hpp"

namespace bsfp {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ amax

__global__ void amax_init_kernel(float* out) { *out = 0.0f; }

// max |x| over n bf16 values.  Non-negative fp32 values order like their
// bit patterns, so the cross-workgroup step is an integer atomic max.  Atomics
// on one address are serialized (about 11 ns each, measured: 1024 workgroups
// spent 11 us in them on a 21 MB tensor), so the grid is one workgroup per
// CU, and a workgroup whose max does not exceed the value already there
// skips its atomic.
constexpr int kAmaxThreads = 1024;

// max |x| over this workgroup's share of the n values (grid-stride, four
// 16-byte loads in flight per lane); the result is valid in thread 0.
__device__ __forceinline__ float workgroup_absmax(const uint16_t* __restrict__ x, int64_t n) {
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t nv = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
  float m = 0.0f;
  // four independent 16-byte loads in flight per lane
  int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
  for (; i + 3 * stride < nv; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = xv[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float f[8];
      unpack8(v[u], f);
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[k]));
    }
  }
  for (; i < nv; i += stride) {
    float f[8];
    unpack8(xv[i], f);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[k]));
  }
  if (blockIdx.x == 0) {  // the n % 8 tail
    int64_t t = (nv << 3) + threadIdx.x;
    if (t < n) m = fmaxf(m, fabsf(bf16_to_f32(x[t])));
  }
  m = team_max<64>(m);
  __shared__ float part[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = part[0];
#pragma unroll
  for (int w = 1; w < kAmaxThreads / 64; ++w) r = fmaxf(r, part[w]);
  return r;
}

__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const uint16_t* __restrict__ x,
                                                             int64_t n, float* __restrict__ out) {
  const float r = workgroup_absmax(x, n);
  if (threadIdx.x == 0) {
    unsigned int* o = reinterpret_cast<unsigned int*>(out);
    const unsigned int cur = __hip_atomic_load(o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__float_as_uint(r) > cur) atomicMax(o, __float_as_uint(r));
  }
}

// The same maximum as per-workgroup partials: parts[blockIdx.x] = max |x|
// over the workgroup's share.  Needs no initialised output and no atomics;
// the consumer takes the max of the gridDim.x partials (max is exact in any
// order, so the result equals amax_kernel's).
__global__ __launch_bounds__(kAmaxThreads) void amax_parts_kernel(const uint16_t* __restrict__ x,
                                                                   int64_t n,
                                                                   float* __restrict__ parts) {
  const float r = workgroup_absmax(x, n);
  if (threadIdx.x == 0) parts[blockIdx.x] = r;
}

// The tensor amax from amax_parts_kernel's nparts (<= kThreads) partial
// maxima, in every thread of a kThreads workgroup.
__device__ __forceinline__ float reduce_parts(const float* __restrict__ parts, int nparts) {
  float a = (int)threadIdx.x < nparts ? parts[threadIdx.x] : 0.0f;
  a = team_max<64>(a);
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) a = fmaxf(a, red[w]);
  return a;
}

// ------------------------------------------------------------------ NVFP4

// The NVFP4 and MXFP4 quantizers take kQuantWords packed words per lane per
// step: lane l takes words c + l and c + 256 + l of a chunk of 512 words c,
// with both 16-byte loads issued before either is used, on a grid that
// strides over the chunks with at most a few workgroups per CU.
//   NVFP4, 8 workgroups per CU: fewer, longer workgroups pay the start-up
// (the read of g or the reduction of the partial maxima, then a barrier)
// once per workgroup slot instead of about four times; measured 20.8 us
// against 23.0 for X[4096, 5120] with g computed (one word per lane at 32
// workgroups per CU; one word at 8: 21.6; four words at 8: 21.7).
//   MXFP4, 16 workgroups per CU: W[5760, 2880] 9.1 us against 10.2 (8: 9.4;
// four words at 8: 9.6).  The same change to the dequantizer measured no
// faster.
constexpr int kQuantWords = 2;
constexpr int kNvfp4WgPerCu = 8;
constexpr int kMxfp4WgPerCu = 16;

// Words c + u * kThreads + lane (u < kQuantWords) of x, zeros past n_words.
__device__ __forceinline__ void load_chunk(const uint4* __restrict__ x, int64_t c, int64_t n_words,
                                           uint4 (&v)[kQuantWords]) {
  if (c + (int64_t)kThreads * kQuantWords <= n_words) {
#pragma unroll
    for (int u = 0; u < kQuantWords; ++u) v[u] = x[c + u * kThreads + threadIdx.x];
  } else {  // the last chunk
#pragma unroll
    for (int u = 0; u < kQuantWords; ++u) {
      const int64_t i = c + u * kThreads + threadIdx.x;
      v[u] = i < n_words ? x[i] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// rbits (stochastic rounding, NULL for nearest): 8 random words per packed
// word, element order.
//   parts / nparts (nparts <= kThreads): per-workgroup partial maxima of |x|
//   from amax_parts_kernel; every workgroup reduces them to the tensor amax
//   and takes g = amax/2688 (g_src is then ignored), and workgroup 0 stores
//   amax in *amax_out.
__global__ __launch_bounds__(kThreads) void quantize_nvfp4_kernel(
    const uint4* __restrict__ x, int64_t n_words, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, const float* __restrict__ g_src, int g_src_is_amax,
    float* __restrict__ g_out, const uint4* __restrict__ rbits,
    const float* __restrict__ parts, int nparts, float* __restrict__ amax_out) {
  float g = 1.0f;
  if (parts) {
    const float a = reduce_parts(parts, nparts);
    g = a / 2688.0f;
    if (amax_out && blockIdx.x == 0 && threadIdx.x == 0) *amax_out = a;
  } else if (g_src) {
    g = g_src_is_amax ? (*g_src / 2688.0f) : *g_src;
  }
  if (g_out && blockIdx.x == 0 && threadIdx.x == 0) *g_out = g;
  const float six_g = 6.0f * g;
  constexpr int64_t kChunk = (int64_t)kThreads * kQuantWords;
  for (int64_t c = (int64_t)blockIdx.x * kChunk; c < n_words; c += (int64_t)gridDim.x * kChunk) {
    uint4 xv[kQuantWords];
    load_chunk(x, c, n_words, xv);
#pragma unroll
    for (int u = 0; u < kQuantWords; ++u) {
      // n_words is even, so a lane pair (2j, 2j+1) is in or out together
      const int64_t i = c + u * kThreads + threadIdx.x;
      if (i >= n_words) break;
      float f[8];
      unpack8(xv[u], f);
      float a = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
      a = team_max<2>(a);  // 16-element group = lanes (2j, 2j+1)
      uint32_t S = 0;
      float d = 0.0f;
      if (g != 0.0f) {
        float sf = a / six_g;
        S = e4m3_encode(sf);
        d = e4m3_decode(S) * g;
      }
      uint32_t w = 0;
      if (d != 0.0f) {
        const float inv = 1.0f / d;
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = f[k] * inv;
        w = rbits ? e2m1_pack8_sr(v, rbits[2 * i], rbits[2 * i + 1]) : e2m1_pack8(v);
      } else {
        S = 0;
      }
      codes[i] = w;
      if ((i & 1) == 0) scales[i >> 1] = (uint8_t)S;
    }
  }
}

// NVFP4 quantize immediately followed by dequantization without the global
// scale: xhat = E2M1(code) * E4M3(S), written as fp16 (exact: at most 6
// significant bits, magnitudes 2^-10 .. 2688).  This is the activation
// operand of the NVFP4 qq GEMM (the pages' fp_quantize_dequantize, "mlx
// 0.30.7.3 -> 0.30.7.6", qqmm.cpp); the codes and scales are those
// bsfp_quantize produces for the same input and global scale.
//   BF16 = true writes bf16 instead (E2M1 * E4M3 has at most 6 significant
//   bits, so it is exact in bf16 too): the x of the qq decode GEMV.
//   parts / nparts (nparts <= kThreads): per-workgroup partial maxima of |x|
//   from amax_parts_kernel; every workgroup reduces them to the tensor amax
//   and takes g = amax/2688 (g_src is then ignored), and workgroup 0 stores
//   amax in *amax_out.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void quantize_dequant_nvfp4_kernel(
    const uint4* __restrict__ x, int64_t n_words, uint4* __restrict__ xhat,
    const float* __restrict__ g_src, int g_src_is_amax, float* __restrict__ g_out,
    const float* __restrict__ parts, int nparts, float* __restrict__ amax_out) {
  float g = 1.0f;
  if (parts) {
    const float a = reduce_parts(parts, nparts);
    g = a / 2688.0f;
    if (amax_out && blockIdx.x == 0 && threadIdx.x == 0) *amax_out = a;
  } else if (g_src) {
    g = g_src_is_amax ? (*g_src / 2688.0f) : *g_src;
  }
  if (g_out && blockIdx.x == 0 && threadIdx.x == 0) *g_out = g;
  const float six_g = 6.0f * g;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_words; i += stride) {
    if constexpr (BF16) {
      xhat[i] = qdq_nvfp4_half_bf16(x[i], g);
      continue;
    }
    float f[8];
    unpack8(x[i], f);
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
    a = team_max<2>(a);
    uint32_t S = 0;
    float d = 0.0f;
    if (g != 0.0f) {
      S = e4m3_encode(a / six_g);
      d = e4m3_decode(S) * g;
    }
    uint4 o = {0u, 0u, 0u, 0u};
    if (d != 0.0f) {
      const float inv = 1.0f / d;
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = f[k] * inv;
      const uint32_t w = e2m1_pack8(v);
      const _Float16 sh = (_Float16)e4m3_decode(S);  // exact in fp16
      const f16x2_t s2 = {sh, sh};
      o.x = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<0>(w) * s2);
      o.y = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<1>(w) * s2);
      o.z = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<2>(w) * s2);
      o.w = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<3>(w) * s2);
    }
    xhat[i] = o;
  }
}

// ------------------------------------------------------------------ MXFP4

__global__ __launch_bounds__(kThreads) void quantize_mxfp4_kernel(
    const uint4* __restrict__ x, int64_t n_words, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, const uint4* __restrict__ rbits) {
  constexpr int64_t kChunk = (int64_t)kThreads * kQuantWords;
  for (int64_t c = (int64_t)blockIdx.x * kChunk; c < n_words; c += (int64_t)gridDim.x * kChunk) {
    uint4 xv[kQuantWords];
    load_chunk(x, c, n_words, xv);
#pragma unroll
    for (int u = 0; u < kQuantWords; ++u) {
      // n_words is a multiple of 4, so a group's 4 lanes are in or out together
      const int64_t i = c + u * kThreads + threadIdx.x;
      if (i >= n_words) break;
      float f[8];
      unpack8(xv[u], f);
      float a = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
      a = team_max<4>(a);  // 32-element group = 4 lanes
      // floor(log2 a) = biased exponent - 127 for normal a; subnormal or zero
      // a gives an exponent below -128, which the clamp maps to -127.
      const int be = (int)(__float_as_uint(a) >> 23);
      const int e = max(be - 129, -127);  // e <= 125 for finite bf16 input
      const float p = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = f[k] * p;
      codes[i] = rbits ? e2m1_pack8_sr(v, rbits[2 * i], rbits[2 * i + 1]) : e2m1_pack8(v);
      if ((i & 3) == 0) scales[i >> 2] = (uint8_t)(e + 127);
    }
  }
}

// MXFP4 quantize followed by exact dequantization, written as bf16: the x of
// the qq decode GEMV (E2M1 * 2^e is exact in bf16 for the exponents a bf16
// input can produce).  Codes and exponents are those quantize_mxfp4_kernel
// produces.
__global__ __launch_bounds__(kThreads) void quantize_dequant_mxfp4_bf16_kernel(
    const uint4* __restrict__ x, int64_t n_words, uint4* __restrict__ xhat) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;  // multiple of 4
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_words; i += stride)
    xhat[i] = qdq_mxfp4_quarter_bf16(x[i]);
}

// ------------------------------------------------------------------ affine

__global__ __launch_bounds__(kThreads) void quantize_affine_kernel(
    const uint4* __restrict__ x, int64_t n_words, uint32_t* __restrict__ codes,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ biases) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;  // multiple of 8
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_words; i += stride) {
    float f[8];
    unpack8(x[i], f);
    float mn = f[0], mx = f[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) { mn = fminf(mn, f[k]); mx = fmaxf(mx, f[k]); }
    mn = team_min<8>(mn);  // 64-element group = 8 lanes
    mx = team_max<8>(mx);
    const float step = (mx - mn) / 15.0f;
    const uint32_t sb = f32_to_bf16(step);
    const uint32_t bb = __float_as_uint(mn) >> 16;  // mn is a bf16 value: exact
    const float sc = __uint_as_float(sb << 16);
    const float inv = (sc == 0.0f) ? 0.0f : 1.0f / sc;
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float q = __builtin_rintf((f[k] - mn) * inv);
      q = fminf(fmaxf(q, 0.0f), 15.0f);
      w |= (uint32_t)q << (4 * k);
    }
    codes[i] = w;
    if ((i & 7) == 0) {
      scales[i >> 3] = (uint16_t)sb;
      biases[i >> 3] = (uint16_t)bb;
    }
  }
}

// ------------------------------------------------------------------ dequantize

// One lane per packed word: 8 codes -> 8 bf16 (one 16-byte store).
template <int MODE>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint32_t* __restrict__ codes, const void* __restrict__ scales,
    const uint16_t* __restrict__ biases, const float* __restrict__ gptr, int64_t n_words,
    uint4* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const float g = gptr ? *gptr : 1.0f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_words; i += stride) {
    const uint32_t w = codes[i];
    float v[8];
    if constexpr (MODE == BSFP_AFFINE) {
      const float s = bf16_to_f32(reinterpret_cast<const uint16_t*>(scales)[i >> 3]);
      const float b = bf16_to_f32(biases[i >> 3]);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(s, (float)((w >> (4 * k)) & 15u), b);
    } else {
      f32x2_t p0 = e2m1x2_to_f32x2<0>(w), p1 = e2m1x2_to_f32x2<1>(w);
      f32x2_t p2 = e2m1x2_to_f32x2<2>(w), p3 = e2m1x2_to_f32x2<3>(w);
      v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
      v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
      const uint8_t* s8 = reinterpret_cast<const uint8_t*>(scales);
      if constexpr (MODE == BSFP_NVFP4) {
        const float sc = e4m3_decode(s8[i >> 1]);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = (v[k] * sc) * g;  // product exact, then one rounding
      } else {
        const float sc = e8m0_decode(s8[i >> 2]);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = v[k] * sc;  // exact power-of-two scaling
      }
    }
    uint4 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    o.z = pack_bf16x2(v[4], v[5]);
    o.w = pack_bf16x2(v[6], v[7]);
    out[i] = o;
  }
}

// ------------------------------------------------------ format variants

// Affine b-bit quantize with group G (4-bit group 64 is
// quantize_affine_kernel; same steps with 2^b - 1 levels): a lane owns 8
// elements, a group is G / 8 adjacent lanes.  8-bit codes go out as two
// words per lane (element k in byte k % 4).
template <int BITS, int G>
__global__ __launch_bounds__(kThreads) void quantize_affine_g_kernel(
    const uint4* __restrict__ x, int64_t n_units, uint32_t* __restrict__ codes,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ biases) {
  constexpr int TEAM = G / 8;
  constexpr float QMAX = (float)((1 << BITS) - 1);
  const int64_t stride = (int64_t)gridDim.x * kThreads;  // multiple of TEAM
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_units; i += stride) {
    float f[8];
    unpack8(x[i], f);
    float mn = f[0], mx = f[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) { mn = fminf(mn, f[k]); mx = fmaxf(mx, f[k]); }
    mn = team_min<TEAM>(mn);
    mx = team_max<TEAM>(mx);
    const float step = (mx - mn) / QMAX;
    const uint32_t sb = f32_to_bf16(step);
    const uint32_t bb = __float_as_uint(mn) >> 16;  // mn is a bf16 value: exact
    const float sc = __uint_as_float(sb << 16);
    const float inv = (sc == 0.0f) ? 0.0f : 1.0f / sc;
    uint32_t q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float t = __builtin_rintf((f[k] - mn) * inv);
      q[k] = (uint32_t)fminf(fmaxf(t, 0.0f), QMAX);
    }
    if constexpr (BITS == 4) {
      uint32_t w = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) w |= q[k] << (4 * k);
      codes[i] = w;
    } else {
      reinterpret_cast<uint2*>(codes)[i] =
          make_uint2(q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24),
                     q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24));
    }
    if (i % TEAM == 0) {
      scales[i / TEAM] = (uint16_t)sb;
      biases[i / TEAM] = (uint16_t)bb;
    }
  }
}

// MXFP8 (OCP MX, E4M3 elements): e = floor(log2 amax) - 8 per 32 elements
// (4 lanes), clamped to [-127, 127]; elements E4M3(x * 2^-e), nearest even,
// saturating at 448, sign bit kept.
__global__ __launch_bounds__(kThreads) void quantize_mxfp8_kernel(
    const uint4* __restrict__ x, int64_t n_units, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;  // multiple of 4
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_units; i += stride) {
    float f[8];
    unpack8(x[i], f);
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
    a = team_max<4>(a);
    // floor(log2 a) = biased exponent - 127 for normal a; subnormal or zero
    // a gives an exponent below -127 after the - 8, which the clamp maps to
    // -127
    const int be = (int)(__float_as_uint(a) >> 23);
    const int e = max(be - 135, -127);
    const float p = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact
    uint32_t c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float v = f[k] * p;
      c[k] = e4m3_encode(fabsf(v)) | ((__float_as_uint(v) >> 31) << 7);
    }
    codes[i] = make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                          c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
    if ((i & 3) == 0) scales[i >> 2] = (uint8_t)(e + 127);
  }
}

// Format variants to bf16: affine bf16(fma(s, q, b)); MXFP8 bf16(E4M3 *
// 2^e) with the product in fp32 (exact unless below fp32's normal range,
// then one rounding).  8 elements per lane.
template <int FMT>
__global__ __launch_bounds__(kThreads) void dequantize_g_kernel(
    const uint32_t* __restrict__ codes, const void* __restrict__ scales,
    const uint16_t* __restrict__ biases, int64_t n_units, uint4* __restrict__ out) {
  constexpr int BITS = fmt_bits(FMT), UPG = fmt_group(FMT) / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_units; i += stride) {
    float v[8];
    if constexpr (BITS == 4) {
      const uint32_t w = codes[i];
      const float s = bf16_to_f32(reinterpret_cast<const uint16_t*>(scales)[i / UPG]);
      const float b = bf16_to_f32(biases[i / UPG]);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(s, (float)((w >> (4 * k)) & 15u), b);
    } else {
      const uint2 w = reinterpret_cast<const uint2*>(codes)[i];
      if constexpr (FMT == FMT_MXFP8) {
        const float sc = e8m0_decode(reinterpret_cast<const uint8_t*>(scales)[i >> 2]);
        const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.x, 1.0f, false);
        const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.x, 1.0f, true);
        const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.y, 1.0f, false);
        const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.y, 1.0f, true);
        v[0] = p0.x * sc; v[1] = p0.y * sc; v[2] = p1.x * sc; v[3] = p1.y * sc;
        v[4] = p2.x * sc; v[5] = p2.y * sc; v[6] = p3.x * sc; v[7] = p3.y * sc;
      } else {
        const float s = bf16_to_f32(reinterpret_cast<const uint16_t*>(scales)[i / UPG]);
        const float b = bf16_to_f32(biases[i / UPG]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t q = ((k < 4 ? w.x : w.y) >> (8 * (k & 3))) & 255u;
          v[k] = __builtin_fmaf(s, (float)q, b);
        }
      }
    }
    uint4 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    o.z = pack_bf16x2(v[4], v[5]);
    o.w = pack_bf16x2(v[6], v[7]);
    out[i] = o;
  }
}

// Grid for a flat streaming kernel: enough workgroups to fill every CU
// several times over, no more than the work needs.
// Workgroups of amax_parts_kernel over n values: enough for four 16-byte
// loads in flight per lane, at most one per CU and at most kAmaxParts.
int amax_parts_grid(int64_t n) {
  const int64_t want = ((n >> 3) / 4 + kAmaxThreads) / kAmaxThreads;
  return (int)std::min<int64_t>(std::max<int64_t>(want, 1),
                                std::min(device_cu_count(), kAmaxParts));
}

// Workgroups of the quantizers that take kQuantWords words per lane, over
// n_words packed words, at most wg_per_cu per CU.
int chunk_grid(int64_t n_words, int wg_per_cu) {
  constexpr int64_t chunk = (int64_t)kThreads * kQuantWords;
  const int64_t want = (n_words + chunk - 1) / chunk;
  const int64_t cap = (int64_t)device_cu_count() * wg_per_cu;
  return (int)std::max<int64_t>(1, std::min(want, cap));
}

int stream_grid(int64_t items) {
  const int64_t want = (items + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 32;
  return (int)(want < cap ? (want > 0 ? want : 1) : cap);
}

}  // namespace

hipError_t launch_amax(const uint16_t* x, int64_t n, float* amax_out, hipStream_t s) {
  hipLaunchKernelGGL(amax_init_kernel, dim3(1), dim3(1), 0, s, amax_out);
  if (n > 0) {
    const int64_t nv = n >> 3;
    const int64_t want = (nv / 4 + kAmaxThreads) / kAmaxThreads;  // 4 loads per lane
    const int grid = (int)std::min<int64_t>(std::max<int64_t>(want, 1), device_cu_count());
    hipLaunchKernelGGL(amax_kernel, dim3(grid), dim3(kAmaxThreads), 0, s, x, n, amax_out);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_nvfp4(const uint16_t* x, int64_t n_words, uint32_t* codes,
                                 uint8_t* scales, const float* g_src, int g_src_is_amax,
                                 float* g_out, hipStream_t s, const uint32_t* rbits) {
  hipLaunchKernelGGL(quantize_nvfp4_kernel, dim3(chunk_grid(n_words, kNvfp4WgPerCu)), dim3(kThreads), 0, s,
                     reinterpret_cast<const uint4*>(x), n_words, codes, scales, g_src,
                     g_src_is_amax, g_out, reinterpret_cast<const uint4*>(rbits),
                     (const float*)nullptr, 0, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_amax_quantize_nvfp4(const uint16_t* x, int64_t n, uint32_t* codes,
                                      uint8_t* scales, float* parts, float* amax_out,
                                      float* g_out, hipStream_t s, const uint32_t* rbits) {
  const int grid = amax_parts_grid(n);
  hipLaunchKernelGGL(amax_parts_kernel, dim3(grid), dim3(kAmaxThreads), 0, s, x, n, parts);
  hipLaunchKernelGGL(quantize_nvfp4_kernel, dim3(chunk_grid(n / 8, kNvfp4WgPerCu)), dim3(kThreads), 0, s,
                     reinterpret_cast<const uint4*>(x), n / 8, codes, scales,
                     (const float*)nullptr, 0, g_out, reinterpret_cast<const uint4*>(rbits),
                     (const float*)parts, grid, amax_out);
  return hipGetLastError();
}

hipError_t launch_quantize_dequant_nvfp4_f16(const uint16_t* x, int64_t n_words, void* xhat,
                                             const float* g_src, int g_src_is_amax,
                                             float* g_out, hipStream_t s) {
  hipLaunchKernelGGL(quantize_dequant_nvfp4_kernel<false>, dim3(stream_grid(n_words)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint4*>(x), n_words,
                     reinterpret_cast<uint4*>(xhat), g_src, g_src_is_amax, g_out,
                     (const float*)nullptr, 0, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_amax_qdq_nvfp4_f16(const uint16_t* x, int64_t n, void* xhat, float* parts,
                                     float* amax_out, float* g_out, hipStream_t s) {
  const int grid = amax_parts_grid(n);
  hipLaunchKernelGGL(amax_parts_kernel, dim3(grid), dim3(kAmaxThreads), 0, s, x, n, parts);
  hipLaunchKernelGGL(quantize_dequant_nvfp4_kernel<false>, dim3(stream_grid(n / 8)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint4*>(x), n / 8,
                     reinterpret_cast<uint4*>(xhat), (const float*)nullptr, 0, g_out,
                     (const float*)parts, grid, amax_out);
  return hipGetLastError();
}

hipError_t launch_quantize_dequant_nvfp4_bf16(const uint16_t* x, int64_t n_words, void* xhat,
                                              const float* g_src, int g_src_is_amax,
                                              float* g_out, hipStream_t s) {
  hipLaunchKernelGGL(quantize_dequant_nvfp4_kernel<true>, dim3(stream_grid(n_words)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint4*>(x), n_words,
                     reinterpret_cast<uint4*>(xhat), g_src, g_src_is_amax, g_out,
                     (const float*)nullptr, 0, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_dequant_mxfp4_bf16(const uint16_t* x, int64_t n_words, void* xhat,
                                              hipStream_t s) {
  hipLaunchKernelGGL(quantize_dequant_mxfp4_bf16_kernel, dim3(stream_grid(n_words)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint4*>(x), n_words,
                     reinterpret_cast<uint4*>(xhat));
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const uint16_t* x, int64_t n_words, uint32_t* codes,
                                 uint8_t* scales, hipStream_t s, const uint32_t* rbits) {
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3(chunk_grid(n_words, kMxfp4WgPerCu)), dim3(kThreads), 0, s,
                     reinterpret_cast<const uint4*>(x), n_words, codes, scales,
                     reinterpret_cast<const uint4*>(rbits));
  return hipGetLastError();
}

hipError_t launch_quantize_affine(const uint16_t* x, int64_t n_words, uint32_t* codes,
                                  uint16_t* scales, uint16_t* biases, hipStream_t s) {
  hipLaunchKernelGGL(quantize_affine_kernel, dim3(stream_grid(n_words)), dim3(kThreads), 0, s,
                     reinterpret_cast<const uint4*>(x), n_words, codes, scales, biases);
  return hipGetLastError();
}

hipError_t launch_quantize_variant(const uint16_t* x, const bsfp_qtensor& q, hipStream_t s) {
  const int64_t n_units = q.rows * q.cols / 8;
  if (n_units == 0) return hipGetLastError();
  const dim3 grid(stream_grid(n_units)), block(kThreads);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint16_t* sc = reinterpret_cast<uint16_t*>(q.scales);
  switch (format_id(q.mode, q.bits, q.group_size)) {
    case FMT_MXFP8:
      hipLaunchKernelGGL(quantize_mxfp8_kernel, grid, block, 0, s, xv, n_units,
                         reinterpret_cast<uint2*>(q.codes), (uint8_t*)q.scales);
      break;
    case FMT_AFF4_G32:
      hipLaunchKernelGGL((quantize_affine_g_kernel<4, 32>), grid, block, 0, s, xv, n_units,
                         q.codes, sc, q.biases);
      break;
    case FMT_AFF4_G128:
      hipLaunchKernelGGL((quantize_affine_g_kernel<4, 128>), grid, block, 0, s, xv, n_units,
                         q.codes, sc, q.biases);
      break;
    case FMT_AFF8_G32:
      hipLaunchKernelGGL((quantize_affine_g_kernel<8, 32>), grid, block, 0, s, xv, n_units,
                         q.codes, sc, q.biases);
      break;
    case FMT_AFF8_G64:
      hipLaunchKernelGGL((quantize_affine_g_kernel<8, 64>), grid, block, 0, s, xv, n_units,
                         q.codes, sc, q.biases);
      break;
    case FMT_AFF8_G128:
      hipLaunchKernelGGL((quantize_affine_g_kernel<8, 128>), grid, block, 0, s, xv, n_units,
                         q.codes, sc, q.biases);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const bsfp_qtensor& q, uint16_t* out, hipStream_t s) {
  const int64_t n_words = q.rows * q.cols / 8;
  if (n_words == 0) return hipGetLastError();
  const dim3 grid(stream_grid(n_words)), block(kThreads);
  uint4* o = reinterpret_cast<uint4*>(out);
  const int fmt = format_id(q.mode, q.bits, q.group_size);
  switch (fmt) {
    case FMT_MXFP8:
      hipLaunchKernelGGL(dequantize_g_kernel<FMT_MXFP8>, grid, block, 0, s, q.codes, q.scales,
                         nullptr, n_words, o);
      return hipGetLastError();
    case FMT_AFF4_G32:
      hipLaunchKernelGGL(dequantize_g_kernel<FMT_AFF4_G32>, grid, block, 0, s, q.codes,
                         q.scales, q.biases, n_words, o);
      return hipGetLastError();
    case FMT_AFF4_G128:
      hipLaunchKernelGGL(dequantize_g_kernel<FMT_AFF4_G128>, grid, block, 0, s, q.codes,
                         q.scales, q.biases, n_words, o);
      return hipGetLastError();
    case FMT_AFF8_G32:
      hipLaunchKernelGGL(dequantize_g_kernel<FMT_AFF8_G32>, grid, block, 0, s, q.codes,
                         q.scales, q.biases, n_words, o);
      return hipGetLastError();
    case FMT_AFF8_G64:
      hipLaunchKernelGGL(dequantize_g_kernel<FMT_AFF8_G64>, grid, block, 0, s, q.codes,
                         q.scales, q.biases, n_words, o);
      return hipGetLastError();
    case FMT_AFF8_G128:
      hipLaunchKernelGGL(dequantize_g_kernel<FMT_AFF8_G128>, grid, block, 0, s, q.codes,
                         q.scales, q.biases, n_words, o);
      return hipGetLastError();
    default:
      break;
  }
  switch (q.mode) {
    case BSFP_AFFINE:
      hipLaunchKernelGGL(dequantize_kernel<BSFP_AFFINE>, grid, block, 0, s, q.codes, q.scales,
                         q.biases, nullptr, n_words, o);
      break;
    case BSFP_MXFP4:
      hipLaunchKernelGGL(dequantize_kernel<BSFP_MXFP4>, grid, block, 0, s, q.codes, q.scales,
                         nullptr, nullptr, n_words, o);
      break;
    default:
      hipLaunchKernelGGL(dequantize_kernel<BSFP_NVFP4>, grid, block, 0, s, q.codes, q.scales,
                         nullptr, q.global_scale, n_words, o);
      break;
  }
  return hipGetLastError();
}

}  // namespace bsfp
