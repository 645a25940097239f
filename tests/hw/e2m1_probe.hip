// e2m1_probe.hip -- test support: the library's E2M1 encoder (the device
// helper bsfp::e2m1_pack2, i.e. v_cvt_scalef32_pk_fp4_f32 with a unit scale)
// applied to arbitrary fp32 inputs, one code per byte, so that a GPU test
// can check the converter's rounding, saturation and sign of zero on every
// fp32 bit pattern against the round-to-nearest-even / satfinite rule of
// cvt.rn.satfinite.e2m1x2.f32 ("perf(cuda): enable hardware NVFP4/MXFP4
// conversion on Blackwell builds", Problem / Background).  Not part of the
// product library.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../block_scaled_bit_fp_amd/csrc/bsfp_device.hpp"

namespace {

// Thread t converts the pair (v[2t], v[2t+1]); n is even.
__global__ __launch_bounds__(256) void e2m1_probe_kernel(const float2* __restrict__ v,
                                                         int64_t pairs,
                                                         uint16_t* __restrict__ codes) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= pairs) return;
  const float2 p = v[t];
  const uint32_t w = bsfp::e2m1_pack2<0>(0u, p.x, p.y);
  codes[t] = (uint16_t)((w & 0xFu) | ((w >> 4 & 0xFu) << 8));  // one code per byte
}

}  // namespace

extern "C" {

// codes[i] = E2M1 code of v[i] for i < n (n even, both device pointers,
// 16-byte aligned; the caller owns them).  Returns a hipError_t value.
int e2m1_probe(const float* v, int64_t n, uint8_t* codes, void* stream) {
  if (n < 0 || (n & 1) || (n > 0 && (!v || !codes))) return (int)hipErrorInvalidValue;
  const int64_t pairs = n / 2;
  if (pairs == 0) return (int)hipSuccess;
  const int64_t blocks = (pairs + 255) / 256;
  if (blocks > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(e2m1_probe_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, reinterpret_cast<const float2*>(v), pairs,
                     reinterpret_cast<uint16_t*>(codes));
  return (int)hipGetLastError();
}

}  // extern "C"
