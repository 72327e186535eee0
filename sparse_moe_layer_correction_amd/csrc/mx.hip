// MX quantisation of bf16 weights on gfx950 (OCP Microscaling formats, one
// E8M0 scale per 32 consecutive elements of a row): MXFP8 (E4M3 elements) and
// MXFP4 (E2M1 elements, two per byte).
//
// The released model keeps its experts in a block-scaled 4-bit format (the QA
// page on the experts' NVFP4 storage); MXFP8 and MXFP4 are the block-scaled
// formats whose decode gfx950 does in one instruction per two elements.
//
// MXFP8. Per block: the shared exponent is e = floor(log2(max |v|)) - 8 (8 = the exponent of E4M3's largest
// normal, 448), clamped to [-127, 127], stored as the code e + 127 (an all-zero
// block takes e = -127); each element is v * 2^-e rounded to the nearest E4M3
// value, ties to even, magnitudes of 448 and above saturating to 448 (E4M3 "fn"
// has no infinities; its NaN codes are never produced). The scaling by 2^-e is
// exact, and so is every step of the rounding below, so the codes are exactly
// those of the definition.
#include "kernels.h"

namespace moe {

__device__ __forceinline__ uint32_t e4m3_code(float r) {
  const uint32_t sign = (__float_as_uint(r) >> 24) & 0x80u;
  const float a = fabsf(r);
  if (a >= 448.f) return sign | 0x7Eu;                       // saturate
  if (a < 0.015625f) {                                        // below 2^-6: grid 2^-9
    const float q = __builtin_rintf(a * 512.f);              // 0..8 (8 = the smallest normal)
    return sign | (uint32_t)q;
  }
  int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6..8
  const float m = a * __builtin_ldexpf(1.f, -e);             // [1, 2)
  float f = __builtin_rintf((m - 1.f) * 8.f);                // 3 mantissa bits, ties to even
  if (f >= 8.f) { f = 0.f; ++e; }
  const uint32_t code = ((uint32_t)(e + 7) << 3) | (uint32_t)f;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// one thread per block of 32 elements
__global__ void __launch_bounds__(256) mxfp8_quantize_kernel(const uint16_t* __restrict__ src, int64_t nblocks,
                                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* p = reinterpret_cast<const u32x4*>(src + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 w = p[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[i * 8 + 2 * q] = bf16_bits_to_f32(ws[q] & 0xFFFFu);
      v[i * 8 + 2 * q + 1] = bf16_bits_to_f32(ws[q] >> 16);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = -127;
  if (amax > 0.f) {
    // amax = mant * 2^x with mant in [0.5, 1): floor(log2 amax) = x - 1
    e = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  const float inv = __builtin_ldexpf(1.f, -e);
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    packed[i] = e4m3_code(v[4 * i] * inv) | (e4m3_code(v[4 * i + 1] * inv) << 8) |
                (e4m3_code(v[4 * i + 2] * inv) << 16) | (e4m3_code(v[4 * i + 3] * inv) << 24);
  }
  u32x4* o = reinterpret_cast<u32x4*>(codes + b * 32);
  o[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
  o[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
  scales[b] = (uint8_t)(e + 127);
}

hipError_t launch_mxfp8_quantize(const uint16_t* src, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                                 hipStream_t st) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st, src, nblocks,
                     codes, scales);
  return hipGetLastError();
}

// MXFP4. E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6: the grid step is 0.5
// below 2, 1 in [2, 4) and 2 in [4, 6]. The block exponent is
// e = floor(log2 amax) - 2 (2 = the exponent of E2M1's largest normal, 6), and
// each element is v * 2^-e rounded to the nearest magnitude, ties to the even
// multiple of the step (the code with mantissa bit 0), saturating at 6.
__device__ __forceinline__ uint32_t e2m1_code(float r) {
  const uint32_t sign = (__float_as_uint(r) >> 28) & 0x8u;
  const float a = fminf(fabsf(r), 6.f);
  const float step = a < 2.f ? 0.5f : (a < 4.f ? 1.f : 2.f);
  const float v = fminf(__builtin_rintf(a / step) * step, 6.f);   // a / step is exact (power-of-two step)
  const uint32_t mag = v < 2.f ? (uint32_t)(v * 2.f) : (v < 4.f ? (uint32_t)v + 2u : (uint32_t)(v * 0.5f) + 4u);
  return sign | mag;
}

// one thread per block of 32 elements: 16 bytes of codes (element 2i in the low
// nibble of byte i) and one scale byte
__global__ void __launch_bounds__(256) mxfp4_quantize_kernel(const uint16_t* __restrict__ src, int64_t nblocks,
                                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* p = reinterpret_cast<const u32x4*>(src + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 w = p[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[i * 8 + 2 * q] = bf16_bits_to_f32(ws[q] & 0xFFFFu);
      v[i * 8 + 2 * q + 1] = bf16_bits_to_f32(ws[q] >> 16);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = -127;
  if (amax > 0.f) {
    e = __builtin_amdgcn_frexp_expf(amax) - 1 - 2;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  const float inv = __builtin_ldexpf(1.f, -e);
  uint32_t packed[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= e2m1_code(v[8 * i + j] * inv) << (4 * j);
    packed[i] = w;
  }
  *reinterpret_cast<u32x4*>(codes + b * 16) = u32x4{packed[0], packed[1], packed[2], packed[3]};
  scales[b] = (uint8_t)(e + 127);
}

hipError_t launch_mxfp4_quantize(const uint16_t* src, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                                 hipStream_t st) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp4_quantize_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st, src, nblocks,
                     codes, scales);
  return hipGetLastError();
}

}  // namespace moe
