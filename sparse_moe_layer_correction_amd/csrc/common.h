// Shared device helpers for the gfx950 kernels of the LatentMoE forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// MFMA operand and accumulator vector types (gfx950 bf16 MFMA takes 8 bf16 per lane).
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native 16-byte vector (HIP's uint4 is a struct that defeats scalar
// replacement of small arrays and ends up in scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// two fp32 -> packed bf16x2 (low half = a)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

// max(v, 0)^2 (0 for NaN). Written as one v_max_f32: the compiler makes any
// max or select of v and 0 a max after a canonicalising max (quieting a
// signalling NaN, which an accumulator never holds), two instructions per
// value in the tiled products' epilogue.
__device__ __forceinline__ float relu2(float v) {
  float r;
  asm("v_max_f32 %0, 0, %1" : "=v"(r) : "v"(v));
  return r * r;
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, mask, kWave);
  hi = __shfl_xor(hi, mask, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// max(v, the value DPP control CTRL brings from another lane), 0 (the identity
// of an unsigned max) where the control brings nothing
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = __builtin_amdgcn_update_dpp(0u, v, CTRL, ROW_MASK, 0xF, true);
  return o > v ? o : v;
}

// Max over the 64 lanes, returned to every lane. DPP moves (VALU latency) rather
// than LDS permutes: row shifts by 1, 2, 4, 8 leave each 16-lane row's max in
// its lane 15; broadcasts of lane 15 and lane 31 carry it to the last lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<0x111, 0xF>(v);   // row_shr:1
  v = dpp_max_u32<0x112, 0xF>(v);   // row_shr:2
  v = dpp_max_u32<0x114, 0xF>(v);   // row_shr:4
  v = dpp_max_u32<0x118, 0xF>(v);   // row_shr:8
  v = dpp_max_u32<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_max_u32<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}

// 64-bit max over the 64 lanes as two 32-bit ones: the high words', then the low
// words' of the lanes that hold that high word (a 64-bit compare and two
// selects per step cost the top-k's serial rounds about twice as much).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan_i32(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

}  // namespace moe
