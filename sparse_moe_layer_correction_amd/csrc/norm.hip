// The layer's neighbours on gfx950: the pre-norm RMSNorm that feeds it and the
// load-balancing update of the routing correction bias.
//
// RMSNorm (the QA page on Nemotron 3 Ultra, CH2 Q2.8): per row,
//   y = gamma * bf16( x * rsqrt(mean(x^2) + eps) )
// with the product by gamma (a bf16 weight) rounded to bf16 again. The page
// computes the statistics in (at least) fp32; here the mean of squares, the
// scale and both products are float64 and each of the two roundings is one
// round-to-nearest-even from that float64 value, so every output is the unique
// bf16 value the definition gives. The work is bound by reading x and writing
// y once (4 bytes per element); float64 arithmetic costs nothing visible here.
//
// Bias update (same page, CH5 Q5.3): b_i <- b_i - eta * (load_i - mean load),
// load_i the slots routed to expert i in the batch (from the permutation's
// offsets), mean load = total slots / E, evaluated in float64 with no fused
// multiply-add and rounded once to the fp32 bias.
#include "kernels.h"

namespace moe {

// Round a float64 value to the nearest bf16 value, ties to even; the result is
// returned as a float64 that is exactly that bf16 value.
__device__ __forceinline__ double round_bf16_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const int ex = (int)((b >> 52) & 0x7FF) - 1023;
  if (ex >= -126) {
    // normal bf16 range: keep 8 significant bits (1 + 7 of the 52 fraction bits)
    const uint64_t lsb = (b >> 45) & 1u;
    const uint64_t r = (b + ((1ull << 44) - 1) + lsb) & ~((1ull << 45) - 1);
    return __longlong_as_double((long long)r);
  }
  // below 2^-126 the bf16 grid is the subnormal spacing 2^-133; both scalings are exact
  return __builtin_rint(v * 0x1p133) * 0x1p-133;
}

__device__ __forceinline__ uint32_t bf16_bits_of(double exact_bf16) {
  return __float_as_uint((float)exact_bf16) >> 16;
}

// y = gamma * bf16(x * r) for the NC 16-byte chunks c of a row, rounded twice as stated.
__device__ __forceinline__ u32x4 norm_chunk(const u32x4 v, const u32x4 g, double r) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const double xv = (double)bf16_bits_to_f32((v[q] >> (16 * h)) & 0xFFFFu);
      const double gv = (double)bf16_bits_to_f32((g[q] >> (16 * h)) & 0xFFFFu);
      const double t = round_bf16_f64(xv * r);
      w |= bf16_bits_of(round_bf16_f64(gv * t)) << (16 * h);
    }
    o[q] = w;
  }
  return o;
}

__device__ __forceinline__ double sumsq_chunk(const u32x4 v) {
  double ss = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const double a = (double)bf16_bits_to_f32(v[q] & 0xFFFFu);
    const double b = (double)bf16_bits_to_f32(v[q] >> 16);
    ss += a * a;
    ss += b * b;
  }
  return ss;
}

// One workgroup of 256 threads per row. Thread i holds the row's 16-byte chunks
// i, i + 256, ... (up to NC of them, H <= 2048 * NC) in registers, so the row is
// read from HBM once; the sum of squares is reduced over the wave (shuffles)
// and then over the 4 waves (LDS, summed in wave order: deterministic).
template <int NC>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const uint16_t* x, const uint16_t* __restrict__ gamma,
                                                      int64_t T, int H, double eps, uint16_t* y) {
  __shared__ double part[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * H);
  const u32x4* gr = reinterpret_cast<const u32x4*>(gamma);
  u32x4* yr = reinterpret_cast<u32x4*>(y + row * H);
  const int nch = H / 8;

  u32x4 v[NC];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + 256 * i;
    v[i] = c < nch ? xr[c] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) ss += sumsq_chunk(v[i]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const double tot = ((part[0] + part[1]) + part[2]) + part[3];
  const double r = 1.0 / __builtin_sqrt(tot / (double)H + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + 256 * i;
    if (c < nch) yr[c] = norm_chunk(v[i], gr[c], r);
  }
}

// Rows longer than 2048 * 8 elements: the same with the row streamed twice
// (the second pass hits the caches).
__global__ void __launch_bounds__(256) rmsnorm_long_kernel(const uint16_t* x, const uint16_t* __restrict__ gamma,
                                                           int64_t T, int H, double eps, uint16_t* y) {
  __shared__ double part[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * H);
  const u32x4* gr = reinterpret_cast<const u32x4*>(gamma);
  u32x4* yr = reinterpret_cast<u32x4*>(y + row * H);
  const int nch = H / 8;
  double ss = 0.0;
  for (int c = tid; c < nch; c += 256) ss += sumsq_chunk(xr[c]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const double tot = ((part[0] + part[1]) + part[2]) + part[3];
  const double r = 1.0 / __builtin_sqrt(tot / (double)H + eps);
  for (int c = tid; c < nch; c += 256) yr[c] = norm_chunk(xr[c], gr[c], r);
}

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, int64_t T, int H, float eps, uint16_t* y,
                          hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)T), block(256);
  const int per = (H / 8 + 255) / 256;         // chunks per thread
  if (per <= 1) hipLaunchKernelGGL(rmsnorm_kernel<1>, grid, block, 0, st, x, gamma, T, H, (double)eps, y);
  else if (per <= 2) hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, block, 0, st, x, gamma, T, H, (double)eps, y);
  else if (per <= 4) hipLaunchKernelGGL(rmsnorm_kernel<4>, grid, block, 0, st, x, gamma, T, H, (double)eps, y);
  else if (per <= 8) hipLaunchKernelGGL(rmsnorm_kernel<8>, grid, block, 0, st, x, gamma, T, H, (double)eps, y);
  else hipLaunchKernelGGL(rmsnorm_long_kernel, grid, block, 0, st, x, gamma, T, H, (double)eps, y);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) bias_update_kernel(const int32_t* __restrict__ offsets, int E, float eta,
                                                          float* __restrict__ bias) {
#pragma clang fp contract(off)
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const double avg = (double)offsets[E] / (double)E;
  const double load = (double)(offsets[e + 1] - offsets[e]);
  const double step = (double)eta * (load - avg);
  bias[e] = (float)((double)bias[e] - step);
}

hipError_t launch_bias_update(const int32_t* offsets, int E, float eta, float* bias, hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, st, offsets, E, eta, bias);
  return hipGetLastError();
}

}  // namespace moe
