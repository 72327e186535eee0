// Gate-weighted combine on gfx950: y_lat[t] = sum_k gate[t,k] * y[slot_row[t,k]].
//
// Each expert's output row is multiplied by its token's gate and the K rows are
// summed in the latent space, before fc2 ("Nemotron 3 Ultra 架构 QA", Q5.5
// point 3 and Q5.1). Written as a gather: one wavefront per token and 512
// columns reads its K permuted rows (16 bytes per lane, consecutive lanes on
// consecutive columns) and sums them in fp32 in slot order, so the result is
// deterministic without atomics. The sum is rounded once to bf16.
#include "kernels.h"

namespace moe {

__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ y, const float* __restrict__ gate,
                                                      const int32_t* __restrict__ slot_row, int T, int K, int L,
                                                      uint16_t* __restrict__ y_lat) {
  // one wavefront per (token, 512-column chunk): few tokens still spread over
  // several waves, and each wave keeps up to 8 rows in flight
  const int lane = threadIdx.x & 63;
  const int nchunk = (L + 511) / 512;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)T * nchunk) return;
  const int t = (int)(w / nchunk);
  const int cb = (int)(w % nchunk) * 512;
  // lane k < K holds slot k's row and gate (K <= 64)
  const int my_row = lane < K ? slot_row[(int64_t)t * K + lane] : 0;
  const float my_g = lane < K ? gate[(int64_t)t * K + lane] : 0.f;

  // every lane runs every iteration; only the loads' columns and the store are
  // guarded when L is not a multiple of 512
  const int c0 = cb + lane * 8;
  const bool act = c0 < L;
  const int64_t col = act ? c0 : 0;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  auto add = [&](const u32x4& v, float g) {
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += g * bf16_bits_to_f32(wv[q] & 0xFFFFu);
      acc[2 * q + 1] += g * bf16_bits_to_f32(wv[q] >> 16);
    }
  };
  // slots in batches of 8 loads in flight (the last batch guarded by a
  // uniform test, so K = 22 is 3 round trips, not 2 plus 6 single loads); a
  // slot's row and gate are read from its lane with readlane (no LDS trip)
  for (int k = 0; k < K; k += 8) {
    u32x4 v[8];
    float g[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k + u < K) {
        const int r = __builtin_amdgcn_readlane(my_row, k + u);
        g[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_g), k + u));
        v[u] = *reinterpret_cast<const u32x4*>(y + (int64_t)r * L + col);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k + u < K) add(v[u], g[u]);     // slot order
  }
  if (act) {
    const u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                     pack_bf16x2(acc[6], acc[7])};
    *reinterpret_cast<u32x4*>(y_lat + (int64_t)t * L + c0) = o;
  }
}

hipError_t launch_combine(const uint16_t* y, const float* gate, const int32_t* slot_row, int T, int K, int L,
                          uint16_t* y_lat, hipStream_t st) {
  const int64_t waves = (int64_t)T * ((L + 511) / 512);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, y, gate, slot_row, T, K, L,
                     y_lat);
  return hipGetLastError();
}

}  // namespace moe
