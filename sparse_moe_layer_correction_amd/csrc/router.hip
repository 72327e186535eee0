// Router of the LatentMoE layer on gfx950.
//
// Logits are fp32 dot products of the bf16 input row with the fp32 router
// weight ("Nemotron 3 Ultra 架构 QA", Q5.2: both operands cast to fp32). The
// weight is split exactly-enough into three bf16 parts w = w0 + w1 + w2 (each
// part takes the next 8 significant bits), so every bf16 x bf16 product is
// exact in fp32 and the logit becomes one bf16 MFMA product with three K
// segments accumulated in fp32 (see gemm.h). The residual after three parts is
// below 2**-24 of |w|, inside fp32 rounding of the weight itself.
//
// Then, per token, one wavefront: sigmoid scores, choice = score + bias (Q5.2,
// Q5.3), K rounds of a wave-wide arg-max over 64-bit keys (choice order key,
// then the complement of the expert index, so equal choices go to the lower
// index), a ballot-based rank that lists the chosen experts in ascending index,
// and gates = routed_scaling * s / sum(s) over the chosen set (walkthrough
// section "路由与共享专家"; QA Q5.8).
#include "kernels.h"

namespace moe {

__global__ void split_router_weight_kernel(const float* __restrict__ w, int64_t n,
                                           uint16_t* __restrict__ parts) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    const float v = w[i];
    const uint32_t b0 = f32_to_bf16_bits(v);
    const float r1 = v - bf16_bits_to_f32(b0);         // exact
    const uint32_t b1 = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(b1);        // exact
    const uint32_t b2 = f32_to_bf16_bits(r2);
    parts[i] = (uint16_t)b0;
    parts[n + i] = (uint16_t)b1;
    parts[2 * n + i] = (uint16_t)b2;
  }
}

template <int VPL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int64_t ldl,
                                                   const float* __restrict__ bias, int T, int E, int K,
                                                   float scale, int32_t* __restrict__ idx,
                                                   float* __restrict__ gate, float* __restrict__ gap) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;

  float s[VPL];
  uint64_t key[VPL];
  const float* lrow = logits + (int64_t)t * ldl;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = j * 64 + lane;
    s[j] = 0.f;
    key[j] = 0;
    if (e < E) {
      const float l = lrow[e];
      const float sv = 1.0f / (1.0f + expf(-l));
      const float cv = sv + bias[e];
      s[j] = sv;
      key[j] = ((uint64_t)f32_order_key(cv) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }

  uint32_t taken = 0;
  uint64_t kth = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (!((taken >> j) & 1u) && key[j] > best) best = key[j];
    best = wave_max_u64(best);
    kth = best;
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    if ((e & 63) == lane) taken |= 1u << (e >> 6);
  }

  float gapv = __builtin_inff();
  if (K < E) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (!((taken >> j) & 1u) && key[j] > best) best = key[j];
    best = wave_max_u64(best);
    gapv = f32_from_order_key((uint32_t)(kth >> 32)) - f32_from_order_key((uint32_t)(best >> 32));
  }

  float ssum = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j)
    if ((taken >> j) & 1u) ssum += s[j];
  ssum = wave_sum_f32(ssum);

  int before = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const bool mine = (taken >> j) & 1u;
    const uint64_t m = __ballot(mine);
    if (mine) {
      const int rank = before + __popcll(m & below);
      idx[(int64_t)t * K + rank] = j * 64 + lane;
      gate[(int64_t)t * K + rank] = scale * s[j] / ssum;
    }
    before += __popcll(m);
  }
  if (gap != nullptr && lane == 0) gap[t] = gapv;
}

hipError_t launch_split_router_weight(const float* w, int E, int H, uint16_t* parts, hipStream_t st) {
  const int64_t n = (int64_t)E * H;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(split_router_weight_kernel, dim3(blocks), dim3(256), 0, st, w, n, parts);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t ldl, const float* bias, int T, int E, int K,
                       float scale, int32_t* idx, float* gate, float* gap, hipStream_t st) {
  const dim3 grid((T + 3) / 4), block(256);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1) hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, st, logits, ldl, bias, T, E, K, scale, idx, gate, gap);
  else if (vpl <= 2) hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, st, logits, ldl, bias, T, E, K, scale, idx, gate, gap);
  else if (vpl <= 4) hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, st, logits, ldl, bias, T, E, K, scale, idx, gate, gap);
  else if (vpl <= 8) hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, st, logits, ldl, bias, T, E, K, scale, idx, gate, gap);
  else hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, st, logits, ldl, bias, T, E, K, scale, idx, gate, gap);
  return hipGetLastError();
}

}  // namespace moe
