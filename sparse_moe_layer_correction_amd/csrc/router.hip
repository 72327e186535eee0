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
// section "路由与共享专家"; QA Q5.8). Optionally the choice is first limited to
// the best groups of experts (see topk_kernel).
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

// Max of a 64-bit key over the wave. The keys of one top-K round are distinct
// (the low word holds the expert index), so when a single lane holds the
// largest high word its key is the answer and the second 32-bit reduction over
// the low words can be skipped; it runs only on a tie of the high words.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  const uint32_t vh = (uint32_t)(v >> 32);
  const uint32_t hi = wave_max_u32(vh);
  const uint64_t holders = __ballot(vh == hi);
  uint32_t lo;
  if (__popcll(holders) == 1)
    lo = __builtin_amdgcn_readlane((uint32_t)v, __builtin_amdgcn_readfirstlane(__ffsll((long long)holders) - 1));
  else
    lo = wave_max_u32(vh == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// Top-K of token t by one wavefront from its logit row lrow (plus lrow2, the
// other half of a K split, when not null).
template <int VPL>
__device__ __forceinline__ void topk_token(int t, int lane, const float* lrow, const float* lrow2, int nparts,
                                           int64_t part_off, const float* __restrict__ bias, int E, int K,
                                           float scale, int n_group, int topk_group, int32_t* __restrict__ idx,
                                           float* __restrict__ gate, float* __restrict__ gap) {
  float s[VPL];
  uint64_t key[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = j * 64 + lane;
    s[j] = 0.f;
    key[j] = 0;
    if (e < E) {
      // a half's logit is the sum of its nparts column blocks (stacked weight parts), in order
      float l = lrow[e];
      for (int p = 1; p < nparts; ++p) l += lrow[p * part_off + e];
      if (lrow2) {
        float l2 = lrow2[e];
        for (int p = 1; p < nparts; ++p) l2 += lrow2[p * part_off + e];
        l += l2;
      }
      const float sv = 1.0f / (1.0f + expf(-l));
      const float cv = sv + bias[e];
      s[j] = sv;
      key[j] = ((uint64_t)f32_order_key(cv) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }

  // Group-limited selection (walkthrough "路由与共享专家": top-K within
  // groups; the DeepSeek-V3 rule of the parent class, QA Q9.2): group g is
  // experts [g*G, (g+1)*G); its score is the sum of its two highest choice
  // scores. Lane g keeps group g's score; topk_group rounds of a wave arg-max
  // over (score, lower group first) admit groups, and the experts of the other
  // groups drop out of the choice (key 0 never wins).
  float ggap = __builtin_inff();
  int admitted = E;
  if (n_group > 1) {
    const int G = E / n_group;
    uint64_t gkey = 0;
    for (int g = 0; g < n_group; ++g) {
      uint64_t b1 = 0;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int e = j * 64 + lane;
        if (e < E && e / G == g && key[j] > b1) b1 = key[j];
      }
      b1 = wave_max_u64(b1);
      float gs = f32_from_order_key((uint32_t)(b1 >> 32));
      if (G > 1) {
        uint64_t b2 = 0;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int e = j * 64 + lane;
          if (e < E && e / G == g && key[j] != b1 && key[j] > b2) b2 = key[j];
        }
        b2 = wave_max_u64(b2);
        gs += f32_from_order_key((uint32_t)(b2 >> 32));
      }
      if (lane == g) gkey = ((uint64_t)f32_order_key(gs) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)g);
    }
    uint64_t allowed = 0, glast = 0;
    for (int r = 0; r < topk_group; ++r) {
      const uint64_t best = wave_max_u64(gkey);
      glast = best;
      const int g = (int)(0xFFFFFFFFu - (uint32_t)best);
      allowed |= 1ull << g;
      if (lane == g) gkey = 0;
    }
    if (topk_group < n_group) {
      const uint64_t next = wave_max_u64(gkey);
      ggap = f32_from_order_key((uint32_t)(glast >> 32)) - f32_from_order_key((uint32_t)(next >> 32));
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = j * 64 + lane;
      if (e < E && !((allowed >> (e / G)) & 1ull)) key[j] = 0;
    }
    admitted = topk_group * G;
  }

  // Each lane sorts its keys in descending order once (a compare-exchange
  // network with no dependence between the pairs of a pass), so the lane's
  // candidate in a round is the head of its list, and a lane whose head wins
  // shifts the list by one. A round is then one wave-wide max instead of a
  // serial scan of the lane's keys followed by it.
  uint64_t q[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) q[j] = key[j];
#pragma unroll
  for (int pass = 0; pass < VPL; ++pass) {
#pragma unroll
    for (int j = pass & 1; j + 1 < VPL; j += 2) {
      const uint64_t a = q[j], b = q[j + 1];
      q[j] = a > b ? a : b;
      q[j + 1] = a > b ? b : a;
    }
  }

  uint32_t taken = 0;
  uint64_t kth = 0;
  for (int k = 0; k < K; ++k) {
    const uint64_t best = wave_max_key(q[0]);
    kth = best;
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    if (q[0] == best) {
      taken |= 1u << (e >> 6);
#pragma unroll
      for (int j = 0; j + 1 < VPL; ++j) q[j] = q[j + 1];
      q[VPL - 1] = 0;
    }
  }

  float gapv = __builtin_inff();
  if (K < admitted) {
    const uint64_t best = wave_max_key(q[0]);
    gapv = f32_from_order_key((uint32_t)(kth >> 32)) - f32_from_order_key((uint32_t)(best >> 32));
  }
  gapv = fminf(gapv, ggap);

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

template <int VPL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ logits2, int64_t ldl,
                                                   int nparts, int64_t part_off,
                                                   const float* __restrict__ bias, int T, int E, int K,
                                                   float scale, int n_group, int topk_group,
                                                   int32_t* __restrict__ idx, float* __restrict__ gate,
                                                   float* __restrict__ gap) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token<VPL>(t, threadIdx.x & 63, logits + (int64_t)t * ldl, logits2 ? logits2 + (int64_t)t * ldl : nullptr,
                  nparts, part_off, bias, E, K, scale, n_group, topk_group, idx, gate, gap);
}

// A few-token forward's router product leaves fp32 partial logits of ksplit
// k ranges, [ksplit, T, ldl] (ldl a multiple of 64). One workgroup per token
// sums its row into LDS and wave 0 takes the top-K from there: one launch
// instead of a reduction pass and a top-K. A thread holds 4 experts; the
// threads that cover the row form a team, and the teams sum consecutive
// ranges of splits side by side (each split row read whole by a wave: 1 KB
// per load, 8 loads in flight), after which the team sums are added in team
// order. The order is fixed, so the logits do not change from call to call.
constexpr int kPartThreads = 512;

template <int VPL>
__global__ void __launch_bounds__(kPartThreads) topk_partials_kernel(const float* __restrict__ partial, int ksplit,
                                                                     int T, int64_t ldl,
                                                                     const float* __restrict__ bias, int E, int K,
                                                                     float scale, int n_group, int topk_group,
                                                                     int32_t* __restrict__ idx,
                                                                     float* __restrict__ gate,
                                                                     float* __restrict__ gap) {
  __shared__ float lg[64 * VPL];
  __shared__ f32x4 team_sum[kPartThreads];
  const int t = blockIdx.x;
  const int64_t stride = (int64_t)T * ldl;
  const int nq = (E + 3) >> 2;                       // 4-expert groups of the row
  const int span = (nq + 63) & ~63;                  // a team: whole waves, <= 256 threads (E <= 1024)
  const int teams = kPartThreads / span;             // 2, 4 or 8
  const int team = threadIdx.x / span, q = threadIdx.x % span;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  if (q < nq) {
    const int k0 = (int)((int64_t)ksplit * team / teams), k1 = (int)((int64_t)ksplit * (team + 1) / teams);
    const float* pq = partial + (int64_t)t * ldl + q * 4;
    int k = k0;
    for (; k + 8 <= k1; k += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(pq + (int64_t)(k + u) * stride);
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; k < k1; ++k) s += *reinterpret_cast<const f32x4*>(pq + (int64_t)k * stride);
  }
  team_sum[threadIdx.x] = s;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPartThreads) {
    float v = team_sum[e >> 2][e & 3];
    for (int m = 1; m < teams; ++m) v += team_sum[m * span + (e >> 2)][e & 3];
    lg[e] = v;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  topk_token<VPL>(t, threadIdx.x, lg, nullptr, 1, 0, bias, E, K, scale, n_group, topk_group, idx, gate, gap);
}

hipError_t launch_split_router_weight(const float* w, int E, int H, uint16_t* parts, hipStream_t st) {
  const int64_t n = (int64_t)E * H;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(split_router_weight_kernel, dim3(blocks), dim3(256), 0, st, w, n, parts);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* logits2, int64_t ldl, int nparts, int64_t part_off,
                       const float* bias, int T, int E, int K,
                       float scale, int n_group, int topk_group, int32_t* idx, float* gate, float* gap,
                       hipStream_t st) {
  const dim3 grid((T + 3) / 4), block(256);
  const int vpl = (E + 63) / 64;
#define MOE_TOPK(V)                                                                                           \
  hipLaunchKernelGGL(topk_kernel<V>, grid, block, 0, st, logits, logits2, ldl, nparts, part_off, bias, T, E, K, scale, n_group,   \
                     topk_group, idx, gate, gap)
  if (vpl <= 1) MOE_TOPK(1);
  else if (vpl <= 2) MOE_TOPK(2);
  else if (vpl <= 4) MOE_TOPK(4);
  else if (vpl <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

hipError_t launch_topk_partials(const float* partial, int ksplit, int T, int64_t ldl, const float* bias, int E, int K,
                                float scale, int n_group, int topk_group, int32_t* idx, float* gate, float* gap,
                                hipStream_t st) {
  const int vpl = (E + 63) / 64;
#define MOE_TOPK(V)                                                                                            \
  hipLaunchKernelGGL(topk_partials_kernel<V>, dim3(T), dim3(kPartThreads), 0, st, partial, ksplit, T, ldl, bias, E, K, scale, \
                     n_group, topk_group, idx, gate, gap)
  if (vpl <= 1) MOE_TOPK(1);
  else if (vpl <= 2) MOE_TOPK(2);
  else if (vpl <= 4) MOE_TOPK(4);
  else if (vpl <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
