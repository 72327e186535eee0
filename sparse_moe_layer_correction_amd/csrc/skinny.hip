// Weight-streaming products for few rows (decode): C[m, n] = epi(sum_s A_s[row(m)] . B_s[n]).
//
// With a handful of rows per product (a decode batch, or the few tokens an
// expert receives from it) the work is bound by reading the [N, K] weights
// from HBM once. Each wavefront owns a slab of 16 output columns and streams
// its 16 weight rows straight from global memory into MFMA operand registers
// (16 bytes per lane per load; no LDS and no barriers), so many independent
// waves per CU keep enough bytes in flight. The rows' activations are loaded
// the same way; they are few and stay in the caches.
//
// v_mfma_f32_16x16x32_bf16 takes the weight fragment as first operand: lane l
// ends up with output row m = l % 16 of its m-tile and the four columns
// n0 + 4*(l / 16) + 0..3.
//
// Dense products (fc1 / shared up, fc2 + shared down, router) split K over
// KSPLIT waves per column block; each writes its fp32 partial and skinny_reduce sums
// the partials in a fixed order and applies the epilogue, so results do not
// depend on timing. Grouped products (experts) need no split: a slab of one
// expert covers its rows, and there are E x N/16 slabs.
#include "kernels.h"

namespace moe {

typedef float f32x4v __attribute__((ext_vector_type(4)));

int skinny_slabs_per_wave(const SkinnyProblem& P) { return (P.offsets == nullptr && P.M > 16) ? 4 : 1; }

// MT m-tiles of 16 rows and NS slabs of 16 columns per wave: per 32-deep k step
// the wave loads NS weight fragments and MT activation fragments and issues
// MT*NS MFMAs, so the activations are read once per NS weight fragments.
template <int MT, int NS, int UNROLL>
__device__ __forceinline__ void skinny_tile(const SkinnyProblem& P, int n_first, int rows, int row0,
                                            const int32_t* gather, int64_t b_base, int k_begin, int k_end,
                                            int out_row0, float* partial, int lane, int epi) {
  // rows of the MT m-tiles this lane loads (clamped: padding lanes re-read a valid row)
  int64_t arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = min(t * 16 + (lane & 15), rows - 1);
    arow[t] = gather ? (int64_t)gather[row0 + m] : (int64_t)(row0 + m);
  }
  int nrow[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) nrow[j] = min(n_first + j * 16 + (lane & 15), P.Nb - 1);
  const int kl = (lane >> 4) * 8;          // this lane's 8 k values within a 32-wide step
  f32x4v acc[NS][MT];
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = f32x4v{0.f, 0.f, 0.f, 0.f};

  // walk the K segments; k indices are global over the concatenated segments
  int seg_k0 = 0;
  for (int s = 0; s < P.nseg; ++s) {
    const KSeg& S = P.seg[s];
    const int lo = max(k_begin, seg_k0), hi = min(k_end, seg_k0 + S.K);
    if (lo < hi) {
      const uint16_t* bp[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) bp[j] = S.B + b_base + (int64_t)nrow[j] * S.ldb + (lo - seg_k0) + kl;
      const uint16_t* ap[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) ap[t] = S.A + arow[t] * S.lda + (lo - seg_k0) + kl;
      const int nsteps = (hi - lo) / 32;
      int st = 0;
      for (; st + UNROLL <= nsteps; st += UNROLL) {
        u32x4 bv[UNROLL][NS], av[UNROLL][MT];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
          for (int j = 0; j < NS; ++j) bv[u][j] = *reinterpret_cast<const u32x4*>(bp[j] + (st + u) * 32);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
          for (int t = 0; t < MT; ++t) av[u][t] = *reinterpret_cast<const u32x4*>(ap[t] + (st + u) * 32);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
          for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int t = 0; t < MT; ++t)
              acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bv[u][j]),
                                                                  __builtin_bit_cast(bf16x8, av[u][t]), acc[j][t], 0, 0,
                                                                  0);
      }
      for (; st < nsteps; ++st) {
        u32x4 bv[NS], av[MT];
#pragma unroll
        for (int j = 0; j < NS; ++j) bv[j] = *reinterpret_cast<const u32x4*>(bp[j] + st * 32);
#pragma unroll
        for (int t = 0; t < MT; ++t) av[t] = *reinterpret_cast<const u32x4*>(ap[t] + st * 32);
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int t = 0; t < MT; ++t)
            acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bv[j]),
                                                                __builtin_bit_cast(bf16x8, av[t]), acc[j][t], 0, 0, 0);
      }
    }
    seg_k0 += S.K;
  }

#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int n = n_first + j * 16 + (lane >> 4) * 4;
    if (n >= P.N) continue;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + (lane & 15);
      if (m >= rows) continue;
      f32x4v v = acc[j][t];
      if (partial != nullptr) {
        *reinterpret_cast<f32x4v*>(partial + (int64_t)(out_row0 + m) * P.N + n) = v;
      } else if (epi == EPI_F32) {
        *reinterpret_cast<f32x4v*>(static_cast<float*>(P.C) + (int64_t)(out_row0 + m) * P.ldc + n) = v;
      } else {
        if (epi == EPI_RELU2_BF16) {
          v[0] = relu2(v[0]); v[1] = relu2(v[1]); v[2] = relu2(v[2]); v[3] = relu2(v[3]);
        }
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P.C) + (int64_t)(out_row0 + m) * P.ldc + n) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

// One wavefront per (group, column block, k split); 4 waves per workgroup. A
// column block is NSB slabs of 16 columns.
// GROUPED_EPI: -1 for dense products (epilogue from the problem), else the
// fixed epilogue of a grouped expert product (which also names up and down
// apart in profiles).
template <int NSB, int GROUPED_EPI>
__global__ void __launch_bounds__(256) skinny_kernel(const SkinnyProblem P) {
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nblocks = (P.N + 16 * NSB - 1) / (16 * NSB);
  const int64_t per_group = (int64_t)nblocks * P.ksplit;
  const int gi = (int)(task / per_group);
  if (gi >= P.groups) return;
  const int rem = (int)(task - (int64_t)gi * per_group);
  const int blk = rem / P.ksplit, ks = rem % P.ksplit;

  int row0 = 0, rows = P.M;
  int64_t b_base = 0;
  if (P.offsets != nullptr) {            // grouped: the gi-th expert with tokens
    if (gi >= *P.n_groups) return;
    const int g = P.group_list[gi];
    row0 = P.offsets[g];
    rows = P.offsets[g + 1] - row0;
    b_base = (int64_t)g * P.b_estride;
  }
  if (rows <= 0) return;

  int ktot = 0;
  for (int s = 0; s < P.nseg; ++s) ktot += P.seg[s].K;
  const int ksteps = ktot / 32;
  const int k_begin = (int)((int64_t)ksteps * ks / P.ksplit) * 32;
  const int k_end = (int)((int64_t)ksteps * (ks + 1) / P.ksplit) * 32;
  float* partial = P.partial ? P.partial + (int64_t)ks * P.M * P.N : nullptr;
  const int n_first = blk * 16 * NSB;
  const int epi = GROUPED_EPI >= 0 ? GROUPED_EPI : P.epi;

  // up to 64 rows in registers per pass; more rows take further passes
  for (int r0 = 0; r0 < rows; r0 += 64) {
    const int rr = min(64, rows - r0);
    if (rr <= 16)
      skinny_tile<1, NSB, 8 / NSB>(P, n_first, rr, row0 + r0, P.gather, b_base, k_begin, k_end, row0 + r0, partial,
                                    lane, epi);
    else if (rr <= 32)
      skinny_tile<2, NSB, (4 / NSB > 0 ? 4 / NSB : 1)>(P, n_first, rr, row0 + r0, P.gather, b_base, k_begin, k_end,
                                                        row0 + r0, partial, lane, epi);
    else
      skinny_tile<4, NSB, (2 / NSB > 0 ? 2 / NSB : 1)>(P, n_first, rr, row0 + r0, P.gather, b_base, k_begin, k_end,
                                                        row0 + r0, partial, lane, epi);
  }
}

// out[m, n] = epi(sum_{s < ksplit} partial[s, m, n]), summed in split order.
__global__ void __launch_bounds__(256) skinny_reduce_kernel(const float* __restrict__ partial, int ksplit, int M, int N,
                                                            void* C, int64_t ldc, int epi) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const int64_t total = (int64_t)M * N;
  if (i >= total) return;
  f32x4v s = *reinterpret_cast<const f32x4v*>(partial + i);
  for (int k = 1; k < ksplit; ++k) s += *reinterpret_cast<const f32x4v*>(partial + (int64_t)k * total + i);
  const int m = (int)(i / N), n = (int)(i % N);
  if (epi == EPI_F32) {
    *reinterpret_cast<f32x4v*>(static_cast<float*>(C) + (int64_t)m * ldc + n) = s;
  } else {
    if (epi == EPI_RELU2_BF16) {
      s[0] = relu2(s[0]); s[1] = relu2(s[1]); s[2] = relu2(s[2]); s[3] = relu2(s[3]);
    }
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + (int64_t)m * ldc + n) =
        u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  }
}

hipError_t launch_skinny(const SkinnyProblem& P, hipStream_t st) {
  // dense products carry up to 64 rows: 4 slabs per wave load the rows once per
  // four weight fragments; grouped products have a few rows per expert
  const int nsb = skinny_slabs_per_wave(P);
  const int64_t nblocks = (P.N + 16 * nsb - 1) / (16 * nsb);
  const int64_t tasks = (int64_t)P.groups * nblocks * P.ksplit;
  if (tasks <= 0) return hipSuccess;
  const dim3 grid((unsigned)((tasks + 3) / 4)), block(256);
  if (nsb == 4) hipLaunchKernelGGL((skinny_kernel<4, -1>), grid, block, 0, st, P);
  else if (P.offsets == nullptr) hipLaunchKernelGGL((skinny_kernel<1, -1>), grid, block, 0, st, P);
  else if (P.epi == EPI_RELU2_BF16) hipLaunchKernelGGL((skinny_kernel<1, EPI_RELU2_BF16>), grid, block, 0, st, P);
  else hipLaunchKernelGGL((skinny_kernel<1, EPI_BF16>), grid, block, 0, st, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.partial == nullptr) return e;
  const int64_t total = (int64_t)P.M * P.N;
  hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)((total / 4 + 255) / 256)), dim3(256), 0, st, P.partial,
                     P.ksplit, P.M, P.N, P.C, P.ldc, P.epi);
  return hipGetLastError();
}

}  // namespace moe
