// Token -> expert permutation on gfx950: histogram, prefix scan, stable scatter.
//
// The rows of one expert are laid out contiguously, tokens ascending -- the
// row set that a loop over the hit experts gathers ("Nemotron 3 Ultra 架构 QA",
// Q5.6 point 3). Everything is exact integer work and deterministic:
//  1. block_masks: tokens in blocks of 64; per block and expert a 64-bit mask of
//     the tokens that chose the expert, built with LDS atomic OR (the result
//     does not depend on the order of the ORs). Stored expert-major.
//  2. expert_scan: one wavefront per expert scans its per-block popcounts.
//  3. offsets: one workgroup scans the expert counts into offsets[E+1] and lays
//     out the M-tile table of the grouped expert products.
//  4. scatter: slot (t,k) of expert e goes to row
//       offsets[e] + base[e][t/64] + popcount(mask[e][t/64] below bit t%64).
//  5. gather: dst[r] = src[row_token[r]] with 16-byte loads and stores (rows
//     past offsets[E] -- slots of skipped entries -- are zero).
// With at most 64 tokens, steps 1-4 run as one workgroup (permute_small_kernel).
#include "kernels.h"

namespace moe {

__global__ void __launch_bounds__(256) block_masks_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                          int E, int nblk, uint64_t* __restrict__ masks) {
  __shared__ unsigned long long m[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) m[e] = 0ull;
  __syncthreads();
  const int t0 = blockIdx.x * 64;
  const int nt = min(64, T - t0);
  const int64_t base = (int64_t)t0 * K;
  for (int s = threadIdx.x; s < nt * K; s += blockDim.x) {
    const int e = idx[base + s];
    if (e >= 0 && e < E) atomicOr(&m[e], 1ull << (s / K));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) masks[(int64_t)e * nblk + blockIdx.x] = m[e];
}

__global__ void __launch_bounds__(256) expert_scan_kernel(const uint64_t* __restrict__ masks, int nblk,
                                                          int E, int32_t* __restrict__ base,
                                                          int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  int running = 0;
  for (int b0 = 0; b0 < nblk; b0 += 64) {
    const int b = b0 + lane;
    const int c = b < nblk ? __popcll(masks[(int64_t)e * nblk + b]) : 0;
    const int inc = wave_inclusive_scan_i32(c);
    if (b < nblk) base[(int64_t)e * nblk + b] = running + inc - c;
    running += __shfl(inc, 63, 64);
  }
  if (lane == 0) counts[e] = running;
}

// Expert offsets and the grouped products' M-tile table from the per-expert
// count c of thread tid (one workgroup of 1024 threads, E <= 1024). Also lists
// the experts that received at least one token, in ascending order. Returns
// the exclusive offset of expert tid.
__device__ __forceinline__ int layout_experts(int c, int E, int BM, int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ tile_info,
                                              int32_t* __restrict__ n_mtiles, int32_t* __restrict__ touched,
                                              int32_t* __restrict__ n_touched, int32_t* __restrict__ gemm_ctr) {
  __shared__ int wsum_c[16], wsum_t[16], wsum_h[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nt = (c + BM - 1) / BM;
  const int hit = c > 0 ? 1 : 0;
  const int ic = wave_inclusive_scan_i32(c);
  const int it = wave_inclusive_scan_i32(nt);
  const int ih = wave_inclusive_scan_i32(hit);
  if (lane == 63) { wsum_c[wave] = ic; wsum_t[wave] = it; wsum_h[wave] = ih; }
  __syncthreads();
  int pc = 0, pt = 0, ph = 0;
  for (int w = 0; w < wave; ++w) { pc += wsum_c[w]; pt += wsum_t[w]; ph += wsum_h[w]; }
  const int ex_c = pc + ic - c, ex_t = pt + it - nt, ex_h = ph + ih - hit;
  if (tid < kGemmCounters) gemm_ctr[tid] = 0;
  if (tid < E) {
    offsets[tid] = ex_c;
    for (int i = 0; i < nt; ++i)
      reinterpret_cast<int4*>(tile_info)[ex_t + i] = make_int4(tid, ex_t, ex_c, ex_c + c);
    if (hit) touched[ex_h] = tid;
  }
  if (tid == E - 1) {
    offsets[E] = ex_c + c;
    *n_mtiles = ex_t + nt;
    *n_touched = ex_h + hit;
  }
  return ex_c;
}

__global__ void __launch_bounds__(1024) offsets_kernel(const int32_t* __restrict__ counts, int E, int BM,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ tile_info,
                                                       int32_t* __restrict__ n_mtiles,
                                                       int32_t* __restrict__ touched,
                                                       int32_t* __restrict__ n_touched,
                                                       int32_t* __restrict__ gemm_ctr) {
  const int c = (int)threadIdx.x < E ? counts[threadIdx.x] : 0;
  layout_experts(c, E, BM, offsets, tile_info, n_mtiles, touched, n_touched, gemm_ctr);
}

// All of steps 1-4 in one workgroup when the tokens fit one 64-token block
// (T <= 64): the masks and offsets stay in LDS, and a few-token forward pays
// one launch instead of four.
__global__ void __launch_bounds__(1024) permute_small_kernel(const int32_t* __restrict__ idx, int T, int K, int E,
                                                             int BM, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ tile_info,
                                                             int32_t* __restrict__ n_mtiles,
                                                             int32_t* __restrict__ touched,
                                                             int32_t* __restrict__ n_touched,
                                                             int32_t* __restrict__ gemm_ctr,
                                                             int32_t* __restrict__ row_token,
                                                             int32_t* __restrict__ slot_row) {
  __shared__ unsigned long long m[kMaxExperts];
  __shared__ int off[kMaxExperts];
  const int tid = threadIdx.x;
  const int tk = T * K;
  for (int e = tid; e < E; e += blockDim.x) m[e] = 0ull;
  __syncthreads();
  for (int s = tid; s < tk; s += blockDim.x) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicOr(&m[e], 1ull << (s / K));
  }
  __syncthreads();
  const int c = tid < E ? __popcll(m[tid]) : 0;
  const int ex = layout_experts(c, E, BM, offsets, tile_info, n_mtiles, touched, n_touched, gemm_ctr);
  if (tid < E) off[tid] = ex;
  __syncthreads();
  for (int s = tid; s < tk; s += blockDim.x) {
    const int t = s / K;
    const int e = idx[s];
    if (e < 0 || e >= E) { slot_row[s] = -1; continue; }
    const uint64_t below = t == 0 ? 0ull : (m[e] & (~0ull >> (64 - t)));
    const int r = off[e] + __popcll(below);
    row_token[r] = t;
    slot_row[s] = r;
  }
}

__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ idx, int T, int K, int E,
                                                      int nblk, const uint64_t* __restrict__ masks,
                                                      const int32_t* __restrict__ base,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ row_token,
                                                      int32_t* __restrict__ slot_row) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= (int64_t)T * K) return;
  const int t = (int)(s / K);
  const int e = idx[s];
  if (e < 0 || e >= E) { slot_row[s] = -1; return; }
  const int blk = t >> 6, tl = t & 63;
  const uint64_t m = masks[(int64_t)e * nblk + blk];
  const uint64_t below = tl == 0 ? 0ull : (m & (~0ull >> (64 - tl)));
  const int r = offsets[e] + base[(int64_t)e * nblk + blk] + __popcll(below);
  row_token[r] = t;
  slot_row[s] = r;
}

// Rows at or past *n_valid (the slots of entries outside [0, E), for which the
// maps leave row_token unwritten) are written as zeros and read nothing.
__global__ void __launch_bounds__(256) gather_rows_kernel(const uint16_t* __restrict__ src, int C,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ n_valid,
                                                          int64_t rows, uint16_t* __restrict__ dst) {
  const int cpr = C / 8;                      // 16-byte chunks per row
  const int64_t n = rows * cpr;
  const int64_t valid = *n_valid;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    const int64_t r = i / cpr;
    const int ch = (int)(i - r * cpr);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (r < valid) v = reinterpret_cast<const u32x4*>(src + (int64_t)row_token[r] * C)[ch];
    reinterpret_cast<u32x4*>(dst + r * C)[ch] = v;
  }
}

hipError_t launch_permute_maps(const int32_t* idx, int T, int K, int E, int BM, const PermuteScratch& ps,
                               int32_t* offsets, int32_t* row_token, int32_t* slot_row, hipStream_t st) {
  const int nblk = (T + 63) / 64;
  if (nblk == 1) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, st, idx, T, K, E, BM, offsets, ps.tile_info,
                       ps.n_mtiles, ps.touched, ps.n_touched, ps.gemm_ctr, row_token, slot_row);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(block_masks_kernel, dim3(nblk), dim3(256), 0, st, idx, T, K, E, nblk, ps.masks);
  hipLaunchKernelGGL(expert_scan_kernel, dim3((E + 3) / 4), dim3(256), 0, st, ps.masks, nblk, E, ps.base, ps.counts);
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(1024), 0, st, ps.counts, E, BM, offsets, ps.tile_info,
                     ps.n_mtiles, ps.touched, ps.n_touched, ps.gemm_ctr);
  const int64_t tk = (int64_t)T * K;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((tk + 255) / 256)), dim3(256), 0, st, idx, T, K, E, nblk,
                     ps.masks, ps.base, offsets, row_token, slot_row);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* src, int C, const int32_t* row_token, const int32_t* n_valid,
                              int64_t rows, uint16_t* dst, hipStream_t st) {
  const int64_t n = rows * (C / 8);
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 65536);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(256), 0, st, src, C, row_token, n_valid, rows, dst);
  return hipGetLastError();
}

}  // namespace moe
