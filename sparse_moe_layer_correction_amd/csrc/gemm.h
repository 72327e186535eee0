// bf16 MFMA GEMM for gfx950: C[m, n] = epi( sum_s sum_k A_s[row(m), k] * B_s[n, k] ).
//
// One kernel serves every matrix product of the layer:
//  * dense products (fc1, shared up, fc2 + shared down, router), and
//  * grouped per-expert products over the permuted rows (expert up / down),
//    where a device-side tile table maps each M tile to an expert, the A rows
//    may be gathered through an index table (dispatch fused into the load) and
//    B is the expert's own [N, K] weight.
// Up to three K segments accumulate into one fp32 accumulator, so
// out = y_lat.W_fc2^T + hs.W_sd^T is one product with K = L + Is, and the
// router's three bf16 weight parts sum into one logit.
//
// Tiling: BM x BN x 64 per workgroup of 64*WM*WN threads (WM x WN wave
// grid), v_mfma_f32_32x32x16_bf16 tiles, both operands staged through LDS
// (double buffered, XOR-swizzled 16-byte chunks so MFMA fragment reads are
// bank-conflict free), global loads for tile k+1 in flight while tile k is
// multiplied. The MFMA takes the B fragment as its first operand so that each
// lane ends up owning 4 consecutive output columns of one output row.
#pragma once

#include "common.h"

namespace moe {

enum Epilogue : int { EPI_BF16 = 0, EPI_RELU2_BF16 = 1, EPI_F32 = 2 };

struct KSeg {
  const uint16_t* A;   // [rows, lda] bf16
  const uint16_t* B;   // [N, ldb] bf16 (expert 0's matrix in grouped mode)
  int64_t lda, ldb;
  int K;               // multiple of 64
};

struct GemmProblem {
  KSeg seg[3];
  int nseg;
  int M;                     // dense: rows of C
  int N;                     // columns of C that are stored (multiple of 4)
  int Nb;                    // valid B rows (columns >= Nb reuse row Nb-1, results unused)
  const int32_t* gather;     // nullable: A row of output row r is gather[r]
  const int32_t* tile_e;     // nullable: grouped mode tile table (expert of M tile)
  const int32_t* tile_m0;    //   first permuted row of M tile
  const int32_t* n_mtiles;   //   device scalar: number of valid M tiles
  const int32_t* offsets;    //   [E+1] expert row offsets
  int64_t b_estride;         //   elements between consecutive experts' B
  void* C;
  int64_t ldc;
  int epi;
  int mtiles;                // M tiles in the grid (an upper bound in grouped mode)
  int ntiles;                // ceil(N / BN)
  int group_m;               // M tiles per raster group
};

struct GemmLaunch {
  GemmProblem p[2];
  int np;
  int tiles0;                // tiles of problem 0 (mtiles * ntiles)
};

// Workgroup i runs on XCD i % 8. Renumber so that each XCD walks a contiguous
// range of logical tiles: neighbours in the raster order then share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  constexpr int NX = 8;
  const int q = nwg / NX, r = nwg % NX;
  const int x = bid % NX, local = bid / NX;
  return (x < r) ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

// Grouped raster: group_m M tiles at a time, M fastest inside a group.
__device__ __forceinline__ void tile_order(int t, int mtiles, int ntiles, int gm_, int& mt, int& nt) {
  const int per_group = gm_ * ntiles;
  const int g = t / per_group;
  const int rem = t - g * per_group;
  const int m_first = g * gm_;
  const int gm = min(gm_, mtiles - m_first);
  mt = m_first + rem % gm;
  nt = rem / gm;
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) gemm_bf16_kernel(const GemmLaunch L) {
  constexpr int NT = 64 * WM * WN;                 // threads
  constexpr int RS = NT / 8;                       // rows covered by one pass of 16-byte loads
  constexpr int WTM = BM / WM, WTN = BN / WN;      // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;      // MFMA tiles per wave
  constexpr int AR = BM / RS, BR = BN / RS;        // 16-byte chunks per thread per k tile
  static_assert(TM >= 1 && TN >= 1 && AR >= 1 && BR >= 1 && BM % RS == 0 && BN % RS == 0, "tile shape");
  __shared__ u32x4 smem[2][(BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_m = wave % WM, wave_n = wave / WM;

  int bid = xcd_remap(blockIdx.x, gridDim.x);
  int pi = 0;
  if (L.np > 1 && bid >= L.tiles0) { pi = 1; bid -= L.tiles0; }
  const GemmProblem& P = L.p[pi];
  int mt, nt;
  tile_order(bid, P.mtiles, P.ntiles, P.group_m, mt, nt);

  int m0, mend;
  int64_t b_base = 0;
  if (P.tile_e != nullptr) {
    if (mt >= *P.n_mtiles) return;
    const int e = P.tile_e[mt];
    m0 = P.tile_m0[mt];
    mend = P.offsets[e + 1];
    b_base = (int64_t)e * P.b_estride;
  } else {
    m0 = mt * BM;
    mend = P.M;
  }
  const int n0 = nt * BN;

  const int c = tid & 7, r0 = tid >> 3;
  int64_t arow[AR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    const int m = min(m0 + r0 + RS * i, mend - 1);
    arow[i] = P.gather ? (int64_t)P.gather[m] : (int64_t)m;
  }
  int brow[BR];
#pragma unroll
  for (int i = 0; i < BR; ++i) brow[i] = min(n0 + r0 + RS * i, P.Nb - 1);

  f32x16 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.f;

  u32x4 ra[AR], rb[BR];
  const u32x4* ap[AR];
  const u32x4* bp[BR];

  for (int s = 0; s < P.nseg; ++s) {
    const KSeg S = P.seg[s];
#pragma unroll
    for (int i = 0; i < AR; ++i) ap[i] = reinterpret_cast<const u32x4*>(S.A + arow[i] * S.lda + c * 8);
#pragma unroll
    for (int i = 0; i < BR; ++i)
      bp[i] = reinterpret_cast<const u32x4*>(S.B + b_base + (int64_t)brow[i] * S.ldb + c * 8);
    const int nk = S.K / 64;

#pragma unroll
    for (int i = 0; i < AR; ++i) ra[i] = ap[i][0];
#pragma unroll
    for (int i = 0; i < BR; ++i) rb[i] = bp[i][0];
#pragma unroll
    for (int i = 0; i < AR; ++i) {
      const int r = r0 + RS * i;
      smem[0][r * 8 + (c ^ (r & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      const int r = r0 + RS * i;
      smem[0][BM * 8 + r * 8 + (c ^ (r & 7))] = rb[i];
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        // a k tile is 64 bf16 = 8 chunks of 16 bytes
#pragma unroll
        for (int i = 0; i < AR; ++i) ra[i] = ap[i][(kt + 1) * 8];
#pragma unroll
        for (int i = 0; i < BR; ++i) rb[i] = bp[i][(kt + 1) * 8];
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int ch = ks * 2 + (lane >> 5);
        bf16x8 af[TM], bf[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int r = wave_m * WTM + tm * 32 + (lane & 31);
          af[tm] = __builtin_bit_cast(bf16x8, smem[cur][r * 8 + (ch ^ (r & 7))]);
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int r = wave_n * WTN + tn * 32 + (lane & 31);
          bf[tn] = __builtin_bit_cast(bf16x8, smem[cur][BM * 8 + r * 8 + (ch ^ (r & 7))]);
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
            acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[tn], af[tm], acc[tn][tm], 0, 0, 0);
      }
      if (more) {
#pragma unroll
        for (int i = 0; i < AR; ++i) {
          const int r = r0 + RS * i;
          smem[cur ^ 1][r * 8 + (c ^ (r & 7))] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BR; ++i) {
          const int r = r0 + RS * i;
          smem[cur ^ 1][BM * 8 + r * 8 + (c ^ (r & 7))] = rb[i];
        }
      }
      __syncthreads();
    }
  }

  // Epilogue: lane owns row m = (lane & 31) of each MFMA tile and, for g = 0..3,
  // the four columns 8g + 4*(lane >> 5) + 0..3.
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = m0 + wave_m * WTM + tm * 32 + (lane & 31);
    if (m >= mend) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wave_n * WTN + tn * 32 + 8 * g + 4 * (lane >> 5);
        if (n >= P.N) continue;
        float v0 = acc[tn][tm][4 * g + 0], v1 = acc[tn][tm][4 * g + 1];
        float v2 = acc[tn][tm][4 * g + 2], v3 = acc[tn][tm][4 * g + 3];
        if (P.epi == EPI_F32) {
          f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(P.C) + (int64_t)m * P.ldc + n);
          *dst = f32x4{v0, v1, v2, v3};
        } else {
          if (P.epi == EPI_RELU2_BF16) {
            v0 = relu2(v0); v1 = relu2(v1); v2 = relu2(v2); v3 = relu2(v3);
          }
          u32x2* dst = reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P.C) + (int64_t)m * P.ldc + n);
          *dst = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        }
      }
    }
  }
}

}  // namespace moe
