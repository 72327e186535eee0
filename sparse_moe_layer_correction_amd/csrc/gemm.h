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
// Data movement (gfx950):
//  * global -> LDS with global_load_lds_dwordx4 (16 bytes per lane, no VGPR
//    staging) into a ring of STAGES separate LDS arrays, one per stage, so the
//    compiler's alias analysis can tell the stage being read from the stages
//    being filled and does not wait for every DMA in flight;
//  * one k tile is 32 bf16 deep (64 bytes per row = 4 chunks of 16 bytes);
//    chunk c of row r sits in slot c ^ ((r >> 2) & 3): gfx950's LDS serves a
//    ds_read_b128 16 lanes per cycle over 64 banks, and the 16 rows those lanes
//    read then fall into the 16 distinct 16-byte slots of a 256-byte window;
//  * the DMA of each lane is chosen so that the 64 lanes of a wave fill 1 KB
//    of LDS contiguously in that swizzled order (rows stay fully coalesced);
//  * every step waits for its own tile (vmcnt), passes one barrier and issues
//    the tile STAGES-1 ahead into the stage freed by the previous step; past
//    the end it re-reads the last tile, so the wait count never changes.
// The MFMA is v_mfma_f32_32x32x16_bf16 with the B fragment as first operand,
// so each lane owns 4 consecutive output columns of one output row.
#pragma once

#include "common.h"

namespace moe {

enum Epilogue : int { EPI_BF16 = 0, EPI_RELU2_BF16 = 1, EPI_F32 = 2 };

struct KSeg {
  const uint16_t* A;   // [rows, lda] bf16
  const uint16_t* B;   // [N, ldb] bf16 (expert 0's matrix in grouped mode)
  int64_t lda, ldb;
  int K;               // multiple of 32
};

struct GemmProblem {
  KSeg seg[3];
  int nseg;
  int M;                     // dense: rows of C
  int N;                     // columns of C that are stored (multiple of 4)
  int Nb;                    // valid B rows (columns >= Nb reuse row Nb-1, results unused)
  const int32_t* gather;     // nullable: A row of output row r is gather[r]
  const int32_t* tile_e;     // nullable: grouped mode tile table (expert of M tile);
                             //   a grouped launch holds exactly one problem
  const int32_t* tile_m0;    //   first permuted row of M tile
  const int32_t* n_mtiles;   //   device scalar: number of valid M tiles
  const int32_t* first_mtile;  // [E] each expert's first M tile in the table
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

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 3) << 14))

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

template <int V>
struct Stage {
  static constexpr int value = V;
};

// slot of logical chunk c of row r (4 chunks of 16 bytes per 64-byte row)
__device__ __forceinline__ int swz_slot(int r, int c) { return c ^ ((r >> 2) & 3); }

// EPI: an Epilogue fixed at compile time, or -1 to take each problem's own.
template <int BM, int BN, int WM, int WN, int STAGES, int EPI>
__global__ void __launch_bounds__(64 * WM * WN, 1) gemm_bf16_kernel(const GemmLaunch L) {
  static_assert(STAGES >= 2 && STAGES <= 5, "stages");
  constexpr int BK = 32, CPR = 4;
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;      // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;      // MFMA tiles per wave
  constexpr int NA = BM * CPR / (64 * NW);         // A DMA instructions per thread per k tile
  constexpr int NB = BN * CPR / (64 * NW);
  constexpr int PER_TILE = NA + NB;
  constexpr int ACH = BM * CPR, BCH = BN * CPR;    // 16-byte chunks per stage
  static_assert(TM >= 1 && TN >= 1 && NA >= 1 && NB >= 1, "tile shape");
  static_assert(NA * 64 * NW == ACH && NB * 64 * NW == BCH, "DMA coverage");
  __shared__ u32x4 sa0[ACH], sb0[BCH], sa1[ACH], sb1[BCH];
  __shared__ u32x4 sa2[STAGES > 2 ? ACH : 1], sb2[STAGES > 2 ? BCH : 1];
  __shared__ u32x4 sa3[STAGES > 3 ? ACH : 1], sb3[STAGES > 3 ? BCH : 1];
  __shared__ u32x4 sa4[STAGES > 4 ? ACH : 1], sb4[STAGES > 4 ? BCH : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WM, wave_n = wave / WM;

  int mt, nt, pi = 0;
  if (L.p[0].tile_e != nullptr) {
    // grouped: the grid is sized for the most M tiles any routing can need; only
    // the first n_mtiles * ntiles workgroups work, and the XCD renumbering runs
    // over exactly those, so every XCD gets an equal share
    const int mtv = *L.p[0].n_mtiles;
    const int ntl = L.p[0].ntiles;
    const int valid = mtv * ntl;
    if ((int)blockIdx.x >= valid) return;
    // expert by expert: the tiles of one expert are contiguous in the order,
    // M fastest, so the M tiles that share a weight panel run side by side
    const int t = xcd_remap(blockIdx.x, valid);
    const int e = L.p[0].tile_e[t / ntl];
    const int f = L.p[0].first_mtile[e];
    const int ne = (L.p[0].offsets[e + 1] - L.p[0].offsets[e] + BM - 1) / BM;
    const int local = t - f * ntl;
    mt = f + local % ne;
    nt = local / ne;
  } else {
    int bid = xcd_remap(blockIdx.x, gridDim.x);
    if (L.np > 1 && bid >= L.tiles0) { pi = 1; bid -= L.tiles0; }
    tile_order(bid, L.p[pi].mtiles, L.p[pi].ntiles, L.p[pi].group_m, mt, nt);
  }
  const GemmProblem& P = L.p[pi];

  int m0, mend;
  int64_t b_base = 0;
  if (P.tile_e != nullptr) {
    const int e = P.tile_e[mt];
    m0 = P.tile_m0[mt];
    mend = P.offsets[e + 1];
    b_base = (int64_t)e * P.b_estride;
  } else {
    m0 = mt * BM;
    mend = P.M;
  }
  const int n0 = nt * BN;

  // Rows and chunks this thread moves: DMA instruction i of wave w fills LDS
  // chunks [(w*NA + i)*64, +64) of the A stage, lane l taking chunk position p.
  int64_t arow[NA];
  int acol[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int p = (wave * NA + i) * 64 + lane;
    const int r = p / CPR;
    const int m = min(m0 + r, mend - 1);
    arow[i] = P.gather ? (int64_t)P.gather[m] : (int64_t)m;
    acol[i] = swz_slot(r, p % CPR) * 8;
  }
  int brow[NB], bcol[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int p = (wave * NB + i) * 64 + lane;
    const int r = p / CPR;
    brow[i] = min(n0 + r, P.Nb - 1);
    bcol[i] = swz_slot(r, p % CPR) * 8;
  }

  // K segments, walked by the DMA issue in increasing tile order.
  int nk = 0;
  for (int s = 0; s < P.nseg; ++s) nk += P.seg[s].K / BK;
  int seg = 0, seg_k0 = 0, seg_end = P.seg[0].K / BK;
  const uint16_t* ap[NA];
  const uint16_t* bp[NB];
  auto point = [&](int s) {
    const KSeg& S = P.seg[s];
#pragma unroll
    for (int i = 0; i < NA; ++i) ap[i] = S.A + arow[i] * S.lda + acol[i];
#pragma unroll
    for (int i = 0; i < NB; ++i) bp[i] = S.B + b_base + (int64_t)brow[i] * S.ldb + bcol[i];
  };
  point(0);

  auto stA = [&](auto st) -> u32x4* {
    constexpr int v = decltype(st)::value;
    if constexpr (v == 0) return sa0;
    else if constexpr (v == 1) return sa1;
    else if constexpr (v == 2) return sa2;
    else if constexpr (v == 3) return sa3;
    else return sa4;
  };
  auto stB = [&](auto st) -> u32x4* {
    constexpr int v = decltype(st)::value;
    if constexpr (v == 0) return sb0;
    else if constexpr (v == 1) return sb1;
    else if constexpr (v == 2) return sb2;
    else if constexpr (v == 3) return sb3;
    else return sb4;
  };
  auto issue = [&](int kt, auto st) {
    while (kt >= seg_end) {          // uniform; at most nseg-1 times in the whole loop
      seg_k0 = seg_end;
      ++seg;
      seg_end += P.seg[seg].K / BK;
      point(seg);
    }
    const int koff = (kt - seg_k0) * BK;
    u32x4* a = stA(st);
    u32x4* b = stB(st);
#pragma unroll
    for (int i = 0; i < NA; ++i)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(ap[i] + koff), (lds_void_ptr)&a[(wave * NA + i) * 64], 16,
                                       0, 0);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(bp[i] + koff), (lds_void_ptr)&b[(wave * NB + i) * 64], 16,
                                       0, 0);
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.f;

  auto step = [&](int kt, auto st) {
    constexpr int S = decltype(st)::value;
    MOE_WAIT_VMCNT((STAGES - 2) * PER_TILE);
    // bare barrier: the wait above covers this wave's DMA of tile kt, the barrier
    // everyone else's, and every wave is done with the stage refilled below
    asm volatile("s_barrier" ::: "memory");
    issue(min(kt + STAGES - 1, nk - 1), Stage<(S + STAGES - 1) % STAGES>{});
    const u32x4* a = stA(st);
    const u32x4* b = stB(st);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      bf16x8 af[TM], bf[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int r = wave_m * WTM + tm * 32 + (lane & 31);
        af[tm] = __builtin_bit_cast(bf16x8, a[r * CPR + swz_slot(r, ch)]);
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int r = wave_n * WTN + tn * 32 + (lane & 31);
        bf[tn] = __builtin_bit_cast(bf16x8, b[r * CPR + swz_slot(r, ch)]);
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[tn], af[tm], acc[tn][tm], 0, 0, 0);
    }
  };

  issue(0, Stage<0>{});
  if constexpr (STAGES > 2) issue(min(1, nk - 1), Stage<1>{});
  if constexpr (STAGES > 3) issue(min(2, nk - 1), Stage<2>{});
  if constexpr (STAGES > 4) issue(min(3, nk - 1), Stage<3>{});
  // The unrolled body has no conditional steps (the compiler's wait analysis then
  // sees the same DMA history on every trip); the remainder runs after it.
  const int nfull = nk - nk % STAGES;
  for (int kt = 0; kt < nfull; kt += STAGES) {
    step(kt, Stage<0>{});
    step(kt + 1, Stage<1>{});
    if constexpr (STAGES > 2) step(kt + 2, Stage<2>{});
    if constexpr (STAGES > 3) step(kt + 3, Stage<3>{});
    if constexpr (STAGES > 4) step(kt + 4, Stage<4>{});
  }
  {
    const int r = nk - nfull;
    if (r > 0) step(nfull, Stage<0>{});
    if constexpr (STAGES > 2)
      if (r > 1) step(nfull + 1, Stage<1>{});
    if constexpr (STAGES > 3)
      if (r > 2) step(nfull + 2, Stage<2>{});
    if constexpr (STAGES > 4)
      if (r > 3) step(nfull + 3, Stage<3>{});
  }
  MOE_WAIT_VMCNT(0);   // no DMA may still be writing this workgroup's LDS when it ends

  // Epilogue: lane owns row m = (lane & 31) of each MFMA tile and, for g = 0..3,
  // the four columns 8g + 4*(lane >> 5) + 0..3.
  const int epi = EPI >= 0 ? EPI : P.epi;
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
        if (epi == EPI_F32) {
          f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(P.C) + (int64_t)m * P.ldc + n);
          *dst = f32x4{v0, v1, v2, v3};
        } else {
          if (epi == EPI_RELU2_BF16) {
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
