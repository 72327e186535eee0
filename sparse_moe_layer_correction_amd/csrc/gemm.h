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
//  * global -> LDS by buffer loads that write LDS directly (16 bytes per lane,
//    no VGPR staging), addressed through a buffer resource per operand with a
//    fixed 32-bit offset per lane and the k position in the scalar offset;
//  * one k tile is 64 bf16 deep, so each row contributes one whole 128-byte
//    line per tile; chunk c of row r sits in slot c ^ ((r >> 1) & 7), which
//    keeps the ds_read_b128 fragment reads free of bank conflicts on gfx950's
//    64-bank LDS;
//  * two LDS stages of A and, in the 256x256 tiles, three of B (the weights,
//    which the grouped products stream from HBM), so a B tile is loaded two k
//    steps ahead; per k tile, one barrier, placed so that the loads of the
//    next tiles and the first fragment reads of the next tile overlap the
//    MFMAs of the current tile's last substep.
// The 256x256 tile runs four waves of 128x128 each: a wave then reads half a
// fragment per MFMA from LDS (a 128x64 wave tile reads three quarters), and
// its 256 fp32 accumulators per lane live in AGPRs.
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
  int K;               // multiple of 64
};

struct GemmProblem {
  KSeg seg[3];
  int nseg;
  int M;                     // dense: rows of C
  int N;                     // columns of C that are stored (multiple of 4)
  int Nb;                    // valid B rows (columns >= Nb reuse row Nb-1, results unused)
  const int32_t* gather;     // nullable: A row of output row r is gather[r]
  const int32_t* tile_info;  // nullable: grouped mode M-tile table, 4 ints per M tile: its
                             //   expert e, e's first M tile, offsets[e], offsets[e+1];
                             //   a grouped launch holds exactly one problem
  const int32_t* n_mtiles;   //   device scalar: number of valid M tiles
  const int32_t* offsets;    //   [E+1] expert row offsets
  int64_t b_estride;         //   elements between consecutive experts' B
  void* C;
  int64_t ldc;
  int epi;
  const uint16_t* residual;  // nullable, dense bf16 epilogues: C = bf16(residual + bf16(acc))
  int64_t ldr;
  int mtiles;                // M tiles in the grid (an upper bound in grouped mode)
  int ntiles;                // ceil(N / BN)
  int group_m;               // M tiles per raster group
  int a_records;             // range of the A buffer resources: kRsrc2G, or kRsrc4G when the
                             //   A rows' byte offsets reach 2 GiB (gathered rows of a large z)
};

struct GemmLaunch {
  GemmProblem p[2];
  int np;
  int tiles0;                // tiles of problem 0 (mtiles * ntiles)
  int* counters;             // grouped launches: nullable, 8 zeroed ints (one per XCD) that hand
                             //   out the tiles; without them workgroup b takes a fixed tile
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

// Order of a grouped expert's tiles. An XCD hands its workgroups, in order, to
// its four shader engines in turn (measured: every fourth workgroup goes to the
// same engine whatever its tile costs, and the hand-out waits for the engine
// whose turn it is). With the short last M tile of an expert next to its full
// ones, tiles of one height went to the same engines (two M tiles per expert:
// two engines had only full tiles, two only short ones). So the N tiles go in
// blocks (all of them up to 8, else 4 at a time): a block holds first the
// expert's full-height M tiles for its N tiles (rasters of gm_ M tiles, M
// fastest in a raster, so that the M tiles sharing a weight panel run side by
// side), then the short M tile for the same N tiles; with a multiple of 4 N
// tiles every run of one tile height is a multiple of 4 long and each engine
// gets the same mix. (Blocks of 4 out of 8 N tiles made an M tile's rows be
// read again half an expert later: Super's 31-tile expert, expert down +1.4 %.)
// ne M tiles, the first nfull of full height.
__host__ __device__ __forceinline__ void grouped_tile_order(int local, int ne, int nfull, int ntl, int gm_, int& mt,
                                                            int& nt) {
  const int PB = ntl <= 8 ? ntl : 4;
  const int blk = local / (ne * PB);
  const int nb = min(PB, ntl - blk * PB);
  const int rem = local - blk * ne * PB;
  if (rem < nfull * nb) {
    const int per = gm_ * nb;
    const int g = rem / per;
    const int gm = min(gm_, nfull - g * gm_);
    const int r2 = rem - g * per;
    mt = g * gm_ + r2 % gm;
    nt = blk * PB + r2 / gm;
  } else {
    mt = ne - 1;
    nt = blk * PB + (rem - nfull * nb);
  }
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

// slot of logical chunk c of row r (8 chunks of 16 bytes per 128-byte row):
// the 16 lanes a ds_read_b128 serves together read rows r0..r0+15 at one
// logical chunk, and land in the 16 distinct slots of a 256-byte window.
__device__ __forceinline__ int swz_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

// two fp32 -> packed bf16x2, round to nearest even (one v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2_t));
}

// Buffer resource over [base, base + num_records): raw (stride 0) descriptor,
// word 3 as the gfx9 family expects for untyped loads. A raw buffer access is
// in range while its byte offset is below num_records; num_records 0 makes
// every lane out of range: the load then touches no memory (buffer range
// checking returns zeros). kRsrc2G covers every offset below 2 GiB; kRsrc4G
// (0xFFFFFFFF) every 32-bit offset but the last, for operands whose rows lie
// past 2 GiB from their base -- measured 17 % slower on every product of the
// Ultra prefill when used for all loads, so it is taken only where needed.
constexpr int kRsrc2G = 0x7FFFFFFF;
constexpr int kRsrc4G = -1;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int num_records = kRsrc2G) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_records, 0x00020000);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Stage<I>{});
    static_for<I + 1, N>(f);
  }
}

// Spread NDMA buffer loads and NREAD ds_reads over NMFMA MFMAs in the order the
// scheduler emits them: per group, loads first, then a read, then MFMAs.
template <int NMFMA, int NREAD, int NDMA>
__device__ __forceinline__ void interleave() {
  constexpr int G = NREAD > 0 ? NREAD : (NDMA > 0 ? NDMA : 1);
  static_for<0, G>([&](auto gi) {
    constexpr int g = decltype(gi)::value;
    constexpr int nd = (g + 1) * NDMA / G - g * NDMA / G;
    constexpr int nr = (g + 1) * NREAD / G - g * NREAD / G;
    constexpr int nm = (g + 1) * NMFMA / G - g * NMFMA / G;
    if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x020, nd, 0);
    if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
    if constexpr (nm > 0) __builtin_amdgcn_sched_group_barrier(0x008, nm, 0);
  });
  __builtin_amdgcn_sched_barrier(0);
}

// EPI: an Epilogue fixed at compile time, or -1 to take each problem's own.
// OCC: waves per SIMD the register allocation is sized for (1 lets the 256x256
// tile keep its 256 accumulators per lane in AGPRs next to 256 VGPRs).
// BST: LDS stages of B, 2 or 3 (3 for the 256x256 tiles: see the main loop).
template <int BM, int BN, int WM, int WN, int EPI, int OCC, int BST = 2>
__global__ void __launch_bounds__(64 * WM * WN, 1) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
gemm_bf16_kernel(const GemmLaunch L) {
  constexpr int BK = 64, CPR = 8;                  // k tile: 64 bf16 = 128 bytes per row
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;      // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;      // 32x32 MFMA tiles per wave
  constexpr int NA = BM * CPR / NT;                // A loads per thread per k tile
  constexpr int NB = BN * CPR / NT;
  constexpr int ACH = BM * CPR, BCH = BN * CPR;    // 16-byte chunks per stage
  static_assert(TM >= 1 && TN >= 1 && NA >= 1 && NB >= 1, "tile shape");
  static_assert(NA * NT == ACH && NB * NT == BCH, "load coverage");
  static_assert(BST == 2 || BST == 3, "B stages");
  // two stages (B: BST), each its own array so that the compiler can tell the
  // stage being filled from the one being read. With three B stages the LDS is
  // full (2 x 32 + 3 x 32 KiB at 256x256), and the tile claim's word lives in
  // the third B stage, which no load fills before every wave has read it.
  __shared__ u32x4 sa0[ACH], sb0[BCH], sa1[ACH], sb1[BCH], sb2[BST == 3 ? BCH : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WM, wave_n = wave / WM;

  int pi = 0, m0, mend, n0;
  int64_t b_base = 0;
  if (L.p[0].tile_info != nullptr) {
    // grouped: the grid is sized for the most M tiles any routing can need, and
    // n_mtiles * ntiles of those workgroups get a tile; the tiles are split over
    // the XCDs in equal contiguous ranges (see xcd_remap)
    const int ntl = L.p[0].ntiles;
    int t;
    // (only the grouped instantiations, the fixed-epilogue ones, carry the
    // claim: its LDS word would push the 64x256 tile past two workgroups per CU)
    if (EPI >= 0 && L.counters != nullptr) {
      // Each XCD's range is split into a fixed part, seven eighths of it, and a
      // tail handed out in order by the XCD's counter: workgroup b (on XCD
      // b % 8) takes fixed tile b / 8 while there is one, then claims from its
      // XCD's tail and, once that is done, from another XCD's. XCDs run the
      // grouped products a few per cent apart, and with fixed tiles the slowest
      // one ended the launch alone; only the tail pays the claim's latency.
      const int valid = *L.p[0].n_mtiles * ntl;
      const int q = valid / 8, r = valid % 8;
      const int x = (int)blockIdx.x % 8, j = (int)blockIdx.x / 8;
      const int size = q + (x < r ? 1 : 0), fixed = size - size / 8;
      if (j < fixed) {
        t = x * q + min(x, r) + j;
      } else {
        int& claim = *reinterpret_cast<int*>(sb2);
        if (tid == 0) {
          int tt = -1;
          for (int d = 0; d < 8 && tt < 0; ++d) {
            const int y = (x + d) & 7;
            const int sy = q + (y < r ? 1 : 0), fy = sy - sy / 8;
            if (d > 0 && __hip_atomic_load(&L.counters[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= sy - fy)
              continue;                                  // that tail is done: no atomic
            const int w = atomicAdd(&L.counters[y], 1);
            if (w < sy - fy) tt = y * q + min(y, r) + fy + w;
          }
          claim = tt;
        }
        __syncthreads();
        t = __builtin_amdgcn_readfirstlane(claim);
        if (t < 0) return;
        if constexpr (BST == 3) __syncthreads();   // every wave has read the word before loads fill sb2
      }
    } else {
      const int valid = *L.p[0].n_mtiles * ntl;
      if ((int)blockIdx.x >= valid) return;
      t = xcd_remap(blockIdx.x, valid);
    }
    // expert by expert: the tiles of one expert are contiguous in the order,
    // in rasters of group_m M tiles (M fastest in a raster), so the M tiles that
    // share a weight panel run side by side
    // (an expert's ne M tiles times ntl N tiles are contiguous in t, starting at
    // its first M tile f times ntl, so t / ntl lands on one of the expert's own
    // M tiles, whose entry holds e, f and the expert's rows; its tiles start at
    // its first permuted row, offsets[e], BM rows apart). Every table read here
    // is one dependent step of the workgroup's start, so the entry is one read.
    const int4 info = reinterpret_cast<const int4*>(L.p[0].tile_info)[t / ntl];
    const int e = info.x, f = info.y, o0 = info.z, o1 = info.w;
    const int ne = (o1 - o0 + BM - 1) / BM;
    const int local = t - f * ntl;
    int mt, nt;
    grouped_tile_order(local, ne, (o1 - o0) / BM, ntl, L.p[0].group_m, mt, nt);
    m0 = o0 + mt * BM;
    mend = o1;
    n0 = nt * BN;
    b_base = (int64_t)e * L.p[0].b_estride;
  } else {
    int bid = xcd_remap(blockIdx.x, gridDim.x);
    if (L.np > 1 && bid >= L.tiles0) { pi = 1; bid -= L.tiles0; }
    int mt, nt;
    tile_order(bid, L.p[pi].mtiles, L.p[pi].ntiles, L.p[pi].group_m, mt, nt);
    m0 = mt * BM;
    mend = L.p[pi].M;
    n0 = nt * BN;
  }

  // In the grouped products (the instantiations with a fixed epilogue), an
  // expert's tail tile with at most BM/4, BM/2 or 3*BM/4 valid rows runs a
  // shorter tile: the same waves split that many rows, so it costs a part of a
  // full tile instead of a whole one (the tail tiles are about a sixth of the
  // padded rows at 704 rows per expert). Mode q runs q quarters of the tile's
  // rows. Quarter tiles (tails of at most 64 rows): Super 5.54 -> 5.49 ms,
  // Nano 2.64 -> 2.63 ms, Ultra prefill unchanged within noise.
  constexpr bool kShortTiles = BM == 256 && WM == 2 && EPI >= 0;
  auto body = [&](const GemmProblem& P, auto mode) __attribute__((always_inline)) {
    constexpr int Q = decltype(mode)::value;       // quarters of BM
    static_assert(Q >= 1 && Q <= 4, "tile height");
    constexpr int NAX = NA * Q / 4;                // A loads per thread per k tile
    constexpr int TMX = TM * Q / 4;                // 32-row MFMA tiles per wave
    constexpr int WTMX = WTM * Q / 4;              // wave tile rows
    static_assert(Q == 4 || (NA * Q % 4 == 0 && TM * Q % 4 == 0), "short tile shape");
    // Load i of a thread fills LDS chunks [(wave*NAX + i)*64, +64) of the A stage
    // (64 lanes x 16 bytes, contiguous), lane l taking chunk position p: row
    // p / 8, slot p % 8, which holds logical chunk swz_slot(row, slot). Rows are
    // taken relative to the tile's first row (gathered rows: absolute), so the
    // 32-bit buffer offsets stay small; rows past the end repeat the last row.
    int arow[NAX], acol[NAX];
  #pragma unroll
    for (int i = 0; i < NAX; ++i) {
      const int p = (wave * NAX + i) * 64 + lane;
      const int r = p / CPR;
      const int m = min(m0 + r, mend - 1);
      arow[i] = P.gather ? P.gather[m] : m - m0;
      acol[i] = swz_slot(r, p % CPR) * 16;
    }
    int brow[NB], bcol[NB];
  #pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int p = (wave * NB + i) * 64 + lane;
      const int r = p / CPR;
      brow[i] = min(n0 + r, P.Nb - 1) - n0;
      bcol[i] = swz_slot(r, p % CPR) * 16;
    }

    // the A buffer range, read once: a kernel-argument load inside the loop
    // would be followed by a wait for all scalar and LDS reads in flight
    const int arec = __builtin_amdgcn_readfirstlane(P.a_records);
    // K segments, walked by the load issue in increasing k-tile order.
    int nk = 0;
    for (int s = 0; s < P.nseg; ++s) nk += P.seg[s].K / BK;
    int seg = 0, seg_k0 = 0, seg_end = P.seg[0].K / BK;
    const uint16_t* abase;
    const uint16_t* bbase;
    uint32_t ao[NAX], bo[NB];
    auto point = [&](int s) {
      const KSeg& S = P.seg[s];
      abase = P.gather ? S.A : S.A + (int64_t)m0 * S.lda;
      bbase = S.B + b_base + (int64_t)n0 * S.ldb;
  #pragma unroll
      for (int i = 0; i < NAX; ++i) ao[i] = (uint32_t)((int64_t)arow[i] * S.lda * 2 + acol[i]);
  #pragma unroll
      for (int i = 0; i < NB; ++i) bo[i] = (uint32_t)((int64_t)brow[i] * S.ldb * 2 + bcol[i]);
    };
    point(0);

    auto stA = [&](auto st) -> u32x4* {
      if constexpr (decltype(st)::value == 0) return sa0;
      else return sa1;
    };
    auto stB = [&](auto st) -> u32x4* {
      if constexpr (decltype(st)::value == 0) return sb0;
      else return sb1;
    };
    // loads of a tile in four quarters: bit 0 / 1 the first / second half of a
    // thread's A loads, bit 2 / 3 the same for B
    auto issue = [&](int kt, auto st, bool live = true, int parts = 15) {
      while (kt >= seg_end) {          // uniform; at most nseg-1 times in the whole loop
        seg_k0 = seg_end;
        ++seg;
        seg_end += P.seg[seg].K / BK;
        point(seg);
      }
      const int so = (kt - seg_k0) * BK * 2;
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(abase, live ? arec : 0),
                                   rb = make_rsrc(bbase, live ? kRsrc2G : 0);
      // (the explicit casts of the lane offsets matter: without them the host
      // pass silently drops this kernel's launch stub)
      u32x4* a = stA(st);
      u32x4* b = stB(st);
  #pragma unroll
      for (int i = 0; i < NAX; ++i)
        if (parts & (i < NAX / 2 ? 1 : 2))
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_ptr)&a[(wave * NAX + i) * 64], 16, (int)ao[i], so, 0,
                                                   0);
  #pragma unroll
      for (int i = 0; i < NB; ++i)
        if (parts & (i < NB / 2 ? 4 : 8))
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_ptr)&b[(wave * NB + i) * 64], 16, (int)bo[i], so, 0,
                                                   0);
    };

    // Fragments of one 16-deep k substep: lane l reads row (l & 31) of each
    // 32-row MFMA tile at logical chunk 2*ks + (l >> 5).
    struct Frag {
      bf16x8 a[TMX], b[TN];
    };
    auto read = [&](Frag& f, auto st, int ks) {
      const u32x4* a = stA(st);
      const u32x4* b = stB(st);
      const int ch = ks * 2 + (lane >> 5);
  #pragma unroll
      for (int tm = 0; tm < TMX; ++tm) {
        const int r = wave_m * WTMX + tm * 32 + (lane & 31);
        f.a[tm] = __builtin_bit_cast(bf16x8, a[r * CPR + swz_slot(r, ch)]);
      }
  #pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int r = wave_n * WTN + tn * 32 + (lane & 31);
        f.b[tn] = __builtin_bit_cast(bf16x8, b[r * CPR + swz_slot(r, ch)]);
      }
    };
    f32x16 acc[TN][TMX];
  #pragma unroll
    for (int a = 0; a < TN; ++a)
  #pragma unroll
      for (int b = 0; b < TMX; ++b)
  #pragma unroll
        for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.f;
    auto mma = [&](const Frag& f) {
  #pragma unroll
      for (int tn = 0; tn < TN; ++tn)
  #pragma unroll
        for (int tm = 0; tm < TMX; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[tn], f.a[tm], acc[tn][tm], 0, 0, 0);
    };

    // Step kt computes k tile kt from stage kt & 1 in four substeps; the reads of
    // substep s+1 overlap the MFMAs of substep s. The one barrier sits before the
    // last substep, whose fragments are then already in registers: past it, tile
    // kt+1 has landed (every wave waited for its own loads) and nobody reads
    // stage kt & 1 any more, so tile kt+2 is loaded into it while the last
    // substep runs and the first fragments of tile kt+1 are read.
    constexpr int NM = TMX * TN, NR = TMX + TN;
    Frag f0, f1;
    // When each quarter of tile kt+2's loads is issued (plan digits for A lo, A hi,
    // B lo, B hi: 3 = after the barrier of step kt, 0 / 1 = in the first / second
    // substep of step kt+1; with three B stages the B quarters are tile kt+3's). All at the barrier left the waves' load issue in one
    // burst that put them out of step (the barrier then waits for the slowest):
    // spreading the B half over the next tile's first substeps took 3-6 % off
    // every product on the Ultra prefill, the best split differing by product.
    // With three B stages (a sweep of 6 plans over the Ultra prefill, Nano and
    // Super): both B halves in the second substep for expert up and the dense
    // products (1-2 % ahead of the two-stage plans at Nano and Super, equal at
    // Ultra), the two-stage plan for expert down; all at the barrier 4-10 % slower.
    constexpr int PLAN = EPI == EPI_BF16 ? 3301 : 3311;
    constexpr int QD[4] = {PLAN / 1000, PLAN / 100 % 10, PLAN / 10 % 10, PLAN % 10};
    constexpr int QN[4] = {NAX / 2, NAX - NAX / 2, NB / 2, NB - NB / 2};
    constexpr int M0 = (QD[0] == 0) | (QD[1] == 0) << 1 | (QD[2] == 0) << 2 | (QD[3] == 0) << 3;
    constexpr int M1 = (QD[0] == 1) | (QD[1] == 1) << 1 | (QD[2] == 1) << 2 | (QD[3] == 1) << 3;
    constexpr int M3 = (QD[0] == 3) | (QD[1] == 3) << 1 | (QD[2] == 3) << 2 | (QD[3] == 3) << 3;
    constexpr int N0 = (M0 & 1 ? QN[0] : 0) + (M0 & 2 ? QN[1] : 0) + (M0 & 4 ? QN[2] : 0) + (M0 & 8 ? QN[3] : 0);
    constexpr int N1 = (M1 & 1 ? QN[0] : 0) + (M1 & 2 ? QN[1] : 0) + (M1 & 4 ? QN[2] : 0) + (M1 & 8 ? QN[3] : 0);
    constexpr int N3 = (M3 & 1 ? QN[0] : 0) + (M3 & 2 ? QN[1] : 0) + (M3 & 4 ? QN[2] : 0) + (M3 & 8 ? QN[3] : 0);
    auto step = [&](int kt, auto st) {
      constexpr int S = decltype(st)::value;
      read(f1, st, 1);
      // quarters of tile kt+1 (in the other stage) planned for this substep
      if constexpr (M0 != 0) {
        if (kt >= 1) issue(min(kt + 1, nk - 1), Stage<1 - S>{}, kt + 1 < nk, M0);
      }
      mma(f0);
      interleave<NM, NR, N0>();
      read(f0, st, 2);
      if constexpr (M1 != 0) {
        if (kt >= 1) issue(min(kt + 1, nk - 1), Stage<1 - S>{}, kt + 1 < nk, M1);
      }
      mma(f1);
      interleave<NM, NR, N1>();
      read(f1, st, 3);
      mma(f0);
      interleave<NM, NR, 0>();
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // past the end the load still runs (the schedule stays the same) but over
      // an empty range, so it moves no data and lands at once
      if constexpr (M3 != 0) issue(min(kt + 2, nk - 1), st, kt + 2 < nk, M3);
      read(f0, Stage<1 - S>{}, 0);
      mma(f1);
      interleave<NM, NR, N3>();
    };

    if constexpr (BST == 2) {
      issue(0, Stage<0>{});
      issue(min(1, nk - 1), Stage<1>{});
      MOE_WAIT_VMCNT(NAX + NB);
      __syncthreads();
      read(f0, Stage<0>{}, 0);
      for (int kt = 0; kt + 1 < nk; kt += 2) {
        step(kt, Stage<0>{});
        step(kt + 1, Stage<1>{});
      }
      if (nk & 1) step(nk - 1, Stage<0>{});
    } else {
      // Three B stages: B tile kt+3 is loaded from the barrier
      // of step kt on, so a B load has two steps to land instead of one (A
      // keeps one). In the grouped products the weight panels come from HBM,
      // and the weights of the 10-20 panels that an XCD's workgroups start on
      // together all miss at once. A tile's stages: A kt % 2, B kt % 3.
      auto stB3 = [&](auto st) -> u32x4* {
        constexpr int v = decltype(st)::value;
        if constexpr (v == 0) return sb0;
        else if constexpr (v == 1) return sb1;
        else return sb2;
      };
      // A and B walk the K segments apart (B one tile ahead): each has its own
      // segment position, and a segment change re-points only its operand. The
      // grouped products (fixed epilogue) have one segment: no walk.
      int sega = 0, sega_k0 = 0, sega_end = P.seg[0].K / BK;
      int segb = 0, segb_k0 = 0, segb_end = sega_end;
      auto issueA = [&](int kt, auto st, bool live) {
        if constexpr (EPI < 0) {
          while (kt >= sega_end) {     // uniform; at most nseg-1 times in the whole loop
            sega_k0 = sega_end;
            ++sega;
            sega_end += P.seg[sega].K / BK;
            const KSeg& S = P.seg[sega];
            abase = P.gather ? S.A : S.A + (int64_t)m0 * S.lda;
  #pragma unroll
            for (int i = 0; i < NAX; ++i) ao[i] = (uint32_t)((int64_t)arow[i] * S.lda * 2 + acol[i]);
          }
        }
        const int so = (kt - sega_k0) * BK * 2;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(abase, live ? arec : 0);
        u32x4* a = stA(st);
  #pragma unroll
        for (int i = 0; i < NAX; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_ptr)&a[(wave * NAX + i) * 64], 16, (int)ao[i], so, 0,
                                                   0);
      };
      auto issueB = [&](int kt, auto st, bool live, int parts) {
        if constexpr (EPI < 0) {
          while (kt >= segb_end) {
            segb_k0 = segb_end;
            ++segb;
            segb_end += P.seg[segb].K / BK;
            const KSeg& S = P.seg[segb];
            bbase = S.B + b_base + (int64_t)n0 * S.ldb;
  #pragma unroll
            for (int i = 0; i < NB; ++i) bo[i] = (uint32_t)((int64_t)brow[i] * S.ldb * 2 + bcol[i]);
          }
        }
        const int so = (kt - segb_k0) * BK * 2;
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bbase, live ? kRsrc2G : 0);
        u32x4* b = stB3(st);
  #pragma unroll
        for (int i = 0; i < NB; ++i)
          if (parts & (i < NB / 2 ? 4 : 8))
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_ptr)&b[(wave * NB + i) * 64], 16, (int)bo[i], so,
                                                     0, 0);
      };
      auto read3 = [&](Frag& f, auto sa, auto sb, int ks) {
        const u32x4* a = stA(sa);
        const u32x4* b = stB3(sb);
        const int ch = ks * 2 + (lane >> 5);
  #pragma unroll
        for (int tm = 0; tm < TMX; ++tm) {
          const int r = wave_m * WTMX + tm * 32 + (lane & 31);
          f.a[tm] = __builtin_bit_cast(bf16x8, a[r * CPR + swz_slot(r, ch)]);
        }
  #pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int r = wave_n * WTN + tn * 32 + (lane & 31);
          f.b[tn] = __builtin_bit_cast(bf16x8, b[r * CPR + swz_slot(r, ch)]);
        }
      };
      // the plan's B quarters: at the barrier of step kt (tile kt+3), or in the
      // first / second substep of step kt+1; A is loaded whole at the barrier,
      // so that the last NB loads issued before a barrier are one B tile's
      static_assert(((M0 | M1) & 3) == 0, "A quarters at the barrier");
      constexpr int NB0 = N0, NB1 = N1, NX3 = NAX + (N3 - (M3 & 1 ? QN[0] : 0) - (M3 & 2 ? QN[1] : 0));
      // s_waitcnt vmcnt(NB) lgkmcnt(0): tile kt+1 has landed once no more than
      // the NB loads of B tile kt+2 are in flight
      constexpr int kWaitB = (NB & 0xF) | (0x7 << 4) | (0x0 << 8) | (((NB >> 4) & 3) << 14);
      // (step 0 is its own copy, FIRST: B tile 2 was loaded whole before it. A
      // run-time test there left the compiler's count of loads in flight
      // unknown at the loop head, and it then waited for B tile kt+2 after
      // the barrier of every sixth step.)
      auto step3 = [&](int kt, auto sa, auto sb, auto first) {
        constexpr int SA = decltype(sa)::value, SB = decltype(sb)::value;
        constexpr bool FIRST = decltype(first)::value != 0;
        read3(f1, sa, sb, 1);
        if constexpr (M0 != 0 && !FIRST) issueB(min(kt + 2, nk - 1), Stage<(SB + 2) % 3>{}, kt + 2 < nk, M0);
        mma(f0);
        interleave<NM, NR, FIRST ? 0 : NB0>();
        read3(f0, sa, sb, 2);
        if constexpr (M1 != 0 && !FIRST) issueB(min(kt + 2, nk - 1), Stage<(SB + 2) % 3>{}, kt + 2 < nk, M1);
        mma(f1);
        interleave<NM, NR, FIRST ? 0 : NB1>();
        read3(f1, sa, sb, 3);
        mma(f0);
        interleave<NM, NR, 0>();
        __builtin_amdgcn_s_waitcnt(kWaitB);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        issueA(min(kt + 2, nk - 1), sa, kt + 2 < nk);
        if constexpr ((M3 & 12) != 0) issueB(min(kt + 3, nk - 1), sb, kt + 3 < nk, M3);
        read3(f0, Stage<1 - SA>{}, Stage<(SB + 1) % 3>{}, 0);
        mma(f1);
        interleave<NM, NR, NX3>();
      };
      issueA(0, Stage<0>{}, true);
      issueB(0, Stage<0>{}, true, 12);
      issueA(min(1, nk - 1), Stage<1>{}, true);
      issueB(min(1, nk - 1), Stage<1>{}, true, 12);
      issueB(min(2, nk - 1), Stage<2>{}, true, 12);
      // tile 0 has landed once tile 1 and B tile 2 are all that is in flight
      // (an explicit wait and barrier: __syncthreads would wait for every load)
      MOE_WAIT_VMCNT(NAX + 2 * NB);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      read3(f0, Stage<0>{}, Stage<0>{}, 0);
      step3(0, Stage<0>{}, Stage<0>{}, Stage<1>{});
      // step kt reads A stage kt % 2 and B stage kt % 3: from kt = 1 the pattern
      // (1,1) (0,2) (1,0) (0,1) (1,2) (0,0) repeats
      int kt = 1;
      for (; kt + 6 <= nk; kt += 6) {
        step3(kt, Stage<1>{}, Stage<1>{}, Stage<0>{});
        step3(kt + 1, Stage<0>{}, Stage<2>{}, Stage<0>{});
        step3(kt + 2, Stage<1>{}, Stage<0>{}, Stage<0>{});
        step3(kt + 3, Stage<0>{}, Stage<1>{}, Stage<0>{});
        step3(kt + 4, Stage<1>{}, Stage<2>{}, Stage<0>{});
        step3(kt + 5, Stage<0>{}, Stage<0>{}, Stage<0>{});
      }
      if (kt < nk) {
        step3(kt, Stage<1>{}, Stage<1>{}, Stage<0>{});
        if (kt + 1 < nk) {
          step3(kt + 1, Stage<0>{}, Stage<2>{}, Stage<0>{});
          if (kt + 2 < nk) {
            step3(kt + 2, Stage<1>{}, Stage<0>{}, Stage<0>{});
            if (kt + 3 < nk) {
              step3(kt + 3, Stage<0>{}, Stage<1>{}, Stage<0>{});
              if (kt + 4 < nk) step3(kt + 4, Stage<1>{}, Stage<2>{}, Stage<0>{});
            }
          }
        }
      }
    }
    MOE_WAIT_VMCNT(0);   // no load may still be writing this workgroup's LDS when it ends

    // Epilogue. Lane l owns row (l & 31) of each 32x32 MFMA tile and, for
    // g = 0..3, the four columns 8g + 4*(l >> 5) + 0..3.
    const int epi = EPI >= 0 ? EPI : P.epi;
    if (EPI < 0 && epi == EPI_F32) {
      // fp32 results (router logits): straight from the accumulators
#pragma unroll
      for (int tm = 0; tm < TMX; ++tm) {
        const int m = m0 + wave_m * WTMX + tm * 32 + (lane & 31);
        if (m >= mend) continue;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wave_n * WTN + tn * 32 + 8 * g + 4 * (lane >> 5);
            if (n >= P.N) continue;
            *reinterpret_cast<f32x4*>(static_cast<float*>(P.C) + (int64_t)m * P.ldc + n) =
                f32x4{acc[tn][tm][4 * g], acc[tn][tm][4 * g + 1], acc[tn][tm][4 * g + 2], acc[tn][tm][4 * g + 3]};
          }
      }
      return;
    }
    // bf16 results go through LDS, so that every store writes whole rows of
    // the wave tile (WTN * 2 bytes) instead of 16-byte pieces of 32 rows. Each
    // wave stages its tile in one of the (now idle) stage arrays, 16-byte chunk
    // c of tile row r at chunk c ^ (r % CPW): the 32 rows a ds_write_b64 hits
    // then fall on distinct banks pairwise, and a row reads back contiguously.
    constexpr int CPW = WTN / 8;                   // 16-byte chunks per wave-tile row
    static_assert(WTMX * WTN * 2 <= ACH * 16 && WTMX * WTN * 2 <= BCH * 16, "staging fits a stage array");
    MOE_WAIT_VMCNT(0);
    __syncthreads();                               // all loads landed, all fragment reads done
    constexpr int NWAVE = WM * WN;
    static_assert(NWAVE <= 4 || (NWAVE == 8 && 2 * WTMX * WTN * 2 <= ACH * 16), "staging areas");
    char* stg;
    if constexpr (NWAVE <= 4) {
      stg = reinterpret_cast<char*>(wave == 0 ? sa0 : wave == 1 ? sb0 : wave == 2 ? sa1 : sb1);
    } else {                                       // eight waves: two wave tiles per stage array
      const int h = wave >> 1;
      stg = reinterpret_cast<char*>(h == 0 ? sa0 : h == 1 ? sb0 : h == 2 ? sa1 : sb1) + (wave & 1) * (WTMX * WTN * 2);
    }
    const bool r2 = epi == EPI_RELU2_BF16;
#pragma unroll
    for (int tm = 0; tm < TMX; ++tm) {
      const int r = tm * 32 + (lane & 31);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v0 = acc[tn][tm][4 * g + 0], v1 = acc[tn][tm][4 * g + 1];
          float v2 = acc[tn][tm][4 * g + 2], v3 = acc[tn][tm][4 * g + 3];
          if (r2) {
            v0 = relu2(v0); v1 = relu2(v1); v2 = relu2(v2); v3 = relu2(v3);
          }
          const int c = tn * 4 + g;
          *reinterpret_cast<u32x2*>(stg + r * (CPW * 16) + ((c ^ (r % CPW)) * 16) + (lane >> 5) * 8) =
              u32x2{cvt_pk_bf16(v0, v1), cvt_pk_bf16(v2, v3)};
        }
    }
    // read back: 64 / CPW rows per instruction, CPW lanes per row. The problem's
    // fields are copied first: read through P after a store, the compiler would
    // load them again (it cannot tell the stores from the kernel arguments),
    // and each such reload serialised one read-back and store.
    constexpr int RPI = 64 / CPW, NRB = WTMX / RPI;
    const int Nc = P.N;
    const int64_t ldc = P.ldc, ldr = P.ldr;
    uint16_t* const Cp = static_cast<uint16_t*>(P.C);
    const uint16_t* const res = EPI < 0 ? P.residual : nullptr;
    u32x4 rb[NRB];
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      const int r = i * RPI + lane / CPW;
      const int c = lane % CPW;
      rb[i] = *reinterpret_cast<const u32x4*>(stg + r * (CPW * 16) + ((c ^ (r % CPW)) * 16));
    }
    // read-back i holds row mfirst + i * RPI of the output at columns n..n+7:
    // the row offsets advance by a fixed stride, and the column tests hold for
    // every row (per row, the 64-bit row products and the tests had cost about
    // 20 instructions per store)
    const int mfirst = m0 + wave_m * WTMX + lane / CPW;
    const int n = n0 + wave_n * WTN + (lane % CPW) * 8;
    const bool cols = n < Nc, full = n + 8 <= Nc;    // else 4 columns (N is a multiple of 4)
    int64_t doff = (int64_t)mfirst * ldc + n, soff = (int64_t)mfirst * ldr + n;
    const int64_t dstep = (int64_t)RPI * ldc, sstep = (int64_t)RPI * ldr;
#pragma unroll
    for (int i = 0; i < NRB; ++i, doff += dstep, soff += sstep) {
      if (!cols || mfirst + i * RPI >= mend) continue;
      const u32x4 v = rb[i];
      u32x4 o = v;
      if (EPI < 0 && res != nullptr) {
        // the block's residual add: bf16 + bf16 in fp32 (exact), rounded once
        const uint16_t* src = res + soff;
        u32x4 rv;
        if (full) rv = *reinterpret_cast<const u32x4*>(src);
        else {
          const u32x2 h = *reinterpret_cast<const u32x2*>(src);
          rv = u32x4{h[0], h[1], 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = cvt_pk_bf16(bf16_bits_to_f32(v[q] & 0xFFFFu) + bf16_bits_to_f32(rv[q] & 0xFFFFu),
                             bf16_bits_to_f32(v[q] >> 16) + bf16_bits_to_f32(rv[q] >> 16));
      }
      uint16_t* dst = Cp + doff;
      if (full) *reinterpret_cast<u32x4*>(dst) = o;
      else *reinterpret_cast<u32x2*>(dst) = u32x2{o[0], o[1]};
    }
  };
  if constexpr (kShortTiles) {
    if (mend - m0 <= BM / 4) {
      body(L.p[0], Stage<1>{});
      return;
    }
    if (mend - m0 <= BM / 2) {
      body(L.p[0], Stage<2>{});
      return;
    }
    if (mend - m0 <= 3 * BM / 4) {
      body(L.p[0], Stage<3>{});
      return;
    }
  }
  body(L.p[pi], Stage<4>{});
}

}  // namespace moe
