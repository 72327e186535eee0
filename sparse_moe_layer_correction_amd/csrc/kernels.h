// Private declarations shared by the kernel sources and the C ABI layer.
#pragma once

#include <algorithm>

#include "common.h"
#include "gemm.h"

namespace moe {

constexpr int kMaxExperts = 1024;
// tile counters of the forward's grouped GEMM launches (8 per launch, one per XCD)
constexpr int kGemmCounters = 16;
constexpr int kMaxTopK = 64;
constexpr int kMaxGroups = 64;      // one group per lane of the top-K wave

// GEMM tile configurations (BM x BN; 256x256 runs 8 waves, the others 4).
// TILE_256x256_GROUPED: the grouped expert products (one problem per launch).
enum TileCfg : int { TILE_256x256 = 0, TILE_128x128 = 1, TILE_64x256 = 2, TILE_256x256_GROUPED = 3, TILE_COUNT = 4 };
struct TileShape { int BM, BN; };
TileShape tile_shape(int cfg);

// Fills mtiles/ntiles-independent fields; the caller sets the problem fields.
hipError_t launch_gemm(GemmLaunch& L, int cfg, hipStream_t st);

// Few-row (decode) product streamed straight from HBM, see skinny.hip.
struct SkinnyProblem {
  KSeg seg[3];
  int nseg;
  int M;                     // dense rows (rows of the split-K partials)
  int N, Nb;                 // stored columns (multiple of 4), valid B rows
  int groups;                // 1 for a dense product; grouped: an upper bound on the experts listed
  const int32_t* offsets;    // grouped: [E+1] permuted row offsets (nullable -> dense)
  const int32_t* group_list; // grouped: the experts to run (those with tokens)
  const int32_t* n_groups;   // grouped: device scalar, length of group_list
  const int32_t* gather;     // nullable: A row of output row r is gather[r]
  int64_t b_estride;         // grouped: elements between experts' B
  void* C;
  int64_t ldc;
  int epi;
  int ksplit;                // dense: K split over this many waves per slab
  float* partial;            // [ksplit, M, N] fp32 when ksplit > 1, else null
  // MX weights (grouped products, one K segment): when set, B comes from
  // E4M3 codes [.., N, K] (b_estride apart per expert, row length seg[0].ldb)
  // and E8M0 scales, one per 32 k; seg[0].B is then unused
  const uint8_t* mx_codes;
  const uint8_t* mx_scales;
  int mx_fp4;                // MX codes are E2M1 (two per byte) rather than E4M3
  // fp32 weights (dense products, one K segment): when set, B is read from here
  // as fp32 [N, seg[0].ldb] and split exactly into three bf16 parts in registers
  const float* f32_b;
  // nullable, dense bf16 epilogue: C = bf16(residual + bf16(acc)) (the block's residual add)
  const uint16_t* residual;
  int64_t ldr;
};
// the weight operand of a skinny product: bf16, MXFP8 or MXFP4 codes and scales, or fp32
enum SkinnyBMode : int { kSkinnyBf16 = 0, kSkinnyMx = 1, kSkinnyF32 = 2, kSkinnyMx4 = 3 };
// reduce = false: leave a split-K product's fp32 partials for the caller to sum
hipError_t launch_skinny(const SkinnyProblem& P, hipStream_t st, bool reduce = true);
// dense bf16 products of 1..16 rows, K split over the waves of a workgroup and
// reduced in LDS (no partials, no second pass); P1: an optional second problem
// in the same launch
hipError_t launch_skinny_wgk(const SkinnyProblem& P0, const SkinnyProblem* P1, hipStream_t st);
constexpr int kWgkMaxRows = 16;
hipError_t launch_mxfp8_quantize(const uint16_t* src, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                                 hipStream_t st);
hipError_t launch_mxfp4_quantize(const uint16_t* src, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                                 hipStream_t st);
int skinny_slabs_per_wave(const SkinnyProblem& P);

struct PermuteScratch {
  uint64_t* masks;     // [E][nblk]
  int32_t* base;       // [E][nblk]
  int32_t* counts;     // [E]
  int32_t* tile_info;  // [max_mtiles][4]: each M tile's expert e, its first M tile, offsets[e], offsets[e+1]
  int32_t* n_mtiles;   // [1]
  int32_t* touched;    // [E] experts with at least one token, ascending
  int32_t* n_touched;  // [1]
  int32_t* gemm_ctr;   // [kGemmCounters] zeroed here for the grouped GEMMs that follow
};

hipError_t launch_split_router_weight(const float* w, int E, int H, uint16_t* parts, hipStream_t st);
// logits2: nullable, the second half of a K-split router product, added to logits
hipError_t launch_topk(const float* logits, const float* logits2, int64_t ldl, int nparts, int64_t part_off,
                       const float* bias, int T, int E, int K,
                       float scale, int n_group, int topk_group, int32_t* idx, float* gate, float* gap, hipStream_t st);
// top-K from a few-token router product's split-K partials [ksplit, T, ldl], summed in split order
hipError_t launch_topk_partials(const float* partial, int ksplit, int T, int64_t ldl, const float* bias, int E, int K,
                                float scale, int n_group, int topk_group, int32_t* idx, float* gate, float* gap,
                                hipStream_t st);
hipError_t launch_permute_maps(const int32_t* idx, int T, int K, int E, int BM, const PermuteScratch& ps,
                               int32_t* offsets, int32_t* row_token, int32_t* slot_row, hipStream_t st);
// n_valid: device scalar, the number of rows the maps filled (offsets[E]); rows past it are zeroed
hipError_t launch_gather_rows(const uint16_t* src, int C, const int32_t* row_token, const int32_t* n_valid,
                              int64_t rows, uint16_t* dst, hipStream_t st);
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, int64_t T, int H, float eps, uint16_t* y,
                          hipStream_t st);
hipError_t launch_bias_update(const int32_t* offsets, int E, float eta, float* bias, hipStream_t st);
hipError_t launch_combine(const uint16_t* y, const float* gate, const int32_t* slot_row, int T, int K, int L,
                          uint16_t* y_lat, hipStream_t st);

}  // namespace moe
