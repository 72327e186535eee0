// Private declarations shared by the kernel sources and the C ABI layer.
#pragma once

#include <algorithm>

#include "common.h"
#include "gemm.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;

// GEMM tile configurations (BM x BN; 256x256 runs 8 waves, the others 4).
enum TileCfg : int { TILE_256x256 = 0, TILE_128x128 = 1, TILE_64x256 = 2, TILE_COUNT = 3 };
struct TileShape { int BM, BN; };
TileShape tile_shape(int cfg);

// Fills mtiles/ntiles-independent fields; the caller sets the problem fields.
hipError_t launch_gemm(GemmLaunch& L, int cfg, hipStream_t st);

struct PermuteScratch {
  uint64_t* masks;     // [E][nblk]
  int32_t* base;       // [E][nblk]
  int32_t* counts;     // [E]
  int32_t* tile_e;     // [max_mtiles]
  int32_t* tile_m0;    // [max_mtiles]
  int32_t* n_mtiles;   // [1]
};

hipError_t launch_split_router_weight(const float* w, int E, int H, uint16_t* parts, hipStream_t st);
hipError_t launch_topk(const float* logits, int64_t ldl, const float* bias, int T, int E, int K, float scale,
                       int32_t* idx, float* gate, float* gap, hipStream_t st);
hipError_t launch_permute_maps(const int32_t* idx, int T, int K, int E, int BM, const PermuteScratch& ps,
                               int32_t* offsets, int32_t* row_token, int32_t* slot_row, hipStream_t st);
hipError_t launch_gather_rows(const uint16_t* src, int C, const int32_t* row_token, int64_t rows, uint16_t* dst,
                              hipStream_t st);
hipError_t launch_combine(const uint16_t* y, const float* gate, const int32_t* slot_row, int T, int K, int L,
                          uint16_t* y_lat, hipStream_t st);

}  // namespace moe
