// Instantiations and launcher of the bf16 MFMA GEMM (gemm.h).
#include "kernels.h"

namespace moe {

TileShape tile_shape(int cfg) {
  switch (cfg) {
    case TILE_256x256: return {256, 256};
    case TILE_128x128: return {128, 128};
    case TILE_64x256: return {64, 256};
    case TILE_256x256_GROUPED: return {256, 256};
    default: return {0, 0};
  }
}

constexpr int64_t kDense8WaveMaxTiles = 2048;

static bool one_segment(const GemmLaunch& L) {
  for (int i = 0; i < L.np; ++i)
    if (L.p[i].nseg != 1) return false;
  return true;
}

hipError_t launch_gemm(GemmLaunch& L, int cfg, hipStream_t st) {
  int64_t total = 0;
  for (int i = 0; i < L.np; ++i) total += (int64_t)L.p[i].mtiles * L.p[i].ntiles;
  L.tiles0 = L.p[0].mtiles * L.p[0].ntiles;
  if (total <= 0) return hipSuccess;
  const dim3 grid((unsigned)total);
  switch (cfg) {
    // The 256x256 tiles fill the 160 KiB of LDS with three B stages (gemm.h).
    // Eight waves of 128x64 (two per SIMD, 128 accumulators each, the same
    // k order per output, so the same bits) against four of 128x128, measured
    // on Ultra prefill, Nano and Super: 2-2.5 % faster for expert up and for
    // dense launches of up to 1536 tiles, 1-4 % slower for expert down and
    // even or 1 % slower for the Ultra prefill's dense launches (2048-3072 tiles)
    // and 5 % slower for its router product (fp32 logits, 256 tiles).
    case TILE_256x256:
      if (total < kDense8WaveMaxTiles && L.p[0].epi != EPI_F32)
        hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 4, -1, 2, 3>), grid, dim3(512), 0, st, L);
      else
        hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 2, -1, 1, 3>), grid, dim3(256), 0, st, L);
      break;
    case TILE_128x128: hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, -1, 2>), grid, dim3(256), 0, st, L); break;
    case TILE_64x256: hipLaunchKernelGGL((gemm_bf16_kernel<64, 256, 1, 4, -1, 2>), grid, dim3(256), 0, st, L); break;
    // grouped expert products: one problem, epilogue fixed at compile time (the
    // up and down products are then also told apart by name in profiles)
    case TILE_256x256_GROUPED:   // one problem of one K segment
      if (L.np != 1 || !one_segment(L)) return hipErrorInvalidValue;
      if (L.p[0].epi == EPI_RELU2_BF16)
        hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 4, EPI_RELU2_BF16, 2, 3>), grid, dim3(512), 0, st, L);
      else
        hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 2, EPI_BF16, 1, 3>), grid, dim3(256), 0, st, L);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
