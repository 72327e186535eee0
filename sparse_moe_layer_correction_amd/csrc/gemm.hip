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
    // the 256x256 tiles fill the 160 KiB of LDS with three B stages (gemm.h)
    case TILE_256x256: hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 2, -1, 1, 3>), grid, dim3(256), 0, st, L); break;
    case TILE_128x128: hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, -1, 2>), grid, dim3(256), 0, st, L); break;
    case TILE_64x256: hipLaunchKernelGGL((gemm_bf16_kernel<64, 256, 1, 4, -1, 2>), grid, dim3(256), 0, st, L); break;
    // grouped expert products: one problem, epilogue fixed at compile time (the
    // up and down products are then also told apart by name in profiles)
    case TILE_256x256_GROUPED:   // one problem of one K segment
      if (L.np != 1 || !one_segment(L)) return hipErrorInvalidValue;
      if (L.p[0].epi == EPI_RELU2_BF16)
        hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 2, EPI_RELU2_BF16, 1, 3>), grid, dim3(256), 0, st, L);
      else
        hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 2, EPI_BF16, 1, 3>), grid, dim3(256), 0, st, L);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
