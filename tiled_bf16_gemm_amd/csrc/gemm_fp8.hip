// Instances and dispatch of the fp8 GEMM (gemm_fp8.hpp).
#include "gemm_fp8.hpp"

namespace tbg {

template <int BM, int BN, int FMT>
static hipError_t launch_fp8_tile(const GemmParams& p, int out_bf16, hipStream_t stream) {
  const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
  if (p.scaled) {
    if (out_bf16) hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, FMT, 1, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, FMT, 0, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else {
    if (out_bf16) hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, FMT, 1, 0>), dim3(grid), dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, FMT, 0, 0>), dim3(grid), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

bool fp8_tile_built(int bm, int bn) {
  return (bm == 256 && bn == 256) || (bm == 128 && bn == 128) || (bm == 64 && bn == 64);
}

hipError_t launch_fp8(GemmParams p, int bm, int bn, int fmt, int out_bf16, hipStream_t stream) {
  p.tiles_m = (int)((p.M + bm - 1) / bm);
  p.tiles_n = (int)((p.N + bn - 1) / bn);
  if ((int64_t)p.tiles_m * p.tiles_n == 0) return hipSuccess;
  if (bm == 256 && bn == 256)
    return fmt ? launch_fp8_tile<256, 256, 1>(p, out_bf16, stream) : launch_fp8_tile<256, 256, 0>(p, out_bf16, stream);
  if (bm == 128 && bn == 128)
    return fmt ? launch_fp8_tile<128, 128, 1>(p, out_bf16, stream) : launch_fp8_tile<128, 128, 0>(p, out_bf16, stream);
  if (bm == 64 && bn == 64)
    return fmt ? launch_fp8_tile<64, 64, 1>(p, out_bf16, stream) : launch_fp8_tile<64, 64, 0>(p, out_bf16, stream);
  return hipErrorInvalidValue;
}

}  // namespace tbg
