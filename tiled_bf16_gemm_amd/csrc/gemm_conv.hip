// Instances and dispatch of the implicit-GEMM convolution (gemm_conv.hpp).
#include "gemm_conv.hpp"

namespace tbg {

template <int BM, int BN>
static hipError_t launch_conv_tile(const ConvParams& cp, int out_bf16, hipStream_t stream) {
  const unsigned grid = (unsigned)cp.g.tiles_m * (unsigned)cp.g.tiles_n;
  if (cp.g.scaled) {
    if (out_bf16) hipLaunchKernelGGL((gemm_conv_kernel<BM, BN, 1, 1>), dim3(grid), dim3(kThreads), 0, stream, cp);
    else hipLaunchKernelGGL((gemm_conv_kernel<BM, BN, 0, 1>), dim3(grid), dim3(kThreads), 0, stream, cp);
  } else {
    if (out_bf16) hipLaunchKernelGGL((gemm_conv_kernel<BM, BN, 1, 0>), dim3(grid), dim3(kThreads), 0, stream, cp);
    else hipLaunchKernelGGL((gemm_conv_kernel<BM, BN, 0, 0>), dim3(grid), dim3(kThreads), 0, stream, cp);
  }
  return hipGetLastError();
}

bool conv_tile_built(int bm, int bn) {
  return (bm == 256 && bn == 256) || (bm == 256 && bn == 128) || (bm == 128 && bn == 128) || (bm == 64 && bn == 64);
}

hipError_t launch_conv(ConvParams cp, int bm, int bn, int out_bf16, hipStream_t stream) {
  cp.g.tiles_m = (int)((cp.g.M + bm - 1) / bm);
  cp.g.tiles_n = (int)((cp.g.N + bn - 1) / bn);
  if ((int64_t)cp.g.tiles_m * cp.g.tiles_n == 0) return hipSuccess;
  if (bm == 256 && bn == 256) return launch_conv_tile<256, 256>(cp, out_bf16, stream);
  if (bm == 256 && bn == 128) return launch_conv_tile<256, 128>(cp, out_bf16, stream);
  if (bm == 128 && bn == 128) return launch_conv_tile<128, 128>(cp, out_bf16, stream);
  if (bm == 64 && bn == 64) return launch_conv_tile<64, 64>(cp, out_bf16, stream);
  return hipErrorInvalidValue;
}

}  // namespace tbg
