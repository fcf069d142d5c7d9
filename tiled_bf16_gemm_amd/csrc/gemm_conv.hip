// Instances and dispatch of the implicit-GEMM convolution (gemm_conv.hpp) and of the halo
// convolution (gemm_conv_halo.hpp).
#include "gemm_conv.hpp"
#include "gemm_conv_halo.hpp"

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

bool plan_conv_halo(HaloParams& hp, int* hs_out, const char** why) {
  const ConvParams& c = hp.c;
  if (c.sh != 1 || c.sw != 1) return (*why = "stride 1"), false;
  const int rs = c.r * c.s;
  if (rs < 2) return (*why = "a filter of two taps or more"), false;
  if (c.c8 % 32 != 0) return (*why = "channels a multiple of 32"), false;
  if (c.ow > kHaloBM) return (*why = "output rows of at most 448 pixels"), false;
  const int tr = min(kHaloBM / c.ow, c.oh);
  const int64_t hh = tr + (int64_t)(c.r - 1) * c.dh, hw = c.ow + (int64_t)(c.s - 1) * c.dw;
  const int64_t hat = (hh * hw * kHaloPitch + 1023) / 1024;
  if (hat > kHaloMaxAtoms) return (*why = "an input window of at most 1008 pixels"), false;
  const int64_t hs = (hat + 4 * (rs - 1) - 1) / (4 * (rs - 1));
  if (hs > 4) return (*why = "an input window that four atoms per wave and tap copy in time"), false;
  const int tpi = (c.oh + tr - 1) / tr;
  const int64_t tiles_m = (int64_t)c.n * tpi, tiles_n = ((int64_t)c.g.N + kHaloBN - 1) / kHaloBN;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return (*why = "fewer than 2^31 tiles"), false;
  hp.tr = tr;
  hp.tpi = tpi;
  hp.hh = (int)hh;
  hp.hw = (int)hw;
  hp.ns = (int)(hh * hw);
  hp.hat = (int)hat;
  hp.hb = (int)hat * 1024;
  hp.cb32 = c.c8 / 32;
  hp.rs = rs;
  hp.div_hw = make_fast_div((uint32_t)hw);
  hp.div_ow = make_fast_div((uint32_t)c.ow);
  for (int v = 0; v < 9; ++v)
    hp.tap_off[v] = v < rs ? (int)(((int64_t)(v / c.s) * c.dh * hw + (int64_t)(v % c.s) * c.dw) * kHaloPitch) : 0;
  hp.c.g.tiles_m = (int)tiles_m;
  hp.c.g.tiles_n = (int)tiles_n;
  *hs_out = (int)hs;
  return true;
}

template <int HS, int TAPS>
static hipError_t launch_halo_taps(const HaloParams& hp, int out_bf16, hipStream_t stream) {
  const unsigned grid = (unsigned)hp.c.g.tiles_m * (unsigned)hp.c.g.tiles_n;
  if (hp.c.g.scaled) {
    if (out_bf16)
      hipLaunchKernelGGL((gemm_conv_halo_kernel<HS, 1, 1, TAPS>), dim3(grid), dim3(kThreads), 0, stream, hp);
    else
      hipLaunchKernelGGL((gemm_conv_halo_kernel<HS, 0, 1, TAPS>), dim3(grid), dim3(kThreads), 0, stream, hp);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((gemm_conv_halo_kernel<HS, 1, 0, TAPS>), dim3(grid), dim3(kThreads), 0, stream, hp);
    else
      hipLaunchKernelGGL((gemm_conv_halo_kernel<HS, 0, 0, TAPS>), dim3(grid), dim3(kThreads), 0, stream, hp);
  }
  return hipGetLastError();
}

// Filters of nine taps (3×3 and the like) run the kernel whose block of taps is unrolled.  With
// nine taps a window of at most 63 atoms needs at most two atoms per wave and tap.
template <int HS>
static hipError_t launch_halo_hs(const HaloParams& hp, int out_bf16, hipStream_t stream) {
  if constexpr (HS <= 2)
    if (hp.rs == 9) return launch_halo_taps<HS, 9>(hp, out_bf16, stream);
  return launch_halo_taps<HS, 0>(hp, out_bf16, stream);
}

hipError_t launch_conv_halo(const HaloParams& hp, int hs, int out_bf16, hipStream_t stream) {
  if ((int64_t)hp.c.g.tiles_m * hp.c.g.tiles_n == 0) return hipSuccess;
  switch (hs) {
    case 1: return launch_halo_hs<1>(hp, out_bf16, stream);
    case 2: return launch_halo_hs<2>(hp, out_bf16, stream);
    case 3: return launch_halo_hs<3>(hp, out_bf16, stream);
    case 4: return launch_halo_hs<4>(hp, out_bf16, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tbg
