// Instances of the barrier ring (gemm_ring.hpp) with 128×128 tiles.
#include "gemm_ring.hpp"

namespace tbg {
template hipError_t launch_ring<128, 128, 2>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 128, 3>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 128, 4>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 128, 5>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
