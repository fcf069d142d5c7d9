// Instances of the barrier ring (gemm_ring.hpp) with 128×128 tiles.
#include "gemm_ring.hpp"

namespace tbg {
template hipError_t launch_ring<128, 128, 2, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 128, 3, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 128, 4, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 128, 5, 0>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
