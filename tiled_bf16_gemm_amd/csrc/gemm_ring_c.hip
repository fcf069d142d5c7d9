// Instances of the barrier ring (gemm_ring.hpp) with 64×64 tiles.
#include "gemm_ring.hpp"

namespace tbg {
template hipError_t launch_ring<64, 64, 2, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 3, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 4, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 5, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 6, 0>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
