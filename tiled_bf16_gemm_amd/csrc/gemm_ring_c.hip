// Instances of the barrier ring (gemm_ring.hpp) with 64×64 tiles.
#include "gemm_ring.hpp"

namespace tbg {
template hipError_t launch_ring<64, 64, 2>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 3>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 4>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 5>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 6>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
