// Instances of the barrier ring (gemm_ring.hpp) with 256-row or 256-column tiles.
#include "gemm_ring.hpp"

namespace tbg {
template hipError_t launch_ring<256, 256, 2, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<256, 128, 2, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<256, 128, 3, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 256, 2, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 256, 3, 0>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
