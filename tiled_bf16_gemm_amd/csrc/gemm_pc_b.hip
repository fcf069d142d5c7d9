// Instances of the producer/consumer ring (gemm_pc.hpp) with 64×64 tiles.
#include "gemm_pc.hpp"

namespace tbg {
template hipError_t launch_pc<64, 64, 2, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<64, 64, 3, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<64, 64, 4, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<64, 64, 5, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<64, 64, 6, 0>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
