// Instances of the producer/consumer ring (gemm_pc.hpp) with 128×128 tiles.
#include "gemm_pc.hpp"

namespace tbg {
template hipError_t launch_pc<128, 128, 2, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<128, 128, 3, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<128, 128, 4, 0>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
