// Instances of the producer/consumer ring (gemm_pc.hpp) with 256×128 and 128×256 tiles.
#include "gemm_pc.hpp"

namespace tbg {
template hipError_t launch_pc<256, 128, 2, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<256, 128, 3, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<128, 256, 2, 0>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<128, 256, 3, 0>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
