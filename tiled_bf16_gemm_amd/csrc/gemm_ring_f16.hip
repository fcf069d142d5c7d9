// fp16-input instances of the barrier ring (gemm_ring.hpp): the configurations the automatic
// choice uses.
#include "gemm_ring.hpp"

namespace tbg {
template hipError_t launch_ring<256, 256, 2, 1>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<256, 128, 2, 1>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 256, 2, 1>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<128, 128, 2, 1>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 2, 1>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_ring<64, 64, 3, 1>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
