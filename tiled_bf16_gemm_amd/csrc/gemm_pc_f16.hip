// fp16-input instances of the producer/consumer ring (gemm_pc.hpp): the configurations the
// automatic choice uses.
#include "gemm_pc.hpp"

namespace tbg {
template hipError_t launch_pc<256, 128, 2, 1>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<128, 256, 2, 1>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<128, 128, 3, 1>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_pc<64, 64, 3, 1>(const GemmParams&, int, int, hipStream_t);
}  // namespace tbg
