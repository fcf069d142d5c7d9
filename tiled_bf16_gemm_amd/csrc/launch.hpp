// Host-side launchers of the kernels, called by the C ABI in api.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tbg_desc.hpp"

namespace tbg {

// Arguments of one GEMM launch (see gemm_kernel.hip).
struct GemmParams {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int64_t lda, ldb, ldc;  // elements
  int M, N, K;
  int kchunks;     // 16-byte chunks along K present in memory (ceil(K/8)); data past K there is zero
  int tiles_m, tiles_n, group_m;
  int vec_store;   // C and its rows are 16-byte aligned: whole 16-byte stores allowed
  float alpha, beta;
  int scaled;      // 0: C = A·B; 1: C = alpha·A·B + beta·C (C read only when beta != 0)
};

hipError_t launch_tiled_store(const DescImpl& d, const int32_t* host_coords, const int32_t* coords_dev, uint32_t n,
                              const void* src, hipStream_t stream);
hipError_t launch_tiled_copy(const DescImpl& d, const int32_t* host_coords, const int32_t* coords_dev, uint32_t n,
                             void* dst, hipStream_t stream);
// Workgroup tile (bm × bn) for an M×N product on a device with num_cus compute units.
void choose_tile(int64_t M, int64_t N, int num_cus, int& bm, int& bn);
// Launch with tile bm × bn (256×256, 256×128, 128×256, 128×128 or 64×64); fills tiles_m/tiles_n.
hipError_t launch_gemm(GemmParams p, int bm, int bn, int b_layout, int out_bf16, hipStream_t stream);
hipError_t launch_pack(const uint16_t* src, int64_t ld_src, int64_t rows, int64_t cols, uint16_t* dst, int64_t ld_dst,
                       hipStream_t stream);

}  // namespace tbg
