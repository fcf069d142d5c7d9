// Host-side launchers of the kernels, called by the C ABI in api.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fast_div.hpp"
#include "tbg_desc.hpp"

namespace tbg {

// Arguments of one GEMM launch (see gemm_kernel.hip).  The barrier ring, the producer ring and
// the fp8 ring read their operands through `da` and `db`, the descriptors of the operand boxes
// that the host encodes with tbg_encode_tiled ("2 · Le Tensor Memory Accelerator" §2.3: built
// once on the host, handed to the kernel): base address, row pitch in bytes and extents (A {K, M};
// B {K, N} stored N×K, {N, K} stored K×N).  A, B, lda and ldb stay for the convolution kernel.
struct GemmParams {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int64_t lda, ldb, ldc;  // elements
  int M, N, K;
  int kchunks;     // 16-byte chunks along K present in memory (ceil(K/8)); data past K there is zero
  int tiles_m, tiles_n, group_m;
  int vec_store;   // C's base and row pitch are multiples of 4 bytes: whole 16-byte pieces may be stored
  float alpha, beta;
  int scaled;      // 0: C = A·B; 1: C = alpha·A·B + beta·C (C read only when beta != 0)
  // Clock-recording instances only (a measurement build outside the C ABI): per workgroup the
  // 100 MHz real-time and shader-clock counter deltas from its start to its end.  Null otherwise.
  uint64_t* clock;
  DescImpl da, db;  // operand box descriptors (zero when K = 0: every copy is masked)
};

// Arguments of one implicit-GEMM convolution launch (gemm_conv.hpp).  `g` carries what the
// GEMM epilogue needs: M = N*OH*OW output pixels, N = K output channels, C = Y, ldc = ldy,
// vec_store, alpha/beta/scaled, and the tile grid.  X and W have a channel pitch of c8 (a
// multiple of 8; channels c8 > c >= C hold zeros after packing).
struct ConvParams {
  GemmParams g;
  const uint16_t* X;   // NHWC, channel pitch c8
  const uint16_t* W;   // K × (R·S·c8): filter k, tap (r, s), channel c at k*ldw + (r*S + s)*c8 + c
  int64_t ldw;         // R * S * c8
  uint32_t x_bytes;    // bytes of X (below 2^31)
  int n, h, w, c8, r, s, oh, ow;
  int ph, pw, sh, sw, dh, dw;
  int cblocks;         // ceil(c8 / 64): 64-channel blocks per tap
};

// Arguments of the halo convolution (gemm_conv_halo.hpp): stride 1, channels a multiple of 32.
// A workgroup computes `tr` whole output rows of one image (tr·ow <= 448 pixels) for 128 output
// channels; the input window those rows need (hh × hw pixels, zero outside the image) is copied
// into LDS once per 32-channel block and every filter tap reads it there.
struct HaloParams {
  ConvParams c;        // c.g.tiles_m = images × tiles per image, c.g.tiles_n = ceil(k / 128)
  int tr, tpi;         // output rows per tile, tiles per image
  int hh, hw, ns;      // window rows, columns, pixels (hh·hw)
  int hat, hb;         // 1 KiB copy atoms per window image, its LDS bytes (hat·1024)
  int cb32, rs;        // 32-channel blocks, filter taps
  FastDiv div_hw, div_ow;
  int tap_off[9];      // LDS byte offset of tap v = r·S + s from tap 0 in a window image (v < rs, rs <= 9)
};

hipError_t launch_im2col_copy(const DescIm2col& d, const int32_t* host_coords, const int32_t* coords_dev, uint32_t n,
                              void* dst, hipStream_t stream);
// Convolution with workgroup tile bm × bn (256×256, 256×128, 128×128 or 64×64); fills the grid.
hipError_t launch_conv(ConvParams cp, int bm, int bn, int out_bf16, hipStream_t stream);
bool conv_tile_built(int bm, int bn);
// Fills the halo fields of `hp` from hp.c (shape fields set); false with `why` set when the shape
// does not fit the halo kernel.  hs_out: window atoms each wave copies per filter tap (1..4).
bool plan_conv_halo(HaloParams& hp, int* hs_out, const char** why);
hipError_t launch_conv_halo(const HaloParams& hp, int hs, int out_bf16, hipStream_t stream);

hipError_t launch_tiled_store(const DescImpl& d, const int32_t* host_coords, const int32_t* coords_dev, uint32_t n,
                              const void* src, hipStream_t stream);
hipError_t launch_tiled_copy(const DescImpl& d, const int32_t* host_coords, const int32_t* coords_dev, uint32_t n,
                             void* dst, hipStream_t stream);
// Operand-copy pipelines of the GEMM (values of tbg_pipeline).
enum GemmPipeline { kPipeRing = 1, kPipeProducer = 2 };

// One built kernel configuration; tiles_m / tiles_n of `p` must be set.
typedef hipError_t (*GemmLauncher)(const GemmParams& p, int b_layout, int out_bf16, hipStream_t stream);
// IN: input element type of the products, 0 bf16, 1 fp16.
template <int BM, int BN, int S, int IN>
hipError_t launch_ring(const GemmParams& p, int b_layout, int out_bf16, hipStream_t stream);
template <int BM, int BN, int S, int IN>
hipError_t launch_pc(const GemmParams& p, int b_layout, int out_bf16, hipStream_t stream);

// The launcher of (pipeline, tile bm × bn, stages) for input type `in`, or nullptr when that
// configuration is not built.
GemmLauncher find_gemm(int pipeline, int bm, int bn, int stages, int in = 0);
// Readable list of the built configurations of a pipeline (for error messages).
const char* gemm_configs_text(int pipeline, int in = 0);

// A kernel configuration for an M×N product on a device with num_cus compute units.  Zero
// arguments are open: pipeline 0 = either pipeline, bm = bn = 0 = any tile, stages 0 = each
// candidate's default.  Returns false when no built configuration matches what is fixed.
struct GemmChoice {
  int pipeline, bm, bn, stages;
};
bool choose_gemm(int64_t M, int64_t N, int num_cus, int pipeline, int bm, int bn, int stages, GemmChoice& out,
                 int in = 0);
// Launch a built configuration; fills tiles_m / tiles_n.  Returns hipErrorInvalidValue for a
// configuration find_gemm does not know.
hipError_t launch_gemm(GemmParams p, int pipeline, int bm, int bn, int stages, int b_layout, int out_bf16,
                       hipStream_t stream, int in = 0);
// One repack: `rows` rows of `row_bytes` bytes at pitch ld_src (bytes, any alignment) into
// pitch ld_dst (bytes, a multiple of 16), zero-filled past row_bytes.
struct PackJob {
  const uint8_t* src;
  int64_t ld_src, rows, row_bytes;
  uint8_t* dst;
  int64_t ld_dst;
};
// Runs n (1 or 2) repacks in one launch.
hipError_t launch_pack_jobs(const PackJob* jobs, int n, hipStream_t stream);
// fp8 GEMM (gemm_fp8.hpp): p in units of two fp8 values (lda, ldb, K, kchunks as for 16-bit data
// of half the width); fmt 0 E4M3, 1 E5M2; tiles 256×256, 128×128, 64×64.
hipError_t launch_fp8(GemmParams p, int bm, int bn, int fmt, int out_bf16, hipStream_t stream);
bool fp8_tile_built(int bm, int bn);

}  // namespace tbg
