// Internal layout of tbg_tensor_desc (128 bytes), shared by the host encoder and the kernels.
//
// The descriptor records what "2 · Le Tensor Memory Accelerator" §2.2 and "H100 · cuTensorMap"
// §5 list: base address, rank (<= 5), elements per dimension, byte strides, the box, element
// strides, the swizzle, the out-of-bounds fill and the element type.  The layout is this
// library's own; only the information matches the pages.
#pragma once
#include <stdint.h>

namespace tbg {

constexpr uint32_t kDescMagic = 0x44474254u;  // "TBGD"
constexpr int kMaxRank = 5;
constexpr uint32_t kMaxBox = 256;
constexpr uint32_t kMaxEstride = 8;
constexpr uint64_t kMaxImageBytes = 64u * 1024u;

struct DescImpl {
  uint32_t magic;
  uint8_t dtype;     // tbg_dtype
  uint8_t elsize;    // bytes per element: 1, 2 or 4
  uint8_t rank;      // 1..5
  uint8_t swizzle;   // tbg_swizzle
  uint8_t oob;       // tbg_oob_fill
  uint8_t l2;        // tbg_l2_hint (recorded, no effect)
  uint8_t estr[5];   // element strides, 1..8 (unused dims: 1)
  uint8_t interleave;  // tbg_interleave (recorded; the copy itself is the tiled one)
  uint64_t base;          // device address of element (0, ..., 0)
  uint64_t dim[5];        // elements per dimension, innermost first (unused dims: 1)
  uint64_t stride[5];     // byte stride per dimension; stride[0] = elsize (unused dims: 0)
  uint16_t box[5];        // traversal box in elements (unused dims: 1)
  uint16_t n[5];          // copied elements per dimension, ceil(box / estr)
  uint32_t image_bytes;   // elsize * prod(n)
};
static_assert(sizeof(DescImpl) == 128, "descriptor must stay 128 bytes");

// Layout of an im2col descriptor (also 128 bytes, told apart by its magic): the NHWC tensor,
// the convolution's window geometry and the box ({channels, pixels}) of one copy.  Per-spatial
// arrays are {along W, along H}.  "2 · Le Tensor Memory Accelerator", section "im2col".
constexpr uint32_t kIm2colMagic = 0x49474254u;  // "TBGI"

struct DescIm2col {
  uint32_t magic;
  uint8_t dtype, elsize, swizzle, oob;
  uint8_t l2;
  uint8_t pad0[7];
  uint64_t base;          // device address of element (n, h, w, c) = (0, 0, 0, 0)
  uint32_t dim[4];        // C, W, H, N
  uint64_t stride[3];     // byte strides of W, H, N (the channel stride is the element size)
  int32_t pad_lo[2], pad_hi[2], cstride[2], dil[2], filt[2];
  uint32_t out[2];        // OW, OH: output extents of the convolution
  uint32_t channels, pixels;
  uint32_t image_bytes;   // elsize * channels * pixels
  uint32_t pad1;
};
static_assert(sizeof(DescIm2col) == 128, "im2col descriptor must stay 128 bytes");

// Extension swizzle mode for gfx950's 64-bank LDS (see tbg.h): a[6:4] ^= a[10:8].
constexpr int kSwizzle128B2Row = 4;
// Layout of the GEMM's B tiles stored K×N, descriptor mode TBG_SWIZZLE_128B_TR: the 16-byte chunk
// index of row r is XORed with (r[3] << 2) | (r[1] << 1) | r[2].  The transposing fragment read takes 32
// bytes from each of 16 rows {r0 + 8a + 2b + c}; LDS serves it 32 lanes (256 bytes) at a time,
// and this XOR gives the 8 rows of each half (rows 2 and 8 apart) distinct 32-byte bank groups,
// which neither the 128B nor the 2-row mode does (measured: 1.65x the cycles of a linear read
// with either, 1.0x with this one).
constexpr int kSwizzleKnTr = 5;

}  // namespace tbg
