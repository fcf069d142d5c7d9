// The im2col copy: one block of the im2col matrix of a 2-D convolution per workgroup, built in
// LDS and written out as a dense image.
//
// "2 · Le Tensor Memory Accelerator", section "im2col": a copy mode dedicated to convolution
// performs the im2col transform during the copy, so the convolution becomes a GEMM without the
// intermediate matrix being stored.  Reading (the page gives no more): the tensor is NHWC; row m
// of the im2col matrix is output pixel m = (n*OH + oh)*OW + ow, column (r, s, c) is filter tap
// (r, s) and channel c; its element is X[n, oh*sh - ph + r*dh, ow*sw - pw + s*dw, c], the fill
// where that position is outside the tensor (the convolution's zero padding), where m is outside
// 0..N*OH*OW-1 or c outside 0..C-1.  A copy takes `pixels` rows from m0 and `channels` channels
// from c0 at one tap: coords {c0, m0, s, r}.  The image is dense, channel fastest, through the
// swizzle like a tiled copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "tbg_desc.hpp"
#include "tile_loader.hpp"

namespace tbg {

struct Coords4 {
  int32_t c[4];
};

// Address of X[n, ih, iw, 0] for output pixel m at tap (r, s), or 0 when the window position is
// outside the tensor (or m outside the output).
__device__ __forceinline__ uint64_t im2col_row_base(const DescIm2col& d, int64_t m, int64_t tap_s, int64_t tap_r) {
  const int64_t OW = d.out[0], OH = d.out[1];
  if (m < 0 || m >= (int64_t)d.dim[3] * OH * OW) return 0;
  const int64_t ow = m % OW, oh = (m / OW) % OH, n = m / (OW * OH);
  const int64_t ih = oh * d.cstride[1] - d.pad_lo[1] + tap_r * d.dil[1];
  const int64_t iw = ow * d.cstride[0] - d.pad_lo[0] + tap_s * d.dil[0];
  if (ih < 0 || ih >= (int64_t)d.dim[2] || iw < 0 || iw >= (int64_t)d.dim[1]) return 0;
  return d.base + (uint64_t)n * d.stride[2] + (uint64_t)ih * d.stride[1] + (uint64_t)iw * d.stride[0];
}

__device__ __forceinline__ void lds_put(uint8_t* lds, uint32_t off, const uint8_t* src, int es) {
  if (es == 1) lds[off] = *src;
  else if (es == 2) *(uint16_t*)(lds + off) = *(const uint16_t*)src;
  else *(uint32_t*)(lds + off) = *(const uint32_t*)src;
}

__device__ __forceinline__ void lds_fill(uint8_t* lds, uint32_t off, uint32_t fill, int es) {
  if (es == 1) lds[off] = (uint8_t)fill;
  else if (es == 2) *(uint16_t*)(lds + off) = (uint16_t)fill;
  else *(uint32_t*)(lds + off) = fill;
}

// Build the image in LDS: 16-byte chunks of whole in-bounds channel runs move as one load
// (rows are 16-byte aligned when channels*elsize and c0*elsize are multiples of 16: the base and
// every stride are); everything else goes element by element.
__device__ void build_im2col(const DescIm2col& d, const int64_t* c, uint8_t* lds, uint32_t fill) {
  const int es = d.elsize;
  const uint32_t row_bytes = d.channels * es;
  const bool chunked = (row_bytes % 16u) == 0 && ((c[0] * es) % 16) == 0;
  if (!chunked) {
    const uint32_t total = d.channels * d.pixels;
    for (uint32_t e = threadIdx.x; e < total; e += blockDim.x) {
      const uint32_t i = e / d.channels, j = e % d.channels;
      const uint64_t row = im2col_row_base(d, c[1] + i, c[2], c[3]);
      const int64_t ch = c[0] + j;
      const uint32_t off = swizzle_offset(e * es, d.swizzle);
      if (row && ch >= 0 && ch < (int64_t)d.dim[0]) lds_put(lds, off, (const uint8_t*)(row + (uint64_t)ch * es), es);
      else lds_fill(lds, off, fill, es);
    }
    return;
  }
  const uint32_t cpr = row_bytes / 16u;
  const int epc = 16 / es;
  const uint32_t total = d.image_bytes / 16u;
  const uint4 fill4 = make_uint4(fill, fill, fill, fill);
  for (uint32_t q = threadIdx.x; q < total; q += blockDim.x) {
    const uint32_t i = q / cpr, jc = q % cpr;
    const uint64_t row = im2col_row_base(d, c[1] + i, c[2], c[3]);
    const int64_t ch0 = c[0] + (int64_t)jc * epc;
    const uint32_t off = swizzle_offset(q * 16u, d.swizzle);
    if (row && ch0 >= 0 && ch0 + epc <= (int64_t)d.dim[0]) {
      *(uint4*)(lds + off) = *(const uint4*)(row + (uint64_t)ch0 * es);
    } else if (!row || ch0 + epc <= 0 || ch0 >= (int64_t)d.dim[0]) {
      *(uint4*)(lds + off) = fill4;
    } else {
      for (int e = 0; e < epc; ++e) {
        const int64_t ch = ch0 + e;
        if (ch >= 0 && ch < (int64_t)d.dim[0]) lds_put(lds, off + e * es, (const uint8_t*)(row + (uint64_t)ch * es), es);
        else lds_fill(lds, off + e * es, fill, es);
      }
    }
  }
}

__global__ void __launch_bounds__(256) im2col_copy_kernel(DescIm2col d, Coords4 host_coords, const int32_t* coords_dev,
                                                          uint8_t* dst, uint32_t box_offset, uint32_t fill) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const uint32_t b = blockIdx.x + box_offset;
  int64_t c[4];
  for (int i = 0; i < 4; ++i) c[i] = coords_dev ? coords_dev[(uint64_t)b * 4 + i] : host_coords.c[i];
  build_im2col(d, c, smem, fill);
  __syncthreads();
  uint8_t* out = dst + (uint64_t)b * d.image_bytes;
  const uint32_t nbytes = d.image_bytes;
  if ((((uintptr_t)out) % 16u) == 0 && (nbytes % 16u) == 0) {
    for (uint32_t i = threadIdx.x; i < nbytes / 16u; i += blockDim.x) ((uint4*)out)[i] = ((const uint4*)smem)[i];
  } else {
    for (uint32_t i = threadIdx.x; i < nbytes; i += blockDim.x) out[i] = smem[i];
  }
}

hipError_t launch_im2col_copy(const DescIm2col& d, const int32_t* host_coords, const int32_t* coords_dev, uint32_t n,
                              void* dst, hipStream_t stream) {
  Coords4 hc{};
  if (host_coords)
    for (int i = 0; i < 4; ++i) hc.c[i] = host_coords[i];
  uint32_t fill = 0;
  if (d.oob == 1) {
    if (d.dtype == 3) fill = 0x7E007E00u;        // f16
    else if (d.dtype == 4) fill = 0x7FC07FC0u;   // bf16
    else if (d.dtype == 6) fill = 0x7F7F7F7Fu;   // fp8 E4M3
    else if (d.dtype == 7) fill = 0x7E7E7E7Eu;   // fp8 E5M2
    else fill = 0x7FC00000u;                     // f32
  }
  const size_t lds_bytes = ((size_t)d.image_bytes + 1023u) & ~(size_t)1023u;
  const uint32_t kMaxGrid = 1u << 20;
  for (uint32_t done = 0; done < n; done += kMaxGrid) {
    const uint32_t cnt = (n - done) < kMaxGrid ? (n - done) : kMaxGrid;
    hipLaunchKernelGGL(im2col_copy_kernel, dim3(cnt), dim3(256), lds_bytes, stream, d, hc, coords_dev, (uint8_t*)dst,
                       done, fill);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tbg
