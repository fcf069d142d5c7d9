// Tiled copy kernels, one workgroup per box.  Load: the box is built in LDS (the page's "shared
// memory" destination) and then written out as a dense image so that it can be checked byte for
// byte.  Store: an image is brought into LDS and scattered into the box's tensor positions.
//
// "2 · Le Tensor Memory Accelerator" §2.2, §2.4, §2.5 and "H100 · cuTensorMap" §8, §9, §11, §14
// define what a copy produces; this file decides how gfx950 produces it:
//  * 2-D boxes of 128-byte rows with a 128-byte-row swizzle and zero fill go through the same
//    direct-to-LDS atom loader the GEMM uses for its operand tiles (tile_loader.hpp), so the
//    copy API checks the GEMM's loader bit for bit;
//  * every other box (rank up to 5, element strides, NaN fill, any swizzle) is staged through
//    registers: whole 16-byte chunks where the box row is chunk-aligned and in bounds, single
//    elements at ragged edges.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "tbg_desc.hpp"
#include "tile_loader.hpp"

namespace tbg {

struct Coords5 {
  int32_t c[5];
};

__device__ __forceinline__ void lds_store_elem(uint8_t* lds, uint32_t off, const uint8_t* src, int elsize) {
  if (elsize == 1) *(lds + off) = *src;
  else if (elsize == 2) *(uint16_t*)(lds + off) = *(const uint16_t*)src;
  else *(uint32_t*)(lds + off) = *(const uint32_t*)src;
}

__device__ __forceinline__ void lds_fill_elem(uint8_t* lds, uint32_t off, uint32_t fill, int elsize) {
  if (elsize == 1) *(lds + off) = (uint8_t)fill;
  else if (elsize == 2) *(uint16_t*)(lds + off) = (uint16_t)fill;
  else *(uint32_t*)(lds + off) = fill;
}

// One element of the box at image element index e (innermost first).
__device__ __forceinline__ void copy_element(const DescImpl& d, const int64_t* c, uint8_t* lds, uint64_t e,
                                             uint32_t fill) {
  uint64_t rem = e;
  bool inside = true;
  uint64_t src = d.base;
  for (int i = 0; i < kMaxRank; ++i) {
    const uint64_t ni = d.n[i];
    const uint64_t j = rem % ni;
    rem /= ni;
    if (i < d.rank) {
      const int64_t x = c[i] + (int64_t)j * (int64_t)d.estr[i];
      if (x < 0 || (uint64_t)x >= d.dim[i]) inside = false;
      else src += (uint64_t)x * d.stride[i];
    }
  }
  const uint32_t off = swizzle_offset((uint32_t)(e * d.elsize), d.swizzle);
  if (inside) lds_store_elem(lds, off, (const uint8_t*)src, d.elsize);
  else lds_fill_elem(lds, off, fill, d.elsize);
}

// Register-staged path for any descriptor.
__device__ void build_box_generic(const DescImpl& d, const int64_t* c, uint8_t* lds, uint32_t fill) {
  const int tid = threadIdx.x;
  const int es = d.elsize;
  const uint32_t row_bytes = (uint32_t)d.n[0] * es;
  const bool chunked = d.estr[0] == 1 && (row_bytes % 16u) == 0 && ((c[0] * es) % 16) == 0;
  if (!chunked) {
    const uint64_t total = d.image_bytes / es;
    for (uint64_t e = tid; e < total; e += blockDim.x) copy_element(d, c, lds, e, fill);
    return;
  }
  const uint32_t chunks_per_row = row_bytes / 16u;
  const int epc = 16 / es;  // elements per chunk
  const uint32_t total_chunks = d.image_bytes / 16u;
  const uint4 fill4 = make_uint4(fill, fill, fill, fill);
  for (uint32_t ch = tid; ch < total_chunks; ch += blockDim.x) {
    const uint32_t row = ch / chunks_per_row;
    const uint32_t cr = ch % chunks_per_row;
    // coordinates of dims 1..rank-1 for this image row
    uint32_t rem = row;
    bool row_inside = true;
    uint64_t src = d.base;
    for (int i = 1; i < kMaxRank; ++i) {
      const uint32_t ni = d.n[i];
      const uint32_t j = rem % ni;
      rem /= ni;
      if (i < d.rank) {
        const int64_t x = c[i] + (int64_t)j * (int64_t)d.estr[i];
        if (x < 0 || (uint64_t)x >= d.dim[i]) row_inside = false;
        else src += (uint64_t)x * d.stride[i];
      }
    }
    const int64_t x0 = c[0] + (int64_t)cr * epc;
    const uint32_t off = swizzle_offset(ch * 16u, d.swizzle);
    if (row_inside && x0 >= 0 && (uint64_t)(x0 + epc) <= d.dim[0]) {
      *(uint4*)(lds + off) = *(const uint4*)(src + (uint64_t)x0 * es);
    } else if (!row_inside || x0 + epc <= 0 || (x0 >= 0 && (uint64_t)x0 >= d.dim[0])) {
      *(uint4*)(lds + off) = fill4;
    } else {
      for (int q = 0; q < epc; ++q) {
        const int64_t x = x0 + q;
        const uint32_t eoff = off + (uint32_t)(q * es);  // a chunk moves whole under the swizzle
        if (x >= 0 && (uint64_t)x < d.dim[0]) lds_store_elem(lds, eoff, (const uint8_t*)(src + (uint64_t)x * es), es);
        else lds_fill_elem(lds, eoff, fill, es);
      }
    }
  }
}

// Direct-to-LDS path: rank 2, 128-byte box rows, box rows a multiple of 8, 128B, 2-row or
// transposing-read swizzle, zero fill, chunk-aligned origin inside the tensor.  Same atoms as the
// GEMM's loads.
template <int SWZ>
__device__ void build_box_dma(const DescImpl& d, const int64_t* c, uint8_t* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const uint32_t pitch = (uint32_t)d.stride[1];
  const uint64_t origin = d.base + (uint64_t)c[1] * d.stride[1] + (uint64_t)c[0] * d.elsize;
  const uint64_t remaining = (d.dim[1] - 1 - (uint64_t)c[1]) * d.stride[1] + (d.dim[0] - (uint64_t)c[0]) * d.elsize;
  const rsrc_t rs = make_rsrc((const void*)origin, remaining);
  const int chunks_valid = (int)(((d.dim[0] - (uint64_t)c[0]) * d.elsize) / 16u);
  const int atoms = d.n[1] / 8;
  for (int a = wave; a < atoms; a += nwaves) {
    const LaneChunk lc = lane_chunk<SWZ>(a * 8, lane, pitch);
    issue_atom(rs, lds_addr_of(lds + a * 1024), lc, chunks_valid);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ void __launch_bounds__(256) tiled_copy_kernel(DescImpl d, Coords5 host_coords, const int32_t* coords_dev,
                                                         uint8_t* dst, uint32_t box_offset, int dma_ok,
                                                         uint32_t fill) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const uint32_t b = blockIdx.x + box_offset;
  int64_t c[kMaxRank];
  for (int i = 0; i < kMaxRank; ++i) {
    c[i] = 0;
    if (i < d.rank) c[i] = coords_dev ? coords_dev[(uint64_t)b * d.rank + i] : host_coords.c[i];
  }
  const bool dma = dma_ok && c[0] >= 0 && c[1] >= 0 && (uint64_t)c[0] < d.dim[0] && (uint64_t)c[1] < d.dim[1] &&
                   ((c[0] * d.elsize) % 16) == 0;
  if (dma) {
    if (d.swizzle == 3) build_box_dma<3>(d, c, smem);
    else if (d.swizzle == kSwizzle128B2Row) build_box_dma<kSwizzle128B2Row>(d, c, smem);
    else build_box_dma<kSwizzleKnTr>(d, c, smem);
  } else {
    build_box_generic(d, c, smem, fill);
  }
  __syncthreads();
  uint8_t* out = dst + (uint64_t)b * d.image_bytes;
  const uint32_t nbytes = d.image_bytes;
  if ((((uintptr_t)out) % 16u) == 0 && (nbytes % 16u) == 0) {
    // Images are written once and not read again here: non-temporal stores keep them from
    // taking L2 space that the source rows of other boxes are using.
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    for (uint32_t i = threadIdx.x; i < nbytes / 16u; i += blockDim.x)
      __builtin_nontemporal_store(((const u32x4_t*)smem)[i], (u32x4_t*)out + i);
  } else {
    for (uint32_t i = threadIdx.x; i < nbytes; i += blockDim.x) out[i] = smem[i];
  }
}

// ---- store direction ("2 · Le Tensor Memory Accelerator" §2.5) -----------------------------
__device__ __forceinline__ void global_store_elem(uint8_t* dst, const uint8_t* lds, uint32_t off, int elsize) {
  if (elsize == 1) *dst = lds[off];
  else if (elsize == 2) *(uint16_t*)dst = *(const uint16_t*)(lds + off);
  else *(uint32_t*)dst = *(const uint32_t*)(lds + off);
}

// Scatter the LDS image of one box into the tensor: each position inside the tensor is written
// from the image offset a load of the same box would fill; positions outside are skipped.
// Whole 16-byte chunks go out as one store where the box row is chunk-aligned and the chunk
// lies inside the tensor (the swizzle moves 16-byte units whole, so a chunk is contiguous in
// the image too); ragged chunks and element-strided boxes go element by element.
__device__ void scatter_box(const DescImpl& d, const int64_t* c, const uint8_t* lds) {
  const int tid = threadIdx.x;
  const int es = d.elsize;
  const uint32_t row_bytes = (uint32_t)d.n[0] * es;
  const bool chunked = d.estr[0] == 1 && (row_bytes % 16u) == 0 && ((c[0] * es) % 16) == 0;
  if (!chunked) {
    const uint64_t total = d.image_bytes / es;
    for (uint64_t e = tid; e < total; e += blockDim.x) {
      uint64_t rem = e;
      bool inside = true;
      uint64_t dst = d.base;
      for (int i = 0; i < kMaxRank; ++i) {
        const uint64_t ni = d.n[i];
        const uint64_t j = rem % ni;
        rem /= ni;
        if (i < d.rank) {
          const int64_t x = c[i] + (int64_t)j * (int64_t)d.estr[i];
          if (x < 0 || (uint64_t)x >= d.dim[i]) inside = false;
          else dst += (uint64_t)x * d.stride[i];
        }
      }
      if (inside) global_store_elem((uint8_t*)dst, lds, swizzle_offset((uint32_t)(e * es), d.swizzle), es);
    }
    return;
  }
  const uint32_t chunks_per_row = row_bytes / 16u;
  const int epc = 16 / es;
  const uint32_t total_chunks = d.image_bytes / 16u;
  for (uint32_t ch = tid; ch < total_chunks; ch += blockDim.x) {
    const uint32_t row = ch / chunks_per_row;
    const uint32_t cr = ch % chunks_per_row;
    uint32_t rem = row;
    bool row_inside = true;
    uint64_t dst = d.base;
    for (int i = 1; i < kMaxRank; ++i) {
      const uint32_t ni = d.n[i];
      const uint32_t j = rem % ni;
      rem /= ni;
      if (i < d.rank) {
        const int64_t x = c[i] + (int64_t)j * (int64_t)d.estr[i];
        if (x < 0 || (uint64_t)x >= d.dim[i]) row_inside = false;
        else dst += (uint64_t)x * d.stride[i];
      }
    }
    if (!row_inside) continue;
    const int64_t x0 = c[0] + (int64_t)cr * epc;
    const uint32_t off = swizzle_offset(ch * 16u, d.swizzle);
    if (x0 >= 0 && (uint64_t)(x0 + epc) <= d.dim[0]) {
      *(uint4*)(dst + (uint64_t)x0 * es) = *(const uint4*)(lds + off);
    } else {
      for (int q = 0; q < epc; ++q) {
        const int64_t x = x0 + q;
        if (x >= 0 && (uint64_t)x < d.dim[0]) global_store_elem((uint8_t*)(dst + (uint64_t)x * es), lds, off + q * es, es);
      }
    }
  }
}

__global__ void __launch_bounds__(256) tiled_store_kernel(DescImpl d, Coords5 host_coords, const int32_t* coords_dev,
                                                          const uint8_t* src, uint32_t box_offset) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const uint32_t b = blockIdx.x + box_offset;
  int64_t c[kMaxRank];
  for (int i = 0; i < kMaxRank; ++i) {
    c[i] = 0;
    if (i < d.rank) c[i] = coords_dev ? coords_dev[(uint64_t)b * d.rank + i] : host_coords.c[i];
  }
  const uint8_t* in = src + (uint64_t)b * d.image_bytes;
  const uint32_t nbytes = d.image_bytes;
  if ((((uintptr_t)in) % 16u) == 0 && (nbytes % 16u) == 0) {
    for (uint32_t i = threadIdx.x; i < nbytes / 16u; i += blockDim.x) ((uint4*)smem)[i] = ((const uint4*)in)[i];
  } else {
    for (uint32_t i = threadIdx.x; i < nbytes; i += blockDim.x) smem[i] = in[i];
  }
  __syncthreads();
  scatter_box(d, c, smem);
}

hipError_t launch_tiled_store(const DescImpl& d, const int32_t* host_coords, const int32_t* coords_dev, uint32_t n,
                              const void* src, hipStream_t stream) {
  Coords5 hc{};
  if (host_coords)
    for (int i = 0; i < d.rank; ++i) hc.c[i] = host_coords[i];
  const size_t lds_bytes = ((size_t)d.image_bytes + 1023u) & ~(size_t)1023u;
  const uint32_t kMaxGrid = 1u << 20;
  for (uint32_t done = 0; done < n; done += kMaxGrid) {
    const uint32_t cnt = (n - done) < kMaxGrid ? (n - done) : kMaxGrid;
    hipLaunchKernelGGL(tiled_store_kernel, dim3(cnt), dim3(256), lds_bytes, stream, d, hc, coords_dev,
                       (const uint8_t*)src, done);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Host launcher.  Returns the HIP error of the launch.
hipError_t launch_tiled_copy(const DescImpl& d, const int32_t* host_coords, const int32_t* coords_dev, uint32_t n,
                             void* dst, hipStream_t stream) {
  Coords5 hc{};
  if (host_coords)
    for (int i = 0; i < d.rank; ++i) hc.c[i] = host_coords[i];
  const int dma_ok = d.rank == 2 && d.estr[0] == 1 && d.estr[1] == 1 && (uint32_t)d.box[0] * d.elsize == 128u &&
                     (d.box[1] % 8) == 0 && (d.swizzle == 3 || d.swizzle == kSwizzle128B2Row || d.swizzle == kSwizzleKnTr) && d.oob == 0 &&
                     ((d.dim[0] * d.elsize) % 16u) == 0 && d.stride[1] < (1ull << 23) &&
                     d.stride[1] >= d.dim[0] * d.elsize;
  uint32_t fill = 0;
  if (d.oob == 1) {
    // canonical quiet NaN of the element type, replicated to 32 bits
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
    hipLaunchKernelGGL(tiled_copy_kernel, dim3(cnt), dim3(256), lds_bytes, stream, d, hc, coords_dev, (uint8_t*)dst,
                       done, dma_ok, fill);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tbg
