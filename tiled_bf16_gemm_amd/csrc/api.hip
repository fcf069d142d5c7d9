// The C ABI (include/tbg.h): argument validation, descriptor encoding, operand packing and
// kernel dispatch.  Everything here runs on the host; kernels are enqueued on the caller's
// stream and never waited for.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "launch.hpp"
#include "tbg.h"
#include "tbg_desc.hpp"


using tbg::DescImpl;

namespace {

thread_local std::string g_last_error;

tbg_status fail(tbg_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tbg_status fail(tbg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

int elsize_of(int dtype) {
  switch (dtype) {
    case TBG_U8: case TBG_F8_E4M3: case TBG_F8_E5M2: return 1;
    case TBG_U16: case TBG_F16: case TBG_BF16: return 2;
    case TBG_U32: case TBG_F32: return 4;
    default: return 0;
  }
}

uint32_t swizzle_span(int mode) {
  switch (mode) {
    case TBG_SWIZZLE_32B: return 32;
    case TBG_SWIZZLE_64B: return 64;
    case TBG_SWIZZLE_128B: case TBG_SWIZZLE_128B_2ROW: case TBG_SWIZZLE_128B_TR: return 128;
    default: return 0;
  }
}

// A usable device: the current HIP device must be gfx950.  Checked once per device id, which
// also records the device's compute-unit count (returned through num_cus when given).
tbg_status check_device(int* num_cus = nullptr) {
  int dev = -1;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(TBG_ERR_NO_DEVICE, "no HIP device is visible");
  }
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(TBG_ERR_NO_DEVICE, "hipGetDevice failed");
  }
  static std::mutex mu;
  static int checked[64] = {0};  // 0 unknown, 1 ok, 2 wrong architecture
  static int cus[64] = {0};
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || dev >= 64) return fail(TBG_ERR_NO_DEVICE, "device id %d out of range", dev);
  if (checked[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(TBG_ERR_NO_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    }
    checked[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    cus[dev] = prop.multiProcessorCount;
    if (checked[dev] == 2) g_last_error = std::string("device is ") + prop.gcnArchName + ", not gfx950";
  }
  if (checked[dev] != 1) return fail(TBG_ERR_NO_DEVICE, "current device %d is not a gfx950 GPU", dev);
  if (num_cus) *num_cus = cus[dev];
  return TBG_OK;
}

bool valid_desc(const tbg_tensor_desc* d, const DescImpl** out) {
  if (!d) return false;
  const DescImpl* di = reinterpret_cast<const DescImpl*>(d);
  if (di->magic != tbg::kDescMagic || di->rank < 1 || di->rank > tbg::kMaxRank || di->image_bytes == 0) return false;
  *out = di;
  return true;
}

bool valid_im2col(const tbg_tensor_desc* d, const tbg::DescIm2col** out) {
  if (!d) return false;
  const tbg::DescIm2col* di = reinterpret_cast<const tbg::DescIm2col*>(d);
  if (di->magic != tbg::kIm2colMagic || di->image_bytes == 0) return false;
  *out = di;
  return true;
}

// Output extent of a convolution along one dimension (0 when the window never fits).
int64_t conv_out_dim(int64_t in, int64_t pad_lo, int64_t pad_hi, int64_t stride, int64_t dil, int64_t filt) {
  const int64_t span = in + pad_lo + pad_hi - dil * (filt - 1) - 1;
  if (stride < 1 || dil < 1 || filt < 1 || span < 0) return 0;
  return span / stride + 1;
}

// TBG_LOG set to anything but "" or "0": every GEMM and convolution call reports the kernel
// configuration it launches on stderr (read once per process).
void log_choice(const char* fmt, ...) {
  static const bool on = [] {
    const char* v = getenv("TBG_LOG");
    return v && *v && strcmp(v, "0") != 0;
  }();
  if (!on) return;
  va_list ap;
  va_start(ap, fmt);
  fputs("tbg: ", stderr);
  vfprintf(stderr, fmt, ap);
  fputc('\n', stderr);
  va_end(ap);
}

// Whether the epilogue may store whole 16-byte pieces of C's rows (8-byte pieces in the scaled
// bf16 path): gfx9's multi-dword memory instructions need only dword-aligned addresses, so C's
// base and its row pitch in bytes must be multiples of 4 (every fp32 C at a 4-byte aligned base;
// a bf16 C when ldc is even).  Otherwise the epilogue stores element by element.
int rows_dword_aligned(const void* C, int64_t ldc, tbg_dtype c_dtype) {
  return (((uintptr_t)C) % 4 == 0) && ((ldc * (c_dtype == TBG_BF16 ? 2 : 4)) % 4 == 0);
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

}  // namespace

extern "C" {

const char* tbg_status_string(tbg_status s) {
  switch (s) {
    case TBG_OK: return "TBG_OK";
    case TBG_ERR_INVALID_VALUE: return "TBG_ERR_INVALID_VALUE";
    case TBG_ERR_MISALIGNED: return "TBG_ERR_MISALIGNED";
    case TBG_ERR_UNSUPPORTED: return "TBG_ERR_UNSUPPORTED";
    case TBG_ERR_OUT_OF_RANGE: return "TBG_ERR_OUT_OF_RANGE";
    case TBG_ERR_NO_DEVICE: return "TBG_ERR_NO_DEVICE";
    case TBG_ERR_HIP: return "TBG_ERR_HIP";
    default: return "TBG_ERR_UNKNOWN";
  }
}

const char* tbg_last_error(void) { return g_last_error.c_str(); }

tbg_status tbg_encode_tiled(tbg_tensor_desc* out, tbg_dtype dtype, uint32_t rank, const void* global_address,
                            const uint64_t* global_dim, const uint64_t* global_strides, const uint32_t* box_dim,
                            const uint32_t* element_strides, tbg_swizzle swizzle, tbg_l2_hint l2, tbg_oob_fill oob) {
  if (!out) return fail(TBG_ERR_INVALID_VALUE, "out is NULL");
  const int es = elsize_of(dtype);
  if (es == 0) return fail(TBG_ERR_INVALID_VALUE, "unknown dtype %d", (int)dtype);
  if (rank < 1 || rank > (uint32_t)tbg::kMaxRank) return fail(TBG_ERR_UNSUPPORTED, "rank %u not in 1..5", rank);
  if (!global_address) return fail(TBG_ERR_INVALID_VALUE, "global_address is NULL");
  if (((uintptr_t)global_address) % 16 != 0)
    return fail(TBG_ERR_MISALIGNED, "global_address %p is not a multiple of 16 bytes", global_address);
  if (!global_dim || !box_dim || !element_strides || (rank > 1 && !global_strides))
    return fail(TBG_ERR_INVALID_VALUE, "a per-dimension array is NULL");
  if ((int)swizzle < TBG_SWIZZLE_NONE || (int)swizzle > TBG_SWIZZLE_128B_TR)
    return fail(TBG_ERR_INVALID_VALUE, "unknown swizzle %d", (int)swizzle);
  if ((int)l2 < TBG_L2_NONE || (int)l2 > TBG_L2_256B) return fail(TBG_ERR_INVALID_VALUE, "unknown l2 hint %d", (int)l2);
  if ((int)oob != TBG_OOB_ZERO && (int)oob != TBG_OOB_NAN)
    return fail(TBG_ERR_INVALID_VALUE, "unknown oob fill %d", (int)oob);
  if (oob == TBG_OOB_NAN && !(dtype == TBG_F16 || dtype == TBG_BF16 || dtype == TBG_F32 || dtype == TBG_F8_E4M3 ||
                              dtype == TBG_F8_E5M2))
    return fail(TBG_ERR_INVALID_VALUE, "NaN fill needs a floating-point element type");

  DescImpl d;
  memset(&d, 0, sizeof(d));
  d.magic = tbg::kDescMagic;
  d.dtype = (uint8_t)dtype;
  d.elsize = (uint8_t)es;
  d.rank = (uint8_t)rank;
  d.swizzle = (uint8_t)swizzle;
  d.oob = (uint8_t)oob;
  d.l2 = (uint8_t)l2;
  d.base = (uint64_t)(uintptr_t)global_address;
  uint64_t image = (uint64_t)es;
  for (int i = 0; i < tbg::kMaxRank; ++i) {
    d.dim[i] = 1;
    d.box[i] = 1;
    d.n[i] = 1;
    d.estr[i] = 1;
    d.stride[i] = 0;
  }
  d.stride[0] = (uint64_t)es;
  for (uint32_t i = 0; i < rank; ++i) {
    if (global_dim[i] < 1 || global_dim[i] > (1ull << 32))
      return fail(TBG_ERR_OUT_OF_RANGE, "global_dim[%u] = %llu not in 1..2^32", i, (unsigned long long)global_dim[i]);
    if (box_dim[i] < 1 || box_dim[i] > tbg::kMaxBox)
      return fail(TBG_ERR_OUT_OF_RANGE, "box_dim[%u] = %u not in 1..256", i, box_dim[i]);
    if (element_strides[i] < 1 || element_strides[i] > tbg::kMaxEstride)
      return fail(TBG_ERR_OUT_OF_RANGE, "element_strides[%u] = %u not in 1..8", i, element_strides[i]);
    d.dim[i] = global_dim[i];
    d.box[i] = (uint16_t)box_dim[i];
    d.estr[i] = (uint8_t)element_strides[i];
    d.n[i] = (uint16_t)((box_dim[i] + element_strides[i] - 1) / element_strides[i]);
    image *= d.n[i];
  }
  for (uint32_t i = 1; i < rank; ++i) {
    const uint64_t s = global_strides[i - 1];
    if (s % 16 != 0)
      return fail(TBG_ERR_MISALIGNED, "global_strides[%u] = %llu is not a multiple of 16 bytes", i - 1,
                  (unsigned long long)s);
    if (s == 0 || s >= (1ull << 40))
      return fail(TBG_ERR_OUT_OF_RANGE, "global_strides[%u] = %llu not in 16..2^40", i - 1, (unsigned long long)s);
    d.stride[i] = s;
  }
  if (image > tbg::kMaxImageBytes)
    return fail(TBG_ERR_OUT_OF_RANGE, "box image of %llu bytes exceeds 64 KiB", (unsigned long long)image);
  if (swizzle != TBG_SWIZZLE_NONE) {
    const uint32_t span = swizzle_span(swizzle);
    if ((uint64_t)box_dim[0] * es > span)
      return fail(TBG_ERR_INVALID_VALUE, "swizzled box inner extent %u bytes exceeds the %u-byte span",
                  (unsigned)(box_dim[0] * es), span);
    if (image % span != 0)
      return fail(TBG_ERR_INVALID_VALUE, "swizzled image of %llu bytes is not a multiple of the %u-byte span",
                  (unsigned long long)image, span);
  }
  d.image_bytes = (uint32_t)image;
  memcpy(out, &d, sizeof(d));
  return TBG_OK;
}

tbg_status tbg_encode_tiled_interleaved(tbg_tensor_desc* out, tbg_dtype dtype, uint32_t rank,
                                        const void* global_address, const uint64_t* global_dim,
                                        const uint64_t* global_strides, const uint32_t* box_dim,
                                        const uint32_t* element_strides, tbg_interleave interleave,
                                        tbg_swizzle swizzle, tbg_l2_hint l2, tbg_oob_fill oob) {
  if ((int)interleave < TBG_INTERLEAVE_NONE || (int)interleave > TBG_INTERLEAVE_32B)
    return fail(TBG_ERR_INVALID_VALUE, "unknown interleave %d", (int)interleave);
  if (interleave != TBG_INTERLEAVE_NONE) {
    const uint64_t width = interleave == TBG_INTERLEAVE_16B ? 16 : 32;
    const int es = elsize_of(dtype);
    if (es == 0) return fail(TBG_ERR_INVALID_VALUE, "unknown dtype %d", (int)dtype);
    if (rank < 3) return fail(TBG_ERR_UNSUPPORTED, "an interleaved layout needs rank >= 3 (got %u)", rank);
    if (rank > (uint32_t)tbg::kMaxRank) return fail(TBG_ERR_UNSUPPORTED, "rank %u not in 3..5", rank);
    if (!global_dim || !box_dim || !element_strides || !global_strides)
      return fail(TBG_ERR_INVALID_VALUE, "a per-dimension array is NULL");
    if (global_dim[0] * (uint64_t)es != width)
      return fail(TBG_ERR_INVALID_VALUE, "dimension 0 must be one %llu-byte channel slice (%llu elements of %d bytes)",
                  (unsigned long long)width, (unsigned long long)global_dim[0], es);
    if (box_dim[0] != global_dim[0] || element_strides[0] != 1)
      return fail(TBG_ERR_INVALID_VALUE, "an interleaved box takes whole channel slices (box_dim[0] = dim 0, "
                  "element_strides[0] = 1)");
    if (((uintptr_t)global_address) % width != 0)
      return fail(TBG_ERR_MISALIGNED, "global_address must be %llu-byte aligned for this interleave",
                  (unsigned long long)width);
    for (uint32_t i = 0; i + 1 < rank; ++i)
      if (global_strides[i] % width != 0)
        return fail(TBG_ERR_MISALIGNED, "global_strides[%u] must be a multiple of %llu bytes for this interleave", i,
                    (unsigned long long)width);
    if (interleave == TBG_INTERLEAVE_32B && swizzle != TBG_SWIZZLE_32B)
      return fail(TBG_ERR_INVALID_VALUE, "32-byte interleave requires the 32B swizzle");
  }
  tbg_status st = tbg_encode_tiled(out, dtype, rank, global_address, global_dim, global_strides, box_dim,
                                   element_strides, swizzle, l2, oob);
  if (st != TBG_OK) return st;
  reinterpret_cast<DescImpl*>(out)->interleave = (uint8_t)interleave;
  return TBG_OK;
}

size_t tbg_box_bytes(const tbg_tensor_desc* d) {
  const DescImpl* di = nullptr;
  if (valid_desc(d, &di)) return di->image_bytes;
  const tbg::DescIm2col* ii = nullptr;
  if (valid_im2col(d, &ii)) return ii->image_bytes;
  return 0;
}

tbg_status tbg_tiled_copy(const tbg_tensor_desc* d, const int32_t* coords, void* dst_image, void* stream) {
  const DescImpl* di = nullptr;
  if (!valid_desc(d, &di)) return fail(TBG_ERR_INVALID_VALUE, "not an encoded descriptor");
  if (!coords || !dst_image) return fail(TBG_ERR_INVALID_VALUE, "coords or dst_image is NULL");
  if (((uintptr_t)dst_image) % 16 != 0) return fail(TBG_ERR_MISALIGNED, "dst_image is not 16-byte aligned");
  tbg_status st = check_device();
  if (st != TBG_OK) return st;
  hipError_t e = tbg::launch_tiled_copy(*di, coords, nullptr, 1, dst_image, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "tiled copy launch: %s", hipGetErrorString(e));
  return TBG_OK;
}

tbg_status tbg_tiled_copy_many(const tbg_tensor_desc* d, const int32_t* coords_dev, uint32_t n, void* dst_images,
                               void* stream) {
  const DescImpl* di = nullptr;
  if (!valid_desc(d, &di)) return fail(TBG_ERR_INVALID_VALUE, "not an encoded descriptor");
  if (n == 0) return TBG_OK;
  if (!coords_dev || !dst_images) return fail(TBG_ERR_INVALID_VALUE, "coords_dev or dst_images is NULL");
  if (((uintptr_t)dst_images) % 16 != 0) return fail(TBG_ERR_MISALIGNED, "dst_images is not 16-byte aligned");
  tbg_status st = check_device();
  if (st != TBG_OK) return st;
  hipError_t e = tbg::launch_tiled_copy(*di, nullptr, coords_dev, n, dst_images, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "tiled copy launch: %s", hipGetErrorString(e));
  return TBG_OK;
}

tbg_status tbg_tiled_store(const tbg_tensor_desc* d, const int32_t* coords, const void* src_image, void* stream) {
  const DescImpl* di = nullptr;
  if (!valid_desc(d, &di)) return fail(TBG_ERR_INVALID_VALUE, "not an encoded descriptor");
  if (!coords || !src_image) return fail(TBG_ERR_INVALID_VALUE, "coords or src_image is NULL");
  if (((uintptr_t)src_image) % 16 != 0) return fail(TBG_ERR_MISALIGNED, "src_image is not 16-byte aligned");
  tbg_status st = check_device();
  if (st != TBG_OK) return st;
  hipError_t e = tbg::launch_tiled_store(*di, coords, nullptr, 1, src_image, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "tiled store launch: %s", hipGetErrorString(e));
  return TBG_OK;
}

tbg_status tbg_tiled_store_many(const tbg_tensor_desc* d, const int32_t* coords_dev, uint32_t n,
                                const void* src_images, void* stream) {
  const DescImpl* di = nullptr;
  if (!valid_desc(d, &di)) return fail(TBG_ERR_INVALID_VALUE, "not an encoded descriptor");
  if (n == 0) return TBG_OK;
  if (!coords_dev || !src_images) return fail(TBG_ERR_INVALID_VALUE, "coords_dev or src_images is NULL");
  if (((uintptr_t)src_images) % 16 != 0) return fail(TBG_ERR_MISALIGNED, "src_images is not 16-byte aligned");
  tbg_status st = check_device();
  if (st != TBG_OK) return st;
  hipError_t e = tbg::launch_tiled_store(*di, nullptr, coords_dev, n, src_images, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "tiled store launch: %s", hipGetErrorString(e));
  return TBG_OK;
}

tbg_status tbg_encode_im2col(tbg_tensor_desc* out, tbg_dtype dtype, const void* global_address,
                             const uint64_t* global_dim, const uint64_t* global_strides, const int32_t* pad_lo,
                             const int32_t* pad_hi, const int32_t* conv_stride, const int32_t* dilation,
                             const int32_t* filter, uint32_t channels, uint32_t pixels, tbg_swizzle swizzle,
                             tbg_l2_hint l2, tbg_oob_fill oob) {
  if (!out) return fail(TBG_ERR_INVALID_VALUE, "out is NULL");
  const int es = elsize_of(dtype);
  if (es == 0) return fail(TBG_ERR_INVALID_VALUE, "unknown dtype %d", (int)dtype);
  if (!global_address) return fail(TBG_ERR_INVALID_VALUE, "global_address is NULL");
  if (!global_dim || !global_strides || !pad_lo || !pad_hi || !conv_stride || !dilation || !filter)
    return fail(TBG_ERR_INVALID_VALUE, "a per-dimension array is NULL");
  if (((uintptr_t)global_address) % 16 != 0)
    return fail(TBG_ERR_MISALIGNED, "global_address %p is not a multiple of 16 bytes", global_address);
  if ((int)swizzle < TBG_SWIZZLE_NONE || (int)swizzle > TBG_SWIZZLE_128B_TR)
    return fail(TBG_ERR_INVALID_VALUE, "unknown swizzle %d", (int)swizzle);
  if ((int)l2 < TBG_L2_NONE || (int)l2 > TBG_L2_256B) return fail(TBG_ERR_INVALID_VALUE, "unknown l2 hint %d", (int)l2);
  if ((int)oob != TBG_OOB_ZERO && (int)oob != TBG_OOB_NAN)
    return fail(TBG_ERR_INVALID_VALUE, "unknown oob fill %d", (int)oob);
  if (oob == TBG_OOB_NAN && !(dtype == TBG_F16 || dtype == TBG_BF16 || dtype == TBG_F32 || dtype == TBG_F8_E4M3 ||
                              dtype == TBG_F8_E5M2))
    return fail(TBG_ERR_INVALID_VALUE, "NaN fill needs a floating-point element type");
  for (int i = 0; i < 4; ++i)
    if (global_dim[i] < 1 || global_dim[i] > (1ull << 31) - 1)
      return fail(TBG_ERR_OUT_OF_RANGE, "global_dim[%d] = %llu not in 1..2^31-1", i, (unsigned long long)global_dim[i]);
  for (int i = 0; i < 3; ++i) {
    if (global_strides[i] % 16 != 0)
      return fail(TBG_ERR_MISALIGNED, "global_strides[%d] = %llu is not a multiple of 16 bytes", i,
                  (unsigned long long)global_strides[i]);
    if (global_strides[i] == 0 || global_strides[i] >= (1ull << 40))
      return fail(TBG_ERR_OUT_OF_RANGE, "global_strides[%d] = %llu not in 16..2^40", i,
                  (unsigned long long)global_strides[i]);
  }
  for (int i = 0; i < 2; ++i) {
    if (filter[i] < 1 || filter[i] > 256) return fail(TBG_ERR_OUT_OF_RANGE, "filter[%d] = %d not in 1..256", i, filter[i]);
    if (conv_stride[i] < 1 || conv_stride[i] > 256)
      return fail(TBG_ERR_OUT_OF_RANGE, "conv_stride[%d] = %d not in 1..256", i, conv_stride[i]);
    if (dilation[i] < 1 || dilation[i] > 256)
      return fail(TBG_ERR_OUT_OF_RANGE, "dilation[%d] = %d not in 1..256", i, dilation[i]);
    if (pad_lo[i] < 0 || pad_lo[i] > 65535 || pad_hi[i] < 0 || pad_hi[i] > 65535)
      return fail(TBG_ERR_OUT_OF_RANGE, "padding along dimension %d not in 0..65535", i);
  }
  const int64_t ow = conv_out_dim((int64_t)global_dim[1], pad_lo[0], pad_hi[0], conv_stride[0], dilation[0], filter[0]);
  const int64_t oh = conv_out_dim((int64_t)global_dim[2], pad_lo[1], pad_hi[1], conv_stride[1], dilation[1], filter[1]);
  if (ow < 1 || oh < 1) return fail(TBG_ERR_INVALID_VALUE, "the filter window does not fit the padded image");
  if ((int64_t)global_dim[3] * oh * ow > INT32_MAX)
    return fail(TBG_ERR_UNSUPPORTED, "more than 2^31-1 output pixels");
  if (channels < 1 || channels > tbg::kMaxBox || pixels < 1 || pixels > tbg::kMaxBox)
    return fail(TBG_ERR_OUT_OF_RANGE, "channels %u and pixels %u must be in 1..256", channels, pixels);
  const uint64_t image = (uint64_t)es * channels * pixels;
  if (image > tbg::kMaxImageBytes)
    return fail(TBG_ERR_OUT_OF_RANGE, "box image of %llu bytes exceeds 64 KiB", (unsigned long long)image);
  if (swizzle != TBG_SWIZZLE_NONE) {
    const uint32_t span = swizzle_span(swizzle);
    if ((uint64_t)channels * es > span)
      return fail(TBG_ERR_INVALID_VALUE, "swizzled box inner extent %u bytes exceeds the %u-byte span",
                  (unsigned)(channels * es), span);
    if (image % span != 0)
      return fail(TBG_ERR_INVALID_VALUE, "swizzled image of %llu bytes is not a multiple of the %u-byte span",
                  (unsigned long long)image, span);
  }
  tbg::DescIm2col d;
  memset(&d, 0, sizeof(d));
  d.magic = tbg::kIm2colMagic;
  d.dtype = (uint8_t)dtype;
  d.elsize = (uint8_t)es;
  d.swizzle = (uint8_t)swizzle;
  d.oob = (uint8_t)oob;
  d.l2 = (uint8_t)l2;
  d.base = (uint64_t)(uintptr_t)global_address;
  for (int i = 0; i < 4; ++i) d.dim[i] = (uint32_t)global_dim[i];
  for (int i = 0; i < 3; ++i) d.stride[i] = global_strides[i];
  for (int i = 0; i < 2; ++i) {
    d.pad_lo[i] = pad_lo[i];
    d.pad_hi[i] = pad_hi[i];
    d.cstride[i] = conv_stride[i];
    d.dil[i] = dilation[i];
    d.filt[i] = filter[i];
  }
  d.out[0] = (uint32_t)ow;
  d.out[1] = (uint32_t)oh;
  d.channels = channels;
  d.pixels = pixels;
  d.image_bytes = (uint32_t)image;
  memcpy(out, &d, sizeof(d));
  return TBG_OK;
}

tbg_status tbg_im2col_copy(const tbg_tensor_desc* d, const int32_t* coords, void* dst_image, void* stream) {
  const tbg::DescIm2col* di = nullptr;
  if (!valid_im2col(d, &di)) return fail(TBG_ERR_INVALID_VALUE, "not an encoded im2col descriptor");
  if (!coords || !dst_image) return fail(TBG_ERR_INVALID_VALUE, "coords or dst_image is NULL");
  if (((uintptr_t)dst_image) % 16 != 0) return fail(TBG_ERR_MISALIGNED, "dst_image is not 16-byte aligned");
  tbg_status st = check_device();
  if (st != TBG_OK) return st;
  hipError_t e = tbg::launch_im2col_copy(*di, coords, nullptr, 1, dst_image, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "im2col copy launch: %s", hipGetErrorString(e));
  return TBG_OK;
}

tbg_status tbg_im2col_copy_many(const tbg_tensor_desc* d, const int32_t* coords_dev, uint32_t n, void* dst_images,
                                void* stream) {
  const tbg::DescIm2col* di = nullptr;
  if (!valid_im2col(d, &di)) return fail(TBG_ERR_INVALID_VALUE, "not an encoded im2col descriptor");
  if (n == 0) return TBG_OK;
  if (!coords_dev || !dst_images) return fail(TBG_ERR_INVALID_VALUE, "coords_dev or dst_images is NULL");
  if (((uintptr_t)dst_images) % 16 != 0) return fail(TBG_ERR_MISALIGNED, "dst_images is not 16-byte aligned");
  tbg_status st = check_device();
  if (st != TBG_OK) return st;
  hipError_t e = tbg::launch_im2col_copy(*di, nullptr, coords_dev, n, dst_images, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "im2col copy launch: %s", hipGetErrorString(e));
  return TBG_OK;
}

}  // extern "C"

namespace {

constexpr int64_t kMaxLd = (1ll << 22) - 1;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Where a call's repacked operands go in the caller's workspace.  A workspace of at least twice
// the need (each half 256-byte aligned) is used by halves, alternately from call to call (one
// counter for the process): a repack that overwrites the copy which the previous product has
// just read runs much slower on MI355X (the 3001×2049×777 operands: ≈8.5 µs, against ≈4.7 µs
// into the other half; kernel trace), and consecutive products usually share one workspace.
// The half only moves where the repack lands, never what the product computes.
uint8_t* repack_area(void* workspace, size_t workspace_bytes, size_t need) {
  static std::atomic<uint32_t> calls{0};
  const size_t half = (size_t)round_up((int64_t)need, 256);
  if (need == 0 || workspace_bytes < 2 * half) return (uint8_t*)workspace;
  return (uint8_t*)workspace + (calls.fetch_add(1, std::memory_order_relaxed) & 1u) * half;
}

struct PackPlan {
  bool pack_a = false, pack_b = false;
  int64_t kext = 0;
  int64_t lda_p = 0, ldb_p = 0;
  size_t a_bytes = 0, b_bytes = 0;
};

PackPlan plan_packs(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int bl, bool a_aligned,
                    bool b_aligned) {
  PackPlan pl;
  pl.kext = round_up(K, 8);
  if (K == 0) return pl;
  pl.pack_a = (lda % 8) != 0 || (K % 8) != 0 || !a_aligned;
  if (bl == TBG_B_NK) pl.pack_b = (ldb % 8) != 0 || (K % 8) != 0 || !b_aligned;
  else pl.pack_b = (ldb % 8) != 0 || !b_aligned;
  if (pl.pack_a) {
    pl.lda_p = pl.kext;
    pl.a_bytes = (size_t)round_up(M * pl.lda_p * 2, 256);
  }
  if (pl.pack_b) {
    if (bl == TBG_B_NK) {
      pl.ldb_p = pl.kext;
      pl.b_bytes = (size_t)round_up(N * pl.ldb_p * 2, 256);
    } else {
      pl.ldb_p = round_up(N, 8);
      pl.b_bytes = (size_t)round_up(K * pl.ldb_p * 2, 256);
    }
  }
  return pl;
}

// Repacks of 8-bit operands: rows whose pitch or K is not a multiple of 16 bytes, or that start
// off a 16-byte boundary, are copied with K rounded up to 16 (zero padded).  B is stored N×K.
struct Fp8PackPlan {
  bool pack_a = false, pack_b = false;
  int64_t k16 = 16;
  size_t a_bytes = 0, b_bytes = 0;
};

Fp8PackPlan plan_fp8_packs(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, bool a_aligned, bool b_aligned) {
  Fp8PackPlan pl;
  pl.k16 = round_up(K > 0 ? K : 1, 16);
  pl.pack_a = K > 0 && ((lda % 16) != 0 || (K % 16) != 0 || !a_aligned);
  pl.pack_b = K > 0 && ((ldb % 16) != 0 || (K % 16) != 0 || !b_aligned);
  pl.a_bytes = pl.pack_a ? (size_t)round_up(M * pl.k16, 256) : 0;
  pl.b_bytes = pl.pack_b ? (size_t)round_up(N * pl.k16, 256) : 0;
  return pl;
}

bool is_f8(tbg_dtype t) { return t == TBG_F8_E4M3 || t == TBG_F8_E5M2; }

}  // namespace

extern "C" {

size_t tbg_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, tbg_b_layout bl) {
  if (M <= 0 || N <= 0 || K <= 0 || lda <= 0 || ldb <= 0) return 0;
  PackPlan pl = plan_packs(M, N, K, lda, ldb, (int)bl, true, true);
  return pl.a_bytes + pl.b_bytes;
}

size_t tbg_gemm_workspace_query(int64_t M, int64_t N, int64_t K, tbg_dtype ab_dtype, const void* A, int64_t lda,
                                const void* B, int64_t ldb, tbg_b_layout bl) {
  if (M <= 0 || N <= 0 || K <= 0 || lda <= 0 || ldb <= 0) return 0;
  const bool a_aligned = ((uintptr_t)A % 16) == 0, b_aligned = ((uintptr_t)B % 16) == 0;
  if (is_f8(ab_dtype)) {
    const Fp8PackPlan pl = plan_fp8_packs(M, N, K, lda, ldb, a_aligned, b_aligned);
    return pl.a_bytes + pl.b_bytes;
  }
  if (ab_dtype != TBG_BF16 && ab_dtype != TBG_F16) return 0;
  const PackPlan pl = plan_packs(M, N, K, lda, ldb, (int)bl, a_aligned, b_aligned);
  return pl.a_bytes + pl.b_bytes;
}

}  // extern "C"

namespace {

tbg_status gemm_impl(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                     int64_t ldb, tbg_b_layout bl, float beta, void* C, int64_t ldc, tbg_dtype c_dtype,
                     const tbg_gemm_config* cfg, void* workspace, size_t workspace_bytes, void* stream, bool scaled,
                     tbg_dtype ab_dtype = TBG_BF16);

// The operand boxes of a product as this library's descriptors, encoded (and so checked) by
// tbg_encode_tiled ("2 · Le Tensor Memory Accelerator" §2.3: the descriptor is built once on the
// host and handed to the kernel): A {K, M} with box {one 128-byte row of K, bm}; B stored N×K
// {K, N} with box {one 128-byte row of K, bn}, both with the 2-row swizzle; B stored K×N {N, K}
// with box {64, 64} and the transposing-read swizzle; zero fill.  These are the boxes and layouts
// the kernels copy into their LDS stages.  K = 0: no operand is read and both stay zero.
tbg_status encode_operand_boxes(tbg::GemmParams& p, tbg_dtype ab, tbg_b_layout bl, int bm, int bn, int64_t M,
                                int64_t N, int64_t K, const void* A, int64_t lda_bytes, const void* B,
                                int64_t ldb_bytes) {
  memset(&p.da, 0, sizeof(p.da));
  memset(&p.db, 0, sizeof(p.db));
  if (K == 0) return TBG_OK;
  static_assert(sizeof(tbg_tensor_desc) == sizeof(tbg::DescImpl), "descriptor sizes");
  const uint32_t row = (ab == TBG_F8_E4M3 || ab == TBG_F8_E5M2) ? 128u : 64u;  // elements per 128 bytes
  const uint32_t one[2] = {1, 1};
  tbg_tensor_desc d;
  {
    const uint64_t dims[2] = {(uint64_t)K, (uint64_t)M};
    const uint64_t strides[1] = {(uint64_t)lda_bytes};
    const uint32_t box[2] = {row, (uint32_t)bm};
    const tbg_status st =
        tbg_encode_tiled(&d, ab, 2, A, dims, strides, box, one, TBG_SWIZZLE_128B_2ROW, TBG_L2_NONE, TBG_OOB_ZERO);
    if (st != TBG_OK) return st;
    memcpy(&p.da, &d, sizeof(d));
  }
  {
    const bool nk = bl == TBG_B_NK;
    const uint64_t dims[2] = {(uint64_t)(nk ? K : N), (uint64_t)(nk ? N : K)};
    const uint64_t strides[1] = {(uint64_t)ldb_bytes};
    const uint32_t box[2] = {nk ? row : 64u, nk ? (uint32_t)bn : 64u};
    const tbg_status st = tbg_encode_tiled(&d, ab, 2, B, dims, strides, box, one,
                                           nk ? TBG_SWIZZLE_128B_2ROW : TBG_SWIZZLE_128B_TR, TBG_L2_NONE, TBG_OOB_ZERO);
    if (st != TBG_OK) return st;
    memcpy(&p.db, &d, sizeof(d));
  }
  return TBG_OK;
}

// The fp8 product: operands are byte matrices, repacked to 16-byte pitches with zero padding
// where needed, then handed to the kernel as 16-bit pairs.
tbg_status gemm_fp8_impl(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                         int64_t ldb, tbg_b_layout bl, tbg_dtype ab_dtype, float beta, void* C, int64_t ldc,
                         tbg_dtype c_dtype, const tbg_gemm_config* cfg, void* workspace, size_t workspace_bytes,
                         void* stream, bool scaled) {
  if (M < 0 || N < 0 || K < 0) return fail(TBG_ERR_INVALID_VALUE, "negative size M=%lld N=%lld K=%lld",
                                          (long long)M, (long long)N, (long long)K);
  if ((int)bl != TBG_B_KN && (int)bl != TBG_B_NK) return fail(TBG_ERR_INVALID_VALUE, "unknown b_layout %d", (int)bl);
  if (bl != TBG_B_NK) return fail(TBG_ERR_UNSUPPORTED, "8-bit inputs need B stored N×K (TBG_B_NK)");
  int bm = 0, bn = 0;
  if (cfg) {
    if (cfg->pipeline != TBG_PIPE_AUTO && cfg->pipeline != TBG_PIPE_RING)
      return fail(TBG_ERR_UNSUPPORTED, "the fp8 product runs on the barrier ring only");
    if (cfg->stages != 0 && cfg->stages != 2) return fail(TBG_ERR_UNSUPPORTED, "the fp8 ring has 2 stages");
    if ((cfg->tile_m == 0) != (cfg->tile_n == 0))
      return fail(TBG_ERR_INVALID_VALUE, "tile_m and tile_n must both be 0 or both be set");
    if (cfg->tile_m != 0 && !tbg::fp8_tile_built(cfg->tile_m, cfg->tile_n))
      return fail(TBG_ERR_UNSUPPORTED, "no fp8 kernel with tile %dx%d (built: 256x256, 128x128, 64x64)", cfg->tile_m,
                  cfg->tile_n);
    bm = cfg->tile_m;
    bn = cfg->tile_n;
  }
  if (scaled && alpha == 0.f)
    return gemm_impl(M, N, 0, 0.f, nullptr, 1, nullptr, 1, TBG_B_NK, beta, C, ldc, c_dtype, nullptr, nullptr, 0,
                     stream, true, TBG_BF16);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(TBG_ERR_UNSUPPORTED, "sizes must stay below 2^31");
  if (c_dtype != TBG_F32 && c_dtype != TBG_BF16) return fail(TBG_ERR_INVALID_VALUE, "C must be TBG_F32 or TBG_BF16");
  if (lda < (K > 0 ? K : 1)) return fail(TBG_ERR_INVALID_VALUE, "lda=%lld < K=%lld", (long long)lda, (long long)K);
  if (ldb < (K > 0 ? K : 1)) return fail(TBG_ERR_INVALID_VALUE, "ldb=%lld < K=%lld", (long long)ldb, (long long)K);
  if (ldc < (N > 0 ? N : 1)) return fail(TBG_ERR_INVALID_VALUE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
  if (lda > 2 * kMaxLd || ldb > 2 * kMaxLd || ldc > (1ll << 40))
    return fail(TBG_ERR_UNSUPPORTED, "leading dimensions are limited to 2^23-2 bytes");
  if (M == 0 || N == 0) return TBG_OK;
  if (!C) return fail(TBG_ERR_INVALID_VALUE, "C is NULL");
  if (K > 0 && (!A || !B)) return fail(TBG_ERR_INVALID_VALUE, "A or B is NULL");
  const Fp8PackPlan fpl = plan_fp8_packs(M, N, K, lda, ldb, ((uintptr_t)A % 16) == 0, ((uintptr_t)B % 16) == 0);
  const int64_t k16 = fpl.k16;
  const bool pack_a = fpl.pack_a, pack_b = fpl.pack_b;
  const size_t a_bytes = fpl.a_bytes, b_bytes = fpl.b_bytes;
  if (a_bytes + b_bytes > 0) {
    if (!workspace || workspace_bytes < a_bytes + b_bytes)
      return fail(TBG_ERR_OUT_OF_RANGE, "workspace of %zu bytes needed to repack unaligned operands (have %zu)",
                  a_bytes + b_bytes, workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace) % 256 != 0) return fail(TBG_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  }
  int num_cus = 0;
  tbg_status st = check_device(&num_cus);
  if (st != TBG_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* Ab = (const uint8_t*)A;
  const uint8_t* Bb = (const uint8_t*)B;
  int64_t lda_b = lda, ldb_b = ldb;
  hipError_t e = hipSuccess;
  tbg::PackJob jobs[2];
  int njobs = 0;
  uint8_t* const area = repack_area(workspace, workspace_bytes, a_bytes + b_bytes);
  if (pack_a) {
    uint8_t* dst = area;
    jobs[njobs++] = tbg::PackJob{Ab, lda, M, K, dst, k16};
    Ab = dst;
    lda_b = k16;
  }
  if (pack_b) {
    uint8_t* dst = area + a_bytes;
    jobs[njobs++] = tbg::PackJob{Bb, ldb, N, K, dst, k16};
    Bb = dst;
    ldb_b = k16;
  }
  e = tbg::launch_pack_jobs(jobs, njobs, s);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "fp8 repack: %s", hipGetErrorString(e));
  tbg::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A = (const uint16_t*)Ab;
  p.B = (const uint16_t*)Bb;
  p.C = C;
  p.lda = lda_b / 2;
  p.ldb = ldb_b / 2;
  p.ldc = ldc;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)(K > 0 ? k16 / 2 : 0);
  p.kchunks = K > 0 ? (int)(k16 / 16) : 0;  // K = 0: every copy lane masked, A and B never read
  p.group_m = 8;
  p.vec_store = rows_dword_aligned(C, ldc, c_dtype);
  p.alpha = alpha;
  p.beta = beta;
  p.scaled = scaled ? 1 : 0;
  if (bm == 0) {
    // the ring's cost model over the fp8 tiles
    double best = 0;
    const struct { int bm, bn; double eff; } tiles[] = {{256, 256, 1.0}, {128, 128, 0.82}, {64, 64, 0.52}};
    const int cus = num_cus > 0 ? num_cus : 256;
    for (const auto& t : tiles) {
      const int64_t ntiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
      const double cost = (double)((ntiles + cus - 1) / cus) * t.bm * t.bn / t.eff;
      if (best == 0 || cost < best * 0.999) {
        best = cost;
        bm = t.bm;
        bn = t.bn;
      }
    }
  }
  st = encode_operand_boxes(p, ab_dtype, bl, bm, bn, M, N, K, Ab, lda_b, Bb, ldb_b);
  if (st != TBG_OK) return st;
  log_choice("gemm M=%lld N=%lld K=%lld B=nk in=%s out=%s: ring %dx%d, 2 stages; repack A %s, B %s", (long long)M,
             (long long)N, (long long)K, ab_dtype == TBG_F8_E5M2 ? "e5m2" : "e4m3", c_dtype == TBG_BF16 ? "bf16" : "f32",
             bm, bn, pack_a ? "yes" : "no", pack_b ? "yes" : "no");
  e = tbg::launch_fp8(p, bm, bn, ab_dtype == TBG_F8_E5M2 ? 1 : 0, c_dtype == TBG_BF16, s);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "fp8 gemm launch: %s", hipGetErrorString(e));
  return TBG_OK;
}

// C = alpha·A·B + beta·C (scaled) or C = A·B.  With alpha == 0 the product is skipped: K is taken
// as 0 and A, B and their leading dimensions are not looked at.
tbg_status gemm_impl(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                     int64_t ldb, tbg_b_layout bl, float beta, void* C, int64_t ldc, tbg_dtype c_dtype,
                     const tbg_gemm_config* cfg, void* workspace, size_t workspace_bytes, void* stream, bool scaled,
                     tbg_dtype ab_dtype) {
  if (ab_dtype == TBG_F8_E4M3 || ab_dtype == TBG_F8_E5M2)
    return gemm_fp8_impl(M, N, K, alpha, A, lda, B, ldb, bl, ab_dtype, beta, C, ldc, c_dtype, cfg, workspace,
                         workspace_bytes, stream, scaled);
  if (ab_dtype != TBG_BF16 && ab_dtype != TBG_F16)
    return fail(TBG_ERR_INVALID_VALUE, "A and B must be TBG_BF16, TBG_F16, TBG_F8_E4M3 or TBG_F8_E5M2 (got %d)",
                (int)ab_dtype);
  const int in = ab_dtype == TBG_F16 ? 1 : 0;
  if (M < 0 || N < 0 || K < 0) return fail(TBG_ERR_INVALID_VALUE, "negative size M=%lld N=%lld K=%lld",
                                          (long long)M, (long long)N, (long long)K);
  if ((int)bl != TBG_B_KN && (int)bl != TBG_B_NK) return fail(TBG_ERR_INVALID_VALUE, "unknown b_layout %d", (int)bl);
  // Kernel configuration: checked in full before anything else can fail on a machine without a
  // device, so that the checks are the same everywhere.
  int pipeline = 0, bm = 0, bn = 0, stages = 0;  // 0: left to the library
  if (cfg) {
    if (cfg->pipeline != TBG_PIPE_AUTO && cfg->pipeline != TBG_PIPE_RING && cfg->pipeline != TBG_PIPE_PRODUCER)
      return fail(TBG_ERR_INVALID_VALUE, "unknown pipeline %d", (int)cfg->pipeline);
    if ((cfg->tile_m == 0) != (cfg->tile_n == 0))
      return fail(TBG_ERR_INVALID_VALUE, "tile_m and tile_n must both be 0 or both be set");
    if (cfg->stages < 0 || cfg->stages == 1) return fail(TBG_ERR_INVALID_VALUE, "stages must be 0 or >= 2");
    pipeline = cfg->pipeline == TBG_PIPE_RING ? tbg::kPipeRing
               : cfg->pipeline == TBG_PIPE_PRODUCER ? tbg::kPipeProducer : 0;
    bm = cfg->tile_m;
    bn = cfg->tile_n;
    stages = cfg->stages;
    tbg::GemmChoice probe;
    // Whether anything built matches what is fixed does not depend on the shape or the device.
    if (!tbg::choose_gemm(256, 256, 256, pipeline, bm, bn, stages, probe, in))
      return fail(TBG_ERR_UNSUPPORTED, "no %s%s kernel with tile %dx%d and %d stages (built: ring %s; producer %s)",
                  in ? "fp16 " : "bf16 ",
                  pipeline == tbg::kPipeProducer ? "producer/consumer" : pipeline == tbg::kPipeRing ? "ring" : "",
                  bm, bn, stages, tbg::gemm_configs_text(tbg::kPipeRing, in),
                  tbg::gemm_configs_text(tbg::kPipeProducer, in));
  }
  if (scaled && alpha == 0.f) {  // the empty product: nothing of A or B is used
    K = 0;
    A = B = nullptr;
    lda = ldb = 1;
    bl = TBG_B_NK;
  }
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(TBG_ERR_UNSUPPORTED, "sizes must stay below 2^31");
  if (c_dtype != TBG_F32 && c_dtype != TBG_BF16) return fail(TBG_ERR_INVALID_VALUE, "C must be TBG_F32 or TBG_BF16");
  if (lda < (K > 0 ? K : 1)) return fail(TBG_ERR_INVALID_VALUE, "lda=%lld < K=%lld", (long long)lda, (long long)K);
  const int64_t ldb_min = bl == TBG_B_KN ? N : K;
  if (ldb < (ldb_min > 0 ? ldb_min : 1))
    return fail(TBG_ERR_INVALID_VALUE, "ldb=%lld below its minimum %lld", (long long)ldb, (long long)ldb_min);
  if (ldc < (N > 0 ? N : 1)) return fail(TBG_ERR_INVALID_VALUE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
  if (lda > kMaxLd || ldb > kMaxLd || ldc > (1ll << 40))
    return fail(TBG_ERR_UNSUPPORTED, "leading dimensions are limited to 2^22-1 elements");
  if (M == 0 || N == 0) return TBG_OK;
  if (!C) return fail(TBG_ERR_INVALID_VALUE, "C is NULL");
  if (K > 0 && (!A || !B)) return fail(TBG_ERR_INVALID_VALUE, "A or B is NULL");

  const bool a_aligned = ((uintptr_t)A % 16) == 0, b_aligned = ((uintptr_t)B % 16) == 0;
  PackPlan pl = plan_packs(M, N, K, lda, ldb, (int)bl, a_aligned, b_aligned);
  const size_t need = pl.a_bytes + pl.b_bytes;
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(TBG_ERR_OUT_OF_RANGE, "workspace of %zu bytes needed to repack unaligned operands (have %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace) % 256 != 0) return fail(TBG_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  }
  int num_cus = 0;
  tbg_status st = check_device(&num_cus);
  if (st != TBG_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* Ae = (const uint16_t*)A;
  const uint16_t* Be = (const uint16_t*)B;
  int64_t lda_e = lda, ldb_e = ldb;
  hipError_t e = hipSuccess;
  tbg::PackJob jobs[2];
  int njobs = 0;
  uint8_t* const area = repack_area(workspace, workspace_bytes, need);
  if (pl.pack_a) {
    uint16_t* dst = (uint16_t*)area;
    jobs[njobs++] = tbg::PackJob{(const uint8_t*)A, lda * 2, M, K * 2, (uint8_t*)dst, pl.lda_p * 2};
    Ae = dst;
    lda_e = pl.lda_p;
  }
  if (pl.pack_b) {
    uint16_t* dst = (uint16_t*)(area + pl.a_bytes);
    const int64_t rows = bl == TBG_B_NK ? N : K, cols = bl == TBG_B_NK ? K : N;
    jobs[njobs++] = tbg::PackJob{(const uint8_t*)B, ldb * 2, rows, cols * 2, (uint8_t*)dst, pl.ldb_p * 2};
    Be = dst;
    ldb_e = pl.ldb_p;
  }
  e = tbg::launch_pack_jobs(jobs, njobs, s);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "operand repack: %s", hipGetErrorString(e));
  tbg::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A = Ae;
  p.B = Be;
  p.C = C;
  p.lda = lda_e;
  p.ldb = ldb_e;
  p.ldc = ldc;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.kchunks = (int)(pl.kext / 8);
  // Kernel configuration: what the caller fixed, the rest chosen from the shape and the device.
  tbg::GemmChoice ch;
  if (!tbg::choose_gemm(M, N, num_cus, pipeline, bm, bn, stages, ch, in))
    return fail(TBG_ERR_UNSUPPORTED, "no built kernel matches tile %dx%d with %d stages", bm, bn, stages);
  p.tiles_m = 0;
  p.tiles_n = 0;
  // Tile-group height of the XCD-aware order: 4 and 8 are level on 8192^3, 4 is ≈0.5 % faster on
  // 16384×14336×4096; 2, 16 and 32 are slower.
  p.group_m = env_int("TBG_GROUP_M", 4);
  if (p.group_m < 1) p.group_m = 1;
  p.vec_store = rows_dword_aligned(C, ldc, c_dtype);
  p.alpha = alpha;
  p.beta = beta;
  p.scaled = scaled ? 1 : 0;
  st = encode_operand_boxes(p, ab_dtype, bl, ch.bm, ch.bn, M, N, K, Ae, lda_e * 2, Be, ldb_e * 2);
  if (st != TBG_OK) return st;
  log_choice("gemm M=%lld N=%lld K=%lld B=%s in=%s out=%s: %s %dx%d, %d stages; repack A %s, B %s", (long long)M,
             (long long)N, (long long)K, bl == TBG_B_KN ? "kn" : "nk", in ? "f16" : "bf16",
             c_dtype == TBG_BF16 ? "bf16" : "f32", ch.pipeline == tbg::kPipeProducer ? "producer" : "ring", ch.bm,
             ch.bn, ch.stages, pl.pack_a ? "yes" : "no", pl.pack_b ? "yes" : "no");
  e = tbg::launch_gemm(p, ch.pipeline, ch.bm, ch.bn, ch.stages, (int)bl, c_dtype == TBG_BF16, s, in);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "gemm launch: %s", hipGetErrorString(e));
  return TBG_OK;
}

}  // namespace

// The allocation-free product's repack area: a file-scope device array, one per GPU the library
// runs on, held until the process ends.  Host code never passes `scratch` itself to a kernel or
// a copy (on the host the name stands for a host-side shadow, not the device memory): it uses the
// device address that hipGetSymbolAddress returns for the current device (scratch_ptr).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per device with that device
// current (each GPU holds its own copy at its own address).
tbg_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return fail(TBG_ERR_NO_DEVICE, "no current HIP device");
  }
  static std::mutex mu;
  static void* ptrs[64] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(TBG_ERR_HIP, "hipGetSymbolAddress of the scratch array on device %d: %s", dev, hipGetErrorString(e));
    }
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return TBG_OK;
}

}  // namespace

extern "C" {

tbg_status tbg_gemm_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                            tbg_b_layout bl, void* C, int64_t ldc, tbg_dtype c_dtype, void* stream) {
  // Sizes and operands that need no repack go straight to tbg_gemm's path; the argument checks
  // are tbg_gemm's own.
  const size_t need = tbg_gemm_workspace_query(M, N, K, TBG_BF16, A, lda, B, ldb, bl);
  if (need == 0)
    return gemm_impl(M, N, K, 1.f, A, lda, B, ldb, bl, 0.f, C, ldc, c_dtype, nullptr, nullptr, 0, stream, false);
  if (need > kNoAllocScratchBytes)
    return fail(TBG_ERR_OUT_OF_RANGE,
                "the operands' repack needs %zu bytes; the allocation-free product holds %zu bytes of scratch "
                "(use tbg_gemm with a workspace)", need, kNoAllocScratchBytes);
  tbg_status st = check_device();
  if (st != TBG_OK) return st;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != TBG_OK) return st;
  return gemm_impl(M, N, K, 1.f, A, lda, B, ldb, bl, 0.f, C, ldc, c_dtype, nullptr, ws, kNoAllocScratchBytes, stream,
                   false);
}

size_t tbg_gemm_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

tbg_status tbg_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                    tbg_b_layout bl, void* C, int64_t ldc, tbg_dtype c_dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return gemm_impl(M, N, K, 1.f, A, lda, B, ldb, bl, 0.f, C, ldc, c_dtype, nullptr, workspace, workspace_bytes, stream,
                   false);
}

tbg_status tbg_gemm_ex(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                       int64_t ldb, tbg_b_layout bl, float beta, void* C, int64_t ldc, tbg_dtype c_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const bool scaled = !(alpha == 1.f && beta == 0.f);
  return gemm_impl(M, N, K, alpha, A, lda, B, ldb, bl, beta, C, ldc, c_dtype, nullptr, workspace, workspace_bytes,
                   stream, scaled);
}

tbg_status tbg_gemm_typed(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                          int64_t ldb, tbg_b_layout bl, tbg_dtype ab_dtype, float beta, void* C, int64_t ldc,
                          tbg_dtype c_dtype, const tbg_gemm_config* cfg, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const bool scaled = !(alpha == 1.f && beta == 0.f);
  return gemm_impl(M, N, K, alpha, A, lda, B, ldb, bl, beta, C, ldc, c_dtype, cfg, workspace, workspace_bytes, stream,
                   scaled, ab_dtype);
}

tbg_status tbg_gemm_configured(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                               const void* B, int64_t ldb, tbg_b_layout bl, float beta, void* C, int64_t ldc,
                               tbg_dtype c_dtype, const tbg_gemm_config* cfg, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!cfg) return fail(TBG_ERR_INVALID_VALUE, "cfg is NULL");
  const bool scaled = !(alpha == 1.f && beta == 0.f);
  return gemm_impl(M, N, K, alpha, A, lda, B, ldb, bl, beta, C, ldc, c_dtype, cfg, workspace, workspace_bytes, stream,
                   scaled);
}


}  // extern "C"

namespace {

struct ConvPlan {
  int64_t oh = 0, ow = 0, m = 0, c8 = 0;
  bool pack = false;
  size_t x_bytes = 0, w_bytes = 0;  // packed sizes (256-byte rounded) when pack
};

tbg_status conv_plan(const tbg_conv2d_shape* sh, bool x_aligned, bool w_aligned, ConvPlan& pl) {
  if (!sh) return fail(TBG_ERR_INVALID_VALUE, "shape is NULL");
  if (sh->n < 1 || sh->h < 1 || sh->w < 1 || sh->c < 1 || sh->k < 1)
    return fail(TBG_ERR_INVALID_VALUE, "n, h, w, c and k must be at least 1");
  if (sh->r < 1 || sh->s < 1 || sh->stride_h < 1 || sh->stride_w < 1 || sh->dil_h < 1 || sh->dil_w < 1)
    return fail(TBG_ERR_INVALID_VALUE, "filter sizes, strides and dilations must be at least 1");
  if (sh->pad_h < 0 || sh->pad_w < 0 || sh->pad_h_end < 0 || sh->pad_w_end < 0)
    return fail(TBG_ERR_INVALID_VALUE, "padding must not be negative");
  if (sh->r > 256 || sh->s > 256 || sh->stride_h > 256 || sh->stride_w > 256 || sh->dil_h > 256 || sh->dil_w > 256 ||
      sh->pad_h > 65535 || sh->pad_w > 65535 || sh->pad_h_end > 65535 || sh->pad_w_end > 65535)
    return fail(TBG_ERR_UNSUPPORTED, "filter, stride and dilation are limited to 256, padding to 65535");
  pl.oh = conv_out_dim(sh->h, sh->pad_h, sh->pad_h_end, sh->stride_h, sh->dil_h, sh->r);
  pl.ow = conv_out_dim(sh->w, sh->pad_w, sh->pad_w_end, sh->stride_w, sh->dil_w, sh->s);
  if (pl.oh < 1 || pl.ow < 1) return fail(TBG_ERR_INVALID_VALUE, "the filter window does not fit the padded image");
  pl.m = sh->n * pl.oh * pl.ow;
  pl.c8 = (sh->c + 7) / 8 * 8;
  if (pl.m > INT32_MAX || sh->k > INT32_MAX || sh->h > 65535 || sh->w > 65535)
    return fail(TBG_ERR_UNSUPPORTED, "sizes beyond this library's limits (output pixels and k below 2^31, h and w below 2^16)");
  const int64_t x_elems = sh->n * sh->h * sh->w * pl.c8;
  const int64_t ldw = (int64_t)sh->r * sh->s * pl.c8;
  if (x_elems * 2 >= (1ll << 31)) return fail(TBG_ERR_UNSUPPORTED, "the input tensor must stay below 2 GiB");
  if (ldw > (1ll << 22) - 1) return fail(TBG_ERR_UNSUPPORTED, "r*s*c is limited to 2^22-1");
  pl.pack = (sh->c % 8) != 0 || !x_aligned || !w_aligned;
  if (pl.pack) {
    pl.x_bytes = (size_t)((x_elems * 2 + 255) / 256 * 256);
    pl.w_bytes = (size_t)((sh->k * ldw * 2 + 255) / 256 * 256);
  }
  return TBG_OK;
}

}  // namespace

extern "C" {

tbg_status tbg_conv2d_out_dims(const tbg_conv2d_shape* shape, int64_t* oh, int64_t* ow) {
  ConvPlan pl;
  tbg_status st = conv_plan(shape, true, true, pl);
  if (st != TBG_OK) return st;
  if (oh) *oh = pl.oh;
  if (ow) *ow = pl.ow;
  return TBG_OK;
}

size_t tbg_conv2d_workspace_bytes(const tbg_conv2d_shape* shape) {
  ConvPlan pl;
  if (conv_plan(shape, true, true, pl) != TBG_OK) return 0;
  return pl.x_bytes + pl.w_bytes;
}

size_t tbg_conv2d_workspace_query(const tbg_conv2d_shape* shape, const void* x, const void* w) {
  ConvPlan pl;
  if (conv_plan(shape, ((uintptr_t)x % 16) == 0, ((uintptr_t)w % 16) == 0, pl) != TBG_OK) return 0;
  return pl.x_bytes + pl.w_bytes;
}

tbg_status tbg_conv2d_fwd(const tbg_conv2d_shape* shape, float alpha, const void* x, const void* w, float beta,
                          void* y, int64_t ldy, tbg_dtype y_dtype, const tbg_gemm_config* cfg, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const bool x_aligned = ((uintptr_t)x % 16) == 0, w_aligned = ((uintptr_t)w % 16) == 0;
  ConvPlan pl;
  tbg_status st = conv_plan(shape, x_aligned, w_aligned, pl);
  if (st != TBG_OK) return st;
  // tile 448x128 names the halo kernel (stride 1: the input window copied once per channel block)
  const bool want_halo = cfg && cfg->tile_m == 448 && cfg->tile_n == 128;
  if (cfg) {
    if (cfg->pipeline != TBG_PIPE_AUTO && cfg->pipeline != TBG_PIPE_RING)
      return fail(TBG_ERR_UNSUPPORTED, "the convolution runs on the barrier ring only");
    if (want_halo ? (cfg->stages != 0 && cfg->stages != 4) : (cfg->stages != 0 && cfg->stages != 2))
      return fail(TBG_ERR_UNSUPPORTED, want_halo ? "the halo convolution has 4 filter stages"
                                                 : "the convolution ring has 2 stages");
    if ((cfg->tile_m == 0) != (cfg->tile_n == 0))
      return fail(TBG_ERR_INVALID_VALUE, "tile_m and tile_n must both be 0 or both be set");
    if (cfg->tile_m != 0 && !want_halo && !tbg::conv_tile_built(cfg->tile_m, cfg->tile_n))
      return fail(TBG_ERR_UNSUPPORTED,
                  "no convolution kernel with tile %dx%d (built: 256x256, 256x128, 128x128, 64x64; 448x128 halo)",
                  cfg->tile_m, cfg->tile_n);
  }
  if (y_dtype != TBG_F32 && y_dtype != TBG_BF16) return fail(TBG_ERR_INVALID_VALUE, "y must be TBG_F32 or TBG_BF16");
  if (ldy < shape->k) return fail(TBG_ERR_INVALID_VALUE, "ldy=%lld < k=%lld", (long long)ldy, (long long)shape->k);
  if (ldy > (1ll << 40)) return fail(TBG_ERR_UNSUPPORTED, "ldy is limited to 2^40");
  if (!y) return fail(TBG_ERR_INVALID_VALUE, "y is NULL");
  const bool scaled = !(alpha == 1.f && beta == 0.f);
  const bool skip_product = scaled && alpha == 0.f;
  if (!skip_product && (!x || !w)) return fail(TBG_ERR_INVALID_VALUE, "x or w is NULL");
  const size_t need = pl.x_bytes + pl.w_bytes;
  if (!skip_product && need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(TBG_ERR_OUT_OF_RANGE, "workspace of %zu bytes needed to repack the channels (have %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace) % 256 != 0) return fail(TBG_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  }
  int num_cus = 0;
  st = check_device(&num_cus);
  if (st != TBG_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (skip_product) {
    // alpha == 0: C <- beta·C through the GEMM's epilogue with an empty product
    return gemm_impl(pl.m, shape->k, 0, 0.f, nullptr, 1, nullptr, 1, TBG_B_NK, beta, y, ldy, y_dtype, nullptr,
                     nullptr, 0, stream, true);
  }
  const uint16_t* X = (const uint16_t*)x;
  const uint16_t* W = (const uint16_t*)w;
  const int64_t ldw = (int64_t)shape->r * shape->s * pl.c8;
  if (pl.pack) {
    uint8_t* const area = repack_area(workspace, workspace_bytes, need);
    uint16_t* xp = (uint16_t*)area;
    uint16_t* wp = (uint16_t*)(area + pl.x_bytes);
    const tbg::PackJob jobs[2] = {
        {(const uint8_t*)X, shape->c * 2, shape->n * shape->h * shape->w, shape->c * 2, (uint8_t*)xp, pl.c8 * 2},
        {(const uint8_t*)W, shape->c * 2, shape->k * shape->r * shape->s, shape->c * 2, (uint8_t*)wp, pl.c8 * 2}};
    e = tbg::launch_pack_jobs(jobs, 2, s);
    if (e != hipSuccess) return fail(TBG_ERR_HIP, "channel repack: %s", hipGetErrorString(e));
    X = xp;
    W = wp;
  }
  tbg::ConvParams cp;
  memset(&cp, 0, sizeof(cp));
  cp.g.A = X;
  cp.g.B = W;
  cp.g.C = y;
  cp.g.lda = pl.c8;
  cp.g.ldb = ldw;
  cp.g.ldc = ldy;
  cp.g.M = (int)pl.m;
  cp.g.N = (int)shape->k;
  cp.g.K = (int)(ldw);
  cp.g.kchunks = (int)(ldw / 8);
  cp.g.group_m = 8;
  cp.g.vec_store = rows_dword_aligned(y, ldy, y_dtype);
  cp.g.alpha = alpha;
  cp.g.beta = beta;
  cp.g.scaled = scaled ? 1 : 0;
  cp.X = X;
  cp.W = W;
  cp.ldw = ldw;
  cp.x_bytes = (uint32_t)(shape->n * shape->h * shape->w * pl.c8 * 2);
  cp.n = (int)shape->n;
  cp.h = (int)shape->h;
  cp.w = (int)shape->w;
  cp.c8 = (int)pl.c8;
  cp.r = shape->r;
  cp.s = shape->s;
  cp.oh = (int)pl.oh;
  cp.ow = (int)pl.ow;
  cp.ph = shape->pad_h;
  cp.pw = shape->pad_w;
  cp.sh = shape->stride_h;
  cp.sw = shape->stride_w;
  cp.dh = shape->dil_h;
  cp.dw = shape->dil_w;
  cp.cblocks = (int)((pl.c8 + 63) / 64);
  // The halo kernel, where the shape allows it (stride 1, channels a multiple of 32 with nothing
  // repacked, a window that fits LDS): forced by tile 448x128, chosen by the library when its
  // tiles use at least 3/4 of their rows and fill at least half of the compute units.
  tbg::HaloParams hp;
  memset(&hp, 0, sizeof(hp));
  int hs = 0;
  const char* why = "channels a multiple of 32 and 16-byte aligned x and w";
  hp.c = cp;
  const bool halo_ok = !pl.pack && shape->c % 32 == 0 && tbg::plan_conv_halo(hp, &hs, &why);
  if (want_halo && !halo_ok) return fail(TBG_ERR_UNSUPPORTED, "the 448x128 halo convolution needs %s", why);
  const int cus_h = num_cus > 0 ? num_cus : 256;
  const bool auto_halo = halo_ok && (!cfg || cfg->tile_m == 0) &&
                         4 * pl.oh * pl.ow >= 3 * (int64_t)hp.tpi * 448 &&
                         2 * (int64_t)hp.c.g.tiles_m * hp.c.g.tiles_n >= cus_h;
  if (want_halo || auto_halo) {
    log_choice("conv2d N=%lld H=%lld W=%lld C=%lld K=%lld %dx%d: halo 448x128, %d output rows per tile, "
               "window %dx%d, %d atoms per wave and tap",
               (long long)shape->n, (long long)shape->h, (long long)shape->w, (long long)shape->c,
               (long long)shape->k, shape->r, shape->s, hp.tr, hp.hh, hp.hw, hs);
    e = tbg::launch_conv_halo(hp, hs, y_dtype == TBG_BF16, s);
    if (e != hipSuccess) return fail(TBG_ERR_HIP, "convolution launch: %s", hipGetErrorString(e));
    return TBG_OK;
  }
  // Workgroup tile: the GEMM ring's cost model (tiles per busiest CU × tile work / measured
  // efficiency relative to 256×256) over the tiles built for convolution.
  int bm = 256, bn = 256;
  double best = 0;
  const struct { int bm, bn; double eff; } tiles[] = {{256, 256, 1.0}, {128, 128, 0.82}, {256, 128, 0.73},
                                                      {64, 64, 0.52}};
  const int cus = num_cus > 0 ? num_cus : 256;
  for (const auto& t : tiles) {
    const int64_t ntiles = ((pl.m + t.bm - 1) / t.bm) * ((shape->k + t.bn - 1) / t.bn);
    const int64_t rounds = (ntiles + cus - 1) / cus;
    const double cost = (double)rounds * t.bm * t.bn / t.eff;
    if (best == 0 || cost < best * 0.999) {
      best = cost;
      bm = t.bm;
      bn = t.bn;
    }
  }
  if (cfg && cfg->tile_m != 0) {
    bm = cfg->tile_m;
    bn = cfg->tile_n;
  }
  log_choice("conv2d N=%lld H=%lld W=%lld C=%lld K=%lld %dx%d (GEMM %lld x %lld x %lld): ring %dx%d, 2 stages",
             (long long)shape->n, (long long)shape->h, (long long)shape->w, (long long)shape->c, (long long)shape->k,
             shape->r, shape->s, (long long)cp.g.M, (long long)cp.g.N, (long long)(shape->r * shape->s * cp.c8), bm, bn);
  e = tbg::launch_conv(cp, bm, bn, y_dtype == TBG_BF16, s);
  if (e != hipSuccess) return fail(TBG_ERR_HIP, "convolution launch: %s", hipGetErrorString(e));
  return TBG_OK;
}

}  // extern "C"
