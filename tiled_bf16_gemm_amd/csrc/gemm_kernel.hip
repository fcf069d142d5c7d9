// GEMM dispatch: the table of built kernel configurations (pipeline × workgroup tile × ring
// stages), the choice of a tile for a shape, and the packing kernel for operands whose rows are
// not 16-byte aligned.  The kernels themselves are in gemm_ring.hpp (every compute wave copies
// its share of each stage, one barrier per stage) and gemm_pc.hpp (dedicated producer waves,
// per-stage full/empty counters), instantiated in gemm_ring_*.hip and gemm_pc_*.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <string>

#include "launch.hpp"

namespace tbg {

// Copy `rows` rows of `cols` bf16 values into a buffer of pitch ld_dst (a multiple of 8),
// zero-filling columns cols..ld_dst-1: the packing step for operands whose rows are not 16-byte
// aligned ("GEMM" page: packing a block into a contiguous area before use; 16-byte alignment of
// the leading dimension, section "In pratica").
__global__ void __launch_bounds__(256) pack_rows_kernel(const uint16_t* src, int64_t ld_src, int64_t rows,
                                                        int64_t cols, uint16_t* dst, int64_t ld_dst) {
  const int64_t cpr = ld_dst / 8;
  const int64_t total = rows * cpr;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / cpr;
    const int64_t c0 = (idx - r * cpr) * 8;
    uint16_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (c0 + j < cols) ? src[r * ld_src + c0 + j] : (uint16_t)0;
    uint4 w;
    w.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
    w.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
    w.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
    w.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
    *(uint4*)(dst + r * ld_dst + c0) = w;
  }
}

hipError_t launch_pack(const uint16_t* src, int64_t ld_src, int64_t rows, int64_t cols, uint16_t* dst, int64_t ld_dst,
                       hipStream_t stream) {
  const int64_t total = rows * (ld_dst / 8);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, ld_src, rows, cols, dst,
                     ld_dst);
  return hipGetLastError();
}

// Byte rows: copy `rows` rows of `cols` bytes into a buffer of pitch ld_dst (a multiple of 16),
// zero-filling bytes cols..ld_dst-1 (the packing step for 8-bit operands).
__global__ void __launch_bounds__(256) pack_bytes_kernel(const uint8_t* src, int64_t ld_src, int64_t rows,
                                                         int64_t cols, uint8_t* dst, int64_t ld_dst) {
  const int64_t cpr = ld_dst / 16;
  const int64_t total = rows * cpr;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / cpr;
    const int64_t c0 = (idx - r * cpr) * 16;
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (c0 + j < cols) w[j >> 2] |= (uint32_t)src[r * ld_src + c0 + j] << (8 * (j & 3));
    *(uint4*)(dst + r * ld_dst + c0) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_pack_bytes(const uint8_t* src, int64_t ld_src, int64_t rows, int64_t cols, uint8_t* dst,
                             int64_t ld_dst, hipStream_t stream) {
  const int64_t total = rows * (ld_dst / 16);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_bytes_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, ld_src, rows, cols, dst,
                     ld_dst);
  return hipGetLastError();
}

namespace {

struct GemmVariant {
  int pipeline, bm, bn, stages, in;
  GemmLauncher fn;
};

// Every built configuration.  The ring runs every tile; 256×256 has room for two stages only
// (2 × 64 KiB of the 160 KiB of LDS).  The producer/consumer ring needs registers for its producer
// waves next to the compute waves, which the 256×256 tile does not leave.
const GemmVariant kVariants[] = {
    {kPipeRing, 256, 256, 2, 0, &launch_ring<256, 256, 2, 0>},
    {kPipeRing, 256, 128, 2, 0, &launch_ring<256, 128, 2, 0>},
    {kPipeRing, 256, 128, 3, 0, &launch_ring<256, 128, 3, 0>},
    {kPipeRing, 128, 256, 2, 0, &launch_ring<128, 256, 2, 0>},
    {kPipeRing, 128, 256, 3, 0, &launch_ring<128, 256, 3, 0>},
    {kPipeRing, 128, 128, 2, 0, &launch_ring<128, 128, 2, 0>},
    {kPipeRing, 128, 128, 3, 0, &launch_ring<128, 128, 3, 0>},
    {kPipeRing, 128, 128, 4, 0, &launch_ring<128, 128, 4, 0>},
    {kPipeRing, 128, 128, 5, 0, &launch_ring<128, 128, 5, 0>},
    {kPipeRing, 64, 64, 2, 0, &launch_ring<64, 64, 2, 0>},
    {kPipeRing, 64, 64, 3, 0, &launch_ring<64, 64, 3, 0>},
    {kPipeRing, 64, 64, 4, 0, &launch_ring<64, 64, 4, 0>},
    {kPipeRing, 64, 64, 5, 0, &launch_ring<64, 64, 5, 0>},
    {kPipeRing, 64, 64, 6, 0, &launch_ring<64, 64, 6, 0>},
    {kPipeProducer, 256, 128, 2, 0, &launch_pc<256, 128, 2, 0>},
    {kPipeProducer, 256, 128, 3, 0, &launch_pc<256, 128, 3, 0>},
    {kPipeProducer, 128, 256, 2, 0, &launch_pc<128, 256, 2, 0>},
    {kPipeProducer, 128, 256, 3, 0, &launch_pc<128, 256, 3, 0>},
    {kPipeProducer, 128, 128, 2, 0, &launch_pc<128, 128, 2, 0>},
    {kPipeProducer, 128, 128, 3, 0, &launch_pc<128, 128, 3, 0>},
    {kPipeProducer, 128, 128, 4, 0, &launch_pc<128, 128, 4, 0>},
    {kPipeProducer, 64, 64, 2, 0, &launch_pc<64, 64, 2, 0>},
    {kPipeProducer, 64, 64, 3, 0, &launch_pc<64, 64, 3, 0>},
    {kPipeProducer, 64, 64, 4, 0, &launch_pc<64, 64, 4, 0>},
    {kPipeProducer, 64, 64, 5, 0, &launch_pc<64, 64, 5, 0>},
    {kPipeProducer, 64, 64, 6, 0, &launch_pc<64, 64, 6, 0>},
    // fp16 inputs: the configurations of the automatic choice
    {kPipeRing, 256, 256, 2, 1, &launch_ring<256, 256, 2, 1>},
    {kPipeRing, 256, 128, 2, 1, &launch_ring<256, 128, 2, 1>},
    {kPipeRing, 128, 256, 2, 1, &launch_ring<128, 256, 2, 1>},
    {kPipeRing, 128, 128, 2, 1, &launch_ring<128, 128, 2, 1>},
    {kPipeRing, 64, 64, 2, 1, &launch_ring<64, 64, 2, 1>},
    {kPipeProducer, 256, 128, 2, 1, &launch_pc<256, 128, 2, 1>},
    {kPipeProducer, 128, 256, 2, 1, &launch_pc<128, 256, 2, 1>},
    {kPipeProducer, 128, 128, 3, 1, &launch_pc<128, 128, 3, 1>},
    {kPipeProducer, 64, 64, 3, 1, &launch_pc<64, 64, 3, 1>},
};

}  // namespace

GemmLauncher find_gemm(int pipeline, int bm, int bn, int stages, int in) {
  for (const GemmVariant& v : kVariants)
    if (v.pipeline == pipeline && v.bm == bm && v.bn == bn && v.stages == stages && v.in == in) return v.fn;
  return nullptr;
}

namespace {
std::string configs_of(int pipeline, int in) {
  std::string t;
  for (const GemmVariant& v : kVariants) {
    if (v.pipeline != pipeline || v.in != in) continue;
    char buf[48];
    snprintf(buf, sizeof(buf), "%s%dx%d/%d", t.empty() ? "" : ", ", v.bm, v.bn, v.stages);
    t += buf;
  }
  return t;
}
}  // namespace

const char* gemm_configs_text(int pipeline, int in) {
  static const std::string ring = configs_of(kPipeRing, 0), pc = configs_of(kPipeProducer, 0);
  static const std::string ring16 = configs_of(kPipeRing, 1), pc16 = configs_of(kPipeProducer, 1);
  if (in == 1) return pipeline == kPipeProducer ? pc16.c_str() : ring16.c_str();
  return pipeline == kPipeProducer ? pc.c_str() : ring.c_str();
}

// Candidates of the automatic choice: every built (pipeline, tile) pair with its default stage
// count and its efficiency — throughput on the 8192³ and 16384×14336×4096 products relative to
// the 256×256 ring (measured with the configuration sweep of bench.py).  Fragment reads and copies
// per product grow as the tile shrinks; the 128×128 ring and the 64×64 tiles run two workgroups
// per compute unit; with dedicated producer waves the 256×128 and 128×256 tiles keep their
// compute waves free of copy instructions and run 18 % faster than as a ring, while the 128×128
// and 64×64 tiles lose the second workgroup per compute unit to the extra waves or the deeper
// ring and run slower.  Deeper rings lose occupancy and never win at the default.
namespace {
struct Candidate {
  int pipeline, bm, bn, stages;
  double eff;
};
const Candidate kCandidates[] = {
    {kPipeRing, 256, 256, 2, 1.00},     {kPipeProducer, 256, 128, 2, 0.86}, {kPipeProducer, 128, 256, 2, 0.86},
    {kPipeRing, 128, 128, 2, 0.82},     {kPipeRing, 256, 128, 2, 0.73},     {kPipeRing, 128, 256, 2, 0.72},
    {kPipeProducer, 128, 128, 3, 0.69}, {kPipeRing, 64, 64, 2, 0.52},       {kPipeProducer, 64, 64, 3, 0.34},
};
}  // namespace

// Each candidate's cost is the number of tiles the busiest compute unit computes times the work
// of one tile divided by the candidate's efficiency; the cheapest wins (the 256×256 ring whenever
// it fills the machine).
bool choose_gemm(int64_t M, int64_t N, int num_cus, int pipeline, int bm, int bn, int stages, GemmChoice& out,
                 int in) {
  const int cus = num_cus > 0 ? num_cus : 256;
  double best = 0;
  bool found = false;
  for (const Candidate& c : kCandidates) {
    if (pipeline != 0 && c.pipeline != pipeline) continue;
    if (bm != 0 && (c.bm != bm || c.bn != bn)) continue;
    const int st = stages != 0 ? stages : c.stages;
    if (!find_gemm(c.pipeline, c.bm, c.bn, st, in)) continue;
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const int64_t rounds = (tiles + cus - 1) / cus;
    const double cost = (double)(rounds > 0 ? rounds : 1) * c.bm * c.bn / c.eff;
    if (!found || cost < best * 0.999) {
      best = cost;
      out = GemmChoice{c.pipeline, c.bm, c.bn, st};
      found = true;
    }
  }
  return found;
}

hipError_t launch_gemm(GemmParams p, int pipeline, int bm, int bn, int stages, int b_layout, int out_bf16,
                       hipStream_t stream, int in) {
  const GemmLauncher fn = find_gemm(pipeline, bm, bn, stages, in);
  if (!fn) return hipErrorInvalidValue;
  p.tiles_m = (int)((p.M + bm - 1) / bm);
  p.tiles_n = (int)((p.N + bn - 1) / bn);
  if ((int64_t)p.tiles_m * p.tiles_n == 0) return hipSuccess;
  return fn(p, b_layout, out_bf16, stream);
}

}  // namespace tbg
