// GEMM dispatch: the table of built kernel configurations (pipeline × workgroup tile × ring
// stages), the choice of a tile for a shape, and the packing kernel for operands whose rows are
// not 16-byte aligned.  The kernels themselves are in gemm_ring.hpp (every compute wave copies
// its share of each stage, one barrier per stage) and gemm_pc.hpp (dedicated producer waves,
// per-stage full/empty counters), instantiated in gemm_ring_*.hip and gemm_pc_*.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <string>

#include "fast_div.hpp"
#include "launch.hpp"

namespace tbg {

// The packing step for operands whose rows are not 16-byte aligned ("GEMM" page: packing a block
// into a contiguous area before use; 16-byte alignment of the leading dimension, section "In
// pratica"): copy `rows` rows of `row_bytes` bytes into a buffer of pitch `ld_dst` bytes (a
// multiple of 16), zero-filling bytes row_bytes..ld_dst-1.  One thread per 16-byte chunk of the
// destination.  The chunk's 16 source bytes may start at any byte: the thread loads the two
// aligned 16-byte blocks that hold them (consecutive lanes load consecutive blocks, so every load
// instruction is one contiguous run) and funnel-shifts them into place.  The second block is
// clamped to the aligned block that holds the row's last byte, and the bytes past the row are
// zeroed, so no load leaves the 16-byte blocks the row touches (those never cross a page).
// Offsets inside a row are 32-bit (a row is below 2^24 bytes; the callers check the pitches).
__device__ __forceinline__ uint4 pack_chunk(const PackJob& j, uint64_t r, uint32_t b0) {
  const uint32_t rb = (uint32_t)j.row_bytes;
  if (b0 >= rb) return make_uint4(0, 0, 0, 0);
  const uint8_t* srow = j.src + r * (uint64_t)j.ld_src;
  const uint32_t mis = (uint32_t)((uintptr_t)srow & 15);  // the row's offset from a 16-byte boundary
  const uint8_t* blocks = srow - mis;                      // the aligned block holding its first byte
  const uint32_t last = ((mis + rb - 1) >> 4) << 4;        // the block holding its last byte
  const uint4 q0 = *(const uint4*)(blocks + b0);
  const uint4 q1 = *(const uint4*)(blocks + (b0 + 16 <= last ? b0 + 16 : last));
  // the 32 loaded bytes shifted down by `mis`: by 8 bytes, by 4, then alignbyte by the rest
  // (named registers: an indexed array here is lowered through memory)
  const bool s8 = mis & 8, s4 = mis & 4;
  const uint32_t sh = mis & 3;
  const uint32_t y0 = s8 ? q0.z : q0.x, y1 = s8 ? q0.w : q0.y, y2 = s8 ? q1.x : q0.z, y3 = s8 ? q1.y : q0.w,
                 y4 = s8 ? q1.z : q1.x, y5 = s8 ? q1.w : q1.y;
  const uint32_t z0 = s4 ? y1 : y0, z1 = s4 ? y2 : y1, z2 = s4 ? y3 : y2, z3 = s4 ? y4 : y3, z4 = s4 ? y5 : y4;
  uint32_t o[4] = {__builtin_amdgcn_alignbyte(z1, z0, sh), __builtin_amdgcn_alignbyte(z2, z1, sh),
                   __builtin_amdgcn_alignbyte(z3, z2, sh), __builtin_amdgcn_alignbyte(z4, z3, sh)};
  const uint32_t valid = rb - b0;  // bytes of this chunk inside the row
  if (valid < 16) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (valid < 4u * k + 4) o[k] &= valid <= 4u * k ? 0u : ((1u << (8 * (valid - 4 * k))) - 1u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Two repacks in one launch.  Workgroups 0..blocks0-1 take j0's chunks, the rest j1's, so the job
// is uniform over a workgroup (its fields stay in scalar registers); chunks are numbered
// row-major over a job's rows × chunks-per-row.
struct PackGrid {
  uint32_t chunks0, chunks1;  // chunks of each repack
  uint32_t cpr0, cpr1;        // destination chunks per row of each repack
  FastDiv div0, div1;         // division by cpr0, cpr1
};

__global__ void __launch_bounds__(256) pack_rows_kernel(PackJob j0, PackJob j1, PackGrid g) {
  const uint32_t blocks0 = (g.chunks0 + 255) / 256;
  const bool second = blockIdx.x >= blocks0;
  const PackJob& j = second ? j1 : j0;
  const uint32_t i = (blockIdx.x - (second ? blocks0 : 0u)) * 256u + threadIdx.x;
  if (i >= (second ? g.chunks1 : g.chunks0)) return;
  const uint32_t r = fast_div(i, second ? g.div1 : g.div0);
  const uint32_t c = i - r * (second ? g.cpr1 : g.cpr0);
  *(uint4*)(j.dst + (uint64_t)r * (uint64_t)j.ld_dst + c * 16u) = pack_chunk(j, r, c * 16u);
}

// The same for repacks of 2^32 - 256 chunks (64 GiB) or more: 64-bit chunk numbers, numbered flat
// over both repacks, the grid stepping through them.
__global__ void __launch_bounds__(256) pack_rows_wide_kernel(PackJob j0, PackJob j1, uint64_t n0, uint64_t total,
                                                             uint32_t cpr0, uint32_t cpr1) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const bool second = t >= n0;
    const PackJob& j = second ? j1 : j0;
    const uint64_t i = second ? t - n0 : t;
    const uint32_t cpr = second ? cpr1 : cpr0;
    const uint64_t r = i / cpr;
    const uint32_t c = (uint32_t)(i % cpr);
    *(uint4*)(j.dst + r * (uint64_t)j.ld_dst + c * 16u) = pack_chunk(j, r, c * 16u);
  }
}

hipError_t launch_pack_jobs(const PackJob* jobs, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  uint64_t chunks[2] = {0, 0};
  uint32_t cpr[2] = {1, 1};
  for (int i = 0; i < n; ++i) {
    if (jobs[i].ld_dst >= (1ll << 31) || jobs[i].row_bytes > jobs[i].ld_dst) return hipErrorInvalidValue;
    cpr[i] = (uint32_t)(jobs[i].ld_dst / 16);
    chunks[i] = (uint64_t)cpr[i] * (uint64_t)jobs[i].rows;
  }
  const PackJob& j1 = n > 1 ? jobs[1] : jobs[0];
  if (chunks[0] + chunks[1] == 0) return hipSuccess;
  const uint64_t limit = (1ull << 32) - 256;
  if (chunks[0] < limit && chunks[1] < limit) {
    const PackGrid g{(uint32_t)chunks[0], (uint32_t)chunks[1], cpr[0], cpr[1], make_fast_div(cpr[0]),
                     make_fast_div(cpr[1])};
    const uint64_t blocks = (chunks[0] + 255) / 256 + (chunks[1] + 255) / 256;
    hipLaunchKernelGGL(pack_rows_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, jobs[0], j1, g);
  } else {
    const uint64_t total = chunks[0] + chunks[1], blocks = (total + 255) / 256;
    const uint32_t grid = blocks < (1u << 20) ? (uint32_t)blocks : (1u << 20);
    hipLaunchKernelGGL(pack_rows_wide_kernel, dim3(grid), dim3(256), 0, stream, jobs[0], j1, chunks[0], total, cpr[0],
                       cpr[1]);
  }
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
    {kPipeRing, 64, 64, 3, 1, &launch_ring<64, 64, 3, 1>},
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
// compute waves free of copy instructions and run ≈8 % faster than as a two-stage ring, while the
// 128×128 and 64×64 tiles lose the second workgroup per compute unit to the extra waves and run
// slower.
namespace {
struct Candidate {
  int pipeline, bm, bn, stages;
  double eff;
};
// Candidates of equal cost keep the first listed: the 128×128 ring comes before the 128×256 producer
// ring (on 3008×2056×784, where their costs tie, the ring's kernel took 19.4 µs, the producer's 21.0).
const Candidate kCandidates[] = {
    {kPipeRing, 256, 256, 2, 1.00},     {kPipeRing, 128, 128, 2, 0.76},     {kPipeProducer, 128, 256, 2, 0.75},
    {kPipeProducer, 256, 128, 2, 0.75}, {kPipeRing, 256, 128, 2, 0.70},     {kPipeRing, 128, 256, 2, 0.69},
    {kPipeProducer, 128, 128, 3, 0.61}, {kPipeRing, 64, 64, 3, 0.43},       {kPipeProducer, 64, 64, 3, 0.33},
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
