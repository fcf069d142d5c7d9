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

// The packing step for operands whose rows are not 16-byte aligned ("GEMM" page: packing a block
// into a contiguous area before use; 16-byte alignment of the leading dimension, section "In
// pratica"): copy `rows` rows of `row_bytes` bytes into a buffer of pitch `ld_dst` bytes (a
// multiple of 16), zero-filling bytes row_bytes..ld_dst-1.  One thread per 16-byte chunk of the
// destination: it reads the five aligned dwords that hold the chunk's source bytes (the source may
// sit at any byte alignment) and funnel-shifts them into place.  Near the row's end the dword
// reads stop at the dword that holds the row's last byte and the bytes past the row are zeroed,
// so every lane runs the same instructions and no read leaves the dwords of the row.  Both
// operands of a product are packed by one launch.
__device__ __forceinline__ uint4 pack_chunk(const PackJob& j, int64_t r, int64_t b0) {
  const int64_t valid = j.row_bytes - b0;  // bytes of this chunk inside the row
  if (valid <= 0) return make_uint4(0, 0, 0, 0);
  const uint8_t* srow = j.src + r * j.ld_src;
  const uintptr_t a = (uintptr_t)(srow + b0);
  const uint32_t* q = (const uint32_t*)(a & ~(uintptr_t)3);
  const uint32_t sh = (uint32_t)(a & 3);
  const uint32_t* qlast = (const uint32_t*)((uintptr_t)(srow + j.row_bytes - 1) & ~(uintptr_t)3);
  const int64_t nlast = qlast - q;
  uint32_t w[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) w[i] = q[i < nlast ? i : nlast];
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[k] = __builtin_amdgcn_alignbyte(w[k + 1], w[k], sh);
    const int64_t keep = valid - 4 * k;  // bytes of this dword inside the row
    if (keep < 4) o[k] &= keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Blocks of 64 chunks × 4 rows, numbered flat: blocks below `b0` pack j0, the rest j1, so each
// repack gets exactly its own blocks when the two operands have different shapes.  Workgroups
// step through the blocks by the grid size.
struct PackGrid {
  uint32_t b0, total;  // blocks of the first repack; blocks of both
  uint32_t gx0, gx1;   // blocks across a row of each repack
};

__global__ void __launch_bounds__(256) pack_rows_kernel(PackJob j0, PackJob j1, PackGrid g) {
  for (uint32_t blk = blockIdx.x; blk < g.total; blk += gridDim.x) {
    const bool second = blk >= g.b0;
    const PackJob& j = second ? j1 : j0;
    const uint32_t w = second ? blk - g.b0 : blk;
    const uint32_t gx = second ? g.gx1 : g.gx0;
    const int64_t r = (int64_t)(w / gx) * 4 + threadIdx.y;
    const int64_t c = (int64_t)(w % gx) * 64 + threadIdx.x;
    if (r >= j.rows || c >= j.ld_dst / 16) continue;
    *(uint4*)(j.dst + r * j.ld_dst + c * 16) = pack_chunk(j, r, c * 16);
  }
}

hipError_t launch_pack_jobs(const PackJob* jobs, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  uint64_t gx[2] = {1, 1}, blocks[2] = {0, 0};
  for (int i = 0; i < n; ++i) {
    gx[i] = (uint64_t)(jobs[i].ld_dst / 16 + 63) / 64;
    blocks[i] = gx[i] * (uint64_t)((jobs[i].rows + 3) / 4);
  }
  if (blocks[0] + blocks[1] >= (1ull << 32)) return hipErrorInvalidValue;
  const PackGrid g{(uint32_t)blocks[0], (uint32_t)(blocks[0] + blocks[1]), (uint32_t)gx[0], (uint32_t)gx[1]};
  if (g.total == 0) return hipSuccess;
  const uint32_t grid = g.total < (1u << 20) ? g.total : (1u << 20);
  hipLaunchKernelGGL(pack_rows_kernel, dim3(grid), dim3(64, 4), 0, stream, jobs[0], n > 1 ? jobs[1] : jobs[0], g);
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
const Candidate kCandidates[] = {
    {kPipeRing, 256, 256, 2, 1.00},     {kPipeProducer, 128, 256, 2, 0.79}, {kPipeProducer, 256, 128, 2, 0.77},
    {kPipeRing, 128, 128, 2, 0.79},     {kPipeRing, 256, 128, 2, 0.72},     {kPipeRing, 128, 256, 2, 0.71},
    {kPipeProducer, 128, 128, 3, 0.65}, {kPipeRing, 64, 64, 3, 0.44},       {kPipeProducer, 64, 64, 3, 0.35},
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
