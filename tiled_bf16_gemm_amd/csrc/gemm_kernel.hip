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
// destination, numbered flat over both operands' chunks (no idle threads at ragged row ends).
// The chunk's 16 source bytes may start at any byte: the thread loads the two aligned 16-byte
// blocks that hold them (consecutive lanes load consecutive blocks, so every load instruction is
// one contiguous run) and funnel-shifts them into place.  The second block is clamped to the
// aligned block that holds the row's last byte, and the bytes past the row are zeroed, so no load
// leaves the 16-byte blocks the row touches (those never cross a page).
__device__ __forceinline__ uint4 pack_chunk(const PackJob& j, int64_t r, int64_t b0) {
  const int64_t valid = j.row_bytes - b0;  // bytes of this chunk inside the row
  if (valid <= 0) return make_uint4(0, 0, 0, 0);
  const uint8_t* srow = j.src + r * j.ld_src;
  const uintptr_t a = (uintptr_t)(srow + b0);
  const uintptr_t base = a & ~(uintptr_t)15;
  const uintptr_t last = (uintptr_t)(srow + j.row_bytes - 1) & ~(uintptr_t)15;
  const uint4 q0 = *(const uint4*)base;
  const uint4 q1 = *(const uint4*)(base + 16 <= last ? base + 16 : last);
  const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  const uint32_t d = (uint32_t)(a & 15) >> 2, sh = (uint32_t)(a & 3);
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // dwords d + k and d + k + 1 of the 32 loaded bytes, selected without indexing registers
    uint32_t lo = w[k], hi = w[k + 1];
#pragma unroll
    for (int s = 1; s < 4; ++s) {
      if (d == (uint32_t)s) {
        lo = w[k + s];
        hi = w[k + s + 1 < 8 ? k + s + 1 : 7];
      }
    }
    o[k] = __builtin_amdgcn_alignbyte(hi, lo, sh);
    const int64_t keep = valid - 4 * k;  // bytes of this dword inside the row
    if (keep < 4) o[k] &= keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Chunks numbered flat: chunks below `n0` belong to j0 (row-major over its rows × cpr0 chunks),
// the rest to j1.  Workgroups step through the chunks by the grid size.
struct PackGrid {
  uint64_t n0, total;  // chunks of the first repack; chunks of both
  uint32_t cpr0, cpr1;  // destination chunks per row of each repack
};

// Index is the chunk number's type: 32-bit when every chunk number fits (a 32-bit division per
// thread instead of the 64-bit division routine), 64-bit otherwise.
template <typename Index>
__global__ void __launch_bounds__(256) pack_rows_kernel(PackJob j0, PackJob j1, PackGrid g) {
  const Index stride = (Index)gridDim.x * blockDim.x;
  const Index n0 = (Index)g.n0, total = (Index)g.total;
  for (Index t = (Index)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const bool second = t >= n0;
    const PackJob& j = second ? j1 : j0;
    const Index i = second ? t - n0 : t;
    const Index cpr = second ? g.cpr1 : g.cpr0;
    const int64_t r = (int64_t)(i / cpr), c = (int64_t)(i % cpr);
    *(uint4*)(j.dst + r * j.ld_dst + c * 16) = pack_chunk(j, r, c * 16);
  }
}

hipError_t launch_pack_jobs(const PackJob* jobs, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  uint64_t chunks[2] = {0, 0};
  uint32_t cpr[2] = {1, 1};
  for (int i = 0; i < n; ++i) {
    if (jobs[i].ld_dst / 16 >= (1ll << 32)) return hipErrorInvalidValue;
    cpr[i] = (uint32_t)(jobs[i].ld_dst / 16);
    chunks[i] = (uint64_t)cpr[i] * (uint64_t)jobs[i].rows;
  }
  const PackGrid g{chunks[0], chunks[0] + chunks[1], cpr[0], cpr[1]};
  if (g.total == 0) return hipSuccess;
  const uint64_t blocks = (g.total + 255) / 256;
  const uint32_t grid = blocks < (1u << 20) ? (uint32_t)blocks : (1u << 20);
  // the grid-stride loop's last step must not wrap the 32-bit index either
  if (g.total + (uint64_t)grid * 256 < (1ull << 32))
    hipLaunchKernelGGL(pack_rows_kernel<uint32_t>, dim3(grid), dim3(256), 0, stream, jobs[0],
                       n > 1 ? jobs[1] : jobs[0], g);
  else
    hipLaunchKernelGGL(pack_rows_kernel<uint64_t>, dim3(grid), dim3(256), 0, stream, jobs[0],
                       n > 1 ? jobs[1] : jobs[0], g);
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
