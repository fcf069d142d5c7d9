// The barrier ring: S LDS stages, every compute wave copies its share of each stage.
//
// "1 · Asynchronisme et mbarrier" §1.3–§1.5 describes a multi-stage ring that loads tile t+S-1
// while tile t is multiplied, with a full and an empty hand-off per stage.  Here the four compute
// waves are also the copiers: each issues T::Atoms direct-to-LDS atoms of every K tile
// (tile_loader.hpp), and one workgroup barrier per tile does both hand-offs at once — before
// it, every wave waits for its own copies of the next tile (`s_waitcnt vmcnt`, leaving the S-2
// newer tiles in flight); after it, those copies are visible to all waves and every wave's
// reads of the stage that the next copies overwrite have completed.
//
// Tile kt: k-step 0 (its products, with the fragment reads of k-step 1), the stage barrier
// (tile kt+1 landed everywhere, stage kt%S free), k-step 1 (its products, with the reads of tile
// kt+1's first fragments and the copies of tile kt+S into stage kt%S interleaved).  The loop body
// holds S tiles, one per stage, so stage addresses are constants; the last ones read fragments
// nobody uses and issue fully masked copies.  The accumulators keep one register assignment
// throughout.
#pragma once
#include "gemm_common.hpp"

namespace tbg {

template <int BM, int BN, int S>
struct RingCfg {
  using T = TileCfg<BM, BN>;
  static constexpr int LdsBytes = S * T::StageBytes;
  // Two workgroups per compute unit when two rings fit in the 160 KiB of LDS.
  static constexpr int MinBlocks = 2 * LdsBytes <= 160 * 1024 ? 2 : 1;
  static_assert(S >= 2, "a ring has at least two stages");
  static_assert(LdsBytes <= 160 * 1024, "the ring must fit in LDS");
  static_assert(T::Atoms * (S - 2) <= 63, "tiles in flight must fit the vmcnt counter");
};

// CLK 1: a measurement instance (never launched by the library) that records, per workgroup, the
// real-time and shader-clock counters' advance from its start to the end of its stores.
// CLK 2: a measurement instance that records a timeline per workgroup (8 values): the 100 MHz
// real-time counter at its start, once its first tile has landed, after its K loop and once its
// stores have completed (wave 0's); the shader-clock advance over the whole; the hardware ids of
// the wave (HW_ID) and of the XCD (XCC_ID) it ran on.
template <int BM, int BN, int S, int IN, int BL, int OUT, int SCALED, int CLK = 0>
__global__ void __launch_bounds__(kThreads, (RingCfg<BM, BN, S>::MinBlocks)) gemm_ring_kernel(GemmParams p) {
  using T = TileCfg<BM, BN, IN>;
  uint64_t clk_r0 = 0, clk_m0 = 0, clk_first = 0, clk_loop = 0;
  if (CLK) {
    clk_r0 = __builtin_amdgcn_s_memrealtime();
    clk_m0 = __builtin_amdgcn_s_memtime();
  }
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RingCfg<BM, BN, S>::LdsBytes];
  const int lane = threadIdx.x & 63;
  // The wave index is uniform: keeping it scalar keeps every address derived from it scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- copies: each wave copies AtomsA atoms (1 KiB each) of A and AtomsB of B per K tile ----
  // A: box {64 k, BM m} at (k0, m0), 2-row swizzle; this wave owns box rows (BM/4)*wave .. +BM/4-1.
  // B stored N×K: the same with n.  B stored K×N: BN/64 boxes {64 n, 64 k} at (n0 + 64*b, k0),
  // K×N layout (kSwizzleKnTr), 8 atoms each; this wave owns atoms AtomsB*wave .. +AtomsB-1 of the boxes in
  // order, all inside one box.
  const uint32_t pitch_a = row_pitch(p.da), pitch_b = row_pitch(p.db);
  const int b_box = (wave * T::AtomsB) >> 3;  // K×N box of this wave's B atoms
  LaneChunk la[T::AtomsA], lb[T::AtomsB];
#pragma unroll
  for (int i = 0; i < T::AtomsA; ++i) {
    la[i] = lane_chunk<kSwizzle128B2Row>((BM / 4) * wave + 8 * i, lane, pitch_a);
    mask_row(la[i], (BM / 4) * wave + 8 * i + (lane >> 3), p.M - m0);
  }
#pragma unroll
  for (int i = 0; i < T::AtomsB; ++i) {
    if (BL == 1) {
      lb[i] = lane_chunk<kSwizzle128B2Row>((BN / 4) * wave + 8 * i, lane, pitch_b);
      mask_row(lb[i], (BN / 4) * wave + 8 * i + (lane >> 3), p.N - n0);
    } else {
      lb[i] = lane_chunk<kSwizzleKnTr>(8 * ((wave * T::AtomsB + i) & 7), lane, pitch_b);
      lb[i].offset += 128u * b_box;
      // columns past N: masked once here; rows past K by the range of the last tile's copy
      if (lb[i].chunk >= kn_box_cvalid(p, n0, b_box)) lb[i].offset = kOobOffset;
    }
  }
  // At least one tile: with K = 0 every copy lane is masked, the products add zeros and the
  // empty sum is stored.  Keeping one straight path from the accumulator initialisation to the
  // epilogue also keeps the accumulators in fixed AGPRs (no register copies next to in-flight
  // products).
  const int ktiles = p.K > 0 ? (p.K + kBK - 1) / kBK : 1;
  const uint32_t smem_addr = lds_addr_of(smem);
  const CopyPlan plan = make_copy_plan<BL>(p, m0, n0);

  // The copies of tile kt into `stage`; INTERIOR (kt < ktiles - 1, the tile lies wholly inside
  // K) takes open ranges and no chunk tests.
  auto make_copy = [&](int kt, int stage, auto interior) __attribute__((always_inline)) {
    const OperandTiles o = decltype(interior)::value ? interior_tiles<BL>(plan, kt) : operand_tiles<BL>(plan, kt, ktiles);
    TileCopy tc;
    const uint32_t sa = smem_addr + stage * T::StageBytes;
    const uint32_t sb = sa + T::ABytes;
    tc.ra = o.ra;
    tc.rb = o.rb;
    tc.cvalid_a = o.cvalid_a;
    tc.cvalid_b = o.cvalid_a;  // B stored K×N: unused (lane offsets and range mask it)
    tc.lds_a = sa + (BM / 4) * wave * 128;
    tc.lds_b = BL == 1 ? sb + (BN / 4) * wave * 128 : sb + wave * T::AtomsB * 1024;
    return tc;
  };

  const FragAddr<T> fa = make_frag_addr<T>(wm, wn, lane);
  f32x4_t acc[T::FN][T::FM];
  zero_acc<T>(acc);

  {
    Frags<T> f0, f1;
    const TileCopy none{};
#pragma unroll
    for (int t = 0; t < S; ++t) {
      const TileCopy tc = make_copy(t, t, std::false_type{});
#pragma unroll
      for (int j = 0; j < T::Atoms; ++j) copy_atom<T, true, BL == 1>(tc, la, lb, j);
    }
    stage_barrier<T::Atoms*(S - 1)>();  // tile 0 landed; tiles 1..S-1 may be in flight
    if (CLK == 2) clk_first = __builtin_amdgcn_s_memrealtime();
#pragma unroll
    for (int idx = 0; idx < T::Reads; ++idx) read_frag<T, BL>(f0, fa, smem, smem + T::ABytes, 0, idx);
    // One K tile on stage CUR (a compile-time constant, so every LDS address below is a fixed
    // offset from the ring: the loop runs S tiles per iteration, one per stage).
    auto tile = [&](int kt, auto stage, auto interior) __attribute__((always_inline)) {
      constexpr int cur = decltype(stage)::value;
      constexpr int nxt = cur + 1 == S ? 0 : cur + 1;
      constexpr bool mask = !decltype(interior)::value;
      const uint8_t* sA = smem + cur * T::StageBytes;
      kstep<T, BL, false>(acc, f0, f1, fa, sA, sA + T::ABytes, 1, none, la, lb);
      stage_barrier<T::Atoms*(S - 2)>();  // tile kt+1 landed; tiles kt+2..kt+S-1 may be in flight
      const uint8_t* nA = smem + nxt * T::StageBytes;
      const TileCopy tc = make_copy(kt + S, cur, interior);
      kstep<T, BL, true, mask, mask && BL == 1>(acc, f1, f0, fa, nA, nA + T::ABytes, 0, tc, la, lb);
    };
    int kt = 0;
    // Iterations whose copies (tiles kt+S .. kt+2S-1) all lie before the last tile: no masking.
    for (; kt + 2 * S < ktiles; kt += S)
      for_stages<S>([&](auto st) __attribute__((always_inline)) {
        tile(kt + decltype(st)::value, st, std::true_type{});
      });
    for (; kt + S <= ktiles; kt += S)
      for_stages<S>([&](auto st) __attribute__((always_inline)) {
        tile(kt + decltype(st)::value, st, std::false_type{});
      });
    // the last ktiles % S tiles, on stages 0.. in order
    for_stages<S - 1>([&](auto st) __attribute__((always_inline)) {
      if (kt + decltype(st)::value < ktiles) tile(kt + decltype(st)::value, st, std::false_type{});
    });
  }

  // Wait states after the last product (drain_acc), then the ring is drained before it becomes
  // the park: the last iterations' masked copies still write zeros into stages, and the other
  // waves may still read their fragments.
  if (CLK == 2) clk_loop = __builtin_amdgcn_s_memrealtime();
  drain_acc<T>(acc);
  stage_barrier<0>();
  store_tile<T, OUT, SCALED>(acc, smem + wave * (T::RingBytes / 4), p, m0 + wm * T::TM, n0 + wn * T::TN, lane);
  if (CLK == 1) {
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime(), m1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
      p.clock[2 * (uint64_t)blockIdx.x] = r1 - clk_r0;
      p.clock[2 * (uint64_t)blockIdx.x + 1] = m1 - clk_m0;
    }
  } else if (CLK == 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have completed
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime(), m1 = __builtin_amdgcn_s_memtime();
    uint32_t hw_id, xcc_id;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw_id));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc_id));
    if (threadIdx.x == 0) {
      uint64_t* o = p.clock + 8 * (uint64_t)blockIdx.x;
      o[0] = clk_r0;
      o[1] = clk_first;
      o[2] = clk_loop;
      o[3] = r1;
      o[4] = m1 - clk_m0;
      o[5] = hw_id;
      o[6] = xcc_id;
      o[7] = 0;
    }
  }
}

template <int BM, int BN, int S, int IN>
hipError_t launch_ring(const GemmParams& p, int b_layout, int out_bf16, hipStream_t stream) {
  TBG_LAUNCH_INSTANCES(gemm_ring_kernel, kThreads, BM, BN, S, IN);
}

}  // namespace tbg
