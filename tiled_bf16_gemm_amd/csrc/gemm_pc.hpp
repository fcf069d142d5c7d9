// The producer/consumer ring: S LDS stages, dedicated producer waves, per-stage full and empty
// counters in LDS instead of a workgroup barrier.
//
// "1 · Asynchronisme et mbarrier" §1.5 gives the N-stage ring with two barriers per stage: the
// producer waits until a stage is empty, fills it and marks it full; the consumers wait until
// it is full, compute on it and mark it empty.  "2 · Le Tensor Memory Accelerator" gives the
// producer role to one thread of one warp.  On gfx950:
//
//  * NP producer waves (each issuing 16 direct-to-LDS atoms per K tile, 8 with more than four
//    stages, so that the S-1 tiles in flight fit the 6-bit vmcnt counter) copy every stage; the
//    four compute waves issue no memory instruction at all;
//  * full[s] and empty[s] are monotonically increasing 32-bit counters in LDS.  A producer wave
//    adds 1 to full[s] once its copies of the stage's tile have landed (its own
//    `s_waitcnt vmcnt`); the f-th fill of stage s is complete when full[s] reaches NP·(f+1).
//    A compute wave adds 1 to empty[s] after its last fragment read of the stage; the stage may
//    be filled for the f-th time once empty[s] reaches 4·f.  Waiters poll the counter with
//    `s_sleep` between reads;
//  * the producer keeps S-1 tiles in flight: after issuing tile t it waits for tile t-(S-2) and
//    marks it full.
//
// Only tiles whose compute waves fit in half a SIMD's registers can host producer waves: the
// 256×256 tile needs the whole register file for its four compute waves and has no variant here.
#pragma once
#include "gemm_common.hpp"

namespace tbg {

template <int BM, int BN, int S>
struct PcCfg {
  using T = TileCfg<BM, BN>;
  static constexpr int TileAtoms = BM / 8 + BN / 8;   // 1 KiB atoms per K tile (A then B)
  // Atoms per producer wave per tile: its S-1 tiles in flight must fit the 6-bit vmcnt counter.
  static constexpr int PA = S <= 4 ? 16 : 8;
  static constexpr int NP = TileAtoms / PA;           // producer waves
  static constexpr int Threads = kThreads + 64 * NP;
  static constexpr int LdsBytes = S * T::StageBytes;
  static constexpr int MinBlocks = 2 * LdsBytes <= 150 * 1024 ? 2 : 1;
  static_assert(TileAtoms % NP == 0, "atoms split evenly between producer waves");
  static_assert(S >= 2, "a ring has at least two stages");
  static_assert(LdsBytes <= 150 * 1024, "the ring and its counters must fit in LDS");
  static_assert(PA * (S - 1) <= 63, "tiles in flight must fit the vmcnt counter");
  static_assert(!T::AsmMfma, "compute waves must leave registers for the producer waves");
};

// Wait until an LDS counter reaches `target`.  The acquire keeps the caller's later LDS reads
// after the observation.  The spin is bounded (about 2^20 sleeps): a counter that never arrives
// would be a bug, and the kernel then finishes with wrong results instead of never finishing.
__device__ __forceinline__ void wait_counter(uint32_t* counter, uint32_t target) {
  for (int spin = 0; spin < (1 << 20); ++spin) {
    if (__hip_atomic_load(counter, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Add 1 to an LDS counter from one lane; the release orders it after the wave's earlier LDS
// accesses.
__device__ __forceinline__ void arrive(uint32_t* counter, int lane) {
  if (lane == 0) __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Producer wave PW: atoms PW*PA .. PW*PA+PA-1 of every K tile.  Atom j < BM/8 is rows 8j..8j+7
// of the A box; atom j = BM/8 + i is rows 8i.. of the N×K B box, or atom i%8 of the K×N box i/8.
// Atom j lands at stage byte 1024 j (the layout the compute waves read, the same as the barrier
// ring's).  Tile t is issued once every compute wave has released the stage's previous tile, and
// marked full once the copies of tile t landed, S-2 tiles later.
template <int BM, int BN, int S, int BL, int PW>
__device__ __forceinline__ void produce(const GemmParams& p, const uint8_t* smem, uint32_t* full, uint32_t* empty,
                                        int m0, int n0, int ktiles, int lane) {
  using C = PcCfg<BM, BN, S>;
  using T = TileCfg<BM, BN>;
  static_assert(PW < C::NP, "producer wave index");
  const uint32_t pitch_a = row_pitch(p.da), pitch_b = row_pitch(p.db);
  const uint32_t smem_addr = lds_addr_of(smem);
  LaneChunk ch[C::PA];
#pragma unroll
  for (int i = 0; i < C::PA; ++i) {
    const int j = PW * C::PA + i;
    if (j < BM / 8) {
      ch[i] = lane_chunk<kSwizzle128B2Row>(8 * j, lane, pitch_a);
      mask_row(ch[i], 8 * j + (lane >> 3), p.M - m0);
    } else if (BL == 1) {
      ch[i] = lane_chunk<kSwizzle128B2Row>(8 * (j - BM / 8), lane, pitch_b);
      mask_row(ch[i], 8 * (j - BM / 8) + (lane >> 3), p.N - n0);
    } else {
      const int jb = j - BM / 8;
      ch[i] = lane_chunk<kSwizzleKnTr>(8 * (jb & 7), lane, pitch_b);
      ch[i].offset += 128u * (uint32_t)(jb >> 3);
    }
  }
  const CopyPlan plan = make_copy_plan<BL>(p, m0, n0);
  int st = 0, fill = 0;     // stage and fill round of tile kt
  int sig = 0, sig_st = 0;  // next tile to mark full, and its stage
  for (int kt = 0; kt < ktiles; ++kt) {
    if (fill > 0) wait_counter(&empty[st], 4u * (uint32_t)fill);
    const OperandTiles o = operand_tiles<BL>(plan, kt, ktiles);
    const uint32_t base = smem_addr + (uint32_t)(st * T::StageBytes);
#pragma unroll
    for (int i = 0; i < C::PA; ++i) {
      const int j = PW * C::PA + i;
      if (j < BM / 8) {
        issue_atom(o.ra, base + 1024u * j, ch[i], o.cvalid_a);
      } else {
        const int cv = BL == 1 ? o.cvalid_a : (o.live ? kn_box_cvalid(p, n0, (j - BM / 8) >> 3) : -1);
        issue_atom(o.rb, base + 1024u * j, ch[i], cv);
      }
    }
    if (TBG_HANDOFF_CHECK) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (kt >= S - 2) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::PA * (S - 2)) : "memory");
      arrive(&full[sig_st], lane);
      ++sig;
      sig_st = sig_st + 1 == S ? 0 : sig_st + 1;
    }
    if (++st == S) {
      st = 0;
      ++fill;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (; sig < ktiles; ++sig) {
    arrive(&full[sig_st], lane);
    sig_st = sig_st + 1 == S ? 0 : sig_st + 1;
  }
}

template <int BM, int BN, int S, int IN, int BL, int OUT, int SCALED>
__global__ void __launch_bounds__((PcCfg<BM, BN, S>::Threads), (PcCfg<BM, BN, S>::MinBlocks))
    gemm_pc_kernel(GemmParams p) {
  using C = PcCfg<BM, BN, S>;
  using T = TileCfg<BM, BN, IN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LdsBytes];
  __shared__ uint32_t full[S], empty[S];
  const int lane = threadIdx.x & 63;
  // The wave index is uniform across the wave: keeping it scalar turns every role and atom-kind
  // test below into a scalar branch instead of an exec-mask region.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x < S) {
    full[threadIdx.x] = 0;
    empty[threadIdx.x] = 0;
  }
  __syncthreads();

  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int ktiles = p.K > 0 ? (p.K + kBK - 1) / kBK : 1;

  if (wave >= 4) {
    // Producer wave pw runs a copy of the loop specialised to its atoms (all index arithmetic
    // and atom kinds then fold at compile time).
    const int pw = wave - 4;
    if (pw == 0) produce<BM, BN, S, BL, 0>(p, smem, full, empty, m0, n0, ktiles, lane);
    if (C::NP > 1 && pw == 1) produce<BM, BN, S, BL, (C::NP > 1 ? 1 : 0)>(p, smem, full, empty, m0, n0, ktiles, lane);
    if (C::NP > 2 && pw == 2) produce<BM, BN, S, BL, (C::NP > 2 ? 2 : 0)>(p, smem, full, empty, m0, n0, ktiles, lane);
    if (C::NP > 3 && pw == 3) produce<BM, BN, S, BL, (C::NP > 3 ? 3 : 0)>(p, smem, full, empty, m0, n0, ktiles, lane);
    __syncthreads();
    return;
  }

  // ---- compute waves ---------------------------------------------------------------------------
  // Iteration kt: k-step 0 of tile kt (reading k-step 1's fragments), release of the stage, wait
  // for tile kt+1, k-step 1 of tile kt (reading tile kt+1's first fragments).  The last
  // iteration reads fragments of a stage nobody writes any more and never uses them.
  const int wm = wave >> 1, wn = wave & 1;
  const FragAddr<T> fa = make_frag_addr<T>(wm, wn, lane);
  f32x4_t acc[T::FN][T::FM];
  zero_acc<T>(acc);
  {
    Frags<T> f0, f1;
    const TileCopy none{};
    const LaneChunk* nolanes = nullptr;
    wait_counter(&full[0], (uint32_t)C::NP);
#pragma unroll
    for (int idx = 0; idx < T::Reads; ++idx) read_frag<T, BL>(f0, fa, smem, smem + T::ABytes, 0, idx);
    int fill_next = 0;  // fill round of tile kt+1
    // Tile kt on stage CUR = kt % S, a compile-time constant: S tiles per loop iteration.
    auto tile = [&](int kt, auto stage) __attribute__((always_inline)) {
      constexpr int cur = decltype(stage)::value;
      constexpr int nxt = cur + 1 == S ? 0 : cur + 1;
      if (nxt == 0) ++fill_next;
      const uint8_t* sA = smem + cur * T::StageBytes;
      kstep<T, BL, false>(acc, f0, f1, fa, sA, sA + T::ABytes, 1, none, nolanes, nolanes);
      if (TBG_HANDOFF_CHECK) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      arrive(&empty[cur], lane);
      if (kt + 1 < ktiles) wait_counter(&full[nxt], (uint32_t)(C::NP * (fill_next + 1)));
      const uint8_t* nA = smem + nxt * T::StageBytes;
      kstep<T, BL, false>(acc, f1, f0, fa, nA, nA + T::ABytes, 0, none, nolanes, nolanes);
    };
    int kt = 0;
    for (; kt + S <= ktiles; kt += S)
      for_stages<S>([&](auto st) __attribute__((always_inline)) { tile(kt + decltype(st)::value, st); });
    for_stages<S - 1>([&](auto st) __attribute__((always_inline)) {
      if (kt + decltype(st)::value < ktiles) tile(kt + decltype(st)::value, st);
    });
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();  // every copy landed and every fragment read retired: the ring becomes the park
  store_tile<T, OUT, SCALED>(acc, smem + wave * (T::RingBytes / 4), p, m0 + wm * T::TM, n0 + wn * T::TN, lane);
}

template <int BM, int BN, int S, int IN>
hipError_t launch_pc(const GemmParams& p, int b_layout, int out_bf16, hipStream_t stream) {
  TBG_LAUNCH_INSTANCES(gemm_pc_kernel, (PcCfg<BM, BN, S>::Threads), BM, BN, S, IN);
}

}  // namespace tbg
