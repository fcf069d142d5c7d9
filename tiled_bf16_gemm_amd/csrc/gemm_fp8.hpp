// GEMM with 8-bit floating-point inputs (OCP E4M3 or E5M2) on gfx950's 16×16×128 matrix
// instruction: C = A·Bᵀ, A row-major M×K, B stored N×K (K contiguous), fp32 accumulation.
//
// "GEMM: la moltiplicazione di matrici sull'hardware", section "Alcune regole pratiche": the
// matrix units reach their peak with 16-bit formats and with shorter ones still, like FP8.  A
// K tile is 128 fp8 values — 128 bytes per row, exactly the rows of the bf16 kernels — so the
// ring, the copy atoms, the 2-row swizzle and the epilogue are the barrier ring's (gemm_ring.hpp,
// two stages).  What changes:
//  * one product per fragment pair per K tile, `v_mfma_f32_16x16x128_f8f6f4`, whose operands are
//    32 bytes per lane: lane l supplies row l%16 of its fragment, the 16-byte chunks l/16 and
//    l/16 + 4 of the tile's row (two ds_read_b128), which the instruction takes as its k =
//    32(l/16)..+31.  It sums over all 128 k of the two operands, and A and B use the same
//    placement, so every k of A meets the same k of B (the sum runs over a permutation of k).
//    The placement keeps the 32 lanes of each read on distinct LDS banks (chunks 2(l/16) and
//    2(l/16)+1 did not: 18 % of the cycles were bank conflicts);
//  * the products run A-fragment outermost: a wave's B fragments stay live for the whole tile and
//    half of its A fragments die in the first half, so one tile's fragments plus the next
//    tile's B fragments and first A fragments fit the register file next to the accumulators;
//  * one barrier per K tile, in its middle (ktile8): it publishes tile kt+1 and frees the stage
//    of tile kt.  The loop runs pairs of tiles; an odd tile count adds one tile of zeros (fully
//    masked copies) to the products.
// The operands are handed over as 16-bit pairs (GemmParams in units of two fp8 values), so the
// copy helpers are the bf16 kernels' own.
#pragma once
#include "gemm_common.hpp"
#include "gemm_ring.hpp"

namespace tbg {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

template <class T>
struct Frags8 {
  i32x8_t a[T::FM];
  i32x8_t b[T::FN];
};

// One 16×16×128 product; FMT 0: E4M3, 1: E5M2 (both operands).  ASM pins the accumulator to
// AGPRs as in mfma16 (drain_acc after the loop).
template <bool ASM, int FMT>
__device__ __forceinline__ void mfma8(f32x4_t& acc, const i32x8_t& a, const i32x8_t& b) {
  if (!ASM)
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, FMT, FMT, 0, 0, 0, 0);
  else if (FMT == 0)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1" : "+a"(acc) : "v"(a), "v"(b));
}

// Per-lane LDS byte offsets of the two 16-byte halves of a fragment row: logical chunks
// l/16 and l/16 + 4 of a 128-byte row at their 2-row-swizzled places.
struct FragAddr8 {
  uint32_t a_lane, a_col[2];
  uint32_t b_lane, b_col[2];
};

template <class T>
__device__ __forceinline__ FragAddr8 make_frag_addr8(int wm, int wn, int lane) {
  FragAddr8 fa;
  const int arow = wm * T::TM + (lane & 15), brow = wn * T::TN + (lane & 15);
  const int ax = (arow >> 1) & 7, bx = (brow >> 1) & 7, c = lane >> 4;
  fa.a_lane = (uint32_t)arow * 128u;
  fa.a_col[0] = (uint32_t)(c ^ ax) * 16u;
  fa.a_col[1] = (uint32_t)((c + 4) ^ ax) * 16u;
  fa.b_lane = (uint32_t)brow * 128u;
  fa.b_col[0] = (uint32_t)(c ^ bx) * 16u;
  fa.b_col[1] = (uint32_t)((c + 4) ^ bx) * 16u;
  return fa;
}

__device__ __forceinline__ i32x8_t read_frag8(const uint8_t* base, uint32_t lane_off, const uint32_t* col) {
  const u32x4_t lo = *(const u32x4_t*)(base + lane_off + col[0]);
  const u32x4_t hi = *(const u32x4_t*)(base + lane_off + col[1]);
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// One K tile on `cur` (held in stage sCur), in two halves around the stage barrier:
//   first half   the products on A fragments 0..H-1 (H = FM/2), with this tile's remaining A
//                fragments H..FM-1 read from sCur;
//   barrier      this wave's copies of tile kt+1 have landed (vmcnt 0: nothing newer is in flight
//                yet) and every wave's reads of sCur have completed, so tile kt+1 is visible and
//                sCur is free;
//   second half  the products on A fragments H..FM-1, with tile kt+1's B fragments and its A
//                fragments 0..H-1 read from sNxt, and tile kt+2's copy atoms into sCur.
// A copy so has from the middle of the tile it is issued in to the middle of the next one to
// land, and no fragment is read before its tile is known to be complete.
template <class T, int FMT, bool MASK>
__device__ __forceinline__ void ktile8(f32x4_t (&acc)[T::FN][T::FM], Frags8<T>& cur, Frags8<T>& nxt,
                                       const FragAddr8& fa, const uint8_t* sCurA, const uint8_t* sNxtA,
                                       const uint8_t* sNxtB, const TileCopy& tc, const LaneChunk* la,
                                       const LaneChunk* lb) {
  constexpr int A = T::Atoms, FN = T::FN, FM = T::FM, H = FM / 2;
  constexpr int P0 = H * FN, P1 = T::Products - P0, NR = FN + H;
#pragma unroll
  for (int i = 0; i < P0; ++i) {
    // serpentine over fn (as kstep in gemm_common.hpp): consecutive products share an operand
    const int fm = i / FN, fn = (fm & 1) ? FN - 1 - i % FN : i % FN;
    if (i % FN == 0) cur.a[H + fm] = read_frag8(sCurA, fa.a_lane + (H + fm) * 2048, fa.a_col);
    mfma8<T::AsmMfma, FMT>(acc[fn][fm], cur.b[fn], cur.a[fm]);
  }
  stage_barrier<0>();
#pragma unroll
  for (int i = 0; i < P1; ++i) {
    const int fm = H + i / FN, fn = (fm & 1) ? FN - 1 - i % FN : i % FN;
    // fragment read q (B first, then A 0..H-1) before product (q * P1) / NR; atom j before (j * P1) / A
#pragma unroll
    for (int q = (i * NR + P1 - 1) / P1; q < ((i + 1) * NR + P1 - 1) / P1 && q < NR; ++q) {
      if (q < FN) nxt.b[q] = read_frag8(sNxtB, fa.b_lane + q * 2048, fa.b_col);
      else nxt.a[q - FN] = read_frag8(sNxtA, fa.a_lane + (q - FN) * 2048, fa.a_col);
    }
#pragma unroll
    for (int j = (i * A + P1 - 1) / P1; j < ((i + 1) * A + P1 - 1) / P1 && j < A; ++j)
      copy_atom<T, MASK, MASK>(tc, la, lb, j);
    mfma8<T::AsmMfma, FMT>(acc[fn][fm], cur.b[fn], cur.a[fm]);
  }
}

template <int BM, int BN, int FMT, int OUT, int SCALED>
__global__ void __launch_bounds__(kThreads, (RingCfg<BM, BN, 2>::MinBlocks)) gemm_fp8_kernel(GemmParams p) {
  using T = TileCfg<BM, BN>;
  constexpr int BL = 1;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::StageBytes];
  const int lane = threadIdx.x & 63;
  // The wave index is uniform: keeping it scalar keeps every address derived from it scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const uint32_t pitch_a = row_pitch(p.da), pitch_b = row_pitch(p.db);
  LaneChunk la[T::AtomsA], lb[T::AtomsB];
#pragma unroll
  for (int i = 0; i < T::AtomsA; ++i) {
    la[i] = lane_chunk<kSwizzle128B2Row>((BM / 4) * wave + 8 * i, lane, pitch_a);
    mask_row(la[i], (BM / 4) * wave + 8 * i + (lane >> 3), p.M - m0);
  }
#pragma unroll
  for (int i = 0; i < T::AtomsB; ++i) {
    lb[i] = lane_chunk<kSwizzle128B2Row>((BN / 4) * wave + 8 * i, lane, pitch_b);
    mask_row(lb[i], (BN / 4) * wave + 8 * i + (lane >> 3), p.N - n0);
  }
  const int ktiles = p.K > 0 ? (p.K + kBK - 1) / kBK : 1;  // K counts pairs: a tile is 64 pairs
  const uint32_t smem_addr = lds_addr_of(smem);
  const CopyPlan plan = make_copy_plan<BL>(p, m0, n0);

  // The copies of tile kt into `stage`; INTERIOR (kt < ktiles - 1: the tile lies wholly inside
  // K) takes open ranges and no chunk tests (rows past M or N stay masked in the lane offsets).
  auto make_copy = [&](int kt, int stage, auto interior) __attribute__((always_inline)) {
    const OperandTiles o = decltype(interior)::value ? interior_tiles<BL>(plan, kt) : operand_tiles<BL>(plan, kt, ktiles);
    TileCopy tc;
    const uint32_t sa = smem_addr + stage * T::StageBytes;
    tc.ra = o.ra;
    tc.rb = o.rb;
    tc.cvalid_a = o.cvalid_a;
    tc.cvalid_b = o.cvalid_a;
    tc.lds_a = sa + (BM / 4) * wave * 128;
    tc.lds_b = sa + T::ABytes + (BN / 4) * wave * 128;
    return tc;
  };

  const FragAddr8 fa = make_frag_addr8<T>(wm, wn, lane);
  f32x4_t acc[T::FN][T::FM];
  zero_acc<T>(acc);
  {
    Frags8<T> f0, f1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const TileCopy tc = make_copy(t, t, std::false_type{});
#pragma unroll
      for (int j = 0; j < T::Atoms; ++j) copy_atom<T>(tc, la, lb, j);
    }
    stage_barrier<T::Atoms>();  // tile 0 landed; tile 1 may be in flight
#pragma unroll
    for (int j = 0; j < T::FM / 2; ++j) f0.a[j] = read_frag8(smem, fa.a_lane + j * 2048, fa.a_col);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) f0.b[j] = read_frag8(smem + T::ABytes, fa.b_lane + j * 2048, fa.b_col);
    const uint8_t* s1 = smem + T::StageBytes;
    // Tile kt (stage 0) with tile kt+1's first fragments from stage 1 and tile kt+2's copies into
    // stage 0; then tile kt+1 (stage 1) with tile kt+2's first fragments and tile kt+3's copies.
    auto pair = [&](int kt, auto interior) __attribute__((always_inline)) {
      constexpr bool mask = !decltype(interior)::value;
      ktile8<T, FMT, mask>(acc, f0, f1, fa, smem, s1, s1 + T::ABytes, make_copy(kt + 2, 0, interior), la, lb);
      ktile8<T, FMT, mask>(acc, f1, f0, fa, s1, smem, smem + T::ABytes, make_copy(kt + 3, 1, interior), la, lb);
    };
    int kt = 0;
    // Pairs whose copies (tiles kt+2, kt+3) both lie before the last tile: no masking.
    for (; kt + 5 <= ktiles; kt += 2) pair(kt, std::true_type{});
    for (; kt < ktiles; kt += 2) pair(kt, std::false_type{});
  }
  drain_acc<T>(acc);
  stage_barrier<0>();
  store_tile<T, OUT, SCALED>(acc, smem + wave * (T::RingBytes / 4), p, m0 + wm * T::TM, n0 + wn * T::TN, lane);
}

}  // namespace tbg
