// Device building blocks shared by the GEMM kernels (gemm_ring.hpp, gemm_pc.hpp): the
// workgroup tile shape, the XCD-aware tile order, the 16×16×32 bf16 product, fragment reads from
// LDS, the copy atoms of a ring stage, one k-step of products with its interleaved reads and
// copies, and the epilogue.
//
// "GEMM: la moltiplicazione di matrici sull'hardware" fixes the product (section "Il conto"),
// the tiling argument (section "Tiling": a B_M×B_N tile of C, operand blocks loaded once into
// on-chip memory and reused, grouped launch order for L2 reuse, a second level of tiles in
// registers) and the mixed precision of the matrix units (tensor-core section).  The descriptor
// pages fix how operand tiles reach on-chip memory (a box copy with out-of-bounds zero fill and
// an XOR swizzle).  Layouts used by every kernel:
//
//  * workgroup tile BM×BN×64, 4 compute waves in a 2×2 arrangement, each owning a
//    (BM/2)×(BN/2) block of C whose 16×16 fp32 accumulator fragments stay in registers for the
//    whole K loop (256 per lane at 256×256);
//  * a ring stage holds the A box {64 k, BM m} with the 2-row swizzle, then B: stored N×K the
//    same way, stored K×N as BN/64 boxes {64 n, 64 k} in the K×N layout (kSwizzleKnTr);
//  * fragments come from LDS with ds_read_b128 (k-contiguous rows) or, for B stored K×N, with
//    ds_read_b64_tr_b16, which transposes 4×16 blocks of 16-bit values across 16 lanes.  Both
//    layouts are chosen so that every fragment read is free of LDS bank conflicts (measured
//    with the counters and a read micro-benchmark: the 16-byte reads here are conflict-free
//    with the 2-row swizzle; the 8-byte transposing read is served 32 lanes at a time from 256
//    bytes and needs the K×N layout);
//  * v_mfma_f32_16x16x32_bf16 with the operands swapped (B fragment first), so each lane ends
//    with four consecutive columns of one row of C; the epilogue regroups them through LDS into
//    whole-row 16-byte stores, masked at the M and N edges.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "launch.hpp"
#include "tbg_desc.hpp"
#include "tile_loader.hpp"

namespace tbg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 64, kThreads = 256;

// Shape of one workgroup tile and everything derived from it.  IN_ is the input element type of
// the products: 0 bf16, 1 fp16 (both 16 bits: only the matrix instruction differs).
template <int BM_, int BN_, int IN_ = 0>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int In = IN_;
  static constexpr int TM = BM / 2, TN = BN / 2;    // block of C per wave (2×2 waves)
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16×16 fragments per wave
  static constexpr int ABytes = BM * kBK * 2, BBytes = BN * kBK * 2;
  static constexpr int StageBytes = ABytes + BBytes;
  // A ring has at least two stages; the epilogue parks each wave's block of C in its own
  // quarter of the first two.
  static constexpr int RingBytes = 2 * StageBytes;
  static constexpr int AtomsA = BM / 32, AtomsB = BN / 32;  // 1 KiB copy atoms per wave per K tile
  static constexpr int Atoms = AtomsA + AtomsB;
  static constexpr int Reads = FM + FN;     // fragment reads per k-step of 32
  static constexpr int Products = FM * FN;  // products per k-step
  // 256 accumulators per lane only fit if they are pinned to AGPRs (inline assembly); smaller
  // blocks use the compiler's builtin, which also inserts the dependency waits that the
  // short accumulator reuse distance of a small block needs.
  static constexpr bool AsmMfma = Products >= 64;
  static_assert(BM % 64 == 0 && BN % 64 == 0 && BM <= 256 && BN <= 256, "tile sizes 64, 128, 256");
};

// Workgroup id -> (tile row, tile column).  Ids are dealt round-robin to the 8 XCDs; the first
// step gives each XCD a contiguous range of logical ids (a bijection for any grid size), the
// second orders logical ids column-major inside groups of `group_m` tile-rows ("GEMM" page,
// section "Tiling": blocks launched together reuse the same operand tiles from L2).
__device__ __forceinline__ void map_tile(int bid, int nwg, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int q = nwg >> 3, r = nwg & 7;
  const int x = bid & 7, i = bid >> 3;
  const int lid = x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
  const int per_group = group_m * tiles_n;
  const int g = lid / per_group;
  const int first = g * group_m;
  const int gsz = min(tiles_m - first, group_m);
  const int in = lid - g * per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

// One 16×16×32 bf16 product-accumulate.  For the 256×256 tile it is inline assembly with the
// accumulator pinned to AGPRs ("+a"): the 256 accumulators of a wave then stay in the
// accumulation registers for the whole K loop and the 256 architectural VGPRs hold the fragments
// and addresses.  Consecutive products there never reuse an accumulator within 63 instructions,
// so no dependency wait is needed between them; after the loop, drain_acc adds the wait states a
// matrix result needs before another instruction may read it.
template <bool ASM, int IN = 0>
__device__ __forceinline__ void mfma16(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  if (IN == 1) {
    // fp16 operands travel in the same registers as bf16 ones: only the instruction differs.
    if (!ASM)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), acc,
                                                   0, 0, 0);
    else
      asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    return;
  }
  if (!ASM)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// TBG_HANDOFF_CHECK 1 builds the hand-off checking variant of every kernel (a library of its own,
// never the product): each stage hand-off waits for all of the wave's copies and LDS reads
// (vmcnt(0), lgkmcnt(0)) instead of only the awaited tile's, so a schedule that read a stage
// before its copies landed, or overwrote it while another wave still read it, would show up as
// a difference from the lean kernels' bits.
#ifndef TBG_HANDOFF_CHECK
#define TBG_HANDOFF_CHECK 0
#endif

// Wait for this wave's outstanding tile copies (down to `N` in flight) and its LDS reads, then
// meet the other waves: afterwards every wave's copies of the awaited tile are visible in LDS
// and no wave still reads the stage that the next copies overwrite ("1 · Asynchronisme et
// mbarrier" §1.5: the full/empty hand-off of a ring stage, done here with one barrier).
// The wait and the barrier are the compiler's builtins, not assembly text, so its own wait
// insertion knows that every LDS read has completed here; with the wait hidden in assembly it
// drained all reads again at the head of the K loop (a full LDS round trip once per
// iteration).  The builtins do not order memory accesses for the optimizer, so an empty
// assembly statement with a memory clobber on each side keeps every LDS read and copy on its
// side of the hand-off.  The vmcnt field is split: bits 3:0 and 15:14; expcnt (bits 6:4) is left
// at 7, no wait.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  constexpr int V = TBG_HANDOFF_CHECK ? 0 : N;
  static_assert(V >= 0 && V <= 63, "vmcnt is a 6-bit count");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <class T>
struct Frags {
  bf16x8_t a[T::FM];
  bf16x8_t b[T::FN];
};

// Per-lane LDS byte offsets of the fragment reads (see the kernel for the layouts).
template <class T>
struct FragAddr {
  static constexpr int Q = T::FN < 4 ? T::FN : 4;
  uint32_t a_lane, a_col[2];
  uint32_t b_lane, b_col[2];
  uint32_t b_tr[Q][2];
  int wn;
};

// Read fragment `idx` (0..FM-1: A fragments, FM..FM+FN-1: B fragments) of k-step `kk` of a stage.
template <class T, int BL>
__device__ __forceinline__ void read_frag(Frags<T>& f, const FragAddr<T>& fa, const uint8_t* sA, const uint8_t* sB,
                                          int kk, int idx) {
  if (idx < T::FM) {
    f.a[idx] = *(const bf16x8_t*)(sA + fa.a_lane + idx * 2048 + fa.a_col[kk]);
  } else {
    const int fn = idx - T::FM;
    if (BL == 1) {
      f.b[fn] = *(const bf16x8_t*)(sB + fa.b_lane + fn * 2048 + fa.b_col[kk]);
    } else {
      // The wave's columns wn*TN .. +TN-1 lie in boxes of 64 columns; fragment fn is 16 of them.
      const int box = T::TN >= 64 ? fa.wn * (T::TN / 64) + (fn >> 2) : 0;
      const int q = T::TN >= 64 ? (fn & 3) : fn;
      const uint8_t* base = sB + box * 8192 + kk * 4096;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4_t*)(base + fa.b_tr[q][0]));
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4_t*)(base + fa.b_tr[q][1]));
      f.b[fn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// Copies of one operand tile pair (A and B boxes of one K tile) into one ring stage: T::Atoms
// atoms per wave, issued one at a time between the products of a k-step.
struct TileCopy {
  rsrc_t ra, rb;
  uint32_t lds_a, lds_b;  // LDS byte address of this wave's first atom of A and of B
  int cvalid_a, cvalid_b;
};

// Atom j of a tile.  A lane's logical chunk depends only on the atom's parity: atoms start
// 8 rows apart at multiples of 16 rows per wave, and the 2-row and K×N XORs of rows 16 apart are
// equal (checked for every tile, wave, lane and atom), so the chunk tests of atoms 0 and 1 serve
// every atom of the tile (two compares per operand instead of one per atom).  MASK_A / MASK_B
// false: no chunk test for that operand (a tile that lies wholly inside it, or an operand whose
// lane offsets and range already mask everything outside it).
template <class T, bool MASK_A = true, bool MASK_B = true>
__device__ __forceinline__ void copy_atom(const TileCopy& tc, const LaneChunk* la, const LaneChunk* lb, int j) {
  if (j < T::AtomsA) {
    issue_atom_if(tc.ra, tc.lds_a, j * 1024, la[j].offset, !MASK_A || la[j & 1].chunk < tc.cvalid_a);
  } else {
    const int i = j - T::AtomsA;
    issue_atom_if(tc.rb, tc.lds_b, i * 1024, lb[i].offset, !MASK_B || lb[i & 1].chunk < tc.cvalid_b);
  }
}

// One k-step: the products on `cur`, with the fragment reads of the next k-step and (if COPY)
// the copy atoms of a later tile spread between them.  The loop's last product is drained after
// the loop (drain_acc), not here.
template <class T, int BL, bool COPY, bool MASK_A = true, bool MASK_B = true>
__device__ __forceinline__ void kstep(f32x4_t (&acc)[T::FN][T::FM], const Frags<T>& cur, Frags<T>& nxt,
                                      const FragAddr<T>& fa, const uint8_t* nA, const uint8_t* nB, int nkk,
                                      const TileCopy& tc, const LaneChunk* la, const LaneChunk* lb) {
  // Read r goes before product (r * Products) / Reads; atom j halfway between that slot and the
  // next, before product (j * Products) / Atoms + Products / (2 * Atoms).  A wave alone on its
  // SIMD issues one instruction every 4 clocks and a product keeps the matrix unit busy for 16,
  // so every run of more than 3 other instructions between products idles the unit: staggering
  // the atoms (5-6 instructions each with their m0 setup and chunk mask) against the reads keeps
  // the runs short.
  constexpr int P = T::Products, R = T::Reads, A = T::Atoms;
#pragma unroll
  for (int i = 0; i < P; ++i) {
#pragma unroll
    for (int r = (i * R + P - 1) / P; r < ((i + 1) * R + P - 1) / P; ++r) read_frag<T, BL>(nxt, fa, nA, nB, nkk, r);
    if (COPY && i >= P / (2 * A)) {
      constexpr int H = P / (2 * A);
#pragma unroll
      for (int j = ((i - H) * A + P - 1) / P; j < ((i + 1 - H) * A + P - 1) / P; ++j) copy_atom<T, MASK_A, MASK_B>(tc, la, lb, j);
    }
    // Serpentine order: row fn of the FN×FM grid of products runs forward when fn is even and
    // backward when odd, so consecutive products always share one operand register (63 operand
    // changes per k-step instead of 70).  Under the power cap the matrix units' input toggling
    // sets the clock (measured: 0.7-0.9 % shorter products on 8192³ and 16384×14336×4096, same
    // bits: every accumulator still sees its k-steps in ascending order).
    const int fn = i / T::FM, fm = (fn & 1) ? T::FM - 1 - i % T::FM : i % T::FM;
    mfma16<T::AsmMfma, T::In>(acc[fn][fm], cur.b[fn], cur.a[fm]);
  }
}

// The wait states between the K loop's last product and the first read of an accumulator, for
// products issued as inline assembly (the compiler cannot see their hazards; for its builtin it
// inserts the waits itself).  The drain is one assembly statement; each accumulator then passes
// through an empty statement that claims to rewrite it, so every later read of it depends on a
// statement that the compiler keeps after the drain.
template <class T>
__device__ __forceinline__ void drain_acc(f32x4_t (&acc)[T::FN][T::FM]) {
  if (!T::AsmMfma) return;
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0][0]));
#pragma unroll
  for (int i = 0; i < T::FN; ++i)
#pragma unroll
    for (int j = 0; j < T::FM; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// LDS chunk swizzle of the epilogue's park: rows of `cpr` 16-byte chunks; XOR the chunk index
// so that 16 rows at one chunk (the fragment writes) and 16 consecutive chunks (the row reads)
// fall on 16 distinct 16-byte bank groups of the 256-byte bank window.
template <int CPR>
__device__ __forceinline__ int park_xor(int r) {
  if (CPR >= 16) return r & 15;
  if (CPR == 8) return (r >> 1) & 7;
  return (r >> 2) & 3;  // CPR == 4
}

// The epilogue: C leaves through LDS as whole rows.  A lane holds C[m][n..n+3] of each fragment,
// so storing fragments directly would write 16 rows × 32 bytes per instruction.  Instead each
// wave parks its block (in one or two bands of rows) in its own quarter of the now idle ring,
// then reads it back as 16-byte pieces of whole rows, so every store instruction writes whole
// row segments.  Whole-row stores are non-temporal: C is written once and not read again here,
// so it should not push operand tiles out of the caches.  With SCALED the park keeps the fp32
// sums and each piece becomes alpha·S + beta·C_old (C_old read only when beta != 0) before it is
// rounded to C's type ("GEMM" page, tensor-core section: C <- alpha·A·B + beta·C).
template <class T, int OUT, int SCALED>
__device__ __forceinline__ void store_tile(const f32x4_t (&acc)[T::FN][T::FM], uint8_t* park, const GemmParams& p,
                                          int row0, int col0, int lane) {
  constexpr int ES = OUT == 1 ? 2 : 4;                     // element size of C
  constexpr int PES = (OUT == 1 && !SCALED) ? 2 : 4;       // element size in the park
  constexpr int RowBytes = T::TN * PES;
  constexpr int CPR = RowBytes / 16;
  constexpr int EPC = 16 / PES;  // elements per 16-byte park chunk
  constexpr int ParkBytes = T::RingBytes / 4;
  constexpr int Bands = (T::TM * RowBytes + ParkBytes - 1) / ParkBytes;
  constexpr int BandFM = T::FM / Bands;
  constexpr int BandRows = 16 * BandFM;
  constexpr int RowsPerRead = 64 / CPR;
  constexpr int ReadsPerBand = BandRows / RowsPerRead;
  static_assert(T::FM % Bands == 0 && BandRows % RowsPerRead == 0, "epilogue bands");
#pragma unroll
  for (int band = 0; band < Bands; ++band) {
#pragma unroll
    for (int f = 0; f < BandFM; ++f)
#pragma unroll
      for (int fn = 0; fn < T::FN; ++fn) {
        const int r = 16 * f + (lane & 15);
        const f32x4_t v = acc[fn][band * BandFM + f];
        if (PES == 2) {
          const int c = 2 * fn + (lane >> 5);
          bf16x4_t h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (__bf16)v[e];
          *(bf16x4_t*)(park + r * RowBytes + ((c ^ park_xor<CPR>(r)) << 4) + ((lane >> 4) & 1) * 8) = h;
        } else {
          const int c = 4 * fn + (lane >> 4);
          *(f32x4_t*)(park + r * RowBytes + ((c ^ park_xor<CPR>(r)) << 4)) = v;
        }
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < ReadsPerBand; ++i) {
      const int r = RowsPerRead * i + lane / CPR, c = lane % CPR;
      const uint4 v = *(const uint4*)(park + r * RowBytes + ((c ^ park_xor<CPR>(r)) << 4));
      const int gm = row0 + BandRows * band + r, gn = col0 + EPC * c;
      if (gm >= p.M) continue;
      uint8_t* dst = (uint8_t*)p.C + ((uint64_t)gm * p.ldc + gn) * ES;
      const bool whole = p.vec_store && gn + EPC - 1 < p.N;
      if (!SCALED) {
        if (whole) {
          __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, (u32x4_t*)dst);
        } else {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            if (gn + e >= p.N) continue;
            if (OUT == 1) ((uint16_t*)dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            else ((uint32_t*)dst)[e] = w[e];
          }
        }
      } else {
        // four fp32 sums per piece
        float x[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
        float old[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.beta != 0.f) {
          if (whole) {
            if (OUT == 1) {
              const uint2 o = *(const uint2*)dst;
              old[0] = __uint_as_float(o.x << 16);
              old[1] = __uint_as_float(o.x & 0xFFFF0000u);
              old[2] = __uint_as_float(o.y << 16);
              old[3] = __uint_as_float(o.y & 0xFFFF0000u);
            } else {
              const uint4 o = *(const uint4*)dst;
              old[0] = __uint_as_float(o.x);
              old[1] = __uint_as_float(o.y);
              old[2] = __uint_as_float(o.z);
              old[3] = __uint_as_float(o.w);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (gn + e >= p.N) continue;
              old[e] = OUT == 1 ? __uint_as_float((uint32_t)((const uint16_t*)dst)[e] << 16) : ((const float*)dst)[e];
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = p.beta != 0.f ? p.alpha * x[e] + p.beta * old[e] : p.alpha * x[e];
        if (OUT == 1) {
          bf16x4_t h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (__bf16)x[e];
          if (whole) {
            *(bf16x4_t*)dst = h;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gn + e < p.N) ((__bf16*)dst)[e] = h[e];
          }
        } else {
          if (whole) {
            *(f32x4_t*)dst = f32x4_t{x[0], x[1], x[2], x[3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gn + e < p.N) ((float*)dst)[e] = x[e];
          }
        }
      }
    }
    // The next band's writes follow these reads in this wave's LDS order.
    if (Bands > 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}


// Copy descriptors of one workgroup's operand boxes, built once before the K loop: the loop only
// advances a base address per K tile.  A and B stored N×K use an open range (0x7FFFFFFF bytes):
// their rows past M (or N) are masked in the per-lane offsets once (mask_row) and their chunks
// past K by the chunk count, so no lane reads outside the operand.  B stored K×N keeps the exact
// range to the end of B: the 16-byte chunk that straddles column N is loaded whole, and in B's
// last row the range check is what keeps it inside the allocation.
struct CopyPlan {
  rsrc_t ra0, rb0;   // the boxes at K tile 0
  int64_t rem_b0;    // B stored K×N: bytes from the box origin to the end of B (range at tile 0)
  uint32_t step_b;   // bytes per K tile along B: 128 for N×K, 64 rows of ldb for K×N
  int kchunks;       // 16-byte K chunks in a row of A (and of N×K B)
};

struct OperandTiles {
  rsrc_t ra, rb;
  int cvalid_a;  // K chunks of tile kt that exist (<= 0 past the end: every lane masked)
  bool live;
};

// Row pitch in bytes of an operand descriptor (its dimension-1 stride).
__device__ __forceinline__ uint32_t row_pitch(const DescImpl& d) { return (uint32_t)d.stride[1]; }

// The copy plan from the operand descriptors the host encoded: A's box origin moves m0 rows down,
// B's n0 rows (stored N×K) or n0 elements along a row (stored K×N); the 16-byte K chunks present
// in a row are A's inner extent in bytes, rounded up.
template <int BL>
__device__ __forceinline__ CopyPlan make_copy_plan(const GemmParams& p, int m0, int n0) {
  CopyPlan c;
  const DescImpl& da = p.da;
  const DescImpl& db = p.db;
  c.kchunks = (int)((da.dim[0] * da.elsize + 15) / 16);
  c.ra0 = make_rsrc((const uint8_t*)da.base + (uint64_t)m0 * da.stride[1], 0x7FFFFFFFull);
  if (BL == 1) {
    c.rb0 = make_rsrc((const uint8_t*)db.base + (uint64_t)n0 * db.stride[1], 0x7FFFFFFFull);
    c.step_b = 128u;
    c.rem_b0 = 0;
  } else {
    c.rb0 = make_rsrc((const uint8_t*)db.base + (uint64_t)n0 * db.elsize, 0);
    c.step_b = (uint32_t)(db.stride[1] * kBK);
    // Round the last row's end up to a whole dword: the range check works on dwords, so a last
    // element in the low half of one is still fetched.  The two bytes past it share that dword
    // (and its page) and only reach columns past N.
    c.rem_b0 = ((int64_t)(db.dim[1] - 1) * (int64_t)db.stride[1] + ((int64_t)db.dim[0] - n0) * db.elsize + 3) &
               ~(int64_t)3;
  }
  return c;
}

// A buffer descriptor with its 48-bit base moved on by `bytes`.
__device__ __forceinline__ rsrc_t rsrc_advance(rsrc_t r, uint64_t bytes) {
  const uint64_t a = (((uint64_t)(uint32_t)r.y << 32) | (uint32_t)r.x) + bytes;
  r.x = (int)(uint32_t)a;
  r.y = (int)((uint32_t)(a >> 32) & 0xFFFFu);
  return r;
}

// Range of B stored K×N from the box origin moved on by `off` bytes: clamp(rem, 0, 2^31-1), or 0
// for a tile past the end.  Computed on the two 32-bit halves with scalar compares (a 64-bit
// signed compare would go to the vector unit).
__device__ __forceinline__ int kn_range(const CopyPlan& c, uint64_t off, bool live) {
  const uint64_t rem = (uint64_t)(c.rem_b0 - (int64_t)off);
  int32_t hi = (int32_t)(rem >> 32);
  uint32_t lo = (uint32_t)rem;
  asm("" : "+s"(hi), "+s"(lo));  // opaque: the optimizer would fuse the halves into a 64-bit compare
  return (!live || hi < 0) ? 0 : ((hi != 0 || lo > 0x7FFFFFFFu) ? 0x7FFFFFFF : (int)lo);
}

// The boxes of K tile kt (tiles at or past `ktiles` are fully masked).
template <int BL>
__device__ __forceinline__ OperandTiles operand_tiles(const CopyPlan& c, int kt, int ktiles) {
  OperandTiles o;
  o.live = kt < ktiles;
  o.cvalid_a = c.kchunks - kt * (kBK / 8);
  o.ra = rsrc_advance(c.ra0, (uint64_t)kt * 128u);
  const uint64_t off = (uint64_t)kt * c.step_b;
  o.rb = rsrc_advance(c.rb0, off);
  if (BL == 0) o.rb.z = kn_range(c, off, o.live);
  return o;
}

// The boxes of K tile kt < ktiles - 1, which lies wholly inside K: open ranges and every chunk
// valid (rows past M or N stay masked in the lane offsets; B stored K×N has its columns past N
// masked there too).
template <int BL>
__device__ __forceinline__ OperandTiles interior_tiles(const CopyPlan& c, int kt) {
  OperandTiles o;
  o.live = true;
  o.cvalid_a = kBK / 8;
  o.ra = rsrc_advance(c.ra0, (uint64_t)kt * 128u);
  o.rb = rsrc_advance(c.rb0, (uint64_t)kt * c.step_b);
  if (BL == 0) o.rb.z = 0x7FFFFFFF;
  return o;
}

// Mask a lane's chunk when its box row is past the operand's last row (set once per kernel).
__device__ __forceinline__ void mask_row(LaneChunk& lc, int row, int rows) {
  if (row >= rows) lc.offset = kOobOffset;
}

// 16-byte chunks of columns that exist in the K×N box b (64 columns from n0 + 64 b).  The chunk
// that straddles column N is loaded whole: its columns past N only feed outputs that are never
// written.
__device__ __forceinline__ int kn_box_cvalid(const GemmParams& p, int n0, int b) { return (p.N - n0 - 64 * b + 7) >> 3; }

// Call f(std::integral_constant<int, s>) for s = 0..N-1 in order (compile-time stage indices).
template <int... I, class F>
__device__ __forceinline__ void for_stages_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void for_stages(F&& f) {
  for_stages_impl(f, std::make_integer_sequence<int, N>{});
}

// Per-lane fragment read addresses of compute wave (wm, wn).
// A (and B stored N×K): lane l reads row (l & 15) of a 16-row fragment, logical chunk
// 4*kk + (l >> 4) (eight consecutive k), at its 2-row-swizzled place.
// B stored K×N, transposing reads: lane 16g + 4e + q supplies the 8 bytes at k row 8g + 4h + e,
// columns 4q..4q+3 of a 16-column group; lane 16g + i then holds column i.  Group f4 of a box is
// the wave's fragment (f4 of its first box, or 2*wn + fn when the wave's 32 columns are half of
// the single box).
template <class T>
__device__ __forceinline__ FragAddr<T> make_frag_addr(int wm, int wn, int lane) {
  FragAddr<T> fa;
  const int arow = wm * T::TM + (lane & 15);
  const int ax = (arow >> 1) & 7;
  fa.a_lane = (uint32_t)arow * 128u;
  fa.a_col[0] = (uint32_t)((lane >> 4) ^ ax) * 16u;
  fa.a_col[1] = (uint32_t)((4 + (lane >> 4)) ^ ax) * 16u;
  const int brow = wn * T::TN + (lane & 15);
  const int bx = (brow >> 1) & 7;
  fa.b_lane = (uint32_t)brow * 128u;
  fa.b_col[0] = (uint32_t)((lane >> 4) ^ bx) * 16u;
  fa.b_col[1] = (uint32_t)((4 + (lane >> 4)) ^ bx) * 16u;
  const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
#pragma unroll
  for (int q = 0; q < FragAddr<T>::Q; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int f4 = T::TN >= 64 ? q : 2 * wn + q;
      const int r = 8 * tg + 4 * h + te;  // row within a 32-row k step
      const int c = f4 * 2 + (tq >> 1);
      fa.b_tr[q][h] = (uint32_t)r * 128u + (uint32_t)((c ^ row_xor<kSwizzleKnTr>(r)) * 16) + (uint32_t)((tq & 1) * 8);
    }
  fa.wn = wn;
  return fa;
}

template <class T>
__device__ __forceinline__ void zero_acc(f32x4_t (&acc)[T::FN][T::FM]) {
#pragma unroll
  for (int i = 0; i < T::FN; ++i)
#pragma unroll
    for (int j = 0; j < T::FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// One launcher per kernel configuration: picks the B layout / C type / scaling instance.
#define TBG_LAUNCH_INSTANCES(KERNEL, THREADS, ...)                                                              \
  do {                                                                                                         \
    const unsigned grid_ = (unsigned)p.tiles_m * (unsigned)p.tiles_n;                                          \
    if (p.scaled) {                                                                                            \
      if (b_layout == 0 && !out_bf16)                                                                          \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 0, 0, 1>), dim3(grid_), dim3(THREADS), 0, stream, p);          \
      else if (b_layout == 0)                                                                                  \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 0, 1, 1>), dim3(grid_), dim3(THREADS), 0, stream, p);          \
      else if (!out_bf16)                                                                                      \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 1, 0, 1>), dim3(grid_), dim3(THREADS), 0, stream, p);          \
      else                                                                                                     \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 1, 1, 1>), dim3(grid_), dim3(THREADS), 0, stream, p);          \
    } else {                                                                                                   \
      if (b_layout == 0 && !out_bf16)                                                                          \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 0, 0, 0>), dim3(grid_), dim3(THREADS), 0, stream, p);          \
      else if (b_layout == 0)                                                                                  \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 0, 1, 0>), dim3(grid_), dim3(THREADS), 0, stream, p);          \
      else if (!out_bf16)                                                                                      \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 1, 0, 0>), dim3(grid_), dim3(THREADS), 0, stream, p);          \
      else                                                                                                     \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 1, 1, 0>), dim3(grid_), dim3(THREADS), 0, stream, p);          \
    }                                                                                                          \
    return hipGetLastError();                                                                                  \
  } while (0)

}  // namespace tbg
