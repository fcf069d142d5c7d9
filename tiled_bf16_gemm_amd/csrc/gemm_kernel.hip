// bf16 GEMM for gfx950: C = A·B with fp32 accumulation in the matrix cores.
//
// "GEMM: la moltiplicazione di matrici sull'hardware" fixes the product (section "Il conto"),
// the tiling argument (section "Tiling": a B_M×B_N tile of C, operand blocks loaded once into
// on-chip memory and reused, grouped launch order for L2 reuse, a second level of tiles in
// registers) and the mixed precision of the matrix units (tensor-core section).  The descriptor
// pages fix how operand tiles reach on-chip memory (a box copy with out-of-bounds zero fill and
// an XOR swizzle), and "1 · Asynchronisme et mbarrier" §1.3–§1.5 the multi-stage ring that loads
// tile t+1 while tile t is multiplied.  The mapping onto gfx950:
//
//  * workgroup tile 256×256×64, 4 waves (one per SIMD), each owning a 128×128 block of C whose
//    8×8 fragments of 16×16 fp32 accumulators (256 per lane) stay in registers for the whole K
//    loop;
//  * operand tiles are boxes copied straight into LDS by `buffer_load_dwordx4 ... lds` atoms
//    (tile_loader.hpp): A as {64 k, 256 m} with the 2-row swizzle, B stored N×K likewise, B
//    stored K×N as four {64 n, 64 k} boxes with the 128B swizzle;
//  * a 2-stage LDS ring (2 × 64 KiB): at the top of iteration t every wave waits for its own
//    copies of tile t (`s_waitcnt vmcnt(0)`), one barrier publishes them to all waves and
//    retires everyone's reads of the other stage, then tile t+1's copies are issued into that
//    stage and tile t is multiplied — the load of t+1 overlaps the math on t;
//  * fragments come from LDS with ds_read_b128 (k-contiguous rows) or, for B stored K×N, with
//    ds_read_b64_tr_b16, which transposes 4×16 blocks of 16-bit values across 16 lanes;
//  * v_mfma_f32_16x16x32_bf16 with the operands swapped (B fragment first), so each lane ends
//    with four consecutive columns of one row of C; the epilogue regroups them through LDS into
//    whole-row 16-byte stores, masked at the M and N edges;
//  * workgroup ids are remapped so that the tiles resident on one XCD (ids are dealt round-robin
//    over the 8 XCDs) form a compact group of tile-rows and share operand tiles in that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "tbg_desc.hpp"
#include "tile_loader.hpp"

namespace tbg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));


constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 256;
constexpr int kWM = 2, kWN = 2;
constexpr int kTM = kBM / kWM, kTN = kBN / kWN;  // 128 × 128 per wave
constexpr int kFM = kTM / 16, kFN = kTN / 16;    // 8 × 8 fragments per wave
constexpr int kABytes = kBM * kBK * 2;           // 32 KiB
constexpr int kBBytes = kBN * kBK * 2;           // 32 KiB
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kStages = 2;

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

// One 16×16×32 bf16 product-accumulate into an AGPR-resident fp32 tile.  Written as inline
// assembly with the accumulator pinned to AGPRs ("+a"): the 256 accumulators of a wave then stay
// in the accumulation registers for the whole K loop and the 256 architectural VGPRs hold the
// fragments and addresses.  Consecutive products in this kernel never reuse an accumulator
// within 63 instructions, so no dependency wait is needed between them.  The last product of a
// loop iteration (DRAIN) is followed by 24 wait states, more than a matrix result needs before
// another instruction may read it, so whatever follows the loop can read the accumulators.
template <bool DRAIN = false>
__device__ __forceinline__ void mfma16(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  if (DRAIN)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc)
                 : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait for this wave's outstanding tile copies (down to `N` in flight) and its LDS reads, then
// meet the other waves: afterwards every wave's copies of the awaited tile are visible in LDS
// and no wave still reads the stage that the next copies overwrite ("1 · Asynchronisme et
// mbarrier" §1.5: the full/empty hand-off of a ring stage, done here with one barrier).
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N == 0 || N == 16, "vmcnt values used by the ring");
  if (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct Frags {
  bf16x8_t a[kFM];
  bf16x8_t b[kFN];
};

// Per-lane LDS byte offsets of the fragment reads (see the kernel for the layouts).
struct FragAddr {
  uint32_t a_lane, a_col[2];
  uint32_t b_lane, b_col[2];
  uint32_t b_tr[4][2];
  int wn;
};

// Read fragment `idx` (0..7: A fragments, 8..15: B fragments) of k-step `kk` of a stage.
template <int BL>
__device__ __forceinline__ void read_frag(Frags& f, const FragAddr& fa, const uint8_t* sA, const uint8_t* sB, int kk,
                                          int idx) {
  if (idx < kFM) {
    f.a[idx] = *(const bf16x8_t*)(sA + fa.a_lane + idx * 2048 + fa.a_col[kk]);
  } else {
    const int fn = idx - kFM;
    if (BL == 1) {
      f.b[fn] = *(const bf16x8_t*)(sB + fa.b_lane + fn * 2048 + fa.b_col[kk]);
    } else {
      const uint8_t* base = sB + (2 * fa.wn + (fn >> 2)) * 8192 + kk * 4096;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4_t*)(base + fa.b_tr[fn & 3][0]));
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4_t*)(base + fa.b_tr[fn & 3][1]));
      f.b[fn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// Copies of one operand tile pair (A and B boxes of one K tile) into one ring stage: 16 atoms
// per wave, issued one at a time between the products of a k-step.
struct TileCopy {
  rsrc_t ra, rb;
  uint32_t lds_a, lds_b;  // LDS byte address of this wave's first atom of A and of B
  int cvalid_a, cvalid_b;
};

template <int BL>
__device__ __forceinline__ void copy_atom(const TileCopy& tc, const LaneChunk* la, const LaneChunk* lb, int j) {
  if (j < 8) issue_atom(tc.ra, tc.lds_a + j * 1024, la[j], tc.cvalid_a);
  else issue_atom(tc.rb, tc.lds_b + (j - 8) * 1024, lb[j - 8], tc.cvalid_b);
}

// One k-step: the 64 products on `cur`, with the 16 fragment reads of the next k-step and (if
// COPY) the 16 copy atoms of a later tile spread between them, four products per slot.  The
// COPY step closes a loop iteration, so its last product drains.
template <int BL, bool COPY>
__device__ __forceinline__ void kstep(f32x4_t (&acc)[kFN][kFM], const Frags& cur, Frags& nxt, const FragAddr& fa,
                                      const uint8_t* nA, const uint8_t* nB, int nkk, const TileCopy& tc,
                                      const LaneChunk* la, const LaneChunk* lb) {
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    read_frag<BL>(nxt, fa, nA, nB, nkk, g);
    if (COPY) copy_atom<BL>(tc, la, lb, g);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * g + u;
      const int fn = i >> 3, fm = i & 7;
      if (COPY && i == 63) mfma16<true>(acc[fn][fm], cur.b[fn], cur.a[fm]);
      else mfma16(acc[fn][fm], cur.b[fn], cur.a[fm]);
    }
  }
}

template <int BL, int OUT>
__global__ void __launch_bounds__(kThreads, 1) gemm_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  // ---- loader: each wave copies 8 atoms (1 KiB each) of A and 8 of B per tile -----------------
  // A: box {64 k, 256 m} at (k0, m0), 2-row swizzle; this wave owns box rows 64*wave .. +63.
  // B stored N×K: the same with n.  B stored K×N: four boxes {64 n, 64 k} at (n0 + 64*w, k0),
  // 128B swizzle; this wave owns box `wave`.
  const uint32_t pitch_a = (uint32_t)(p.lda * 2), pitch_b = (uint32_t)(p.ldb * 2);
  LaneChunk la[8], lb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    la[i] = lane_chunk<kSwizzle128B2Row>(64 * wave + 8 * i, lane, pitch_a);
    if (BL == 1) {
      lb[i] = lane_chunk<kSwizzle128B2Row>(64 * wave + 8 * i, lane, pitch_b);
    } else {
      lb[i] = lane_chunk<3>(8 * i, lane, pitch_b);
      lb[i].offset += 128u * wave;
    }
  }
  const int kext = p.kchunks * 8;
  // Columns past N in the straddling chunk are loaded as they are: they only feed outputs that
  // are never written.
  const int b_kn_cvalid = (p.N - n0 - 64 * wave + 7) >> 3;
  // At least one tile: with K = 0 every copy lane is masked, the products add zeros and the
  // empty sum is stored.  Keeping one straight path from the accumulator initialisation to the
  // epilogue also keeps the accumulators in fixed AGPRs (no register copies next to in-flight
  // products).
  const int ktiles = p.K > 0 ? (p.K + kBK - 1) / kBK : 1;
  const uint32_t smem_addr = lds_addr_of(smem);

  // Copies of tile kt into `stage`.  A tile past the end of K is issued with every lane masked
  // (zeros land in a stage nobody reads), which keeps the loop body a single path.
  auto make_copy = [&](int kt, int stage) {
    TileCopy tc;
    const int k0 = kt * kBK;
    const bool live = kt < ktiles;
    const uint32_t sa = smem_addr + stage * kStageBytes;
    const uint32_t sb = sa + kABytes;
    tc.cvalid_a = live ? p.kchunks - (k0 >> 3) : -1;
    {
      const uint16_t* origin = p.A + (uint64_t)m0 * p.lda + (live ? k0 : 0);
      const int64_t rem = live ? ((int64_t)(p.M - 1 - m0) * p.lda + (kext - k0)) * 2 : 0;
      tc.ra = make_rsrc(origin, rem > 0 ? (uint64_t)rem : 0);
      tc.lds_a = sa + 64 * wave * 128;
    }
    if (BL == 1) {
      const uint16_t* origin = p.B + (uint64_t)n0 * p.ldb + (live ? k0 : 0);
      const int64_t rem = live ? ((int64_t)(p.N - 1 - n0) * p.ldb + (kext - k0)) * 2 : 0;
      tc.rb = make_rsrc(origin, rem > 0 ? (uint64_t)rem : 0);
      tc.lds_b = sb + 64 * wave * 128;
      tc.cvalid_b = tc.cvalid_a;
    } else {
      const uint16_t* origin = p.B + (uint64_t)(live ? k0 : 0) * p.ldb + n0;
      // The range check works on whole dwords: round the last row's end up to one, so a last
      // element in the low half of a dword is still fetched.  The two bytes past it share that
      // dword (and its page) and only reach columns past N.
      const int64_t rem = live ? (((int64_t)(p.K - 1 - k0) * p.ldb + (p.N - n0)) * 2 + 3) & ~(int64_t)3 : 0;
      tc.rb = make_rsrc(origin, rem > 0 ? (uint64_t)rem : 0);
      tc.lds_b = sb + wave * 8192;
      tc.cvalid_b = live ? b_kn_cvalid : -1;
    }
    return tc;
  };
  auto copy_tile = [&](int kt, int stage) {
    const TileCopy tc = make_copy(kt, stage);
#pragma unroll
    for (int j = 0; j < 16; ++j) copy_atom<BL>(tc, la, lb, j);
  };

  // ---- fragment addresses ---------------------------------------------------------------------
  // A (and B stored N×K): lane l reads row (l & 15) of a 16-row fragment, logical chunk
  // 4*kk + (l >> 4) (eight consecutive k), at its 2-row-swizzled place.
  FragAddr fa;
  {
    const int arow = wm * kTM + (lane & 15);
    const int ax = (arow >> 1) & 7;
    fa.a_lane = (uint32_t)arow * 128u;
    fa.a_col[0] = (uint32_t)((lane >> 4) ^ ax) * 16u;
    fa.a_col[1] = (uint32_t)((4 + (lane >> 4)) ^ ax) * 16u;
    const int brow = wn * kTN + (lane & 15);
    const int bx = (brow >> 1) & 7;
    fa.b_lane = (uint32_t)brow * 128u;
    fa.b_col[0] = (uint32_t)((lane >> 4) ^ bx) * 16u;
    fa.b_col[1] = (uint32_t)((4 + (lane >> 4)) ^ bx) * 16u;
    // B stored K×N, transposing reads: lane 16g + 4e + q supplies the 8 bytes at k row
    // 8g + 4h + e, columns 4q..4q+3 of a 16-column group; lane 16g + i then holds column i.
    const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
#pragma unroll
    for (int f4 = 0; f4 < 4; ++f4)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * tg + 4 * h + te;  // row within a 32-row k step
        const int c = f4 * 2 + (tq >> 1);
        fa.b_tr[f4][h] = (uint32_t)r * 128u + (uint32_t)((c ^ (r & 7)) * 16) + (uint32_t)((tq & 1) * 8);
      }
    fa.wn = wn;
  }

  f32x4_t acc[kFN][kFM];
#pragma unroll
  for (int i = 0; i < kFN; ++i)
#pragma unroll
    for (int j = 0; j < kFM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // ---- the ring: 2 stages of {A tile, B tile}, 2 k-steps of 32 per tile ------------------------
  // Iteration kt: k-step 0 of tile kt (reading k-step 1's fragments), the stage barrier (tile
  // kt+1 landed everywhere, stage kt&1 free), k-step 1 of tile kt (reading tile kt+1's first
  // fragments and copying tile kt+2 into stage kt&1).  Every iteration runs the same code —
  // the last one reads fragments nobody uses and issues fully masked copies — so all products
  // sit in one loop body and the accumulators keep one register assignment throughout.
  {
    Frags f0, f1;
    const TileCopy none{};
    copy_tile(0, 0);
    copy_tile(1, 1);
    stage_barrier<16>();
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) read_frag<BL>(f0, fa, smem, smem + kABytes, 0, idx);
    for (int kt = 0; kt < ktiles; ++kt) {
      const uint8_t* sA = smem + (kt & 1) * kStageBytes;
      kstep<BL, false>(acc, f0, f1, fa, sA, sA + kABytes, 1, none, la, lb);
      stage_barrier<0>();
      const uint8_t* nA = smem + ((kt + 1) & 1) * kStageBytes;
      const TileCopy tc = make_copy(kt + 2, kt & 1);
      kstep<BL, true>(acc, f1, f0, fa, nA, nA + kABytes, 0, tc, la, lb);
    }
  }

  // The loop's last product ends with the drain wait states (mfma16<true>): the accumulators
  // are now safe to read.

  // ---- epilogue: C leaves through LDS as whole rows ------------------------------------------
  // A lane holds C[m][n..n+3] of each fragment, so storing fragments directly writes 16 rows ×
  // 32 bytes per instruction.  Instead each wave parks its 128×128 block in its own quarter of
  // the (now idle) ring, then reads it back as 16-byte pieces of whole rows: a store instruction
  // writes four (bf16) or two (fp32) rows of 256 contiguous bytes, whole cache lines.  The LDS
  // image keeps 16-byte chunks whole and XORs the chunk index with (row & 15), so both the
  // fragment writes (16 rows at one logical chunk) and the row reads (16 chunks of one row) fall
  // on 16 distinct 16-byte bank groups.  Whole-row stores are non-temporal: C is written once and
  // not read again here, so it should not push operand tiles out of the caches.  The ring is
  // drained first: the last iteration's masked copies still write zeros into a stage, and the
  // other waves may still read their fragments.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  uint8_t* park = smem + wave * 32768;
  const int row0 = m0 + wm * kTM, col0 = n0 + wn * kTN;
  if (OUT == 1) {
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn) {
        const int r = 16 * fm + (lane & 15);
        const int c = 2 * fn + (lane >> 5);
        bf16x4_t h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (__bf16)acc[fn][fm][e];
        *(bf16x4_t*)(park + r * 256 + ((c ^ (r & 15)) << 4) + ((lane >> 4) & 1) * 8) = h;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
      const int r = 4 * i + (lane >> 4), c = lane & 15;
      const uint4 v = *(const uint4*)(park + r * 256 + ((c ^ (r & 15)) << 4));
      const int gm = row0 + r, gn = col0 + 8 * c;
      if (gm >= p.M) continue;
      __bf16* dst = (__bf16*)p.C + (uint64_t)gm * p.ldc + gn;
      if (p.vec_store && gn + 7 < p.N) {
        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, (u32x4_t*)dst);
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gn + e < p.N) ((uint16_t*)dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
  } else {
    // fp32: 64 KiB per wave, parked in two halves of 64 rows.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int f = 0; f < kFM / 2; ++f)
#pragma unroll
        for (int fn = 0; fn < kFN; ++fn) {
          const int r = 16 * f + (lane & 15);
          const int c = 4 * fn + (lane >> 4);
          *(f32x4_t*)(park + r * 512 + ((c ^ (r & 15)) << 4)) = acc[fn][half * (kFM / 2) + f];
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const int r = 2 * i + (lane >> 5), c = lane & 31;
        const f32x4_t v = *(const f32x4_t*)(park + r * 512 + ((c ^ (r & 15)) << 4));
        const int gm = row0 + 64 * half + r, gn = col0 + 4 * c;
        if (gm >= p.M) continue;
        float* dst = (float*)p.C + (uint64_t)gm * p.ldc + gn;
        if (p.vec_store && gn + 3 < p.N) {
          __builtin_nontemporal_store(v, (f32x4_t*)dst);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gn + e < p.N) dst[e] = v[e];
        }
      }
      // The second half overwrites the same LDS: its writes follow this wave's reads in LDS
      // order, and the reads' values are already in registers.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

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

hipError_t launch_gemm(const GemmParams& p, int b_layout, int out_bf16, hipStream_t stream) {
  const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
  if (grid == 0) return hipSuccess;
  if (b_layout == 0 && !out_bf16)
    hipLaunchKernelGGL((gemm_bf16_kernel<0, 0>), dim3(grid), dim3(kThreads), 0, stream, p);
  else if (b_layout == 0)
    hipLaunchKernelGGL((gemm_bf16_kernel<0, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
  else if (!out_bf16)
    hipLaunchKernelGGL((gemm_bf16_kernel<1, 0>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<1, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

int gemm_tile_m() { return kBM; }
int gemm_tile_n() { return kBN; }

}  // namespace tbg

