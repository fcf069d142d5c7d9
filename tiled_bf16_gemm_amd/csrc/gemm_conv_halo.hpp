// Halo convolution: a 2-D convolution with stride 1 whose input window is copied into LDS once
// and read there by every filter tap.
//
// The im2col form ("2 · Le Tensor Memory Accelerator", section "im2col"; gemm_conv.hpp) copies one
// box of the im2col matrix per filter tap, so each input pixel crosses from L2 into LDS once per
// tap that reads it (nine times for a 3×3 filter).  With stride 1 the boxes of all taps are
// shifted views of one window of the input: for output rows oh0 .. oh0+tr-1 (whole rows, all ow
// columns) and taps (r, s), the pixels read are input rows oh0 − ph + [0, hh) and columns
// −pw + [0, hw), hh = tr + (R−1)·dh, hw = ow + (S−1)·dw.  That window is a tiled box of X
// ("H100 · cuTensorMap": box copy with out-of-bounds zero fill), and the fill is the zero padding.
// The workgroup copies it once per 32-channel block and reads the A fragment of tap (r, s) at
// window pixel (oh − oh0 + r·dh)·hw + ow + s·dw: the GEMM's A tile becomes an address offset.
//
// Workgroup tile: 448 output pixels (tr·ow of them used, tr = min(448 / ow, oh)) × 128 output
// channels; four waves, each 112 pixels × 128 channels (7 × 8 fragments of 16×16, 224
// accumulators per lane in AGPRs); K loop over 32-channel blocks, and inside each over the taps:
// one 16×16×32 product step per (block, tap), so the sums run block by block, tap by tap inside
// a block (another order than the im2col kernels', which run tap by tap, 64 channels inside).
//
// LDS: four filter tiles (128 channels-out × 32 channels-in, 8 KiB each) in a ring, two window
// images (one per channel block, alternating: the next block's window is copied while the
// current one is read), one spare 1 KiB atom for copies that carry nothing.  A window pixel takes
// its 64 channel bytes, unpadded: a 16-byte read of 16 consecutive pixels at two chunks then meets
// each bank group twice (a pitch of 80 or 96 bytes halves that, but each window atom would carry a
// fifth or a third of unused bytes, and the kernel is bound by its copies, not by LDS reads); the
// filter tiles use 64-byte rows with the chunk XOR (row >> 2) & 3.
//
// Copies per product step and wave: 2 filter atoms of the tile four steps ahead, then HS window
// atoms of the next block's window (spread over the first R·S − 1 taps of the current block; a
// wave with nothing left to copy issues an atom that lands zeros in the spare atom, so that every
// step issues the same number and the waits have fixed counts).
#pragma once
#include "fast_div.hpp"
#include "gemm_common.hpp"

namespace tbg {

constexpr int kHaloBM = 448, kHaloBN = 128;
constexpr int kHaloFM = 7, kHaloFN = 8;  // fragments per wave: 112 pixels × 128 channels
constexpr int kHaloStages = 4;           // filter tiles in the ring
constexpr int kHaloBStage = kHaloBN * 64;
constexpr int kHaloPitch = 64;           // LDS bytes per window pixel
constexpr int kHaloMaxAtoms = 63;        // 1 KiB atoms per window image
constexpr int kHaloOff0 = kHaloStages * kHaloBStage;
constexpr int kHaloJunk = kHaloOff0 + 2 * kHaloMaxAtoms * 1024;
constexpr int kHaloSmem = kHaloJunk + 1024;

// Epilogue shape for store_tile: each wave parks its 112 × 128 block in one band (bf16) or in
// seven bands of 16 rows (fp32 sums).
template <int OUT, int SCALED>
struct HaloTile {
  static constexpr int TM = 112, TN = kHaloBN, FM = kHaloFM, FN = kHaloFN;
  static constexpr bool AsmMfma = true;
  static constexpr int RingBytes = (OUT == 1 && !SCALED) ? 4 * TM * TN * 2 : 4 * 16 * TN * 4;
};
static_assert(HaloTile<1, 0>::RingBytes <= kHaloSmem && HaloTile<0, 0>::RingBytes <= kHaloSmem, "park");

// issue_atom_if preceded by 5 wait states inside the same statement.  The filter tile's buffer
// descriptor changes every step, and the compiler may write its scalar registers with a vector
// instruction (v_readfirstlane); gfx9 needs 5 wait states between a vector write of a scalar
// register and a memory instruction reading it, which the compiler cannot insert in front of
// inline assembly.
__device__ __forceinline__ void issue_atom_settled(rsrc_t rs, uint32_t lds_base, int lds_imm, uint32_t offset) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(offset), "s"(rs), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base) + (uint32_t)lds_imm)
               : "memory");
}

// A direct-to-LDS atom whose source is voff + soff bytes into the buffer: soff (uniform) carries
// what is the same for every lane, here a channel block's or a filter column's offset.
// Offsets with bit 31 set stay out of the buffer's range with the scalar offset added (it is
// below 2^31), so those lanes still land zeros.
__device__ __forceinline__ void issue_atom_so(rsrc_t rs, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(soff), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

struct HaloFrags {
  bf16x8_t a[kHaloFM];
  bf16x8_t b[kHaloFN];
};

// TAPS 0: any filter, the step's tap and channel block kept in counters.  TAPS 9: filters of nine
// taps (r·s == 9), one block of taps unrolled: every tap offset, copy position and wait count is
// a compile-time choice, and each window atom reuses per-lane offsets computed once.
template <int HS, int OUT, int SCALED, int TAPS = 0>
__global__ void __launch_bounds__(kThreads, 1) gemm_conv_halo_kernel(HaloParams hp) {
  using T = HaloTile<OUT, SCALED>;
  const ConvParams& cp = hp.c;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kHaloSmem];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, cp.g.tiles_m, cp.g.tiles_n, cp.g.group_m, tm, tn);
  const int img = tm / hp.tpi;
  const int oh0 = (tm - img * hp.tpi) * hp.tr;
  const int n0 = tn * kHaloBN;
  const int rows = min(hp.tr, cp.oh - oh0) * cp.ow;  // output pixels of the tile
  const int m0 = (img * cp.oh + oh0) * cp.ow;        // Y rows m0 .. m0 + rows - 1

  // A fragment f of this wave: lane row p = 112·wave + 16f + (lane & 15), chunk (lane >> 4);
  // its window pixel at tap (0, 0), as an LDS byte offset.  Rows past the tile read pixel 0.
  const uint32_t q16 = (uint32_t)(lane >> 4) * 16u;
  uint32_t a0[kHaloFM];
#pragma unroll
  for (int f = 0; f < kHaloFM; ++f) {
    const int p = 112 * wave + 16 * f + (lane & 15);
    uint32_t slot = 0;
    if (p < rows) {
      const uint32_t ohl = fast_div((uint32_t)p, hp.div_ow);
      slot = ohl * (uint32_t)hp.hw + ((uint32_t)p - ohl * (uint32_t)cp.ow);
    }
    a0[f] = slot * kHaloPitch + q16;
  }
  // B fragment fn: output channel 16fn + (lane & 15), chunk (lane >> 4) at its XORed place.
  const int br = lane & 15;
  const uint32_t b0 = (uint32_t)br * 64u + (uint32_t)(((lane >> 4) ^ ((br >> 2) & 3)) << 4);

  // Filter copies: atoms 2·wave and 2·wave + 1 of each tile (16 output channels each); lane l
  // fills row l >> 2, physical chunk l & 3 with logical chunk (l & 3) ^ ((l >> 4) & 3).
  const int64_t ldw2 = cp.ldw * 2;
  uint32_t ob[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = 16 * (2 * wave + j) + (lane >> 2);
    const int c = (lane & 3) ^ ((lane >> 4) & 3);
    ob[j] = n0 + n < cp.g.N ? (uint32_t)(n * ldw2) + (uint32_t)c * 16u : kOobOffset;
  }
  const rsrc_t rw = make_rsrc(cp.W + (int64_t)n0 * cp.ldw, 0x7FFFFFFFull);
  const rsrc_t rx = make_rsrc(cp.X, cp.x_bytes);
  const uint32_t smem_addr = lds_addr_of(smem);

  // Window copies: atom a covers 16-byte units 64a .. 64a + 63 of the window image, unit U being
  // chunk U % 4 of window pixel U / 4; pixel s is window row s / hw, column s % hw, i.e. input
  // row oh0 − ph + s / hw, column s % hw − pw.  Units outside the image or past the window take
  // an offset with bit 31 set, which the buffer's range rejects (they land zeros).
  const int ih_base = oh0 - cp.ph;
  const uint32_t img_base = (uint32_t)img * (uint32_t)cp.h * (uint32_t)cp.w * (uint32_t)cp.c8 * 2u;
  const uint32_t pix_bytes = (uint32_t)cp.c8 * 2u;
  const int h1 = cp.h - 1, w1 = cp.w - 1;
  auto halo_src = [&](int a, int cb) __attribute__((always_inline)) {
    const uint32_t u = (uint32_t)a * 64u + (uint32_t)lane;
    const uint32_t s = u >> 2;
    const uint32_t ch = u & 3u;
    const uint32_t hr = fast_div(s, hp.div_hw);
    const int ix = (int)(s - hr * (uint32_t)hp.hw) - cp.pw;
    const int iy = ih_base + (int)hr;
    const uint32_t bad =
        (uint32_t)(iy | (h1 - iy) | ix | (w1 - ix) | (hp.ns - 1 - (int)s)) & kOobOffset;
    // modulo 2^32: exact for pixels inside the image, the only ones not rejected
    const uint32_t pix = (uint32_t)iy * (uint32_t)cp.w + (uint32_t)ix;
    return (img_base + pix * pix_bytes + (uint32_t)cb * 64u + ch * 16u) | bad;
  };
  auto halo_lds = [&](int buf) __attribute__((always_inline)) {
    return smem_addr + (uint32_t)kHaloOff0 + (uint32_t)(buf * hp.hb);
  };
  // Window atom a of channel block cb into image buf, or (real false) an atom of zeros into the
  // spare one.
  auto issue_halo = [&](int a, int cb, int buf, bool real) __attribute__((always_inline)) {
    if (real)
      issue_atom_if(rx, halo_lds(buf), a * 1024, halo_src(a, cb), true);
    else
      issue_atom_if(rx, smem_addr + (uint32_t)kHaloJunk, 0, kOobOffset, true);
  };
  // Filter tile of (channel block cb, tap) into ring slot `stage` (a tile past the end reads
  // nothing and lands zeros).
  auto issue_b = [&](int stage, int cb, int tap, bool live) __attribute__((always_inline)) {
    // (the step counters are uniform; read from the first lane, the descriptor is built with
    // scalar instructions)
    const uint32_t col = __builtin_amdgcn_readfirstlane((uint32_t)(tap * cp.c8 + cb * 32) * 2u);
    const int lv = __builtin_amdgcn_readfirstlane(live ? 1 : 0);
    rsrc_t r = rsrc_advance(rw, col);
    if (!lv) r.z = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      issue_atom_settled(r, smem_addr + (uint32_t)(stage * kHaloBStage), (2 * wave + j) * 1024, ob[j]);
  };

  const int cb32 = hp.cb32, rs = hp.rs, S = cp.s, R = cp.r;
  const int steps = cb32 * rs;
  // Counters, stepped once per product step (no division): the step whose fragments are read
  // next (channel block, filter row and column) and the step whose filter tile is copied next.
  int rd_cb = 0, rd_r = 0, rd_s = 0;
  int bc_cb = 0, bc_tap = 0;
  auto step_rd = [&]() __attribute__((always_inline)) {
    if (++rd_s == S) {
      rd_s = 0;
      if (++rd_r == R) {
        rd_r = 0;
        ++rd_cb;
      }
    }
  };
  auto copy_b_next = [&](int stage) __attribute__((always_inline)) {
    issue_b(stage, bc_cb, bc_tap, bc_cb < cb32);
    if (++bc_tap == rs) {
      bc_tap = 0;
      ++bc_cb;
    }
  };

  // ---- prologue: window of block 0, filter tiles 0..3, and the first window atoms of block 1,
  // in the order the loop's waits count on (each "step" before step 0 issues its filter tile,
  // then HS window atoms).
  {
    const int per_wave = (hp.hat + 3) >> 2;
    for (int i = 0; i < per_wave; ++i) {
      const int a = wave * per_wave + i;
      issue_halo(a, 0, 0, a < hp.hat);
    }
  }
  copy_b_next(0);
  copy_b_next(1);
#pragma unroll
  for (int i = 0; i < HS; ++i) issue_halo(0, 0, 0, false);
  copy_b_next(2);
#pragma unroll
  for (int i = 0; i < HS; ++i) issue_halo(0, 0, 0, false);
  copy_b_next(3);
#pragma unroll
  for (int i = 0; i < HS; ++i) {
    const int a = wave * HS + i;
    issue_halo(a, 1, 1, a < hp.hat && 1 < cb32);
  }
  // window 0 and filter tile 0 landed (the 3 later tiles and their window atoms may be in flight)
  stage_barrier<6 + 3 * HS>();

  f32x4_t acc[kHaloFN][kHaloFM];
  zero_acc<T>(acc);
  HaloFrags f0, f1;
#pragma unroll
  for (int f = 0; f < kHaloFM; ++f) f0.a[f] = *(const bf16x8_t*)(smem + kHaloOff0 + a0[f]);
#pragma unroll
  for (int fn = 0; fn < kHaloFN; ++fn) f0.b[fn] = *(const bf16x8_t*)(smem + b0 + fn * 1024);
  step_rd();  // fragments of step 1 come next

  // One product step t on `cur` (stage SI = t % 4 holds its filter tile), reading the fragments
  // of step t + 1 into `nxt`, copying filter tile t + 4 into stage SI and HS window atoms.
  auto step = [&](auto si, const HaloFrags& cur, HaloFrags& nxt) __attribute__((always_inline)) {
    constexpr int SI = decltype(si)::value;
    // Step t + 1 reads a new window: every window atom of it (issued at least two steps ago)
    // must have landed; otherwise only filter tile t + 1.
    if (rd_r == 0 && rd_s == 0)
      stage_barrier<2 + HS>();
    else
      stage_barrier<4 + 3 * HS>();
    const uint8_t* hA = smem + kHaloOff0 + (rd_cb & 1) * hp.hb +
                        (rd_r * cp.dh * hp.hw + rd_s * cp.dw) * kHaloPitch;
    const uint8_t* sB = smem + ((SI + 1) % kHaloStages) * kHaloBStage + b0;
    // Window atoms of this step: position u of block rd_cb's copy window for block rd_cb + 1.
    const int u = rd_r * S + rd_s;
    const bool win = u <= rs - 2 && rd_cb + 1 < cb32;
    const int nbuf = (rd_cb + 1) & 1;
    constexpr int P = kHaloFM * kHaloFN, RD = kHaloFM + kHaloFN, CP = 2 + HS, H = P / (2 * CP);
    // Product i is preceded by at most one fragment read (read r before product r·P/RD) and at
    // most one copy (copy j halfway between products j·P/CP and (j+1)·P/CP; copy 0 issues both
    // filter atoms, copy 1 none): compile-time indices throughout.
    for_stages<P>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      constexpr int r = (i * RD + P - 1) / P;
      if constexpr (r < ((i + 1) * RD + P - 1) / P) {
        if constexpr (r < kHaloFM)
          nxt.a[r] = *(const bf16x8_t*)(hA + a0[r]);
        else
          nxt.b[r - kHaloFM] = *(const bf16x8_t*)(sB + (r - kHaloFM) * 1024);
      }
      if constexpr (i >= H) {
        constexpr int j = ((i - H) * CP + P - 1) / P;
        if constexpr (j < ((i + 1 - H) * CP + P - 1) / P) {
          if constexpr (j == 0) copy_b_next(SI);
          if constexpr (j >= 2) {
            const int a = (u * 4 + wave) * HS + (j - 2);
            issue_halo(a, rd_cb + 1, nbuf, win && a < hp.hat);
          }
        }
      }
      mfma16<true, 0>(acc[i / kHaloFM][i % kHaloFM], cur.b[i / kHaloFM], cur.a[i % kHaloFM]);
    });
    step_rd();
  };

  if constexpr (TAPS == 0) {
    int t = 0;
    for (; t + 4 <= steps; t += 4) {
      step(std::integral_constant<int, 0>{}, f0, f1);
      step(std::integral_constant<int, 1>{}, f1, f0);
      step(std::integral_constant<int, 2>{}, f0, f1);
      step(std::integral_constant<int, 3>{}, f1, f0);
    }
    if (t < steps) step(std::integral_constant<int, 0>{}, f0, f1);
    if (t + 1 < steps) step(std::integral_constant<int, 1>{}, f1, f0);
    if (t + 2 < steps) step(std::integral_constant<int, 2>{}, f0, f1);
  } else {
    // The same steps, copies and waits as above, with the taps of a block unrolled.  Window
    // offsets of this wave's atoms at every copy position of a block, for channel block 0 (a
    // block's 64-byte channel offset goes in as the atom's scalar offset): a position's atoms
    // cover the same pixels in every block.  Units outside the image or the window get exactly
    // 2^31.
    static_assert(TAPS >= 4, "a filter tile four steps ahead lies at most one block ahead");
    uint32_t woff[TAPS - 1][HS];
#pragma unroll
    for (int u = 0; u < TAPS - 1; ++u)
#pragma unroll
      for (int j = 0; j < HS; ++j) {
        const uint32_t o = halo_src((u * 4 + wave) * HS + j, 0);
        woff[u][j] = (o & kOobOffset) ? kOobOffset : o;
      }
    const uint32_t junk = smem_addr + (uint32_t)kHaloJunk;
    const uint32_t c8x2 = (uint32_t)cp.c8 * 2u;
    // Step t = cb·TAPS + K (K a compile-time tap index): the products on `cur`, the fragments of
    // step t+1 into `nxt`, filter tile t+4 into stage t % 4, and the window atoms of copy
    // position K+1 of block cb+1 (K <= TAPS-3), none (K = TAPS-2: atoms of zeros into the spare
    // one) or position 0 of block cb+2 (K = TAPS-1), as the counters of the general loop give.
    auto step_t = [&](auto kc, const HaloFrags& cur, HaloFrags& nxt, int cb, int t) __attribute__((always_inline)) {
      constexpr int K = decltype(kc)::value;
      if constexpr (K == TAPS - 1)
        stage_barrier<2 + HS>();  // step t+1 opens block cb+1: its whole window has landed
      else
        stage_barrier<4 + 3 * HS>();
      const int nblk = K == TAPS - 1 ? cb + 1 : cb;
      const uint32_t hA = (uint32_t)kHaloOff0 + (uint32_t)(nblk & 1) * (uint32_t)hp.hb +
                          (uint32_t)hp.tap_off[K == TAPS - 1 ? 0 : K + 1];
      const uint32_t vB = b0 + (uint32_t)((t + 1) & 3) * (uint32_t)kHaloBStage;
      constexpr int FB = (K + 4) / TAPS, FT = (K + 4) % TAPS;  // filter tile t+4: block cb+FB, tap FT
      // (a tile past the last block re-reads block 0's first tile into a stage nobody reads again)
      const uint32_t fcol = cb + FB < cb32 ? (uint32_t)FT * c8x2 + (uint32_t)(cb + FB) * 64u : 0u;
      const uint32_t fst = smem_addr + (uint32_t)(t & 3) * (uint32_t)kHaloBStage;
      constexpr int WP = K <= TAPS - 3 ? K + 1 : (K == TAPS - 1 ? 0 : -1);
      const int wblk = K == TAPS - 1 ? cb + 2 : cb + 1;
      const int lim = WP >= 0 && wblk < cb32 ? hp.hat : 0;  // atoms below lim are real
      // (a block past the last copies block 0's channels, into the spare atom)
      const uint32_t wsoff = lim ? (uint32_t)wblk * 64u : 0u;
      const uint32_t wbase = smem_addr + (uint32_t)kHaloOff0 + (uint32_t)(wblk & 1) * (uint32_t)hp.hb;
      constexpr int P = kHaloFM * kHaloFN, RD = kHaloFM + kHaloFN, CP = 2 + HS, H = P / (2 * CP);
      for_stages<P>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        constexpr int r = (i * RD + P - 1) / P;
        if constexpr (r < ((i + 1) * RD + P - 1) / P) {
          if constexpr (r < kHaloFM)
            nxt.a[r] = *(const bf16x8_t*)(smem + hA + a0[r]);
          else
            nxt.b[r - kHaloFM] = *(const bf16x8_t*)(smem + vB + (r - kHaloFM) * 1024);
        }
        if constexpr (i >= H) {
          constexpr int j = ((i - H) * CP + P - 1) / P;
          if constexpr (j < ((i + 1 - H) * CP + P - 1) / P) {
            if constexpr (j == 0) {
              issue_atom_so(rw, fst + (uint32_t)(2 * wave) * 1024u, ob[0], fcol);
              issue_atom_so(rw, fst + (uint32_t)(2 * wave + 1) * 1024u, ob[1], fcol);
            }
            if constexpr (j >= 2) {
              if constexpr (WP < 0) {
                issue_atom_so(rx, junk, kOobOffset, 0u);
              } else {
                const int a = (WP * 4 + wave) * HS + (j - 2);
                const uint32_t place = wbase + (uint32_t)a * 1024u;
                uint32_t lds;
                // (a scalar select written out: the compiler would branch on the uniform test)
                asm("s_cmp_lt_i32 %1, %2\n\ts_cselect_b32 %0, %3, %4"
                    : "=s"(lds)
                    : "s"(a), "s"(lim), "s"(place), "s"(junk)
                    : "scc");
                issue_atom_so(rx, lds, woff[WP][j - 2], wsoff);
              }
            }
          }
        }
        // serpentine over the fragment grid (as the GEMM's k-step): consecutive products share
        // an operand
        constexpr int fn = i / kHaloFM, fm = (fn & 1) ? kHaloFM - 1 - i % kHaloFM : i % kHaloFM;
        mfma16<true, 0>(acc[fn][fm], cur.b[fn], cur.a[fm]);
      });
    };
    // Two blocks per iteration keep each step's fragment sets (f0 at even steps) compile-time.
    auto block = [&](auto odd, int cb) __attribute__((always_inline)) {
      const int t0 = cb * TAPS;
      for_stages<TAPS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int K = decltype(kc)::value;
        if constexpr ((decltype(odd)::value * TAPS + K) % 2 == 0)
          step_t(kc, f0, f1, cb, t0 + K);
        else
          step_t(kc, f1, f0, cb, t0 + K);
      });
    };
    int cb = 0;
    for (; cb + 2 <= cb32; cb += 2) {
      block(std::false_type{}, cb);
      block(std::true_type{}, cb + 1);
    }
    if (cb < cb32) block(std::false_type{}, cb);
  }

  drain_acc<T>(acc);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  stage_barrier<0>();  // every copy landed and every wave done reading: LDS becomes the park
  GemmParams pe = cp.g;
  pe.M = m0 + rows;
  store_tile<T, OUT, SCALED>(acc, smem + wave * (T::RingBytes / 4), pe, m0 + 112 * wave, n0, lane);
}

}  // namespace tbg
