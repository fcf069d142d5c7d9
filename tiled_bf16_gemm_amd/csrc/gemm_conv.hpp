// Implicit-GEMM 2-D convolution: the barrier ring of gemm_ring.hpp (two stages) whose A tiles
// are blocks of the im2col matrix, formed by the copy itself.
//
// "2 · Le Tensor Memory Accelerator", section "im2col": the copy performs the im2col transform,
// so the convolution becomes a GEMM and the im2col matrix is never stored.  The GEMM here is
//   Y (N·OH·OW × K) = im2col(X) (N·OH·OW × R·S·C) · Wᵀ,  W viewed as K × (R·S·C),
// its K loop running over filter taps (r, s) and, inside each tap, 64-channel blocks.  For the
// A tile of output pixels m0..m0+BM-1 at tap (r, s) and channels c0..c0+63, each lane's 16-byte
// atom chunk comes from X[n, oh·sh − ph + r·dh, ow·sw − pw + s·dw, c0 + 8·chunk .. +7] of its
// pixel; a window position outside the image (the zero padding), a pixel past the output and a
// chunk past the channels all take the buffer's out-of-range offset and land zeros — the
// out-of-bounds fill that "removes the edge guards of convolutions" in the same page.  The B
// tile is the filters' N×K box at column (r·S + s)·c8 + c0.  Fragment reads, products and the
// epilogue are the GEMM's.
#pragma once
#include "gemm_common.hpp"
#include "gemm_ring.hpp"

namespace tbg {

template <int BM, int BN, int OUT, int SCALED>
__global__ void __launch_bounds__(kThreads, (RingCfg<BM, BN, 2>::MinBlocks)) gemm_conv_kernel(ConvParams cp) {
  using T = TileCfg<BM, BN>;
  constexpr int BL = 1;  // the filters are stored K × (R·S·c8): the GEMM's B stored N×K
  const GemmParams& p = cp.g;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::StageBytes];
  const int lane = threadIdx.x & 63;
  // The wave index is uniform: keeping it scalar keeps every address derived from it scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- im2col atoms of A: this wave owns box rows (BM/4)*wave .. +BM/4-1 (as the ring) ----------
  // Per atom, the lane's output pixel as its window origin (ih0, iw0) and the byte offset of
  // X[n, ih0, iw0, 0] (negative when the origin is in the padding); a pixel past the output gets
  // an origin no tap can bring inside.
  const int cpix = cp.c8 * 2;  // bytes per pixel
  int ih0[T::AtomsA], iw0[T::AtomsA], pix[T::AtomsA];
#pragma unroll
  for (int j = 0; j < T::AtomsA; ++j) {
    const int row = (BM / 4) * wave + 8 * j + (lane >> 3);
    const int m = m0 + row;
    if (m < p.M) {
      const int per_img = cp.oh * cp.ow;
      const int n = m / per_img;
      const int rem = m - n * per_img;
      const int oh = rem / cp.ow;
      const int ow = rem - oh * cp.ow;
      ih0[j] = oh * cp.sh - cp.ph;
      iw0[j] = ow * cp.sw - cp.pw;
      pix[j] = ((n * cp.h + ih0[j]) * cp.w + iw0[j]) * cpix;
    } else {
      ih0[j] = -(1 << 28);
      iw0[j] = 0;
      pix[j] = 0;
    }
  }
  // The lane's chunk of each atom is fixed (its row's 2-row swizzle); pixc folds its byte offset
  // into the pixel's.
  LaneChunk la[T::AtomsA];
  int pixc[T::AtomsA];
#pragma unroll
  for (int j = 0; j < T::AtomsA; ++j) {
    const int row = (BM / 4) * wave + 8 * j + (lane >> 3);
    la[j].chunk = (lane & 7) ^ row_xor<kSwizzle128B2Row>(row);
    pixc[j] = pix[j] + la[j].chunk * 16;
  }
  const uint32_t pitch_b = (uint32_t)(cp.ldw * 2);
  LaneChunk lb[T::AtomsB];
#pragma unroll
  for (int i = 0; i < T::AtomsB; ++i) {
    lb[i] = lane_chunk<kSwizzle128B2Row>((BN / 4) * wave + 8 * i, lane, pitch_b);
    mask_row(lb[i], (BN / 4) * wave + 8 * i + (lane >> 3), p.N - n0);
  }
  const int ktiles = cp.r * cp.s * cp.cblocks;
  const uint32_t smem_addr = lds_addr_of(smem);
  const rsrc_t rx = make_rsrc(cp.X, cp.x_bytes);
  // The filters' rows n0.. as one open-range buffer (rows past N are masked per lane above,
  // channels past c8 by the chunk count); each K tile moves its base to the tap's columns.
  const rsrc_t rw = make_rsrc(cp.W + (uint64_t)n0 * cp.ldw, 0x7FFFFFFFull);

  // The copies of one K tile into `stage`; la receives the tile's per-lane A sources.  make_copy
  // is called once per K tile, in order (tiles 0 and 1 before the loop, then tile kt+2 during
  // tile kt), so it keeps the next tile's position as counters and steps them: channel block cb
  // of filter tap (rr, ss), K tile (rr·S + ss)·cblocks + cb; no division per tile.  A lane whose
  // window position (iy, ix) lies outside the image takes an offset with bit 31 set, which the
  // buffer's range (below 2^31) rejects: bit 31 of iy | (h-1-iy) | ix | (w-1-ix) is set exactly
  // when iy or ix is outside [0, h) or [0, w), so the test needs no compare or branch.  Tiles
  // past the end are issued fully masked the same way.
  int nx_kt = 0, nx_cb = 0, nx_rr = 0, nx_ss = 0;
  const int h1 = cp.h - 1, w1 = cp.w - 1;
  auto make_copy = [&](int stage, LaneChunk* la) __attribute__((always_inline)) {
    const bool live = nx_kt < ktiles;
    const int c0 = nx_cb * 64;
    const int dy = nx_rr * cp.dh, dx = nx_ss * cp.dw;
    const int tap = nx_rr * cp.s + nx_ss;
    // modulo 2^32: exact wherever the window lies in the image, the only places it is used
    const uint32_t tap_off = ((uint32_t)dy * (uint32_t)cp.w + (uint32_t)dx) * (uint32_t)cpix + (uint32_t)c0 * 2u;
    const uint32_t dead = live ? 0u : kOobOffset;
#pragma unroll
    for (int j = 0; j < T::AtomsA; ++j) {
      const int iy = ih0[j] + dy, ix = iw0[j] + dx;
      const uint32_t outside = (uint32_t)(iy | (h1 - iy) | ix | (w1 - ix)) & kOobOffset;
      la[j].offset = ((uint32_t)pixc[j] + tap_off) | outside | dead;
    }
    TileCopy tc;
    const uint32_t sa = smem_addr + stage * T::StageBytes;
    tc.ra = rx;
    tc.lds_a = sa + (BM / 4) * wave * 128;
    tc.cvalid_a = live ? (cp.c8 - c0) >> 3 : -1;
    tc.rb = rsrc_advance(rw, (uint64_t)(tap * cp.c8 + c0) * 2u);
    if (!live) tc.rb.z = 0;  // a tile past the end reads no filter column
    tc.lds_b = sa + T::ABytes + (BN / 4) * wave * 128;
    tc.cvalid_b = tc.cvalid_a;
    ++nx_kt;
    if (++nx_cb == cp.cblocks) {
      nx_cb = 0;
      if (++nx_ss == cp.s) {
        nx_ss = 0;
        ++nx_rr;
      }
    }
    return tc;
  };

  const FragAddr<T> fa = make_frag_addr<T>(wm, wn, lane);
  f32x4_t acc[T::FN][T::FM];
  zero_acc<T>(acc);
  {
    Frags<T> f0, f1;
    const TileCopy none{};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const TileCopy tc = make_copy(t, la);
#pragma unroll
      for (int j = 0; j < T::Atoms; ++j) copy_atom<T>(tc, la, lb, j);
    }
    stage_barrier<T::Atoms>();  // tile 0 landed; tile 1 may be in flight
#pragma unroll
    for (int idx = 0; idx < T::Reads; ++idx) read_frag<T, BL>(f0, fa, smem, smem + T::ABytes, 0, idx);
    // Tile kt on stage CUR = kt & 1, a compile-time constant: two tiles per loop iteration.
    // MASK false (channels a multiple of 64: every channel block whole) leaves out the chunk
    // tests of the copies; the offsets and ranges of make_copy still mask the window, the rows
    // past N and the tiles past the end.
    auto kloop = [&](auto maskc) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(maskc)::value;
      auto tile = [&](int kt, auto stage) __attribute__((always_inline)) {
        constexpr int cur = decltype(stage)::value;
        const uint8_t* sA = smem + cur * T::StageBytes;
        kstep<T, BL, false>(acc, f0, f1, fa, sA, sA + T::ABytes, 1, none, la, lb);
        stage_barrier<0>();  // tile kt+1 landed everywhere; stage kt&1 free
        const uint8_t* nA = smem + (cur ^ 1) * T::StageBytes;
        const TileCopy tc = make_copy(cur, la);  // tile kt+2
        kstep<T, BL, true, MASK, MASK>(acc, f1, f0, fa, nA, nA + T::ABytes, 0, tc, la, lb);
      };
      int kt = 0;
      for (; kt + 2 <= ktiles; kt += 2) {
        tile(kt, std::integral_constant<int, 0>{});
        tile(kt + 1, std::integral_constant<int, 1>{});
      }
      if (kt < ktiles) tile(kt, std::integral_constant<int, 0>{});
    };
    // (the second copy of the loop only where registers allow it: two loops of the 256-row
    // tiles would spill)
    if (BM * BN <= 128 * 128 && cp.c8 % 64 == 0)
      kloop(std::integral_constant<bool, !(BM * BN <= 128 * 128)>{});
    else
      kloop(std::true_type{});
  }
  drain_acc<T>(acc);
  stage_barrier<0>();
  store_tile<T, OUT, SCALED>(acc, smem + wave * (T::RingBytes / 4), p, m0 + wm * T::TM, n0 + wn * T::TN, lane);
}

}  // namespace tbg
