/*
 * oracle.c — plain, slow CPU reference for the tiled copy, the bf16 GEMM, the im2col copy and
 * the 2-D convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load this file's
 * library: only the test suite, the smoke check and the CPU-baseline leg of the benchmark do.
 * It shares no code, header, table or constant with the GPU library; it takes raw parameters,
 * never the packed descriptor.
 *
 * Sources (web pages; cited by title and section):
 *   [TMA]   "2 · Le Tensor Memory Accelerator" (mkdocs.reaper.mx, cuda-moderne/02-tma)
 *   [MAP]   "H100 · cuTensorMap（TMA 描述符）" (runguoli.com, h100-cuda-programming/l4)
 *   [GEMM]  "GEMM: la moltiplicazione di matrici sull'hardware" (book.paithon.it)
 *
 * Parity pins: every function here is pinned by CPU tests against facts the pages or plain
 * mathematics fix (per-bit swizzle formulas, the worked descriptor example, brute-force index
 * decoding, exact rational dot products, closed forms).  The one part left unpinned beyond
 * the tolerance is the hardware's own accumulation order inside a matrix instruction.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------
 * Element conversions, written from the IEEE-754 binary16/bfloat16/binary32 definitions.
 * bfloat16 is the top half of a binary32: widening is a 16-bit shift, which is exact.
 * ---------------------------------------------------------------------------------------- */
static double bf16_to_f64(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.  Exponent field 0:
 * subnormal, (-1)^s * f * 2^-24; 1..30: (-1)^s * (1024 + f) * 2^(e-25); 31: infinity (f = 0) or
 * NaN.  Every binary16 value is exact in binary64. */
static double f16_to_f64(uint16_t h) {
    const int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

/* A 16-bit input element of the GEMM: kind 0 bfloat16, 1 binary16. */
static double in_to_f64(uint16_t h, int kind) { return kind == 1 ? f16_to_f64(h) : bf16_to_f64(h); }

void oracle_f16_to_f64_array(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f16_to_f64(in[i]);
}

/* binary32 -> bfloat16, round to nearest, ties to even.  A NaN stays a NaN (quiet bit set,
 * sign and upper payload kept); everything else follows the rounding definition on the bit
 * pattern: add half an ulp of the kept part, plus one if the kept part is odd, and truncate. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------------------------
 * O1 — swizzle.  [MAP] §11.3: a' = a ^ ((a & Y_mask) >> 3), low bits a[3:0] never change.
 * The section's per-mode bit lists (32B: a[4]^=a[7]; 64B: a[5:4]^=a[8:7]; 128B: a[6:4]^=a[9:7])
 * fix Y_mask as bits 7, 8:7 and 9:7 respectively (the single "1 << 7" printed there only
 * reproduces the 32B row).  mode: 0 none, 1 32B, 2 64B, 3 128B.
 * mode 4 is the library's extension of the same XOR form with the row bits taken one place
 * higher, a ^ ((a & 0x700) >> 4), i.e. a[6:4] ^= a[10:8]; it is defined by that mask and shift.
 * mode 5 is the library's layout for boxes read back with the transposing 8-byte read; it is
 * not of that form and is defined bit by bit: a[4] ^= a[9], a[5] ^= a[8], a[6] ^= a[10].
 * ---------------------------------------------------------------------------------------- */
uint64_t oracle_swizzle_general(uint64_t a, uint64_t y_mask, unsigned shift) {
    return a ^ ((a & y_mask) >> shift);
}

uint64_t oracle_swizzle(uint64_t a, int mode) {
    switch (mode) {
        case 0: return a;
        case 1: return oracle_swizzle_general(a, 0x080u, 3);
        case 2: return oracle_swizzle_general(a, 0x180u, 3);
        case 3: return oracle_swizzle_general(a, 0x380u, 3);
        case 4: return oracle_swizzle_general(a, 0x700u, 4);
        case 5: return a ^ (((a >> 9) & 1u) << 4) ^ (((a >> 8) & 1u) << 5) ^ (((a >> 10) & 1u) << 6);
        default: return (uint64_t)-1;
    }
}

void oracle_swizzle_array(const uint64_t* in, uint64_t* out, int64_t n, int mode) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_swizzle(in[i], mode);
}

/* Size in bytes of the aligned block inside which a mode permutes 16-byte units. */
static uint64_t swizzle_span(int mode) {
    return mode == 1 ? 32u : mode == 2 ? 64u : (mode == 3 || mode == 4 || mode == 5) ? 128u : 1u;
}

/* ------------------------------------------------------------------------------------------
 * O2 — tiled copy of one box into a dense image.
 *   [MAP] §8.2 globalDim: elements per dimension, innermost first.
 *   [MAP] §8.3 globalStrides: rank-1 byte strides of dims 1..rank-1; dim 0's stride is the
 *         element size.
 *   [MAP] §9.1 elementStrides: per-dimension step in elements (nonzero, at most 8).
 *   [MAP] §9.2 boxDim: the traversal box, in elements.
 *   [MAP] §14 / [TMA] §2.5: elements outside the tensor are filled in the destination only
 *         (zero, or NaN); the source is not touched.
 *   [MAP] §11: the destination byte offset goes through the swizzle.
 * Readings (pages silent): the box covers box[i] elements of traversal, of which every
 * estr[i]-th is copied, so n[i] = ceil(box[i]/estr[i]) land densely, innermost first, with no
 * padding; coordinates are signed; the swizzle acts on the byte offset inside the image.
 * NaN fill writes the canonical quiet NaN of the element type.
 *   elsize: 1, 2 or 4 bytes; nan_kind: 0 none (integer), 1 bf16, 2 f16, 3 f32, 4 E4M3 (0x7F),
 *   5 E5M2 (0x7E, the quiet NaN with the top fraction bit set).
 * Returns the image size in bytes, or 0 on an argument this plain reference does not take.
 * ---------------------------------------------------------------------------------------- */
uint64_t oracle_tiled_copy(int elsize, int rank, const void* src, const uint64_t* dims,
                           const uint64_t* strides_bytes, const uint32_t* box, const uint32_t* estr,
                           int swizzle, int oob_nan, int nan_kind, const int32_t* coords, void* dst) {
    if (rank < 1 || rank > 5 || (elsize != 1 && elsize != 2 && elsize != 4)) return 0;
    uint64_t S[5], n[5], dim[5];
    int64_t c[5];
    for (int i = 0; i < 5; ++i) { S[i] = 0; n[i] = 1; dim[i] = 1; c[i] = 0; }
    S[0] = (uint64_t)elsize;
    for (int i = 1; i < rank; ++i) S[i] = strides_bytes[i - 1];
    for (int i = 0; i < rank; ++i) {
        if (estr[i] == 0) return 0;
        n[i] = (box[i] + estr[i] - 1) / estr[i];
        dim[i] = dims[i];
        c[i] = coords[i];
    }
    uint64_t image = (uint64_t)elsize * n[0] * n[1] * n[2] * n[3] * n[4];
    if (swizzle != 0 && image % swizzle_span(swizzle) != 0) return 0;

    uint8_t fill[4] = {0, 0, 0, 0};
    if (oob_nan) {
        if (nan_kind == 1) { fill[0] = 0xC0; fill[1] = 0x7F; }                   /* bf16 0x7FC0 */
        else if (nan_kind == 2) { fill[0] = 0x00; fill[1] = 0x7E; }              /* f16  0x7E00 */
        else if (nan_kind == 3) { fill[2] = 0xC0; fill[3] = 0x7F; }              /* f32  0x7FC00000 */
        else if (nan_kind == 4) { fill[0] = 0x7F; }                              /* E4M3 0x7F */
        else if (nan_kind == 5) { fill[0] = 0x7E; }                              /* E5M2 0x7E */
        else return 0;
    }
    const uint8_t* s = (const uint8_t*)src;
    uint8_t* d = (uint8_t*)dst;

    uint64_t j[5];
    for (j[4] = 0; j[4] < n[4]; ++j[4])
    for (j[3] = 0; j[3] < n[3]; ++j[3])
    for (j[2] = 0; j[2] < n[2]; ++j[2])
    for (j[1] = 0; j[1] < n[1]; ++j[1])
    for (j[0] = 0; j[0] < n[0]; ++j[0]) {
        int inside = 1;
        uint64_t src_off = 0;
        for (int i = 0; i < rank; ++i) {
            int64_t x = c[i] + (int64_t)j[i] * (int64_t)estr[i];
            if (x < 0 || (uint64_t)x >= dim[i]) inside = 0;
            else src_off += (uint64_t)x * S[i];
        }
        uint64_t lin = j[0] + n[0] * (j[1] + n[1] * (j[2] + n[2] * (j[3] + n[3] * j[4])));
        uint64_t off = oracle_swizzle(lin * (uint64_t)elsize, swizzle);
        if (off + (uint64_t)elsize > image) return 0; /* never writes past the image */
        if (inside) memcpy(d + off, s + src_off, (size_t)elsize);
        else memcpy(d + off, fill, (size_t)elsize);
    }
    return image;
}

/* ------------------------------------------------------------------------------------------
 * O2s — tiled store, the other direction of the same copy.  [TMA] §2.5: the copy engine also
 * moves shared memory to global memory, with the same descriptors (the store of a GEMM
 * epilogue).  Box position j takes its value from the image at byte offset
 * swizzle(elsize * lin(j)), exactly where a load of that box puts it, and goes to tensor
 * coordinates coords[i] + j[i]*estr[i].
 * Reading (pages silent on the store's edges): a position outside the tensor is not written —
 * the fill of [MAP] §14 exists only on the load side, and a store never touches memory outside
 * the tensor.
 *   dst: the tensor's bytes (modified in place); image: image_len bytes.
 * Returns the image size in bytes, or 0 on an argument this plain reference does not take.
 * ---------------------------------------------------------------------------------------- */
uint64_t oracle_tiled_store(int elsize, int rank, void* dst, const uint64_t* dims,
                            const uint64_t* strides_bytes, const uint32_t* box, const uint32_t* estr,
                            int swizzle, const int32_t* coords, const void* image, uint64_t image_len) {
    if (rank < 1 || rank > 5 || (elsize != 1 && elsize != 2 && elsize != 4)) return 0;
    uint64_t S[5], n[5], dim[5];
    int64_t c[5];
    for (int i = 0; i < 5; ++i) { S[i] = 0; n[i] = 1; dim[i] = 1; c[i] = 0; }
    S[0] = (uint64_t)elsize;
    for (int i = 1; i < rank; ++i) S[i] = strides_bytes[i - 1];
    for (int i = 0; i < rank; ++i) {
        if (estr[i] == 0) return 0;
        n[i] = (box[i] + estr[i] - 1) / estr[i];
        dim[i] = dims[i];
        c[i] = coords[i];
    }
    uint64_t size = (uint64_t)elsize * n[0] * n[1] * n[2] * n[3] * n[4];
    if (size > image_len) return 0;
    if (swizzle != 0 && size % swizzle_span(swizzle) != 0) return 0;
    const uint8_t* img = (const uint8_t*)image;
    uint8_t* d = (uint8_t*)dst;

    uint64_t j[5];
    for (j[4] = 0; j[4] < n[4]; ++j[4])
    for (j[3] = 0; j[3] < n[3]; ++j[3])
    for (j[2] = 0; j[2] < n[2]; ++j[2])
    for (j[1] = 0; j[1] < n[1]; ++j[1])
    for (j[0] = 0; j[0] < n[0]; ++j[0]) {
        int inside = 1;
        uint64_t dst_off = 0;
        for (int i = 0; i < rank; ++i) {
            int64_t x = c[i] + (int64_t)j[i] * (int64_t)estr[i];
            if (x < 0 || (uint64_t)x >= dim[i]) inside = 0;
            else dst_off += (uint64_t)x * S[i];
        }
        if (!inside) continue;
        uint64_t lin = j[0] + n[0] * (j[1] + n[1] * (j[2] + n[2] * (j[3] + n[3] * j[4])));
        uint64_t off = oracle_swizzle(lin * (uint64_t)elsize, swizzle);
        if (off + (uint64_t)elsize > size) return 0;
        memcpy(d + dst_off, img + off, (size_t)elsize);
    }
    return size;
}

/* ------------------------------------------------------------------------------------------
 * O3 — GEMM.  [GEMM] "Il conto": C = A·B, A (M,K), B (K,N), C (M,N), C_ij = Σ_k A_ik B_kj.
 * [GEMM] tensor-core section: 16-bit inputs (bfloat16 or float16, ab_kind 0 or 1), the sum kept in
 * a wide format.  Here every 16-bit·16-bit product is exact in binary64, the sum runs over k in ascending order in binary64,
 * and the result is rounded once to binary32 (round to nearest even, the C cast).
 *   A: bf16 bits, row-major M×K, leading dimension lda (elements).
 *   B: bf16 bits; b_layout 0: row-major K×N (ldb >= N); 1: N×K with K contiguous (ldb >= K).
 *   rows [m0, m1) of C are produced; out64 (if non-null) gets the binary64 sums and out32
 *   (if non-null) the binary32 results, both row-major with leading dimension ldo, indexed
 *   from row m0.  threads: worker count (0 = library default).
 * ---------------------------------------------------------------------------------------- */
void oracle_gemm_rows(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                      const uint16_t* B, int64_t ldb, int b_layout, int64_t m0, int64_t m1,
                      double* out64, float* out32, int64_t ldo, int threads, double* scratch, int ab_kind) {
    (void)M;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
    if (b_layout == 0) {
        /* Each row's N sums are kept side by side; k runs outermost, so each sum still adds
         * its terms in ascending k. scratch holds N doubles per worker. */
#pragma omp parallel
        {
            int t = 0;
#ifdef _OPENMP
            t = omp_get_thread_num();
#endif
            double* acc = scratch + (size_t)t * (size_t)N;
#pragma omp for schedule(dynamic, 1)
            for (int64_t m = m0; m < m1; ++m) {
                for (int64_t n = 0; n < N; ++n) acc[n] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double a = in_to_f64(A[m * lda + k], ab_kind);
                    const uint16_t* brow = B + k * ldb;
                    for (int64_t n = 0; n < N; ++n) acc[n] += a * in_to_f64(brow[n], ab_kind);
                }
                for (int64_t n = 0; n < N; ++n) {
                    if (out64) out64[(m - m0) * ldo + n] = acc[n];
                    if (out32) out32[(m - m0) * ldo + n] = (float)acc[n];
                }
            }
        }
    } else {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t m = m0; m < m1; ++m) {
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += in_to_f64(A[m * lda + k], ab_kind) * in_to_f64(B[n * ldb + k], ab_kind);
                if (out64) out64[(m - m0) * ldo + n] = acc;
                if (out32) out32[(m - m0) * ldo + n] = (float)acc;
            }
        }
    }
}

/* The same sum at individual (m, n) points, for sampled checks of large products. */
void oracle_gemm_points(int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                        int b_layout, int64_t npts, const int64_t* ms, const int64_t* ns,
                        double* out64, float* out32, int ab_kind) {
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npts; ++p) {
        int64_t m = ms[p], n = ns[p];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            uint16_t b = b_layout == 0 ? B[k * ldb + n] : B[n * ldb + k];
            acc += in_to_f64(A[m * lda + k], ab_kind) * in_to_f64(b, ab_kind);
        }
        if (out64) out64[p] = acc;
        if (out32) out32[p] = (float)acc;
    }
}

/* ------------------------------------------------------------------------------------------
 * Output extent of a convolution along one spatial dimension: the number of window positions
 * p >= 0 with p*stride - pad_lo + dil*(filt-1) <= in - 1 + pad_hi, i.e.
 * floor((in + pad_lo + pad_hi - dil*(filt-1) - 1) / stride) + 1, or 0 if the window never fits.
 * ---------------------------------------------------------------------------------------- */
int64_t oracle_conv_out_dim(int64_t in, int64_t pad_lo, int64_t pad_hi, int64_t stride, int64_t dil,
                            int64_t filt) {
    int64_t span = in + pad_lo + pad_hi - dil * (filt - 1) - 1;
    if (stride < 1 || dil < 1 || filt < 1 || span < 0) return 0;
    return span / stride + 1;
}

/* ------------------------------------------------------------------------------------------
 * O2i — im2col copy: one block of the im2col matrix of a 2-D convolution.
 * [TMA] section "im2col": a copy mode dedicated to convolution performs the im2col transform
 * while copying, so the convolution becomes a GEMM and the intermediate matrix is never stored.
 * The page gives nothing more; the reading taken (plain im2col with the tiled mode's image,
 * swizzle and fill rules):
 *   - the tensor X is NHWC: dims = {C, W, H, N} innermost first, byte strides {sW, sH, sN}
 *     (the channel stride is the element size);
 *   - row m of the im2col matrix is output pixel m = (n*OH + oh)*OW + ow; column (r, s, c) is
 *     filter tap (r along H, s along W) and channel c; its element is
 *     X[n, oh*sh - ph + r*dh, ow*sw - pw + s*dw, c], zero (or the fill) where that position is
 *     outside the tensor — the zero padding of the convolution — and for rows m outside
 *     0..N*OH*OW-1 and channels outside 0..C-1;
 *   - one copy takes `pixels` consecutive rows from m0 and `channels` consecutive channels from
 *     c0 at one tap (r, s): coords = {c0, m0, s, r}; the image is dense, channel fastest
 *     (element (i, j) at byte elsize*(j + channels*i)), through the swizzle like a tiled copy.
 *   pad_lo/pad_hi/cstride/dil/filt: {along W, along H}.  elsize, nan_kind as oracle_tiled_copy.
 * Returns the image size in bytes, or 0 on an argument this plain reference does not take.
 * ---------------------------------------------------------------------------------------- */
uint64_t oracle_im2col_copy(int elsize, const void* src, const uint64_t* dims, const uint64_t* strides_bytes,
                            const int32_t* pad_lo, const int32_t* pad_hi, const int32_t* cstride,
                            const int32_t* dil, const int32_t* filt, uint32_t channels, uint32_t pixels,
                            int swizzle, int oob_nan, int nan_kind, const int32_t* coords, void* dst) {
    if (elsize != 1 && elsize != 2 && elsize != 4) return 0;
    const int64_t C = (int64_t)dims[0], W = (int64_t)dims[1], H = (int64_t)dims[2], N = (int64_t)dims[3];
    const int64_t OW = oracle_conv_out_dim(W, pad_lo[0], pad_hi[0], cstride[0], dil[0], filt[0]);
    const int64_t OH = oracle_conv_out_dim(H, pad_lo[1], pad_hi[1], cstride[1], dil[1], filt[1]);
    if (OW < 1 || OH < 1) return 0;
    const uint64_t image = (uint64_t)elsize * channels * pixels;
    if (swizzle != 0 && image % swizzle_span(swizzle) != 0) return 0;
    uint8_t fill[4] = {0, 0, 0, 0};
    if (oob_nan) {
        if (nan_kind == 1) { fill[0] = 0xC0; fill[1] = 0x7F; }
        else if (nan_kind == 2) { fill[0] = 0x00; fill[1] = 0x7E; }
        else if (nan_kind == 3) { fill[2] = 0xC0; fill[3] = 0x7F; }
        else if (nan_kind == 4) { fill[0] = 0x7F; }
        else if (nan_kind == 5) { fill[0] = 0x7E; }
        else return 0;
    }
    const int64_t c0 = coords[0], m0 = coords[1], tap_s = coords[2], tap_r = coords[3];
    const uint8_t* x = (const uint8_t*)src;
    uint8_t* d = (uint8_t*)dst;
    for (uint64_t i = 0; i < pixels; ++i) {
        const int64_t m = m0 + (int64_t)i;
        int row_inside = m >= 0 && m < N * OH * OW;
        int64_t n = 0, ih = 0, iw = 0;
        if (row_inside) {
            const int64_t ow = m % OW, oh = (m / OW) % OH;
            n = m / (OW * OH);
            ih = oh * cstride[1] - pad_lo[1] + tap_r * dil[1];
            iw = ow * cstride[0] - pad_lo[0] + tap_s * dil[0];
            row_inside = ih >= 0 && ih < H && iw >= 0 && iw < W;
        }
        for (uint64_t j = 0; j < channels; ++j) {
            const int64_t c = c0 + (int64_t)j;
            const uint64_t off = oracle_swizzle((uint64_t)elsize * (j + (uint64_t)channels * i), swizzle);
            if (off + (uint64_t)elsize > image) return 0;
            if (row_inside && c >= 0 && c < C) {
                const uint64_t so = (uint64_t)c * (uint64_t)elsize + (uint64_t)iw * strides_bytes[0] +
                                    (uint64_t)ih * strides_bytes[1] + (uint64_t)n * strides_bytes[2];
                memcpy(d + off, x + so, (size_t)elsize);
            } else {
                memcpy(d + off, fill, (size_t)elsize);
            }
        }
    }
    return image;
}

/* ------------------------------------------------------------------------------------------
 * O5 — 2-D convolution, by its definition (the product that [TMA]'s im2col mode turns into a
 * GEMM):  Y[n, oh, ow, k] = Σ_r Σ_s Σ_c X[n, oh*sh - ph + r*dh, ow*sw - pw + s*dw, c] · Wt[k, r, s, c],
 * terms whose input position lies outside X counting as zero (zero padding).  Layouts: X NHWC
 * dense, Wt KRSC dense, Y row-major (N*OH*OW) × K with leading dimension ldy (row m = output
 * pixel (n*OH + oh)*OW + ow).  Every bf16·bf16 product is exact in binary64; each sum runs over
 * (r, s, c) in ascending order in binary64 and is rounded once to binary32.  Rows [m0, m1) of Y
 * are produced (indexed from m0 in out32 / out64, either may be null).
 *   geom: {pad_h, pad_w, pad_h_end, pad_w_end, stride_h, stride_w, dil_h, dil_w}.
 * ---------------------------------------------------------------------------------------- */
void oracle_conv2d_rows(const uint16_t* X, const uint16_t* Wt, int64_t N, int64_t H, int64_t Wd, int64_t C,
                        int64_t K, int64_t R, int64_t S, const int32_t* geom, int64_t m0, int64_t m1,
                        double* out64, float* out32, int64_t ldy, int threads) {
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
    const int64_t ph = geom[0], pw = geom[1], sh = geom[4], sw = geom[5], dh = geom[6], dw = geom[7];
    const int64_t OH = oracle_conv_out_dim(H, geom[0], geom[2], sh, dh, R);
    const int64_t OW = oracle_conv_out_dim(Wd, geom[1], geom[3], sw, dw, S);
    (void)N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = m0; m < m1; ++m) {
        const int64_t ow = m % OW, oh = (m / OW) % OH, n = m / (OW * OH);
        for (int64_t k = 0; k < K; ++k) {
            double acc = 0.0;
            for (int64_t r = 0; r < R; ++r) {
                const int64_t ih = oh * sh - ph + r * dh;
                if (ih < 0 || ih >= H) continue;
                for (int64_t s = 0; s < S; ++s) {
                    const int64_t iw = ow * sw - pw + s * dw;
                    if (iw < 0 || iw >= Wd) continue;
                    const uint16_t* xp = X + ((n * H + ih) * Wd + iw) * C;
                    const uint16_t* wp = Wt + ((k * R + r) * S + s) * C;
                    for (int64_t c = 0; c < C; ++c) acc += bf16_to_f64(xp[c]) * bf16_to_f64(wp[c]);
                }
            }
            if (out64) out64[(m - m0) * ldy + k] = acc;
            if (out32) out32[(m - m0) * ldy + k] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------------------------------
 * 8-bit floating point inputs ([GEMM] "Alcune regole pratiche": the matrix units reach their
 * peak with 16-bit formats "and shorter ones still, like FP8").  The two OCP 8-bit formats:
 *   E4M3 (fmt 0): 1 sign, 4 exponent bits (bias 7), 3 fraction bits; exponent field 0 is
 *                 subnormal (f * 2^-9); S.1111.111 is NaN; there is no infinity (max 448).
 *   E5M2 (fmt 1): 1 sign, 5 exponent bits (bias 15), 2 fraction bits; exponent field 0 is
 *                 subnormal (f * 2^-16); exponent 31 is infinity (f = 0) or NaN.
 * Every value is exact in binary64.
 * ---------------------------------------------------------------------------------------- */
static double f8_to_f64(uint8_t v, int fmt) {
    const int s = v >> 7;
    double r;
    if (fmt == 0) {
        const int e = (v >> 3) & 15, f = v & 7;
        if (e == 15 && f == 7) return NAN;
        r = e == 0 ? ldexp((double)f, -9) : ldexp((double)(8 + f), e - 10);
    } else {
        const int e = (v >> 2) & 31, f = v & 3;
        if (e == 31) return f ? NAN : (s ? -INFINITY : INFINITY);
        r = e == 0 ? ldexp((double)f, -16) : ldexp((double)(4 + f), e - 17);
    }
    return s ? -r : r;
}

void oracle_f8_to_f64_array(const uint8_t* in, double* out, int64_t n, int fmt) {
    for (int64_t i = 0; i < n; ++i) out[i] = f8_to_f64(in[i], fmt);
}

/* O3 for 8-bit inputs: C rows [m0, m1) of A·Bᵀ with A (M×K, lda) and B stored N×K (ldb), both
 * in format fmt; products exact in binary64, sums in ascending k in binary64, one rounding to
 * binary32.  Output layout as oracle_gemm_rows. */
void oracle_gemm_f8_rows(int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                         int fmt, int64_t m0, int64_t m1, double* out64, float* out32, int64_t ldo, int threads) {
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += f8_to_f64(A[m * lda + k], fmt) * f8_to_f64(B[n * ldb + k], fmt);
            if (out64) out64[(m - m0) * ldo + n] = acc;
            if (out32) out32[(m - m0) * ldo + n] = (float)acc;
        }
    }
}

/* binary32 array -> bfloat16 bits (round to nearest even), for bf16 outputs. */
void oracle_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
