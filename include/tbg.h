/*
 * tbg.h — C ABI of the MI355X (gfx950) tiled bf16 GEMM library with descriptor-driven tile copies.
 *
 * The library computes C = A·B with bf16 inputs and fp32 accumulation, feeding its matrix cores
 * from tiles that are copied global memory -> LDS as the descriptor pages describe them: a
 * host-built tensor descriptor (rank <= 5, byte strides, a box, element strides, an XOR swizzle
 * of the destination, out-of-bounds fill) plus coordinates per copy.
 *
 * Sources, cited by page title and section:
 *   [TMA]  "2 · Le Tensor Memory Accelerator" (mkdocs.reaper.mx, cuda-moderne/02-tma)
 *   [MAP]  "H100 · cuTensorMap（TMA 描述符）" (runguoli.com, h100-cuda-programming/l4)
 *   [PIPE] "1 · Asynchronisme et mbarrier" (mkdocs.reaper.mx, cuda-moderne/01-asynchronisme...)
 *   [GEMM] "GEMM: la moltiplicazione di matrici sull'hardware" (book.paithon.it)
 *
 * Conventions for every call:
 *   - No HIP or framework types cross this boundary.  `stream` is a hipStream_t passed as
 *     void* (NULL = the legacy default stream).  Device pointers are plain addresses of device
 *     memory that the caller owns; the library never allocates, frees or retains memory.
 *   - All argument checks run synchronously on the host and return a status; nothing is
 *     enqueued when a check fails.  Device work is enqueued on `stream` and the call returns
 *     without waiting; a fault inside a kernel surfaces at the caller's next synchronisation.
 *   - No exception crosses the ABI.  tbg_last_error() gives a readable detail of the last
 *     failure on the calling thread.
 *   - Every array of per-dimension values is ordered innermost dimension first ([MAP] §8.2).
 *   - With the environment variable TBG_LOG set to a value other than "" or "0", every GEMM and
 *     convolution call prints the kernel configuration it launches (pipeline, tile, stages, which
 *     operands were repacked) as one line on stderr.
 */
#ifndef TBG_H_
#define TBG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TBG_OK = 0,
    TBG_ERR_INVALID_VALUE = 1, /* a null pointer, a negative size, inconsistent arguments      */
    TBG_ERR_MISALIGNED = 2,    /* base or stride not a multiple of 16 bytes ([TMA] §2.3)      */
    TBG_ERR_UNSUPPORTED = 3,   /* rank outside 1..5, or a size this library does not take     */
    TBG_ERR_OUT_OF_RANGE = 4,  /* a dimension, box, element stride or workspace out of range  */
    TBG_ERR_NO_DEVICE = 5,     /* no usable gfx950 device                                     */
    TBG_ERR_HIP = 6            /* the HIP runtime refused a launch                             */
} tbg_status;

/* Element type of a copy ([MAP] §7).  A copy moves bits: no conversion, no flush to zero.
 * TBG_F8_E4M3 and TBG_F8_E5M2 are the two OCP 8-bit floating-point formats (E4M3: 4 exponent
 * bits, bias 7, no infinity, NaN S.1111.111; E5M2: 5 exponent bits, bias 15, IEEE-style
 * infinities and NaNs). */
typedef enum {
    TBG_U8 = 0, TBG_U16 = 1, TBG_U32 = 2, TBG_F16 = 3, TBG_BF16 = 4, TBG_F32 = 5,
    TBG_F8_E4M3 = 6, TBG_F8_E5M2 = 7
} tbg_dtype;

/* Destination swizzle ([MAP] §11.3): for a byte offset a inside the box image,
 *   a' = a ^ ((a & Y_mask) >> 3),  Y_mask = 0x080 (32B), 0x180 (64B), 0x380 (128B),
 * i.e. 32B: a[4] ^= a[7]; 64B: a[5:4] ^= a[8:7]; 128B: a[6:4] ^= a[9:7].  16-byte units move
 * whole ([MAP] §11.4).
 * TBG_SWIZZLE_128B_2ROW is this library's extension of the same XOR form for gfx950's LDS,
 * which serves 16 lanes of a 16-byte read per cycle from 64 four-byte banks (256 bytes):
 *   a' = a ^ ((a & 0x700) >> 4),  i.e. a[6:4] ^= a[10:8],
 * so sixteen consecutive 128-byte rows read at one logical 16-byte column hit 16 distinct
 * 16-byte bank groups.  It permutes 16-byte units inside each aligned 128-byte block.
 * TBG_SWIZZLE_128B_TR is the library's layout for a 128-byte-row box read back with gfx950's
 * transposing 8-byte LDS read (ds_read_b64_tr_b16, which the GEMM uses for B stored K×N): the
 * 16-byte unit index of 128-byte row r is XORed with 4·r[3] + 2·r[1] + r[2], i.e.
 *   a[4] ^= a[9],  a[5] ^= a[8],  a[6] ^= a[10]
 * (not of the single-shift form above).  That read takes 32 bytes from each of the rows
 * {r0 + 8t + e : t < 2, e < 4} per 32 lanes, served from one 256-byte bank window; this XOR puts
 * the eight 32-byte pieces on eight distinct 32-byte bank groups, which neither 128B nor
 * 128B_2ROW does.  It permutes 16-byte units inside each aligned 128-byte block and repeats every
 * 16 rows (2048 bytes). */
typedef enum {
    TBG_SWIZZLE_NONE = 0,
    TBG_SWIZZLE_32B = 1,
    TBG_SWIZZLE_64B = 2,
    TBG_SWIZZLE_128B = 3,
    TBG_SWIZZLE_128B_2ROW = 4,
    TBG_SWIZZLE_128B_TR = 5
} tbg_swizzle;

/* Out-of-bounds fill ([MAP] §14; [TMA] §2.5): box elements outside the tensor are written to
 * the destination as zero bytes (TBG_OOB_ZERO, the pages' FILL_NONE) or as the element type's
 * canonical quiet NaN (TBG_OOB_NAN: bf16 0x7FC0, f16 0x7E00, f32 0x7FC00000, E4M3 0x7F, E5M2
 * 0x7E; floating types only).  The source is never touched outside the tensor. */
typedef enum { TBG_OOB_ZERO = 0, TBG_OOB_NAN = 1 } tbg_oob_fill;

/* L2 promotion hint ([MAP] §13).  Accepted and recorded; it does not change any result. */
typedef enum { TBG_L2_NONE = 0, TBG_L2_64B = 1, TBG_L2_128B = 2, TBG_L2_256B = 3 } tbg_l2_hint;

/* Layout of the GEMM's B operand: TBG_B_KN = row-major K×N (N contiguous);
 * TBG_B_NK = N×K with K contiguous (B transposed, as weights are usually stored). */
typedef enum { TBG_B_KN = 0, TBG_B_NK = 1 } tbg_b_layout;

/* A host-built tensor descriptor: 128 bytes, plain data, copied by value ([TMA] §2.2; [MAP]
 * §3, §5).  It records a raw device address and does not keep that memory alive. */
typedef struct {
    uint64_t opaque[16];
} tbg_tensor_desc;

/* Encode a tiled-copy descriptor ([TMA] §2.3; [MAP] §6, §8, §9).
 *   out             caller storage for the descriptor.
 *   dtype           element type (sets the element size).
 *   rank            number of dimensions, 1..5 ([TMA] §2.2).
 *   global_address  device address of element (0,...,0); must be a multiple of 16 bytes.
 *   global_dim      [rank] elements per dimension, innermost first; each in 1..2^32 ([MAP] §8.2).
 *   global_strides  [rank-1] byte distance between consecutive indices of dimensions 1..rank-1
 *                   (dimension 0's stride is the element size, [MAP] §8.3); each a multiple of 16
 *                   and below 2^40.  May be NULL when rank == 1.
 *   box_dim         [rank] traversal box per copy, in elements, each 1..256 ([MAP] §9.2).
 *   element_strides [rank] step between copied elements, each 1..8 ([MAP] §9.1); a box copies
 *                   n[i] = ceil(box_dim[i] / element_strides[i]) elements per dimension.
 *   swizzle, l2, oob as documented above.
 * The image of one copy is dense, innermost first, elsize * prod(n[i]) bytes, at most 64 KiB.
 * With a swizzle, box_dim[0] * elsize must not exceed 128 bytes for the 128-byte modes (32/64
 * for the 32B/64B modes, [MAP] §9.2; [TMA] §2.3) and the image size must be a multiple of that
 * span so the permutation stays inside the image.
 * Returns TBG_OK, or UNSUPPORTED (rank), MISALIGNED (base/strides), OUT_OF_RANGE (dims, box,
 * element strides, image size), INVALID_VALUE (null pointers, enum values, swizzle width, NaN
 * fill of an integer type). */
tbg_status tbg_encode_tiled(tbg_tensor_desc* out, tbg_dtype dtype, uint32_t rank, const void* global_address,
                            const uint64_t* global_dim, const uint64_t* global_strides, const uint32_t* box_dim,
                            const uint32_t* element_strides, tbg_swizzle swizzle, tbg_l2_hint l2,
                            tbg_oob_fill oob);

/* Interleaved layouts ([MAP] §12): tensors stored NC/xHWCx, i.e. channels cut into slices of x
 * channels that are 16 or 32 bytes wide, each slice stored contiguously per position
 * (memory order N, C/x, H, W, x).  The copy that reads them back is a tiled copy; interleave adds
 * the page's rules (§12.3, §12.4): rank >= 3; base and every stride a multiple of the slice
 * width; 32-byte slices require the 32B swizzle.  Reading (the page's table of the two modes is
 * lost in the text): dimension 0 is one channel slice, global_dim[0] * elsize equals the width,
 * and a box takes whole slices (box_dim[0] = global_dim[0], element_strides[0] = 1); channel
 * counts that are not a multiple of x carry the zero padding of the last slice in memory, as the
 * page asks of the tensor's producer. */
typedef enum { TBG_INTERLEAVE_NONE = 0, TBG_INTERLEAVE_16B = 1, TBG_INTERLEAVE_32B = 2 } tbg_interleave;

/* tbg_encode_tiled with an interleave mode (TBG_INTERLEAVE_NONE is tbg_encode_tiled itself).
 * Returns what tbg_encode_tiled returns, plus UNSUPPORTED (rank < 3), INVALID_VALUE (dimension 0
 * not one slice, a box that splits a slice, 32B interleave without the 32B swizzle, unknown
 * interleave) and MISALIGNED (base or strides not multiples of the slice width).  The descriptor
 * is used with tbg_tiled_copy / tbg_tiled_store like any tiled descriptor. */
tbg_status tbg_encode_tiled_interleaved(tbg_tensor_desc* out, tbg_dtype dtype, uint32_t rank,
                                        const void* global_address, const uint64_t* global_dim,
                                        const uint64_t* global_strides, const uint32_t* box_dim,
                                        const uint32_t* element_strides, tbg_interleave interleave,
                                        tbg_swizzle swizzle, tbg_l2_hint l2, tbg_oob_fill oob);

/* Bytes of one copy's image for an encoded descriptor: for a tiled descriptor elsize times the
 * product over dimensions of n[i] = ceil(box_dim[i] / element_strides[i]), the elements one copy
 * lands ("H100 · cuTensorMap" §9.1-§9.2: the box is the traversal extent and every
 * element_strides[i]-th element along it is copied); for an im2col descriptor elsize * channels *
 * pixels.  0 if `d` is not a valid descriptor. */
size_t tbg_box_bytes(const tbg_tensor_desc* d);

/* Copy one box ([TMA] §2.2, §2.4): the element at box position j (innermost first) comes from
 * tensor coordinates coords[i] + j[i] * element_strides[i] and lands at image byte offset
 * swizzle(elsize * (j[0] + n[0]*(j[1] + n[1]*(...)))); positions outside the tensor get the
 * fill.  The box passes through LDS on its way to `dst_image`.
 *   coords     [rank] signed int32 coordinates in host memory (negative values allowed).
 *   dst_image  device memory of tbg_box_bytes(d) bytes, 16-byte aligned.
 * Returns INVALID_VALUE for null arguments or a bad descriptor, MISALIGNED for dst_image,
 * NO_DEVICE / HIP for runtime failures. */
tbg_status tbg_tiled_copy(const tbg_tensor_desc* d, const int32_t* coords, void* dst_image, void* stream);

/* Copy n boxes of the same descriptor: box b uses coords_dev[b*rank .. b*rank+rank-1] (device
 * memory, int32) and writes its image at dst_images + b * tbg_box_bytes(d).  n == 0 is a no-op.
 * dst_images must be 16-byte aligned. */
tbg_status tbg_tiled_copy_many(const tbg_tensor_desc* d, const int32_t* coords_dev, uint32_t n, void* dst_images,
                               void* stream);

/* Store one box: the other direction of tbg_tiled_copy ([TMA] §2.5: the copy engine also moves
 * shared memory to global memory, with the same descriptors, as a GEMM epilogue does).  Box
 * position j takes the element at image byte offset swizzle(elsize * lin(j)), where a load of
 * the same box puts it, and writes it at tensor coordinates coords[i] + j[i] * element_strides[i].
 * Positions outside the tensor are not written (the fill mode applies to loads only; this
 * reading is the library's, the pages do not describe the store's edges).  The image passes
 * through LDS on its way to the tensor.
 *   coords     [rank] signed int32 coordinates in host memory (negative values allowed).
 *   src_image  device memory of tbg_box_bytes(d) bytes, 16-byte aligned; not modified.
 * Returns INVALID_VALUE for null arguments or a bad descriptor, MISALIGNED for src_image,
 * NO_DEVICE / HIP for runtime failures. */
tbg_status tbg_tiled_store(const tbg_tensor_desc* d, const int32_t* coords, const void* src_image, void* stream);

/* Store n boxes of the same descriptor: box b uses coords_dev[b*rank .. b*rank+rank-1] (device
 * memory, int32) and reads its image at src_images + b * tbg_box_bytes(d).  n == 0 is a no-op.
 * Boxes that overlap in the tensor are written in an unspecified order. */
tbg_status tbg_tiled_store_many(const tbg_tensor_desc* d, const int32_t* coords_dev, uint32_t n,
                                const void* src_images, void* stream);

/* Workspace bytes tbg_gemm needs for these sizes, assuming A and B start on 16-byte
 * boundaries.  It is non-zero only when an operand has to be repacked first ([GEMM] section
 * "I tensor core", packing of a block into a contiguous area; "In pratica", 16-byte alignment of
 * the leading dimension): A when lda % 8 != 0 or K % 8 != 0; B (N×K) likewise with ldb; B (K×N)
 * when ldb % 8 != 0. */
size_t tbg_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, tbg_b_layout bl);

/* The exact workspace bytes a product of these sizes and operands needs, for every input type
 * (tbg_gemm, tbg_gemm_ex, tbg_gemm_configured, tbg_gemm_typed; the same repack rules, [GEMM]
 * "In pratica": 16-byte leading dimensions, and "I tensor core": packing a block into a
 * contiguous area).  Unlike tbg_gemm_workspace_bytes it looks at the operands' base addresses
 * (A and B are only compared against 16-byte boundaries, never dereferenced) and at the type:
 *   TBG_BF16, TBG_F16  A is repacked when lda % 8, K % 8 or A % 16 is non-zero; B (N×K) likewise
 *                      with ldb; B (K×N) when ldb % 8 or B % 16 is non-zero;
 *   TBG_F8_E4M3/E5M2   A (B, stored N×K) is repacked when lda (ldb) % 16, K % 16 or its base
 *                      % 16 is non-zero, with K rounded up to 16.
 * Each repack takes its rows at the rounded pitch, 256-byte rounded.  Returns 0 when no repack
 * is needed, for non-positive sizes or leading dimensions, and for any other ab_dtype. */
size_t tbg_gemm_workspace_query(int64_t M, int64_t N, int64_t K, tbg_dtype ab_dtype, const void* A, int64_t lda,
                                const void* B, int64_t ldb, tbg_b_layout bl);

/* C = A·B ([GEMM] "Il conto": C_ij = Σ_k A_ik B_kj, 2MNK flops), bf16 inputs, fp32 accumulation
 * in the matrix cores ([GEMM] tensor-core section), fp32 or bf16 (round to nearest even) output.
 *   A          bf16, row-major M×K, lda >= K (elements).
 *   B          bf16, TBG_B_KN: row-major K×N, ldb >= N;  TBG_B_NK: N×K, ldb >= K.
 *   C          TBG_F32 or TBG_BF16, row-major M×N, ldc >= N.  Only C[m][n] with m < M, n < N is
 *              written; C must not overlap A, B or the workspace.
 *   workspace  device memory of at least tbg_gemm_workspace_query(...) bytes (the exact need,
 *              misaligned bases included; tbg_gemm_workspace_bytes gives it for 16-byte aligned
 *              operands), 256-byte aligned; may be NULL when 0.  With at least twice the need,
 *              successive calls (of any of the products) put their repacked operands alternately
 *              in its two halves: a repack that overwrites the copy the previous product has just
 *              read is much slower on MI355X (≈8.5 µs against ≈4.7 µs for 3001×2049×777).
 * The operand boxes the kernels copy are encoded with tbg_encode_tiled (A {K, M}, B {K, N} or
 * {N, K}, with this library's LDS layouts) and handed to the kernels, which take base, row pitch
 * and extents from them.
 * M == 0 or N == 0 is a no-op; K == 0 writes zeros (the empty sum).  Leading dimensions are
 * limited to 2^22 - 1 elements.
 * Returns INVALID_VALUE (negative sizes, ld below its minimum, null pointers, bad enum),
 * UNSUPPORTED (leading dimension too large), OUT_OF_RANGE (workspace too small; the detail
 * names the size needed), NO_DEVICE / HIP for runtime failures. */
tbg_status tbg_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                    tbg_b_layout bl, void* C, int64_t ldc, tbg_dtype c_dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/* tbg_gemm for callers that cannot allocate device memory or pass a workspace: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.  The same
 * product, kernels and results as tbg_gemm; operands that need a repack (see
 * tbg_gemm_workspace_query) are repacked into a scratch array that the library holds in device
 * memory, one per GPU it runs on, for the life of the process: tbg_gemm_noalloc_scratch_bytes()
 * bytes (32 MiB).  The call allocates nothing (no hipMalloc, no hipFree).
 * The scratch array is shared by every call on a GPU and keeps the last call's contents (each
 * repack writes every byte it reads back, zero padding included): calls that overlap on one GPU
 * (on different streams, or from different threads) race on it and must be serialised by the
 * caller; calls on one stream are ordered.
 * Returns what tbg_gemm returns; OUT_OF_RANGE when the repack needs more than the scratch array
 * holds (the detail names both sizes), HIP when the array's device address cannot be found. */
tbg_status tbg_gemm_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                            tbg_b_layout bl, void* C, int64_t ldc, tbg_dtype c_dtype, void* stream);

/* Size in bytes of the scratch array behind tbg_gemm_noalloc. */
size_t tbg_gemm_noalloc_scratch_bytes(void);

/* C <- alpha·A·B + beta·C, the general form of the BLAS product that [GEMM]'s tensor-core section
 * gives for the matrix units.  Arguments, layouts, checks and workspace as tbg_gemm, plus:
 *   alpha, beta  binary32 scalars.  The product's fp32 sum S is combined as alpha·S + beta·C_old
 *                in binary32 and rounded once to C's type.
 *   beta == 0    C is not read: whatever it holds (NaN included) does not reach the result.
 *   alpha == 0   the product is skipped and A and B are not read (they may be NULL); C becomes
 *                beta·C.
 * tbg_gemm is tbg_gemm_ex with alpha = 1 and beta = 0. */
tbg_status tbg_gemm_ex(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                       int64_t ldb, tbg_b_layout bl, float beta, void* C, int64_t ldc, tbg_dtype c_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Operand-copy pipeline of the GEMM ([PIPE] §1.3-§1.5: an S-stage ring in on-chip memory whose
 * stages are filled by asynchronous copies while earlier stages are multiplied).
 *   TBG_PIPE_RING      every compute wave copies its share of each stage; one workgroup barrier
 *                      per K tile both publishes the next stage and frees the oldest one.
 *   TBG_PIPE_PRODUCER  dedicated producer waves copy every stage ([TMA] §2.1: the copy is issued
 *                      by one thread); the compute waves issue no copies.  Each stage has a full
 *                      and an empty counter in LDS ([PIPE] §1.5: the two barriers per stage),
 *                      polled with short sleeps.
 *   TBG_PIPE_AUTO      the library's choice, made with the tile from measured throughput: the
 *                      ring for 256x256, 128x128 and 64x64 tiles, producer waves for 256x128 and
 *                      128x256 tiles. */
typedef enum { TBG_PIPE_AUTO = 0, TBG_PIPE_RING = 1, TBG_PIPE_PRODUCER = 2 } tbg_pipeline;

/* Kernel configuration of tbg_gemm_configured.  Zero fields are left to the library.
 *   tile_m, tile_n  workgroup tile of C ([GEMM] "Tiling"): both 0 (chosen from the shape), or
 *                   one of 256x256, 256x128, 128x256, 128x128, 64x64.
 *   stages          LDS stages of the ring: 0 (default: 2; 3 for 64x64 tiles and for the
 *                   producer pipeline's 128x128 tiles) or >= 2.  Each stage holds one tile_m x 64 block of A and
 *                   one 64 x tile_n block of B in bf16, so the count is bounded by the 160 KiB
 *                   of LDS.
 *   pipeline        a tbg_pipeline value.
 * Built configurations (tile / stages):
 *   ring:      256x256/2; 256x128 and 128x256/2-3; 128x128/2-5; 64x64/2-6
 *   producer:  256x128 and 128x256/2-3; 128x128/2-4; 64x64/2-6
 * (the 256x256 tile needs every register of its four compute waves and leaves none for
 * producer waves). */
typedef struct {
    int32_t tile_m, tile_n;
    int32_t stages;
    int32_t pipeline;
} tbg_gemm_config;

/* tbg_gemm_ex with an explicit kernel configuration; same arguments, layouts, results and checks,
 * plus cfg (host memory, not retained).  Every configuration accumulates each C element over K in
 * the same ascending order of 32-wide steps, so all configurations give bit-identical results.
 * Returns INVALID_VALUE for a NULL cfg or a malformed field (unknown pipeline, only one tile
 * size set, stages == 1 or negative) and UNSUPPORTED for a configuration that is not built (the
 * detail lists the built ones); these checks come before any device check. */
tbg_status tbg_gemm_configured(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                               const void* B, int64_t ldb, tbg_b_layout bl, float beta, void* C, int64_t ldc,
                               tbg_dtype c_dtype, const tbg_gemm_config* cfg, void* workspace,
                               size_t workspace_bytes, void* stream);

/* C <- alpha·A·B + beta·C with the input element type given ([GEMM] "Alcune regole pratiche": the
 * matrix units reach their peak with 16-bit formats and shorter ones still, like FP8).  A and B
 * are both of type ab_dtype:
 *   TBG_BF16, TBG_F16   as tbg_gemm_configured.  fp16 inputs are built for the configurations
 *                       the automatic choice uses (ring 256x256, 256x128, 128x256, 128x128
 *                       with 2 stages, 64x64 with 2 and 3; producer 256x128 and 128x256 with 2
 *                       stages, 128x128 and 64x64 with 3); others are UNSUPPORTED.
 *   TBG_F8_E4M3, TBG_F8_E5M2
 *                       8-bit inputs on the 16x16x128 matrix instruction.  B must be stored N×K
 *                       (TBG_B_NK; TBG_B_KN is UNSUPPORTED); lda, ldb in elements (bytes); rows
 *                       whose pitch or K is not a multiple of 16 bytes, or operands off a 16-byte
 *                       boundary, are repacked into the workspace (tbg_gemm_workspace_query
 *                       gives the exact size; the OUT_OF_RANGE detail names it too).
 *                       Configurations: ring, 2 stages, tiles 256x256, 128x128, 64x64.
 * Every product of two inputs is exact in fp32; accumulation is fp32, output fp32 or bf16.  cfg
 * may be NULL (the library's choice).  Other arguments, layouts and checks as tbg_gemm_ex; any
 * other ab_dtype is INVALID_VALUE.  tbg_gemm_configured is this call with ab_dtype = TBG_BF16. */
tbg_status tbg_gemm_typed(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                          int64_t ldb, tbg_b_layout bl, tbg_dtype ab_dtype, float beta, void* C, int64_t ldc,
                          tbg_dtype c_dtype, const tbg_gemm_config* cfg, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Encode an im2col descriptor ([TMA] section "im2col": a copy mode dedicated to convolution that
 * performs the im2col transform during the copy, so that a convolution becomes a GEMM whose
 * im2col matrix is never stored).  The page gives no more than that; this library's reading:
 *   - the tensor X is NHWC: global_dim = {C, W, H, N} (innermost first), global_strides = byte
 *     strides of W, H and N (each a multiple of 16; the channel stride is the element size);
 *   - pad_lo, pad_hi, conv_stride, dilation, filter: {along W, along H}; the convolution has
 *     OW = floor((W + pad_lo[0] + pad_hi[0] - dilation[0]*(filter[0]-1) - 1) / conv_stride[0]) + 1
 *     output columns, OH likewise; the window must fit (OW, OH >= 1);
 *   - row m of the im2col matrix is output pixel m = (n*OH + oh)*OW + ow, column (r, s, c) is
 *     filter tap r (along H), s (along W) and channel c; its element is
 *     X[n, oh*sh - ph + r*dh, ow*sw - pw + s*dw, c], or the fill where that position is outside
 *     the tensor (the convolution's padding), where m >= N*OH*OW or m < 0, and where c is
 *     outside 0..C-1;
 *   - a copy takes `pixels` consecutive rows (1..256) and `channels` consecutive channels
 *     (1..256) at one tap; its image is dense, channel fastest (element (i, j) at byte
 *     elsize*(j + channels*i)), through `swizzle` like a tiled copy (channels*elsize must fit the
 *     swizzle span and the image must be a whole number of spans), at most 64 KiB.
 * Limits: each dimension below 2^31, strides below 2^40, filter, stride and dilation 1..256,
 * padding 0..65535, fewer than 2^31 output pixels.
 * Returns MISALIGNED (base/strides), OUT_OF_RANGE (dims, strides, box, geometry), INVALID_VALUE
 * (null pointers, enum values, a window that does not fit, swizzle width, NaN fill of an integer
 * type), UNSUPPORTED (too many output pixels). */
tbg_status tbg_encode_im2col(tbg_tensor_desc* out, tbg_dtype dtype, const void* global_address,
                             const uint64_t* global_dim, const uint64_t* global_strides, const int32_t* pad_lo,
                             const int32_t* pad_hi, const int32_t* conv_stride, const int32_t* dilation,
                             const int32_t* filter, uint32_t channels, uint32_t pixels, tbg_swizzle swizzle,
                             tbg_l2_hint l2, tbg_oob_fill oob);

/* Copy one im2col block: coords = {c0, m0, s, r} in host memory (first channel, first output
 * pixel, filter tap along W, filter tap along H; signed).  dst_image: tbg_box_bytes(d) bytes of
 * device memory, 16-byte aligned.  The block passes through LDS.  Errors as tbg_tiled_copy
 * (a tiled descriptor here is INVALID_VALUE). */
tbg_status tbg_im2col_copy(const tbg_tensor_desc* d, const int32_t* coords, void* dst_image, void* stream);

/* n im2col blocks of one descriptor: block b uses coords_dev[4b .. 4b+3] (device memory, int32)
 * and writes its image at dst_images + b * tbg_box_bytes(d).  n == 0 is a no-op. */
tbg_status tbg_im2col_copy_many(const tbg_tensor_desc* d, const int32_t* coords_dev, uint32_t n, void* dst_images,
                                void* stream);

/* Shape of a 2-D convolution (cross-correlation, as deep-learning frameworks define it):
 *   Y[n, oh, ow, k] = sum over r < R, s < S, c < C of
 *                     X[n, oh*stride_h - pad_h + r*dil_h, ow*stride_w - pad_w + s*dil_w, c] * W[k, r, s, c],
 * with X read as zero outside its H x W extent.  OH = floor((h + pad_h + pad_h_end - dil_h*(r-1)
 * - 1) / stride_h) + 1, OW likewise.  X is NHWC, W is KRSC (both bf16, dense), Y is row-major
 * (N*OH*OW) x K (NHWK) with leading dimension ldy. */
typedef struct {
    int64_t n, h, w, c;            /* input batch, height, width, channels */
    int64_t k;                     /* output channels */
    int32_t r, s;                  /* filter height and width */
    int32_t pad_h, pad_w;          /* zero padding before the first row and column */
    int32_t pad_h_end, pad_w_end;  /* zero padding after the last row and column */
    int32_t stride_h, stride_w;
    int32_t dil_h, dil_w;
} tbg_conv2d_shape;

/* Output extents OH, OW of a shape (either pointer may be NULL).  Returns INVALID_VALUE for a
 * size, stride or dilation below 1, negative padding or a window that does not fit;
 * UNSUPPORTED beyond the limits of tbg_conv2d_fwd. */
tbg_status tbg_conv2d_out_dims(const tbg_conv2d_shape* shape, int64_t* oh, int64_t* ow);

/* Workspace bytes tbg_conv2d_fwd needs: 0 when c is a multiple of 8 (and x, w are 16-byte
 * aligned, which this function assumes); else room to repack X and W with the channel pitch
 * rounded up to 8 (zero channels added), 256-byte aligned.  0 for an invalid shape. */
size_t tbg_conv2d_workspace_bytes(const tbg_conv2d_shape* shape);

/* The exact workspace bytes tbg_conv2d_fwd needs for this shape and these operands: as
 * tbg_conv2d_workspace_bytes, and also when x or w is not 16-byte aligned (only compared against
 * 16-byte boundaries, never dereferenced); 0 when nothing is repacked or the shape is invalid. */
size_t tbg_conv2d_workspace_query(const tbg_conv2d_shape* shape, const void* x, const void* w);

/* Y <- alpha * conv2d(X, W) + beta * Y as an implicit GEMM ([TMA] section "im2col": the im2col
 * matrix of X is formed tile by tile by the operand copies and never stored; [GEMM] the product).
 * The GEMM is (N*OH*OW) x K with reduction R*S*C over filter taps and channels; bf16 inputs,
 * fp32 accumulation, fp32 or bf16 (RNE) output; alpha/beta as tbg_gemm_ex (beta == 0 does not
 * read Y; alpha == 0 reads neither X nor W).
 *   x, w       device memory, NHWC and KRSC bf16; any c (c % 8 != 0, or an operand not 16-byte
 *              aligned, needs the workspace of tbg_conv2d_workspace_bytes, plus that much again
 *              for a misaligned operand; with twice the need the repack alternates between the
 *              workspace's halves, as for tbg_gemm).
 *   y          fp32 or bf16 device memory, (N*OH*OW) rows of ldy >= k elements; only the first k
 *              of each row are written.
 *   cfg        NULL (the library's choice) or a tbg_gemm_config with pipeline AUTO or RING and
 *              one of:
 *                tile 0x0, 256x256, 256x128, 128x128 or 64x64, stages 0 or 2: the im2col
 *                kernels, whose sums run tap by tap with 64 channels inside; these tiles give
 *                bit-identical results;
 *                tile 448x128, stages 0 or 4: the halo kernel (stride 1 and r*s >= 2 only; c a
 *                multiple of 32 and x, w 16-byte aligned, so nothing is repacked; OW <= 448; an
 *                input window of at most 1008 pixels that four 1 KiB copies per wave and tap
 *                bring in time), which copies each input window into LDS once per
 *                32-channel block for all taps.  Its sums run block by block, tap by tap inside
 *                a block, so its results may differ from the im2col tiles' in rounding (both are
 *                fp32 sums of the same exact products; small-integer inputs give equal bits);
 *              anything else is UNSUPPORTED.  With cfg NULL or tile 0x0 the library takes the
 *              halo kernel where it applies, its tiles use at least 3/4 of their 448 rows and
 *              there are at least half as many tiles as compute units; else an im2col tile by
 *              the GEMM's cost model.
 * Limits: h, w below 2^16; N*OH*OW and k below 2^31; X (with its channel pitch rounded up to 8)
 * below 2 GiB; r*s*c below 2^22; filter, stride, dilation up to 256; padding up to 65535.
 * Returns INVALID_VALUE (bad shape, ldy < k, null pointers, y type), UNSUPPORTED (limits),
 * OUT_OF_RANGE (workspace too small), MISALIGNED (workspace), NO_DEVICE / HIP. */
tbg_status tbg_conv2d_fwd(const tbg_conv2d_shape* shape, float alpha, const void* x, const void* w, float beta,
                          void* y, int64_t ldy, tbg_dtype y_dtype, const tbg_gemm_config* cfg, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* tbg_status_string(tbg_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char* tbg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TBG_H_ */
