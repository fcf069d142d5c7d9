/* A plain C99 caller of the library: builds against include/tbg.h alone and links libtbg.so,
 * and the HIP runtime (for device memory only), with no Python and no framework.  Modes:
 *   host                 descriptor encoding and argument checks, no device needed;
 *   gemm M N K IN OUT    device run: reads bf16 A (M×K) and B (K×N, row-major) from the files
 *                        IN.a and IN.b, allocates device memory with the HIP runtime, runs
 *                        tbg_gemm with fp32 output and writes C (M×N fp32) to OUT.
 * Prints "ok" and exits 0 on success; prints the failing check and exits 1 otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tbg.h"

#define CHECK(cond)                                                                          \
    do {                                                                                     \
        if (!(cond)) {                                                                       \
            fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #cond,            \
                    tbg_last_error());                                                       \
            return 1;                                                                        \
        }                                                                                    \
    } while (0)

static int host_checks(void) {
    /* The worked descriptor: a 256×256 bf16 matrix, a box of 64 columns × 128 rows, 128-byte
     * swizzle, zero fill; any 16-byte-aligned address (encoding reads no memory). */
    const void* base = (const void*)(uintptr_t)0x7F0000000000ull;
    uint64_t dims[2] = {256, 256}, strides[1] = {512};
    uint32_t box[2] = {64, 128}, estr[2] = {1, 1};
    tbg_tensor_desc d;
    CHECK(sizeof(tbg_tensor_desc) == 128);
    CHECK(tbg_encode_tiled(&d, TBG_BF16, 2, base, dims, strides, box, estr, TBG_SWIZZLE_128B, TBG_L2_NONE,
                           TBG_OOB_ZERO) == TBG_OK);
    CHECK(tbg_box_bytes(&d) == 16384);
    /* rank 6, a misaligned base, a stride off 16 bytes, an element stride of 9 */
    CHECK(tbg_encode_tiled(&d, TBG_BF16, 6, base, dims, strides, box, estr, TBG_SWIZZLE_NONE, TBG_L2_NONE,
                           TBG_OOB_ZERO) == TBG_ERR_UNSUPPORTED);
    CHECK(tbg_encode_tiled(&d, TBG_BF16, 2, (const char*)base + 8, dims, strides, box, estr, TBG_SWIZZLE_NONE,
                           TBG_L2_NONE, TBG_OOB_ZERO) == TBG_ERR_MISALIGNED);
    strides[0] = 520;
    CHECK(tbg_encode_tiled(&d, TBG_BF16, 2, base, dims, strides, box, estr, TBG_SWIZZLE_NONE, TBG_L2_NONE,
                           TBG_OOB_ZERO) == TBG_ERR_MISALIGNED);
    strides[0] = 512;
    estr[0] = 9;
    CHECK(tbg_encode_tiled(&d, TBG_BF16, 2, base, dims, strides, box, estr, TBG_SWIZZLE_NONE, TBG_L2_NONE,
                           TBG_OOB_ZERO) == TBG_ERR_OUT_OF_RANGE);
    /* GEMM argument checks come before any device access */
    CHECK(tbg_gemm(-1, 4, 4, base, 4, base, 4, TBG_B_KN, (void*)base, 4, TBG_F32, NULL, 0, NULL) ==
          TBG_ERR_INVALID_VALUE);
    CHECK(tbg_gemm(4, 4, 8, base, 4, base, 4, TBG_B_KN, (void*)base, 4, TBG_F32, NULL, 0, NULL) ==
          TBG_ERR_INVALID_VALUE); /* lda < K */
    CHECK(tbg_gemm(0, 4, 4, base, 4, base, 4, TBG_B_KN, (void*)base, 4, TBG_F32, NULL, 0, NULL) == TBG_OK);
    CHECK(strcmp(tbg_status_string(TBG_OK), "") != 0);
    return 0;
}

static void* read_file(const char* path, size_t n) {
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(n);
    if (p && fread(p, 1, n, f) != n) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

static int gemm_run(int64_t M, int64_t N, int64_t K, const char* in, const char* out) {
    char pa[4096], pb[4096];
    snprintf(pa, sizeof pa, "%s.a", in);
    snprintf(pb, sizeof pb, "%s.b", in);
    const size_t na = (size_t)(M * K * 2), nb = (size_t)(K * N * 2), nc = (size_t)(M * N * 4);
    void* ha = read_file(pa, na);
    void* hb = read_file(pb, nb);
    void* hc = malloc(nc);
    CHECK(ha && hb && hc);
    void *da = NULL, *db = NULL, *dc = NULL;
    CHECK(hipMalloc(&da, na) == hipSuccess && hipMalloc(&db, nb) == hipSuccess && hipMalloc(&dc, nc) == hipSuccess);
    CHECK(hipMemcpy(da, ha, na, hipMemcpyHostToDevice) == hipSuccess &&
          hipMemcpy(db, hb, nb, hipMemcpyHostToDevice) == hipSuccess);
    /* dense row-major bf16 rows whose pitch is a multiple of 16 bytes need no workspace */
    CHECK(tbg_gemm_workspace_bytes(M, N, K, K, N, TBG_B_KN) == 0);
    CHECK(tbg_gemm(M, N, K, da, K, db, N, TBG_B_KN, dc, N, TBG_F32, NULL, 0, NULL) == TBG_OK);
    CHECK(hipDeviceSynchronize() == hipSuccess);
    CHECK(hipMemcpy(hc, dc, nc, hipMemcpyDeviceToHost) == hipSuccess);
    FILE* f = fopen(out, "wb");
    CHECK(f && fwrite(hc, 1, nc, f) == nc);
    fclose(f);
    (void)hipFree(da);
    (void)hipFree(db);
    (void)hipFree(dc);
    free(ha);
    free(hb);
    free(hc);
    return 0;
}

int main(int argc, char** argv) {
    if (argc >= 2 && strcmp(argv[1], "host") == 0) {
        if (host_checks()) return 1;
    } else if (argc == 7 && strcmp(argv[1], "gemm") == 0) {
        if (gemm_run(atoll(argv[2]), atoll(argv[3]), atoll(argv[4]), argv[5], argv[6])) return 1;
    } else {
        fprintf(stderr, "usage: %s host | gemm M N K IN OUT\n", argv[0]);
        return 2;
    }
    printf("ok\n");
    return 0;
}
