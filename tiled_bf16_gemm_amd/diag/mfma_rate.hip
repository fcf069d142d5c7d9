// Measurement aid for the benchmark, not part of the library's ABI: the rate at which this chip
// sustains matrix products when nothing else runs, the ceiling a GEMM kernel can reach at the
// clock the power limit allows.  Each wave issues one product instruction back to back on
// register-resident operand fragments filled from a buffer of random values (the matrix units'
// energy depends on operand bits), accumulators in AGPRs, never reusing an accumulator within 64
// products; one workgroup of four waves per CU (the full register file, as the 256x256 GEMM
// tile), `nwg` workgroups.  KIND 0: v_mfma_f32_16x16x32_bf16 (16 bytes of operand per lane),
// KIND 1: v_mfma_f32_16x16x128_f8f6f4 with E4M3 operands (32 bytes per lane).  Each workgroup
// records its shader-clock and 100 MHz real-time counter deltas, from which the caller derives the
// clock the products ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "gemm_ring.hpp"

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ void __launch_bounds__(256, 1) mfma_rate_kernel(const i32x4_t* src, float* out, int iters, uint64_t* clk) {
  const int t = threadIdx.x;
  // 16 operand fragments of 16 bytes per lane (KIND 0) or 8 of 32 bytes (KIND 1), 256 bytes per lane
  i32x4_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = src[((uint64_t)blockIdx.x * 16 + i) * 256 + t];
  f32x4_t acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime(), m0 = __builtin_amdgcn_s_memtime();
  // The fragment grid is walked in serpentine order, as the GEMM's k-step walks it: consecutive
  // products share one operand register (the order of least operand toggling, so of least energy).
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (KIND == 0) {
        const int x = ((i >> 3) & 1) ? 7 - (i & 7) : (i & 7);
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i]) : "v"(v[x]), "v"(v[8 + (i >> 3)]));
      } else {
        const int x = ((i >> 2) & 1) ? 3 - (i & 3) : (i & 3);
        const i32x8_t a = __builtin_shufflevector(v[2 * x], v[2 * x + 1], 0, 1, 2, 3, 4, 5, 6, 7);
        const i32x8_t b = __builtin_shufflevector(v[8 + 2 * ((i >> 2) & 3)], v[9 + 2 * ((i >> 2) & 3)], 0, 1, 2, 3, 4,
                                                  5, 6, 7);
        asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc[i]) : "v"(a), "v"(b));
      }
    }
  }
  // wait states before the accumulators are read (the products are inline assembly)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime(), m1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    f32x4_t a = acc[i];
    asm volatile("" : "+v"(a));
    s += a[0] + a[1] + a[2] + a[3];
  }
  out[(uint64_t)blockIdx.x * 256 + t] = s;
  if (t == 0) {
    clk[2 * (uint64_t)blockIdx.x] = r1 - r0;
    clk[2 * (uint64_t)blockIdx.x + 1] = m1 - m0;
  }
}

// src: nwg * 16 * 256 16-byte values (nwg * 64 KiB of random bf16 for kind 0, random E4M3 bytes
// for kind 1); out: nwg * 256 floats; clk: 2 * nwg uint64 (real-time ticks at 100 MHz,
// shader-clock ticks).  Flops per launch: nwg * 4 waves * iters * 64 products * (16384 for kind
// 0, 65536 for kind 1).  Returns the launch's hipError_t as an int.
extern "C" int tbg_diag_mfma_rate(int kind, const void* src, void* out, int nwg, int iters, void* clk, void* stream) {
  if ((kind != 0 && kind != 1) || nwg <= 0 || iters <= 0 || !src || !out || !clk) return (int)hipErrorInvalidValue;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(nwg), dim3(256), 0, (hipStream_t)stream, (const i32x4_t*)src,
                       (float*)out, iters, (uint64_t*)clk);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(nwg), dim3(256), 0, (hipStream_t)stream, (const i32x4_t*)src,
                       (float*)out, iters, (uint64_t*)clk);
  return (int)hipGetLastError();
}

// The library's 256x256 two-stage ring on a bf16 product with B stored K×N and bf16 output (the
// kernel the library runs on the 8192^3 workload), built with clock recording: each workgroup
// writes {real-time ticks at 100 MHz, shader-clock ticks} from its start to the end of its stores
// into clk[2 * workgroup].  Operands must need no repack (16-byte aligned, lda, ldb, ldc and K
// multiples of 8).  Returns the launch's hipError_t as an int; the number of workgroups through
// nwg_out.
extern "C" int tbg_diag_gemm_clock(const void* A, const void* B, void* C, int M, int N, int K, long long lda,
                                   long long ldb, long long ldc, void* clk, int* nwg_out, void* stream) {
  if (!A || !B || !C || !clk || M <= 0 || N <= 0 || K <= 0 || lda % 8 || ldb % 8 || ldc % 8 || K % 8 || lda < K ||
      ldb < N || ldc < N || ((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) % 16)
    return (int)hipErrorInvalidValue;
  tbg::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  p.C = C;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = M;
  p.N = N;
  p.K = K;
  p.kchunks = K / 8;
  p.tiles_m = (M + 255) / 256;
  p.tiles_n = (N + 255) / 256;
  p.group_m = 4;
  p.vec_store = 1;
  p.alpha = 1.f;
  p.clock = (uint64_t*)clk;
  // the operand descriptors the library's encoder would produce (the fields the kernel reads):
  // A {K, M}, B stored K×N {N, K}, bf16, row pitches in bytes
  p.da.elsize = p.db.elsize = 2;
  p.da.base = (uint64_t)(uintptr_t)A;
  p.da.dim[0] = (uint64_t)K;
  p.da.dim[1] = (uint64_t)M;
  p.da.stride[1] = (uint64_t)lda * 2;
  p.db.base = (uint64_t)(uintptr_t)B;
  p.db.dim[0] = (uint64_t)N;
  p.db.dim[1] = (uint64_t)K;
  p.db.stride[1] = (uint64_t)ldb * 2;
  const int nwg = p.tiles_m * p.tiles_n;
  if (nwg_out) *nwg_out = nwg;
  hipLaunchKernelGGL((tbg::gemm_ring_kernel<256, 256, 2, 0, 0, 1, 0, 1>), dim3(nwg), dim3(tbg::kThreads), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

// Per-workgroup timelines of the library's barrier ring (gemm_ring.hpp, CLK 2) on a bf16 product
// with B stored K×N, for the configurations the library picks on small and ragged products:
// cfg 0: 128x128, 2 stages; 1: 256x128, 3 stages; 2: 256x256, 2 stages; 3: 64x64, 3 stages.
// out_bf16 selects the output type (else fp32).  Each workgroup writes 8 uint64 into
// tl[8 * workgroup] (see gemm_ring.hpp).  Operands must need no repack (16-byte aligned bases,
// lda, ldb and K multiples of 8); C's base and row pitch multiples of 4 bytes.  Returns the
// launch's hipError_t as an int; the number of workgroups through nwg_out.
template <int BM, int BN, int S>
static int diag_timeline(const void* A, const void* B, void* C, int M, int N, int K, long long lda, long long ldb,
                         long long ldc, int out_bf16, void* tl, int* nwg_out, hipStream_t stream) {
  tbg::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  p.C = C;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = M;
  p.N = N;
  p.K = K;
  p.kchunks = K / 8;
  p.tiles_m = (M + BM - 1) / BM;
  p.tiles_n = (N + BN - 1) / BN;
  p.group_m = 4;
  p.vec_store = 1;
  p.alpha = 1.f;
  p.clock = (uint64_t*)tl;
  p.da.elsize = p.db.elsize = 2;
  p.da.base = (uint64_t)(uintptr_t)A;
  p.da.dim[0] = (uint64_t)K;
  p.da.dim[1] = (uint64_t)M;
  p.da.stride[1] = (uint64_t)lda * 2;
  p.db.base = (uint64_t)(uintptr_t)B;
  p.db.dim[0] = (uint64_t)N;
  p.db.dim[1] = (uint64_t)K;
  p.db.stride[1] = (uint64_t)ldb * 2;
  const int nwg = p.tiles_m * p.tiles_n;
  if (nwg_out) *nwg_out = nwg;
  if (out_bf16)
    hipLaunchKernelGGL((tbg::gemm_ring_kernel<BM, BN, S, 0, 0, 1, 0, 2>), dim3(nwg), dim3(tbg::kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((tbg::gemm_ring_kernel<BM, BN, S, 0, 0, 0, 0, 2>), dim3(nwg), dim3(tbg::kThreads), 0, stream, p);
  return (int)hipGetLastError();
}

extern "C" int tbg_diag_gemm_timeline(int cfg, const void* A, const void* B, void* C, int M, int N, int K,
                                      long long lda, long long ldb, long long ldc, int out_bf16, void* tl,
                                      int* nwg_out, void* stream) {
  const int es = out_bf16 ? 2 : 4;
  if (!A || !B || !C || !tl || M <= 0 || N <= 0 || K <= 0 || lda % 8 || ldb % 8 || K % 8 || lda < K || ldb < N ||
      ldc < N || ((uintptr_t)A | (uintptr_t)B) % 16 || ((uintptr_t)C) % 4 || (ldc * es) % 4)
    return (int)hipErrorInvalidValue;
  const hipStream_t s = (hipStream_t)stream;
  switch (cfg) {
    case 0: return diag_timeline<128, 128, 2>(A, B, C, M, N, K, lda, ldb, ldc, out_bf16, tl, nwg_out, s);
    case 1: return diag_timeline<256, 128, 3>(A, B, C, M, N, K, lda, ldb, ldc, out_bf16, tl, nwg_out, s);
    case 2: return diag_timeline<256, 256, 2>(A, B, C, M, N, K, lda, ldb, ldc, out_bf16, tl, nwg_out, s);
    case 3: return diag_timeline<64, 64, 3>(A, B, C, M, N, K, lda, ldb, ldc, out_bf16, tl, nwg_out, s);
  }
  return (int)hipErrorInvalidValue;
}
