// Measurement aid for the benchmark, not part of the library's ABI: the rate at which this chip
// sustains bf16 matrix products when nothing else runs, the ceiling a GEMM kernel can reach at
// the clock the power limit allows.  Each wave issues v_mfma_f32_16x16x32_bf16 back to back on
// register-resident operand fragments filled from a buffer of random bf16 values (the matrix
// units' energy depends on operand bits), accumulators in AGPRs, never reusing an accumulator
// within 64 products; one workgroup of four waves per CU (the full register file, as the 256x256
// GEMM tile), `nwg` workgroups.  Each workgroup records its shader-clock and 100 MHz real-time
// counter deltas, from which the caller derives the clock the products ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256, 1) mfma_rate_kernel(const bf16x8_t* src, float* out, int iters,
                                                            uint64_t* clk) {
  const int t = threadIdx.x;
  bf16x8_t a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[((uint64_t)blockIdx.x * 16 + i) * 256 + t];
    b[i] = src[((uint64_t)blockIdx.x * 16 + 8 + i) * 256 + t];
  }
  f32x4_t acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime(), m0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 64; ++i)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i]) : "v"(a[i & 7]), "v"(b[i >> 3]));
  }
  // wait states before the accumulators are read (the products are inline assembly)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime(), m1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    f32x4_t v = acc[i];
    asm volatile("" : "+v"(v));
    s += v[0] + v[1] + v[2] + v[3];
  }
  out[(uint64_t)blockIdx.x * 256 + t] = s;
  if (t == 0) {
    clk[2 * (uint64_t)blockIdx.x] = r1 - r0;
    clk[2 * (uint64_t)blockIdx.x + 1] = m1 - m0;
  }
}

// src: nwg * 16 * 256 bf16x8 values (nwg * 64 KiB); out: nwg * 256 floats; clk: 2 * nwg uint64
// (real-time ticks at 100 MHz, shader-clock ticks).  Flops per launch: nwg * 4 waves * iters * 64
// products * 16384.  Returns the launch's hipError_t as an int.
extern "C" int tbg_diag_mfma_rate(const void* src, void* out, int nwg, int iters, void* clk, void* stream) {
  if (nwg <= 0 || iters <= 0 || !src || !out || !clk) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(nwg), dim3(256), 0, (hipStream_t)stream, (const bf16x8_t*)src,
                     (float*)out, iters, (uint64_t*)clk);
  return (int)hipGetLastError();
}
