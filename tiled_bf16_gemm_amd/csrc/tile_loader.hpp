// Device side of the descriptor-driven tile copy on gfx950: swizzle, buffer resources, and the
// direct-to-LDS loader shared by the copy kernel and the GEMM.
//
// The pages ("2 · Le Tensor Memory Accelerator" §2.1–§2.2; "H100 · cuTensorMap" §1–§4) describe
// a copy engine that, given a descriptor and box coordinates, generates addresses, applies the
// bounds check and the swizzle, and writes the box into on-chip memory.  On gfx950 the same
// contract is met by the whole wave: each lane issues one 16-byte `buffer_load_dwordx4 ... lds`
// whose destination is LDS[M0 + 16 * lane].  The buffer resource's range check returns zeros
// for every dword at or past `num_records`, which gives the out-of-bounds zero fill ("H100 ·
// cuTensorMap" §14) without any branch, and because a wave writes one contiguous 1 KiB block of
// LDS, the swizzle is applied by choosing which source chunk each lane fetches: the XOR swizzle
// is an involution, so LDS slot s receives logical chunk swizzle(s).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tbg {

typedef __attribute__((address_space(3))) void lds_void_t;

// ---- swizzle ("H100 · cuTensorMap" §11.3) ---------------------------------------------------
// Byte offset inside an image -> LDS byte offset.  mode 0 none, 1 32B, 2 64B, 3 128B,
// 4 the 2-row extension a ^ ((a & 0x700) >> 4), 5 the transposing-read layout (the 16-byte unit
// of 128-byte row r XORed with row_xor<5>(r)).
__host__ __device__ __forceinline__ uint32_t swizzle_offset(uint32_t a, int mode) {
  switch (mode) {
    case 1: return a ^ ((a & 0x080u) >> 3);
    case 2: return a ^ ((a & 0x180u) >> 3);
    case 3: return a ^ ((a & 0x380u) >> 3);
    case 4: return a ^ ((a & 0x700u) >> 4);
    case 5: {
      const uint32_t r = a >> 7;
      return a ^ (((((r >> 3) & 1u) << 2) | (((r >> 1) & 1u) << 1) | ((r >> 2) & 1u)) << 4);
    }
    default: return a;
  }
}

// For images made of 128-byte rows: the XOR applied to the 16-byte chunk index of row r (modes
// 3, 4 and 5 of swizzle_offset).
template <int SWZ>
__device__ __forceinline__ int row_xor(int r) {
  static_assert(SWZ == 3 || SWZ == 4 || SWZ == 5, "128-byte-row loader takes the 128B, 2-row or K×N layout");
  if (SWZ == 3) return r & 7;
  if (SWZ == 4) return (r >> 1) & 7;
  return (((r >> 3) & 1) << 2) | (((r >> 1) & 1) << 1) | ((r >> 2) & 1);
}

// ---- buffer resources --------------------------------------------------------------------
// A raw buffer descriptor (stride 0) in four scalar registers: base address bits [47:0],
// num_records, and dword 3 = 0x00020000, the gfx9 data format for raw dword access.  Every
// field goes through readfirstlane so the descriptor lives in SGPRs even when the compiler
// cannot prove the inputs uniform.  num_records is kept below 2^31 so that the 0x80000000 offset
// used to mask a lane is always out of range.
typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFFFull ? 0x7FFFFFFFu : (uint32_t)bytes;
  const uint64_t a = (uint64_t)(uintptr_t)base;
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)n);
  r.w = 0x00020000;
  return r;
}

constexpr uint32_t kOobOffset = 0x80000000u;

// s_waitcnt immediate for gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
__host__ __device__ constexpr int waitcnt_vm(int n) {
  return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 0x3) << 14);
}

// ---- the 128-byte-row box loader ---------------------------------------------------------
// A box whose rows are 128 bytes (64 bf16) and whose row count is a multiple of 8 is loaded in
// 1 KiB atoms of 8 rows.  For the atom starting at box row `row0`, lane l fills LDS slot l,
// i.e. physical row row0 + l/8, physical chunk l%8, which holds logical chunk
// (l%8) ^ row_xor(row).  The lane's source is row `row` and logical chunk c of the box:
//   byte offset = row * row_pitch + c * 16   (relative to the box origin).
struct LaneChunk {
  uint32_t offset;  // byte offset from the box origin
  int chunk;        // logical 16-byte chunk index within the 128-byte row (0..7)
};

template <int SWZ>
__device__ __forceinline__ LaneChunk lane_chunk(int row0, int lane, uint32_t row_pitch) {
  const int row = row0 + (lane >> 3);
  const int c = (lane & 7) ^ row_xor<SWZ>(row);
  return LaneChunk{(uint32_t)row * row_pitch + (uint32_t)c * 16u, c};
}

// Issue one atom: every lane moves 16 bytes into LDS[dst + 16 * lane].  Lanes whose logical
// chunk starts at or beyond `chunks_valid` fetch from an out-of-range offset and write zeros.
// `lds_addr` is the LDS byte address of the atom, the same for the whole wave, 16-byte aligned
// (1 KiB for swizzled images).  The instruction is emitted as inline assembly so that the
// compiler does not add its own vmcnt waits before every later LDS read: completion is awaited
// explicitly with `s_waitcnt vmcnt` before the barrier that publishes a stage.  The LDS
// destination goes in through the "{m0}" operand constraint: the compiler itself writes M0
// before the statement, so it knows M0's contents and keeps no value of its own there.
__device__ __forceinline__ void issue_atom(rsrc_t rs, uint32_t lds_addr, LaneChunk lc,
                                           int chunks_valid) {
  const uint32_t off = lc.chunk < chunks_valid ? lc.offset : kOobOffset;
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rs), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// issue_atom with the lane's chunk test already made (`valid` false: the lane lands zeros) and
// the atom's LDS address as a base plus an offset that is a compile-time constant where this is
// inlined (the atom index of an unrolled loop): the compiler then sets M0 with one scalar add.
__device__ __forceinline__ void issue_atom_if(rsrc_t rs, uint32_t lds_base, int lds_imm, uint32_t offset, bool valid) {
  const uint32_t off = valid ? offset : kOobOffset;
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rs), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base) + (uint32_t)lds_imm)
               : "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace tbg
