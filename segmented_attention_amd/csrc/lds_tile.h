// LDS staging of packed-latent rows (512 nope + 64 RoPE bf16 dims, 1152 bytes) shared by the
// attention and projection kernels.
//
// Layout of a tile of R rows: a nope region of R rows x 64 16-byte chunks (chunk c of row r at
// r * 64 + (c ^ fn(r))) followed by a RoPE region of R rows x 8 chunks (chunk c of row r at
// r * 8 + (c ^ fr(r))). With 64 LDS banks (16 chunk slots per 256 bytes):
// * the MFMA operand read of 16 consecutive rows, one chunk each (16 lanes, b128), and
// * the transposing read of 4 consecutive rows x 4 chunks (32 lanes, ds_read_b64_tr_b16)
// each land in 16 distinct slots in both regions.
//
// Rows are copied with global->LDS loads issued from inline assembly (see dma16): a nope row
// is one 64-lane instruction (64 x 16 bytes), 8 RoPE rows are one instruction.
#pragma once
#include <cstdint>

namespace segmla {

typedef __attribute__((address_space(3))) char lds_char;

// nope-region swizzle: a bijection on row bits 0..3 whose top two bits follow row bits 0..1
__device__ __forceinline__ int fn(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// RoPE-region swizzle, a bijection on row bits 1..3 (row bit 0 selects the half of the
// 256-byte bank line) whose top bit follows row bit 1
__device__ __forceinline__ int fr(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// LDS byte address of a pointer into dynamic shared memory
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// Lane id from v_mbcnt in a volatile statement: values derived from it are recomputed where
// they are used instead of being kept live (and possibly spilled) across a loop.
__device__ __forceinline__ int lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// One 64-lane global->LDS copy of 16 bytes per lane: lane L's bytes from sbase + voff land at
// LDS byte address lds + 16 L. Issued from inline assembly so that the compiler does not see
// an LDS write in flight: it would otherwise wait for every outstanding copy before each later
// LDS read. The consumer orders it explicitly (s_waitcnt vmcnt, then a barrier). M0 needs one
// wait state after the SALU write before the load reads it. Nothing else in these kernels
// keeps a value in M0 (checked on the generated assembly by the CPU tests).
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
// The same with a full 64-bit address per lane.
__device__ __forceinline__ void dma16_v(const char* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(vaddr), "s"(lds)
               : "memory", "m0");
}

}  // namespace segmla
