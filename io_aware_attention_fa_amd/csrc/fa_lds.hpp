// LDS staging helpers for gfx950 kernels that stream row-major tiles through shared memory:
// direct global-to-LDS loads, vector-memory waits, the LDS reads that feed MFMA operands, and
// 16-byte LDS writes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"

namespace fa {

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8),
// waiting on vector-memory operations only.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Buffer resource words for the LDS loads below: base, stride 0, byte range (reads at offsets
// >= range return zeros), raw 32-bit dword format.
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// One buffer_load ... lds: lane l reads 16 (dwordx4) or 4 (dword) bytes at byte offset voff of
// the buffer and writes them to LDS at m0 + 16*l (or m0 + 4*l).  Inline assembly, so that the
// compiler neither tracks the load (it would otherwise wait for it before any later LDS read it
// cannot prove disjoint) nor moves LDS accesses across it; kernels wait for these loads with
// s_waitcnt vmcnt themselves.
__device__ __forceinline__ void lds_dma16(u32x4_t rsrc, uint32_t m0, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(u32x4_t rsrc, uint32_t m0, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// 16-byte LDS reads at a byte address.
__device__ __forceinline__ bf16x8_t lds_read_bf16x8(uint32_t addr) {
  typedef __attribute__((address_space(3))) const bf16x8_t* lds_ptr_t;
  return *(lds_ptr_t)(uintptr_t)addr;
}
__device__ __forceinline__ f32x4_t lds_read_f32x4(uint32_t addr) {
  typedef __attribute__((address_space(3))) const f32x4_t* lds_ptr_t;
  return *(lds_ptr_t)(uintptr_t)addr;
}

__device__ __forceinline__ u32x4_t lds_read_u32x4(uint32_t addr) {
  typedef __attribute__((address_space(3))) const u32x4_t* lds_ptr_t;
  return *(lds_ptr_t)(uintptr_t)addr;
}

// 8- and 16-byte LDS writes at a byte address.
__device__ __forceinline__ void lds_write_u32x2(uint32_t addr, u32x2_t v) {
  typedef __attribute__((address_space(3))) u32x2_t* lds_ptr_t;
  *(lds_ptr_t)(uintptr_t)addr = v;
}
__device__ __forceinline__ void lds_write_f32x4(uint32_t addr, f32x4_t v) {
  typedef __attribute__((address_space(3))) f32x4_t* lds_ptr_t;
  *(lds_ptr_t)(uintptr_t)addr = v;
}
__device__ __forceinline__ void lds_write_bf16x8(uint32_t addr, bf16x8_t v) {
  typedef __attribute__((address_space(3))) bf16x8_t* lds_ptr_t;
  *(lds_ptr_t)(uintptr_t)addr = v;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane j receives,
// for t = 0..3, the 16-bit element j % 4 of the 8 bytes addressed by lane 4t + j / 4.
__device__ __forceinline__ u32x2_t lds_read_tr(uint32_t addr) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4_t* lds_ptr_t;
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr_t)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2_t, v);
}

// Two transposing reads 8 rows apart form one MFMA A operand (8 bf16).
__device__ __forceinline__ bf16x8_t lds_read_tr_pair(uint32_t a0, uint32_t a1) {
  const u32x2_t lo = lds_read_tr(a0);
  const u32x2_t hi = lds_read_tr(a1);
  const u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf16x8(w);
}

}  // namespace fa
