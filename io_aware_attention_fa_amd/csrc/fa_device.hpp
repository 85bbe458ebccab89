// Device helpers for gfx950 (CDNA4): vector types, buffer loads, MFMA, exp2/log2, bf16 packing.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// (1.0, 1.0) in bf16: a v_dot2 against it sums a bf16 pair in fp32.
__device__ __forceinline__ bf16x2_t ones_bf16x2() {
  return __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
}

// Buffer resource over [base, base + bytes): loads at byte offsets >= bytes return zeros, which
// gives free, fault-free handling of ragged tails.  Word 3 selects 32-bit raw dword data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
// The same load marked non-temporal (cache policy bit 1: `nt` on gfx950), for data read once.
__device__ __forceinline__ u32x4_t buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2);
}

// D = A(32x16) * B(16x32) + C(32x32), bf16 inputs, fp32 accumulate.
// Lane l holds A row (l % 32) and B column (l % 32), each with 8 consecutive k-slots chosen by
// l / 32; D column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4) for register i.
__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Scalar helpers take their operand by value: this compiler mis-lowers a bit cast applied
// directly to a subscripted vector element (it reads element 0), so never write
// __builtin_bit_cast(T, vec[i]).
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Round four fp32 values to bf16 (round to nearest even) and pack them into 8 bytes.
__device__ __forceinline__ u32x2_t pack_bf16x4(float a, float b, float c, float d) {
  f32x4_t f = {a, b, c, d};
  bf16x4_t h = __builtin_convertvector(f, bf16x4_t);
  return __builtin_bit_cast(u32x2_t, h);
}

// bf16 element e (0..7) of a 16-byte chunk, widened to fp32 exactly.
__device__ __forceinline__ float bf16_elem(u32x4_t v, int e) {
  const uint32_t w = v[e >> 1];
  return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
}

}  // namespace fa
