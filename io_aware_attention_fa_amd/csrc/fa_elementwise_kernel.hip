// Fused elementwise chains for gfx950: GELU (fp32 or bf16) and bias -> GELU -> dropout (bf16).
//
// The method (page "Chapter 10 Writing and Benchmarking Custom Kernels", section 10.2.1, the GeLU
// case study: one read and one write per element instead of one HBM round trip per
// sub-operation, with 16-byte vector accesses; page "Fusion and IO-aware kernels", "The idea in
// one minute": a bias add, a GELU and a dropout fused into one kernel).  GELU is the tanh form
// 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), evaluated as x * sigmoid(2u) with
// u = sqrt(2/pi) (x + 0.044715 x^3) (the same function: 0.5 (1 + tanh u) = 1 / (1 + e^(-2u))).
//
// Dropout draws from Philox4x32-10 (Salmon et al., SC 2011), written here from its published
// definition: element e of the row-major activation uses 16 bits, half e % 2 (low for even e)
// of word (e % 8) / 2 of the generator applied to the counter (e / 8 low, e / 8 high, offset
// low, offset high) under the key (seed low, seed high), and is dropped iff that value is below
// floor(p * 2^16); kept elements are scaled by 1 / (1 - p).  One generator call thus serves
// eight elements (its 40 64-bit multiplies per call had made the kernel bound by them rather
// than by HBM).  The decision is an integer comparison, so it is reproducible bit for bit.
//
// MI355X mapping (our design): streaming kernels with 16-byte nontemporal loads and stores,
// 4 (fp32) or 8 (bf16) elements per lane per access, several accesses in flight per lane; the
// dropout kernel gives each lane 8 consecutive columns of two rows (one Philox block per row),
// so that the bias needs no division by the row length and is unpacked once for both rows.
// Lengths that do not fit the vector layout take a scalar path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kThreadsEw = 256;
// vector accesses in flight per lane: 1, with one 256-lane workgroup per 256 vectors (up to 65536
// workgroups), ran the 64M-element fp32 GELU 7.6% faster than 4 per lane with a quarter of the
// workgroups (same box), and 2 per lane 3.8% faster
constexpr int kUnrollEw = 1;

// -2 sqrt(2/pi) log2(e) and the cubic coefficient: gelu(x) = x / (1 + 2^(K1 x (1 + A x^2)))
constexpr float kGeluK1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
constexpr float kGeluK1A = -2.0f * 0.7978845608028654f * 1.4426950408889634f * 0.044715f;

// x / (1 + 2^z) with z = x (K1 + K1 A x^2) and the hardware reciprocal (within an ulp or so;
// 1 + 2^z >= 1, and an infinite 2^z gives 0, the limit).
__device__ __forceinline__ float gelu(float x) {
  const float z = x * __builtin_fmaf(x * x, kGeluK1A, kGeluK1);
  return x * __builtin_amdgcn_rcpf(1.0f + fast_exp2(z));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// ---- Philox4x32-10 ----
struct Philox4 {
  uint32_t v[4];
};
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    // three-input XORs as one gfx950 v_bitop3_b32 each (truth table 0x96: odd parity)
    c0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
    c1 = lo1;
    c2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
    c3 = lo0;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// ---- GELU, fp32 ----
__global__ __launch_bounds__(kThreadsEw) void fa_gelu_f32_kernel(const float* __restrict__ x,
                                                                 float* __restrict__ y,
                                                                 int64_t n) {
  const int64_t nv = n / 4;   // full float4 groups
  const int64_t stride = (int64_t)gridDim.x * kThreadsEw;
  int64_t i = (int64_t)blockIdx.x * kThreadsEw + threadIdx.x;
  const f32x4_t* xv = reinterpret_cast<const f32x4_t*>(x);
  f32x4_t* yv = reinterpret_cast<f32x4_t*>(y);
  for (; i + (kUnrollEw - 1) * stride < nv; i += kUnrollEw * stride) {
    f32x4_t a[kUnrollEw];
#pragma unroll
    for (int u = 0; u < kUnrollEw; ++u) a[u] = __builtin_nontemporal_load(xv + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnrollEw; ++u) {
      const f32x4_t r = {gelu(a[u][0]), gelu(a[u][1]), gelu(a[u][2]), gelu(a[u][3])};
      __builtin_nontemporal_store(r, yv + i + u * stride);
    }
  }
  for (; i < nv; i += stride) {
    const f32x4_t a = __builtin_nontemporal_load(xv + i);
    const f32x4_t r = {gelu(a[0]), gelu(a[1]), gelu(a[2]), gelu(a[3])};
    __builtin_nontemporal_store(r, yv + i);
  }
  // the last n % 4 elements
  const int64_t t = (int64_t)blockIdx.x * kThreadsEw + threadIdx.x;
  if (t < n - 4 * nv) y[4 * nv + t] = gelu(x[4 * nv + t]);
}

// ---- GELU, bf16 (fp32 arithmetic, round to nearest even on output) ----
__device__ __forceinline__ u32x4_t gelu_bf16x8(u32x4_t a) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x2_t p = pack_bf16x4(gelu(bf16_lo(a[j])), gelu(bf16_hi(a[j])), 0.f, 0.f);
    r[j] = p[0];
  }
  return r;
}

__global__ __launch_bounds__(kThreadsEw) void fa_gelu_bf16_kernel(const uint16_t* __restrict__ x,
                                                                  uint16_t* __restrict__ y,
                                                                  int64_t n) {
  const int64_t nv = n / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreadsEw;
  int64_t i = (int64_t)blockIdx.x * kThreadsEw + threadIdx.x;
  const u32x4_t* xv = reinterpret_cast<const u32x4_t*>(x);
  u32x4_t* yv = reinterpret_cast<u32x4_t*>(y);
  for (; i + (kUnrollEw - 1) * stride < nv; i += kUnrollEw * stride) {
    u32x4_t a[kUnrollEw];
#pragma unroll
    for (int u = 0; u < kUnrollEw; ++u) a[u] = __builtin_nontemporal_load(xv + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnrollEw; ++u)
      __builtin_nontemporal_store(gelu_bf16x8(a[u]), yv + i + u * stride);
  }
  for (; i < nv; i += stride) __builtin_nontemporal_store(gelu_bf16x8(__builtin_nontemporal_load(xv + i)), yv + i);
  const int64_t t = (int64_t)blockIdx.x * kThreadsEw + threadIdx.x;
  if (t < n - 8 * nv) {
    const int64_t e = 8 * nv + t;
    const u32x2_t p = pack_bf16x4(gelu(bf16_lo(x[e])), 0.f, 0.f, 0.f);
    y[e] = (uint16_t)p[0];
  }
}

// ---- bias -> GELU -> dropout, bf16 ----
struct DropoutParams {
  const uint16_t* x;
  const uint16_t* bias;
  uint16_t* y;
  int64_t rows, cols;
  uint32_t threshold;   // drop iff word < threshold
  float scale;          // 1 / (1 - p)
  uint32_t seed_lo, seed_hi, off_lo, off_hi;
};

// Computed for every element and selected, so that the wave never branches on the mask.  The
// element's 16-bit draw is compared in the high half of a word: bits is the generator word for
// an odd element and the word shifted left by 16 for an even one, and p.threshold is
// floor(p * 2^16) * 2^16.
__device__ __forceinline__ float dropout_one(float xb, uint32_t bits, const DropoutParams& p) {
  const float g = gelu(xb) * p.scale;
  return bits >= p.threshold ? g : 0.f;
}

// Vector path (cols % 8 == 0, 16-byte aligned rows): lane -> the same 8 consecutive columns of
// two rows (2 * blockIdx.y and the next one, if any), so that the bias is loaded and unpacked once
// and both rows' loads are in flight together.
__device__ __forceinline__ u32x4_t dropout_8(u32x4_t a, const float (&bf)[8], int64_t e,
                                            const DropoutParams& p) {
  const uint64_t blk = (uint64_t)e >> 3;   // e is a multiple of 8: one generator block
  const Philox4 w = philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), p.off_lo, p.off_hi,
                                  p.seed_lo, p.seed_hi);
  float r[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // elements 2j and 2j + 1: the two halves of word j
    r[2 * j] = dropout_one(bf16_lo(a[j]) + bf[2 * j], w.v[j] << 16, p);
    r[2 * j + 1] = dropout_one(bf16_hi(a[j]) + bf[2 * j + 1], w.v[j], p);
  }
  const u32x2_t lo = pack_bf16x4(r[0], r[1], r[2], r[3]);
  const u32x2_t hi = pack_bf16x4(r[4], r[5], r[6], r[7]);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

__global__ __launch_bounds__(kThreadsEw) void fa_bias_gelu_dropout_vec_kernel(DropoutParams p) {
  const int64_t row = 2 * (int64_t)blockIdx.y;
  const int64_t col = ((int64_t)blockIdx.x * kThreadsEw + threadIdx.x) * 8;
  if (col >= p.cols) return;
  const bool two = row + 1 < p.rows;
  const int64_t e = row * p.cols + col;   // a multiple of 8
  const u32x4_t a0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.x + e));
  u32x4_t a1 = u32x4_t{0u, 0u, 0u, 0u};
  if (two) a1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.x + e + p.cols));
  const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p.bias + col);
  float bf[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf[2 * j] = bf16_lo(b[j]);
    bf[2 * j + 1] = bf16_hi(b[j]);
  }
  __builtin_nontemporal_store(dropout_8(a0, bf, e, p), reinterpret_cast<u32x4_t*>(p.y + e));
  if (two)
    __builtin_nontemporal_store(dropout_8(a1, bf, e + p.cols, p),
                                reinterpret_cast<u32x4_t*>(p.y + e + p.cols));
}

// Scalar path: one element per lane, any shape.
__global__ __launch_bounds__(kThreadsEw) void fa_bias_gelu_dropout_scalar_kernel(DropoutParams p) {
  const int64_t n = p.rows * p.cols;
  const int64_t stride = (int64_t)gridDim.x * kThreadsEw;
  for (int64_t e = (int64_t)blockIdx.x * kThreadsEw + threadIdx.x; e < n; e += stride) {
    const int64_t col = e % p.cols;
    const uint64_t blk = (uint64_t)e >> 3;
    const Philox4 w = philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), p.off_lo, p.off_hi,
                                    p.seed_lo, p.seed_hi);
    const uint32_t word = w.v[(e >> 1) & 3];
    const float xb = bf16_lo(p.x[e]) + bf16_lo(p.bias[col]);
    const u32x2_t o = pack_bf16x4(dropout_one(xb, (e & 1) ? word : word << 16, p), 0.f, 0.f, 0.f);
    p.y[e] = (uint16_t)o[0];
  }
}

int grid_for(int64_t groups) {
  const int64_t per = (int64_t)kThreadsEw * kUnrollEw;
  int64_t g = (groups + per - 1) / per;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;   // grid-stride beyond this
  return (int)g;
}

}  // namespace

hipError_t launch_gelu(const GeluLaunch& a, hipStream_t s) {
  if (a.bf16) {
    hipLaunchKernelGGL(fa_gelu_bf16_kernel, dim3(grid_for(a.n / 8 + 1)), dim3(kThreadsEw), 0, s,
                       static_cast<const uint16_t*>(a.x), static_cast<uint16_t*>(a.y), a.n);
  } else {
    hipLaunchKernelGGL(fa_gelu_f32_kernel, dim3(grid_for(a.n / 4 + 1)), dim3(kThreadsEw), 0, s,
                       static_cast<const float*>(a.x), static_cast<float*>(a.y), a.n);
  }
  return hipGetLastError();
}

hipError_t launch_bias_gelu_dropout(const DropoutLaunch& a, hipStream_t s) {
  DropoutParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.bias = static_cast<const uint16_t*>(a.bias);
  p.y = static_cast<uint16_t*>(a.y);
  p.rows = a.rows;
  p.cols = a.cols;
  p.threshold = a.threshold;
  p.scale = a.scale;
  p.seed_lo = (uint32_t)a.seed;
  p.seed_hi = (uint32_t)(a.seed >> 32);
  p.off_lo = (uint32_t)a.offset;
  p.off_hi = (uint32_t)(a.offset >> 32);
  const bool vec = a.cols % 8 == 0 && reinterpret_cast<uintptr_t>(a.x) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.y) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.bias) % 16 == 0 && a.rows <= 65535;
  if (vec) {
    const int64_t gx = (a.cols / 8 + kThreadsEw - 1) / kThreadsEw;
    const int64_t gy = (a.rows + 1) / 2;   // row pairs
    hipLaunchKernelGGL(fa_bias_gelu_dropout_vec_kernel, dim3((unsigned)gx, (unsigned)gy),
                       dim3(kThreadsEw), 0, s, p);
  } else {
    int64_t g = (a.rows * a.cols + kThreadsEw - 1) / kThreadsEw;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(fa_bias_gelu_dropout_scalar_kernel, dim3((unsigned)g), dim3(kThreadsEw), 0,
                       s, p);
  }
  return hipGetLastError();
}

}  // namespace fa
