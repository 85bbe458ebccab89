// Row-wise softmax for gfx950: y = softmax(x) over each row of a [rows][cols] fp32 matrix, and
// optionally each row's log-sum-exp.
//
// The method (page "Chapter 10 Writing and Benchmarking Custom Kernels", section 10.2.2, the
// worked example and its closing question; page "Kernels -- fusion and FlashAttention",
// section 3): one HBM read and one write per element, the row's max subtracted before
// exponentiating, and the running (max, sum) pair of the online recurrence, whose merge rescales
// a partial sum by exp(m_part - m_new) when the max grows.
//
// MI355X mapping (our design, not the pages'):
//   * Four waves per workgroup, no LDS and no barriers.  Up to 8192 columns a wave holds a
//     whole row in registers (up to 4096 columns two rows each, the next row's loads issued
//     before the current row is written): lane l holds, for chunk c, the 16-byte group of columns
//     c*256 + 4*l .. +3 (fully coalesced 1 KB wave loads), read once with nontemporal hints.
//   * Each lane reduces its own entries to (m, l) -- the max, then the sum of exp(x - m) with the
//     exponentials kept in registers -- and the 64 lanes merge their pairs by the recurrence's
//     rescale: M = max m, L = sum l * exp(m - M).  The outputs are the kept exponentials times
//     exp(m - M) / L: one multiply per element, no second exponential.
//   * Wider rows take the streamed form of the same recurrence: pass 1 folds 2048-column tiles
//     into (m, l) with the rescale, pass 2 reads the row again and writes exp(x - M) / L.
//   * Rows whose length is not a multiple of 4 (or unaligned pointers) use 4-byte accesses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kRowsPerBlock = 4;   // one wave per row
constexpr int kStreamChunks = 8;   // chunks per tile of the streamed form

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) v = fmaxf(v, __shfl_xor(v, w));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) v += __shfl_xor(v, w);
  return v;
}

// exp(a - b) for b >= a, with b = -inf (nothing seen yet) giving 0.
__device__ __forceinline__ float exp_diff(float a, float b) {
  return b == -INFINITY ? 0.f : fast_exp2((a - b) * kLog2e);
}

// VEC consecutive columns starting at col (masked columns read as -inf).
template <int VEC>
__device__ __forceinline__ void load_vec(const float* __restrict__ r, int col, int cols, float* v) {
  if (col + VEC <= cols) {
    if constexpr (VEC == 4) {
      const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(r + col));
      v[0] = t[0];
      v[1] = t[1];
      v[2] = t[2];
      v[3] = t[3];
    } else {
      v[0] = __builtin_nontemporal_load(r + col);
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = col + e < cols ? r[col + e] : -INFINITY;
  }
}

template <int VEC>
__device__ __forceinline__ void store_vec(float* __restrict__ r, int col, int cols, const float* v) {
  if (col + VEC <= cols) {
    if constexpr (VEC == 4) {
      __builtin_nontemporal_store(f32x4_t{v[0], v[1], v[2], v[3]},
                                  reinterpret_cast<f32x4_t*>(r + col));
    } else {
      __builtin_nontemporal_store(v[0], r + col);
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (col + e < cols) r[col + e] = v[e];
  }
}

// Row held in registers: CH chunks of 64 * VEC columns.  Up to 16 chunks each wave takes rows
// row0, row0 + W, ... (W waves in the grid, launched for two rows per wave), issuing the next
// row's loads before it works on and stores the current one, so that reads and writes overlap:
// 4-7% faster than one row per wave at 4096 and 2048 columns (bit-identical).  32 chunks hold
// one row at a time (two would spill).
template <int VEC, int CH>
__device__ __forceinline__ void softmax_row(float* v, float* __restrict__ yr,
                                            float* __restrict__ lse, int64_t row, int cols,
                                            int lane) {
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int i = 0; i < CH * VEC; ++i) mx[i & 3] = fmaxf(mx[i & 3], v[i]);
  const float m = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CH * VEC; ++i) {
    v[i] = exp_diff(v[i], m);
    ls[i & 3] += v[i];
  }
  const float l = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  const float M = wave_max(m);
  const float f = exp_diff(m, M);
  const float L = wave_sum(l * f);
  const float s = f / L;
#pragma unroll
  for (int i = 0; i < CH * VEC; ++i) v[i] *= s;
#pragma unroll
  for (int c = 0; c < CH; ++c) store_vec<VEC>(yr, (c * 64 + lane) * VEC, cols, v + c * VEC);
  if (lse != nullptr && lane == 0) lse[row] = M + fast_log2(L) * kLn2;
}

template <int VEC, int CH>
__global__ __launch_bounds__(64 * kRowsPerBlock) void fa_softmax_reg_kernel(
    const float* __restrict__ x, float* __restrict__ y, float* __restrict__ lse, int64_t rows,
    int cols) {
  const int lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;   // whole waves leave; there is no barrier
  float va[CH * VEC];
#pragma unroll
  for (int c = 0; c < CH; ++c)
    load_vec<VEC>(x + row * cols, (c * 64 + lane) * VEC, cols, va + c * VEC);
  if constexpr (CH > 16) {
    softmax_row<VEC, CH>(va, y + row * cols, lse, row, cols, lane);
    return;
  }
  float vb[CH * VEC];
  for (;;) {
    const int64_t nb = row + W;
    if (nb < rows) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
        load_vec<VEC>(x + nb * cols, (c * 64 + lane) * VEC, cols, vb + c * VEC);
    }
    softmax_row<VEC, CH>(va, y + row * cols, lse, row, cols, lane);
    if (nb >= rows) break;
    const int64_t na = nb + W;
    if (na < rows) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
        load_vec<VEC>(x + na * cols, (c * 64 + lane) * VEC, cols, va + c * VEC);
    }
    softmax_row<VEC, CH>(vb, y + nb * cols, lse, nb, cols, lane);
    if (na >= rows) break;
    row = na;
  }
}

// Streamed form for wide rows: (m, l) over tiles of kStreamChunks chunks, then a second pass.
template <int VEC>
__global__ __launch_bounds__(64 * kRowsPerBlock) void fa_softmax_stream_kernel(
    const float* __restrict__ x, float* __restrict__ y, float* __restrict__ lse, int64_t rows,
    int cols) {
  constexpr int TILE = kStreamChunks * 64 * VEC;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + row * cols;
  float* yr = y + row * cols;
  float m = -INFINITY, l = 0.f;
  for (int t0 = 0; t0 < cols; t0 += TILE) {
    float v[kStreamChunks * VEC];
#pragma unroll
    for (int c = 0; c < kStreamChunks; ++c)
      load_vec<VEC>(xr, t0 + (c * 64 + lane) * VEC, cols, v + c * VEC);
    float tm = -INFINITY;
#pragma unroll
    for (int i = 0; i < kStreamChunks * VEC; ++i) tm = fmaxf(tm, v[i]);
    const float m_new = fmaxf(m, tm);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kStreamChunks * VEC; ++i) acc += exp_diff(v[i], m_new);
    l = l * exp_diff(m, m_new) + acc;   // the rescale of the running sum
    m = m_new;
  }
  const float M = wave_max(m);
  const float L = wave_sum(l * exp_diff(m, M));
  const float inv = 1.f / L;
  for (int t0 = 0; t0 < cols; t0 += TILE) {
    float v[kStreamChunks * VEC];
#pragma unroll
    for (int c = 0; c < kStreamChunks; ++c)
      load_vec<VEC>(xr, t0 + (c * 64 + lane) * VEC, cols, v + c * VEC);
#pragma unroll
    for (int i = 0; i < kStreamChunks * VEC; ++i) v[i] = exp_diff(v[i], M) * inv;
#pragma unroll
    for (int c = 0; c < kStreamChunks; ++c)
      store_vec<VEC>(yr, t0 + (c * 64 + lane) * VEC, cols, v + c * VEC);
  }
  if (lse != nullptr && lane == 0) lse[row] = M + fast_log2(L) * kLn2;
}

template <int VEC>
hipError_t launch_vec(const SoftmaxLaunch& a, hipStream_t s) {
  const int64_t grid = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int chunks = (int)((a.cols + 64 * VEC - 1) / (64 * VEC));
  const dim3 g((unsigned)grid), b(64 * kRowsPerBlock);
  // two rows a wave for the pipelined register kernel
  const dim3 g2((unsigned)((a.rows + 2 * kRowsPerBlock - 1) / (2 * kRowsPerBlock)));
  const float* x = a.x;
  float* y = a.y;
  float* lse = a.lse;
  const int64_t rows = a.rows;
  const int cols = (int)a.cols;
  if (chunks <= 1) hipLaunchKernelGGL((fa_softmax_reg_kernel<VEC, 1>), g2, b, 0, s, x, y, lse, rows, cols);
  else if (chunks <= 2) hipLaunchKernelGGL((fa_softmax_reg_kernel<VEC, 2>), g2, b, 0, s, x, y, lse, rows, cols);
  else if (chunks <= 4) hipLaunchKernelGGL((fa_softmax_reg_kernel<VEC, 4>), g2, b, 0, s, x, y, lse, rows, cols);
  else if (chunks <= 8) hipLaunchKernelGGL((fa_softmax_reg_kernel<VEC, 8>), g2, b, 0, s, x, y, lse, rows, cols);
  else if (chunks <= 16) hipLaunchKernelGGL((fa_softmax_reg_kernel<VEC, 16>), g2, b, 0, s, x, y, lse, rows, cols);
  else if (chunks <= 32) hipLaunchKernelGGL((fa_softmax_reg_kernel<VEC, 32>), g, b, 0, s, x, y, lse, rows, cols);
  else hipLaunchKernelGGL((fa_softmax_stream_kernel<VEC>), g, b, 0, s, x, y, lse, rows, cols);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax(const SoftmaxLaunch& a, hipStream_t stream) {
  const bool vec4 = a.cols % 4 == 0 && reinterpret_cast<uintptr_t>(a.x) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(a.y) % 16 == 0;
  return vec4 ? launch_vec<4>(a, stream) : launch_vec<1>(a, stream);
}

}  // namespace fa
