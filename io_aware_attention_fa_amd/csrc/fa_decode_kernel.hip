// Split-KV decode for gfx950: one query per (batch, head) against a KV cache of Tk keys.
//
// Decode reads the whole KV cache once and does little arithmetic per byte, so it is bound by
// HBM bandwidth; the sequence is split into chunks processed by independent workgroups, and a
// second pass merges the chunks (page "Fusion and IO-aware kernels", "Where it breaks": decode
// is dominated by reading the KV cache and is split across the sequence).  The merge is the
// rescale of the online-softmax recurrence (page "Kernels -- fusion and FlashAttention",
// section 3): every chunk's (max, denominator, output) is brought onto the common max by
// exp(m_s - m*) and summed.
//
// Split pass: grid (num_splits, h, B), 4 to 16 waves per workgroup (enough to cover a chunk in
// one pass).  A key row of d bf16 is read by d/8 lanes with 16-byte loads, so one wave-wide load
// covers 64*16 = 1 KB of consecutive key rows; each lane issues U K-loads and U V-loads before
// using any of them, so every wave keeps 2*U*1 KB of HBM reads in flight.  The loads are marked
// non-temporal: the cache is read once, and keeping it out of the caches' normal replacement made
// the split pass 7-9% faster.  Each lane keeps its own online-softmax state for the keys it sees;
// the states are merged across lanes and waves at the end with the same rescale.
//
// Combine pass: one 64-lane wave per (batch, head) reads the num_splits partials, rescales and
// writes O (bf16) and LSE (fp32).
//
// Workspace layout (fp32): o_s [B][h][S][d] followed by (m_s, l_s) [B][h][S][2]; m_s is in
// log2 units (scores * scale * log2 e) and o_s is unnormalised relative to m_s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* ws_o;    // [B][h][S][D]
  float* ws_ml;   // [B][h][S][2]
  uint16_t* o;
  float* lse;
  int H, Tk, S, chunk;
  float scale_log2;
  // general layouts (GEN variants): the true head dim d <= D (columns d .. D - 1 are zero
  // padding on chip) and element strides: q and o (batch, head), k and v (batch, head, row)
  int d;
  int64_t q_b, q_h, o_b, o_h, k_b, k_h, v_b, v_h;
  uint32_t k_t, v_t;
};

// A buffer offset beyond every head's range (heads are < 2^31 bytes): loads return zeros.
constexpr uint32_t kPadOffset = 0x80000000u;

// Merge the online-softmax state (m, l, o) of another lane / wave into this one.
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float (&o)[N], float m2, float l2,
                                            const float (&o2)[N]) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;   // both empty
  const float a = fast_exp2(m - mm), b = fast_exp2(m2 - mm);
  l = l * a + l2 * b;
#pragma unroll
  for (int j = 0; j < N; ++j) o[j] = o[j] * a + o2[j] * b;
  m = mm;
}

// GEN = false: contiguous tensors with d = D; GEN = true: the strides and d of DecodeParams.
// WAVES waves per workgroup (4, 8 or 16; the launch picks the fewest that cover a chunk in one
// pass where possible).
template <int D, bool GEN, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void fa_decode_split_kernel(DecodeParams p) {
  constexpr int LPK = D / 8;     // lanes per key row
  constexpr int KPW = 64 / LPK;  // key rows per wave-wide load
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane / LPK, c = lane % LPK;
  const int hd = GEN ? p.d : D;                       // true head dim
  const bool live = !GEN || 8 * c < hd;               // this lane's columns are not padding
  const uint32_t k_t = GEN ? p.k_t : D, v_t = GEN ? p.v_t : D;

  const size_t bh = (size_t)b * p.H + h;
  const int64_t kbase = GEN ? b * p.k_b + h * p.k_h : (int64_t)bh * p.Tk * D;
  const int64_t vbase = GEN ? b * p.v_b + h * p.v_h : (int64_t)bh * p.Tk * D;
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(p.k + kbase, ((uint32_t)(p.Tk - 1) * k_t + (uint32_t)hd) * 2u);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(p.v + vbase, ((uint32_t)(p.Tk - 1) * v_t + (uint32_t)hd) * 2u);
  // padding lanes load from past the buffers' ranges (zeros)
  const uint32_t kcol = live ? 16u * (uint32_t)c : kPadOffset;

  // this lane's 8 query components, pre-multiplied by scale * log2(e)
  float qv[8];
  {
    const int64_t qoff = GEN ? b * p.q_b + h * p.q_h : (int64_t)bh * D;
    u32x4_t qr = u32x4_t{0u, 0u, 0u, 0u};
    if (live) qr = *reinterpret_cast<const u32x4_t*>(p.q + qoff + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = bf16_elem(qr, e) * p.scale_log2;
  }

  const int k_begin = s * p.chunk;
  const int k_end = min(p.Tk, k_begin + p.chunk);

  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  constexpr int STEP = WAVES * KPW * kUnroll;   // keys per workgroup iteration
  for (int base = k_begin + wave * KPW * kUnroll; base < k_end; base += STEP) {
    u32x4_t kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = base + u * KPW + slot;
      kr[u] = buf_load16_nt(rk, (uint32_t)key * (k_t * 2u) + kcol);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = base + u * KPW + slot;
      vr[u] = buf_load16_nt(rv, (uint32_t)key * (v_t * 2u) + kcol);
    }
    float sc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(qv[e], bf16_elem(kr[u], e), acc);
      sc[u] = acc;
    }
    // sum the partial dot products over the LPK lanes of each key row
#pragma unroll
    for (int w = 1; w < LPK; w <<= 1)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) sc[u] += __shfl_xor(sc[u], w);
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (base + u * KPW + slot >= k_end) sc[u] = -INFINITY;
      mt = fmaxf(mt, sc[u]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new == -INFINITY) continue;   // nothing visible to this lane yet
    const float corr = fast_exp2(m - m_new);
    l *= corr;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= corr;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float pu = fast_exp2(sc[u] - m_new);
      l += pu;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(pu, bf16_elem(vr[u], e), o[e]);
    }
    m = m_new;
  }

  // merge the KPW key slots of the wave (lanes with equal c)
#pragma unroll
  for (int w = LPK; w < 64; w <<= 1) {
    float o2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[e], w);
    const float m2 = __shfl_xor(m, w), l2 = __shfl_xor(l, w);
    merge_state(m, l, o, m2, l2, o2);
  }

  // merge the waves through LDS
  __shared__ float sm_o[WAVES][D];
  __shared__ float sm_ml[WAVES][2];
  if (slot == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[wave][8 * c + e] = o[e];
    if (c == 0) {
      sm_ml[wave][0] = m;
      sm_ml[wave][1] = l;
    }
  }
  __syncthreads();
  if (tid < LPK) {
    float mw = sm_ml[0][0], lw = sm_ml[0][1], ow[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ow[e] = sm_o[0][8 * tid + e];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      float o2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o2[e] = sm_o[w][8 * tid + e];
      merge_state(mw, lw, ow, sm_ml[w][0], sm_ml[w][1], o2);
    }
    const size_t part = bh * p.S + s;
    float* dst = p.ws_o + part * D + 8 * tid;
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{ow[0], ow[1], ow[2], ow[3]};
    *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{ow[4], ow[5], ow[6], ow[7]};
    if (tid == 0) {
      p.ws_ml[part * 2 + 0] = mw;
      p.ws_ml[part * 2 + 1] = lw;
    }
  }
}

template <int D, bool GEN>
__global__ __launch_bounds__(kThreads) void fa_decode_combine_kernel(DecodeParams p, int BH) {
  constexpr int PER = D / 64;   // output elements per lane
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (bh >= BH) return;
  const float* ml = p.ws_ml + (size_t)bh * p.S * 2;
  float mstar = -INFINITY;
  for (int s = 0; s < p.S; ++s) mstar = fmaxf(mstar, ml[2 * s]);
  float l = 0.f, acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  for (int s = 0; s < p.S; ++s) {
    const float ms = ml[2 * s];
    if (ms == -INFINITY) continue;   // empty chunk
    const float w = fast_exp2(ms - mstar);
    l = fmaf(w, ml[2 * s + 1], l);
    const float* os = p.ws_o + ((size_t)bh * p.S + s) * D;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = fmaf(w, os[lane + 64 * j], acc[j]);
  }
  const float inv = 1.0f / l;
  int64_t obase = (int64_t)bh * D;
  if (GEN) {
    const int b = bh / p.H;
    obase = b * p.o_b + (bh - b * p.H) * p.o_h;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const __bf16 hv = (__bf16)(acc[j] * inv);
    if (!GEN || lane + 64 * j < p.d)
      p.o[obase + lane + 64 * j] = __builtin_bit_cast(uint16_t, hv);
  }
  if (lane == 0) p.lse[bh] = (mstar + fast_log2(l)) * kLn2;
}

template <int D, bool GEN>
hipError_t launch(const DecodeLaunch& a, hipStream_t stream) {
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  const size_t parts = (size_t)a.B * a.H * a.num_splits;
  p.ws_o = a.workspace;
  p.ws_ml = a.workspace + parts * D;
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.H = a.H;
  p.Tk = a.Tk;
  p.S = a.num_splits;
  p.chunk = (a.Tk + a.num_splits - 1) / a.num_splits;
  p.scale_log2 = a.scale * kLog2e;
  p.d = a.d;
  p.q_b = a.q_s[0]; p.q_h = a.q_s[1];
  p.o_b = a.o_s[0]; p.o_h = a.o_s[1];
  p.k_b = a.k_s[0]; p.k_h = a.k_s[1]; p.k_t = (uint32_t)a.k_s[2];
  p.v_b = a.v_s[0]; p.v_h = a.v_s[1]; p.v_t = (uint32_t)a.v_s[2];
  {
    // Workgroup size: enough waves to cover a chunk in one pass (each wave takes kUnroll loads
    // of 512 / D keys per pass), at least 4 and at most 16.  With the whole chunk's loads in
    // flight at once the split pass ran 5.5% faster at 512-key chunks and d = 128 (16 waves
    // against 4), and 1% faster at d = 64 (8 waves); 16 waves at d = 64, half of them idle,
    // ran 9% slower.
    constexpr int kKeysPerWave = (512 / D) * kUnroll;
    const int need = (p.chunk + kKeysPerWave - 1) / kKeysPerWave;
    const void* fn = need > 8   ? reinterpret_cast<const void*>(&fa_decode_split_kernel<D, GEN, 16>)
                     : need > 4 ? reinterpret_cast<const void*>(&fa_decode_split_kernel<D, GEN, 8>)
                                : reinterpret_cast<const void*>(&fa_decode_split_kernel<D, GEN, 4>);
    const int waves = need > 8 ? 16 : need > 4 ? 8 : 4;
    void* args[] = {&p};
    const hipError_t e =
        hipLaunchKernel(fn, dim3(a.num_splits, a.H, a.B), dim3(64 * waves), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  int BH = a.B * a.H;
  void* args[] = {&p, &BH};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa_decode_combine_kernel<D, GEN>),
                         dim3((BH + kWaves - 1) / kWaves), dim3(kThreads), args, 0, stream);
}

// GEN = false for contiguous tensors with d = D (64 or 128), else the general kernels.
template <int D>
hipError_t launch_d(const DecodeLaunch& a, hipStream_t stream) {
  const int64_t H = a.H, T = a.Tk;
  const bool dense = a.d == D && a.q_s[0] == H * D && a.q_s[1] == D && a.o_s[0] == H * D &&
                     a.o_s[1] == D && a.k_s[2] == D && a.k_s[1] == T * D &&
                     a.k_s[0] == H * T * D && a.v_s[2] == D && a.v_s[1] == T * D &&
                     a.v_s[0] == H * T * D;
  return dense ? launch<D, false>(a, stream) : launch<D, true>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream) {
  if (a.d <= 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace fa
