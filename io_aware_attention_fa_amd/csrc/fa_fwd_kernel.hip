// Attention forward (prefill) for gfx950: one workgroup per (128-row query block, head, batch).
//
// The method (page "Fusion and IO-aware kernels", "How it really works", FlashAttention steps
// 1-4; page "Kernels -- fusion and FlashAttention", sections 3-5): a block of query rows stays
// on chip, K/V tiles stream past it, and each query row keeps a running max m, a running
// denominator l and an fp32 output accumulator; after the last tile O = acc / l and
// LSE = m + ln l.  The score tile never leaves registers.
//
// MI355X mapping (our design, not the pages'):
//   * 4 waves x 32 query rows = 128 rows per workgroup; key tiles of 64 rows.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the Q
//     fragment is the B operand and lives in registers for the whole kernel, K is the A operand
//     read from LDS.  In the MFMA output layout every lane then owns ONE query row (lane % 32)
//     and 16 of the tile's keys per 32-key block, so the row max and row sum are in-lane
//     reductions plus one exchange with lane ^ 32.
//   * The P V contraction is also computed transposed, O^T += V^T P^T: P^T comes straight from
//     the score registers (rounded to bf16) as the B operand, V^T is the A operand read from
//     LDS.  For that, V is transposed while it is staged into LDS, with its key columns
//     permuted so that the 8 keys a lane holds in P are 8 adjacent LDS columns.
//   * The output accumulator (d x 32 rows per wave) stays in registers; the per-row rescale
//     by exp(m_old - m_new) is an in-lane multiply.
//   * exp is computed as exp2 with scale * log2(e) folded into one multiply-add per score.
//   * K/V tiles are double-buffered in LDS: the next tile's global loads are issued before the
//     current tile's math, and written to the other LDS buffer after it (one barrier per tile).
//   * Buffer loads with a per-head range return zeros past the end of Q/K/V, so ragged tails
//     need only the -inf score mask (page "Chapter 10 Writing and Benchmarking Custom
//     Kernels", section 10.3.1, "What You Actually Decide in Practice": the final partial tile).
//   * Causal: key tiles entirely above the diagonal are never loaded or computed; per wave,
//     tiles above that wave's rows are skipped; only tiles crossing the diagonal are masked.
//   * Workgroup -> (head, query block) order is XCD-aware (consecutive blocks of one head land
//     on one XCD, so its K/V stay in that XCD's L2) and, for causal, heaviest blocks first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kBM = 128;      // query rows per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kThreads = 256;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int Tq, Tk, nqb, total_wg;
  float scale_log2;
};

// Column of the V^T tile that holds key c (an involution): inside each group of 16 keys the
// 4-key blocks 1 and 2 swap places.  This makes LDS columns [16s + 8g, 16s + 8g + 8) hold
// exactly the keys that lane group g holds in registers 8*(s%2) .. 8*(s%2)+7 of the score
// block s/2 (MFMA output rows 8*(i/4) + 4g + (i%4)).
__host__ __device__ constexpr int vt_col(int c) {
  const int blk = (c >> 2) & 3;
  const int nb = blk == 1 ? 2 : (blk == 2 ? 1 : blk);
  return (c & ~15) | (nb << 2) | (c & 3);
}

template <int D>
struct Tile {
  static constexpr int KSTR = D + 8;           // bf16 per K row in LDS (16-byte pad)
  static constexpr int VSTR = kBN + 8;         // bf16 per V^T row in LDS (16-byte pad)
  static constexpr int KELEMS = kBN * KSTR;
  static constexpr int VELEMS = D * VSTR;
  static constexpr int STAGE = KELEMS + VELEMS;
  static constexpr int KCHUNKS = kBN * D / 8 / kThreads;   // 16-byte K chunks per thread
  static constexpr int VPAIRS = 16 * (D / 8);              // (4-key group, 8-d chunk) pairs
};

// Global -> registers for one K/V tile starting at key j0.
template <int D>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          int j0, int tid, u32x4_t (&kr)[Tile<D>::KCHUNKS],
                                          u32x4_t (&vr)[4]) {
#pragma unroll
  for (int it = 0; it < Tile<D>::KCHUNKS; ++it) {
    const int c = tid + kThreads * it;
    const int row = c / (D / 8), col8 = c % (D / 8);
    kr[it] = buf_load16(rk, (uint32_t)((j0 + row) * D + col8 * 8) * 2u);
  }
  if (tid < Tile<D>::VPAIRS) {
    const int kg = tid & 15, dc = tid >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vr[r] = buf_load16(rv, (uint32_t)((j0 + 4 * kg + r) * D + dc * 8) * 2u);
  }
}

// Registers -> LDS stage: K row-major, V transposed with permuted key columns.
template <int D>
__device__ __forceinline__ void store_tile(uint16_t* stage, int tid,
                                           const u32x4_t (&kr)[Tile<D>::KCHUNKS],
                                           const u32x4_t (&vr)[4]) {
  using T = Tile<D>;
#pragma unroll
  for (int it = 0; it < T::KCHUNKS; ++it) {
    const int c = tid + kThreads * it;
    const int row = c / (D / 8), col8 = c % (D / 8);
    *reinterpret_cast<u32x4_t*>(stage + row * T::KSTR + col8 * 8) = kr[it];
  }
  if (tid < T::VPAIRS) {
    const int kg = tid & 15, dc = tid >> 4;
    uint16_t* vt = stage + T::KELEMS + vt_col(4 * kg);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
      const int w = dd >> 1;
      u32x2_t pk;
      pk[0] = __builtin_amdgcn_perm(vr[1][w], vr[0][w], sel);   // keys 4kg, 4kg+1
      pk[1] = __builtin_amdgcn_perm(vr[3][w], vr[2][w], sel);   // keys 4kg+2, 4kg+3
      *reinterpret_cast<u32x2_t*>(vt + (dc * 8 + dd) * T::VSTR) = pk;
    }
  }
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_kernel(FwdParams p) {
  using T = Tile<D>;
  constexpr int NS = D / 16;   // k-steps of S^T = K Q^T
  constexpr int ND = D / 32;   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;

  // ---- workgroup -> (batch*head, query block) ----
  const int n = blockIdx.x;
  const int per = p.total_wg >> 3, rem = p.total_wg & 7, xcd = n & 7, loc = n >> 3;
  const int logical =
      xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int bh = logical / p.nqb;
  const int qr = logical - bh * p.nqb;
  const int qb = CAUSAL ? p.nqb - 1 - qr : qr;
  const int i0 = qb * kBM;
  const int off = p.Tk - p.Tq;   // query i sits at key position i + off (causal)

  const size_t qbase = (size_t)bh * (size_t)p.Tq * D;
  const size_t kbase = (size_t)bh * (size_t)p.Tk * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + qbase, (uint32_t)p.Tq * D * 2u);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + kbase, (uint32_t)p.Tk * D * 2u);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + kbase, (uint32_t)p.Tk * D * 2u);

  // ---- this wave's 32 query rows; Q fragment kept in registers ----
  const int qw0 = i0 + wave * 32;
  const int qrow = qw0 + r32;
  const int qw_last = min(qw0 + 31, p.Tq - 1);
  const bool wave_has_rows = qw0 < p.Tq;
  bf16x8_t qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = as_bf16x8(buf_load16(rq, (uint32_t)(qrow * D + 16 * s + 8 * g) * 2u));

  // keys the workgroup needs: all, or (causal) up to the block's last row
  int kend = p.Tk;
  if (CAUSAL) kend = min(p.Tk, min(i0 + kBM, p.Tq) + off);
  const int ntiles = (kend + kBN - 1) / kBN;

  float m_run = -INFINITY;   // running max, log2 units (scores * scale * log2 e)
  float l_run = 0.f;         // this lane's partial running denominator
  f32x16_t oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x16_t{};

  u32x4_t kr[T::KCHUNKS], vr[4];
  load_tile<D>(rk, rv, 0, tid, kr, vr);
  store_tile<D>(lds, tid, kr, vr);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kBN;
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_tile<D>(rk, rv, j0 + kBN, tid, kr, vr);

    const bool active = wave_has_rows && !(CAUSAL && j0 > qw_last + off);
    if (active) {
      const uint16_t* ks = lds + (t & 1) * T::STAGE;
      const uint16_t* vt = ks + T::KELEMS;

      // S^T block kb: keys j0 + 32kb + [0, 32) x this wave's 32 queries
      f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              ks + (32 * kb + r32) * T::KSTR + 16 * s + 8 * g);
          sacc[kb] = mfma_32x32x16(a, qf[s], sacc[kb]);
        }
      }

      // ---- online softmax for this lane's query row ----
      float x[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[kb * 16 + i] = sacc[kb][i] * p.scale_log2;

      const bool need_mask = (j0 + kBN > p.Tk) || (CAUSAL && j0 + kBN - 1 > qw0 + off);
      if (need_mask) {
        const int lim = CAUSAL ? min(p.Tk - 1, qrow + off) : p.Tk - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key > lim) x[kb * 16 + i] = -INFINITY;
          }
      }

      float mt = x[0];
#pragma unroll
      for (int i = 1; i < 32; ++i) mt = fmaxf(mt, x[i]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);   // finite: key 0 is visible to every row
      const float corr = fast_exp2(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        x[i] = fast_exp2(x[i] - m_new);
        psum += x[i];
      }
      l_run = l_run * corr + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= corr;

      // P^T as bf16 B operands: 16 keys per k-step, registers 8*(ks%2).. of score block ks/2
      bf16x8_t pb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int base = (ks >> 1) * 16 + (ks & 1) * 8;
        u32x4_t w;
        const u32x2_t lo = pack_bf16x4(x[base], x[base + 1], x[base + 2], x[base + 3]);
        const u32x2_t hi = pack_bf16x4(x[base + 4], x[base + 5], x[base + 6], x[base + 7]);
        w[0] = lo[0]; w[1] = lo[1]; w[2] = hi[0]; w[3] = hi[1];
        pb[ks] = as_bf16x8(w);
      }

      // O^T block db: d rows 32db + [0, 32) x this wave's 32 queries
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              vt + (32 * db + r32) * T::VSTR + 16 * ks + 8 * g);
          oacc[db] = mfma_32x32x16(a, pb[ks], oacc[db]);
        }
      }
    }

    if (has_next) store_tile<D>(lds + ((t + 1) & 1) * T::STAGE, tid, kr, vr);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2 ----
  if (!wave_has_rows) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow >= p.Tq) return;
  const float inv = 1.0f / l_tot;
  const size_t orow = qbase + (size_t)qrow * D;
#pragma unroll
  for (int db = 0; db < ND; ++db) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * db + 8 * i4 + 4 * g;
      const float a0 = oacc[db][4 * i4 + 0] * inv, a1 = oacc[db][4 * i4 + 1] * inv;
      const float a2 = oacc[db][4 * i4 + 2] * inv, a3 = oacc[db][4 * i4 + 3] * inv;
      if (OUT_F32) {
        f32x4_t f = {a0, a1, a2, a3};
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.o) + orow + d0) = f;
      } else {
        *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.o) + orow + d0) =
            pack_bf16x4(a0, a1, a2, a3);
      }
    }
  }
  if (g == 0) p.lse[(size_t)bh * p.Tq + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch(const FwdLaunch& a, hipStream_t stream) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.lse = a.lse;
  p.Tq = a.Tq;
  p.Tk = a.Tk;
  p.nqb = (a.Tq + kBM - 1) / kBM;
  p.total_wg = p.nqb * a.B * a.H;
  p.scale_log2 = a.scale * kLog2e;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_kernel<D, CAUSAL, OUT_F32>),
                         dim3(p.total_wg), dim3(kThreads), args, 0, stream);
}

template <int D>
hipError_t launch_d(const FwdLaunch& a, hipStream_t s) {
  if (a.causal) return a.out_f32 ? launch<D, true, true>(a, s) : launch<D, true, false>(a, s);
  return a.out_f32 ? launch<D, false, true>(a, s) : launch<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd(const FwdLaunch& a, hipStream_t stream) {
  if (a.d == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace fa
