// Attention backward for gfx950: dQ, dK and dV from Q, K, V, O, dO and the forward's LSE.
//
// The method (page "Chapter 10 Writing and Benchmarking Custom Kernels", section 10.3.2, the
// backward pass with recomputation; page "Kernels -- fusion and FlashAttention", the note that
// the backward recomputes attention from the saved statistics): the Tq x Tk probability matrix
// is never stored.  Tile by tile the scores S = scale Q K^T are recomputed and
// P = exp(S - LSE) is rebuilt from the stored log-sum-exp; with dP = dO V^T and the per-row
// scalar D_i = <dO_i, O_i>, the score gradient is dS = P (dP - D), and
//     dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K.
//
// MI355X mapping (our design, not the pages'): three kernels on the caller's stream.
//   * fa_bwd_prep: D_i and LSE_i * log2(e) per query row into the workspace (HBM-bound, one
//     pass over O and dO).
//   * fa_bwd_dkdv: one workgroup per (128-key block, head); each lane owns one key.  Q, dO and
//     the per-row L, D stream through LDS in 64-row tiles; K and V stay in registers as MFMA B
//     operands.  Per tile: S = Q K^T and dP = dO V^T (A operands: Q and dO rows from LDS),
//     then P and dS in the lane-per-key layout, then dV^T += dO^T P and dK^T += Q^T dS with
//     dO^T and Q^T read by the transposing LDS read (ds_read_b64_tr_b16) from the same
//     row-major tiles.  No atomics: every key's dK and dV are finished by one workgroup.
//   * fa_bwd_dq: one workgroup per (128-query block, head); each lane owns one query.  K and V
//     stream through LDS; S^T = K Q^T and dP^T = V dO^T with Q and dO in registers, then
//     dQ^T += K^T dS^T with K^T from the transposing read.  The two gradient kernels share no
//     partial sums, so the result is deterministic.
//   * A tile's 16-byte chunks are XOR-swizzled by row so that both the row reads (16 rows x one
//     chunk per 16 lanes) and the transposing reads (4 rows x 4 chunks per 32 lanes) hit
//     distinct LDS banks; tiles are filled by direct global-to-LDS loads, two tiles ahead.
//   * Ragged tails: buffer loads return zeros past the end of a head, so out-of-range rows
//     contribute nothing; out-of-range keys and causally hidden entries get P = 0.
//   * MFMA v_mfma_f32_32x32x16_bf16 throughout; P and dS are rounded to bf16 (round to nearest
//     even) as MFMA operands, every product accumulates in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"
#include "fa_lds.hpp"

namespace fa {
namespace {

constexpr int kRows = 64;     // rows of a streamed tile
constexpr int kStages = 4;    // LDS ring depth
constexpr int kOwn = 128;     // own rows (keys or queries) per workgroup
constexpr int kWaves = 4;     // one wave per SIMD, 32 own rows each
constexpr int kThreads = 64 * kWaves;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* l2;   // LSE_i * log2(e), [BH][Tq]
  const float* dd;   // D_i = <dO_i, O_i>, [BH][Tq]
  void* dq;
  void* dk;
  void* dv;
  int Tq, Tk, BH, nblk;   // nblk: 128-row own blocks per head
  int groups;             // 8: workgroup n works on heads n % 8, n % 8 + 8, ... (XCD-local)
  float c;                // scale * log2(e)
  float scale;
};

template <int D>
struct BTile {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int TILE = kRows * D;             // bf16 per tile
  static constexpr uint32_t BYTES = TILE * 2;
  static constexpr int ROWS_PER_LOAD = 64 / CH;      // rows one 64-lane 1 KB load covers
  static constexpr int LOADS = kRows / ROWS_PER_LOAD;
  static constexpr int LPW = LOADS / kWaves;         // 1 KB loads per wave per tile
  static_assert(LPW >= 1 && LOADS % kWaves == 0, "staging layout");
  // Row term of the chunk swizzle (physical chunk = logical chunk ^ f(r), an involution).
  // d = 128: a row is 256 bytes (all 64 banks); f takes 16 distinct values over rows 0..15
  // (row reads) and moves each of 4 consecutive rows to its own 64-byte quarter (transposing
  // reads).  d = 64: two rows share the banks; the same two properties hold per row pair.
  static __device__ __forceinline__ int f(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};

template <int D>
struct Lanes {
  // Per-lane byte offsets inside a tile (add the tile's LDS address; stages are 1 KB-aligned).
  //  Row operand (MFMA A operand from a row-major tile): tile row 32*blk + r32, logical chunk
  //  2*s + g; the swizzle makes this row_off ^ (32*s), plus blk * 32 rows.
  //  Transposed operand (A operand = tile^T, 32-column block db, k-step ks, half hf): lane l of
  //  16-lane group (g, dh) addresses row 16*ks + 8*hf + 4*g + (l % 16) / 4, column
  //  32*db + 16*dh + 4*(l % 4), and receives tile^T row 32*db + (l % 32) at rows
  //  16*ks + 8*hf + 4*g + 0..3.  The swizzle depends on the row through (l % 16) / 4, g and hf
  //  only, which makes this (tr_off ^ (64*db) ^ (32*hf)) + (16*ks + 8*hf) rows.
  uint32_t row_off, tr_off;
  uint32_t dma_l[BTile<D>::LPW], dma_g[BTile<D>::LPW];   // LDS / global offsets of loads
  __device__ __forceinline__ Lanes(int wave, int lane) {
    using T = BTile<D>;
    const int g = lane >> 5, r32 = lane & 31;
    row_off = 2u * (uint32_t)(r32 * D) + 16u * (uint32_t)(g ^ T::f(r32));
    const int x = (lane & 15) >> 2, dh = (lane >> 4) & 1, b = (lane & 3) >> 1;
    const int xr = D == 128 ? x : ((x >> 1) & 1);
    const int phys0 = (2 * dh + b) ^ (4 * xr + g);
    tr_off = 2u * (uint32_t)((4 * g + x) * D) + 16u * (uint32_t)phys0 + 8u * (uint32_t)(lane & 1);
#pragma unroll
    for (int i = 0; i < T::LPW; ++i) {
      // load n fills tile rows n*ROWS_PER_LOAD.. : lane l -> row + l / CH, physical chunk l % CH
      const int nld = wave * T::LPW + i;
      const int r = nld * T::ROWS_PER_LOAD + lane / T::CH, pc = lane % T::CH;
      dma_l[i] = (uint32_t)nld * 1024u;
      dma_g[i] = 2u * (uint32_t)(r * D + 8 * (pc ^ T::f(r)));
    }
  }
};

template <int D>
__device__ __forceinline__ bf16x8_t row_opnd(uint32_t at, int blk, int s) {
  return lds_read_bf16x8((at ^ (32u * (uint32_t)s)) + (uint32_t)blk * (32u * D * 2u));
}
template <int D>
__device__ __forceinline__ bf16x8_t tr_opnd(uint32_t at, int db, int ks) {
  const uint32_t a = at ^ (64u * (uint32_t)db);
  return lds_read_tr_pair(a + (uint32_t)(16 * ks) * (D * 2u),
                          (a ^ 32u) + (uint32_t)(16 * ks + 8) * (D * 2u));
}

// Stores 4 consecutive columns of one row (fp32 or rounded to bf16).
template <bool OUT_F32>
__device__ __forceinline__ void store4(void* base, size_t elem, float a, float b, float c,
                                       float d) {
  if (OUT_F32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(base) + elem) = f32x4_t{a, b, c, d};
  } else {
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(base) + elem) = pack_bf16x4(a, b, c, d);
  }
}

// Workgroup n -> (head, own block).  With groups == 8 the workgroups dispatched to one XCD
// (n % 8) take the blocks of heads n % 8, n % 8 + 8, ... in order, so the tiles a head streams
// are shared in that XCD's L2; `heavy_first_desc` reverses the block order within a head.
__device__ __forceinline__ void block_of(const BwdParams& p, bool heavy_last_blocks, int& bh,
                                         int& blk) {
  const int n = blockIdx.x;
  int hl, j;
  if (p.groups == 8) {
    const int x = n & 7, c = n >> 3;
    hl = c / p.nblk;
    j = c - hl * p.nblk;
    hl = x + 8 * hl;
  } else {
    hl = n / p.nblk;
    j = n - hl * p.nblk;
  }
  bh = __builtin_amdgcn_readfirstlane(hl);
  blk = __builtin_amdgcn_readfirstlane(heavy_last_blocks ? p.nblk - 1 - j : j);
}

// ---------------------------------------------------------------------------------------------
// Preprocess: D_i = <dO_i, O_i> (fp32 sum of bf16 products) and LSE_i * log2(e).
// One row per D/8 lanes (16 bytes each); rows = B * h * Tq.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                          const uint16_t* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ l2,
                                                          float* __restrict__ dd, int64_t rows) {
  constexpr int LPR = D / 8;   // lanes per row
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t e = (size_t)row * D + 8 * part;
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(o + e);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(dout + e);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[i]), as_bf16x2(b[i]), acc, false);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < rows && part == 0) {
    dd[row] = acc;
    l2[row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------------------------
// Software pipeline of the two gradient kernels.  The work on one streamed tile has three parts:
//   A: the score-side products (S and dP) of the tile, from row operands in LDS;
//   V: the elementwise part, P = exp2(S * scale * log2 e - L2), dS = P (dP - D), rounded to bf16;
//   C: the gradient products that consume P and dS, from transposed operands in LDS.
// Step s runs C of tile s - 1 with V of tile s scheduled between its MFMAs (one wave per SIMD:
// the vector instructions issue while the matrix core works), then A of tile s + 1.  V of tile s
// reads the score registers A filled in the previous step and writes the bf16 operands of the
// next step's C, which are handed over by register moves at the end of the step.  Every MFMA
// operand streams from LDS through a ring of kRing registers, each read issued kRing MFMAs ahead
// of its use.  Tiles go through a 4-stage LDS ring: at step s, tile s + 2 is requested into the
// stage tile s - 2 left (its last use, C of step s - 1, is behind the barrier that ended that
// step), and the step ends once it has landed.
constexpr int kRing = 8;

// A step's MFMA stream: NC C-part MFMAs (two transposing reads each), then NA A-part MFMAs (one
// LDS read each); VPM vector instructions are scheduled after each C-part MFMA (after each
// A-part MFMA when there is no C part), and the step issues XR extra LDS reads up front.
template <int NC, int NA, int VPM, int XR>
struct StepSeq {
  static constexpr int n = NC + NA;
  static constexpr __device__ int reads(int i) { return i < NC ? 2 : 1; }
  static constexpr __device__ int valu(int i) { return (NC > 0 ? i < NC : i < NA) ? VPM : 0; }
  static constexpr __device__ int initial_reads() {
    int r = XR;
    for (int i = 0; i < kRing && i < n; ++i) r += reads(i);
    return r;
  }
};

template <class S, int I>
__device__ __forceinline__ void sched_step() {
  if constexpr (I < S::n) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA I
    if constexpr (I + kRing < S::n)
      __builtin_amdgcn_sched_group_barrier(0x100, S::reads(I + kRing), 0);   // its ring refill
    if constexpr (S::valu(I) > 0) __builtin_amdgcn_sched_group_barrier(0x002, S::valu(I), 0);
    sched_step<S, I + 1>();
  }
}
template <class S>
__device__ __forceinline__ void sched_pattern() {
  if constexpr (S::initial_reads() > 0)
    __builtin_amdgcn_sched_group_barrier(0x100, S::initial_reads(), 0);
  sched_step<S, 0>();
}

// Packs registers 8*(ks%2) .. +7 of a 16-register MFMA result block into one bf16 B operand
// (RNE): the 16 streamed rows of k-step ks.
__device__ __forceinline__ bf16x8_t pack_kstep(const f32x16_t& x, int half) {
  const int b0 = 8 * half;
  const u32x2_t lo = pack_bf16x4(x[b0], x[b0 + 1], x[b0 + 2], x[b0 + 3]);
  const u32x2_t hi = pack_bf16x4(x[b0 + 4], x[b0 + 5], x[b0 + 6], x[b0 + 7]);
  return as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}

template <bool C, bool V, bool A, bool M>
struct Parts {
  static constexpr bool c = C, v = V, a = A, m = M;
};

// ---------------------------------------------------------------------------------------------
// dK, dV: one workgroup per (128-key block, head), lane = key.
template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkdv_kernel(BwdParams p) {
  using T = BTile<D>;
  constexpr int NS = D / 16;   // k-steps over d
  constexpr int ND = D / 32;   // 32-row blocks of dK^T / dV^T
  constexpr int NA = 4 * NS;   // S and dP MFMAs per tile
  constexpr int NC = 8 * ND;   // dV^T and dK^T MFMAs per tile
  // LDS: Q stages, dO stages, then 64 floats of L2 and of D per stage.
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * kStages * T::TILE];
  __shared__ __attribute__((aligned(256))) float lds_ld[2 * kStages * kRows];
  const uint32_t lq = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  const uint32_t ldo = lq + kStages * T::BYTES;
  const uint32_t ll = (uint32_t)reinterpret_cast<uintptr_t>(lds_ld);
  const uint32_t ld = ll + kStages * kRows * 4;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const Lanes<D> ln(wave, lane);

  int bh, blk;
  block_of(p, false, bh, blk);
  const int off = p.Tk - p.Tq;   // query i sits at key position i + off (causal)
  const int kw0 = blk * kOwn + wave * 32;   // this wave's first key
  const int key = kw0 + r32;
  // P is zeroed for queries below thr: keys past the end see nothing; causal keys see queries
  // from key - off on
  const int thr = key >= p.Tk ? INT32_MAX : (CAUSAL ? key - off : INT32_MIN);

  // K and V rows of this lane's key as B operands (k = 8 columns per lane half).
  bf16x8_t kf[NS], vf[NS];
  {
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(p.k + (size_t)bh * (size_t)p.Tk * D, (uint32_t)p.Tk * D * 2u);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(p.v + (size_t)bh * (size_t)p.Tk * D, (uint32_t)p.Tk * D * 2u);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t o = (uint32_t)(key * D + 16 * s + 8 * g) * 2u;
      kf[s] = as_bf16x8(buf_load16(rk, o));
      vf[s] = as_bf16x8(buf_load16(rv, o));
    }
  }

  // query tiles this block needs: from the first query that sees its first key
  const int nqt = (p.Tq + kRows - 1) / kRows;
  const int t0 = CAUSAL ? __builtin_amdgcn_readfirstlane(max(0, blk * kOwn - off) / kRows) : 0;
  const int nt = nqt - t0;

  const u32x4_t rq = rsrc_words(p.q + (size_t)bh * (size_t)p.Tq * D, (uint32_t)p.Tq * D * 2u);
  const u32x4_t rdo =
      rsrc_words(p.dout + (size_t)bh * (size_t)p.Tq * D, (uint32_t)p.Tq * D * 2u);
  const u32x4_t rl = rsrc_words(p.l2 + (size_t)bh * (size_t)p.Tq, (uint32_t)p.Tq * 4u);
  const u32x4_t rd = rsrc_words(p.dd + (size_t)bh * (size_t)p.Tq, (uint32_t)p.Tq * 4u);
  auto request = [&](int it) {   // tile t0 + it into stage it % kStages
    const int st = it & (kStages - 1);
    const uint32_t g0 = (uint32_t)(t0 + it) * (kRows * D * 2);
#pragma unroll
    for (int i = 0; i < T::LPW; ++i) {
      lds_dma16(rq, lq + st * T::BYTES + ln.dma_l[i], g0 + ln.dma_g[i]);
      lds_dma16(rdo, ldo + st * T::BYTES + ln.dma_l[i], g0 + ln.dma_g[i]);
    }
    // every wave writes the same 64 values of L2 and D (identical data, so the copies agree)
    const uint32_t r0 = (uint32_t)((t0 + it) * kRows + lane) * 4u;
    lds_dma4(rl, ll + st * (kRows * 4), r0);
    lds_dma4(rd, ld + st * (kRows * 4), r0);
  };

  f32x16_t accv[ND], acck[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    accv[db] = f32x16_t{};
    acck[db] = f32x16_t{};
  }
  f32x16_t sacc[2], dpacc[2];   // [32-query block]: S then P, dP then dS
  bf16x8_t pb[4], dsb[4];       // P and dS of the previous tile (C operands)
  bf16x8_t ring[kRing];

  // Step s (see the pipeline above).  In the MFMA result layout, register i of 32-query block
  // qb holds query 64*(t0 + s) + 32*qb + 8*(i/4) + 4*g + i%4 for key `key`.
  auto step = [&](auto parts, const int s) {
    using PT = decltype(parts);
    constexpr int nc = PT::c ? NC : 0, na = PT::a ? NA : 0;
    using S = StepSeq<nc, na, PT::v ? 7 : 0, PT::v ? 16 : 0>;
    if (s + 2 < nt) request(s + 2);
    const uint32_t qc = lq + ((s - 1) & 3) * T::BYTES + ln.tr_off;
    const uint32_t doc = ldo + ((s - 1) & 3) * T::BYTES + ln.tr_off;
    const uint32_t qa = lq + ((s + 1) & 3) * T::BYTES + ln.row_off;
    const uint32_t doa = ldo + ((s + 1) & 3) * T::BYTES + ln.row_off;
    auto opnd = [&](int i) -> bf16x8_t {
      if (i < nc) {
        const int r = i % (2 * ND);
        return tr_opnd<D>((r & 1) ? qc : doc, r >> 1, i / (2 * ND));
      }
      const int j = i - nc;
      return row_opnd<D>((j & 1) ? doa : qa, (j >> 1) & 1, j >> 2);
    };
#pragma unroll
    for (int i = 0; i < kRing && i < S::n; ++i) ring[i] = opnd(i);
    bf16x8_t pn[4], dsn[4];
    if constexpr (PT::v) {
      const uint32_t lo = ll + (s & 3) * (kRows * 4), dof = ld + (s & 3) * (kRows * 4);
      f32x4_t L4[2][4], D4[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const uint32_t o4 = 4u * (uint32_t)(32 * qb + 8 * a + 4 * g);
          L4[qb][a] = lds_read_f32x4(lo + o4);
          D4[qb][a] = lds_read_f32x4(dof + o4);
        }
      const int q0 = (t0 + s) * kRows + 4 * g;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int a = i >> 2, e = i & 3;
          float pv = fast_exp2(__builtin_fmaf(sacc[qb][i], p.c, -L4[qb][a][e]));
          if (q0 + 32 * qb + 8 * a + e < thr) pv = 0.f;
          sacc[qb][i] = pv;
          dpacc[qb][i] = pv * (dpacc[qb][i] - D4[qb][a][e]);
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        pn[ks] = pack_kstep(sacc[ks >> 1], ks & 1);
        dsn[ks] = pack_kstep(dpacc[ks >> 1], ks & 1);
      }
    }
#pragma unroll
    for (int i = 0; i < S::n; ++i) {
      const bf16x8_t a = ring[i % kRing];
      if (i + kRing < S::n) ring[i % kRing] = opnd(i + kRing);
      if (i < nc) {
        const int r = i % (2 * ND), ks = i / (2 * ND);
        if (r & 1)
          acck[r >> 1] = mfma_32x32x16(a, dsb[ks], acck[r >> 1]);
        else
          accv[r >> 1] = mfma_32x32x16(a, pb[ks], accv[r >> 1]);
      } else {
        const int j = i - nc, ss = j >> 2, qb = (j >> 1) & 1;
        const bool first = ss == 0;
        if (j & 1)
          dpacc[qb] = mfma_32x32x16(a, vf[ss], first ? f32x16_t{} : dpacc[qb]);
        else
          sacc[qb] = mfma_32x32x16(a, kf[ss], first ? f32x16_t{} : sacc[qb]);
      }
    }
    sched_pattern<S>();
    if constexpr (PT::v) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        pb[ks] = pn[ks];
        dsb[ks] = dsn[ks];
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // tile s + 2 has landed (this wave's part)
    __syncthreads();
  };

  request(0);
  if (nt > 1) request(1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  // steps -1 .. nt: A of tile 0; then C of s - 1, V of s, A of s + 1; then the last C
  step(Parts<false, false, true, false>{}, -1);
  if (nt > 1) {
    step(Parts<false, true, true, false>{}, 0);
    for (int s = 1; s + 1 < nt; ++s) step(Parts<true, true, true, false>{}, s);
    step(Parts<true, true, false, false>{}, nt - 1);
  } else {
    step(Parts<false, true, false, false>{}, 0);
  }
  step(Parts<true, false, false, false>{}, nt);

  // ---- epilogue: register i of block db is column 32*db + 8*(i/4) + 4*g + i%4 of row `key`
  if (key < p.Tk) {
    const size_t row = ((size_t)bh * (size_t)p.Tk + (size_t)key) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const size_t e = row + 32 * db + 8 * a + 4 * g;
        store4<OUT_F32>(p.dv, e, accv[db][4 * a], accv[db][4 * a + 1], accv[db][4 * a + 2],
                        accv[db][4 * a + 3]);
        store4<OUT_F32>(p.dk, e, p.scale * acck[db][4 * a], p.scale * acck[db][4 * a + 1],
                        p.scale * acck[db][4 * a + 2], p.scale * acck[db][4 * a + 3]);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// dQ: one workgroup per (128-query block, head), lane = query.
template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dq_kernel(BwdParams p) {
  using T = BTile<D>;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int NA = 4 * NS;   // S^T and dP^T MFMAs per tile
  constexpr int NC = 4 * ND;   // dQ^T MFMAs per tile
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * kStages * T::TILE];
  const uint32_t lk = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  const uint32_t lv = lk + kStages * T::BYTES;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const Lanes<D> ln(wave, lane);

  int bh, blk;
  block_of(p, CAUSAL, bh, blk);   // causal: the longest key ranges (last query blocks) first
  const int off = p.Tk - p.Tq;
  const int i0 = blk * kOwn;
  const int qw0 = i0 + wave * 32;
  const int qrow = qw0 + r32;
  // keys above lim get P = 0 (past the end, or above the diagonal)
  const int lim = CAUSAL ? min(p.Tk - 1, qrow + off) : p.Tk - 1;

  // Q and dO rows of this lane's query as B operands, and its L2 and D.
  bf16x8_t qf[NS], dof[NS];
  float l2q = 0.f, dq_d = 0.f;
  {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(p.q + (size_t)bh * (size_t)p.Tq * D, (uint32_t)p.Tq * D * 2u);
    const __amdgpu_buffer_rsrc_t rdo =
        make_rsrc(p.dout + (size_t)bh * (size_t)p.Tq * D, (uint32_t)p.Tq * D * 2u);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t o = (uint32_t)(qrow * D + 16 * s + 8 * g) * 2u;
      qf[s] = as_bf16x8(buf_load16(rq, o));
      dof[s] = as_bf16x8(buf_load16(rdo, o));
    }
    if (qrow < p.Tq) {
      l2q = p.l2[(size_t)bh * p.Tq + qrow];
      dq_d = p.dd[(size_t)bh * p.Tq + qrow];
    }
  }

  int kend = p.Tk;
  if (CAUSAL) kend = min(p.Tk, min(i0 + kOwn, p.Tq) + off);
  const int nt = __builtin_amdgcn_readfirstlane((kend + kRows - 1) / kRows);

  const u32x4_t rk = rsrc_words(p.k + (size_t)bh * (size_t)p.Tk * D, (uint32_t)p.Tk * D * 2u);
  const u32x4_t rv = rsrc_words(p.v + (size_t)bh * (size_t)p.Tk * D, (uint32_t)p.Tk * D * 2u);
  auto request = [&](int it) {
    const int st = it & (kStages - 1);
    const uint32_t g0 = (uint32_t)it * (kRows * D * 2);
#pragma unroll
    for (int i = 0; i < T::LPW; ++i) {
      lds_dma16(rk, lk + st * T::BYTES + ln.dma_l[i], g0 + ln.dma_g[i]);
      lds_dma16(rv, lv + st * T::BYTES + ln.dma_l[i], g0 + ln.dma_g[i]);
    }
  };

  f32x16_t accq[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) accq[db] = f32x16_t{};
  f32x16_t sacc[2], dpacc[2];   // [32-key block]: S^T, dP^T (then dS^T)
  bf16x8_t dsb[4], ring[kRing];

  // Step s.  Register i of 32-key block kb holds key 64*s + 32*kb + 8*(i/4) + 4*g + i%4 for
  // query `qrow`.
  auto step = [&](auto parts, const int s) {
    using PT = decltype(parts);
    constexpr int nc = PT::c ? NC : 0, na = PT::a ? NA : 0;
    using S = StepSeq<nc, na, PT::v ? (PT::m ? 12 : 8) : 0, 0>;
    if (s + 2 < nt) request(s + 2);
    const uint32_t kc = lk + ((s - 1) & 3) * T::BYTES + ln.tr_off;
    const uint32_t ka = lk + ((s + 1) & 3) * T::BYTES + ln.row_off;
    const uint32_t va = lv + ((s + 1) & 3) * T::BYTES + ln.row_off;
    auto opnd = [&](int i) -> bf16x8_t {
      if (i < nc) return tr_opnd<D>(kc, i % ND, i / ND);
      const int j = i - nc;
      return row_opnd<D>((j & 1) ? va : ka, (j >> 1) & 1, j >> 2);
    };
#pragma unroll
    for (int i = 0; i < kRing && i < S::n; ++i) ring[i] = opnd(i);
    bf16x8_t dsn[4];
    if constexpr (PT::v) {
      const int kj0 = s * kRows + 4 * g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = fast_exp2(__builtin_fmaf(sacc[kb][i], p.c, -l2q));
          if (PT::m && kj0 + 32 * kb + 8 * (i >> 2) + (i & 3) > lim) pv = 0.f;
          dpacc[kb][i] = pv * (dpacc[kb][i] - dq_d);
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) dsn[ks] = pack_kstep(dpacc[ks >> 1], ks & 1);
    }
#pragma unroll
    for (int i = 0; i < S::n; ++i) {
      const bf16x8_t a = ring[i % kRing];
      if (i + kRing < S::n) ring[i % kRing] = opnd(i + kRing);
      if (i < nc) {
        accq[i % ND] = mfma_32x32x16(a, dsb[i / ND], accq[i % ND]);
      } else {
        const int j = i - nc, ss = j >> 2, kb = (j >> 1) & 1;
        const bool first = ss == 0;
        if (j & 1)
          dpacc[kb] = mfma_32x32x16(a, dof[ss], first ? f32x16_t{} : dpacc[kb]);
        else
          sacc[kb] = mfma_32x32x16(a, qf[ss], first ? f32x16_t{} : sacc[kb]);
      }
    }
    sched_pattern<S>();
    if constexpr (PT::v) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) dsb[ks] = dsn[ks];
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  };
  // tile s needs masking for this wave if a key is past the end or above a query's diagonal
  auto need_mask = [&](int s) {
    return (s * kRows + kRows > p.Tk) || (CAUSAL && s * kRows + kRows - 1 > qw0 + off);
  };

  request(0);
  if (nt > 1) request(1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  step(Parts<false, false, true, false>{}, -1);
  if (nt > 1) {
    if (need_mask(0)) step(Parts<false, true, true, true>{}, 0);
    else step(Parts<false, true, true, false>{}, 0);
    for (int s = 1; s + 1 < nt; ++s) {
      if (need_mask(s)) step(Parts<true, true, true, true>{}, s);
      else step(Parts<true, true, true, false>{}, s);
    }
    step(Parts<true, true, false, true>{}, nt - 1);
  } else {
    step(Parts<false, true, false, true>{}, 0);
  }
  step(Parts<true, false, false, false>{}, nt);

  if (qrow < p.Tq) {
    const size_t row = ((size_t)bh * (size_t)p.Tq + (size_t)qrow) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        store4<OUT_F32>(p.dq, row + 32 * db + 8 * a + 4 * g, p.scale * accq[db][4 * a],
                        p.scale * accq[db][4 * a + 1], p.scale * accq[db][4 * a + 2],
                        p.scale * accq[db][4 * a + 3]);
  }
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch(const BwdLaunch& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.Tq;
  {
    constexpr int rows_per_block = 256 / (D / 8);
    const int64_t grid = (rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL(fa_bwd_prep_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout),
                       a.lse, a.l2, a.dd, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.l2 = a.l2;
  p.dd = a.dd;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.Tq = a.Tq;
  p.Tk = a.Tk;
  p.BH = a.B * a.H;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.groups = (p.BH % 8 == 0) ? 8 : 1;
  {
    p.nblk = (a.Tk + kOwn - 1) / kOwn;
    void* args[] = {&p};
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<D, CAUSAL, OUT_F32>),
                        dim3(p.BH * p.nblk), dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  {
    p.nblk = (a.Tq + kOwn - 1) / kOwn;
    void* args[] = {&p};
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void*>(&fa_bwd_dq_kernel<D, CAUSAL, OUT_F32>),
                        dim3(p.BH * p.nblk), dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_d(const BwdLaunch& a, hipStream_t s) {
  if (a.causal) return a.out_f32 ? launch<D, true, true>(a, s) : launch<D, true, false>(a, s);
  return a.out_f32 ? launch<D, false, true>(a, s) : launch<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_bwd(const BwdLaunch& a, hipStream_t stream) {
  if (a.d == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace fa
