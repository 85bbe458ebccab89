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
//     pass over O and dO); it also zeroes the dQ kernel's item counters.
//   * fa_bwd_dkdv: persistent workgroups of 8 waves, each running (128-key block, head) items
//     dealt as pairs of blocks with equal total work; each lane owns one key.
//     Q, dO and the per-row L, D stream through LDS in 32-row tiles; K and V stay in registers
//     as MFMA B operands.  The two waves on a SIMD own the same 32 keys and split the work: one
//     computes S = Q K^T, P and dV^T += dO^T P, the other dP = dO V^T, dS and dK^T += Q^T dS;
//     P goes from the first to the second through LDS.  dO^T and Q^T come from the transposing
//     LDS read (ds_read_b64_tr_b16) of the same row-major tiles.  No atomics: every key's dK
//     and dV are finished by one workgroup.
//   * fa_bwd_dq: persistent workgroups of 8 waves, each taking (256-query block, head) items
//     from XCD-local queues (an atomic counter each) until none is left; each lane owns one query.
//     K and V stream through LDS; S^T = K Q^T and dP^T = V dO^T with Q and dO in registers, then
//     dQ^T += K^T dS^T with K^T from the transposing read.  The two gradient kernels share no
//     partial sums, so the result is deterministic.
//   * A tile's 16-byte chunks are XOR-swizzled by row so that both the row reads (16 rows x one
//     chunk per 16 lanes) and the transposing reads (4 rows x 4 chunks per 32 lanes) hit
//     distinct LDS banks; tiles are filled by direct global-to-LDS loads into a ring of stages,
//     several tiles ahead.
//   * Both gradient kernels run two waves per SIMD (each wave's state fits in half of the SIMD's
//     registers), so one wave's LDS reads and vector work overlap the other's MFMAs; within a
//     wave, software pipelining schedules the exp / dS work of one tile between the MFMAs of the
//     gradient products of the tile before, and every MFMA operand streams from LDS through a
//     register ring.
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

constexpr int kOwnK = 128;    // dK/dV: keys per workgroup
constexpr int kWavesK = 8;    // dK/dV: four wave pairs, two waves per SIMD
constexpr int kThreadsK = 64 * kWavesK;
constexpr int kWavesQ = 8;    // dQ: two waves per SIMD, 32 own queries each
constexpr int kOwnQ = 32 * kWavesQ;
constexpr int kThreadsQ = 64 * kWavesQ;
constexpr int kQueues = 8;     // XCD groups of the persistent kernels; dQ's item queues
// the workspace reserves 1 KB for dQ's item counters, 64 bytes apart
static_assert(kQueues * 64 <= 1024, "counters exceed their workspace area");

// Layout of one [B][h][T][d] tensor: element (b, h, t, c) at base[b*sb + h*sh + t*st + c].
struct Lay {
  int64_t sb, sh;
  uint32_t st;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* l2;   // LSE_i * log2(e), [BH][Tq] (workspace)
  float* dd;   // -D_i = -<dO_i, O_i>, [BH][Tq] (workspace)
  void* dq;
  void* dk;
  void* dv;
  uint32_t* ctr;          // dQ's item counters (workspace, 64 B apart; the preprocess zeroes)
  int Tq, Tk, BH, nblk;   // nblk: own blocks (128 keys or 256 queries) per head
  int groups;             // XCD groups: group x works on heads x, x + groups, ...
  float c;                // scale * log2(e)
  float scale;
  // general layouts (used by the GEN variants): heads per batch entry, the true head dim
  // d <= D (columns d .. D - 1 are zero padding on chip) and each tensor's strides
  int H, d;
  Lay lq, lk, lv, lo, ldo, ldq, ldk, ldv;
};

// A buffer offset beyond every head's range (heads are < 2^31 bytes): loads return zeros.
constexpr uint32_t kPadOffset = 0x80000000u;

// Layout helpers: with GEN = false (contiguous, d = D) they reduce to compile-time strides.
template <int D, bool GEN>
__device__ __forceinline__ int64_t head_elem(const BwdParams& p, const Lay& l, int bh, int T) {
  if (!GEN) return (int64_t)bh * T * D;
  const int b = __builtin_amdgcn_readfirstlane(bh / p.H);
  return (int64_t)b * l.sb + (int64_t)(bh - b * p.H) * l.sh;
}
template <int D, bool GEN>
__device__ __forceinline__ uint32_t row_stride(const Lay& l) {
  return GEN ? l.st : (uint32_t)D;
}
// a head's byte range: rows 0 .. T - 1 of stride st, the last one d columns wide
__device__ __forceinline__ uint32_t head_bytes(int T, uint32_t st, int d) {
  return ((uint32_t)(T - 1) * st + (uint32_t)d) * 2u;
}
// byte offset of the 16 bytes at (row, col) of a head; padding columns read zeros
__device__ __forceinline__ uint32_t off16(int row, int col, uint32_t st, int d) {
  return col < d ? ((uint32_t)row * st + (uint32_t)col) * 2u : kPadOffset;
}

// A streamed tile of ROWS rows of D bf16 and how the W waves of a workgroup load it.
template <int D, int ROWS, int W>
struct BTile {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int TILE = ROWS * D;              // bf16 per tile
  static constexpr uint32_t BYTES = TILE * 2;
  static constexpr int ROWS_PER_LOAD = 64 / CH;      // rows one 64-lane 1 KB load covers
  static constexpr int LOADS = ROWS / ROWS_PER_LOAD;
  static constexpr int LPW = LOADS / W;              // 1 KB loads per wave per tile
  static_assert(LPW >= 1 && LOADS % W == 0, "staging layout");
  // Row term of the chunk swizzle (physical chunk = logical chunk ^ f(r), an involution).
  // d = 128: a row is 256 bytes (all 64 banks); f takes 16 distinct values over rows 0..15
  // (row reads) and moves each of 4 consecutive rows to its own 64-byte quarter (transposing
  // reads).  d = 64: two rows share the banks; the same two properties hold per row pair.
  static __device__ __forceinline__ int f(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};

// Per-lane byte offsets inside a tile (add the tile's LDS address; tiles are 1 KB-aligned).
//  Row operand (MFMA A operand from a row-major tile): tile row 32*blk + r32, logical chunk
//  2*s + g; the swizzle makes this row_off ^ (32*s), plus blk * 32 rows.
//  Transposed operand (A operand = tile^T, 32-column block db, k-step ks, half hf): lane l of
//  16-lane group (g, dh) addresses row 16*ks + 8*hf + 4*g + (l % 16) / 4, column
//  32*db + 16*dh + 4*(l % 4), and receives tile^T row 32*db + (l % 32) at rows
//  16*ks + 8*hf + 4*g + 0..3.  The swizzle depends on the row through (l % 16) / 4, g and hf
//  only, which makes this (tr_off ^ (64*db) ^ (32*hf)) + (16*ks + 8*hf) rows.
template <int D, int ROWS, int W>
struct Lanes {
  using T = BTile<D, ROWS, W>;
  uint32_t row_off, tr_off;
  uint32_t dma_l[T::LPW];   // LDS byte offsets of this wave's loads
  int w_, l_;
  __device__ __forceinline__ Lanes(int wave, int lane) : w_(wave), l_(lane) {
    const int g = lane >> 5, r32 = lane & 31;
    row_off = 2u * (uint32_t)(r32 * D) + 16u * (uint32_t)(g ^ T::f(r32));
    const int x = (lane & 15) >> 2, dh = (lane >> 4) & 1, b = (lane & 3) >> 1;
    const int xr = D == 128 ? x : ((x >> 1) & 1);
    const int phys0 = (2 * dh + b) ^ (4 * xr + g);
    tr_off = 2u * (uint32_t)((4 * g + x) * D) + 16u * (uint32_t)phys0 + 8u * (uint32_t)(lane & 1);
#pragma unroll
    for (int i = 0; i < T::LPW; ++i) dma_l[i] = (uint32_t)(wave * T::LPW + i) * 1024u;
  }
  // Global byte offset (within a tile of rows of stride st, d real columns) of load i: load n
  // fills tile rows n*ROWS_PER_LOAD.. : lane l -> row + l / CH, physical chunk l % CH, which
  // holds the logical chunk the swizzle maps there.
  __device__ __forceinline__ uint32_t goff(int i, uint32_t st, int d) const {
    const int nld = w_ * T::LPW + i;
    const int r = nld * T::ROWS_PER_LOAD + l_ / T::CH, c = (l_ % T::CH) ^ T::f(r);
    return 8 * c < d ? 2u * ((uint32_t)r * st + 8u * (uint32_t)c) : kPadOffset;
  }
};

// Per-lane LDS addresses of one region (a ring of tiles at `base`): the row operand of k-step s
// and the transposed operand halves of column block db are base + row[s] and base + tr[db][hf];
// the stage, the 32-row block and the k-step add byte offsets that are compile-time constants,
// which the LDS instructions take as immediates.
template <int D>
struct Region {
  static constexpr uint32_t kRowBlock = 32u * D * 2u;   // bytes of 32 tile rows
  uint32_t row[D / 16], tr[D / 32][2];
  __device__ __forceinline__ Region(uint32_t base, uint32_t row_off, uint32_t tr_off) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      row[s] = base + (row_off ^ (32u * (uint32_t)s));
      // opaque to the optimiser: a base above 64 KB would otherwise be folded into per-stage
      // addresses (beyond the 16-bit LDS immediate) that are kept in registers
      asm volatile("" : "+v"(row[s]));
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        tr[db][hf] = base + (tr_off ^ (64u * (uint32_t)db) ^ (32u * (uint32_t)hf));
        asm volatile("" : "+v"(tr[db][hf]));
      }
  }
  // A operand: rows 32*blk + (lane % 32), k-step s, of the tile at byte offset so
  __device__ __forceinline__ bf16x8_t row_opnd(uint32_t so, int blk, int s) const {
    return lds_read_bf16x8(row[s] + so + (uint32_t)blk * kRowBlock);
  }
  // A operand = tile^T: rows 32*db + (lane % 32), k-step ks (16 tile rows)
  __device__ __forceinline__ bf16x8_t tr_opnd(uint32_t so, int db, int ks) const {
    return lds_read_tr_pair(tr[db][0] + so + (uint32_t)(16 * ks) * (D * 2u),
                            tr[db][1] + so + (uint32_t)(16 * ks + 8) * (D * 2u));
  }
};

template <int ST>
using Stage = std::integral_constant<int, ST>;

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

// Stores a wave's 32 x D block of results as bf16: register i of acc[db] holds column
// 32 db + 8 (i / 4) + 4 g + i % 4 of row row0 + l31 (l31 = lane % 32, g = lane / 32), scaled by
// sc.  The rows pass through the wave's own 32 (2D + 16) bytes of LDS at ew (idle once the last
// step's barrier has passed) so that each store writes whole rows, 16 bytes per lane, instead of
// 16 bytes in each of 32 rows; the 16-byte skew per row keeps both the 8-byte writes and the
// 16-byte reads free of bank conflicts.  Rows from nrows on and columns from hd on are dropped
// by the buffer range (rd covers the head, rs is its row stride in elements).
template <int D, bool GEN>
__device__ __forceinline__ void store_rows_bf16(const f32x16_t (&acc)[D / 32], float sc,
                                                uint32_t ew, int l31, int g, int row0, int nrows,
                                                __amdgpu_buffer_rsrc_t rd, uint32_t rs, int hd) {
  constexpr uint32_t RS = 2 * D + 16;
  constexpr int LPR = D / 8;      // lanes per row
  constexpr int RPP = 64 / LPR;   // rows per store
  const uint32_t wr = ew + (uint32_t)l31 * RS + 8u * (uint32_t)g;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      lds_write_u32x2(wr + 2u * (uint32_t)(32 * db + 8 * a),
                      pack_bf16x4(sc * acc[db][4 * a], sc * acc[db][4 * a + 1],
                                  sc * acc[db][4 * a + 2], sc * acc[db][4 * a + 3]));
  const int ln = l31 | (g << 5);
  const int rr = ln / LPR, cc = 8 * (ln % LPR);
#pragma unroll
  for (int i = 0; i < 32 / RPP; ++i) {
    const int r = RPP * i + rr;
    const u32x4_t v = lds_read_u32x4(ew + (uint32_t)r * RS + 2u * (uint32_t)cc);
    const bool ok = row0 + r < nrows && (!GEN || cc < hd);
    const uint32_t off = ok ? 2u * ((uint32_t)(row0 + r) * rs + (uint32_t)cc) : kPadOffset;
    __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, 0);
  }
}

// Persistent schedule of the dK/dV kernel: at most one workgroup per CU, each running several
// (head, key block) items one after the other, so that a CU starts its next block without a new
// workgroup's dispatch (which cost about as much as 15-20 of its pipeline steps).  Blocks are
// paired as (nblk - 1 - j, j): under the causal mask block j sees Tq - 128 j queries, so the costs
// of a pair add up to the same total for every j and dealing pairs round-robin balances the CUs.
// With groups == 8 workgroup n belongs to group n % 8 (the XCD it is dispatched to) and takes the
// pairs of heads n % 8, n % 8 + 8, ..., so the tiles a head streams are shared in that XCD's L2.
// body(bh, blk, tid) runs one item with tid, the thread index, rebuilt per item from the wave
// index (a scalar) and the lane's position in the wave, which an opaque instruction pair computes
// inside the loop: every lane-dependent value of an item is then computed inside it, so the
// compiler neither hoists such values out of the item loop nor keeps them live across an item
// (the kernel's steady state fills the registers).  The barrier between items lets the next item's loads reuse the LDS.
template <class F>
__device__ __forceinline__ void for_each_block(const BwdParams& p, F&& body) {
  const int wave0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  for (int u = 0;; ++u) {
    const int X = p.groups, n = blockIdx.x;
    const int x = n % X, c = n / X;
    const int C = ((int)gridDim.x - x + X - 1) / X;   // workgroups of group x
    const int np = (p.nblk + 1) / 2;                   // block pairs per head
    const int PX = ((p.BH - x + X - 1) / X) * np;      // pairs of group x
    const int pp = c + (u >> 1) * C;
    if (pp >= PX) break;
    const int hl = pp / np, j = pp - hl * np;
    const int blk = (u & 1) ? j : p.nblk - 1 - j;
    if ((u & 1) && blk == p.nblk - 1 - j) continue;   // the middle block of an odd count
    if (u > 0) __syncthreads();
    int ml;   // the lane's position, computed here (the builtins' result would be hoisted)
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ml));
    const int tid = wave0 * 64 + ml;
    body(__builtin_amdgcn_readfirstlane(x + X * hl), __builtin_amdgcn_readfirstlane(blk), tid);
  }
}

// Persistent schedule of the dQ kernel: at most one workgroup per CU, each taking (head, query
// block) items from shared queues until none is left, so that no CU idles while items remain
// (a fixed deal ends with the slowest XCD; the XCDs of one device differ in speed by several
// percent).  Queue x < groups holds the items of heads x, x + groups, ... head by head, nblk per
// head, and counter x (ctr[16 x], 64 bytes apart; the preprocess zeroes them) counts the items
// taken.  Workgroup n takes from queue n % groups (with groups == 8, the queue of the XCD it is
// dispatched to: the workgroups working on a head at one time share its streamed tiles in their
// L2) and, once that queue is empty, from the others in turn.  With REV a head's blocks are
// taken from the last one, which under the causal mask sees the most keys, so the items left at
// the end are the short ones.  (The dK/dV kernel keeps the fixed deal of pairs above: taken from
// queues its items ran 2-3% slower.)

// Items of queue x.
__device__ __forceinline__ int queue_items(const BwdParams& p, int x) {
  return ((p.BH - x + p.groups - 1) / p.groups) * p.nblk;
}

// Completes taking an item (one lane): k0 is what the counter of queue x0 returned.  If that
// queue is empty, takes from the others in turn.  x = the item's queue (-1: none left), k = its
// index there.
__device__ __forceinline__ void take_item(const BwdParams& p, uint32_t* ctr, int x0, int k0,
                                          int& x, int& k) {
  x = x0;
  k = k0;
  if (k < queue_items(p, x)) return;
  for (int q = 1; q < p.groups; ++q) {
    x = x0 + q;
    if (x >= p.groups) x -= p.groups;
    k = (int)atomicAdd(ctr + 16 * x, 1u);
    if (k < queue_items(p, x)) return;
  }
  x = -1;
}

// Runs body(bh, blk, tid, claim, publish) for every item this workgroup takes.  One lane (lane 0
// of wave 0) takes items; the item is passed to the waves through a two-int LDS slot.  The body
// calls claim() as its last step ends and publish(c) after its stores (the counter's atomic
// completes during the stores; every wave read the slot at the item's start).  Taking the next
// item only then keeps the items a queue's workgroups run at one time contiguous in the queue,
// so they share their heads' tiles in L2: taken one item ahead (at an item's start), the short
// blocks of a head ran long after its long ones and fetched 2.6 times the bytes.  tid is the thread index, rebuilt
// per item as in for_each_block.  The barrier between items lets the next item's loads reuse
// the LDS.
template <bool REV, class F>
__device__ __forceinline__ void for_each_item(const BwdParams& p, uint32_t* ctr, int* slot,
                                              F&& body) {
  const int wave0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int x0 = (int)blockIdx.x % p.groups;
  auto lane_pos = []() {
    int ml;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ml));
    return ml;
  };
  auto claim = [&]() -> int {
    int k0 = 0;
    if (wave0 == 0 && lane_pos() == 0) k0 = (int)atomicAdd(ctr + 16 * x0, 1u);
    return k0;
  };
  auto publish = [&](int k0) {
    if (wave0 == 0 && lane_pos() == 0) {
      int x, k;
      take_item(p, ctr, x0, k0, x, k);
      slot[0] = x;
      slot[1] = k;
    }
  };
  publish(claim());
  __syncthreads();
  for (;;) {
    const int x = __builtin_amdgcn_readfirstlane(slot[0]);
    if (x < 0) break;
    const int k = __builtin_amdgcn_readfirstlane(slot[1]);
    const int hl = k / p.nblk, r = k - hl * p.nblk;
    body(__builtin_amdgcn_readfirstlane(x + p.groups * hl),
         __builtin_amdgcn_readfirstlane(REV ? p.nblk - 1 - r : r), wave0 * 64 + lane_pos(), claim,
         publish);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// Preprocess: -D_i = -<dO_i, O_i> (fp32 sum of bf16 products) and LSE_i * log2(e).
// One row per D/8 lanes (16 bytes each); rows = B * h * Tq.
template <int D, bool GEN>
__global__ __launch_bounds__(256) void fa_bwd_prep_kernel(BwdParams p, int64_t rows) {
  constexpr int LPR = D / 8;   // lanes per row
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    int64_t eo, ed;
    if (!GEN) {
      eo = ed = row * D + 8 * part;
    } else {
      const int bh = (int)(row / p.Tq), t = (int)(row - (int64_t)bh * p.Tq), b = bh / p.H;
      const int hh = bh - b * p.H;
      eo = b * p.lo.sb + hh * p.lo.sh + (int64_t)t * p.lo.st + 8 * part;
      ed = b * p.ldo.sb + hh * p.ldo.sh + (int64_t)t * p.ldo.st + 8 * part;
    }
    if (!GEN || 8 * part < p.d) {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p.o + eo);
      const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p.dout + ed);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[i]), as_bf16x2(b[i]), acc, false);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < rows && part == 0) {
    p.dd[row] = -acc;
    p.l2[row] = p.lse[row] * kLog2e;
  }
  if (blockIdx.x == 0 && threadIdx.x < kQueues) p.ctr[16 * threadIdx.x] = 0u;
}

// ---------------------------------------------------------------------------------------------
// Software pipeline of the two gradient kernels.  The work on one streamed tile has three parts:
//   A: the score-side products (S and dP) of the tile, from row operands in LDS;
//   V: the elementwise part, P = exp2(S * scale * log2 e - L2), dS = P (dP - D), rounded to bf16;
//   C: the gradient products that consume P and dS, from transposed operands in LDS.
// A wave's step s runs C of an earlier tile with V of a later one between its MFMAs (the vector
// instructions issue while the matrix core works; the dQ kernel runs V first, having too few
// registers for V's values and a deep operand ring at once), then A of the next tile; V reads
// the score registers that A filled in the step before.  (dQ: C of tile s - 1, V of s, A of
// s + 1; the two roles of the dK/dV kernel are listed there.)  The bf16 operands that V makes
// for C are double-buffered by tile parity.  Every MFMA operand streams from LDS through a ring
// of registers, each read issued as many MFMAs ahead of its use as the ring holds; where the
// next step starts with a C part the ring runs across steps: the last MFMAs of step s read the
// first operands of step s + 1 (resident tiles) before the barrier that ends the step.  Tiles
// are loaded AHEAD steps ahead into a ring of NST stages; the stage of every step is a
// compile-time constant (the steady state is a chain of the NST stage variants, left after the
// last step), so that all LDS addresses are per-lane registers plus immediates.  The last steps
// run the V part (and, in the dK/dV kernel, the A part) on stages holding stale tiles and produce
// values that are never used; the dQ kernel skips its A part there behind one wave-uniform
// branch (the same branch in the dK/dV roles measured no faster, and in role V it spills).

// A step's MFMA stream: NC C-part MFMAs, then NA A-part MFMAs, with RING operands in flight.
// The stream is issued in program order (a scheduling barrier after each MFMA): left to itself
// the scheduler moved each operand read next to its MFMA, exposing the LDS latency once per
// MFMA, and ran the V part's vector work apart from the MFMAs.
template <int NC, int NA, int RING>
struct StepSeq {
  static constexpr int n = NC + NA;
  static_assert(n % RING == 0, "the ring restarts at slot 0 every step");
};

// Packs registers 8*half .. +7 of a 16-register MFMA result block into one bf16 B operand
// (RNE): the 16 streamed rows of one k-step.
__device__ __forceinline__ bf16x8_t pack_kstep(const f32x16_t& x, int half) {
  const int b0 = 8 * half;
  const u32x2_t lo = pack_bf16x4(x[b0], x[b0 + 1], x[b0 + 2], x[b0 + 3]);
  const u32x2_t hi = pack_bf16x4(x[b0 + 4], x[b0 + 5], x[b0 + 6], x[b0 + 7]);
  return as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}

// Parts of a step: C (gradient products of tile s - 1), V (elementwise part of tile s),
// A (score products of tile s + 1), M (V applies the mask).
template <bool C, bool V, bool A, bool M>
struct Parts {
  static constexpr bool c = C, v = V, a = A, m = M;
};

// Waits until this wave's loads of tile `need` have landed, when tiles up to `last` have been
// requested (each tile is `per` vector-memory operations; they complete in issue order).
template <int PER, int AHEAD>
__device__ __forceinline__ void wait_tile(int need, int last) {
  const int after = min(AHEAD, max(0, last - need));
  static_assert(AHEAD <= 2, "wait_tile handles up to two later tiles");
  if (after >= 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER));
  else if (after == 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---------------------------------------------------------------------------------------------
// dK, dV: 8 waves per (128-key block, head) item, lane = key; query tiles of 32 rows.
// Waves w and w + 4 (which share a SIMD) own the same 32 keys and split the work: wave w (role K)
// holds the K rows and computes S, P and dV; wave w + 4 (role V) holds the V rows and computes
// dP - D, dS and dK.  P goes from role K to role V through LDS (fp32, double-buffered by tile
// parity).  Each role holds half of a key block's state, so two waves fit per SIMD and one's LDS
// reads and vector work overlap the other's MFMAs.
//   role K, step s: dV += dO^T P of tile s - 1, with P of tile s (from S, computed in the step
//     before) scheduled between its MFMAs and stored to LDS; then S of tile s + 1.
//   role V, step s: dK += Q^T dS of tile s - 2, with dS of tile s - 1 (P from role K, dP - D
//     from the step before) scheduled between its MFMAs; then dP - D of tile s (the accumulator
//     starts from -D).
// Both roles end every step at the same barrier, which publishes P; role V runs one step behind
// role K, so both run steps -1 .. nt + 1 (role K's last one is empty).
template <int D, bool CAUSAL, bool OUT_F32, bool GEN>
__global__ __launch_bounds__(kThreadsK) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(BwdParams p) {
  constexpr int R = 32;        // query rows per streamed tile (one 32-row MFMA block)
  constexpr int NST = 6;       // LDS stages: tiles s - 2 .. s + 1 in use, two in flight
  constexpr int AHEAD = 3;     // step s requests tile s + AHEAD
  constexpr int kRing = 4;     // MFMA operands in flight
  constexpr int NS = D / 16;   // k-steps over d
  constexpr int ND = D / 32;   // 32-row blocks of dK^T / dV^T
  constexpr int NA = NS;       // S (or dP) MFMAs per tile
  constexpr int NC = 2 * ND;   // dV^T (or dK^T) MFMAs per tile (two 16-query k-steps)
  // Staging: every wave issues the same number of 1 KB loads per tile.  d = 128: each wave loads
  // one piece of Q and one of dO; d = 64 (four pieces per tile): waves 0-3 load Q, 4-7 load dO.
  constexpr bool SPLIT = BTile<D, R, 4>::LOADS < kWavesK;
  using T = BTile<D, R, SPLIT ? 4 : kWavesK>;
  constexpr int LDS_LD = 64;   // floats of L2 (or of -D) per stage (one 64-lane load)
  constexpr uint32_t PF = 16u * 64u * 4u;   // P of one tile and wave pair: 4 x 64 lanes x 16 B
  // LDS: Q stages, dO stages, L2 and -D per stage, then P [pair][parity].
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * NST * T::TILE];
  __shared__ __attribute__((aligned(1024))) float lds_p[4 * 2 * PF / 4];
  __shared__ __attribute__((aligned(256))) float lds_ld[2 * NST * LDS_LD];
  for_each_block(p, [&](const int bh, const int blk, const int tid) {
  const uint32_t lq = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  const uint32_t ldo = lq + NST * T::BYTES;
    const uint32_t ll = (uint32_t)reinterpret_cast<uintptr_t>(lds_ld);
    const uint32_t ld = ll + NST * LDS_LD * 4;

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pr = wave & 3;     // wave pair
    const bool role_k = wave < 4;
    const int g = lane >> 5;
    const Lanes<D, R, SPLIT ? 4 : kWavesK> ln(SPLIT ? pr : wave, lane);
    // this lane's slot of the pair's P buffers (parity and part add immediates)
    const uint32_t pfb =
        (uint32_t)reinterpret_cast<uintptr_t>(lds_p) + (uint32_t)pr * (2 * PF) + 16u * lane;

    const int off = p.Tk - p.Tq;   // query i sits at key position i + off (causal)
    const int key = blk * kOwnK + pr * 32 + (lane & 31);

    // query tiles this block needs: from the first query that sees its first key
    const int nqt = (p.Tq + R - 1) / R;
    const int t0 = CAUSAL ? __builtin_amdgcn_readfirstlane(max(0, blk * kOwnK - off) / R) : 0;
    const int nt = nqt - t0;

    const int hd = GEN ? p.d : D;   // true head dim
    const uint32_t st_q = row_stride<D, GEN>(p.lq), st_do = row_stride<D, GEN>(p.ldo);
    const u32x4_t rq = rsrc_words(p.q + head_elem<D, GEN>(p, p.lq, bh, p.Tq),
                                  head_bytes(p.Tq, st_q, hd));
    const u32x4_t rdo = rsrc_words(p.dout + head_elem<D, GEN>(p, p.ldo, bh, p.Tq),
                                   head_bytes(p.Tq, st_do, hd));
    uint32_t gq[T::LPW], gdo[T::LPW];   // this wave's global load offsets within a tile
  #pragma unroll
    for (int i = 0; i < T::LPW; ++i) {
      gq[i] = ln.goff(i, st_q, hd);
      gdo[i] = ln.goff(i, st_do, hd);
    }
    // role K stages L2 (for P), role V stages -D (the dP seed); four identical copies each
    const u32x4_t rld = role_k ? rsrc_words(p.l2 + (size_t)bh * (size_t)p.Tq, (uint32_t)p.Tq * 4u)
                               : rsrc_words(p.dd + (size_t)bh * (size_t)p.Tq, (uint32_t)p.Tq * 4u);
    const uint32_t lld = role_k ? ll : ld;
    auto request = [&](int it) {   // tile t0 + it into stage it % NST
      const int st = it % NST;
      const uint32_t g0q = (uint32_t)(t0 + it) * (R * 2u) * st_q;
      const uint32_t g0d = (uint32_t)(t0 + it) * (R * 2u) * st_do;
  #pragma unroll
      for (int i = 0; i < T::LPW; ++i) {
        if (SPLIT) {
          lds_dma16(role_k ? rq : rdo, (role_k ? lq : ldo) + st * T::BYTES + ln.dma_l[i],
                    role_k ? g0q + gq[i] : g0d + gdo[i]);
        } else {
          lds_dma16(rq, lq + st * T::BYTES + ln.dma_l[i], g0q + gq[i]);
          lds_dma16(rdo, ldo + st * T::BYTES + ln.dma_l[i], g0d + gdo[i]);
        }
      }
      // 64 values from the tile's first row on (the tile uses the first 32)
      lds_dma4(rld, lld + st * (LDS_LD * 4), (uint32_t)((t0 + it) * R + lane) * 4u);
    };
    constexpr int PER = (SPLIT ? 1 : 2) * T::LPW + 1;   // vector-memory operations per tile

    // K (role K) or V (role V) rows of this lane's key as B operands (k = 8 columns per half).
    bf16x8_t kvf[NS];
    {
      const uint16_t* src = role_k ? p.k : p.v;
      const Lay& lkv = role_k ? p.lk : p.lv;
      const uint32_t st = row_stride<D, GEN>(lkv);
      const __amdgpu_buffer_rsrc_t rkv =
          make_rsrc(src + head_elem<D, GEN>(p, lkv, bh, p.Tk), head_bytes(p.Tk, st, hd));
  #pragma unroll
      for (int s = 0; s < NS; ++s)
        kvf[s] = as_bf16x8(buf_load16(rkv, off16(key, 16 * s + 8 * g, st, hd)));
    }

    for (int it = 0; it < AHEAD - 1 && it < nt; ++it) request(it);
    wait_tile<PER, AHEAD - 2>(1, min(AHEAD - 2, nt - 1));   // tiles 0 and 1 (and the K/V rows)
    __syncthreads();

    f32x16_t acc[ND];   // dV^T (role K) or dK^T (role V)
  #pragma unroll
    for (int db = 0; db < ND; ++db) acc[db] = f32x16_t{};
    bf16x8_t ring[kRing];
    const Region<D> rQ(lq, ln.row_off, ln.tr_off), rO(ldo, ln.row_off, ln.tr_off);

    if (role_k) {
      // ------------------------------- role K -------------------------------
      // P is zeroed for queries below thr: keys past the end see nothing; causal keys see
      // queries from key - off on.  thr4: thr relative to the first query this lane holds.
      const int thr4 = key >= p.Tk ? (1 << 30) : (CAUSAL ? key - off - 4 * g : -(1 << 30));
      // Tiles from s_free on need no mask (wave-uniform): no key of this wave is past the end,
      // and the tile starts at or below the diagonal of this wave's last key.
      const int kw0 = blk * kOwnK + pr * 32;
      int s_free = 0;
      if (kw0 + 31 >= p.Tk) {
        s_free = INT32_MAX;
      } else if (CAUSAL) {
        const int x = kw0 + 31 - off;   // the first query that sees every key of this wave
        s_free = x <= 0 ? 0 : (x + R - 1) / R - t0;
      }
      f32x16_t sacc;         // S of the next tile (32 queries x this key)
      bf16x8_t pb[2][2];     // [tile parity][k-step]: P as C-part operands
      auto step = [&](auto parts, auto stage, int s) {
        using PT = decltype(parts);
        constexpr int ST = decltype(stage)::value;
        constexpr int nc = PT::c ? NC : 0, na = PT::a ? NA : 0;
        constexpr bool next = PT::v;   // the next step (if any) starts with a C part
        using S = StepSeq<nc, na, kRing>;
        constexpr uint32_t so_c = ((ST + NST - 1) % NST) * T::BYTES;   // tile s - 1
        constexpr uint32_t so_v = ST * T::BYTES;                       // tile s
        constexpr uint32_t so_a = ((ST + 1) % NST) * T::BYTES;         // tile s + 1
        constexpr int PC = (ST + 1) & 1, PV = ST & 1;                  // parities (NST is even)
        asm volatile("" : "+s"(s));
        if (s + AHEAD < nt) request(s + AHEAD);
        auto c_opnd = [&](uint32_t so, int i) -> bf16x8_t {
          return rO.tr_opnd(so, i % ND, i / ND);
        };
        auto opnd = [&](int i) -> bf16x8_t {
          if (i < nc) return c_opnd(so_c, i);
          return rQ.row_opnd(so_a, 0, i - nc);
        };
        if constexpr (!PT::c) {
  #pragma unroll
          for (int i = 0; i < kRing && i < S::n; ++i) ring[i] = opnd(i);
        }
        // V part (P of tile s from its scores) in 8 chunks of two scores each
        f32x4_t L4[4];
        int lt = 0;
        if constexpr (PT::v) {
  #pragma unroll
          for (int a = 0; a < 4; ++a)
            L4[a] = lds_read_f32x4(ll + ST * (LDS_LD * 4) + 4u * (uint32_t)(8 * a + 4 * g));
          lt = thr4 - (t0 + s) * R;
        }
        auto vchunk = [&](int c) {
  #pragma unroll
          for (int i = 2 * c; i < 2 * c + 2; ++i) {
            const int a = i >> 2, e = i & 3;
            float pv = fast_exp2(__builtin_fmaf(sacc[i], p.c, -L4[a][e]));
            if (PT::m && 8 * a + e < lt) pv = 0.f;
            sacc[i] = pv;
          }
          if (c & 1) {
            const int a = c >> 1;
            lds_write_f32x4(pfb + PV * PF + 1024u * a,
                            f32x4_t{sacc[4 * a], sacc[4 * a + 1], sacc[4 * a + 2],
                                    sacc[4 * a + 3]});
          }
          if (c == 3) pb[PV][0] = pack_kstep(sacc, 0);
          if (c == 7) pb[PV][1] = pack_kstep(sacc, 1);
        };
        if constexpr (PT::v && !PT::c) {
  #pragma unroll
          for (int c = 0; c < 8; ++c) vchunk(c);
        }
        // MFMAs in program order (pinned by scheduling barriers): operand i + kRing is read
        // while MFMA i runs, and the V part's chunks follow the C-part MFMAs, which do not
        // depend on it (the A part overwrites the scores it reads, so it comes last).
  #pragma unroll
        for (int i = 0; i < S::n; ++i) {
          const bf16x8_t a = ring[i % kRing];
          if (i + kRing < S::n)
            ring[i % kRing] = opnd(i + kRing);
          else if (next)
            ring[i % kRing] = c_opnd(so_v, i + kRing - S::n);
          if (i < nc) {
            acc[i % ND] = mfma_32x32x16(a, pb[PC][i / ND], acc[i % ND]);
          } else {
            const int j = i - nc;
            sacc = mfma_32x32x16(a, kvf[j], j == 0 ? f32x16_t{} : sacc);
          }
          if constexpr (PT::v && PT::c) {
            if (i < nc) {
  #pragma unroll
              for (int c = i * 8 / nc; c < (i + 1) * 8 / nc; ++c) vchunk(c);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // the next step reads tile s + 2 (role K's S)
        wait_tile<PER, AHEAD - 2>(s + 2, min(s + AHEAD, nt - 1));
        __syncthreads();
      };
      step(Parts<false, false, true, true>{}, Stage<NST - 1>{}, -1);
      step(Parts<false, true, true, true>{}, Stage<0>{}, 0);
      {
        // steps 1 .. nt: whole chains of the NST stage variants with the mask while a chain may
        // hold a tile that needs it, then chains without (each chain left after step nt)
        int s = 1;
        auto chain = [&](auto parts) {
          step(parts, Stage<1>{}, s); if (++s > nt) return true;
          step(parts, Stage<2>{}, s); if (++s > nt) return true;
          step(parts, Stage<3>{}, s); if (++s > nt) return true;
          step(parts, Stage<4>{}, s); if (++s > nt) return true;
          step(parts, Stage<5>{}, s); if (++s > nt) return true;
          step(parts, Stage<0>{}, s); if (++s > nt) return true;
          return false;
        };
        bool fin = false;
        while (!fin && s < s_free) fin = chain(Parts<true, true, true, true>{});
        while (!fin) fin = chain(Parts<true, true, true, false>{});
      }
      step(Parts<false, false, false, false>{}, Stage<0>{}, nt + 1);   // role V's last step
    } else {
      // ------------------------------- role V -------------------------------
      // (fewer live registers than role K: a deeper operand ring at d = 128)
      constexpr int kRingV = D == 128 ? 8 : kRing;
      bf16x8_t ringv[kRingV];
      f32x16_t dpacc;        // dP - D of tile s (kept for the dS of the next step)
      bf16x8_t dsb[2][2];    // [tile parity][k-step]: dS as C-part operands
      auto step = [&](auto parts, auto stage, int s) {
        using PT = decltype(parts);
        constexpr int ST = decltype(stage)::value;
        constexpr int nc = PT::c ? NC : 0, na = PT::a ? NA : 0;
        constexpr bool next = PT::v;   // the next step (if any) starts with a C part
        using S = StepSeq<nc, na, kRingV>;
        constexpr uint32_t so_c = ((ST + NST - 2) % NST) * T::BYTES;   // tile s - 2
        constexpr uint32_t so_n = ((ST + NST - 1) % NST) * T::BYTES;   // tile s - 1
        constexpr uint32_t so_a = ST * T::BYTES;                       // tile s
        constexpr int PC = ST & 1, PV = (ST + 1) & 1;   // parities of tiles s - 2 and s - 1
        asm volatile("" : "+s"(s));
        if (s + AHEAD < nt) request(s + AHEAD);
        auto c_opnd = [&](uint32_t so, int i) -> bf16x8_t {
          return rQ.tr_opnd(so, i % ND, i / ND);
        };
        auto opnd = [&](int i) -> bf16x8_t {
          if (i < nc) return c_opnd(so_c, i);
          return rO.row_opnd(so_a, 0, i - nc);
        };
        if constexpr (!PT::c) {
  #pragma unroll
          for (int i = 0; i < kRingV && i < S::n; ++i) ringv[i] = opnd(i);
        }
        // V part: dS of tile s - 1 (P from role K times dP - D), in 8 chunks of two scores
        f32x4_t P4[4];
        f32x16_t ds;
        if constexpr (PT::v) {
  #pragma unroll
          for (int a = 0; a < 4; ++a) P4[a] = lds_read_f32x4(pfb + PV * PF + 1024u * a);
        }
        auto vchunk = [&](int c) {
  #pragma unroll
          for (int i = 2 * c; i < 2 * c + 2; ++i) ds[i] = P4[i >> 2][i & 3] * dpacc[i];
          if (c == 3) dsb[PV][0] = pack_kstep(ds, 0);
          if (c == 7) dsb[PV][1] = pack_kstep(ds, 1);
        };
        if constexpr (PT::v && !PT::c) {
  #pragma unroll
          for (int c = 0; c < 8; ++c) vchunk(c);
        }
        // the dP accumulator starts from -D of the tile's rows
        f32x16_t nd0;
        if constexpr (PT::a) {
  #pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4_t v4 =
                lds_read_f32x4(ld + ST * (LDS_LD * 4) + 4u * (uint32_t)(8 * a + 4 * g));
  #pragma unroll
            for (int e = 0; e < 4; ++e) nd0[4 * a + e] = v4[e];
          }
        }
  #pragma unroll
        for (int i = 0; i < S::n; ++i) {
          const bf16x8_t a = ringv[i % kRingV];
          if (i + kRingV < S::n)
            ringv[i % kRingV] = opnd(i + kRingV);
          else if (next)
            ringv[i % kRingV] = c_opnd(so_n, i + kRingV - S::n);
          if (i < nc) {
            acc[i % ND] = mfma_32x32x16(a, dsb[PC][i / ND], acc[i % ND]);
          } else {
            const int j = i - nc;
            dpacc = mfma_32x32x16(a, kvf[j], j == 0 ? nd0 : dpacc);
          }
          if constexpr (PT::v && PT::c) {
            if (i < nc) {
  #pragma unroll
              for (int c = i * 8 / nc; c < (i + 1) * 8 / nc; ++c) vchunk(c);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        wait_tile<PER, AHEAD - 2>(s + 2, min(s + AHEAD, nt - 1));
        __syncthreads();
      };
      step(Parts<false, false, false, false>{}, Stage<NST - 1>{}, -1);
      step(Parts<false, false, true, false>{}, Stage<0>{}, 0);
      step(Parts<false, true, true, false>{}, Stage<1>{}, 1);
      {
        using P = Parts<true, true, true, false>;
        int s = 2;
        for (;;) {
          step(P{}, Stage<2>{}, s); if (++s > nt + 1) break;
          step(P{}, Stage<3>{}, s); if (++s > nt + 1) break;
          step(P{}, Stage<4>{}, s); if (++s > nt + 1) break;
          step(P{}, Stage<5>{}, s); if (++s > nt + 1) break;
          step(P{}, Stage<0>{}, s); if (++s > nt + 1) break;
          step(P{}, Stage<1>{}, s); if (++s > nt + 1) break;
        }
      }
    }

    // ---- epilogue: register i of block db is column 32*db + 8*(i/4) + 4*g + i%4 of row `key`
    const Lay& lg = role_k ? p.ldv : p.ldk;
    const float sc = role_k ? 1.f : p.scale;
    if constexpr (OUT_F32) {
      if (key < p.Tk) {
        const size_t row = (size_t)(head_elem<D, GEN>(p, lg, bh, p.Tk) +
                                    (int64_t)key * row_stride<D, GEN>(lg));
        void* dst = role_k ? p.dv : p.dk;
  #pragma unroll
        for (int db = 0; db < ND; ++db)
  #pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int col = 32 * db + 8 * a + 4 * g;
            if (!GEN || col < hd)
              store4<OUT_F32>(dst, row + col, sc * acc[db][4 * a], sc * acc[db][4 * a + 1],
                              sc * acc[db][4 * a + 2], sc * acc[db][4 * a + 3]);
          }
      }
    } else {
      // the lane's row is key % 32 (key and g stay live through the steps; lane does not)
      static_assert(kWavesK * 32 * (2 * D + 16) <= sizeof(lds), "rows exceed the stage area");
      const int key0 = key - (key & 31);
      const uint32_t rs = row_stride<D, GEN>(lg);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(
          static_cast<uint16_t*>(role_k ? p.dv : p.dk) + head_elem<D, GEN>(p, lg, bh, p.Tk),
          head_bytes(p.Tk, rs, hd));
      store_rows_bf16<D, GEN>(acc, sc, lq + (uint32_t)wave * (32u * (2 * D + 16)), key & 31, g,
                              key0, p.Tk, rd, rs, hd);
    }
  });
}

// ---------------------------------------------------------------------------------------------
// dQ: 8 waves (two per SIMD) per (256-query block, head) item; lane = query; key tiles of 32
// rows (d = 128) or 64 rows (d = 64).  The per-wave state fits in half of a SIMD's
// registers, so the two waves of a SIMD overlap one's LDS reads and vector work with the
// other's MFMAs.
template <int D, bool CAUSAL, bool OUT_F32, bool GEN>
__global__ __launch_bounds__(kThreadsQ) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(BwdParams p) {
  constexpr int R = D == 128 ? 32 : 64;   // keys per streamed tile
  constexpr int KB = R / 32;              // 32-key MFMA blocks per tile
  constexpr int NK = R / 16;              // 16-key k-steps of the dQ product per tile
  constexpr int NST = 8;                  // LDS stages
  constexpr int AHEAD = 4;                // step s requests tile s + AHEAD
  constexpr int kRing = 2;                // MFMA operands in flight (4 would spill)
  using T = BTile<D, R, kWavesQ>;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int NA = 2 * KB * NS;   // S^T and dP^T MFMAs per tile
  constexpr int NC = ND * NK;       // dQ^T MFMAs per tile
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * NST * T::TILE];
  const uint32_t lk = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  const uint32_t lv = lk + NST * T::BYTES;

  __shared__ int slot[2];
  // causal: a head's last query blocks (the longest key ranges) first
  for_each_item<CAUSAL>(p, p.ctr, slot, [&](const int bh, const int blk, const int tid,
                                            auto&& claim, auto&& publish) {
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const Lanes<D, R, kWavesQ> ln(wave, lane);

    const int off = p.Tk - p.Tq;
    const int i0 = blk * kOwnQ;
    const int qw0 = i0 + wave * 32;
    const int qrow = qw0 + (lane & 31);
    // keys above lim get P = 0 (past the end, or above the diagonal); lim4 is lim relative to the
    // first key this lane holds in a tile
    const int lim = CAUSAL ? min(p.Tk - 1, qrow + off) : p.Tk - 1;
    const int lim4 = lim - 4 * g;
    // Tiles before s_mask need no mask (wave-uniform): their last key is within the limit of
    // this wave's first query.
    const int lim_w = CAUSAL ? min(p.Tk - 1, qw0 + off) : p.Tk - 1;
    const int s_mask = (lim_w + 1) / R;

    // Q and dO rows of this lane's query as B operands, and its L2 and -D.
    const int hd = GEN ? p.d : D;   // true head dim
    bf16x8_t qf[NS], dof[NS];
    float l2q = 0.f, ndq = 0.f;
    {
      const uint32_t st_q = row_stride<D, GEN>(p.lq), st_do = row_stride<D, GEN>(p.ldo);
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + head_elem<D, GEN>(p, p.lq, bh, p.Tq),
                                                  head_bytes(p.Tq, st_q, hd));
      const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + head_elem<D, GEN>(p, p.ldo, bh, p.Tq),
                                                   head_bytes(p.Tq, st_do, hd));
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        qf[s] = as_bf16x8(buf_load16(rq, off16(qrow, 16 * s + 8 * g, st_q, hd)));
        dof[s] = as_bf16x8(buf_load16(rdo, off16(qrow, 16 * s + 8 * g, st_do, hd)));
      }
      if (qrow < p.Tq) {
        l2q = p.l2[(size_t)bh * p.Tq + qrow];
        ndq = p.dd[(size_t)bh * p.Tq + qrow];
      }
    }

    int kend = p.Tk;
    if (CAUSAL) kend = min(p.Tk, min(i0 + kOwnQ, p.Tq) + off);
    const int nt = __builtin_amdgcn_readfirstlane((kend + R - 1) / R);

    const uint32_t st_k = row_stride<D, GEN>(p.lk), st_v = row_stride<D, GEN>(p.lv);
    const u32x4_t rk = rsrc_words(p.k + head_elem<D, GEN>(p, p.lk, bh, p.Tk),
                                  head_bytes(p.Tk, st_k, hd));
    const u32x4_t rv = rsrc_words(p.v + head_elem<D, GEN>(p, p.lv, bh, p.Tk),
                                  head_bytes(p.Tk, st_v, hd));
    uint32_t gk[T::LPW], gv[T::LPW];   // this wave's global load offsets within a tile
#pragma unroll
    for (int i = 0; i < T::LPW; ++i) {
      gk[i] = ln.goff(i, st_k, hd);
      gv[i] = ln.goff(i, st_v, hd);
    }
    auto request = [&](int it) {
      const int st = it & (NST - 1);
      const uint32_t g0k = (uint32_t)it * (R * 2u) * st_k, g0v = (uint32_t)it * (R * 2u) * st_v;
#pragma unroll
      for (int i = 0; i < T::LPW; ++i) {
        lds_dma16(rk, lk + st * T::BYTES + ln.dma_l[i], g0k + gk[i]);
        lds_dma16(rv, lv + st * T::BYTES + ln.dma_l[i], g0v + gv[i]);
      }
    };
    constexpr int PER = 2 * T::LPW;

    f32x16_t accq[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) accq[db] = f32x16_t{};
    f32x16_t sacc[KB], dpacc[KB];   // [32-key block]: S^T, dP^T (then dS^T)
    bf16x8_t dsb[2][NK];            // [tile parity][k-step]: dS^T as C operands
    bf16x8_t ring[kRing];
    const Region<D> rK(lk, ln.row_off, ln.tr_off), rV(lv, ln.row_off, ln.tr_off);

    // Step s with stage ST = s % NST.  Register i of 32-key block kb holds key
    // R*s + 32*kb + 8*(i/4) + 4*g + i%4 for query `qrow`.
    auto step = [&](auto parts, auto stage, int s) {
      using PT = decltype(parts);
      constexpr int ST = decltype(stage)::value;
      constexpr int nc = PT::c ? NC : 0, na = PT::a ? NA : 0;
      constexpr bool next = PT::v;
      using S = StepSeq<nc, na, kRing>;
      // s as an opaque scalar: otherwise the optimiser keeps a per-lane copy of each value derived
      // from it for every stage variant of the chain
      asm volatile("" : "+s"(s));
      constexpr uint32_t so_c = ((ST + NST - 1) % NST) * T::BYTES;
      constexpr uint32_t so_v = ST * T::BYTES;
      constexpr uint32_t so_a = ((ST + 1) % NST) * T::BYTES;
      constexpr int PC = (ST + 1) & 1, PV = ST & 1;
      if (s + AHEAD < nt) request(s + AHEAD);
      auto c_opnd = [&](uint32_t so, int i) -> bf16x8_t { return rK.tr_opnd(so, i % ND, i / ND); };
      auto opnd = [&](int i) -> bf16x8_t {
        if (i < nc) return c_opnd(so_c, i);
        const int j = i - nc;
        return ((j & 1) ? rV : rK).row_opnd(so_a, (j >> 1) % KB, (j >> 1) / KB);
      };
      if constexpr (!PT::c) {
#pragma unroll
        for (int i = 0; i < kRing && i < S::n; ++i) ring[i] = opnd(i);
      }
      // V part (dS of tile s from its scores), in 8 chunks of 2 KB scores; k-step ks of dS is
      // packed once the chunk holding its last score is done
      const int lt = lim4 - s * R;   // lim relative to the tile's first key
      auto vchunk = [&](int c) {
        constexpr int PERC = 2 * KB;
#pragma unroll
        for (int f = c * PERC; f < (c + 1) * PERC; ++f) {
          const int kb = f >> 4, i = f & 15;
          float pv = fast_exp2(__builtin_fmaf(sacc[kb][i], p.c, -l2q));
          if (PT::m && 32 * kb + 8 * (i >> 2) + (i & 3) > lt) pv = 0.f;
          dpacc[kb][i] = pv * (dpacc[kb][i] + ndq);
        }
#pragma unroll
        for (int ks = 0; ks < NK; ++ks)
          if ((8 * ks + 7) / PERC == c) dsb[PV][ks] = pack_kstep(dpacc[ks >> 1], ks & 1);
      };
      if constexpr (PT::v) {
#pragma unroll
        for (int c = 0; c < 8; ++c) vchunk(c);
      }
      // MFMAs in program order (pinned by scheduling barriers): operand i + kRing is read while
      // MFMA i runs, and the V part's chunks follow the C-part MFMAs, which do not depend on it
      // (the A part overwrites the scores it reads, so it comes last).  The MFMA parts run at
      // raised issue priority, so that on a SIMD the wave past its V part keeps the matrix core
      // fed while the other still issues its vector work (about 1% faster per backward call).
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < nc; ++i) {
        const bf16x8_t a = ring[i % kRing];
        if (i + kRing < S::n)
          ring[i % kRing] = opnd(i + kRing);
        else if (next)
          ring[i % kRing] = c_opnd(so_v, i + kRing - S::n);
        accq[i % ND] = mfma_32x32x16(a, dsb[PC][i / ND], accq[i % ND]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // The A part's tile s + 1 exists only for s + 1 < nt: the last two steps skip it (one
      // wave-uniform branch) and only read the next step's first operands.
      if (s + 1 < nt) {
#pragma unroll
        for (int i = nc; i < S::n; ++i) {
          const bf16x8_t a = ring[i % kRing];
          if (i + kRing < S::n)
            ring[i % kRing] = opnd(i + kRing);
          else if (next)
            ring[i % kRing] = c_opnd(so_v, i + kRing - S::n);
          const int j = i - nc, ss = (j >> 1) / KB, kb = (j >> 1) % KB;
          if (j & 1)
            dpacc[kb] = mfma_32x32x16(a, dof[ss], ss == 0 ? f32x16_t{} : dpacc[kb]);
          else
            sacc[kb] = mfma_32x32x16(a, qf[ss], ss == 0 ? f32x16_t{} : sacc[kb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else if constexpr (next) {
#pragma unroll
        for (int i = (nc > S::n - kRing ? nc : S::n - kRing); i < S::n; ++i)
          ring[i % kRing] = c_opnd(so_v, i + kRing - S::n);
      }
      __builtin_amdgcn_s_setprio(0);
      wait_tile<PER, AHEAD - 2>(s + 2, min(s + AHEAD, nt - 1));
      __syncthreads();
    };
    for (int it = 0; it < AHEAD - 1 && it < nt; ++it) request(it);
    wait_tile<PER, AHEAD - 2>(1, min(AHEAD - 2, nt - 1));
    __syncthreads();
    step(Parts<false, false, true, true>{}, Stage<NST - 1>{}, -1);
    step(Parts<false, true, true, true>{}, Stage<0>{}, 0);
    // steps 1 .. nt: a chain of the NST stage variants, left after step nt; each step in a masked
    // or an unmasked variant (the mask costs two vector instructions per score)
    {
      // whole chains of the NST stage variants without the mask while every step of a chain is
      // before s_mask, then chains with it (each chain left after step nt)
      int s = 1;
      auto chain = [&](auto parts) {
        step(parts, Stage<1>{}, s); if (++s > nt) return true;
        step(parts, Stage<2>{}, s); if (++s > nt) return true;
        step(parts, Stage<3>{}, s); if (++s > nt) return true;
        step(parts, Stage<4>{}, s); if (++s > nt) return true;
        step(parts, Stage<5>{}, s); if (++s > nt) return true;
        step(parts, Stage<6>{}, s); if (++s > nt) return true;
        step(parts, Stage<7>{}, s); if (++s > nt) return true;
        step(parts, Stage<0>{}, s); if (++s > nt) return true;
        return false;
      };
      bool fin = false;
      while (!fin && s + NST <= s_mask) fin = chain(Parts<true, true, true, false>{});
      while (!fin) fin = chain(Parts<true, true, true, true>{});
    }

    const int next = claim();   // the next item, taken as this one ends
    if constexpr (OUT_F32 || GEN) {   // (through LDS the strided variant spills in its steps)
      if (qrow < p.Tq) {
        const size_t row = (size_t)(head_elem<D, GEN>(p, p.ldq, bh, p.Tq) +
                                    (int64_t)qrow * row_stride<D, GEN>(p.ldq));
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int col = 32 * db + 8 * a + 4 * g;
            if (!GEN || col < hd)
              store4<OUT_F32>(p.dq, row + col, p.scale * accq[db][4 * a],
                              p.scale * accq[db][4 * a + 1], p.scale * accq[db][4 * a + 2],
                              p.scale * accq[db][4 * a + 3]);
          }
      }
    } else {
      static_assert(kWavesQ * 32 * (2 * D + 16) <= sizeof(lds), "dQ rows exceed the stage area");
      const uint32_t rs = row_stride<D, GEN>(p.ldq);
      const __amdgpu_buffer_rsrc_t rd =
          make_rsrc(static_cast<uint16_t*>(p.dq) + head_elem<D, GEN>(p, p.ldq, bh, p.Tq),
                    head_bytes(p.Tq, rs, hd));
      store_rows_bf16<D, GEN>(accq, p.scale, lk + (uint32_t)wave * (32u * (2 * D + 16)),
                              lane & 31, g, qw0, p.Tq, rd, rs, hd);
    }
    publish(next);
  });
}

Lay to_lay(const int64_t* s3) { return Lay{s3[0], s3[1], (uint32_t)s3[2]}; }

template <int D, bool CAUSAL, bool OUT_F32, bool GEN>
hipError_t launch(const BwdLaunch& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<const uint16_t*>(a.o);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
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
  p.ctr = a.ctr;
  p.groups = 1;
  p.H = a.H;
  p.d = a.d;
  p.lq = to_lay(a.q_s);
  p.lk = to_lay(a.k_s);
  p.lv = to_lay(a.v_s);
  p.lo = to_lay(a.o_s);
  p.ldo = to_lay(a.do_s);
  p.ldq = to_lay(a.dq_s);
  p.ldk = to_lay(a.dk_s);
  p.ldv = to_lay(a.dv_s);
  {
    const int64_t rows = (int64_t)a.B * a.H * a.Tq;
    constexpr int rows_per_block = 256 / (D / 8);
    const int64_t grid = (rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((fa_bwd_prep_kernel<D, GEN>), dim3((unsigned)grid), dim3(256), 0, stream,
                       p, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    // both gradient kernels are persistent: one workgroup per CU (each needs most of a CU's LDS
    // and registers), at most one per work unit; 8 XCD groups when there are more units than CUs
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cus < 1) cus = 1;
    auto grid_for = [&](BwdParams& q, long long units) {
      if (units > cus && cus >= kQueues) {
        q.groups = kQueues;
        return cus - cus % kQueues;
      }
      q.groups = 1;
      return (int)(units < cus ? units : cus);
    };
    // dK/dV: (nblk - 1 - j, j) key-block pairs dealt to the workgroups
    BwdParams pk = p;
    pk.nblk = (a.Tk + kOwnK - 1) / kOwnK;
    const int grid_k = grid_for(pk, (long long)pk.BH * ((pk.nblk + 1) / 2));
    void* args_k[] = {&pk};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<D, CAUSAL, OUT_F32, GEN>),
                        dim3(grid_k), dim3(kThreadsK), args_k, 0, stream);
    if (e != hipSuccess) return e;
    // dQ: query blocks taken from the item queues
    p.nblk = (a.Tq + kOwnQ - 1) / kOwnQ;
    const int grid_q = grid_for(p, (long long)p.BH * p.nblk);
    void* args_q[] = {&p};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_bwd_dq_kernel<D, CAUSAL, OUT_F32, GEN>),
                        dim3(grid_q), dim3(kThreadsQ), args_q, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// GEN = false for contiguous [B][h][T][D] tensors (d = D), else the general-layout kernels.
template <int D>
hipError_t launch_d(const BwdLaunch& a, hipStream_t s) {
  const int64_t H = a.H;
  auto dense = [&](const int64_t* s3, int64_t T) {
    return s3[2] == D && s3[1] == T * D && s3[0] == H * T * D;
  };
  const bool gen = a.d != D || !dense(a.q_s, a.Tq) || !dense(a.k_s, a.Tk) ||
                   !dense(a.v_s, a.Tk) || !dense(a.o_s, a.Tq) || !dense(a.do_s, a.Tq) ||
                   !dense(a.dq_s, a.Tq) || !dense(a.dk_s, a.Tk) || !dense(a.dv_s, a.Tk);
  if (gen) {   // general layouts: bf16 outputs only
    if (a.out_f32) return hipErrorInvalidValue;
    return a.causal ? launch<D, true, false, true>(a, s) : launch<D, false, false, true>(a, s);
  }
  if (a.causal)
    return a.out_f32 ? launch<D, true, true, false>(a, s) : launch<D, true, false, false>(a, s);
  return a.out_f32 ? launch<D, false, true, false>(a, s) : launch<D, false, false, false>(a, s);
}

}  // namespace

hipError_t launch_bwd(const BwdLaunch& a, hipStream_t stream) {
  if (a.d <= 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace fa
