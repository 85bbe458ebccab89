// Attention forward (prefill) for gfx950: one workgroup per (256-row query block, head, batch).
//
// The method (page "Fusion and IO-aware kernels", "How it really works", FlashAttention steps
// 1-4; page "Kernels -- fusion and FlashAttention", sections 3-5): a block of query rows stays
// on chip, K/V tiles stream past it, and each query row keeps a running max m, a running
// denominator l and an fp32 output accumulator; after the last tile O = acc / l and
// LSE = m + ln l.  The score tile never leaves registers.
//
// MI355X mapping (our design, not the pages'):
//   * 8 waves x 32 query rows = 256 rows per workgroup, two waves per SIMD; key tiles of 64.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the Q
//     fragment is the B operand and lives in registers for the whole kernel, K is the A operand
//     read from LDS.  In the MFMA output layout every lane then owns ONE query row (lane % 32)
//     and 16 of the tile's keys per 32-key block, so the row max and row sum are in-lane
//     reductions plus one exchange with lane ^ 32 (v_permlane32_swap).
//   * The P V contraction is also computed transposed, O^T += V^T P^T: P^T comes straight from
//     the score registers (rounded to bf16) as the B operand; the V^T A operand is read from
//     row-major V in LDS with the gfx950 transposing LDS read (two ds_read_b64_tr_b16 per
//     MFMA), whose lane layout lands on exactly the keys each lane holds in P.
//   * Ping-pong: waves 0-3 (group A) and 4-7 (group B) share the four SIMDs pairwise and run
//     the same program half a step apart.  Each step is a matrix section (this tile's S^T and
//     the previous tile's O^T, 32 MFMAs, issued at raised priority) followed by a vector section
//     (online softmax of this tile and staging of a later K/V tile into LDS), each closed by a
//     workgroup barrier; group B starts one section late, so on every SIMD one wave feeds the
//     matrix core while the other runs the exp/max/sum work.
//   * K/V tiles live in a 4-deep ring of LDS stages (4 x 32 KB at d = 128), filled by direct
//     global-to-LDS loads (buffer_load ... lds): no registers, no LDS store instructions and no
//     waits in the vector sections.  Tile t+2 is requested at the start of matrix section t and
//     waited for at the end of matrix section t+1.  Each 64-lane load writes 1 KB of LDS
//     contiguously, so rows cannot be padded; instead the 16-byte chunks of each row are
//     XOR-swizzled so that the MFMA operand reads hit distinct LDS banks.
//   * Online softmax in log2 units with scale * log2(e) folded into one fused multiply-add per
//     score; the row max is taken on the raw scores.  P is rounded to bf16 for the O^T MFMA and
//     O is normalised by the sum of those rounded values (a v_dot2 against (1, 1) per pair), so
//     O is an exact convex combination of the V rows the MFMA used; the LSE takes the sum of
//     the fp32 p.  The rescale of the accumulator by exp(m_old - m_new) is skipped (one
//     wave-uniform branch) unless some row's max has grown by more than 2^8 since the last
//     rescale: stale maxima only scale p, l and acc by the same factor (at most 256), so
//     O = acc / l and LSE = m + log l are unchanged.
//   * Buffer loads with a per-head range return zeros past the end of Q/K/V, so ragged tails
//     need only the -inf score mask (page "Chapter 10 Writing and Benchmarking Custom
//     Kernels", section 10.3.1, "What You Actually Decide in Practice": the final partial tile).
//   * Causal: key tiles entirely above the diagonal are never loaded or computed; per wave,
//     tiles above that wave's rows are skipped; only tiles crossing the diagonal are masked.
//   * Workgroup -> (head, query block) order is XCD-aware (consecutive blocks of one head land
//     on one XCD, so its K/V stay in that XCD's L2) and, for causal, heaviest blocks first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"
#include "fa_lds.hpp"

namespace fa {
namespace {

constexpr int kBM = 256;       // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;     // LDS ring depth
constexpr float kRescaleThreshold = 8.0f;   // log2 units

constexpr int kVmcnt0 = vmcnt_imm(0);

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int Tq, Tk, nqb;
  int BH, npairs;   // heads (batch * heads) and query-block pairs per head
  int groups;       // workgroup groups (one per XCD); group x takes heads x, x + groups, ...
  float scale_log2;   // |scale| * log2(e), > 0
  uint32_t q_sign;    // 0x80008000 when scale < 0 (Q is negated instead), else 0
  // Layout: element (b, h, t, c) of q is at q[b*q_b + h*q_h + t*q_t + c], likewise for k, v, o;
  // d <= D is the true head dimension (columns d .. D - 1 are zero padding on chip).
  int H, d;
  int64_t q_b, q_h, k_b, k_h, v_b, v_h, o_b, o_h;
  uint32_t q_t, k_t, v_t, o_t;
};

// A buffer offset beyond every head's range (heads are < 2^31 bytes): loads return zeros.
constexpr uint32_t kPadOffset = 0x80000000u;

template <int D>
struct Tile {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int TILE = kBN * D;               // bf16 per K (or V) tile
  static constexpr int STAGE = 2 * TILE;             // K then V
  static constexpr int ROWS_PER_LOAD = 64 / CH;      // rows one 64-lane load (1 KB) covers
  static constexpr int LOADS = kBN / ROWS_PER_LOAD;  // 1 KB loads per tile and tensor
  static constexpr int LOADS_PER_WAVE = LOADS / kWaves;
  static_assert(LOADS_PER_WAVE >= 1 && LOADS % kWaves == 0, "staging layout");
  // Physical 16-byte chunk of logical chunk c in row r (an involution, so it also maps back).
  // LDS serves 256 bytes per clock: one d = 128 row, or two d = 64 rows.  K is read 16 rows x
  // one chunk per 16 lanes, so rows that share banks get distinct chunks.  V is read by the
  // transposing load, 4 rows x 4 chunks per 32 lanes, so each row's 4-chunk group moves to its
  // own 64-byte quarter of the banks.
  static __device__ __forceinline__ int kchunk(int r, int c) {
    return D == 128 ? c ^ (r & 15) : c ^ ((r >> 1) & 7);
  }
  static __device__ __forceinline__ int vchunk(int r, int c) {
    return D == 128 ? c ^ (4 * (r & 3)) : c ^ (4 * ((r >> 1) & 1));
  }
};

// Loads one wave issues per tile (K and V).
template <int D>
constexpr int kVmcntTile = vmcnt_imm(2 * Tile<D>::LOADS_PER_WAVE);
// ... plus the D/16 loads of a wave's Q rows.
template <int D>
constexpr int kVmcntQ = vmcnt_imm(D / 16);
template <int D>
constexpr int kVmcntQTile = vmcnt_imm(D / 16 + 2 * Tile<D>::LOADS_PER_WAVE);

// Matrix sections (see the kernel): scores only (first tile of a block), both products, or the
// P^T product only (after the last tile).
constexpr int kSecScores = 0, kSecBoth = 1, kSecValues = 2;

// Operand order of a matrix section: scores only = the NK K operands; both = VH V^T operands,
// the NK K operands, the other NV - VH V^T operands; values only = the NV V^T operands.  kPre
// operands are in the ring of kRing registers on entry.  K operands take one LDS read, V^T
// operands two.
template <int MODE, int NV, int NK, int VH, int RING>
struct OpSeq {
  static constexpr int kRing = RING;
  static constexpr int n = MODE == kSecScores ? NK : (MODE == kSecBoth ? NV + NK : NV);
  static constexpr bool kScores = MODE != kSecValues;
  static constexpr int kPre = MODE == kSecScores ? kRing : (VH < kRing ? VH : kRing);
  static constexpr __device__ bool is_k(int i) {
    return MODE == kSecScores || (MODE == kSecBoth && i >= VH && i < VH + NK);
  }
  static constexpr __device__ int k_index(int i) { return MODE == kSecScores ? i : i - VH; }
  static constexpr __device__ int v_index(int i) {
    return MODE == kSecBoth && i >= VH + NK ? i - NK : i;
  }
  static constexpr __device__ int reads(int i) { return is_k(i) ? 1 : 2; }
  static constexpr __device__ int initial_reads() {
    int r = 0;
    for (int i = kPre; i < kRing && i < n; ++i) r += reads(i);
    return r;
  }
};

// Scheduling pattern of a section's steady state: MFMA i, then the reads of operand i + kRing.
template <class S, int R>
__device__ __forceinline__ void sched_refills() {
  if constexpr (R < S::n) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, S::reads(R), 0);
    sched_refills<S, R + 1>();
  }
}

// 16- and 8-byte LDS accesses at a byte address.
__device__ __forceinline__ u32x4_t lds_read16u(uint32_t addr) {
  typedef __attribute__((address_space(3))) const u32x4_t* lds_ptr_t;
  return *(lds_ptr_t)(uintptr_t)addr;
}
__device__ __forceinline__ void lds_write8(uint32_t addr, u32x2_t v) {
  typedef __attribute__((address_space(3))) u32x2_t* lds_ptr_t;
  *(lds_ptr_t)(uintptr_t)addr = v;
}

// A lane's value and the value of lane l ^ 32.  With both operands holding v,
// v_permlane32_swap leaves lanes 0-31 with (v[l], v[l+32]) and lanes 32-63 with (v[l-32], v[l]).
// The two halves of the result are copied into named scalars before use: reading them through
// a bit cast of the subscripted result made this compiler substitute half 0 for half 1.
__device__ __forceinline__ void xhalf_pair(float v, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t s0 = s[0], s1 = s[1];
  a = __builtin_bit_cast(float, s0);
  b = __builtin_bit_cast(float, s1);
}
__device__ __forceinline__ float xhalf_max(float v) {
  float a, b;
  xhalf_pair(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xhalf_sum(float v) {
  float a, b;
  xhalf_pair(v, a, b);
  return a + b;
}

// GEN = false: contiguous [B][h][T][D] tensors with d = D, every stride a compile-time multiple of
// D (the layout of fa_fwd at d_head = 64 or 128); GEN = true: the strides and d of FwdParams.
template <int D, bool CAUSAL, bool OUT_F32, bool GEN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(FwdParams p) {
  using T = Tile<D>;
  // layout (compile-time constants in the contiguous case)
  const int dd = GEN ? p.d : D;
  const uint32_t q_t = GEN ? p.q_t : D, k_t = GEN ? p.k_t : D, v_t = GEN ? p.v_t : D,
                 o_t = GEN ? p.o_t : D;
  constexpr int NS = D / 16;   // k-steps of S^T = K Q^T
  constexpr int ND = D / 32;   // 32-row blocks of O^T
  constexpr int NK = 2 * NS, NV = 4 * ND;            // K and V^T operands per tile
  // V^T operands before the scores: half for the causal d = 128 kernels; a quarter elsewhere
  // (3-4% faster at d = 64, where the scores are half as long and the vector section that waits
  // for them sets the pace; 1% faster non-causal at d = 128; 2-3% slower causal at d = 128)
  constexpr int VH = D == 128 && CAUSAL ? NV / 2 : NV / 4;
  // Operand registers in flight per matrix section: 8 for the causal contiguous kernels (1-2%
  // faster than 4 there), 4 elsewhere (the non-causal kernels ran 1% slower with 8, and the
  // general-layout ones spill).
  constexpr int kRing = CAUSAL && !GEN ? 8 : 4;
  constexpr int PRE = VH < kRing ? VH : kRing;       // of which read ahead of the barrier
  // LDS: the four K stages, then the four V stages.  Every access below is a per-lane base
  // address (fixed for the whole kernel) plus a compile-time offset below 64 KB, which the
  // LDS instructions take as an immediate.
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * kStages * T::TILE];
  // Output staging: 32 rows x 64 columns of bf16 per wave (the rest of the CU's 160 KB).
  __shared__ __attribute__((aligned(1024))) uint16_t ostage[kWaves * 32 * 64];
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  constexpr uint32_t kTileBytes = T::TILE * 2, kVRegion = kStages * kTileBytes;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  // waves w and w + 4 share a SIMD: one from each group
  const bool group_b = wave >= 4;

  // Per-lane LDS byte addresses of the MFMA A operands in stage 0; stage x adds x * kTileBytes.
  //  K (S^T = K Q^T), k-step s, key block kb: row 32*kb + r32, logical chunk 2*s + g.  The
  //  swizzle is an XOR on the chunk index and depends on the row only through r32, so the
  //  address is k_base ^ (32*s), plus 32*kb*D*2 bytes.
  //  V^T (O^T += V^T P^T) via the transposing read, 32-row block db of O^T, k-step ks, half hf:
  //  lane l of 16-lane group (g, dh) addresses key 16*ks + 8*hf + 4*g + (l % 16) / 4,
  //  d = 32*db + 16*dh + 4*(l % 4), and receives V^T row d = 32*db + (l % 32), keys
  //  16*ks + 8*hf + 4*g + 0..3 (the keys it holds in P registers 8*(ks%2) + 4*hf .. +3 of score
  //  block ks/2).  The swizzle depends on the key only through (l % 16) / 4, so the address is
  //  v_base ^ (64*db), plus (16*ks + 8*hf)*D*2 bytes.
  const uint32_t k_base = lds0 + 2 * (r32 * D + 8 * T::kchunk(r32, g));
  uint32_t v_base;
  {
    const int x = (lane & 15) >> 2, dh = (lane >> 4) & 1, r = 4 * g + x;
    v_base = lds0 + kVRegion +
             2 * (r * D + 8 * T::vchunk(r, 2 * dh + ((lane & 3) >> 1)) + 4 * (lane & 1));
  }
  // This wave's share of a tile load: LOADS_PER_WAVE 1 KB pieces of K and of V.  Lane l of
  // piece n fills tile row n * ROWS_PER_LOAD + l / CH, physical chunk l % CH, so it reads the
  // logical chunk that the swizzle maps there.
  uint32_t dk[T::LOADS_PER_WAVE], dv[T::LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < T::LOADS_PER_WAVE; ++i) {
    const int r = (wave * T::LOADS_PER_WAVE + i) * T::ROWS_PER_LOAD + lane / T::CH;
    const int pc = lane % T::CH;
    // (padding columns, logical chunk >= d / 8, read zeros from past the buffer's end)
    const int ck = T::kchunk(r, pc), cv = T::vchunk(r, pc);
    dk[i] = 8 * ck < dd ? 2u * ((uint32_t)r * k_t + 8u * (uint32_t)ck) : kPadOffset;
    dv[i] = 8 * cv < dd ? 2u * ((uint32_t)r * v_t + 8u * (uint32_t)cv) : kPadOffset;
  }

  // ---- static schedule ----
  // The grid is at most one workgroup per CU.  Workgroup n belongs to group x = n % groups
  // (the XCD it is dispatched to) and takes heads x, x + groups, ... of that group; the group's
  // (head, block pair) list is dealt round-robin over its workgroups, so the workgroups of one
  // XCD work on a few heads at a time and share their K/V in that XCD's L2.  A pair holds query
  // blocks nqb-1-j and j, whose causal costs add up to the same total for every j.  A workgroup
  // runs its items (one query block each) back to back as one stream of K/V tiles: the first
  // tiles and the Q rows of the next item are loaded while the current one finishes.
  const int n = blockIdx.x, X = p.groups;
  const int x = __builtin_amdgcn_readfirstlane(n % X), c = __builtin_amdgcn_readfirstlane(n / X);
  const int C = __builtin_amdgcn_readfirstlane(((int)gridDim.x - x + X - 1) / X);
  const int PX = __builtin_amdgcn_readfirstlane(((p.BH - x + X - 1) / X) * p.npairs);
  const int off = p.Tk - p.Tq;   // query i sits at key position i + off (causal)

  struct Item {
    int pp, half;   // pair index in the group, 0 = block nqb-1-j / 1 = block j
    int bh, i0, ntiles;
  };
  auto describe = [&](int pp, int half) {
    Item it;
    it.pp = pp;
    it.half = half;
    const int hl = __builtin_amdgcn_readfirstlane(pp / p.npairs);
    const int j = pp - hl * p.npairs;
    it.bh = x + X * hl;
    it.i0 = __builtin_amdgcn_readfirstlane((half == 0 ? p.nqb - 1 - j : j) * kBM);
    // keys the block needs: all, or (causal) up to its last row
    int kend = p.Tk;
    if (CAUSAL) kend = min(p.Tk, min(it.i0 + kBM, p.Tq) + off);
    it.ntiles = __builtin_amdgcn_readfirstlane((kend + kBN - 1) / kBN);
    return it;
  };
  auto following = [&](const Item& it) {   // (pp >= PX: no item)
    const int j = it.pp - (it.pp / p.npairs) * p.npairs;
    if (it.half == 0 && p.nqb - 1 - j != j) return describe(it.pp, 1);
    return describe(it.pp + C, 0);
  };
  // a head's element offset (rows of T elements of stride D when contiguous)
  auto head_off = [&](int bh, int64_t sb, int64_t sh, int T_) -> int64_t {
    if (!GEN) return (int64_t)bh * T_ * D;
    const int b = __builtin_amdgcn_readfirstlane(bh / p.H);
    return (int64_t)b * sb + (int64_t)(bh - b * p.H) * sh;
  };
  // a head's byte range: rows 0 .. T - 1 of stride st, the last one d columns wide
  auto range = [&](int T_, uint32_t st) { return ((uint32_t)(T_ - 1) * st + (uint32_t)dd) * 2u; };
  auto k_rsrc = [&](const Item& it) {
    return rsrc_words(p.k + head_off(it.bh, p.k_b, p.k_h, p.Tk), range(p.Tk, k_t));
  };
  auto v_rsrc = [&](const Item& it) {
    return rsrc_words(p.v + head_off(it.bh, p.v_b, p.v_h, p.Tk), range(p.Tk, v_t));
  };
  // this wave's 32 query rows of an item, as the B operand fragment of S^T = K Q^T
  bf16x8_t qf[NS];
  auto load_q = [&](const Item& it) {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(p.q + head_off(it.bh, p.q_b, p.q_h, p.Tq), range(p.Tq, q_t));
    const int qrow = it.i0 + wave * 32 + r32;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int col = 16 * s + 8 * g;
      // (the loaded value is not touched here: the loads stay in flight until the item's first
      // matrix section, which applies the sign of a negative scale)
      qf[s] = as_bf16x8(buf_load16(
          rq, col < dd ? ((uint32_t)qrow * q_t + (uint32_t)col) * 2u : kPadOffset));
    }
  };
  // one K/V tile of an item into stage st
  auto dma = [&](u32x4_t rk, u32x4_t rv, int tile, int st) {
    const uint32_t g0k = (uint32_t)tile * (kBN * 2u) * k_t;
    const uint32_t g0v = (uint32_t)tile * (kBN * 2u) * v_t;
    const uint32_t so = (uint32_t)st * kTileBytes;
#pragma unroll
    for (int i = 0; i < T::LOADS_PER_WAVE; ++i) {
      const uint32_t piece = (uint32_t)(wave * T::LOADS_PER_WAVE + i) * 1024u;
      lds_dma16(rk, lds0 + so + piece, g0k + dk[i]);
      lds_dma16(rv, lds0 + kVRegion + so + piece, g0v + dv[i]);
    }
  };

  // ---- matrix-section operands ----
  // A section is a list of MFMAs whose A operands stream from LDS through a ring of kRing
  // registers, each read issued kRing MFMAs ahead of its use.  Section t (1 <= t < ntiles)
  // applies the previous tile's P^T (O^T += V^T P^T, operands: V^T of tile t - 1) and computes
  // this tile's scores (S^T = K Q^T, operands: K of tile t), in the order: first half of the
  // V^T operands, all K operands, second half of the V^T operands.  Section 0 has only the
  // scores, section ntiles only the P^T product.
  //  * The leading V^T operands may be read by a wave as soon as its own vector section t - 1
  //    has run (tile t - 1 was published two barriers earlier), so they are issued at the end of
  //    that vector section and their latency hides behind the barrier.
  //  * The scores are finished half a section before its end, so the vector section that follows
  //    does not wait for the matrix pipe to drain.
  bf16x8_t ring[kRing];
  // K operand kk: rows 32*(kk%2) + r32, k-step kk/2 of the tile at ks.
  auto k_opnd = [&](uint32_t ks, int kk) -> bf16x8_t {
    return lds_read_bf16x8((ks ^ (32u * (kk >> 1))) + 2 * 32 * (kk & 1) * D);
  };
  // V^T operand j: block db = j%ND, k-step j/ND of the tile at vs (two transposing reads).
  auto v_opnd = [&](uint32_t vs, int j) -> bf16x8_t {
    const uint32_t base = (vs ^ (64u * (j % ND))) + 2 * 16 * (j / ND) * D;
    return lds_read_tr_pair(base, base + 2 * 8 * D);
  };
  auto k_at = [&](int st) { return k_base + (uint32_t)st * kTileBytes; };
  auto v_at = [&](int st) { return v_base + (uint32_t)st * kTileBytes; };

  f32x16_t oacc[ND];
  f32x16_t sacc[2];
  bf16x8_t pb[4];
  // On entry ring[0 .. kPre-1] hold the first operands (kPre: kRing for scores only, else PRE).
  auto section = [&](auto mode, uint32_t ks, uint32_t vs) {
    using S = OpSeq<decltype(mode)::value, NV, NK, VH, kRing>;
    constexpr int pre = S::kPre;
    auto opnd = [&](int i) {
      return S::is_k(i) ? k_opnd(ks, S::k_index(i)) : v_opnd(vs, S::v_index(i));
    };
#pragma unroll
    for (int i = pre; i < kRing; ++i) ring[i] = opnd(i);
    if (S::kScores) {
      sacc[0] = f32x16_t{};
      sacc[1] = f32x16_t{};
    }
#pragma unroll
    for (int i = 0; i < S::n; ++i) {
      const bf16x8_t a = ring[i % kRing];
      if (i + kRing < S::n) ring[i % kRing] = opnd(i + kRing);
      if (S::is_k(i)) {
        const int kk = S::k_index(i);
        sacc[kk & 1] = mfma_32x32x16(a, qf[kk >> 1], sacc[kk & 1]);
      } else {
        const int j = S::v_index(i);
        oacc[j % ND] = mfma_32x32x16(a, pb[j / ND], oacc[j % ND]);
      }
    }
    // the remaining initial reads, then (MFMA, refill reads) pairs, then the last kRing MFMAs
    if (S::initial_reads() > 0) __builtin_amdgcn_sched_group_barrier(0x100, S::initial_reads(), 0);
    sched_refills<S, kRing>();
    __builtin_amdgcn_sched_group_barrier(0x008, kRing, 0);
  };
  using ScoresOnly = std::integral_constant<int, kSecScores>;
  using Both = std::integral_constant<int, kSecBoth>;
  using ValuesOnly = std::integral_constant<int, kSecValues>;

  Item cur = describe(c, 0);
  int g0 = 0;   // stream position of the current item's tile 0 (tile x sits in stage x % 4)
  if (cur.pp < PX) {
    // ---- prologue: Q and the first two tiles of the stream loaded and published ----
    load_q(cur);
    {
      const u32x4_t rk = k_rsrc(cur), rv = v_rsrc(cur);
      dma(rk, rv, 0, 0);
      if (cur.ntiles > 1) {
        dma(rk, rv, 1, 1);
      } else {
        const Item nx = following(cur);
        if (nx.pp < PX) dma(k_rsrc(nx), v_rsrc(nx), 0, 1);
      }
    }
    // (a full wait: it also settles the Q loads, which the compiler would otherwise wait for
    // at their first use, behind later tile loads)
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (group_b) __syncthreads();   // group B runs one section behind group A
  }

  while (cur.pp < PX) {
    const Item nxt = following(cur);
    const bool has_nxt = nxt.pp < PX;
    const int ntiles = cur.ntiles;
    const u32x4_t rk = k_rsrc(cur), rv = v_rsrc(cur);
    const u32x4_t rk_n = k_rsrc(nxt), rv_n = v_rsrc(nxt);

    const int qw0 = cur.i0 + wave * 32;
    const int qrow = qw0 + r32;
    const int qw_last = min(qw0 + 31, p.Tq - 1);
    const bool wave_has_rows = qw0 < p.Tq;
    auto active = [&](int t) { return wave_has_rows && !(CAUSAL && t * kBN > qw_last + off); };

    float m_run = -INFINITY;   // running max used for the exponentials (log2 units)
    float m_thr = -INFINITY;   // m_run + rescale threshold
    // This lane's running sums, kept as four partial sums each (independent add chains):
    float l_run[4] = {0.f, 0.f, 0.f, 0.f};     // of p (fp32): the LSE
    float l16_run[4] = {0.f, 0.f, 0.f, 0.f};   // of bf16(p): normalises O
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] = f32x16_t{};

    // Stream tile x of this item (x >= ntiles: tile x - ntiles of the next item).  Tile x + 2 is
    // requested at the start of matrix section x; each wave waits for its own part of tile
    // x + 1 at the end of matrix section x (one more tile may still be in flight), and the
    // barrier that follows publishes it to all waves.
    auto exists = [&](int xt) { return xt < ntiles || (has_nxt && xt - ntiles < nxt.ntiles); };
    auto request = [&](int xt) {
      const int st = (g0 + xt) & (kStages - 1);
      if (xt < ntiles) dma(rk, rv, xt, st);
      else if (exists(xt)) dma(rk_n, rv_n, xt - ntiles, st);
    };
    // Vector-memory operations complete in issue order.  Before tile 1 of an item has landed,
    // the previous item's last step issued this item's Q rows and the previous output stores,
    // after tile 1's loads; allowing the Q loads to stay in flight keeps the stores (the younger
    // part) out of the wait as well.  (For the first item, tiles 0 and 1 were waited for fully.)
    auto wait_next = [&](int t) {   // stream tile t + 1 has landed (this wave's part)
      if (t == 0) {
        if (exists(2))
          __builtin_amdgcn_s_waitcnt(kVmcntQTile<D>);
        else
          __builtin_amdgcn_s_waitcnt(kVmcntQ<D>);
      } else if (exists(t + 2)) {
        __builtin_amdgcn_s_waitcnt(kVmcntTile<D>);
      } else {
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
      }
    };

    // q_next: this is the item's last score step (t = ntiles - 1, ntiles > 1); it requests the
    // next item's Q rows.  It is a separate instantiation, outside the loop over the other
    // steps, so that no step in that loop has Q loads in flight into the fragment it reads.
    auto step = [&](const int t, auto mode, auto q_next) {
      constexpr int MODE = decltype(mode)::value;
      const int st = (g0 + t) & (kStages - 1), st_prev = (g0 + t + kStages - 1) & (kStages - 1);
      // ================= matrix section =================
      __builtin_amdgcn_s_setprio(1);
      request(t + 2);
      if (MODE == kSecScores) {
        // the item's Q rows are needed from here on: negate them for a negative scale (exact)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8_t x = qf[s];
          qf[s] = as_bf16x8(__builtin_bit_cast(u32x4_t, x) ^ p.q_sign);
        }
      }
      // A wave's tiles form a prefix (causal skipping is monotone in t), so after step 0 a wave
      // that has the previous tile's P^T to apply runs both products; at the step after its
      // last tile the S^T product is wasted (and ignored), which keeps a single code path for
      // the accumulators.
      if (MODE == kSecScores) {
        if (active(0)) section(ScoresOnly{}, k_at(st), 0u);
      } else {
        if (active(t - 1)) section(Both{}, k_at(st), v_at(st_prev));
      }
      wait_next(t);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();

      // ================= vector section =================
      if (active(t)) {
        const int j0 = t * kBN;
        const bool need_mask = (j0 + kBN > p.Tk) || (CAUSAL && j0 + kBN - 1 > qw0 + off);
        if (need_mask) {
          const int lim = CAUSAL ? min(p.Tk - 1, qrow + off) : p.Tk - 1;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = j0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
              if (key > lim) sacc[kb][i] = -INFINITY;
            }
        }
        // Every reduction below runs as four independent chains: one wave per SIMD does this
        // work while the other issues MFMAs, so dependent-issue latency is not hidden by others.
        float mx[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) mx[cc] = fmaxf(sacc[0][cc], sacc[0][cc + 4]);
#pragma unroll
        for (int i = 8; i < 32; ++i) mx[i & 3] = fmaxf(mx[i & 3], sacc[i >> 4][i & 15]);
        float mt = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
        mt = xhalf_max(mt) * p.scale_log2;
        // lazy rescale: only when some row's max outgrew the max in use by > 2^8
        if (__any(mt > m_thr)) {
          const float m_new = fmaxf(m_run, mt);
          const float corr = fast_exp2(m_run - m_new);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            l_run[cc] *= corr;
            l16_run[cc] *= corr;
          }
#pragma unroll
          for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= corr;
          m_run = m_new;
          m_thr = m_new + kRescaleThreshold;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = fast_exp2(__builtin_fmaf(sacc[kb][i], p.scale_log2, -m_run));
            sacc[kb][i] = e;
            l_run[i & 3] += e;
          }
        // P^T as bf16 B operands: 16 keys per k-step, registers 8*(ks%2).. of score block ks/2
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const f32x16_t& sb = sacc[ks >> 1];
          const int b0 = (ks & 1) * 8;
          const u32x2_t lo = pack_bf16x4(sb[b0], sb[b0 + 1], sb[b0 + 2], sb[b0 + 3]);
          const u32x2_t hi = pack_bf16x4(sb[b0 + 4], sb[b0 + 5], sb[b0 + 6], sb[b0 + 7]);
          u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
          pb[ks] = as_bf16x8(w);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            l16_run[e] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[e]), ones_bf16x2(),
                                                         l16_run[e], false);
        }
        // the next section's leading operands: V^T of this tile
#pragma unroll
        for (int i = 0; i < PRE; ++i) ring[i] = v_opnd(v_at(st), i);
      }
      // After the item's last S^T section the Q fragment is free: the next item's Q rows are
      // requested here, a whole step before its first S^T section needs them.  (They follow
      // the request of the next item's tile 1 and precede this item's output stores, the order
      // the waits below count on.)
      if constexpr (decltype(q_next)::value) {
        if (has_nxt) load_q(nxt);
      }
      __syncthreads();
    };

    // section 0's first operands: K of tile 0
    {
      const uint32_t ks0 = k_at(g0 & (kStages - 1));
#pragma unroll
      for (int i = 0; i < kRing; ++i) ring[i] = k_opnd(ks0, i);
    }
    using NoQ = std::false_type;
    using WithQ = std::true_type;
    step(0, ScoresOnly{}, NoQ{});
    for (int t = 1; t < ntiles - 1; ++t) step(t, Both{}, NoQ{});
    if (ntiles > 1) step(ntiles - 1, Both{}, WithQ{});

    // ---- last step: the last tile's P^T, then the epilogue in the vector slot ----
    __builtin_amdgcn_s_setprio(1);
    if (active(ntiles - 1))
      section(ValuesOnly{}, 0u, v_at((g0 + ntiles - 1) & (kStages - 1)));
    // (an item with a single tile, Tk <= 64 only: its Q request comes after the P^T section)
    if (ntiles == 1 && has_nxt) load_q(nxt);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    // O = acc / l16, LSE = (m + log2 l) * ln 2 (touches only this wave's output staging)
    const float l_tot = xhalf_sum((l_run[0] + l_run[1]) + (l_run[2] + l_run[3]));
    const float l16_tot = xhalf_sum((l16_run[0] + l16_run[1]) + (l16_run[2] + l16_run[3]));
    const float inv = 1.0f / l16_tot;
    if (OUT_F32) {
      if (wave_has_rows && qrow < p.Tq) {
        const int64_t orow = head_off(cur.bh, p.o_b, p.o_h, p.Tq) + (int64_t)qrow * o_t;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int col = 32 * db + 8 * i4 + 4 * g;
            const f32x4_t f = {oacc[db][4 * i4] * inv, oacc[db][4 * i4 + 1] * inv,
                               oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv};
            if (col < dd)
              *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.o) + orow + col) = f;
          }
      }
    } else {
      // In the MFMA layout a lane holds 8-byte pieces of one row; the rows go through this
      // wave's 4 KB of LDS, 64 columns at a time (16-byte chunks XOR-swizzled by row), so that
      // each store writes whole 128-byte row segments.  The stores are buffer stores that every
      // wave issues, rows past Tq (or every row of a wave without rows) and padding columns at
      // an offset past the buffer's range, which the hardware drops: with no branch around them
      // the compiler counts them in every path, so the next item's first score product waits
      // only for its Q rows, not for these stores.
      const uint32_t ob = (uint32_t)reinterpret_cast<uintptr_t>(ostage) + (uint32_t)wave * 4096u;
      const int rows = p.Tq - qw0;   // valid rows of this wave (<= 0: none)
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(
          static_cast<uint16_t*>(p.o) + head_off(cur.bh, p.o_b, p.o_h, p.Tq), range(p.Tq, o_t));
#pragma unroll
      for (int h = 0; h < ND / 2; ++h) {
#pragma unroll
        for (int db2 = 0; db2 < 2; ++db2)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f32x16_t& a = oacc[2 * h + db2];
            const int ch = 4 * db2 + i4;   // columns 8*ch + 4*g .. + 3 of this half
            lds_write8(ob + r32 * 128u + 16u * (ch ^ (r32 & 7)) + 8u * g,
                       pack_bf16x4(a[4 * i4] * inv, a[4 * i4 + 1] * inv, a[4 * i4 + 2] * inv,
                                   a[4 * i4 + 3] * inv));
          }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * i + (lane >> 3), ch = lane & 7;
          const u32x4_t w = lds_read16u(ob + row * 128u + 16u * (ch ^ (row & 7)));
          const uint32_t off =
              row < rows && 64 * h + 8 * ch < dd
                  ? ((uint32_t)(qw0 + row) * o_t + (uint32_t)(64 * h + 8 * ch)) * 2u
                  : kPadOffset;
          __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
        }
      }
    }
    {
      // LSE, one lane per row (the lanes of the other half hold the same rows)
      const __amdgpu_buffer_rsrc_t rl =
          make_rsrc(p.lse + (size_t)cur.bh * p.Tq, (uint32_t)p.Tq * 4u);
      const float lse = (m_run + fast_log2(l_tot)) * kLn2;
      const uint32_t off = wave_has_rows && qrow < p.Tq && g == 0 ? (uint32_t)qrow * 4u
                                                                  : kPadOffset;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), rl, off, 0, 0);
    }
    __syncthreads();

    g0 += ntiles;
    cur = nxt;
  }
  if (describe(c, 0).pp < PX && !group_b) __syncthreads();   // match group B's extra barrier
}

template <int D, bool CAUSAL, bool OUT_F32, bool GEN>
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
  p.BH = a.B * a.H;
  p.npairs = (p.nqb + 1) / 2;
  // A zero scale would make every score 0; a tiny positive factor gives the same softmax.
  p.scale_log2 = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  p.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  p.H = a.H;
  p.d = a.d;
  p.q_b = a.q_s[0]; p.q_h = a.q_s[1]; p.q_t = (uint32_t)a.q_s[2];
  p.k_b = a.k_s[0]; p.k_h = a.k_s[1]; p.k_t = (uint32_t)a.k_s[2];
  p.v_b = a.v_s[0]; p.v_h = a.v_s[1]; p.v_t = (uint32_t)a.v_s[2];
  p.o_b = a.o_s[0]; p.o_h = a.o_s[1]; p.o_t = (uint32_t)a.o_s[2];
  // One workgroup per CU (each needs a whole CU's LDS), in 8 groups (one per XCD) when there
  // are more block pairs than CUs; otherwise one workgroup per pair.  The kernel looks two tiles
  // ahead in its stream and resolves a stream position only within the current and the next
  // item, so a workgroup that runs three or more items needs every item after its first to
  // have at least two tiles.  Items have a single tile only when Tk <= kBN (every causal block
  // with Tk > kBN sees at least min(Tk, 256) keys); those shapes take one workgroup per pair,
  // i.e. at most two items per workgroup.
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long long pairs = (long long)p.BH * p.npairs;
  const bool single_tile_items = a.Tk <= kBN;
  int grid;
  if (single_tile_items) {
    p.groups = 1;
    grid = (int)pairs;
  } else if (pairs > cus && cus >= 8) {
    p.groups = 8;
    grid = cus - cus % 8;
  } else {
    p.groups = 1;
    grid = (int)(pairs < cus ? pairs : (cus > 0 ? cus : 1));
  }
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_kernel<D, CAUSAL, OUT_F32, GEN>),
                         dim3(grid), dim3(kThreads), args, 0, stream);
}

template <int D, bool GEN>
hipError_t launch_g(const FwdLaunch& a, hipStream_t s) {
  if (a.causal)
    return a.out_f32 ? launch<D, true, true, GEN>(a, s) : launch<D, true, false, GEN>(a, s);
  return a.out_f32 ? launch<D, false, true, GEN>(a, s) : launch<D, false, false, GEN>(a, s);
}

// the contiguous layout with d = D takes the specialised kernel
template <int D>
hipError_t launch_d(const FwdLaunch& a, hipStream_t s) {
  auto contiguous = [&](const int64_t* st, int T_) {
    return st[2] == D && st[1] == (int64_t)T_ * D && st[0] == (int64_t)a.H * T_ * D;
  };
  const bool plain = a.d == D && contiguous(a.q_s, a.Tq) && contiguous(a.k_s, a.Tk) &&
                     contiguous(a.v_s, a.Tk) && contiguous(a.o_s, a.Tq);
  return plain ? launch_g<D, false>(a, s) : launch_g<D, true>(a, s);
}

}  // namespace

hipError_t launch_fwd(const FwdLaunch& a, hipStream_t stream) {
  // head dimensions up to 64 run the 64-wide kernel, larger ones the 128-wide one, padded
  if (a.d <= 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace fa
