// Host-side argument validation, status strings and workspace sizing of the C ABI in fa.h.
// Pure C++ (no HIP): it runs before any HIP call, so an invalid call enqueues nothing and
// leaves its outputs untouched.  Compiles with g++ alone for host-only checks.
#include <cmath>
#include <cstdint>

#include "fa.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The kernels pad any multiple of 8 up to 128 on chip (16-byte chunks of 8 bf16) to 64 or 128.
bool head_dim_ok(int64_t d) { return d >= 8 && d <= 128 && d % 8 == 0; }

// Strided head: rows of stride t (>= d, a multiple of 8 elements so that rows stay 16-byte
// aligned), the head's bytes including one 128-row block of reads past the end below 2^31.
bool strides_ok(const int64_t* s, int64_t T, int64_t d, int64_t B, int64_t h) {
  if (!s) return false;
  const int64_t sb = s[0], sh = s[1], st = s[2];
  if (st < d || st % 8 != 0 || sb < 0 || sh < 0 || sb % 8 != 0 || sh % 8 != 0) return false;
  if (st > (FA_MAX_HEAD_BYTES / 2) / (T + 128)) return false;
  // the largest element offset must fit in int64 comfortably
  const int64_t big = INT64_MAX / 4;
  if ((B > 1 && sb > big / (B - 1)) || (h > 1 && sh > big / (h - 1))) return false;
  return true;
}

// An output written by many workgroups must not alias itself: with its dimensions of extent > 1
// ordered by stride, each stride must step past everything the smaller ones span (the usual
// sufficient condition for a non-overlapping strided tensor; gaps between rows or heads are
// allowed, interleavings that this order cannot express are rejected).  Inputs may broadcast
// (stride 0, e.g. one K/V head shared by several query heads); outputs may not.
bool no_self_overlap(const int64_t* stride, const int64_t* extent, int n) {
  int64_t s[4], e[4];
  int m = 0;
  for (int i = 0; i < n; ++i)
    if (extent[i] > 1) {
      s[m] = stride[i];
      e[m] = extent[i];
      ++m;
    }
  for (int i = 1; i < m; ++i)   // insertion sort by stride
    for (int j = i; j > 0 && s[j] < s[j - 1]; --j) {
      const int64_t ts = s[j], te = e[j];
      s[j] = s[j - 1]; e[j] = e[j - 1];
      s[j - 1] = ts; e[j - 1] = te;
    }
  int64_t span = 0;   // largest element offset reachable through the dimensions so far
  for (int i = 0; i < m; ++i) {
    if (s[i] <= span) return false;
    span += (e[i] - 1) * s[i];   // strides and extents were bounded by the callers' checks
  }
  return true;
}

// A [B][h][T][d] output with element strides s (batch, head, row) and a contiguous last dim.
bool output4_ok(const int64_t* s, int64_t B, int64_t h, int64_t T, int64_t d) {
  const int64_t stride[4] = {s[0], s[1], s[2], 1}, extent[4] = {B, h, T, d};
  return no_self_overlap(stride, extent, 4);
}

// Per-head tensors are addressed with 32-bit byte offsets inside the kernels.
bool head_bytes_ok(int64_t rows, int64_t d) {
  // one extra 128-row block of zero-filled reads past the end must still fit in 32 bits
  return rows <= (FA_MAX_HEAD_BYTES / (2 * d)) - 128;
}

}  // namespace

extern "C" int fa_validate_fwd_strided(const void* q, const void* k, const void* v,
                                       const void* o, const float* lse, int64_t B, int64_t h,
                                       int64_t Tq, int64_t Tk, int64_t d_head,
                                       const int64_t* q_strides, const int64_t* k_strides,
                                       const int64_t* v_strides, const int64_t* o_strides,
                                       int causal, float scale) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || h < 1 || Tq < 1 || Tk < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d_head)) return FA_ERR_HEAD_DIM;
  if (!strides_ok(q_strides, Tq, d_head, B, h) || !strides_ok(k_strides, Tk, d_head, B, h) ||
      !strides_ok(v_strides, Tk, d_head, B, h) || !strides_ok(o_strides, Tq, d_head, B, h))
    return FA_ERR_SHAPE;
  if (!output4_ok(o_strides, B, h, Tq, d_head)) return FA_ERR_SHAPE;
  const int64_t nqb = (Tq + 127) / 128;
  if (B > INT32_MAX / h || B * h > INT32_MAX / nqb) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SCALE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (causal && Tq > Tk) return FA_ERR_CAUSAL_TQ_GT_TK;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  return FA_OK;
}

extern "C" int fa_validate_fwd(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, int64_t B, int64_t h, int64_t Tq, int64_t Tk,
                               int64_t d_head, int causal, float scale) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || h < 1 || Tq < 1 || Tk < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d_head)) return FA_ERR_HEAD_DIM;
  if (!head_bytes_ok(Tq, d_head) || !head_bytes_ok(Tk, d_head)) return FA_ERR_SHAPE;
  // (batch, head, query block) counts are kept in 32-bit integers on the device and the grid
  // may run one workgroup per pair of query blocks: the count at 128-row granularity bounds both
  const int64_t nqb = (Tq + 127) / 128;
  if (B > INT32_MAX / h || B * h > INT32_MAX / nqb) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SCALE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (causal && Tq > Tk) return FA_ERR_CAUSAL_TQ_GT_TK;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  return FA_OK;
}

extern "C" size_t fa_decode_workspace_size(int64_t B, int64_t h, int64_t d_head,
                                           int64_t num_splits) {
  if (B < 1 || h < 1 || d_head < 1 || num_splits < 1) return 0;
  // partials are kept at the padded width (64 or 128) the kernels compute in
  const int64_t dw = d_head <= 64 ? 64 : (d_head <= 128 ? 128 : d_head);
  return static_cast<size_t>(B) * static_cast<size_t>(h) * static_cast<size_t>(num_splits) *
         static_cast<size_t>(dw + 2) * sizeof(float);
}

extern "C" int fa_validate_decode(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, int64_t B, int64_t h, int64_t Tk,
                                  int64_t d_head, float scale, int64_t num_splits,
                                  const void* workspace, size_t workspace_bytes) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || h < 1 || Tk < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d_head)) return FA_ERR_HEAD_DIM;
  if (!head_bytes_ok(Tk, d_head)) return FA_ERR_SHAPE;
  if (B > 65535 || h > 65535) return FA_ERR_SHAPE;   // grid y / z extents of the split pass
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (num_splits < 1 || num_splits > Tk || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 16) ||
      workspace_bytes < fa_decode_workspace_size(B, h, d_head, num_splits))
    return FA_ERR_WORKSPACE;
  return FA_OK;
}

namespace {
// (batch, head) strides of a one-row-per-head tensor (decode's q and o)
bool strides2_ok(const int64_t* s, int64_t B, int64_t h) {
  if (!s) return false;
  const int64_t sb = s[0], sh = s[1];
  if (sb < 0 || sh < 0 || sb % 8 != 0 || sh % 8 != 0) return false;
  const int64_t big = INT64_MAX / 4;
  return !((B > 1 && sb > big / (B - 1)) || (h > 1 && sh > big / (h - 1)));
}
}  // namespace

extern "C" int fa_validate_decode_strided(const void* q, const void* k, const void* v,
                                          const void* o, const float* lse, int64_t B, int64_t h,
                                          int64_t Tk, int64_t d_head, const int64_t* q_strides,
                                          const int64_t* k_strides, const int64_t* v_strides,
                                          const int64_t* o_strides, float scale,
                                          int64_t num_splits, const void* workspace,
                                          size_t workspace_bytes) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || h < 1 || Tk < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d_head)) return FA_ERR_HEAD_DIM;
  if (!strides2_ok(q_strides, B, h) || !strides2_ok(o_strides, B, h)) return FA_ERR_SHAPE;
  {
    const int64_t stride[3] = {o_strides[0], o_strides[1], 1}, extent[3] = {B, h, d_head};
    if (!no_self_overlap(stride, extent, 3)) return FA_ERR_SHAPE;
  }
  // the split pass reads up to 256 rows past a chunk's end (zero-filled), so one more block
  if (!strides_ok(k_strides, Tk + 128, d_head, B, h) ||
      !strides_ok(v_strides, Tk + 128, d_head, B, h))
    return FA_ERR_SHAPE;
  if (B > 65535 || h > 65535) return FA_ERR_SHAPE;   // grid y / z extents of the split pass
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (num_splits < 1 || num_splits > Tk || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 2) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 16) ||
      workspace_bytes < fa_decode_workspace_size(B, h, d_head, num_splits))
    return FA_ERR_WORKSPACE;
  return FA_OK;
}

namespace {
size_t round256(size_t x) { return (x + 255) / 256 * 256; }
// the backward's item counters: 2 kernels x 8 queues, 64 bytes apart (fa_bwd_kernel.hip)
constexpr size_t kBwdCounterBytes = 1024;
}  // namespace

extern "C" size_t fa_bwd_workspace_size(int64_t B, int64_t h, int64_t Tq) {
  if (B < 1 || h < 1 || Tq < 1) return 0;
  return 2 * round256(static_cast<size_t>(B) * static_cast<size_t>(h) * static_cast<size_t>(Tq) *
                      sizeof(float)) +
         kBwdCounterBytes;
}

extern "C" int fa_validate_bwd(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, const void* dq, const void* dk,
                               const void* dv, int64_t B, int64_t h, int64_t Tq, int64_t Tk,
                               int64_t d_head, int causal, float scale, const void* workspace,
                               size_t workspace_bytes) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B < 1 || h < 1 || Tq < 1 || Tk < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d_head)) return FA_ERR_HEAD_DIM;
  if (!head_bytes_ok(Tq, d_head) || !head_bytes_ok(Tk, d_head)) return FA_ERR_SHAPE;
  // grids: one workgroup per (128-row block, head); the preprocess takes >= 16 rows per
  // workgroup and indexes rows in 64 bits
  const int64_t nb = ((Tq > Tk ? Tq : Tk) + 127) / 128;
  if (B > INT32_MAX / h || B * h > INT32_MAX / nb) return FA_ERR_SHAPE;
  if (B * h > (int64_t)UINT32_MAX * 16 / Tq) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SCALE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (causal && Tq > Tk) return FA_ERR_CAUSAL_TQ_GT_TK;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 16) ||
      workspace_bytes < fa_bwd_workspace_size(B, h, Tq))
    return FA_ERR_WORKSPACE;
  return FA_OK;
}

extern "C" int fa_validate_bwd_strided(
    const void* q, const void* k, const void* v, const void* o, const void* dout,
    const float* lse, const void* dq, const void* dk, const void* dv, int64_t B, int64_t h,
    int64_t Tq, int64_t Tk, int64_t d_head, const int64_t* q_strides, const int64_t* k_strides,
    const int64_t* v_strides, const int64_t* o_strides, const int64_t* do_strides,
    const int64_t* dq_strides, const int64_t* dk_strides, const int64_t* dv_strides, int causal,
    float scale, const void* workspace, size_t workspace_bytes) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B < 1 || h < 1 || Tq < 1 || Tk < 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d_head)) return FA_ERR_HEAD_DIM;
  if (!strides_ok(q_strides, Tq, d_head, B, h) || !strides_ok(o_strides, Tq, d_head, B, h) ||
      !strides_ok(do_strides, Tq, d_head, B, h) || !strides_ok(dq_strides, Tq, d_head, B, h) ||
      !strides_ok(k_strides, Tk, d_head, B, h) || !strides_ok(v_strides, Tk, d_head, B, h) ||
      !strides_ok(dk_strides, Tk, d_head, B, h) || !strides_ok(dv_strides, Tk, d_head, B, h))
    return FA_ERR_SHAPE;
  if (!output4_ok(dq_strides, B, h, Tq, d_head) || !output4_ok(dk_strides, B, h, Tk, d_head) ||
      !output4_ok(dv_strides, B, h, Tk, d_head))
    return FA_ERR_SHAPE;
  const int64_t nb = ((Tq > Tk ? Tq : Tk) + 127) / 128;
  if (B > INT32_MAX / h || B * h > INT32_MAX / nb) return FA_ERR_SHAPE;
  if (B * h > (int64_t)UINT32_MAX * 16 / Tq) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SCALE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (causal && Tq > Tk) return FA_ERR_CAUSAL_TQ_GT_TK;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  if (!workspace || !aligned(workspace, 16) ||
      workspace_bytes < fa_bwd_workspace_size(B, h, Tq))
    return FA_ERR_WORKSPACE;
  return FA_OK;
}

extern "C" int fa_validate_softmax(const float* x, const float* y, const float* lse, int64_t rows,
                                   int64_t cols) {
  if (!x || !y) return FA_ERR_NULL;
  if (rows < 1 || cols < 1 || cols > INT32_MAX) return FA_ERR_SHAPE;
  // four rows per workgroup; the grid's x extent is below 2^31
  if ((rows + 3) / 4 > INT32_MAX) return FA_ERR_SHAPE;
  if (!aligned(x, 4) || !aligned(y, 4) || (lse && !aligned(lse, 4))) return FA_ERR_ALIGN;
  return FA_OK;
}

extern "C" int fa_validate_gelu(const void* x, const void* y, int64_t n) {
  if (!x || !y) return FA_ERR_NULL;
  if (n < 1) return FA_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16)) return FA_ERR_ALIGN;
  return FA_OK;
}

extern "C" int fa_validate_bias_gelu_dropout(const void* x, const void* bias, const void* y,
                                             int64_t rows, int64_t cols, float p) {
  if (!x || !bias || !y) return FA_ERR_NULL;
  if (rows < 1 || cols < 1 || rows > INT64_MAX / cols / 2) return FA_ERR_SHAPE;
  if (!aligned(x, 2) || !aligned(bias, 2) || !aligned(y, 2)) return FA_ERR_ALIGN;
  if (!(p >= 0.0f && p < 1.0f)) return FA_ERR_PROB;   // also rejects NaN
  return FA_OK;
}

extern "C" const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size is < 1 or exceeds the kernels' limits";
    case FA_ERR_HEAD_DIM:
      return "FA_ERR_HEAD_DIM: d_head must be 64 or 128 (forward: a multiple of 8 up to 128)";
    case FA_ERR_CAUSAL_TQ_GT_TK: return "FA_ERR_CAUSAL_TQ_GT_TK: causal attention needs Tq <= Tk";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensors must be 16-byte aligned (lse 4-byte)";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and causal 0 or 1";
    case FA_ERR_SPLITS: return "FA_ERR_SPLITS: num_splits must be in [1, min(Tk, FA_MAX_SPLITS)]";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace NULL, misaligned or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP launch failed (see fa_last_hip_error)";
    case FA_ERR_PROB: return "FA_ERR_PROB: the dropout probability must be in [0, 1)";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the decode partials exceed the static scratch array "
             "(FA_NOALLOC_SCRATCH_BYTES); use fewer splits or fa_decode with a workspace";
    default: return "unknown fa status code";
  }
}
