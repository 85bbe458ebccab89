/*
 * fa.h -- C ABI of the MI355X (gfx950) IO-aware attention library (libfa_mi355x.so).
 *
 * What it computes.  For every batch b and head h, with S = scale * Q K^T:
 *     O   = softmax(S masked) V                  (row softmax over the visible keys)
 *     LSE = log(sum_j exp(S_ij)) over visible j   (natural log, one fp32 per query row)
 * This is the forward pass of FlashAttention-style attention as defined on the page
 * "Kernels -- fusion and FlashAttention" (section 3, the online-softmax recurrence, and section 5,
 * the Triton tile program that writes O and m + log l), computed without ever storing the
 * Tq x Tk score matrix: query rows are tiled into blocks, K/V tiles stream through on-chip
 * memory, and a running max m, denominator l and output accumulator o are kept per query row
 * (page "Fusion and IO-aware kernels", "How it really works", FlashAttention steps 1-4).
 * The result is exact softmax attention up to floating-point rounding.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers (memory from hipMalloc / torch on the GPU), row-major
 *     and contiguous.  bf16 tensors are passed as raw 16-bit bfloat16 storage.
 *   - Ownership: the caller allocates and frees every buffer (outputs and the decode workspace).
 *     The library never allocates, frees, memsets or synchronises; it writes every element of
 *     every output it is given.
 *   - Asynchrony: a successful call only enqueues work on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream) and returns FA_OK.  Results are valid once the caller has
 *     synchronised that stream.
 *   - Errors: arguments are validated on the host before any HIP call.  An invalid call returns a
 *     nonzero FA_ERR_* code, enqueues nothing and leaves every output untouched.  A failed kernel
 *     launch returns FA_ERR_HIP; fa_last_hip_error() then gives the hipError_t (per thread).
 *     No C++ exception crosses this interface.
 *   - Thread safety: the library holds no state besides the per-thread last HIP error.
 *   - Precision: bf16 inputs, fp32 accumulation of both contractions and of the softmax state.
 *     In fa_fwd, P is rounded to bf16 (round to nearest even) for the P V contraction and O is
 *     divided by the fp32 sum of those rounded values (so O is a convex combination of the V
 *     rows); the LSE uses the fp32 sum of the unrounded p.  fa_decode keeps p in fp32
 *     throughout.  O is rounded to bf16 (round to nearest even) at the end; LSE is fp32.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,             /* a required pointer is NULL                                    */
  FA_ERR_SHAPE = 2,            /* a size is < 1, or too large for the kernels' 32-bit offsets   */
  FA_ERR_HEAD_DIM = 3,         /* d_head not a multiple of 8 in [8, 128] (fa_bwd_f32: not 64 or */
                               /* 128)                                                          */
  FA_ERR_CAUSAL_TQ_GT_TK = 4,  /* causal with Tq > Tk (a query row would see no key)            */
  FA_ERR_ALIGN = 5,            /* a tensor pointer is not 16-byte aligned (LSE: 4-byte)          */
  FA_ERR_SCALE = 6,            /* scale is not finite, or causal is not 0 / 1                   */
  FA_ERR_SPLITS = 7,           /* num_splits outside [1, min(Tk, FA_MAX_SPLITS)]                */
  FA_ERR_WORKSPACE = 8,        /* decode workspace NULL, misaligned or smaller than required     */
  FA_ERR_HIP = 9,              /* a HIP launch failed; see fa_last_hip_error()                  */
  FA_ERR_PROB = 10,            /* a dropout probability outside [0, 1)                          */
  FA_ERR_SCRATCH = 11          /* fa_decode_noalloc: partials beyond FA_NOALLOC_SCRATCH_BYTES   */
};

/* Largest per-head tensor the kernels address with 32-bit byte offsets: T * d_head * 2 bytes
 * (strided forward: (T + 128) * row_stride * 2 bytes) must stay below 2^31 (so T <= 8,388,607 at
 * d_head = 128, contiguous). */
#define FA_MAX_HEAD_BYTES 2147483647LL
/* Largest split count of the decode entry point. */
#define FA_MAX_SPLITS 256
/* Size of the static per-GPU array that holds fa_decode_noalloc's partials (32 MiB). */
#define FA_NOALLOC_SCRATCH_BYTES 33554432

/*
 * fa_fwd -- attention forward (prefill).
 *   q    [B][h][Tq][d_head] bf16        k, v [B][h][Tk][d_head] bf16
 *   o    [B][h][Tq][d_head] bf16 (out)  lse  [B][h][Tq] fp32 (out, natural log)
 *   causal = 1: query i sees key j iff j <= i + (Tk - Tq) (bottom-right aligned; with Tq == Tk
 *     the lower triangle including the diagonal).  Key tiles entirely above the diagonal are
 *     skipped and the diagonal tiles are masked on chip (page "Chapter 10 Writing and Benchmarking
 *     Custom Kernels", section 10.3.1, "What You Actually Decide in Practice": causal masking and
 *     the final partial tile).  causal = 0: every key is visible.
 *   scale multiplies Q K^T before the softmax (usually 1/sqrt(d_head)); it must be finite.
 *   d_head: any multiple of 8 from 8 to 128.  Head dimensions other than 64 and 128 run the
 *   64- or 128-wide kernel with the extra columns zero on chip (page "Chapter 10 Writing and
 *   Benchmarking Custom Kernels", section 10.3.1, "What You Actually Decide in Practice": pad
 *   d_head = 80 to 128 inside the kernel); the padding changes no result.
 *   Preconditions: B, h, Tq, Tk >= 1; d_head as above; causal => Tq <= Tk;
 *   q, k, v, o 16-byte aligned, lse 4-byte aligned; Tq*d_head*2 and Tk*d_head*2 <= FA_MAX_HEAD_BYTES.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head,
           int causal, float scale, void* stream);

/*
 * fa_fwd_o32 -- the same computation and kernel, with O stored in fp32 instead of bf16.
 *   o [B][h][Tq][d_head] fp32 (out).  For parity diagnostics: the bf16 output of fa_fwd is the
 *   round-to-nearest-even of this output, bit for bit.  Same preconditions as fa_fwd.
 */
int fa_fwd_o32(const void* q, const void* k, const void* v, float* o, float* lse,
               int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head,
               int causal, float scale, void* stream);

/*
 * fa_fwd_strided -- fa_fwd on strided tensors (layout variants).
 *   Element (b, h, t, c) of q is q[b*q_strides[0] + h*q_strides[1] + t*q_strides[2] + c], and
 *   likewise for k, v and o with their own strides (counted in elements; the last dimension is
 *   contiguous).  For example a [B][T][h][d] tensor has strides {T*h*d, d, h*d}.  lse stays
 *   contiguous [B][h][Tq] fp32; o is bf16.  Same computation, kernel and results as fa_fwd.
 *   Preconditions: as fa_fwd, and for each tensor: row stride >= d_head, every stride a
 *   non-negative multiple of 8 elements (rows stay 16-byte aligned), and
 *   (T + 128) * row_stride * 2 <= FA_MAX_HEAD_BYTES.  o must not overlap q, k, v or lse, and
 *   its strides must not make it overlap itself (FA_ERR_SHAPE otherwise; q, k, v may broadcast
 *   with stride 0).
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head,
                   const int64_t* q_strides, const int64_t* k_strides,
                   const int64_t* v_strides, const int64_t* o_strides,
                   int causal, float scale, void* stream);

/*
 * fa_decode_workspace_size -- bytes of device workspace fa_decode / fa_decode_strided need
 *   (the caller allocates it, as the host wrapper of page "Chapter 10 Writing and Benchmarking
 *   Custom Kernels", section 10.2.1, allocates the kernel's output before launching it):
 *   B * h * num_splits * (w + 2) fp32 partials (chunk max, denominator, w outputs), where w is
 *   the width the kernels compute in: 64 for d_head <= 64, 128 for d_head <= 128 (d_head
 *   itself when larger).  Returns 0 for sizes < 1.
 */
size_t fa_decode_workspace_size(int64_t B, int64_t h, int64_t d_head, int64_t num_splits);

/*
 * fa_decode -- split-KV decode: one query per (batch, head) against a KV cache, no mask.
 *   q [B][h][d_head] bf16; k, v [B][h][Tk][d_head] bf16; o [B][h][d_head] bf16 (out);
 *   lse [B][h] fp32 (out).  The Tk keys are cut into num_splits chunks of ceil(Tk/num_splits)
 *   keys; one pass computes each chunk's (max, denominator, unnormalised output) into
 *   `workspace`, a second pass rescales the chunks onto their common max and normalises
 *   (page "Fusion and IO-aware kernels", "Where it breaks": decode is KV-cache bound and is split
 *   across the sequence; the merge is the rescale of the online-softmax recurrence).
 *   The result does not depend on num_splits beyond rounding.  d_head as fa_fwd (any multiple
 *   of 8 in [8, 128], padded to 64 or 128 with zeros on chip).
 *   Preconditions: as fa_fwd for pointers and sizes; 1 <= num_splits <= min(Tk, FA_MAX_SPLITS);
 *   workspace 16-byte aligned with workspace_bytes >= fa_decode_workspace_size(B, h, d_head,
 *   num_splits).  The workspace holds no state between calls; calls that may run at the same
 *   time (on different streams) need separate workspaces.
 */
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int64_t B, int64_t h, int64_t Tk, int64_t d_head, float scale,
              int64_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_noalloc -- fa_decode without a workspace argument, for callers that cannot allocate
 *   device memory (code under graph capture, tight serving loops, harnesses that forbid
 *   allocation).  The per-split partials go to a static array of FA_NOALLOC_SCRATCH_BYTES that
 *   the library's code object holds on each GPU it runs on until the process ends; the call
 *   itself allocates nothing.  Same arguments (less the workspace), kernels and results as
 *   fa_decode, bit for bit.
 *   Errors: as fa_decode, and FA_ERR_SCRATCH (nothing enqueued, outputs untouched) when
 *   fa_decode_workspace_size(B, h, d_head, num_splits) exceeds FA_NOALLOC_SCRATCH_BYTES
 *   (e.g. B = 64, h = 32, d_head = 128 allows up to 31 splits).  The first call on a device
 *   looks up that device's address of the array (a HIP call; failure gives FA_ERR_HIP).
 *   All calls on one GPU share its array: calls that overlap in time on one GPU (different
 *   streams, or unordered threads) race on it and give undefined results.  Nothing in the
 *   array needs clearing between calls: each call writes every partial it reads.
 */
int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t h, int64_t Tk, int64_t d_head, float scale,
                      int64_t num_splits, void* stream);

/*
 * fa_decode_strided -- fa_decode on strided tensors and any head dim (layout variants).
 *   Element (b, h, c) of q is q[b*q_strides[0] + h*q_strides[1] + c], likewise o with
 *   o_strides; element (b, h, t, c) of k is k[b*k_strides[0] + h*k_strides[1] + t*k_strides[2]
 *   + c], likewise v (strides in elements; the last dimension contiguous), e.g. a [B][Tk][h][d]
 *   KV cache has strides {Tk*h*d, d, h*d}.  d_head may be any multiple of 8 in [8, 128]: the
 *   kernels pad it to 64 or 128 with zeros on chip.  lse stays contiguous [B][h] fp32.  Same
 *   method, kernels and results as fa_decode (bit for bit for contiguous d_head 64 / 128).
 *   Preconditions: as fa_decode, with d_head as above; q, k, v 16-byte aligned, o 2-byte
 *   aligned; every stride a non-negative multiple of 8 elements; k and v row strides >= d_head
 *   with (Tk + 256) * row_stride * 2 <= FA_MAX_HEAD_BYTES; o must not overlap the inputs, and
 *   its strides must not make it overlap itself (FA_ERR_SHAPE otherwise).
 */
int fa_decode_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t h, int64_t Tk, int64_t d_head,
                      const int64_t* q_strides, const int64_t* k_strides,
                      const int64_t* v_strides, const int64_t* o_strides, float scale,
                      int64_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd / fa_bwd_f32 need: two fp32 values
 *   per query row (D_i and LSE_i * log2(e)), each array starting on a 256-byte boundary, then
 *   1024 bytes of work counters for the dQ kernel's item queues (zeroed by the backward itself
 *   on every call).  Returns 0 for sizes < 1.
 */
size_t fa_bwd_workspace_size(int64_t B, int64_t h, int64_t Tq);

/*
 * fa_bwd -- attention backward: the gradients of sum(dout * O) with respect to q, k and v,
 *   where O, lse are fa_fwd's outputs for the same q, k, v, causal and scale.
 *   q, o, dout [B][h][Tq][d_head] bf16; k, v [B][h][Tk][d_head] bf16; lse [B][h][Tq] fp32
 *   (natural log, as fa_fwd writes it);
 *   dq [B][h][Tq][d_head], dk, dv [B][h][Tk][d_head] bf16 (out).
 *   The method is the recomputing backward of page "Chapter 10 Writing and Benchmarking Custom
 *   Kernels", section 10.3.2: S = scale q k^T is recomputed tile by tile, P = exp(S - lse) is
 *   rebuilt from the stored log-sum-exp, D_i = <dout_i, O_i>, dP = dout v^T and
 *   dS = P (dP - D); then dv = P^T dout, dk = scale dS^T q, dq = scale dS k.  Nothing of size
 *   Tq x Tk is stored.  Masking as in fa_fwd (causal: query i sees key j iff j <= i + Tk - Tq).
 *   Precision: bf16 inputs, fp32 accumulation; P and dS are rounded to bf16 (round to nearest
 *   even) as operands of the gradient products; outputs rounded to bf16.  The result is
 *   deterministic (no atomic accumulation; which CU computes an item does not change its
 *   bits): the same inputs give the same bits.
 *   d_head as fa_fwd (any multiple of 8 in [8, 128], padded to 64 or 128 with zeros on chip).
 *   Preconditions: as fa_fwd for sizes and alignment (all tensors 16-byte aligned, lse 4-byte);
 *   workspace 16-byte aligned with workspace_bytes >= fa_bwd_workspace_size(B, h, Tq); the
 *   outputs and the workspace must not overlap the inputs or each other.  Every element of dq,
 *   dk and dv is written.  The workspace holds no state between calls; calls that may run at
 *   the same time (on different streams) need separate workspaces.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head, int causal,
           float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_f32 -- the same computation and kernels with dq, dk, dv stored in fp32 (parity
 *   diagnostics: fa_bwd's outputs are the round-to-nearest-even of these, bit for bit).
 *   d_head must be 64 or 128 (FA_ERR_HEAD_DIM otherwise); everything else as fa_bwd.
 */
int fa_bwd_f32(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, float* dq, float* dk, float* dv,
               int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head, int causal,
               float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_strided -- fa_bwd on strided tensors and any head dim (layout variants of the backward).
 *   Element (b, h, t, c) of each of q, k, v, o, dout, dq, dk, dv is at
 *   base[b*s[0] + h*s[1] + t*s[2] + c] with that tensor's strides s (elements; the last
 *   dimension is contiguous), e.g. {T*h*d, d, h*d} for [B][T][h][d] storage.  d_head may be any
 *   multiple of 8 in [8, 128]: the kernels pad it to 64 or 128 on chip with zeros, which
 *   changes no product.  lse stays contiguous [B][h][Tq] fp32; dq, dk, dv are bf16.  Same method,
 *   kernels and precision as fa_bwd; for contiguous tensors with d_head 64 or 128 the results are
 *   fa_bwd's bit for bit.
 *   Preconditions: as fa_bwd, with d_head as above, and for each tensor: row stride >= d_head,
 *   every stride a non-negative multiple of 8 elements, and
 *   (T + 128) * row_stride * 2 <= FA_MAX_HEAD_BYTES (T = Tq for q, o, dout, dq; Tk for k, v,
 *   dk, dv).  The outputs must not overlap the inputs, the workspace or each other, and the
 *   strides of dq, dk and dv must not make one overlap itself (FA_ERR_SHAPE otherwise).
 */
int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head,
                   const int64_t* q_strides, const int64_t* k_strides,
                   const int64_t* v_strides, const int64_t* o_strides,
                   const int64_t* do_strides, const int64_t* dq_strides,
                   const int64_t* dk_strides, const int64_t* dv_strides,
                   int causal, float scale, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * fa_softmax_rows -- row-wise softmax of a [rows][cols] fp32 matrix, in one pass over HBM.
 *   x [rows][cols] fp32 (in); y [rows][cols] fp32 (out); lse [rows] fp32 (out, natural log) or
 *   NULL.  y_ij = exp(x_ij - m_i) / sum_k exp(x_ik - m_i) with m_i the row max, and
 *   lse_i = m_i + log(sum_k exp(x_ik - m_i)).  The workload of page "Chapter 10 Writing and
 *   Benchmarking Custom Kernels", section 10.2.2 (the worked example: one block per row, the max
 *   subtracted before exponentiating), computed with the running (max, sum) recurrence of that
 *   section's closing question and of page "Kernels -- fusion and FlashAttention", section 3:
 *   partial sums are rescaled by exp(m_part - m_new) when merged.  Rows of up to 8192 columns
 *   are read once and written once; wider rows are read twice (the (max, sum) pass, then the
 *   output pass).
 *   Entries equal to -inf are masked (y = 0).  A row with no finite entry, or one holding +inf or
 *   NaN, has no defined softmax and its outputs are unspecified.
 *   Preconditions: rows, cols >= 1, cols <= INT32_MAX, (rows + 3) / 4 <= INT32_MAX; x, y (and lse)
 *   4-byte aligned; y must not overlap x.  16-byte aligned x and y with cols % 4 == 0 take the
 *   vector path.
 */
int fa_softmax_rows(const float* x, float* y, float* lse, int64_t rows, int64_t cols,
                    void* stream);

/*
 * fa_gelu_f32, fa_gelu_bf16 -- y = gelu(x) elementwise over n contiguous values, in one pass over
 *   HBM (one read, one write per element).  GELU in the tanh form of page "Chapter 10 Writing and
 *   Benchmarking Custom Kernels", section 10.2.1 (the GeLU case study, whose workload is 64M fp32
 *   values): gelu(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), computed in fp32 as
 *   x / (1 + exp(-2 sqrt(2/pi) (x + 0.044715 x^3))).  fa_gelu_bf16 reads and writes bf16 (round
 *   to nearest even), computing in fp32.
 *   Preconditions: n >= 1; x, y 16-byte aligned; y equal to x or not overlapping it.
 */
int fa_gelu_f32(const float* x, float* y, int64_t n, void* stream);
int fa_gelu_bf16(const void* x, void* y, int64_t n, void* stream);

/*
 * fa_bias_gelu_dropout_bf16 -- the fused chain y = dropout(gelu(x + bias)) over a row-major
 *   [rows][cols] bf16 activation with one bf16 bias per column (page "Fusion and IO-aware
 *   kernels", "The idea in one minute": bias add, GELU and dropout as one kernel that reads x once
 *   and writes y once).  Arithmetic in fp32, y rounded to bf16 (round to nearest even).
 *   Dropout: element e = row * cols + col draws 16 bits, half e % 2 (low 16 bits for even e,
 *   high for odd) of word (e % 8) / 2 of Philox4x32-10 (Salmon et al., "Parallel random
 *   numbers: as easy as 1, 2, 3", SC 2011) at counter (e / 8 low 32 bits, e / 8 high 32 bits,
 *   offset low, offset high) and key (seed low, seed high); it is dropped (y = 0) iff that value
 *   is below floor(p * 2^16), else y = gelu(x + bias) * (1 / (1 - p)) with the factor rounded to
 *   fp32.  The drop probability is p to within 2^-16.  The same (seed, offset) reproduces the
 *   same mask bit for bit.
 *   Preconditions: rows, cols >= 1; 0 <= p < 1 (else FA_ERR_PROB); x, bias, y 2-byte aligned
 *   (16-byte aligned with cols % 8 == 0 and rows <= 65535 takes the vector path); y equal to x
 *   or not overlapping it.
 */
int fa_bias_gelu_dropout_bf16(const void* x, const void* bias, void* y, int64_t rows,
                              int64_t cols, float p, uint64_t seed, uint64_t offset, void* stream);

/* Host-only argument checks used by fa_fwd / fa_fwd_o32, fa_fwd_strided, fa_decode(_strided),
 * fa_bwd / fa_bwd_f32, fa_bwd_strided, fa_softmax_rows, fa_gelu_* and fa_bias_gelu_dropout_bf16
 * (no HIP call is made).  Return FA_OK or the FA_ERR_* code the entry point would return
 * (fa_validate_bwd checks fa_bwd's rules; fa_bwd_f32 also needs d_head 64 or 128).
 * They are the checking half of the host wrapper of page "Chapter 10 Writing and Benchmarking
 * Custom Kernels", section 10.2.1 (check the inputs, allocate the output, size the grid by
 * ceiling division, launch), returning a status code where that wrapper raises; the strided
 * checks also reject an output whose strides make it overlap itself (a stride of 0 or one
 * inside the span of a smaller one), which inputs may do (e.g. one K/V head broadcast to
 * several query heads). */
int fa_validate_bwd(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, const void* dq, const void* dk,
                    const void* dv, int64_t B, int64_t h, int64_t Tq, int64_t Tk,
                    int64_t d_head, int causal, float scale, const void* workspace,
                    size_t workspace_bytes);
int fa_validate_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, const void* dq, const void* dk,
                            const void* dv, int64_t B, int64_t h, int64_t Tq, int64_t Tk,
                            int64_t d_head, const int64_t* q_strides, const int64_t* k_strides,
                            const int64_t* v_strides, const int64_t* o_strides,
                            const int64_t* do_strides, const int64_t* dq_strides,
                            const int64_t* dk_strides, const int64_t* dv_strides, int causal,
                            float scale, const void* workspace, size_t workspace_bytes);
int fa_validate_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head,
                    int causal, float scale);
int fa_validate_fwd_strided(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, int64_t B, int64_t h, int64_t Tq, int64_t Tk,
                            int64_t d_head, const int64_t* q_strides, const int64_t* k_strides,
                            const int64_t* v_strides, const int64_t* o_strides, int causal,
                            float scale);
int fa_validate_decode_strided(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, int64_t B, int64_t h, int64_t Tk,
                               int64_t d_head, const int64_t* q_strides,
                               const int64_t* k_strides, const int64_t* v_strides,
                               const int64_t* o_strides, float scale, int64_t num_splits,
                               const void* workspace, size_t workspace_bytes);
int fa_validate_decode(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, int64_t B, int64_t h, int64_t Tk, int64_t d_head,
                       float scale, int64_t num_splits, const void* workspace,
                       size_t workspace_bytes);
int fa_validate_softmax(const float* x, const float* y, const float* lse, int64_t rows,
                        int64_t cols);
int fa_validate_gelu(const void* x, const void* y, int64_t n);
int fa_validate_bias_gelu_dropout(const void* x, const void* bias, const void* y, int64_t rows,
                                  int64_t cols, float p);

/* Static, NUL-terminated description of a status code (never NULL): the message of the failed
 * check, which the wrapper of page "Chapter 10 Writing and Benchmarking Custom Kernels", section
 * 10.2.1 raises as an exception and the Python binding raises from this string. */
const char* fa_status_str(int status);

/* The hipError_t behind this thread's last FA_ERR_HIP (0 if none): the launch-error check that
 * follows the kernel launch in that wrapper. */
int fa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
