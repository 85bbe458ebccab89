// C-ABI entry points: validate on the host, then enqueue the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>

#include "fa.h"
#include "fa_internal.hpp"

namespace {
thread_local int g_last_hip_error = 0;
}  // namespace

void fa::note_hip_error(int hip_error) { g_last_hip_error = hip_error; }

namespace {
int map_hip(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  fa::note_hip_error(static_cast<int>(e));
  return FA_ERR_HIP;
}

int fwd_launch(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
               int64_t h, int64_t Tq, int64_t Tk, int64_t d, const int64_t* qs,
               const int64_t* ks, const int64_t* vs, const int64_t* os, int causal, float scale,
               void* stream, bool out_f32) {
  fa::FwdLaunch a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = static_cast<int>(B); a.H = static_cast<int>(h);
  a.Tq = static_cast<int>(Tq); a.Tk = static_cast<int>(Tk); a.d = static_cast<int>(d);
  a.causal = causal != 0; a.out_f32 = out_f32; a.scale = scale;
  for (int i = 0; i < 3; ++i) {
    a.q_s[i] = qs[i]; a.k_s[i] = ks[i]; a.v_s[i] = vs[i]; a.o_s[i] = os[i];
  }
  return map_hip(fa::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
               int64_t h, int64_t Tq, int64_t Tk, int64_t d, int causal, float scale,
               void* stream, bool out_f32) {
  const int st = fa_validate_fwd(q, k, v, o, lse, B, h, Tq, Tk, d, causal, scale);
  if (st != FA_OK) return st;
  // contiguous [B][h][T][d]
  const int64_t qs[3] = {h * Tq * d, Tq * d, d}, ks[3] = {h * Tk * d, Tk * d, d};
  return fwd_launch(q, k, v, o, lse, B, h, Tq, Tk, d, qs, ks, ks, qs, causal, scale, stream,
                    out_f32);
}
}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head, int causal,
                      float scale, void* stream) {
  return fwd_common(q, k, v, o, lse, B, h, Tq, Tk, d_head, causal, scale, stream, false);
}

extern "C" int fa_fwd_o32(const void* q, const void* k, const void* v, float* o, float* lse,
                          int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head,
                          int causal, float scale, void* stream) {
  return fwd_common(q, k, v, o, lse, B, h, Tq, Tk, d_head, causal, scale, stream, true);
}

extern "C" int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head,
                              const int64_t* q_strides, const int64_t* k_strides,
                              const int64_t* v_strides, const int64_t* o_strides, int causal,
                              float scale, void* stream) {
  const int st = fa_validate_fwd_strided(q, k, v, o, lse, B, h, Tq, Tk, d_head, q_strides,
                                         k_strides, v_strides, o_strides, causal, scale);
  if (st != FA_OK) return st;
  return fwd_launch(q, k, v, o, lse, B, h, Tq, Tk, d_head, q_strides, k_strides, v_strides,
                    o_strides, causal, scale, stream, false);
}

namespace {
int decode_launch(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                  int64_t h, int64_t Tk, int64_t d, const int64_t* qs, const int64_t* ks,
                  const int64_t* vs, const int64_t* os, float scale, int64_t num_splits,
                  void* workspace, void* stream) {
  fa::DecodeLaunch a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.workspace = static_cast<float*>(workspace);
  a.B = static_cast<int>(B); a.H = static_cast<int>(h); a.Tk = static_cast<int>(Tk);
  a.d = static_cast<int>(d); a.num_splits = static_cast<int>(num_splits); a.scale = scale;
  for (int i = 0; i < 2; ++i) {
    a.q_s[i] = qs[i]; a.o_s[i] = os[i];
  }
  for (int i = 0; i < 3; ++i) {
    a.k_s[i] = ks[i]; a.v_s[i] = vs[i];
  }
  return map_hip(fa::launch_decode(a, static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t h, int64_t Tk, int64_t d_head, float scale,
                         int64_t num_splits, void* workspace, size_t workspace_bytes,
                         void* stream) {
  const int st = fa_validate_decode(q, k, v, o, lse, B, h, Tk, d_head, scale, num_splits,
                                    workspace, workspace_bytes);
  if (st != FA_OK) return st;
  // contiguous q, o [B][h][d] and k, v [B][h][Tk][d]
  const int64_t qs[2] = {h * d_head, d_head}, ks[3] = {h * Tk * d_head, Tk * d_head, d_head};
  return decode_launch(q, k, v, o, lse, B, h, Tk, d_head, qs, ks, ks, qs, scale, num_splits,
                       workspace, stream);
}

extern "C" int fa_decode_strided(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int64_t B, int64_t h, int64_t Tk, int64_t d_head,
                                 const int64_t* q_strides, const int64_t* k_strides,
                                 const int64_t* v_strides, const int64_t* o_strides, float scale,
                                 int64_t num_splits, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  const int st = fa_validate_decode_strided(q, k, v, o, lse, B, h, Tk, d_head, q_strides,
                                            k_strides, v_strides, o_strides, scale, num_splits,
                                            workspace, workspace_bytes);
  if (st != FA_OK) return st;
  return decode_launch(q, k, v, o, lse, B, h, Tk, d_head, q_strides, k_strides, v_strides,
                       o_strides, scale, num_splits, workspace, stream);
}

namespace {
// Enqueues the backward; strides s[8][3] of q, k, v, o, dout, dq, dk, dv (validated).
int bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t h, int64_t Tq,
               int64_t Tk, int64_t d, const int64_t* const s[8], int causal, float scale,
               void* workspace, void* stream, bool out_f32) {
  fa::BwdLaunch a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  // the workspace holds two arrays of B*h*Tq floats, each from a 256-byte boundary, then the
  // item counters
  const size_t arr = (static_cast<size_t>(B * h * Tq) * sizeof(float) + 255) / 256 * 256;
  a.l2 = static_cast<float*>(workspace);
  a.dd = reinterpret_cast<float*>(static_cast<char*>(workspace) + arr);
  a.ctr = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + 2 * arr);
  a.B = static_cast<int>(B); a.H = static_cast<int>(h);
  a.Tq = static_cast<int>(Tq); a.Tk = static_cast<int>(Tk); a.d = static_cast<int>(d);
  a.causal = causal != 0; a.out_f32 = out_f32; a.scale = scale;
  int64_t* dst[8] = {a.q_s, a.k_s, a.v_s, a.o_s, a.do_s, a.dq_s, a.dk_s, a.dv_s};
  for (int t = 0; t < 8; ++t)
    for (int i = 0; i < 3; ++i) dst[t][i] = s[t][i];
  return map_hip(fa::launch_bwd(a, static_cast<hipStream_t>(stream)));
}

int bwd_common(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t h, int64_t Tq,
               int64_t Tk, int64_t d, int causal, float scale, void* workspace,
               size_t workspace_bytes, void* stream, bool out_f32) {
  const int st = fa_validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, h, Tq, Tk, d, causal, scale,
                                 workspace, workspace_bytes);
  if (st != FA_OK) return st;
  // the fp32-output kernels exist for the unpadded head dims only
  if (out_f32 && d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  // contiguous [B][h][T][d]
  const int64_t qs[3] = {h * Tq * d, Tq * d, d}, ks[3] = {h * Tk * d, Tk * d, d};
  const int64_t* const s[8] = {qs, ks, ks, qs, qs, qs, ks, ks};
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, B, h, Tq, Tk, d, s, causal, scale,
                    workspace, stream, out_f32);
}
}  // namespace

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head, int causal,
                      float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, h, Tq, Tk, d_head, causal, scale,
                    workspace, workspace_bytes, stream, false);
}

extern "C" int fa_bwd_f32(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, float* dq, float* dk, float* dv,
                          int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head,
                          int causal, float scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, h, Tq, Tk, d_head, causal, scale,
                    workspace, workspace_bytes, stream, true);
}

extern "C" int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              int64_t B, int64_t h, int64_t Tq, int64_t Tk, int64_t d_head,
                              const int64_t* q_strides, const int64_t* k_strides,
                              const int64_t* v_strides, const int64_t* o_strides,
                              const int64_t* do_strides, const int64_t* dq_strides,
                              const int64_t* dk_strides, const int64_t* dv_strides, int causal,
                              float scale, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const int st = fa_validate_bwd_strided(
      q, k, v, o, dout, lse, dq, dk, dv, B, h, Tq, Tk, d_head, q_strides, k_strides, v_strides,
      o_strides, do_strides, dq_strides, dk_strides, dv_strides, causal, scale, workspace,
      workspace_bytes);
  if (st != FA_OK) return st;
  const int64_t* const s[8] = {q_strides,  k_strides,  v_strides,  o_strides,
                               do_strides, dq_strides, dk_strides, dv_strides};
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, B, h, Tq, Tk, d_head, s, causal, scale,
                    workspace, stream, false);
}

extern "C" int fa_softmax_rows(const float* x, float* y, float* lse, int64_t rows, int64_t cols,
                               void* stream) {
  const int st = fa_validate_softmax(x, y, lse, rows, cols);
  if (st != FA_OK) return st;
  fa::SoftmaxLaunch a;
  a.x = x; a.y = y; a.lse = lse; a.rows = rows; a.cols = cols;
  return map_hip(fa::launch_softmax(a, static_cast<hipStream_t>(stream)));
}

extern "C" int fa_gelu_f32(const float* x, float* y, int64_t n, void* stream) {
  const int st = fa_validate_gelu(x, y, n);
  if (st != FA_OK) return st;
  fa::GeluLaunch a;
  a.x = x; a.y = y; a.n = n; a.bf16 = false;
  return map_hip(fa::launch_gelu(a, static_cast<hipStream_t>(stream)));
}

extern "C" int fa_gelu_bf16(const void* x, void* y, int64_t n, void* stream) {
  const int st = fa_validate_gelu(x, y, n);
  if (st != FA_OK) return st;
  fa::GeluLaunch a;
  a.x = x; a.y = y; a.n = n; a.bf16 = true;
  return map_hip(fa::launch_gelu(a, static_cast<hipStream_t>(stream)));
}

extern "C" int fa_bias_gelu_dropout_bf16(const void* x, const void* bias, void* y, int64_t rows,
                                         int64_t cols, float p, uint64_t seed, uint64_t offset,
                                         void* stream) {
  const int st = fa_validate_bias_gelu_dropout(x, bias, y, rows, cols, p);
  if (st != FA_OK) return st;
  fa::DropoutLaunch a;
  a.x = x; a.bias = bias; a.y = y; a.rows = rows; a.cols = cols;
  // drop iff the element's 16-bit draw < floor(p * 2^16) (compared in the high half of a word,
  // so the threshold is scaled by 2^16); kept values scaled by 1 / (1 - p)
  const double t = std::floor(static_cast<double>(p) * 65536.0);
  a.threshold = static_cast<uint32_t>(t >= 65535.0 ? 65535.0 : t) << 16;
  a.scale = static_cast<float>(1.0 / (1.0 - static_cast<double>(p)));
  a.seed = seed; a.offset = offset;
  return map_hip(fa::launch_bias_gelu_dropout(a, static_cast<hipStream_t>(stream)));
}

extern "C" int fa_last_hip_error(void) { return g_last_hip_error; }
