// Launch descriptors shared by the host entry points (fa_host.cpp) and the kernel translation
// units.  Internal to the library; not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Tq, Tk, d;
  bool causal;
  bool out_f32;
  float scale;
  // element strides (batch, head, row) of q, k, v, o; the last dimension is contiguous
  int64_t q_s[3], k_s[3], v_s[3], o_s[3];
};

struct DecodeLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* workspace;
  int B, H, Tk, d, num_splits;
  float scale;
  // element strides: q and o (batch, head), k and v (batch, head, row); last dim contiguous
  int64_t q_s[2], o_s[2], k_s[3], v_s[3];
};

struct BwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* l2;   // workspace: LSE * log2(e) per query row
  float* dd;   // workspace: D_i = <dO_i, O_i> per query row
  uint32_t* ctr;   // workspace: 1 KB of item counters of the persistent kernels
  int B, H, Tq, Tk, d;
  bool causal;
  bool out_f32;
  float scale;
  // element strides (batch, head, row) of each tensor; the last dimension is contiguous
  int64_t q_s[3], k_s[3], v_s[3], o_s[3], do_s[3], dq_s[3], dk_s[3], dv_s[3];
};

struct SoftmaxLaunch {
  const float* x;
  float* y;
  float* lse;   // may be null
  int64_t rows, cols;
};

struct GeluLaunch {
  const void* x;
  void* y;
  int64_t n;
  bool bf16;
};

struct DropoutLaunch {
  const void* x;
  const void* bias;
  void* y;
  int64_t rows, cols;
  uint32_t threshold;   // floor(p * 2^16) * 2^16: drop iff the element's draw * 2^16 is below it
  float scale;          // 1 / (1 - p)
  uint64_t seed, offset;
};

// Records the hipError_t behind an FA_ERR_HIP for fa_last_hip_error() (per thread).
void note_hip_error(int hip_error);

hipError_t launch_fwd(const FwdLaunch& a, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream);
hipError_t launch_bwd(const BwdLaunch& a, hipStream_t stream);
hipError_t launch_softmax(const SoftmaxLaunch& a, hipStream_t stream);
hipError_t launch_gelu(const GeluLaunch& a, hipStream_t stream);
hipError_t launch_bias_gelu_dropout(const DropoutLaunch& a, hipStream_t stream);

}  // namespace fa
