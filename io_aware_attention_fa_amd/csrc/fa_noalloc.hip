// fa_decode_noalloc: the split-KV decode with its per-split partials kept in a static device
// array instead of a caller-provided workspace, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array lives in this file's device code object: each GPU the library runs on holds its own
// copy (FA_NOALLOC_SCRATCH_BYTES) until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the first call on a device
// looks up that device's address of the array with hipGetSymbolAddress, with the device
// current, and every later call on that device passes the remembered address to the kernels,
// exactly where fa_decode passes its workspace.
//
// Nothing has to start at zero: the split pass writes every (max, denominator, output) partial
// of every (batch, head, split), empty chunks included, before the combine pass of the same call
// reads them.  All calls on one GPU share its array, so calls that overlap in time on that GPU
// (on different streams, or from different threads without ordering) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_internal.hpp"

static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up once per device with that device current.
hipError_t device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int64_t B, int64_t h, int64_t Tk, int64_t d_head,
                                 float scale, int64_t num_splits, void* stream) {
  // Every check of fa_decode except the workspace's, which this entry point replaces by the
  // static array's size: a non-null, aligned stand-in with an unbounded size passes it.
  const int st = fa_validate_decode(q, k, v, o, lse, B, h, Tk, d_head, scale, num_splits,
                                    reinterpret_cast<const void*>(uintptr_t{256}),
                                    ~size_t{0});
  if (st != FA_OK) return st;
  if (fa_decode_workspace_size(B, h, d_head, num_splits) > FA_NOALLOC_SCRATCH_BYTES)
    return FA_ERR_SCRATCH;
  void* ws = nullptr;
  hipError_t e = device_scratch(&ws);
  if (e == hipSuccess) {
    fa::DecodeLaunch a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.workspace = static_cast<float*>(ws);
    a.B = static_cast<int>(B); a.H = static_cast<int>(h); a.Tk = static_cast<int>(Tk);
    a.d = static_cast<int>(d_head); a.num_splits = static_cast<int>(num_splits);
    a.scale = scale;
    // contiguous q, o [B][h][d] and k, v [B][h][Tk][d]
    a.q_s[0] = a.o_s[0] = h * d_head;
    a.q_s[1] = a.o_s[1] = d_head;
    a.k_s[0] = a.v_s[0] = h * Tk * d_head;
    a.k_s[1] = a.v_s[1] = Tk * d_head;
    a.k_s[2] = a.v_s[2] = d_head;
    e = fa::launch_decode(a, static_cast<hipStream_t>(stream));
  }
  if (e == hipSuccess) return FA_OK;
  fa::note_hip_error(static_cast<int>(e));
  return FA_ERR_HIP;
}
