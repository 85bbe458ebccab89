// Calibration microbenchmarks for gfx950: the ceilings the attention kernels run against.
//   mfma   : dense bf16 v_mfma_f32_32x32x16_bf16 throughput (8 independent accumulators / wave)
//   exp    : v_exp_f32 throughput (16 independent chains / lane, x <- 2^-x stays in [0.5, 1])
//   lds    : ds_read_b128 and ds_read_b64_tr_b16 bandwidth (conflict-free addresses)
//   ldsmfma: MFMAs whose A operands stream from LDS (random bf16 data), with or without
//            operand reuse and a share of fma/exp vector work, at two waves per SIMD
//   hbm    : streaming read of a large buffer with 16-byte loads (grid-stride, and in
//            contiguous 128 KB blocks per 16-wave workgroup)
//   atomic : fp32 atomic adds (no return value) into an L2-sized or an HBM-sized buffer
//   clock  : shader clock from s_memtime against the 100 MHz s_memrealtime counter
// Every kernel reads and writes only inside the buffers it is given.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// NACC independent accumulator chains per wave; wave 0 of block 0 records the shader clock
// (s_memtime) and the 100 MHz reference (s_memrealtime) around its loop.
template <int NACC>
__global__ __launch_bounds__(256) void k_mfma(float* out, int iters, unsigned long long* clk) {
  const int l = threadIdx.x;
  bf16x8_t a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (l + j));
    b[j] = (__bf16)(0.002f * (l - j));
  }
  f32x16_t c[NACC];
  for (int i = 0; i < NACC; ++i) c[i] = f32x16_t{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NACC; ++i)
      c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int i = 0; i < NACC; ++i)
    for (int j = 0; j < 16; ++j) s += c[i][j];
  out[blockIdx.x * blockDim.x + l] = s;
  if (blockIdx.x == 0 && l == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

__global__ __launch_bounds__(256) void k_exp(float* out, int iters) {
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = 0.5f + 0.01f * i + 1e-6f * threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// VALU throughput of one opcode: 16 independent chains per lane.
//   op 0: v_add_f32, 1: v_fma_f32, 2: v_dot2c_f32_bf16, 3: v_cvt_pk_bf16_f32 (+ v_add to chain),
//   4: v_max3_f32
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <int OP>
__global__ __launch_bounds__(256) void k_valu(float* out, int iters) {
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = 0.5f + 0.01f * i + 1e-6f * threadIdx.x;
  const float c = 1.0000001f, d = -0.0000001f;
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (OP == 0) x[i] = x[i] + d;
      if (OP == 1) x[i] = __builtin_fmaf(x[i], c, d);
      if (OP == 2) {
        const uint32_t u = __builtin_bit_cast(uint32_t, x[i]) & 0x3F803F80u;
        x[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u), ones, x[i], false);
      }
      if (OP == 3) {
        typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        f2 f = {x[i], x[(i + 1) & 15]};
        bf16x2v h = __builtin_convertvector(f, bf16x2v);
        x[i] = __builtin_bit_cast(float, h);
      }
      if (OP == 4) x[i] = fmaxf(fmaxf(x[i], x[(i + 1) & 15]), x[(i + 2) & 15]) * c;
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// MFMA / VALU co-execution: 512-thread workgroups (two waves per SIMD); waves 0-3 run an MFMA
// loop (4 accumulator chains), waves 4-7 an fp32 FMA + v_exp loop.  mode 0 runs both, 1 only
// the MFMA waves, 2 only the VALU waves.
__global__ __launch_bounds__(512) void k_coexec(float* out, int mfma_iters, int valu_iters,
                                                int mode) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  float s = 0.f;
  if (w < 4) {
    if (mode == 2) return;
    bf16x8_t a, b;
    for (int j = 0; j < 8; ++j) {
      a[j] = (__bf16)(0.001f * (l + j));
      b[j] = (__bf16)(0.002f * (l - j));
    }
    f32x16_t c[4];
    for (int i = 0; i < 4; ++i) c[i] = f32x16_t{};
    for (int it = 0; it < mfma_iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
    }
    for (int i = 0; i < 4; ++i)
      for (int j = 0; j < 16; ++j) s += c[i][j];
  } else {
    if (mode == 1) return;
    float x[8];
    for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.01f * i + 1e-6f * l;
    for (int it = 0; it < valu_iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-__builtin_fmaf(x[i], 0.999f, 0.001f));
    }
    for (int i = 0; i < 8; ++i) s += x[i];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// LDS: 64 KB per workgroup; lane l of wave w reads 16 bytes at ((w*64 + l + 64*k) * 16) mod 64 KB.
__global__ __launch_bounds__(256) void k_lds_b128(uint32_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t sm[16384];
  for (int i = threadIdx.x; i < 16384; i += 256) sm[i] = i * 2654435761u;
  __syncthreads();
  uint32_t acc0 = 0, acc1 = 0;
  const uint32_t base = threadIdx.x * 16u;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t addr = (base + (uint32_t)k * 4096u + (uint32_t)it * 64u) & 0xFFF0u;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(sm) + addr);
      acc0 = acc0 ^ v[0] ^ v[1];
      acc1 = acc1 ^ v[2] ^ v[3];
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc0 + acc1;
}

__global__ __launch_bounds__(256) void k_lds_tr(uint32_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint16_t sm[32768];
  for (int i = threadIdx.x; i < 32768; i += 256) sm[i] = (uint16_t)(i * 40503u);
  __syncthreads();
  typedef __attribute__((address_space(3))) s16x4_t* lp;
  uint32_t acc = 0;
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // element offset: 16 rows x 64 elements tile, 8-byte chunks, inside 32768 elements
      const uint32_t e = ((lane % 16) * 64 + (lane / 16) * 4 + wave * 1024 + k * 4096 +
                          (uint32_t)(it & 3) * 16) & 32767u;
      const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(sm + e));
      acc ^= (uint32_t)(uint16_t)v[0] ^ ((uint32_t)(uint16_t)v[3] << 16);
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// MFMA fed from LDS, the prefill forward's operand mix: 128 KB of random bf16 in LDS (one
// workgroup per CU), every A operand a row read (ds_read_b128) or a transposing read (two
// ds_read_b64_tr_b16), alternately, through an 8-deep register ring; B operands in registers.
// REUSE = 1: each A operand feeds one MFMA (a wave owning 32 query rows); REUSE = 2: two MFMAs
// with two B operands (a wave owning 64).  NV vector instructions per 16 MFMAs, 16 of them
// v_exp_f32 when NV > 0, the rest v_fma_f32.  All LDS addresses stay inside the 128 KB array.
template <int REUSE, int NV>
__global__ __launch_bounds__(512) void k_lds_mfma(float* out, int iters) {
  __shared__ __attribute__((aligned(1024))) uint16_t sm[65536];
  for (int i = threadIdx.x; i < 65536; i += blockDim.x) {
    uint32_t h = (uint32_t)i * 2654435761u + blockIdx.x * 40503u;
    h ^= h >> 15;
    h *= 2246822519u;
    h ^= h >> 13;
    sm[i] = (uint16_t)(0x3f00u | (h & 0x807fu));   // +-[0.5, 1) with random mantissas
  }
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t base = (uint32_t)reinterpret_cast<uintptr_t>(sm);
  const uint32_t r32 = lane & 31, g = lane >> 5;
  // row reads: 256-byte rows, chunk XOR-swizzled by row (conflict-free); at most 57.6 KB + 8 KB
  uint32_t ra = base + (w & 3) * 16384u + r32 * 256u + 16u * (g ^ (r32 & 15));
  // transposing reads: 16-lane groups read 4 rows x 16 bytes; at most 82 KB
  const uint32_t x = (lane & 15) >> 2, dh = (lane >> 4) & 1, r = 4 * g + x;
  uint32_t ta = base + (w & 3) * 16384u + r * 256u +
                16u * ((2 * dh + ((lane & 3) >> 1)) ^ (4 * (r & 3))) + 8u * (lane & 1);
  asm volatile("" : "+v"(ra), "+v"(ta));
  constexpr int NACC = REUSE == 1 ? 4 : 8, NA = 16 / REUSE, RING = 8;
  f32x16_t acc[NACC];
  for (int i = 0; i < NACC; ++i) acc[i] = f32x16_t{};
  bf16x8_t b[2];
  for (int j = 0; j < 2; ++j)
    for (int i = 0; i < 8; ++i) {
      uint32_t h = (threadIdx.x * 16u + 8u * j + i) * 2654435761u;
      h ^= h >> 15;
      h *= 2246822519u;
      h ^= h >> 13;
      b[j][i] = __builtin_bit_cast(__bf16, (uint16_t)(0x3f00u | (h & 0x807fu)));
    }
  float xv[16];
  for (int i = 0; i < 16; ++i) xv[i] = 0.5f + 0.01f * i + 1e-6f * threadIdx.x;
  auto rd = [&](int i) -> bf16x8_t {
    typedef __attribute__((address_space(3))) s16x4_t* lp;
    if (i & 1) {
      const uint32_t a0 = ta + (uint32_t)((i >> 1) & 7) * 4096u + 64u * ((i >> 4) & 3);
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(uintptr_t)a0);
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(uintptr_t)(a0 + 2048));
      const u32x4_t v = {(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                         (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                         (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                         (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
      return __builtin_bit_cast(bf16x8_t, v);
    }
    const uint32_t a0 = (ra ^ (32u * ((i >> 1) & 7))) + 8192u * ((i >> 4) & 1);
    return *(__attribute__((address_space(3))) const bf16x8_t*)(uintptr_t)a0;
  };
  bf16x8_t ring[RING];
#pragma unroll
  for (int i = 0; i < RING; ++i) ring[i] = rd(i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const bf16x8_t av = ring[a % RING];
      ring[a % RING] = rd(a + RING);
#pragma unroll
      for (int u = 0; u < REUSE; ++u) {
        const int m = a * REUSE + u;
        acc[m % NACC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b[u], acc[m % NACC], 0, 0, 0);
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if (v < 16)
        xv[v & 15] = __builtin_amdgcn_exp2f(xv[v & 15]);
      else
        xv[v & 15] = __builtin_fmaf(xv[v & 15], 1.0000001f, -0.0000001f);
    }
    // per A operand: its MFMAs, each followed by NV / 16 vector instructions, then its reads
#pragma unroll
    for (int a = 0; a < NA; ++a) {
#pragma unroll
      for (int u = 0; u < REUSE; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (NV) __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, NV / 16, 0);
      }
      if (a & 1)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += xv[i] + acc[i % NACC][i];
  for (int i = 0; i < RING; ++i) s += (float)ring[i][i & 7];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Streaming read: thread t reads 16-byte chunks t, t + stride, ... of n16 chunks.
__global__ __launch_bounds__(256) void k_hbm_read(const u32x4_t* __restrict__ src, long n16,
                                                  uint32_t* out) {
  const long stride = (long)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
    const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a[0] ^ b[1] ^ c[2] ^ d[3] ^ a[3] ^ b[2] ^ c[1] ^ d[0];
  }
  for (; i < n16; i += stride) acc ^= src[i][0];
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Streaming read in contiguous blocks (the access pattern of the decode's split pass): workgroup
// g of 16 waves reads the 128 KB block g, each wave 8 KB as 8 consecutive 1 KB wave-wide loads,
// all issued before any is used.  The result feeds a store that never happens (the data are
// ones), so the loads cannot be dropped.
__global__ __launch_bounds__(1024) void k_hbm_read_blocked(const u32x4_t* __restrict__ src,
                                                           long n16, uint32_t* out) {
  const long base = (long)blockIdx.x * 8192 + (long)(threadIdx.x >> 6) * 512 + (threadIdx.x & 63);
  u32x4_t a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const long i = base + 64 * u;
    a[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) acc ^= a[u][u & 3];
  if (acc == 0x12345678u) out[0] = acc;
}

// fp32 atomic adds without a return value (global_atomic_add_f32): each wave adds to one
// 256-byte run of 64 floats per iteration; consecutive iterations of a wave move by a large odd
// stride, so the runs spread over the buffer.  n_mask = (floats in the buffer) - 1, a power of
// two minus one: every index stays inside the buffer.
__global__ __launch_bounds__(256) void k_atomic_add(float* buf, uint32_t n_mask, int iters) {
  const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6, lane = threadIdx.x & 63;
  uint32_t run = wave * 2654435761u;
  for (int it = 0; it < iters; ++it) {
    unsafeAtomicAdd(buf + (((run & ~63u) + lane) & n_mask), 1.0f);
    run += 40503u * 64u + 64u;
  }
}

__global__ void k_clock(unsigned long long* out, int spin) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  float x = threadIdx.x;
  for (int i = 0; i < spin; ++i) x = __builtin_fmaf(x, 0.999999f, 1e-7f);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = t1 - t0;
    out[1] = r1 - r0;
    out[2] = (unsigned long long)(x > 1e30f);
  }
}

extern "C" {
int calib_mfma(float* out, int blocks, int iters, int nacc, unsigned long long* clk, void* s) {
  const hipStream_t st = (hipStream_t)s;
  switch (nacc) {
    case 1: hipLaunchKernelGGL(k_mfma<1>, dim3(blocks), dim3(256), 0, st, out, iters, clk); break;
    case 2: hipLaunchKernelGGL(k_mfma<2>, dim3(blocks), dim3(256), 0, st, out, iters, clk); break;
    case 4: hipLaunchKernelGGL(k_mfma<4>, dim3(blocks), dim3(256), 0, st, out, iters, clk); break;
    default: hipLaunchKernelGGL(k_mfma<8>, dim3(blocks), dim3(256), 0, st, out, iters, clk); break;
  }
  return (int)hipGetLastError();
}
int calib_exp(float* out, int blocks, int iters, void* s) {
  hipLaunchKernelGGL(k_exp, dim3(blocks), dim3(256), 0, (hipStream_t)s, out, iters);
  return (int)hipGetLastError();
}
int calib_valu(float* out, int blocks, int iters, int op, void* s) {
  const hipStream_t st = (hipStream_t)s;
  switch (op) {
    case 0: hipLaunchKernelGGL(k_valu<0>, dim3(blocks), dim3(256), 0, st, out, iters); break;
    case 1: hipLaunchKernelGGL(k_valu<1>, dim3(blocks), dim3(256), 0, st, out, iters); break;
    case 2: hipLaunchKernelGGL(k_valu<2>, dim3(blocks), dim3(256), 0, st, out, iters); break;
    case 3: hipLaunchKernelGGL(k_valu<3>, dim3(blocks), dim3(256), 0, st, out, iters); break;
    default: hipLaunchKernelGGL(k_valu<4>, dim3(blocks), dim3(256), 0, st, out, iters); break;
  }
  return (int)hipGetLastError();
}
int calib_coexec(float* out, int blocks, int mfma_iters, int valu_iters, int mode, void* s) {
  hipLaunchKernelGGL(k_coexec, dim3(blocks), dim3(512), 0, (hipStream_t)s, out, mfma_iters,
                     valu_iters, mode);
  return (int)hipGetLastError();
}
int calib_lds_b128(uint32_t* out, int blocks, int iters, void* s) {
  hipLaunchKernelGGL(k_lds_b128, dim3(blocks), dim3(256), 0, (hipStream_t)s, out, iters);
  return (int)hipGetLastError();
}
int calib_lds_tr(uint32_t* out, int blocks, int iters, void* s) {
  hipLaunchKernelGGL(k_lds_tr, dim3(blocks), dim3(256), 0, (hipStream_t)s, out, iters);
  return (int)hipGetLastError();
}
int calib_lds_mfma(float* out, int blocks, int iters, int reuse, int nv, void* s) {
  const hipStream_t st = (hipStream_t)s;
#define FA_CALIB_LM(R, N)                                                                  \
  if (reuse == R && nv == N) {                                                             \
    hipLaunchKernelGGL((k_lds_mfma<R, N>), dim3(blocks), dim3(512), 0, st, out, iters);   \
    return (int)hipGetLastError();                                                         \
  }
  FA_CALIB_LM(1, 0) FA_CALIB_LM(2, 0) FA_CALIB_LM(1, 48) FA_CALIB_LM(2, 48) FA_CALIB_LM(1, 80)
  FA_CALIB_LM(2, 80)
#undef FA_CALIB_LM
  return (int)hipErrorInvalidValue;
}
int calib_hbm_read(const void* src, long n16, uint32_t* out, int blocks, void* s) {
  hipLaunchKernelGGL(k_hbm_read, dim3(blocks), dim3(256), 0, (hipStream_t)s,
                     (const u32x4_t*)src, n16, out);
  return (int)hipGetLastError();
}
int calib_hbm_read_blocked(const void* src, long n16, uint32_t* out, void* s) {
  const long blocks = (n16 + 8191) / 8192;
  hipLaunchKernelGGL(k_hbm_read_blocked, dim3((unsigned)blocks), dim3(1024), 0, (hipStream_t)s,
                     (const u32x4_t*)src, n16, out);
  return (int)hipGetLastError();
}
int calib_atomic_add(float* buf, unsigned int n_mask, int blocks, int iters, void* s) {
  hipLaunchKernelGGL(k_atomic_add, dim3(blocks), dim3(256), 0, (hipStream_t)s, buf, n_mask,
                     iters);
  return (int)hipGetLastError();
}
int calib_clock(unsigned long long* out, int spin, void* s) {
  hipLaunchKernelGGL(k_clock, dim3(1), dim3(64), 0, (hipStream_t)s, out, spin);
  return (int)hipGetLastError();
}
}
