// Row softmax and fused GELU for gfx950 (MI355X): the two memory-bound steps
// of the first page's kernel ladder ("Guia Pratico de Programacao de GPU com
// Tiles", Passo a Passo step 3 "GELU Fundido" and step 4 "Softmax por Linha").
// Both read their inputs from HBM once and write their output once; the
// arithmetic is in fp32 whatever the storage type (fp32 or bf16).
//
// Softmax: out[r, :] = exp(x[r, :] - max) / sum(exp(x[r, :] - max)), one
// workgroup per row (256 threads, 512 above 4096 columns, where the wider
// workgroup was 1-11% faster).  Rows of up to 16384 columns stay in
// registers between the max, the sum and the store (one read, one write);
// longer rows take an online max/sum pass and a second pass that writes.
// Reductions: xor shuffles inside a wave, then LDS across the 4 waves.
// exp(t) is computed as exp2(t * log2 e) with the hardware exp2, and the
// division by the sum as one correctly rounded reciprocal per row times each
// numerator.
//
// GELU: h = x * w + b elementwise, out = 0.5 h (1 + tanh(c (h + 0.044715 h^3))),
// c = sqrt(2/pi).  0.5 (1 + tanh(z)) equals 1 / (1 + exp(-2z)), so the kernel
// evaluates out = h / (1 + exp(-2z)), which stays finite for every z (written
// with exp(-2z) as numerator and denominator, as on the page, the tanh is
// inf/inf for z below about -44 in fp32).  Grid-stride loop over 16-byte
// pieces of the four arrays, nontemporal loads and stores, one workgroup
// per CU.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "tileattn.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kVec = 8;        // elements per thread per access
constexpr int kRowChunk = kThreads * kVec;
constexpr float kLog2e = 1.4426950408889634f;
constexpr long long kGeluWorkgroups = 256;
#ifndef TILEATTN_SOFTMAX_F32_WIDE
#define TILEATTN_SOFTMAX_F32_WIDE 512
#endif
#ifndef TILEATTN_SOFTMAX_BF16_WIDE
#define TILEATTN_SOFTMAX_BF16_WIDE 512
#endif

// Streaming data is read and written once: nontemporal hints keep it from
// displacing cached lines, and on this part they also raise the sustained
// HBM rate of these kernels.
__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

struct F32 {
  using T = float;
  static constexpr int kBytes = 4;
  static constexpr int kPer16 = 4;    // elements per 16 bytes
  static constexpr int kWideThreads = TILEATTN_SOFTMAX_F32_WIDE;  // threads per row above 4096 columns
  static constexpr int kUnroll = 2;   // 16-byte accesses per array in flight per thread (GELU)
  static constexpr bool kRcpDiv = false;  // GELU divides correctly rounded (see gelu_tanh)
  __device__ static void widen16(u32x4 u, float (&v)[kPer16]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(u[e]);
  }
  __device__ static u32x4 narrow16(const float (&v)[kPer16]) {
    return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  }
  __device__ static void load8(const float* p, float (&v)[kVec]) {
    const f32x4 a = __builtin_bit_cast(f32x4, ld_nt(p));
    const f32x4 b = __builtin_bit_cast(f32x4, ld_nt(p + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[e + 4] = b[e];
    }
  }
  __device__ static void store8(float* p, const float (&v)[kVec]) {
    st_nt(p, __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}));
    st_nt(p + 4, __builtin_bit_cast(u32x4, f32x4{v[4], v[5], v[6], v[7]}));
  }
  __device__ static float load1(const float* p) { return *p; }
  __device__ static void store1(float* p, float v) { *p = v; }
};

struct BF16 {
  using T = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kPer16 = 8;
  static constexpr int kUnroll = 4;
  static constexpr bool kRcpDiv = true;
  static constexpr int kWideThreads = TILEATTN_SOFTMAX_BF16_WIDE;
  __device__ static float widen(uint16_t u) { return __uint_as_float((unsigned)u << 16); }
  __device__ static uint16_t narrow(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }  // RNE
  __device__ static void widen16(u32x4 u, float (&v)[kPer16]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(u[e] << 16);
      v[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
  }
  __device__ static u32x4 narrow16(const float (&v)[kPer16]) {
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (unsigned)narrow(v[2 * e]) | ((unsigned)narrow(v[2 * e + 1]) << 16);
    return u;
  }
  __device__ static void load8(const uint16_t* p, float (&v)[kVec]) {
    const u32x4 u = ld_nt(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(u[e] << 16);
      v[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
  }
  __device__ static void store8(uint16_t* p, const float (&v)[kVec]) {
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (unsigned)narrow(v[2 * e]) | ((unsigned)narrow(v[2 * e + 1]) << 16);
    st_nt(p, u);
  }
  __device__ static float load1(const uint16_t* p) { return widen(*p); }
  __device__ static void store1(uint16_t* p, float v) { *p = narrow(v); }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Workgroup reductions over NW waves: every thread gets the result.  `red`
// holds NW floats.
template <int NW>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red may still be read by an earlier reduction
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w]);
  return r;
}
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += red[w];
  return r;
}

// Rows held in registers: CH chunks of 8 elements per thread
// (n_cols <= CH * 8 * THREADS).
template <typename IO, int CH, int THREADS>
__global__ __launch_bounds__(THREADS) void softmax_rows_kernel(const typename IO::T* x,
                                                               typename IO::T* out, int n_cols,
                                                               long long stride) {
  using T = typename IO::T;
  constexpr int NW = THREADS / 64;
  __shared__ float red[NW];
  const size_t row = blockIdx.x;
  const T* xr = x + row * (size_t)stride;
  T* orow = out + row * (size_t)stride;
  const int tid = threadIdx.x;
  float v[CH][kVec];
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = (c * THREADS + tid) * kVec;
    if (col + kVec <= n_cols) {
      IO::load8(xr + col, v[c]);
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e) v[c][e] = (col + e < n_cols) ? IO::load1(xr + col + e) : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) mx = fmaxf(mx, v[c][e]);
  }
  mx = block_max<NW>(mx, red);
  const float mc = mx * kLog2e;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      v[c][e] = __builtin_amdgcn_exp2f(fmaf(v[c][e], kLog2e, -mc));
      s += v[c][e];
    }
  s = block_sum<NW>(s, red);
  const float inv = 1.0f / s;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = (c * THREADS + tid) * kVec;
#pragma unroll
    for (int e = 0; e < kVec; ++e) v[c][e] *= inv;
    if (col + kVec <= n_cols) {
      IO::store8(orow + col, v[c]);
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        if (col + e < n_cols) IO::store1(orow + col + e, v[c][e]);
    }
  }
}

// Rows too long for registers: pass 1 keeps a running max and a running sum
// per thread (the sum rescaled by exp(m_old - m_new) when the max rises),
// merges them across the workgroup, and pass 2 re-reads the row and writes.
template <typename IO>
__global__ __launch_bounds__(kThreads) void softmax_rows_online_kernel(const typename IO::T* x,
                                                                       typename IO::T* out, int n_cols,
                                                                       long long stride) {
  using T = typename IO::T;
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const T* xr = x + row * (size_t)stride;
  T* orow = out + row * (size_t)stride;
  const int tid = threadIdx.x;
  auto load = [&](int col, float (&v)[kVec]) {
    if (col + kVec <= n_cols) {
      IO::load8(xr + col, v);
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e) v[e] = (col + e < n_cols) ? IO::load1(xr + col + e) : -INFINITY;
    }
  };
  float m = -INFINITY, s = 0.f;
  for (int col = tid * kVec; col < n_cols; col += kRowChunk) {
    float v[kVec];
    load(col, v);
    float lm = v[0];
#pragma unroll
    for (int e = 1; e < kVec; ++e) lm = fmaxf(lm, v[e]);
    const float mn = fmaxf(m, lm);
    if (mn == -INFINITY) continue;  // nothing finite seen yet
    s *= __builtin_amdgcn_exp2f((m - mn) * kLog2e);  // m = -inf: s is 0 and stays 0
    const float mc = mn * kLog2e;
#pragma unroll
    for (int e = 0; e < kVec; ++e) s += __builtin_amdgcn_exp2f(fmaf(v[e], kLog2e, -mc));
    m = mn;
  }
  const float M = block_max<4>(m, red);
  const float scaled = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
  const float S = block_sum<4>(scaled, red);
  const float inv = 1.0f / S;
  const float Mc = M * kLog2e;
  for (int col = tid * kVec; col < n_cols; col += kRowChunk) {
    float v[kVec];
    load(col, v);
#pragma unroll
    for (int e = 0; e < kVec; ++e) v[e] = __builtin_amdgcn_exp2f(fmaf(v[e], kLog2e, -Mc)) * inv;
    if (col + kVec <= n_cols) {
      IO::store8(orow + col, v);
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        if (col + e < n_cols) IO::store1(orow + col + e, v[e]);
    }
  }
}

// tanh-approximate GELU of h, as h * sigmoid(2z), z = c (h + 0.044715 h^3).
// RCP: h times the hardware reciprocal (v_rcp_f32, about 1 ulp) instead of
// the correctly rounded division, whose fix-up sequence makes the 16-bit
// kernel issue-bound.  The extra ulp in fp32 is far below the half ulp of
// the 16-bit rounding that follows; the edge cases are unchanged (1 + e is
// 1 or more, or +inf, whose reciprocal is 0 as in h / inf).
template <bool RCP>
__device__ __forceinline__ float gelu_tanh(float h) {
  constexpr float kC = 0.7978845608028654f;  // sqrt(2/pi)
  const float z = kC * fmaf(0.044715f * h, h * h, h);
  const float den = 1.0f + __builtin_amdgcn_exp2f(-2.0f * kLog2e * z);
  return RCP ? h * __builtin_amdgcn_rcpf(den) : h / den;
}

// One 16-byte piece of every array per access; each thread keeps
// IO::kUnroll accesses, a grid stride apart, in flight.  One workgroup per
// CU: on this part fewer, deeper streams sustain a higher HBM rate than a
// full grid (the concurrently touched window of each array stays small).
template <typename IO>
__global__ __launch_bounds__(kThreads) void gelu_kernel(const typename IO::T* x, const typename IO::T* w,
                                                        const typename IO::T* b, typename IO::T* out,
                                                        long long n) {
  constexpr int P = IO::kPer16, U = IO::kUnroll;
  const long long pieces = n / P;
  const long long step = (long long)gridDim.x * kThreads;
  long long g = (long long)blockIdx.x * kThreads + threadIdx.x;
  for (; g + (U - 1) * step < pieces; g += U * step) {
    u32x4 xv[U], wv[U], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xv[u] = ld_nt(x + (g + u * step) * P);
      wv[u] = ld_nt(w + (g + u * step) * P);
      bv[u] = ld_nt(b + (g + u * step) * P);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xf[P], wf[P], bf[P];
      IO::widen16(xv[u], xf);
      IO::widen16(wv[u], wf);
      IO::widen16(bv[u], bf);
#pragma unroll
      for (int e = 0; e < P; ++e) xf[e] = gelu_tanh<IO::kRcpDiv>(fmaf(xf[e], wf[e], bf[e]));
      st_nt(out + (g + u * step) * P, IO::narrow16(xf));
    }
  }
  for (; g < pieces; g += step) {
    float xf[P], wf[P], bf[P];
    IO::widen16(ld_nt(x + g * P), xf);
    IO::widen16(ld_nt(w + g * P), wf);
    IO::widen16(ld_nt(b + g * P), bf);
#pragma unroll
    for (int e = 0; e < P; ++e) xf[e] = gelu_tanh<IO::kRcpDiv>(fmaf(xf[e], wf[e], bf[e]));
    st_nt(out + g * P, IO::narrow16(xf));
  }
  for (long long i = pieces * P + (long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += step)
    IO::store1(out + i, gelu_tanh<IO::kRcpDiv>(fmaf(IO::load1(x + i), IO::load1(w + i), IO::load1(b + i))));
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

template <typename IO>
int softmax_launch(const void* x, void* out, int n_rows, int n_cols, long long stride, hipStream_t st) {
  using T = typename IO::T;
  auto xp = static_cast<const T*>(x);
  auto op = static_cast<T*>(out);
  void* args[] = {(void*)&xp, (void*)&op, (void*)&n_cols, (void*)&stride};
  // Rows up to 16384 columns stay in registers (CH * 8 * threads >= n_cols
  // in every bucket); rows above 4096 columns take IO::kWideThreads threads.
  constexpr int W = IO::kWideThreads;
  const void* k;
  int threads = kThreads;
  if (n_cols <= 1 * kRowChunk) k = reinterpret_cast<const void*>(softmax_rows_kernel<IO, 1, kThreads>);
  else if (n_cols <= 2 * kRowChunk) k = reinterpret_cast<const void*>(softmax_rows_kernel<IO, 2, kThreads>);
  else if (n_cols <= 4 * kRowChunk) { k = reinterpret_cast<const void*>(softmax_rows_kernel<IO, 4 * kThreads / W, W>); threads = W; }
  else if (n_cols <= 8 * kRowChunk) { k = reinterpret_cast<const void*>(softmax_rows_kernel<IO, 8 * kThreads / W, W>); threads = W; }
  else k = reinterpret_cast<const void*>(softmax_rows_online_kernel<IO>);
  const hipError_t e = hipLaunchKernel(k, dim3(n_rows), dim3(threads), args, 0, st);
  return e == hipSuccess ? TILEATTN_OK : TILEATTN_ERR_LAUNCH;
}

template <typename IO>
int gelu_launch(const void* x, const void* w, const void* b, void* out, long long n, hipStream_t st) {
  using T = typename IO::T;
  auto xp = static_cast<const T*>(x);
  auto wp = static_cast<const T*>(w);
  auto bp = static_cast<const T*>(b);
  auto op = static_cast<T*>(out);
  // One workgroup per CU (256 on MI355X); the grid-stride loop covers the rest.
  const long long pieces = n / IO::kPer16;
  long long blocks = (pieces + kThreads - 1) / kThreads;
  blocks = blocks < 1 ? 1 : (blocks > kGeluWorkgroups ? kGeluWorkgroups : blocks);
  void* args[] = {(void*)&xp, (void*)&wp, (void*)&bp, (void*)&op, (void*)&n};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(gelu_kernel<IO>), dim3((unsigned)blocks),
                                       dim3(kThreads), args, 0, st);
  return e == hipSuccess ? TILEATTN_OK : TILEATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int tileattn_softmax(const void* x, void* out, int n_rows, int n_cols, long long stride,
                                int dtype, void* stream) {
  if (dtype != TILEATTN_DTYPE_F32 && dtype != TILEATTN_DTYPE_BF16) return TILEATTN_ERR_DTYPE;
  if (n_rows < 0 || n_cols < 1 || stride < n_cols) return TILEATTN_ERR_BAD_SHAPE;
  const int per16 = dtype == TILEATTN_DTYPE_F32 ? 4 : 8;  // elements per 16 bytes
  if (stride % per16 != 0) return TILEATTN_ERR_ALIGNMENT;
  if (n_rows == 0) return TILEATTN_OK;
  if (!x || !out) return TILEATTN_ERR_NULL_POINTER;
  if (misaligned(x) || misaligned(out)) return TILEATTN_ERR_ALIGNMENT;
  if (n_cols > INT_MAX - kRowChunk) return TILEATTN_ERR_TOO_LARGE;  // column indices stay in int
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dtype == TILEATTN_DTYPE_F32 ? softmax_launch<F32>(x, out, n_rows, n_cols, stride, st)
                                     : softmax_launch<BF16>(x, out, n_rows, n_cols, stride, st);
}

extern "C" int tileattn_gelu(const void* x, const void* w, const void* b, void* out, long long n,
                             int dtype, void* stream) {
  if (dtype != TILEATTN_DTYPE_F32 && dtype != TILEATTN_DTYPE_BF16) return TILEATTN_ERR_DTYPE;
  if (n < 0) return TILEATTN_ERR_BAD_SHAPE;
  if (n == 0) return TILEATTN_OK;
  if (!x || !w || !b || !out) return TILEATTN_ERR_NULL_POINTER;
  if (misaligned(x) || misaligned(w) || misaligned(b) || misaligned(out)) return TILEATTN_ERR_ALIGNMENT;
  if (n > LLONG_MAX / 2 - (long long)kThreads * 2048 * kVec) return TILEATTN_ERR_TOO_LARGE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dtype == TILEATTN_DTYPE_F32 ? gelu_launch<F32>(x, w, b, out, n, st)
                                     : gelu_launch<BF16>(x, w, b, out, n, st);
}
