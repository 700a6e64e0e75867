// Helpers of the attention kernels: vector types, the buffer resources, the
// lane-pair reductions of the 32x32 MFMA layout, the 16-bit MFMA and
// rounding, the XCD-aware workgroup map, and the build switches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <float.h>
#include <math.h>
#include <type_traits>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native vector type for 16-byte staging registers: arrays of HIP's uint4
// wrapper struct are not always promoted to registers and can land in
// scratch memory.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// no swizzle, no stride): loads past num_records return 0.
constexpr int kBufferFlags = 0x00020000;

// Raw buffer resource over [base, base + bytes) for a wave-uniform range,
// built from readfirstlane'd values so it lives in scalar registers (a
// resource the compiler cannot prove uniform costs a loop around every
// buffer access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_buffer(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), 0,
                                           __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

__device__ __forceinline__ float wave_pair_max(float x) {
  // Lanes l and l^32 hold the same query row; combine their partial maxima.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The 16-bit kernel holds bf16 and fp16 operands in one bit container
// (bf16x8); IS_F16 selects which MFMA reads the bits and how fp32 values are
// rounded into them (round to nearest even either way).
template <bool IS_F16>
__device__ __forceinline__ f32x16 mfma16(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (IS_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool IS_F16>
__device__ __forceinline__ __bf16 round16(float x) {
  if constexpr (IS_F16)
    return __builtin_bit_cast(__bf16, (_Float16)x);
  else
    return (__bf16)x;
}

// Map a hardware workgroup id to (batch, query head, query tile).  Ids are
// dealt to the 8 XCDs round-robin (XCD = id % 8, position on it = id / 8).
// The remap gives every XCD whole (batch, kv head) slots, so its resident
// workgroups share K/V in its L2, and orders each XCD's share by query tile,
// heaviest first when causal, across all of its slots (longest jobs first on
// its 32 CUs), then by query head within the group.  With fewer than 8 slots
// a slot's query tiles are spread over 8/slots XCDs by residue, so every XCD
// gets the same mix of heavy and light tiles.  Shapes that divide unevenly
// keep contiguous XCD ranges of the order (batch, kv head, query tile, query
// head), or the plain order.
__device__ __forceinline__ void map_workgroup(int hw_id, int nwg, int Hkv, int G, int nqt,
                                              bool causal, int& b, int& hq, int& qt) {
  const int P = nwg / (G * nqt);  // (batch, kv head) slots
  const int x = hw_id & 7, pos = hw_id >> 3;
  int slot, tq, g;
  if ((P & 7) == 0) {
    const int per = P >> 3;
    g = pos % G;
    const int rest = pos / G;
    slot = x * per + rest % per;
    tq = rest / per;
  } else if (P < 8 && 8 % P == 0 && nqt % (8 / P) == 0) {
    const int r = 8 / P;
    g = pos % G;
    slot = x / r;
    tq = x % r + (pos / G) * r;
  } else {
    const int logical = (nwg & 7) == 0 ? x * (nwg >> 3) + pos : hw_id;
    g = logical % G;
    const int rest = logical / G;
    tq = rest % nqt;
    slot = rest / nqt;
  }
  const int hk = slot % Hkv;
  b = slot / Hkv;
  hq = hk * G + g;
  qt = causal ? (nqt - 1 - tq) : tq;
}

// Largest sum of one lane's p of a tile before the reference max is raised
// (2^8: every p stays <= 2^8).
#ifndef TILEATTN_RESCALE_SUM
#define TILEATTN_RESCALE_SUM 256.0f
#endif
#ifndef TILEATTN_SETPRIO
#define TILEATTN_SETPRIO 1
#endif
// Race-check build: with TILEATTN_SYNC_CHECK defined, extra workgroup
// barriers close the staging step and both phases of every iteration, in the
// same number on both wave groups.  Only the order of LDS accesses across
// waves changes, not the arithmetic, so that build's results must equal the
// normal build's bit for bit; a difference would expose an LDS read that
// races the write it depends on.
#ifdef TILEATTN_SYNC_CHECK
#define TILEATTN_CHECK_BARRIER() __syncthreads()
#else
#define TILEATTN_CHECK_BARRIER() ((void)0)
#endif

}  // namespace
