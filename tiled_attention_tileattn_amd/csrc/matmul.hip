// Tiled matrix product C = A * B for gfx950 (MI355X): bf16 inputs, fp32
// accumulation, C stored as fp32 or bf16.
//
// This is the tiled K-loop of the first page ("Guia Pratico de Programacao de
// GPU com Tiles", Passo a Passo step 5): one workgroup per output tile, an
// fp32 accumulator, and a loop over K that adds the product of an A block and
// a B block (the page's Troubleshooting note: an fp16 accumulator loses
// precision on large matrices).  It is the building block of both attention
// products, here standalone.
//
// Layout: A is [M, K], B is [K, N] and C is [M, N], all row-major and dense.
//
// Design:
//   * a 256 x 256 tile of C per workgroup of 8 waves, each wave a 128 (M) x
//     64 (N) sub-tile held as 8 accumulators of v_mfma_f32_32x32x16_bf16;
//   * the MFMA computes transposed blocks, C^T = B^T A^T: with B as the first
//     operand a lane ends up owning 4 consecutive columns of C per register
//     group, so the epilogue writes 16-byte (fp32) or 8-byte (bf16) pieces;
//   * K steps of 64: the next A and B tiles are loaded with buffer loads into
//     registers at the top of a step, the current tiles are multiplied out
//     of LDS, and the registers are written to the other LDS slot between
//     the MFMA blocks of the step's middle sub-steps (double buffering, one
//     barrier per step);
//   * A operand fragments are 16-byte LDS reads along K; B fragments are read
//     down the columns of the row-major B tile with ds_read_b64_tr_b16;
//   * padded LDS rows (A: 144 B, B: 576 B) make every operand read phase
//     bank-conflict free;
//   * ragged edges: each workgroup's buffer starts at its own tile, so rows
//     past M (A) and K (B) fall outside the buffer's range and read as 0;
//     column chunks past N (B) and past K (A, last step) get an offset
//     outside the range.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "tileattn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 512;                 // 8 waves: 2 along M x 4 along N
constexpr int kWaveM = 128, kWaveN = 64;
constexpr int kAPitch = kBK * 2 + 16;         // bytes per A row in LDS
constexpr int kBPitch = kBN * 2 + 64;         // bytes per B row in LDS
constexpr int kABytes = kBM * kAPitch;
constexpr int kBBytes = kBK * kBPitch;
constexpr int kStage = kABytes + kBBytes;
constexpr int kLoads = kBM * kBK / 8 / kThreads;  // 16-byte loads per thread per tile
static_assert(kLoads == 4 && kBK * kBN / 8 / kThreads == 4, "tile / thread count mismatch");
constexpr unsigned kOutOfRange = 0x80000000u;  // beyond any buffer range used here
constexpr int kBufferFlags = 0x00020000;
#ifndef TILEATTN_MM_GROUP
#define TILEATTN_MM_GROUP 4
#endif
constexpr int kGroupM = TILEATTN_MM_GROUP;      // tile rows per group of the tile order

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Map a hardware workgroup id to a tile (tm, tn).  Ids are dealt to the 8 XCDs
// round-robin; the remap gives each XCD a contiguous range of the logical
// order, and the logical order walks groups of kGroupM tile rows column by
// column, so the workgroups resident on one XCD share A rows and B columns.
__device__ __forceinline__ void map_tile(int hw_id, int ntm, int ntn, int& tm, int& tn) {
  const int nwg = ntm * ntn;
  int logical = hw_id;
  if ((nwg & 7) == 0) logical = (hw_id & 7) * (nwg >> 3) + (hw_id >> 3);
  const int group = logical / (kGroupM * ntn);
  const int first = group * kGroupM;
  const int rows = min(ntm - first, kGroupM);
  const int in = logical - group * kGroupM * ntn;
  tm = first + in % rows;
  tn = in / rows;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void matmul_bf16_kernel(const uint16_t* A, const uint16_t* B,
                                                               void* __restrict__ C, int M, int N,
                                                               int K, int ntm, int ntn) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int s16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  int tm, tn;
  map_tile(blockIdx.x, ntm, ntn, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int nk = (K + kBK - 1) / kBK;

  // Per-thread load offsets.  A chunk i: row idx/8, 16-byte chunk idx%8 of the
  // 64-wide K slice; B chunk i: row idx/32, chunk idx%32 of the 256 columns.
  int a_off[kLoads], a_col[kLoads], b_off[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int idx = tid + i * kThreads;
    const int ar = idx >> 3, ac = idx & 7;
    a_off[i] = ar * K * 2 + ac * 16;
    a_col[i] = ac * 8;
    const int br = idx >> 5, bc = idx & 31;
    b_off[i] = (n0 + bc * 8 < N) ? br * N * 2 + bc * 16 : (int)kOutOfRange;
  }
  const long long a_rows_bytes = (long long)(M - m0) * K * 2;
  const long long b_rows_bytes = (long long)K * N * 2 - (long long)n0 * 2;

  u32x4 areg[kLoads], breg[kLoads];
  auto load_tiles = [&](int kt) {
    const int k0 = kt * kBK;
    const long long na = a_rows_bytes - (long long)k0 * 2;
    const long long nb = b_rows_bytes - (long long)k0 * N * 2;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + (size_t)m0 * K + k0), 0, (int)min(na, (long long)INT_MAX), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(B + (size_t)k0 * N + n0), 0, (int)min(nb, (long long)INT_MAX), kBufferFlags);
    const bool k_edge = k0 + kBK > K;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int off = (k_edge && a_col[i] >= K - k0) ? (int)kOutOfRange : a_off[i];
      areg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
      breg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off[i], 0, 0));
    }
  };
  auto store_a = [&](int stage) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = tid + i * kThreads;
      *reinterpret_cast<u32x4*>(smem + stage + (idx >> 3) * kAPitch + (idx & 7) * 16) = areg[i];
    }
  };
  auto store_b = [&](int stage) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = tid + i * kThreads;
      *reinterpret_cast<u32x4*>(smem + stage + kABytes + (idx >> 5) * kBPitch + (idx & 31) * 16) = breg[i];
    }
  };

  // Operand fragments.  A: lane (row l32, k half) reads 8 consecutive k of
  // one row.  B: ds_read_b64_tr_b16 hands output lane 4a+b of each 16-lane
  // group element b of source lanes a, a+4, a+8, a+12; source lane s reads 4
  // columns 4(s%4).. of k-row s/4, so a lane receives 4 consecutive k of one
  // column, and the second read (4 rows further) the next 4.
  const int a_lane = (wm * kWaveM + l32) * kAPitch + half * 16;
  const int b_lane = kABytes + (8 * half + (s16 >> 2)) * kBPitch +
                     2 * (wn * kWaveN + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3));
  auto a_frag = [&](int base, int mb, int t) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(smem + base + mb * 32 * kAPitch + t * 32);
  };
  auto b_frag = [&](int base, int nb, int t) -> bf16x8 {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const unsigned char* p = smem + base + t * 16 * kBPitch + nb * 64;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(p + 4 * kBPitch));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x16{};

  if (nk > 0) {
    load_tiles(0);
    store_a(0);
    store_b(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_tiles(kt + 1);
    int stage = (kt & 1) * kStage;
    asm volatile("" : "+s"(stage));  // one runtime base: operand addresses stay base + immediate
    const int abase = stage + a_lane, bbase = stage + b_lane;
    bf16x8 af[2][4], bfr[2][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) af[0][mb] = a_frag(abase, mb, 0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bfr[0][nb] = b_frag(bbase, nb, 0);
#pragma unroll
    for (int t = 0; t < kBK / 16; ++t) {
      const int cur = t & 1, nxt = cur ^ 1;
      if (t + 1 < kBK / 16) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) af[nxt][mb] = a_frag(abase, mb, t + 1);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bfr[nxt][nb] = b_frag(bbase, nb, t + 1);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma(bfr[cur][nb], af[cur][mb], acc[nb][mb]);
      // The staged next tile goes to the other slot (last read in the
      // previous step, before its closing barrier) between the MFMA blocks of
      // the middle sub-steps, A after the second and B after the third.
      if (kt + 1 < nk && t == 1) store_a(((kt + 1) & 1) * kStage);
      if (kt + 1 < nk && t == 2) store_b(((kt + 1) & 1) * kStage);
    }
    __syncthreads();
  }

  // Epilogue.  acc[nb][mb] is the block C^T[n][m]: lane (l32, half) holds
  // column m = l32 and, in register group g, the 4 consecutive columns
  // n = 8g + 4*half .. +3 of C's row m.
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + wm * kWaveM + mb * 32 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * kWaveN + nb * 32 + 8 * g + 4 * half;
        if (n >= N) continue;
        const f32x4 v = {acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                         acc[nb][mb][4 * g + 3]};
        if constexpr (OUT_BF16) {
          uint2 u;
          u.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[0]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[1]) << 16);
          u.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[3]) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + (size_t)m * N + n) = u;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(C) + (size_t)m * N + n) = v;
        }
      }
  }
}

}  // namespace

extern "C" int tileattn_matmul(const void* a, const void* b, void* c, int M, int N, int K,
                               int out_bf16, void* stream) {
  if (M < 0 || N < 0 || K < 0 || (N & 7) != 0 || (K & 7) != 0) return TILEATTN_ERR_BAD_SHAPE;
  if (M == 0 || N == 0) return TILEATTN_OK;
  if (!c || (K > 0 && (!a || !b))) return TILEATTN_ERR_NULL_POINTER;  // K = 0 reads neither
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (misaligned(a) || misaligned(b) || misaligned(c)) return TILEATTN_ERR_ALIGNMENT;
  // 32-bit buffer offsets inside one tile (256 rows of A, 64 rows of B), and
  // row indices inside the kernel within int (M <= 2^30).
  if ((long long)kBM * K * 2 > INT_MAX || (long long)kBK * N * 2 > INT_MAX || M > (1 << 30))
    return TILEATTN_ERR_TOO_LARGE;
  const long long tiles = (long long)((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (tiles > INT_MAX) return TILEATTN_ERR_TOO_LARGE;
  const int ntm = (M + kBM - 1) / kBM, ntn = (N + kBN - 1) / kBN;
  auto A = static_cast<const uint16_t*>(a);
  auto B = static_cast<const uint16_t*>(b);
  void* args[] = {(void*)&A, (void*)&B, (void*)&c, (void*)&M, (void*)&N, (void*)&K, (void*)&ntm, (void*)&ntn};
  const void* kernel = out_bf16 ? reinterpret_cast<const void*>(matmul_bf16_kernel<true>)
                                : reinterpret_cast<const void*>(matmul_bf16_kernel<false>);
  const hipError_t e = hipLaunchKernel(kernel, dim3(ntm * ntn), dim3(kThreads), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TILEATTN_OK : TILEATTN_ERR_LAUNCH;
}
