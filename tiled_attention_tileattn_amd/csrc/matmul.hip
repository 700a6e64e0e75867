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
//   * K steps of 64: the next A and B tiles go from memory straight into the
//     other LDS slot at the top of a step (buffer_load_dwordx4 with the LDS
//     flag: 64 lanes x 16 bytes written at M0 + 16 * lane), while the current
//     tiles are multiplied out of LDS (double buffering, one barrier per
//     step);
//   * A operand fragments are 16-byte LDS reads along K; B fragments are read
//     down the columns of the row-major B tile with ds_read_b64_tr_b16;
//   * LDS rows are unpadded (A: 128 B, B: 512 B, as the 1 KiB loads write
//     them) and their 16-byte chunks XOR-swizzled so that every operand read
//     phase is bank-conflict free: chunk c of A row r sits at position
//     c ^ ((r >> 1) & 7), chunk c of B row r at c ^ 4 (r & 3); each lane
//     loads the global chunk its LDS position holds;
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
constexpr int kAPitch = kBK * 2;              // bytes per A row in LDS
constexpr int kBPitch = kBN * 2;              // bytes per B row in LDS
constexpr int kABytes = kBM * kAPitch;
constexpr int kBBytes = kBK * kBPitch;
constexpr int kStage = kABytes + kBBytes;
constexpr int kPieces = kABytes / 1024 / (kThreads / 64);  // 1 KiB loads per wave per tile
static_assert(kPieces == 4 && kBBytes / 1024 / (kThreads / 64) == 4, "tile / wave count mismatch");
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

  // Tile loads.  Wave w moves the 1 KiB pieces n = 4w + e (e = 0..3) of each
  // tile: A rows 8n .. 8n + 7 (lane: row 8n + lane / 8, chunk position
  // lane % 8), B rows 2n, 2n + 1 (lane: row 2n + lane / 32, position
  // lane % 32).  The lane's byte offset in the tile is its global chunk's:
  // the swizzle is applied on the load side.  A chunks past K (last step)
  // and B chunks past N get an offset outside the buffer range (zeros).
  int a_off[kPieces], a_col[kPieces], b_off[kPieces];
#pragma unroll
  for (int e = 0; e < kPieces; ++e) {
    const int n = wave * kPieces + e;
    const int ar = 8 * n + (lane >> 3);
    const int ac = (lane & 7) ^ ((ar >> 1) & 7);
    a_off[e] = ar * K * 2 + ac * 16;
    a_col[e] = ac * 8;
    const int br = 2 * n + (lane >> 5);
    const int bc = (lane & 31) ^ (4 * (br & 3));
    b_off[e] = (n0 + bc * 8 < N) ? br * N * 2 + bc * 16 : (int)kOutOfRange;
  }
  const long long a_rows_bytes = (long long)(M - m0) * K * 2;
  const long long b_rows_bytes = (long long)K * N * 2 - (long long)n0 * 2;
  const unsigned smem_base = (unsigned)(uintptr_t)smem;  // LDS byte address of smem

  // The loads are inline asm: the compiler would otherwise wait for every one
  // of them before each LDS read.  They are the kernel's only vector-memory
  // loads; each wave waits for its own (vmcnt) before the step's closing
  // barrier.
  auto dma = [&](const __amdgpu_buffer_rsrc_t& r, int voff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r) : "memory", "m0");
  };
  auto load_tiles = [&](int kt, int stage) {
    const int k0 = kt * kBK;
    const long long na = a_rows_bytes - (long long)k0 * 2;
    const long long nb = b_rows_bytes - (long long)k0 * N * 2;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + (size_t)m0 * K + k0), 0, (int)min(na, (long long)INT_MAX), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(B + (size_t)k0 * N + n0), 0, (int)min(nb, (long long)INT_MAX), kBufferFlags);
    const bool k_edge = k0 + kBK > K;
#pragma unroll
    for (int e = 0; e < kPieces; ++e) {
      const int n = wave * kPieces + e;
      const int off = (k_edge && a_col[e] >= K - k0) ? (int)kOutOfRange : a_off[e];
      dma(ra, off, smem_base + stage + n * 1024);
      dma(rb, b_off[e], smem_base + stage + kABytes + n * 1024);
    }
  };
  auto dma_wait = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // Operand fragments.  A: lane (row l32, k half) reads 8 consecutive k of
  // one row.  B: ds_read_b64_tr_b16 hands output lane 4a+b of each 16-lane
  // group element b of source lanes a, a+4, a+8, a+12; source lane s reads 4
  // columns 4(s%4).. of k-row s/4, so a lane receives 4 consecutive k of one
  // column, and the second read (4 rows further) the next 4.
  // With the swizzle: A row wm*128 + mb*32 + l32 has (row >> 1) & 7 =
  // (l32 >> 1) & 7, so the lane's offset of k chunk 2t + half is aofs[t]
  // plus an immediate per mb; B row 16t + 8*half + s16/4 (+4) has row & 3 =
  // s16 >> 2, and the lane's 64-byte column group 2*(wn & 1) + nb of the
  // 256-byte half wn >> 1 moves by XOR with it: bofs[nb] plus an immediate
  // per t.
  int aofs[kBK / 16], bofs[2];
#pragma unroll
  for (int t = 0; t < kBK / 16; ++t)
    aofs[t] = (wm * kWaveM + l32) * kAPitch + (((2 * t + half) ^ ((l32 >> 1) & 7)) << 4);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
    bofs[nb] = kABytes + (8 * half + (s16 >> 2)) * kBPitch + 256 * (wn >> 1) +
               64 * ((2 * (wn & 1) + nb) ^ (s16 >> 2)) + 32 * ((lane >> 4) & 1) + 8 * (s16 & 3);
  auto a_frag = [&](int base, int mb, int t) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(smem + base + aofs[t] + mb * 32 * kAPitch);
  };
  auto b_frag = [&](int base, int nb, int t) -> bf16x8 {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const unsigned char* p = smem + base + bofs[nb] + t * 16 * kBPitch;
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
    load_tiles(0, 0);
    dma_wait();
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    // The other slot was last read in the previous step, before its closing
    // barrier.
    if (kt + 1 < nk) load_tiles(kt + 1, ((kt + 1) & 1) * kStage);
    int stage = (kt & 1) * kStage;
    asm volatile("" : "+s"(stage));  // one runtime base: operand addresses stay base + immediate
    const int abase = stage, bbase = stage;
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
    }
    dma_wait();
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
