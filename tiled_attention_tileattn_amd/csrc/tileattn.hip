// tileattn — exact attention forward for MI355X (gfx950 / CDNA4).
//
// Method: the tiled flash-attention loop of "Guia Prático de Programação de GPU
// com Tiles: de Kernels cuTile e Triton ao Flash Attention" (Passo a Passo,
// step 6 "Flash Attention — Softmax Online"): a block of query rows stays
// resident, key/value tiles stream past it, and per tile the kernel
//   (1) forms the scores of the query block against the key tile,
//   (2) raises the running row maximum,
//   (3) exponentiates the shifted scores,
//   (4) rescales the running sum and the output accumulator by
//       exp(old max - new max) and adds the new tile's contribution, with the
//       probabilities cast to the value dtype before the second product,
// and divides the accumulator by the running sum at the end.  Both products
// accumulate in fp32 (step 5 "Multiplicação de Matrizes Tiled" and the
// Troubleshooting note on fp16 accumulators).
//
// CDNA4 mapping (our design, not the pages'):
//   * One workgroup = 8 waves = 256 query rows: P query heads that share one
//     KV head (P the largest power of two dividing the group size, at most
//     8) times 256 / P consecutive positions; each wave owns 32 query rows
//     (one head, 32 positions) for the whole key loop.  Two waves share each
//     SIMD (wave w and w+4).
//   * The kernel computes the transposed products S^T = K * Q^T and
//     O^T = V^T * P^T with v_mfma_f32_32x32x16_bf16.  In the 32x32 result
//     layout a lane holds 16 entries of ONE output column, so with queries as
//     columns every lane owns one query row: the row max and row sum are
//     in-lane reductions plus one v_permlane32_swap between the two lanes
//     that share the row, and the rescale factor is a per-lane scalar.
//   * The fp32 S^T tile, once exponentiated and packed to bf16, is already
//     in the B-operand layout of the P*V product (no LDS round trip); the V
//     operand is read from row-major LDS with ds_read_b64_tr_b16, whose
//     transpose yields exactly the key order that P^T carries.
//   * Q lives in VGPRs for the whole loop (B operand of the first product).
//     It arrives, and O leaves, whole rows at a time through a per-wave LDS
//     area, since in the MFMA layouts a lane holds only pieces of a row.
//   * K and V tiles are double-buffered in LDS as unpadded rows with an XOR
//     swizzle of their 16-byte chunks, which makes the operand reads free of
//     bank conflicts; buffer loads write them straight into LDS (no staging
//     registers).  Operands are read into a small register ring a few MFMAs
//     ahead of use.
//   * Ping-pong: the waves of a SIMD alternate between a matrix phase (only
//     MFMAs: the scores of tile j and the P*V update of tile j-1) and a
//     vector phase (the online softmax), half a tile apart (one group starts
//     an iteration with its matrix phase, the other with its vector phase),
//     so that one wave keeps the matrix core busy while the other
//     exponentiates.
//   * exp is computed as exp2 with scale*log2(e) folded into one FMA; the
//     reference max is raised lazily, only when a tile's exponentials grow
//     too large (see softmax_tile), which is exact.
//   * Causal: tiles entirely above a workgroup's diagonal are never loaded;
//     masking code runs only on tiles that cross a wave's diagonal or the
//     ragged end.  A wave whose rows end before the workgroup's last tile
//     runs the remaining tiles fully masked (p = 0), which keeps both wave
//     groups in step with the shared barriers; with heads packed, a
//     workgroup spans fewer positions and so fewer such tiles (none at 64).
//   * Workgroup ids are remapped so the workgroups that one XCD (8 per chip,
//     ids dealt round-robin) runs share key/value heads and read their K/V
//     tiles from that XCD's L2, and each XCD takes its causal query tiles
//     heaviest first across all of its heads (see map_workgroup).
//   * Grids too small to fill the chip with 256-row workgroups take the key
//     split instead: 128 query rows per workgroup, which both wave groups
//     hold, each group running the same ping-pong over its own half of the
//     key tiles (its own LDS slots); at the end the two partial
//     (acc, l, max) states of a row merge through LDS by the online-softmax
//     update itself.  Where a few query tiles own long key ranges, the
//     workspace entry point also cuts those ranges into chunks run by
//     separate workgroups, whose partial states a second kernel merges
//     (attn_merge_kernel).
//   * Instances with a block mask compact the visible key tiles into an LDS
//     list and skip, per wave, the tiles its rows cannot see; instances with
//     a linear (ALiBi) bias start the score product from the bias, and walk
//     the key tiles from the diagonal down when causal.

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/tileattn.h"
#include "attn_common.h"

namespace {

constexpr int kRowsPerWave = 32;                       // query rows owned by one wave
constexpr int kBlockN = 64;                            // keys per tile (bf16 path)
constexpr int kF32Waves = 4;                           // fp32 path: waves per workgroup
constexpr int kF32Threads = kF32Waves * 64;
constexpr int kF32BlockM = kF32Waves * kRowsPerWave;   // fp32 path: 128 query rows
constexpr int kBlockNF32 = 32;                         // keys per tile (fp32 path)

// Capacity of the per-workgroup tile list of block-masked calls: Sk <= 64 * this.
constexpr int kMaxMaskedTiles = 2048;
// Chunked key split: workspace floats per chunk (one 128-row workgroup): the
// fp32 accumulator, then the rows' reference max and running sum.
constexpr int kChunkRows = 128;
template <int D>
constexpr int kChunkFloats = kChunkRows * D + 2 * kChunkRows;

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
// Depth (in MFMAs) of the LDS operand prefetch ring of each product.
#ifndef TILEATTN_PREFETCH
#define TILEATTN_PREFETCH 4
#endif

// The 8-wave ping-pong workgroup: 256 query rows, every wave with its own 32.
// SPLIT: 128 query rows, which both wave groups hold, each group visiting
// half of the key tiles; the two partial results merge at the end.  That is
// for grids too small to fill the chip with 256-row workgroups.
template <int D, bool SPLIT = false>
struct Bf16Tile {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRowWaves = SPLIT ? kWaves / 2 : kWaves;  // waves with distinct query rows
  static constexpr int kRowWavesShift = SPLIT ? 2 : 3;            // log2 kRowWaves
  static constexpr int kBlockM = kRowWaves * kRowsPerWave;      // query rows per workgroup
  static constexpr int kSets = SPLIT ? 2 : 1;                    // K/V slot pairs (one per group)
  static constexpr int kChunks = D / 8;                    // 16-byte chunks per K/V row
  // A slot holds one tile's 64 unpadded rows (D * 2 bytes each, chunks
  // swizzled; see the kernel's tile loaders).  K slots are 16 bytes a row
  // larger: room that lets the split kernel's merge area (64 (D/2 + 2)
  // floats per row pair, over the K slots) fit.
  static constexpr int kKBytes = kBlockN * (D * 2 + 16);
  static constexpr int kVBytes = kBlockN * D * 2;
  // Per-wave staging area for Q on the way in and O on the way out: the
  // wave's 32 rows padded by 16 bytes, so the 16 rows of one operand-layout
  // read phase of Q start 16 bytes apart modulo 256 and hit distinct banks.
  static constexpr int kKPitch = D * 2 + 16;
  static constexpr int kStageBytes = kRowsPerWave * kKPitch;
  static constexpr int kRowLoads = kRowsPerWave * kChunks / 64;  // 16-byte chunks per lane
  // LDS layout: K slots 0 and 1, V slots 0 and 1, then the staging areas
  // (one per row wave).  The split kernel has two such slot pairs per tensor
  // (set g for group g) and lays its staging areas over the V slots instead
  // (Q is staged before the first V tile is written, O after the last one is
  // read), which keeps it within 132 KiB at D = 128.
  static constexpr bool kStageOverV = SPLIT;
  static constexpr int kVOff = kSets * 2 * kKBytes;
  static constexpr int kStageOff = kVOff + (kStageOverV ? 0 : kSets * 2 * kVBytes);
  static constexpr int kSmemBytes = kVOff + kSets * 2 * kVBytes + (kStageOverV ? 0 : kRowWaves * kStageBytes);
  static_assert(!kStageOverV || kRowWaves * kStageBytes <= kSets * 2 * kVBytes,
                "staging areas must fit in the V slots");
};

// Steps (2)-(4a) of the tile update for one lane's 32 scores of its query row.
// mref is the row's reference maximum in exp2 units (m * c).  The tile is
// first exponentiated against the current reference, p = exp2(s c - mref).
// Only if some lane's sum of those p exceeds TILEATTN_RESCALE_SUM (a
// wave-uniform ballot; rare after a row's first tile) is the reference
// raised to the row's tile maximum, the accumulator and running sum scaled
// by alpha = exp2(mref_old - mref_new), and the tile exponentiated again.
// Numerator and denominator are always accumulated against the same
// reference, so the result is exact, and every p stays at most
// TILEATTN_RESCALE_SUM, far from fp32/bf16/fp16 overflow.  The reference
// starts at -FLT_MAX (finite): against it a visible score gives p = inf,
// which takes the raising branch, and a masked (-inf) score gives 0, so no
// step forms inf - inf.  The running sum adds the fp32 p; p is packed to
// 16 bits (round to nearest even) in the B-operand layout of the P*V
// product.
//
// MAX_FIRST takes the tile max before exponentiating instead (a v_max3 tree
// on every tile, the reference raised when the max exceeds it by more than
// 8 in log2 units): for score layouts whose max keeps rising from tile to
// tile, as with a two-sided linear bias, it avoids exponentiating twice.
template <bool IS_F16, bool MAX_FIRST, int NACC>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[2], float& mref, float& l_run,
                                             float c, f32x16 (&acc)[NACC],
                                             bf16x8 (&pf)[2][2]) {
  auto exponentiate = [&](float m) -> float {
    float psum0, psum1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * t + e], c, -m));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * t + e + 1], c, -m));
          const bool first = kb == 0 && t == 0 && e == 0;
          psum0 = first ? p0 : psum0 + p0;
          psum1 = first ? p1 : psum1 + p1;
          pf[kb][t][e] = round16<IS_F16>(p0);
          pf[kb][t][e + 1] = round16<IS_F16>(p1);
        }
    return psum0 + psum1;
  };
  auto raise_to_tile_max = [&]() {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
    return wave_pair_max(mx) * c;  // c > 0
  };
  auto rescale = [&](float m_new) {
    const float alpha = __builtin_amdgcn_exp2f(mref - m_new);
    mref = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] *= alpha;
  };
  float ps;
  if constexpr (MAX_FIRST) {
    const float mxc = raise_to_tile_max();
    if (__builtin_expect(__ballot(mxc - mref > 8.0f) != 0, 0)) rescale(fmaxf(mref, mxc));
    ps = exponentiate(mref);
  } else {
    ps = exponentiate(mref);
    if (__builtin_expect(__ballot(!(ps <= TILEATTN_RESCALE_SUM)) != 0, 0)) {
      rescale(fmaxf(mref, raise_to_tile_max()));
      ps = exponentiate(mref);
    }
  }
  l_run += ps;
}

// Ping-pong schedule.  The 8 waves form two groups (waves 0-3 and 4-7, one
// wave of each on every SIMD).  Per 64-key tile j a wave runs a matrix phase
// M(j) (MFMAs only: S_j = K_j Q^T interleaved with acc += V_{j-1}^T P_{j-1}^T)
// and a vector phase V(j) (the online softmax of S_j into P_j).  Group 0 runs
// M(j) then V(j) in the two halves of iteration j; group 1 runs V(j-1) then
// M(j).  A barrier closes every iteration (and, in the key split, one
// separates its halves), so on every SIMD one wave drives the matrix core
// while the other works through its exponentials.
// MASK: a block mask (tile list, per-wave skipping, rows with no visible key);
// ALIBI: the linear bias.  The plain kernel has neither.  SPLIT: the key
// split of the plain kernel (see Bf16Tile): the same schedule, with group g
// on its own half of the tiles, staged into its own slots.
template <int D, bool CAUSAL, bool IS_F16, bool MASK, bool ALIBI, bool SPLIT = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* K,
    const uint16_t* V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Hq, int Hkv, int Sq, int Sk, float scale, int nqt, int nwg,
    const float* __restrict__ slopes, const unsigned char* __restrict__ bmask, int mask_heads,
    int chunk_tiles, float* __restrict__ ws, int pack_shift) {
  using T = Bf16Tile<D, SPLIT>;
  static_assert(T::kThreads == 512, "two groups of four waves");
  static_assert(!SPLIT || T::kBlockM == kChunkRows, "a chunk is one key-split workgroup");
  __shared__ __attribute__((aligned(16)))
  unsigned char smem[T::kSmemBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int group = wave >> 2;
  const int G = Hq / Hkv;

  // Chunked key split (key-split instances with chunk_tiles > 0): the grid
  // is chunk-major, workgroup u = c * nwg + w taking key tiles
  // c * chunk_tiles to c * chunk_tiles + chunk_tiles - 1 of the query tile
  // that workgroup w of the plain grid has.  chunk_tiles is even, so only a
  // query tile's last chunk can be odd.  A chunk past the query tile's last
  // key tile has nothing to do.
  const bool chunked = SPLIT && chunk_tiles > 0;
  const int chunk = chunked ? (int)blockIdx.x / nwg : 0;
  // Head packing: the workgroup's rows are 2^pack_shift consecutive query
  // heads of one KV head (they share its K and V tiles) times PW = kBlockM /
  // 2^pack_shift consecutive positions (a query tile).  Row wave rw takes
  // head rw >> wph_shift of the group and positions (rw & (2^wph_shift - 1))
  // * 32 ... + 31 of the tile.  The grid map works on head groups.
  const int wph_shift = T::kRowWavesShift - pack_shift;  // log2 row waves per head
  const int PW = T::kBlockM >> pack_shift;
  int b, hgrp, qt;
  map_workgroup((int)blockIdx.x - chunk * nwg, nwg, Hkv, G >> pack_shift, nqt, CAUSAL, b, hgrp, qt);
  const int hq0 = hgrp << pack_shift;  // first query head of the group
  const int hk = hq0 / G;
  const int q0 = qt * PW;
  const int rw = SPLIT ? (wave & 3) : wave;  // row wave: which 32 rows of the workgroup
  const int hq = hq0 + (rw >> wph_shift);    // the wave's query head
  const int qw = q0 + ((rw & ((1 << wph_shift) - 1)) << 5);
  const int my_row = qw + l32;

  const size_t q_head = ((size_t)b * Hq + hq) * (size_t)Sq;
  const size_t kv_head = ((size_t)b * Hkv + hk) * (size_t)Sk;
  const uint16_t* Kh = K + kv_head * D;
  const uint16_t* Vh = V + kv_head * D;

  int nkt = (Sk + kBlockN - 1) / kBlockN;
  if (CAUSAL) {
    const int last_row = min(q0 + PW - 1, Sq - 1);
    nkt = min(nkt, last_row / kBlockN + 1);
  }
  const int nchunks = chunked ? (nkt + chunk_tiles - 1) / chunk_tiles : 1;
  if (chunk >= nchunks) return;

  // Key tiles the workgroup visits.  Without a block mask: tiles 0..nkt-1.
  // With one: the tiles that any of the workgroup's 64-row query blocks
  // (kBlockM / 64 of them: (head, 64 positions) pairs, two row waves each;
  // block i = row waves 2i and 2i+1) may see, in order, compacted into an
  // LDS list by wave 0; entry = tile index (bits 0-11) | visibility of
  // query block i (bit 12 + i).  Packing keeps PW >= 64 with a mask.
  __shared__ unsigned short tlist[MASK ? kMaxMaskedTiles : 1];
  __shared__ int tcount;
  int nt = nkt;
  if (MASK) {
    if (wave == 0) {
      const int nqb = (Sq + kBlockN - 1) / kBlockN, nkb = (Sk + kBlockN - 1) / kBlockN;
      const int qb0 = q0 / kBlockN;
      const int nb_shift = wph_shift - 1;  // log2 query blocks per head
      int count = 0;
      for (int base = 0; base < nkt; base += 64) {
        const int kb = base + lane;
        unsigned bits = 0;
        if (kb < nkt) {
#pragma unroll
          for (int i = 0; i < T::kBlockM / kBlockN; ++i) {
            const int qb = qb0 + (i & ((1 << nb_shift) - 1));
            const unsigned char* plane = bmask + (size_t)(mask_heads == Hq ? hq0 + (i >> nb_shift) : 0) * nqb * nkb;
            if (qb < nqb && plane[(size_t)qb * nkb + kb] != 0) bits |= 1u << i;
          }
        }
        const unsigned long long vis = __ballot(bits != 0);
        const int pos = count + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(vis >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((unsigned)vis, 0u));
        if (bits != 0) tlist[pos] = (unsigned short)(kb | (bits << 12));
        count += __popcll(vis);
      }
      if (lane == 0) tcount = count;
    }
    __syncthreads();
    nt = __builtin_amdgcn_readfirstlane(tcount);  // wave-uniform, so branches on it stay scalar
  }
  // With a causal linear bias the largest scores of a row sit next to its
  // diagonal: walking the tiles from the diagonal down finds the row max on
  // the first visible tile, so the lazy reference is rarely raised after it.
  constexpr bool kReversed = ALIBI && CAUSAL;
  auto order = [&](int j) -> int { return kReversed ? nt - 1 - j : j; };
  // Key split: group g visits entries g*h to g*h + h - 1 of the nl tiles
  // (the tile list with a block mask, else tiles 0 to nkt - 1), with
  // h = ceil(nl / 2).  When nl is odd, group 1's last entry lies past the
  // end: without a mask, a tile past the keys (past Sk, or past every row's
  // diagonal), whose loads read zeros and whose scores the mask hides; with
  // one, no list entry, which no wave sees.  Either way it changes nothing.
  // A chunk covers tiles t0 to t0 + nl - 1; only the last chunk of a query
  // tile can have an odd count, so only there does group 1 reach one past
  // the end, the tile nkt past the keys, as without chunks.  (The block-mask
  // instances take no chunks.)
  const int t0 = chunk * chunk_tiles;
  const int nl = chunked ? min(chunk_tiles, nkt - t0) : nt;
  const int lbase = (chunked ? t0 : 0) + (SPLIT ? group * ((nl + 1) / 2) : 0);
  if (SPLIT) nt = (nl + 1) / 2;
  auto in_list = [&](int j) -> bool { return !SPLIT || lbase + order(j) < nl; };
  auto tile = [&](int j) -> int {
    if constexpr (MASK)
      return in_list(j) ? (int)(tlist[lbase + order(j)] & 0xFFF) : nkt;
    else
      return lbase + order(j);
  };
  // This wave's 64-row query block may see tile j (block mask).
  auto wave_sees = [&](int j) -> bool {
    return !MASK || (in_list(j) && ((tlist[lbase + order(j)] >> (12 + (rw >> 1))) & 1));
  };

  // With the bias, scores are kept in units of 1/kscale: the S product
  // starts from bias/kscale instead of 0 (see bias_init), so the softmax and
  // lse below are those of the plain kernel with kscale for scale.  A scale
  // under 2^-64 (zero included) counts as zero there: the products q.k drop
  // out (Q is zeroed) and the scores are the bias alone, kscale = 1.
  const bool q_dropped = ALIBI && !(scale >= 0x1p-64f);
  const float kscale = !ALIBI ? scale : (q_dropped ? 1.f : scale);
  const float sigma = ALIBI ? slopes[hq] / kscale : 0.f;

  // The wave's 32 query rows are contiguous in memory.  They are loaded
  // whole-row (64 lanes x 16 bytes = 1 KiB per instruction; rows past Sq,
  // or every row when Q drops out, lie outside the buffer range and read as
  // 0), staged in the wave's LDS area, and read back in the B-operand layout
  // after the prologue barrier.  O leaves the same way in the epilogue.
  // Split: the two waves of a row pair share one staging area; group 0
  // stages Q there and writes O out of it.
  const bool row_owner = !SPLIT || group == 0;
  unsigned char* const stage = smem + T::kStageOff + rw * T::kStageBytes;
  u32x4 qreg[T::kRowLoads];
  if (row_owner) {
    const int rows_here = q_dropped ? 0 : max(0, min(kRowsPerWave, Sq - qw));
    const __amdgpu_buffer_rsrc_t qrsrc = wave_buffer(Q + (q_head + (size_t)(rows_here > 0 ? qw : 0)) * D, rows_here * D * 2);
#pragma unroll
    for (int i = 0; i < T::kRowLoads; ++i)
      qreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrsrc, (i * 64 + lane) * 16, 0, 0));
  }
  bf16x8 qf[D / 16];

  // ---- tile loaders ---------------------------------------------------------
  // K and V rows go from memory straight into LDS (buffer_load_dwordx4 with
  // the LDS flag: 64 lanes x 16 bytes, lane l's bytes written at M0 + 16 l),
  // 1 KiB per instruction, with no staging registers and no LDS-write
  // instructions.  The loads are buffer loads over this head's K or V: rows
  // past Sk fall outside the buffer range and arrive as 0 (those keys are
  // masked).  The slots hold unpadded rows (D * 2 bytes) with their 16-byte
  // chunks XOR-swizzled, so that the operand reads have no bank conflicts
  // (64 banks x 4 bytes = one 256-byte line, holding kRowsPerLine rows):
  //   * K: chunk c of key r sits at position c ^ kswz(r).  The 16 lanes of
  //     one operand-read phase read the same chunk of 16 consecutive keys,
  //     which then land in 16 distinct 16-byte slots of a line;
  //   * V: chunk c of key r sits at c ^ vswz(r), which moves the 64-byte
  //     column groups: one transposed-read phase reads 4 consecutive keys x
  //     64 bytes, which then cover a line.
  // Each lane loads the global chunk its LDS position holds.  The waves that
  // stage a tile (a group's four in the key split, else all eight) move its
  // pieces n (rows (1024 / kRowBytes) n on) in turn.  The loads are inline
  // asm: the compiler would otherwise wait for every one of them before each
  // LDS read (it cannot tell the rows from the operands).  They are the only
  // vector-memory loads of the tile loop, and each wave waits for its own
  // (vmcnt) before the barrier that publishes them.
  constexpr int kRowBytes = D * 2;
  constexpr int kChunksRow = kRowBytes / 16;       // 16-byte chunks per row: 16 or 8
  constexpr int kRowsPerLine = 16 / kChunksRow;    // rows per 256-byte bank line: 1 or 2
  constexpr int kRowsPiece = 1024 / kRowBytes;     // rows per 1 KiB load
  constexpr int kStagers = SPLIT ? 4 : 8;          // waves staging one tile
  constexpr int kDmaPieces = kBlockN * kRowBytes / 1024 / kStagers;  // per wave and tile
  static_assert(kDmaPieces >= 1 && kDmaPieces * 1024 * kStagers == kBlockN * kRowBytes &&
                kBlockN * kRowBytes <= T::kKBytes && kBlockN * kRowBytes <= T::kVBytes,
                "whole pieces; an unpadded tile fits a slot");
  auto kswz = [](int r) { return (r / kRowsPerLine) & (kChunksRow - 1); };
  auto vswz = [](int r) { return 4 * ((r / kRowsPerLine) & (4 / kRowsPerLine - 1)); };
  const int kv_bytes = Sk * D * 2;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, 0, kv_bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, 0, kv_bytes, kBufferFlags);
  const int set = SPLIT ? group : 0;  // this group's slot pair
  auto kslot = [&](int j) { return (2 * set + (j & 1)) * T::kKBytes; };
  auto vslot = [&](int j) { return T::kVOff + (2 * set + (j & 1)) * T::kVBytes; };
  const int dma_wave = SPLIT ? (wave & 3) : wave;  // this wave's rank among a tile's stagers
  const unsigned smem_base = (unsigned)(uintptr_t)smem;  // LDS byte address of smem
  // The lane's byte offset in piece e: row row_in of the piece, the global
  // chunk that its position p holds.  vswz of a piece's rows does not depend
  // on the piece (a piece starts at a multiple of 4 lines' rows).
  unsigned k_voff[kDmaPieces], v_voff;
  {
    const int row_in = lane / kChunksRow, p = lane % kChunksRow;
#pragma unroll
    for (int e = 0; e < kDmaPieces; ++e) {
      const int r = (dma_wave * kDmaPieces + e) * kRowsPiece + row_in;
      k_voff[e] = row_in * kRowBytes + ((p ^ kswz(r)) << 4);
    }
    v_voff = row_in * kRowBytes + ((p ^ vswz(row_in)) << 4);
  }
  auto dma_tile = [&](__amdgpu_buffer_rsrc_t rsrc, bool is_k, int t, int slot) {
    const int tile_off = t * kBlockN * kRowBytes;
#pragma unroll
    for (int e = 0; e < kDmaPieces; ++e) {
      const int n = dma_wave * kDmaPieces + e;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                   :: "s"(__builtin_amdgcn_readfirstlane(smem_base + slot + n * 1024)),
                      "v"(is_k ? k_voff[e] : v_voff), "s"(rsrc),
                      "s"(__builtin_amdgcn_readfirstlane(tile_off + n * 1024))
                   : "memory", "m0");
    }
  };
  auto dma_wait_all = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // Operand addresses.  K: lane (l32, half) reads chunk 2a + half of key
  // 32 (i & 1) + l32 for MFMA i (a = i / 2); kswz of that key is kswz(l32).
  // V: lane reads rows 16 g + 4 half + s16 / 4 (+ 8) at column group db,
  // 32 ((lane >> 4) & 1) + 8 (s16 & 3) bytes in; vswz of those rows is
  // vswz(4 half + s16 / 4).  Offsets per chunk pair and column group, the
  // rest immediates.
  const int s16 = lane & 15;
  unsigned kofs[D / 16], vofs[D / 32];
  // The offsets include this group's slot pair, so that within a tile
  // iteration only the slot parity (a compile-time immediate) is added.
#pragma unroll
  for (int a = 0; a < D / 16; ++a)
    kofs[a] = kslot(0) + l32 * kRowBytes + (((2 * a + half) ^ kswz(l32)) << 4);
  {
    const int vr = 4 * half + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      vofs[db] = vslot(0) + vr * kRowBytes + 64 * (db ^ (vswz(vr) >> 2)) + 32 * ((lane >> 4) & 1) +
                 8 * (s16 & 3);
  }
  auto k_operand = [&](int kbase, int i) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(smem + kbase + kofs[i >> 1] + (i & 1) * 32 * kRowBytes);
  };
  auto v_operand = [&](int vbase, int i) -> bf16x8 {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int g = i / (D / 32), db = i % (D / 32);
    const unsigned char* vs = smem + vbase + vofs[db] + 16 * g * kRowBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)vs);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vs + 8 * kRowBytes));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  f32x16 s[2] = {f32x16{}, f32x16{}};
  bf16x8 pf[2][2];
  float mref = -FLT_MAX;  // reference max in exp2 units (see softmax_tile)
  float l_run = 0.f;
  // exp2 argument scale, scale*log2(e), kept >= the smallest normal float: a
  // zero (or tiny) scale then still gives every visible key p = exp2(~0) = 1
  // exactly, as scale = 0 does, while masked -inf scores keep p = 0.  With
  // the bias, kscale >= 2^-64 already.
  const float c = ALIBI ? kscale * kLog2e : fmaxf(scale * kLog2e, 1.17549435e-38f);

  constexpr int kN = 2 * (D / 16);  // MFMAs of each product per tile
  static_assert(kN == 4 * (D / 32), "both products take the same number of MFMAs");
  constexpr int kP = TILEATTN_PREFETCH;

  // Matrix phase: S_j (WITH_S) and acc += V_{j-1}^T P_{j-1}^T (WITH_PV),
  // MFMA by MFMA alternating, operands read kP steps ahead.
  auto matrix_body = [&](auto with_s_c, auto with_pv_c, int j, auto par) {
    constexpr bool WITH_S = decltype(with_s_c)::value;
    constexpr bool WITH_PV = decltype(with_pv_c)::value;
    // Tile j's K and tile j-1's V sit in the slots of parity j & 1 and
    // (j - 1) & 1: byte offsets from the pair's first slots (compile-time
    // constants inside the loop, where par is an integral_constant).
    const int kb = static_cast<int>(par) * T::kKBytes;
    const int vb = (1 - static_cast<int>(par)) * T::kVBytes;
    // Keep the operand offsets opaque here, so that the compiler folds
    // kb + ... into each read's immediate instead of hoisting every
    // offset + constant out of the loop into a register of its own (not in
    // the bias instances, which take runtime parities; see the tile loop).
    if constexpr (!ALIBI) {
#pragma unroll
      for (int a = 0; a < D / 16; ++a) asm volatile("" : "+v"(kofs[a]));
#pragma unroll
      for (int d = 0; d < D / 32; ++d) asm volatile("" : "+v"(vofs[d]));
    }
    if (TILEATTN_SETPRIO) __builtin_amdgcn_s_setprio(1);
    bf16x8 kring[kP], vring[kP];
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      if (WITH_S) kring[i] = k_operand(kb, i);
      if (WITH_PV) vring[i] = v_operand(vb, i);
    }
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (WITH_S)
        s[i & 1] = mfma16<IS_F16>(kring[i % kP], qf[i >> 1], (i < 2 && !ALIBI) ? f32x16{} : s[i & 1]);
      if (WITH_PV) {
        const int g = i / (D / 32), db = i % (D / 32);
        acc[db] = mfma16<IS_F16>(vring[i % kP], pf[g >> 1][g & 1], acc[db]);
      }
      if (i + kP < kN) {
        if (WITH_S) kring[i % kP] = k_operand(kb, i + kP);
        if (WITH_PV) vring[i % kP] = v_operand(vb, i + kP);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (TILEATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
  };
  // With a block mask, a wave skips the products of the tiles its query
  // block cannot see: their probabilities would all be 0.
  auto matrix_phase = [&](auto with_s_c, auto with_pv_c, int j, auto par) {
    using TT_ = std::true_type;
    using FF_ = std::false_type;
    constexpr bool WITH_S = decltype(with_s_c)::value;
    constexpr bool WITH_PV = decltype(with_pv_c)::value;
    if constexpr (!MASK) {
      matrix_body(with_s_c, with_pv_c, j, par);
    } else {
      // Two independent products, one after the other, each behind its own
      // wave-uniform branch (one body with both would need four variants).
      if (WITH_S && wave_sees(j)) matrix_body(TT_{}, FF_{}, j, par);
      if (WITH_PV && wave_sees(j - 1)) matrix_body(FF_{}, TT_{}, j, par);
    }
  };

  // Bias of tile j in units of 1/kscale, written into s as the starting value
  // of the S product: key - row = d, bias = slope * d (causal: every visible
  // d <= 0) or -slope * |d| (non-causal).  One FMA per score when causal.
  auto bias_init = [&](int j) {
    const float d0 = (float)(tile(j) * kBlockN + 4 * half - my_row);
    const float b0 = sigma * d0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float kr = (float)(kb * 32 + 8 * (r >> 2) + (r & 3));
        s[kb][r] = CAUSAL ? fmaf(sigma, kr, b0) : -sigma * fabsf(d0 + kr);
      }
  };

  // Vector phase: mask tile j where needed, online softmax, pack P_j; with
  // the bias, then the starting value of S_{j+1}.
  // Tiles past a causal wave's diagonal come out fully masked (p = 0): the
  // tile max is -inf, the reference max stays, and acc and l are unchanged.
  // With a block mask, a tile this wave cannot see changes nothing (its
  // matrix phases skip it too).
  auto vector_phase = [&](int j) {
    if (!MASK || wave_sees(j)) {
      const int key0 = tile(j) * kBlockN;
      const bool need_mask = (CAUSAL && key0 + kBlockN - 1 > qw) || (key0 + kBlockN > Sk);
      if (need_mask) {
        const int lim = (CAUSAL ? min(Sk - 1, my_row) : Sk - 1) - key0 - 4 * half;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3) <= lim) ? s[kb][r] : -INFINITY;
      }
      // c > 0 here, so a masked (-inf) score gives p = exp2(-inf) = 0 without
      // a separate masked code path.
      softmax_tile<IS_F16, ALIBI && !CAUSAL>(s, mref, l_run, c, acc, pf);
    }
    if constexpr (ALIBI)
      if (j + 1 < nt) bias_init(j + 1);
  };

  using TT = std::true_type;
  using FF = std::false_type;
  // One iteration (both groups): the first half runs; K_{j+1} and V_j go
  // into the slots that K_{j-1} and V_{j-2} left (free since the previous
  // closing barrier); the second half runs; and the rows land before the
  // closing barrier, which publishes them for iteration j+1.  (Issued
  // between the halves rather than at the top: 1-2% faster.)  No LDS access
  // of one half depends on the other group's other half, so the barrier
  // between the halves only paces the ping-pong: the key split keeps it
  // (2-10% faster with it); the 256-row kernel runs without it (2-4% faster
  // so).
  auto iteration = [&](int j, auto first, auto second) {
    TILEATTN_CHECK_BARRIER();
    first();
    if (j + 1 < nt) dma_tile(krsrc, true, tile(j + 1), kslot(j + 1));
    if (j < nt) dma_tile(vrsrc, false, tile(j), vslot(j));
    TILEATTN_CHECK_BARRIER();
    if constexpr (SPLIT) __builtin_amdgcn_s_barrier();
    second();
    TILEATTN_CHECK_BARRIER();
    dma_wait_all();
    __syncthreads();
  };

  // A workgroup whose block mask shows it no tile skips the loop: its rows
  // have no visible key (o = 0, lse = -inf below).
  if (!MASK || nt > 0) {
    if constexpr (ALIBI) bias_init(0);
    dma_tile(krsrc, true, tile(0), kslot(0));
    if (row_owner) {
#pragma unroll
      for (int i = 0; i < T::kRowLoads; ++i) {
        const int idx = i * 64 + lane;
        *reinterpret_cast<u32x4*>(stage + (idx / T::kChunks) * T::kKPitch + (idx % T::kChunks) * 16) = qreg[i];
      }
    }
    dma_wait_all();
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(stage + l32 * T::kKPitch + kk * 32 + half * 16);
    // Staging over the V slots: every wave's Q reads complete before any
    // wave writes V_0 there.
    if constexpr (T::kStageOverV) __syncthreads();

    // Tiles in pairs (odd j, then even j), so that each matrix phase has its
    // slot parity as a compile-time constant and the slot offsets fold into
    // the LDS instructions' immediates (the compiler does not unroll a loop
    // with barriers by itself).  The bias instances, at the register limit,
    // keep one tile per loop step and a runtime parity.
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    constexpr bool kPairs = !ALIBI;
    int j = 1;
    if (group == 0) {
      iteration(0, [&] { matrix_phase(TT{}, FF{}, 0, P0{}); }, [&] { vector_phase(0); });
      if constexpr (kPairs) {
        for (; j + 1 < nt; j += 2) {
          iteration(j, [&] { matrix_phase(TT{}, TT{}, j, P1{}); }, [&] { vector_phase(j); });
          iteration(j + 1, [&] { matrix_phase(TT{}, TT{}, j + 1, P0{}); }, [&] { vector_phase(j + 1); });
        }
        if (j < nt) iteration(j, [&] { matrix_phase(TT{}, TT{}, j, P1{}); }, [&] { vector_phase(j); });
      } else {
        for (; j < nt; ++j)
          iteration(j, [&] { matrix_phase(TT{}, TT{}, j, j & 1); }, [&] { vector_phase(j); });
      }
      iteration(nt, [&] { matrix_phase(FF{}, TT{}, nt, nt & 1); }, [&] {});
    } else {
      iteration(0, [&] {}, [&] { matrix_phase(TT{}, FF{}, 0, P0{}); });
      if constexpr (kPairs) {
        for (; j + 1 < nt; j += 2) {
          iteration(j, [&] { vector_phase(j - 1); }, [&] { matrix_phase(TT{}, TT{}, j, P1{}); });
          iteration(j + 1, [&] { vector_phase(j); }, [&] { matrix_phase(TT{}, TT{}, j + 1, P0{}); });
        }
        if (j < nt) iteration(j, [&] { vector_phase(j - 1); }, [&] { matrix_phase(TT{}, TT{}, j, P1{}); });
      } else {
        for (; j < nt; ++j)
          iteration(j, [&] { vector_phase(j - 1); }, [&] { matrix_phase(TT{}, TT{}, j, j & 1); });
      }
      iteration(nt, [&] { vector_phase(nt - 1); }, [&] { matrix_phase(FF{}, TT{}, nt, nt & 1); });
    }
  }

  // ---- key split: merge group 1's partial state into group 0's -------------
  // Each group holds acc, l and the reference max of the same 32 rows over
  // its half of the keys, both against their own reference.  Group 1's goes
  // through LDS (over the K slots, free after the loop); group 0 rescales
  // both to the larger reference and adds: the same update as the online
  // softmax takes between two tiles.
  if constexpr (SPLIT) {
    constexpr int kXchg = 64 * (D / 2 + 2);  // floats per row pair
    static_assert(T::kRowWaves * kXchg * 4 <= T::kVOff, "exchange must fit in the K slots");
    float* const xchg = reinterpret_cast<float*>(smem) + rw * kXchg;
    if (group == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(xchg + ((db * 4 + q4) * 64 + lane) * 4) =
              f32x4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]};
      xchg[64 * (D / 2) + lane] = mref;
      xchg[64 * (D / 2) + 64 + lane] = l_run;
    }
    __syncthreads();
    if (group == 0) {
      const float m1 = xchg[64 * (D / 2) + lane];
      const float l1 = xchg[64 * (D / 2) + 64 + lane];
      const float m = fmaxf(mref, m1);
      const float a0 = __builtin_amdgcn_exp2f(mref - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(xchg + ((db * 4 + q4) * 64 + lane) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * q4 + e] = fmaf(acc[db][4 * q4 + e], a0, x[e] * a1);
        }
      l_run = fmaf(l_run, a0, l1 * a1);
      mref = m;
    }
  }

  // ---- a chunk of several: its partial state goes to the workspace --------
  // The unnormalised acc in the accumulator's own register layout (entry
  // ((rw * D/32 + db) * 4 + g) * 64 + lane of f32x4, i.e. 1 KiB per store
  // instruction), then the rows' reference max (exp2 units) and sum;
  // attn_merge_kernel combines the chunks of the query tile.  Rows past Sq
  // are not written.
  const float l_tot = wave_pair_sum(l_run);
  if (chunked && nchunks > 1) {
    if (group == 0 && my_row < Sq) {
      float* const part = ws + (size_t)blockIdx.x * kChunkFloats<D>;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(part + (((rw * (D / 32) + db) * 4 + g) * 64 + lane) * 4) =
              f32x4{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
      if (half == 0) {
        part[kChunkRows * D + rw * kRowsPerWave + l32] = mref;
        part[kChunkRows * D + kChunkRows + rw * kRowsPerWave + l32] = l_tot;
      }
    }
    return;
  }

  // ---- epilogue: O = acc / l, lse = m*scale + ln l = mref*ln2 + ln l ---------
  // Block mask: a row with no visible key (l = 0, mref = -FLT_MAX) gets
  // o = 0, lse = -inf.
  const float inv = (MASK && !(l_tot > 0.f)) ? 0.f : 1.0f / l_tot;
  // The lane's pieces of its row (4 x 4 consecutive d) go to the wave's LDS
  // area, and the rows leave it whole: 1 KiB per store instruction.  Split:
  // group 0 alone writes the rows (group 1 only meets the barrier).
  if (row_owner) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __bf16 o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = round16<IS_F16>(acc[db][4 * g + e] * inv);
        uint2 u;
        u.x = (uint32_t)__builtin_bit_cast(uint16_t, o4[0]) |
              ((uint32_t)__builtin_bit_cast(uint16_t, o4[1]) << 16);
        u.y = (uint32_t)__builtin_bit_cast(uint16_t, o4[2]) |
              ((uint32_t)__builtin_bit_cast(uint16_t, o4[3]) << 16);
        *reinterpret_cast<uint2*>(stage + l32 * T::kKPitch + (db * 32 + 8 * g + 4 * half) * 2) = u;
      }
  }
  __syncthreads();
  if (row_owner) {
    // All reads first, then the stores: a buffer store past the wave's last
    // row (Sq) falls outside the buffer range and is dropped, so no store
    // needs a branch (which would serialise each read with its store).
    const int rows_here = max(0, min(kRowsPerWave, Sq - qw));
    const __amdgpu_buffer_rsrc_t orsrc = wave_buffer(O + (q_head + (size_t)(rows_here > 0 ? qw : 0)) * D, rows_here * D * 2);
    u32x4 orow[T::kRowLoads];
#pragma unroll
    for (int i = 0; i < T::kRowLoads; ++i) {
      const int idx = i * 64 + lane;
      orow[i] = *reinterpret_cast<const u32x4*>(stage + (idx / T::kChunks) * T::kKPitch + (idx % T::kChunks) * 16);
    }
#pragma unroll
    for (int i = 0; i < T::kRowLoads; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(orow[i], orsrc, (i * 64 + lane) * 16, 0, 0);
  }
  if (row_owner && half == 0 && my_row < Sq) LSE[q_head + my_row] = mref * kLn2 + logf(l_tot);
}

// ---------------------------------------------------------------------------
// Merge of a chunked key split: per query tile with several chunks, the
// chunks' partial states (acc, reference max m and sum l of every row, over
// disjoint key ranges) combine as the online softmax combines two tiles:
// with M = max_c m_c, O = sum_c 2^(m_c - M) acc_c / L, L = sum_c 2^(m_c - M) l_c,
// lse = M ln 2 + ln L.  Workgroup 4 w + s takes row wave s of workgroup w
// (32 positions of one query head, as the attention kernel's head packing
// assigns them); its 256 threads read the chunks' accumulators in their
// stored order (a thread keeps one row and D / 8 of its columns), and the
// rows leave through LDS whole.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool IS_F16>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const float* __restrict__ ws, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Hq, int Hkv, int Sq, int Sk, int nqt, int nwg, int chunk_tiles, int pack_shift) {
  constexpr int kPitch = D * 2 + 16;  // bytes per staged output row
  __shared__ __attribute__((aligned(16))) unsigned char stage[kRowsPerWave * kPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = tid >> 6;
  const int w = (int)blockIdx.x >> 2, slice = (int)blockIdx.x & 3;
  const int wph_shift = 2 - pack_shift;  // log2 row waves per head (4 row waves)
  const int PW = kChunkRows >> pack_shift;
  int b, hgrp, qt;
  map_workgroup(w, nwg, Hkv, (Hq / Hkv) >> pack_shift, nqt, CAUSAL, b, hgrp, qt);
  const int hq = (hgrp << pack_shift) + (slice >> wph_shift);
  const int q0 = qt * PW + ((slice & ((1 << wph_shift) - 1)) << 5);
  int nkt = (Sk + kBlockN - 1) / kBlockN;
  if (CAUSAL) nkt = min(nkt, min(qt * PW + PW - 1, Sq - 1) / kBlockN + 1);
  const int nchunks = (nkt + chunk_tiles - 1) / chunk_tiles;
  if (nchunks < 2 || q0 >= Sq) return;  // a single chunk wrote its own rows

  const int r = slice * kRowsPerWave + (lane & 31);  // row within the query tile
  const bool live = q0 + (lane & 31) < Sq;             // rows past Sq were not written
  float M = -FLT_MAX, L = 0.f;
  f32x4 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Chunks in batches of kBatch: all loads of a batch are issued before the
  // first is used.  A chunk past the last (m = -FLT_MAX, l = 0, acc = 0)
  // adds nothing.
  constexpr int kBatch = 4;
  for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
    float m[kBatch], l[kBatch];
    f32x4 x[kBatch][D / 32];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      m[u] = -FLT_MAX;
      l[u] = 0.f;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) x[u][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (live && c0 + u < nchunks) {
        const float* part = ws + (size_t)((c0 + u) * nwg + w) * kChunkFloats<D>;
        m[u] = part[kChunkRows * D + r];
        l[u] = part[kChunkRows * D + kChunkRows + r];
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
          x[u][i] = *reinterpret_cast<const f32x4*>(part + (((slice * (D / 32) + i) * 4 + g) * 64 + lane) * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float mn = fmaxf(M, m[u]);
      const float a = __builtin_amdgcn_exp2f(M - mn), bw = __builtin_amdgcn_exp2f(m[u] - mn);
      M = mn;
      L = fmaf(L, a, l[u] * bw);
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(acc[i][e], a, x[u][i][e] * bw);
    }
  }
  const float inv = 1.0f / L;
  // Element e of acc[i] is column 32 i + 8 g + 4 (lane / 32) + e of row r.
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    __bf16 o4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] = round16<IS_F16>(acc[i][e] * inv);
    uint2 u;
    u.x = (uint32_t)__builtin_bit_cast(uint16_t, o4[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, o4[1]) << 16);
    u.y = (uint32_t)__builtin_bit_cast(uint16_t, o4[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, o4[3]) << 16);
    *reinterpret_cast<uint2*>(stage + (lane & 31) * kPitch + (32 * i + 8 * g + 4 * (lane >> 5)) * 2) = u;
  }
  const size_t q_head = ((size_t)b * Hq + hq) * (size_t)Sq;
  if (tid < kRowsPerWave && q0 + tid < Sq) LSE[q_head + q0 + tid] = M * kLn2 + logf(L);
  __syncthreads();
  constexpr int kPieces = kRowsPerWave * D * 2 / 16;  // 16-byte pieces of the slice
#pragma unroll
  for (int p = tid; p < kPieces; p += 256) {
    const int row = p / (D / 8), col = p % (D / 8);
    if (q0 + row < Sq)
      *reinterpret_cast<u32x4*>(O + (q_head + q0 + row) * D + col * 8) =
          *reinterpret_cast<const u32x4*>(stage + row * kPitch + col * 16);
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: same structure, v_mfma_f32_32x32x2_f32, 32-key tiles, P in fp32.
// ---------------------------------------------------------------------------
template <int D>
struct F32Layout {
  static constexpr int kPitch = D + 1;                       // floats per LDS row (pad: banks)
  static constexpr int kTileFloats = kBlockNF32 * kPitch;
  static constexpr int kLoadsPerThread = kBlockNF32 * D / 4 / kF32Threads;  // float4 loads
  static_assert(kLoadsPerThread * kF32Threads * 4 == kBlockNF32 * D, "tile/threads mismatch");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Threads) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Sq, int Sk,
    float scale, int nqt, int nwg) {
  using L = F32Layout<D>;
  __shared__ float ks[L::kTileFloats];
  __shared__ float vs[L::kTileFloats];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wave = tid >> 6;
  const int G = Hq / Hkv;

  int b, hq, qt;
  map_workgroup(blockIdx.x, nwg, Hkv, G, nqt, CAUSAL, b, hq, qt);
  const int hk = hq / G;
  const int q0 = qt * kF32BlockM;
  const int qw = q0 + wave * kRowsPerWave;
  const int my_row = qw + l32;

  const size_t q_head = ((size_t)b * Hq + hq) * (size_t)Sq;
  const size_t kv_head = ((size_t)b * Hkv + hk) * (size_t)Sk;
  const float* Kh = K + kv_head * D;
  const float* Vh = V + kv_head * D;

  int nkt = (Sk + kBlockNF32 - 1) / kBlockNF32;
  if (CAUSAL) {
    const int last_row = min(q0 + kF32BlockM - 1, Sq - 1);
    nkt = min(nkt, last_row / kBlockNF32 + 1);
  }

  // Q fragment: B operand (k = d, n = query); lane holds d = 2*kk + half.
  float qf[D / 2];
  {
    const bool ok = my_row < Sq;
    const float* qrow = Q + (q_head + (size_t)(ok ? my_row : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) qf[kk] = ok ? qrow[2 * kk + half] : 0.f;
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = scale * kLog2e;

  for (int j = 0; j < nkt; ++j) {
    const int key0 = j * kBlockNF32;
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < L::kLoadsPerThread; ++i) {
      const int idx = tid + i * kF32Threads;
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
      if (key0 + r < Sk) {
        kv4 = *reinterpret_cast<const float4*>(Kh + (size_t)(key0 + r) * D + c4 * 4);
        vv4 = *reinterpret_cast<const float4*>(Vh + (size_t)(key0 + r) * D + c4 * 4);
      }
      float* kd = ks + r * L::kPitch + c4 * 4;
      float* vd = vs + r * L::kPitch + c4 * 4;
      kd[0] = kv4.x; kd[1] = kv4.y; kd[2] = kv4.z; kd[3] = kv4.w;
      vd[0] = vv4.x; vd[1] = vv4.y; vd[2] = vv4.z; vd[3] = vv4.w;
    }
    __syncthreads();

    const bool wave_active = !CAUSAL || key0 <= qw + kRowsPerWave - 1;
    if (!wave_active) continue;

    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
      const float a = ks[l32 * L::kPitch + 2 * kk + half];
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[kk], s, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
      const bool vis = key < Sk && (!CAUSAL || key <= my_row);
      s[r] = vis ? s[r] : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = wave_pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f((m_run - m_new) * c);
    m_run = m_new;
    const float mc = m_new * c;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = s[r];
      const float p = (x == -INFINITY) ? 0.f : exp2f(fmaf(x, c, -mc));
      s[r] = p;
      psum += p;
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      acc[db] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * half + (r & 3);
        const float a = vs[key * L::kPitch + db * 32 + l32];
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[r], acc[db], 0, 0, 0);
      }
    }
  }

  const float l_tot = wave_pair_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (my_row < Sq) {
    float* orow = O + (q_head + my_row) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 u = make_float4(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
                               acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
        *reinterpret_cast<float4*>(orow + db * 32 + 8 * g + 4 * half) = u;
      }
    if (half == 0) LSE[q_head + my_row] = m_run * scale + logf(l_tot);
  }
}

// ---------------------------------------------------------------------------
// Host side: validation and launch.
// ---------------------------------------------------------------------------
int validate(const void* q, const void* k, const void* v, const void* o, const void* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale, bool* empty) {
  *empty = false;
  if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 1 || Sk < 1) return TILEATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0) return TILEATTN_ERR_GQA_RATIO;
  if (D != 64 && D != 128) return TILEATTN_ERR_HEAD_DIM;
  if (!(scale >= 0.f) || isinf(scale)) return TILEATTN_ERR_SCALE;
  // Row indices inside the kernels stay within int: Sq <= 2^30.
  if (Sq > (1 << 30)) return TILEATTN_ERR_TOO_LARGE;
  // 64-bit index range: elements of q/o and of k/v, and the workgroup count.
  const double q_elems = (double)B * Hq * Sq * D;
  const double kv_elems = (double)B * Hkv * Sk * D;
  const double nwg = (double)B * Hq * ((Sq + kF32BlockM - 1) / kF32BlockM);  // smallest block_m
  // One head's K or V is addressed with 32-bit buffer offsets.
  const double head_bytes = (double)Sk * D * 4;
  if (q_elems > 9.0e18 || kv_elems > 9.0e18 || nwg > 2147483647.0 || head_bytes > 2147483647.0)
    return TILEATTN_ERR_TOO_LARGE;
  if (B == 0 || Hq == 0 || Sq == 0) {
    *empty = true;
    return TILEATTN_OK;
  }
  if (!q || !k || !v || !o || !lse) return TILEATTN_ERR_NULL_POINTER;
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return TILEATTN_ERR_ALIGNMENT;
  return TILEATTN_OK;
}

template <int BLOCK_M, int THREADS, typename Kern, typename TIn, typename TOut>
int launch(Kern kernel, const TIn* q, const TIn* k, const TIn* v, TOut* o, float* lse, int B,
           int Hq, int Hkv, int Sq, int Sk, float scale, void* stream) {
  const int nqt = (Sq + BLOCK_M - 1) / BLOCK_M;
  const int nwg = B * Hq * nqt;
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse, (void*)&Hq,
                  (void*)&Hkv, (void*)&Sq, (void*)&Sk, (void*)&scale, (void*)&nqt, (void*)&nwg};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(nwg), dim3(THREADS),
                                 args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TILEATTN_OK : TILEATTN_ERR_LAUNCH;
}

// The 16-bit kernel takes five more arguments (bias slopes, block mask and
// its head count, and the chunked key split's chunk length and workspace);
// the plain entry points pass none.  With chunks the grid is chunk-major:
// max_chunks copies of the plain grid.
// Head packing (see the kernel): log2 of the query heads one workgroup of
// `row_waves` row waves holds: the largest power of two that divides G, at
// most row_waves, and with a block mask at most row_waves / 2 (so that every
// 64-position query block of the mask lies within one workgroup).
int pack_shift_for(int G, int row_waves, bool mask) {
  const int cap = mask ? row_waves / 2 : row_waves;
  int s = 0;
  while ((2 << s) <= cap && G % (2 << s) == 0) ++s;
  return s;
}

// Workgroups of a grid of `rows`-row workgroups with head packing ps:
// B * (Hq / 2^ps) head groups times ceil(Sq / (rows / 2^ps)) query tiles.
long long grid_workgroups(int B, int Hq, int Sq, int rows, int ps) {
  const int pw = rows >> ps;
  return (long long)B * (Hq >> ps) * ((Sq + pw - 1) / pw);
}

template <int BLOCK_M, int THREADS, typename Kern>
int launch16(Kern kernel, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
             float* lse, int B, int Hq, int Hkv, int Sq, int Sk, float scale,
             const float* slopes, const unsigned char* bmask, int mask_heads, int pack_shift, void* stream,
             int chunk_tiles = 0, int max_chunks = 1, float* ws = nullptr) {
  const int pw = BLOCK_M >> pack_shift;
  const int nqt = (Sq + pw - 1) / pw;
  const int nwg = B * (Hq >> pack_shift) * nqt;
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse, (void*)&Hq,
                  (void*)&Hkv, (void*)&Sq, (void*)&Sk, (void*)&scale, (void*)&nqt, (void*)&nwg,
                  (void*)&slopes, (void*)&bmask, (void*)&mask_heads, (void*)&chunk_tiles, (void*)&ws,
                  (void*)&pack_shift};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(nwg * max_chunks), dim3(THREADS),
                                 args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TILEATTN_OK : TILEATTN_ERR_LAUNCH;
}

// Compute units of the current device, queried once per device.
int compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> count[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The 16-bit kernel runs 256-row workgroups unless that grid would leave at
// least half the compute units idle; then the key split's 128-row
// workgroups, each wave with half the tiles.
bool use_split(int B, int Hq, int Hkv, int Sq, bool mask) {
  const long long wg256 = grid_workgroups(B, Hq, Sq, 256, pack_shift_for(Hq / Hkv, 8, mask));
  return 2 * wg256 <= compute_units();
}

// Chunked key split (tileattn_fwd_ws): on a key-split grid whose heaviest
// query tile has far more key tiles than the chip's balanced share, the
// query tiles' key ranges are cut into chunks of about that share (an even
// number of tiles, at least kMinChunkTiles), each its own workgroup, and a
// second kernel merges the chunks of each query tile.  Without it the grid
// lasts as long as its heaviest query tile while most compute units idle.
// The merge and the partial states cost about 5 us; measured on MI355X, a
// split pays once the heaviest query tile has 1.5 chunks and at least
// kMinSplitTiles key tiles (at 32 tiles, a 2K causal grid, it lost 15%).
constexpr int kMinChunkTiles = 16;
constexpr int kMinSplitTiles = 48;

struct ChunkPlan {
  int chunk_tiles = 0;  // 0: no chunks
  int max_chunks = 1;   // chunks of the heaviest query tile
  int pack_shift = 0;   // head packing of the key-split grid
  size_t bytes = 0;     // workspace bytes
};

ChunkPlan chunk_plan(int B, int Hq, int Hkv, int Sq, int Sk, int D, bool causal) {
  ChunkPlan plan;
  if (B == 0 || Hq == 0 || Sq == 0 || !use_split(B, Hq, Hkv, Sq, false)) return plan;
  const int ps = pack_shift_for(Hq / Hkv, 4, false);
  const int pw = kChunkRows >> ps;
  const int nqt = (Sq + pw - 1) / pw;
  const int n = (Sk + kBlockN - 1) / kBlockN;
  long long per_group = 0;
  int max_nk = 0;
  for (int qt = 0; qt < nqt; ++qt) {
    const int nk = causal ? std::min(n, std::min(qt * pw + pw - 1, Sq - 1) / kBlockN + 1) : n;
    per_group += nk;
    max_nk = std::max(max_nk, nk);
  }
  const long long nwg = (long long)B * (Hq >> ps) * nqt;
  const long long units = compute_units();
  const long long share = (nwg / nqt * per_group + units - 1) / units;
  const int c = (int)std::max<long long>(kMinChunkTiles, (share + 1) & ~1LL);
  if (2 * max_nk < 3 * c || max_nk < kMinSplitTiles) return plan;
  plan.chunk_tiles = c;
  plan.max_chunks = (max_nk + c - 1) / c;
  plan.pack_shift = ps;
  plan.bytes = (size_t)plan.max_chunks * nwg * (size_t)(kChunkRows * D + 2 * kChunkRows) * sizeof(float);
  return plan;
}

template <int D, bool IS_F16, bool ALIBI>
int launch_chunked(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                   int B, int Hq, int Hkv, int Sq, int Sk, float scale, int causal, const float* slopes,
                   const ChunkPlan& plan, float* ws, void* stream) {
  using T = Bf16Tile<D, true>;
  const int st = causal
      ? launch16<T::kBlockM, T::kThreads>(attn_fwd_16_kernel<D, true, IS_F16, false, ALIBI, true>, q, k, v, o,
                                          lse, B, Hq, Hkv, Sq, Sk, scale, slopes, nullptr, 1, plan.pack_shift,
                                          stream, plan.chunk_tiles, plan.max_chunks, ws)
      : launch16<T::kBlockM, T::kThreads>(attn_fwd_16_kernel<D, false, IS_F16, false, ALIBI, true>, q, k, v, o,
                                          lse, B, Hq, Hkv, Sq, Sk, scale, slopes, nullptr, 1, plan.pack_shift,
                                          stream, plan.chunk_tiles, plan.max_chunks, ws);
  if (st != TILEATTN_OK) return st;
  int pack_shift = plan.pack_shift;
  const int pw = kChunkRows >> pack_shift;
  int nqt = (Sq + pw - 1) / pw;
  int nwg = B * (Hq >> pack_shift) * nqt;
  int chunk_tiles = plan.chunk_tiles;
  const float* wsc = ws;
  void* args[] = {(void*)&wsc, (void*)&o, (void*)&lse, (void*)&Hq, (void*)&Hkv, (void*)&Sq,
                  (void*)&Sk, (void*)&nqt, (void*)&nwg, (void*)&chunk_tiles, (void*)&pack_shift};
  const void* merge = causal ? reinterpret_cast<const void*>(attn_merge_kernel<D, true, IS_F16>)
                             : reinterpret_cast<const void*>(attn_merge_kernel<D, false, IS_F16>);
  hipError_t e = hipLaunchKernel(merge, dim3(4 * nwg), dim3(256), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TILEATTN_OK : TILEATTN_ERR_LAUNCH;
}

template <int D, bool IS_F16, bool MASK, bool ALIBI, bool SPLIT>
int launch_waves(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, float scale, int causal,
                 const float* slopes, const unsigned char* bmask, int mask_heads, void* stream) {
  using T = Bf16Tile<D, SPLIT>;
  const int ps = pack_shift_for(Hq / Hkv, T::kRowWaves, MASK);
  return causal ? launch16<T::kBlockM, T::kThreads>(attn_fwd_16_kernel<D, true, IS_F16, MASK, ALIBI, SPLIT>,
                                                    q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, scale, slopes, bmask,
                                                    mask_heads, ps, stream)
                : launch16<T::kBlockM, T::kThreads>(attn_fwd_16_kernel<D, false, IS_F16, MASK, ALIBI, SPLIT>,
                                                    q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, scale, slopes, bmask,
                                                    mask_heads, ps, stream);
}

// bf16 and fp16 inputs share one kernel template (IS_F16); a block mask and
// the linear bias select the MASK / ALIBI instances.
template <int D, bool IS_F16, bool MASK, bool ALIBI>
int launch_variant(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                   int B, int Hq, int Hkv, int Sq, int Sk, float scale, int causal,
                   const float* slopes, const unsigned char* bmask, int mask_heads, void* stream) {
  // Small grids take the key split.
  if (use_split(B, Hq, Hkv, Sq, MASK))
    return launch_waves<D, IS_F16, MASK, ALIBI, true>(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, scale, causal,
                                                      slopes, bmask, mask_heads, stream);
  return launch_waves<D, IS_F16, MASK, ALIBI, false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, scale, causal,
                                                     slopes, bmask, mask_heads, stream);
}

template <bool IS_F16>
int fwd16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
          int Hkv, int Sq, int Sk, int D, float scale, int causal, const float* slopes,
          const unsigned char* bmask, int mask_heads, void* stream) {
  bool empty;
  const int st = validate(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, &empty);
  if (st != TILEATTN_OK) return st;
  if (bmask != nullptr && mask_heads != 1 && mask_heads != Hq) return TILEATTN_ERR_BAD_SHAPE;
  if (bmask != nullptr && Sk > 64 * kMaxMaskedTiles) return TILEATTN_ERR_TOO_LARGE;
  if (slopes != nullptr && (reinterpret_cast<uintptr_t>(slopes) & 3u) != 0) return TILEATTN_ERR_ALIGNMENT;
  if (empty) return TILEATTN_OK;
  auto qq = static_cast<const uint16_t*>(q), kk = static_cast<const uint16_t*>(k),
       vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(o);
#define TILEATTN_V16(MM, AA)                                                                        \
  (D == 128 ? launch_variant<128, IS_F16, MM, AA>(qq, kk, vv, oo, lse, B, Hq, Hkv, Sq, Sk, scale,  \
                                                  causal, slopes, bmask, mask_heads, stream)       \
            : launch_variant<64, IS_F16, MM, AA>(qq, kk, vv, oo, lse, B, Hq, Hkv, Sq, Sk, scale,   \
                                                 causal, slopes, bmask, mask_heads, stream))
  if (bmask != nullptr) return slopes != nullptr ? TILEATTN_V16(true, true) : TILEATTN_V16(true, false);
  return slopes != nullptr ? TILEATTN_V16(false, true) : TILEATTN_V16(false, false);
#undef TILEATTN_V16
}

// tileattn_fwd_ws: the chunked key split where chunk_plan takes it (bf16 /
// fp16, with or without the linear bias), else the unsplit kernel.
int fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
           int Hkv, int Sq, int Sk, int D, float scale, int causal, const float* slopes, int is_f16,
           void* workspace, size_t workspace_bytes, void* stream) {
  bool empty;
  const int st = validate(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, &empty);
  if (st != TILEATTN_OK || empty) return st;
  if (slopes != nullptr && (reinterpret_cast<uintptr_t>(slopes) & 3u) != 0) return TILEATTN_ERR_ALIGNMENT;
  const ChunkPlan plan = chunk_plan(B, Hq, Hkv, Sq, Sk, D, causal != 0);
  if (plan.chunk_tiles == 0)
    return is_f16 ? fwd16<true>(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, slopes, nullptr, 1, stream)
                  : fwd16<false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, slopes, nullptr, 1, stream);
  if (workspace == nullptr || workspace_bytes < plan.bytes) return TILEATTN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return TILEATTN_ERR_ALIGNMENT;
  auto qq = static_cast<const uint16_t*>(q), kk = static_cast<const uint16_t*>(k),
       vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(o);
  auto ws = static_cast<float*>(workspace);
#define TILEATTN_CHUNKED(DD, FF, AA) \
  launch_chunked<DD, FF, AA>(qq, kk, vv, oo, lse, B, Hq, Hkv, Sq, Sk, scale, causal, slopes, plan, ws, stream)
  if (slopes != nullptr) {
    if (D == 128) return is_f16 ? TILEATTN_CHUNKED(128, true, true) : TILEATTN_CHUNKED(128, false, true);
    return is_f16 ? TILEATTN_CHUNKED(64, true, true) : TILEATTN_CHUNKED(64, false, true);
  }
  if (D == 128) return is_f16 ? TILEATTN_CHUNKED(128, true, false) : TILEATTN_CHUNKED(128, false, false);
  return is_f16 ? TILEATTN_CHUNKED(64, true, false) : TILEATTN_CHUNKED(64, false, false);
#undef TILEATTN_CHUNKED
}

}  // namespace

// Workspace of tileattn_fwd_noalloc: one array per device, loaded with the
// code object and held until the process ends.  Host code never passes its
// name to a kernel (on the host it is a stand-in, not a device address);
// scratch_address() looks up the device address once per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

// Device address of `scratch` on the current device, or nullptr if the
// lookup fails.  The first call on a device looks it up with that device
// current and keeps it.
float* scratch_address() {
  constexpr int kMaxDevices = 64;
  static std::atomic<float*> addr[kMaxDevices];
  static std::mutex lookup;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  float* p = addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> guard(lookup);
  p = addr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) return nullptr;
    p = static_cast<float*>(a);
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int tileattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                            int causal, void* stream) {
  return fwd16<false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, nullptr, nullptr, 1, stream);
}

extern "C" int tileattn_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                                int causal, void* stream) {
  return fwd16<true>(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, nullptr, nullptr, 1, stream);
}

extern "C" int tileattn_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                                int causal, const float* alibi_slopes,
                                const unsigned char* block_mask, int mask_heads, int is_f16,
                                void* stream) {
  return is_f16 ? fwd16<true>(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, alibi_slopes,
                              block_mask, mask_heads, stream)
                : fwd16<false>(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, alibi_slopes,
                               block_mask, mask_heads, stream);
}

extern "C" long long tileattn_fwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                                 int causal) {
  bool empty;
  static const float dummy[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  const int st = validate(dummy, dummy, dummy, dummy, dummy, B, Hq, Hkv, Sq, Sk, D, 1.0f, &empty);
  if (st != TILEATTN_OK) return st;
  return empty ? 0 : (long long)chunk_plan(B, Hq, Hkv, Sq, Sk, D, causal != 0).bytes;
}

extern "C" int tileattn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                               int causal, const float* alibi_slopes, int is_f16, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return fwd_ws(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, alibi_slopes, is_f16, workspace,
                workspace_bytes, stream);
}

extern "C" int tileattn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                                    int causal, const float* alibi_slopes, int is_f16, void* stream) {
  bool empty;
  const int st = validate(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, &empty);
  if (st != TILEATTN_OK || empty) return st;
  if (alibi_slopes != nullptr && (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u) != 0) return TILEATTN_ERR_ALIGNMENT;
  const ChunkPlan plan = chunk_plan(B, Hq, Hkv, Sq, Sk, D, causal != 0);
  if (plan.chunk_tiles == 0)  // no chunks: the unsplit kernel, no workspace
    return fwd_ws(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, alibi_slopes, is_f16, nullptr, 0,
                  stream);
  if (plan.bytes > kScratchBytes) return TILEATTN_ERR_SCRATCH;
  float* const ws = scratch_address();
  if (ws == nullptr) return TILEATTN_ERR_LAUNCH;
  return fwd_ws(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, alibi_slopes, is_f16, ws, kScratchBytes,
                stream);
}

extern "C" int tileattn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                                float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                float scale, int causal, void* stream) {
  bool empty;
  const int st = validate(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, &empty);
  if (st != TILEATTN_OK || empty) return st;
  if (D == 128)
    return causal ? launch<kF32BlockM, kF32Threads>(attn_fwd_f32_kernel<128, true>, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, scale, stream)
                  : launch<kF32BlockM, kF32Threads>(attn_fwd_f32_kernel<128, false>, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, scale, stream);
  return causal ? launch<kF32BlockM, kF32Threads>(attn_fwd_f32_kernel<64, true>, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, scale, stream)
                : launch<kF32BlockM, kF32Threads>(attn_fwd_f32_kernel<64, false>, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, scale, stream);
}

extern "C" const char* tileattn_strerror(int status) {
  switch (status) {
    case TILEATTN_OK: return "ok";
    case TILEATTN_ERR_NULL_POINTER: return "a tensor pointer is NULL";
    case TILEATTN_ERR_BAD_SHAPE: return "bad shape: sizes must be >= 0 (attention: Hkv, Sk >= 1; matmul: N, K multiples of 8)";
    case TILEATTN_ERR_GQA_RATIO: return "Hq must be a multiple of Hkv";
    case TILEATTN_ERR_HEAD_DIM: return "head dimension D must be 64 or 128";
    case TILEATTN_ERR_SCALE: return "scale must be finite and >= 0";
    case TILEATTN_ERR_ALIGNMENT: return "tensor pointers must be 16-byte aligned";
    case TILEATTN_ERR_TOO_LARGE: return "problem exceeds the index range";
    case TILEATTN_ERR_LAUNCH: return "kernel launch failed (is a gfx950 device current?)";
    case TILEATTN_ERR_DTYPE: return "unknown dtype code";
    case TILEATTN_ERR_WORKSPACE: return "workspace is NULL or smaller than tileattn_fwd_workspace_size";
    case TILEATTN_ERR_SCRATCH: return "problem needs more than the 64 MiB static workspace of tileattn_fwd_noalloc";
    default: return "unknown tileattn status";
  }
}

extern "C" int tileattn_launch_shape(int dtype_bytes, int B, int Hq, int Hkv, int Sq, int Sk,
                                     int D, int causal, int* block_m, int* block_n,
                                     long long* workgroups) {
  (void)causal;
  if (dtype_bytes != 2 && dtype_bytes != 4) return TILEATTN_ERR_BAD_SHAPE;
  bool empty;
  // Shape checks only: pass dummy aligned non-null pointers.
  static const float dummy[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  const int st = validate(dummy, dummy, dummy, dummy, dummy, B, Hq, Hkv, Sq, Sk, D, 1.0f, &empty);
  if (st != TILEATTN_OK) return st;
  // 16-bit: the plain entry points' choice, rows = query heads x positions
  // (head packing) per workgroup.
  const bool split = dtype_bytes == 2 && use_split(B, Hq, Hkv, Sq, false);
  const int bm = dtype_bytes == 2 ? (split ? Bf16Tile<128, true>::kBlockM : Bf16Tile<128>::kBlockM) : kF32BlockM;
  const int ps = dtype_bytes == 2 ? pack_shift_for(Hq / Hkv, split ? 4 : 8, false) : 0;
  if (block_m) *block_m = bm;
  // 16-bit: 64-key tiles.
  if (block_n) *block_n = dtype_bytes == 2 ? kBlockN : kBlockNF32;
  if (workgroups) *workgroups = empty ? 0 : grid_workgroups(B, Hq, Sq, bm, ps);
  return TILEATTN_OK;
}
