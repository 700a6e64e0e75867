/*
 * tileattn — exact attention forward for AMD Instinct MI355X (gfx950), C ABI.
 *
 * Computes, for every batch b, query head h and query row i,
 *
 *     s_ij   = scale * <q[b,h,i,:], k[b,hk,j,:]>          for visible keys j
 *     o[b,h,i,:] = sum_j softmax_j(s_i) * v[b,hk,j,:]
 *     lse[b,h,i] = ln( sum_j exp(s_ij) )                  (natural log)
 *
 * tile by tile with an online (running max / running sum) softmax, so the
 * Sq x Sk score matrix never exists in memory.  That method is the flash
 * attention kernel of "Guia Prático de Programação de GPU com Tiles: de
 * Kernels cuTile e Triton ao Flash Attention" (Passo a Passo, step 6
 * "Flash Attention — Softmax Online"): a query tile stays resident while key
 * and value tiles stream past it; per tile the scores are formed, the running
 * row maximum is raised, the running sum and the accumulator are rescaled by
 * exp(old max - new max), and probabilities (cast to the value dtype) are
 * multiplied into the accumulator, which is divided by the running sum at the
 * end.  Products accumulate in fp32 (step 5 "Multiplicação de Matrizes Tiled"
 * and its Troubleshooting note on fp16 accumulators).
 *
 * Readings of what the pages leave open:
 *   - GQA (named for the final kernel of "Como Domar o Blackwell Sem
 *     Enlouquecer com CUDA", section "O Que Tem Dentro Deste Tutorial"):
 *     query head h reads key/value head hk = h / (Hq / Hkv).
 *   - causal (named in the FAQ of the first page as a production feature):
 *     key j is visible to query i iff j <= i, top-left aligned for any Sq, Sk.
 *   - lse is not on the pages: natural log of the softmax denominator of the
 *     scaled scores, stored as fp32.
 *
 * Layout: every tensor is dense row-major with the head dimension innermost:
 *     q   [B, Hq,  Sq, D]      k, v [B, Hkv, Sk, D]
 *     o   [B, Hq,  Sq, D]      lse  [B, Hq,  Sq]      (fp32)
 * All pointers are device pointers on the current HIP device, 16-byte
 * aligned.  The caller owns every buffer, and no call allocates memory.
 * Between calls the library keeps only per-device constants (the compute
 * unit count; for tileattn_fwd_noalloc, the address of its static device
 * workspace), and it is safe to call from several host threads (calls that
 * share a workspace must still be ordered).  o and lse must not overlap q,
 * k or v.
 *
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 * stream).  Argument errors are reported before anything is launched; a
 * launch failure is reported as TILEATTN_ERR_LAUNCH; faults inside the kernel
 * surface at the caller's next synchronisation with the stream.
 */
#ifndef TILEATTN_H
#define TILEATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TILEATTN_OK = 0,
  TILEATTN_ERR_NULL_POINTER = -1, /* q, k, v, o or lse is NULL (non-empty problem)   */
  TILEATTN_ERR_BAD_SHAPE = -2,    /* a size < 0; attention: Hkv < 1 or Sk < 1;         */
                                  /* matmul: N or K not a multiple of 8               */
  TILEATTN_ERR_GQA_RATIO = -3,    /* Hq is not a multiple of Hkv                      */
  TILEATTN_ERR_HEAD_DIM = -4,     /* D is not 64 or 128                               */
  TILEATTN_ERR_SCALE = -5,        /* scale is negative, NaN or infinite               */
  TILEATTN_ERR_ALIGNMENT = -6,    /* a pointer is not 16-byte aligned                 */
  TILEATTN_ERR_TOO_LARGE = -7,    /* a size product exceeds the 64-bit index range,   */
                                  /* or Sk*D*4 > 2^31-1 (one head's K or V is read    */
                                  /* with 32-bit buffer offsets)                      */
  TILEATTN_ERR_LAUNCH = -8,       /* the HIP launch failed (e.g. no gfx950 device)    */
  TILEATTN_ERR_DTYPE = -9,        /* unknown tileattn_dtype code                      */
  TILEATTN_ERR_WORKSPACE = -10,   /* workspace NULL or below the size it needs        */
  TILEATTN_ERR_SCRATCH = -11      /* tileattn_fwd_noalloc: over its static workspace  */
} tileattn_status;

/* Storage type codes of tileattn_softmax and tileattn_gelu. */
typedef enum {
  TILEATTN_DTYPE_F32 = 0,         /* IEEE binary32                                    */
  TILEATTN_DTYPE_BF16 = 1         /* bfloat16; results rounded to nearest even        */
} tileattn_dtype;

/*
 * bfloat16 attention forward (the hot path).
 *   q, k, v : bf16 inputs, layouts above.
 *   o       : bf16 output [B, Hq, Sq, D], rounded to nearest even from fp32.
 *   lse     : fp32 output [B, Hq, Sq].
 *   B, Hq, Sq may be 0 (nothing is launched, TILEATTN_OK).  Hkv >= 1, Sk >= 1.
 *   D in {64, 128}.  scale >= 0 and finite (usually 1/sqrt(D)).
 *   causal != 0 applies the top-left causal mask (key j visible iff j <= i).
 *   stream  : hipStream_t to launch on, NULL for the default stream.
 * Returns TILEATTN_OK or a tileattn_status error code.
 */
int tileattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int D,
                 float scale, int causal, void* stream);

/*
 * float16 attention forward: the same contract as tileattn_fwd with fp16
 * (IEEE binary16) q, k, v and o.  The first page's own kernel is written for
 * fp16 inputs with fp32 accumulation, casting the probabilities to the value
 * dtype before the second product (Passo a Passo, step 6, and its
 * Troubleshooting note on fp16 accumulators); this entry point runs that
 * dtype on the same kernel with fp16 matrix-core instructions.  The
 * probabilities are rounded to fp16 (nearest even); they never exceed 2^8,
 * far inside fp16 range, and o stays within the range of v.
 */
int tileattn_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D,
                     float scale, int causal, void* stream);

/*
 * 16-bit attention forward with an ALiBi bias and/or a block-sparse mask.
 * The first page's FAQ names both (with causal masking) as what the official
 * flash-attention library adds over its tutorial kernel; it does not define
 * them, so this entry point takes the plainest readings:
 *   - ALiBi ("Train Short, Test Long: Attention with Linear Biases"): a slope
 *     m_h per query head adds a bias linear in the query-key distance to the
 *     scaled score:  s_ij = scale * <q_i, k_j> + b_ij  with
 *     b_ij = -m_h * (i - j) when causal, -m_h * |i - j| otherwise.
 *   - block mask: uint8 map [mask_heads, ceil(Sq/64), ceil(Sk/64)]; block
 *     (qb, kb) is visible iff its byte is nonzero (query rows 64*qb..64*qb+63,
 *     keys 64*kb..64*kb+63).  mask_heads is 1 (one map for every head and
 *     batch) or Hq (query head h uses plane h).  It combines with causal (a
 *     key must pass both).  Tiles no query block of a workgroup can see are
 *     neither loaded nor computed.
 *   - a row with no visible key gets o = 0 and lse = -inf.
 *   q, k, v, o as for tileattn_fwd (is_f16 = 0: bf16, else fp16); lse is the
 *   natural log of the softmax denominator of the biased scaled scores.
 *   alibi_slopes : NULL (no bias) or device pointer to Hq fp32 slopes
 *                  (4-byte aligned), |m_h| <= 1e6 (the kernel carries the
 *                  bias divided by scale).  With slopes, a scale below 2^-64
 *                  (zero included) is taken as 0: the scores are the bias
 *                  alone.
 *   block_mask   : NULL (no mask) or device pointer to the uint8 map above.
 * Extra errors: TILEATTN_ERR_BAD_SHAPE if block_mask is given and mask_heads
 * is not 1 or Hq; TILEATTN_ERR_TOO_LARGE if block_mask is given and
 * Sk > 131072 (the per-workgroup tile list holds 2048 tiles);
 * TILEATTN_ERR_ALIGNMENT for a misaligned alibi_slopes.
 */
int tileattn_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D,
                     float scale, int causal, const float* alibi_slopes,
                     const unsigned char* block_mask, int mask_heads, int is_f16,
                     void* stream);

/*
 * 16-bit attention forward with the key range of a query tile optionally
 * split over several workgroups.  The online softmax of the page's step 6
 * ("Flash Attention — Softmax Online") folds the tiles of a row one after
 * another into (running max, running sum, accumulator); two such states over
 * disjoint key ranges fold together by the same rescale-and-add, so a query
 * tile's keys can be cut into chunks that run in parallel and are merged at
 * the end.  The result is the attention of tileattn_fwd (bf16, is_f16 = 0)
 * or tileattn_fwd_f16 (is_f16 != 0), up to the rounding order of that fold.
 * It pays where few query tiles cover long key ranges (a small batch of
 * heads, causal heads whose diagonal query tiles dominate, short queries
 * against a long context): there the plain grid leaves most compute units
 * idle while its heaviest query tiles run.
 *   alibi_slopes    : NULL, or the linear bias of tileattn_fwd_ext (Hq fp32
 *                     slopes on the device, 4-byte aligned; same reading
 *                     and limits): the call is then tileattn_fwd_ext
 *                     without a block mask, up to the rounding order of the
 *                     fold.
 *   workspace       : device memory, 16-byte aligned, of at least
 *                     tileattn_fwd_workspace_size(...) bytes for the same
 *                     problem on the same device; owned by the caller, its
 *                     contents on entry do not matter and on return are
 *                     undefined.  Calls that share a workspace must be
 *                     ordered (one stream, or synchronised).
 *   workspace_bytes : its size in bytes.
 * Where tileattn_fwd_workspace_size is 0 the call is tileattn_fwd /
 * tileattn_fwd_f16 (with slopes: tileattn_fwd_ext) and workspace may be
 * NULL.  Otherwise it launches two kernels on `stream`.  Extra errors:
 * TILEATTN_ERR_WORKSPACE (workspace NULL or workspace_bytes too small),
 * TILEATTN_ERR_ALIGNMENT for a misaligned workspace or alibi_slopes.
 */
int tileattn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int Sq, int Sk, int D,
                    float scale, int causal, const float* alibi_slopes, int is_f16,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes tileattn_fwd_ws needs for this problem on the current
 * device (0: it needs none), or a negative tileattn_status for a bad shape.
 * The split depends on the device's compute unit count.
 */
long long tileattn_fwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal);

/*
 * tileattn_fwd_ws without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: the workspace is
 * a static 64 MiB device array of the library, one per device, loaded with
 * the library's code and held until the process ends; the first call on a
 * device looks up its address (hipGetSymbolAddress) with that device
 * current.  Same arguments, results and errors as tileattn_fwd_ws (bitwise
 * the same results), plus TILEATTN_ERR_SCRATCH for a problem whose
 * tileattn_fwd_workspace_size exceeds 64 MiB (none does on a 256-CU device:
 * the largest split needs about 51 MB at D = 128); TILEATTN_ERR_LAUNCH if
 * the address lookup fails.  Every call on a device shares its array and
 * nothing in it needs clearing between calls (each call writes every part
 * it reads), so calls that overlap on one device (different streams or
 * host threads without ordering) race and must be serialised by the caller.
 */
int tileattn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Sq, int Sk, int D,
                         float scale, int causal, const float* alibi_slopes, int is_f16,
                         void* stream);

/*
 * float32 attention forward: the same contract as tileattn_fwd with fp32
 * q, k, v and o.  Both products use fp32 matrix-core instructions and the
 * probabilities stay fp32 (there is no narrower value dtype to cast them to).
 */
int tileattn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D,
                     float scale, int causal, void* stream);

/*
 * Tiled matrix product C = A * B with bf16 inputs and an fp32 accumulator:
 * the first page's step 5 (Passo a Passo, "Multiplicacao de Matrizes
 * Tiled"): per output tile, an fp32 accumulator adds the products of A and B
 * blocks over the K loop; its Troubleshooting section explains why the
 * accumulator must be fp32 even for 16-bit inputs.
 *   a : bf16 [M, K] row-major, device pointer, 16-byte aligned.
 *   b : bf16 [K, N] row-major, device pointer, 16-byte aligned.
 *   c : [M, N] row-major output, fp32 (out_bf16 = 0: the accumulator as it
 *       is) or bf16 (out_bf16 != 0: rounded to nearest even), 16-byte aligned.
 *   M >= 0; N and K >= 0 and multiples of 8.  M or N = 0 launches nothing;
 *   K = 0 writes zeros (a and b are not read and may be NULL).  The caller owns every buffer; nothing is allocated.
 *   stream : hipStream_t to launch on, NULL for the default stream.
 * Errors: TILEATTN_ERR_BAD_SHAPE (negative size, N or K not a multiple of 8),
 * TILEATTN_ERR_NULL_POINTER, TILEATTN_ERR_ALIGNMENT, TILEATTN_ERR_TOO_LARGE
 * (512*K or 128*N bytes above 2^31-1: 32-bit offsets within one tile),
 * TILEATTN_ERR_LAUNCH.
 */
int tileattn_matmul(const void* a, const void* b, void* c, int M, int N, int K, int out_bf16,
                    void* stream);

/*
 * Row softmax: the first page's step 4 (Passo a Passo, "Softmax por Linha"):
 * per row, subtract the row maximum, exponentiate, divide by the sum of the
 * exponentials (the max subtraction keeps the largest term at 1).
 *   out[r, c] = exp(x[r, c] - max_c' x[r, c']) / sum_c'' exp(x[r, c''] - max)
 * for r < n_rows, c < n_cols; element (r, c) of x and out is at r*stride + c.
 *   x, out : device pointers, 16-byte aligned, dtype (tileattn_dtype) storage;
 *            out may be x (in place).  Arithmetic is fp32.
 *   n_rows >= 0 (0: nothing is launched), 1 <= n_cols <= stride, stride a
 *   multiple of 16 bytes.  A row whose entries are all -inf gives NaN, as
 *   the definition does (-inf - -inf).
 * Errors: TILEATTN_ERR_DTYPE, TILEATTN_ERR_BAD_SHAPE, TILEATTN_ERR_ALIGNMENT
 * (pointer or stride), TILEATTN_ERR_NULL_POINTER, TILEATTN_ERR_TOO_LARGE,
 * TILEATTN_ERR_LAUNCH.
 */
int tileattn_softmax(const void* x, void* out, int n_rows, int n_cols, long long stride, int dtype,
                     void* stream);

/*
 * Fused GELU: the first page's step 3 (Passo a Passo, "GELU Fundido"): one
 * pass computes h = x*w + b elementwise and the tanh approximation of GELU,
 *   out[i] = 0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3))),  h = x[i]*w[i] + b[i],
 * for i < n (x, w, b, out all of n elements).  Arithmetic is fp32.
 *   x, w, b, out : device pointers, 16-byte aligned, dtype storage; out may be
 *                  one of the inputs.  n >= 0 (0: nothing is launched).
 * Errors: TILEATTN_ERR_DTYPE, TILEATTN_ERR_BAD_SHAPE (n < 0),
 * TILEATTN_ERR_NULL_POINTER, TILEATTN_ERR_ALIGNMENT, TILEATTN_ERR_TOO_LARGE,
 * TILEATTN_ERR_LAUNCH.
 */
int tileattn_gelu(const void* x, const void* w, const void* b, void* out, long long n, int dtype,
                  void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* tileattn_strerror(int status);

/*
 * Launch geometry the library uses for a problem: query rows per workgroup
 * (block_m), keys per tile (block_n) and the number of workgroups.  For
 * reporting and tests; host arithmetic plus, for 16-bit inputs, the current
 * device's compute-unit count (queried once per device; 256 when no device
 * answers).  dtype_bytes is 2 (bf16 or fp16: the plain entry points, which
 * use 256-row workgroups, or the key split's 128-row ones when the 256-row
 * grid would fill at most half of the compute units) or 4 (fp32).  A 16-bit
 * workgroup's rows are P query heads that share a KV head times
 * block_m / P consecutive positions, P the largest power of two dividing
 * Hq / Hkv and at most block_m / 32; the workgroup count is
 * B * (Hq / P) * ceil(Sq / (block_m / P)).  (tileattn_fwd_ext with a block
 * mask takes P at most block_m / 64.)  Returns TILEATTN_OK or the error
 * tileattn_fwd would.
 */
int tileattn_launch_shape(int dtype_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                          int causal, int* block_m, int* block_n, long long* workgroups);

#ifdef __cplusplus
}
#endif

#endif /* TILEATTN_H */
