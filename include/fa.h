/*
 * fa.h -- C ABI of the exact tiled attention forward pass for AMD Instinct
 * MI355X (gfx950).
 *
 * What is computed.  For every batch b and head h, with Q, K, V in R^{N x d}:
 *     S = scale * Q K^T,  S_ij = -inf for j > i when causal,
 *     O = softmax_rows(S) V,   LSE_i = ln sum_j exp(S_ij)   (natural log).
 * The result is the one standard attention gives (FlashAttention-2 wiki page,
 * introduction and section "Leistung und Effizienz": identical results, exact
 * and deterministic); it is obtained without ever materialising S, by an
 * outer loop over blocks of queries and an inner loop over tiles of keys and
 * values that are staged in on-chip memory (same page, section "Hintergrund",
 * and page "FlashAttention-Skalierung, Multi-GPU-Training und
 * Gewichtsquantisierung", section 1), with the online softmax whose
 * normalisation is applied once, after the last key tile (same section; wiki
 * page, section "Technische Architektur", item 1).  The causal mask aligns
 * queries and keys (query i sees keys 0..i); LSE is the logsumexp of the
 * scaled, masked scores of each query row.
 *
 * Conventions shared by every entry point.
 *  - Pointers named as tensors are DEVICE pointers owned by the caller; the
 *    library never allocates, frees or keeps them.
 *  - Tensors are contiguous and row-major: Q, K, V, O are [B, H, N, d];
 *    LSE is float32 [B, H, N].
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it and return; they never synchronise.
 *  - Arguments are validated before anything is enqueued; on any non-zero
 *    status nothing was launched and no output was written.
 *  - B, H or N equal to 0 is an empty problem: FA_OK, nothing is launched and
 *    the tensor pointers are not inspected.
 *  - Input values are not inspected; non-finite inputs propagate.
 *  - Results are bitwise repeatable for the same inputs, shape and device
 *    (no atomics, fixed reduction order).
 *  - Calls are reentrant; the library holds no mutable state (except
 *    fa_bwd_noalloc's static scratch, described there).
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 4

/* Row length (keys) of transposed V codes: N rounded up to a multiple of 64. */
#define FA_FP8_VT_COLS(N) ((((N) + 63) / 64) * 64)

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  FA_ERR_SHAPE = 2,       /* a negative size, an element count beyond int64,  */
                          /* N * d * 4 beyond INT32_MAX (per-head size), or    */
                          /* B * H * ceil(N / 16) beyond 2^23 (one launch)     */
  FA_ERR_UNSUPPORTED = 3, /* head dim, dtype, flag or layout not provided      */
  FA_ERR_SCALE = 4,       /* scale is NaN or infinite                          */
  FA_ERR_ALIAS = 5,       /* an output overlaps an input                       */
  FA_ERR_HIP = 6,         /* the HIP runtime rejected a launch                 */
  FA_ERR_SCRATCH = 7      /* the problem needs more than the library's static  */
                          /* scratch (fa_bwd_noalloc: B * H * N rows)          */
};

/* Rows (B * H * N) that fa_bwd_noalloc's static scratch holds: 16 MiB of fp32. */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 22)

enum fa_dtype { FA_F32 = 0, FA_BF16 = 1 };

/* Version of this interface (FA_ABI_VERSION).  The pages define no interface;
 * the version lets a caller check the layout of the calls below. */
int fa_abi_version(void);

/* Static, human-readable name of a status code ("unknown status" otherwise);
 * the codes are the validation results listed with each call below. */
const char* fa_status_string(int status);

/*
 * fa_fwd -- attention forward in fp32 or bf16: the exact, IO-aware tiled
 * forward pass of page "FlashAttention-Skalierung, Multi-GPU-Training und
 * Gewichtsquantisierung", section 1, FlashAttention-2 items (the online
 * softmax with its rescaling moved to the end of the inner loop; the outer
 * loop over query blocks and the inner loop over K/V tiles, with the work of
 * one head spread over the sequence), also the FlashAttention-2 wiki page,
 * section "Technische Architektur und Funktionsprinzipien", items 1 and 2;
 * it returns O and the row logsumexp.
 *   q, k, v : [B, H, N, d] of `dtype` (FA_F32: float32, FA_BF16: bfloat16).
 *   o       : [B, H, N, d] of `dtype`, fully overwritten.
 *   lse     : float32 [B, H, N], fully overwritten.
 *   d       : 64 or 128.  N: any value >= 1 (no tile-size restriction).
 *   causal  : 0 or 1.  scale: any finite value (0 gives uniform weights).
 * Arithmetic: products and sums in fp32 (bf16 inputs multiply on bf16 MFMA
 * with fp32 accumulation; the probabilities feeding the second product are
 * rounded to bf16); O is rounded to `dtype` once, at the end.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (d, dtype, causal),
 * FA_ERR_SCALE, FA_ERR_ALIAS (o or lse overlapping q, k or v, or each other),
 * FA_ERR_HIP.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
           int dtype, void* stream);

/*
 * fa_quant_rotate_fp8 -- the FP8 pre-pass: block quantisation of one tensor,
 * after an optional random orthogonal rotation (page "FlashAttention-
 * Skalierung, Multi-GPU-Training und Gewichtsquantisierung", section 1, the
 * FlashAttention-3 FP8 item: per-tile scales, and Q and K multiplied by random
 * orthogonal matrices to spread outliers before quantisation).
 *   x       : bfloat16 [B, H, N, d].
 *   signs   : int8 [d] of +1/-1 (device), or NULL for no rotation (use NULL
 *             for V).  With signs, each row x is replaced by x R with
 *             R = diag(signs) H_d / sqrt(d), H_d the Sylvester-ordered
 *             Hadamard matrix; Q and K must use the same signs.
 *   x8      : OCP e4m3 codes (uint8).  transpose_out = 0: [B, H, N, d];
 *             transpose_out = 1: [B, H, d, FA_FP8_VT_COLS(N)], columns N and
 *             beyond holding code 0 (the layout fa_fwd_fp8 wants for V).
 *   x_scale : float32 [B, H, ceil(N/128)]: one scale per tile of 128 rows
 *             (the last tile may be partial) = max |value| over the tile / 448,
 *             or 1 for an all-zero tile -- a tile whose largest magnitude is
 *             below 2^-96 (of the rotated values times sqrt(d) with signs)
 *             counts as all-zero.  code = e4m3(value / scale), rounded to
 *             nearest even and saturated at +-448.
 *   d       : 64 or 128.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (d, transpose_out),
 * FA_ERR_ALIAS, FA_ERR_HIP.
 */
int fa_quant_rotate_fp8(const void* x, uint8_t* x8, float* x_scale, const int8_t* signs,
                        int64_t B, int64_t H, int64_t N, int64_t d, int transpose_out,
                        void* stream);

/*
 * fa_quant_rotate_fp8_tensor -- fa_quant_rotate_fp8 with ONE scale for the whole
 * tensor instead of one per 128-row tile: the baseline against which the
 * pages' block quantisation (independent scales of small tiles; page
 * "FlashAttention-Skalierung, Multi-GPU-Training und Gewichtsquantisierung",
 * section 1, FlashAttention-3 FP8 item) is measured.  The scale is the largest
 * magnitude over all B, H, N, d (after the rotation) / 448 -- 1 if that is
 * below 2^-96 as above -- and is written into every entry of x_scale, so the
 * output goes to fa_fwd_fp8 unchanged.  Three launches (tile maxima, their
 * maximum, the quantisation).
 *   Arguments, layouts and errors: as fa_quant_rotate_fp8.
 */
int fa_quant_rotate_fp8_tensor(const void* x, uint8_t* x8, float* x_scale, const int8_t* signs,
                               int64_t B, int64_t H, int64_t N, int64_t d, int transpose_out,
                               void* stream);

/*
 * fa_quant_rotate_fp8_qkv -- the whole FP8 pre-pass in one launch: the three
 * fa_quant_rotate_fp8 calls the FP8 path makes (same page and item as above),
 * with identical results -- Q and K with `signs` (rotated; NULL: not rotated)
 * into row-major codes, V without rotation into transposed codes.
 *   q, k, v : bfloat16 [B, H, N, d].
 *   q8, k8  : e4m3 codes [B, H, N, d];  v8t: e4m3 codes [B, H, d, FA_FP8_VT_COLS(N)].
 *   q_scale, k_scale, v_scale : float32 [B, H, ceil(N/128)].
 *   signs   : int8 [d] of +1/-1 (device) or NULL.   d: 64 or 128.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (d, alignment),
 * FA_ERR_ALIAS (an output overlapping an input, the signs or another output),
 * FA_ERR_HIP.
 */
int fa_quant_rotate_fp8_qkv(const void* q, const void* k, const void* v, uint8_t* q8, uint8_t* k8,
                            uint8_t* v8t, float* q_scale, float* k_scale, float* v_scale,
                            const int8_t* signs, int64_t B, int64_t H, int64_t N, int64_t d,
                            void* stream);

/*
 * fa_fwd_fp8 -- attention forward on e4m3 operands with per-tile scales: the
 * FP8 variant of the pages (page "FlashAttention-Skalierung, Multi-GPU-
 * Training und Gewichtsquantisierung", section 1, FlashAttention-3 FP8 item:
 * FP8 matrix products at twice the raw rate of 16-bit ones, kept accurate by
 * block quantisation with one scale per small tile and by the random
 * orthogonal rotation of Q and K that fa_quant_rotate_fp8 applies; the news
 * article on FlashAttention-3, section "Innovationen von FlashAttention-3",
 * third item), computed with the same tiled online softmax as fa_fwd.
 *   q8, k8  : e4m3 codes [B, H, N, d] from fa_quant_rotate_fp8 with the same signs.
 *   v8      : e4m3 codes of V (not rotated); v_transposed must be 1 and v8
 *             laid out [B, H, d, FA_FP8_VT_COLS(N)] with zero codes in the
 *             padding columns, as fa_quant_rotate_fp8 writes it.
 *   q_scale, k_scale, v_scale : float32 [B, H, ceil(N/128)] tile scales.
 *   o       : bfloat16 [B, H, N, d];  lse: float32 [B, H, N].
 *   d       : 128.  causal: 0 or 1.  scale: finite.
 * Arithmetic: Q K^T and P V on fp8 MFMA with fp32 accumulation; the score of
 * a (query tile, key tile) pair is multiplied by scale * q_scale * k_scale;
 * the probabilities of a key tile are multiplied by 2^6 * v_scale / (largest
 * v_scale of the head) and rounded to e4m3 for the P V product (the factors
 * are divided out at the end); O is normalised by the sum of those rounded
 * probabilities (the weights the P V product used), LSE by the sum of the
 * unrounded fp32 ones.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (d, v_transposed,
 * causal), FA_ERR_SCALE, FA_ERR_ALIAS, FA_ERR_HIP.
 */
int fa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
               const float* q_scale, const float* k_scale, const float* v_scale,
               int v_transposed, void* o, float* lse, int64_t B, int64_t H, int64_t N,
               int64_t d, int causal, float scale, void* stream);

/*
 * fa_fwd_fp8_pbf16 -- fa_fwd_fp8 with the probabilities kept in bf16: the same
 * fp8 operands, scales and Q K^T product, but P is rounded to bf16 (not e4m3)
 * and P V runs on the bf16 matrix core with V's codes widened exactly to
 * bf16.  It isolates the effect of rounding P to FP8 for the accuracy study of
 * the pages' FP8 item (page "FlashAttention-Skalierung, Multi-GPU-Training und
 * Gewichtsquantisierung", section 1, FlashAttention-3 FP8 item: FP8 precision
 * losses and the measures against them); it is not tuned for speed.
 *   Arguments, layouts and errors: as fa_fwd_fp8.
 */
int fa_fwd_fp8_pbf16(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                     const float* q_scale, const float* k_scale, const float* v_scale,
                     int v_transposed, void* o, float* lse, int64_t B, int64_t H, int64_t N,
                     int64_t d, int causal, float scale, void* stream);

/*
 * fa_fwd_partial -- attention of queries against one range of keys: the
 * building block of a split-KV forward and of merging results computed apart
 * (on other streams or devices).  The softmax of a row over a union of key
 * ranges follows exactly from the ranges' own outputs and logsumexps
 * (fa_merge), by the same rescaling that the online softmax applies tile by
 * tile (page "FlashAttention-Skalierung, Multi-GPU-Training und
 * Gewichtsquantisierung", section 1; FlashAttention-2 wiki page,
 * "Technische Architektur", item 1).
 *   q        : bfloat16 [B, H, Nq, d]; query i sits at key position q_pos0 + i.
 *   k, v     : bfloat16 [B, H, Nk, d]; keys k_begin <= j < k_end are used
 *              (and, when causal, only j <= q_pos0 + i).
 *   o_part   : float32 [B, H, Nq, d]: O normalised over the visible keys of the
 *              range; 0 for a row that sees none of them.
 *   lse_part : float32 [B, H, Nq]: natural logsumexp of the scaled visible
 *              scores; -inf for a row that sees none of them.
 *   d        : 64 or 128.  dtype: FA_BF16.  causal: 0 or 1.  scale: finite.
 *   0 <= k_begin <= k_end <= Nk;  0 <= q_pos0 <= INT32_MAX / 2 - Nq.
 * fa_fwd(q, k, v) with Nq = Nk = N equals this call with q_pos0 = 0 and the
 * range [0, N), up to the precision of O (fp32 here, bf16 there).
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (d, dtype, causal),
 * FA_ERR_SCALE, FA_ERR_ALIAS, FA_ERR_HIP.
 */
int fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t q_pos0,
                   int64_t k_begin, int64_t k_end, int causal, float scale, int dtype, void* stream);

/*
 * fa_fwd_split -- fa_fwd_partial over n_splits consecutive key ranges in one
 * launch, so that short query blocks (decode) still fill the device: range s
 * (0 <= s < n_splits) is [k_begin + floor((k_end - k_begin) * s / n_splits),
 * k_begin + floor((k_end - k_begin) * (s + 1) / n_splits)).
 *   o_parts   : float32 [n_splits, B, H, Nq, d];  lse_parts: float32 [n_splits, B, H, Nq]:
 *               slice s as fa_fwd_partial writes it for range s (ready for fa_merge).
 *   1 <= n_splits <= 65535; all other arguments as for fa_fwd_partial.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (d, dtype, causal),
 * FA_ERR_SCALE, FA_ERR_ALIAS, FA_ERR_HIP.
 */
int fa_fwd_split(const void* q, const void* k, const void* v, float* o_parts, float* lse_parts,
                 int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t q_pos0,
                 int64_t k_begin, int64_t k_end, int64_t n_splits, int causal, float scale, int dtype,
                 void* stream);

/*
 * fa_merge -- O and LSE over the union of n_parts disjoint key ranges from
 * their partial results: LSE = log(sum_s exp(LSE_s)), O = sum_s exp(LSE_s - LSE) O_s.
 *   o_parts   : float32 [n_parts, B, H, N, d];  lse_parts: float32 [n_parts, B, H, N]
 *               (as written by fa_fwd_partial; -inf marks a range a row does not see).
 *   o         : [B, H, N, d] of dtype (FA_F32 or FA_BF16);  lse: float32 [B, H, N].
 *   A row that sees no key in any range gets O = 0 and LSE = -inf.
 *   d         : 64 or 128.  n_parts >= 1.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (d, dtype),
 * FA_ERR_ALIAS, FA_ERR_HIP.
 */
int fa_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, void* o, float* lse,
             int64_t B, int64_t H, int64_t N, int64_t d, int dtype, void* stream);

/*
 * fa_bwd -- attention backward: the gradients dQ, dK, dV of the forward
 * output for an output gradient dO, recomputing the probabilities tile by
 * tile from the LSE the forward saved (training is the pages' motivating use:
 * FlashAttention-2 wiki page, "Leistung und Effizienz").  With S = scale Q K^T
 * (masked), P = softmax(S):  dV = P^T dO;  D = rowsum(dO * O);
 * dS = P * (dO V^T - D);  dQ = scale dS K;  dK = scale dS^T Q.
 *   q, k, v, o, dout : bfloat16 [B, H, N, d] (o: the forward's output).
 *   lse              : float32 [B, H, N], the forward's logsumexp.
 *   dq, dk, dv       : bfloat16 [B, H, N, d], fully overwritten.
 *   delta            : float32 [B, H, N] workspace (caller-owned), overwritten
 *                      with D.
 *   d: 64 or 128.  dtype: FA_BF16.  causal: 0 or 1.  scale: finite, the one
 *   the forward used.
 * Arithmetic: products on bf16 MFMA with fp32 accumulation; P and dS are
 * rounded to bf16 for the products that use them; no atomics (bitwise
 * reproducible).
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (d, dtype, causal,
 * alignment), FA_ERR_SCALE, FA_ERR_ALIAS (any output or the workspace
 * overlapping an input or each other), FA_ERR_HIP.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H,
           int64_t N, int64_t d, int causal, float scale, int dtype, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving or training loops, harnesses that
 * forbid hipMalloc): the same kernels and results, with the row-sum workspace
 * `delta` taken from a static device array of FA_BWD_NOALLOC_MAX_ROWS floats
 * (16 MiB per GPU, held until the process ends) instead of an argument.
 *   Arguments: as fa_bwd, without delta.
 *   The call allocates nothing (no hipMalloc, hipFree or allocating library
 *   routine).  Its first call on a device looks up that device's copy of the
 *   array (hipGetSymbolAddress, with the device current).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (on different streams, or from several threads) race and give wrong
 *   gradients; calls one after another on a stream are safe.  The array needs
 *   no clearing: each call overwrites the rows it reads.
 * Errors: those of fa_bwd, and FA_ERR_SCRATCH when B * H * N exceeds
 * FA_BWD_NOALLOC_MAX_ROWS (checked before any pointer or device access).
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                   int64_t N, int64_t d, int causal, float scale, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
