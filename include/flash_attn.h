/*
 * flash_attn.h - C ABI of the MI355X (gfx950) exact-attention library.
 *
 * The library computes exact scaled-dot-product attention the IO-aware way:
 * one fused forward kernel streams K/V tiles past a resident Q tile, keeps the
 * softmax statistics online, and writes back only O and the per-row
 * log-sum-exp; the backward recomputes the probabilities from those saved
 * statistics instead of reading an N x N matrix.
 *
 * Passages defining the operations (page title, section):
 *   - codechina.net CUDA/FlashAttention article, section 3: Q, K, V are N x d,
 *     S = Q K^T, P = softmax(S), O = P V.
 *   - 52jiny.com FlashAttention explainer, "why standard attention is
 *     IO-bound": scaling and a mask sit between Q K^T and the softmax.
 *   - 52jiny.com, "key ideas" parts 1-3: tile Q, K, V into on-chip memory,
 *     online softmax (running max and sum, rescale on update), fused kernel
 *     that writes back only the output and a few normalisation statistics.
 *   - 52jiny.com, "key ideas" part 4: the backward saves the output and the
 *     softmax statistics and recomputes intermediates block by block.
 *
 * Conventions shared by every entry point
 *   Layout     Q, K, V, O, dO, dQ, dK, dV: contiguous row-major [B, H, N, d],
 *              d fastest. LSE: contiguous [B, H, N] float32. Q, K and V share
 *              one N (square self-attention).
 *   Pointers   DEVICE pointers on the current HIP device, 16-byte aligned.
 *              The caller owns all memory; the library allocates and frees
 *              nothing and keeps no state between calls.
 *   Scale      Multiplies Q K^T in float32 before the mask and softmax; must be
 *              finite (any sign).
 *   Causal     causal != 0 masks key j for query i when j > i.
 *   LSE        Natural-log log-sum-exp of row i of the scaled, masked scores:
 *              ln(sum_j exp(scale * q_i . k_j)).
 *   Streams    Every call is asynchronous on `stream` (a hipStream_t; NULL is
 *              the null stream) and never synchronises. All arguments are
 *              validated before anything is launched; a call that returns an
 *              error status has launched nothing and written nothing.
 *   Errors     The library never aborts and never prints. Launch failures are
 *              reported as FA_ERR_HIP.
 *   Support    (any call outside this matrix returns FA_ERR_UNSUPPORTED)
 *              bf16, fp16: d in {32, 64, 96, 128, 256}; every entry point (forward,
 *                          key-split, masked with optional dropout, backward and its
 *                          stages, masked backward). fp16 is IEEE binary16.
 *              fp32:       d in {64, 128}; flash_attn_fwd only (no masks, no backward).
 *              B, H, N >= 1, B*H*N*d < 2^31 elements per tensor and
 *              N*d < 2^29 (one head is addressed with 32-bit byte offsets).
 */
#ifndef FLASH_ATTN_H_
#define FLASH_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  FA_ERR_BAD_SHAPE = 2,    /* B, H, N or d < 1, a tensor exceeds 2^31 elements, N*d >= 2^29,
                              or (key-split forward) Nq > Nk or num_splits outside 0..64 */
  FA_ERR_UNSUPPORTED = 3,  /* (dtype, d, pass) outside the support matrix, or a block map with
                              more than FA_MAX_MASK_BLOCKS blocks per row */
  FA_ERR_BAD_SCALE = 4,    /* scale is NaN or infinite */
  FA_ERR_MISALIGNED = 5,   /* a pointer is not 16-byte aligned (lse, seqlens: 4-byte) */
  FA_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than flash_attn_bwd_workspace_size() */
  FA_ERR_HIP = 7,          /* the HIP runtime reported an error at launch */
  FA_ERR_BAD_DROPOUT = 8,  /* dropout_p is NaN, infinite, negative or above 511/512 */
  FA_ERR_SCRATCH_LIMIT = 9 /* (no-allocation entry point) the call needs more scratch than
                              FA_NOALLOC_SCRATCH_BYTES */
} fa_status_t;

typedef enum { FA_DTYPE_FP32 = 0, FA_DTYPE_BF16 = 1, FA_DTYPE_FP16 = 2 } fa_dtype_t;

/* Block-sparse maps: one byte per FA_MASK_BLOCK x FA_MASK_BLOCK block of scores, at most
 * FA_MAX_MASK_BLOCKS blocks per row (N <= 131072 with a map). */
#define FA_MASK_BLOCK 128
#define FA_MAX_MASK_BLOCKS 1024

/*
 * Forward: O = softmax(scale * Q K^T [+ causal mask]) V and LSE.
 * Defined by codechina.net CUDA/FlashAttention article, section 3 (S = Q K^T, P = softmax(S),
 * O = P V) and section 4.2 (per-block running maximum m and sum l merged across key blocks);
 * 52jiny.com FlashAttention explainer, "key ideas" parts 1-3 (tiles in on-chip memory, online
 * softmax, one fused kernel that writes back only O and the row statistics, here LSE = m + ln l).
 *   q, k, v  [B,H,N,d] of `dtype`, read only.
 *   o        [B,H,N,d] of `dtype`, written (rounded to nearest even for bf16 and fp16).
 *   lse      [B,H,N] float32, written; may be NULL when not wanted.
 * Arithmetic: products on the matrix cores with float32 accumulation,
 * softmax in float32; for the 16-bit types the probabilities that multiply V
 * are rounded to that type. fp16 shares bf16's algorithm; its narrower range
 * means scores whose dot products, or gradients, exceed 65504 in magnitude
 * overflow where bf16 would not. Deterministic: the same inputs give
 * bitwise-identical outputs.
 */
fa_status_t flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, int causal,
                           int dtype, void* stream);

/*
 * Forward under padding and block-sparse masks (the mask step of 52jiny.com FlashAttention
 * explainer, "why standard attention is IO-bound"; sparse attention as named in yunthe.com
 * "FlashAttention explained", section 5, and codechina.net article, section 7.2).
 *   seqlens     int32 [B] on the device, or NULL: sequence b occupies rows 0 .. L_b - 1 of Q, K
 *               and V; the rest is padding. Values are clamped to [0, N] (not checked on the host).
 *   block_mask  uint8 [B,H,ceil(N/128),ceil(N/128)] on the device, or NULL: entry (r, c) == 0
 *               removes scores of query rows 128r .. 128r+127 against keys 128c .. 128c+127;
 *               whole blocks are skipped, never loaded.
 * Query i sees key j iff i < L_b, j < L_b, (not causal or j <= i) and the block of (i, j) is
 * enabled. A row that sees no key (padding rows included) gets O = 0 and LSE = -inf.
 *   dropout_p, seed  attention dropout (52jiny.com, "why standard attention is IO-bound": the
 *               step between the softmax and the product with V). Each probability P_ij is kept
 *               or zeroed by a byte of the counter-based generator Philox4x32-10 (Salmon, Moraes,
 *               Dror, Shaw, SC 2011): counter (i, j / 32, b * H + h, (j / 4) % 2), key
 *               (seed & 0xffffffff, seed >> 32); byte j % 4 of output word (j % 32) / 8 (byte 0 =
 *               least significant); kept iff byte < T = round(256 (1 - dropout_p)). Kept
 *               probabilities are scaled by 256 / T. LSE stays that of the undropped softmax.
 *               dropout_p = 0 (T = 256) disables dropout; flash_attn_dropout_mask returns the mask.
 * bf16 and fp16; other arguments as flash_attn_fwd. Deterministic for a given seed.
 */
fa_status_t flash_attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int B, int H, int N, int d, float scale, int causal,
                                  const int32_t* seqlens, const uint8_t* block_mask,
                                  float dropout_p, uint64_t seed, int dtype, void* stream);

/*
 * The dropout keep mask flash_attn_fwd_masked applies for (dropout_p, seed), for inspection and
 * testing: keep [B,H,Nq,Nk] uint8 on the device, written 1 (kept) or 0 (dropped) per score
 * element. Not needed to run attention.
 */
fa_status_t flash_attn_dropout_mask(uint8_t* keep, int B, int H, int Nq, int Nk, float dropout_p,
                                    uint64_t seed, void* stream);

/*
 * Forward of Nq queries against Nk >= Nq keys (decoding one or a few new
 * positions against a long key/value history, or a chunk of a longer
 * sequence), with the key range split across workgroups.
 *   q, o     [B,H,Nq,d] of `dtype` (bf16 or fp16); lse [B,H,Nq] float32 or NULL.
 *   k, v     [B,H,Nk,d] of `dtype`.
 *   causal   query i is position Nk - Nq + i of the key sequence and sees keys
 *            j <= Nk - Nq + i (with Nq == Nk this is flash_attn_fwd's mask).
 *   seqlens_k  int32 [B] on the device, or NULL: sequence b's cache holds L_b <= Nk valid
 *            keys (rows L_b .. Nk-1 of K and V are ignored); its queries are positions
 *            L_b - Nq .. L_b - 1, so with causal query i sees keys j <= L_b - Nq + i. A query
 *            that sees no key gets O = 0 and LSE = -inf. Values are clamped to [0, Nk].
 *   num_splits  0 = as many as give every compute unit two workgroups; else
 *            1..64. Each split covers a contiguous run of 64-key tiles.
 * Each split writes its rows' partial softmax (O_s normalised within the
 * split, LSE_s) in float32 to the workspace; a second kernel merges them with
 * the rule the online softmax uses for consecutive blocks (52jiny.com
 * FlashAttention explainer, "key ideas" part 2; codechina.net article,
 * section 4.2): LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 * O and LSE equal those of the plain softmax over all Nk keys. When the launch has a
 * single split (d <= 128) its workgroups write O and LSE directly, which is what the
 * merge would produce with one split; the workspace is then left untouched.
 * workspace: device scratch of at least flash_attn_fwd_kvsplit_workspace_size()
 * bytes for the same shape and num_splits (16-byte aligned); its contents on
 * entry are ignored. Deterministic.
 */
size_t flash_attn_fwd_kvsplit_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits, int dtype);
fa_status_t flash_attn_fwd_kvsplit(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                                   const int32_t* seqlens_k, int num_splits, void* workspace,
                                   size_t workspace_bytes, int dtype, void* stream);

/*
 * flash_attn_fwd_kvsplit without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory: code being captured into a HIP graph, tight decoding loops, and
 * harnesses that forbid hipMalloc. Same arguments, checks, kernels and results as
 * flash_attn_fwd_kvsplit (bitwise equal for the same inputs and num_splits).
 * The fp32 partials live in a fixed device array of FA_NOALLOC_SCRATCH_BYTES inside the library: one
 * copy on each GPU the library runs on, held until the process ends. A call whose
 * flash_attn_fwd_kvsplit_workspace_size() exceeds FA_NOALLOC_SCRATCH_BYTES returns
 * FA_ERR_SCRATCH_LIMIT and launches nothing. Every call on a GPU shares that GPU's array: calls that
 * may overlap on one GPU (different streams, or threads issuing without ordering) race on it and
 * must be serialised by the caller. The array's contents on entry are ignored (every partial is
 * written before it is read). The first call on a device looks up the array's address there; a
 * failure of that lookup returns FA_ERR_HIP.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
fa_status_t flash_attn_fwd_kvsplit_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                           int B, int H, int Nq, int Nk, int d, float scale, int causal,
                                           const int32_t* seqlens_k, int num_splits, int dtype,
                                           void* stream);

/*
 * Bytes of device workspace flash_attn_bwd needs for this shape (the per-row
 * term D = rowsum(dO * O), float32 [B,H,N]). Returns 0 for an invalid shape.
 */
size_t flash_attn_bwd_workspace_size(int B, int H, int N, int d, int dtype);

/*
 * Backward with recomputation, for the loss sum(O * dO). Defined by 52jiny.com FlashAttention
 * explainer, "key ideas" part 4 (the backward keeps only O and the softmax statistics and
 * recomputes the probabilities block by block instead of storing the N x N matrix) and
 * codechina.net article, section 4.2 (the statistics m, l that make the recomputation exact);
 * the gradient formulas below are the chain rule through the row softmax of section 3.
 *   D  = rowsum(dO * O)                     (into the workspace)
 *   P  = exp(scale * Q K^T - LSE)           (recomputed tile by tile)
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q.
 *   q, k, v, o, dout   [B,H,N,d] of `dtype`, read only; o and lse are the
 *                      forward's outputs for the same q, k, v, scale, causal.
 *   lse                [B,H,N] float32, read only (must not be NULL).
 *   dq, dk, dv         [B,H,N,d] of `dtype`, written.
 *   workspace          device scratch of at least workspace_bytes >=
 *                      flash_attn_bwd_workspace_size(); its contents on entry
 *                      are ignored; on return it holds delta (float32 [B,H,N]).
 * Runs flash_attn_bwd_dq and then flash_attn_bwd_dkdv (below) on `stream`.
 * Deterministic (no atomics). bf16 and fp16 only.
 */
fa_status_t flash_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout,
                           void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes,
                           int B, int H, int N, int d, float scale, int causal,
                           int dtype, void* stream);

/*
 * Backward of flash_attn_fwd_masked (same seqlens, block_mask, dropout_p and seed; o and lse from
 * that call). Rows that see no key contribute nothing; dQ rows of such queries and dK, dV rows of
 * keys that no query sees are 0 (padding rows included). With dropout the keep mask is
 * regenerated from the seed: dV = (P Z)^T dO, dP = (dO V^T) Z, dS = P (dP - D), with
 * Z = keep * 256 / T and D = rowsum(dO * O). Workspace and other arguments as flash_attn_bwd.
 */
fa_status_t flash_attn_bwd_masked(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv,
                                  void* workspace, size_t workspace_bytes,
                                  int B, int H, int N, int d, float scale, int causal,
                                  const int32_t* seqlens, const uint8_t* block_mask,
                                  float dropout_p, uint64_t seed, int dtype, void* stream);

/*
 * Backward stages, exposed so a caller can run (or time) them separately. Same
 * conventions and validation as flash_attn_bwd; bf16 and fp16; deterministic.
 * flash_attn_bwd runs flash_attn_bwd_dq and then flash_attn_bwd_dkdv.
 *
 * flash_attn_bwd_delta: delta[b,h,i] = sum_c dout[b,h,i,c] * o[b,h,i,c]
 * (float32 [B,H,N], written). This is the row term the softmax Jacobian
 * subtracts: it equals sum_j P_ij dP_ij. (flash_attn_bwd_dq computes the same
 * values as a by-product; this stage exists for callers that want delta alone.)
 */
fa_status_t flash_attn_bwd_delta(const void* o, const void* dout, float* delta,
                                 int B, int H, int N, int d, int dtype, void* stream);

/*
 * Query-outer stage: for every query tile, compute delta from o and dout
 * (written to `delta`, float32 [B,H,N]), recompute P = exp(scale*Q K^T - LSE)
 * and dP = dO V^T over the key tiles, and accumulate
 *   dQ = scale * (P * (dP - delta)) K.      dq is written.
 */
fa_status_t flash_attn_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, float* delta, void* dq,
                              int B, int H, int N, int d, float scale, int causal,
                              int dtype, void* stream);

/*
 * Key-outer stage: for every key tile, recompute P and dP over all query tiles
 * and accumulate dV = P^T dO and dK = scale * (P * (dP - delta))^T Q.
 * lse and delta (as written by flash_attn_bwd_dq or flash_attn_bwd_delta) are
 * read only; dk and dv are written.
 */
fa_status_t flash_attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                                const void* dout, const float* delta, void* dk, void* dv,
                                int B, int H, int N, int d, float scale, int causal,
                                int dtype, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* flash_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H_ */
