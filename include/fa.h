/*
 * fa.h - exact fused attention on AMD MI355X (gfx950): C ABI.
 *
 * What is computed.  For every batch b and head h, with Q [Nq, d], K [Nk, d], V [Nk, d]:
 *     S = scale * Q K^T,  P = softmax(S) row-wise,  O = P V,  LSE_i = ln sum_j exp(S_ij)
 * This is standard attention as the Day-21 page ("GPU 学习日报 Day 21：FlashAttention：GPU
 * Memory Hierarchy 下的 IO 优化", §3.1) writes it; the result is exact, only the floating-point
 * summation order differs from the unfused form (same page, FAQ Q1; M4-047 card
 * "高效注意力与 FlashAttention", §5).  The GPU never materialises S or P: K/V tiles are staged
 * through LDS and a running max m, a running sum l and a rescaled accumulator replace them
 * (Day-21 page §4-§5.3).  LSE is the per-row statistic a backward pass recomputes from
 * (M4-047 card §3, point (c)).
 *
 * Conventions shared by every entry point.
 *   - Layouts: q, k, v, o are row-major, contiguous [B, H, N, d] (N = Nq for q and o, Nk for
 *     k and v); lse is [B, H, Nq] float32.  O has the storage type of the inputs.
 *   - dtype: FA_DTYPE_BF16 (inputs and O bfloat16; fp32 accumulation, P rounded to bf16 with
 *     round-to-nearest-even before the P V product, O rounded to nearest-even) or FA_DTYPE_F32
 *     (everything float32, no down-conversion anywhere).
 *   - scale must be finite and > 0 (1/sqrt(d) in the pages).
 *   - Every pointer is DEVICE memory owned by the caller.  The library allocates nothing,
 *     keeps no global mutable state, prints nothing, and is safe to call from several threads.
 *     The one exception is fa_decode_noalloc, which uses a fixed scratch array the library
 *     holds per device (see there).
 *   - Work is enqueued on `stream` (NULL = the default stream); calls return without
 *     synchronising.  Inputs must stay valid and unmodified until the work completes.
 *   - Errors: arguments are validated on the host before any HIP call; on any error nothing is
 *     launched and a status other than FA_OK is returned.  A failed launch returns FA_ERR_HIP.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_F32 = 1 } fa_dtype_t;

/* Causal alignment for fa_fwd_ex.  Query row i (0-based) may attend to key j iff
 *   FA_MASK_NONE:                 always;
 *   FA_MASK_CAUSAL:               j <= i                (top-left diagonal, any Nq and Nk);
 *   FA_MASK_CAUSAL_BOTTOM_RIGHT:  j <= i + (Nk - Nq)    (the last query sees every key: Nq new
 *                                 tokens appended to a KV cache of Nk - Nq earlier ones, the
 *                                 prefill-against-a-cache case of the Day-21 page §9; needs
 *                                 Nk >= Nq so that every row sees at least one key).
 * The pages do not fix an alignment for Nq != Nk; both are offered, and with Nq == Nk they agree. */
typedef enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1, FA_MASK_CAUSAL_BOTTOM_RIGHT = 2 } fa_mask_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_ALIGN = 2,       /* q/k/v/o/workspace not 16-byte aligned, lse not 4-byte aligned, or the
                             mask of fa_fwd_masked not 8-byte aligned */
  FA_ERR_SHAPE = 3,       /* a size <= 0, H_kv not dividing H, causal with Nq != Nk (fa_fwd) or
                             bottom-right with Nk < Nq, or sizes beyond the index limits */
  FA_ERR_UNSUPPORTED = 4, /* d not in {64, 128}, unknown dtype, or fp32 in the backward */
  FA_ERR_WORKSPACE = 5,   /* workspace smaller than fa_decode_workspace_bytes() / fa_bwd_workspace_bytes() */
  FA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
  FA_ERR_ARG = 7,         /* scale not finite and > 0, num_splits outside [1, Nk], or an unknown
                             fa_mask_t */
  FA_ERR_SCRATCH = 8      /* fa_decode_noalloc: the split partials, fa_decode_workspace_bytes(B, H, d,
                             num_splits) bytes, exceed FA_DECODE_NOALLOC_SCRATCH_BYTES */
} fa_status_t;

/*
 * Fused attention forward (prefill / training forward).
 *   q [B,H,Nq,d], k and v [B,H,Nk,d]  (in), o [B,H,Nq,d] and lse [B,H,Nq] float32 (out).
 *   causal != 0 applies the mask "key j is allowed iff j <= i" for query row i; it requires
 *   Nq == Nk.  Fully masked key tiles are skipped and only tiles on the diagonal are masked
 *   element by element (Day-21 page §6 table, last row).
 *   Limits: B*H*ceil(Nq/128) < 2^31 and N*d*sizeof(elt) < 2^31 per head.
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   int causal, float scale, fa_dtype_t dtype, hipStream_t stream);

/*
 * Fused attention forward with grouped K/V heads and a choice of causal alignment.
 *   q [B,H,Nq,d], k and v [B,H_kv,Nk,d]  (in), o [B,H,Nq,d] and lse [B,H,Nq] float32 (out).
 *   H_kv must divide H; query head h reads K/V head h / (H / H_kv) (grouped-query attention,
 *   which the Day-21 page's FAQ Q5 lists among the techniques that matter once reading K/V
 *   dominates; H_kv == H is multi-head attention, H_kv == 1 multi-query attention).
 *   mask: see fa_mask_t.  Everything else (dtypes, layouts, precision, limits, errors) is as
 *   for fa_fwd, which equals fa_fwd_ex with H_kv = H and mask = causal ? FA_MASK_CAUSAL :
 *   FA_MASK_NONE (fa_fwd additionally rejects causal with Nq != Nk).
 */
fa_status_t fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t H_kv, int64_t Nq, int64_t Nk, int64_t d,
                      fa_mask_t mask, float scale, fa_dtype_t dtype, hipStream_t stream);

/*
 * Forward with FP8 inputs (the Day-21 page names FP8 as a FlashAttention-3 feature at the close of
 * its §6): q [B,H,Nq,d], k and v [B,H_kv,Nk,d] are OCP FP8 E4M3 codes, one byte per element
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinity, S.1111.111 =
 * NaN); q_scale [B,H], k_scale and v_scale [B,H_kv] float32: an element's value is the E4M3 value
 * of its code times the scale of its (batch, head).  o [B,H,Nq,d] bf16 and lse [B,H,Nq] float32
 * (out), as fa_fwd_ex computes them on the decoded values: O = softmax(scale * Q K^T) V with the
 * mask, LSE natural log.  Both products run on the FP8 matrix core; P is rounded to E4M3 (round
 * to nearest even) for the second, with values kept between 2^-10 and 2^8 of the running row
 * max so that none but the negligible ones fall into the E4M3 subnormals; the row sums and LSE
 * use the unrounded P.  Grouped heads, masks, layouts, limits and errors as for fa_fwd_ex
 * (q, k, v, o 16-byte aligned; the scales and lse 4-byte aligned).
 */
fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                       const float* k_scale, const float* v_scale, void* o, float* lse, int64_t B,
                       int64_t H, int64_t H_kv, int64_t Nq, int64_t Nk, int64_t d, fa_mask_t mask,
                       float scale, hipStream_t stream);

/*
 * Forward with an arbitrary element mask (the Day-21 page's §6 table, last row: blocks the mask
 * leaves empty are skipped, partly visible blocks are masked element by element; the Q31 answer
 * "FlashAttention 为什么快", §2, names arbitrary masks as what FlashAttention-2 lacks).
 *   q [B,H,Nq,d], k and v [B,H_kv,Nk,d] bf16 (in); o [B,H,Nq,d] bf16 and lse [B,H,Nq] float32
 *   (out), as fa_fwd_ex with no mask except that key j is visible to query row i iff bit (j % 64)
 *   of mask[i * ceil(Nk/64) + j / 64] is 1.  The mask is one [Nq][ceil(Nk/64)] array of 64-bit
 *   words in device memory, shared by every batch and head; bits of keys >= Nk are ignored.  A row
 *   with no visible key gets O = 0 and LSE = -inf.
 *   workspace: caller-owned device memory of at least fa_fwd_masked_workspace_bytes(Nq, Nk)
 *   bytes, 16-byte aligned.  Small kernels classify every (block of 256 query rows, 64-key
 *   tile) of the mask as empty, full or partial and write each block's list of non-empty tiles
 *   there, and a counter from which the forward's workgroups claim (block, head) items, the
 *   blocks with the most tiles first; the forward then streams only the listed tiles and applies
 *   the element mask only on the partial ones.  The workspace holds nothing across calls; two
 *   calls that overlap on one workspace race.
 *   dtype must be FA_DTYPE_BF16; d 64 or 128; Nk <= 131072 (FA_ERR_SHAPE beyond); mask 8-byte
 *   aligned.  Other limits and errors as for fa_fwd_ex.
 */
size_t fa_fwd_masked_workspace_bytes(int64_t Nq, int64_t Nk);
fa_status_t fa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t H_kv, int64_t Nq, int64_t Nk, int64_t d,
                          const uint64_t* mask, void* workspace, size_t workspace_bytes, float scale,
                          fa_dtype_t dtype, hipStream_t stream);

/*
 * Split-KV decode (one query token per (b, h) against a KV cache): the keys are split into
 * num_splits contiguous chunks of ceil(Nk / num_splits) keys that are processed in parallel,
 * then the partial results are merged (Q31 answer, "FlashAttention 为什么快", follow-up 3;
 * the merge rescales each partial by exp(m_s - max_s m_s), follow-up 2).  A trailing chunk may
 * be short or empty; the result does not depend on num_splits beyond rounding.
 *
 * Workspace (float32, owned by the caller, 16-byte aligned), as written by fa_decode_split
 * and read by fa_decode_combine:
 *     float O_part[B][H][num_splits][d];  - sum_j exp(s_j - m_s) v_j over the split (unnormalised)
 *     float ml[B][H][num_splits][2];      - (m_s, l_s): max score of the split (natural-log units,
 *                                           -inf for an empty split) and sum_j exp(s_j - m_s)
 *   ml starts right after O_part.  fa_decode_workspace_bytes returns B*H*num_splits*(d+2)*4.
 */
size_t fa_decode_workspace_bytes(int64_t B, int64_t H, int64_t d, int num_splits);

/* q [B,H,1,d], k and v [B,H,Nk,d] (in); fills the workspace.  1 <= num_splits <= Nk. */
fa_status_t fa_decode_split(const void* q, const void* k, const void* v,
                            void* workspace, size_t workspace_bytes,
                            int64_t B, int64_t H, int64_t Nk, int64_t d, float scale,
                            int num_splits, fa_dtype_t dtype, hipStream_t stream);

/*
 * Split step of decode with grouped K/V heads: q [B,H,1,d], k and v [B,H_kv,Nk,d], H_kv
 * dividing H; query head h reads K/V head h / (H / H_kv) (see fa_fwd_ex).  The workspace, its
 * size (per query head: fa_decode_workspace_bytes(B, H, d, num_splits)), the merge
 * (fa_decode_combine, unchanged) and the errors are as for fa_decode_split, which equals
 * fa_decode_split_ex with H_kv = H.
 */
fa_status_t fa_decode_split_ex(const void* q, const void* k, const void* v,
                               void* workspace, size_t workspace_bytes,
                               int64_t B, int64_t H, int64_t H_kv, int64_t Nk, int64_t d, float scale,
                               int num_splits, fa_dtype_t dtype, hipStream_t stream);

/* Merges the workspace into o [B,H,1,d] (dtype) and lse [B,H,1] float32. */
fa_status_t fa_decode_combine(const void* workspace, size_t workspace_bytes, void* o, float* lse,
                              int64_t B, int64_t H, int64_t d, int num_splits,
                              fa_dtype_t dtype, hipStream_t stream);

/*
 * One-token decode that allocates nothing: for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  It is
 * fa_decode_split_ex followed by fa_decode_combine on the same stream, with the same kernels and
 * the same results bit for bit, except that the split partials go to a fixed scratch array that
 * the library holds in device memory instead of a caller's workspace.
 *   q [B,H,1,d], k and v [B,H_kv,Nk,d] (in); o [B,H,1,d] (dtype) and lse [B,H,1] float32 (out).
 *   Requires fa_decode_workspace_bytes(B, H, d, num_splits) <= FA_DECODE_NOALLOC_SCRATCH_BYTES
 *   (32 MiB; e.g. B16 H32 d128 with 64 splits needs 17.0 MB), else FA_ERR_SCRATCH and nothing is
 *   launched.  Other errors as for fa_decode_split_ex, plus o (16 bytes) and lse (4 bytes)
 *   alignment.  `stream` must belong to the current device.
 *   Unlike the other entry points, this one keeps state: each GPU holds one 32 MiB scratch array
 *   from the library's load until the process ends, and the library remembers its address per
 *   device after the first call there.  Every call on a GPU shares that GPU's array, so calls
 *   that overlap on one GPU (on different streams, or from different threads without ordering)
 *   race and give wrong results; calls ordered on one stream are safe.  Nothing in the scratch
 *   needs clearing: every call writes all the partials it reads.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
fa_status_t fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t H_kv, int64_t Nk, int64_t d, float scale,
                              int num_splits, fa_dtype_t dtype, hipStream_t stream);

/*
 * Split step of decode against an FP8 KV cache (KV-cache quantisation, which the Day-21 page's
 * FAQ Q5 names among the decode-side techniques; the cache is read with half the bytes of bf16):
 *   q [B,H,1,d] bf16; k and v [B,H_kv,Nk,d] OCP FP8 E4M3 codes, one byte per element (sign,
 *   4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinity, S.1111.111 = NaN);
 *   k_scale and v_scale [B,H_kv] float32: the value of a code of K/V head (b, j) is its E4M3
 *   value times k_scale[b*H_kv + j] (resp. v_scale).  Everything else (grouped heads, splits, the
 *   workspace and its size, errors) is as for fa_decode_split_ex; fa_decode_combine with dtype
 *   FA_DTYPE_BF16 merges the partials into a bf16 o.  NaN codes give NaN results.
 */
fa_status_t fa_decode_split_fp8kv(const void* q, const void* k, const void* v, const float* k_scale,
                                  const float* v_scale, void* workspace, size_t workspace_bytes,
                                  int64_t B, int64_t H, int64_t H_kv, int64_t Nk, int64_t d,
                                  float scale, int num_splits, hipStream_t stream);

/*
 * Backward pass: the gradients of a loss with respect to q, k and v, given its gradient dout
 * with respect to the forward's output o.  The probabilities are recomputed tile by tile from
 * q, k and the forward's lse instead of being stored (M4-047 card "高效注意力与 FlashAttention",
 * §3 point (c)); with Dr_i = dout_i . o_i:
 *     P = exp(scale q k^T - lse) (0 where masked),  dv = P^T dout,  dS = P * (dout v^T - Dr),
 *     dq = scale dS k,  dk = scale dS^T q.
 *   q, o, dout [B,H,Nq,d]; k, v [B,H_kv,Nk,d]; lse [B,H,Nq] float32 as fa_fwd / fa_fwd_ex wrote
 *   it for the same q, k, v, mask and scale  (in);
 *   dq [B,H,Nq,d], dk and dv [B,H_kv,Nk,d]  (out, bf16, RNE; fp32 accumulation inside; the
 *   gradient of a K/V head sums over the query heads that read it).
 *   mask, H_kv, scale: as for fa_fwd_ex.  dtype must be FA_DTYPE_BF16.
 *   workspace: caller-owned device memory of at least fa_bwd_workspace_bytes(B, H, Nq) bytes,
 *   16-byte aligned; it holds two floats per query row (lse in log2 units and Dr) between the
 *   launches of one call, and nothing across calls.
 *   The result is deterministic (no atomics).  Limits as for fa_fwd, and B*H*Nq*8 < 2^31.
 */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq);
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, int64_t B, int64_t H, int64_t H_kv, int64_t Nq,
                   int64_t Nk, int64_t d, fa_mask_t mask, float scale, fa_dtype_t dtype,
                   hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_string(fa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
