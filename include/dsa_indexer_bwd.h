/*
 * dsa_indexer_bwd.h — C ABI of the MI355X (gfx950) backward pass of the
 * DeepSeek-Sparse-Attention lightning indexer.
 *
 * The indexer scores query t against key s as
 *     I[t,s] = sum_h w[t,h] * relu(q[t,h,:] . k[s,:])
 * restricted to per-query top-k key ids.  The backward pass defined by the
 * fp64 reference of NVIDIA/cudnn-frontend PR #730 (its posted A/B benchmark
 * harness, `ref_grads`, together with the kernel-1 score-gradient contract in
 * the same harness docstring) is, per query row t with valid slot set
 * V = { j : 0 <= id_j < S_k }:
 *     dI_j      = grad_loss * sm_scale * (softmax_V(sm_scale * I[t,:])_j - p[t,j])
 *     S[h,j]    = q[t,h,:] . k[id_j,:]
 *     G[h,j]    = dI_j * w[t,h] * [S[h,j] > 0]
 *     d_w[t,h]  = sum_{j in V} dI_j * max(S[h,j], 0)
 *     d_q[t,h,:]= sum_{j in V} G[h,j] * k[id_j,:]
 *     d_k[s,:]  = sum over every (t, j in V) with id_j = s of sum_h G[h,j] * q[t,h,:]
 * (index_score is I, attn_score is the target distribution p.)
 *
 * The step before it is declared here too: indexer_fwd_scores computes I for
 * every key and indexer_topk selects each row's top-k, whose ids and scores
 * are this backward's topk_ids and index_score.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, contiguous, and live in device memory
 *     of the current HIP device.  bf16 tensors are passed as their 16-bit
 *     patterns (`const void*`).
 *   - Shapes: q [B,S_q,H,D] bf16, k [B,S_k,D] bf16, w [B,S_q,H] fp32,
 *     d_q [B,S_q,H,D], d_w [B,S_q,H], d_k [B,S_k,D], all fp32, or all bf16
 *     with IBWD_FLAG_BF16_OUT.
 *   - Ids are local to each batch: 0 <= id < S_k selects key id of the same
 *     batch; every other value (-1 canonically, any negative, any >= S_k) is a
 *     padding slot that contributes nothing, whatever index_score/attn_score
 *     hold there (PR #730 review thread: a positive out-of-range local id is
 *     padding and must not alias the next batch; harness padding battery).
 *     Duplicate ids are independent slots.
 *   - Ownership: the caller owns every buffer.  The library allocates nothing,
 *     frees nothing, keeps no state between calls apart from a per-device cache
 *     of the device check (and the optional profiling hook below), never
 *     synchronises, and only enqueues work on
 *     `stream` (0 = the null stream).  Inputs are read-only (attn_score too).
 *     d_q, d_w and d_k are overwritten in full (d_k is zeroed by the library).
 *   - Alignment: q, k, d_q, d_k must be 16-byte aligned; w, index_score,
 *     attn_score, topk_ids, d_w 4-byte aligned.
 *   - Supported shapes: 1 <= H <= 64, D in {32, 64, 128}; every dimension >= 1;
 *     element counts below 2^31 per tensor; S_k <= 262144.
 *   - Errors: every argument is validated before anything is written or
 *     launched, so on error the outputs are untouched.  Launch failures are
 *     reported by the HIP error of the launch; execution errors surface on the
 *     stream as usual for HIP.
 *   - dK routes.  The default route reduces the dK scatter in two passes: a
 *     prep kernel lays out each row's records by key range and computes every
 *     slot's dI, the row kernel exports each slot's sign mask [S > 0] and dI
 *     into the caller's workspace, and a range-major kernel computes the dK of
 *     every 128-key
 *     range as a GEMM over (query, head) whose accumulators stay in the matrix
 *     cores (dI enters that GEMM rounded to bf16, like w*q), then the per
 *     query-block partial sums are added in a fixed order.  d_q, d_w and d_k
 *     are all bitwise reproducible run to run.
 *     When a row selects few keys per 128-key range (topk*8 <= S_k by
 *     default; IBWD_FLAG_DK_SLOT_ROWS / IBWD_FLAG_DK_KEY_RANGES force either
 *     way) the deterministic call takes the slot-row route instead: the row
 *     kernel computes each valid slot's dK row dI * sum_h [S > 0] (w*q)[h,:]
 *     (PR #730 harness `ref_grads`, the `contrib` rows before `index_add_`)
 *     on the matrix cores, rounds it to bf16 and stores it with the slot's key,
 *     and a second kernel adds the rows of each key in a fixed order.  d_q and
 *     d_w are the same bits on both routes; d_k differs by the rounding of the
 *     rows (relRMS about 3e-3 against the fp64 reference, 2e-3 on the key
 *     ranges) and is again bitwise reproducible.
 *     IBWD_FLAG_ATOMIC_DK selects the single-pass route of the pages' design
 *     instead: fp32 global atomics straight from the row kernel, no workspace,
 *     and d_k may then differ in the last bits between runs (PR #549: dK uses
 *     fp32 atomicAdd and is run-to-run nondeterministic).
 */
#ifndef DSA_INDEXER_BWD_H
#define DSA_INDEXER_BWD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define IBWD_OK 0
#define IBWD_ERR_INVALID_ARGUMENT -1 /* null pointer, bad shape (topk > S_k included), misaligned,
                                        workspace too small */
#define IBWD_ERR_UNSUPPORTED_DEVICE -2 /* the current device is not gfx950 */
#define IBWD_ERR_HIP -3              /* a HIP runtime call or launch failed */

/* Flags. */
#define IBWD_FLAG_DETERMINISTIC 1u /* request the bitwise-reproducible route (the default
                                      two-pass route; conflicts with IBWD_FLAG_ATOMIC_DK) */
#define IBWD_FLAG_ATOMIC_DK 2u     /* single-pass dK with fp32 global atomics; no workspace;
                                      d_k not bitwise reproducible */
#define IBWD_FLAG_GLOBAL_IDS 4u    /* indexer_bwd_sparse only: topk_ids index the flattened
                                      [B*S_k] key array instead of the batch's own keys */
#define IBWD_FLAG_BF16_OUT 8u      /* d_q, d_w and d_k are bf16 arrays (PR #730 harness: bf16
                                      dQ and dW, dK cast to bf16), each rounded to nearest
                                      even from fp32: d_w and d_k from the fp32 results of the
                                      same call without this flag, d_q from a dQ whose G enters
                                      its product as two bf16 terms (bf16(G) and the bf16 of
                                      the remainder), so that the output rounding is its only
                                      error of note.  Default route only; not with
                                      IBWD_FLAG_ATOMIC_DK, whose dK accumulates in d_k */
#define IBWD_FLAG_DK_KEY_RANGES 16u /* deterministic dK by the key-range GEMM at any selection
                                       density (by default a sparse call with topk*8 > S_k) */
#define IBWD_FLAG_DK_SLOT_ROWS 32u  /* indexer_bwd_sparse only: deterministic dK from per-slot
                                       rows at any density (by default when topk*8 <= S_k);
                                       needs (B*S_q*topk + 1)*D*2 < 2^32 (the default falls
                                       back to key ranges beyond); excludes
                                       IBWD_FLAG_DK_KEY_RANGES */

/*
 * indexer_bwd_sparse — backward of the top-k (sparse) indexer.
 *
 *   topk_ids     [B,S_q,topk] int32, batch-local key ids (see padding above);
 *                1 <= topk <= S_k (a larger topk is IBWD_ERR_INVALID_ARGUMENT).
 *                With IBWD_FLAG_GLOBAL_IDS the ids are global instead (the
 *                factory flag topk_indices_global of PR #730's benchmark
 *                harness): a row of batch b selects key id - b*S_k of its own
 *                batch when b*S_k <= id < (b+1)*S_k, and every other id,
 *                another batch's key included, is a padding slot.  At B = 1
 *                the two conventions coincide.
 *   index_score  [B,S_q,topk] fp32, the forward scores I of the selected slots
 *   attn_score   [B,S_q,topk] fp32, the target distribution p over the valid
 *                slots (read-only; the kernel never writes it)
 *   sm_scale     scale applied to I inside the softmax and as chain factor
 *   grad_loss    upstream gradient of the KL loss (a scalar)
 *   flags        0, IBWD_FLAG_DETERMINISTIC or IBWD_FLAG_ATOMIC_DK, optionally or-ed
 *                with IBWD_FLAG_GLOBAL_IDS and (not with IBWD_FLAG_ATOMIC_DK)
 *                IBWD_FLAG_BF16_OUT
 *   d_q, d_w, d_k  outputs: fp32, or bf16 bit patterns with IBWD_FLAG_BF16_OUT
 *   workspace    device scratch of at least indexer_bwd_workspace_bytes(...)
 *                bytes (may be NULL when that size is 0); 256-byte aligned
 *   stream       HIP stream the work is enqueued on
 *
 * Returns IBWD_OK or one of the IBWD_ERR_* codes.
 */
int indexer_bwd_sparse(const void* q, const void* k, const float* w, const int32_t* topk_ids,
                       const float* index_score, const float* attn_score, void* d_q, void* d_w,
                       void* d_k, int64_t B, int64_t S_q, int64_t S_k, int64_t H, int64_t D,
                       int64_t topk, float sm_scale, float grad_loss, uint32_t flags,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * indexer_bwd_sparse_noalloc — indexer_bwd_sparse for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace; its scratch is a
 * library-owned device array of IBWD_NOALLOC_SCRATCH_BYTES bytes (a
 * file-scope device variable: each GPU the library runs on holds its own copy
 * until the process ends).  The call allocates and frees nothing; the first
 * call on a device resolves the array's address on that device (make one
 * before capturing a graph).  The caller passes inputs and outputs exactly as
 * for indexer_bwd_sparse.
 *   - A call whose indexer_bwd_workspace_bytes(0, B, S_q, S_k, H, D, topk,
 *     flags) exceeds IBWD_NOALLOC_SCRATCH_BYTES returns
 *     IBWD_ERR_INVALID_ARGUMENT before anything is written or launched (at
 *     H=64, D=128, S_k=4096, topk=1024 the limit is 2354 query rows).
 *   - Every call on a GPU shares that GPU's array, which keeps the last call's
 *     contents; no part of it needs clearing (each location a kernel reads is
 *     written earlier in the same call).  Calls that overlap on one GPU (other
 *     streams, other threads) race on the array: the caller must order them.
 * Arguments, flags, results and other errors as for indexer_bwd_sparse.
 */
#define IBWD_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int indexer_bwd_sparse_noalloc(const void* q, const void* k, const float* w,
                               const int32_t* topk_ids, const float* index_score,
                               const float* attn_score, void* d_q, void* d_w, void* d_k, int64_t B,
                               int64_t S_q, int64_t S_k, int64_t H, int64_t D, int64_t topk,
                               float sm_scale, float grad_loss, uint32_t flags,
                               hipStream_t stream);

/*
 * indexer_bwd_dense — backward of the dense causal indexer: query t of a batch
 * selects every key s with 0 <= s <= t + q_offset (and s < S_k); a row with no
 * such key contributes nothing (PR #549 names a separate dense indexer-backward
 * test; PR #730 keeps the q-causal-offset behaviour).
 *
 *   index_score  [B,S_q,S_k] fp32, I[t,s]; entries with s > t + q_offset are ignored
 *   attn_score   [B,S_q,S_k] fp32, p[t,s]; same masking
 *   q_offset     causal offset (may be negative)
 *
 * Other arguments as for indexer_bwd_sparse.
 */
int indexer_bwd_dense(const void* q, const void* k, const float* w, const float* index_score,
                      const float* attn_score, void* d_q, void* d_w, void* d_k, int64_t B,
                      int64_t S_q, int64_t S_k, int64_t H, int64_t D, int64_t q_offset,
                      float sm_scale, float grad_loss, uint32_t flags, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * indexer_bwd_workspace_bytes — device scratch needed by a call with these
 * arguments (dense != 0 selects indexer_bwd_dense; topk is ignored then).
 * The key-range route needs 16 bytes per record entry (topk + 3 per 128-key
 * range per row, for aligning the ranges), 8 bytes per slot for each slot's
 * record position and dI, 8 bytes per row and key range for the range table,
 * (w*q)^T in bf16 (2*H_pad*D bytes per row, H_pad = 32 or 64) and the per
 * query-block dK partial sums (about 385 MB in all at B=1, S_q=8192, S_k=4096,
 * H=64, D=128, topk=1024; about 511 MB for the dense variant at that shape).
 * The slot-row route needs 8 + 4 + 2*D bytes per slot (position and dI, key,
 * bf16 dK row), one spare row, the range table and the partial sums (about
 * 317 MB at topk=128 of the same shape).  The flags choose the route, so pass
 * the call's flags.  IBWD_FLAG_ATOMIC_DK needs none (0).
 * Returns 0 for invalid shapes as well; the call itself reports those.
 */
size_t indexer_bwd_workspace_bytes(int dense, int64_t B, int64_t S_q, int64_t S_k, int64_t H,
                                   int64_t D, int64_t topk, uint32_t flags);

/*
 * indexer_fwd_scores — the indexer scores that the top-k step selects from:
 *     scores[b,t,s] = sum_h w[b,t,h] * relu(q[b,t,h,:] . k[b,s,:])
 * for every key s of the batch (the score whose gradients the PR #730
 * harness's fp64 reference computes; bf16 products, fp32 accumulation).  With
 * causal != 0, key s is visible to query t only when s <= t + q_offset, and
 * the other keys score -inf.
 *
 *   q [B,S_q,H,D] bf16, k [B,S_k,D] bf16, w [B,S_q,H] fp32 (as above)
 *   scores       [B,S_q,S_k] fp32, overwritten in full
 * Shapes as for the backward (H <= 64, D in {32, 64, 128}); B*S_q*S_k below
 * 2^31.  No workspace.  Returns IBWD_OK or an IBWD_ERR_* code.
 */
int indexer_fwd_scores(const void* q, const void* k, const float* w, float* scores, int64_t B,
                       int64_t S_q, int64_t S_k, int64_t H, int64_t D, int causal,
                       int64_t q_offset, hipStream_t stream);

/*
 * indexer_topk — per row of scores [rows, S_k] fp32: the min(topk, n) largest
 * of its n finite scores (a tie at the threshold goes to the lower key id),
 * written to topk_ids [rows, topk] int32 in ascending key id, followed by -1
 * for the slots left over; topk_scores [rows, topk] fp32 (may be NULL)
 * receives the selected scores and -inf after them.  -0 and +0 rank equal.
 * 1 <= topk <= S_k; rows*S_k below 2^31; pointers 4-byte aligned.  With rows
 * = B*S_q, the outputs are the topk_ids and index_score arguments of
 * indexer_bwd_sparse.  No workspace.
 */
int indexer_topk(const float* scores, int32_t* topk_ids, float* topk_scores, int64_t rows,
                 int64_t S_k, int64_t topk, hipStream_t stream);

/* indexer_bwd_strerror — static text for a status code (never NULL). */
const char* indexer_bwd_strerror(int status);

/*
 * indexer_bwd_set_stage_hook — profiling aid, outside the numerical contract.
 * While a hook is set, every call of indexer_bwd_sparse / indexer_bwd_dense
 * calls hook(user, stage, kernel) on the host right after it has enqueued its
 * kernel number `stage` (0, 1, ...) on the call's stream; `kernel` is a static
 * name.  A hook that records a HIP event on that stream therefore separates
 * the kernels of a call in stream order, which lets a caller time each kernel
 * with events.  The hook must not enqueue work that changes the call's
 * buffers.  The setting is process-wide and not synchronised: set it while no
 * other thread calls the library.  hook = NULL removes it.  Returns IBWD_OK.
 */
typedef void (*indexer_bwd_stage_hook_t)(void* user, int stage, const char* kernel);
int indexer_bwd_set_stage_hook(indexer_bwd_stage_hook_t hook, void* user);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEXER_BWD_H */
