/*
 * fa_bwd.h -- single-pass attention backward on AMD MI355X (gfx950), C ABI.
 *
 * Computes the gradients dQ, dK, dV of softmax attention from the forward's
 * inputs Q, K, V, its output O, the incoming gradient dO and the forward's
 * softmax row statistics m (row max) and l (row sum). The per-tile arithmetic
 * is the eight steps of the PyPTO-Gym SK-16 article ("single-pass attention
 * backward (FA Grad)"), section 3.1:
 *     S = Q K^T, P = exp(S*scale - m) / l, dP = dO V^T, D = rowsum(O*dO),
 *     dS = P*(dP - D), dV = P^T dO, dK = scale * dS^T Q, dQ = scale * dS K,
 * with the inputs in bf16, all softmax arithmetic and accumulation in fp32 and
 * the outputs in bf16 (the article's dtype table, section 4.2).
 *
 * Layout (the article's [total, heads, head_dim] tensors, section 三, and the
 * BTNH layout with the batch and sequence axes flattened, jax cuDNN wrapper,
 * AttentionLayout): every bf16 tensor is a contiguous row-major
 * [T][H][d] array (token-major, then head, then feature), with d = head_dim
 * for Q, K, dQ, dK and d = head_dim_v for V, O, dO, dV; m and l are
 * contiguous fp32 [T_q][H]. All tensor pointers are DEVICE pointers, owned by
 * the caller, 16-byte aligned.
 *
 * Sequences (the article's actual_q / actual_kv offsets, section 三; jax
 * cuDNN wrapper, dot_product_attention and _fix_seqlen_offsets):
 *   cu_seqlens_q/kv are DEVICE int32 arrays of batch+1 non-decreasing entries
 *   with cu[0] = 0. L_b = cu[b+1] - cu[b] is the valid length of sequence b.
 *   - FA_BWD_MASK_NONE, FA_BWD_MASK_CAUSAL (packed varlen): sequence b is rows
 *     [cu[b], cu[b+1]); no attention across sequences; cu[batch] <= total.
 *   - FA_BWD_MASK_PADDING, FA_BWD_MASK_PADDING_CAUSAL (padded): sequence b
 *     occupies the slot of rows [b*max_seqlen, (b+1)*max_seqlen) and its first
 *     L_b <= max_seqlen rows are valid; the rest of the slot is padding.
 *   Causal masks are top-left aligned in sequence-local coordinates: key j is
 *   visible from query i iff j <= i.
 *   Rows outside every sequence (padding, or rows at or after cu[batch]) are
 *   never read, and their dQ/dK/dV are written as 0. The contents of
 *   cu_seqlens are preconditions: the library does not read them on the host;
 *   device code never touches a row outside [0, total) whatever they hold.
 *
 * Outputs dq/dk/dv are fully overwritten (no pre-zeroing needed).
 * Masks use the codes of jax's cuDNN MaskType (NO_MASK, PADDING, CAUSAL,
 * PADDING_CAUSAL); ALIBI is not supported.
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fa_bwd_handle fa_bwd_handle; /* opaque: sizes + device workspace */

typedef enum {
  FA_BWD_MASK_NONE = 0,
  FA_BWD_MASK_PADDING = 1,
  FA_BWD_MASK_CAUSAL = 2,
  FA_BWD_MASK_PADDING_CAUSAL = 3
} fa_bwd_mask;

/* How dQ is formed. All forms compute the same per-tile math (steps 1-8) and
 * agree within the fp32 rounding of the accumulation order. */
typedef enum {
  FA_BWD_ALGO_DEFAULT = 0,      /* the faster form on this GPU: FA_BWD_ALGO_STORED_DS where runs take the
                                   64-key layout (head dims of 128, no window, grids that balance) or
                                   the wide-head kernels (a head dim above 128, no window) and its dS
                                   workspace is at most 8 GiB, else FA_BWD_ALGO_RECOMPUTE_DQ */
  FA_BWD_ALGO_SINGLE_PASS = 1,  /* the article's single-pass structure: one main kernel forms the dK, dV and
                                   dQ contributions of every (q tile, kv tile) pair; dQ partial sums are
                                   added to an fp32 workspace with global atomics (summation order not
                                   fixed), then cast to bf16 */
  FA_BWD_ALGO_RECOMPUTE_DQ = 2, /* the article's two-pass fallback: a kv-outer kernel forms dK, dV and a
                                   q-outer kernel recomputes S and dP to form dQ in registers; no
                                   atomics, no dQ workspace, bitwise reproducible. For head dims up to
                                   128 the kv-outer kernel has two layouts, chosen per run by load
                                   balance (the four-wave one when the largest workgroup, doubled,
                                   fits within the average work per compute unit) */
  FA_BWD_ALGO_SPLIT_REDUCE = 3, /* the single-pass structure with a fixed-order dQ reduction in place of
                                   the atomics (the article gives a fixed summation order as a reason for
                                   its two-pass fallback; this keeps one pass): 8 workgroups per (head,
                                   sequence) each walk every 8th kv tile and keep their dQ partial sums
                                   in a buffer of their own (8 fp32 copies of dQ in the workspace); a
                                   last kernel sums the 8 buffers in a fixed order and casts to bf16;
                                   bitwise reproducible. Same restrictions as FA_BWD_ALGO_SINGLE_PASS */
  FA_BWD_ALGO_RECOMPUTE_DQ_8W = 4, /* FA_BWD_ALGO_RECOMPUTE_DQ with the eight-wave layout of the kv-outer
                                   kernel: one workgroup per compute unit, the two waves of each 32-key
                                   group split every 64-row q step */
  FA_BWD_ALGO_RECOMPUTE_DQ_4W = 5, /* FA_BWD_ALGO_RECOMPUTE_DQ with the four-wave layout: two workgroups
                                   per compute unit, each wave takes whole 32-row q steps for its 32
                                   keys. Both layouts give the same results within fp32 rounding (the
                                   order of the dK, dV sums differs); for head dims above 128 both
                                   codes run the one wide-head layout */
  FA_BWD_ALGO_RECOMPUTE_DQ_64K = 6, /* FA_BWD_ALGO_RECOMPUTE_DQ with the 64-key layout of the kv-outer
                                   kernel: one four-wave workgroup per compute unit over 256 keys, each
                                   wave holding 64 keys and their dK, dV sums, 32-row q steps; head
                                   dims of exactly 128 (else FA_BWD_ERR_UNSUPPORTED), with or without
                                   a window */
  FA_BWD_ALGO_STORED_DS = 7        /* the kv-outer kernel also writes dS (bf16) to a workspace, and
                                   dQ = scale * dS K (SK-16 article, section 3.1, step 8) runs as a
                                   q-outer pass over it instead of forming S and dP a second time.
                                   Head dims of exactly 128: the 64-key kernel, with or without a
                                   window; workspace batch * num_heads * ceil(max_seqlen_q / 32) *
                                   ceil(max_seqlen_kv / 256) blocks of 16 KiB. A head dim above 128
                                   (the wide-head kernels), no window: the same bytes as pieces of
                                   32 x 32 (2 KiB). Other head dims, or a window with a head dim
                                   above 128: FA_BWD_ERR_UNSUPPORTED. Deterministic (every output
                                   row has one owner) */
} fa_bwd_algo;

typedef enum {
  FA_BWD_OK = 0,
  FA_BWD_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad mask code, bad scale, misalignment */
  FA_BWD_ERR_UNSUPPORTED = 2,      /* a head dim that is not a multiple of 8 in [8, 256]; in the
                                      single-pass and split-reduce forms: head dims other than 64 or
                                      128, unequal head dims, grouped heads or a window */
  FA_BWD_ERR_OUT_OF_MEMORY = 3,    /* workspace allocation failed in fa_bwd_create */
  FA_BWD_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
  FA_BWD_ERR_SCRATCH_LIMIT = 5     /* fa_bwd_run_noalloc: total_q * num_heads exceeds
                                      FA_BWD_NOALLOC_MAX_ROWS */
} fa_bwd_status;

typedef struct {
  int32_t batch;         /* number of sequences (entries of cu_seqlens minus one), >= 1 */
  int32_t num_heads;     /* heads of Q, O, dO, dQ, m, l, >= 1 */
  int32_t head_dim;      /* head dim of Q, K, dQ, dK: a multiple of 8 from 8 to 256 (the head dim
                            limits of the jax cuDNN wrapper's bf16 path); the single-pass form takes
                            64 and 128 */
  int32_t max_seqlen_q;  /* >= every L_b of the queries; the slot length in padded modes; 1 .. 2^30 */
  int32_t max_seqlen_kv; /* same for keys/values */
  int64_t total_q;       /* rows of q, o, do, dq, m, l; >= 1 */
  int64_t total_kv;      /* rows of k, v, dk, dv; >= 1 */
  int32_t algorithm;     /* an fa_bwd_algo code */
  int32_t num_heads_kv;  /* heads of K and V (and dK, dV): 0 = num_heads, else a divisor of num_heads;
                            query head h reads K/V head h / (num_heads / num_heads_kv), and the
                            gradient of a shared head sums over its query heads (grouped heads, as
                            the jax cuDNN wrapper's API allows; recompute form only) */
  int32_t window;        /* 0: no window; w > 0: every query i sees only its left local window of keys
                            (i - w, i] (the jax cuDNN wrapper's sliding_window_length), which implies
                            the causal bound whatever the mask code; any w >= max_seqlen_q acts as
                            w = max_seqlen_q (the causal bound alone); recompute form and forward only */
  int32_t head_dim_v;    /* head dim of V, O, dO and dV: 0 = head_dim. It may differ from head_dim
                            (latent attention: the jax cuDNN wrapper's qH != vH); then S = Q K^T runs
                            over head_dim and O = P V over head_dim_v. Recompute form and forward only */
} fa_bwd_desc;

/* Validates desc (a num_heads_kv of 0 is stored as num_heads) and allocates
 * the device workspace of the handle on the current HIP device: two fp32 [H][total_q] row-statistic arrays and, for
 * FA_BWD_ALGO_SINGLE_PASS only, an fp32 dQ accumulator of total_q*H*head_dim
 * floats (8 of them for FA_BWD_ALGO_SPLIT_REDUCE), and for the stored-dS form (FA_BWD_ALGO_STORED_DS,
 * or FA_BWD_ALGO_DEFAULT where it takes that form) its dS workspace. For FA_BWD_ALGO_DEFAULT and
 * FA_BWD_ALGO_RECOMPUTE_DQ it also fixes the kv-outer kernel's layout for runs
 * without and with a causal bound, from the descriptor (every sequence taken at
 * the maximum lengths) and the device's compute-unit count; planned runs use the
 * same layout. On success *out holds a new handle; on failure *out is set to NULL.
 * Host-side checks run before any HIP call. */
fa_bwd_status fa_bwd_create(const fa_bwd_desc* desc, fa_bwd_handle** out);

/* Enqueues the backward on `stream` (a hipStream_t; NULL = the default
 * stream) and returns without waiting. The caller synchronises its stream
 * before reading dq/dk/dv.
 *   q:          bf16 [total_q][H][head_dim]        (read only)
 *   o, dout:    bf16 [total_q][H][head_dim_v]      (read only)
 *   k:          bf16 [total_kv][H_kv][head_dim]    (read only; H_kv = num_heads_kv)
 *   v:          bf16 [total_kv][H_kv][head_dim_v]  (read only)
 *   m, l:       fp32 [total_q][H], row max of the scaled visible logits and
 *               the row sum of exp(scaled logit - m) over visible keys, as the
 *               forward produced them (not recomputed here; l > 0 on valid rows)
 *   cu_seqlens_q, cu_seqlens_kv: int32 [batch+1] device arrays (see above)
 *   scale:      the softmax scale applied to Q K^T (finite, > 0), e.g. 1/sqrt(head_dim)
 *   mask:       an fa_bwd_mask code
 *   dq:         bf16 [total_q][H][head_dim]       (written)
 *   dk:         bf16 [total_kv][H_kv][head_dim]   (written)
 *   dv:         bf16 [total_kv][H_kv][head_dim_v] (written)
 * Every argument is checked on the host first; an invalid one returns
 * FA_BWD_ERR_INVALID_ARGUMENT with nothing enqueued. FA_BWD_ERR_HIP reports a
 * failed launch. The handle's workspace is reused by every call, so one
 * handle must not be used by two calls that can overlap in time (two streams). */
fa_bwd_status fa_bwd_run(fa_bwd_handle* h, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* m, const float* l, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_kv, float scale, int32_t mask, void* dq, void* dk, void* dv,
                         void* stream);

/* The same backward with the softmax statistics as one log-sum-exp per row (the single statistic
 * the jax cuDNN wrapper keeps): lse = m + ln(l), fp32 [total_q][H], so that step 2 reads
 * P = exp(S*scale - lse). Every other argument, check and error as for fa_bwd_run; lse must not be
 * NULL and must be 4-byte aligned. */
fa_bwd_status fa_bwd_run_lse(fa_bwd_handle* h, const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_kv, float scale, int32_t mask, void* dq, void* dk, void* dv,
                             void* stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The backward of fa_bwd_run for the recompute form
 * (FA_BWD_ALGO_RECOMPUTE_DQ, _RECOMPUTE_DQ_8W, _RECOMPUTE_DQ_4W, _RECOMPUTE_DQ_64K: the same kernels,
 * the same layout rule and bitwise the same results as a handle created from `desc`; with
 * FA_BWD_ALGO_DEFAULT, those of a handle created with FA_BWD_ALGO_RECOMPUTE_DQ, since the stored-dS
 * form the default may take needs its dS workspace), without a handle
 * and without any allocation: the two fp32 [H][total_q] row-statistic arrays live in a fixed
 * device array of the library, 32 MiB, which every GPU the library runs on holds until the process
 * ends. The caller passes the descriptor and every input and output, with the meanings, layouts,
 * checks and errors of fa_bwd_create and fa_bwd_run (the dense grid: no host schedule, no
 * profiling). The first call on a device looks up that device's copy of the array (the caller
 * makes the device of `stream` current, as for any HIP call); no call allocates or frees memory.
 *   FA_BWD_ERR_SCRATCH_LIMIT: total_q * num_heads > FA_BWD_NOALLOC_MAX_ROWS (nothing enqueued).
 *   FA_BWD_ERR_UNSUPPORTED: the single-pass, split-reduce and stored-dS forms (their dQ or dS
 *     workspace is not part of the fixed array).
 * All calls on one GPU share its array: calls that can overlap in time on one GPU (two streams,
 * or a graph replayed beside a direct call) race on it and give wrong gradients. Each call rewrites
 * every row statistic it reads, so the array needs no clearing between calls. */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 22)
fa_bwd_status fa_bwd_run_noalloc(const fa_bwd_desc* desc, const void* q, const void* k, const void* v,
                                 const void* o, const void* dout, const float* m, const float* l,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, float scale,
                                 int32_t mask, void* dq, void* dk, void* dv, void* stream);

/* Forward that produces the backward's inputs, for callers without one of their own: enqueues on
 * `stream` O = softmax(scale * Q K^T, masked) V together with the row statistics the backward
 * consumes, for the sizes of the handle (its workspace is not used; FA_BWD_ALGO_* is ignored).
 * The softmax is the one step 2 of the SK-16 article inverts, P = exp(S*scale - m) / l.
 *   q:          bf16 [total_q][H][head_dim]   (read only)
 *   k:          bf16 [total_kv][H_kv][head_dim]  (read only)
 *   v:          bf16 [total_kv][H_kv][head_dim_v]  (read only)
 *   cu_seqlens_q, cu_seqlens_kv, scale, mask: as for fa_bwd_run
 *   o:          bf16 [total_q][H][head_dim_v] (written)
 *   m:          fp32 [total_q][H]  (written) row max of the scaled visible logits
 *   l:          fp32 [total_q][H]  (written) row sum of exp(scaled logit - m) over visible keys
 * Rows outside every sequence get O = 0, m = 0, l = 1; a row whose sequence has no keys gets the
 * same. Argument checks and errors as for fa_bwd_run (m, l need 4-byte, the rest 16-byte
 * alignment). With profiling enabled, the recorded row holds (fill of rows outside sequences,
 * forward kernel, 0). */
fa_bwd_status fa_fwd_run(fa_bwd_handle* h, const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_kv, float scale, int32_t mask, void* o, float* m, float* l,
                         void* stream);

/* Longest-first schedule from host copies of the sequence offsets (the SK-16 article lets its
 * control flow read actual_q / actual_kv on the host, section 三). Builds the list of work items
 * of the recompute-form kernels and of the forward, one per (tile, head, sequence) that holds rows
 * of a sequence, ordered by decreasing work (number of tile pairs it visits; ties in the dense
 * grid's order: tile, then sequence and head), and keeps it in device memory owned by the handle. Later fa_bwd_run,
 * fa_bwd_run_lse and fa_fwd_run calls whose mask equals `mask` launch one workgroup per item instead
 * of the dense grid of max_seqlen tiles x heads x sequences; calls with another mask use the dense
 * grid. The results are bitwise the same either way: only the launch order and the empty
 * workgroups change.
 *   cu_seqlens_q_host, cu_seqlens_kv_host: HOST int32 [batch+1], the values the device arrays of
 *     those later calls hold (the library cannot compare them; a mismatch gives wrong gradients).
 *     Checked here: cu[0] = 0, non-decreasing, every length <= its max_seqlen, and cu[batch] <=
 *     total (packed masks); otherwise FA_BWD_ERR_INVALID_ARGUMENT and the previous plan is kept.
 *   mask: the fa_bwd_mask code of the later calls (it sets the causal bound of the work counts).
 * Both arrays NULL: drop the plan. FA_BWD_ERR_UNSUPPORTED for a single-pass or split-reduce handle. Blocks until
 * the schedule is on the device; must not overlap a run that uses the handle. */
fa_bwd_status fa_bwd_plan(fa_bwd_handle* h, const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_kv_host,
                          int32_t mask);

/* Frees the workspace and the handle (NULL is accepted). Waits for the
 * device to finish work that may still use the workspace. */
fa_bwd_status fa_bwd_destroy(fa_bwd_handle* h);

/* Static English text for a status code. */
const char* fa_bwd_status_string(fa_bwd_status s);

/* Descriptor the handle was created with (for bindings); NULL on NULL. */
const fa_bwd_desc* fa_bwd_get_desc(const fa_bwd_handle* h);

/* Layout of the dK/dV kernel that fa_bwd_run takes on this handle under `mask`
 * (a causal mask, with or without padding, can select another layout than none
 * or padding), chosen when the handle was created from the descriptor and the
 * device's compute-unit count: FA_BWD_ALGO_RECOMPUTE_DQ_8W,
 * FA_BWD_ALGO_RECOMPUTE_DQ_4W or FA_BWD_ALGO_RECOMPUTE_DQ_64K for head dims up
 * to 128, and FA_BWD_ALGO_RECOMPUTE_DQ for wider heads (whose kernels have one
 * layout), whether or not the run stores dS (fa_bwd_dq_form).
 * Returns FA_BWD_ALGO_SINGLE_PASS or FA_BWD_ALGO_SPLIT_REDUCE for handles of
 * those forms, and -1 for a NULL handle or an invalid mask. Host only; does
 * not touch the device. */
int32_t fa_bwd_dkdv_layout(const fa_bwd_handle* h, int32_t mask);

/* How fa_bwd_run forms dQ on this handle under `mask`, fixed when the handle was
 * created: FA_BWD_ALGO_STORED_DS (the dK/dV kernel writes dS and a q-outer pass
 * forms dQ = scale * dS K) or FA_BWD_ALGO_RECOMPUTE_DQ (a q-outer kernel forms S
 * and dP again), as FA_BWD_ALGO_DEFAULT chooses by the rule stated with it or
 * the algorithm code forces; FA_BWD_ALGO_SINGLE_PASS or
 * FA_BWD_ALGO_SPLIT_REDUCE for handles of those forms; -1 for a NULL handle or
 * an invalid mask. Host only; does not touch the device. */
int32_t fa_bwd_dq_form(const fa_bwd_handle* h, int32_t mask);

/* Per-kernel timing for benchmarks. While enabled, every fa_bwd_run (and
 * fa_bwd_run_lse) also records four HIP events on its stream, around its three
 * kernels (row preprocessing; the main kernel in single-pass form or the dK/dV
 * kernel in recompute form; then the dQ cast, the split sum or the dQ kernel); an fa_fwd_run
 * records the fill of rows outside sequences, the forward kernel and an empty
 * third interval. Recording does not wait.
 * Enabling or disabling forgets the runs recorded so far. At most 4096 runs
 * are kept; later runs are not recorded. */
fa_bwd_status fa_bwd_profile_enable(fa_bwd_handle* h, int32_t enable);

/* Waits for the recorded runs, writes min(max_runs, recorded) rows of three
 * floats (milliseconds of the first, second and third kernels above) to the
 * HOST array ms, stores the row count in *n_runs, and forgets the runs. */
fa_bwd_status fa_bwd_profile_collect(fa_bwd_handle* h, float* ms, int32_t max_runs, int32_t* n_runs);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
