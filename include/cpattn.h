/*
 * cpattn.h — C ABI of libcpattn.so: partial causal GQA attention and exact
 * log-sum-exp (LSE) merge for context parallelism, on AMD MI355X (gfx950).
 *
 * What is computed comes from three vLLM pull-request pages:
 *   [PCP-GQA]  "[Feature] Support Prefill Context Parallel (PCP) for GQA flashinfer"
 *   [PASSKV]   "Add utility functions to enable pass-kv prefill and allgather decode"
 *   [PCP-BASE] "[Feature] Prefill Context Parallel (PCP) basic support"
 * Context parallelism (CP) shards a sequence over cp ranks. Attention is the
 * only sequence-coupled operation ([PASSKV], Purpose), so a rank's queries
 * attend to one KV shard at a time ("partial attention"), each step giving a
 * partial output O and its LSE, and the partials are merged exactly.
 *
 * Conventions (all entry points):
 *  - Every call returns cpa_status: 0 on success, a negative code on error.
 *    cpa_last_error() then returns a message (thread-local, valid until the
 *    next failing call on the same thread). No exception crosses the ABI.
 *  - Ownership: the caller allocates every buffer. Host calls read and write
 *    caller host arrays synchronously. Device calls take device pointers,
 *    validate every host-side argument before touching the GPU, enqueue their
 *    kernels on `stream` (a hipStream_t; NULL is the default stream) and
 *    return without synchronising. Errors the GPU could only report later
 *    (an out-of-range block-table entry, say) are not detected.
 *  - The library allocates no device memory. Scratch space, where a call
 *    needs any, is a caller-supplied workspace whose size is queried first.
 *  - Layouts are row-major and token-major:
 *      q, o      [T][hq][d]          k, v   [T][hkv][d]
 *      lse       [T][hq]             paged k/v cache [num_blocks][hkv][block_size][d]
 *    Query head h reads KV head h / (hq / hkv) (contiguous GQA groups).
 *  - LSE is the natural logarithm of the sum over visible keys of
 *    exp(scale * <q, k>). A row that sees no key has O = 0 and LSE = -inf.
 *  - Positions are global token positions within a sequence and must be
 *    non-decreasing within each sequence (zigzag shards and round-robin
 *    local orders are). The kernels use this to skip masked tiles.
 *  - Device calls run on gfx950 only; any other device gives
 *    CPA_ERR_UNSUPPORTED.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CPA_OK = 0,
  CPA_ERR_INVALID_ARG = -1, /* bad pointer, size, shape or enum value */
  CPA_ERR_UNSUPPORTED = -2, /* valid but not implemented (d, dtype, device) */
  CPA_ERR_CAPACITY = -3,    /* an output or workspace is too small */
  CPA_ERR_HIP = -4          /* the HIP runtime reported an error */
} cpa_status;

typedef enum { CPA_BF16 = 0, CPA_F32 = 1 } cpa_dtype;

/* CPA_MASK_CAUSAL: query i sees key j iff k_pos[j] <= q_pos[i] (global
 * positions). The offset-causal mask of chunked prefill is this mask with the
 * new queries' positions starting at the cached length.
 * CPA_MASK_NONE: every query sees every key of its sequence's shard. */
typedef enum { CPA_MASK_NONE = 0, CPA_MASK_CAUSAL = 1 } cpa_mask;

/* Message for the last failing call on this thread ("" if none). */
const char* cpa_last_error(void);

/* ---------------------------------------------------------------------------
 * cpa_cp_partition — the query/KV shard one CP rank holds at prefill (host).
 *
 * [PCP-GQA] and [PCP-BASE], Purpose: prefill CP partitions the sequence
 * dimension across ranks. Each sequence of length L is cut into 2*cp
 * contiguous chunks (sizes floor(L/2cp), the first L mod 2cp chunks one
 * larger) and rank r owns chunk r and chunk 2cp-1-r, the zigzag pairing that
 * gives every rank the same number of causal pairs when 2cp divides L.
 * A shard lists its tokens in ascending position; shards of a batch are
 * packed sequence after sequence.
 *
 * In:  num_seqs >= 0; seq_lens[num_seqs] >= 0 (host); cp_size >= 1;
 *      0 <= rank < cp_size.
 * Out (host arrays, caller-allocated):
 *      chunk_bounds [num_seqs][2*cp_size+1] chunk starts then L (may be NULL)
 *      cu_seqlens   [num_seqs+1]            shard offsets          (may be NULL)
 *      positions    [cap] global position of each shard token      (may be NULL)
 *      src_index    [cap] index of the token in the packed unsharded batch
 *                         (may be NULL)
 *      *n_out = total shard tokens (required, never NULL).
 * Size query: with positions == src_index == NULL, only *n_out (and the
 * non-NULL small arrays) are written. CPA_ERR_CAPACITY if n_out > cap while
 * positions or src_index is non-NULL; nothing is then written to them.
 * Errors: CPA_ERR_INVALID_ARG on NULL seq_lens with num_seqs > 0, negative
 * lengths, cp_size < 1, rank out of range, or totals above INT32_MAX.
 * ------------------------------------------------------------------------- */
cpa_status cpa_cp_partition(int32_t num_seqs, const int32_t* seq_lens, int32_t cp_size,
                            int32_t rank, int32_t* chunk_bounds, int32_t* cu_seqlens,
                            int32_t* positions, int32_t* src_index, int64_t cap,
                            int64_t* n_out);

/* ---------------------------------------------------------------------------
 * cpa_rr_placement — round-robin KV placement with an interleave size (host).
 *
 * [PASSKV], Purpose: for decode the KV cache is stored on the CP ranks in a
 * round-robin manner; [PCP-GQA], Test Plan, and [PCP-BASE], review summary:
 * the placement has an interleave size shared by prefill and decode CP.
 * Position t is stored on rank (t / I) mod cp at local slot
 * (t / (I*cp))*I + t mod I; positions [0, I) go to rank 0.
 *
 * In:  num_seqs >= 0; seq_lens[num_seqs] (host); cp_size >= 1;
 *      0 <= rank < cp_size; interleave I >= 1.
 * Out: local_lens[num_seqs] (required); local_to_global[cap] the global
 *      position of each local slot, packed sequence after sequence (may be
 *      NULL); *n_out = sum(local_lens) (required).
 * Errors: as cpa_cp_partition; CPA_ERR_INVALID_ARG also for interleave < 1.
 * ------------------------------------------------------------------------- */
cpa_status cpa_rr_placement(int32_t num_seqs, const int32_t* seq_lens, int32_t cp_size,
                            int32_t rank, int32_t interleave, int32_t* local_lens,
                            int32_t* local_to_global, int64_t cap, int64_t* n_out);

/* ---------------------------------------------------------------------------
 * cpa_choose_pass — pass KV or pass Q for a prefill batch (host).
 *
 * [PASSKV], Purpose: which shard to exchange follows the relative sizes of
 * the Q and KV tensors; full prefill passes KV because a KV head usually
 * serves more than two query heads, chunked prefill with a cache much longer
 * than the new tokens passes Q. The rule here compares the bytes each scheme
 * moves for the batch: K and V of every context token (2*hkv*d*elem_bytes
 * each) against Q of every new token (hq*d*elem_bytes each); pass KV iff
 * strictly fewer. With kv_lens == q_lens (full prefill) this is hq/hkv > 2.
 *
 * In:  num_seqs >= 0; q_lens[num_seqs] new tokens and kv_lens[num_seqs]
 *      context tokens (cached + new) per sequence, all >= 0 (host);
 *      hq, hkv, d, elem_bytes >= 1.
 * Out: *pass_kv = 1 (pass KV) or 0 (pass Q), required; *kv_bytes, *q_bytes
 *      the two totals (each may be NULL).
 * Errors: CPA_ERR_INVALID_ARG on NULL arrays with num_seqs > 0, negative
 *      lengths, sizes < 1, or totals above INT64_MAX.
 * ------------------------------------------------------------------------- */
cpa_status cpa_choose_pass(int32_t num_seqs, const int32_t* q_lens, const int32_t* kv_lens,
                           int32_t hq, int32_t hkv, int32_t d, int32_t elem_bytes,
                           int32_t* pass_kv, int64_t* kv_bytes, int64_t* q_bytes);

/* ---------------------------------------------------------------------------
 * cpa_pass_cost — per-step transfer and compute of the two exchange schemes
 * for a prefill batch (host).
 *
 * [PASSKV], Purpose: the shard to exchange follows the relative sizes of Q
 * and KV, and the partial attention of a step is the compute that hides the
 * transfer of the next shard. A rank's work is 1/cp of the batch's (the
 * zigzag and round-robin shards balance it) and one step is 1/cp of a rank's
 * work: step_flops = 4*d*hq*pairs / cp^2, where pairs counts the (new token,
 * context key) pairs of the causal mask (new token i of a sequence with c
 * cached tokens sees c + i + 1 keys). A step moves one rank's shard over one
 * link: kv_bytes / cp under pass-KV, q_bytes / cp under pass-Q (the byte
 * totals of cpa_choose_pass). A transfer is hidden when it takes no longer
 * than the step's compute at mfma_flops_per_s.
 *
 * In:  as cpa_choose_pass, plus cp_size >= 1 and the two rates (> 0, finite):
 *      link_bytes_per_s (one link, e.g. ~153e9 for one xGMI link) and
 *      mfma_flops_per_s (the partial-attention rate the caller achieves).
 *      q_lens[b] <= kv_lens[b].
 * Out: *out (required), every field written.
 * Errors: CPA_ERR_INVALID_ARG as cpa_choose_pass, and for cp_size < 1, a rate
 *      that is not a positive finite number, or q_lens[b] > kv_lens[b].
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t pass_kv;       /* the choice of cpa_choose_pass */
  int32_t kv_hidden;     /* pass-KV: a step's KV transfer fits under its compute */
  int32_t q_hidden;      /* pass-Q: a step's Q transfer fits under its compute */
  int64_t kv_bytes;      /* K+V bytes of the batch's context */
  int64_t q_bytes;       /* Q bytes of the batch's new tokens */
  int64_t pairs;         /* causal (new token, context key) pairs of the batch */
  double kv_step_bytes;  /* kv_bytes / cp */
  double q_step_bytes;   /* q_bytes / cp */
  double step_flops;     /* 4*d*hq*pairs / cp^2 */
  double kv_transfer_s;  /* kv_step_bytes / link_bytes_per_s */
  double q_transfer_s;   /* q_step_bytes / link_bytes_per_s */
  double step_compute_s; /* step_flops / mfma_flops_per_s */
} cpa_pass_cost_t;

cpa_status cpa_pass_cost(int32_t num_seqs, const int32_t* q_lens, const int32_t* kv_lens, int32_t hq,
                         int32_t hkv, int32_t d, int32_t elem_bytes, int32_t cp_size,
                         double link_bytes_per_s, double mfma_flops_per_s, cpa_pass_cost_t* out);

/* ---------------------------------------------------------------------------
 * cpa_partial_attn — one pass-KV step: a packed Q shard against one packed,
 * contiguous KV shard, giving partial O and LSE (device).
 *
 * [PASSKV], Purpose: Q and KV are both sharded at prefill; each step of the
 * exchange computes a partial attention of the local queries against one
 * KV shard, and the partials are merged (cpa_lse_merge).
 *
 * In (device pointers):
 *   q      [Tq][hq][d]   in_dtype          q_pos [Tq] int32, cu_q [num_seqs+1] int32
 *   k, v   [Tk][hkv][d]  in_dtype          k_pos [Tk] int32, cu_k [num_seqs+1] int32
 *   Sequence b's queries are rows cu_q[b]..cu_q[b+1]-1 and its keys rows
 *   cu_k[b]..cu_k[b+1]-1; q_pos and k_pos must be non-decreasing within a
 *   sequence.
 * In (host values): num_seqs >= 1; max_q >= max_b(cu_q[b+1]-cu_q[b]);
 *   hq % hkv == 0; d in {64, 128}; in_dtype CPA_BF16 or CPA_F32; scale > 0
 *   (normally 1/sqrt(d)); mask.
 * Out (device): o [Tq][hq][d] in o_dtype (CPA_F32, or CPA_BF16 when
 *   in_dtype is CPA_BF16); lse [Tq][hq] float.
 * The caller guarantees max_q; rows beyond it are not computed.
 * Errors: CPA_ERR_INVALID_ARG (NULL pointer, bad sizes), CPA_ERR_UNSUPPORTED
 *   (d, dtype combination, device), CPA_ERR_HIP (launch failure).
 * ------------------------------------------------------------------------- */
cpa_status cpa_partial_attn(const void* q, const int32_t* q_pos, const int32_t* cu_q,
                            const void* k, const void* v, const int32_t* k_pos,
                            const int32_t* cu_k, int32_t num_seqs, int32_t max_q, int32_t hq,
                            int32_t hkv, int32_t d, cpa_dtype in_dtype, float scale,
                            cpa_mask mask, void* o, cpa_dtype o_dtype, float* lse,
                            void* stream);

/* ---------------------------------------------------------------------------
 * cpa_partial_attn_multi — several pass-KV steps in one call: the same Q
 * shard against n_shards contiguous KV shards that are all resident, one
 * partial (O, LSE) per shard (device).
 *
 * [PASSKV], Purpose: the step partials of pass-KV prefill are independent
 * computations over disjoint key sets (they only meet in the merge); when the
 * shards are already resident they can run as one launch. With causal masks
 * over zigzag shards the work of a query tile differs by an order of
 * magnitude between tiles and shards; given a workspace, a small pre-pass
 * orders the launch heaviest tile first, which keeps its tail short (it also
 * records each tile's visible key-tile count there for the kernel). Each
 * shard's result is exactly what cpa_partial_attn returns for it, whatever
 * the order.
 *
 * In: n_shards in [1, 8]; k, v, k_pos, cu_k, o, lse are HOST arrays of
 *   n_shards DEVICE pointers with the meaning, layout and constraints of the
 *   corresponding cpa_partial_attn arguments (k_pos entries may be NULL
 *   under CPA_MASK_NONE); every other tensor argument is shared by all
 *   shards. workspace: device memory of workspace_bytes >= the size
 *   cpa_partial_attn_multi_workspace reports, overwritten by the call; it
 *   may be NULL (or too small, or the reported size 0), and then the tiles
 *   run in a fixed order (heaviest query tile of each sequence first).
 * Errors: as cpa_partial_attn; CPA_ERR_INVALID_ARG for n_shards out of range
 *   or a NULL pointer array / entry.
 * ------------------------------------------------------------------------- */
cpa_status cpa_partial_attn_multi_workspace(int32_t n_shards, int32_t num_seqs, int32_t max_q,
                                            size_t* bytes);
cpa_status cpa_partial_attn_multi(int32_t n_shards, const void* q, const int32_t* q_pos,
                                  const int32_t* cu_q, const void* const* k, const void* const* v,
                                  const int32_t* const* k_pos, const int32_t* const* cu_k,
                                  int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv,
                                  int32_t d, cpa_dtype in_dtype, float scale, cpa_mask mask,
                                  void* const* o, cpa_dtype o_dtype, float* const* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * cpa_partial_attn_multi_noalloc — cpa_partial_attn_multi for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same results, with the
 * launch-order workspace taken from a scratch array the library holds in each
 * GPU's memory (8192 tile units, 32 KiB) instead of a caller buffer. Calls no
 * allocating routine.
 *
 * In / out: as cpa_partial_attn_multi without workspace arguments.
 * Limit: cdiv(max_q, 128) * num_seqs * n_shards <= 8192 tile units;
 *   larger problems get CPA_ERR_CAPACITY (use cpa_partial_attn_multi).
 * Every call on one GPU shares that GPU's scratch array (the pre-pass rewrites
 * all of it that a call uses): calls that overlap on one GPU, on different
 * streams say, race and must be serialised by the caller.
 * Errors: as cpa_partial_attn_multi; CPA_ERR_CAPACITY as above; CPA_ERR_HIP if
 *   the scratch address cannot be obtained on the current device.
 * ------------------------------------------------------------------------- */
cpa_status cpa_partial_attn_multi_noalloc(int32_t n_shards, const void* q, const int32_t* q_pos,
                                          const int32_t* cu_q, const void* const* k,
                                          const void* const* v, const int32_t* const* k_pos,
                                          const int32_t* const* cu_k, int32_t num_seqs,
                                          int32_t max_q, int32_t hq, int32_t hkv, int32_t d,
                                          cpa_dtype in_dtype, float scale, cpa_mask mask,
                                          void* const* o, cpa_dtype o_dtype, float* const* lse,
                                          void* stream);

/* ---------------------------------------------------------------------------
 * cpa_partial_attn_merged — the merged result of the pass-KV steps over
 * n_shards resident contiguous KV shards, computed in one walk (device).
 *
 * [PASSKV], Purpose: a rank's queries attend to every KV shard in turn and
 * the step partials are merged exactly. The merge of disjoint key sets is the
 * softmax over their union, so one workgroup per query tile can walk the
 * visible keys of all shards with a single online softmax and write the
 * merged (O, LSE) directly: the same result as cpa_partial_attn_multi
 * followed by cpa_lse_merge (up to rounding order), without the fp32
 * partials or the separate merge pass.
 *
 * In: as cpa_partial_attn_multi (n_shards in [1, 8], host arrays of device
 *   pointers k, v, k_pos, cu_k; workspace as there, optional).
 * Out (device): o [Tq][hq][d] in o_dtype; lse [Tq][hq] float (natural log).
 * Supported: in_dtype CPA_BF16 with an even GQA group (hq / hkv); anything
 *   else is CPA_ERR_UNSUPPORTED (compute the partials and merge instead).
 * Errors: as cpa_partial_attn_multi.
 * ------------------------------------------------------------------------- */
cpa_status cpa_partial_attn_merged(int32_t n_shards, const void* q, const int32_t* q_pos,
                                   const int32_t* cu_q, const void* const* k, const void* const* v,
                                   const int32_t* const* k_pos, const int32_t* const* cu_k,
                                   int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv,
                                   int32_t d, cpa_dtype in_dtype, float scale, cpa_mask mask,
                                   void* o, cpa_dtype o_dtype, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * cpa_partial_attn_accumulate — one pass-KV step folded into a running merge
 * (device).
 *
 * [PASSKV], Purpose: in the pass-KV exchange a rank computes one partial per
 * arriving KV shard and the partials are merged exactly. This call computes
 * the partial of one contiguous KV shard (as cpa_partial_attn) and merges it
 * in its epilogue with the running (o_acc, lse_acc) of the earlier steps, in
 * place, by the rule of cpa_lse_merge; no partial is written.
 *
 * In: q ... mask as cpa_partial_attn (one shard). o_acc [Tq][hq][d] float and
 *   lse_acc [Tq][hq] float (device, read and written): the merge of the
 *   earlier steps; a row with lse_acc = -inf counts as empty and its o_acc
 *   values do not enter the result, whatever they are (start a ring with
 *   lse_acc = -inf, or with a cpa_partial_attn result in fp32). A row this
 *   step adds nothing to (no visible key) keeps its o_acc and lse_acc
 *   untouched. o_out (device, may be NULL) also receives the merged O
 *   in o_out_dtype (for the last step, say). workspace (device, optional):
 *   cpa_partial_attn_multi_workspace(1, num_seqs, max_q) bytes for the
 *   heaviest-first launch order, as in cpa_partial_attn_multi (NULL or short:
 *   index order, same results).
 * Supported: in_dtype CPA_BF16 with an even GQA group; anything else is
 *   CPA_ERR_UNSUPPORTED.
 * Errors: as cpa_partial_attn; CPA_ERR_INVALID_ARG for NULL o_acc / lse_acc.
 * ------------------------------------------------------------------------- */
cpa_status cpa_partial_attn_accumulate(const void* q, const int32_t* q_pos, const int32_t* cu_q,
                                       const void* k, const void* v, const int32_t* k_pos,
                                       const int32_t* cu_k, int32_t num_seqs, int32_t max_q,
                                       int32_t hq, int32_t hkv, int32_t d, cpa_dtype in_dtype,
                                       float scale, cpa_mask mask, float* o_acc, float* lse_acc,
                                       void* o_out, cpa_dtype o_out_dtype, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * cpa_partial_attn_paged_workspace — bytes of device workspace that
 * cpa_partial_attn_paged needs for these sizes (host, no GPU access).
 * Zero when no workspace is needed (max_q > 1).
 * ------------------------------------------------------------------------- */
cpa_status cpa_partial_attn_paged_workspace(int32_t num_seqs, int32_t max_q,
                                            int32_t max_blocks, int32_t block_size,
                                            int32_t hq, int32_t d, size_t* bytes);

/* ---------------------------------------------------------------------------
 * cpa_partial_attn_paged — partial attention against one rank's paged,
 * round-robin-placed KV shard (device).
 *
 * [PASSKV], Purpose: for chunked prefill, passing Q is preferred when the KV
 * cache is much longer than the new tokens, so every rank attends the visiting
 * queries to its resident KV; for decode, Q is all-gathered and each rank
 * attends to its round-robin share of the cache. [PCP-BASE], Purpose: the
 * KV-cache block tables are extended for CP. Local slot l of sequence b is
 * at physical block block_table[b][l / block_size], row l mod block_size,
 * and holds global position ((l / I)*cp_size + cp_rank)*I + l mod I.
 * max_q > 1 selects the prefill kernel (pass-Q, offset-causal mask);
 * max_q == 1 selects the split-KV decode kernel, which needs the workspace.
 *
 * In (device): q [Tq][hq][d], q_pos [Tq], cu_q [num_seqs+1] as in
 *   cpa_partial_attn; k_cache, v_cache [num_blocks][hkv][block_size][d];
 *   block_table [num_seqs][max_blocks] int32; local_kv_lens [num_seqs] int32
 *   with local_kv_lens[b] <= max_blocks*block_size.
 * In (host): block_size == 16; cp_size >= 1; 0 <= cp_rank < cp_size;
 *   interleave >= 1; d in {64, 128}; in_dtype CPA_BF16; hq % hkv == 0.
 * Out (device): o [Tq][hq][d] (o_dtype CPA_F32 or CPA_BF16), lse [Tq][hq].
 * workspace: device memory of at least the queried size (may be NULL when
 *   the query returned 0); contents on return are unspecified.
 * Errors: as cpa_partial_attn; CPA_ERR_CAPACITY if workspace_bytes is short.
 * ------------------------------------------------------------------------- */
cpa_status cpa_partial_attn_paged(const void* q, const int32_t* q_pos, const int32_t* cu_q,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* local_kv_lens, int32_t block_size,
                                  int32_t cp_size, int32_t cp_rank, int32_t interleave,
                                  int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv,
                                  int32_t d, cpa_dtype in_dtype, float scale, cpa_mask mask,
                                  void* o, cpa_dtype o_dtype, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * cpa_partial_attn_paged_merged — partial attention against this rank's
 * paged shard, merged in the same call with the other ranks' partials of the
 * same rows (device).
 *
 * [PASSKV], Purpose: in allgather decode every rank attends the gathered
 * decode queries to its round-robin share of the KV cache, and in pass-Q
 * chunked prefill the new queries visit every rank's resident cache; the
 * per-rank partials are merged exactly. Once the other ranks' partials are
 * resident (received), this call computes the rank's own partial as
 * cpa_partial_attn_paged does and folds the received ones into it by the rule
 * of cpa_lse_merge in the kernel that finishes it (the decode kernels' final
 * merge; the prefill kernel's epilogue), so no separate merge launch follows.
 *
 * In: every argument of cpa_partial_attn_paged (max_q > 1 needs an even GQA
 *   group, hq / hkv);
 *   n_parts in [0, 15]; o_parts and lse_parts are HOST arrays of n_parts
 *   DEVICE pointers: o_parts[j] [Tq][hq][d] in part_dtype (CPA_F32 or
 *   CPA_BF16), lse_parts[j] [Tq][hq] natural-log LSE, -inf for a row with no
 *   visible key (its O is then not read).
 * Out (device): o [Tq][hq][d] in o_dtype and lse [Tq][hq]: the exact merge of
 *   this rank's partial with the n_parts partials (O = 0, LSE = -inf where
 *   every part is empty); own_o [Tq][hq][d] in part_dtype and own_lse
 *   [Tq][hq] (each may be NULL): this rank's own partial, for the ranks that
 *   still need it. Rows of sequences without a query are not written.
 *   Outputs must not overlap the parts.
 * workspace: as cpa_partial_attn_paged (cpa_partial_attn_paged_workspace).
 * Errors: as cpa_partial_attn_paged; CPA_ERR_UNSUPPORTED for max_q > 1 with
 *   an odd GQA group; CPA_ERR_INVALID_ARG for n_parts out of range, NULL part
 *   arrays or pointers, or a bad part_dtype.
 * ------------------------------------------------------------------------- */
cpa_status cpa_partial_attn_paged_merged(const void* q, const int32_t* q_pos, const int32_t* cu_q,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, int32_t max_blocks,
                                         const int32_t* local_kv_lens, int32_t block_size,
                                         int32_t cp_size, int32_t cp_rank, int32_t interleave,
                                         int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv,
                                         int32_t d, cpa_dtype in_dtype, float scale, cpa_mask mask,
                                         int32_t n_parts, const void* const* o_parts,
                                         const float* const* lse_parts, cpa_dtype part_dtype,
                                         void* own_o, float* own_lse, void* o, cpa_dtype o_dtype,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* ---------------------------------------------------------------------------
 * cpa_lse_merge — exact n-way merge of partial (O, LSE) results (device).
 *
 * The partials come from disjoint key sets (the KV shards of the ranks), so
 * with M = max_s LSE_s, LSE = M + log sum_s exp(LSE_s - M) and
 * O = sum_s exp(LSE_s - LSE) O_s equals attention over the union of the key
 * sets ([PASSKV], Purpose: partial attention over exchanged shards). Rows
 * whose partials are all -inf give O = 0, LSE = -inf.
 *
 * In: n_parts in [1, 16]; o_parts and lse_parts are HOST arrays of n_parts
 *   DEVICE pointers: o_parts[s] [rows][d] in part_dtype, lse_parts[s]
 *   [rows] float; rows = tokens * hq >= 0; d in {64, 128}.
 * Out (device): o_out [rows][d] in out_dtype; lse_out [rows] (may be NULL).
 * Outputs may alias part 0 only when part_dtype == out_dtype.
 * ------------------------------------------------------------------------- */
cpa_status cpa_lse_merge(int32_t n_parts, const void* const* o_parts,
                         const float* const* lse_parts, cpa_dtype part_dtype, int64_t rows,
                         int32_t d, void* o_out, cpa_dtype out_dtype, float* lse_out,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
