// C-ABI entry points for partial attention: host-side validation, then
// dispatch to the fp32 kernel, the bf16 MFMA kernel (contiguous or paged
// prefill) or the split-KV decode kernels. Nothing here touches the GPU
// before every argument has been checked.
#include "cpa_internal.h"

using namespace cpa;

namespace {

cpa_status check_common(const char* fn, const void* q, const int32_t* q_pos, const int32_t* cu_q, const void* k,
                        const void* v, int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv, int32_t d,
                        float scale, int mask, const void* o, const float* lse) {
  if (num_seqs < 0) return fail(CPA_ERR_INVALID_ARG, "%s: num_seqs < 0", fn);
  if (max_q < 0) return fail(CPA_ERR_INVALID_ARG, "%s: max_q < 0", fn);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(CPA_ERR_INVALID_ARG, "%s: need hq, hkv >= 1 and hq %% hkv == 0 (hq=%d, hkv=%d)", fn, hq, hkv);
  if (d != 64 && d != 128) return fail(CPA_ERR_UNSUPPORTED, "%s: d = %d (supported: 64, 128)", fn, d);
  if (!(scale > 0.f) || scale != scale || scale > 1e30f) return fail(CPA_ERR_INVALID_ARG, "%s: bad scale", fn);
  if (mask != CPA_MASK_NONE && mask != CPA_MASK_CAUSAL) return fail(CPA_ERR_INVALID_ARG, "%s: bad mask", fn);
  if (num_seqs > 0 && max_q > 0) {
    if (!q || !cu_q || !k || !v || !o || !lse) return fail(CPA_ERR_INVALID_ARG, "%s: NULL tensor pointer", fn);
    if (mask == CPA_MASK_CAUSAL && !q_pos) return fail(CPA_ERR_INVALID_ARG, "%s: q_pos is NULL", fn);
  }
  return CPA_OK;
}

}  // namespace

extern "C" cpa_status cpa_partial_attn(const void* q, const int32_t* q_pos, const int32_t* cu_q, const void* k,
                                       const void* v, const int32_t* k_pos, const int32_t* cu_k, int32_t num_seqs,
                                       int32_t max_q, int32_t hq, int32_t hkv, int32_t d, cpa_dtype in_dtype,
                                       float scale, cpa_mask mask, void* o, cpa_dtype o_dtype, float* lse,
                                       void* stream) {
  const char* fn = "cpa_partial_attn";
  cpa_status st = check_common(fn, q, q_pos, cu_q, k, v, num_seqs, max_q, hq, hkv, d, scale, mask, o, lse);
  if (st != CPA_OK) return st;
  if (in_dtype != CPA_BF16 && in_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad in_dtype", fn);
  if (o_dtype != CPA_BF16 && o_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad o_dtype", fn);
  if (in_dtype == CPA_F32 && o_dtype != CPA_F32)
    return fail(CPA_ERR_UNSUPPORTED, "%s: fp32 inputs need an fp32 output", fn);
  if (num_seqs > 0 && max_q > 0) {
    if (!cu_k) return fail(CPA_ERR_INVALID_ARG, "%s: cu_k is NULL", fn);
    if (mask == CPA_MASK_CAUSAL && !k_pos) return fail(CPA_ERR_INVALID_ARG, "%s: k_pos is NULL", fn);
  }
  st = check_device();
  if (st != CPA_OK) return st;
  if (num_seqs == 0 || max_q == 0) return CPA_OK;
  AttnArgs a;
  a.q = q;
  a.q_pos = q_pos;
  a.cu_q = cu_q;
  a.k = k;
  a.v = v;
  a.k_pos = k_pos;
  a.cu_k = cu_k;
  a.num_seqs = num_seqs;
  a.max_q = max_q;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.scale = scale;
  a.causal = mask == CPA_MASK_CAUSAL;
  a.o = o;
  a.o_bf16 = o_dtype == CPA_BF16;
  a.lse = lse;
  hipStream_t s = (hipStream_t)stream;
  if (in_dtype == CPA_F32) return launch_attn_f32(a, s);
  return attn_pp_supported(a) ? launch_attn_pp(&a, 1, /*paged=*/false, s) : launch_attn_mfma(a, /*paged=*/false, s);
}

extern "C" cpa_status cpa_partial_attn_multi_workspace(int32_t n_shards, int32_t num_seqs, int32_t max_q,
                                                       size_t* bytes) {
  if (!bytes) return fail(CPA_ERR_INVALID_ARG, "cpa_partial_attn_multi_workspace: bytes is NULL");
  if (n_shards < 1 || n_shards > kMaxShards || num_seqs < 0 || max_q < 0)
    return fail(CPA_ERR_INVALID_ARG, "cpa_partial_attn_multi_workspace: bad sizes");
  *bytes = attn_pp_order_bytes(n_shards, num_seqs, max_q);
  return CPA_OK;
}

namespace {

// Validation and argument setup shared by the batched pass-KV calls.
cpa_status prepare_multi(const char* fn, int32_t n_shards, const void* q, const int32_t* q_pos, const int32_t* cu_q,
                         const void* const* k, const void* const* v, const int32_t* const* k_pos,
                         const int32_t* const* cu_k, int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv,
                         int32_t d, cpa_dtype in_dtype, float scale, cpa_mask mask, void* const* o,
                         cpa_dtype o_dtype, float* const* lse, AttnArgs* args) {
  if (n_shards < 1 || n_shards > kMaxShards)
    return fail(CPA_ERR_INVALID_ARG, "%s: n_shards %d not in [1, %d]", fn, n_shards, kMaxShards);
  if (!k || !v || !cu_k || !o || !lse || (mask == CPA_MASK_CAUSAL && !k_pos))
    return fail(CPA_ERR_INVALID_ARG, "%s: NULL pointer array", fn);
  if (in_dtype != CPA_BF16 && in_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad in_dtype", fn);
  if (o_dtype != CPA_BF16 && o_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad o_dtype", fn);
  if (in_dtype == CPA_F32 && o_dtype != CPA_F32)
    return fail(CPA_ERR_UNSUPPORTED, "%s: fp32 inputs need an fp32 output", fn);
  for (int i = 0; i < n_shards; ++i) {
    const int32_t* kp = (mask == CPA_MASK_CAUSAL) ? k_pos[i] : nullptr;
    cpa_status st = check_common(fn, q, q_pos, cu_q, k[i], v[i], num_seqs, max_q, hq, hkv, d, scale, mask, o[i], lse[i]);
    if (st != CPA_OK) return st;
    if (num_seqs > 0 && max_q > 0) {
      if (!cu_k[i]) return fail(CPA_ERR_INVALID_ARG, "%s: cu_k[%d] is NULL", fn, i);
      if (mask == CPA_MASK_CAUSAL && !kp) return fail(CPA_ERR_INVALID_ARG, "%s: k_pos[%d] is NULL", fn, i);
    }
    AttnArgs& a = args[i];
    a.q = q;
    a.q_pos = q_pos;
    a.cu_q = cu_q;
    a.k = k[i];
    a.v = v[i];
    a.k_pos = kp;
    a.cu_k = cu_k[i];
    a.num_seqs = num_seqs;
    a.max_q = max_q;
    a.hq = hq;
    a.hkv = hkv;
    a.d = d;
    a.scale = scale;
    a.causal = mask == CPA_MASK_CAUSAL;
    a.o = o[i];
    a.o_bf16 = o_dtype == CPA_BF16;
    a.lse = lse[i];
  }
  return CPA_OK;
}

// The batched launch: one launch over every shard (bf16, even GQA group), or
// one launch per shard otherwise.
cpa_status run_multi(const AttnArgs* args, int32_t n_shards, cpa_dtype in_dtype, void* order_ws,
                     size_t order_ws_bytes, hipStream_t s) {
  if (in_dtype == CPA_BF16 && attn_pp_supported(args[0]))
    return launch_attn_pp(args, n_shards, /*paged=*/false, s, order_ws, order_ws_bytes);
  for (int i = 0; i < n_shards; ++i) {
    const cpa_status st =
        (in_dtype == CPA_F32) ? launch_attn_f32(args[i], s) : launch_attn_mfma(args[i], /*paged=*/false, s);
    if (st != CPA_OK) return st;
  }
  return CPA_OK;
}

}  // namespace

extern "C" cpa_status cpa_partial_attn_multi(int32_t n_shards, const void* q, const int32_t* q_pos,
                                             const int32_t* cu_q, const void* const* k, const void* const* v,
                                             const int32_t* const* k_pos, const int32_t* const* cu_k,
                                             int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv, int32_t d,
                                             cpa_dtype in_dtype, float scale, cpa_mask mask, void* const* o,
                                             cpa_dtype o_dtype, float* const* lse, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  AttnArgs args[kMaxShards];
  cpa_status st = prepare_multi("cpa_partial_attn_multi", n_shards, q, q_pos, cu_q, k, v, k_pos, cu_k, num_seqs,
                                max_q, hq, hkv, d, in_dtype, scale, mask, o, o_dtype, lse, args);
  if (st != CPA_OK) return st;
  st = check_device();
  if (st != CPA_OK) return st;
  if (num_seqs == 0 || max_q == 0) return CPA_OK;
  return run_multi(args, n_shards, in_dtype, workspace, workspace_bytes, (hipStream_t)stream);
}

extern "C" cpa_status cpa_partial_attn_multi_noalloc(int32_t n_shards, const void* q, const int32_t* q_pos,
                                                     const int32_t* cu_q, const void* const* k, const void* const* v,
                                                     const int32_t* const* k_pos, const int32_t* const* cu_k,
                                                     int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv,
                                                     int32_t d, cpa_dtype in_dtype, float scale, cpa_mask mask,
                                                     void* const* o, cpa_dtype o_dtype, float* const* lse,
                                                     void* stream) {
  const char* fn = "cpa_partial_attn_multi_noalloc";
  AttnArgs args[kMaxShards];
  cpa_status st = prepare_multi(fn, n_shards, q, q_pos, cu_q, k, v, k_pos, cu_k, num_seqs, max_q, hq, hkv, d,
                                in_dtype, scale, mask, o, o_dtype, lse, args);
  if (st != CPA_OK) return st;
  const int64_t units = attn_pp_tile_units(n_shards, num_seqs, max_q);
  if (units > attn_pp_scratch_units())
    return fail(CPA_ERR_CAPACITY, "%s: %lld tile units (query tiles x sequences x shards); at most %d fit the "
                "library's launch-order scratch", fn, (long long)units, attn_pp_scratch_units());
  st = check_device();
  if (st != CPA_OK) return st;
  if (num_seqs == 0 || max_q == 0) return CPA_OK;
  void* scratch_ptr = nullptr;
  size_t scratch_bytes = 0;
  st = attn_pp_scratch(&scratch_ptr, &scratch_bytes);
  if (st != CPA_OK) return st;
  return run_multi(args, n_shards, in_dtype, scratch_ptr, scratch_bytes, (hipStream_t)stream);
}

extern "C" cpa_status cpa_partial_attn_merged(int32_t n_shards, const void* q, const int32_t* q_pos,
                                              const int32_t* cu_q, const void* const* k, const void* const* v,
                                              const int32_t* const* k_pos, const int32_t* const* cu_k,
                                              int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv, int32_t d,
                                              cpa_dtype in_dtype, float scale, cpa_mask mask, void* o,
                                              cpa_dtype o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                                              void* stream) {
  const char* fn = "cpa_partial_attn_merged";
  if (n_shards < 1 || n_shards > kMaxShards)
    return fail(CPA_ERR_INVALID_ARG, "%s: n_shards %d not in [1, %d]", fn, n_shards, kMaxShards);
  if (!k || !v || !cu_k || (mask == CPA_MASK_CAUSAL && !k_pos))
    return fail(CPA_ERR_INVALID_ARG, "%s: NULL pointer array", fn);
  if (in_dtype != CPA_BF16 && in_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad in_dtype", fn);
  if (o_dtype != CPA_BF16 && o_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad o_dtype", fn);
  AttnArgs args[kMaxShards];
  for (int i = 0; i < n_shards; ++i) {
    const int32_t* kp = (mask == CPA_MASK_CAUSAL) ? k_pos[i] : nullptr;
    cpa_status st = check_common(fn, q, q_pos, cu_q, k[i], v[i], num_seqs, max_q, hq, hkv, d, scale, mask, o, lse);
    if (st != CPA_OK) return st;
    if (num_seqs > 0 && max_q > 0) {
      if (!cu_k[i]) return fail(CPA_ERR_INVALID_ARG, "%s: cu_k[%d] is NULL", fn, i);
      if (mask == CPA_MASK_CAUSAL && !kp) return fail(CPA_ERR_INVALID_ARG, "%s: k_pos[%d] is NULL", fn, i);
    }
    AttnArgs& a = args[i];
    a.q = q;
    a.q_pos = q_pos;
    a.cu_q = cu_q;
    a.k = k[i];
    a.v = v[i];
    a.k_pos = kp;
    a.cu_k = cu_k[i];
    a.num_seqs = num_seqs;
    a.max_q = max_q;
    a.hq = hq;
    a.hkv = hkv;
    a.d = d;
    a.scale = scale;
    a.causal = mask == CPA_MASK_CAUSAL;
    a.o = o;
    a.o_bf16 = o_dtype == CPA_BF16;
    a.lse = lse;
  }
  if (in_dtype != CPA_BF16 || !attn_pp_supported(args[0]))
    return fail(CPA_ERR_UNSUPPORTED, "%s: needs bf16 inputs and an even GQA group (hq / hkv)", fn);
  cpa_status st = check_device();
  if (st != CPA_OK) return st;
  if (num_seqs == 0 || max_q == 0) return CPA_OK;
  const MergedOut out{o, o_dtype == CPA_BF16, lse};
  return launch_attn_pp(args, n_shards, /*paged=*/false, (hipStream_t)stream, workspace, workspace_bytes, &out);
}

extern "C" cpa_status cpa_partial_attn_accumulate(const void* q, const int32_t* q_pos, const int32_t* cu_q,
                                                  const void* k, const void* v, const int32_t* k_pos,
                                                  const int32_t* cu_k, int32_t num_seqs, int32_t max_q, int32_t hq,
                                                  int32_t hkv, int32_t d, cpa_dtype in_dtype, float scale,
                                                  cpa_mask mask, float* o_acc, float* lse_acc, void* o_out,
                                                  cpa_dtype o_out_dtype, void* workspace, size_t workspace_bytes,
                                                  void* stream) {
  const char* fn = "cpa_partial_attn_accumulate";
  if (in_dtype != CPA_BF16 && in_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad in_dtype", fn);
  if (o_out_dtype != CPA_BF16 && o_out_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad o_out_dtype", fn);
  cpa_status st = check_common(fn, q, q_pos, cu_q, k, v, num_seqs, max_q, hq, hkv, d, scale, mask, o_acc, lse_acc);
  if (st != CPA_OK) return st;
  if (num_seqs > 0 && max_q > 0) {
    if (!cu_k) return fail(CPA_ERR_INVALID_ARG, "%s: cu_k is NULL", fn);
    if (mask == CPA_MASK_CAUSAL && !k_pos) return fail(CPA_ERR_INVALID_ARG, "%s: k_pos is NULL", fn);
  }
  AttnArgs a{};
  a.q = q;
  a.q_pos = q_pos;
  a.cu_q = cu_q;
  a.k = k;
  a.v = v;
  a.k_pos = mask == CPA_MASK_CAUSAL ? k_pos : nullptr;
  a.cu_k = cu_k;
  a.num_seqs = num_seqs;
  a.max_q = max_q;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.scale = scale;
  a.causal = mask == CPA_MASK_CAUSAL;
  a.o = o_out;
  a.o_bf16 = o_out_dtype == CPA_BF16;
  a.lse = lse_acc;
  if (in_dtype != CPA_BF16 || !attn_pp_supported(a))
    return fail(CPA_ERR_UNSUPPORTED, "%s: needs bf16 inputs and an even GQA group (hq / hkv)", fn);
  st = check_device();
  if (st != CPA_OK) return st;
  if (num_seqs == 0 || max_q == 0) return CPA_OK;
  const AccumIO io{o_acc, lse_acc, o_out};
  return launch_attn_pp(&a, 1, /*paged=*/false, (hipStream_t)stream, workspace, workspace_bytes, nullptr, &io);
}

extern "C" cpa_status cpa_partial_attn_paged_workspace(int32_t num_seqs, int32_t max_q, int32_t max_blocks,
                                                       int32_t block_size, int32_t hq, int32_t d, size_t* bytes) {
  const char* fn = "cpa_partial_attn_paged_workspace";
  if (!bytes) return fail(CPA_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  if (num_seqs < 0 || max_q < 0 || max_blocks < 0 || hq < 1)
    return fail(CPA_ERR_INVALID_ARG, "%s: negative size or hq < 1", fn);
  if (block_size != 16) return fail(CPA_ERR_UNSUPPORTED, "%s: block_size %d (supported: 16)", fn, block_size);
  if (d != 64 && d != 128) return fail(CPA_ERR_UNSUPPORTED, "%s: d = %d (supported: 64, 128)", fn, d);
  *bytes = (max_q == 1) ? decode_workspace_bytes(num_seqs, max_blocks, block_size, hq, d) : 0;
  return CPA_OK;
}

// Checks of the paged entry points and their arguments; num_seqs == 0 or
// max_q == 0 leaves *empty true (nothing to launch).
static cpa_status prepare_paged(const char* fn, const void* q, const int32_t* q_pos, const int32_t* cu_q,
                                const void* k_cache, const void* v_cache, const int32_t* block_table,
                                int32_t max_blocks, const int32_t* local_kv_lens, int32_t block_size,
                                int32_t cp_size, int32_t cp_rank, int32_t interleave, int32_t num_seqs,
                                int32_t max_q, int32_t hq, int32_t hkv, int32_t d, cpa_dtype in_dtype, float scale,
                                cpa_mask mask, void* o, cpa_dtype o_dtype, float* lse, void* workspace,
                                size_t workspace_bytes, AttnArgs* a, bool* empty) {
  *empty = true;
  cpa_status st =
      check_common(fn, q, q_pos, cu_q, k_cache, v_cache, num_seqs, max_q, hq, hkv, d, scale, mask, o, lse);
  if (st != CPA_OK) return st;
  if (in_dtype != CPA_BF16) return fail(CPA_ERR_UNSUPPORTED, "%s: only bf16 caches are supported", fn);
  if (o_dtype != CPA_BF16 && o_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad o_dtype", fn);
  if (block_size != 16) return fail(CPA_ERR_UNSUPPORTED, "%s: block_size %d (supported: 16)", fn, block_size);
  if (cp_size < 1 || cp_rank < 0 || cp_rank >= cp_size)
    return fail(CPA_ERR_INVALID_ARG, "%s: need 0 <= cp_rank < cp_size (got %d, %d)", fn, cp_rank, cp_size);
  if (interleave < 1) return fail(CPA_ERR_INVALID_ARG, "%s: interleave %d < 1", fn, interleave);
  if ((int64_t)interleave * cp_size > INT32_MAX / 2)
    return fail(CPA_ERR_INVALID_ARG, "%s: interleave * cp_size too large", fn);
  if (max_blocks < 0) return fail(CPA_ERR_INVALID_ARG, "%s: max_blocks < 0", fn);
  if (num_seqs > 0 && max_q > 0 && (!block_table || !local_kv_lens) && max_blocks > 0)
    return fail(CPA_ERR_INVALID_ARG, "%s: block_table or local_kv_lens is NULL", fn);
  if (num_seqs > 0 && max_q > 0 && !local_kv_lens)
    return fail(CPA_ERR_INVALID_ARG, "%s: local_kv_lens is NULL", fn);
  if (max_q == 1) {
    const size_t need = decode_workspace_bytes(num_seqs, max_blocks, block_size, hq, d);
    if (workspace_bytes < need)
      return fail(CPA_ERR_CAPACITY, "%s: workspace has %zu bytes, decode needs %zu", fn, workspace_bytes, need);
    if (need > 0 && !workspace) return fail(CPA_ERR_INVALID_ARG, "%s: workspace is NULL", fn);
  }
  st = check_device();
  if (st != CPA_OK) return st;
  if (num_seqs == 0 || max_q == 0) return CPA_OK;
  *empty = false;
  a->q = q;
  a->q_pos = q_pos;
  a->cu_q = cu_q;
  a->k = k_cache;
  a->v = v_cache;
  a->block_table = block_table;
  a->max_blocks = max_blocks;
  a->local_kv_lens = local_kv_lens;
  a->cp = cp_size;
  a->rank = cp_rank;
  a->interleave = interleave;
  a->num_seqs = num_seqs;
  a->max_q = max_q;
  a->hq = hq;
  a->hkv = hkv;
  a->d = d;
  a->scale = scale;
  a->causal = mask == CPA_MASK_CAUSAL;
  a->o = o;
  a->o_bf16 = o_dtype == CPA_BF16;
  a->lse = lse;
  a->workspace = workspace;
  a->workspace_bytes = workspace_bytes;
  return CPA_OK;
}

extern "C" cpa_status cpa_partial_attn_paged(const void* q, const int32_t* q_pos, const int32_t* cu_q,
                                             const void* k_cache, const void* v_cache, const int32_t* block_table,
                                             int32_t max_blocks, const int32_t* local_kv_lens, int32_t block_size,
                                             int32_t cp_size, int32_t cp_rank, int32_t interleave, int32_t num_seqs,
                                             int32_t max_q, int32_t hq, int32_t hkv, int32_t d, cpa_dtype in_dtype,
                                             float scale, cpa_mask mask, void* o, cpa_dtype o_dtype, float* lse,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  AttnArgs a;
  bool empty;
  cpa_status st = prepare_paged("cpa_partial_attn_paged", q, q_pos, cu_q, k_cache, v_cache, block_table, max_blocks,
                                local_kv_lens, block_size, cp_size, cp_rank, interleave, num_seqs, max_q, hq, hkv,
                                d, in_dtype, scale, mask, o, o_dtype, lse, workspace, workspace_bytes, &a, &empty);
  if (st != CPA_OK || empty) return st;
  hipStream_t s = (hipStream_t)stream;
  if (max_q == 1) return launch_attn_decode(a, s);
  return attn_pp_supported(a) ? launch_attn_pp(&a, 1, /*paged=*/true, s) : launch_attn_mfma(a, /*paged=*/true, s);
}

extern "C" cpa_status cpa_partial_attn_paged_merged(
    const void* q, const int32_t* q_pos, const int32_t* cu_q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, int32_t max_blocks, const int32_t* local_kv_lens, int32_t block_size,
    int32_t cp_size, int32_t cp_rank, int32_t interleave, int32_t num_seqs, int32_t max_q, int32_t hq, int32_t hkv,
    int32_t d, cpa_dtype in_dtype, float scale, cpa_mask mask, int32_t n_parts, const void* const* o_parts,
    const float* const* lse_parts, cpa_dtype part_dtype, void* own_o, float* own_lse, void* o, cpa_dtype o_dtype,
    float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "cpa_partial_attn_paged_merged";
  if (n_parts < 0 || n_parts > kMaxFoldParts)
    return fail(CPA_ERR_INVALID_ARG, "%s: n_parts %d not in [0, %d]", fn, n_parts, kMaxFoldParts);
  if (n_parts > 0 && (!o_parts || !lse_parts)) return fail(CPA_ERR_INVALID_ARG, "%s: part arrays are NULL", fn);
  if (part_dtype != CPA_BF16 && part_dtype != CPA_F32) return fail(CPA_ERR_INVALID_ARG, "%s: bad part_dtype", fn);
  AttnArgs a;
  bool empty;
  cpa_status st = prepare_paged(fn, q, q_pos, cu_q, k_cache, v_cache, block_table, max_blocks, local_kv_lens,
                                block_size, cp_size, cp_rank, interleave, num_seqs, max_q, hq, hkv, d, in_dtype,
                                scale, mask, o, o_dtype, lse, workspace, workspace_bytes, &a, &empty);
  if (st != CPA_OK || empty) return st;
  RankFold f{};
  f.n = n_parts;
  for (int j = 0; j < n_parts; ++j) {
    if (!o_parts[j] || !lse_parts[j]) return fail(CPA_ERR_INVALID_ARG, "%s: part %d pointer is NULL", fn, j);
    f.o[j] = o_parts[j];
    f.lse[j] = lse_parts[j];
  }
  f.part_bf16 = part_dtype == CPA_BF16;
  f.own_o = own_o;
  f.own_lse = own_lse;
  if (max_q == 1) return launch_attn_decode(a, (hipStream_t)stream, &f);
  if (!attn_pp_supported(a))
    return fail(CPA_ERR_UNSUPPORTED, "%s: prefill (max_q > 1) needs an even GQA group (hq / hkv)", fn);
  return launch_attn_pp(&a, 1, /*paged=*/true, (hipStream_t)stream, nullptr, 0, nullptr, nullptr, &f);
}
