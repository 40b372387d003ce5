// Host-side integer work of the C ABI: zigzag partition, round-robin
// placement, error reporting and the device check.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstring>
#include <mutex>
#include <vector>

#include "cpa_internal.h"

namespace cpa {

static thread_local std::string g_last_error;

cpa_status fail(cpa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

cpa_status check_device() {
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CPA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(CPA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(CPA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    known[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    if (known[dev] < 0) return fail(CPA_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (known[dev] < 0) return fail(CPA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return CPA_OK;
}

cpa_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CPA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return CPA_OK;
}

}  // namespace cpa

using cpa::fail;

extern "C" const char* cpa_last_error(void) { return cpa::g_last_error.c_str(); }

// Zigzag split: 2*cp contiguous chunks per sequence (the first L mod 2cp one
// token longer), rank r owns chunk r and chunk 2cp-1-r, in ascending position.
extern "C" cpa_status cpa_cp_partition(int32_t num_seqs, const int32_t* seq_lens, int32_t cp_size,
                                       int32_t rank, int32_t* chunk_bounds, int32_t* cu_seqlens,
                                       int32_t* positions, int32_t* src_index, int64_t cap,
                                       int64_t* n_out) {
  if (!n_out) return fail(CPA_ERR_INVALID_ARG, "cpa_cp_partition: n_out is NULL");
  if (num_seqs < 0) return fail(CPA_ERR_INVALID_ARG, "cpa_cp_partition: num_seqs < 0");
  if (num_seqs > 0 && !seq_lens) return fail(CPA_ERR_INVALID_ARG, "cpa_cp_partition: seq_lens is NULL");
  if (cp_size < 1) return fail(CPA_ERR_INVALID_ARG, "cpa_cp_partition: cp_size %d < 1", cp_size);
  if (rank < 0 || rank >= cp_size)
    return fail(CPA_ERR_INVALID_ARG, "cpa_cp_partition: rank %d not in [0, %d)", rank, cp_size);
  const int64_t n = 2LL * cp_size;
  int64_t total = 0, all = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t L = seq_lens[b];
    if (L < 0) return fail(CPA_ERR_INVALID_ARG, "cpa_cp_partition: seq_lens[%d] = %lld < 0", b, (long long)L);
    const int64_t base = L / n, rem = L % n;
    const int64_t lo = rank, hi = n - 1 - rank;
    total += (base + (lo < rem)) + (base + (hi < rem));
    all += L;
  }
  if (all > INT32_MAX) return fail(CPA_ERR_INVALID_ARG, "cpa_cp_partition: total tokens exceed INT32_MAX");
  *n_out = total;
  if ((positions || src_index) && total > cap)
    return fail(CPA_ERR_CAPACITY, "cpa_cp_partition: need %lld output slots, cap is %lld", (long long)total,
                (long long)cap);
  int64_t out = 0, seq_start = 0;
  if (cu_seqlens && num_seqs >= 0) cu_seqlens[0] = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t L = seq_lens[b];
    const int64_t base = L / n, rem = L % n;
    // chunk c starts at c*base + min(c, rem)
    auto start = [&](int64_t c) { return c * base + (c < rem ? c : rem); };
    if (chunk_bounds)
      for (int64_t c = 0; c <= n; ++c) chunk_bounds[b * (n + 1) + c] = (int32_t)start(c);
    const int64_t own[2] = {rank, n - 1 - rank};
    for (int k = 0; k < 2; ++k) {
      const int64_t a = start(own[k]), e = start(own[k] + 1);
      for (int64_t p = a; p < e; ++p, ++out) {
        if (positions) positions[out] = (int32_t)p;
        if (src_index) src_index[out] = (int32_t)(seq_start + p);
      }
    }
    if (cu_seqlens) cu_seqlens[b + 1] = (int32_t)out;
    seq_start += L;
  }
  return CPA_OK;
}

// Round-robin placement with interleave I: position t lives on rank
// (t / I) mod cp at local slot (t / (I*cp))*I + t mod I.
extern "C" cpa_status cpa_rr_placement(int32_t num_seqs, const int32_t* seq_lens, int32_t cp_size,
                                       int32_t rank, int32_t interleave, int32_t* local_lens,
                                       int32_t* local_to_global, int64_t cap, int64_t* n_out) {
  if (!n_out) return fail(CPA_ERR_INVALID_ARG, "cpa_rr_placement: n_out is NULL");
  if (num_seqs < 0) return fail(CPA_ERR_INVALID_ARG, "cpa_rr_placement: num_seqs < 0");
  if (num_seqs > 0 && (!seq_lens || !local_lens))
    return fail(CPA_ERR_INVALID_ARG, "cpa_rr_placement: seq_lens or local_lens is NULL");
  if (cp_size < 1) return fail(CPA_ERR_INVALID_ARG, "cpa_rr_placement: cp_size %d < 1", cp_size);
  if (rank < 0 || rank >= cp_size)
    return fail(CPA_ERR_INVALID_ARG, "cpa_rr_placement: rank %d not in [0, %d)", rank, cp_size);
  if (interleave < 1) return fail(CPA_ERR_INVALID_ARG, "cpa_rr_placement: interleave %d < 1", interleave);
  int64_t total = 0, all = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (seq_lens[b] < 0) return fail(CPA_ERR_INVALID_ARG, "cpa_rr_placement: seq_lens[%d] < 0", b);
    total += cpa::rr_local_len(seq_lens[b], cp_size, rank, interleave);
    all += seq_lens[b];
  }
  if (all > INT32_MAX) return fail(CPA_ERR_INVALID_ARG, "cpa_rr_placement: total tokens exceed INT32_MAX");
  *n_out = total;
  if (local_to_global && total > cap)
    return fail(CPA_ERR_CAPACITY, "cpa_rr_placement: need %lld output slots, cap is %lld", (long long)total,
                (long long)cap);
  int64_t out = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t n = cpa::rr_local_len(seq_lens[b], cp_size, rank, interleave);
    local_lens[b] = (int32_t)n;
    if (local_to_global)
      for (int64_t l = 0; l < n; ++l, ++out)
        local_to_global[out] = (int32_t)(((l / interleave) * cp_size + rank) * interleave + l % interleave);
  }
  return CPA_OK;
}

// Exchanged-shard choice: bytes of K+V over the context against bytes of Q over
// the new tokens; pass KV iff strictly fewer.
extern "C" cpa_status cpa_choose_pass(int32_t num_seqs, const int32_t* q_lens, const int32_t* kv_lens, int32_t hq,
                                      int32_t hkv, int32_t d, int32_t elem_bytes, int32_t* pass_kv, int64_t* kv_bytes,
                                      int64_t* q_bytes) {
  const char* fn = "cpa_choose_pass";
  if (!pass_kv) return fail(CPA_ERR_INVALID_ARG, "%s: pass_kv is NULL", fn);
  if (num_seqs < 0 || (num_seqs > 0 && (!q_lens || !kv_lens)))
    return fail(CPA_ERR_INVALID_ARG, "%s: bad sequence arrays", fn);
  if (hq < 1 || hkv < 1 || d < 1 || elem_bytes < 1) return fail(CPA_ERR_INVALID_ARG, "%s: sizes must be >= 1", fn);
  __int128 t_q = 0, t_kv = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (q_lens[b] < 0 || kv_lens[b] < 0) return fail(CPA_ERR_INVALID_ARG, "%s: negative length", fn);
    t_q += q_lens[b];
    t_kv += kv_lens[b];
  }
  const __int128 kvb = t_kv * 2 * hkv * d * elem_bytes;
  const __int128 qb = t_q * hq * d * elem_bytes;
  const __int128 lim = INT64_MAX;
  if (kvb > lim || qb > lim) return fail(CPA_ERR_INVALID_ARG, "%s: byte totals overflow int64", fn);
  *pass_kv = kvb < qb ? 1 : 0;
  if (kv_bytes) *kv_bytes = (int64_t)kvb;
  if (q_bytes) *q_bytes = (int64_t)qb;
  return CPA_OK;
}

// Per-step cost of the two schemes: a step moves one rank's shard (1/cp of the
// byte totals) and computes 1/cp^2 of the batch's causal pairs.
extern "C" cpa_status cpa_pass_cost(int32_t num_seqs, const int32_t* q_lens, const int32_t* kv_lens, int32_t hq,
                                    int32_t hkv, int32_t d, int32_t elem_bytes, int32_t cp_size,
                                    double link_bytes_per_s, double mfma_flops_per_s, cpa_pass_cost_t* out) {
  const char* fn = "cpa_pass_cost";
  if (!out) return fail(CPA_ERR_INVALID_ARG, "%s: out is NULL", fn);
  if (cp_size < 1) return fail(CPA_ERR_INVALID_ARG, "%s: cp_size %d < 1", fn, cp_size);
  auto good_rate = [](double r) { return r > 0.0 && r <= 1.7e308; };  // also false for NaN
  if (!good_rate(link_bytes_per_s) || !good_rate(mfma_flops_per_s))
    return fail(CPA_ERR_INVALID_ARG, "%s: rates must be positive and finite", fn);
  int32_t pass_kv = 0;
  int64_t kvb = 0, qb = 0;
  cpa_status st = cpa_choose_pass(num_seqs, q_lens, kv_lens, hq, hkv, d, elem_bytes, &pass_kv, &kvb, &qb);
  if (st != CPA_OK) return st;
  __int128 pairs = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t ql = q_lens[b], kl = kv_lens[b];
    if (ql > kl) return fail(CPA_ERR_INVALID_ARG, "%s: q_lens[%d] > kv_lens[%d]", fn, b, b);
    // new token i sees (kl - ql) + i + 1 keys: sum over i < ql
    pairs += (__int128)ql * (kl - ql) + (__int128)ql * (ql + 1) / 2;
  }
  const __int128 flops = pairs * 4 * d * hq;
  if (flops > (__int128)INT64_MAX) return fail(CPA_ERR_INVALID_ARG, "%s: pair count overflows", fn);
  const double cp = (double)cp_size;
  out->pass_kv = pass_kv;
  out->kv_bytes = kvb;
  out->q_bytes = qb;
  out->pairs = (int64_t)pairs;
  out->kv_step_bytes = (double)kvb / cp;
  out->q_step_bytes = (double)qb / cp;
  out->step_flops = (double)(int64_t)flops / (cp * cp);
  out->kv_transfer_s = out->kv_step_bytes / link_bytes_per_s;
  out->q_transfer_s = out->q_step_bytes / link_bytes_per_s;
  out->step_compute_s = out->step_flops / mfma_flops_per_s;
  out->kv_hidden = out->kv_transfer_s <= out->step_compute_s ? 1 : 0;
  out->q_hidden = out->q_transfer_s <= out->step_compute_s ? 1 : 0;
  return CPA_OK;
}
