// Exact n-way merge of partial attention results (O_s, LSE_s) computed over
// disjoint key sets: LSE = M + log sum_s exp(LSE_s - M), M = max_s LSE_s, and
// O = sum_s exp(LSE_s - LSE) O_s. This is how partial attentions over the
// exchanged KV shards of context parallelism combine into full attention
// ("Add utility functions to enable pass-kv prefill and allgather decode",
// Purpose).
//
// HBM-bound: every byte of every partial is read once and the result written
// once. One thread owns two groups of 4 elements of a row, half a row apart,
// issues all of its loads before any arithmetic, and the LSE arithmetic is
// done in base 2 on
// v_exp_f32 / v_log_f32. Two and four parts (the common CP sizes) have their
// own instantiations so the registers are sized for them.
#include "cpa_internal.h"
#include "device_common.h"

namespace cpa {

constexpr int kMaxParts = 16;

struct MergeParts {
  const void* o[kMaxParts];
  const float* lse[kMaxParts];
};

// NP > 0: exactly NP parts (compile time, registers sized for them); NP == 0:
// n_parts at run time, up to kMaxParts. Each thread owns two groups of 4
// elements of a row, half a row apart, so that every part adds two loads to
// the thread's loads in flight while each load instruction of a wave still
// reads one contiguous span.
template <int D, int NP, bool PART_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeParts parts, int n_parts, int64_t rows,
                                                        void* __restrict__ o_out, float* __restrict__ lse_out) {
  constexpr int kThreadsPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kThreadsPerRow;
  constexpr int kP = NP > 0 ? NP : kMaxParts;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  const int c = threadIdx.x % kThreadsPerRow;
  if (row >= rows) return;
  const int np = NP > 0 ? NP : n_parts;
  const int64_t elem = row * D + c * 4;  // and elem + D / 2

  float l2[kP];
  f32x4 xa[kP], xb[kP];
#pragma unroll
  for (int s = 0; s < kP; ++s) {
    if (s < np) {
      l2[s] = parts.lse[s][row] * kLog2e;
      if constexpr (PART_BF16) {
        const u32x2 wa = __builtin_nontemporal_load((const u32x2*)((const uint16_t*)parts.o[s] + elem));
        const u32x2 wb = __builtin_nontemporal_load((const u32x2*)((const uint16_t*)parts.o[s] + elem + D / 2));
        xa[s] = f32x4{bf16_lo(wa[0]), bf16_hi(wa[0]), bf16_lo(wa[1]), bf16_hi(wa[1])};
        xb[s] = f32x4{bf16_lo(wb[0]), bf16_hi(wb[0]), bf16_lo(wb[1]), bf16_hi(wb[1])};
      } else {
        xa[s] = __builtin_nontemporal_load((const f32x4*)((const float*)parts.o[s] + elem));
        xb[s] = __builtin_nontemporal_load((const f32x4*)((const float*)parts.o[s] + elem + D / 2));
      }
    }
  }
  float m = kNegInf;
#pragma unroll
  for (int s = 0; s < kP; ++s)
    if (s < np) m = fmaxf(m, l2[s]);
  f32x4 acc_a = {0.f, 0.f, 0.f, 0.f}, acc_b = {0.f, 0.f, 0.f, 0.f};
  float lse2 = kNegInf;
  if (m != kNegInf) {
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < kP; ++s)
      if (s < np) sum += hw_exp2(l2[s] - m);
    lse2 = m + hw_log2(sum);
#pragma unroll
    for (int s = 0; s < kP; ++s)
      if (s < np) {
        const float w = hw_exp2(l2[s] - lse2);  // 0 for an empty (-inf) part
        acc_a += w * xa[s];
        acc_b += w * xb[s];
      }
  }
  if constexpr (OUT_BF16) {
    const u32x2 wa = {pack_bf16x2(acc_a[0], acc_a[1]), pack_bf16x2(acc_a[2], acc_a[3])};
    const u32x2 wb = {pack_bf16x2(acc_b[0], acc_b[1]), pack_bf16x2(acc_b[2], acc_b[3])};
    __builtin_nontemporal_store(wa, (u32x2*)((uint16_t*)o_out + elem));
    __builtin_nontemporal_store(wb, (u32x2*)((uint16_t*)o_out + elem + D / 2));
  } else {
    __builtin_nontemporal_store(acc_a, (f32x4*)((float*)o_out + elem));
    __builtin_nontemporal_store(acc_b, (f32x4*)((float*)o_out + elem + D / 2));
  }
  if (c == 0 && lse_out) lse_out[row] = lse2 * kLn2;
}

template <int D, int NP, bool PB, bool OB>
static void launch_merge_np(const MergeParts& p, int n, int64_t rows, void* o, float* lse, hipStream_t st) {
  constexpr int kRowsPerBlock = 256 / (D / 8);
  const int64_t blocks = cdiv(rows, kRowsPerBlock);
  hipLaunchKernelGGL((lse_merge_kernel<D, NP, PB, OB>), dim3((uint32_t)blocks), dim3(256), 0, st, p, n, rows, o,
                     lse);
}

template <int D, bool PB, bool OB>
static void launch_merge(const MergeParts& p, int n, int64_t rows, void* o, float* lse, hipStream_t st) {
  switch (n) {
    case 2: launch_merge_np<D, 2, PB, OB>(p, n, rows, o, lse, st); break;
    case 4: launch_merge_np<D, 4, PB, OB>(p, n, rows, o, lse, st); break;
    default: launch_merge_np<D, 0, PB, OB>(p, n, rows, o, lse, st); break;
  }
}

}  // namespace cpa

using namespace cpa;

extern "C" cpa_status cpa_lse_merge(int32_t n_parts, const void* const* o_parts, const float* const* lse_parts,
                                    cpa_dtype part_dtype, int64_t rows, int32_t d, void* o_out,
                                    cpa_dtype out_dtype, float* lse_out, void* stream) {
  if (n_parts < 1 || n_parts > kMaxParts)
    return fail(CPA_ERR_INVALID_ARG, "cpa_lse_merge: n_parts %d not in [1, %d]", n_parts, kMaxParts);
  if (!o_parts || !lse_parts) return fail(CPA_ERR_INVALID_ARG, "cpa_lse_merge: part arrays are NULL");
  if (rows < 0) return fail(CPA_ERR_INVALID_ARG, "cpa_lse_merge: rows < 0");
  if (d != 64 && d != 128) return fail(CPA_ERR_UNSUPPORTED, "cpa_lse_merge: d = %d (supported: 64, 128)", d);
  if ((part_dtype != CPA_BF16 && part_dtype != CPA_F32) || (out_dtype != CPA_BF16 && out_dtype != CPA_F32))
    return fail(CPA_ERR_INVALID_ARG, "cpa_lse_merge: bad dtype");
  if (rows > 0 && !o_out) return fail(CPA_ERR_INVALID_ARG, "cpa_lse_merge: o_out is NULL");
  MergeParts p{};
  for (int s = 0; s < n_parts; ++s) {
    if (rows > 0 && (!o_parts[s] || !lse_parts[s]))
      return fail(CPA_ERR_INVALID_ARG, "cpa_lse_merge: part %d pointer is NULL", s);
    p.o[s] = o_parts[s];
    p.lse[s] = lse_parts[s];
  }
  if (rows > (int64_t)INT32_MAX * 16) return fail(CPA_ERR_INVALID_ARG, "cpa_lse_merge: rows too large");
  cpa_status st = check_device();
  if (st != CPA_OK) return st;
  if (rows == 0) return CPA_OK;
  hipStream_t s = (hipStream_t)stream;
  const bool pb = part_dtype == CPA_BF16, ob = out_dtype == CPA_BF16;
  if (d == 64) {
    if (pb && ob) launch_merge<64, true, true>(p, n_parts, rows, o_out, lse_out, s);
    else if (pb) launch_merge<64, true, false>(p, n_parts, rows, o_out, lse_out, s);
    else if (ob) launch_merge<64, false, true>(p, n_parts, rows, o_out, lse_out, s);
    else launch_merge<64, false, false>(p, n_parts, rows, o_out, lse_out, s);
  } else {
    if (pb && ob) launch_merge<128, true, true>(p, n_parts, rows, o_out, lse_out, s);
    else if (pb) launch_merge<128, true, false>(p, n_parts, rows, o_out, lse_out, s);
    else if (ob) launch_merge<128, false, true>(p, n_parts, rows, o_out, lse_out, s);
    else launch_merge<128, false, false>(p, n_parts, rows, o_out, lse_out, s);
  }
  return check_launch("cpa_lse_merge");
}
