// Partial attention for fp32 inputs against a contiguous KV shard.
//
// Query i of sequence b attends to the keys of sequence b's shard with
// k_pos <= q_pos[i] (or to all of them without a mask) and returns the
// partial output and its natural-log LSE ("Add utility functions to enable
// pass-kv prefill and allgather decode", Purpose: partial attention against
// one exchanged KV shard).
//
// fp32 inputs only appear in tiny, launch-bound problems, so this kernel is
// written for clarity rather than speed: one wave per (query row, head), one
// lane per key for the scores (64 keys per step), online softmax with wave
// reductions, and one lane per output element for P.V. The bf16 path, which
// carries the real workloads, is the MFMA kernel in attn_mfma.hip.
#include "cpa_internal.h"
#include "device_common.h"

namespace cpa {

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ q, const int* __restrict__ q_pos,
                                                       const int* __restrict__ cu_q, const float* __restrict__ k,
                                                       const float* __restrict__ v, const int* __restrict__ k_pos,
                                                       const int* __restrict__ cu_k, int hq, int hkv, float scale_log2,
                                                       int causal, float* __restrict__ o, float* __restrict__ lse) {
  constexpr int kPer = D / 64;  // output elements per lane
  __shared__ float q_sh[4][D];
  __shared__ float p_sh[4][64];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int seq = blockIdx.z, h = blockIdx.y;
  const int qa = cu_q[seq], qe = cu_q[seq + 1];
  const int r = blockIdx.x * 4 + wave;
  if (qa + r >= qe) return;  // whole wave leaves together; no block barrier below
  const int row = qa + r;
  const int kvh = h / (hq / hkv);
  const int my_pos = q_pos[row];
  const float* qrow = q + ((int64_t)row * hq + h) * D;
  for (int d = lane; d < D; d += 64) q_sh[wave][d] = qrow[d];
  __builtin_amdgcn_wave_barrier();

  const int ka = cu_k[seq], ke = cu_k[seq + 1];
  float m = kNegInf, l = 0.f;
  float acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.f;

  for (int j0 = ka; j0 < ke; j0 += 64) {
    if (causal && k_pos[j0] > my_pos) break;  // positions ascend: the rest is masked too
    const int j = j0 + lane;
    float s = kNegInf;
    if (j < ke && (!causal || k_pos[j] <= my_pos)) {
      const float* krow = k + ((int64_t)j * hkv + kvh) * D;
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) dot = fmaf(q_sh[wave][d], krow[d], dot);
      s = dot * scale_log2;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float base = (m_new == kNegInf) ? 0.f : m_new;
    const float p = hw_exp2(s - base);
    const float alpha = hw_exp2(m - base);
    l = l * alpha + wave_sum(p);
    m = m_new;
    p_sh[wave][lane] = p;
    __builtin_amdgcn_wave_barrier();
    const int nk = min(64, ke - j0);
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] *= alpha;
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = p_sh[wave][jj];
      const float* vrow = v + ((int64_t)(j0 + jj) * hkv + kvh) * D;
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = fmaf(pj, vrow[lane + 64 * i], acc[i]);
    }
    __builtin_amdgcn_wave_barrier();
  }
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  float* orow = o + ((int64_t)row * hq + h) * D;
#pragma unroll
  for (int i = 0; i < kPer; ++i) orow[lane + 64 * i] = acc[i] * inv;
  if (lane == 0) lse[(int64_t)row * hq + h] = (l > 0.f) ? (m + hw_log2(l)) * kLn2 : kNegInf;
}

cpa_status launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((uint32_t)cdiv(a.max_q, 4), (uint32_t)a.hq, (uint32_t)a.num_seqs);
  const float sl2 = a.scale * kLog2e;
  if (a.d == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, st, (const float*)a.q, a.q_pos, a.cu_q,
                       (const float*)a.k, (const float*)a.v, a.k_pos, a.cu_k, a.hq, a.hkv, sl2, a.causal,
                       (float*)a.o, a.lse);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, st, (const float*)a.q, a.q_pos, a.cu_q,
                       (const float*)a.k, (const float*)a.v, a.k_pos, a.cu_k, a.hq, a.hkv, sl2, a.causal,
                       (float*)a.o, a.lse);
  return check_launch("cpa_partial_attn (fp32)");
}

}  // namespace cpa
