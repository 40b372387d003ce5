// Decode partial attention against one rank's paged, round-robin KV shard.
//
// Allgather decode ("Add utility functions to enable pass-kv prefill and
// allgather decode", Purpose): the decode query of every sequence is gathered
// on all CP ranks, each rank attends it to its round-robin share of the KV
// cache, and the per-rank partials (O, LSE) are merged exactly.
//
// One query per sequence makes this HBM-bound: every K/V byte of the local
// shard is read once. The work is split over (sequence, KV head, split of
// 512-2048 local tokens) so that sequences of very different lengths still
// fill the GPU, and a second small kernel merges the splits of each (sequence,
// head) with the same exact LSE rule used across ranks. That kernel can also
// fold in the other ranks' partials of the same rows when they are already
// resident (received), so that a rank's decode step ends with the merged
// result after two launches, without a separate cross-rank merge.
//
// Inside a workgroup (4 waves, each walking every 4th 16-token block):
//  * S^T = K q^T with v_mfma_f32_16x16x32_bf16: the 16 keys of a block are the
//    M dimension and loaded straight from HBM in operand layout (16 contiguous
//    bytes per lane); the query heads of the GQA group are the N columns.
//  * P.V on the vector ALUs in fp32: each lane owns 8 contiguous dims of 4 of
//    the block's keys, so V is read with fully coalesced 16-byte loads, and
//    the P values and rescale factors reach those lanes through LDS.
//  * Keys past the visible count are masked and their rows clamped to a valid
//    row of the same block, so no uninitialised cache memory enters a sum.
#include <climits>

#include "cpa_internal.h"
#include "device_common.h"

namespace cpa {
namespace {

// Local KV tokens per split: the largest of 2048, 1024 and 512 that still
// gives kMinSplitItems (sequence, split) pairs at the longest local length.
// Longer splits spend less of the run on each workgroup's first load and its
// final reduction; shorter ones keep a few long sequences spread over the GPU.
constexpr int kMaxSplit = 2048, kMinSplit = 512;
constexpr int64_t kMinSplitItems = 1024;
int split_tokens(int64_t num_seqs, int64_t max_len) {
  int s = kMaxSplit;
  while (s > kMinSplit && num_seqs * ((max_len + s - 1) / s) < kMinSplitItems) s >>= 1;
  return s;
}
constexpr int kThreads = 256;
constexpr int kWaves = 4;

struct DecParams {
  const uint16_t* q;
  const int* q_pos;
  const int* cu_q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int* block_table;
  int max_blocks;
  const int* local_kv_lens;
  int cp, rank, il;
  int num_seqs, hq, hkv, g, head_chunk, n_hchunks, split, n_splits_max, causal;
  float scale_log2;
  float* ws_o;    // [num_seqs][hq][n_splits_max][D]
  float* ws_lse;  // [num_seqs][hq][n_splits_max], base-2 LSE of each split
  void* o;
  float* lse;
  // other ranks' partials of the same rows, folded in by the merge kernel
  int n_fold;
  const void* fold_o[kMaxFoldParts];
  const float* fold_lse[kMaxFoldParts];
  void* own_o;  // this rank's own partial (may be NULL), in the parts' dtype
  float* own_lse;
};

// Local KV slots of `seq` visible to its query at packed row `row`: the round-
// robin order is ascending in global position, so they form a prefix.
__device__ __forceinline__ int visible_local(const DecParams& p, int seq, int row) {
  const int len = min(p.local_kv_lens[seq], p.max_blocks * 16);  // never index past the block table
  if (!p.causal) return len;
  return min(len, rr_count_below(p.q_pos[row] + 1, p.cp, p.rank, p.il));
}

template <int D, int HC>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecParams p) {
  __shared__ __attribute__((aligned(16))) float p_sh[kWaves][HC][16];
  __shared__ float a_sh[kWaves][HC];
  __shared__ float red_m[kWaves][HC], red_l[kWaves][HC];
  __shared__ __attribute__((aligned(16))) float red_o[kWaves][HC][D];

  // heads vary fastest over the grid: the workgroups that run together read
  // the slices of the same physical blocks
  const int split = blockIdx.y;
  const int kvh = blockIdx.x / p.n_hchunks, hc = blockIdx.x % p.n_hchunks;
  const int seq = blockIdx.z;
  const int row = p.cu_q[seq];
  if (p.cu_q[seq + 1] <= row) return;
  const int n_vis = visible_local(p, seq, row);
  if (split * p.split >= n_vis) return;  // the merge kernel reads only the splits that exist
  const int k_end = min(n_vis, (split + 1) * p.split);
  const int b_begin = split * (p.split / 16), b_end = (k_end + 15) / 16;
  const int h0 = kvh * p.g + hc * HC;
  const int nh = min(HC, p.g - hc * HC);

  // V role: lane owns dims 8*dc .. 8*dc+7 of keys kg*kKPL .. kg*kKPL+kKPL-1 of a block
  constexpr int kDC = D / 8;        // 16-byte chunks per row
  constexpr int kKPL = 16 * kDC / 64;  // keys per lane per block
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, ks = lane >> 4;          // S role: head column n, keys 4ks..4ks+3
  const int dc = lane % kDC, kg = lane / kDC;       // V role

  // q^T fragments (B operand): lane holds head h0+n, dims 32*kk + 8*ks .. +8
  bf16x8 qf[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    if (n < nh) qf[kk] = *(const bf16x8*)(p.q + ((int64_t)row * p.hq + h0 + n) * D + 32 * kk + 8 * ks);
    else qf[kk] = bf16x8{};
  }
  const float sl2 = p.scale_log2;
  float m_run = kNegInf, l_run = 0.f;  // softmax state of head n (this lane's keys only for l)
  float acc[HC][8];                    // sum_k p[h][k] v[k][8dc + e] over this lane's keys
#pragma unroll
  for (int h = 0; h < HC; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  const int64_t head_stride = 16LL * D;  // one (block, kv head) slab
  // This wave's blocks are b_begin + wave + kWaves*i, i < nb (at most
  // kBlocksPerWave); lane i holds the physical block of the i-th, read once.
  constexpr int kBlocksPerWave = kMaxSplit / 16 / kWaves;
  static_assert(kBlocksPerWave <= 64, "one block-table entry per lane");
  const int first_b = b_begin + wave;
  const int nb = first_b < b_end ? (b_end - first_b + kWaves - 1) / kWaves : 0;
  const int phys_lane =
      lane < nb ? p.block_table[(int64_t)seq * p.max_blocks + first_b + kWaves * lane] : 0;

  // K and V of a block in registers; the next block's loads are issued before
  // the current block is computed, so HBM latency overlaps the math
  struct Blk {
    bf16x8 ka[D / 32];
    u32x4 vr[kKPL];
  };
  auto load_blk = [&](int i, Blk& r) {
    const int b = first_b + kWaves * i;
    const int phys = __builtin_amdgcn_readlane(phys_lane, i);
    const int nvalid = min(16, k_end - b * 16);
    const int64_t slab = ((int64_t)phys * p.hkv + kvh) * head_stride;
    const uint16_t* kb = p.kc + slab;
    const uint16_t* vb = p.vc + slab;
    const int krow = min(n, nvalid - 1);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) r.ka[kk] = *(const bf16x8*)(kb + krow * D + 32 * kk + 8 * ks);
#pragma unroll
    for (int i2 = 0; i2 < kKPL; ++i2) r.vr[i2] = *(const u32x4*)(vb + min(kg * kKPL + i2, nvalid - 1) * D + 8 * dc);
  };
  auto compute_blk = [&](int i, const Blk& r) {
    const int b = first_b + kWaves * i;
    const int nvalid = min(16, k_end - b * 16);
    f32x4 s = {};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.ka[kk], qf[kk], s, 0, 0, 0);
    // s[i]: key 4*ks + i of this block, head column n
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = (4 * ks + j < nvalid) ? s[j] * sl2 : kNegInf;
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float base = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = hw_exp2(m_run - base);
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = hw_exp2(s[j] - base);
    l_run = l_run * alpha + (s[0] + s[1]) + (s[2] + s[3]);
    m_run = m_new;
    if (n < HC) {
      *(f32x4*)&p_sh[wave][n][4 * ks] = s;
      if (ks == 0) a_sh[wave][n] = alpha;
    }
    __builtin_amdgcn_wave_barrier();
    // acc[h][e] = acc[h][e] * alpha[h] + sum over this lane's keys of p[h][key] v[key][8 dc + e]
    // (heads past nh carry zero queries; their sums are never written)
    float pv[HC][kKPL];
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      const float al = a_sh[wave][h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al;
#pragma unroll
      for (int i2 = 0; i2 < kKPL; ++i2) pv[h][i2] = p_sh[wave][h][kg * kKPL + i2];
    }
#pragma unroll
    for (int i2 = 0; i2 < kKPL; ++i2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(r.vr[i2][e]), hi = bf16_hi(r.vr[i2][e]);
#pragma unroll
        for (int h = 0; h < HC; ++h) {
          acc[h][2 * e] = fmaf(pv[h][i2], lo, acc[h][2 * e]);
          acc[h][2 * e + 1] = fmaf(pv[h][i2], hi, acc[h][2 * e + 1]);
        }
      }
    __builtin_amdgcn_wave_barrier();
  };
  Blk bufa, bufb;
  if (nb > 0) load_blk(0, bufa);
  for (int i = 0; i < nb; i += 2) {
    if (i + 1 < nb) load_blk(i + 1, bufb);
    compute_blk(i, bufa);
    if (i + 1 < nb) {
      if (i + 2 < nb) load_blk(i + 2, bufa);
      compute_blk(i + 1, bufb);
    }
  }

  // reduce over the key subsets of the wave
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
#pragma unroll
  for (int h = 0; h < HC; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[h][e];
#pragma unroll
      for (int off = kDC; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
      acc[h][e] = x;
    }
  if (ks == 0 && n < HC) {
    red_m[wave][n] = m_run;
    red_l[wave][n] = l_run;
  }
  if (kg == 0) {
#pragma unroll
    for (int h = 0; h < HC; ++h)
#pragma unroll
      for (int e = 0; e < 8; e += 4)
        *(f32x4*)&red_o[wave][h][8 * dc + e] = f32x4{acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]};
  }
  __syncthreads();
  // merge the 4 waves and write this split's (O, base-2 LSE)
  for (int idx = tid; idx < nh * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, red_m[w][h]);
    float ll = 0.f, oo = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = hw_exp2(red_m[w][h] - mm);  // 0 for a wave that saw no block
      ll += red_l[w][h] * f;
      oo += red_o[w][h][d] * f;
    }
    const int64_t slot = ((int64_t)seq * p.hq + h0 + h) * p.n_splits_max + split;
    p.ws_o[slot * D + d] = oo / ll;
    if (d == 0) p.ws_lse[slot] = mm + hw_log2(ll);
  }
}

template <int D, bool BF16>
__device__ __forceinline__ void store_row_part(void* base, int64_t off, int lane, const float (&x)[D / 64]) {
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    if constexpr (BF16) ((__bf16*)base)[off + lane + 64 * i] = (__bf16)x[i];
    else ((float*)base)[off + lane + 64 * i] = x[i];
  }
}

// One wave per (sequence, query head): merges the splits of this rank's
// partial. FOLD: then merges that partial with the other ranks' partials of
// the same row (p.fold_o / fold_lse, PART_BF16 giving their dtype) by the same
// exact LSE rule, writes the result to p.o / p.lse and this rank's own partial
// to p.own_o / own_lse when those are set. A part whose LSE is -inf has no
// visible key; its O is not read.
template <int D, bool OUT_BF16, bool FOLD, bool PART_BF16>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecParams p) {
  constexpr int kPer = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
  if (item >= (int64_t)p.num_seqs * p.hq) return;
  const int seq = (int)(item / p.hq), h = (int)(item % p.hq);
  const int row = p.cu_q[seq];
  if (p.cu_q[seq + 1] <= row) return;
  const int64_t ri = (int64_t)row * p.hq + h;
  // the other ranks' LSEs (base 2) are read first, so their latency overlaps
  // the split loop
  float lf[FOLD ? kMaxFoldParts : 1];
  if constexpr (FOLD) {
#pragma unroll
    for (int j = 0; j < kMaxFoldParts; ++j) lf[j] = j < p.n_fold ? p.fold_lse[j][ri] * kLog2e : kNegInf;
  }
  const int n_vis = visible_local(p, seq, row);
  const int n_splits = (n_vis + p.split - 1) / p.split;
  const int64_t slot0 = ((int64_t)seq * p.hq + h) * p.n_splits_max;
  float mx = kNegInf;
  for (int s = lane; s < n_splits; s += 64) mx = fmaxf(mx, p.ws_lse[slot0 + s]);
  mx = wave_max(mx);
  float lse2 = kNegInf;
  float acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
  if (mx != kNegInf) {
    float sum = 0.f;
    for (int s = lane; s < n_splits; s += 64) sum += hw_exp2(p.ws_lse[slot0 + s] - mx);
    lse2 = mx + hw_log2(wave_sum(sum));
    // 8 splits' reads issued before their sums (one round trip per 8 splits
    // instead of one per split); the sums stay in split order. Reads past the
    // last split repeat it and get weight 0.
    constexpr int kU = 8;
    for (int s0 = 0; s0 < n_splits; s0 += kU) {
      float lv[kU], x[kU][kPer];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int s = min(s0 + u, n_splits - 1);
        lv[u] = p.ws_lse[slot0 + s];
        const float* src = p.ws_o + (slot0 + s) * D;
#pragma unroll
        for (int i = 0; i < kPer; ++i) x[u][i] = src[lane + 64 * i];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float w = s0 + u < n_splits ? hw_exp2(lv[u] - lse2) : 0.f;
#pragma unroll
        for (int i = 0; i < kPer; ++i) acc[i] = fmaf(w, x[u][i], acc[i]);
      }
    }
  }
  if constexpr (FOLD) {
    if (p.own_o) store_row_part<D, PART_BF16>(p.own_o, ri * D, lane, acc);
    if (p.own_lse && lane == 0) p.own_lse[ri] = lse2 * kLn2;
    float m = lse2;
#pragma unroll
    for (int j = 0; j < kMaxFoldParts; ++j) m = fmaxf(m, lf[j]);
    if (m == kNegInf) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
      lse2 = kNegInf;
    } else {
      float sum = hw_exp2(lse2 - m);
#pragma unroll
      for (int j = 0; j < kMaxFoldParts; ++j) sum += hw_exp2(lf[j] - m);
      const float lt = m + hw_log2(sum);
      const float w_own = hw_exp2(lse2 - lt);
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] *= w_own;
#pragma unroll
      for (int j = 0; j < kMaxFoldParts; ++j) {
        if (j >= p.n_fold || lf[j] == kNegInf) continue;  // wave-uniform
        const float w = hw_exp2(lf[j] - lt);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          float x;
          if constexpr (PART_BF16) x = (float)((const __bf16*)p.fold_o[j])[ri * D + lane + 64 * i];
          else x = ((const float*)p.fold_o[j])[ri * D + lane + 64 * i];
          acc[i] = fmaf(w, x, acc[i]);
        }
      }
      lse2 = lt;
    }
  }
  store_row_part<D, OUT_BF16>(p.o, ri * D, lane, acc);
  if (lane == 0) p.lse[ri] = lse2 * kLn2;
}

int head_chunk_for(int g) { return g >= 8 ? 8 : (g >= 4 ? 4 : (g >= 2 ? 2 : 1)); }

template <int D, int HC>
void launch_split(const DecParams& p, hipStream_t st) {
  const dim3 grid((uint32_t)(p.hkv * p.n_hchunks), (uint32_t)p.n_splits_max, (uint32_t)p.num_seqs);
  hipLaunchKernelGGL((decode_split_kernel<D, HC>), grid, dim3(kThreads), 0, st, p);
}

template <int D>
void launch_split_d(const DecParams& p, hipStream_t st) {
  switch (p.head_chunk) {
    case 8: launch_split<D, 8>(p, st); break;
    case 4: launch_split<D, 4>(p, st); break;
    case 2: launch_split<D, 2>(p, st); break;
    default: launch_split<D, 1>(p, st); break;
  }
}

template <int D>
void launch_merge_d(const DecParams& p, bool o_bf16, const RankFold* fold, hipStream_t st) {
  const dim3 grid((uint32_t)cdiv((int64_t)p.num_seqs * p.hq, kWaves)), block(kThreads);
  if (!fold) {
    if (o_bf16) hipLaunchKernelGGL((decode_merge_kernel<D, true, false, false>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((decode_merge_kernel<D, false, false, false>), grid, block, 0, st, p);
  } else if (fold->part_bf16) {
    if (o_bf16) hipLaunchKernelGGL((decode_merge_kernel<D, true, true, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((decode_merge_kernel<D, false, true, true>), grid, block, 0, st, p);
  } else {
    if (o_bf16) hipLaunchKernelGGL((decode_merge_kernel<D, true, true, false>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((decode_merge_kernel<D, false, true, false>), grid, block, 0, st, p);
  }
}

}  // namespace

size_t decode_workspace_bytes(int32_t num_seqs, int32_t max_blocks, int32_t block_size, int32_t hq, int32_t d) {
  const int64_t max_len = (int64_t)max_blocks * block_size;
  const int64_t n_splits = cdiv(max_len, split_tokens(num_seqs, max_len));
  return (size_t)num_seqs * hq * n_splits * (d + 1) * sizeof(float);
}

cpa_status launch_attn_decode(const AttnArgs& a, hipStream_t st, const RankFold* fold) {
  DecParams p{};
  p.q = (const uint16_t*)a.q;
  p.q_pos = a.q_pos;
  p.cu_q = a.cu_q;
  p.kc = (const uint16_t*)a.k;
  p.vc = (const uint16_t*)a.v;
  p.block_table = a.block_table;
  p.max_blocks = a.max_blocks;
  p.local_kv_lens = a.local_kv_lens;
  p.cp = a.cp;
  p.rank = a.rank;
  p.il = a.interleave;
  p.num_seqs = a.num_seqs;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.g = a.hq / a.hkv;
  p.head_chunk = head_chunk_for(p.g);
  p.n_hchunks = (int)cdiv(p.g, p.head_chunk);
  p.split = split_tokens(a.num_seqs, (int64_t)a.max_blocks * 16);
  p.n_splits_max = (int)cdiv((int64_t)a.max_blocks * 16, p.split);
  p.causal = a.causal;
  p.scale_log2 = a.scale * kLog2e;
  const int64_t slots = (int64_t)a.num_seqs * a.hq * p.n_splits_max;
  p.ws_o = (float*)a.workspace;
  p.ws_lse = p.ws_o + slots * a.d;
  p.o = a.o;
  p.lse = a.lse;
  if (a.num_seqs == 0) return CPA_OK;
  if (p.n_splits_max > 65535 || (int64_t)p.hkv * p.n_hchunks > 65535 || a.num_seqs > 65535)
    return fail(CPA_ERR_INVALID_ARG, "cpa_partial_attn_paged (decode): grid too large");
  if (p.n_splits_max > 0) {
    if (a.d == 64) launch_split_d<64>(p, st);
    else launch_split_d<128>(p, st);
    cpa_status s = check_launch("cpa_partial_attn_paged (decode splits)");
    if (s != CPA_OK) return s;
  }
  if (fold) {
    p.n_fold = fold->n;
    for (int j = 0; j < fold->n; ++j) {
      p.fold_o[j] = fold->o[j];
      p.fold_lse[j] = fold->lse[j];
    }
    p.own_o = fold->own_o;
    p.own_lse = fold->own_lse;
  }
  if (a.d == 64) launch_merge_d<64>(p, a.o_bf16, fold, st);
  else launch_merge_d<128>(p, a.o_bf16, fold, st);
  return check_launch("cpa_partial_attn_paged (decode merge)");
}

}  // namespace cpa
