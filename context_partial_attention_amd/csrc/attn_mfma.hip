// Partial causal GQA attention on bf16 inputs with gfx950 matrix cores.
//
// One call computes, for a packed shard of queries against one KV shard, the
// softmax-weighted values over the keys each query may see (k_pos <= q_pos in
// global positions, or all keys without a mask) together with the natural-log
// LSE of the scores. That is the partial attention of one step of pass-KV
// prefill, of pass-Q chunked prefill against a rank's resident cache, and of
// allgather decode ("Add utility functions to enable pass-kv prefill and
// allgather decode", Purpose); the partials are then merged exactly.
//
// Design (one workgroup = 4 waves = 128 query rows of one head):
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys are the M dimension and
//    queries the N dimension, so every lane owns one query row (lane % 32) and
//    the row max / row sum of the online softmax need a single cross-lane step
//    (lane ^ 32). Q stays in registers as the B operand for the whole loop.
//  * O^T = V^T P^T with the same instruction: P^T is built in registers from
//    the S^T accumulator (the lane that owns a query row owns its P values),
//    and the key order inside each 16-key step is the order the accumulator
//    produces; V is written to LDS transposed (d-major) with the matching key
//    permutation, so each A operand is one 16-byte LDS read.
//  * K and V tiles of 64 keys are double-buffered in LDS; the next tile's
//    global loads are in flight while the current tile is computed.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA per score.
//  * Positions ascend within a sequence, so a tile is skipped once its first
//    key is past the last query, and masking is only applied on tiles that
//    straddle a wave's diagonal.
//  * Work order: query tiles of a sequence run last-first (the causal mask
//    makes later tiles heavier), and the heads of one GQA group run on the
//    same XCD (workgroup ids are dealt to the 8 XCDs round-robin) so they
//    share K/V through that XCD's L2.
// Contiguous shards read k_pos; paged shards derive each key's global
// position from round-robin placement and gather 16-token blocks through the
// block table ("[Feature] Prefill Context Parallel (PCP) basic support",
// Purpose: block tables extended for context parallelism).
#include <climits>

#include "cpa_internal.h"
#include "device_common.h"

namespace cpa {
namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per main-loop step
constexpr int kThreads = 256;

template <int D>
struct Tile {
  static constexpr int kKStride = D + 8;    // LDS row stride of a K tile (bf16 elements)
  static constexpr int kVStride = kBN + 8;  // LDS row stride of a transposed V tile
  static constexpr int kKElems = kBN * kKStride;
  static constexpr int kVElems = D * kVStride;
  static constexpr int kBufElems = kKElems + kVElems;
  static constexpr int kKChunks = kBN * D / 8 / kThreads;  // 16-byte K pieces per thread
  static constexpr int kVUnits = (kBN / 4) * (D / 8);      // pieces of 4 keys x 8 dims
  static_assert(kKChunks * kThreads * 8 == kBN * D, "K tile must split evenly");
  static_assert(kVUnits <= kThreads, "one V piece per thread at most");
};

struct Params {
  const uint16_t* q;
  const int* q_pos;
  const int* cu_q;
  const uint16_t* k;
  const uint16_t* v;
  const int* k_pos;
  const int* cu_k;
  const int* block_table;
  int max_blocks;
  const int* local_kv_lens;
  int cp, rank, il;
  int num_seqs, hq, hkv, g, n_groups;
  float scale_log2;
  int causal;
  void* o;
  float* lse;
};

// LDS slot of key `key` inside a transposed V tile: within every 16 keys the
// groups of 4 are stored in the order 0,2,1,3 (bits 2 and 3 swapped), which is
// the order in which a lane's half of the S^T accumulator lists them.
__device__ __forceinline__ int v_slot(int key) { return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1); }

// Number of entries of the ascending array a[0..n) that are <= x, found by
// the whole workgroup: each round tests 256 evenly spaced points.
__device__ int block_count_le(const int* __restrict__ a, int n, int x) {
  int lo = 0, hi = n;
  while (true) {
    const int span = hi - lo;
    if (span <= 0) return lo;
    const int step = (span + kThreads - 1) / kThreads;
    const int idx = lo + (int)(threadIdx.x + 1) * step - 1;
    const int c = __syncthreads_count(idx < hi && a[idx] <= x);
    const int new_lo = lo + c * step;
    if (step == 1) return new_lo;
    hi = min(hi, new_lo + step - 1);
    lo = new_lo;
  }
}

template <int D, bool PAGED, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void attn_mfma_kernel(Params p) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::kBufElems];
  __shared__ int kpos_sh[2][kBN];

  // ---- which (sequence, query tile, head) this workgroup owns
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int member = rest % p.g;
  const int grp = (rest / p.g) * 8 + xcd;
  if (grp >= p.n_groups) return;
  const int kvh = grp % p.hkv;
  const int t2 = grp / p.hkv;
  const int seq = t2 % p.num_seqs;
  const int t_desc = t2 / p.num_seqs;
  const int qa = p.cu_q[seq], qe = p.cu_q[seq + 1];
  const int n_tiles = (qe - qa + kBM - 1) / kBM;
  if (t_desc >= n_tiles) return;
  const int row0 = qa + (n_tiles - 1 - t_desc) * kBM;
  const int h = kvh * p.g + member;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lc = lane >> 5;

  // ---- query rows and their positions
  const int my_row = row0 + wave * 32 + lr;
  const bool row_ok = my_row < qe;
  const int wave_first = row0 + wave * 32;
  const bool wave_active = wave_first < qe;
  const int wave_last = min(wave_first + 31, qe - 1);
  const int blk_last = min(row0 + kBM - 1, qe - 1);
  int my_pos, wave_qmin, wave_qmax, blk_qmax;
  if (p.causal) {
    my_pos = row_ok ? p.q_pos[my_row] : INT_MIN;
    wave_qmin = wave_active ? p.q_pos[wave_first] : INT_MIN;
    wave_qmax = wave_active ? p.q_pos[wave_last] : INT_MIN;
    blk_qmax = p.q_pos[blk_last];
  } else {  // every key of the shard is visible: treat rows as lying after all keys
    my_pos = row_ok ? INT_MAX - 1 : INT_MIN;
    wave_qmin = wave_qmax = wave_active ? INT_MAX - 1 : INT_MIN;
    blk_qmax = INT_MAX - 1;
  }

  // ---- key range [ka, n_end) that some row of this workgroup can see
  int ka, ke;
  if constexpr (PAGED) {
    ka = 0;
    ke = min(p.local_kv_lens[seq], p.max_blocks * 16);  // never index past the block table
  } else {
    ka = p.cu_k[seq];
    ke = p.cu_k[seq + 1];
  }
  int n_end = ke;
  if (p.causal) {
    if constexpr (PAGED) {
      n_end = min(ke, rr_count_below(blk_qmax + 1, p.cp, p.rank, p.il));
    } else {
      n_end = ka + block_count_le(p.k_pos + ka, ke - ka, blk_qmax);
    }
  }
  const int n_iter = n_end > ka ? (n_end - ka + kBN - 1) / kBN : 0;

  // ---- Q^T fragments (B operand): lane owns query row lr, dims 8*lc + 16*kk ...
  bf16x8 qf[D / 16];
  {
    const int qrow = row_ok ? my_row : qa;
    const uint16_t* src = p.q + ((int64_t)qrow * p.hq + h) * D + 8 * lc;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(src + 16 * kk);
  }

  // ---- tile staging through registers
  u32x4 kreg[T::kKChunks];
  u32x4 vreg[4];
  int kp_reg = INT_MAX;

  auto key_row = [&](const uint16_t* base, int j) -> const uint16_t* {
    if constexpr (PAGED) {
      const int blk = p.block_table[(int64_t)seq * p.max_blocks + (j >> 4)];
      return base + (((int64_t)blk * p.hkv + kvh) * 16 + (j & 15)) * D;
    } else {
      return base + ((int64_t)j * p.hkv + kvh) * D;
    }
  };

  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int u = tid + i * kThreads;
      const int r = u / (D / 8), c8 = u % (D / 8);
      const int j = min(j0 + r, n_end - 1);
      kreg[i] = *(const u32x4*)(key_row(p.k, j) + c8 * 8);
    }
    if (tid < T::kVUnits) {
      const int gk = tid & 15, dc = tid >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = min(j0 + 4 * gk + r, n_end - 1);
        vreg[r] = *(const u32x4*)(key_row(p.v, j) + dc * 8);
      }
    }
    if (tid < kBN) {
      const int j = j0 + tid;
      if (j < n_end) {
        if constexpr (PAGED) kp_reg = rr_global_pos(j, p.cp, p.rank, p.il);
        else kp_reg = p.causal ? p.k_pos[j] : 0;
      } else {
        kp_reg = INT_MAX;
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * T::kBufElems;
    uint16_t* vs = ks + T::kKElems;
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int u = tid + i * kThreads;
      const int r = u / (D / 8), c8 = u % (D / 8);
      *(u32x4*)(ks + r * T::kKStride + c8 * 8) = kreg[i];
    }
    if (tid < T::kVUnits) {
      const int gk = tid & 15, dc = tid >> 4;
      const int slot = v_slot(4 * gk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w0 = vreg[0][e], w1 = vreg[1][e], w2 = vreg[2][e], w3 = vreg[3][e];
        const u32x2 even = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
        const u32x2 odd = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
        *(u32x2*)(vs + (dc * 8 + 2 * e) * T::kVStride + slot) = even;
        *(u32x2*)(vs + (dc * 8 + 2 * e + 1) * T::kVStride + slot) = odd;
      }
    }
    if (tid < kBN) kpos_sh[buf][tid] = kp_reg;
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float sl2 = p.scale_log2;

  if (n_iter > 0) {
    load_tile(ka);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    const bool has_next = it + 1 < n_iter;
    if (has_next) load_tile(ka + (it + 1) * kBN);

    const int* kp = kpos_sh[buf];
    const int kfirst = kp[0], klast = kp[kBN - 1];
    if (kfirst <= wave_qmax) {
      const uint16_t* ks = smem + buf * T::kBufElems;
      const uint16_t* vs = ks + T::kKElems;
      // S^T for keys 0..31 (s0) and 32..63 (s1) of the tile
      f32x16 s0 = {}, s1 = {};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a0 = *(const bf16x8*)(ks + lr * T::kKStride + 16 * kk + 8 * lc);
        const bf16x8 a1 = *(const bf16x8*)(ks + (32 + lr) * T::kKStride + 16 * kk + 8 * lc);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], s1, 0, 0, 0);
      }
      // accumulator element v of this lane holds key 8*(v/4) + 4*lc + v%4 (+32 for s1)
      if (klast > wave_qmin) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = 8 * (v >> 2) + 4 * lc + (v & 3);
          if (kp[key] > my_pos) s0[v] = kNegInf;
          if (kp[32 + key] > my_pos) s1[v] = kNegInf;
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx * sl2);
      const float base = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = hw_exp2(m_run - base);
      float ps = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s0[v] = hw_exp2(fmaf(s0[v], sl2, -base));
        s1[v] = hw_exp2(fmaf(s1[v], sl2, -base));
        ps += s0[v] + s1[v];
      }
      l_run = l_run * alpha + ps;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      // P^T operands: k-step ks covers tile keys 16*ks .. 16*ks+15
      bf16x8 pb[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[0][e] = (__bf16)s0[e];
        pb[1][e] = (__bf16)s0[8 + e];
        pb[2][e] = (__bf16)s1[e];
        pb[3][e] = (__bf16)s1[8 + e];
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int kst = 0; kst < 4; ++kst) {
          const bf16x8 a = *(const bf16x8*)(vs + (32 * db + lr) * T::kVStride + 16 * kst + 8 * lc);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kst], oacc[db], 0, 0, 0);
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise and store O and LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t obase = ((int64_t)my_row * p.hq + h) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * lc;
      const f32x4 val = {oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv, oacc[db][4 * q4 + 2] * inv,
                         oacc[db][4 * q4 + 3] * inv};
      if constexpr (OUT_BF16) {
        const u32x2 w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
        *(u32x2*)((uint16_t*)p.o + obase + d0) = w;
      } else {
        *(f32x4*)((float*)p.o + obase + d0) = val;
      }
    }
  }
  if (lc == 0) p.lse[(int64_t)my_row * p.hq + h] = l_tot > 0.f ? (m_run + hw_log2(l_tot)) * kLn2 : kNegInf;
}

template <int D, bool PAGED, bool OUT_BF16>
void launch(const Params& p, uint32_t blocks, hipStream_t st) {
  hipLaunchKernelGGL((attn_mfma_kernel<D, PAGED, OUT_BF16>), dim3(blocks), dim3(kThreads), 0, st, p);
}

}  // namespace

cpa_status launch_attn_mfma(const AttnArgs& a, bool paged, hipStream_t st) {
  Params p{};
  p.q = (const uint16_t*)a.q;
  p.q_pos = a.q_pos;
  p.cu_q = a.cu_q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.k_pos = a.k_pos;
  p.cu_k = a.cu_k;
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
  p.scale_log2 = a.scale * kLog2e;
  p.causal = a.causal;
  p.o = a.o;
  p.lse = a.lse;
  const int64_t n_qtiles = cdiv(a.max_q, kBM);
  const int64_t n_groups = n_qtiles * a.num_seqs * a.hkv;
  const int64_t blocks = cdiv(n_groups, 8) * 8 * p.g;
  if (blocks > INT32_MAX) return fail(CPA_ERR_INVALID_ARG, "cpa_partial_attn: problem too large for one launch");
  p.n_groups = (int)n_groups;
  if (blocks == 0) return CPA_OK;
  const uint32_t nb = (uint32_t)blocks;
  if (a.d == 64) {
    if (paged) a.o_bf16 ? launch<64, true, true>(p, nb, st) : launch<64, true, false>(p, nb, st);
    else a.o_bf16 ? launch<64, false, true>(p, nb, st) : launch<64, false, false>(p, nb, st);
  } else {
    if (paged) a.o_bf16 ? launch<128, true, true>(p, nb, st) : launch<128, true, false>(p, nb, st);
    else a.o_bf16 ? launch<128, false, true>(p, nb, st) : launch<128, false, false>(p, nb, st);
  }
  return check_launch(paged ? "cpa_partial_attn_paged (prefill)" : "cpa_partial_attn (bf16)");
}

}  // namespace cpa
