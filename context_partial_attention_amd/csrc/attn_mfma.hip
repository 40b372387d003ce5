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
// Design (one workgroup = 4 waves; each wave owns 32*RB query rows of one
// head, RB = 1 or 2):
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys are the M dimension and
//    queries the N dimension, so every lane owns one query row per 32-row
//    block (lane % 32) and the row max of the online softmax needs a single
//    cross-lane step (lane ^ 32); the row sum needs none until the end. Q
//    stays in registers as the B operand for the whole loop.
//  * O^T = V^T P^T with the same instruction: P^T is taken from the S^T
//    accumulator registers (the lane that owns a query row owns its P values).
//    V is staged in LDS row-major, exactly like K, and each V^T operand is
//    assembled by two ds_read_b64_tr_b16 transposing reads, each giving a lane
//    4 consecutive keys of its d column; the key order they produce matches
//    the order in which the S^T accumulator lists a lane's keys.
//  * With RB = 2 every K and V operand read from LDS would feed two MFMAs (one
//    per 32-row block), halving LDS traffic per FLOP; the wave then holds ~400
//    registers and runs alone on its SIMD, with no room left to compute the
//    next tile's S during the softmax. Written that way it measured slower
//    than RB = 1 (two 32-row waves per SIMD), so only RB = 1 is built.
// The two-group kernel (attn_pp.hip) serves every even GQA group; this one
// serves odd groups.
//  * K and V tiles of 64 keys are double-buffered in LDS, K one tile ahead of
//    V, so the QK^T MFMAs of tile t+1 are issued while the softmax of tile t
//    runs on the vector ALUs; the next tiles' global loads are in flight
//    during the step. Loads use a workgroup-uniform tile base plus per-thread
//    offsets fixed for the whole loop; only the last tile clamps rows to the
//    last visible key.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA per score.
//    The running max is raised lazily: O and the row sum are rescaled only
//    when a row's tile max exceeds the running max by more than 2^8, so the
//    P values stay below 256 and the rescale of O is rare.
//  * Positions ascend within a sequence, so a tile is skipped once its first
//    key is past a wave's last query, and masking is only applied on tiles
//    that straddle a wave's diagonal.
//  * Work order: query tiles of a sequence run last-first (the causal mask
//    makes later tiles heavier), and the heads of one GQA group run on the
//    same XCD (workgroup ids are dealt to the 8 XCDs round-robin) so they
//    share K/V through that XCD's L2; consecutive groups rotate over the XCDs
//    so no sequence's tiles pile up on a few of them.
// Contiguous shards read k_pos; paged shards derive each key's global
// position from round-robin placement and gather 16-token blocks through the
// block table ("[Feature] Prefill Context Parallel (PCP) basic support",
// Purpose: block tables extended for context parallelism).
#include <climits>

#include "cpa_internal.h"
#include "device_common.h"

namespace cpa {
namespace {

constexpr int kBN = 64;   // keys per main-loop step
constexpr int kThreads = 256;

template <int D>
struct Tile {
  // LDS row strides (bf16 elements), padded so that the 16-byte K reads (16
  // rows per 16 lanes: stride = 4 banks mod 64) and the transposing V reads
  // (4 rows x 64 bytes per 32 lanes: stride = 16 banks mod 64) hit distinct
  // banks.
  static constexpr int kKStride = D + 8;
  static constexpr int kVStride = D + 32;
  static constexpr int kKElems = kBN * kKStride;
  static constexpr int kVElems = kBN * kVStride;
  static constexpr int kBufElems = kKElems + kVElems;
  static constexpr int kChunksPerRow = D / 8;                    // 16-byte pieces per row
  static constexpr int kChunks = kBN * kChunksPerRow / kThreads;  // pieces per thread per tile
  static constexpr int kRowsPerPass = kThreads / kChunksPerRow;   // rows covered by one piece index
  static_assert(kChunks * kThreads == kBN * kChunksPerRow, "tile must split evenly");
  // the rows one wave covers with one piece index stay inside one 16-token block
  static_assert(kRowsPerPass % 16 == 0 && 16 % (64 / kChunksPerRow) == 0, "wave rows must share a block");
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

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, source lane 4k+q names 4
// consecutive bf16 of row k of a 4-row block; result lane 4q+t receives column
// t of that lane quad's chunk from rows 0..3, i.e. one column of the block as
// 4 consecutive rows.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

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

template <int D, int RB, bool PIPE, bool PAGED, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 3 - RB) void attn_mfma_kernel(Params p) {
  using T = Tile<D>;
  constexpr int kRowsPerWave = 32 * RB;
  constexpr int kBM = 4 * kRowsPerWave;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (T::kKElems + T::kVElems)];
  __shared__ int kpos_sh[2][kBN];

  // ---- which (sequence, query tile, head) this workgroup owns
  // Workgroup ids are dealt to the 8 XCDs round-robin. The g heads (members)
  // of a group (query tile, sequence, KV head) share an XCD; group G of row
  // G/8 goes to XCD (G + G/8) mod 8, so groups that differ only in query tile
  // (the heavy and light tiles of one sequence) spread over all XCDs even
  // when sequences x KV heads is a multiple of 8.
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int member = rest % p.g;
  const int grow = rest / p.g;
  const int grp = grow * 8 + ((xcd - grow) & 7);
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

  // ---- query rows (lane owns row lr of each 32-row block rb) and positions
  const int wave_first = row0 + wave * kRowsPerWave;
  const bool wave_active = wave_first < qe;
  const int wave_last = min(wave_first + kRowsPerWave - 1, qe - 1);
  const int blk_last = min(row0 + kBM - 1, qe - 1);
  int my_row[RB], my_pos[RB];
  bool row_ok[RB];
  int wave_qmin, wave_qmax, blk_qmax;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    my_row[rb] = wave_first + 32 * rb + lr;
    row_ok[rb] = my_row[rb] < qe;
  }
  if (p.causal) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) my_pos[rb] = row_ok[rb] ? p.q_pos[my_row[rb]] : INT_MIN;
    wave_qmin = __builtin_amdgcn_readfirstlane(wave_active ? p.q_pos[wave_first] : INT_MIN);
    wave_qmax = __builtin_amdgcn_readfirstlane(wave_active ? p.q_pos[wave_last] : INT_MIN);
    blk_qmax = p.q_pos[blk_last];
  } else {  // every key of the shard is visible: treat rows as lying after all keys
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) my_pos[rb] = row_ok[rb] ? INT_MAX - 1 : INT_MIN;
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

  // ---- Q^T fragments (B operand): lane owns query row lr of block rb, dims 8*lc + 16*kk ...
  bf16x8 qf[RB][D / 16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qrow = row_ok[rb] ? my_row[rb] : qa;
    const uint16_t* src = p.q + ((int64_t)qrow * p.hq + h) * D + 8 * lc;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[rb][kk] = *(const bf16x8*)(src + 16 * kk);
  }

  // ---- tile staging through registers: thread piece i covers row
  // r_i = tid / kChunksPerRow + i * kRowsPerPass, bytes [16 c8, 16 c8 + 16).
  // Tile t covers keys ka + 64 t .. ka + 64 t + 63. K(t) lives in K buffer
  // t % 2 and is consumed one step before V(t) (with its key positions) in V
  // buffer t % 2.
  const int c8 = tid % T::kChunksPerRow;
  const int r_first = tid / T::kChunksPerRow;
  const int64_t row_stride = (int64_t)p.hkv * D;  // elements between consecutive keys (contiguous)
  uint32_t off[T::kChunks];                         // per-thread element offsets, fixed for the loop
#pragma unroll
  for (int i = 0; i < T::kChunks; ++i) {
    const int r = r_first + i * T::kRowsPerPass;
    if constexpr (PAGED) off[i] = (uint32_t)((r & 15) * D + c8 * 8);
    else off[i] = (uint32_t)(r * row_stride + c8 * 8);
  }

  // 16-byte pieces of tile t of `src` (K or V) into regs; the last tile
  // clamps rows to the last visible key
  auto load_tile = [&](const uint16_t* __restrict__ src, int t, u32x4* regs) {
    const int j0 = ka + t * kBN;
    const bool last = j0 + kBN > n_end;
    if constexpr (PAGED) {
      const int64_t slab = (int64_t)p.hkv * 16 * D;
      const int* tab = p.block_table + (int64_t)seq * p.max_blocks;
#pragma unroll
      for (int i = 0; i < T::kChunks; ++i) {
        const int r = r_first + i * T::kRowsPerPass;
        if (!last) {
          // every row of this wave's piece i lies in the same 16-token block
          const int blk = tab[__builtin_amdgcn_readfirstlane((j0 + r) >> 4)];
          regs[i] = *(const u32x4*)(src + (int64_t)blk * slab + (int64_t)kvh * 16 * D + off[i]);
        } else {
          const int j = min(j0 + r, n_end - 1);
          const int blk = tab[j >> 4];
          regs[i] = *(const u32x4*)(src + (int64_t)blk * slab + ((int64_t)kvh * 16 + (j & 15)) * D + c8 * 8);
        }
      }
    } else {
      const uint16_t* b = src + ((int64_t)j0 * p.hkv + kvh) * D;
#pragma unroll
      for (int i = 0; i < T::kChunks; ++i) {
        uint32_t o = off[i];
        if (last) o = (uint32_t)(min(r_first + i * T::kRowsPerPass, n_end - 1 - j0) * row_stride + c8 * 8);
        regs[i] = *(const u32x4*)(b + o);
      }
    }
  };
  auto key_pos = [&](int t) -> int {  // position of key tid of tile t (tid < 64), INT_MAX past the end
    const int j = ka + t * kBN + tid;
    if (j >= n_end) return INT_MAX;
    if constexpr (PAGED) return rr_global_pos(j, p.cp, p.rank, p.il);
    else return p.causal ? p.k_pos[j] : 0;
  };
  auto store_tile = [&](uint16_t* dst, int stride, const u32x4* regs) {
#pragma unroll
    for (int i = 0; i < T::kChunks; ++i)
      *(u32x4*)(dst + (r_first + i * T::kRowsPerPass) * stride + c8 * 8) = regs[i];
  };
  auto kbuf = [&](int b) { return smem + b * T::kKElems; };
  auto vbuf = [&](int b) { return smem + 2 * T::kKElems + b * T::kVElems; };

  f32x16 oacc[RB][D / 32];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[rb][db] = f32x16{};
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
  }
  const float sl2 = p.scale_log2;
  constexpr float kTau = 8.f;  // lazy-rescale threshold (log2 units)

  // per-lane LDS element offsets of the MFMA operands
  const int k_lane = lr * T::kKStride + 8 * lc;  // K rows lr (+32), dims 16 kk + 8 lc
  const int g16 = lane >> 4, j16 = lane & 15;
  // transposing V read: rows 4 lc + j16/4 (+16 kst, +8 for the second half),
  // columns 16 (g16 & 1) + 4 (j16 & 3) (+32 db)
  const int v_lane = (4 * lc + (j16 >> 2)) * T::kVStride + 16 * (g16 & 1) + 4 * (j16 & 3);

  // S^T of tile in K buffer kb for every row block: acc[rb][0] keys 0..31, acc[rb][1] keys 32..63
  auto qk = [&](int kb, f32x16 (&acc)[RB][2]) {
    const uint16_t* ks = kbuf(kb) + k_lane;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][0] = acc[rb][1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 a0 = *(const bf16x8*)(ks + 16 * kk);
      const bf16x8 a1 = *(const bf16x8*)(ks + 32 * T::kKStride + 16 * kk);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[rb][kk], acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[rb][kk], acc[rb][1], 0, 0, 0);
      }
    }
  };

  u32x4 kreg[T::kChunks], vreg[T::kChunks];
  int kp_reg = INT_MAX;

  // One pipelined step for tile t: S(t) is in c; S(t+1) is produced in x while
  // P(t) is formed, then O += V(t)^T P(t)^T. All waves take part in the loads,
  // stores and barrier; a wave whose rows see nothing of tile t (and hence of
  // any later tile, positions ascending) skips the math.
  // Softmax and P.V of tile t on S(t) in c; when pipelined, also S(t+1) into x.
  auto tile_math = [&](int t, f32x16 (&c)[RB][2], f32x16 (&x)[RB][2]) {
    const int* kp = kpos_sh[t & 1];
    if (__builtin_amdgcn_readfirstlane(kp[0]) <= wave_qmax) {
      // accumulator element v of this lane holds key 8*(v/4) + 4*lc + v%4 (+32 for c[rb][1])
      if (__builtin_amdgcn_readfirstlane(kp[kBN - 1]) > wave_qmin) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = 8 * (v >> 2) + 4 * lc + (v & 3);
          const int k0 = kp[key], k1 = kp[32 + key];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            if (k0 > my_pos[rb]) c[rb][0][v] = kNegInf;
            if (k1 > my_pos[rb]) c[rb][1][v] = kNegInf;
          }
        }
      }
      float mx[RB];
      bool need = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float m = fmaxf(c[rb][0][0], c[rb][1][0]);
#pragma unroll
        for (int v = 1; v < 16; ++v) m = max3(m, c[rb][0][v], c[rb][1][v]);
        mx[rb] = fmaxf(m, __shfl_xor(m, 32, 64)) * sl2;
        need |= mx[rb] > m_run[rb] + kTau;
      }
      // raise the running max only when some row's tile max exceeds it by > kTau
      if (__ballot(need) != 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float m_new = fmaxf(m_run[rb], mx[rb]);
          // 0 when the row had no key yet, 1 when its max is unchanged; rows
          // that still see no key keep O = 0 and l = 0
          const float alpha = (m_new == kNegInf) ? 1.f : hw_exp2(m_run[rb] - m_new);
          l_run[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[rb][db] *= alpha;
          m_run[rb] = m_new;
        }
      }
      // S^T of tile t+1 on the matrix cores while P of tile t is formed (past
      // the last tile the K buffer holds stale data and the result is unused)
      if constexpr (PIPE) qk((t + 1) & 1, x);
      bf16x8 pb[RB][4];  // P^T operands: k-step kst covers tile keys 16*kst .. 16*kst+15
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float base = (m_run[rb] == kNegInf) ? 0.f : m_run[rb];
        float ps = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          c[rb][0][v] = hw_exp2(fmaf(c[rb][0][v], sl2, -base));
          c[rb][1][v] = hw_exp2(fmaf(c[rb][1][v], sl2, -base));
          ps += c[rb][0][v] + c[rb][1][v];
        }
        l_run[rb] += ps;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[rb][0][e] = (__bf16)c[rb][0][e];
          pb[rb][1][e] = (__bf16)c[rb][0][8 + e];
          pb[rb][2][e] = (__bf16)c[rb][1][e];
          pb[rb][3][e] = (__bf16)c[rb][1][8 + e];
        }
      }
      const uint16_t* vs = vbuf(t & 1) + v_lane;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int kst = 0; kst < 4; ++kst) {
          const uint16_t* src = vs + 16 * kst * T::kVStride + 32 * db;
          const s16x4 lo = lds_read_tr(src);
          const s16x4 hi = lds_read_tr(src + 8 * T::kVStride);
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[rb][kst], oacc[rb][db], 0, 0, 0);
        }
      }
    }
  };

  auto step = [&](int t, f32x16 (&c)[RB][2], f32x16 (&x)[RB][2]) {
    const bool has_k2 = t + 2 < n_iter, has_v1 = t + 1 < n_iter;
    if constexpr (PIPE) {
      if (has_k2) load_tile(p.k, t + 2, kreg);
    } else {
      if (has_v1) load_tile(p.k, t + 1, kreg);
    }
    if (has_v1) {
      load_tile(p.v, t + 1, vreg);
      if (tid < kBN) kp_reg = key_pos(t + 1);
    }
    if constexpr (PIPE) {
      tile_math(t, c, x);
    } else {
      // S(t) local to the step: nothing of it is carried across tiles
      f32x16 cl[RB][2];
      if (__builtin_amdgcn_readfirstlane(kpos_sh[t & 1][0]) <= wave_qmax) qk(t & 1, cl);
      tile_math(t, cl, cl);
    }
    // pipelined: K(t) was last read in step t-1, V(t-1) and its positions in
    // step t-1. Otherwise K(t+1) was loaded one step ahead into buffer (t+1)%2.
    if constexpr (PIPE) {
      if (has_k2) store_tile(kbuf(t & 1), T::kKStride, kreg);
    } else {
      if (has_v1) store_tile(kbuf((t + 1) & 1), T::kKStride, kreg);
    }
    if (has_v1) {
      store_tile(vbuf((t + 1) & 1), T::kVStride, vreg);
      if (tid < kBN) kpos_sh[(t + 1) & 1][tid] = kp_reg;
    }
    lds_barrier();
  };

  // The loop is reached only through the prologue, which waits for every load
  // issued so far (Q included): the loop body then never waits on Q.
  if (n_iter > 0) {
    load_tile(p.k, 0, kreg);
    load_tile(p.v, 0, vreg);
    if (tid < kBN) kp_reg = key_pos(0);
    store_tile(kbuf(0), T::kKStride, kreg);
    store_tile(vbuf(0), T::kVStride, vreg);
    if (tid < kBN) kpos_sh[0][tid] = kp_reg;
    if (PIPE && n_iter > 1) {
      load_tile(p.k, 1, kreg);
      store_tile(kbuf(1), T::kKStride, kreg);
    }
    __syncthreads();
    f32x16 sa[RB][2], sb[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sa[rb][0] = sa[rb][1] = sb[rb][0] = sb[rb][1] = f32x16{};
    if (PIPE && __builtin_amdgcn_readfirstlane(kpos_sh[0][0]) <= wave_qmax) qk(0, sa);
    // unrolled by two so the S(t) / S(t+1) registers swap roles without copies
    for (int t = 0; t < n_iter; t += 2) {
      step(t, sa, sb);
      if (t + 1 < n_iter) step(t + 1, sb, sa);
    }
  }

  // ---- epilogue: normalise and store O and LSE
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = l_run[rb] + __shfl_xor(l_run[rb], 32, 64);
    if (!row_ok[rb]) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t obase = ((int64_t)my_row[rb] * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * lc;
        const f32x4 val = {oacc[rb][db][4 * q4] * inv, oacc[rb][db][4 * q4 + 1] * inv,
                           oacc[rb][db][4 * q4 + 2] * inv, oacc[rb][db][4 * q4 + 3] * inv};
        if constexpr (OUT_BF16) {
          const u32x2 w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
          *(u32x2*)((uint16_t*)p.o + obase + d0) = w;
        } else {
          *(f32x4*)((float*)p.o + obase + d0) = val;
        }
      }
    }
    if (lc == 0)
      p.lse[(int64_t)my_row[rb] * p.hq + h] = l_tot > 0.f ? (m_run[rb] + hw_log2(l_tot)) * kLn2 : kNegInf;
  }
}

template <int D, int RB, bool PAGED, bool OUT_BF16>
void launch(const Params& p, uint32_t blocks, hipStream_t st) {
  // one 32-row block per wave: two waves per SIMD, S of the next tile
  // computed during the softmax; two blocks: one wave per SIMD, no room for a
  // second S
  hipLaunchKernelGGL((attn_mfma_kernel<D, RB, RB == 1, PAGED, OUT_BF16>), dim3(blocks), dim3(kThreads), 0, st, p);
}

template <int D, int RB>
void launch_d(const Params& p, uint32_t blocks, bool paged, bool o_bf16, hipStream_t st) {
  if (paged) o_bf16 ? launch<D, RB, true, true>(p, blocks, st) : launch<D, RB, true, false>(p, blocks, st);
  else o_bf16 ? launch<D, RB, false, true>(p, blocks, st) : launch<D, RB, false, false>(p, blocks, st);
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
  const int64_t n_qtiles = cdiv(a.max_q, 128);
  const int64_t n_groups = n_qtiles * a.num_seqs * a.hkv;
  const int64_t blocks = cdiv(n_groups, 8) * 8 * p.g;
  if (blocks > INT32_MAX) return fail(CPA_ERR_INVALID_ARG, "cpa_partial_attn: problem too large for one launch");
  p.n_groups = (int)n_groups;
  if (blocks == 0) return CPA_OK;
  const uint32_t nb = (uint32_t)blocks;
  if (a.d == 64) launch_d<64, 1>(p, nb, paged, a.o_bf16, st);
  else launch_d<128, 1>(p, nb, paged, a.o_bf16, st);
  return check_launch(paged ? "cpa_partial_attn_paged (prefill)" : "cpa_partial_attn (bf16)");
}

}  // namespace cpa
