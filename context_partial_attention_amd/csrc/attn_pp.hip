// Partial causal GQA attention on bf16 inputs: two-group ("ping-pong")
// workgroup for GQA groups of even size.
//
// Computes the same partial attention as attn_mfma.hip (a packed query shard
// against one KV shard, causal in global positions, returning O and the
// natural-log LSE; "Add utility functions to enable pass-kv prefill and
// allgather decode", Purpose) with a schedule built to keep the matrix cores
// busy while the softmax runs.
//
// A workgroup of 8 waves owns 128 query rows of two heads h0, h0+1 of one GQA
// group (they read the same KV head). Waves 0-3 (group 0) take head h0,
// waves 4-7 (group 1) head h0+1; each wave owns 32 rows, so every SIMD holds
// one wave of each group. Work on KV tile t is split into two phases:
//   A(t): O += V(t-1)^T P(t-1)^T and S(t)^T = K(t) Q^T   (matrix cores)
//   B(t): mask, online softmax of S(t) -> P(t)           (vector ALUs)
// Group 1 runs one phase behind group 0, so on each SIMD one wave issues
// MFMAs while the other does its softmax. A workgroup barrier ends every odd
// phase (it publishes the next slot); between two barriers each group runs
// one A and one B phase in opposite orders, which keeps the groups a phase
// apart without a barrier in the middle (one there only added the waves'
// skew). Both groups see the same rows, hence the same masks and tile
// counts, so neither waits on the other. The wave in phase A raises its
// issue priority: left to the hardware, the older wave (group 0) wins every
// conflict and group 1's matrix work stalls behind group 0's softmax.
//
// LDS holds two slots; slot t carries K(t), V(t-1) and the key positions of
// tile t and is read in phases 2t and 2t+1. Its K and V tiles travel from
// global memory straight into LDS (gfx950's 16-byte global->LDS loads, no
// registers and no LDS write instructions in the waves): they are issued at
// the start of phase 2t-2 and waited for at the end of phase 2t-1, so every
// load has two phases to arrive. Both tiles are row-major with the 16-byte
// pieces of each row swizzled so that the K operand reads (16 bytes) and the
// transposing V^T operand reads (ds_read_b64_tr_b16, which hand each lane 4
// consecutive keys of one dim) are bank-conflict free.
//
// One launch covers up to kMaxShards contiguous KV shards, each into its own
// partial (a group is then (query tile, sequence, shard, KV head)), or with
// MERGED one walk over the visible key tiles of every shard with a single
// online softmax, which yields the exact merge of the shards' partials. With a
// running accumulator (o_acc) the epilogue folds the partial into it instead
// of writing it. An optional pre-pass (pp_schedule_kernel) orders the launch
// heaviest query tile first (shard-major for long launches). Paged shards
// (pass-Q prefill) take one shard, their block table read through the scalar
// cache; there the epilogue can also merge the other ranks' partials of the
// same rows into the result (the rank fold).
#include <climits>
#include <mutex>

#include "attn_pp_common.h"

namespace cpa {
namespace {

constexpr int kThreads = 512;  // 8 waves
using namespace pp;

template <int D, bool PAGED, bool OUT_BF16, bool MERGED>
__global__ __launch_bounds__(kThreads, 1) void attn_pp_kernel(PPParams p) {
  using T = PPTile<D, kThreads>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::kSlotElems];
  __shared__ int kpos_sh[4][kBN];

  // ---- (sequence, query tile, KV head) group and head pair. Workgroup ids
  // are dealt round-robin to the 8 XCDs; group grow * 8 + xcd runs on XCD
  // xcd, so its KV head (the group index modulo hkv) is fixed per XCD and
  // each XCD's L2 holds the K/V of its own heads only (8x less L2-to-fabric
  // traffic on the 128K launch than rotating groups over the XCDs); the head
  // pairs of a group share its XCD
  const int pairs = p.g >> 1;
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int pair = rest % pairs;
  const int grow = rest / pairs;
  int grp = grow * 8 + xcd;
  if (grp >= p.n_groups) return;
  // visible key tiles of the unit as the launch-order pre-pass counted them
  // (-1: not known, search below)
  int pre_n = -1;
  if constexpr (!PAGED) {
    if (p.order) {
      const int e = p.order[grp / p.hkv];
      grp = (e & kOrderUnitMask) * p.hkv + grp % p.hkv;
      if (!MERGED && (e >> kOrderUnitBits) != kOrderWorkUnknown) pre_n = e >> kOrderUnitBits;
    }
  }
  // group = ((tile_desc * num_seqs + seq) * n_shards + shard) * hkv + kvh
  // (no shard term when MERGED: one group walks every shard): the heaviest
  // query tiles of every sequence and shard come first
  const int n_sh_grid = MERGED ? 1 : p.n_shards;
  const int kvh = grp % p.hkv;
  const int t2 = grp / p.hkv;
  const int shard = t2 % n_sh_grid;
  const int t3 = t2 / n_sh_grid;
  const int seq = t3 % p.num_seqs;
  const int t_desc = t3 / p.num_seqs;
  const int qa = p.cu_q[seq], qe = p.cu_q[seq + 1];
  const int n_tiles = (qe - qa + kRows - 1) / kRows;
  if (t_desc >= n_tiles) return;
  const int row0 = qa + (n_tiles - 1 - t_desc) * kRows;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int gp = wave >> 2, wq = wave & 3;  // group, 32-row block
  const int lr = lane & 31, lc = lane >> 5;
  const int h = kvh * p.g + 2 * pair + gp;

  // ---- rows and positions (both groups see the same rows)
  const int my_row = row0 + 32 * wq + lr;
  const bool row_ok = my_row < qe;
  const int wave_first = row0 + 32 * wq;
  const bool wave_active = wave_first < qe;
  const int wave_last = min(wave_first + 31, qe - 1);
  const int blk_last = min(row0 + kRows - 1, qe - 1);
  int my_pos, wave_qmin, wave_qmax, blk_qmax;
  if (p.causal) {
    my_pos = row_ok ? p.q_pos[my_row] : INT_MIN;
    wave_qmin = __builtin_amdgcn_readfirstlane(wave_active ? p.q_pos[wave_first] : INT_MIN);
    wave_qmax = __builtin_amdgcn_readfirstlane(wave_active ? p.q_pos[wave_last] : INT_MIN);
    blk_qmax = p.q_pos[blk_last];
  } else {
    my_pos = row_ok ? INT_MAX - 1 : INT_MIN;
    wave_qmin = wave_qmax = wave_active ? INT_MAX - 1 : INT_MIN;
    blk_qmax = INT_MAX - 1;
  }

  // ---- key segments: the workgroup's own shard, or (MERGED) every shard in
  // turn. A segment holds the keys [ka, end) of its shard that some row of
  // the workgroup can see; its 64-key tiles are consecutive tiles of the
  // walk. One online softmax runs over the whole walk, so a MERGED workgroup
  // ends with the exact merge of the shards' partials.
  __shared__ int seg_sh[MERGED ? kMaxShards : 1][3];  // ka, end, first tile of the walk
  auto seg_range = [&](int sh, int& ka, int& ke) {
    if constexpr (PAGED) {
      ka = 0;
      ke = min(p.local_kv_lens[seq], p.max_blocks * 16);  // never index past the block table
      if (p.causal) ke = min(ke, rr_count_below(blk_qmax + 1, p.cp, p.rank, p.il));
    } else {
      ka = p.cu_k[sh][seq];
      ke = p.cu_k[sh][seq + 1];
      if (p.causal) ke = ka + pp_count_le<kThreads>(p.k_pos[sh] + ka, ke - ka, blk_qmax);
    }
  };
  int seg0_ka = 0, seg0_end = 0, n = 0;  // n: tiles of the walk
  if constexpr (!MERGED) {
    if (!PAGED && pre_n >= 0) {
      // the pre-pass counted the key tiles whose first key some row sees; the
      // last of them may hold keys past the visible end, which the per-key
      // mask removes like any other masked key
      seg0_ka = p.cu_k[shard][seq];
      seg0_end = min(seg0_ka + pre_n * kBN, p.cu_k[shard][seq + 1]);
      n = pre_n;
    } else {
      seg_range(shard, seg0_ka, seg0_end);
      n = seg0_end > seg0_ka ? (seg0_end - seg0_ka + kBN - 1) / kBN : 0;
    }
  } else {
    for (int sg = 0; sg < p.n_shards; ++sg) {
      int ka, ke;
      seg_range(sg, ka, ke);
      if (tid == 0) {
        seg_sh[sg][0] = ka;
        seg_sh[sg][1] = ke;
        seg_sh[sg][2] = n;
      }
      n += ke > ka ? (ke - ka + kBN - 1) / kBN : 0;
    }
    __syncthreads();
  }
  // Tiles t < n_fast need no position read in the matrix phase: every key of
  // them is visible to every row of the workgroup. A shard's key positions
  // increase strictly, and tile t+3 < n starts at or below blk_qmax, so tile
  // t ends below blk_qmax - 128; when the workgroup's rows hold consecutive
  // positions (the first at blk_qmax - (blk_last - row0)), that is below every
  // row's position. (Not for a walk over several shards, whose positions do
  // not increase across shards.)
  int n_fast = 0;
  if constexpr (!MERGED) {
    if (!p.causal) {
      n_fast = max(0, n - 1);  // only a partial last tile has masked keys
    } else if (blk_qmax - p.q_pos[row0] == blk_last - row0) {
      n_fast = max(0, n - 3);
    }
  }
  // tile t of the walk: its shard's K, V and positions, first key index, end of the visible keys
  struct TileRef {
    const uint16_t* k;
    const uint16_t* v;
    const int* kp;
    int j0, end;
  };
  // MERGED: a cursor over the segments that only moves forward (tiles are
  // staged in walk order), so each tile costs one comparison
  int cur_sg = -1, cur_ka = 0, cur_end = 0, cur_base = 0, cur_next = 0;
  auto tile_ref = [&](int t) -> TileRef {
    if constexpr (!MERGED) {
      return TileRef{p.k[shard], p.v[shard], p.k_pos[shard], seg0_ka + t * kBN, seg0_end};
    } else {
      while (t >= cur_next) {
        ++cur_sg;
        cur_ka = __builtin_amdgcn_readfirstlane(seg_sh[cur_sg][0]);
        cur_end = __builtin_amdgcn_readfirstlane(seg_sh[cur_sg][1]);
        cur_base = __builtin_amdgcn_readfirstlane(seg_sh[cur_sg][2]);
        cur_next = cur_sg + 1 < p.n_shards ? __builtin_amdgcn_readfirstlane(seg_sh[cur_sg + 1][2]) : INT_MAX;
      }
      return TileRef{p.k[cur_sg], p.v[cur_sg], p.k_pos[cur_sg], cur_ka + (t - cur_base) * kBN, cur_end};
    }
  };

  // ---- Q^T fragments
  bf16x8 qf[D / 16];
  {
    const int qrow = row_ok ? my_row : qa;
    const uint16_t* src = p.q + ((int64_t)qrow * p.hq + h) * D + 8 * lc;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(src + 16 * kk);
  }

  // ---- slot staging: load instruction i of this wave fills tile rows
  // ld_row(i) .. ld_row(i) + kRowsPerLoad - 1 of a matrix; this lane fetches
  // the piece of row ld_row(i) + lane / kChunksPerRow that belongs at its
  // place in the swizzled row
  const int ld_rowbase = wave * T::kLoads * T::kRowsPerLoad + lane / T::kChunksPerRow;
  auto ld_row = [&](int i) { return ld_rowbase + i * T::kRowsPerLoad; };
  auto ld_piece = [&](int i) { return (lane % T::kChunksPerRow) ^ T::swz(ld_row(i)); };
  // LDS byte address of load instruction i of this wave in the matrix that
  // starts mat_off elements into smem (wave-uniform)
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)smem + (uint32_t)wave * T::kLoads * 1024u);
  auto ld_lds = [&](int mat_off, int i) { return wave_lds + (uint32_t)mat_off * 2u + (uint32_t)i * 1024u; };
  const int64_t row_stride = (int64_t)p.hkv * D;
  // paged: physical block of this wave's rows in the next slot's K tile and
  // in its V tile, read one slot ahead. A wave loads kWaveRows consecutive
  // rows of a tile starting at a multiple of kWaveRows, a divisor of 16, so
  // clamped to the visible range or not its rows lie in one 16-key block:
  // that of its clamped first row.
  constexpr int kWaveRows = T::kLoads * T::kRowsPerLoad;
  static_assert(16 % kWaveRows == 0, "a wave's rows of a tile must share a 16-key block");
  int pre_k = 0, pre_v = 0;
  // contiguous shards: byte offset of this lane's piece of load instruction i
  // from the start of the tile's first row, the same in every tile that needs
  // no clamping
  uint32_t ld_off[T::kLoads];
#pragma unroll
  for (int i = 0; i < T::kLoads; ++i) ld_off[i] = (uint32_t)(ld_row(i) * (int)row_stride + ld_piece(i) * 8) * 2u;
  const int kvh_u = __builtin_amdgcn_readfirstlane(kvh);
  // direct global->LDS loads of one matrix tile; rows past the visible range
  // are clamped to its last row. In a contiguous shard a tile with every row
  // visible (all but the last) is addressed from a uniform base, with no
  // vector arithmetic (paged tiles measured slower that way: their base waits
  // on the block-table read).
  auto load_mat = [&](const uint16_t* __restrict__ src, const TileRef& tr, int blk, int mat) {
    const int j0 = tr.j0, n_end = tr.end;
    if constexpr (!PAGED) {
      if (__builtin_amdgcn_readfirstlane(j0 + kBN <= n_end)) {
        const uint16_t* base = src + (int64_t)__builtin_amdgcn_readfirstlane(j0) * row_stride + kvh_u * D;
#pragma unroll
        for (int i = 0; i < T::kLoads; ++i) lds_dma16_s(base, ld_off[i], ld_lds(mat, i));
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
      const int j = min(j0 + ld_row(i), n_end - 1);
      const uint16_t* g;
      if constexpr (PAGED) {
        g = src + ((int64_t)blk * p.hkv + kvh) * 16 * D + (j & 15) * D + ld_piece(i) * 8;
      } else {
        g = src + (int64_t)j * row_stride + kvh * D + ld_piece(i) * 8;
      }
      lds_dma16(g, ld_lds(mat, i));
    }
  };
  // The table is read with uniform indices, through the scalar cache
  // (consecutive tiles read consecutive entries). A tile outside the walk
  // (tile n, or tile -1 before the first V) reads an entry inside the table
  // that no load then uses.
  auto prefetch_tab = [&](int tk, int tv) {  // K tile tk, V tile tv
    if constexpr (PAGED) {
      using ctab_t = const __attribute__((address_space(4))) int*;
      const ctab_t tab = (ctab_t)(p.block_table + (int64_t)seq * p.max_blocks);
      const int w_row0 = wave * kWaveRows;
      const int last = __builtin_amdgcn_readfirstlane(seg0_end - 1);
      const int bk = __builtin_amdgcn_readfirstlane(max(0, min(tk * kBN + w_row0, last)) >> 4);
      const int bv = __builtin_amdgcn_readfirstlane(max(0, min(tv * kBN + w_row0, last)) >> 4);
      pre_k = tab[bk];
      pre_v = tab[bv];
    }
  };
  // position of key tid of the tile (tid < 64): read (or derived) when the
  // slot's loads are issued, finished when it is stored (INT_MAX past the
  // end). The register is written only by the load itself, so issuing it
  // never waits on the previous slot's read of the same register.
  auto key_pos_issue = [&](const TileRef& tr) -> int {
    const int j = min(tr.j0 + tid, tr.end - 1);
    if constexpr (PAGED) return rr_global_pos(j, p.cp, p.rank, p.il);
    else return p.causal ? tr.kp[j] : 0;
  };
  int kp_j0 = 0, kp_end = 0;  // tile of the pending position read
  auto kslot = [&](int s) { return smem + s * T::kSlotElems; };
  auto vslot = [&](int s) { return smem + s * T::kSlotElems + T::kKElems; };

  int kp_reg = INT_MAX;
  // slot t = {K(t), V(t-1), positions of tile t}
  // slots are loaded for t = 0, 1, ..., n in order; the V of a slot is the
  // previous tile's, whose reference the last call kept
  TileRef prev_tr{};
  auto load_slot = [&](int t) {
    TileRef tr{};
    if (t < n) {
      tr = tile_ref(t);
      // positions first: any wait the compiler puts before reusing their
      // register then precedes this slot's tile loads
      if (tid < kBN) {
        if constexpr (PAGED) {
          kp_reg = key_pos_issue(tr);
        } else if (p.causal) {
          kp_reg = tr.kp[min(tr.j0 + tid, tr.end - 1)];
        }
        kp_j0 = tr.j0;
        kp_end = tr.end;
      }
      load_mat(tr.k, tr, pre_k, (t & 1) * T::kSlotElems);
    }
    if (t >= 1) {
      const TileRef vr = MERGED ? prev_tr : tile_ref(t - 1);
      load_mat(vr.v, vr, pre_v, (t & 1) * T::kSlotElems + T::kKElems);
    }
    prev_tr = tr;
  };
  // the slot's tiles are in LDS once this wave's loads have completed (and,
  // for the other waves, after the barrier that follows)
  auto store_slot = [&](int t) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    if (t < n && tid < kBN) {
      const int kp = PAGED || p.causal ? kp_reg : 0;
      kpos_sh[t & 3][tid] = kp_j0 + tid >= kp_end ? INT_MAX : kp;
    }
    // paged: the blocks of the next slot (K(t+1), V(t)), read here at the end
    // of a phase, not on the way into the matrix work
    prefetch_tab(t + 1, t);
  };

  // ---- per-wave state
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float sl2 = p.scale_log2;
  constexpr float kTau = 8.f;  // lazy-rescale threshold (log2 units)
  f32x16 s0 = {}, s1 = {};  // S(t) after phase A, P(t) in fp32 after phase B
  bool p_valid = false;     // s0/s1 hold P of the previous tile for this wave
  bool b_valid = false, b_mask = false;  // tile of the next B phase: any key visible / some masked

  // K operand k-step kk: row lr (+32 for the second key half), piece 2 kk + lc
  int k_off[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = lr * D + 8 * ((2 * kk + lc) ^ T::swz(lr));
  // V^T operand (d-block db, k-step kst) from two transposing reads: within
  // each 16 lanes, lane j16 names 4 bf16 of key row 4 lc + j16/4 (+8 for the
  // second read, +16 kst), dims 32 db + 16 (g16 & 1) + 4 (j16 & 3); a lane
  // receives 4 consecutive keys of dim 32 db + lr, which is the key order of
  // its P values in the S^T accumulator
  const int g16 = lane >> 4, j16 = lane & 15;
  int v_off[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 4 * lc + (j16 >> 2) + 8 * hi;
      const int piece = 4 * db + 2 * (g16 & 1) + ((j16 >> 1) & 1);
      v_off[db][hi] = r * D + 8 * (piece ^ T::swz(r)) + 4 * (j16 & 1);
    }
  }

  // A(t): O += V(t-1)^T P(t-1)^T, then S(t)^T = K(t) Q^T. The bf16 packing of
  // P(t-1) and its row sum run here, under the matrix work, to keep the
  // softmax phase short.
  //
  // PV operand i: d-block i % (D/32), k-step i / (D/32) (consecutive MFMAs
  // accumulate into different d-blocks). QK operand i: key half i % 2, d-step
  // i / 2 (the two accumulators alternate). When both run, they form one
  // pipeline of 4 D/32 + D/8 MFMAs whose LDS operands are read kRing MFMAs
  // ahead from a single register ring, so the first K reads are in flight
  // while the PV MFMAs run. The row sum of P is a pairwise tree whose adds
  // are spread over the PV MFMAs.
  auto phase_a_body = [&](int t) {
    // the wave feeding the matrix core issues first when both waves of a
    // SIMD have an instruction ready (by default the older wave would)
    __builtin_amdgcn_s_setprio(2);
    const int s = t & 1;
    const bool do_pv = t >= 1 && p_valid;
    const bool do_qk =
        t < n && (t < n_fast ? wave_active : __builtin_amdgcn_readfirstlane(kpos_sh[t & 3][0]) <= wave_qmax);
    b_valid = do_qk;  // B(t) has work iff some key of tile t is visible to this wave
    const uint16_t* vs = vslot(s);
    const uint16_t* ks = kslot(s);
    constexpr int kPV = 4 * (D / 32), kQK = D / 8, kRing = 6;
    constexpr int kSumPer = (31 + kPV - 1) / kPV;  // row-sum adds per PV MFMA
    auto vop = [&](int i) {
      const int db = i % (D / 32), kst = i / (D / 32);
      const s16x4 lo = lds_read_tr(vs + 16 * kst * D + v_off[db][0]);
      const s16x4 hi = lds_read_tr(vs + 16 * kst * D + v_off[db][1]);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto kop = [&](int i) { return *(const bf16x8*)(ks + (i & 1) * 32 * D + k_off[i >> 1]); };
    bf16x8 pb[4];
    float sums[31];  // [0, 16): s0[v] + s1[v]; node a >= 16: sums[2(a-16)] + sums[2(a-16)+1]
    auto pack_p = [&]() {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[0][e] = (__bf16)s0[e];
        pb[1][e] = (__bf16)s0[8 + e];
        pb[2][e] = (__bf16)s1[e];
        pb[3][e] = (__bf16)s1[8 + e];
      }
    };
    auto sum_step = [&](int a) {
      if (a < 16) sums[a] = s0[a] + s1[a];
      else if (a < 31) sums[a] = sums[2 * (a - 16)] + sums[2 * (a - 16) + 1];
    };
    auto pv_mfma = [&](int i, const bf16x8& a) {
      const int db = i % (D / 32), kst = i / (D / 32);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kst], oacc[db], 0, 0, 0);
    };
    auto qk_mfma = [&](int i, const bf16x8& a) {
      if (i & 1) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i >> 1], i < 2 ? f32x16{} : s1, 0, 0, 0);
      else s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i >> 1], i < 2 ? f32x16{} : s0, 0, 0, 0);
    };
    if (do_pv && do_qk) {
      auto op = [&](int j) { return j < kPV ? vop(j) : kop(j - kPV); };
      bf16x8 ring[kRing];
#pragma unroll
      for (int j = 0; j < kRing; ++j) ring[j] = op(j);
      pack_p();
#pragma unroll
      for (int j = 0; j < kPV + kQK; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        if (j < kPV) pv_mfma(j, ring[j % kRing]);
        else qk_mfma(j - kPV, ring[j % kRing]);
        if (j + kRing < kPV + kQK) ring[j % kRing] = op(j + kRing);
        if (j < kPV) {
#pragma unroll
          for (int u = 0; u < kSumPer; ++u) sum_step(kSumPer * j + u);
        }
      }
      l_run += sums[30];
      return;
    }
    if (do_pv) {
      bf16x8 ring[kRing];
#pragma unroll
      for (int j = 0; j < kRing; ++j) ring[j] = vop(j);
      pack_p();
#pragma unroll
      for (int j = 0; j < kPV; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        pv_mfma(j, ring[j % kRing]);
        if (j + kRing < kPV) ring[j % kRing] = vop(j + kRing);
#pragma unroll
        for (int u = 0; u < kSumPer; ++u) sum_step(kSumPer * j + u);
      }
      l_run += sums[30];
    }
    if (do_qk) {
      bf16x8 ring[kRing];
#pragma unroll
      for (int j = 0; j < kRing; ++j) ring[j] = kop(j);
#pragma unroll
      for (int j = 0; j < kQK; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        qk_mfma(j, ring[j % kRing]);
        if (j + kRing < kQK) ring[j % kRing] = kop(j + kRing);
      }
    }
  };

  // the flags B(t) needs, read here after the matrix work is issued rather
  // than as the first (dependent) LDS reads of the softmax phase
  auto phase_a = [&](int t) {
    phase_a_body(t);
    b_mask = b_valid && t >= n_fast && __builtin_amdgcn_readfirstlane(kpos_sh[t & 3][kBN - 1]) > wave_qmin;
  };

  // B(t): mask and online softmax of S(t) -> P(t) (fp32, in place)
  auto phase_b = [&](int t) {
    __builtin_amdgcn_s_setprio(0);
    const int* kp = kpos_sh[t & 3];
    p_valid = b_valid;
    if (!p_valid) return;
    // accumulator element v of this lane holds key 8*(v/4) + 4*lc + v%4 (+32 for s1)
    if (b_mask) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 8 * (v >> 2) + 4 * lc + (v & 3);
        if (kp[key] > my_pos) s0[v] = kNegInf;
        if (kp[32 + key] > my_pos) s1[v] = kNegInf;
      }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = pp_max3(mx, s0[v], s1[v]);
    mx = pp_half_max(mx) * sl2;
    if (__ballot(mx > m_run + kTau) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : hw_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float base = (m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s0[v] = hw_exp2(fmaf(s0[v], sl2, -base));
      s1[v] = hw_exp2(fmaf(s1[v], sl2, -base));
    }
  };

  if (n > 0) {
    prefetch_tab(0, -1);
    load_slot(0);
    store_slot(0);
    __syncthreads();
    // phases 0 .. 2n+1; group 0 runs A(t) in phase 2t and B(t) in 2t+1,
    // group 1 one phase later; slot t+1 is loaded during phases 2t, 2t+1.
    // Only odd phases end in a barrier: a wave may then run a phase ahead of
    // the other group, which is why the positions of a tile have four
    // buffers (tile t's are read until phase 2t+2 and rewritten for tile t+4)
    // while K and V need two (slot t+1's buffer is last read in phase 2t-1)
    for (int ph = 0; ph <= 2 * n + 1; ++ph) {
      const int t_ld = ph >> 1;
      if (!(ph & 1) && t_ld + 1 <= n) load_slot(t_ld + 1);
      const int q = ph - gp;  // this group's own phase index
      if (q >= 0 && q <= 2 * n) {
        if (!(q & 1)) phase_a(q >> 1);
        else phase_b(q >> 1);
      }
      if (ph & 1) {
        if (t_ld + 1 <= n) store_slot(t_ld + 1);
        // the last phase publishes no slot and no LDS is read after it, so
        // group 0 goes on to its epilogue while group 1 runs its last PV
        if (ph < 2 * n + 1) lds_barrier();
      }
    }
  }

  // ---- epilogue
  const float l_tot = pp_half_sum(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t obase = ((int64_t)my_row * p.hq + h) * D;
  if constexpr (!PAGED && !MERGED) {
    if (p.o_acc) {
      // exact merge of (o_acc, lse_acc) with this partial, in base 2: weights
      // 2^(lse_s - lse) with lse = M + log2(sum_s 2^(lse_s - M)); an empty side
      // (LSE -inf) has weight 0 and its O does not enter the sum
      const int64_t li = (int64_t)my_row * p.hq + h;
      const float lse_new = l_tot > 0.f ? m_run + hw_log2(l_tot) : kNegInf;
      const float lse_old = p.lse_acc[li] * kLog2e;
      // the old O is loaded together with its LSE rather than after it: a row
      // whose LSE is -inf has its loaded values replaced by zero bits (an
      // integer select, which no floating-point simplification can drop)
      u32x4 old_bits[D / 32][4];
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) old_bits[db][q4] = *(const u32x4*)(p.o_acc + obase + 32 * db + 8 * q4 + 4 * lc);
      const float mx = fmaxf(lse_old, lse_new);
      float w_old = 0.f, c_new = 0.f, lse_m = kNegInf;
      if (mx != kNegInf) {
        const float e_old = hw_exp2(lse_old - mx), e_new = hw_exp2(lse_new - mx);
        const float sum = e_old + e_new;
        lse_m = mx + hw_log2(sum);
        w_old = e_old / sum;
        c_new = (e_new / sum) * inv;
      }
      const bool use_old = lse_old != kNegInf;
      // an empty partial leaves a non-empty accumulator as it is (weight 1 on
      // the old side, exactly): only the copy in o_out is written then
      const bool write_acc = lse_new != kNegInf || !use_old;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * db + 8 * q4 + 4 * lc;
          const u32x4 ob = use_old ? old_bits[db][q4] : u32x4{0u, 0u, 0u, 0u};
          f32x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = fmaf(w_old, __uint_as_float(ob[e]), c_new * oacc[db][4 * q4 + e]);
          if (write_acc) *(f32x4*)(p.o_acc + obase + d0) = val;
          if (p.o[0]) {
            if constexpr (OUT_BF16) {
              const u32x2 w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
              *(u32x2*)((uint16_t*)p.o[0] + obase + d0) = w;
            } else {
              *(f32x4*)((float*)p.o[0] + obase + d0) = val;
            }
          }
        }
      }
      if (lc == 0 && write_acc) p.lse_acc[li] = lse_m * kLn2;
      return;
    }
  }
  if constexpr (PAGED) {
    if (p.n_fold > 0 || p.own_o || p.own_lse) {
      // this rank's partial merged with the other ranks' partials of the row,
      // by the rule of the LSE merge in base 2: weights 2^(lse_s - lse) with
      // lse = M + log2(sum_s 2^(lse_s - M)); a part with LSE -inf has weight 0
      // and its O is not read
      const int64_t li = (int64_t)my_row * p.hq + h;
      const float lse_own = l_tot > 0.f ? m_run + hw_log2(l_tot) : kNegInf;
      if (p.own_o) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * db + 8 * q4 + 4 * lc;
            const f32x4 val = {oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv, oacc[db][4 * q4 + 2] * inv,
                               oacc[db][4 * q4 + 3] * inv};
            if (p.fold_bf16) {
              const u32x2 w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
              *(u32x2*)((uint16_t*)p.own_o + obase + d0) = w;
            } else {
              *(f32x4*)((float*)p.own_o + obase + d0) = val;
            }
          }
        }
      }
      if (p.own_lse && lc == 0) p.own_lse[li] = lse_own * kLn2;
      float mx = lse_own;
      for (int j = 0; j < p.n_fold; ++j) mx = fmaxf(mx, p.fold_lse[j][li] * kLog2e);
      float lt = kNegInf;
      if (mx == kNegInf) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
      } else {
        float sum = hw_exp2(lse_own - mx);
        for (int j = 0; j < p.n_fold; ++j) sum += hw_exp2(p.fold_lse[j][li] * kLog2e - mx);
        lt = mx + hw_log2(sum);
        const float w_own = hw_exp2(lse_own - lt) * inv;  // oacc is not yet normalised
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= w_own;
        for (int j = 0; j < p.n_fold; ++j) {
          const float w = hw_exp2(p.fold_lse[j][li] * kLog2e - lt);
          if (w != 0.f) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = 32 * db + 8 * q4 + 4 * lc;
                f32x4 x;
                if (p.fold_bf16) {
                  const u32x2 r = *(const u32x2*)((const uint16_t*)p.fold_o[j] + obase + d0);
                  x = f32x4{bf16_lo(r[0]), bf16_hi(r[0]), bf16_lo(r[1]), bf16_hi(r[1])};
                } else {
                  x = *(const f32x4*)((const float*)p.fold_o[j] + obase + d0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) oacc[db][4 * q4 + e] = fmaf(w, x[e], oacc[db][4 * q4 + e]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * db + 8 * q4 + 4 * lc;
          const f32x4 val = {oacc[db][4 * q4], oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]};
          if constexpr (OUT_BF16) {
            const u32x2 w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
            *(u32x2*)((uint16_t*)p.o[0] + obase + d0) = w;
          } else {
            *(f32x4*)((float*)p.o[0] + obase + d0) = val;
          }
        }
      }
      if (lc == 0) p.lse[0][li] = lt * kLn2;
      return;
    }
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * lc;
      const f32x4 val = {oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv, oacc[db][4 * q4 + 2] * inv,
                         oacc[db][4 * q4 + 3] * inv};
      if constexpr (OUT_BF16) {
        const u32x2 w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
        *(u32x2*)((uint16_t*)p.o[shard] + obase + d0) = w;
      } else {
        *(f32x4*)((float*)p.o[shard] + obase + d0) = val;
      }
    }
  }
  if (lc == 0) p.lse[shard][(int64_t)my_row * p.hq + h] = l_tot > 0.f ? (m_run + hw_log2(l_tot)) * kLn2 : kNegInf;
}

// ---- launch order, heaviest tile units first (contiguous shards)
//
// A tile unit is (query tile, sequence, shard); its work is the number of
// 64-key tiles some row of it can see. With causal masks over zigzag shards
// that work differs by an order of magnitude between units, and running the
// heaviest first keeps the tail of the launch short. One workgroup counts
// every unit's key tiles (a binary search over the first positions of the
// shard's key tiles) and counting-sorts the units by it, descending. Units
// of equal work keep no particular order; the results do not depend on it.
// When the launch holds several shards and is long against its heaviest
// unit (each CU's share of the key tiles at least kShardMajorRatio times the
// heaviest unit's), the order is shard-major instead, heaviest first within
// each shard (counts from 511 tiles up rank as equal there): the workgroups
// running together then read the K/V of one shard, which the L2 keeps, and
// the heavy units of the last shard still start early enough for the end of
// the launch to stay short. Each entry also carries the unit's count, so the
// attention kernel starts its first tile loads without searching the key
// positions itself.
constexpr int kSchedThreads = 1024;
constexpr int kSchedBuckets = 4096;
constexpr int kSchedMaxUnits = 8192;
constexpr int kShardMajorRatio = 12;

// wg_per_unit: workgroups per unit (KV heads x head pairs); n_cus: compute
// units of the device
__global__ __launch_bounds__(kSchedThreads) void pp_schedule_kernel(PPParams p, int n_units, int merged,
                                                                     int wg_per_unit, int n_cus, int* order) {
  static_assert(kSchedMaxUnits <= 1 << kOrderUnitBits, "unit index must fit its field");
  __shared__ int bucket[kSchedBuckets];
  __shared__ int work_sh[kSchedMaxUnits];
  __shared__ int wave_tot[kSchedThreads / 64];
  __shared__ unsigned long long total_sh;
  __shared__ int max_sh;
  const int tid = threadIdx.x;
  for (int b = tid; b < kSchedBuckets; b += kSchedThreads) bucket[b] = 0;
  if (tid == 0) {
    total_sh = 0;
    max_sh = 0;
  }
  __syncthreads();
  // a unit is (tile_desc, seq, shard), or (tile_desc, seq) when merged (its
  // work is then summed over the shards it walks)
  const int n_sh_unit = merged ? 1 : p.n_shards;
  for (int u = tid; u < n_units; u += kSchedThreads) {
    const int t3 = u / n_sh_unit;
    const int seq = t3 % p.num_seqs;
    const int t_desc = t3 / p.num_seqs;
    const int qa = p.cu_q[seq], qe = p.cu_q[seq + 1];
    const int n_tiles = (qe - qa + kRows - 1) / kRows;
    int work = 0;
    if (t_desc < n_tiles) {
      const int row0 = qa + (n_tiles - 1 - t_desc) * kRows;
      const int qmax = p.causal ? p.q_pos[min(row0 + kRows - 1, qe - 1)] : 0;
      const int sh0 = merged ? 0 : u % p.n_shards, sh1 = merged ? p.n_shards : sh0 + 1;
      for (int shard = sh0; shard < sh1; ++shard) {
        const int ka = p.cu_k[shard][seq], ke = p.cu_k[shard][seq + 1];
        const int nk = (ke - ka + kBN - 1) / kBN;
        if (!p.causal) {
          work += nk;
        } else {
          const int* kp = p.k_pos[shard] + ka;
          int lo = 0, hi = nk;  // key tiles whose first key is visible: [0, lo)
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (kp[mid * kBN] <= qmax) lo = mid + 1;
            else hi = mid;
          }
          work += lo;
        }
      }
    }
    work_sh[u] = work;
    atomicAdd(&total_sh, (unsigned long long)work);
    atomicMax(&max_sh, work);
  }
  __syncthreads();
  // sort key: the work, or (shard-major) the shard's rank above the work
  constexpr int kPerShard = kSchedBuckets / kMaxShards;
  const bool shard_major = !merged && p.n_shards > 1 &&
                           total_sh * (unsigned long long)wg_per_unit >=
                               (unsigned long long)kShardMajorRatio * (unsigned long long)max_sh * n_cus;
  auto key = [&](int u) {
    const int work = work_sh[u];
    if (!shard_major) return min(work, kSchedBuckets - 1);
    return (p.n_shards - 1 - u % p.n_shards) * kPerShard + min(work, kPerShard - 1);
  };
  for (int u = tid; u < n_units; u += kSchedThreads) atomicAdd(&bucket[key(u)], 1);
  __syncthreads();
  // exclusive scan over the buckets in descending key order: thread t owns
  // the four buckets 4095-4t .. 4092-4t
  constexpr int kPer = kSchedBuckets / kSchedThreads;
  int c[kPer], run = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    c[j] = bucket[kSchedBuckets - 1 - (kPer * tid + j)];
    run += c[j];
  }
  int incl = run;  // inclusive scan of `run` over the threads
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = incl - run;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    bucket[kSchedBuckets - 1 - (kPer * tid + j)] = base;
    base += c[j];
  }
  __syncthreads();
  for (int u = tid; u < n_units; u += kSchedThreads) {
    const int work = work_sh[u];
    order[atomicAdd(&bucket[key(u)], 1)] =
        u | (min(work, kOrderWorkUnknown) << kOrderUnitBits);
  }
}

// Launch-order scratch of cpa_partial_attn_multi_noalloc: one entry per tile
// unit, written in full by the pre-pass before the attention kernel reads it.
// Host code never uses this name as an address: the address comes from
// hipGetSymbolAddress (attn_pp_scratch), per device.
static __device__ __align__(256) int scratch[kSchedMaxUnits];

template <int D, bool PAGED, bool OUT_BF16, bool MERGED = false>
void pp_launch(const PPParams& p, uint32_t blocks, hipStream_t st) {
  hipLaunchKernelGGL((attn_pp_kernel<D, PAGED, OUT_BF16, MERGED>), dim3(blocks), dim3(kThreads), 0, st, p);
}

}  // namespace

bool attn_pp_supported(const AttnArgs& a) { return (a.hq / a.hkv) % 2 == 0; }

int attn_pp_scratch_units() { return kSchedMaxUnits; }

cpa_status attn_pp_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CPA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(CPA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !a)
      return fail(CPA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = a;
  }
  *ptr = addr[dev];
  *bytes = sizeof(scratch);
  return CPA_OK;
}

int64_t attn_pp_tile_units(int n_shards, int num_seqs, int max_q) {
  return cdiv(max_q, kRows) * (int64_t)num_seqs * n_shards;
}

size_t attn_pp_order_bytes(int n_shards, int num_seqs, int max_q) {
  const int64_t units = attn_pp_tile_units(n_shards, num_seqs, max_q);
  if (units <= 0 || units > kSchedMaxUnits) return 0;
  return (size_t)cdiv(units * (int64_t)sizeof(int), 256) * 256;
}

cpa_status launch_attn_pp(const AttnArgs* shards, int n_shards, bool paged, hipStream_t st, void* order_ws,
                          size_t order_ws_bytes, const MergedOut* merged, const AccumIO* accum, const RankFold* fold) {
  if (merged && paged) return fail(CPA_ERR_INVALID_ARG, "partial attention: a merged walk needs contiguous shards");
  if (fold && (!paged || n_shards != 1 || fold->n < 0 || fold->n > kMaxFoldParts))
    return fail(CPA_ERR_INVALID_ARG, "partial attention: folding other ranks' partials needs one paged shard");
  if (accum && (paged || merged || n_shards != 1))
    return fail(CPA_ERR_INVALID_ARG, "partial attention: a running merge takes one contiguous shard");
  if (n_shards < 1 || n_shards > kMaxShards) return fail(CPA_ERR_INVALID_ARG, "partial attention: bad shard count");
  const AttnArgs& a = shards[0];
  PPParams p{};
  p.q = (const uint16_t*)a.q;
  p.q_pos = a.q_pos;
  p.cu_q = a.cu_q;
  p.n_shards = n_shards;
  for (int i = 0; i < n_shards; ++i) {
    p.k[i] = (const uint16_t*)shards[i].k;
    p.v[i] = (const uint16_t*)shards[i].v;
    p.k_pos[i] = shards[i].k_pos;
    p.cu_k[i] = shards[i].cu_k;
    p.o[i] = shards[i].o;
    p.lse[i] = shards[i].lse;
  }
  if (merged) {  // one output: the exact merge over all shards
    p.o[0] = merged->o;
    p.lse[0] = merged->lse;
  }
  if (accum) {  // fold into the running (O, LSE); o[0] is the optional merged copy
    p.o_acc = accum->o_acc;
    p.lse_acc = accum->lse_acc;
    p.o[0] = accum->o_out;
    p.lse[0] = nullptr;
  }
  if (fold) {
    p.n_fold = fold->n;
    p.fold_bf16 = fold->part_bf16;
    for (int j = 0; j < fold->n; ++j) {
      p.fold_o[j] = fold->o[j];
      p.fold_lse[j] = fold->lse[j];
    }
    p.own_o = fold->own_o;
    p.own_lse = fold->own_lse;
  }
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
  const int64_t n_groups = cdiv(a.max_q, kRows) * a.num_seqs * (merged ? 1 : n_shards) * a.hkv;
  const int64_t blocks = cdiv(n_groups, 8) * 8 * (p.g / 2);
  if (blocks > INT32_MAX) return fail(CPA_ERR_INVALID_ARG, "partial attention: problem too large for one launch");
  p.n_groups = (int)n_groups;
  if (blocks == 0) return CPA_OK;
  const uint32_t nb = (uint32_t)blocks;
  const size_t order_bytes = paged ? 0 : attn_pp_order_bytes(n_shards, a.num_seqs, a.max_q);
  if (order_bytes > 0 && order_ws && order_ws_bytes >= order_bytes) {
    p.order = (const int*)order_ws;
    const int n_units = (int)(n_groups / a.hkv);
    int dev = 0, n_cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return fail(CPA_ERR_HIP, "partial attention: cannot read the device's compute-unit count");
    hipLaunchKernelGGL(pp_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, st, p, n_units, merged ? 1 : 0,
                       a.hkv * (p.g / 2), n_cus, (int*)order_ws);
  }
  if (merged) {
    if (a.d == 64) merged->o_bf16 ? pp_launch<64, false, true, true>(p, nb, st) : pp_launch<64, false, false, true>(p, nb, st);
    else merged->o_bf16 ? pp_launch<128, false, true, true>(p, nb, st) : pp_launch<128, false, false, true>(p, nb, st);
    return check_launch("cpa_partial_attn_merged");
  }
  if (a.d == 64) {
    if (paged) a.o_bf16 ? pp_launch<64, true, true>(p, nb, st) : pp_launch<64, true, false>(p, nb, st);
    else a.o_bf16 ? pp_launch<64, false, true>(p, nb, st) : pp_launch<64, false, false>(p, nb, st);
  } else {
    if (paged) a.o_bf16 ? pp_launch<128, true, true>(p, nb, st) : pp_launch<128, true, false>(p, nb, st);
    else a.o_bf16 ? pp_launch<128, false, true>(p, nb, st) : pp_launch<128, false, false>(p, nb, st);
  }
  return check_launch(paged ? "cpa_partial_attn_paged (prefill)"
                             : (accum ? "cpa_partial_attn_accumulate" : "cpa_partial_attn (bf16)"));
}

}  // namespace cpa
