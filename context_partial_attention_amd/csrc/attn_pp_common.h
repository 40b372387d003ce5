// Shared pieces of the bf16 prefill kernel (attn_pp.hip) and its helpers:
// tile geometry and LDS layout of the K/V tiles, the kernel parameters, the
// launch-order encoding, and small device helpers. Internal to the library.
#pragma once

#include "cpa_internal.h"
#include "device_common.h"

namespace cpa {
namespace pp {

constexpr int kBN = 64;        // keys per tile
constexpr int kRows = 128;     // query rows per workgroup (per head)
// launch-order entry: unit index in the low bits, its visible key-tile count
// above them (kOrderWorkUnknown when it does not fit)
constexpr int kOrderUnitBits = 13;
constexpr int kOrderUnitMask = (1 << kOrderUnitBits) - 1;
constexpr int kOrderWorkUnknown = (1 << (31 - kOrderUnitBits)) - 1;

// NT: threads of the workgroup that stages the tile
template <int D, int NT>
struct PPTile {
  // K and V tiles are stored row-major ([64 keys][D], no padding) as the
  // global->LDS loads write them: each load instruction fills 1 KiB of LDS
  // with 16 bytes per lane in lane order, and which 16-byte piece of a row a
  // lane fetches sets the layout. Pieces are swizzled within a row (the
  // piece index is XORed with swz(row)) so that both operand reads are
  // bank-conflict free: 16 lanes reading one piece column of 16 rows, and the
  // transposing V reads (4 rows x 4 pieces per 32 lanes).
  static constexpr int kChunksPerRow = D / 8;                  // 16-byte pieces per row
  static constexpr int kKElems = kBN * D;
  static constexpr int kVElems = kBN * D;
  static constexpr int kSlotElems = kKElems + kVElems;
  static constexpr int kRowsPerLoad = 512 / D;                 // rows one 1 KiB load instruction fills
  static constexpr int kLoads = kBN * D * 2 / 1024 / (NT / 64);  // load instructions per wave per matrix
  static_assert(kLoads >= 1 && kLoads * (NT / 64) * 1024 == kBN * D * 2, "tile must split evenly");
  static_assert(16 % kRowsPerLoad == 0, "a load instruction's rows must share a 16-key block");
  // piece swizzle of row r. d = 128 (16 pieces, one row per 256-byte bank
  // period): the low two row bits move to piece bits 2-3 and the next two to
  // bits 0-1, a bijection on 16 consecutive rows (16 rows of one piece
  // column land on 16 bank groups) that gives 4 consecutive rows distinct
  // piece bits 2-3 (the 4 rows x 4 pieces of a transposing read). d = 64
  // (8 pieces, two rows per bank period): row bit 1 to piece bit 2, row bits
  // 2-3 to bits 0-1, so the 8 rows of each parity land on 8 groups.
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
};

struct PPParams {
  const uint16_t* q;
  const int* q_pos;
  const int* cu_q;
  // one entry per KV shard of a batched launch (contiguous shards only)
  const uint16_t* k[kMaxShards];
  const uint16_t* v[kMaxShards];
  const int* k_pos[kMaxShards];
  const int* cu_k[kMaxShards];
  void* o[kMaxShards];
  float* lse[kMaxShards];
  int n_shards;
  const int* block_table;
  int max_blocks;
  const int* local_kv_lens;
  int cp, rank, il;
  int num_seqs, hq, hkv, g, n_groups;
  float scale_log2;
  int causal;
  // Optional launch order (contiguous shards): order[i] is the tile unit
  // (group / hkv) the i-th unit slot runs; NULL runs units in index order.
  const int* order;
  // Running merge (one contiguous shard): when o_acc is set, the partial is
  // folded into (o_acc, lse_acc) in place, and o[0] (may be NULL) receives a
  // copy of the merged O in the output dtype.
  float* o_acc;
  float* lse_acc;
  // Paged (one shard): the other ranks' partials of the same rows, merged into
  // this partial in the epilogue when n_fold > 0 or own_o / own_lse is set
  // (o[0], lse[0] then receive the merge, own_o / own_lse this rank's own
  // partial in the parts' dtype).
  int n_fold;
  bool fold_bf16;
  const void* fold_o[kMaxFoldParts];
  const float* fold_lse[kMaxFoldParts];
  void* own_o;
  float* own_lse;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, source lane 4k+q names 4
// consecutive bf16 of row k of a 4-row block; result lane 4q+t receives
// column t of that lane quad's piece from rows 0..3, i.e. one column of the
// block as 4 consecutive rows.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// 16 bytes per lane from global memory straight into LDS: lane i writes
// bytes [16 i, 16 i + 16) after lds_base (wave-uniform). Written as a
// statement of its own rather than the compiler builtin: the compiler treats
// every later LDS read as possibly aliasing such a load and waits for it to
// complete, which would stall the matrix phase on the next slot's loads. The
// statement has no output register (the data goes to LDS); the kernel waits
// for these loads (vmcnt 0) itself before the barrier that publishes the
// slot. Loads the compiler issues itself are counted in order with these, so
// its own waits can only wait longer than needed, never shorter.
// lds_addr is the LDS byte address (wave-uniform).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  // m0 is reserved to the compiler (a clobber of it is ignored), so the
  // statement restores it
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(src), "s"(m0v)
               : "memory");
}

// The same load addressed as a wave-uniform base (scalar registers) plus this
// lane's 32-bit byte offset, so a tile whose per-lane offsets do not change
// costs no vector arithmetic to address.
__device__ __forceinline__ void lds_dma16_s(const void* base, uint32_t off, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(off), "s"(base), "s"(m0v)
               : "memory");
}

// Value of the lane 32 apart (lane ^ 32), combined: v_permlane32_swap
// exchanges the upper half of one register with the lower half of another;
// with both operands x, each lane ends with x and its partner's x, one in
// each result, so a symmetric combination needs no lane test. A VALU swap
// rather than an LDS permute, which would queue behind the other wave's
// operand reads.
__device__ __forceinline__ float pp_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pp_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float pp_max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Entries of the ascending array a[0..n) that are <= x (whole workgroup of NT
// threads).
template <int NT>
__device__ int pp_count_le(const int* __restrict__ a, int n, int x) {
  int lo = 0, hi = n;
  while (true) {
    const int span = hi - lo;
    if (span <= 0) return lo;
    const int step = (span + NT - 1) / NT;
    const int idx = lo + (int)(threadIdx.x + 1) * step - 1;
    const int c = __syncthreads_count(idx < hi && a[idx] <= x);
    const int new_lo = lo + c * step;
    if (step == 1) return new_lo;
    hi = min(hi, new_lo + step - 1);
    lo = new_lo;
  }
}


}  // namespace pp
}  // namespace cpa
