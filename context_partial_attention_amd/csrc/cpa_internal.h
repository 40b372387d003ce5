// Internal helpers shared by the library's translation units (not installed).
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include <hip/hip_runtime.h>

#include "cpattn.h"

namespace cpa {

// Records a formatted message for cpa_last_error() and returns `s`.
cpa_status fail(cpa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Checks that the current HIP device is gfx950 (cached per device).
cpa_status check_device();

// Checks hipGetLastError() after a launch and converts it to a status.
cpa_status check_launch(const char* what);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of positions in [0, n) that round-robin placement (groups of
// `interleave` positions dealt to the ranks in turn, starting with rank 0)
// stores on `rank`: each full cycle of interleave*cp positions gives
// `interleave` to every rank, and the leftover fills rank 0's group first.
inline int64_t rr_local_len(int64_t n, int64_t cp, int64_t rank, int64_t interleave) {
  const int64_t cyc = interleave * cp;
  int64_t rest = n % cyc - rank * interleave;
  rest = rest < 0 ? 0 : (rest > interleave ? interleave : rest);
  return (n / cyc) * interleave + rest;
}

// Arguments of one partial-attention launch, validated on the host. The
// contiguous form uses k/v/k_pos/cu_k; the paged form uses k/v as the block
// caches plus block_table/max_blocks/local_kv_lens/cp/rank/interleave.
struct AttnArgs {
  const void* q = nullptr;
  const int32_t* q_pos = nullptr;
  const int32_t* cu_q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* k_pos = nullptr;
  const int32_t* cu_k = nullptr;
  const int32_t* block_table = nullptr;
  int32_t max_blocks = 0;
  const int32_t* local_kv_lens = nullptr;
  int32_t cp = 1, rank = 0, interleave = 1;
  int32_t num_seqs = 0, max_q = 0, hq = 0, hkv = 0, d = 0;
  float scale = 1.f;
  int causal = 1;
  void* o = nullptr;
  bool o_bf16 = false;
  float* lse = nullptr;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
};

// Other ranks' partials (O, LSE) of the same rows, folded into this rank's
// own partial by the kernel that finishes it (the decode merge kernel, or the
// paged prefill kernel's epilogue): a.o, a.lse receive the exact merge of this
// rank's partial with o[0..n), and own_o / own_lse (either may be NULL)
// receive this rank's own partial in the parts' dtype.
constexpr int kMaxFoldParts = 15;
struct RankFold {
  int n;
  const void* o[kMaxFoldParts];
  const float* lse[kMaxFoldParts];
  bool part_bf16;
  void* own_o;
  float* own_lse;
};
cpa_status launch_attn_f32(const AttnArgs& a, hipStream_t st);
cpa_status launch_attn_mfma(const AttnArgs& a, bool paged, hipStream_t st);
// Two-group workgroup for GQA groups of even size (hq / hkv even); one launch
// covers up to kMaxShards contiguous KV shards (a single one when paged),
// each with its own output. With contiguous shards an optional order
// workspace of attn_pp_order_bytes() lets a pre-pass run the heaviest tile
// units first (0 bytes: the problem is too large to sort, index order).
// With `merged`, one workgroup walks the visible keys of every shard in one
// online softmax and writes only the merged (O, LSE) (the shards' own o, lse
// are not used).
constexpr int kMaxShards = 8;
struct MergedOut {
  void* o;
  bool o_bf16;
  float* lse;
};
bool attn_pp_supported(const AttnArgs& a);
size_t attn_pp_order_bytes(int n_shards, int num_seqs, int max_q);
// Tile units (query tiles x sequences x shards) the launch-order pre-pass sorts.
int64_t attn_pp_tile_units(int n_shards, int num_seqs, int max_q);
// The library's own launch-order scratch (a device array in attn_pp.hip, one
// copy per GPU): its address on the current device, looked up once per device,
// and the number of tile units it holds.
cpa_status attn_pp_scratch(void** ptr, size_t* bytes);
int attn_pp_scratch_units();
// With `accum` (one contiguous shard), the partial is folded into the running
// (o_acc, lse_acc) in place; o_out (may be NULL) gets a copy of the merged O in
// the shard's output dtype.
struct AccumIO {
  float* o_acc;
  float* lse_acc;
  void* o_out;
};
// With `fold` (paged, one shard), the epilogue merges the other ranks'
// partials of its rows into the rank's own partial (see RankFold).
cpa_status launch_attn_pp(const AttnArgs* shards, int n_shards, bool paged, hipStream_t st,
                          void* order_ws = nullptr, size_t order_ws_bytes = 0, const MergedOut* merged = nullptr,
                          const AccumIO* accum = nullptr, const RankFold* fold = nullptr);
size_t decode_workspace_bytes(int32_t num_seqs, int32_t max_blocks, int32_t block_size, int32_t hq, int32_t d);
cpa_status launch_attn_decode(const AttnArgs& a, hipStream_t st, const RankFold* fold = nullptr);

}  // namespace cpa
