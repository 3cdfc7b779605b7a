// Internal launch interface between the C-ABI host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace oxa {

struct DecodeLaunch {
  const uint16_t* q;
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* seq_lens;
  uint16_t* o;
  float* lse;
  int32_t* status;
  float* ws_o;      // [batch][hq][P][128] when num_partitions > 1
  float* ws_lse;    // [batch][hq][P]
  int32_t batch, hq, hkv, layout;
  int32_t num_pages, num_page_entries, max_seq_len, num_partitions, chunk_pages;
  float sm_scale;
};
hipError_t launch_paged_decode(const DecodeLaunch& a, hipStream_t stream);
// Load-balanced decode (equal page ranges per work-group, pieces merged by a
// second kernel), used for calls with the workspace for it.  Workspace after
// the partition states: the unit page starts (int32 [units + 1]), then the
// piece states: o f32 [G + units][hq][128] and lse f32 [G + units][hq].
constexpr int kBalancedMaxUnits = 2048;   // batch * partitions
constexpr int kBalancedMaxRanges = 512;   // G, the page ranges
struct BalancedLayout {
  int32_t* meta;
  float* piece_o;
  float* piece_lse;
};
hipError_t launch_paged_decode_balanced(const DecodeLaunch& a, const BalancedLayout& ws, int G,
                                        hipStream_t stream);
// Compute units of the current device (queried once per device).
hipError_t device_cu_count(int* cus);

// Bytes of the per-device static scratch behind the allocation-free decode,
// and its device address on the current device (resolved once per device).
constexpr size_t kDecodeScratchBytes = (size_t)8 << 20;
hipError_t decode_scratch_address(void** ptr);

struct AppendLaunch {
  const uint16_t* q_in;
  uint16_t* q_out;
  const uint16_t* k_in;
  const uint16_t* v_in;
  const int32_t* batch_indices;
  const int32_t* positions;
  uint16_t* k_pages;
  uint16_t* v_pages;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* page_refcounts;
  int32_t* status;
  int32_t* check;  // workspace: [kAppendCheckGroups][2] per-work-group check records
  int32_t hq, hkv, nnz, num_pages, layout, batch, num_page_entries;
  int32_t rope;         // 1: k is stored rotated (and q rotated if given); 0: k stored as is
  double inv_freq[64];  // rope_theta^(-2i/128), i < 64, computed on the host in double
};
// Work-groups of the append check pass, at most: the workspace holds one
// 8-byte record per work-group.
constexpr int kAppendCheckGroups = 1024;
hipError_t launch_paged_append_rope(const AppendLaunch& a, hipStream_t stream);

struct PrefillLaunch {
  const uint16_t* q;
  const uint16_t* k;        // ragged: [nnz_kv][hkv][128]; paged: the K pool
  const uint16_t* v;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;    // ragged only
  const int32_t* page_indptr;  // paged only
  const int32_t* page_indices;
  const int32_t* seq_lens;
  uint16_t* o;
  float* lse;
  int32_t* status;
  int32_t paged, layout, batch, nnz_qo, nnz_kv, hq, hkv, max_qo_len, max_kv_len, causal;
  int32_t num_pages, num_page_entries;
  float sm_scale;
  // key-range split of small calls: chunk states [max_split][nnz_qo][hq][128]
  // f32 and their lse [max_split][nnz_qo][hq]; max_split <= 1 disables it
  float* ws_o;
  float* ws_lse;
  int32_t max_split;
};
// Largest key-range split, and the largest nnz_qo * hq a split call may have
// (its workspace grows with both).
constexpr int kPrefillMaxSplit = 8;
constexpr int64_t kPrefillSplitMaxRowHeads = 1 << 15;
hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream);

// Attention-state merge over (row, head) units.  State s of unit (row, h)
// has its 128 values at element offset row * v_row + h * v_head + s * v_state
// of v[0] (or at row * v_row + h * v_head of v[s] for a pair), and its lse at
// row * l_row + h * l_head + s * l_state of lse[0] (lse[s] for a pair).
// Outputs are contiguous: out [units][128], lse_out [units] (may be null).
struct MergeLaunch {
  const void* v[2];
  const float* lse[2];
  int64_t v_row, v_head, v_state;
  int64_t l_row, l_head, l_state;
  int64_t units;  // rows * heads
  int32_t heads, states, in_f32, out_f32, pair;
  void* out;
  float* lse_out;
};
hipError_t launch_merge_states(const MergeLaunch& a, hipStream_t stream);
// Work-groups launch_merge_states uses for `units` units.
int64_t merge_states_groups(int64_t units, int in_f32);

// Standalone NeoX RoPE: q (if q_in) and k (if k_in) of nnz tokens rotated at
// positions[t] with the given double-precision frequency table.
struct RopeLaunch {
  const uint16_t* q_in;
  uint16_t* q_out;
  const uint16_t* k_in;
  uint16_t* k_out;
  const int32_t* positions;
  int32_t hq, hkv, nnz;
  double inv_freq[64];
};
hipError_t launch_rope(const RopeLaunch& a, hipStream_t stream);

}  // namespace oxa
