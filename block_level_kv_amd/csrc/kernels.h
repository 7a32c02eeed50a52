// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace infllm {

constexpr int kMaxTopK = 256;

struct BuildArgs {
  int batch, Hq, Hkv, d, B, n_init, W, r_k, rep_mode, U;
  int u_begin, u_end, u_stride;   // units built, rows of the output pool
  bool bf16;
  const void* q;
  int64_t q_cap;
  const void* k;
  int64_t kv_cap, n_ctx;
  int32_t* rep_idx;
  float* unit_repr;
  void* ws;
  double* block_qsum;  // optional out [batch, H_kv, ceil(n_ctx/B), d]: fp64 block query sums
};

struct ScoreArgs {
  int batch, Hq, Hkv, d, B, n_init, W, L, n_chunks, U;
  bool bf16;
  const void* q;
  int64_t q_cap, q_off, q_pos;
  const int64_t* pos;  // device [batch] first query position per sequence, or null (q_pos)
  const float* repr;
  float* scores;
  void* ws;  // fp64 partial query sums of long chunks
  int k_m;       // fused selection: units kept per row
  int32_t* sel;  // fused selection output, or null (scores only)
  const double* block_qsum;  // chunk sums from block query sums (B-aligned chunks), or null
  int64_t n_blocks;          // blocks per (sequence, KV head) in block_qsum
};

struct TopkArgs {
  int batch, Hkv, n_chunks, U, k_m;
  const float* scores;
  int32_t* sel;
};

struct AttendArgs {
  int batch, Hq, Hkv, d, B, n_init, W, k_m, L, n_chunks, n_pos;
  bool bf16;
  const void* q;
  int64_t q_cap, q_off, q_pos;
  const int64_t* pos;  // device [batch] first query position per sequence, or null (q_pos)
  const void* k;
  const void* v;
  int64_t kv_cap;
  const int32_t* sel;
  void* out;
  float* lse;
  int64_t out_cap, out_off;
  float* ws_o;   // split-K partial outputs
  float* ws_ml;  // split-K partial (max, sum) pairs
  int* ws_count; // split-K arrival counters (zero between calls)
};

size_t build_workspace_bytes(const BuildArgs& a);
size_t build_range_workspace_bytes(const BuildArgs& a, int64_t n_units);
size_t build_qsum_workspace_bytes(const BuildArgs& a);
hipError_t launch_build(const BuildArgs& a, hipStream_t st);
size_t score_workspace_bytes(const ScoreArgs& a);
size_t select_workspace_bytes(const ScoreArgs& a);
hipError_t launch_score(const ScoreArgs& a, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

// vector-ALU attention, one query position per workgroup
int rows_num_splits(const AttendArgs& a);
hipError_t launch_attend_rows(const AttendArgs& a, int splits, hipStream_t st);
int64_t rows_num_counters(const AttendArgs& a);

// fused decode step (bf16): unit scores, selection and attention of single
// query positions in one launch; false when the shapes need the separate calls
struct StepPlan {
  int n_slices;         // scoring slices per row
  int s_local, s_unit;  // attention splits per row over the local and the unit keys
                        // (s_unit >= n_slices; splits past the slices only attend)
};
bool select_attend_plan(const ScoreArgs& s, const AttendArgs& a, StepPlan* p);
int64_t select_attend_sync_ints(const AttendArgs& a);   // ready flags
hipError_t launch_select_attend(const ScoreArgs& s, const AttendArgs& a, const StepPlan& p,
                                int* ready, hipStream_t st);

// bf16 MFMA attention tiles for query chunks (head_dim 128)
bool prefill_supported(const AttendArgs& a);
int prefill_num_splits(const AttendArgs& a);
int64_t prefill_num_counters(const AttendArgs& a);
int64_t prefill_partial_rows(const AttendArgs& a);   // per split
hipError_t launch_attend_prefill(const AttendArgs& a, int splits, hipStream_t st);

}  // namespace infllm
