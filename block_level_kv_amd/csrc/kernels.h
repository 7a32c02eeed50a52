// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace infllm {

constexpr int kMaxTopK = 256;

// Every workspace that holds counters starts with a header (word 0: waits
// that timed out, the rest reserved) and a counter region of at least
// kWsCounterBytes, then the call's data (partial sums, partial rows).  Every
// call leaves its counters at zero, and counters of every call kind and
// shape lie in the region's first bytes, so a zero-filled workspace can be
// reused by calls of other kinds and shapes as long as their counters fit
// the fixed-size region.
constexpr size_t kWsHeaderBytes = 256;
constexpr size_t kWsCounterBytes = 65536;
inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t ws_counter_region(size_t counter_bytes) {
  const size_t r = round256(counter_bytes);
  return r > kWsCounterBytes ? r : kWsCounterBytes;
}

// Tuning overrides (split counts), read from the environment once per
// process: INFLLM_PREFILL_SPLITS, INFLLM_ROWS_WGS, INFLLM_STEP_SPLITS.
// Zero: the built-in choice.
struct Tuning {
  int prefill_splits, rows_wgs, step_splits;
  int step_prespin;   // -1: the default bound
  int build_spin;     // -1: the default bound
};
const Tuning& tuning();

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
  double rope_theta;   // 0: logits of q and k as given; > 0: re-positioned (rope.h)
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
  // unit cache (decode attention only): k, v hold the initial tokens and a
  // ring of the later ones (local_cap rows per (sequence, KV head): row p
  // for p < n_init, n_init + (p - n_init) mod (local_cap - n_init) after),
  // kv_cap is the context's capacity; units' keys come from the slabs
  const void* ck;           // [b, H_kv, n_slots, B, d]
  const void* cv;
  const int32_t* c_slot;    // [b, H_kv, n_units]: slot + 1, 0 = not cached
  int n_units, n_slots;
  int64_t local_cap;
};

// Unit cache: tables in a caller-owned, zero-filled state buffer
// [header: hits, misses (int64)][slot_of int32 rows x U][unit_of int32
// rows x C][stamp int64 rows x C], each part 256-byte aligned.
constexpr int kCacheMaxSlots = 1024;
constexpr int kCacheMaxUnits = 65536;
constexpr size_t kCacheHeaderBytes = 256;
struct CacheTables {
  int64_t* stats;
  int32_t* slot_of;
  int32_t* unit_of;
  int64_t* stamp;
};
size_t cache_state_bytes(int64_t rows, int n_units, int n_slots);
CacheTables cache_tables(void* state, int64_t rows, int n_units, int n_slots);
struct CacheArgs {
  int batch, Hkv, d, B, n_init, k_m, n_pos, n_units, n_slots, elem;
  const int32_t* sel;       // [b, H_kv, n_pos, k_m]
  int64_t step;
  const void* k_host;       // [b, H_kv, host_cap, d], device-accessible host memory
  const void* v_host;
  int64_t host_cap;
  void* ck;                 // [b, H_kv, n_slots, B, d]
  void* cv;
  int64_t* stats;
  int32_t* slot_of;
  int32_t* unit_of;
  int64_t* stamp;
};
hipError_t launch_cache_fetch(const CacheArgs& a, hipStream_t st);

size_t build_workspace_bytes(const BuildArgs& a);
size_t build_range_workspace_bytes(const BuildArgs& a, int64_t n_units);
size_t build_counter_region(const BuildArgs& a, int64_t n_units);   // bytes after the header
size_t build_qsum_workspace_bytes(const BuildArgs& a);
size_t build_qsum_counter_region(const BuildArgs& a);   // bytes after the header
hipError_t launch_build(const BuildArgs& a, hipStream_t st);
size_t score_workspace_bytes(const ScoreArgs& a);
size_t select_workspace_bytes(const ScoreArgs& a);
hipError_t launch_score(const ScoreArgs& a, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

// vector-ALU attention, one query position per workgroup
int rows_num_splits(const AttendArgs& a);
hipError_t launch_attend_rows(const AttendArgs& a, int splits, hipStream_t st);
// the same over a unit cache (a.ck set)
hipError_t launch_attend_rows_cached(const AttendArgs& a, int splits, hipStream_t st);
int64_t rows_num_counters(const AttendArgs& a);

// fused decode step (bf16): unit scores, selection and attention of single
// query positions in one launch; false when the shapes need the separate calls.
// Every row (position x KV head x sequence) has n_splits workgroups; the
// first s_score of them score a slice of units_per units each.  Every
// workgroup attends an equal share of the selected units' keys and a share
// of the local keys (initial tokens and window) weighted w_score (scoring
// workgroups) or w_unit (the others).
struct StepPlan {
  int n_splits;            // workgroups per row (<= 64)
  int s_score;             // scoring workgroups per row
  int units_per;           // units per scoring workgroup: 64, 128, 192 or 256
  int cand;                // candidates each scoring workgroup publishes
  int w_score, w_unit;     // local-key weights of a scoring / another workgroup
  int pre_spin;            // polls of an attention workgroup for the selector's flag
};
bool select_attend_plan(const ScoreArgs& s, const AttendArgs& a, StepPlan* p);
int64_t step_rows(const AttendArgs& a);                  // rows of one call
// per row: arrival mask (2), ready flag, exit counter (attention
// workgroups in the low 16 bits, the selector above), started bytes (16)
constexpr int kStepSyncInts = 20;
// Row state, candidates and partials of one call: sync [rows][kStepSyncInts]
// in the workspace's counter region, then candidate scores and ids, partial
// rows and (max, sum) pairs.
struct StepPtrs {
  int* sync;
  float* cand_s;
  int* cand_i;
  int* status;   // workspace word 0: waits that timed out
};
hipError_t launch_select_attend(const ScoreArgs& s, AttendArgs a, const StepPlan& p,
                                const StepPtrs& w, hipStream_t st);

// bf16 MFMA attention tiles for query chunks (head_dim 128)
bool prefill_supported(const AttendArgs& a);
int prefill_num_splits(const AttendArgs& a);
int64_t prefill_num_counters(const AttendArgs& a);
int64_t prefill_partial_rows(const AttendArgs& a);   // per split
hipError_t launch_attend_prefill(const AttendArgs& a, int splits, hipStream_t st);

}  // namespace infllm
