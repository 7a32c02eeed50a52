// C ABI of libinfllm.so (declared in include/infllm.h): host-side argument
// validation, workspace sizing and kernel dispatch.  Validation never touches
// the device, so every error path can be exercised without a GPU.
#include "../../include/infllm.h"

#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

using namespace infllm;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

infllm_status check_config(const infllm_config* c) {
  if (!c) return INFLLM_ERR_INVALID_ARG;
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads != 0)
    return INFLLM_ERR_INVALID_ARG;
  if (c->head_dim < 1 || c->block < 1 || c->n_init < 0 || c->window < 1 || c->top_k < 0)
    return INFLLM_ERR_INVALID_ARG;
  if (c->rep_mode != INFLLM_REP_TOKENS && c->rep_mode != INFLLM_REP_MEAN)
    return INFLLM_ERR_INVALID_ARG;
  if (c->dtype != INFLLM_F32 && c->dtype != INFLLM_BF16) return INFLLM_ERR_INVALID_ARG;
  if (c->rep_mode == INFLLM_REP_TOKENS && (c->rep_k < 1 || c->rep_k > c->block))
    return INFLLM_ERR_INVALID_ARG;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return INFLLM_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return INFLLM_ERR_UNSUPPORTED;
  if (c->block % 64 != 0 || c->block > 1024) return INFLLM_ERR_UNSUPPORTED;
  if (c->top_k > kMaxTopK) return INFLLM_ERR_UNSUPPORTED;
  return INFLLM_OK;
}

int64_t num_units(const infllm_config* c, int64_t n) {
  const int64_t u = n / c->block - c->n_init / c->block;
  return u > 0 ? u : 0;
}

infllm_status launched(hipError_t e) { return e == hipSuccess ? INFLLM_OK : INFLLM_ERR_HIP; }

ScoreArgs score_args(const infllm_config* c, int32_t batch, int32_t chunk_len, int32_t n_chunks) {
  ScoreArgs a{};
  a.batch = batch;
  a.Hq = c->n_q_heads;
  a.Hkv = c->n_kv_heads;
  a.d = c->head_dim;
  a.B = c->block;
  a.n_init = c->n_init;
  a.W = c->window;
  a.L = chunk_len;
  a.n_chunks = n_chunks;
  a.bf16 = c->dtype == INFLLM_BF16;
  return a;
}

BuildArgs build_args(const infllm_config* c, int32_t batch, int64_t n_ctx) {
  BuildArgs a{};
  a.batch = batch;
  a.Hq = c->n_q_heads;
  a.Hkv = c->n_kv_heads;
  a.d = c->head_dim;
  a.B = c->block;
  a.n_init = c->n_init;
  a.W = c->window;
  a.r_k = c->rep_k;
  a.rep_mode = c->rep_mode;
  a.bf16 = c->dtype == INFLLM_BF16;
  a.n_ctx = n_ctx;
  a.U = (int)num_units(c, n_ctx);
  a.u_begin = 0;
  a.u_end = a.U;
  a.u_stride = a.U;
  return a;
}

AttendArgs attend_args(const infllm_config* c, int32_t batch, int32_t chunk_len, int32_t n_chunks) {
  AttendArgs a{};
  a.batch = batch;
  a.Hq = c->n_q_heads;
  a.Hkv = c->n_kv_heads;
  a.d = c->head_dim;
  a.B = c->block;
  a.n_init = c->n_init;
  a.W = c->window;
  a.k_m = c->top_k;
  a.L = chunk_len;
  a.n_chunks = n_chunks;
  a.n_pos = chunk_len * n_chunks;
  a.bf16 = c->dtype == INFLLM_BF16;
  return a;
}

// Which attention path runs, and its split-K factor.
void attend_plan(const AttendArgs& a, bool* mfma, int* splits) {
  *mfma = prefill_supported(a);
  *splits = *mfma ? prefill_num_splits(a) : rows_num_splits(a);
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Attention workspace: [split-K counters][partial outputs][partial (max, sum)].
struct AttendWs {
  size_t count_bytes, o_bytes, ml_bytes;
  size_t total() const { return count_bytes + o_bytes + ml_bytes; }
};

AttendWs attend_ws_layout(const AttendArgs& a) {
  bool mfma;
  int splits;
  attend_plan(a, &mfma, &splits);
  AttendWs w{0, 0, 0};
  if (splits <= 1) return w;
  const size_t rows =
      (size_t)splits * (mfma ? (size_t)prefill_partial_rows(a) : (size_t)a.batch * a.Hq * a.n_pos);
  const int64_t counters = mfma ? prefill_num_counters(a) : rows_num_counters(a);
  w.count_bytes = round256((size_t)counters * sizeof(int));
  w.o_bytes = round256(rows * a.d * sizeof(float));
  w.ml_bytes = rows * 2 * sizeof(float);
  return w;
}

size_t attend_ws_bytes(const AttendArgs& a) { return attend_ws_layout(a).total(); }

// Decode step workspace.  Fused: [ready flags][selection
// counters][attention counters, partials of s_local + s_unit splits].
// Separate calls: [selection workspace][attention workspace].  Sized for
// the larger of the two.
struct StepWs {
  bool fused;
  StepPlan plan;
  size_t sync_bytes, sel_bytes;   // fused: ready flags, selection counters
  AttendWs att;                   // fused attention part
  size_t sep_sel_bytes;           // separate calls: selection workspace
  size_t total;
};

StepWs step_ws_layout(const infllm_config* c, int32_t batch, int32_t n_pos, int32_t n_units) {
  StepWs w{};
  ScoreArgs sa = score_args(c, batch, 1, n_pos);
  sa.U = n_units;
  sa.k_m = c->top_k;
  const AttendArgs aa = attend_args(c, batch, 1, n_pos);
  w.sep_sel_bytes = round256(select_workspace_bytes(sa));
  const size_t sep = w.sep_sel_bytes + attend_ws_bytes(aa);
  w.fused = select_attend_plan(sa, aa, &w.plan);
  size_t fused = 0;
  if (w.fused) {
    const size_t rows = (size_t)batch * c->n_kv_heads * n_pos;
    w.sync_bytes = round256((size_t)select_attend_sync_ints(aa) * sizeof(int));
    w.sel_bytes = round256(rows * sizeof(int));
    const size_t prow = (size_t)(w.plan.s_local + w.plan.s_unit) * batch * c->n_q_heads * n_pos;
    w.att.count_bytes = round256(rows * sizeof(int));
    w.att.o_bytes = round256(prow * c->head_dim * sizeof(float));
    w.att.ml_bytes = prow * 2 * sizeof(float);
    fused = w.sync_bytes + w.sel_bytes + w.att.total();
  }
  w.total = sep > fused ? sep : fused;
  return w;
}

}  // namespace

extern "C" {

int32_t infllm_abi_version(void) { return INFLLM_ABI_VERSION; }

const char* infllm_status_string(int32_t s) {
  switch (s) {
    case INFLLM_OK: return "ok";
    case INFLLM_ERR_INVALID_ARG: return "invalid argument";
    case INFLLM_ERR_UNSUPPORTED: return "unsupported configuration";
    case INFLLM_ERR_WORKSPACE: return "workspace missing or too small";
    case INFLLM_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t infllm_num_units(const infllm_config* cfg, int64_t n_ctx) {
  if (check_config(cfg) != INFLLM_OK || n_ctx < 0) return -1;
  const int64_t u = num_units(cfg, n_ctx);
  return u > INT32_MAX ? -1 : (int32_t)u;
}

int32_t infllm_num_eligible(const infllm_config* cfg, int64_t t_last, int32_t n_units) {
  if (check_config(cfg) != INFLLM_OK || n_units < 0) return -1;
  return (int32_t)eligible_units(t_last, n_units, cfg->block, cfg->n_init, cfg->window);
}

size_t infllm_workspace_size(const infllm_config* cfg, int32_t call, int32_t batch, int64_t n,
                             int32_t chunk_len, int32_t n_chunks) {
  if (check_config(cfg) != INFLLM_OK || batch < 1) return 0;
  switch (call) {
    case INFLLM_CALL_BUILD:
      return n < 1 ? 0 : build_workspace_bytes(build_args(cfg, batch, n));
    case INFLLM_CALL_BUILD_QSUM:
      return n < 1 ? 0 : build_qsum_workspace_bytes(build_args(cfg, batch, n));
    case INFLLM_CALL_BUILD_RANGE:
      return n < 1 ? 0 : build_range_workspace_bytes(build_args(cfg, batch, 0), n);
    case INFLLM_CALL_SCORE:
      if (chunk_len < 1 || n_chunks < 1) return 0;
      return score_workspace_bytes(score_args(cfg, batch, chunk_len, n_chunks));
    case INFLLM_CALL_SELECT:
      if (chunk_len < 1 || n_chunks < 1) return 0;
      return select_workspace_bytes(score_args(cfg, batch, chunk_len, n_chunks));
    case INFLLM_CALL_ATTEND:
      if (chunk_len < 1 || n_chunks < 1) return 0;
      return attend_ws_bytes(attend_args(cfg, batch, chunk_len, n_chunks));
    case INFLLM_CALL_SELECT_ATTEND:   // n = units, one query per chunk
      if (chunk_len != 1 || n_chunks < 1 || n < 0 || n > INT32_MAX) return 0;
      return step_ws_layout(cfg, batch, n_chunks, (int32_t)n).total;
    default:
      return 0;
  }
}

infllm_status infllm_build_units(const infllm_config* cfg, int32_t batch, const void* q,
                                 int64_t q_cap, const void* k, int64_t kv_cap, int64_t n_ctx,
                                 int32_t* rep_idx, float* unit_repr, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  infllm_status st = check_config(cfg);
  if (st != INFLLM_OK) return st;
  if (batch < 1 || n_ctx < 1 || q_cap < n_ctx || kv_cap < n_ctx) return INFLLM_ERR_INVALID_ARG;
  const bool tokens = cfg->rep_mode == INFLLM_REP_TOKENS;
  if (!k || !aligned16(k) || (tokens && (!q || !aligned16(q)))) return INFLLM_ERR_INVALID_ARG;
  BuildArgs a = build_args(cfg, batch, n_ctx);
  if (a.U > 0) {
    if (!unit_repr || !aligned16(unit_repr)) return INFLLM_ERR_INVALID_ARG;
    if (tokens && (!rep_idx || !aligned16(rep_idx))) return INFLLM_ERR_INVALID_ARG;
  }
  const size_t need = build_workspace_bytes(a);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return INFLLM_ERR_WORKSPACE;
  a.q = q;
  a.q_cap = q_cap;
  a.k = k;
  a.kv_cap = kv_cap;
  a.rep_idx = rep_idx;
  a.unit_repr = unit_repr;
  a.ws = workspace;
  return launched(launch_build(a, (hipStream_t)stream));
}

infllm_status infllm_build_units_qsum(const infllm_config* cfg, int32_t batch, const void* q,
                                      int64_t q_cap, const void* k, int64_t kv_cap, int64_t n_ctx,
                                      int32_t* rep_idx, float* unit_repr, double* block_qsum,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  infllm_status st = check_config(cfg);
  if (st != INFLLM_OK) return st;
  if (batch < 1 || n_ctx < 1 || q_cap < n_ctx || kv_cap < n_ctx) return INFLLM_ERR_INVALID_ARG;
  const bool tokens = cfg->rep_mode == INFLLM_REP_TOKENS;
  if (!k || !aligned16(k) || !q || !aligned16(q) || !block_qsum || !aligned16(block_qsum))
    return INFLLM_ERR_INVALID_ARG;
  BuildArgs a = build_args(cfg, batch, n_ctx);
  if (a.U > 0) {
    if (!unit_repr || !aligned16(unit_repr)) return INFLLM_ERR_INVALID_ARG;
    if (tokens && (!rep_idx || !aligned16(rep_idx))) return INFLLM_ERR_INVALID_ARG;
  }
  const size_t need = build_qsum_workspace_bytes(a);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return INFLLM_ERR_WORKSPACE;
  a.q = q;
  a.q_cap = q_cap;
  a.k = k;
  a.kv_cap = kv_cap;
  a.rep_idx = rep_idx;
  a.unit_repr = unit_repr;
  a.ws = workspace;
  a.block_qsum = block_qsum;
  return launched(launch_build(a, (hipStream_t)stream));
}

infllm_status infllm_build_units_range(const infllm_config* cfg, int32_t batch, const void* q,
                                       int64_t q_cap, const void* k, int64_t kv_cap,
                                       int64_t n_ctx, int32_t u_begin, int32_t u_end,
                                       int32_t pool_units, int32_t* rep_idx, float* unit_repr,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  infllm_status st = check_config(cfg);
  if (st != INFLLM_OK) return st;
  if (batch < 1 || n_ctx < 1 || q_cap < n_ctx || kv_cap < n_ctx) return INFLLM_ERR_INVALID_ARG;
  BuildArgs a = build_args(cfg, batch, n_ctx);
  if (u_begin < 0 || u_end < u_begin || u_end > a.U || pool_units < u_end)
    return INFLLM_ERR_INVALID_ARG;
  const bool tokens = cfg->rep_mode == INFLLM_REP_TOKENS;
  if (!k || !aligned16(k) || (tokens && (!q || !aligned16(q)))) return INFLLM_ERR_INVALID_ARG;
  if (u_end > u_begin) {
    if (!unit_repr || !aligned16(unit_repr)) return INFLLM_ERR_INVALID_ARG;
    if (tokens && (!rep_idx || !aligned16(rep_idx))) return INFLLM_ERR_INVALID_ARG;
  }
  const size_t need = build_range_workspace_bytes(a, u_end - u_begin);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return INFLLM_ERR_WORKSPACE;
  a.u_begin = u_begin;
  a.u_end = u_end;
  a.u_stride = pool_units;
  a.q = q;
  a.q_cap = q_cap;
  a.k = k;
  a.kv_cap = kv_cap;
  a.rep_idx = rep_idx;
  a.unit_repr = unit_repr;
  a.ws = workspace;
  return launched(launch_build(a, (hipStream_t)stream));
}

}  // extern "C"

// Shared by the single-position and per-sequence-position forms: pos (device,
// [batch]) replaces q_pos when non-null.
// sel non-null: the top-k_m selection is fused into the scoring launch.
static infllm_status score_impl(const infllm_config* cfg, int32_t batch, const void* q,
                                int64_t q_cap, int64_t q_off, int64_t q_pos, const int64_t* pos,
                                int32_t chunk_len, int32_t n_chunks, const float* unit_repr,
                                int32_t n_units, float* scores, int32_t* sel, void* workspace,
                                size_t workspace_bytes, void* stream, bool dry = false) {
  infllm_status st = check_config(cfg);
  if (st != INFLLM_OK) return st;
  if (batch < 1 || chunk_len < 1 || n_chunks < 1 || n_units < 0 || q_off < 0 || q_pos < 0)
    return INFLLM_ERR_INVALID_ARG;
  if (q_off + (int64_t)chunk_len * n_chunks > q_cap) return INFLLM_ERR_INVALID_ARG;
  if ((int64_t)n_chunks * cfg->n_kv_heads > 65535) return INFLLM_ERR_UNSUPPORTED;
  if (!q || !aligned16(q)) return INFLLM_ERR_INVALID_ARG;
  if (n_units > 0 && (!unit_repr || !scores || !aligned16(unit_repr) || !aligned16(scores)))
    return INFLLM_ERR_INVALID_ARG;
  ScoreArgs a = score_args(cfg, batch, chunk_len, n_chunks);
  a.U = n_units;
  if (sel && cfg->top_k > 0) {
    if (!aligned16(sel)) return INFLLM_ERR_INVALID_ARG;
    a.k_m = cfg->top_k;
    a.sel = sel;
  }
  if (dry) return INFLLM_OK;   // arguments only
  const size_t need = a.sel ? select_workspace_bytes(a) : score_workspace_bytes(a);
  if ((n_units > 0 || a.sel) && need > 0 &&
      (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return INFLLM_ERR_WORKSPACE;
  a.ws = workspace;
  a.q = q;
  a.q_cap = q_cap;
  a.q_off = q_off;
  a.q_pos = q_pos;
  a.pos = pos;
  a.repr = unit_repr;
  a.scores = scores;
  return launched(launch_score(a, (hipStream_t)stream));
}

extern "C" {

infllm_status infllm_score_units(const infllm_config* cfg, int32_t batch, const void* q,
                                 int64_t q_cap, int64_t q_off, int64_t q_pos, int32_t chunk_len,
                                 int32_t n_chunks, const float* unit_repr, int32_t n_units,
                                 float* scores, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return score_impl(cfg, batch, q, q_cap, q_off, q_pos, nullptr, chunk_len, n_chunks, unit_repr,
                    n_units, scores, nullptr, workspace, workspace_bytes, stream);
}

infllm_status infllm_score_units_qsum(const infllm_config* cfg, int32_t batch,
                                      const double* block_qsum, int64_t n_blocks, int64_t q_pos,
                                      int32_t chunk_len, int32_t n_chunks, const float* unit_repr,
                                      int32_t n_units, float* scores, void* stream) {
  infllm_status st = check_config(cfg);
  if (st != INFLLM_OK) return st;
  if (batch < 1 || chunk_len < 1 || n_chunks < 1 || n_units < 0 || q_pos < 0 || n_blocks < 1)
    return INFLLM_ERR_INVALID_ARG;
  // chunks made of whole blocks
  if (q_pos % cfg->block != 0 || chunk_len % cfg->block != 0) return INFLLM_ERR_INVALID_ARG;
  if ((q_pos + (int64_t)chunk_len * n_chunks) / cfg->block > n_blocks) return INFLLM_ERR_INVALID_ARG;
  if ((int64_t)n_chunks * cfg->n_kv_heads > 65535) return INFLLM_ERR_UNSUPPORTED;
  if (!block_qsum || !aligned16(block_qsum)) return INFLLM_ERR_INVALID_ARG;
  if (n_units > 0 && (!unit_repr || !scores || !aligned16(unit_repr) || !aligned16(scores)))
    return INFLLM_ERR_INVALID_ARG;
  ScoreArgs a = score_args(cfg, batch, chunk_len, n_chunks);
  a.U = n_units;
  a.q_pos = q_pos;
  a.block_qsum = block_qsum;
  a.n_blocks = n_blocks;
  a.repr = unit_repr;
  a.scores = scores;
  return launched(launch_score(a, (hipStream_t)stream));
}

infllm_status infllm_select_units(const infllm_config* cfg, int32_t batch, const void* q,
                                  int64_t q_cap, int64_t q_off, int64_t q_pos, const int64_t* pos,
                                  int32_t chunk_len, int32_t n_chunks, const float* unit_repr,
                                  int32_t n_units, float* scores, int32_t* sel, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (cfg && cfg->top_k > 0 && !sel) return INFLLM_ERR_INVALID_ARG;
  if (pos && (uintptr_t)pos % 8 != 0) return INFLLM_ERR_INVALID_ARG;
  return score_impl(cfg, batch, q, q_cap, q_off, pos ? 0 : q_pos, pos, chunk_len, n_chunks,
                    unit_repr, n_units, scores, sel, workspace, workspace_bytes, stream);
}

infllm_status infllm_score_units_varlen(const infllm_config* cfg, int32_t batch, const void* q,
                                        int64_t q_cap, int64_t q_off, const int64_t* pos,
                                        int32_t chunk_len, int32_t n_chunks,
                                        const float* unit_repr, int32_t n_units, float* scores,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!pos || (uintptr_t)pos % 8 != 0) return INFLLM_ERR_INVALID_ARG;
  return score_impl(cfg, batch, q, q_cap, q_off, 0, pos, chunk_len, n_chunks, unit_repr, n_units,
                    scores, nullptr, workspace, workspace_bytes, stream);
}

infllm_status infllm_topk_units(const infllm_config* cfg, int32_t batch, int32_t n_chunks,
                                const float* scores, int32_t n_units, int32_t* sel,
                                void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  infllm_status st = check_config(cfg);
  if (st != INFLLM_OK) return st;
  if (batch < 1 || n_chunks < 1 || n_units < 0) return INFLLM_ERR_INVALID_ARG;
  if (cfg->top_k == 0) return INFLLM_OK;
  if (!sel || !aligned16(sel) || (n_units > 0 && (!scores || !aligned16(scores))))
    return INFLLM_ERR_INVALID_ARG;
  TopkArgs a{};
  a.batch = batch;
  a.Hkv = cfg->n_kv_heads;
  a.n_chunks = n_chunks;
  a.U = n_units;
  a.k_m = cfg->top_k;
  a.scores = scores;
  a.sel = sel;
  return launched(launch_topk(a, (hipStream_t)stream));
}

}  // extern "C"

// Shared by the single-position and per-sequence-position forms.  With pos
// (device, [batch]) the positions are checked in the kernels: a sequence
// whose position does not fit kv_cap gets NaN rows.
static infllm_status attend_impl(const infllm_config* cfg, int32_t batch, const void* q,
                                 int64_t q_cap, int64_t q_off, int64_t q_pos, const int64_t* pos,
                                 int32_t chunk_len, int32_t n_chunks, const void* k,
                                 const void* v, int64_t kv_cap, const int32_t* sel, void* out,
                                 float* lse, int64_t out_cap, int64_t out_off, void* workspace,
                                 size_t workspace_bytes, void* stream, bool dry = false) {
  infllm_status st = check_config(cfg);
  if (st != INFLLM_OK) return st;
  if (batch < 1 || chunk_len < 1 || n_chunks < 1 || q_off < 0 || q_pos < 0 || out_off < 0)
    return INFLLM_ERR_INVALID_ARG;
  const int64_t n_pos = (int64_t)chunk_len * n_chunks;
  if ((int64_t)batch * cfg->n_kv_heads > 65535) return INFLLM_ERR_UNSUPPORTED;
  if (q_off + n_pos > q_cap || q_pos + n_pos > kv_cap || out_off + n_pos > out_cap)
    return INFLLM_ERR_INVALID_ARG;
  if (q_pos + n_pos > kPosLimit) return INFLLM_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return INFLLM_ERR_INVALID_ARG;
  if (cfg->top_k > 0 && (!sel || !aligned16(sel))) return INFLLM_ERR_INVALID_ARG;
  AttendArgs a = attend_args(cfg, batch, chunk_len, n_chunks);
  bool mfma;
  int splits;
  attend_plan(a, &mfma, &splits);
  if (!mfma && n_pos > 65535) return INFLLM_ERR_UNSUPPORTED;   // one grid row per position
  if (dry) return INFLLM_OK;   // arguments only
  const size_t need = attend_ws_bytes(a);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return INFLLM_ERR_WORKSPACE;
  a.q = q;
  a.q_cap = q_cap;
  a.q_off = q_off;
  a.q_pos = q_pos;
  a.pos = pos;
  a.k = k;
  a.v = v;
  a.kv_cap = kv_cap;
  a.sel = cfg->top_k > 0 ? sel : nullptr;
  a.out = out;
  a.lse = lse;
  a.out_cap = out_cap;
  a.out_off = out_off;
  if (need > 0) {
    const AttendWs lay = attend_ws_layout(a);
    a.ws_count = (int*)workspace;
    a.ws_o = (float*)((char*)workspace + lay.count_bytes);
    a.ws_ml = (float*)((char*)workspace + lay.count_bytes + lay.o_bytes);
  }
  hipStream_t s = (hipStream_t)stream;
  return launched(mfma ? launch_attend_prefill(a, splits, s) : launch_attend_rows(a, splits, s));
}

extern "C" {

infllm_status infllm_attend(const infllm_config* cfg, int32_t batch, const void* q, int64_t q_cap,
                            int64_t q_off, int64_t q_pos, int32_t chunk_len, int32_t n_chunks,
                            const void* k, const void* v, int64_t kv_cap, const int32_t* sel,
                            void* out, float* lse, int64_t out_cap, int64_t out_off,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return attend_impl(cfg, batch, q, q_cap, q_off, q_pos, nullptr, chunk_len, n_chunks, k, v,
                     kv_cap, sel, out, lse, out_cap, out_off, workspace, workspace_bytes, stream);
}

infllm_status infllm_attend_varlen(const infllm_config* cfg, int32_t batch, const void* q,
                                   int64_t q_cap, int64_t q_off, const int64_t* pos,
                                   int32_t chunk_len, int32_t n_chunks, const void* k,
                                   const void* v, int64_t kv_cap, const int32_t* sel, void* out,
                                   float* lse, int64_t out_cap, int64_t out_off, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!pos || (uintptr_t)pos % 8 != 0) return INFLLM_ERR_INVALID_ARG;
  // q_pos = 0 here only checks that kv_cap can hold one sequence's positions
  return attend_impl(cfg, batch, q, q_cap, q_off, 0, pos, chunk_len, n_chunks, k, v, kv_cap, sel,
                     out, lse, out_cap, out_off, workspace, workspace_bytes, stream);
}

infllm_status infllm_select_attend(const infllm_config* cfg, int32_t batch, const void* q,
                                   int64_t q_cap, int64_t q_off, int64_t q_pos,
                                   const int64_t* pos, int32_t n_pos, const float* unit_repr,
                                   int32_t n_units, const void* k, const void* v, int64_t kv_cap,
                                   float* scores, int32_t* sel, void* out, float* lse,
                                   int64_t out_cap, int64_t out_off, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (cfg && cfg->top_k > 0 && !sel) return INFLLM_ERR_INVALID_ARG;
  if (pos && (uintptr_t)pos % 8 != 0) return INFLLM_ERR_INVALID_ARG;
  const int64_t qp = pos ? 0 : q_pos;
  // both halves' argument checks, before anything is enqueued
  infllm_status st = score_impl(cfg, batch, q, q_cap, q_off, qp, pos, 1, n_pos, unit_repr, n_units,
                                scores, sel, nullptr, 0, stream, true);
  if (st != INFLLM_OK) return st;
  st = attend_impl(cfg, batch, q, q_cap, q_off, qp, pos, 1, n_pos, k, v, kv_cap, sel, out, lse,
                   out_cap, out_off, nullptr, 0, stream, true);
  if (st != INFLLM_OK) return st;
  const StepWs w = step_ws_layout(cfg, batch, n_pos, n_units);
  if (w.total > 0 && (!workspace || workspace_bytes < w.total || !aligned16(workspace)))
    return INFLLM_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  if (!w.fused) {
    st = score_impl(cfg, batch, q, q_cap, q_off, qp, pos, 1, n_pos, unit_repr, n_units, scores,
                    sel, ws, w.sep_sel_bytes, stream);
    if (st != INFLLM_OK) return st;
    return attend_impl(cfg, batch, q, q_cap, q_off, qp, pos, 1, n_pos, k, v, kv_cap, sel, out,
                       lse, out_cap, out_off, ws + w.sep_sel_bytes,
                       workspace_bytes - w.sep_sel_bytes, stream);
  }
  ScoreArgs sa = score_args(cfg, batch, 1, n_pos);
  sa.U = n_units;
  sa.k_m = cfg->top_k;
  sa.sel = sel;
  sa.q = q;
  sa.q_cap = q_cap;
  sa.q_off = q_off;
  sa.q_pos = qp;
  sa.pos = pos;
  sa.repr = unit_repr;
  sa.scores = scores;
  sa.ws = ws + w.sync_bytes;   // selection counters
  AttendArgs aa = attend_args(cfg, batch, 1, n_pos);
  aa.q = q;
  aa.q_cap = q_cap;
  aa.q_off = q_off;
  aa.q_pos = qp;
  aa.pos = pos;
  aa.k = k;
  aa.v = v;
  aa.kv_cap = kv_cap;
  aa.sel = sel;
  aa.out = out;
  aa.lse = lse;
  aa.out_cap = out_cap;
  aa.out_off = out_off;
  char* att = ws + w.sync_bytes + w.sel_bytes;
  aa.ws_count = (int*)att;
  aa.ws_o = (float*)(att + w.att.count_bytes);
  aa.ws_ml = (float*)(att + w.att.count_bytes + w.att.o_bytes);
  return launched(launch_select_attend(sa, aa, w.plan, (int*)ws, (hipStream_t)stream));
}

}  // extern "C"
