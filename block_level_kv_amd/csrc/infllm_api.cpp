// C ABI of libinfllm.so (declared in include/infllm.h): host-side argument
// validation, workspace sizing and kernel dispatch.  Validation never touches
// the device, so every error path can be exercised without a GPU.
#include "../../include/infllm.h"

#include <hip/hip_runtime.h>
#include <stdlib.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

using namespace infllm;

namespace infllm {

// Read once per process, so that workspace sizes and launch shapes cannot
// change between sizing a workspace and the calls that use it.
const Tuning& tuning() {
  static const Tuning t = [] {
    auto get = [](const char* name, int lo, int hi) {
      const char* e = getenv(name);
      const int v = e ? atoi(e) : 0;
      return v >= lo && v <= hi ? v : 0;
    };
    Tuning x{};
    x.prefill_splits = get("INFLLM_PREFILL_SPLITS", 1, 16);
    x.rows_wgs = get("INFLLM_ROWS_WGS", 1, 65536);
    x.step_splits = get("INFLLM_STEP_SPLITS", 2, 64);
    const char* e = getenv("INFLLM_STEP_PRESPIN");
    x.step_prespin = e && atoi(e) >= 0 && atoi(e) <= (1 << 20) ? atoi(e) : -1;
    e = getenv("INFLLM_BUILD_SPIN");
    x.build_spin = e && atoi(e) >= 0 && atoi(e) <= (1 << 20) ? atoi(e) : -1;
    return x;
  }();
  return t;
}

}  // namespace infllm

// Scratch memory of infllm_select_attend_static: the workspace of one decode
// step, for callers that cannot allocate.  Each GPU holds its own copy until
// the process ends; device globals start zero-filled, and every call leaves
// the counters in it at zero.  Host code never passes the array's name to a
// kernel (on the host it only names the symbol): the device address comes
// from hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device.
infllm_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return INFLLM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return INFLLM_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return INFLLM_OK;
}

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
  // 0 (off) or a finite positive base; NaN fails both tests
  if (!(c->rope_theta == 0.0 || (c->rope_theta > 0.0 && c->rope_theta < 1e300)))
    return INFLLM_ERR_INVALID_ARG;
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
  a.rope_theta = c->rope_theta;
  return a;
}

// Which attention path runs, and its split-K factor.
void attend_plan(const AttendArgs& a, bool* mfma, int* splits) {
  *mfma = prefill_supported(a);
  *splits = *mfma ? prefill_num_splits(a) : rows_num_splits(a);
}

// Attention workspace: [header][split-K counters][partial outputs][partial
// (max, sum)].
struct AttendWs {
  size_t count_bytes, o_bytes, ml_bytes;   // count_bytes: header + counter region
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
  w.count_bytes = kWsHeaderBytes + ws_counter_region((size_t)counters * sizeof(int));
  w.o_bytes = round256(rows * a.d * sizeof(float));
  w.ml_bytes = rows * 2 * sizeof(float);
  return w;
}

size_t attend_ws_bytes(const AttendArgs& a) { return attend_ws_layout(a).total(); }

// Decode step workspace.  Fused: [header][counter region: per-row sync
// ints][candidate scores][candidate ids][partial rows of n_splits
// splits][(max, sum)].  Separate calls: [header][counter region: selection
// counters, then attention counters][attention partial rows][(max, sum)].
// Sized for the larger of the two; both keep every counter in the region.
struct StepWs {
  bool fused;
  StepPlan plan;
  size_t sync_bytes;              // header + counter region (either form)
  size_t cand_bytes;              // fused: candidate scores, then ids
  AttendWs att;                   // partial rows and (max, sum) (count_bytes 0)
  size_t sep_sel_count;           // separate calls: bytes of selection counters
  size_t total;
};

StepWs step_ws_layout(const infllm_config* c, int32_t batch, int32_t n_pos, int32_t n_units) {
  StepWs w{};
  ScoreArgs sa = score_args(c, batch, 1, n_pos);
  sa.U = n_units;
  sa.k_m = c->top_k;
  const AttendArgs aa = attend_args(c, batch, 1, n_pos);
  w.fused = select_attend_plan(sa, aa, &w.plan);
  if (w.fused) {
    const size_t rows = (size_t)step_rows(aa);
    const size_t cands = rows * w.plan.s_score * w.plan.cand;
    w.sync_bytes = kWsHeaderBytes + ws_counter_region(rows * kStepSyncInts * sizeof(int));
    w.cand_bytes = round256(cands * sizeof(float)) + round256(cands * sizeof(int));
    const size_t prow = (size_t)w.plan.n_splits * batch * c->n_q_heads * n_pos;
    w.att.o_bytes = round256(prow * c->head_dim * sizeof(float));
    w.att.ml_bytes = prow * 2 * sizeof(float);
  } else {
    w.sep_sel_count = round256((size_t)batch * c->n_kv_heads * n_pos * sizeof(int));
    const AttendWs at = attend_ws_layout(aa);
    const size_t at_count = at.count_bytes > 0 ? (size_t)rows_num_counters(aa) * sizeof(int) : 0;
    w.sync_bytes = kWsHeaderBytes + ws_counter_region(w.sep_sel_count + at_count);
    w.att.o_bytes = at.o_bytes;
    w.att.ml_bytes = at.ml_bytes;
  }
  w.att.count_bytes = 0;
  w.total = w.sync_bytes + w.cand_bytes + w.att.total();
  return w;
}

// Counter region [begin, end) of a call's workspace (begin = end = 0 when
// it has none).
void counter_region(const infllm_config* cfg, int32_t call, int32_t batch, int64_t n,
                    int32_t chunk_len, int32_t n_chunks, size_t* begin, size_t* end) {
  *begin = *end = 0;
  size_t region = 0;
  switch (call) {
    case INFLLM_CALL_BUILD: {
      const BuildArgs a = build_args(cfg, batch, n);
      region = build_counter_region(a, a.u_end - a.u_begin);
      if (region == 0) return;
      break;
    }
    case INFLLM_CALL_BUILD_RANGE: {
      region = build_counter_region(build_args(cfg, batch, 0), n);
      if (region == 0) return;
      break;
    }
    case INFLLM_CALL_BUILD_QSUM: {
      region = build_qsum_counter_region(build_args(cfg, batch, n));
      if (region == 0) return;
      break;
    }
    case INFLLM_CALL_SCORE:
    case INFLLM_CALL_SELECT: {
      ScoreArgs a = score_args(cfg, batch, chunk_len, n_chunks);
      if (call == INFLLM_CALL_SCORE && score_workspace_bytes(a) == 0) return;
      region = ws_counter_region((size_t)batch * cfg->n_kv_heads * n_chunks * sizeof(int));
      break;
    }
    case INFLLM_CALL_ATTEND: {
      const AttendWs w = attend_ws_layout(attend_args(cfg, batch, chunk_len, n_chunks));
      if (w.count_bytes == 0) return;
      region = w.count_bytes - kWsHeaderBytes;
      break;
    }
    case INFLLM_CALL_SELECT_ATTEND: {
      const StepWs w = step_ws_layout(cfg, batch, n_chunks, (int32_t)n);
      region = w.sync_bytes - kWsHeaderBytes;
      break;
    }
    default:
      return;
  }
  *begin = kWsHeaderBytes;
  *end = kWsHeaderBytes + region;
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
  // the merge addresses partial rows with 32-bit byte offsets
  if (attend_ws_layout(a).o_bytes >= ((size_t)1 << 32)) return INFLLM_ERR_UNSUPPORTED;
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
    a.ws_count = (int*)((char*)workspace + kWsHeaderBytes);
    a.ws_o = (float*)((char*)workspace + lay.count_bytes);
    a.ws_ml = (float*)((char*)workspace + lay.count_bytes + lay.o_bytes);
  }
  hipStream_t s = (hipStream_t)stream;
  return launched(mfma ? launch_attend_prefill(a, splits, s) : launch_attend_rows(a, splits, s));
}

// Both halves' argument checks of a decode step, before anything is
// enqueued, and the step's workspace layout.
static infllm_status step_check(const infllm_config* cfg, int32_t batch, const void* q,
                                int64_t q_cap, int64_t q_off, int64_t q_pos, const int64_t* pos,
                                int32_t n_pos, const float* unit_repr, int32_t n_units,
                                const void* k, const void* v, int64_t kv_cap, float* scores,
                                int32_t* sel, void* out, float* lse, int64_t out_cap,
                                int64_t out_off, void* stream, StepWs* w);

// One decode step on a workspace laid out by step_ws_layout (arguments
// already validated): the fused launch, or the selection and attention
// launches with both sets of counters in the workspace's counter region.
static infllm_status step_launch(const infllm_config* cfg, int32_t batch, const void* q,
                                 int64_t q_cap, int64_t q_off, int64_t qp, const int64_t* pos,
                                 int32_t n_pos, const float* unit_repr, int32_t n_units,
                                 const void* k, const void* v, int64_t kv_cap, float* scores,
                                 int32_t* sel, void* out, float* lse, int64_t out_cap,
                                 int64_t out_off, const StepWs& w, char* ws, hipStream_t st) {
  ScoreArgs sa = score_args(cfg, batch, 1, n_pos);
  sa.U = n_units;
  sa.q = q;
  sa.q_cap = q_cap;
  sa.q_off = q_off;
  sa.q_pos = qp;
  sa.pos = pos;
  sa.repr = unit_repr;
  sa.scores = scores;
  if (cfg->top_k > 0) {
    sa.k_m = cfg->top_k;
    sa.sel = sel;
  }
  sa.ws = ws;   // header; counters from kWsHeaderBytes
  AttendArgs aa = attend_args(cfg, batch, 1, n_pos);
  aa.q = q;
  aa.q_cap = q_cap;
  aa.q_off = q_off;
  aa.q_pos = qp;
  aa.pos = pos;
  aa.k = k;
  aa.v = v;
  aa.kv_cap = kv_cap;
  aa.sel = cfg->top_k > 0 ? sel : nullptr;
  aa.out = out;
  aa.lse = lse;
  aa.out_cap = out_cap;
  aa.out_off = out_off;
  char* data = ws + w.sync_bytes;
  aa.ws_o = (float*)(data + w.cand_bytes);
  aa.ws_ml = (float*)(data + w.cand_bytes + w.att.o_bytes);
  if (!w.fused) {
    bool mfma;
    int splits;
    attend_plan(aa, &mfma, &splits);
    aa.ws_count = splits > 1 ? (int*)(ws + kWsHeaderBytes + w.sep_sel_count) : nullptr;
    const infllm_status s1 = launched(launch_score(sa, st));
    if (s1 != INFLLM_OK) return s1;
    return launched(launch_attend_rows(aa, splits, st));
  }
  StepPtrs p{};
  p.status = (int*)ws;
  p.sync = (int*)(ws + kWsHeaderBytes);
  const size_t cands = (size_t)step_rows(aa) * w.plan.s_score * w.plan.cand;
  p.cand_s = (float*)data;
  p.cand_i = (int*)(data + round256(cands * sizeof(float)));
  return launched(launch_select_attend(sa, aa, w.plan, p, st));
}

static infllm_status step_check(const infllm_config* cfg, int32_t batch, const void* q,
                                int64_t q_cap, int64_t q_off, int64_t q_pos, const int64_t* pos,
                                int32_t n_pos, const float* unit_repr, int32_t n_units,
                                const void* k, const void* v, int64_t kv_cap, float* scores,
                                int32_t* sel, void* out, float* lse, int64_t out_cap,
                                int64_t out_off, void* stream, StepWs* w) {
  if (cfg && cfg->top_k > 0 && !sel) return INFLLM_ERR_INVALID_ARG;
  if (pos && (uintptr_t)pos % 8 != 0) return INFLLM_ERR_INVALID_ARG;
  const int64_t qp = pos ? 0 : q_pos;
  infllm_status st = score_impl(cfg, batch, q, q_cap, q_off, qp, pos, 1, n_pos, unit_repr, n_units,
                                scores, sel, nullptr, 0, stream, true);
  if (st != INFLLM_OK) return st;
  st = attend_impl(cfg, batch, q, q_cap, q_off, qp, pos, 1, n_pos, k, v, kv_cap, sel, out, lse,
                   out_cap, out_off, nullptr, 0, stream, true);
  if (st != INFLLM_OK) return st;
  *w = step_ws_layout(cfg, batch, n_pos, n_units);
  return INFLLM_OK;
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
  StepWs w;
  infllm_status st = step_check(cfg, batch, q, q_cap, q_off, q_pos, pos, n_pos, unit_repr, n_units,
                                k, v, kv_cap, scores, sel, out, lse, out_cap, out_off, stream, &w);
  if (st != INFLLM_OK) return st;
  if (!workspace || workspace_bytes < w.total || !aligned16(workspace))
    return INFLLM_ERR_WORKSPACE;
  return step_launch(cfg, batch, q, q_cap, q_off, pos ? 0 : q_pos, pos, n_pos, unit_repr, n_units,
                     k, v, kv_cap, scores, sel, out, lse, out_cap, out_off, w, (char*)workspace,
                     (hipStream_t)stream);
}

infllm_status infllm_select_attend_static(const infllm_config* cfg, int32_t batch, const void* q,
                                          int64_t q_cap, int64_t q_off, int64_t q_pos,
                                          const int64_t* pos, int32_t n_pos,
                                          const float* unit_repr, int32_t n_units, const void* k,
                                          const void* v, int64_t kv_cap, float* scores,
                                          int32_t* sel, void* out, float* lse, int64_t out_cap,
                                          int64_t out_off, void* stream) {
  StepWs w;
  infllm_status st = step_check(cfg, batch, q, q_cap, q_off, q_pos, pos, n_pos, unit_repr, n_units,
                                k, v, kv_cap, scores, sel, out, lse, out_cap, out_off, stream, &w);
  if (st != INFLLM_OK) return st;
  // the step must fit the scratch array, with its counters inside the
  // fixed-size counter region (so that calls of any shape can follow)
  if (w.total > kStaticScratchBytes || w.sync_bytes > kWsHeaderBytes + kWsCounterBytes)
    return INFLLM_ERR_WORKSPACE;
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != INFLLM_OK) return st;
  return step_launch(cfg, batch, q, q_cap, q_off, pos ? 0 : q_pos, pos, n_pos, unit_repr, n_units,
                     k, v, kv_cap, scores, sel, out, lse, out_cap, out_off, w, (char*)ws,
                     (hipStream_t)stream);
}

int32_t infllm_workspace_layout(const infllm_config* cfg, int32_t call, int32_t batch, int64_t n,
                                int32_t chunk_len, int32_t n_chunks, size_t* counters_begin,
                                size_t* counters_end, size_t* total) {
  if (!counters_begin || !counters_end || !total) return INFLLM_ERR_INVALID_ARG;
  *counters_begin = *counters_end = *total = 0;
  if (check_config(cfg) != INFLLM_OK || batch < 1) return INFLLM_ERR_INVALID_ARG;
  *total = infllm_workspace_size(cfg, call, batch, n, chunk_len, n_chunks);
  if (*total > 0) counter_region(cfg, call, batch, n, chunk_len, n_chunks, counters_begin, counters_end);
  return INFLLM_OK;
}

int32_t infllm_step_plan(const infllm_config* cfg, int32_t batch, int32_t n_units, int32_t n_pos,
                         int32_t* plan) {
  if (!plan) return INFLLM_ERR_INVALID_ARG;
  for (int i = 0; i < 7; ++i) plan[i] = 0;
  if (check_config(cfg) != INFLLM_OK || batch < 1 || n_units < 0 || n_pos < 1)
    return INFLLM_ERR_INVALID_ARG;
  const StepWs w = step_ws_layout(cfg, batch, n_pos, n_units);
  if (!w.fused) return INFLLM_OK;
  plan[0] = 1;
  plan[1] = w.plan.n_splits;
  plan[2] = w.plan.s_score;
  plan[3] = w.plan.units_per;
  plan[4] = w.plan.cand;
  plan[5] = w.plan.w_score;
  plan[6] = w.plan.w_unit;
  return INFLLM_OK;
}

int32_t infllm_workspace_status(const void* workspace, size_t workspace_bytes, int32_t* timeouts,
                                void* stream) {
  if (!timeouts) return INFLLM_ERR_INVALID_ARG;
  *timeouts = 0;
  if (!workspace || workspace_bytes < kWsHeaderBytes || !aligned16(workspace))
    return INFLLM_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return INFLLM_ERR_HIP;
  int32_t v = 0;
  if (hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
    return INFLLM_ERR_HIP;
  *timeouts = v;
  return INFLLM_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ unit cache
namespace {

// Host memory the kernels may read at the same address: pinned (registered
// with the runtime) and mapped into the GPU's address space as is.  Pageable
// memory would fault on the device, so it is refused here.
bool device_readable_host(const void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the error this query leaves
    return false;
  }
  return at.type == hipMemoryTypeHost && at.devicePointer == p;
}

infllm_status cache_shape_check(const infllm_config* cfg, int32_t batch, int32_t n_units,
                                int32_t n_slots) {
  const infllm_status st = check_config(cfg);
  if (st != INFLLM_OK) return st;
  if (batch < 1 || n_units < 1 || n_slots < 1) return INFLLM_ERR_INVALID_ARG;
  if (n_units > kCacheMaxUnits || n_slots > kCacheMaxSlots) return INFLLM_ERR_UNSUPPORTED;
  if ((int64_t)batch * cfg->n_kv_heads > ((int64_t)1 << 31) - 1) return INFLLM_ERR_UNSUPPORTED;
  return INFLLM_OK;
}

}  // namespace

extern "C" {

size_t infllm_cache_state_size(const infllm_config* cfg, int32_t batch, int32_t n_units,
                               int32_t n_slots) {
  if (cache_shape_check(cfg, batch, n_units, n_slots) != INFLLM_OK) return 0;
  return cache_state_bytes((int64_t)batch * cfg->n_kv_heads, n_units, n_slots);
}

infllm_status infllm_cache_fetch(const infllm_config* cfg, int32_t batch, int32_t n_pos,
                                 const int32_t* sel, int32_t n_units, int64_t step,
                                 const void* k_host, const void* v_host, int64_t host_cap,
                                 void* cache_k, void* cache_v, int32_t n_slots, void* state,
                                 void* stream) {
  infllm_status st = cache_shape_check(cfg, batch, n_units, n_slots);
  if (st != INFLLM_OK) return st;
  if (n_pos < 1 || step < 1) return INFLLM_ERR_INVALID_ARG;
  if ((int64_t)n_pos * cfg->top_k > n_slots) return INFLLM_ERR_INVALID_ARG;   // union must fit
  // every unit's block lies in the host pool
  if (host_cap < ((int64_t)n_units + cfg->n_init / cfg->block) * cfg->block)
    return INFLLM_ERR_INVALID_ARG;
  if (!k_host || !v_host || !cache_k || !cache_v || !state || !aligned16(k_host) ||
      !aligned16(v_host) || !aligned16(cache_k) || !aligned16(cache_v) || !aligned16(state))
    return INFLLM_ERR_INVALID_ARG;
  if (cfg->top_k == 0) return INFLLM_OK;   // nothing selected
  if (!sel || !aligned16(sel)) return INFLLM_ERR_INVALID_ARG;
  if (!device_readable_host(k_host) || !device_readable_host(v_host)) return INFLLM_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)batch * cfg->n_kv_heads;
  const CacheTables t = cache_tables(state, rows, n_units, n_slots);
  CacheArgs a{};
  a.batch = batch;
  a.Hkv = cfg->n_kv_heads;
  a.d = cfg->head_dim;
  a.B = cfg->block;
  a.n_init = cfg->n_init;
  a.k_m = cfg->top_k;
  a.n_pos = n_pos;
  a.n_units = n_units;
  a.n_slots = n_slots;
  a.elem = cfg->dtype == INFLLM_BF16 ? 2 : 4;
  a.sel = sel;
  a.step = step;
  a.k_host = k_host;
  a.v_host = v_host;
  a.host_cap = host_cap;
  a.ck = cache_k;
  a.cv = cache_v;
  a.stats = t.stats;
  a.slot_of = t.slot_of;
  a.unit_of = t.unit_of;
  a.stamp = t.stamp;
  return launched(launch_cache_fetch(a, (hipStream_t)stream));
}

infllm_status infllm_attend_cached(const infllm_config* cfg, int32_t batch, const void* q,
                                   int64_t q_cap, int64_t q_off, int64_t q_pos,
                                   const int64_t* pos, int32_t n_pos, const void* k_local,
                                   const void* v_local, int64_t local_cap, int64_t ctx_cap,
                                   const int32_t* sel, int32_t n_units, const void* cache_k,
                                   const void* cache_v, int32_t n_slots, const void* state,
                                   void* out, float* lse, int64_t out_cap, int64_t out_off,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  infllm_status st = cache_shape_check(cfg, batch, n_units, n_slots);
  if (st != INFLLM_OK) return st;
  if (cfg->rope_theta != 0.0) return INFLLM_ERR_UNSUPPORTED;
  if (n_pos < 1 || q_off < 0 || q_pos < 0 || out_off < 0) return INFLLM_ERR_INVALID_ARG;
  if ((int64_t)batch * cfg->n_kv_heads > 65535 || n_pos > 65535) return INFLLM_ERR_UNSUPPORTED;
  if (q_off + n_pos > q_cap || out_off + n_pos > out_cap) return INFLLM_ERR_INVALID_ARG;
  if (!pos && q_pos + n_pos > ctx_cap) return INFLLM_ERR_INVALID_ARG;
  if (ctx_cap > kPosLimit) return INFLLM_ERR_UNSUPPORTED;
  // the ring holds every window of the call: W + n_pos - 1 positions
  if (local_cap <= cfg->n_init || local_cap - cfg->n_init < (int64_t)cfg->window + n_pos - 1)
    return INFLLM_ERR_INVALID_ARG;
  if (!q || !k_local || !v_local || !out || !state || !cache_k || !cache_v || !aligned16(q) ||
      !aligned16(k_local) || !aligned16(v_local) || !aligned16(out) || !aligned16(state) ||
      !aligned16(cache_k) || !aligned16(cache_v))
    return INFLLM_ERR_INVALID_ARG;
  if (pos && ((uintptr_t)pos & 7u)) return INFLLM_ERR_INVALID_ARG;
  if (cfg->top_k > 0 && (!sel || !aligned16(sel))) return INFLLM_ERR_INVALID_ARG;
  AttendArgs a = attend_args(cfg, batch, 1, n_pos);
  int splits = rows_num_splits(a);
  if (attend_ws_layout(a).o_bytes >= ((size_t)1 << 32)) return INFLLM_ERR_UNSUPPORTED;
  const size_t need = attend_ws_bytes(a);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return INFLLM_ERR_WORKSPACE;
  a.q = q;
  a.q_cap = q_cap;
  a.q_off = q_off;
  a.q_pos = q_pos;
  a.pos = pos;
  a.k = k_local;
  a.v = v_local;
  a.kv_cap = ctx_cap;
  a.local_cap = local_cap;
  a.sel = cfg->top_k > 0 ? sel : nullptr;
  a.out = out;
  a.lse = lse;
  a.out_cap = out_cap;
  a.out_off = out_off;
  a.ck = cache_k;
  a.cv = cache_v;
  a.c_slot = cache_tables(const_cast<void*>(state), (int64_t)batch * cfg->n_kv_heads, n_units,
                          n_slots).slot_of;
  a.n_units = n_units;
  a.n_slots = n_slots;
  if (need > 0) {
    const AttendWs lay = attend_ws_layout(a);
    a.ws_count = (int*)((char*)workspace + kWsHeaderBytes);
    a.ws_o = (float*)((char*)workspace + lay.count_bytes);
    a.ws_ml = (float*)((char*)workspace + lay.count_bytes + lay.o_bytes);
  }
  return launched(launch_attend_rows_cached(a, splits, (hipStream_t)stream));
}

int32_t infllm_cache_stats(const void* state, int64_t* hits, int64_t* misses, void* stream) {
  if (!state || !hits || !misses || !aligned16(state)) return INFLLM_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return INFLLM_ERR_HIP;
  int64_t v[2] = {0, 0};
  if (hipMemcpy(v, state, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return INFLLM_ERR_HIP;
  *hits = v[0];
  *misses = v[1];
  return INFLLM_OK;
}

}  // extern "C"
