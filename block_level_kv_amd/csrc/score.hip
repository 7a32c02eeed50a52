// Unit relevance scores: for chunk c and KV head h,
//     score[u] = (sum of the chunk's queries over the group's heads) . repr[u]
// for eligible u, -inf otherwise (InfLLM Guide, "Core Innovation 2", item 2;
// authors' rebuttal, "Latency Across Different Context Windows").  The query
// sum and the dot products accumulate in fp64, so the ranking that follows
// is decided on scores accurate far below the near-tie margin.
//
// Long chunks: the query sum is spread over workgroups of ROWS rows
// each (16-byte loads, all G heads), whose fp64 partial sums are added in
// part order, so results do not depend on scheduling.  Up to
// kFusedMaxUnits units this is one launch (k_score_fused: the last
// workgroup of a chunk to arrive adds the parts and scores every unit);
// beyond, k_chunk_qsum writes the parts and k_score_units adds them.
// Short chunks (decode: one query x G heads) skip the parts and sum their
// few rows directly in k_score_units, which scores a slice of kUnitsPerWG
// units.  Each unit is read as one coalesced fp32 row by D/8 lanes.  Every
// phase issues all of its loads before it uses any of them (clamped
// indices or bounds-checked buffer loads instead of branches), so a phase
// costs one memory round trip.
#include "common.h"
#include "kernels.h"
#include "score_units.h"

namespace infllm {

// chunk rows per partial sum: 128 when a call has enough of them to fill
// the chip (fewer, longer workgroups amortize the publication), else 32
constexpr int kRowsShort = 32, kRowsLong = 128;
constexpr int kFusedMaxUnits = 2048;
constexpr int kBatchUnits = 64;      // units whose rows the fused kernel requests together

static int score_rows(const ScoreArgs& a) {
  const int64_t long_parts = (int64_t)a.batch * a.Hkv * a.n_chunks * ((a.L + kRowsLong - 1) / kRowsLong);
  return long_parts >= 512 ? kRowsLong : kRowsShort;
}

static int score_num_parts(const ScoreArgs& a) {
  const int G = a.Hq / a.Hkv, rows = score_rows(a);
  return a.L * G <= kDirectRows ? 0 : (a.L + rows - 1) / rows;
}

// Column sums of rows [r0, r1) of one chunk over the G heads of a KV head,
// fp64: thread (8-column group, row lane) adds its rows head by head, then
// the row lanes are added in order through LDS.  qb points at row 0 of the
// chunk in the first head; heads are hs elements apart.  Threads tid < D
// return column tid's sum.
template <typename T, int G, int D, int ROWS>
__device__ __forceinline__ double rows_colsum(const T* __restrict__ qb, int64_t hs, int r0, int r1,
                                              double (*sm)[D]) {
  constexpr int kCgs = D / 8, kNrl = kScoreThreads / kCgs;
  constexpr int kIt = (ROWS + kNrl - 1) / kNrl;
  const int tid = threadIdx.x, cg = tid % kCgs, rl = tid / kCgs;
  Raw8<T> raw[G][kIt];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int i = r0 + rl + it * kNrl;
      raw[g][it].load(qb + g * hs + (int64_t)(i < r1 ? i : r1 - 1) * D + cg * 8);
    }
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int it = 0; it < kIt; ++it)
      if (r0 + rl + it * kNrl < r1) raw[g][it].add(acc);
#pragma unroll
  for (int j = 0; j < 8; ++j) sm[rl][cg * 8 + j] = acc[j];
  __syncthreads();
  double t = 0.0;
  if (tid < D) {
#pragma unroll
    for (int r = 0; r < kNrl; ++r) t += sm[r][tid];
  }
  return t;
}

// Partial query sums: part p of chunk c covers rows [p*ROWS, ...) of the
// chunk, all G heads.  grid (parts, H_kv, batch * n_chunks).
template <typename T, int G, int D, int ROWS>
__global__ __launch_bounds__(kScoreThreads) void k_chunk_qsum(
    const T* __restrict__ q, int64_t q_cap, int64_t q_off, int L, int Hq, int Hkv, int n_chunks,
    double* __restrict__ parts) {
  const int part = blockIdx.x, h = blockIdx.y;
  const int ch = blockIdx.z % n_chunks, bi = blockIdx.z / n_chunks;
  __shared__ double sm[kScoreThreads / (D / 8)][D];
  const T* qb = q + (((int64_t)bi * Hq + (int64_t)h * G) * q_cap + q_off + (int64_t)ch * L) * D;
  const int r0 = part * ROWS;
  const int r1 = r0 + ROWS < L ? r0 + ROWS : L;
  const double t = rows_colsum<T, G, D, ROWS>(qb, q_cap * D, r0, r1, sm);
  if (threadIdx.x < D) {
    const int n_parts = gridDim.x;
    parts[((((int64_t)bi * Hkv + h) * n_chunks + ch) * n_parts + part) * D + threadIdx.x] = t;
  }
}

// Scores of a slice of kUnitsPerWG units.  grid (slices, n_chunks * H_kv, batch).
// SEL >= 0: the selection is fused (score_slice).
template <typename T, int G, int D, int SEL>
__global__ __launch_bounds__(kScoreThreads) void k_score_units(
    const T* __restrict__ q, int64_t q_cap, int64_t q_off, int64_t q_pos,
    const int64_t* __restrict__ pos, int L, int Hq, int Hkv,
    int B, int n_init, int W, const float* __restrict__ repr, int U, float* __restrict__ scores,
    int n_chunks, const double* __restrict__ parts, int n_parts, int64_t part_stride,
    int64_t part0, int* __restrict__ count,
    int k_m, int32_t* __restrict__ sel) {
  const int ch = blockIdx.y % n_chunks, h = blockIdx.y / n_chunks, bi = blockIdx.z;
  const int64_t prob = ((int64_t)bi * Hkv + h) * n_chunks + ch;
  score_slice<T, G, D, SEL>(blockIdx.x, gridDim.x, ch, h, bi, q, q_cap, q_off, q_pos, pos, L, Hq,
                            Hkv, B, n_init, W, repr, U, scores, n_chunks, parts, n_parts,
                            part_stride, part0, count, k_m, sel ? sel + prob * k_m : nullptr);
}

// Long chunks with a moderate unit count, in one launch: each workgroup
// sums ROWS query rows of one chunk (all G heads) in fp64 and publishes
// the partial sum with device-scope stores; the last workgroup of a
// (sequence, KV head, chunk) to arrive -- found with a counter in the
// workspace, which it resets -- adds the partial sums in part order (so the
// result does not depend on arrival order) and scores every unit.  Its
// part loads and its first batch of unit rows are requested together.
// grid (parts, H_kv, batch * n_chunks).
template <typename T, int G, int D, int ROWS>
__global__ __launch_bounds__(kScoreThreads) void k_score_fused(
    const T* __restrict__ q, int64_t q_cap, int64_t q_off, int64_t q_pos,
    const int64_t* __restrict__ pos, int L, int Hq, int Hkv,
    int B, int n_init, int W, const float* __restrict__ repr, int U, float* __restrict__ scores,
    int n_chunks, double* __restrict__ parts, int* __restrict__ count) {
  using Rows = UnitRows<D, kBatchUnits / UnitRows<D, 1>::kPerSlot>;
  const int part = blockIdx.x, h = blockIdx.y;
  const int ch = blockIdx.z % n_chunks, bi = blockIdx.z / n_chunks;
  const int n_parts = gridDim.x;
  const int tid = threadIdx.x;
  __shared__ double sm[kScoreThreads / (D / 8)][D];
  __shared__ double qsum[D];
  __shared__ int last_sh;
  const T* qb = q + (((int64_t)bi * Hq + (int64_t)h * G) * q_cap + q_off + (int64_t)ch * L) * D;
  const int r0 = part * ROWS;
  const int r1 = r0 + ROWS < L ? r0 + ROWS : L;
  const double t = rows_colsum<T, G, D, ROWS>(qb, q_cap * D, r0, r1, sm);
  const int64_t prob = ((int64_t)bi * Hkv + h) * n_chunks + ch;
  double* pp = parts + prob * n_parts * D;
  if (tid < D)
    __hip_atomic_store(&pp[(int64_t)part * D + tid], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid == 0) {
    const int done = __hip_atomic_fetch_add(&count[prob], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    last_sh = done == n_parts - 1;
    if (last_sh)   // ready for the next call
      __hip_atomic_store(&count[prob], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last_sh) return;
  const float* rb = repr + ((int64_t)bi * Hkv + h) * U * D;
  Rows rows;
  rows.load(rb, U, 0);
  const double qs = sum_parts<D>(pp, n_parts, tid % D);
  if (tid < D) qsum[tid] = qs;
  __syncthreads();
  // a position out of range leaves no unit eligible (negative) or all of
  // them (large); the clamp keeps the sum below overflow
  int64_t t0 = seq_base(pos, q_pos, bi);
  t0 = t0 < -kPosLimit ? -kPosLimit : (t0 > kPosLimit ? kPosLimit : t0);
  const int64_t t_last = t0 + (int64_t)ch * L + L - 1;
  const int64_t e = eligible_units(t_last, U, B, n_init, W);
  const int cg = tid % 64 % (D / 8);
  double qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qv[j] = qsum[cg * 8 + j];
  float* sb = scores + prob * U;
  for (int base = 0; base < U; base += kBatchUnits) {
    if (base > 0) rows.load(rb, U, base);
    rows.score(qv, base, U, e, sb);
  }
}

static bool score_fused(const ScoreArgs& a) {
  return score_num_parts(a) > 0 && a.U <= kFusedMaxUnits;
}

// header and counter region (arrival counters at the region's start)
static size_t score_counter_bytes(const ScoreArgs& a) {
  return kWsHeaderBytes + ws_counter_region((size_t)a.batch * a.Hkv * a.n_chunks * sizeof(int));
}
static int* score_counters(const ScoreArgs& a) { return (int*)((char*)a.ws + kWsHeaderBytes); }

// [header][arrival counters][fp64 partial query sums]; sized for either
// path (the unit count is not known here)
size_t score_workspace_bytes(const ScoreArgs& a) {
  const int parts = score_num_parts(a);
  if (parts == 0) return 0;
  return score_counter_bytes(a) + (size_t)parts * a.batch * a.Hkv * a.n_chunks * a.d * sizeof(double);
}

// Scoring with the fused selection: the counters are needed by every path
// (the two-launch path for long chunks leaves them unused).
size_t select_workspace_bytes(const ScoreArgs& a) {
  const size_t w = score_workspace_bytes(a);
  return w > 0 ? w : score_counter_bytes(a);
}

static TopkArgs select_topk_args(const ScoreArgs& a) {
  TopkArgs t{};
  t.batch = a.batch;
  t.Hkv = a.Hkv;
  t.n_chunks = a.n_chunks;
  t.U = a.U;
  t.k_m = a.k_m;
  t.scores = a.scores;
  t.sel = a.sel;
  return t;
}

template <typename T, int G, int D, int ROWS>
static void launch_parts(const ScoreArgs& a, int parts, double* pw, hipStream_t st) {
  const dim3 grid(parts, a.Hkv, a.batch * a.n_chunks);
  if (score_fused(a))
    k_score_fused<T, G, D, ROWS><<<grid, kScoreThreads, 0, st>>>(
        (const T*)a.q, a.q_cap, a.q_off, a.q_pos, a.pos, a.L, a.Hq, a.Hkv, a.B, a.n_init, a.W, a.repr,
        a.U, a.scores, a.n_chunks, pw, score_counters(a));
  else
    k_chunk_qsum<T, G, D, ROWS><<<grid, kScoreThreads, 0, st>>>(
        (const T*)a.q, a.q_cap, a.q_off, a.L, a.Hq, a.Hkv, a.n_chunks, pw);
}

template <typename T, int G, int D>
static hipError_t launch_score_tgd(const ScoreArgs& a, hipStream_t st) {
  // chunk sums from block query sums: the chunk's L/B blocks are its parts
  const bool from_blocks = a.block_qsum != nullptr;
  const int parts = from_blocks ? a.L / a.B : score_num_parts(a);
  const double* pw = from_blocks ? a.block_qsum
                   : parts > 0   ? (const double*)((char*)a.ws + score_counter_bytes(a))
                                 : nullptr;
  const int64_t part_stride = from_blocks ? a.n_blocks : (int64_t)a.n_chunks * parts;
  const int64_t part0 = from_blocks ? a.q_pos / a.B : 0;
  if (parts > 0 && !from_blocks) {
    double* pwm = const_cast<double*>(pw);
    if (score_rows(a) == kRowsLong) launch_parts<T, G, D, kRowsLong>(a, parts, pwm, st);
    else launch_parts<T, G, D, kRowsShort>(a, parts, pwm, st);
    if (score_fused(a)) {
      // one workgroup scores each chunk; the selection is a launch of its own
      if (!a.sel) return hipGetLastError();
      return launch_topk(select_topk_args(a), st);
    }
  }
  dim3 grid((a.U + kUnitsPerWG - 1) / kUnitsPerWG, a.n_chunks * a.Hkv, a.batch);
#define INFLLM_SCORE_UNITS(SEL, CNT)                                                            \
  k_score_units<T, G, D, SEL><<<grid, kScoreThreads, 0, st>>>(                                 \
      (const T*)a.q, a.q_cap, a.q_off, a.q_pos, a.pos, a.L, a.Hq, a.Hkv, a.B, a.n_init, a.W,     \
      a.repr, a.U, a.scores, a.n_chunks, pw, parts, part_stride, part0, CNT, a.k_m, a.sel)
  if (!a.sel || grid.x > kMaxSelSlices) {
    INFLLM_SCORE_UNITS(-1, nullptr);
    if (a.sel) return launch_topk(select_topk_args(a), st);
  } else {
    // keys per lane of the 4-wave search: ceil(U / 256) <= 8
    static_assert(kMaxSelSlices * kUnitsPerWG <= 8 * kScoreThreads, "keys per lane");
    int* cnt = score_counters(a);
    if (a.U <= 4 * kScoreThreads) INFLLM_SCORE_UNITS(4, cnt);
    else INFLLM_SCORE_UNITS(8, cnt);
  }
#undef INFLLM_SCORE_UNITS
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_score_td(const ScoreArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_score_tgd<T, 1, D>(a, st);
    case 2: return launch_score_tgd<T, 2, D>(a, st);
    case 4: return launch_score_tgd<T, 4, D>(a, st);
    case 8: return launch_score_tgd<T, 8, D>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_score_t(const ScoreArgs& a, hipStream_t st) {
  return a.d == 128 ? launch_score_td<T, 128>(a, st) : launch_score_td<T, 64>(a, st);
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  if (a.n_chunks <= 0) return hipSuccess;
  if (a.U <= 0) return a.sel ? launch_topk(select_topk_args(a), st) : hipSuccess;   // all -1
  return a.bf16 ? launch_score_t<bf16_t>(a, st) : launch_score_t<float>(a, st);
}

}  // namespace infllm
