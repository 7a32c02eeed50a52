// Unit relevance scores: for chunk c and KV head h,
//     score[u] = (sum of the chunk's queries over the group's heads) . repr[u]
// for eligible u, -inf otherwise (InfLLM Guide, "Core Innovation 2", item 2;
// authors' rebuttal, "Latency Across Different Context Windows").  The query
// sum and the dot products accumulate in fp64, so the ranking that follows
// is decided on scores accurate far below the near-tie margin.
//
// Long chunks (unit count above kFusedMaxUnits; smaller counts take the
// one-launch k_score_fused below): k_chunk_qsum spreads the query sum over many workgroups
// (16-byte loads, kQsumRows query rows each) and writes fp64 partial sums;
// k_score_units adds them in a fixed order, so results do not depend on
// scheduling.  Short chunks (decode: one query x G heads) skip the first
// pass and sum their few rows directly.  k_score_units then scores a slice
// of up to kUnitsPerWG units, one wave per unit at a time with a coalesced
// read of its fp32 representation.
#include "common.h"
#include "kernels.h"

namespace infllm {

constexpr int kScoreThreads = 256;
constexpr int kUnitsPerWG = 64;
constexpr int kQsumRows = 32;        // chunk rows per partial sum
constexpr int kDirectRows = 64;      // L*G up to this: sum in the scoring kernel

template <typename T> struct Load8;
template <> struct Load8<bf16_t> {
  static __device__ __forceinline__ void add(const bf16_t* p, double* acc) {
    const u32x4 w = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += (double)__uint_as_float(w[i] << 16);
      acc[2 * i + 1] += (double)__uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Load8<float> {
  static __device__ __forceinline__ void add(const float* p, double* acc) {
    const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
};

int score_num_parts(int L, int G) {
  return L * G <= kDirectRows ? 0 : (L + kQsumRows - 1) / kQsumRows;
}

// Partial query sums: part p of chunk c covers rows [p*kQsumRows, ...) of
// the chunk, all G heads.  grid (parts, H_kv, batch * n_chunks).
template <typename T>
__global__ __launch_bounds__(kScoreThreads) void k_chunk_qsum(
    const T* __restrict__ q, int64_t q_cap, int64_t q_off, int L, int Hq, int Hkv, int d,
    int n_chunks, double* __restrict__ parts) {
  const int part = blockIdx.x, h = blockIdx.y;
  const int ch = blockIdx.z % n_chunks, bi = blockIdx.z / n_chunks;
  const int G = Hq / Hkv;
  const int cgs = d / 8;                            // 8-column groups per row
  const int cg = threadIdx.x % cgs, rl = threadIdx.x / cgs, nrl = kScoreThreads / cgs;
  const int r0 = part * kQsumRows;
  const int r1 = r0 + kQsumRows < L ? r0 + kQsumRows : L;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int g = 0; g < G; ++g) {
    const T* qh = q + (((int64_t)bi * Hq + (int64_t)h * G + g) * q_cap + q_off +
                       (int64_t)ch * L) * d + cg * 8;
    for (int i = r0 + rl; i < r1; i += nrl) Load8<T>::add(qh + (int64_t)i * d, acc);
  }
  __shared__ double sm[kScoreThreads / 8][128];     // [row lane][column]
#pragma unroll
  for (int j = 0; j < 8; ++j) sm[rl][cg * 8 + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < d) {
    double s = 0.0;
    for (int r = 0; r < nrl; ++r) s += sm[r][threadIdx.x];
    const int n_parts = gridDim.x;
    parts[((((int64_t)bi * Hkv + h) * n_chunks + ch) * n_parts + part) * d + threadIdx.x] = s;
  }
}

template <typename T>
__global__ __launch_bounds__(kScoreThreads) void k_score_units(
    const T* __restrict__ q, int64_t q_cap, int64_t q_off, int64_t q_pos, int L, int Hq, int Hkv,
    int d, int B, int n_init, int W, const float* __restrict__ repr, int U,
    float* __restrict__ scores, int n_chunks, const double* __restrict__ parts, int n_parts) {
  const int slice = blockIdx.x;
  const int ch = blockIdx.y % n_chunks, h = blockIdx.y / n_chunks, bi = blockIdx.z;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  __shared__ double part_sm[kScoreThreads];
  __shared__ double qsum[128];

  if (n_parts > 0) {
    if (tid < d) {
      const double* pp = parts + (((int64_t)bi * Hkv + h) * n_chunks + ch) * n_parts * d + tid;
      double s = 0.0;
      for (int p = 0; p < n_parts; ++p) s += pp[(int64_t)p * d];
      qsum[tid] = s;
    }
    __syncthreads();
  } else {
    // few rows: thread -> (column, row phase)
    const int c = tid % d, phase = tid / d, nph = kScoreThreads / d;
    double acc = 0.0;
    const int64_t row0 = q_off + (int64_t)ch * L;
    for (int g = 0; g < G; ++g) {
      const T* qh = q + (((int64_t)bi * Hq + (int64_t)h * G + g) * q_cap + row0) * d + c;
      for (int i = phase; i < L; i += nph) acc += (double)to_f32(qh[(int64_t)i * d]);
    }
    part_sm[tid] = acc;
    __syncthreads();
    if (phase == 0) {
      for (int p = 1; p < nph; ++p) acc += part_sm[p * d + c];
      qsum[c] = acc;
    }
    __syncthreads();
  }

  const int64_t t_last = q_pos + (int64_t)ch * L + L - 1;
  const int64_t e = eligible_units(t_last, U, B, n_init, W);
  const int wave = tid / 64, lane = tid % 64;
  const int u0 = slice * kUnitsPerWG;
  const int u1 = u0 + kUnitsPerWG < U ? u0 + kUnitsPerWG : U;
  const float* rb = repr + ((int64_t)bi * Hkv + h) * U * d;
  float* sb = scores + (((int64_t)bi * Hkv + h) * n_chunks + ch) * U;
  // d/8 lanes per unit (a DPP row or half row), 8 columns each
  const int lpu = d / 8, upw = 64 / lpu;
  const int sub = lane / lpu, cg = lane % lpu;
  double qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qv[j] = qsum[cg * 8 + j];
  for (int ub = u0 + wave * upw; ub < u1; ub += (kScoreThreads / 64) * upw) {
    const int u = ub + sub;
    double s = 0.0;
    if (u < u1 && u < e) {
      const float4* rp = (const float4*)(rb + (int64_t)u * d + cg * 8);
      const float4 x = rp[0], y = rp[1];
      s = fma((double)x.x, qv[0], s);
      s = fma((double)x.y, qv[1], s);
      s = fma((double)x.z, qv[2], s);
      s = fma((double)x.w, qv[3], s);
      s = fma((double)y.x, qv[4], s);
      s = fma((double)y.y, qv[5], s);
      s = fma((double)y.z, qv[6], s);
      s = fma((double)y.w, qv[7], s);
    }
    s += dpp_f64<INFLLM_DPP_XOR1>(s);
    s += dpp_f64<INFLLM_DPP_XOR2>(s);
    s += dpp_f64<INFLLM_DPP_HALF_MIRROR>(s);
    if (lpu == 16) s += dpp_f64<INFLLM_DPP_MIRROR>(s);
    if (u < u1 && cg == 0) sb[u] = u < e ? (float)s : -INFINITY;
  }
}

// Long chunks with a moderate unit count, in one launch: each workgroup
// sums kQsumRows query rows of one chunk (all G heads) in fp64 and publishes
// the partial sum with device-scope stores; the last workgroup of a
// (sequence, KV head, chunk) to arrive -- found with a counter in the
// workspace, which it resets -- adds the partial sums in part order (so the
// result does not depend on arrival order) and scores every unit.
// grid (parts, H_kv, batch * n_chunks).
constexpr int kFusedMaxUnits = 2048;

template <typename T>
__global__ __launch_bounds__(kScoreThreads) void k_score_fused(
    const T* __restrict__ q, int64_t q_cap, int64_t q_off, int64_t q_pos, int L, int Hq, int Hkv,
    int d, int B, int n_init, int W, const float* __restrict__ repr, int U,
    float* __restrict__ scores, int n_chunks, double* __restrict__ parts, int* __restrict__ count) {
  const int part = blockIdx.x, h = blockIdx.y;
  const int ch = blockIdx.z % n_chunks, bi = blockIdx.z / n_chunks;
  const int n_parts = gridDim.x;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int cgs = d / 8;
  const int cg = tid % cgs, rl = tid / cgs, nrl = kScoreThreads / cgs;
  const int r0 = part * kQsumRows;
  const int r1 = r0 + kQsumRows < L ? r0 + kQsumRows : L;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int g = 0; g < G; ++g) {
    const T* qh = q + (((int64_t)bi * Hq + (int64_t)h * G + g) * q_cap + q_off +
                       (int64_t)ch * L) * d + cg * 8;
    for (int i = r0 + rl; i < r1; i += nrl) Load8<T>::add(qh + (int64_t)i * d, acc);
  }
  __shared__ double sm[kScoreThreads / 8][128];     // [row lane][column]
  __shared__ double qsum[128];
  __shared__ int last_sh;
#pragma unroll
  for (int j = 0; j < 8; ++j) sm[rl][cg * 8 + j] = acc[j];
  __syncthreads();
  const int64_t prob = ((int64_t)bi * Hkv + h) * n_chunks + ch;
  double* pp = parts + prob * n_parts * d;
  if (tid < d) {
    double t = 0.0;
    for (int r = 0; r < nrl; ++r) t += sm[r][tid];
    __hip_atomic_store(&pp[(int64_t)part * d + tid], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
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
  if (tid < d) {
    double t = 0.0;
    for (int p = 0; p < n_parts; ++p)
      t += __hip_atomic_load(&pp[(int64_t)p * d + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    qsum[tid] = t;
  }
  __syncthreads();
  const int64_t t_last = q_pos + (int64_t)ch * L + L - 1;
  const int64_t e = eligible_units(t_last, U, B, n_init, W);
  const int wave = tid / 64, lane = tid % 64;
  const float* rb = repr + ((int64_t)bi * Hkv + h) * U * d;
  float* sb = scores + prob * U;
  const int lpu = d / 8, upw = 64 / lpu;
  const int sub = lane / lpu, cgl = lane % lpu;
  double qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qv[j] = qsum[cgl * 8 + j];
  for (int ub = wave * upw; ub < U; ub += (kScoreThreads / 64) * upw) {
    const int u = ub + sub;
    double t = 0.0;
    if (u < U && u < e) {
      const float4* rp = (const float4*)(rb + (int64_t)u * d + cgl * 8);
      const float4 x = rp[0], y = rp[1];
      t = fma((double)x.x, qv[0], t);
      t = fma((double)x.y, qv[1], t);
      t = fma((double)x.z, qv[2], t);
      t = fma((double)x.w, qv[3], t);
      t = fma((double)y.x, qv[4], t);
      t = fma((double)y.y, qv[5], t);
      t = fma((double)y.z, qv[6], t);
      t = fma((double)y.w, qv[7], t);
    }
    t += dpp_f64<INFLLM_DPP_XOR1>(t);
    t += dpp_f64<INFLLM_DPP_XOR2>(t);
    t += dpp_f64<INFLLM_DPP_HALF_MIRROR>(t);
    if (lpu == 16) t += dpp_f64<INFLLM_DPP_MIRROR>(t);
    if (u < U && cgl == 0) sb[u] = u < e ? (float)t : -INFINITY;
  }
}

static bool score_fused(const ScoreArgs& a) {
  return score_num_parts(a.L, a.Hq / a.Hkv) > 0 && a.U <= kFusedMaxUnits;
}

static size_t score_counter_bytes(const ScoreArgs& a) {
  return ((size_t)a.batch * a.Hkv * a.n_chunks * sizeof(int) + 255) & ~(size_t)255;
}

// [arrival counters, 256-byte aligned][fp64 partial query sums]; sized for
// either path (the unit count is not known here)
size_t score_workspace_bytes(const ScoreArgs& a) {
  const int parts = score_num_parts(a.L, a.Hq / a.Hkv);
  if (parts == 0) return 0;
  return score_counter_bytes(a) + (size_t)parts * a.batch * a.Hkv * a.n_chunks * a.d * sizeof(double);
}

template <typename T>
static hipError_t launch_score_t(const ScoreArgs& a, hipStream_t st) {
  const int parts = score_num_parts(a.L, a.Hq / a.Hkv);
  double* pw = parts > 0 ? (double*)((char*)a.ws + score_counter_bytes(a)) : nullptr;
  if (score_fused(a)) {
    k_score_fused<T><<<dim3(parts, a.Hkv, a.batch * a.n_chunks), kScoreThreads, 0, st>>>(
        (const T*)a.q, a.q_cap, a.q_off, a.q_pos, a.L, a.Hq, a.Hkv, a.d, a.B, a.n_init, a.W,
        a.repr, a.U, a.scores, a.n_chunks, pw, (int*)a.ws);
    return hipGetLastError();
  }
  if (parts > 0)
    k_chunk_qsum<T><<<dim3(parts, a.Hkv, a.batch * a.n_chunks), kScoreThreads, 0, st>>>(
        (const T*)a.q, a.q_cap, a.q_off, a.L, a.Hq, a.Hkv, a.d, a.n_chunks, pw);
  dim3 grid((a.U + kUnitsPerWG - 1) / kUnitsPerWG, a.n_chunks * a.Hkv, a.batch);
  k_score_units<T><<<grid, kScoreThreads, 0, st>>>(
      (const T*)a.q, a.q_cap, a.q_off, a.q_pos, a.L, a.Hq, a.Hkv, a.d, a.B, a.n_init, a.W, a.repr,
      a.U, a.scores, a.n_chunks, pw, parts);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  if (a.U <= 0 || a.n_chunks <= 0) return hipSuccess;
  return a.bf16 ? launch_score_t<bf16_t>(a, st) : launch_score_t<float>(a, st);
}

}  // namespace infllm
