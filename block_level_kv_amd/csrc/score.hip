// Unit relevance scores: for chunk c and KV head h,
//     score[u] = (sum of the chunk's queries over the group's heads) . repr[u]
// for eligible u, -inf otherwise (InfLLM Guide, "Core Innovation 2", item 2;
// authors' rebuttal, "Latency Across Different Context Windows").  The query
// sum and the dot products accumulate in fp64, so the ranking that follows
// is decided on scores accurate far below the near-tie margin.
//
// A workgroup handles one (chunk, KV head, sequence) and a slice of up to
// kUnitsPerWG units: the chunk query sum is formed once in LDS, then each
// wave scores one unit at a time with a coalesced read of its fp32 row.
#include "common.h"
#include "kernels.h"

namespace infllm {

constexpr int kScoreThreads = 256;
constexpr int kUnitsPerWG = 512;

template <typename T>
__global__ __launch_bounds__(kScoreThreads) void k_score_units(
    const T* __restrict__ q, int64_t q_cap, int64_t q_off, int64_t q_pos, int L, int Hq, int Hkv,
    int d, int B, int n_init, int W, const float* __restrict__ repr, int U,
    float* __restrict__ scores, int n_chunks) {
  const int slice = blockIdx.x;
  const int ch = blockIdx.y % n_chunks, h = blockIdx.y / n_chunks, bi = blockIdx.z;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  __shared__ double part[kScoreThreads];
  __shared__ double qsum[128];

  // chunk query sum, fp64: thread -> (column, row phase)
  {
    const int c = tid % d, phase = tid / d, nph = kScoreThreads / d;
    double acc = 0.0;
    const int64_t row0 = q_off + (int64_t)ch * L;
    for (int g = 0; g < G; ++g) {
      const T* qh = q + (((int64_t)bi * Hq + (int64_t)h * G + g) * q_cap + row0) * d + c;
      for (int i = phase; i < L; i += nph) acc += (double)to_f32(qh[(int64_t)i * d]);
    }
    part[tid] = acc;
    __syncthreads();
    if (phase == 0) {
      for (int p = 1; p < nph; ++p) acc += part[p * d + c];
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
  for (int u = u0 + wave; u < u1; u += kScoreThreads / 64) {
    if (u >= e) {
      if (lane == 0) sb[u] = -INFINITY;
      continue;
    }
    double s = 0.0;
    for (int c = lane; c < d; c += 64) s += (double)rb[(int64_t)u * d + c] * qsum[c];
    s = wave_sum_f64(s);
    if (lane == 0) sb[u] = (float)s;
  }
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  if (a.U <= 0 || a.n_chunks <= 0) return hipSuccess;
  dim3 grid((a.U + kUnitsPerWG - 1) / kUnitsPerWG, a.n_chunks * a.Hkv, a.batch);
  if (a.bf16)
    k_score_units<bf16_t><<<grid, kScoreThreads, 0, st>>>(
        (const bf16_t*)a.q, a.q_cap, a.q_off, a.q_pos, a.L, a.Hq, a.Hkv, a.d, a.B, a.n_init, a.W,
        a.repr, a.U, a.scores, a.n_chunks);
  else
    k_score_units<float><<<grid, kScoreThreads, 0, st>>>(
        (const float*)a.q, a.q_cap, a.q_off, a.q_pos, a.L, a.Hq, a.Hkv, a.d, a.B, a.n_init, a.W,
        a.repr, a.U, a.scores, a.n_chunks);
  return hipGetLastError();
}

}  // namespace infllm
