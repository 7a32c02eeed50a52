// Unit scoring by slices of kUnitsPerWG units, shared by the scoring
// kernels and the fused decode step (see score.hip for the scheme).
#pragma once

#include "common.h"
#include "topk_select.h"

namespace infllm {

constexpr int kScoreThreads = 256;
constexpr int kUnitsPerWG = 64;
constexpr int kDirectRows = 64;      // L*G up to this: sum in the scoring kernel
constexpr int kPartBatch = 16;       // partial sums requested together
// Fused selection up to this many slices per row: beyond, the arrivals on
// one row's counter serialize (measured: 128 slices cost more than a
// separate top-k launch)
constexpr int kMaxSelSlices = 32;

// Sum of the n_parts partial sums of column c (part p at pp[p*D + c]), in
// part order.  Loads past the last part return 0 and leave the sum as is.
template <int D>
__device__ __forceinline__ double sum_parts(const double* pp, int n_parts, int c) {
  const __amdgpu_buffer_rsrc_t r = dev_rsrc(pp, (uint32_t)((int64_t)n_parts * D * 8));
  double t = 0.0;
  for (int p0 = 0; p0 < n_parts; p0 += kPartBatch) {
    double v[kPartBatch];
#pragma unroll
    for (int j = 0; j < kPartBatch; ++j) v[j] = ld1_dev_f64(r, (uint32_t)(((p0 + j) * D + c) * 8));
#pragma unroll
    for (int j = 0; j < kPartBatch; ++j) t += v[j];
  }
  return t;
}

// Unit rows for scoring: D/8 lanes per unit, 8 columns each; slot s of
// wave w holds units base + s*(4*upw) + w*upw + lane/(D/8).  Indices past
// the last unit are clamped (their scores are not stored).
template <int D, int kSlots>
struct UnitRows {
  static constexpr int kLpu = D / 8, kUpw = 64 / kLpu, kPerSlot = (kScoreThreads / 64) * kUpw;
  Raw8<float> x[kSlots];
  __device__ __forceinline__ static int unit(int base, int s) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    return base + s * kPerSlot + wave * kUpw + lane / kLpu;
  }
  __device__ __forceinline__ void load(const float* rb, int U, int base) {
    const int cg = threadIdx.x % 64 % kLpu;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const int u = unit(base, s);
      x[s].load(rb + (int64_t)(u < U ? u : U - 1) * D + cg * 8);
    }
  }
  // score[u] = qsum . repr[u] (fp64), -inf for u >= e; units in [base, u1).
  // DEV: device-scope stores, for a selection by another workgroup.
  template <bool DEV = false>
  __device__ __forceinline__ void score(const double* qv, int base, int u1, int64_t e,
                                        float* sb) const {
    const int cg = threadIdx.x % 64 % kLpu;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const int u = unit(base, s);
      double t = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) t = fma(x[s].get(j), qv[j], t);
      t += dpp_f64<INFLLM_DPP_XOR1>(t);
      t += dpp_f64<INFLLM_DPP_XOR2>(t);
      t += dpp_f64<INFLLM_DPP_HALF_MIRROR>(t);
      if (kLpu == 16) t += dpp_f64<INFLLM_DPP_MIRROR>(t);
      if (u < u1 && cg == 0) {
        const float v = u < e ? (float)t : -INFINITY;
        if (DEV) st_dev(sb + u, v);
        else sb[u] = v;
      }
    }
  }
  // The same scores, written to sb[u] and to lds[u - lds0].
  __device__ __forceinline__ void score_lds(const double* qv, int base, int u1, int64_t e,
                                            float* sb, float* lds, int lds0) const {
    const int cg = threadIdx.x % 64 % kLpu;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const int u = unit(base, s);
      double t = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) t = fma(x[s].get(j), qv[j], t);
      t += dpp_f64<INFLLM_DPP_XOR1>(t);
      t += dpp_f64<INFLLM_DPP_XOR2>(t);
      t += dpp_f64<INFLLM_DPP_HALF_MIRROR>(t);
      if (kLpu == 16) t += dpp_f64<INFLLM_DPP_MIRROR>(t);
      if (u < u1 && cg == 0) {
        const float v = u < e ? (float)t : -INFINITY;
        sb[u] = v;
        lds[u - lds0] = v;
      }
    }
  }
};

// Scores of slice `slice` (of n_slices, kUnitsPerWG units each) for chunk ch
// of KV head h of sequence bi, by one workgroup of kScoreThreads threads.
// SEL >= 0: the selection is fused -- the scores are published with
// device-scope stores, and the last slice of a (sequence, KV head, chunk)
// to arrive (arrival counter in `count`, which it resets) selects that
// row's top k_m into sel_row with the workgroup search, SEL keys per lane
// (0: re-read from memory) and returns true; every other workgroup returns
// false.
template <typename T, int G, int D, int SEL>
__device__ __forceinline__ bool score_slice(
    int slice, int n_slices, int ch, int h, int bi, const T* __restrict__ q, int64_t q_cap, int64_t q_off, int64_t q_pos,
    const int64_t* __restrict__ pos, int L, int Hq, int Hkv,
    int B, int n_init, int W, const float* __restrict__ repr, int U, float* __restrict__ scores,
    int n_chunks, const double* __restrict__ parts, int n_parts, int64_t part_stride,
    int64_t part0, int* __restrict__ count,
    int k_m, int32_t* sel_row) {
  using Rows = UnitRows<D, kUnitsPerWG / UnitRows<D, 1>::kPerSlot>;
  const int tid = threadIdx.x;
  __shared__ double part_sm[kScoreThreads];
  __shared__ double qsum[D];
  const int u0 = slice * kUnitsPerWG;
  const int u1 = u0 + kUnitsPerWG < U ? u0 + kUnitsPerWG : U;
  const float* rb = repr + ((int64_t)bi * Hkv + h) * U * D;
  Rows rows;
  rows.load(rb, U, u0);              // in flight while the query sum forms

  if (n_parts > 0) {
    // partial sums of chunk ch: n_parts rows from row part0 + ch * n_parts
    // of this (sequence, KV head)'s part_stride rows
    const double* pp = parts + (((int64_t)bi * Hkv + h) * part_stride + part0 +
                                (int64_t)ch * n_parts) * D;
    const double t = sum_parts<D>(pp, n_parts, tid % D);
    if (tid < D) qsum[tid] = t;
    __syncthreads();
  } else {
    // few rows (L*G <= kDirectRows): thread -> (column, row phase)
    constexpr int kNph = kScoreThreads / D;
    constexpr int kIt = (kDirectRows / G + kNph - 1) / kNph;
    const int c = tid % D, phase = tid / D;
    const T* qb = q + (((int64_t)bi * Hq + (int64_t)h * G) * q_cap + q_off + (int64_t)ch * L) * D + c;
    const int n_it = (L + kNph - 1) / kNph;     // row iterations the chunk needs
    T v[G][kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      if (it >= n_it) break;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int i = phase + it * kNph;
        v[g][it] = qb[g * q_cap * D + (int64_t)(i < L ? i : L - 1) * D];
      }
    }
    double acc = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        if (it >= n_it) break;
        if (phase + it * kNph < L) acc += (double)to_f32(v[g][it]);
      }
    part_sm[tid] = acc;
    __syncthreads();
    if (phase == 0) {
#pragma unroll
      for (int p = 1; p < kNph; ++p) acc += part_sm[p * D + c];
      qsum[c] = acc;
    }
    __syncthreads();
  }

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
  const int64_t prob = ((int64_t)bi * Hkv + h) * n_chunks + ch;
  float* sb = scores + prob * U;
  if constexpr (SEL < 0) {
    rows.score(qv, u0, u1, e, sb);
  } else {
    __shared__ TopkShared tsm;
    __shared__ int last_sh;
    rows.template score<true>(qv, u0, u1, e, sb);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
      const int done = __hip_atomic_fetch_add(&count[prob], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      last_sh = done == n_slices - 1;
      if (last_sh)   // ready for the next call
        __hip_atomic_store(&count[prob], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_sh) return false;
    block_topk<kScoreThreads / 64, SEL, true>(sb, U, k_m, sel_row, tsm);
    return true;
  }
  return false;
}

}  // namespace infllm
