// Working-context attention for one query position per workgroup, on the
// vector ALUs.  This is the decode path (one query per step, the G query
// heads of a KV head share every K/V row loaded) and the path for fp32 and
// head sizes the MFMA kernel does not take.
//
// For a single position t the working context (InfLLM Guide, "Core
// Innovation 2", item 3; "Core Innovation 1", items 1-2) is a union of
// disjoint key intervals:
//     [0, min(n_init, t+1))                     initial tokens
//     [first_key(u), min(end(u), t-W+1))        each selected unit u
//     [max(n_init, t-W+1), t+1)                 local window (t included)
// so no per-key mask is needed.  The intervals' keys are numbered 0..n-1 and
// split evenly over gridDim.x workgroups (split-K); each writes a partial
// (max, sum, unnormalised output) that k_combine merges.  Within a workgroup
// 16 lanes share a key (each holds D/16 columns: one coalesced 16-byte load
// per lane for bf16, D = 128) and the 16 key lanes run independent online
// softmaxes that are merged through LDS at the end.
#include "common.h"
#include "kernels.h"

namespace infllm {

constexpr int kRowsThreads = 256;
constexpr int kMaxIntervals = kMaxTopK + 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T, int CPT> struct RowLoad;
template <> struct RowLoad<bf16_t, 8> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* o) {
    const u32x4 w = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct RowLoad<bf16_t, 4> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* o) {
    const uint2 w = *(const uint2*)p;
    o[0] = __uint_as_float(w.x << 16);
    o[1] = __uint_as_float(w.x & 0xffff0000u);
    o[2] = __uint_as_float(w.y << 16);
    o[3] = __uint_as_float(w.y & 0xffff0000u);
  }
};
template <> struct RowLoad<float, 8> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
    const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};
template <> struct RowLoad<float, 4> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
    const float4 a = *(const float4*)p;
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  }
};

constexpr int kKeysPerIter = 4;  // keys per lane between softmax rescales

template <typename T, int D, int G>
__global__ __launch_bounds__(kRowsThreads) void k_attend_rows(AttendArgs a) {
  constexpr int CPT = D / 16;
  const int split = blockIdx.x, pos = blockIdx.y;
  const int h = blockIdx.z % a.Hkv, bi = blockIdx.z / a.Hkv;
  const int tid = threadIdx.x, seg = tid % 16, kl = tid / 16;
  const int ch = pos / a.L;
  const int64_t t = a.q_pos + pos;

  __shared__ int64_t iv_lo[kMaxIntervals];
  __shared__ int64_t iv_end[kMaxIntervals + 1];  // exclusive prefix of lengths
  __shared__ int n_iv;
  if (tid == 0) {
    int n = 0;
    int64_t total = 0;
    auto add = [&](int64_t lo, int64_t hi) {
      if (hi > lo) {
        iv_lo[n] = lo;
        total += hi - lo;
        iv_end[n] = total;
        ++n;
      }
    };
    add(0, a.n_init < t + 1 ? a.n_init : t + 1);
    const int64_t unit_cap = t - a.W + 1;
    for (int m = 0; m < a.k_m; ++m) {
      const int32_t u = a.sel[(((int64_t)bi * a.Hkv + h) * a.n_chunks + ch) * a.k_m + m];
      if (u < 0) continue;
      const int64_t lo = unit_first_key(u, a.B, a.n_init);
      const int64_t hi = ((int64_t)u + a.n_init / a.B + 1) * a.B;
      add(lo, hi < unit_cap ? hi : unit_cap);
    }
    add(a.n_init > unit_cap ? a.n_init : unit_cap, t + 1);
    n_iv = n;
  }
  __syncthreads();
  const int niv = n_iv;
  const int64_t n_keys = niv > 0 ? iv_end[niv - 1] : 0;
  const int64_t per = (n_keys + gridDim.x - 1) / gridDim.x;
  const int64_t k_begin = (int64_t)split * per;
  const int64_t k_stop = k_begin + per < n_keys ? k_begin + per : n_keys;

  const T* kb = (const T*)a.k + ((int64_t)bi * a.Hkv + h) * a.kv_cap * D + seg * CPT;
  const T* vb = (const T*)a.v + ((int64_t)bi * a.Hkv + h) * a.kv_cap * D + seg * CPT;
  const float qscale = kLog2e / sqrtf((float)D);
  float qv[G][CPT];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const T* qp = (const T*)a.q +
                  (((int64_t)bi * a.Hq + (int64_t)h * G + g) * a.q_cap + a.q_off + pos) * D +
                  seg * CPT;
    RowLoad<T, CPT>::load(qp, qv[g]);
#pragma unroll
    for (int c = 0; c < CPT; ++c) qv[g][c] *= qscale;
  }
  float m[G], l[G], acc[G][CPT];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[g][c] = 0.f;
  }

  int cur = 0;
  auto key_pos = [&](int64_t idx) -> int64_t {
    while (idx >= iv_end[cur]) ++cur;
    return iv_lo[cur] + (idx - (cur ? iv_end[cur - 1] : 0));
  };

  for (int64_t base = k_begin; base < k_stop; base += 16 * kKeysPerIter) {
    float kr[kKeysPerIter][CPT], vr[kKeysPerIter][CPT];
    bool ok[kKeysPerIter];
#pragma unroll
    for (int j = 0; j < kKeysPerIter; ++j) {
      const int64_t idx = base + kl + 16 * j;
      ok[j] = idx < k_stop;
      const int64_t p = ok[j] ? key_pos(idx) : 0;
      RowLoad<T, CPT>::load(kb + p * D, kr[j]);
      RowLoad<T, CPT>::load(vb + p * D, vr[j]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s[kKeysPerIter];
      float mx = m[g];
#pragma unroll
      for (int j = 0; j < kKeysPerIter; ++j) {
        float d0 = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) d0 = fmaf(qv[g][c], kr[j][c], d0);
        const float r = row16_sum(d0);  // the 16 lanes of a row share key j
        s[j] = ok[j] ? r : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      if (mx == -INFINITY) continue;  // no valid key yet for this lane group
      const float alpha = exp2f(m[g] - mx);
      m[g] = mx;
      float lsum = l[g] * alpha;
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[g][c] *= alpha;
#pragma unroll
      for (int j = 0; j < kKeysPerIter; ++j) {
        const float p = exp2f(s[j] - mx);
        lsum += p;
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[g][c] = fmaf(p, vr[j][c], acc[g][c]);
      }
      l[g] = lsum;
    }
  }

  // merge the 16 key lanes
  __shared__ float sm_m[16][G], sm_l[16][G];
  __shared__ float sm_o[16][G][D];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (seg == 0) {
      sm_m[kl][g] = m[g];
      sm_l[kl][g] = l[g];
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) sm_o[kl][g][seg * CPT + c] = acc[g][c];
  }
  __syncthreads();
  for (int o = tid; o < G * D; o += kRowsThreads) {
    const int g = o / D, col = o % D;
    float M = -INFINITY;
    for (int r = 0; r < 16; ++r) M = fmaxf(M, sm_m[r][g]);
    float Lsum = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int r = 0; r < 16; ++r) {
        const float w = exp2f(sm_m[r][g] - M);
        Lsum += sm_l[r][g] * w;
        O += sm_o[r][g][col] * w;
      }
    }
    const int64_t qh = (int64_t)bi * a.Hq + (int64_t)h * G + g;
    if (gridDim.x == 1) {
      T* out = (T*)a.out + (qh * a.out_cap + a.out_off + pos) * D + col;
      *out = from_f32<T>(O / Lsum);
      if (a.lse && col == 0) a.lse[qh * a.out_cap + a.out_off + pos] = (M + log2f(Lsum)) * kLn2;
    } else {
      const int64_t row = (((int64_t)split * a.batch * a.Hq) + qh) * a.n_pos + pos;
      a.ws_o[row * D + col] = O;
      if (col == 0) {
        a.ws_ml[2 * row] = M;
        a.ws_ml[2 * row + 1] = Lsum;
      }
    }
  }
}

// Merge split-K partials: o = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// grid (n_pos, H_q, batch), D threads.
template <typename T, int D>
__global__ void k_combine(AttendArgs a, int n_splits) {
  const int pos = blockIdx.x, qh_in = blockIdx.y, bi = blockIdx.z, col = threadIdx.x;
  const int64_t qh = (int64_t)bi * a.Hq + qh_in;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) {
    const int64_t row = ((int64_t)s * a.batch * a.Hq + qh) * a.n_pos + pos;
    M = fmaxf(M, a.ws_ml[2 * row]);
  }
  float Lsum = 0.f, O = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const int64_t row = ((int64_t)s * a.batch * a.Hq + qh) * a.n_pos + pos;
    const float ms = a.ws_ml[2 * row];
    if (ms == -INFINITY) continue;
    const float w = exp2f(ms - M);
    Lsum += a.ws_ml[2 * row + 1] * w;
    O += a.ws_o[row * D + col] * w;
  }
  T* out = (T*)a.out + (qh * a.out_cap + a.out_off + pos) * D + col;
  *out = from_f32<T>(O / Lsum);
  if (a.lse && col == 0) a.lse[qh * a.out_cap + a.out_off + pos] = (M + log2f(Lsum)) * kLn2;
}

int rows_num_splits(const AttendArgs& a) {
  // enough workgroups to cover the chip twice, at least ~256 keys per split
  const int64_t max_keys = (int64_t)a.n_init + (int64_t)a.k_m * a.B + a.W;
  const int64_t wgs = (int64_t)a.n_pos * a.batch * a.Hkv;
  int64_t s = (512 + wgs - 1) / wgs;
  const int64_t cap = (max_keys + 255) / 256;
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  return s < 1 ? 1 : (int)s;
}

hipError_t launch_combine(const AttendArgs& a, int splits, hipStream_t st) {
  const dim3 grid(a.n_pos, a.Hq, a.batch);
  if (a.bf16) {
    if (a.d == 128) k_combine<bf16_t, 128><<<grid, 128, 0, st>>>(a, splits);
    else k_combine<bf16_t, 64><<<grid, 64, 0, st>>>(a, splits);
  } else {
    if (a.d == 128) k_combine<float, 128><<<grid, 128, 0, st>>>(a, splits);
    else k_combine<float, 64><<<grid, 64, 0, st>>>(a, splits);
  }
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t launch_rows_tdg(const AttendArgs& a, int splits, hipStream_t st) {
  k_attend_rows<T, D, G><<<dim3(splits, a.n_pos, a.batch * a.Hkv), kRowsThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_combine(a, splits, st);
}

template <typename T, int D>
static hipError_t launch_rows_td(const AttendArgs& a, int splits, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_rows_tdg<T, D, 1>(a, splits, st);
    case 2: return launch_rows_tdg<T, D, 2>(a, splits, st);
    case 4: return launch_rows_tdg<T, D, 4>(a, splits, st);
    case 8: return launch_rows_tdg<T, D, 8>(a, splits, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attend_rows(const AttendArgs& a, int splits, hipStream_t st) {
  if (a.n_pos <= 0) return hipSuccess;
  if (a.bf16)
    return a.d == 128 ? launch_rows_td<bf16_t, 128>(a, splits, st)
                      : launch_rows_td<bf16_t, 64>(a, splits, st);
  return a.d == 128 ? launch_rows_td<float, 128>(a, splits, st)
                    : launch_rows_td<float, 64>(a, splits, st);
}

}  // namespace infllm
