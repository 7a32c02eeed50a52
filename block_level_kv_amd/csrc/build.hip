// Unit build: representative-token selection and unit representations.
//
// Representative tokens (InfLLM summary page, "Approach"; authors' rebuttal,
// "Representative Tokens"): key p of KV head h earns
//     s_p = k_p . w_p,   w_p = sum_{g in group(h)} sum_{i=p+1}^{e_p} q_i^(g),
//     e_p = min(p + W, n_ctx - 1),
// and each unit keeps its r_k best keys.  With F the inclusive prefix sum of
// the group-summed queries, w_p = F(e_p) - F(p).  The kernels below get F at
// block starts from per-block sums (one streaming pass over Q), then walk
// the 128 positions of a unit keeping F(p) and F(e_p) as running fp64 sums,
// so the whole build reads Q about three times instead of W/B times.
#include "common.h"
#include "kernels.h"

namespace infllm {

// Eight consecutive columns of a row, widened to fp64 and added to acc.
template <typename T> struct Cols8;
template <> struct Cols8<bf16_t> {
  static __device__ __forceinline__ void add(const bf16_t* p, double* acc) {
    const u32x4 w = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += (double)__uint_as_float(w[i] << 16);
      acc[2 * i + 1] += (double)__uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void get(const bf16_t* p, double* v) {
    const u32x4 w = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (double)__uint_as_float(w[i] << 16);
      v[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Cols8<float> {
  static __device__ __forceinline__ void add(const float* p, double* acc) {
    const float4 x = ((const float4*)p)[0], y = ((const float4*)p)[1];
    acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
    acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
  }
  static __device__ __forceinline__ void get(const float* p, double* v) {
    const float4 x = ((const float4*)p)[0], y = ((const float4*)p)[1];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  }
};

// Raw 8-column piece of a row: loaded first, widened later, so that a batch
// of loads is in flight before any of them is waited on.
// S[b][h][j][c] = sum over rows of block j (clipped to n_ctx) and over the
// group's query heads of q[.][c], fp64.  grid (n_blocks, H_kv, batch), 256
// threads: thread -> (8-column group, row phase), 16-byte loads.
constexpr int kSumThreads = 256;
template <typename T>
__global__ __launch_bounds__(kSumThreads) void k_block_sums(const T* __restrict__ q, int64_t q_cap,
                                                            int Hq, int Hkv, int d, int B,
                                                            int64_t n_ctx, int n_blocks,
                                                            double* __restrict__ S) {
  const int j = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int G = Hq / Hkv;
  const int cgs = d / 8, cg = threadIdx.x % cgs, ph = threadIdx.x / cgs, nph = kSumThreads / cgs;
  const int64_t r0 = (int64_t)j * B;
  const int64_t r1 = r0 + B < n_ctx ? r0 + B : n_ctx;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int g = 0; g < G; ++g) {
    const T* qh = q + ((int64_t)bi * Hq + (int64_t)h * G + g) * q_cap * d + cg * 8;
    for (int64_t r = r0 + ph; r < r1; r += nph) Cols8<T>::add(qh + r * d, acc);
  }
  __shared__ double part[kSumThreads / 8][128];   // [phase][column]
#pragma unroll
  for (int i = 0; i < 8; ++i) part[ph][cg * 8 + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < d) {
    double t = 0.0;
    for (int p2 = 0; p2 < nph; ++p2) t += part[p2][threadIdx.x];
    S[(((int64_t)bi * Hkv + h) * n_blocks + j) * d + threadIdx.x] = t;
  }
}

// BP[b][h][j][c] = sum_{j' < j} S[b][h][j'][c] for j = 0..n_blocks.
// grid (H_kv, batch), d threads.
__global__ void k_block_prefix(const double* __restrict__ S, double* __restrict__ BP, int Hkv,
                               int d, int n_blocks) {
  const int h = blockIdx.x, bi = blockIdx.y, c = threadIdx.x;
  const double* s = S + ((int64_t)bi * Hkv + h) * n_blocks * d;
  double* bp = BP + ((int64_t)bi * Hkv + h) * (n_blocks + 1) * d;
  double acc = 0.0;
  int j = 0;
  for (; j + 8 <= n_blocks; j += 8) {
    double v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = s[(int64_t)(j + t) * d + c];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bp[(int64_t)(j + t) * d + c] = acc;
      acc += v[t];
    }
  }
  for (; j < n_blocks; ++j) {
    bp[(int64_t)j * d + c] = acc;
    acc += s[(int64_t)j * d + c];
  }
  bp[(int64_t)n_blocks * d + c] = acc;
}

// One workgroup per (unit, KV head, sequence), four waves.  Wave w scores
// the w-th quarter of the unit's keys; its lanes are (8-column group,
// query-head slot) pairs, a lane summing HPL heads: g = slot + hs * i.
// With F the inclusive prefix of the group-summed queries, key p needs
// F(p) and F(e_p); both advance by one row per key (e_p only while p + W
// stays inside the context).  Pass 1: each wave sums the rows its keys add
// to F(p) and to F(e_p); a prefix over the waves gives each wave its
// starting sums.  Pass 2: each wave walks its keys, and s_p = k_p . (F(e_p)
// - F(p)) is one fp64 reduction over the wave.  Both passes load a batch of
// rows before using any.  Then the r_k best keys are kept (score desc,
// position asc), written ascending, and summed.
constexpr int kMaxBlock = 1024;
constexpr int kRepWaves = 4;
constexpr int kPass1Batch = 8;
constexpr int kPass2Batch = 4;

template <typename T, int HPL>
__global__ __launch_bounds__(64 * kRepWaves) void k_rep_select(
    const T* __restrict__ q, int64_t q_cap, const T* __restrict__ k, int64_t kv_cap, int Hq,
    int Hkv, int d, int B, int n_init, int W, int r_k, int64_t n_ctx, int U, int n_blocks,
    const double* __restrict__ BP, int32_t* __restrict__ rep_idx, float* __restrict__ unit_repr) {
  const int u = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int c = tid;   // column owner in the final phases (c < d)
  const int64_t j = u + n_init / B;
  const int64_t lo = unit_first_key(u, B, n_init), hi = (j + 1) * B;
  const int nk = (int)(hi - lo);
  const int cgs = d / 8, cg = lane % cgs, slot = lane / cgs, hs = 64 / cgs;

  __shared__ double seg[2][kRepWaves][64][8];   // per wave: rows added to F(p), to F(e_p)
  __shared__ double score[kMaxBlock];
  __shared__ int picked[kMaxBlock];

  // this lane's heads (a head past the group repeats head 0 with weight 0)
  const T* qh[HPL];
  bool hv[HPL];
#pragma unroll
  for (int x = 0; x < HPL; ++x) {
    const int g = slot + hs * x;
    hv[x] = g < G;
    qh[x] = q + ((int64_t)bi * Hq + (int64_t)h * G + (hv[x] ? g : 0)) * q_cap * d + cg * 8;
  }
  const T* kb = k + ((int64_t)bi * Hkv + h) * kv_cap * d;
  const double* bp = BP + ((int64_t)bi * Hkv + h) * (n_blocks + 1) * d + cg * 8;
  const int64_t last = n_ctx - 1;
  // this wave's keys: lo + [k0, k1)
  const int per = (nk + kRepWaves - 1) / kRepWaves;
  const int k0 = wave * per < nk ? wave * per : nk;
  const int k1 = k0 + per < nk ? k0 + per : nk;

  // pass 1: rows that keys k0..k1-1 add (key lo adds none: its sums are
  // the starting values); rows past the context are loaded clamped and
  // not added
  {
    double sl[8] = {0, 0, 0, 0, 0, 0, 0, 0}, su[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int o0 = k0 > 0 ? k0 : 1; o0 < k1; o0 += kPass1Batch) {
      Raw8<T> rl[kPass1Batch][HPL], ru[kPass1Batch][HPL];
#pragma unroll
      for (int y = 0; y < kPass1Batch; ++y) {
        const int64_t p = lo + (o0 + y < k1 ? o0 + y : k1 - 1);
        const int64_t pe = p + W < last ? p + W : last;
#pragma unroll
        for (int x = 0; x < HPL; ++x) {
          rl[y][x].load(qh[x] + p * d);
          ru[y][x].load(qh[x] + pe * d);
        }
      }
#pragma unroll
      for (int y = 0; y < kPass1Batch; ++y) {
        const int64_t p = lo + o0 + y;
        if (o0 + y >= k1) break;
#pragma unroll
        for (int x = 0; x < HPL; ++x) {
          if (!hv[x]) continue;
          rl[y][x].add(sl);
          if (p + W <= last) ru[y][x].add(su);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      seg[0][wave][lane][i] = sl[i];
      seg[1][wave][lane][i] = su[i];
    }
  }
  // starting sums F(lo), F(e_lo): block prefix + the in-block rows (the
  // block prefix holds every head of the group: only slot 0 takes it).
  // F(n_ctx - 1) is the prefix past the last block.  In-block rows are
  // added in batches whose loads are all in flight together.
  double fp[8], fe[8];
  {
    const int64_t e = lo + W < last ? lo + W : last;
    const bool e_end = e == last;
    const int64_t be = e_end ? n_blocks : e / B;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fp[i] = slot == 0 ? bp[j * d + i] : 0.0;
      fe[i] = slot == 0 ? bp[be * d + i] : 0.0;
    }
    auto add_rows = [&](int64_t r0, int64_t r1, double* acc) {   // rows r0 .. r1
      for (int64_t i0 = r0; i0 <= r1; i0 += kPass1Batch) {
        Raw8<T> r[kPass1Batch][HPL];
#pragma unroll
        for (int y = 0; y < kPass1Batch; ++y)
#pragma unroll
          for (int x = 0; x < HPL; ++x) r[y][x].load(qh[x] + (i0 + y <= r1 ? i0 + y : r1) * d);
#pragma unroll
        for (int y = 0; y < kPass1Batch; ++y)
#pragma unroll
          for (int x = 0; x < HPL; ++x)
            if (hv[x] && i0 + y <= r1) r[y][x].add(acc);
      }
    };
    add_rows(j * B, lo, fp);
    if (!e_end) add_rows(be * B, e, fe);
  }
  __syncthreads();
  for (int w2 = 0; w2 < wave; ++w2)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fp[i] += seg[0][w2][lane][i];
      fe[i] += seg[1][w2][lane][i];
    }
  // pass 2: walk the keys; a batch's rows are loaded first, and its
  // reductions overlap
  for (int o0 = k0; o0 < k1; o0 += kPass2Batch) {
    Raw8<T> rl[kPass2Batch][HPL], ru[kPass2Batch][HPL], rk[kPass2Batch];
#pragma unroll
    for (int y = 0; y < kPass2Batch; ++y) {
      const int64_t p = lo + (o0 + y < k1 ? o0 + y : k1 - 1);
      const int64_t pe = p + W < last ? p + W : last;
#pragma unroll
      for (int x = 0; x < HPL; ++x) {
        rl[y][x].load(qh[x] + p * d);
        ru[y][x].load(qh[x] + pe * d);
      }
      rk[y].load(kb + p * d + cg * 8);
    }
    double t[kPass2Batch];
#pragma unroll
    for (int y = 0; y < kPass2Batch; ++y) {
      const int o = o0 + y;
      const int64_t p = lo + o;
      t[y] = 0.0;
      if (o >= k1) continue;
      if (o > 0) {
#pragma unroll
        for (int x = 0; x < HPL; ++x) {
          if (!hv[x]) continue;
          rl[y][x].add(fp);
          if (p + W <= last) ru[y][x].add(fe);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) t[y] = fma(rk[y].get(i), fe[i] - fp[i], t[y]);
    }
#pragma unroll
    for (int y = 0; y < kPass2Batch; ++y) {
      const double tt = wave_sum_f64_dpp(t[y]);
      if (lane == 0 && o0 + y < k1) score[o0 + y] = tt;
    }
  }
  __syncthreads();

  // rank each key: #keys ahead of it in (score desc, position asc)
  for (int a = c; a < nk; a += blockDim.x) {
    const double sa = score[a];
    int rank = 0;
    for (int b2 = 0; b2 < nk; ++b2) {
      const double sb = score[b2];
      rank += (sb > sa) || (sb == sa && b2 < a);
    }
    picked[a] = rank < r_k;
  }
  __syncthreads();
  const int64_t out_row = ((int64_t)bi * Hkv + h) * U + u;
  int32_t* ri = rep_idx + out_row * r_k;
  __shared__ int chosen[kMaxBlock];     // kept key offsets, ascending
  for (int a = c; a < nk; a += blockDim.x) {
    if (picked[a]) {
      int at = 0;
      for (int b2 = 0; b2 < a; ++b2) at += picked[b2];
      ri[at] = (int32_t)(lo + a);
      chosen[at] = a;
    }
  }
  for (int s = nk + c; s < r_k; s += blockDim.x) ri[s] = -1;  // fewer keys than r_k
  __syncthreads();
  // the representation: kept keys summed in ascending position, their rows
  // requested together
  const int n_kept = nk < r_k ? nk : r_k;
  if (c < d) {
    double acc = 0.0;
    for (int a0 = 0; a0 < n_kept; a0 += 8) {
      float v[8];
#pragma unroll
      for (int y = 0; y < 8; ++y)
        v[y] = to_f32(kb[(lo + chosen[a0 + y < n_kept ? a0 + y : n_kept - 1]) * d + c]);
#pragma unroll
      for (int y = 0; y < 8; ++y)
        if (a0 + y < n_kept) acc += (double)v[y];
    }
    unit_repr[out_row * d + c] = (float)acc;
  }
}

// Mean-of-keys representation (summary page, "Measured effects": mean key-
// vector representations).  grid (U, H_kv, batch), d threads.
template <typename T>
__global__ void k_mean_repr(const T* __restrict__ k, int64_t kv_cap, int Hkv, int d, int B,
                            int n_init, int U, float* __restrict__ unit_repr) {
  const int u = blockIdx.x, h = blockIdx.y, bi = blockIdx.z, c = threadIdx.x;
  const int64_t lo = unit_first_key(u, B, n_init), hi = (u + n_init / B + 1) * (int64_t)B;
  const T* kb = k + ((int64_t)bi * Hkv + h) * kv_cap * d + c;
  double acc = 0.0;
  for (int64_t p = lo; p < hi; ++p) acc += (double)to_f32(kb[p * d]);
  unit_repr[(((int64_t)bi * Hkv + h) * U + u) * d + c] = (float)(acc / (double)(hi - lo));
}

size_t build_workspace_bytes(const BuildArgs& a) {
  if (a.rep_mode != 0) return 0;
  const int64_t nb = (a.n_ctx + a.B - 1) / a.B;
  const size_t s = (size_t)a.batch * a.Hkv * nb * a.d * sizeof(double);
  const size_t bp = (size_t)a.batch * a.Hkv * (nb + 1) * a.d * sizeof(double);
  return ((s + 255) & ~(size_t)255) + bp;
}

template <typename T>
static hipError_t launch_build_t(const BuildArgs& a, hipStream_t st) {
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  if (a.U <= 0) return hipSuccess;
  if (a.rep_mode != 0) {
    k_mean_repr<T><<<dim3(a.U, a.Hkv, a.batch), a.d, 0, st>>>(k, a.kv_cap, a.Hkv, a.d, a.B,
                                                              a.n_init, a.U, a.unit_repr);
    return hipGetLastError();
  }
  const int nb = (int)((a.n_ctx + a.B - 1) / a.B);
  double* S = (double*)a.ws;
  const size_t s_bytes = (size_t)a.batch * a.Hkv * nb * a.d * sizeof(double);
  double* BP = (double*)((char*)a.ws + ((s_bytes + 255) & ~(size_t)255));
  k_block_sums<T><<<dim3(nb, a.Hkv, a.batch), kSumThreads, 0, st>>>(q, a.q_cap, a.Hq, a.Hkv, a.d, a.B,
                                                            a.n_ctx, nb, S);
  k_block_prefix<<<dim3(a.Hkv, a.batch), a.d, 0, st>>>(S, BP, a.Hkv, a.d, nb);
  // heads per lane: 64 / (d / 8) head slots per wave
  const int hs = 64 / (a.d / 8), G = a.Hq / a.Hkv;
  const dim3 grid(a.U, a.Hkv, a.batch);
  if (G <= hs)
    k_rep_select<T, 1><<<grid, 64 * kRepWaves, 0, st>>>(
        q, a.q_cap, k, a.kv_cap, a.Hq, a.Hkv, a.d, a.B, a.n_init, a.W, a.r_k, a.n_ctx, a.U, nb,
        BP, a.rep_idx, a.unit_repr);
  else if (G <= 2 * hs)
    k_rep_select<T, 2><<<grid, 64 * kRepWaves, 0, st>>>(
        q, a.q_cap, k, a.kv_cap, a.Hq, a.Hkv, a.d, a.B, a.n_init, a.W, a.r_k, a.n_ctx, a.U, nb,
        BP, a.rep_idx, a.unit_repr);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_build(const BuildArgs& a, hipStream_t st) {
  return a.bf16 ? launch_build_t<bf16_t>(a, st) : launch_build_t<float>(a, st);
}

}  // namespace infllm
