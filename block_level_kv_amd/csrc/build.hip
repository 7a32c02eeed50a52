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

// S[b][h][j][c] = sum over rows of block j (clipped to n_ctx) and over the
// group's query heads of q[.][c], fp64.  grid (n_blocks, H_kv, batch), 256 thr.
template <typename T>
__global__ __launch_bounds__(256) void k_block_sums(const T* __restrict__ q, int64_t q_cap, int Hq,
                                                    int Hkv, int d, int B, int64_t n_ctx,
                                                    int n_blocks, double* __restrict__ S) {
  const int j = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int G = Hq / Hkv;
  const int c = threadIdx.x % d, phase = threadIdx.x / d, nph = blockDim.x / d;
  const int64_t r0 = (int64_t)j * B;
  const int64_t r1 = r0 + B < n_ctx ? r0 + B : n_ctx;
  double acc = 0.0;
  for (int g = 0; g < G; ++g) {
    const T* qh = q + ((int64_t)bi * Hq + (int64_t)h * G + g) * q_cap * d;
    for (int64_t r = r0 + phase; r < r1; r += nph) acc += (double)to_f32(qh[r * d + c]);
  }
  __shared__ double part[256];
  part[threadIdx.x] = acc;
  __syncthreads();
  if (phase == 0) {
    for (int p = 1; p < nph; ++p) acc += part[p * d + c];
    S[(((int64_t)bi * Hkv + h) * n_blocks + j) * d + c] = acc;
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

// One workgroup per (unit, KV head, sequence); thread c owns column c.
// Scores every key of the unit in fp64, keeps the r_k best (score desc,
// position asc), writes them ascending and sums their keys.
constexpr int kRepRows = 16;  // positions reduced per LDS pass
constexpr int kMaxBlock = 1024;

template <typename T>
__global__ __launch_bounds__(128) void k_rep_select(
    const T* __restrict__ q, int64_t q_cap, const T* __restrict__ k, int64_t kv_cap, int Hq,
    int Hkv, int d, int B, int n_init, int W, int r_k, int64_t n_ctx, int U, int n_blocks,
    const double* __restrict__ BP, int32_t* __restrict__ rep_idx, float* __restrict__ unit_repr) {
  const int u = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int G = Hq / Hkv;
  const int c = threadIdx.x;  // blockDim.x == d
  const int64_t j = u + n_init / B;
  const int64_t lo = unit_first_key(u, B, n_init), hi = (j + 1) * B;
  const int nk = (int)(hi - lo);

  __shared__ double contrib[kRepRows][128];
  __shared__ double score[kMaxBlock];
  __shared__ int picked[kMaxBlock];

  const T* qb = q + ((int64_t)bi * Hq + (int64_t)h * G) * q_cap * d + c;
  const T* kb = k + ((int64_t)bi * Hkv + h) * kv_cap * d + c;
  const double* bp = BP + ((int64_t)bi * Hkv + h) * (n_blocks + 1) * d + c;
  auto qg = [&](int64_t i) -> double {  // group-summed query, column c
    double s = 0.0;
    for (int g = 0; g < G; ++g) s += (double)to_f32(qb[(int64_t)g * q_cap * d + i * d]);
    return s;
  };

  // F(lo) and F(e_lo) from the block prefix plus the in-block rows
  double Fp = bp[j * d];
  for (int64_t i = j * B; i <= lo; ++i) Fp += qg(i);
  int64_t e = lo + W < n_ctx - 1 ? lo + W : n_ctx - 1;
  const int64_t be = e / B;
  double Fe = bp[be * d];
  for (int64_t i = be * B; i <= e; ++i) Fe += qg(i);

  const int tpr = d / kRepRows;  // threads per row in the reduction
  for (int base = 0; base < nk; base += kRepRows) {
    const int rows = nk - base < kRepRows ? nk - base : kRepRows;
    for (int r = 0; r < rows; ++r) {
      const int64_t p = lo + base + r;
      if (p > lo) {
        Fp += qg(p);
        const int64_t ep = p + W < n_ctx - 1 ? p + W : n_ctx - 1;
        if (ep > e) {
          e = ep;
          Fe += qg(e);
        }
      }
      contrib[r][c] = (double)to_f32(kb[p * d]) * (Fe - Fp);
    }
    __syncthreads();
    {
      const int r = c / tpr, part = c % tpr;
      double s = 0.0;
      for (int cc = part * kRepRows; cc < (part + 1) * kRepRows; ++cc) s += contrib[r][cc];
      for (int m = 1; m < tpr; m <<= 1) s += shfl_xor_f64(s, m);
      if (part == 0 && r < rows) score[base + r] = s;
    }
    __syncthreads();
  }

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
  for (int a = c; a < nk; a += blockDim.x) {
    if (picked[a]) {
      int slot = 0;
      for (int b2 = 0; b2 < a; ++b2) slot += picked[b2];
      ri[slot] = (int32_t)(lo + a);
    }
  }
  for (int s = nk + c; s < r_k; s += blockDim.x) ri[s] = -1;  // fewer keys than r_k
  double acc = 0.0;
  for (int a = 0; a < nk; ++a)
    if (picked[a]) acc += (double)to_f32(kb[(lo + a) * d]);
  unit_repr[out_row * d + c] = (float)acc;
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
  k_block_sums<T><<<dim3(nb, a.Hkv, a.batch), 256, 0, st>>>(q, a.q_cap, a.Hq, a.Hkv, a.d, a.B,
                                                            a.n_ctx, nb, S);
  k_block_prefix<<<dim3(a.Hkv, a.batch), a.d, 0, st>>>(S, BP, a.Hkv, a.d, nb);
  k_rep_select<T><<<dim3(a.U, a.Hkv, a.batch), a.d, 0, st>>>(
      q, a.q_cap, k, a.kv_cap, a.Hq, a.Hkv, a.d, a.B, a.n_init, a.W, a.r_k, a.n_ctx, a.U, nb, BP,
      a.rep_idx, a.unit_repr);
  return hipGetLastError();
}

hipError_t launch_build(const BuildArgs& a, hipStream_t st) {
  return a.bf16 ? launch_build_t<bf16_t>(a, st) : launch_build_t<float>(a, st);
}

}  // namespace infllm
