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
// S[b][h][j][c] = sum over rows of block j (clipped to n_ctx) and over the
// group's query heads of q[.][c], fp64.  With NSUB = 4 (blocks of 128 rows)
// the sums of the block's four 32-row sub-blocks are stored too
// (S32[b][h][j][s][c]) and S[j] is their sum in order.  Blocks jb0 ..
// jb0 + n_blocks - 1 are summed, stored at local index j - jb0.  grid
// (n_blocks, H_kv, batch), 256 threads: thread -> (8-column group, row
// phase); each thread requests 8 rows of a head at a time before adding any.
constexpr int kSumThreads = 256;
template <typename T, int NSUB>
__global__ __launch_bounds__(kSumThreads) void k_block_sums(const T* __restrict__ q, int64_t q_cap,
                                                            int Hq, int Hkv, int d, int B,
                                                            int64_t n_ctx, int64_t jb0,
                                                            int n_blocks, double* __restrict__ S,
                                                            double* __restrict__ S32) {
  const int jl = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int64_t j = jb0 + jl;
  const int G = Hq / Hkv;
  const int cgs = d / 8, cg = threadIdx.x % cgs, ph = threadIdx.x / cgs, nph = kSumThreads / cgs;
  const int64_t r0 = (int64_t)j * B;
  const int64_t r1 = r0 + B < n_ctx ? r0 + B : n_ctx;
  const int sub_rows = B / NSUB;
  double acc[NSUB][8];
#pragma unroll
  for (int s2 = 0; s2 < NSUB; ++s2)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[s2][i] = 0.0;
  // two query heads per batch of loads (16 rows of 16 bytes per thread in
  // flight); a head past G re-reads the last one and is not added
  for (int g0 = 0; g0 < G; g0 += 2) {
    const T* qh0 = q + ((int64_t)bi * Hq + (int64_t)h * G + g0) * q_cap * d + cg * 8;
    const T* qh1 = g0 + 1 < G ? qh0 + q_cap * d : qh0;
    for (int64_t rb = r0 + ph; rb < r1; rb += 8 * nph) {
      Raw8<T> raw[2][8];
#pragma unroll
      for (int y = 0; y < 8; ++y) {
        const int64_t r = rb + (int64_t)y * nph;
        raw[0][y].load(qh0 + (r < r1 ? r : r1 - 1) * d);
        raw[1][y].load(qh1 + (r < r1 ? r : r1 - 1) * d);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if (g0 + hh >= G) break;
#pragma unroll
        for (int y = 0; y < 8; ++y) {
          const int64_t r = rb + (int64_t)y * nph;
          if (r >= r1) break;
          const int sb = NSUB == 1 ? 0 : (int)((r - r0) / sub_rows);
#pragma unroll
          for (int s2 = 0; s2 < NSUB; ++s2)
            if (s2 == sb) raw[hh][y].add(acc[s2]);
        }
      }
    }
  }
  __shared__ double part[kSumThreads / 8][128];   // [phase][column]
  double blk = 0.0;
#pragma unroll
  for (int s2 = 0; s2 < NSUB; ++s2) {
    if (s2 > 0) __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) part[ph][cg * 8 + i] = acc[s2][i];
    __syncthreads();
    if (threadIdx.x < d) {
      double t = 0.0;
      for (int p2 = 0; p2 < nph; ++p2) t += part[p2][threadIdx.x];
      if (NSUB > 1) S32[((((int64_t)bi * Hkv + h) * n_blocks + jl) * NSUB + s2) * d + threadIdx.x] = t;
      blk += t;
    }
  }
  if (threadIdx.x < d) S[(((int64_t)bi * Hkv + h) * n_blocks + jl) * d + threadIdx.x] = blk;
}

// BP[b][h][j][c] = sum_{j' < j} S[b][h][j'][c] for j = 0..n_blocks.
// grid (H_kv, batch), d threads.
__global__ void k_block_prefix(const double* __restrict__ S, double* __restrict__ BP, int Hkv,
                               int d, int n_blocks) {
  const int h = blockIdx.x, bi = blockIdx.y, c = threadIdx.x;
  const double* s = S + ((int64_t)bi * Hkv + h) * n_blocks * d;
  double* bp = BP + ((int64_t)bi * Hkv + h) * (n_blocks + 1) * d;
  // batches of kPrefixBatch block sums, the next batch requested before the
  // current one is added (a dependent chain of one add per block)
  constexpr int kPrefixBatch = 16;
  double acc = 0.0;
  double v[kPrefixBatch], w[kPrefixBatch];
  auto load = [&](double* x, int j0) {
#pragma unroll
    for (int t = 0; t < kPrefixBatch; ++t) {
      const int j = j0 + t < n_blocks ? j0 + t : n_blocks - 1;
      x[t] = s[(int64_t)j * d + c];
    }
  };
  auto add = [&](const double* x, int j0) {
#pragma unroll
    for (int t = 0; t < kPrefixBatch; ++t) {
      if (j0 + t >= n_blocks) break;
      bp[(int64_t)(j0 + t) * d + c] = acc;
      acc += x[t];
    }
  };
  if (n_blocks > 0) load(v, 0);
  for (int j = 0; j < n_blocks; j += 2 * kPrefixBatch) {
    if (j + kPrefixBatch < n_blocks) load(w, j + kPrefixBatch);
    add(v, j);
    if (j + kPrefixBatch >= n_blocks) break;
    if (j + 2 * kPrefixBatch < n_blocks) load(v, j + 2 * kPrefixBatch);
    add(w, j + kPrefixBatch);
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
constexpr int kPass2Batch = 8;

template <typename T, int HPL>
__global__ __launch_bounds__(64 * kRepWaves) void k_rep_select(
    const T* __restrict__ q, int64_t q_cap, const T* __restrict__ k, int64_t kv_cap, int Hq,
    int Hkv, int d, int B, int n_init, int W, int r_k, int64_t n_ctx, int u_begin, int u_stride,
    int64_t jb0, int n_blocks, const double* __restrict__ BP, const double* __restrict__ S32,
    int32_t* __restrict__ rep_idx, float* __restrict__ unit_repr) {
  const int u = u_begin + (int)blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
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

  // Without pass 1: for a 128-key unit aligned to its block, with W a
  // multiple of 32 and 32-row sub-block sums at hand, every wave's keys
  // start at a 32-row boundary, so the sums before them are block prefixes
  // plus sub-block sums: F(32x - 1) = BP[x / 4] + sum_{s < x % 4} S32[x / 4][s].
  const bool sub = S32 != nullptr && nk == B && lo == j * B && B == 4 * 32 && W % 32 == 0;
  auto f_at = [&](int64_t x, double* out) {   // F(32x - 1) (local prefix), slot 0 only
    const int64_t blk = x / 4 - jb0;
    const int s_in = (int)(x % 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = slot == 0 ? bp[blk * d + i] : 0.0;
    if (slot == 0) {
      const double* sp = S32 + ((((int64_t)bi * Hkv + h) * n_blocks + blk) * 4) * d + cg * 8;
      for (int s2 = 0; s2 < s_in; ++s2)
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] += sp[s2 * d + i];
    }
  };
  // pass 1: rows that keys k0..k1-1 add (key lo adds none: its sums are
  // the starting values); rows past the context are loaded clamped and
  // not added
  if (!sub) {
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
    const int64_t be = e_end ? jb0 + n_blocks : e / B;   // absolute block
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fp[i] = slot == 0 ? bp[(j - jb0) * d + i] : 0.0;
      fe[i] = slot == 0 ? bp[(be - jb0) * d + i] : 0.0;
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
  if (!sub) {
    for (int w2 = 0; w2 < wave; ++w2)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        fp[i] += seg[0][w2][lane][i];
        fe[i] += seg[1][w2][lane][i];
      }
  } else if (k0 > 0) {
    // F(lo + k0 - 1) and F(min(lo + k0 - 1 + W, last)); the in-block rows
    // of the starting sums above belong to wave 0 only
    f_at((lo + k0) / 32, fp);
    if (lo + k0 - 1 + W >= last) {
#pragma unroll
      for (int i = 0; i < 8; ++i) fe[i] = slot == 0 ? bp[(int64_t)n_blocks * d + i] : 0.0;   // F(last)
    } else {
      f_at((lo + k0 + W) / 32, fe);
    }
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
  const int64_t out_row = ((int64_t)bi * Hkv + h) * u_stride + u;
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
                            int n_init, int u_begin, int u_stride, float* __restrict__ unit_repr) {
  const int u = u_begin + (int)blockIdx.x, h = blockIdx.y, bi = blockIdx.z, c = threadIdx.x;
  const int64_t lo = unit_first_key(u, B, n_init), hi = (u + n_init / B + 1) * (int64_t)B;
  const T* kb = k + ((int64_t)bi * Hkv + h) * kv_cap * d + c;
  double acc = 0.0;
  for (int64_t p0 = lo; p0 < hi; p0 += 16) {   // 16 rows requested before any is added
    T v[16];
#pragma unroll
    for (int y = 0; y < 16; ++y) v[y] = kb[(p0 + y < hi ? p0 + y : hi - 1) * d];
#pragma unroll
    for (int y = 0; y < 16; ++y)
      if (p0 + y < hi) acc += (double)to_f32(v[y]);
  }
  unit_repr[(((int64_t)bi * Hkv + h) * u_stride + u) * d + c] = (float)(acc / (double)(hi - lo));
}

// Blocks that units u_begin .. u_end-1 read: from the first unit's block to
// ceil(W/B) + 2 blocks past the last one's (its keys' windows), clipped to
// the context.  Sums and prefixes are local to this range: only differences
// of the prefix enter a score.
static void build_blocks(const BuildArgs& a, int64_t* jb0, int64_t* nbl) {
  const int64_t nb = (a.n_ctx + a.B - 1) / a.B;
  if (a.block_qsum) {   // the caller's block sums cover every block of the context
    *jb0 = 0;
    *nbl = nb;
    return;
  }
  const int64_t j0 = a.n_init / a.B;
  *jb0 = a.u_begin + j0;
  int64_t jb1 = (int64_t)(a.u_end - 1) + j0 + (a.W + a.B - 1) / a.B + 2;
  jb1 = jb1 < nb ? jb1 : nb;
  *nbl = jb1 - *jb0;
}

// [block sums S][block prefix BP][32-row sub-block sums S32 (128-row blocks only)]
struct BuildWs {
  size_t s, bp, s32;
};
static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
static BuildWs build_ws_layout(const BuildArgs& a, int64_t nbl) {
  BuildWs w;
  w.s = a.block_qsum ? 0 : round256((size_t)a.batch * a.Hkv * nbl * a.d * sizeof(double));
  w.bp = round256((size_t)a.batch * a.Hkv * (nbl + 1) * a.d * sizeof(double));
  w.s32 = a.B == 128 ? (size_t)a.batch * a.Hkv * nbl * 4 * a.d * sizeof(double) : 0;
  return w;
}
static size_t ws_total(const BuildWs& w) { return w.s + w.bp + w.s32; }

size_t build_workspace_bytes(const BuildArgs& a) {
  if (a.rep_mode != 0 || a.u_end <= a.u_begin) return 0;
  int64_t jb0, nbl;
  build_blocks(a, &jb0, &nbl);
  return ws_total(build_ws_layout(a, nbl));
}

// the build that also writes the block query sums (S in the caller's buffer)
size_t build_qsum_workspace_bytes(const BuildArgs& a) {
  if (a.rep_mode != 0 || a.U < 1) return 0;
  BuildArgs b = a;
  b.block_qsum = reinterpret_cast<double*>(16);   // any non-null: the layout without S
  int64_t jb0, nbl;
  build_blocks(b, &jb0, &nbl);
  return ws_total(build_ws_layout(b, nbl));
}

size_t build_range_workspace_bytes(const BuildArgs& a, int64_t n_units) {
  if (a.rep_mode != 0 || n_units < 1) return 0;
  return ws_total(build_ws_layout(a, n_units + (a.W + a.B - 1) / a.B + 2));
}

template <typename T>
static hipError_t launch_build_t(const BuildArgs& a, hipStream_t st) {
  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const int n_u = a.u_end - a.u_begin;
  if (a.block_qsum && (a.rep_mode != 0 || n_u <= 0)) {
    // block query sums of the whole context, for chunk scores; MEAN builds
    // need nothing else from the queries
    const int64_t nb_all = (a.n_ctx + a.B - 1) / a.B;
    k_block_sums<T, 1><<<dim3((unsigned)nb_all, a.Hkv, a.batch), kSumThreads, 0, st>>>(
        q, a.q_cap, a.Hq, a.Hkv, a.d, a.B, a.n_ctx, 0, (int)nb_all, a.block_qsum, nullptr);
    if (n_u <= 0) return hipGetLastError();
  }
  if (n_u <= 0) return hipSuccess;
  if (a.rep_mode != 0) {
    k_mean_repr<T><<<dim3(n_u, a.Hkv, a.batch), a.d, 0, st>>>(k, a.kv_cap, a.Hkv, a.d, a.B,
                                                              a.n_init, a.u_begin, a.u_stride,
                                                              a.unit_repr);
    return hipGetLastError();
  }
  int64_t jb0, nbl;
  build_blocks(a, &jb0, &nbl);
  const BuildWs lay = build_ws_layout(a, nbl);
  double* S = a.block_qsum ? a.block_qsum : (double*)a.ws;
  double* BP = (double*)((char*)a.ws + lay.s);
  double* S32 = lay.s32 > 0 ? (double*)((char*)a.ws + lay.s + lay.bp) : nullptr;
  const int nb = (int)nbl;
  const dim3 sgrid(nb, a.Hkv, a.batch);
  if (S32)
    k_block_sums<T, 4><<<sgrid, kSumThreads, 0, st>>>(q, a.q_cap, a.Hq, a.Hkv, a.d, a.B, a.n_ctx,
                                                      jb0, nb, S, S32);
  else
    k_block_sums<T, 1><<<sgrid, kSumThreads, 0, st>>>(q, a.q_cap, a.Hq, a.Hkv, a.d, a.B, a.n_ctx,
                                                      jb0, nb, S, nullptr);
  k_block_prefix<<<dim3(a.Hkv, a.batch), a.d, 0, st>>>(S, BP, a.Hkv, a.d, nb);
  // heads per lane: 64 / (d / 8) head slots per wave
  const int hs = 64 / (a.d / 8), G = a.Hq / a.Hkv;
  const dim3 grid(n_u, a.Hkv, a.batch);
  if (G <= hs)
    k_rep_select<T, 1><<<grid, 64 * kRepWaves, 0, st>>>(
        q, a.q_cap, k, a.kv_cap, a.Hq, a.Hkv, a.d, a.B, a.n_init, a.W, a.r_k, a.n_ctx, a.u_begin,
        a.u_stride, jb0, nb, BP, S32, a.rep_idx, a.unit_repr);
  else if (G <= 2 * hs)
    k_rep_select<T, 2><<<grid, 64 * kRepWaves, 0, st>>>(
        q, a.q_cap, k, a.kv_cap, a.Hq, a.Hkv, a.d, a.B, a.n_init, a.W, a.r_k, a.n_ctx, a.u_begin,
        a.u_stride, jb0, nb, BP, S32, a.rep_idx, a.unit_repr);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_build(const BuildArgs& a, hipStream_t st) {
  return a.bf16 ? launch_build_t<bf16_t>(a, st) : launch_build_t<float>(a, st);
}

}  // namespace infllm
