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
// so no per-key mask is needed.  The work is split over gridDim.x workgroups
// (split-K): each takes an equal share of the local keys (initial tokens and
// window, known from t alone, so its first loads go out before the
// selection is read) and an equal share of the units' keys.  Within a
// workgroup 16 lanes share a key (each holds D/16 columns: one coalesced
// 16-byte load per lane for bf16, D = 128); the 16 key lanes run independent
// online softmaxes merged through LDS, and the next group of keys is loaded
// while the current one is reduced.  Splits publish partial (max, sum, unnormalised output)
// rows; the last one to arrive merges them in split order (see common.h for
// the publication protocol), so one launch produces the output.
#include <stdlib.h>

#include "common.h"
#include "kernels.h"
#include "score_units.h"

namespace infllm {

constexpr int kRowsThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T, int CPT> struct RowRaw;   // CPT columns of one row, raw bits
template <> struct RowRaw<bf16_t, 8> {
  u32x4 w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *(const u32x4*)p; }
  __device__ __forceinline__ void to_f32(float* o) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct RowRaw<bf16_t, 4> {
  uint2 w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *(const uint2*)p; }
  __device__ __forceinline__ void to_f32(float* o) const {
    o[0] = __uint_as_float(w.x << 16);
    o[1] = __uint_as_float(w.x & 0xffff0000u);
    o[2] = __uint_as_float(w.y << 16);
    o[3] = __uint_as_float(w.y & 0xffff0000u);
  }
};
template <> struct RowRaw<float, 8> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = ((const float4*)p)[0];
    b = ((const float4*)p)[1];
  }
  __device__ __forceinline__ void to_f32(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};
template <> struct RowRaw<float, 4> {
  float4 a;
  __device__ __forceinline__ void load(const float* p) { a = *(const float4*)p; }
  __device__ __forceinline__ void to_f32(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  }
};

constexpr int kKeysPerIter = 4;  // keys per lane between softmax rescales
constexpr int kMaxSplits = 64;

// The work of one workgroup: split `split` of the n_splits splits of one
// (position, KV head, sequence) row.  It attends share l_part of the local
// keys cut into l_parts equal shares and share u_part of the units' keys
// cut into u_parts (0 parts: none of them).  `ready` (fused decode step,
// every split of the row): the row's selection is written in this launch --
// splits with unit keys wait until ready[row] is set and read it with
// device-scope loads, and the split that merges the row clears the flag.
struct RowsJob {
  int split, n_splits, pos, h, bi;
  int l_part, l_parts, u_part, u_parts;
  const int* ready;
};

// bounded wait for a selection made in the same launch (polls of a few
// hundred ns each; the selection takes microseconds)
constexpr int kSpinLimit = 1 << 18;

template <typename T, int D, int G>
__device__ __forceinline__ void attend_rows_body(const AttendArgs& a, const RowsJob& job) {
  constexpr int CPT = D / 16;
  const int split = job.split, pos = job.pos, h = job.h, bi = job.bi;
  const int tid = threadIdx.x, lane = tid % 64, seg = tid % 16, kl = tid / 16;
  const int ch = pos / a.L;
  const int64_t base = seq_base(a.pos, a.q_pos, bi);
  if (a.pos && !seq_pos_ok(base, a.n_pos, a.kv_cap)) {
    // a sequence whose position does not fit its KV buffer: every split
    // leaves before any key load or arrival count, split 0 writes NaN rows
    if (split == 0)
      nan_rows<T>((T*)a.out, a.lse, (int64_t)bi * a.Hq + (int64_t)h * G, G, a.out_cap,
                  a.out_off + pos, 1, D, tid, kRowsThreads);
    return;
  }
  const int64_t t = base + pos;

  __shared__ int64_t iv_lo[kMaxTopK];               // first key position of unit m
  __shared__ int64_t iv_first[kMaxTopK + 1];        // first unit-key index of unit m
  __shared__ int wave_tot[kRowsThreads / 64];
  __shared__ int last_sh;

  // query rows first: their loads overlap the interval scan below
  RowRaw<T, CPT> qraw[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qraw[g].load((const T*)a.q +
                 (((int64_t)bi * a.Hq + (int64_t)h * G + g) * a.q_cap + a.q_off + pos) * D +
                 seg * CPT);

  // ---------------------------------------------------------- key sets
  // Local keys (initial tokens, then the window) follow from t alone; the
  // units' keys need the selection.  Every split takes an equal share of
  // each: local keys [l_begin, l_stop) of the local numbering first, then
  // unit keys [u_begin, u_stop) of the units' numbering (sel order, each
  // unit at most B keys).  Its first local keys are requested before the
  // selection is read and the unit table formed.
  const int64_t unit_cap = t - a.W + 1;
  const int64_t init_len = a.n_init < t + 1 ? a.n_init : t + 1;
  const int64_t win_lo = a.n_init > unit_cap ? a.n_init : unit_cap;
  const int64_t win_len = t + 1 - win_lo > 0 ? t + 1 - win_lo : 0;
  const int64_t n_local = init_len + win_len;
  const int64_t pl = job.l_parts > 0 ? (n_local + job.l_parts - 1) / job.l_parts : 0;
  const int64_t l_begin = (int64_t)job.l_part * pl < n_local ? (int64_t)job.l_part * pl : n_local;
  const int64_t l_stop = l_begin + pl < n_local ? l_begin + pl : n_local;
  const int64_t nl = l_stop - l_begin;
  const int64_t pu = job.u_parts > 0 ? ((int64_t)a.k_m * a.B + job.u_parts - 1) / job.u_parts : 0;
  const int64_t u_begin = (int64_t)job.u_part * pu;
  const int64_t row_id = ((int64_t)bi * a.Hkv + h) * a.n_pos + pos;
  __shared__ int ready_sh;
  bool stale = false;                                // the selection never arrived
  if (job.ready && job.u_parts > 0) {
    if (tid == 0) {
      int ok = 0;
      for (int it = 0; it < kSpinLimit && !ok; ++it) {
        ok = __hip_atomic_load(job.ready + row_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!ok) __builtin_amdgcn_s_sleep(2);
      }
      ready_sh = ok;
    }
    __syncthreads();
    stale = !ready_sh;
  }
  int32_t my_unit = -1;                              // sel entry `tid`, requested now
  if (tid < a.k_m && job.u_parts > 0 && !stale) {
    const int32_t* sp = a.sel + (((int64_t)bi * a.Hkv + h) * a.n_chunks + ch) * a.k_m + tid;
    my_unit = job.ready ? __hip_atomic_load(const_cast<int32_t*>(sp), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                        : *sp;
  }

  const T* kb = (const T*)a.k + ((int64_t)bi * a.Hkv + h) * a.kv_cap * D + seg * CPT;
  const T* vb = (const T*)a.v + ((int64_t)bi * a.Hkv + h) * a.kv_cap * D + seg * CPT;
  // split-local key index i -> position: i < nl local keys, then unit keys
  // through the table (each lane's indices only grow, so a cursor works)
  int cur = 0;
  int64_t n_split = nl;                              // + the unit keys, once known
  auto key_pos = [&](int64_t i) -> int64_t {
    if (i < nl) {
      const int64_t x = l_begin + i;
      return x < init_len ? x : win_lo + (x - init_len);
    }
    const int64_t y = u_begin + (i - nl);
    while (y >= iv_first[cur + 1]) ++cur;
    return iv_lo[cur] + (y - iv_first[cur]);
  };
  RowRaw<T, CPT> kn[kKeysPerIter], vn[kKeysPerIter];
  bool okn[kKeysPerIter];
  auto fetch = [&](int64_t base) {
#pragma unroll
    for (int j = 0; j < kKeysPerIter; ++j) {
      const int64_t idx = base + kl + 16 * j;
      okn[j] = idx < n_split;
      const int64_t p = okn[j] ? key_pos(idx) : 0;
      kn[j].load(kb + p * D);
      vn[j].load(vb + p * D);
    }
  };
  // the first group of keys, if local only, is in flight during the table
  const bool early = nl >= 16 * kKeysPerIter;
  if (early) fetch(0);

  // unit table: thread m computes unit m's length, a block scan the offsets
  {
    int64_t lo = 0, len = 0;
    if (my_unit >= 0) {
      lo = unit_first_key(my_unit, a.B, a.n_init);
      const int64_t hi = ((int64_t)my_unit + a.n_init / a.B + 1) * a.B;
      len = (hi < unit_cap ? hi : unit_cap) - lo;
      len = len > 0 ? len : 0;
    }
    // inclusive scan of the unit lengths (each <= B)
    int x = (int)len;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int y = __shfl_up(x, m);
      if (lane >= m) x += y;
    }
    if (lane == 63) wave_tot[tid / 64] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w2 = 0; w2 < kRowsThreads / 64; ++w2) {
      before += w2 < tid / 64 ? wave_tot[w2] : 0;
      all += wave_tot[w2];
    }
    if (tid < a.k_m) {
      iv_lo[tid] = lo;
      iv_first[tid] = before + x - len;
    }
    if (tid == 0) iv_first[a.k_m] = all;
  }
  __syncthreads();
  {
    const int64_t n_unit = iv_first[a.k_m];
    const int64_t u_stop = u_begin + pu < n_unit ? u_begin + pu : n_unit;
    n_split = nl + (u_stop > u_begin ? u_stop - u_begin : 0);
  }

  const float qscale = kLog2e / sqrtf((float)D);
  float qv[G][CPT];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    qraw[g].to_f32(qv[g]);
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

  if (!early) fetch(0);
  for (int64_t base = 0; base < n_split; base += 16 * kKeysPerIter) {
    RowRaw<T, CPT> kc[kKeysPerIter], vc[kKeysPerIter];
    bool ok[kKeysPerIter];
#pragma unroll
    for (int j = 0; j < kKeysPerIter; ++j) {
      kc[j] = kn[j];
      vc[j] = vn[j];
      ok[j] = okn[j];
    }
    if (base + 16 * kKeysPerIter < n_split) fetch(base + 16 * kKeysPerIter);  // in flight
    // logits of the current keys for every head (each key row converted once)
    float s[G][kKeysPerIter];
#pragma unroll
    for (int j = 0; j < kKeysPerIter; ++j) {
      float kf[CPT];
      kc[j].to_f32(kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d0 = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) d0 = fmaf(qv[g][c], kf[c], d0);
        const float r = row16_sum(d0);  // the 16 lanes of a row share key j
        s[g][j] = ok[j] ? r : -INFINITY;
      }
    }
    // online softmax update per head; s becomes the weights p
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int j = 0; j < kKeysPerIter; ++j) mx = fmaxf(mx, s[g][j]);
      const float mu = mx == -INFINITY ? 0.f : mx;   // no valid key yet: weights 0
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mu);
      m[g] = mx;
      float lsum = l[g] * alpha;
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[g][c] *= alpha;
#pragma unroll
      for (int j = 0; j < kKeysPerIter; ++j) {
        s[g][j] = __builtin_amdgcn_exp2f(s[g][j] - mu);
        lsum += s[g][j];
      }
      l[g] = lsum;
    }
#pragma unroll
    for (int j = 0; j < kKeysPerIter; ++j) {
      float vf[CPT];
      vc[j].to_f32(vf);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[g][c] = fmaf(s[g][j], vf[c], acc[g][c]);
    }
  }

  // ---------------------------------------------------------- merge 16 key lanes
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
  constexpr int kOut = (G * D + kRowsThreads - 1) / kRowsThreads;  // outputs per thread
  float Mv[kOut], Lv[kOut], Ov[kOut];
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int o = tid + i * kRowsThreads;
    Mv[i] = -INFINITY;
    Lv[i] = 0.f;
    Ov[i] = 0.f;
    if (o >= G * D) continue;
    const int g = o / D, col = o % D;
    for (int r = 0; r < 16; ++r) Mv[i] = fmaxf(Mv[i], sm_m[r][g]);
    if (Mv[i] != -INFINITY) {
      for (int r = 0; r < 16; ++r) {
        const float w = __builtin_amdgcn_exp2f(sm_m[r][g] - Mv[i]);
        Lv[i] = fmaf(sm_l[r][g], w, Lv[i]);
        Ov[i] = fmaf(sm_o[r][g][col], w, Ov[i]);
      }
    }
  }

  if (stale) {
#pragma unroll
    for (int i = 0; i < kOut; ++i) Mv[i] = Lv[i] = Ov[i] = __builtin_nanf("");
  }

  // ---------------------------------------------------------- split-K merge
  const int splits = job.n_splits;
  const int64_t qh0 = (int64_t)bi * a.Hq + (int64_t)h * G;
  if (splits > 1) {
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      const int o = tid + i * kRowsThreads;
      if (o >= G * D) continue;
      const int g = o / D, col = o % D;
      const int64_t row = ((int64_t)split * a.batch * a.Hq + qh0 + g) * a.n_pos + pos;
      st_dev(a.ws_o + row * D + col, Ov[i]);
      if (col == 0) {
        st_dev(a.ws_ml + 2 * row, Mv[i]);
        st_dev(a.ws_ml + 2 * row + 1, Lv[i]);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
      int* ctr = a.ws_count + row_id;
      const int done = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_sh = done == splits - 1;
      if (last_sh) {
        __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // every split of the row is past its wait: ready for the next call
        if (job.ready) __hip_atomic_store(const_cast<int*>(job.ready) + row_id, 0,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (!last_sh) return;
    // Merge every split's published rows (this one's included).  Each
    // thread's (max, sum) pairs and its output columns' first batch of split
    // values are requested together: one memory round trip when the splits
    // fit a batch.  The (max, sum) table is padded to kMaxSplits with
    // (-inf, 0), so the weight pass and the weighted sums run without
    // per-split branches (padding weights are 0 and padding loads return 0).
    float* sm_w = &sm_o[0][0][0];                  // reuse: [kMaxSplits][G] weights
    float* sm_sl = sm_w + kMaxSplits * G;          // [kMaxSplits][G] sums
    constexpr int kMlPer = (kMaxSplits * G + kRowsThreads - 1) / kRowsThreads;
    constexpr int kBatch = kOut <= 2 ? 32 : (kOut <= 64 ? 64 / kOut : 1);  // splits per batch
    static_assert(kMaxSplits <= 64 && kMaxSplits % kBatch == 0, "one split per lane of wave 0");
    const int64_t stride = (int64_t)a.batch * a.Hq * a.n_pos * D;   // between splits
    float mlm[kMlPer], mll[kMlPer];
#pragma unroll
    for (int j = 0; j < kMlPer; ++j) {
      const int idx = tid + j * kRowsThreads;
      const int s = idx / G, g = idx % G;
      const int64_t row = ((int64_t)s * a.batch * a.Hq + qh0 + g) * a.n_pos + pos;
      mlm[j] = idx < splits * G ? ld_dev(a.ws_ml + 2 * row) : -INFINITY;
      mll[j] = idx < splits * G ? ld_dev(a.ws_ml + 2 * row + 1) : 0.f;
    }
    // Output columns through a buffer resource that ends at the last
    // split: loads of splits beyond it return 0, so a batch is issued
    // without branches (the workspace of a split-K launch stays far below
    // 4 GiB, so byte offsets fit 32 bits).
    const __amdgpu_buffer_rsrc_t ro = dev_rsrc(a.ws_o, (uint32_t)(splits * stride * 4));
    float vb[kOut][kBatch];
    auto load_batch = [&](int s0) {
#pragma unroll
      for (int i = 0; i < kOut; ++i) {
        const int o = tid + i * kRowsThreads;
        const int g = (o < G * D ? o : 0) / D, col = o % D;
        const uint32_t base = (uint32_t)(((qh0 + g) * a.n_pos + pos) * D + col);
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          vb[i][j] = ld1_dev(ro, (base + (uint32_t)((s0 + j) * stride)) * 4u);
      }
    };
    load_batch(0);
#pragma unroll
    for (int j = 0; j < kMlPer; ++j) {
      const int idx = tid + j * kRowsThreads;
      if (idx < kMaxSplits * G) {
        sm_w[idx] = mlm[j];
        sm_sl[idx] = mll[j];
      }
    }
    __syncthreads();
    // wave 0, one split per lane: M = max_s m_s, w_s = 2^(m_s - M),
    // L = sum_s l_s w_s (fixed reduction tree)
    __shared__ float sm_M[G], sm_L[G];
    if (tid < 64) {
      float mv[G], lv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        mv[g] = sm_w[lane * G + g];
        lv[g] = sm_sl[lane * G + g];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float M = wave_max_f32(mv[g]);
        const float w = mv[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[g] - M);
        const float Ls = wave_sum_f32(lv[g] * w);
        sm_w[lane * G + g] = w;
        if (lane == 0) {
          sm_M[g] = M;
          sm_L[g] = Ls;
        }
      }
    }
    __syncthreads();
    float Os[kOut];
#pragma unroll
    for (int i = 0; i < kOut; ++i) Os[i] = 0.f;
    for (int s0 = 0; s0 < splits; s0 += kBatch) {
      if (s0 > 0) load_batch(s0);
#pragma unroll
      for (int i = 0; i < kOut; ++i) {
        const int o = tid + i * kRowsThreads;
        const int g = (o < G * D ? o : 0) / D;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) Os[i] = fmaf(vb[i][j], sm_w[(s0 + j) * G + g], Os[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      const int o = tid + i * kRowsThreads;
      if (o >= G * D) continue;
      const int g = o / D;
      Mv[i] = sm_M[g];
      Lv[i] = sm_L[g];
      Ov[i] = Os[i];
    }
  }
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int o = tid + i * kRowsThreads;
    if (o >= G * D) continue;
    const int g = o / D, col = o % D;
    const int64_t qh = qh0 + g;
    T* out = (T*)a.out + (qh * a.out_cap + a.out_off + pos) * D + col;
    *out = from_f32<T>(Ov[i] / Lv[i]);
    if (a.lse && col == 0) a.lse[qh * a.out_cap + a.out_off + pos] = (Mv[i] + log2f(Lv[i])) * kLn2;
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kRowsThreads) void k_attend_rows(AttendArgs a) {
  const int s = blockIdx.x, n = gridDim.x;
  const RowsJob job{s, n, (int)blockIdx.y, (int)(blockIdx.z % a.Hkv), (int)(blockIdx.z / a.Hkv),
                    s, n, s, n, nullptr};
  attend_rows_body<T, D, G>(a, job);
}

int rows_num_splits(const AttendArgs& a) {
  // enough workgroups to cover the chip several times, >= ~256 keys each
  const int64_t max_keys = (int64_t)a.n_init + (int64_t)a.k_m * a.B + a.W;
  const int64_t wgs = (int64_t)a.n_pos * a.batch * a.Hkv;
  int64_t target = 512;
  if (const char* e = getenv("INFLLM_ROWS_WGS")) {  // tuning override
    const int v = atoi(e);
    if (v >= 1 && v <= 65536) target = v;
  }
  int64_t s = (target + wgs - 1) / wgs;
  const int64_t cap = (max_keys + 255) / 256;
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

int64_t rows_num_counters(const AttendArgs& a) { return (int64_t)a.n_pos * a.batch * a.Hkv; }

template <typename T, int D, int G>
static hipError_t launch_rows_tdg(const AttendArgs& a, int splits, hipStream_t st) {
  k_attend_rows<T, D, G><<<dim3(splits, a.n_pos, a.batch * a.Hkv), kRowsThreads, 0, st>>>(a);
  return hipGetLastError();
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

// ------------------------------------------------------------ fused decode step
// Selection and attention of decode positions in one launch.  A row (one
// position of one KV head of one sequence) has s_unit unit splits and
// s_local local splits.  Unit split i first scores units [64i, 64i + 64)
// of the row (none past the last unit: splits may outnumber the slices)
// and counts itself in; the last to arrive selects the row, publishes the
// selection with device-scope stores and sets the row's ready flag; every
// unit split then waits for the flag and attends its share of the selected
// units' keys.  A waiting split has itself arrived, so the one it waits on
// is already running and never waits: the waits end without any
// assumption on dispatch order (and are bounded all the same: a stale
// selection gives NaN outputs).  Local splits attend their share of the
// initial tokens and the window, which need no selection, meanwhile.  The
// row's merging split clears the flag.
template <typename T, int D, int G, int SEL>
__global__ __launch_bounds__(kRowsThreads) void k_select_attend(ScoreArgs s, AttendArgs a,
                                                                StepPlan p, int* ready) {
  static_assert(kRowsThreads == kScoreThreads, "one workgroup size for both roles");
  __shared__ int32_t sel_sm[kMaxTopK];
  const int tid = threadIdx.x;
  const int n_unit = a.batch * a.Hkv * a.n_pos * p.s_unit;
  const bool unit = (int)blockIdx.x < n_unit;
  const int per = unit ? p.s_unit : p.s_local;
  const int x = unit ? (int)blockIdx.x : (int)blockIdx.x - n_unit;
  // row = (sequence * H_kv + KV head) * positions + position; one chunk per position
  const int row = x / per, part = x % per;
  const int pos = row % a.n_pos, h = row / a.n_pos % a.Hkv, bi = row / a.n_pos / a.Hkv;
  if (unit) {
    if (score_slice<T, G, D, SEL>(part, p.s_unit, pos, h, bi, (const T*)s.q, s.q_cap, s.q_off,
                                  s.q_pos, s.pos, 1, s.Hq, s.Hkv, s.B, s.n_init, s.W, s.repr, s.U,
                                  s.scores, s.n_chunks, nullptr, 0, 0, 0, (int*)s.ws, s.k_m,
                                  sel_sm)) {
      __syncthreads();
      int32_t* dst = s.sel + (int64_t)row * s.k_m;
      for (int m = tid; m < s.k_m; m += kRowsThreads)
        __hip_atomic_store(dst + m, sel_sm[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      // a row whose position does not fit its KV buffer attends nothing
      // (every split leaves before waiting), so its flag stays clear
      const bool valid = !a.pos || seq_pos_ok(seq_base(a.pos, a.q_pos, bi), a.n_pos, a.kv_cap);
      if (tid == 0 && valid)
        __hip_atomic_store(ready + row, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const int n_splits = p.s_local + p.s_unit;
  const RowsJob job = unit ? RowsJob{p.s_local + part, n_splits, pos, h, bi, 0, 0, part,
                                     p.s_unit, ready}
                           : RowsJob{part, n_splits, pos, h, bi, part, p.s_local, 0, 0, ready};
  attend_rows_body<T, D, G>(a, job);
}

// workgroups of k_select_attend resident at once: 3 per CU (its LDS and
// registers allow 3) on the 256 CUs
constexpr int64_t kStepResidentWGs = 3 * 256;

bool select_attend_plan(const ScoreArgs& s, const AttendArgs& a, StepPlan* p) {
  const int64_t rows = (int64_t)a.batch * a.Hkv * a.n_pos;
  const int n_slices = (s.U + kUnitsPerWG - 1) / kUnitsPerWG;
  if (!a.bf16 || a.L != 1 || s.U < 1 || a.k_m < 1 || a.k_m > kMaxTopK || n_slices > kMaxSelSlices)
    return false;
  const int G = a.Hq / a.Hkv;
  if (G > kDirectRows || (G != 1 && G != 2 && G != 4 && G != 8)) return false;
  // about 256 workgroups on each key set, >= ~256 keys each; at least one
  // unit split per scoring slice
  const int64_t each = (256 + rows - 1) / rows;
  int64_t sl = each, su = each;
  if (const char* e = getenv("INFLLM_STEP_LOCAL_SPLITS")) {   // tuning override
    const int v = atoi(e);
    if (v >= 1 && v <= kMaxSplits) sl = v;
  }
  const int64_t cap_l = ((int64_t)a.n_init + a.W + 255) / 256;
  const int64_t cap_u = ((int64_t)a.k_m * a.B + 255) / 256;
  sl = sl < cap_l ? sl : cap_l;
  sl = sl < 1 ? 1 : sl;
  su = su < cap_u ? su : cap_u;
  su = su < kMaxSplits / 2 ? su : kMaxSplits / 2;
  su = su > n_slices ? su : n_slices;
  if (sl + su > kMaxSplits) sl = kMaxSplits - su;
  // the whole launch resident at once where it can be: split counts past
  // that left a last round of local splits to start late (measured at 128K:
  // 8 local splits 40.4 us per step, 10 splits 47.8 us)
  const int64_t fit = kStepResidentWGs / rows - su;
  if (sl > fit) sl = fit;
  if (sl < 1) sl = 1;
  if (sl + su > kMaxSplits) return false;
  if (rows * (su + sl) > (int64_t)1 << 30) return false;
  p->n_slices = n_slices;
  p->s_local = (int)sl;
  p->s_unit = (int)su;
  return true;
}

int64_t select_attend_sync_ints(const AttendArgs& a) {
  return (int64_t)a.batch * a.Hkv * a.n_pos;   // ready flags
}

template <int D, int G>
static hipError_t launch_step_dg(const ScoreArgs& s, const AttendArgs& a, const StepPlan& p,
                                 int* ready, hipStream_t st) {
  const int64_t rows = (int64_t)a.batch * a.Hkv * a.n_pos;
  const dim3 grid((unsigned)(rows * (p.s_local + p.s_unit)));
  // keys per lane of the 4-wave search: ceil(U / 256) <= 8
  static_assert(kMaxSelSlices * kUnitsPerWG <= 8 * kScoreThreads, "keys per lane");
  if (s.U <= 4 * kScoreThreads)
    k_select_attend<bf16_t, D, G, 4><<<grid, kRowsThreads, 0, st>>>(s, a, p, ready);
  else
    k_select_attend<bf16_t, D, G, 8><<<grid, kRowsThreads, 0, st>>>(s, a, p, ready);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_step_d(const ScoreArgs& s, const AttendArgs& a, const StepPlan& p,
                                int* ready, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_step_dg<D, 1>(s, a, p, ready, st);
    case 2: return launch_step_dg<D, 2>(s, a, p, ready, st);
    case 4: return launch_step_dg<D, 4>(s, a, p, ready, st);
    case 8: return launch_step_dg<D, 8>(s, a, p, ready, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_select_attend(const ScoreArgs& s, const AttendArgs& a, const StepPlan& p,
                                int* ready, hipStream_t st) {
  if (a.n_pos <= 0) return hipSuccess;
  return a.d == 128 ? launch_step_d<128>(s, a, p, ready, st) : launch_step_d<64>(s, a, p, ready, st);
}

}  // namespace infllm
