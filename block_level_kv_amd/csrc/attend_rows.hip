// Working-context attention of single query positions on the vector ALUs:
// the decode path (one query per step; the G query heads of a KV head share
// every K/V row loaded), the path for fp32 and the head sizes the MFMA
// kernel does not take, and the decode step in one launch (scores,
// selection and attention).
//
// For a single position t the working context (InfLLM Guide, "Core
// Innovation 2", item 3; "Core Innovation 1", items 1-2) is a union of
// disjoint key intervals:
//     [0, min(n_init, t+1))                     initial tokens
//     [first_key(u), min(end(u), t-W+1))        each selected unit u
//     [max(n_init, t-W+1), t+1)                 local window (t included)
// so no per-key mask is needed.  The work of a row is split over several
// workgroups (split-K), each with a share of the local keys and a share of
// the units' keys.  They publish partial (max, sum, unnormalised output)
// rows; the last one to arrive merges them in split order (see common.h for
// the publication protocol), so one launch produces the output.
#include "common.h"
#include "kernels.h"
#include "rope.h"
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

// Bounded wait for a selection made in the same launch (polls of a few
// hundred ns each; a selection takes microseconds).  The wait always ends
// before the bound (see k_select_attend); the bound only turns a broken
// invariant into NaN rows and a nonzero status word instead of a hang.
constexpr int kSpinLimit = 1 << 18;
// The selector's first, bounded spin on the arrival mask before it checks
// for slices nobody started (normally the row's scorers finish within it),
// and an attention workgroup's on the selector's flag before it selects
// the row itself (INFLLM_STEP_PRESPIN overrides the latter).
constexpr int kPreSpin = 1 << 12;

// LDS of one decode attention workgroup.
template <int G, int D, bool ROPE = false>
struct RowsShared {
  int64_t iv_lo[kMaxTopK];            // first key position of unit m
  int32_t iv_first[kMaxTopK + 1];     // first unit-key index of unit m (< k_m * B)
  int32_t ids[kMaxTopK];
  int32_t iv_turn[ROPE ? kMaxTopK : 1];   // RoPE: shift E_m of unit m (rope.h)
  double turns[ROPE ? D / 2 : 1];         // RoPE: frequencies, turns per position
  int wave_tot[kRowsThreads / 64];
  int flag, last, all_in;
  uint64_t todo;
  float sm_m[16][G], sm_l[16][G];
  float sm_o[16][G][D];
  float sm_M[G], sm_L[G];
};

// The attention of one workgroup over its share of one (position, KV head,
// sequence) row's working context.  The local keys (initial tokens, then
// the window; they follow from the position alone) are numbered
// 0 .. n_local-1 and the workgroup takes [n_local*l_lo/l_den,
// n_local*l_hi/l_den); the selected units' keys are numbered in selection
// order (each unit at most B keys) and cut into u_parts equal shares, of
// which it takes u_part.  Its keys are indexed 0 .. nl-1 (local) and
// nl .. nl+nu-1 (units) and can be streamed in any order of ranges.
// Within the workgroup 16 lanes share a key (each holds D/16 columns: one
// coalesced 16-byte load per lane for bf16, D = 128); the 16 key lanes run
// independent online softmaxes merged through LDS, and the next group of
// keys is loaded while the current one is reduced.
// ROPE: every key is turned by the shift of its place in the working
// context (rope.h) as it is converted: lanes seg and seg ^ 8 hold the two
// halves of each rotary pair, the cosines and sines of the last shift stay
// in registers until a key of another shift comes.
// CACHED: the local keys come from a buffer of the initial tokens and a
// ring of the later positions, the units' keys from their slots in a unit
// cache (the unit table holds slab rows instead of positions).
template <typename T, int D, int G, bool ROPE = false, bool CACHED = false>
struct RowsAttn {
  static constexpr int CPT = D / 16;
  static constexpr int kGroup = 16 * kKeysPerIter;   // keys per iteration
  const AttendArgs& a;
  RowsShared<G, D, ROPE>& sh;
  int tid, lane, seg, kl, pos, h, bi;
  bool valid;
  int64_t t, unit_cap, init_len, win_lo, n_local, l_begin, nl, u_begin, pu, nu;
  const int32_t* sel_row;
  const T* kb;   // K and V of the row's KV head (uniform); a lane reads columns seg*CPT ..
  const T* vb;
  const T* cb;   // CACHED: the row's cache slabs
  const T* cvb;
  int64_t ring_off, ring_len;   // CACHED: window position p sits at row p + ring_off (wrapped)
  int cur;
  RowRaw<T, CPT> qraw[G];
  float qv[G][CPT], m[G], l[G], acc[G][CPT];
  RowRaw<T, CPT> kn[kKeysPerIter], vn[kKeysPerIter];
  bool okn[kKeysPerIter];
  // RoPE: first local place lo, shift of the initial tokens, shift of each
  // key in flight, and the shift whose cos / sin (sign folded in) are held
  int64_t lo_ctx;
  int e_sink, e_have;
  int en[kKeysPerIter];
  float rc[CPT], rs[CPT];

  // A sequence whose position does not fit its KV buffer reads no key and
  // gets NaN rows; its workgroups still take part in the merge.
  __device__ __forceinline__ RowsAttn(const AttendArgs& a_, RowsShared<G, D, ROPE>& sh_, int pos_,
                                      int h_, int bi_)
      : a(a_), sh(sh_), pos(pos_), h(h_), bi(bi_) {
    tid = threadIdx.x;
    lane = tid % 64;
    seg = tid % 16;
    kl = tid / 16;
    const int64_t base = seq_base(a.pos, a.q_pos, bi);
    valid = !a.pos || seq_pos_ok(base, a.n_pos, a.kv_cap);
    t = valid ? base + pos : 0;
    load_q();   // first: the loads overlap what follows
    unit_cap = t - a.W + 1;
    init_len = !valid ? 0 : (a.n_init < t + 1 ? a.n_init : t + 1);
    win_lo = a.n_init > unit_cap ? a.n_init : unit_cap;
    const int64_t win_len = valid && t + 1 - win_lo > 0 ? t + 1 - win_lo : 0;
    n_local = init_len + win_len;
    const int ch = pos / a.L;
    sel_row = a.sel ? a.sel + (((int64_t)bi * a.Hkv + h) * a.n_chunks + ch) * a.k_m : nullptr;
    const int64_t stride = CACHED ? a.local_cap : a.kv_cap;
    kb = (const T*)a.k + ((int64_t)bi * a.Hkv + h) * stride * D;
    vb = (const T*)a.v + ((int64_t)bi * a.Hkv + h) * stride * D;
    if constexpr (CACHED) {
      const int64_t slab = ((int64_t)bi * a.Hkv + h) * a.n_slots * a.B * D;
      cb = (const T*)a.ck + slab;
      cvb = (const T*)a.cv + slab;
      ring_len = a.local_cap - a.n_init;
      ring_off = a.n_init + (win_lo - a.n_init) % ring_len - win_lo;
    }
    cur = 0;
    nu = 0;
    if constexpr (ROPE) {
      // chunk start t0 -> first local place; published by build_table's barrier
      const int64_t t0 = valid ? base + (int64_t)(pos / a.L) * a.L : 0;
      lo_ctx = rope_local_start(t0, a.n_init, a.W);
      e_sink = (int)(a.n_init + (int64_t)a.k_m * a.B - lo_ctx);
      e_have = 0;   // 0 is never turned: nothing held yet
      if (tid < D / 2) sh.turns[tid] = rope_turns(a.rope_theta, D, tid);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[g][c] = 0.f;
    }
  }

  __device__ __forceinline__ void load_q() {
#pragma unroll
    for (int g = 0; g < G; ++g)
      qraw[g].load((const T*)a.q +
                   (((int64_t)bi * a.Hq + (int64_t)h * G + g) * a.q_cap + a.q_off + pos) * D +
                   seg * CPT);
  }

  // The softmax state to LDS (park) and back with the query rows reloaded
  // (restore), so that nothing of it stays live in registers across the
  // work in between.  The 16 lanes of a key lane hold the same m and l.
  __device__ __forceinline__ void restore() {
    load_q();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = sh.sm_m[kl][g];
      l[g] = sh.sm_l[kl][g];
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[g][c] = sh.sm_o[kl][g][seg * CPT + c];
    }
    make_qv();
    __syncthreads();
  }

  __device__ __forceinline__ void park() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (seg == 0) {
        sh.sm_m[kl][g] = m[g];
        sh.sm_l[kl][g] = l[g];
      }
#pragma unroll
      for (int c = 0; c < CPT; ++c) sh.sm_o[kl][g][seg * CPT + c] = acc[g][c];
    }
    __syncthreads();
  }
  __device__ __forceinline__ void shares(int64_t l_lo, int64_t l_hi, int64_t l_den, int u_part,
                                         int u_parts) {
    l_begin = n_local * l_lo / l_den;
    nl = n_local * l_hi / l_den - l_begin;
    pu = u_parts > 0 ? ((int64_t)a.k_m * a.B + u_parts - 1) / u_parts : 0;
    u_begin = (int64_t)u_part * pu;
  }

  // Position of key b0 + li (b0 uniform, li the lane's offset in the
  // group): keys below nl are local, then unit keys through the table (within
  // the unit range each lane's indices only grow, so a cursor works).  The
  // per-lane comparisons are 32-bit.
  __device__ __forceinline__ static int clamp32(int64_t v) {
    return v > INT32_MAX ? INT32_MAX : (v < INT32_MIN ? INT32_MIN : (int)v);
  }
  // KIND: kMixed, or a range known to hold only local (kLocal) or only unit
  // (kUnits) keys.
  static constexpr int kMixed = 0, kLocal = 1, kUnits = 2;
  template <int KIND>
  __device__ __forceinline__ int64_t key_pos(int64_t b0, int li) {
    if (KIND == kLocal || (KIND == kMixed && li < clamp32(nl - b0))) {
      const int64_t x0 = l_begin + b0;
      return li < clamp32(init_len - x0) ? x0 + li : x0 + (win_lo - init_len) + li;
    }
    const int y = (int)(u_begin + b0 - nl) + li;   // unit-key index, < k_m * B
    while (y >= sh.iv_first[cur + 1]) ++cur;
    return sh.iv_lo[cur] + (y - sh.iv_first[cur]);
  }

  template <int KIND = kMixed>
  __device__ __forceinline__ void fetch(int64_t b0, int64_t end) {
    // keys of the group left in the range (uniform), so that the per-lane
    // index within the group stays 32-bit
    const int rem = end - b0 < kGroup ? (int)(end - b0) : kGroup;
#pragma unroll
    for (int j = 0; j < kKeysPerIter; ++j) {
      const int li = kl + 16 * j;
      okn[j] = li < rem;
      const int64_t p = okn[j] ? key_pos<KIND>(b0, li) : 0;
      if constexpr (CACHED) {
        // unit keys: p is a slab row; local ones: the ring row of position p
        const bool unit = KIND == kUnits || (KIND == kMixed && li >= clamp32(nl - b0));
        int64_t r = p;
        if (!unit && p >= a.n_init) {
          r = p + ring_off;
          if (r >= a.local_cap) r -= ring_len;
        }
        const int64_t off = r * D + seg * CPT;
        kn[j].load((unit ? cb : kb) + off);
        vn[j].load((unit ? cvb : vb) + off);
      } else {
        const int64_t off = p * D + seg * CPT;
        kn[j].load(kb + off);
        vn[j].load(vb + off);
      }
      if constexpr (ROPE)   // only unit keys lie in [n_init, lo): cur is theirs
        en[j] = !okn[j] || p >= lo_ctx ? 0 : (p < a.n_init ? e_sink : sh.iv_turn[cur]);
    }
  }

  // Unit table of the row's selection (thread m passes entry m; repeated ids
  // count once): each unit's first key and first unit-key index, by a block
  // scan of the unit lengths.  Sets nu, this workgroup's unit keys.  Every
  // thread calls it.  CACHED: the first key's slab row instead of its
  // position; returns true if a unit with keys to attend is not cached.
  __device__ __forceinline__ bool build_table(int32_t u) {
    u = drop_repeats(u, tid, a.k_m, sh.ids);
    int64_t lo = 0, len = 0;
    bool absent = false;
    if (u >= 0) {
      lo = unit_first_key(u, a.B, a.n_init);
      const int64_t hi = ((int64_t)u + a.n_init / a.B + 1) * a.B;
      len = (hi < unit_cap ? hi : unit_cap) - lo;
      len = len > 0 ? len : 0;
      if constexpr (CACHED) {
        const int s = u < a.n_units ? a.c_slot[((int64_t)bi * a.Hkv + h) * a.n_units + u] - 1 : -1;
        if (s < 0) {
          absent = len > 0;
          len = 0;
        } else {
          lo = (int64_t)s * a.B + (lo - hi + a.B);   // row of the first key in slot s
        }
      }
    }
    int x = (int)len;   // inclusive scan of the unit lengths (each <= B)
#pragma unroll
    for (int mm = 1; mm < 64; mm <<= 1) {
      const int y = __shfl_up(x, mm);
      if (lane >= mm) x += y;
    }
    if (lane == 63) sh.wave_tot[tid / 64] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w2 = 0; w2 < kRowsThreads / 64; ++w2) {
      before += w2 < tid / 64 ? sh.wave_tot[w2] : 0;
      all += sh.wave_tot[w2];
    }
    if (tid < a.k_m) {
      sh.iv_lo[tid] = lo;
      sh.iv_first[tid] = before + x - (int)len;
      if constexpr (ROPE)   // slot tid: E_m = (k_m - m) B + jB - lo
        sh.iv_turn[tid] = u < 0 ? 0 : (int)((int64_t)(a.k_m - tid) * a.B +
                                            ((int64_t)u + a.n_init / a.B) * a.B - lo_ctx);
    }
    if (tid == 0) sh.iv_first[a.k_m] = all;
    __syncthreads();
    const int64_t n_unit = sh.iv_first[a.k_m];
    const int64_t u_stop = u_begin + pu < n_unit ? u_begin + pu : n_unit;
    nu = u_stop > u_begin ? u_stop - u_begin : 0;
    cur = 0;
    if constexpr (CACHED) return __syncthreads_or(absent);
    return false;
  }

  // cos / sin of shift E at this lane's columns, sign of its half folded in
  __device__ __forceinline__ void hold_turn(int E) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      rope_cs(E, sh.turns[(seg & 7) * CPT + i], &rc[i], &rs[i]);
      if (seg >= 8) rs[i] = -rs[i];
    }
    e_have = E;
  }
  // x (this lane's CPT columns of one vector) turned by -E; both lanes of
  // every pair take the same branch (same key, or the row's query)
  __device__ __forceinline__ void turn(float* x, int E) {
    if (E == 0) return;
    if (E != e_have) hold_turn(E);
    float px[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) px[i] = dpp_f32<INFLLM_DPP_ROR8>(x[i]);
#pragma unroll
    for (int i = 0; i < CPT; ++i) x[i] = fmaf(px[i], rs[i], x[i] * rc[i]);
  }

  // A query before n_init sees initial tokens only; they are turned by
  // -E_s, so it is turned by -E_s too (every lane of the workgroup holds
  // the same position: a uniform branch).
  __device__ __forceinline__ void make_qv() {
    const float qscale = kLog2e / sqrtf((float)D);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      qraw[g].to_f32(qv[g]);
      if constexpr (ROPE) {
        if (valid && t < a.n_init) turn(qv[g], e_sink);
      }
#pragma unroll
      for (int c = 0; c < CPT; ++c) qv[g][c] *= qscale;
    }
  }

  // Keys [lo, hi), kGroup per iteration, the next group in flight while the
  // current one is reduced.
  template <int KIND = kMixed>
  __device__ __forceinline__ void stream(int64_t lo, int64_t hi, bool in_flight) {
    if (lo >= hi) return;
    if (!in_flight) fetch<KIND>(lo, hi);
    for (int64_t b0 = lo; b0 < hi; b0 += kGroup) {
      RowRaw<T, CPT> kc[kKeysPerIter], vc[kKeysPerIter];
      bool ok[kKeysPerIter];
      int ec[kKeysPerIter];
#pragma unroll
      for (int j = 0; j < kKeysPerIter; ++j) {
        kc[j] = kn[j];
        vc[j] = vn[j];
        ok[j] = okn[j];
        if constexpr (ROPE) ec[j] = en[j];
      }
      if (b0 + kGroup < hi) fetch<KIND>(b0 + kGroup, hi);  // in flight
      step(kc, vc, ok, ec);
    }
  }

  // One group of keys: logits for every head (each key row converted once),
  // then the online softmax update; s becomes the weights p.
  __device__ __forceinline__ void step(const RowRaw<T, CPT>* kc, const RowRaw<T, CPT>* vc,
                                       const bool* ok, const int* ec) {
    float s[G][kKeysPerIter];
#pragma unroll
    for (int j = 0; j < kKeysPerIter; ++j) {
      float kf[CPT];
      kc[j].to_f32(kf);
      if constexpr (ROPE) turn(kf, ec[j]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d0 = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) d0 = fmaf(qv[g][c], kf[c], d0);
        const float r = row16_sum(d0);  // the 16 lanes of a row share key j
        s[g][j] = ok[j] ? r : -INFINITY;
      }
    }
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

  // Merge of the 16 key lanes, then of the n_splits workgroups of the row
  // (split-K): each publishes its partial (max, sum, row) with device-scope
  // stores and counts itself in on merge_count (adding 1); the last of them
  // merges every partial in split order and writes the output.  `others`
  // more workgroups of the row count in with 1 << 16 and merge nothing;
  // whichever arrival completes the count clears the counter and the
  // n_reset ints at reset (the fused step's row state).  stale: the
  // selection never arrived, the row gets NaN.
  __device__ __forceinline__ void finish(int split, int n_splits, int* merge_count, int others,
                                         int* reset, int n_reset, bool stale) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (seg == 0) {
        sh.sm_m[kl][g] = m[g];
        sh.sm_l[kl][g] = l[g];
      }
#pragma unroll
      for (int c = 0; c < CPT; ++c) sh.sm_o[kl][g][seg * CPT + c] = acc[g][c];
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
      for (int r = 0; r < 16; ++r) Mv[i] = fmaxf(Mv[i], sh.sm_m[r][g]);
      if (Mv[i] != -INFINITY) {
        for (int r = 0; r < 16; ++r) {
          const float w = __builtin_amdgcn_exp2f(sh.sm_m[r][g] - Mv[i]);
          Lv[i] = fmaf(sh.sm_l[r][g], w, Lv[i]);
          Ov[i] = fmaf(sh.sm_o[r][g][col], w, Ov[i]);
        }
      }
    }
    if (stale) {
#pragma unroll
      for (int i = 0; i < kOut; ++i) Mv[i] = Lv[i] = Ov[i] = __builtin_nanf("");
    }

    const int splits = n_splits;
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
        const int done =
            __hip_atomic_fetch_add(merge_count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.last = (done & 0xFFFF) == splits - 1;
        sh.all_in = done + 1 == ((others << 16) | splits);
      }
      __syncthreads();
      if (sh.all_in) {
        // every workgroup of the row has counted in (and is past everything
        // it does before that): the row's counters are ready for the next call
        if (tid == 0) __hip_atomic_store(merge_count, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid < n_reset)
          __hip_atomic_store(reset + tid, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (!sh.last) return;
      // Merge every split's published rows (this one's included).  Each
      // thread's (max, sum) pairs and its output columns' first batch of
      // split values are requested together: one memory round trip when the
      // splits fit a batch.  The (max, sum) table is padded to kMaxSplits
      // with (-inf, 0), so the weight pass and the weighted sums run without
      // per-split branches (padding weights are 0 and padding loads return 0).
      float* sm_w = &sh.sm_o[0][0][0];               // reuse: [kMaxSplits][G] weights
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
      // without branches (byte offsets fit 32 bits: the plans keep the
      // partial rows below 4 GiB).
      const __amdgpu_buffer_rsrc_t ro = dev_rsrc(a.ws_o, (uint32_t)(splits * stride * 4));
      float vbuf[kOut][kBatch];
      auto load_batch = [&](int s0) {
#pragma unroll
        for (int i = 0; i < kOut; ++i) {
          const int o = tid + i * kRowsThreads;
          const int g = (o < G * D ? o : 0) / D, col = o % D;
          const uint32_t off = (uint32_t)(((qh0 + g) * a.n_pos + pos) * D + col);
#pragma unroll
          for (int j = 0; j < kBatch; ++j)
            vbuf[i][j] = ld1_dev(ro, (off + (uint32_t)((s0 + j) * stride)) * 4u);
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
            sh.sm_M[g] = M;
            sh.sm_L[g] = Ls;
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
          for (int j = 0; j < kBatch; ++j) Os[i] = fmaf(vbuf[i][j], sm_w[(s0 + j) * G + g], Os[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < kOut; ++i) {
        const int o = tid + i * kRowsThreads;
        if (o >= G * D) continue;
        const int g = o / D;
        Mv[i] = sh.sm_M[g];
        Lv[i] = sh.sm_L[g];
        Ov[i] = Os[i];
      }
    }
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      const int o = tid + i * kRowsThreads;
      if (o >= G * D) continue;
      const int g = o / D, col = o % D;
      const int64_t qh = qh0 + g;
      T* out = (T*)a.out + (qh * a.out_cap + a.out_off + pos) * D + col;
      *out = from_f32<T>(valid ? Ov[i] / Lv[i] : nan);
      if (a.lse && col == 0)
        a.lse[qh * a.out_cap + a.out_off + pos] = valid ? (Mv[i] + log2f(Lv[i])) * kLn2 : nan;
    }
  }
};

// Decode attention (and the fp32 / head-size paths): gridDim.x splits per
// (position, KV head, sequence) row, each an equal share of the local keys
// and of the units' keys.  Its first local keys are requested before the
// selection is read and the unit table formed.
template <typename T, int D, int G, bool ROPE, bool CACHED = false>
__global__ __launch_bounds__(kRowsThreads) void k_attend_rows(AttendArgs a) {
  using Attn = RowsAttn<T, D, G, ROPE, CACHED>;
  __shared__ RowsShared<G, D, ROPE> sh;
  const int s = blockIdx.x, n = gridDim.x;
  const int pos = blockIdx.y, h = blockIdx.z % a.Hkv, bi = blockIdx.z / a.Hkv;
  const int64_t row = ((int64_t)bi * a.Hkv + h) * a.n_pos + pos;
  Attn r(a, sh, pos, h, bi);
  r.shares(s, s + 1, n, s, n);
  int32_t u = -1;   // this thread's sel entry, requested now
  if (r.valid && threadIdx.x < a.k_m) u = r.sel_row[threadIdx.x];
  const bool early = r.nl >= Attn::kGroup;   // first group local only: in flight
  if (early) r.template fetch<Attn::kLocal>(0, r.nl);
  const bool absent = r.build_table(u);
  r.make_qv();
  r.stream(0, r.nl + r.nu, early);
  r.finish(s, n, a.ws_count ? a.ws_count + row : nullptr, 0, nullptr, 0, absent);
}

int rows_num_splits(const AttendArgs& a) {
  // enough workgroups to cover the chip several times, >= ~256 keys each
  const int64_t max_keys = (int64_t)a.n_init + (int64_t)a.k_m * a.B + a.W;
  const int64_t wgs = (int64_t)a.n_pos * a.batch * a.Hkv;
  const int64_t target = tuning().rows_wgs > 0 ? tuning().rows_wgs : 512;
  int64_t s = (target + wgs - 1) / wgs;
  const int64_t cap = (max_keys + 255) / 256;
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

int64_t rows_num_counters(const AttendArgs& a) { return (int64_t)a.n_pos * a.batch * a.Hkv; }

template <typename T, int D, int G>
static hipError_t launch_rows_tdg(const AttendArgs& a, int splits, hipStream_t st) {
  const dim3 grid(splits, a.n_pos, a.batch * a.Hkv);
  if (a.rope_theta > 0.0)
    k_attend_rows<T, D, G, true><<<grid, kRowsThreads, 0, st>>>(a);
  else
    k_attend_rows<T, D, G, false><<<grid, kRowsThreads, 0, st>>>(a);
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

template <typename T, int D>
static hipError_t launch_cached_td(const AttendArgs& a, int splits, hipStream_t st) {
  const dim3 grid(splits, a.n_pos, a.batch * a.Hkv);
  switch (a.Hq / a.Hkv) {
    case 1: k_attend_rows<T, D, 1, false, true><<<grid, kRowsThreads, 0, st>>>(a); break;
    case 2: k_attend_rows<T, D, 2, false, true><<<grid, kRowsThreads, 0, st>>>(a); break;
    case 4: k_attend_rows<T, D, 4, false, true><<<grid, kRowsThreads, 0, st>>>(a); break;
    case 8: k_attend_rows<T, D, 8, false, true><<<grid, kRowsThreads, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attend_rows_cached(const AttendArgs& a, int splits, hipStream_t st) {
  if (a.n_pos <= 0) return hipSuccess;
  if (a.bf16)
    return a.d == 128 ? launch_cached_td<bf16_t, 128>(a, splits, st)
                      : launch_cached_td<bf16_t, 64>(a, splits, st);
  return a.d == 128 ? launch_cached_td<float, 128>(a, splits, st)
                    : launch_cached_td<float, 64>(a, splits, st);
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
// Scores, selection and attention of decode positions in one launch.  A row
// (one position of one KV head of one sequence) has p.n_splits workgroups;
// the first p.s_score of them each score a slice of p.units_per units.
//
// A scoring workgroup marks its slice started (a flag), scores it, publishes
// its candidates -- all of the slice's scores, or its best min(k_m, units)
// when the row has too many to search at once (the row's top k_m is among
// the union of every slice's top k_m, ties to the lower index in both) --
// and sets the slice's bit in the row's arrival mask with an atomic OR.
// One more workgroup per row, the selector, waits for the full mask,
// selects the row's k_m units from the candidates, publishes them and sets
// the row's ready flag.  Every other workgroup of the row (scoring ones
// after their slice) attends its share of the local keys, which need no
// selection, then reads the ready flag and attends its share of the
// selected units' keys.
//
// Why every wait ends, whatever the dispatch order, the grid size or the
// number of workgroups resident at once: no workgroup waits on one that
// may not be running.  Before waiting for the mask (the selector, or an
// attention workgroup whose flag is not set yet) a workgroup checks the
// slices' started flags and scores every slice not started itself
// (publishing the same candidates and setting the same bit, so a slice
// scored twice is harmless); scoring never waits, so the mask fills.  An
// attention workgroup then spins a bounded time for the selector's flag;
// if it has not come, it selects the row itself: the same candidates and
// the same search give the same units, so every copy it or the selector
// stores is the same.  All attention workgroups publish their partial rows
// and the last of them merges; the selector counts in on the same counter
// (with a separate field), and the last arrival of all clears the row's
// mask, flags and counter for the next call.
struct StepRow {
  uint64_t* mask;      // arrival mask of the slices
  int* ready;          // the selection is published
  int* merge;          // merge counter
  uint8_t* started;    // one byte per slice
};
__device__ __forceinline__ StepRow step_row(const StepPtrs& w, int64_t row) {
  int* base = w.sync + row * kStepSyncInts;
  return StepRow{(uint64_t*)base, base + 2, base + 3, (uint8_t*)(base + 4)};
}

// LDS of the scoring and selection parts of a fused step (one copy per
// workgroup, shared by both).
struct StepShared {
  double qsum[128];
  float sc[4 * kUnitsPerWG];
  int32_t pick[kMaxTopK];
  TopkShared tsm;
  uint64_t todo;
  int last;
};

// The row's selection from its s_score * C published candidates (candidate
// order is ascending unit order, so positions map to ascending unit ids):
// entry m for thread m < k_m.  Every thread calls it.
template <int VPT>
__device__ __forceinline__ int32_t step_select(const ScoreArgs& s, const StepPlan& p, int row,
                                               const StepPtrs& w, StepShared& ss) {
  const int64_t c0 = (int64_t)row * p.s_score * p.cand;
  __syncthreads();   // the scratch may still be read by an earlier part
  block_topk<kRowsThreads / 64, VPT, true>(w.cand_s + c0, p.s_score * p.cand, s.k_m, ss.pick,
                                           ss.tsm);
  __syncthreads();
  const int tid = threadIdx.x;
  const int pp = tid < s.k_m ? ss.pick[tid] : -1;
  return pp >= 0 ? __hip_atomic_load(w.cand_i + c0 + pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : -1;
}

// One slice's scores, candidates and arrival bit.  SERIAL: the slice's
// 64-unit parts are loaded one after another (fewer registers; for the rare
// scoring of a slice that was not started).
template <typename T, int G, int D, int NSUB, bool SERIAL>
__device__ __forceinline__ void step_score(const ScoreArgs& s, const StepPlan& p, int sl, int row,
                                           int pos, int h, int bi, const StepRow& y,
                                           const StepPtrs& w, StepShared& ss) {
  using Rows = UnitRows<D, kUnitsPerWG / UnitRows<D, 1>::kPerSlot>;   // 64 units
  static_assert(D <= 128 && NSUB <= 4, "StepShared sizes");
  double* qsum = ss.qsum;
  float* sc_sm = ss.sc;
  int32_t* pick_sm = ss.pick;
  TopkShared& tsm = ss.tsm;
  const int tid = threadIdx.x;
  const int U = s.U;
  const int u0 = sl * p.units_per;
  const int u1 = u0 + p.units_per < U ? u0 + p.units_per : U;
  const float* rb = s.repr + ((int64_t)bi * s.Hkv + h) * U * D;
  constexpr int kHeld = SERIAL ? 1 : NSUB;   // 64-unit parts whose rows are held at once
  Rows rows[kHeld];
#pragma unroll
  for (int j = 0; j < kHeld; ++j) rows[j].load(rb, U, u0 + j * kUnitsPerWG);   // in flight
  // the group's query sum for this position (fp64, heads in order)
  if (tid < D) {
    const T* qb = (const T*)s.q +
                  (((int64_t)bi * s.Hq + (int64_t)h * G) * s.q_cap + s.q_off + pos) * D + tid;
    T v[G];
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = qb[(int64_t)g * s.q_cap * D];
    double acc = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g) acc += (double)to_f32(v[g]);
    qsum[tid] = acc;
  }
  __syncthreads();
  // a position out of range leaves no unit eligible (negative) or all of
  // them (large); the clamp keeps the sum below overflow
  int64_t t0 = seq_base(s.pos, s.q_pos, bi);
  t0 = t0 < -kPosLimit ? -kPosLimit : (t0 > kPosLimit ? kPosLimit : t0);
  const int64_t e = eligible_units(t0 + pos, U, s.B, s.n_init, s.W);
  const int cg = tid % 64 % (D / 8);
  double qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qv[j] = qsum[cg * 8 + j];
  float* sb = s.scores + (int64_t)row * U;
  if constexpr (SERIAL) {
    for (int j = 0; j < NSUB; ++j) {
      if (j > 0) rows[0].load(rb, U, u0 + j * kUnitsPerWG);
      rows[0].score_lds(qv, u0 + j * kUnitsPerWG, u1, e, sb, sc_sm, u0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NSUB; ++j) rows[j].score_lds(qv, u0 + j * kUnitsPerWG, u1, e, sb, sc_sm, u0);
  }
  __syncthreads();
  // candidates: the slice's best C units (all of them if it holds at most C)
  const int n = u1 - u0, C = p.cand;
  const int64_t slot = ((int64_t)row * p.s_score + sl) * C;
  if (n > C) {
    block_topk<kRowsThreads / 64, 1, false>(sc_sm, n, C, pick_sm, tsm);
    __syncthreads();
  }
  for (int m = tid; m < C; m += kRowsThreads) {
    const int idx = n > C ? pick_sm[m] : (m < n ? m : -1);
    st_dev(w.cand_s + slot + m, idx >= 0 ? sc_sm[idx] : -INFINITY);
    __hip_atomic_store(w.cand_i + slot + m, idx >= 0 ? u0 + idx : -1, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid == 0)
    __hip_atomic_fetch_or(y.mask, 1ull << sl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Scores every slice of the row not started yet (the check that makes a
// wait safe), then waits until `done` holds, polling `flag`; returns false
// (and counts the time-out in the status word) if the bound ran out.
// Every thread calls it.
template <typename T, int G, int D, int NSUB, int VPT, typename Done>
__device__ __forceinline__ bool step_wait(const ScoreArgs& s, const StepPlan& p, int row, int pos,
                                          int h, int bi, const StepRow& y, const StepPtrs& w,
                                          StepShared& ss, const Done& done) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const uint64_t mk = __hip_atomic_load(y.mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool todo = tid < p.s_score && !((mk >> tid) & 1) &&
                      __hip_atomic_load(y.started + tid, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == 0;
    const uint64_t b = __ballot(todo);
    if (tid == 0) ss.todo = b;
  }
  __syncthreads();
  uint64_t todo = ss.todo;
  while (todo) {
    const int sl = __builtin_ctzll(todo);
    todo &= todo - 1;
    if (tid == 0)
      __hip_atomic_store(y.started + sl, (uint8_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    step_score<T, G, D, NSUB, true>(s, p, sl, row, pos, h, bi, y, w, ss);
  }
  if (tid == 0) {
    int ok = 0;
    for (int it = 0; it < kSpinLimit && !ok; ++it) {
      ok = done();
      if (!ok) __builtin_amdgcn_s_sleep(2);
    }
    if (!ok) __hip_atomic_fetch_add(w.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ss.last = ok;
  }
  __syncthreads();
  return ss.last;
}

// ROPE: keys turned to their places in the working context; the turned
// keys' registers fit two workgroups per CU (the plan puts at most two
// there), the others three.
template <typename T, int D, int G, int NSUB, int VPT, bool ROPE>
__global__ __launch_bounds__(kRowsThreads) __attribute__((amdgpu_waves_per_eu(ROPE ? 2 : 3)))
void k_select_attend(ScoreArgs s, AttendArgs a, StepPlan p, StepPtrs w) {
  static_assert(kRowsThreads == kScoreThreads, "one workgroup size for both roles");
  using Attn = RowsAttn<T, D, G, ROPE>;
  __shared__ RowsShared<G, D, ROPE> sh;
  __shared__ StepShared ss;
  const int N = p.n_splits, S = p.s_score;
  // row = (sequence * H_kv + KV head) * positions + position; one chunk per
  // position.  Workgroup N of a row is its selector.
  const int row = (int)blockIdx.x / (N + 1), j = (int)blockIdx.x % (N + 1);
  const int pos = row % a.n_pos, h = row / a.n_pos % a.Hkv, bi = row / a.n_pos / a.Hkv;
  const StepRow y = step_row(w, row);
  const int tid = threadIdx.x;
  const uint64_t full = S == 64 ? ~0ull : (1ull << S) - 1ull;
  auto mask_full = [&]() {
    return __hip_atomic_load(y.mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == full;
  };
  if (j == N) {
    // the selector: waits for the mask (a bounded spin first, during which
    // the row's scorers normally finish; then the check that makes the
    // wait safe), selects and publishes the row's units
    if (tid == 0) {
      int ok = 0;
      for (int it = 0; it < kPreSpin && !ok; ++it) {
        ok = mask_full();
        if (!ok) __builtin_amdgcn_s_sleep(2);
      }
      ss.last = ok;
    }
    __syncthreads();
    const bool ok = ss.last || step_wait<T, G, D, NSUB, VPT>(s, p, row, pos, h, bi, y, w, ss,
                                                             mask_full);
    if (ok) {
      const int32_t u = step_select<VPT>(s, p, row, w, ss);
      if (tid < s.k_m)
        __hip_atomic_store(s.sel + (int64_t)row * s.k_m + tid, u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
      if (ok) {
        __hip_atomic_store(y.ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {   // a time-out marks the row unless an attention workgroup selected it
        int zero = 0;
        __hip_atomic_compare_exchange_strong(y.ready, &zero, -1, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // the flag lands before the count
      const int done =
          __hip_atomic_fetch_add(y.merge, 1 << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh.all_in = done + (1 << 16) == ((1 << 16) | N);
    }
    __syncthreads();
    if (sh.all_in && tid < kStepSyncInts)   // the last of the row: clear its state
      __hip_atomic_store(w.sync + (int64_t)row * kStepSyncInts + tid, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (j < S) {
    if (tid == 0)
      __hip_atomic_store(y.started + j, (uint8_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    step_score<T, G, D, NSUB, false>(s, p, j, row, pos, h, bi, y, w, ss);
  }
  Attn r(a, sh, pos, h, bi);
  if constexpr (ROPE) __syncthreads();   // the frequency table, before the first turn
  const int64_t l_lo = j < S ? (int64_t)j * p.w_score
                             : (int64_t)S * p.w_score + (int64_t)(j - S) * p.w_unit;
  r.shares(l_lo, l_lo + (j < S ? p.w_score : p.w_unit),
           (int64_t)S * p.w_score + (int64_t)(N - S) * p.w_unit, j, N);
  r.make_qv();
  // the local keys need no selection
  r.template stream<Attn::kLocal>(0, r.nl, false);
  r.park();
  if (tid == 0) sh.flag = __hip_atomic_load(y.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int rd = sh.flag;
  int32_t u = -1;
  bool own = false;   // u holds this workgroup's own selection
  if (rd == 0) {
    // not published yet: every slice started, then the full mask (neither
    // wait depends on a workgroup that may not be running), then a bounded
    // spin for the selector's flag, and the selection here if it has not come
    if (step_wait<T, G, D, NSUB, VPT>(s, p, row, pos, h, bi, y, w, ss, mask_full)) {
      if (tid == 0) {
        int f = 0;
        for (int it = 0; it < p.pre_spin && f == 0; ++it) {
          f = __hip_atomic_load(y.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (f == 0) __builtin_amdgcn_s_sleep(2);
        }
        sh.flag = f;
      }
      __syncthreads();
      rd = sh.flag;
      if (rd == 0) {
        u = step_select<VPT>(s, p, row, w, ss);
        if (tid < s.k_m)
          __hip_atomic_store(s.sel + (int64_t)row * s.k_m + tid, u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (tid == 0) {
          __hip_atomic_store(y.ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_fetch_add(w.status + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        rd = 1;
        own = true;
      }
    } else {
      rd = -1;
    }
  }
  const bool stale = rd != 1;
  // the row's units, then their keys
  if (stale || !r.valid) u = -1;
  else if (!own && tid < a.k_m)
    u = __hip_atomic_load(const_cast<int32_t*>(r.sel_row + tid), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  r.restore();
  r.build_table(u);
  r.template stream<Attn::kUnits>(r.nl, r.nl + r.nu, false);
  r.finish(j, N, y.merge, 1, w.sync + (int64_t)row * kStepSyncInts, kStepSyncInts, stale);
}

// Plan of a fused step.  One, two or three workgroups per CU in all (a
// whole number per CU, so that every CU ends together, and at most what is
// resident at once), a selector and n_splits attention workgroups per row.
// Scoring workgroups take the fewest units (64 .. 256) that leave
// at least a sixteenth of a row's workgroups without a slice; every
// workgroup takes an equal share of the units' keys, and the local keys
// are shared so that every workgroup moves about the same number of bytes.
constexpr int64_t kStepCUs = 256;                // MI355X compute units
constexpr int64_t kStepBytesPerWave = 64ll << 20;   // step bytes per workgroup per CU
constexpr int kStepMaxCand = 8 * kRowsThreads;   // candidates of a row: 8 per lane

int64_t step_rows(const AttendArgs& a) { return (int64_t)a.batch * a.Hkv * a.n_pos; }

bool select_attend_plan(const ScoreArgs& s, const AttendArgs& a, StepPlan* p) {
  if (!a.bf16 || a.L != 1 || s.U < 1 || a.k_m < 1 || a.k_m > kMaxTopK) return false;
  const int G = a.Hq / a.Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  // re-positioned keys (head_dim 128, up to 4 query heads a KV head):
  // turning them needs ~40 more VGPRs than three workgroups per CU leave
  // (with the spills, 96 against 53 us per step at 128K in two launches),
  // so such a launch holds at most two; with 8 heads they spill even then
  const bool rope = a.rope_theta > 0.0;
  if (rope && (a.d != 128 || G > 4)) return false;
  const int64_t rows = step_rows(a);
  if (rows > ((int64_t)1 << 24)) return false;
  // one, two or three workgroups per CU, about one per CU for every 64 MiB
  // the step moves (measured at 128K, 153 MB: 43.3 us with 2 per CU, 44.2
  // with 3; Mistral 64K, 36 MB: 24.0 us with 1, 26.4 with 2; a grid that is
  // not a whole number of workgroups per CU leaves some CUs one more and
  // ends late: 49-52 us at 128K with 576 or 640)
  const double row_bytes = (double)s.U * (a.d + 1) * 4.0 +
                           ((double)a.n_init + a.W + (double)a.k_m * a.B) * 2.0 * a.d * 2.0;
  int64_t per_cu = (int64_t)(rows * row_bytes / (double)kStepBytesPerWave + 0.5);
  per_cu = per_cu < 1 ? 1 : (per_cu > (rope ? 2 : 3) ? (rope ? 2 : 3) : per_cu);
  int64_t n = kStepCUs * per_cu / rows - 1;   // attention workgroups (the selector is one more)
  if (tuning().step_splits > 0) n = tuning().step_splits;
  n = n < 2 ? 2 : (n > kMaxSplits ? kMaxSplits : n);
  int up = 0;
  int64_t S = 0;
  for (int c = kUnitsPerWG; c <= 4 * kUnitsPerWG; c += kUnitsPerWG) {
    up = c;
    S = (s.U + c - 1) / c;
    if (S <= n - (n / 16 > 1 ? n / 16 : 1)) break;
  }
  if (S >= n) n = S + (S / 16 > 1 ? S / 16 : 1);
  if (n > kMaxSplits) return false;
  // every score is a candidate when the row has few enough of them.  Rows
  // with more take the separate calls unless the split count is set by
  // hand: the first cut of candidates in every slice makes the one launch
  // slower than the scoring, selection and attention launches there
  // (measured at 8,191 units: 49.8 against 44.5 us per step).
  const bool all_scores = S * up <= kStepMaxCand;
  if (!all_scores && tuning().step_splits == 0) return false;
  const int C = all_scores ? up : (a.k_m < up ? a.k_m : up);
  if (S * C > kStepMaxCand) return false;
  // partial rows are addressed with 32-bit byte offsets in the merge
  if ((double)n * a.batch * a.Hq * a.n_pos * a.d * 4.0 >= 4294967296.0) return false;
  // bytes per workgroup: scoring ones move up*(d+1)*4 more, counted twice
  // (scoring is a latency chain ahead of their local keys, measured to
  // leave them behind the others at equal bytes)
  const double esz = 2.0;
  const double rb = 2.0 * (double)up * (a.d + 1) * 4.0;
  const double ut = (double)a.k_m * a.B * 2.0 * a.d * esz;
  const double lt = (double)(a.n_init + a.W) * 2.0 * a.d * esz;
  const double each = ((double)S * rb + lt + ut) / (double)n;
  double x = each - ut / (double)n - rb;   // local bytes of a scoring workgroup
  double y = each - ut / (double)n;        // ... of the others
  if (x < 0) {
    x = 0;
    y = lt / (double)(n - S);
  }
  p->n_splits = (int)n;
  p->s_score = (int)S;
  p->units_per = up;
  p->cand = C;
  p->w_score = (int)(x / 1024.0 + 0.5);
  p->w_unit = (int)(y / 1024.0 + 0.5);
  if (p->w_score + p->w_unit == 0) p->w_unit = 1;
  p->pre_spin = tuning().step_prespin >= 0 ? tuning().step_prespin : kPreSpin;
  return true;
}

template <int D, int G, int NSUB>
static hipError_t launch_step_dgn(const ScoreArgs& s, const AttendArgs& a, const StepPlan& p,
                                  const StepPtrs& w, hipStream_t st) {
  const dim3 grid((unsigned)(step_rows(a) * (p.n_splits + 1)));
  static_assert(kStepMaxCand <= 8 * kRowsThreads, "candidate keys per lane");
  if constexpr (D == 128 && G <= 4) {   // the shapes the plan takes with rope_theta > 0
    if (a.rope_theta > 0.0) {
      k_select_attend<bf16_t, D, G, NSUB, 8, true><<<grid, kRowsThreads, 0, st>>>(s, a, p, w);
      return hipGetLastError();
    }
  }
  k_select_attend<bf16_t, D, G, NSUB, 8, false><<<grid, kRowsThreads, 0, st>>>(s, a, p, w);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_step_dg(const ScoreArgs& s, const AttendArgs& a, const StepPlan& p,
                                 const StepPtrs& w, hipStream_t st) {
  switch (p.units_per / kUnitsPerWG) {
    case 1: return launch_step_dgn<D, G, 1>(s, a, p, w, st);
    case 2: return launch_step_dgn<D, G, 2>(s, a, p, w, st);
    case 3: return launch_step_dgn<D, G, 3>(s, a, p, w, st);
    case 4: return launch_step_dgn<D, G, 4>(s, a, p, w, st);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_step_d(const ScoreArgs& s, const AttendArgs& a, const StepPlan& p,
                                const StepPtrs& w, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_step_dg<D, 1>(s, a, p, w, st);
    case 2: return launch_step_dg<D, 2>(s, a, p, w, st);
    case 4: return launch_step_dg<D, 4>(s, a, p, w, st);
    case 8: return launch_step_dg<D, 8>(s, a, p, w, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_select_attend(const ScoreArgs& s, AttendArgs a, const StepPlan& p,
                                const StepPtrs& w, hipStream_t st) {
  if (a.n_pos <= 0) return hipSuccess;
  a.ws_count = nullptr;   // the merge counts on the rows' sync ints
  return a.d == 128 ? launch_step_d<128>(s, a, p, w, st) : launch_step_d<64>(s, a, p, w, st);
}

}  // namespace infllm
