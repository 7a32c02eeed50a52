// Top-k_m selection over one row of unit scores: the search shared by the
// top-k kernels and by the scoring kernel's fused selection (InfLLM Guide,
// "Core Innovation 2", item 2: keep the k highest-scoring units).
//
// Scores become order-preserving 32-bit keys (0 for -inf, never kept).  The
// K-th largest key tau (K = min(k_m, #finite)) is found on the keys' bits,
// bit by bit by one wave (a candidate is kept when at least K keys reach
// it; the search stops once exactly K keys reach the candidate).  A
// workgroup first narrows the keys to those at or above a lower bound on
// tau and hands them to one wave (block_topk below), or, with too many
// candidates, searches 8 bits per pass with LDS histograms.  Keys above tau
// are kept, keys equal to tau fill the remaining slots lowest index first
// (ties go to the lower index).  Integer work on the fp32 scores: exact and
// deterministic.
//
// Layout: a wave owns a contiguous index range and lane l holds indices
// base + l + 64*i (one coalesced load per i).  Counts are ballots and
// popcounts; output slots come from mbcnt over the keep ballot, column by
// column, so the kept indices are written in ascending order without a scan.
#pragma once

#include "common.h"

namespace infllm {

__device__ __forceinline__ uint32_t score_key(float f) {
  return f > -INFINITY ? orderable(f) : 0u;
}

__device__ __forceinline__ int popc(uint64_t m) { return __builtin_popcountll(m); }
// lanes below this one whose bit is set in m
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// max / min over the wave: DPP within 16-lane rows, then the four rows'
// results through scalar registers
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t x) {
  auto pick = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  x = pick(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, INFLLM_DPP_XOR1, 0xF, 0xF, true));
  x = pick(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, INFLLM_DPP_XOR2, 0xF, 0xF, true));
  x = pick(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, INFLLM_DPP_HALF_MIRROR, 0xF, 0xF, true));
  x = pick(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, INFLLM_DPP_MIRROR, 0xF, 0xF, true));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return pick(pick(r0, r1), pick(r2, r3));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) { return wave_ext_u32<true>(x); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return wave_ext_u32<false>(x); }

// The keys of one wave's index range [base, base + 64*VPT) (clipped to U).
// VPT == 0: keys are re-read from memory at every use.  DEV: scores written
// by other workgroups of the same launch, read with device-scope loads.
template <int VPT, bool DEV = false>
struct WaveKeys {
  __device__ __forceinline__ static float ld(const float* p) { return DEV ? ld_dev(p) : *p; }
  uint32_t k[VPT > 0 ? VPT : 1];
  const float* s;
  int base, U, cols;   // cols: columns of 64 indices in the range
  __device__ __forceinline__ void init(const float* s_, int base_, int end, int U_) {
    s = s_;
    base = base_;
    U = U_;
    cols = (end - base + 63) / 64;
    end_ = end;
    if constexpr (VPT > 0) {
      // unconditional loads from clamped indices: all of them in flight at once
      const int lane = threadIdx.x % 64;
      float f[VPT];
      if (end > base) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
          const int u = base + lane + 64 * i;
          f[i] = ld(s + (u < end ? u : end - 1));
        }
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int u = base + lane + 64 * i;
        k[i] = end > base && u < end ? score_key(f[i]) : 0u;
      }
    }
  }
  int end_ = 0;
  __device__ __forceinline__ int n_cols() const { return VPT > 0 ? VPT : cols; }
  __device__ __forceinline__ uint32_t key(int i) const {
    if constexpr (VPT > 0) return k[i];
    const int u = base + threadIdx.x % 64 + 64 * i;   // only for columns of a non-empty range
    const float f = ld(s + (u < end_ ? u : end_ - 1));
    return u < end_ ? score_key(f) : 0u;
  }
  // number of keys >= c (c >= 1)
  __device__ __forceinline__ int count_ge(uint32_t c) const {
    int n = 0;
    if constexpr (VPT > 0) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) n += popc(__ballot(k[i] >= c));
    } else {
#pragma unroll 8
      for (int i = 0; i < cols; ++i) n += popc(__ballot(key(i) >= c));
    }
    return n;
  }
  // (finite keys, largest key, smallest finite key) of this wave
  __device__ __forceinline__ void stats(int& nv, uint32_t& hi, uint32_t& lo) const {
    nv = 0;
    uint32_t h = 0u, l = 0xffffffffu;
    for (int i = 0; i < n_cols(); ++i) {
      const uint32_t x = key(i);
      nv += popc(__ballot(x != 0u));
      h = x > h ? x : h;
      l = x != 0u && x < l ? x : l;
    }
    hi = wave_max_u32(h);
    lo = wave_min_u32(l);
  }
  // The maximum over each group of GL lanes' keys (every lane of a group
  // gets its group's value; 0 for an empty group).
  template <int GL>
  __device__ __forceinline__ uint32_t group_max() const {
    static_assert(GL == 4 || GL == 8 || GL == 16, "group of 4, 8 or 16 lanes");
    uint32_t h = 0u;
    for (int i = 0; i < n_cols(); ++i) {
      const uint32_t x = key(i);
      h = x > h ? x : h;
    }
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    h = mx(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, INFLLM_DPP_XOR1, 0xF, 0xF, true));
    h = mx(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, INFLLM_DPP_XOR2, 0xF, 0xF, true));
    if (GL >= 8)
      h = mx(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, INFLLM_DPP_HALF_MIRROR, 0xF, 0xF, true));
    if (GL >= 16)
      h = mx(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, INFLLM_DPP_MIRROR, 0xF, 0xF, true));
    return h;
  }
  // keys >= c of this wave
  __device__ __forceinline__ int count_ge_any(uint32_t c) const {
    int n = 0;
    for (int i = 0; i < n_cols(); ++i) n += popc(__ballot(key(i) >= c));
    return n;
  }
  // Keys >= c, with their indices, to ck/ci from slot `slot` on, in
  // ascending index order.
  __device__ __forceinline__ void compact_ge(uint32_t c, int slot, uint32_t* ck, int* ci) const {
    const int lane = threadIdx.x % 64;
    for (int i = 0; i < n_cols(); ++i) {
      const uint32_t x = key(i);
      const uint64_t m = __ballot(x >= c);
      if (x >= c) {
        const int j = slot + lanes_below(m);
        ck[j] = x;
        ci[j] = base + lane + 64 * i;
      }
      slot += popc(m);
    }
  }
  // smallest key >= c (c >= 1)
  __device__ __forceinline__ uint32_t min_ge(uint32_t c) const {
    uint32_t l = 0xffffffffu;
    for (int i = 0; i < n_cols(); ++i) {
      const uint32_t x = key(i);
      l = x >= c && x < l ? x : l;
    }
    return wave_min_u32(l);
  }
  // (keys > tau, keys == tau) of this wave
  __device__ __forceinline__ void split(uint32_t tau, int& n_gt, int& n_eq) const {
    n_gt = n_eq = 0;
    for (int i = 0; i < n_cols(); ++i) {
      const uint32_t x = key(i);
      n_gt += popc(__ballot(x > tau));
      n_eq += popc(__ballot(x == tau));
    }
  }
  // Write kept indices in ascending order from out[slot]: keys above tau,
  // and keys equal to tau whose rank among ties (from tie_rank) is < rem.
  __device__ __forceinline__ void emit(uint32_t tau, int rem, int tie_rank, int slot,
                                       int32_t* out) const {
    const int lane = threadIdx.x % 64;
    for (int i = 0; i < n_cols(); ++i) {
      const uint32_t x = key(i);
      const uint64_t eq = __ballot(x == tau);
      const bool keep = x > tau || (x == tau && tie_rank + lanes_below(eq) < rem);
      const uint64_t kb = __ballot(keep);
      if (keep) out[slot + lanes_below(kb)] = base + lane + 64 * i;
      slot += popc(kb);
      tie_rank += popc(eq);
    }
  }
};

// Threshold search on one wave's keys when the wave holds the whole
// problem; Sum(x) adds a per-wave count over the problem's waves.
template <typename Keys, typename Sum, typename MinAll>
__device__ __forceinline__ uint32_t find_tau(const Keys& keys, int K, int n_valid, uint32_t hi,
                                             uint32_t lo, Sum sum, MinAll min_all) {
  if (K == n_valid || hi == lo) return lo;       // every finite key is kept, or all equal
  const uint32_t diff = hi ^ lo;
  const int top = 31 - __builtin_clz(diff);      // highest bit where keys can differ
  uint32_t tau = top == 31 ? 0u : hi & ~((2u << top) - 1u);
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    const int c = sum(keys.count_ge(cand));
    if (c >= K) {
      tau = cand;
      if (c == K) return min_all(keys.min_ge(tau));   // exactly the top K reach cand
    }
  }
  return tau;
}

// Radix form of the same search, for a workgroup: 8 bits of the threshold
// per pass instead of one.  Among the keys that share the bits above `top`
// with the threshold found so far, an LDS histogram of the next 8 bits
// gives the digit that holds the krem-th largest key; krem then becomes its
// rank inside that digit.  Three barriers per pass, at most four passes
// (fewer after skipping the common leading bits of the largest and
// smallest finite key).
constexpr int kRadixBins = 256;
// lb: a lower bound on the K-th largest key (the smallest finite key, or a
// tighter bound); only the bits where hi and lb differ are searched.
template <typename Keys>
__device__ __forceinline__ uint32_t radix_tau(const Keys& keys, int K, int n_valid, uint32_t hi,
                                              uint32_t lo, uint32_t lb, int* hist, int* pick) {
  if (K == n_valid) return lo;                   // every finite key is kept
  if (hi == lb) return hi;                       // K keys at the maximum
  const int tid = threadIdx.x, lane = tid % 64;
  int top = 31 - __builtin_clz(hi ^ lb);         // highest bit where hi and the bound differ
  uint32_t prefix = top == 31 ? 0u : hi & ~((2u << top) - 1u);
  int krem = K;
  while (top >= 0) {
    const int shift = top >= 7 ? top - 7 : 0;
    const uint32_t dmask = (2u << (top - shift)) - 1u;
    for (int i = tid; i < kRadixBins; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = 0; i < keys.n_cols(); ++i) {
      const uint32_t x = keys.key(i);
      const bool in = x != 0u && (top == 31 || (x >> (top + 1)) == (prefix >> (top + 1)));
      if (in) atomicAdd(&hist[(x >> shift) & dmask], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 4l .. 4l+3; keys above a bin = later bins
      int h[4], own = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[j] = hist[4 * lane + j];
        own += h[j];
      }
      int suf = own;   // inclusive suffix sum over lanes lane .. 63
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int y = __shfl_down(suf, m);
        if (lane + m < 64) suf += y;
      }
      int above = suf - own;   // keys in the bins of later lanes
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < krem && above + h[j] >= krem) {
          pick[0] = 4 * lane + j;
          pick[1] = above;
        }
        above += h[j];
      }
    }
    __syncthreads();
    const int d = pick[0];
    krem -= pick[1];
    prefix |= (uint32_t)d << shift;
    top = shift - 1;
  }
  return prefix;
}

// The candidates of a workgroup search (at most kCand, compacted in LDS in
// ascending index order), loaded into one wave's registers, with the
// interface find_tau expects.
constexpr int kCand = 256;
struct CandKeys {
  static constexpr int kCols = kCand / 64;
  uint32_t k[kCols];
  int idx[kCols];
  __device__ __forceinline__ void load(const uint32_t* ck, const int* ci, int n) {
    const int lane = threadIdx.x % 64;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
      const int j = lane + 64 * i;
      k[i] = j < n ? ck[j] : 0u;
      idx[i] = j < n ? ci[j] : -1;
    }
  }
  __device__ __forceinline__ int count_ge(uint32_t c) const {
    int m = 0;
#pragma unroll
    for (int i = 0; i < kCols; ++i) m += popc(__ballot(k[i] >= c));
    return m;
  }
  __device__ __forceinline__ uint32_t min_ge(uint32_t c) const {
    uint32_t l = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < kCols; ++i) l = k[i] >= c && k[i] < l ? k[i] : l;
    return wave_min_u32(l);
  }
  // keys above tau, then keys equal to tau lowest index first, K in all
  __device__ __forceinline__ void emit(uint32_t tau, int K, int32_t* out) const {
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < kCols; ++i) n_gt += popc(__ballot(k[i] > tau));
    const int rem = K - n_gt;
    int slot = 0, tie_rank = 0;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
      const uint64_t eq = __ballot(k[i] == tau);
      const bool keep = k[i] > tau || (k[i] == tau && tie_rank + lanes_below(eq) < rem);
      const uint64_t kb = __ballot(keep);
      if (keep) out[slot + lanes_below(kb)] = idx[i];
      slot += popc(kb);
      tie_rank += popc(eq);
    }
  }
};

// -------------------------------------------------------- workgroup variant
// NW waves per problem; wave w owns indices [w*R, (w+1)*R), R a multiple of
// 64.  Per-wave values meet in LDS, double-buffered: one barrier per
// exchange.
//
// The search narrows the keys before it looks for the threshold: the keys
// are cut into 64 groups (NW lanes of one wave each) whose maxima are
// distinct keys, so the K-th largest group maximum is at or below the K-th
// largest key.  Only keys at or above it can be kept: usually a few times
// K of them.  They are compacted into LDS in index order and one wave finds
// the threshold among them bit by bit and writes the selection.  With more
// than kCand candidates, the radix search runs over all keys from that
// bound instead.
struct TopkShared {
  uint32_t xch[2][5][16];
  int hist[kRadixBins];
  int pick[2];
  uint32_t gmax[64];
  uint32_t ck[kCand];
  int ci[kCand];
};

template <int NW, int VPT, bool DEV>
__device__ __forceinline__ void block_topk(const float* __restrict__ row, int U, int k_m,
                                           int32_t* __restrict__ out, TopkShared& sm) {
  static_assert(NW == 4 || NW == 8 || NW == 16, "4, 8 or 16 waves");
  constexpr int kGroupsPerWave = 64 / NW;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int R = ((U + NW - 1) / NW + 63) / 64 * 64;
  const int b0 = wave * R < U ? wave * R : U;
  const int b1 = b0 + R < U ? b0 + R : U;
  int phase = 0;
  // all-reduce of one value per wave (sum, max or min)
  auto exchange = [&](uint32_t v, int slot) {
    if (lane == 0) sm.xch[phase][slot][wave] = v;
  };
  auto sync = [&]() {
    __syncthreads();
    phase ^= 1;
  };
  auto got = [&](int slot, int w) { return sm.xch[phase ^ 1][slot][w]; };

  WaveKeys<VPT, DEV> keys;
  keys.init(row, b0, b1, U);
  int nv_w;
  uint32_t hi_w, lo_w;
  keys.stats(nv_w, hi_w, lo_w);
  const uint32_t gm = keys.template group_max<NW>();
  if (lane % NW == 0) sm.gmax[wave * kGroupsPerWave + lane / NW] = gm;
  exchange((uint32_t)nv_w, 0);
  exchange(hi_w, 1);
  exchange(lo_w, 2);
  sync();
  int n_valid = 0;
  uint32_t hi = 0u, lo = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    n_valid += (int)got(0, w);
    hi = got(1, w) > hi ? got(1, w) : hi;
    lo = got(2, w) < lo ? got(2, w) : lo;
  }
  const int K = k_m < n_valid ? k_m : n_valid;
  if (K > 0) {
    // the K-th largest group maximum (every wave finds it; one key per lane)
    uint32_t lb = lo;
    {
      const uint32_t x = sm.gmax[lane];
      if (popc(__ballot(x != 0u)) >= K) {
        uint32_t t = 0u;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = t | (1u << bit);
          if (popc(__ballot(x >= cand)) >= K) t = cand;
        }
        lb = t;
      }
    }
    exchange((uint32_t)keys.count_ge_any(lb), 3);
    sync();
    int n_cand = 0, before = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      before += w < wave ? (int)got(3, w) : 0;
      n_cand += (int)got(3, w);
    }
    if (n_cand <= kCand) {
      keys.compact_ge(lb, before, sm.ck, sm.ci);
      __syncthreads();
      if (wave == 0) {
        CandKeys cand;
        cand.load(sm.ck, sm.ci, n_cand);
        const uint32_t tau = find_tau(cand, K, n_cand, hi, lb, [](int c) { return c; },
                                      [](uint32_t m) { return m; });
        cand.emit(tau, K, out);
      }
    } else {
      const uint32_t tau = radix_tau(keys, K, n_valid, hi, lo, lb, sm.hist, sm.pick);
      int n_gt, n_eq;
      keys.split(tau, n_gt, n_eq);
      exchange((uint32_t)n_gt, 0);
      exchange((uint32_t)n_eq, 1);
      sync();
      int gt_all = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) gt_all += (int)got(0, w);
      const int rem = K - gt_all;                // ties kept, lowest indices first
      int slot = 0, tie_rank = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (w >= wave) break;
        const int eq_w = (int)got(1, w);
        const int kept_eq = rem - tie_rank < 0 ? 0 : (rem - tie_rank < eq_w ? rem - tie_rank : eq_w);
        slot += (int)got(0, w) + kept_eq;
        tie_rank += eq_w;
      }
      keys.emit(tau, rem, tie_rank, slot, out);
    }
  }
  for (int m = K + tid; m < k_m; m += NW * 64) out[m] = -1;
}

}  // namespace infllm
