// Top-k_m unit selection per (sequence, KV head, chunk) (InfLLM Guide,
// "Core Innovation 2", item 2: keep the k highest-scoring units).
//
// Scores become order-preserving 32-bit keys (0 for -inf, never kept).  The
// K-th largest key tau (K = min(k_m, #finite)) is found bit by bit: a
// candidate threshold is kept when at least K keys reach it.  The search
// starts below the common leading bits of the largest and the smallest
// finite key, and stops early once exactly K keys reach the threshold (tau
// is then the smallest of them).  Keys above tau are kept, and keys equal
// to tau fill the remaining slots lowest index first (ties go to the lower
// index).  Everything is integer work on the fp32 scores: exact and
// deterministic.
//
// Layout: a wave owns a contiguous index range and lane l holds indices
// base + l + 64*i (one coalesced load per i).  Counts are ballots and
// popcounts (scalar, no cross-lane reduction); output slots come from
// mbcnt over the keep ballot, column by column, so the kept indices are
// written in ascending order without a scan.
//
// U <= 64*32: one wave per problem (four problems per workgroup).  Larger
// U: one workgroup of four waves per problem, one barrier per round; keys
// in registers up to 4*64*64 units, beyond that re-read every round.
#include "common.h"
#include "kernels.h"

namespace infllm {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / 64;

__device__ __forceinline__ uint32_t score_key(float f) {
  return f > -INFINITY ? orderable(f) : 0u;
}

__device__ __forceinline__ int popc(uint64_t m) { return __builtin_popcountll(m); }
// lanes below this one whose bit is set in m
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)x, m);
    x = y > x ? y : x;
  }
  return x;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)x, m);
    x = y < x ? y : x;
  }
  return x;
}

// The keys of one wave's index range [base, base + 64*VPT) (clipped to U).
// VPT == 0: keys are re-read from memory at every use.
template <int VPT>
struct WaveKeys {
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
          f[i] = s[u < end ? u : end - 1];
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
    const float f = s[u < end_ ? u : end_ - 1];
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

// ------------------------------------------------------------- wave variant
template <int VPT>
__global__ __launch_bounds__(kTopkThreads) void k_topk_wave(const float* __restrict__ scores,
                                                            int64_t problems, int U, int k_m,
                                                            int32_t* __restrict__ sel) {
  const int lane = threadIdx.x % 64;
  const int64_t prob = (int64_t)blockIdx.x * kTopkWaves + threadIdx.x / 64;
  if (prob >= problems) return;              // the whole wave leaves together
  int32_t* out = sel + prob * k_m;
  WaveKeys<VPT> keys;
  keys.init(scores + prob * U, 0, U, U);
  int n_valid;
  uint32_t hi, lo;
  keys.stats(n_valid, hi, lo);
  const int K = k_m < n_valid ? k_m : n_valid;
  if (K > 0) {
    const uint32_t tau = find_tau(keys, K, n_valid, hi, lo, [](int c) { return c; },
                                  [](uint32_t m) { return m; });
    int n_gt, n_eq;
    keys.split(tau, n_gt, n_eq);
    keys.emit(tau, K - n_gt, 0, 0, out);
  }
  for (int m = K + lane; m < k_m; m += 64) out[m] = -1;
}

// -------------------------------------------------------- workgroup variant
// Wave w owns indices [w*R, (w+1)*R), R a multiple of 64.  Per-wave values
// meet in LDS, double-buffered: one barrier per exchange.
template <int VPT>
__global__ __launch_bounds__(kTopkThreads) void k_topk_block(const float* __restrict__ scores,
                                                             int U, int k_m,
                                                             int32_t* __restrict__ sel) {
  const int64_t prob = blockIdx.x;
  int32_t* out = sel + prob * k_m;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int R = ((U + kTopkWaves - 1) / kTopkWaves + 63) / 64 * 64;
  const int b0 = wave * R < U ? wave * R : U;
  const int b1 = b0 + R < U ? b0 + R : U;
  __shared__ uint32_t xch[2][3][kTopkWaves];
  int phase = 0;
  // all-reduce of one value per wave (sum, max or min)
  auto exchange = [&](uint32_t v, int slot) {
    if (lane == 0) xch[phase][slot][wave] = v;
  };
  auto sync = [&]() {
    __syncthreads();
    phase ^= 1;
  };
  auto got = [&](int slot, int w) { return xch[phase ^ 1][slot][w]; };

  WaveKeys<VPT> keys;
  keys.init(scores + prob * U, b0, b1, U);
  int nv_w;
  uint32_t hi_w, lo_w;
  keys.stats(nv_w, hi_w, lo_w);
  exchange((uint32_t)nv_w, 0);
  exchange(hi_w, 1);
  exchange(lo_w, 2);
  sync();
  int n_valid = 0;
  uint32_t hi = 0u, lo = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    n_valid += (int)got(0, w);
    hi = got(1, w) > hi ? got(1, w) : hi;
    lo = got(2, w) < lo ? got(2, w) : lo;
  }
  const int K = k_m < n_valid ? k_m : n_valid;
  if (K > 0) {
    auto sum = [&](int c) {
      exchange((uint32_t)c, 0);
      sync();
      int t = 0;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) t += (int)got(0, w);
      return t;
    };
    auto min_all = [&](uint32_t m) {
      exchange(m, 0);
      sync();
      uint32_t t = 0xffffffffu;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) t = got(0, w) < t ? got(0, w) : t;
      return t;
    };
    const uint32_t tau = find_tau(keys, K, n_valid, hi, lo, sum, min_all);
    int n_gt, n_eq;
    keys.split(tau, n_gt, n_eq);
    exchange((uint32_t)n_gt, 0);
    exchange((uint32_t)n_eq, 1);
    sync();
    int gt_all = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) gt_all += (int)got(0, w);
    const int rem = K - gt_all;                // ties kept, lowest indices first
    int slot = 0, tie_rank = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      if (w >= wave) break;
      const int eq_w = (int)got(1, w);
      const int kept_eq = rem - tie_rank < 0 ? 0 : (rem - tie_rank < eq_w ? rem - tie_rank : eq_w);
      slot += (int)got(0, w) + kept_eq;
      tie_rank += eq_w;
    }
    keys.emit(tau, rem, tie_rank, slot, out);
  }
  for (int m = K + tid; m < k_m; m += kTopkThreads) out[m] = -1;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int64_t problems = (int64_t)a.batch * a.Hkv * a.n_chunks;
  if (problems <= 0 || a.k_m <= 0) return hipSuccess;
  const int cols = (a.U + 63) / 64;
  if (cols <= 32) {
    const dim3 wgrid((unsigned)((problems + kTopkWaves - 1) / kTopkWaves));
    if (cols <= 4)
      k_topk_wave<4><<<wgrid, kTopkThreads, 0, st>>>(a.scores, problems, a.U, a.k_m, a.sel);
    else if (cols <= 16)
      k_topk_wave<16><<<wgrid, kTopkThreads, 0, st>>>(a.scores, problems, a.U, a.k_m, a.sel);
    else
      k_topk_wave<32><<<wgrid, kTopkThreads, 0, st>>>(a.scores, problems, a.U, a.k_m, a.sel);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)problems);
  const int wcols = (cols + kTopkWaves - 1) / kTopkWaves;   // columns per wave
  if (wcols <= 16) k_topk_block<16><<<grid, kTopkThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else if (wcols <= 32) k_topk_block<32><<<grid, kTopkThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else if (wcols <= 64) k_topk_block<64><<<grid, kTopkThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else k_topk_block<0><<<grid, kTopkThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  return hipGetLastError();
}

}  // namespace infllm
