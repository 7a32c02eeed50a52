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
// Up to 256 units (or up to 2,048 with many problems): one wave per
// problem, four problems per workgroup, the bit-by-bit search.  Otherwise
// one workgroup of 16 waves per problem and a radix search (8 bits per
// pass, LDS histograms); keys in registers up to 16*64*32 units, beyond
// that re-read every pass.
#include "common.h"
#include "kernels.h"

namespace infllm {

constexpr int kTopkThreads = 256;                  // wave variant: 4 problems per workgroup
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBlockThreads = 1024;                // workgroup variant: 16 waves per problem
constexpr int kBlockWaves = kBlockThreads / 64;

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
  // A lower bound on the K-th largest key from this wave's four 16-lane
  // rows: their maxima are distinct keys, so with `rows` nonempty rows
  // (summed over the problem's waves) >= K, the smallest row maximum is at
  // or below the K-th largest key.  Empty rows give (0 rows, ~0u).
  __device__ __forceinline__ void row_bound(int& rows, uint32_t& lb) const {
    uint32_t h = 0u;
    for (int i = 0; i < n_cols(); ++i) {
      const uint32_t x = key(i);
      h = x > h ? x : h;
    }
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    h = mx(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, INFLLM_DPP_XOR1, 0xF, 0xF, true));
    h = mx(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, INFLLM_DPP_XOR2, 0xF, 0xF, true));
    h = mx(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, INFLLM_DPP_HALF_MIRROR, 0xF, 0xF, true));
    h = mx(h, (uint32_t)__builtin_amdgcn_mov_dpp((int)h, INFLLM_DPP_MIRROR, 0xF, 0xF, true));
    rows = 0;
    lb = 0xffffffffu;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)h, 16 * r);
      rows += m != 0u;
      lb = m != 0u && m < lb ? m : lb;
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

// -------------------------------------------------------- workgroup variant
// Wave w owns indices [w*R, (w+1)*R), R a multiple of 64.  Per-wave values
// meet in LDS, double-buffered: one barrier per exchange; the threshold
// comes from the radix search.
template <int VPT>
__global__ __launch_bounds__(kBlockThreads) void k_topk_block(const float* __restrict__ scores,
                                                             int U, int k_m,
                                                             int32_t* __restrict__ sel) {
  const int64_t prob = blockIdx.x;
  int32_t* out = sel + prob * k_m;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int R = ((U + kBlockWaves - 1) / kBlockWaves + 63) / 64 * 64;
  const int b0 = wave * R < U ? wave * R : U;
  const int b1 = b0 + R < U ? b0 + R : U;
  __shared__ uint32_t xch[2][5][kBlockWaves];
  __shared__ int hist[kRadixBins];
  __shared__ int pick[2];
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
  int rows_w;
  uint32_t lb_w;
  keys.row_bound(rows_w, lb_w);
  exchange((uint32_t)nv_w, 0);
  exchange(hi_w, 1);
  exchange(lo_w, 2);
  exchange((uint32_t)rows_w, 3);
  exchange(lb_w, 4);
  sync();
  int n_valid = 0, rows = 0;
  uint32_t hi = 0u, lo = 0xffffffffu, lb = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < kBlockWaves; ++w) {
    n_valid += (int)got(0, w);
    hi = got(1, w) > hi ? got(1, w) : hi;
    lo = got(2, w) < lo ? got(2, w) : lo;
    rows += (int)got(3, w);
    lb = got(4, w) < lb ? got(4, w) : lb;
  }
  const int K = k_m < n_valid ? k_m : n_valid;
  if (K > 0) {
    const uint32_t tau = radix_tau(keys, K, n_valid, hi, lo, rows >= K ? lb : lo, hist, pick);
    int n_gt, n_eq;
    keys.split(tau, n_gt, n_eq);
    exchange((uint32_t)n_gt, 0);
    exchange((uint32_t)n_eq, 1);
    sync();
    int gt_all = 0;
#pragma unroll
    for (int w = 0; w < kBlockWaves; ++w) gt_all += (int)got(0, w);
    const int rem = K - gt_all;                // ties kept, lowest indices first
    int slot = 0, tie_rank = 0;
#pragma unroll
    for (int w = 0; w < kBlockWaves; ++w) {
      if (w >= wave) break;
      const int eq_w = (int)got(1, w);
      const int kept_eq = rem - tie_rank < 0 ? 0 : (rem - tie_rank < eq_w ? rem - tie_rank : eq_w);
      slot += (int)got(0, w) + kept_eq;
      tie_rank += eq_w;
    }
    keys.emit(tau, rem, tie_rank, slot, out);
  }
  for (int m = K + tid; m < k_m; m += kBlockThreads) out[m] = -1;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int64_t problems = (int64_t)a.batch * a.Hkv * a.n_chunks;
  if (problems <= 0 || a.k_m <= 0) return hipSuccess;
  const int cols = (a.U + 63) / 64;
  // few columns: a wave per problem; more: a workgroup of 16 waves (each
  // threshold round then costs one ballot column or a few per wave)
  if (cols <= 4 || (cols <= 32 && problems >= 1024)) {
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
  const int wcols = (cols + kBlockWaves - 1) / kBlockWaves;   // columns per wave
  if (wcols <= 2) k_topk_block<2><<<grid, kBlockThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else if (wcols <= 8) k_topk_block<8><<<grid, kBlockThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else if (wcols <= 32) k_topk_block<32><<<grid, kBlockThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else k_topk_block<0><<<grid, kBlockThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  return hipGetLastError();
}

}  // namespace infllm
