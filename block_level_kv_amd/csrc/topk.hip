// Top-k_m unit selection per (sequence, KV head, chunk) (InfLLM Guide,
// "Core Innovation 2", item 2: keep the k highest-scoring units).
//
// Scores become order-preserving 32-bit keys (0 for -inf, never kept).  The
// K-th largest key tau (K = min(k_m, #finite)) is found bit by bit from the
// top: a candidate threshold is kept when at least K keys reach it.  Each of
// the 32 rounds is compares plus one reduction -- no histograms, so keys
// that share their exponent bits cost nothing extra.  Keys above tau are
// kept, and keys equal to tau fill the remaining slots lowest index first
// (ties go to the lower index).  Each thread owns a contiguous run of
// indices, so one exclusive scan of per-thread counts orders the output.
// Everything is integer work on the fp32 scores: exact and deterministic.
//
// U <= 64*32: one wave per problem (four problems per workgroup), keys in
// registers, lane scans.  Larger U: one workgroup per problem, keys in
// registers up to 256*64, one barrier per round.
#include "common.h"
#include "kernels.h"

namespace infllm {

constexpr int kTopkThreads = 256;

__device__ __forceinline__ uint32_t score_key(float f) {
  return f > -INFINITY ? orderable(f) : 0u;
}

// Sum over the wave: DPP all-reduce inside each 16-lane row, then the four
// row sums read into scalar registers (no LDS-permute round trips).
__device__ __forceinline__ int wave_sum_i32(int x) {
  x += __builtin_amdgcn_mov_dpp(x, INFLLM_DPP_XOR1, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, INFLLM_DPP_XOR2, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, INFLLM_DPP_HALF_MIRROR, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, INFLLM_DPP_MIRROR, 0xF, 0xF, true);
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

__device__ __forceinline__ int wave_excl_scan(int x, int lane) {
  int v = x;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int y = __shfl_up(v, m);
    if (lane >= m) v += y;
  }
  return v - x;
}

// ------------------------------------------------------------- wave variant
template <int VPT>
__global__ __launch_bounds__(kTopkThreads) void k_topk_wave(const float* __restrict__ scores,
                                                            int64_t problems, int U, int k_m,
                                                            int32_t* __restrict__ sel) {
  const int lane = threadIdx.x % 64;
  const int64_t prob = (int64_t)blockIdx.x * (kTopkThreads / 64) + threadIdx.x / 64;
  if (prob >= problems) return;              // the whole wave leaves together
  const float* s = scores + prob * U;
  int32_t* out = sel + prob * k_m;
  const int u0 = lane * VPT;                 // this lane's indices u0 .. u0+VPT-1

  uint32_t key[VPT];
  int nv = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    key[i] = u0 + i < U ? score_key(s[u0 + i]) : 0u;
    nv += key[i] != 0u;
  }
  const int n_valid = wave_sum_i32(nv);
  const int K = k_m < n_valid ? k_m : n_valid;

  uint32_t tau = 0;
  if (K > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < VPT; ++i) c += key[i] >= cand;
      if (wave_sum_i32(c) >= K) tau = cand;
    }
  }
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    n_gt += K > 0 && key[i] > tau;
    n_eq += K > 0 && key[i] == tau;
  }
  const int rem = K - wave_sum_i32(n_gt);     // keys equal to tau that are kept
  int eq_rank = wave_excl_scan(n_eq, lane);
  int kept = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const bool keep = K > 0 && (key[i] > tau || (key[i] == tau && eq_rank++ < rem));
    kept += keep;
  }
  int slot = wave_excl_scan(kept, lane);
  eq_rank = wave_excl_scan(n_eq, lane);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const bool keep = K > 0 && (key[i] > tau || (key[i] == tau && eq_rank++ < rem));
    if (keep) out[slot++] = u0 + i;
  }
  for (int m = K + lane; m < k_m; m += 64) out[m] = -1;
}

// -------------------------------------------------------- workgroup variant
// Block reduction with double-buffered wave partials: one barrier per call.
struct BlockSum {
  int* buf;    // [2][kTopkThreads / 64]
  int phase;
  __device__ __forceinline__ int operator()(int x) {
    x = wave_sum_i32(x);
    int* b = buf + phase * (kTopkThreads / 64);
    if (threadIdx.x % 64 == 0) b[threadIdx.x / 64] = x;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kTopkThreads / 64; ++w) t += b[w];
    phase ^= 1;
    return t;
  }
};

// exclusive scan over the workgroup (two barriers)
__device__ __forceinline__ int block_excl_scan(int x, int* wave_tot) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int e = wave_excl_scan(x, lane);
  if (lane == 63) wave_tot[wave] = e + x;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) before += w < wave ? wave_tot[w] : 0;
  __syncthreads();
  return before + e;
}

// VPT > 0: thread t's keys (indices t*VPT ..) in registers; VPT == 0: the
// generic path re-reads scores from global memory every round.
template <int VPT>
__global__ __launch_bounds__(kTopkThreads) void k_topk_block(const float* __restrict__ scores,
                                                             int U, int k_m,
                                                             int32_t* __restrict__ sel) {
  const int64_t prob = blockIdx.x;
  const float* s = scores + prob * U;
  int32_t* out = sel + prob * k_m;
  const int tid = threadIdx.x;
  __shared__ int red_buf[2 * (kTopkThreads / 64)];
  __shared__ int scan_buf[kTopkThreads / 64];
  BlockSum bsum{red_buf, 0};
  const int per = VPT > 0 ? VPT : (U + kTopkThreads - 1) / kTopkThreads;
  const int u0 = tid * per;

  uint32_t kreg[VPT > 0 ? VPT : 1];
  if constexpr (VPT > 0) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) kreg[i] = u0 + i < U ? score_key(s[u0 + i]) : 0u;
  }
  auto key_of = [&](int i) -> uint32_t {
    if constexpr (VPT > 0) return kreg[i];
    return u0 + i < U ? score_key(s[u0 + i]) : 0u;
  };

  int nv = 0;
  for (int i = 0; i < per; ++i) nv += key_of(i) != 0u;
  const int n_valid = bsum(nv);
  const int K = k_m < n_valid ? k_m : n_valid;
  uint32_t tau = 0;
  if (K > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int c = 0;
      for (int i = 0; i < per; ++i) c += key_of(i) >= cand;
      if (bsum(c) >= K) tau = cand;
    }
  }
  int n_gt = 0, n_eq = 0;
  for (int i = 0; i < per; ++i) {
    const uint32_t k = key_of(i);
    n_gt += K > 0 && k > tau;
    n_eq += K > 0 && k == tau;
  }
  const int rem = K - bsum(n_gt);
  int eq_rank = block_excl_scan(n_eq, scan_buf);
  const int eq0 = eq_rank;
  int kept = 0;
  for (int i = 0; i < per; ++i) {
    const uint32_t k = key_of(i);
    kept += K > 0 && (k > tau || (k == tau && eq_rank++ < rem));
  }
  int slot = block_excl_scan(kept, scan_buf);
  eq_rank = eq0;
  for (int i = 0; i < per; ++i) {
    const uint32_t k = key_of(i);
    if (K > 0 && (k > tau || (k == tau && eq_rank++ < rem))) out[slot++] = u0 + i;
  }
  for (int m = K + tid; m < k_m; m += kTopkThreads) out[m] = -1;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int64_t problems = (int64_t)a.batch * a.Hkv * a.n_chunks;
  if (problems <= 0 || a.k_m <= 0) return hipSuccess;
  const int wslots = (a.U + 63) / 64;
  if (wslots <= 32) {
    const dim3 wgrid((unsigned)((problems + 3) / 4));
    if (wslots <= 4)
      k_topk_wave<4><<<wgrid, kTopkThreads, 0, st>>>(a.scores, problems, a.U, a.k_m, a.sel);
    else if (wslots <= 16)
      k_topk_wave<16><<<wgrid, kTopkThreads, 0, st>>>(a.scores, problems, a.U, a.k_m, a.sel);
    else
      k_topk_wave<32><<<wgrid, kTopkThreads, 0, st>>>(a.scores, problems, a.U, a.k_m, a.sel);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)problems);
  const int slots = (a.U + kTopkThreads - 1) / kTopkThreads;
  if (slots <= 16) k_topk_block<16><<<grid, kTopkThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else if (slots <= 32) k_topk_block<32><<<grid, kTopkThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else if (slots <= 64) k_topk_block<64><<<grid, kTopkThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else k_topk_block<0><<<grid, kTopkThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  return hipGetLastError();
}

}  // namespace infllm
