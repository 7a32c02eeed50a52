// Top-k_m unit selection kernels, one problem per (sequence, KV head,
// chunk) (InfLLM Guide, "Core Innovation 2", item 2: keep the k highest-
// scoring units); the search itself is in topk_select.h.
//
// Up to 256 units (or up to 2,048 with many problems): one wave per
// problem, four problems per workgroup, the bit-by-bit search.  Otherwise
// one workgroup of 16 waves per problem and the workgroup search (the keys
// above a lower bound compacted and searched by one wave; radix passes over
// all keys past 256 candidates); keys in registers up to 16*64*32 units,
// beyond that re-read at every use.
#include "kernels.h"
#include "topk_select.h"

namespace infllm {

constexpr int kTopkThreads = 256;                  // wave variant: 4 problems per workgroup
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBlockThreads = 1024;                // workgroup variant: 16 waves per problem
constexpr int kBlockWaves = kBlockThreads / 64;

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
template <int VPT>
__global__ __launch_bounds__(kBlockThreads) void k_topk_block(const float* __restrict__ scores,
                                                             int U, int k_m,
                                                             int32_t* __restrict__ sel) {
  __shared__ TopkShared sm;
  const int64_t prob = blockIdx.x;
  block_topk<kBlockWaves, VPT, false>(scores + prob * U, U, k_m, sel + prob * k_m, sm);
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
  else if (wcols <= 16) k_topk_block<16><<<grid, kBlockThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else if (wcols <= 32) k_topk_block<32><<<grid, kBlockThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  else k_topk_block<0><<<grid, kBlockThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  return hipGetLastError();
}

}  // namespace infllm
