// Top-k_m unit selection per (sequence, KV head, chunk) (InfLLM Guide,
// "Core Innovation 2", item 2: keep the k highest-scoring units).
//
// One workgroup per problem.  A 4-pass radix select over order-preserving
// 32-bit keys finds the k-th largest finite score tau; units scoring above
// tau are kept, and among units equal to tau the lowest indices fill the
// remaining slots (ties go to the lower index).  A block-wide ordered scan
// then writes the kept indices in ascending order.  Every step is integer
// work on the fp32 scores, so the result is exact and deterministic.
#include "common.h"
#include "kernels.h"

namespace infllm {

constexpr int kTopkThreads = 256;

// Inclusive scan over the workgroup (256 threads); returns this thread's
// inclusive prefix and stores the total in *total.
__device__ __forceinline__ int block_scan_incl(int x, int* total, int* wave_sums) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    int y = __shfl_up(x, m);
    if (lane >= m) x += y;
  }
  if (lane == 63) wave_sums[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const int s = wave_sums[w];
    before += w < wave ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return x + before;
}

__device__ __forceinline__ bool finite_score(float s) { return s > -INFINITY; }

__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ scores, int U,
                                                       int k_m, int32_t* __restrict__ sel) {
  const int64_t prob = blockIdx.x;
  const float* s = scores + prob * U;
  int32_t* out = sel + prob * k_m;
  const int tid = threadIdx.x;
  __shared__ int hist[256];
  __shared__ int wave_sums[kTopkThreads / 64];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_rem;

  // number of finite scores
  int nv = 0;
  for (int u = tid; u < U; u += kTopkThreads) nv += finite_score(s[u]);
  int n_valid;
  block_scan_incl(nv, &n_valid, wave_sums);
  const int K = k_m < n_valid ? k_m : n_valid;

  uint32_t prefix = 0, mask = 0;
  int rem = K;
  if (K > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int u = tid; u < U; u += kTopkThreads) {
        const float f = s[u];
        if (!finite_score(f)) continue;
        const uint32_t key = orderable(f);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      // suffix counts: thread t looks at bin 255 - t
      const int bin = 255 - tid;
      const int cnt = hist[bin];
      int dummy;
      const int incl = block_scan_incl(cnt, &dummy, wave_sums);  // keys in bins >= bin
      if (incl >= rem && incl - cnt < rem) {
        sh_prefix = prefix | ((uint32_t)bin << shift);
        sh_rem = rem - (incl - cnt);
      }
      __syncthreads();
      prefix = sh_prefix;
      rem = sh_rem;
      mask |= 255u << shift;
      __syncthreads();
    }
  }
  const uint32_t tau = prefix;  // exact key of the K-th best score
  // rem = how many keys equal to tau are kept (lowest indices first)

  int eq_before = 0, kept_before = 0;
  for (int base = 0; base < U; base += kTopkThreads) {
    const int u = base + tid;
    bool valid = false, eq = false, gt = false;
    if (u < U && K > 0) {
      const float f = s[u];
      valid = finite_score(f);
      const uint32_t key = valid ? orderable(f) : 0u;
      gt = valid && key > tau;
      eq = valid && key == tau;
    }
    int eq_tot;
    const int eq_incl = block_scan_incl(eq ? 1 : 0, &eq_tot, wave_sums);
    const bool keep = gt || (eq && eq_before + eq_incl - 1 < rem);
    int kept_tot;
    const int kept_incl = block_scan_incl(keep ? 1 : 0, &kept_tot, wave_sums);
    if (keep) out[kept_before + kept_incl - 1] = u;
    eq_before += eq_tot;
    kept_before += kept_tot;
  }
  for (int m = K + tid; m < k_m; m += kTopkThreads) out[m] = -1;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int64_t problems = (int64_t)a.batch * a.Hkv * a.n_chunks;
  if (problems <= 0 || a.k_m <= 0) return hipSuccess;
  k_topk<<<dim3((unsigned)problems), kTopkThreads, 0, st>>>(a.scores, a.U, a.k_m, a.sel);
  return hipGetLastError();
}

}  // namespace infllm
