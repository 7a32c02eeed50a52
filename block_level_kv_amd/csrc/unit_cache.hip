// GPU cache of memory units in front of a host-resident unit pool (InfLLM
// Guide, "Core Innovation 3": every unit's K/V in host memory, a
// least-recently-used pool of hot units in GPU memory, misses brought in
// over the host link while the representatives stay resident for scoring).
//
// One workgroup per (sequence, KV head) row does a fetch without any host
// round trip: it reads the call's selections from device memory, updates
// the row's LRU tables, and copies each missed unit's B rows of K and V
// straight from pinned host memory (loads over the host link, issued eight
// 16-byte chunks per lane at a time) into the slot it takes.  The policy:
//   hits       the selected units already cached: stamp = step
//   misses     the other selected units, ascending unit order
//   victims    slots this call does not use, ascending (stamp, slot): empty
//              slots (stamp 0) first, then least recently used
//   the i-th miss takes the i-th victim, whose old unit leaves the cache.
// Tables (zero-filled = empty cache): slot_of[u] = slot + 1 (0: absent),
// unit_of[c] = unit + 1 (0: empty), stamp[c] = last step that used slot c.
#include "common.h"
#include "kernels.h"

namespace infllm {

constexpr int kCacheThreads = 256;
constexpr int kCacheWords = kCacheMaxUnits / 32;   // selection bitmap
constexpr int kCopyUnroll = 8;                     // 16-byte chunks in flight per lane

// Inclusive scan over the workgroup of one int per thread; returns the
// inclusive value, *total = the sum of all.
__device__ __forceinline__ int block_scan(int x, int* wave_tot, int* total) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int y = __shfl_up(x, m);
    if (lane >= m) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kCacheThreads / 64; ++w) {
    before += w < wave ? wave_tot[w] : 0;
    all += wave_tot[w];
  }
  __syncthreads();   // wave_tot may be reused
  *total = all;
  return before + x;
}

// Copy n bytes (a multiple of 16) from src to dst, the whole workgroup.
__device__ __forceinline__ void copy_rows(const char* src, char* dst, int64_t n) {
  const int64_t step = (int64_t)kCacheThreads * 16 * kCopyUnroll;
  for (int64_t o = (int64_t)threadIdx.x * 16; o < n; o += step) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t x = o + (int64_t)j * kCacheThreads * 16;
      if (x < n) v[j] = *(const u32x4*)(src + x);
    }
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t x = o + (int64_t)j * kCacheThreads * 16;
      if (x < n) *(u32x4*)(dst + x) = v[j];
    }
  }
}

__global__ __launch_bounds__(kCacheThreads) void k_cache_fetch(CacheArgs a) {
  __shared__ uint32_t bits[kCacheWords];
  __shared__ int32_t chosen[kCacheMaxSlots];   // selected units, ascending
  __shared__ int32_t miss[kCacheMaxSlots];     // misses, ascending
  __shared__ int32_t victim[kCacheMaxSlots];   // victim slots, LRU first
  __shared__ int64_t st[kCacheMaxSlots];       // stamps before this call
  __shared__ uint8_t used[kCacheMaxSlots];     // slot holds a selected unit
  __shared__ int wave_tot[kCacheThreads / 64];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;              // sequence * H_kv + KV head
  const int U = a.n_units, C = a.n_slots;
  int32_t* slot_of = a.slot_of + row * U;
  int32_t* unit_of = a.unit_of + row * C;
  int64_t* stamp = a.stamp + row * C;
  const int n_words = (U + 31) / 32;

  for (int i = tid; i < n_words; i += kCacheThreads) bits[i] = 0;
  for (int c = tid; c < C; c += kCacheThreads) {
    st[c] = stamp[c];
    used[c] = 0;
  }
  __syncthreads();
  // the union of the row's selections (ids outside [0, U) ignored)
  const int n_sel = a.n_pos * a.k_m;
  const int32_t* sel = a.sel + row * (int64_t)n_sel;
  for (int i = tid; i < n_sel; i += kCacheThreads) {
    const int32_t u = sel[i];
    if (u >= 0 && u < U) atomicOr(&bits[u >> 5], 1u << (u & 31));
  }
  __syncthreads();
  // compaction in ascending order: thread t owns words [t*wpt, (t+1)*wpt)
  const int wpt = (n_words + kCacheThreads - 1) / kCacheThreads;
  int cnt = 0;
  for (int i = 0; i < wpt; ++i) {
    const int wd = tid * wpt + i;
    if (wd < n_words) cnt += __popc(bits[wd]);
  }
  int n_chosen;
  int at = block_scan(cnt, wave_tot, &n_chosen) - cnt;
  for (int i = 0; i < wpt; ++i) {
    const int wd = tid * wpt + i;
    uint32_t b = wd < n_words ? bits[wd] : 0u;
    while (b) {
      const int k = __builtin_ctz(b);
      b &= b - 1;
      chosen[at++] = wd * 32 + k;
    }
  }
  __syncthreads();
  // hits: refresh their stamps, mark their slots
  int is_miss[kCacheMaxSlots / kCacheThreads];
#pragma unroll
  for (int r = 0; r < kCacheMaxSlots / kCacheThreads; ++r) {
    const int i = tid * (kCacheMaxSlots / kCacheThreads) + r;   // contiguous: keeps the order
    is_miss[r] = 0;
    if (i < n_chosen) {
      const int s = slot_of[chosen[i]] - 1;
      if (s >= 0) {
        used[s] = 1;
        stamp[s] = a.step;
      } else {
        is_miss[r] = 1;
      }
    }
  }
  int mc = 0;
#pragma unroll
  for (int r = 0; r < kCacheMaxSlots / kCacheThreads; ++r) mc += is_miss[r];
  int n_miss;
  at = block_scan(mc, wave_tot, &n_miss) - mc;
#pragma unroll
  for (int r = 0; r < kCacheMaxSlots / kCacheThreads; ++r)
    if (is_miss[r]) miss[at++] = chosen[tid * (kCacheMaxSlots / kCacheThreads) + r];
  __syncthreads();   // used[] and miss[] complete
  // victims: rank of each unused slot in (stamp, slot) order
  if (n_miss > 0) {
    for (int c = tid; c < C; c += kCacheThreads) {
      if (used[c]) continue;
      const int64_t s0 = st[c];
      int rank = 0;
      for (int c2 = 0; c2 < C; ++c2)
        rank += !used[c2] && (st[c2] < s0 || (st[c2] == s0 && c2 < c));
      if (rank < n_miss) victim[rank] = c;
    }
  }
  __syncthreads();
  // the i-th miss into the i-th victim
  for (int i = tid; i < n_miss; i += kCacheThreads) {
    const int c = victim[i], u = miss[i];
    const int old = unit_of[c] - 1;
    if (old >= 0) slot_of[old] = 0;
    unit_of[c] = u + 1;
    slot_of[u] = c + 1;
    stamp[c] = a.step;
  }
  if (tid == 0) {
    atomicAdd((unsigned long long*)&a.stats[0], (unsigned long long)(n_chosen - n_miss));
    atomicAdd((unsigned long long*)&a.stats[1], (unsigned long long)n_miss);
  }
  // the missed units' rows from host memory: unit u is block u + n_init/B,
  // B contiguous rows of this (sequence, KV head)
  const int64_t unit_bytes = (int64_t)a.B * a.d * a.elem;
  const int64_t host_row0 = row * a.host_cap;
  for (int i = 0; i < n_miss; ++i) {
    const int64_t first = ((int64_t)miss[i] + a.n_init / a.B) * a.B;
    const int64_t src = (host_row0 + first) * a.d * a.elem;
    const int64_t dst = (row * C + victim[i]) * unit_bytes;
    copy_rows((const char*)a.k_host + src, (char*)a.ck + dst, unit_bytes);
    copy_rows((const char*)a.v_host + src, (char*)a.cv + dst, unit_bytes);
  }
}

size_t cache_state_bytes(int64_t rows, int n_units, int n_slots) {
  return kCacheHeaderBytes + round256((size_t)rows * n_units * 4) +
         round256((size_t)rows * n_slots * 4) + round256((size_t)rows * n_slots * 8);
}

CacheTables cache_tables(void* state, int64_t rows, int n_units, int n_slots) {
  char* p = (char*)state;
  CacheTables t;
  t.stats = (int64_t*)p;
  p += kCacheHeaderBytes;
  t.slot_of = (int32_t*)p;
  p += round256((size_t)rows * n_units * 4);
  t.unit_of = (int32_t*)p;
  p += round256((size_t)rows * n_slots * 4);
  t.stamp = (int64_t*)p;
  return t;
}

hipError_t launch_cache_fetch(const CacheArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.batch * a.Hkv;
  if (rows <= 0) return hipSuccess;
  k_cache_fetch<<<dim3((unsigned)rows), kCacheThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace infllm
