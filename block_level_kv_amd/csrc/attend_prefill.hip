// Working-context attention for query chunks on bf16 MFMA (gfx950,
// head_dim 128): the chunked-encoding hot loop.
//
// A workgroup owns 128 query rows of one KV head -- the G query heads that
// share that KV head times 128/G consecutive queries of one chunk -- and
// walks a list of 64-key tiles: the initial tokens, each selected unit's
// block, and the local-window band of its queries (InfLLM Guide, "Core
// Innovation 2", item 3, Working Context).  Tiles that straddle a boundary
// (causal edge, t - W edge, the sink/unit edge) get a per-element mask:
//     initial tokens:  p < n_init, p <= t
//     unit keys:       p >= n_init, p <= t - W
//     window keys:     p >= n_init, t - W < p <= t
// all other tiles run mask-free.  Each of the 4 waves holds 32 rows:
//     S^T = K Q^T   (v_mfma_f32_32x32x16_bf16; A = K rows from LDS,
//                    B = the wave's Q rows kept in registers)
//     online softmax in fp32 (exp2, log2-scaled logits)
//     O^T += V^T P^T (A = V^T from LDS, B = P^T straight from the S^T
//                    accumulators, rounded to bf16)
// The rows of K fed to the first product are permuted (bits 2 and 3 of the
// row index swapped) so that each lane's S^T values come out as runs of 8
// consecutive keys: exactly the B-operand layout of the second product.  V
// is transposed into LDS while it is staged; both tiles are double-buffered
// and the next tile's global loads are in flight during the current tile's
// math.  To fill the chip the tile list is split over several workgroups
// (split-K): each publishes its partial (max, sum, unnormalised output) rows
// and the last one to finish, found with a per-tile counter in the
// workspace, merges them and writes the output.  The counters return to
// zero at the end of every call.
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace infllm {

constexpr int kD = 128;
constexpr int kRows = 128;            // query rows per workgroup
constexpr int kKT = 64;               // keys per tile
constexpr int kKsStride = kD + 8;     // bf16 per K row in LDS (272 B)
constexpr int kVtStride = kKT + 8;    // bf16 per V^T row in LDS (144 B)
constexpr int kKsElems = kKT * kKsStride;
constexpr int kVtElems = kD * kVtStride;
constexpr int kMaxTiles = 1024;
constexpr int kXcds = 8;             // MI355X: 8 XCDs, each with its own L2
constexpr int kThreads = 256;

enum : int { kTileInit = 0, kTileUnit = 1, kTileWin = 2, kTileMask = 4 };

constexpr float kLog2eP = 1.4426950408889634f;

__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Workgroup -> work mapping.  The hardware hands workgroup i to XCD i % 8;
// when the (sequence, KV head) groups divide evenly over the XCDs, every
// workgroup of a group is placed on one XCD so that the group's K/V tiles
// are shared through that XCD's L2.
struct PrefillGeom {
  int n_qtiles, TQ, splits;
  int per_group;   // workgroups per (sequence, KV head): chunks x query tiles x splits
  int xcd_groups;  // 1: group g runs on XCD g % 8
};

// Valid key offsets [lo, hi] within a 64-key tile for a query at t, per tile
// type (offsets relative to the tile's first key p0).
__device__ __forceinline__ void tile_window(int type, int64_t p0, int64_t t, int n_init, int W,
                                            int* lo, int* hi) {
  int64_t l, h;
  if (type == kTileInit) {
    l = 0;
    h = (n_init - 1 < t ? n_init - 1 : t) - p0;
  } else if (type == kTileUnit) {
    l = n_init - p0;
    h = t - W - p0;
  } else {
    const int64_t a = t - W + 1;
    l = (n_init > a ? n_init : a) - p0;
    h = t - p0;
  }
  *lo = (int)(l < -1 ? -1 : (l > kKT ? kKT : l));
  *hi = (int)(h < -1 ? -1 : (h > kKT ? kKT : h));
}

template <int G>
__global__ __launch_bounds__(kThreads, 2) void k_attend_prefill(AttendArgs a, PrefillGeom geo) {
  constexpr int TQ = kRows / G;  // queries per workgroup
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int n = lane % 32, half = lane / 32;
  int gidx, item;
  if (geo.xcd_groups) {
    const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    gidx = x + kXcds * (j / geo.per_group);
    item = j % geo.per_group;
  } else {
    gidx = blockIdx.x / geo.per_group;
    item = blockIdx.x % geo.per_group;
  }
  const int h = gidx % a.Hkv, bi = gidx / a.Hkv;
  const int split = item % geo.splits;
  item /= geo.splits;
  const int qt = item % geo.n_qtiles, ch = item / geo.n_qtiles;

  const int q_first = qt * TQ;                          // within the chunk
  const int nq = a.L - q_first < TQ ? a.L - q_first : TQ;
  const int64_t ta = a.q_pos + (int64_t)ch * a.L + q_first;  // first query position
  const int64_t tb = ta + nq - 1;                            // last valid query position

  __shared__ __attribute__((aligned(16))) bf16_t lds_k[2][kKsElems];
  __shared__ __attribute__((aligned(16))) bf16_t lds_vt[2][kVtElems];
  __shared__ int tiles[kMaxTiles];
  __shared__ int n_tiles_sh;
  __shared__ int last_sh;

  // ---------------------------------------------------------- tile list
  // [initial-token tiles][unit tiles, in sel order][window-band tiles];
  // thread m handles sel entry m (k_m <= kThreads), a block scan places them.
  {
    const int W = a.W, n_init = a.n_init;
    const int64_t init_end = n_init < tb + 1 ? n_init : tb + 1;
    const int n_init_tiles = (int)((init_end + kKT - 1) / kKT);
    const int64_t wlo = n_init > ta - W + 1 ? n_init : ta - W + 1;
    const int64_t w0 = (wlo / kKT) * kKT;
    const int n_win_tiles = tb >= w0 ? (int)((tb - w0) / kKT + 1) : 0;
    // this thread's unit: how many of its 64-key tiles hold a usable key
    int64_t jb = 0;
    int cnt = 0, s_first = 0;
    if (tid < a.k_m) {
      const int32_t u = a.sel[(((int64_t)bi * a.Hkv + h) * a.n_chunks + ch) * a.k_m + tid];
      if (u >= 0) {
        jb = ((int64_t)u + n_init / a.B) * a.B;
        for (int s = 0; s < a.B / kKT; ++s) {
          const int64_t p0 = jb + (int64_t)s * kKT;
          if (p0 > tb - W) break;                   // no key at least W behind any query
          if (p0 + kKT - 1 < n_init) { s_first = s + 1; continue; }  // initial tokens only
          ++cnt;
        }
      }
    }
    // exclusive scan of cnt over the workgroup
    const int wv = tid / 64;
    int x = cnt;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int y = __shfl_up(x, m);
      if (lane >= m) x += y;
    }
    __shared__ int wave_tot[kThreads / 64];
    if (lane == 63) wave_tot[wv] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w2 = 0; w2 < kThreads / 64; ++w2) {
      before += w2 < wv ? wave_tot[w2] : 0;
      all += wave_tot[w2];
    }
    const int off = n_init_tiles + before + x - cnt;
    for (int i = 0; i < cnt; ++i) {
      const int64_t p0 = jb + (int64_t)(s_first + i) * kKT;
      const bool fast = p0 >= n_init && p0 + kKT - 1 <= ta - W;
      tiles[off + i] = (int)p0 | kTileUnit | (fast ? 0 : kTileMask);
    }
    for (int i = tid; i < n_init_tiles; i += kThreads) {
      const int64_t p0 = (int64_t)i * kKT;
      const bool fast = p0 + kKT - 1 < n_init && p0 + kKT - 1 <= ta;
      tiles[i] = (int)p0 | kTileInit | (fast ? 0 : kTileMask);
    }
    for (int i = tid; i < n_win_tiles; i += kThreads) {
      const int64_t p0 = w0 + (int64_t)i * kKT;
      const bool fast = p0 >= n_init && p0 > tb - W && p0 + kKT - 1 <= ta;
      tiles[n_init_tiles + all + i] = (int)p0 | kTileWin | (fast ? 0 : kTileMask);
    }
    if (tid == 0) n_tiles_sh = n_init_tiles + all + n_win_tiles;
  }
  __syncthreads();
  const int n_tiles = n_tiles_sh;
  const int tile_begin = (int)((int64_t)n_tiles * split / geo.splits);
  const int tile_end = (int)((int64_t)n_tiles * (split + 1) / geo.splits);

  // ---------------------------------------------------------- this lane's row
  const int row = wave * 32 + n;            // 0..127
  const int g = row / TQ, qi = row % TQ;    // head within the group, query within tile
  const bool row_ok = qi < nq;
  const int64_t t_row = ta + qi;
  const int64_t qh = (int64_t)bi * a.Hq + (int64_t)h * G + g;
  const bf16_t* Q = (const bf16_t*)a.q;
  const int64_t q_row = a.q_off + (int64_t)ch * a.L + q_first + (row_ok ? qi : 0);
  bf16x8 qreg[8];
  {
    const bf16_t* qp = Q + (qh * a.q_cap + q_row) * kD + half * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = *(const bf16x8*)(qp + ks * 16);
  }

  // ---------------------------------------------------------- staging
  const bf16_t* Kg = (const bf16_t*)a.k + ((int64_t)bi * a.Hkv + h) * a.kv_cap * kD;
  const bf16_t* Vg = (const bf16_t*)a.v + ((int64_t)bi * a.Hkv + h) * a.kv_cap * kD;
  const int64_t last_row = a.kv_cap - 1;
  u32x4 pk[4], pv[4];
  // K: thread -> (key = tid/16 + 16 i, 16-byte chunk tid%16), coalesced rows
  // V: thread -> (key pair kp = tid%32, 8-column group dg = tid/32 + 8 i)
  auto load_tile = [&](int desc) {
    const int64_t p0 = desc & ~7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t r = p0 + tid / 16 + 16 * i;
      r = r < last_row ? r : last_row;
      pk[i] = *(const u32x4*)(Kg + r * kD + (tid % 16) * 8);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int dg = tid / 32 + 8 * i, kp = tid % 32;
      int64_t r0 = p0 + 2 * kp, r1 = r0 + 1;
      r0 = r0 < last_row ? r0 : last_row;
      r1 = r1 < last_row ? r1 : last_row;
      pv[2 * i] = *(const u32x4*)(Vg + r0 * kD + dg * 8);
      pv[2 * i + 1] = *(const u32x4*)(Vg + r1 * kD + dg * 8);
    }
  };
  auto store_tile = [&](int buf) {
    bf16_t* ks = lds_k[buf];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(u32x4*)(ks + (tid / 16 + 16 * i) * kKsStride + (tid % 16) * 8) = pk[i];
    uint32_t* vt = (uint32_t*)lds_vt[buf];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int dg = tid / 32 + 8 * i, kp = tid % 32;
      const u32x4 x = pv[2 * i], y = pv[2 * i + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // columns 8dg+2j and 8dg+2j+1 of keys 2kp and 2kp+1
        const uint32_t lo = (x[j] & 0xffffu) | (y[j] << 16);
        const uint32_t hi = (x[j] >> 16) | (y[j] & 0xffff0000u);
        vt[((8 * dg + 2 * j) * kVtStride) / 2 + kp] = lo;
        vt[((8 * dg + 2 * j + 1) * kVtStride) / 2 + kp] = hi;
      }
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = kLog2eP / sqrtf((float)kD);
  const int kperm = swap_bits23(n);   // key row this lane feeds to S^T

  if (tile_begin < tile_end) {
    load_tile(tiles[tile_begin]);
    store_tile(0);
  }
  __syncthreads();

  for (int tix = tile_begin; tix < tile_end; ++tix) {
    const int buf = (tix - tile_begin) & 1;
    const int desc = tiles[tix];
    const bool more = tix + 1 < tile_end;
    if (more) load_tile(tiles[tix + 1]);

    // S^T = K Q^T for 64 keys x 32 rows: two 32-key sub-tiles
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    {
      const bf16_t* k0 = lds_k[buf] + kperm * kKsStride + half * 8;
      const bf16_t* k1 = k0 + 32 * kKsStride;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a0 = *(const bf16x8*)(k0 + ks * 16);
        const bf16x8 a1 = *(const bf16x8*)(k1 + ks * 16);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], s1, 0, 0, 0);
      }
    }
    // register r of sub-tile kt holds key offset 32kt + 16(r/8) + 8 half + r%8
    if (desc & kTileMask) {
      int lo, hi;
      tile_window(desc & 3, (int64_t)(desc & ~7), t_row, a.n_init, a.W, &lo, &hi);
      lo -= half * 8;
      hi -= half * 8;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = 16 * (r / 8) + (r % 8);
        if (o < lo || o > hi) s0[r] = -INFINITY;
        if (o + 32 < lo || o + 32 > hi) s1[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    if (__any(m_new != m_run)) {   // rescale only when some row's max moved
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
    }
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p0v = __builtin_amdgcn_exp2f(fmaf(s0[r], c, -m_use));
      const float p1v = __builtin_amdgcn_exp2f(fmaf(s1[r], c, -m_use));
      psum += p0v + p1v;
      pb[r / 8][r % 8] = (__bf16)p0v;
      pb[2 + r / 8][r % 8] = (__bf16)p1v;
    }
    l_run += psum;

    // O^T += V^T P^T: 4 key steps of 16 x 4 d-tiles of 32
    {
      const bf16_t* vt = lds_vt[buf] + kperm * kVtStride + half * 8;
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 av = *(const bf16x8*)(vt + (32 * dt) * kVtStride + sp * 16);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[sp], acc[dt], 0, 0, 0);
        }
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------- epilogue
  float l_tot = l_run + __shfl_xor(l_run, 32);
  const int64_t pos = (int64_t)ch * a.L + q_first + qi;     // row within this call
  // register r of d-tile dt holds column 32dt + 16(r/8) + 8 half + r%8
  if (geo.splits > 1) {
    // Every split publishes its partial rows; the last split to finish
    // merges.  Publication uses device-scope (sc1) stores, drained with
    // s_waitcnt vmcnt(0) before the barrier that precedes the arrival
    // counter; the merger reads with device-scope loads.  No L2 writeback or
    // invalidate is needed, so the K/V lines other workgroups share in L2
    // survive.
    const int64_t wrow = ((int64_t)split * a.batch * a.Hq + qh) * a.n_pos + pos;
    // this workgroup's rows of split s start at region_row(s); lane offsets
    // (head g, query qi, column) stay below G * n_pos rows
    const int64_t qh0 = (int64_t)bi * a.Hq + (int64_t)h * G;
    const int64_t pos0 = (int64_t)ch * a.L + q_first;
    auto region = [&](int s) {
      return dev_rsrc(a.ws_o + (((int64_t)s * a.batch * a.Hq + qh0) * a.n_pos + pos0) * kD,
                      (uint32_t)((int64_t)G * a.n_pos * kD * sizeof(float)));
    };
    const uint32_t lane_off =
        (uint32_t)((((int64_t)g * a.n_pos + qi) * kD + half * 8) * sizeof(float));
    if (row_ok) {
      const __amdgpu_buffer_rsrc_t r = region(split);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = acc[dt][4 * q4 + j];
          // registers 4q4..4q4+3 hold columns 32dt + 16(q4/2) + 8half + 4(q4%2) + j
          st4_dev(r, lane_off + (32 * dt + 16 * (q4 / 2) + 4 * (q4 % 2)) * 4, v);
        }
      if (half == 0) {
        st_dev(&a.ws_ml[2 * wrow], m_run);
        st_dev(&a.ws_ml[2 * wrow + 1], l_tot);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
      const int64_t tile_id = (((int64_t)bi * a.Hkv + h) * a.n_chunks + ch) * geo.n_qtiles + qt;
      const int done = __hip_atomic_fetch_add(&a.ws_count[tile_id], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      last_sh = done == geo.splits - 1;
      if (last_sh)   // ready for the next call
        __hip_atomic_store(&a.ws_count[tile_id], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_sh || !row_ok) return;
    // merge: own registers + the other splits' published rows
    float M = m_run;
    for (int s = 0; s < geo.splits; ++s) {
      if (s == split) continue;
      const int64_t r2 = ((int64_t)s * a.batch * a.Hq + qh) * a.n_pos + pos;
      M = fmaxf(M, ld_dev(&a.ws_ml[2 * r2]));
    }
    // splits are summed in index order whichever one merges, so the result
    // does not depend on arrival order
    const float mu = M == -INFINITY ? 0.f : M;
    f32x16 res[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) res[dt] = f32x16{};
    float l_sum = 0.f;
    for (int s = 0; s < geo.splits; ++s) {
      if (s == split) {
        const float w = __builtin_amdgcn_exp2f(m_run - mu);
        l_sum = fmaf(l_tot, w, l_sum);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int j = 0; j < 16; ++j) res[dt][j] = fmaf(acc[dt][j], w, res[dt][j]);
        continue;
      }
      const int64_t r2 = ((int64_t)s * a.batch * a.Hq + qh) * a.n_pos + pos;
      const float ms = ld_dev(&a.ws_ml[2 * r2]);
      const float w = __builtin_amdgcn_exp2f(ms - mu);
      l_sum = fmaf(ld_dev(&a.ws_ml[2 * r2 + 1]), w, l_sum);
      const __amdgpu_buffer_rsrc_t r = region(s);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = ld4_dev(r, lane_off + (32 * dt + 16 * (q4 / 2) + 4 * (q4 % 2)) * 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) res[dt][4 * q4 + j] = fmaf(v[j], w, res[dt][4 * q4 + j]);
        }
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = res[dt];
    l_tot = l_sum;
    m_run = M;
  }
  if (!row_ok) return;
  const float inv = 1.f / l_tot;
  bf16_t* o = (bf16_t*)a.out + (qh * a.out_cap + a.out_off + pos) * kD + half * 8;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (__bf16)(acc[dt][8 * hh + j] * inv);
      *(bf16x8*)(o + 32 * dt + 16 * hh) = v;
    }
  }
  if (a.lse && half == 0)
    a.lse[qh * a.out_cap + a.out_off + pos] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
}

static int max_tiles(const AttendArgs& a, int TQ) {
  return (a.n_init + kKT - 1) / kKT + a.k_m * (a.B / kKT) + (a.W + TQ + 2 * kKT - 2) / kKT + 1;
}

bool prefill_supported(const AttendArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (!a.bf16 || a.d != kD || a.B % kKT != 0) return false;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (a.L < 16) return false;  // decode-sized chunks take the vector path
  return max_tiles(a, kRows / G) <= kMaxTiles;
}

int prefill_num_splits(const AttendArgs& a) {
  if (const char* e = getenv("INFLLM_PREFILL_SPLITS")) {  // tuning override
    const int v = atoi(e);
    if (v >= 1 && v <= 16) return v;
  }
  const int G = a.Hq / a.Hkv;
  const int TQ = kRows / G;
  const int64_t wgs = (int64_t)((a.L + TQ - 1) / TQ) * a.n_chunks * a.Hkv * a.batch;
  const int tiles = max_tiles(a, TQ);
  int s = 1;
  while (wgs * s < 512 && tiles / (2 * s) >= 8 && s < 8) s *= 2;
  return s;
}

int64_t prefill_num_counters(const AttendArgs& a) {
  const int TQ = kRows / (a.Hq / a.Hkv);
  return (int64_t)((a.L + TQ - 1) / TQ) * a.n_chunks * a.Hkv * a.batch;
}

template <int G>
static void launch_g(const AttendArgs& a, int splits, hipStream_t st) {
  constexpr int TQ = kRows / G;
  PrefillGeom geo;
  geo.TQ = TQ;
  geo.n_qtiles = (a.L + TQ - 1) / TQ;
  geo.splits = splits;
  geo.per_group = geo.n_qtiles * a.n_chunks * splits;
  const int groups = a.Hkv * a.batch;
  geo.xcd_groups = groups % kXcds == 0;
  k_attend_prefill<G><<<dim3(geo.per_group * groups), kThreads, 0, st>>>(a, geo);
}

hipError_t launch_attend_prefill(const AttendArgs& a, int splits, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: launch_g<1>(a, splits, st); break;
    case 2: launch_g<2>(a, splits, st); break;
    case 4: launch_g<4>(a, splits, st); break;
    case 8: launch_g<8>(a, splits, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace infllm
