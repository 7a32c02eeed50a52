// Working-context attention for query chunks on bf16 MFMA (gfx950,
// head_dim 128): the chunked-encoding hot loop.
//
// A workgroup owns 256 query rows of one KV head -- the G query heads that
// share that KV head times 256/G consecutive queries of one chunk -- and
// walks a list of 64-key tiles: the initial tokens, each selected unit's
// block, and the local-window band of its queries (InfLLM Guide, "Core
// Innovation 2", item 3, Working Context).  Tiles that straddle a boundary
// (causal edge, t - W edge, the sink/unit edge) get a per-element mask:
//     initial tokens:  p < n_init, p <= t
//     unit keys:       p >= n_init, p <= t - W
//     window keys:     p >= n_init, t - W < p <= t
// all other tiles run mask-free.  Each of the 8 waves holds 32 rows:
//     S^T = K Q^T   (v_mfma_f32_32x32x16_bf16; A = K rows from LDS,
//                    B = the wave's Q rows kept in registers)
//     online softmax in fp32 (exp2, log2-scaled logits)
//     O^T += V^T P^T (A = V^T read from row-major V with the transposing
//                    LDS load, B = P^T straight from the S^T accumulators,
//                    rounded to bf16)
// The rows of K fed to the first product are permuted (bits 2 and 3 of the
// row index swapped) so that each lane's S^T values come out as runs of 8
// consecutive keys: exactly the B-operand layout of the second product.
//
// K and V tiles travel from global memory straight into LDS (16-byte
// global_load_lds per lane, no register staging) through a ring of four
// buffers, three tiles ahead of the math.  Within a row the 16-byte chunks
// are XOR-swizzled so that both the K operand reads and the transposing V
// reads are free of bank conflicts.  To fill the chip the tile list is
// split over several workgroups (split-K): each publishes its partial
// (max, sum, unnormalised output) rows and the last one to finish, found
// with a per-tile counter in the workspace, merges them and writes the
// output.  The counters return to zero at the end of every call.
//
// RoPE (rope.h): window tiles need nothing; each initial-token or unit tile
// has one shift, and the wave that loaded a tile's rows turns them by it in
// LDS after its loads land and before the barrier that hands the tile to
// the other waves (lanes pos and pos ^ 8 of a 16-lane row hold the two
// halves of every rotary pair); the turned keys are rounded to bf16.  The
// tile's cosines and sines are computed two tiles ahead into one of two LDS
// tables, so the ring keeps one barrier per tile.  Unit keys at or past the
// chunk's first local place keep their own position; queries before n_init
// are turned once, when loaded.

#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace infllm {

constexpr int kD = 128;
constexpr int kRows = 256;            // query rows per workgroup (32 per wave)
constexpr int kKT = 64;               // keys per tile
constexpr int kTileElems = kKT * kD;  // one K or V tile in LDS: 64 rows of 256 B
constexpr int kStages = 4;            // LDS ring depth
constexpr int kMaxTiles = 1024;
constexpr int kXcds = 8;             // MI355X: 8 XCDs, each with its own L2
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

enum : int { kTileInit = 0, kTileUnit = 1, kTileWin = 2, kTileMask = 4 };

constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kSlack = 8.f;         // weights below 2^8 between rescales

// max of three floats in one instruction (no NaN reaches it)
__device__ __forceinline__ float max3(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
// s_waitcnt vmcnt(4 (kStages - 2)) lgkmcnt(0): the loads of the next tile
// have landed and no LDS read of this wave is still in flight
constexpr int kWaitRing = 0x0078;
// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their maxima)
constexpr int kWaitLgkm0 = 0xC07F;
// vmcnt(0) lgkmcnt(0): the paired ring's wait before each barrier
constexpr int kWaitPair = 0x0070;
static_assert(kStages == 4, "kWaitRing encodes 4 loads x 2 tiles in flight");

__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// 16-byte chunk position of chunk c of row r within its 256-byte LDS row.
// K rows are read 16 rows x one chunk at a time: XOR with r % 16 spreads
// them over all banks.  V rows are read through the transposing load, four
// consecutive keys x four chunks per 16 lanes: XOR with 4 (r % 4).
__device__ __forceinline__ int k_pos(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int v_pos(int r, int c) { return c ^ ((r & 3) << 2); }

typedef short short4_t __attribute__((ext_vector_type(4)));
#define INFLLM_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define INFLLM_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))

// Workgroup -> work mapping.  The hardware hands workgroup i to XCD i % 8;
// when the (sequence, KV head) groups divide evenly over the XCDs, every
// workgroup of a group is placed on one XCD so that the group's K/V tiles
// are shared through that XCD's L2.
struct PrefillGeom {
  int n_qtiles, TQ, splits;
  int n_items;     // work items (query tile x chunk x sequence x KV head) per split
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

// bf16 pair <-> two floats; packing rounds to nearest even
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t bf_pack(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <int G, bool ROPE>
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
  // chunks in reverse order: later chunks have the longer tile lists, and
  // the short ones dispatched last fill the tail of the launch
  const int qt = item % geo.n_qtiles, ch = a.n_chunks - 1 - item / geo.n_qtiles;

  const int q_first = qt * TQ;                          // within the chunk
  const int nq = a.L - q_first < TQ ? a.L - q_first : TQ;
  const int64_t base = seq_base(a.pos, a.q_pos, bi);
  if (a.pos && !seq_pos_ok(base, a.n_pos, a.kv_cap)) {
    // a sequence whose position does not fit its KV buffer: every split
    // leaves before any key load or arrival count, split 0 writes NaN rows
    if (split == 0)
      nan_rows<bf16_t>((bf16_t*)a.out, a.lse, (int64_t)bi * a.Hq + (int64_t)h * G, G, a.out_cap,
                       a.out_off + (int64_t)ch * a.L + q_first, nq, kD, tid, kThreads);
    return;
  }
  const int64_t ta = base + (int64_t)ch * a.L + q_first;    // first query position
  const int64_t tb = ta + nq - 1;                            // last valid query position

  // the ring: one variable per stage and operand, so that the compiler can
  // tell the buffer being read from the buffers being loaded
  __shared__ __attribute__((aligned(16))) bf16_t lds_k0[kTileElems], lds_k1[kTileElems],
      lds_k2[kTileElems], lds_k3[kTileElems];
  __shared__ __attribute__((aligned(16))) bf16_t lds_v0[kTileElems], lds_v1[kTileElems],
      lds_v2[kTileElems], lds_v3[kTileElems];
  __shared__ int tiles[kMaxTiles];
  __shared__ int n_tiles_sh;
  __shared__ int last_sh;
  // RoPE: each tile's shift (0: none), the frequencies, and two tables of
  // cos / sin (the tile after next is computed while one is in use)
  __shared__ int tile_turn[ROPE ? kMaxTiles : 1];
  __shared__ double turns_sm[ROPE ? kD / 2 : 1];
  __shared__ __attribute__((aligned(16))) float turn_cs[ROPE ? 2 : 1][2][kD / 2];
  // chunk start -> first local place; shift of the initial tokens
  const int64_t lo_ctx = rope_local_start(base + (int64_t)ch * a.L, a.n_init, a.W);
  const int e_sink = (int)(a.n_init + (int64_t)a.k_m * a.B - lo_ctx);

  // ---------------------------------------------------------- this lane's row
  // (its Q loads go out first: their latency runs beside the tile list's)
  const int row = wave * 32 + n;            // 0..255
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
    __shared__ int32_t ids_sm[kMaxTopK];
    int32_t u = tid < a.k_m ? a.sel[(((int64_t)bi * a.Hkv + h) * a.n_chunks + ch) * a.k_m + tid] : -1;
    u = drop_repeats(u, tid, a.k_m, ids_sm);   // a repeated id is attended once
    if (tid < a.k_m) {
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
    // slot tid: E_m = (k_m - m) B + jB - lo
    const int e_unit = (int)((int64_t)(a.k_m - tid) * a.B + jb - lo_ctx);
    for (int i = 0; i < cnt; ++i) {
      const int64_t p0 = jb + (int64_t)(s_first + i) * kKT;
      const bool fast = p0 >= n_init && p0 + kKT - 1 <= ta - W;
      tiles[off + i] = (int)p0 | kTileUnit | (fast ? 0 : kTileMask);
      if constexpr (ROPE) tile_turn[off + i] = e_unit;
    }
    for (int i = tid; i < n_init_tiles; i += kThreads) {
      const int64_t p0 = (int64_t)i * kKT;
      const bool fast = p0 + kKT - 1 < n_init && p0 + kKT - 1 <= ta;
      tiles[i] = (int)p0 | kTileInit | (fast ? 0 : kTileMask);
      if constexpr (ROPE) tile_turn[i] = e_sink;
    }
    for (int i = tid; i < n_win_tiles; i += kThreads) {
      const int64_t p0 = w0 + (int64_t)i * kKT;
      const bool fast = p0 >= n_init && p0 > tb - W && p0 + kKT - 1 <= ta;
      tiles[n_init_tiles + all + i] = (int)p0 | kTileWin | (fast ? 0 : kTileMask);
      if constexpr (ROPE) tile_turn[n_init_tiles + all + i] = 0;
    }
    if (tid == 0) n_tiles_sh = n_init_tiles + all + n_win_tiles;
    if constexpr (ROPE) {
      if (tid < kD / 2) turns_sm[tid] = rope_turns(a.rope_theta, kD, tid);
    }
  }
  __syncthreads();
  const int n_tiles = n_tiles_sh;
  const int tile_begin = (int)((int64_t)n_tiles * split / geo.splits);
  const int tile_end = (int)((int64_t)n_tiles * (split + 1) / geo.splits);

  if constexpr (ROPE) {
    // a query before n_init sees initial tokens only, which are turned by
    // -E_s: turn it by -E_s too.  qreg[ks] holds columns 8 (2 ks + half) ..
    // +7, so the pairs (c, c + 64) are qreg[ks] and qreg[ks + 4], ks < 4.
    if (row_ok && t_row < a.n_init && e_sink != 0) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c0 = 8 * (2 * ks + half);
        u32x4 wl = __builtin_bit_cast(u32x4, qreg[ks]), wh = __builtin_bit_cast(u32x4, qreg[ks + 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float c2[2], s2[2];
          rope_cs(e_sink, turns_sm[c0 + 2 * i], &c2[0], &s2[0]);
          rope_cs(e_sink, turns_sm[c0 + 2 * i + 1], &c2[1], &s2[1]);
          const float l0 = bf_lo(wl[i]), l1 = bf_hi(wl[i]), h0 = bf_lo(wh[i]), h1 = bf_hi(wh[i]);
          wl[i] = bf_pack(rope_turn(l0, h0, c2[0], s2[0], true), rope_turn(l1, h1, c2[1], s2[1], true));
          wh[i] = bf_pack(rope_turn(h0, l0, c2[0], s2[0], false), rope_turn(h1, l1, c2[1], s2[1], false));
        }
        qreg[ks] = __builtin_bit_cast(bf16x8, wl);
        qreg[ks + 4] = __builtin_bit_cast(bf16x8, wh);
      }
    }
  }

  // ---------------------------------------------------------- staging
  // One global_load_lds instruction of a wave fills 1 KB of LDS: four rows,
  // lane l writing position l % 16 of row l / 16.  Wave w fills row groups w
  // and w + 8 of the K tile and of the V tile; each lane fetches the chunk
  // that the swizzle puts at its position (rows past the cache end are
  // clamped to the last row: those keys are always masked).
  const bf16_t* Kg = (const bf16_t*)a.k + ((int64_t)bi * a.Hkv + h) * a.kv_cap * kD;
  const bf16_t* Vg = (const bf16_t*)a.v + ((int64_t)bi * a.Hkv + h) * a.kv_cap * kD;
  const int64_t last_row = a.kv_cap - 1;
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = kLog2eP / sqrtf((float)kD);
  const int kperm = swap_bits23(n);   // key row this lane feeds to S^T
  // transposing V reads: within each 16 lanes, lane s supplies key
  // 4h + s/4 (of the 8-key run) and 4 columns starting at vcol; the lane
  // then receives column kperm(n) of the four keys 4h .. 4h+3
  const int vs = lane % 16;
  const int vcol = 16 * ((lane % 32) / 16) + 4 * (((vs & 1) << 1) | ((vs >> 1) & 1));
  const int vkey = 8 * half + (vs >> 2);

  // Ring of kStages buffers, loads kStages-1 tiles ahead.  Every iteration
  // issues the loads of one tile (a repeat of the last tile past the end,
  // into a buffer nobody reads) so that each lane always has the same
  // number of loads in flight, and "tile i+1 has landed" is
  // s_waitcnt vmcnt(4 * (kStages - 2)).
  const int nt = tile_end - tile_begin;
  // wave w fills row groups w and w + 8 of a tile: one global_load_lds
  // fills four rows (1 KB), lane l writing position l % 16 of row l / 16
  // with the chunk that the swizzle puts there; rows past the cache end are
  // clamped to the last row (those keys are always masked)
  auto load_tile = [&](int desc, bf16_t* kn, bf16_t* vn) {
    const int64_t p0 = desc & ~7;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int grp = wave + kWaves * j;
      const int r = 4 * grp + lane / 16, pos = lane % 16;
      int64_t row = p0 + r;
      row = row < last_row ? row : last_row;
      __builtin_amdgcn_global_load_lds(INFLLM_GLOBAL(Kg + row * kD + 8 * k_pos(r, pos)),
                                       INFLLM_LDS(kn + grp * 4 * kD), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(INFLLM_GLOBAL(Vg + row * kD + 8 * v_pos(r, pos)),
                                       INFLLM_LDS(vn + grp * 4 * kD), 16, 0, 0);
    }
  };
  // Between tiles: tile i+1 has landed (this lane's loads; vmcnt counts the
  // direct-to-LDS loads in issue order) and every LDS read of tile i has
  // returned (lgkmcnt), so after the barrier all lanes' parts of tile i+1
  // are visible and buffer i can be refilled.  A plain s_barrier:
  // __syncthreads' fence would also wait for the loads of tiles i+2 and
  // i+3.  The empty asm statements keep the compiler from moving LDS
  // accesses across it.
  //
  // RoPE: cos / sin of tile j's shift into table j % 2, frequency 8 w + l
  // by lane l < 8 of wave w.  Table j % 2 was last read while tile j - 2 was
  // turned, before the barrier that preceded tile j - 2's math.
  auto turn_table = [&](int j) {
    if (j >= nt) return;
    const int E = tile_turn[tile_begin + j];
    if (E == 0 || lane >= 8) return;
    const int f = 8 * wave + lane;
    rope_cs(E, turns_sm[f], &turn_cs[j & 1][0][f], &turn_cs[j & 1][1][f]);
  };
  // RoPE: turn this wave's rows of tile j (landed in kbuf) by its shift.
  // Lane l holds position l % 16 of row r = 4 grp + l / 16, i.e. chunk c =
  // (l % 16) ^ (r % 16) (the same for both of its rows); chunk c ^ 8, the
  // other half of its pairs, sits in lane l ^ 8.
  auto turn_tile = [&](int j, bf16_t* kbuf) {
    if (j >= nt) return;
    const int E = tile_turn[tile_begin + j];
    if (E == 0) return;
    const int desc = tiles[tile_begin + j];
    const int64_t p0 = desc & ~7;
    const bool unit = (desc & 3) == kTileUnit;
    const int c = (lane % 16) ^ ((4 * wave + lane / 16) & 15);
    const bool low = c < 8;
    const f32x4* ct = (const f32x4*)&turn_cs[j & 1][0][8 * (c & 7)];
    const f32x4* st = (const f32x4*)&turn_cs[j & 1][1][8 * (c & 7)];
    const f32x4 c0 = ct[0], c1 = ct[1], s0 = st[0], s1 = st[1];
    const float cs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int grp = wave + kWaves * jj;
      const int r = 4 * grp + lane / 16;
      u32x4* at = (u32x4*)(kbuf + grp * 4 * kD) + lane;   // row r, position lane % 16
      u32x4 w = *at, pw;
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = __builtin_amdgcn_mov_dpp(w[i], INFLLM_DPP_ROR8, 0xF, 0xF, true);
      // unit keys past the chunk's first local place sit at their own place
      if (!(unit && p0 + r >= lo_ctx)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = bf_pack(rope_turn(bf_lo(w[i]), bf_lo(pw[i]), cs[2 * i], sn[2 * i], low),
                         rope_turn(bf_hi(w[i]), bf_hi(pw[i]), cs[2 * i + 1], sn[2 * i + 1], low));
        *at = w;
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  };
  // tile j landed in kbuf: turn it (RoPE), then the barrier
  auto ring_barrier = [&](int j, bf16_t* kbuf) {
    __builtin_amdgcn_s_waitcnt(kWaitRing);
    asm volatile("" ::: "memory");
    if constexpr (ROPE) {
      turn_tile(j, kbuf);
      asm volatile("" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  if (nt > 0) {
    const int* tl = tiles + tile_begin;
    load_tile(tl[0], lds_k0, lds_v0);
    load_tile(tl[1 < nt ? 1 : nt - 1], lds_k1, lds_v1);
    if constexpr (ROPE) load_tile(tl[2 < nt ? 2 : nt - 1], lds_k2, lds_v2);
  }
  if constexpr (ROPE) {
    turn_table(0);
    turn_table(1);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  if constexpr (ROPE) {
    ring_barrier(0, lds_k0);   // tile 0 landed
  } else {
    __builtin_amdgcn_s_waitcnt(kWaitPair);   // tiles 0 and 1 landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // One tile: issue the loads of tile i+3, then the math on tile i.  The
  // ring buffers are separate variables and the loop below is unrolled over
  // the ring, so every LDS read names a buffer that the compiler can tell
  // apart from the ones being loaded (otherwise it would make every LDS read
  // wait for all loads in flight).
  auto tile_step = [&](const int* tl, const bf16_t* kb, const bf16_t* vb, bf16_t* kn,
                       bf16_t* vn, int i) {
    const int desc = tl[i];
    if constexpr (ROPE) {
      load_tile(tl[i + kStages - 1 < nt ? i + kStages - 1 : nt - 1], kn, vn);
      turn_table(i + 2);
    }

    // S^T = K Q^T for 64 keys x 32 rows: two 32-key sub-tiles
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    {
      const int r0 = kperm, r1 = 32 + kperm;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int cch = 2 * ks + half;
        const bf16x8 a0 = *(const bf16x8*)(kb + r0 * kD + 8 * k_pos(r0, cch));
        const bf16x8 a1 = *(const bf16x8*)(kb + r1 * kD + 8 * k_pos(r1, cch));
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
    for (int r = 0; r < 16; ++r) mx = max3(mx, s0[r], s1[r]);
    {
      // the other half of the wave holds the row's other keys
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // m_run is a reference maximum, not necessarily the running one: the
    // accumulators are rescaled only when some row's tile maximum exceeds
    // its reference by more than kSlack (log2 units), so weights stay
    // below 2^kSlack and most tiles skip the rescale
    const float mxs = mx * c;
    if (__any(mxs > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, mxs);
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
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

    // O^T += V^T P^T: 4 key steps of 16 x 4 d-tiles of 32; the V^T operand
    // (column kperm(n) + 32 dt, keys 16 sp + 8 half + j) comes from two
    // transposing reads of four keys each
    {
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int col = 32 * dt + vcol;
          const int k0 = 16 * sp + vkey, k1 = k0 + 4;
          const short4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4_t*)(vb + k0 * kD + 8 * v_pos(k0, col / 8) + col % 8));
          const short4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4_t*)(vb + k1 * kD + 8 * v_pos(k1, col / 8) + col % 8));
          // whole-vector concatenation and bit cast: building the operand
          // element by element makes the compiler splat element 0
          const bf16x8 av = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[sp], acc[dt], 0, 0, 0);
        }
      }
    }
  };

  // unrolled over the ring so that every copy names fixed buffers; after
  // each tile: tile i+1 landed (this lane's part), and the barrier makes
  // all parts visible and frees buffer i for the loads of the next tile
  if constexpr (ROPE) {
    const int* tl = tiles + tile_begin;
    for (int i = 0; i < nt; i += kStages) {
      tile_step(tl, lds_k0, lds_v0, lds_k3, lds_v3, i);
      ring_barrier(i + 1, lds_k1);
      if (i + 1 >= nt) break;
      tile_step(tl, lds_k1, lds_v1, lds_k0, lds_v0, i + 1);
      ring_barrier(i + 2, lds_k2);
      if (i + 2 >= nt) break;
      tile_step(tl, lds_k2, lds_v2, lds_k1, lds_v1, i + 2);
      ring_barrier(i + 3, lds_k3);
      if (i + 3 >= nt) break;
      tile_step(tl, lds_k3, lds_v3, lds_k2, lds_v2, i + 3);
      ring_barrier(i + 4, lds_k0);
    }
  } else {
    // Without RoPE the ring is taken in pairs of tiles, one barrier per
    // pair: buffers 0-1 and 2-3 alternate, each pair's math first issues
    // the loads of the next pair into the other two buffers (freed by the
    // barrier just passed), and the barrier after it waits for them.
    const int* tl = tiles + tile_begin;
    auto pair_barrier = [&]() {
      __builtin_amdgcn_s_waitcnt(kWaitPair);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    for (int i = 0; i < nt; i += kStages) {
      load_tile(tl[i + 2 < nt ? i + 2 : nt - 1], lds_k2, lds_v2);
      load_tile(tl[i + 3 < nt ? i + 3 : nt - 1], lds_k3, lds_v3);
      tile_step(tl, lds_k0, lds_v0, nullptr, nullptr, i);
      if (i + 1 < nt) tile_step(tl, lds_k1, lds_v1, nullptr, nullptr, i + 1);
      if (i + 2 >= nt) break;
      pair_barrier();
      load_tile(tl[i + 4 < nt ? i + 4 : nt - 1], lds_k0, lds_v0);
      load_tile(tl[i + 5 < nt ? i + 5 : nt - 1], lds_k1, lds_v1);
      tile_step(tl, lds_k2, lds_v2, nullptr, nullptr, i + 2);
      if (i + 3 < nt) tile_step(tl, lds_k3, lds_v3, nullptr, nullptr, i + 3);
      if (i + 4 >= nt) break;
      pair_barrier();
    }
  }
  // the repeat loads past the end must land before the workgroup's LDS can
  // be handed to another workgroup
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // ---------------------------------------------------------- epilogue
  float l_tot = l_run + __shfl_xor(l_run, 32);
  // register r of d-tile dt holds column 32dt + 16(r/8) + 8 half + r%8
  if (geo.splits > 1) {
    // Every split publishes its partial rows; the last split to finish
    // merges.  Publication uses device-scope (sc1) stores, drained with
    // s_waitcnt vmcnt(0) before the barrier that precedes the arrival
    // counter; the merger reads with device-scope loads.  No L2 writeback or
    // invalidate is needed, so the K/V lines other workgroups share in L2
    // survive.  Only a workgroup with this same row-to-lane mapping reads
    // the partials back, so they are stored lane-major -- [split][work
    // item][16-byte chunk][thread] -- and every store and load instruction
    // covers 1 KB per wave; (max, sum) pairs are stored per row.
    const int64_t item = (((int64_t)bi * a.Hkv + h) * a.n_chunks + ch) * geo.n_qtiles + qt;
    auto region = [&](int s) {
      return dev_rsrc(a.ws_o + ((int64_t)s * geo.n_items + item) * (kRows * kD),
                      (uint32_t)(kRows * kD * sizeof(float)));
    };
    auto ml_at = [&](int s) { return a.ws_ml + 2 * (((int64_t)s * geo.n_items + item) * kRows + row); };
    const uint32_t lane_off = (uint32_t)tid * 16;
    {
      const __amdgpu_buffer_rsrc_t r = region(split);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = acc[dt][4 * q4 + j];
          st4_dev(r, lane_off + (uint32_t)((4 * dt + q4) * kThreads * 16), v);
        }
      if (half == 0) {
        st_dev(ml_at(split), m_run);
        st_dev(ml_at(split) + 1, l_tot);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
      const int done = __hip_atomic_fetch_add(&a.ws_count[item], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      last_sh = done == geo.splits - 1;
      if (last_sh)   // ready for the next call
        __hip_atomic_store(&a.ws_count[item], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_sh || !row_ok) return;
    // merge: own registers + the other splits' published rows
    float M = m_run;
    for (int s2 = 0; s2 < geo.splits; ++s2)
      if (s2 != split) M = fmaxf(M, ld_dev(ml_at(s2)));
    // splits are summed in index order whichever one merges, so the result
    // does not depend on arrival order
    const float mu = M == -INFINITY ? 0.f : M;
    f32x16 res[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) res[dt] = f32x16{};
    float l_sum = 0.f;
    for (int s2 = 0; s2 < geo.splits; ++s2) {
      if (s2 == split) {
        const float w = __builtin_amdgcn_exp2f(m_run - mu);
        l_sum = fmaf(l_tot, w, l_sum);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int j = 0; j < 16; ++j) res[dt][j] = fmaf(acc[dt][j], w, res[dt][j]);
        continue;
      }
      const float w = __builtin_amdgcn_exp2f(ld_dev(ml_at(s2)) - mu);
      l_sum = fmaf(ld_dev(ml_at(s2) + 1), w, l_sum);
      const __amdgpu_buffer_rsrc_t r = region(s2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = ld4_dev(r, lane_off + (uint32_t)((4 * dt + q4) * kThreads * 16));
#pragma unroll
          for (int j = 0; j < 4; ++j) res[dt][4 * q4 + j] = fmaf(v[j], w, res[dt][4 * q4 + j]);
        }
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = res[dt];
    l_tot = l_sum;
    m_run = M;
  }
  const int64_t pos = (int64_t)ch * a.L + q_first + qi;     // row within this call
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
  if (tuning().prefill_splits > 0) return tuning().prefill_splits;   // override
  const int G = a.Hq / a.Hkv;
  const int TQ = kRows / G;
  const int64_t wgs = (int64_t)((a.L + TQ - 1) / TQ) * a.n_chunks * a.Hkv * a.batch;
  const int tiles = max_tiles(a, TQ);
  int s = 1;
  while (wgs * s < 256 && tiles / (2 * s) >= 8 && s < 8) s *= 2;
  return s;
}

int64_t prefill_partial_rows(const AttendArgs& a) { return prefill_num_counters(a) * kRows; }

int64_t prefill_num_counters(const AttendArgs& a) {
  const int TQ = kRows / (a.Hq / a.Hkv);
  return (int64_t)((a.L + TQ - 1) / TQ) * a.n_chunks * a.Hkv * a.batch;
}

template <int G, bool ROPE>
static void launch_gr(const AttendArgs& a, int splits, hipStream_t st) {
  constexpr int TQ = kRows / G;
  PrefillGeom geo;
  geo.TQ = TQ;
  geo.n_qtiles = (a.L + TQ - 1) / TQ;
  geo.splits = splits;
  geo.per_group = geo.n_qtiles * a.n_chunks * splits;
  const int groups = a.Hkv * a.batch;
  geo.n_items = geo.n_qtiles * a.n_chunks * groups;
  geo.xcd_groups = groups % kXcds == 0;
  k_attend_prefill<G, ROPE><<<dim3(geo.per_group * groups), kThreads, 0, st>>>(a, geo);
}

template <int G>
static void launch_g(const AttendArgs& a, int splits, hipStream_t st) {
  if (a.rope_theta > 0.0) launch_gr<G, true>(a, splits, st);
  else launch_gr<G, false>(a, splits, st);
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
