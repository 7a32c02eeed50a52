// Device helpers shared by the gfx950 kernels of libinfllm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infllm {

typedef uint16_t bf16_t;  // bf16 stored as its 16-bit pattern
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(bf16_t, h);
}

// Unit table and eligibility, host and device.  Unit u is absolute block
// j = u + floor(n_init/B) with keys [max(j*B, n_init), (j+1)*B).
__host__ __device__ __forceinline__ int64_t unit_first_key(int64_t u, int B, int n_init) {
  int64_t j = u + n_init / B;
  int64_t lo = j * B;
  return lo > n_init ? lo : n_init;
}

// Units whose first key lies at or before t_last - W (a prefix of [0, U)).
// lo(0) = n_init and lo(u) = (u + n_init/B)*B for u >= 1.
__host__ __device__ __forceinline__ int64_t eligible_units(int64_t t_last, int64_t U, int B,
                                                          int n_init, int W) {
  int64_t x = t_last - W;
  if (U <= 0 || x < n_init) return 0;
  int64_t e = x / B - n_init / B + 1;
  return e < U ? e : U;
}

// Per-sequence positions (variable-length batches).  Positions are kept
// below 2^31 - 128 so that key indices and tile ends fit 32 bits.
constexpr int64_t kPosLimit = ((int64_t)1 << 31) - 128;

// Whether a sequence whose first query sits at `base` can hold `n_pos`
// query positions in a KV buffer of kv_cap rows.
__host__ __device__ __forceinline__ bool seq_pos_ok(int64_t base, int64_t n_pos, int64_t kv_cap) {
  return base >= 0 && base <= kv_cap - n_pos && base <= kPosLimit - n_pos;
}

// First query position of sequence bi: the per-sequence array when there is
// one (read through the scalar cache, uniform per workgroup), else the
// call's single position.
__device__ __forceinline__ int64_t seq_base(const int64_t* pos, int64_t q_pos, int bi) {
  return pos ? pos[bi] : q_pos;
}

// Output rows [row0, row0 + n_rows) of query heads [qh0, qh0 + n_heads) set
// to NaN (and their log-sum-exp, if any): what a sequence with an invalid
// position receives.  Executed by the n_threads threads of a workgroup.
template <typename T>
__device__ __forceinline__ void nan_rows(T* out, float* lse, int64_t qh0, int n_heads,
                                         int64_t out_cap, int64_t row0, int n_rows, int D,
                                         int tid, int n_threads) {
  const float nan = __builtin_nanf("");
  const int per_head = n_rows * D;
  for (int i = tid; i < n_heads * per_head; i += n_threads) {
    const int g = i / per_head, r = (i % per_head) / D, c = i % D;
    const int64_t row = (qh0 + g) * out_cap + row0 + r;
    out[row * D + c] = from_f32<T>(nan);
    if (lse && c == 0) lse[row] = nan;
  }
}

// A selection is a set of units (the working context is a set of keys): an
// id repeated in one row of a selection counts once.  Every thread of the
// workgroup calls this (it synchronises); thread m < n passes entry m (u;
// -1 = empty slot) and gets u back, or -1 if an earlier entry holds the
// same id.  ids_sm: LDS for n ids.  Ascending ids (what the top-k calls
// write) are recognised with one comparison per entry; other orders pay a
// scan of the earlier entries.
__device__ __forceinline__ int32_t drop_repeats(int32_t u, int m, int n, int32_t* ids_sm) {
  if (m < n) ids_sm[m] = u;
  __syncthreads();
  const bool asc = !(m < n && m > 0 && u >= 0) || (ids_sm[m - 1] >= 0 && ids_sm[m - 1] < u);
  if (__syncthreads_count(!asc) > 0 && m < n && u >= 0) {
    for (int j = 0; j < m; ++j)
      if (ids_sm[j] == u) {
        u = -1;
        break;
      }
  }
  return u;
}

// Eight consecutive columns of a row, raw bits, widened to fp64 on use.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *(const u32x4*)p; }
  __device__ __forceinline__ void add(double* acc) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += (double)__uint_as_float(w[i] << 16);
      acc[2 * i + 1] += (double)__uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ void sub(double* acc) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] -= (double)__uint_as_float(w[i] << 16);
      acc[2 * i + 1] -= (double)__uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ double get(int i) const {
    return (double)__uint_as_float(i & 1 ? w[i / 2] & 0xffff0000u : w[i / 2] << 16);
  }
};
template <> struct Raw8<float> {
  float4 x, y;
  __device__ __forceinline__ void load(const float* p) {
    x = ((const float4*)p)[0];
    y = ((const float4*)p)[1];
  }
  __device__ __forceinline__ void add(double* acc) const {
    acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
    acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
  }
  __device__ __forceinline__ void sub(double* acc) const {
    acc[0] -= x.x; acc[1] -= x.y; acc[2] -= x.z; acc[3] -= x.w;
    acc[4] -= y.x; acc[5] -= y.y; acc[6] -= y.z; acc[7] -= y.w;
  }
  __device__ __forceinline__ double get(int i) const {
    const float v[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    return (double)v[i];
  }
};

// ------------------------------------------------------------ lane shuffles
// DPP controls (gfx9 encoding): quad_perm [1,0,3,2], [2,3,0,1]; row_half_mirror;
// row_mirror.  Applied in this order they all-reduce a 16-lane row.
#define INFLLM_DPP_XOR1 0xB1
#define INFLLM_DPP_XOR2 0x4E
#define INFLLM_DPP_HALF_MIRROR 0x141
#define INFLLM_DPP_MIRROR 0x140

template <int CTRL> __device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

template <int CTRL> __device__ __forceinline__ double dpp_f64(double x) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), CTRL, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<INFLLM_DPP_XOR1>(x);
  x += dpp_f32<INFLLM_DPP_XOR2>(x);
  x += dpp_f32<INFLLM_DPP_HALF_MIRROR>(x);
  x += dpp_f32<INFLLM_DPP_MIRROR>(x);
  return x;
}

__device__ __forceinline__ double shfl_xor_f64(double x, int m) {
  int lo = __double2loint(x), hi = __double2hiint(x);
  lo = __shfl_xor(lo, m);
  hi = __shfl_xor(hi, m);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += shfl_xor_f64(x, m);
  return x;
}

// Max / sum over the wave: DPP within each 16-lane row, then the four row
// results read into scalars (a fixed order: deterministic sums).
__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f32<INFLLM_DPP_XOR1>(x));
  x = fmaxf(x, dpp_f32<INFLLM_DPP_XOR2>(x));
  x = fmaxf(x, dpp_f32<INFLLM_DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp_f32<INFLLM_DPP_MIRROR>(x));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  x = row16_sum(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

// Sum over the wave in a fixed order without LDS round trips: DPP sums
// within each 16-lane row, then the four row sums read into scalars.
__device__ __forceinline__ double readlane_f64(double x, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), l);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_sum_f64_dpp(double x) {
  x += dpp_f64<INFLLM_DPP_XOR1>(x);
  x += dpp_f64<INFLLM_DPP_XOR2>(x);
  x += dpp_f64<INFLLM_DPP_HALF_MIRROR>(x);
  x += dpp_f64<INFLLM_DPP_MIRROR>(x);
  return (readlane_f64(x, 0) + readlane_f64(x, 16)) + (readlane_f64(x, 32) + readlane_f64(x, 48));
}

// ------------------------------------------------ cross-workgroup publication
// Split-K partial results are handed from one workgroup to another without
// device-scope fences (on gfx950 a __threadfence() writes back and
// invalidates the L2, evicting what other workgroups share there).  Writers
// use device-scope (sc1) stores and drain them with s_waitcnt vmcnt(0)
// before the barrier that precedes their arrival-counter increment; the
// last arriver reads with device-scope loads.

// s_waitcnt immediate (gfx9 encoding) for vmcnt(0), expcnt/lgkmcnt untouched
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte device-scope accesses through a raw buffer resource (cache policy
// sc1); `bytes` bounds the range, checked by the hardware.
constexpr int kCachePolicySc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void st4_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCachePolicySc1);
}
__device__ __forceinline__ float ld1_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  // past the resource's range the hardware returns 0 (no fault)
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCachePolicySc1));
}
__device__ __forceinline__ double ld1_dev_f64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCachePolicySc1));
}
__device__ __forceinline__ f32x4 ld4_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicySc1));
}

// Order-preserving map of an fp32 to uint32 (larger float -> larger key);
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace infllm
