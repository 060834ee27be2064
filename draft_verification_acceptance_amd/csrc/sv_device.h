// Device helpers of libspecverify (gfx950, wave64).
#pragma once

#include "sv_internal.h"

namespace sv {

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element access for the two logit dtypes. A 16-byte vector holds 8 bf16 or 4 fp32 logits.
template <typename DT>
struct Elem;

template <>
struct Elem<uint16_t> {
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ float load(const uint16_t* p, int64_t i) {
    return __uint_as_float(uint32_t(p[i]) << 16);
  }
  __device__ static __forceinline__ void unpack(const uint4& q, float* x) {
    x[0] = bf_lo(q.x); x[1] = bf_hi(q.x); x[2] = bf_lo(q.y); x[3] = bf_hi(q.y);
    x[4] = bf_lo(q.z); x[5] = bf_hi(q.z); x[6] = bf_lo(q.w); x[7] = bf_hi(q.w);
  }
};

template <>
struct Elem<float> {
  static constexpr int kPerVec = 4;
  __device__ static __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void unpack(const uint4& q, float* x) {
    x[0] = __uint_as_float(q.x); x[1] = __uint_as_float(q.y);
    x[2] = __uint_as_float(q.z); x[3] = __uint_as_float(q.w);
  }
};

// A 16-byte load that bypasses cache retention: every logit is read once per pass.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// v_exp_f32: 2^x (inputs below -126 give 0 or a denormal; such masses never matter at fp32 resolution).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Greedy candidate order: larger value first, then lower index.
__device__ __forceinline__ bool better(float va, int32_t ia, float vb, int32_t ib) {
  return va > vb || (va == vb && ia < ib);
}

// Merge two (max, sum of exp2(x - max)) pairs. An empty side has m = -inf and z = 0.
__device__ __forceinline__ void merge_mz(float& m, float& z, float m2, float z2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) {
    z = z + z2;
    return;
  }
  // An empty side (m = -inf) has z = 0, or NaN when a NaN logit poisoned it: add it unscaled.
  const float a = (m == -INFINITY) ? z : z * exp2_fast(m - M);
  const float c = (m2 == -INFINITY) ? z2 : z2 * exp2_fast(m2 - M);
  m = M;
  z = a + c;
}

// Caller uniform -> value used: NaN -> 0, outside [0,1) -> clamped to [0, 1 - 2^-24]; `bad` reports both.
__device__ __forceinline__ float sanitize_u(float u, bool& bad) {
  if (!(u == u)) {
    bad = true;
    return 0.f;
  }
  if (u >= 0.f && u < 1.f) return u;
  bad = true;
  return fminf(fmaxf(u, 0.f), 0x1.fffffep-1f);
}

// Cross-workgroup hand-off without cache-wide fences. Partial results travel through agent-scope
// atomic stores and loads (coherent across the XCDs' separate L2s) and a per-request completion counter;
// the writer waits for its stores to complete before counting, so the workgroup that sees the final count
// reads complete partials.
__device__ __forceinline__ void store_agent(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long load_agent(unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every memory operation this thread issued has completed (vmcnt = lgkmcnt = expcnt = 0); also keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void complete_memory_ops() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Vocab mask rows: bit (v % 32) of word v / 32 is 1 iff token v is allowed. mask_bits8 returns the bits of
// tokens [v, v + 8) (bit i = token v + i) for any v < V with two word loads and no branch (a load under a
// branch would cost the stream a wait for every load in flight); mask_bits8_aligned is the one-load form
// for v % 8 == 0 (and, for the 4 bits of an fp32 run, v % 4 == 0), where the bits lie in one word.
__device__ __forceinline__ uint32_t mask_bits8(const uint32_t* mrow, int64_t v, int64_t nwords) {
  const int64_t w = v >> 5;
  const uint32_t lo = mrow[w];
  const uint32_t hi = mrow[w + 1 < nwords ? w + 1 : w];
  return uint32_t(((uint64_t(hi) << 32) | lo) >> (v & 31));
}

__device__ __forceinline__ uint32_t mask_bits8_aligned(const uint32_t* mrow, int64_t v) {
  return mrow[v >> 5] >> uint32_t(v & 31);
}

__device__ __forceinline__ bool mask_allows(const uint32_t* mrow, int64_t v) { return (mrow[v >> 5] >> (v & 31)) & 1u; }

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Maximum and sum over the 64 lanes of a wave, the result in every lane: a butterfly inside each 16-lane
// row (DPP quad permutes [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors), then the four row
// results read out. Every lane must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_lanes(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(row_lanes(v, 0), row_lanes(v, 16)), fmaxf(row_lanes(v, 32), row_lanes(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (row_lanes(v, 0) + row_lanes(v, 16)) + (row_lanes(v, 32) + row_lanes(v, 48));
}

// The same for float64 (each DPP move takes one 32-bit half), and an inclusive prefix sum: a Hillis-Steele
// scan inside each 16-lane row (DPP row shifts by 1, 2, 4, 8; lanes shifted in from outside the row read 0),
// then the totals of the rows before added in. Every lane must be active.
template <int CTRL, bool ZERO_OUTSIDE>
__device__ __forceinline__ double dpp_d(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(b)), CTRL, 0xF, 0xF, ZERO_OUTSIDE);
  const int hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(b >> 32)), CTRL, 0xF, 0xF, ZERO_OUTSIDE);
  return __longlong_as_double((long long)((unsigned long long)uint32_t(hi) << 32 | uint32_t(lo)));
}
__device__ __forceinline__ double row_lanes_d(double v, int l) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b >> 32)), l));
  return __longlong_as_double((long long)((unsigned long long)hi << 32 | lo));
}
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_d<0xB1, false>(v);
  v += dpp_d<0x4E, false>(v);
  v += dpp_d<0x141, false>(v);
  v += dpp_d<0x140, false>(v);
  return (row_lanes_d(v, 0) + row_lanes_d(v, 16)) + (row_lanes_d(v, 32) + row_lanes_d(v, 48));
}
__device__ __forceinline__ double wave_inclusive_sum_dpp(double v) {
  v += dpp_d<0x111, true>(v);
  v += dpp_d<0x112, true>(v);
  v += dpp_d<0x114, true>(v);
  v += dpp_d<0x118, true>(v);
  const double r0 = row_lanes_d(v, 15), r1 = row_lanes_d(v, 31), r2 = row_lanes_d(v, 47);
  const int row = int(threadIdx.x & (kWave - 1)) >> 4;
  const double before = row == 0 ? 0.0 : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
  return v + before;
}

// The same inclusive prefix sum for int.
__device__ __forceinline__ int wave_inclusive_sum_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = int(threadIdx.x & (kWave - 1)) >> 4;
  return v + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2);
}

// And for uint64 (each DPP move takes one 32-bit half; the sums are exact modulo 2^64).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(v)), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(v >> 32)), CTRL, 0xF, 0xF, true);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), l));
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_inclusive_sum_dpp(uint64_t v) {
  v += dpp_u64<0x111>(v);
  v += dpp_u64<0x112>(v);
  v += dpp_u64<0x114>(v);
  v += dpp_u64<0x118>(v);
  const uint64_t r0 = readlane_u64(v, 15), r1 = readlane_u64(v, 31), r2 = readlane_u64(v, 47);
  const int row = int(threadIdx.x & (kWave - 1)) >> 4;
  return v + (row == 0 ? 0ull : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Block-wide min over NT threads; every thread gets the result. `red` holds >= NT / 64 ints of LDS.
template <int NT = kThreads>
__device__ __forceinline__ int block_min_i(int v, int* red) {
  v = wave_min_i(v);
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) r = min(r, red[w]);
  __syncthreads();
  return r;
}

template <int NT = kThreads>
__device__ __forceinline__ int block_max_i(int v, int* red) {
  v = wave_max_i(v);
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) r = max(r, red[w]);
  __syncthreads();
  return r;
}

// Inclusive wave prefix sum (lane order).
template <typename T>
__device__ __forceinline__ T wave_inclusive_sum(T v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    T n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  return v;
}

// Block prefix sums of doubles over kThreads threads. The bounds are consistent: thread t's `incl` is
// bit-identical to thread t+1's `excl`, so [excl, incl) ranges partition [0, total).
__device__ __forceinline__ void block_scan_d(double v, double* red, double& excl, double& incl, double& total) {
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const double inc = wave_inclusive_sum_dpp(v);
  const double prev = dpp_d<0x138, true>(inc);   // wave_shr:1, lane i reads lane i - 1's value exactly
  __syncthreads();
  if (lane == kWave - 1) red[w] = inc;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) {
    if (i < w) base = base + red[i];
    tot = tot + red[i];
  }
  __syncthreads();
  total = tot;
  excl = lane == 0 ? base : base + prev;
  incl = base + inc;
}

}  // namespace sv
