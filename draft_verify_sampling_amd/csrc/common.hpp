// Device helpers shared by the verify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kBlock = 256;            // threads per block for the streaming kernels
constexpr int kWave = 64;
constexpr float kLn2 = 0.6931471805599453f;


// Status bits (the public header documents them).
constexpr int kFlagBadRequest = 1;
constexpr int kFlagBadToken = 2;
constexpr int kFlagNonfinite = 4;
constexpr int kFlagOverBudget = 8;
constexpr int kFlagFallback = 16;
constexpr int kFlagBadTree = 32;
constexpr int kFlagSyncTimeout = 64;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Element formats.  A 16-byte vector holds kPerVec elements.
// ---------------------------------------------------------------------------
struct F32 {
  static constexpr int kSize = 4;
  static constexpr int kPerVec = 4;
  __device__ __forceinline__ static float at(const void* row, int64_t i) {
    return static_cast<const float*>(row)[i];
  }
  __device__ __forceinline__ static void unpack(const uint4& w, float* v) {
    v[0] = __uint_as_float(w.x);
    v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z);
    v[3] = __uint_as_float(w.w);
  }
};

struct BF16 {
  static constexpr int kSize = 2;
  static constexpr int kPerVec = 8;
  // bfloat16 -> float is exact: the pattern is the upper half of a float.
  __device__ __forceinline__ static float at(const void* row, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[i]) << 16);
  }
  __device__ __forceinline__ static void unpack(const uint4& w, float* v) {
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xffff0000u);
    v[4] = __uint_as_float(w.z << 16);
    v[5] = __uint_as_float(w.z & 0xffff0000u);
    v[6] = __uint_as_float(w.w << 16);
    v[7] = __uint_as_float(w.w & 0xffff0000u);
  }
};

template <class D>
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t row, int64_t V) {
  return static_cast<const char*>(base) + row * V * D::kSize;
}

// Number of leading elements of a row before its first 16-byte boundary.
template <class D>
__device__ __forceinline__ int64_t head_elems(const void* row, int64_t V) {
  int64_t h = static_cast<int64_t>((16u - (reinterpret_cast<uintptr_t>(row) & 15u)) & 15u) / D::kSize;
  return h < V ? h : V;
}

// ---------------------------------------------------------------------------
// Online softmax pairs over scaled scores y = l * c (c = log2(e) / T):
// m = max of the rounded products l * c, s = sum 2^(l * c - m) with each term
// formed by one fused multiply-add.  Because m is itself a representable value
// of the scaled domain, merging two pairs rescales by 2^(m_a - M) with the
// dominant side's factor exactly 1, so no rounding of the max leaks into s.
// Every multiply-add that is meant to be fused is written as fmaf, and the
// library is built without implicit contraction, so each kernel that forms a
// pair or a weight rounds exactly alike.
// ---------------------------------------------------------------------------
struct MS {
  float m;
  float s;
};

__device__ __forceinline__ MS ms_combine(MS a, MS b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return MS{M, 0.f};
  return MS{M, fmaf(a.s, ex2(a.m - M), b.s * ex2(b.m - M))};
}

// Fold n raw scores into a running pair: one rescale per group, pairwise group sum.
template <int n>
__device__ __forceinline__ void ms_fold(MS& acc, const float* x, float c) {
  float cm = x[0];
#pragma unroll
  for (int j = 1; j < n; ++j) cm = fmaxf(cm, x[j]);
  const float M = fmaxf(acc.m, cm * c);
  if (M == -INFINITY) return;
  float e[n];
#pragma unroll
  for (int j = 0; j < n; ++j) e[j] = ex2(fmaf(x[j], c, -M));
#pragma unroll
  for (int w = 1; w < n; w *= 2) {
#pragma unroll
    for (int j = 0; j + w < n; j += 2 * w) e[j] += e[j + w];
  }
  acc.s = fmaf(acc.s, ex2(acc.m - M), e[0]);
  acc.m = M;
}

// ---------------------------------------------------------------------------
// Wave-level scans with DPP lane moves (GFX9 row shifts and row broadcasts):
// each step is a register move between lanes, no LDS round trip.  Lanes whose
// source is outside the move's reach read `ident`.
// ---------------------------------------------------------------------------
template <int ctrl, int row_mask>
__device__ __forceinline__ float dpp_f(float v, float ident) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(v), ctrl,
                                                    row_mask, 0xf, false));
}

template <int ctrl, int row_mask>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), ctrl, row_mask, 0xf, false));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), ctrl, row_mask, 0xf, false));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

template <int ctrl, int row_mask>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), ctrl, row_mask, 0xf, false));
}

// Largest value over the wave's lanes (0 is the identity), valid in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xf>(v));  // row_shr:1
  v = max(v, dpp_u32<0x112, 0xf>(v));  // row_shr:2
  v = max(v, dpp_u32<0x114, 0xf>(v));  // row_shr:4
  v = max(v, dpp_u32<0x118, 0xf>(v));  // row_shr:8
  v = max(v, dpp_u32<0x142, 0xa>(v));  // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_u32<0x143, 0xc>(v));  // row_bcast:31 into rows 2 and 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), kWave - 1));
}

// Largest 64-bit key over the wave (0 is the identity), valid in every lane:
// the largest high word, then the largest low word among the lanes holding it.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = static_cast<uint32_t>(v >> 32);
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? static_cast<uint32_t>(v) : 0u);
  return (static_cast<uint64_t>(mh) << 32) | ml;
}

// Inclusive prefix sum over the 64 lanes of a wave (lane order).
__device__ __forceinline__ double wave_incl_scan(double x) {
  x += dpp_d<0x111, 0xf>(x);  // row_shr:1
  x += dpp_d<0x112, 0xf>(x);  // row_shr:2
  x += dpp_d<0x114, 0xf>(x);  // row_shr:4
  x += dpp_d<0x118, 0xf>(x);  // row_shr:8
  x += dpp_d<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_d<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

__device__ __forceinline__ double lane_value(double x, int lane) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), lane);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Sum over the wave, valid in every lane.
__device__ __forceinline__ double wave_total(double x) { return lane_value(wave_incl_scan(x), kWave - 1); }

// Online-softmax pair over the wave, valid in every lane.
__device__ __forceinline__ MS wave_ms_dpp(MS v) {
#define SV_MS_STEP(ctrl, rm)                                                     \
  v = ms_combine(v, MS{dpp_f<ctrl, rm>(v.m, -INFINITY), dpp_f<ctrl, rm>(v.s, 0.f)});
  SV_MS_STEP(0x111, 0xf)
  SV_MS_STEP(0x112, 0xf)
  SV_MS_STEP(0x114, 0xf)
  SV_MS_STEP(0x118, 0xf)
  SV_MS_STEP(0x142, 0xa)
  SV_MS_STEP(0x143, 0xc)
#undef SV_MS_STEP
  return MS{__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.m), kWave - 1)),
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.s), kWave - 1))};
}

// Canonical combine of n per-segment pairs, shared by every consumer that
// must agree bit for bit: lane l folds segments l, l + 64, l + 128, ... in
// order, then the wave combines its lanes (wave_ms_dpp).  Valid in every lane
// of the calling wave.  `pair(s)` returns segment s's pair.
template <class Pair>
__device__ __forceinline__ MS wave_combine_segments(int n, Pair pair) {
  const int lane = threadIdx.x & (kWave - 1);
  MS acc{-INFINITY, 0.f};
  for (int s = lane; s < n; s += kWave) acc = ms_combine(acc, pair(s));
  return wave_ms_dpp(acc);
}

__device__ __forceinline__ void flag(int32_t* status, int bits) {
  if (status != nullptr && bits != 0) atomicOr(status, bits);
}

// ---- counter-based uniforms: Philox4x64-10 ----
// Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
// 3" (SC 2011): ten rounds of two 64 x 64 -> 128-bit products of counter
// words with the multipliers, high halves xored with the other words and the
// round keys, the words permuted, the key bumped by the Weyl constants.
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ void philox4x64_10(uint64_t& x0, uint64_t& x1, uint64_t& x2, uint64_t& x3,
                                              uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kPhiloxM0, x0), lo0 = kPhiloxM0 * x0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, x2), lo1 = kPhiloxM1 * x2;
    const uint64_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
    x0 = y0;
    x1 = lo1;
    x2 = y2;
    x3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
}

// Uniform of slot i of request b: word i mod 4 of the Philox block at
// counter (i div 4, b, offset, 0) under key (seed, 0), its top 24 bits
// times 2^-24 (a value on the 2^-24 grid in [0, 1), exact in float).
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t offset, int64_t b, int i) {
  uint64_t x0 = static_cast<uint64_t>(i) >> 2, x1 = static_cast<uint64_t>(b), x2 = offset, x3 = 0;
  philox4x64_10(x0, x1, x2, x3, seed, 0);
  const int w = i & 3;
  const uint64_t v = w == 0 ? x0 : (w == 1 ? x1 : (w == 2 ? x2 : x3));
  return static_cast<float>(v >> 40) * 0x1p-24f;
}

// Uniform slot i of request b: the caller's array u [B, slots], or the
// Philox stream (seed, offset) when u is null.
__device__ __forceinline__ float slot_uniform(const float* u, uint64_t seed, uint64_t offset, int64_t b,
                                              int slots, int i) {
  return u != nullptr ? u[b * slots + i] : philox_uniform(seed, offset, b, i);
}

}  // namespace sv
