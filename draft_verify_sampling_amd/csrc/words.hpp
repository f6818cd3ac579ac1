// 64-bit words that carry data between workgroups of one kernel: each is
// stored with a relaxed agent-scope atomic store and polled with relaxed
// agent-scope atomic loads until its bit 63 is set, so the data itself travels
// inside the atomic word and no fence is needed.  A word is zero before its
// writer stores it: zeroed before the kernel, or (tree walks) by its writer,
// whose completed zeroing a per-call ticket certifies.
#pragma once

#include "common.hpp"

namespace sv {

constexpr uint64_t kValid = 1ull << 63;

// A softmax pair (s >= 0 or NaN frees the sign bit of s).
__device__ __forceinline__ uint64_t enc_ms(MS v) {
  return (static_cast<uint64_t>(__float_as_uint(v.s) | 0x80000000u) << 32) | __float_as_uint(v.m);
}
__device__ __forceinline__ MS dec_ms(uint64_t w) {
  return MS{__uint_as_float(static_cast<uint32_t>(w)),
            __uint_as_float(static_cast<uint32_t>(w >> 32) & 0x7fffffffu)};
}
// A sum of non-negative terms (or NaN): its sign bit carries the valid bit.
__device__ __forceinline__ uint64_t enc_sum(double x) {
  if (isnan(x)) return 0xfff8000000000001ull;
  return static_cast<uint64_t>(__double_as_longlong(x)) | kValid;
}
__device__ __forceinline__ double dec_sum(uint64_t w) {
  return __longlong_as_double(static_cast<long long>(w & ~kValid));
}
// Class of a partial sum of a draft row: NaN, +inf, -inf.  The row's total is
// NaN iff some part is NaN or the parts hold both infinities.
__device__ __forceinline__ uint64_t enc_qclass(double q) {
  return kValid | (isnan(q) ? 1u : 0u) | (q == INFINITY ? 2u : 0u) | (q == -INFINITY ? 4u : 0u);
}
__device__ __forceinline__ bool qclass_nan(uint64_t cls) { return (cls & 1u) || ((cls & 2u) && (cls & 4u)); }

__device__ __forceinline__ void store_word(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_word(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sv
