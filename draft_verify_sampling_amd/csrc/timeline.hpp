// Optional in-kernel timestamps, for the time lines of the tree walk, the
// softmax statistics (all rows, and the lazy chain statistics) and the chain
// draw.  Compiled in only with -DSV_TIMELINE (python -m
// draft_verify_sampling_amd.build --timeline builds that copy of the library,
// libspecverify_timeline.so); the normal library has none of it.
//
// A record is a fixed number of 64-bit readings of the 100 MHz real-time
// counter (s_memrealtime), 0 where a point was not reached.  Each translation
// unit that stamps keeps its own record arrays (device code is not linked
// across translation units) and exports a reader and a clearer for each.
#pragma once

#include <cstdint>

namespace sv {

constexpr int kTimelineSlots = 64;
constexpr int kTimelineRecords = 16384;

__device__ __forceinline__ uint64_t timeline_now() { return __builtin_amdgcn_s_memrealtime(); }

}  // namespace sv

#ifdef SV_TIMELINE
// A record array `name` of `records` records of `slots` readings, with its
// host reader and clearer: extern "C" int <name>_read(unsigned long long* host,
// int64_t records) copies the first `records` records, and extern "C" int
// <name>_clear(void) zeroes the array; both synchronous, returning a
// hipError_t.
#define SV_TIMELINE_ARRAY_SIZED(name, records, slots)                                                   \
  constexpr int64_t name##_nrec = (records);                                                            \
  constexpr int64_t name##_nslot = (slots);                                                             \
  __device__ uint64_t name##_records[(records) * (slots)];                                              \
  extern "C" int name##_read(unsigned long long* host, int64_t n) {                                     \
    if (n < 0 || n > name##_nrec) return static_cast<int>(hipErrorInvalidValue);                        \
    return static_cast<int>(                                                                            \
        hipMemcpyFromSymbol(host, HIP_SYMBOL(name##_records), sizeof(uint64_t) * name##_nslot * n));    \
  }                                                                                                     \
  extern "C" int name##_clear(void) {                                                                   \
    void* p = nullptr;                                                                                  \
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(name##_records));                                 \
    if (e == hipSuccess) e = hipMemset(p, 0, sizeof(name##_records));                                   \
    if (e == hipSuccess) e = hipDeviceSynchronize();                                                    \
    return static_cast<int>(e);                                                                         \
  }
#define SV_TIMELINE_ARRAY(name) SV_TIMELINE_ARRAY_SIZED(name, sv::kTimelineRecords, sv::kTimelineSlots)
// Store the counter into slot `slot` of record `rec` of array `array` (from
// the calling thread; records past the array are dropped).
#define SV_STAMP(array, rec, slot)                                                                      \
  do {                                                                                                  \
    const int64_t sv_r_ = (rec);                                                                        \
    if (sv_r_ >= 0 && sv_r_ < array##_nrec) array##_records[sv_r_ * array##_nslot + (slot)] = sv::timeline_now(); \
  } while (0)
#else
#define SV_TIMELINE_ARRAY_SIZED(name, records, slots)
#define SV_TIMELINE_ARRAY(name)
#define SV_STAMP(array, rec, slot) ((void)0)
#endif
