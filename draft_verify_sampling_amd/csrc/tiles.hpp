// Tile-level steps of an inverse-CDF draw over one vocabulary row, shared by
// the chain and the tree verify kernels.  A tile is kSampleTile = 2048
// consecutive ids and one wave handles one tile.
//
// Draw weights of a row: p = 2^(l c - Mc) / S, the temperature softmax of the
// target logits l (c = log2(e) / T, Mc the row's scaled-domain max, S its
// normaliser), either as they are or as the residual w = max(0, p - coef q)
// against the draft probabilities q ("投机解码:为什么一个字都不改", section
// "改进:接受概率 min(1, p/q),拒绝时从残差重采"; the tree walk of "Speculative
// Decoding II", EAGLE section, applies it with a growing coef).  The drawn id
// is the smallest one whose running weight exceeds u times the total weight:
// ids of weight zero are never drawn, and when rounding leaves the target at or
// beyond the last running sum the last id of positive weight is taken.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace sv {

struct DrawRow {
  const void* t;   // target logits of the row
  const void* q;   // draft probabilities of the row, read only when use_q
  float c;         // log2(e) / T
  float Mc;        // scaled-domain max of the target row
  float invS;      // 1 / softmax normaliser of the target row
  float coef;      // residual coefficient
  bool use_q;      // true: w = max(0, p - coef q); false: w = p
  const int32_t* excl = nullptr;  // ids whose weight is 0 (point-mass residual),
  int nexcl = 0;                  // honoured by the one-tile steps built with kExcl
};

template <int n>
__device__ __forceinline__ float pairwise(const float* x) {
  float t[n];
#pragma unroll
  for (int j = 0; j < n; ++j) t[j] = x[j];
#pragma unroll
  for (int w = 1; w < n; w *= 2) {
#pragma unroll
    for (int j = 0; j + w < n; j += 2 * w) t[j] += t[j + w];
  }
  return t[0];
}

template <class D>
__device__ __forceinline__ uint4 ld16(const void* row, int64_t e) {
  return *reinterpret_cast<const uint4*>(static_cast<const char*>(row) + e * D::kSize);
}

template <class D>
__device__ __forceinline__ bool aligned16(const void* row, int64_t e) {
  return ((reinterpret_cast<uintptr_t>(row) + e * D::kSize) & 15u) == 0;
}

// Shift a wave-inclusive scan into an exclusive one (lane 0 reads 0).
__device__ __forceinline__ double wave_exclusive_from_inclusive(double incl) {
  return dpp_d<0x138, 0xf>(incl);  // wave_shr:1
}

__device__ __forceinline__ float draw_p(const DrawRow& r, float l) {
  return ex2(fmaf(l, r.c, -r.Mc)) * r.invS;
}

__device__ __forceinline__ float draw_w(const DrawRow& r, float p, float q) {
  return r.use_q ? fmaxf(fmaf(-r.coef, q, p), 0.f) : p;
}

// Layout of a tile for the sums: runs of kPer consecutive elements (the wider
// of the two rows' 16-byte vector widths, so each row's share of a run is a
// whole number of vectors); lane l takes runs l, l + 64, l + 128, ... so every
// load instruction of the wave is coalesced.
template <class DT, class DQ>
struct TileRuns {
  static constexpr int kPer = DT::kPerVec > DQ::kPerVec ? DT::kPerVec : DQ::kPerVec;
  static constexpr int kRuns = kSampleTile / (kWave * kPer);  // runs per lane per tile
  static constexpr int nt = kPer * DT::kSize / 16;            // target vectors per run
  static constexpr int nq = kPer * DQ::kSize / 16;            // draft vectors per run
  static_assert(nt >= 1 && nq >= 1, "a run must cover whole vectors of both rows");
};

// An LDS copy of one tile's draw inputs under a residual pass: p (draw_p of
// each element) and the draft probability q, as floats, laid out as the tile
// sums visit them (run k, group j4 of four elements of the run, lane), so a
// later residual pass over the same row pair rebuilds the same weights in the
// same order, and so the same sums, without reading or exponentiating the
// rows again.  Elements beyond the row's end hold p = q = 0, which adds zero.
template <class DT, class DQ>
struct TileCache {
  using L = TileRuns<DT, DQ>;
  static constexpr int kVec = L::kPer / 4;                  // float4 per run and lane
  static constexpr int kFloat4 = L::kRuns * kVec * kWave;  // float4 per tile and array
  static_assert(L::kPer % 4 == 0, "runs of whole float4");
  float4* p = nullptr;
  float4* q = nullptr;
  __device__ __forceinline__ void put(int run, int lane, const float* pv, const float* qv) const {
#pragma unroll
    for (int j4 = 0; j4 < kVec; ++j4) {
      const int i = (run * kVec + j4) * kWave + lane;
      p[i] = make_float4(pv[4 * j4], pv[4 * j4 + 1], pv[4 * j4 + 2], pv[4 * j4 + 3]);
      q[i] = make_float4(qv[4 * j4], qv[4 * j4 + 1], qv[4 * j4 + 2], qv[4 * j4 + 3]);
    }
  }
  __device__ __forceinline__ void put_zero(int run, int lane) const {
#pragma unroll
    for (int j4 = 0; j4 < kVec; ++j4) {
      const int i = (run * kVec + j4) * kWave + lane;
      p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      q[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
};

// Sums (w, p, q) of tile t, in fp32 within a lane and fp64 across lanes; valid
// in every lane.  Handles any tile.  On 16-byte aligned rows every complete
// run is one predicated vector load, all in flight at once (the row's last
// partial tile costs one load round like any other); a run that the row's
// end cuts (rows whose length is not a multiple of the vector width) and
// unaligned rows take element loads.
// kFill: also leave the tile's p and q in `cache` (residual passes only).
// kPSum false: the p sum is not formed (v[1] = 0).  kQAlways: the row is a
// residual row (r.use_q holds), so w = max(0, p - coef q) without a select.
template <class DT, class DQ, bool kQ = true, bool kFill = false, bool kPSum = true, bool kQAlways = false>
__device__ __forceinline__ void wave_tile_sums_any(const DrawRow& r, int64_t V, int t, double* v,
                                                   TileCache<DT, DQ> cache = {}) {
  using L = TileRuns<DT, DQ>;
  constexpr int kPer = L::kPer;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t0 = static_cast<int64_t>(t) * kSampleTile;
  const bool use_q = kQ && (kQAlways || r.use_q);
  const bool al = aligned16<DT>(r.t, t0) && (!use_q || aligned16<DQ>(r.q, t0));
  float ws = 0.f, ps = 0.f, qs = 0.f;
  constexpr int kAB = (L::nt + L::nq == 2) ? 4 : 2;  // runs per load round (<= 8 vectors)
  static_assert(L::kRuns % kAB == 0, "whole rounds");
  if (al) {
#pragma unroll
    for (int k0 = 0; k0 < L::kRuns; k0 += kAB) {
    uint4 tw[kAB][L::nt], qw[kAB][L::nq];
#pragma unroll
    for (int kk = 0; kk < kAB; ++kk) {
      const int64_t e = t0 + static_cast<int64_t>((k0 + kk) * kWave + lane) * kPer;
      if (e + kPer <= V) {
#pragma unroll
        for (int j = 0; j < L::nt; ++j) tw[kk][j] = ld16<DT>(r.t, e + j * DT::kPerVec);
        if (use_q) {
#pragma unroll
          for (int j = 0; j < L::nq; ++j) qw[kk][j] = ld16<DQ>(r.q, e + j * DQ::kPerVec);
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < kAB; ++kk) {
      const int64_t e = t0 + static_cast<int64_t>((k0 + kk) * kWave + lane) * kPer;
      if (e >= V) continue;
      float l[kPer], q[kPer];
      if (e + kPer <= V) {
#pragma unroll
        for (int j = 0; j < L::nt; ++j) DT::unpack(tw[kk][j], l + j * DT::kPerVec);
        if (use_q) {
#pragma unroll
          for (int j = 0; j < L::nq; ++j) DQ::unpack(qw[kk][j], q + j * DQ::kPerVec);
        } else {
#pragma unroll
          for (int j = 0; j < kPer; ++j) q[j] = 0.f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const bool in = e + j < V;
          l[j] = in ? DT::at(r.t, e + j) : -INFINITY;
          q[j] = (in && use_q) ? DQ::at(r.q, e + j) : 0.f;
        }
      }
      float w[kPer], p[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        p[j] = draw_p(r, l[j]);
        w[j] = kQAlways ? fmaxf(fmaf(-r.coef, q[j], p[j]), 0.f) : draw_w(r, p[j], q[j]);
      }
      if constexpr (kFill) cache.put(k0 + kk, lane, p, q);
      ws += pairwise<kPer>(w);
      if constexpr (kPSum) ps += pairwise<kPer>(p);
      qs += pairwise<kPer>(q);
    }
    }
  } else {
#pragma unroll 1
    for (int k = 0; k < L::kRuns; ++k) {
      const int64_t e = t0 + static_cast<int64_t>(k * kWave + lane) * kPer;
      if (e >= V) break;
      float l[kPer], q[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const bool in = e + j < V;
        l[j] = in ? DT::at(r.t, e + j) : -INFINITY;
        q[j] = (in && use_q) ? DQ::at(r.q, e + j) : 0.f;
      }
      float w[kPer], p[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        p[j] = draw_p(r, l[j]);
        w[j] = kQAlways ? fmaxf(fmaf(-r.coef, q[j], p[j]), 0.f) : draw_w(r, p[j], q[j]);
      }
      if constexpr (kFill) cache.put(k, lane, p, q);
      ws += pairwise<kPer>(w);
      if constexpr (kPSum) ps += pairwise<kPer>(p);
      qs += pairwise<kPer>(q);
    }
  }
  if constexpr (kFill) {  // runs wholly beyond the row's end were skipped above
#pragma unroll 1
    for (int k = 0; k < L::kRuns; ++k)
      if (t0 + static_cast<int64_t>(k * kWave + lane) * kPer >= V) cache.put_zero(k, lane);
  }
  v[0] = wave_total(static_cast<double>(ws));
  v[1] = kPSum ? wave_total(static_cast<double>(ps)) : 0.0;
  v[2] = wave_total(static_cast<double>(qs));
}

// Sums (w, p, q) of the kT tiles t, t + tstride, ... into v[i]; all of a
// lane's loads for a batch of runs are in flight before the first is used.
// Falls back to wave_tile_sums_any tile by tile unless every tile is complete
// and the rows are 16-byte aligned.
// kMaxBatch (0: up to 16 vectors) caps the runs whose loads are in flight
// together, for callers that must keep registers low; the runs are summed in
// the same order either way, so the sums are the same bits.  kFill (one tile):
// also leave the tile's p and q in `cache`.  kPSum, kQAlways: as for
// wave_tile_sums_any.
template <class DT, class DQ, int kT, bool kQ = true, int kMaxBatch = 0, bool kFill = false, bool kPSum = true,
          bool kQAlways = false>
__device__ __forceinline__ void wave_tile_sums(const DrawRow& r, int64_t V, int t, int tstride,
                                               double (*v)[3], TileCache<DT, DQ> cache = {}) {
  static_assert(!kFill || kT == 1, "the cache holds one tile");
  using L = TileRuns<DT, DQ>;
  constexpr int kPer = L::kPer;
  constexpr int kAll = kT * L::kRuns;                           // runs per lane in total
  constexpr int kCap0 = (L::nt + L::nq == 2) ? 8 : 4;           // runs per batch (<= 16 vectors)
  constexpr int kCap = (kMaxBatch > 0 && kMaxBatch < kCap0) ? kMaxBatch : kCap0;
  constexpr int kBatch = kAll < kCap ? kAll : kCap;
  static_assert(kAll % kBatch == 0, "whole batches");
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t tlast = static_cast<int64_t>(t + (kT - 1) * tstride);
  const bool use_q = kQ && (kQAlways || r.use_q);
  const bool fast = (tlast + 1) * kSampleTile <= V && aligned16<DT>(r.t, 0) &&
                    (!use_q || aligned16<DQ>(r.q, 0));
  if (!fast) {
#pragma unroll 1
    for (int i = 0; i < kT; ++i)
      wave_tile_sums_any<DT, DQ, kQ, kFill, kPSum, kQAlways>(r, V, t + i * tstride, v[i], cache);
    return;
  }
  float ws[kT], ps[kT], qs[kT];
#pragma unroll
  for (int i = 0; i < kT; ++i) ws[i] = ps[i] = qs[i] = 0.f;
#pragma unroll
  for (int r0 = 0; r0 < kAll; r0 += kBatch) {
    uint4 tw[kBatch][L::nt];
    uint4 qw[kBatch][L::nq];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int run = r0 + k, ti = run / L::kRuns, kr = run % L::kRuns;
      const int64_t e = static_cast<int64_t>(t + ti * tstride) * kSampleTile +
                        static_cast<int64_t>(kr * kWave + lane) * kPer;
#pragma unroll
      for (int j = 0; j < L::nt; ++j) tw[k][j] = ld16<DT>(r.t, e + j * DT::kPerVec);
      if (use_q) {
#pragma unroll
        for (int j = 0; j < L::nq; ++j) qw[k][j] = ld16<DQ>(r.q, e + j * DQ::kPerVec);
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int ti = (r0 + k) / L::kRuns;
      float l[kPer], q[kPer], w[kPer], p[kPer];
#pragma unroll
      for (int j = 0; j < L::nt; ++j) DT::unpack(tw[k][j], l + j * DT::kPerVec);
      if (use_q) {
#pragma unroll
        for (int j = 0; j < L::nq; ++j) DQ::unpack(qw[k][j], q + j * DQ::kPerVec);
      } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) q[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        p[j] = draw_p(r, l[j]);
        w[j] = kQAlways ? fmaxf(fmaf(-r.coef, q[j], p[j]), 0.f) : draw_w(r, p[j], q[j]);
      }
      if constexpr (kFill) cache.put(r0 + k, lane, p, q);
      ws[ti] += pairwise<kPer>(w);
      if constexpr (kPSum) ps[ti] += pairwise<kPer>(p);
      qs[ti] += pairwise<kPer>(q);
    }
  }
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    v[i][0] = wave_total(static_cast<double>(ws[i]));
    v[i][1] = kPSum ? wave_total(static_cast<double>(ps[i])) : 0.0;
    v[i][2] = wave_total(static_cast<double>(qs[i]));
  }
}

// Weight sum of a tile from its LDS copy under the residual max(0, p - coef q):
// the same weights summed in the same order as the pass that filled the copy,
// so the same bits as wave_tile_sums would give; valid in every lane.
template <class DT, class DQ>
__device__ __forceinline__ double wave_tile_wsum_cached(const TileCache<DT, DQ>& c, float coef) {
  using C = TileCache<DT, DQ>;
  constexpr int kPer = C::L::kPer, kRuns = C::L::kRuns, kVec = C::kVec;
  const int lane = threadIdx.x & (kWave - 1);
  float4 pv[kRuns][kVec], qv[kRuns][kVec];
#pragma unroll
  for (int k = 0; k < kRuns; ++k) {
#pragma unroll
    for (int j4 = 0; j4 < kVec; ++j4) {
      pv[k][j4] = c.p[(k * kVec + j4) * kWave + lane];
      qv[k][j4] = c.q[(k * kVec + j4) * kWave + lane];
    }
  }
  float ws = 0.f;
#pragma unroll
  for (int k = 0; k < kRuns; ++k) {
    float w[kPer];
#pragma unroll
    for (int j4 = 0; j4 < kVec; ++j4) {
      w[4 * j4] = fmaxf(fmaf(-coef, qv[k][j4].x, pv[k][j4].x), 0.f);
      w[4 * j4 + 1] = fmaxf(fmaf(-coef, qv[k][j4].y, pv[k][j4].y), 0.f);
      w[4 * j4 + 2] = fmaxf(fmaf(-coef, qv[k][j4].z, pv[k][j4].z), 0.f);
      w[4 * j4 + 3] = fmaxf(fmaf(-coef, qv[k][j4].w, pv[k][j4].w), 0.f);
    }
    ws += pairwise<kPer>(w);
  }
  return wave_total(static_cast<double>(ws));
}

// Online-softmax pair (scaled domain, as in common.hpp) of tile t of a target
// row, valid in every lane, for any tile: on aligned rows every complete
// 16-byte vector is one predicated load, all in flight at once; a vector the
// row's end cuts and unaligned rows take element loads.
template <class D>
__device__ MS wave_tile_ms_any(const void* row, int64_t V, float c, int t) {
  constexpr int kPer = D::kPerVec;
  constexpr int kRuns = kSampleTile / (kWave * kPer);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t0 = static_cast<int64_t>(t) * kSampleTile;
  MS acc{-INFINITY, 0.f};
  if (aligned16<D>(row, t0)) {
    constexpr int kAB = kRuns < 4 ? kRuns : 4;  // runs per load round
#pragma unroll
    for (int k0 = 0; k0 < kRuns; k0 += kAB) {
      uint4 w[kAB];
#pragma unroll
      for (int kk = 0; kk < kAB; ++kk) {
        const int64_t e = t0 + static_cast<int64_t>((k0 + kk) * kWave + lane) * kPer;
        if (e + kPer <= V) w[kk] = ld16<D>(row, e);
      }
#pragma unroll
      for (int kk = 0; kk < kAB; ++kk) {
        const int64_t e = t0 + static_cast<int64_t>((k0 + kk) * kWave + lane) * kPer;
        float x[kPer];
        if (e + kPer <= V) {
          D::unpack(w[kk], x);
        } else {
#pragma unroll
          for (int j = 0; j < kPer; ++j) x[j] = e + j < V ? D::at(row, e + j) : -INFINITY;
        }
        ms_fold<kPer>(acc, x, c);
      }
    }
  } else {
#pragma unroll 1
    for (int k = 0; k < kRuns; ++k) {
      const int64_t e = t0 + static_cast<int64_t>(k * kWave + lane) * kPer;
      if (e >= V) break;
      float x[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) x[j] = e + j < V ? D::at(row, e + j) : -INFINITY;
      ms_fold<kPer>(acc, x, c);
    }
  }
  return wave_ms_dpp(acc);
}

// Online-softmax pairs of tile t of one target row (kTwo false; row1 unused) or two,
// valid in every lane.  Lane l takes the 16-byte vectors l, l + 64, ... of the
// tile; the loads of both rows are in flight at once and each row is folded
// with one rescale.
template <class D, bool kTwo>
__device__ __forceinline__ void wave_tile_ms(const void* row0, const void* row1, int64_t V, float c, int t,
                                             MS& out0, MS& out1) {
  constexpr int kPer = D::kPerVec;
  constexpr int kRuns = kSampleTile / (kWave * kPer);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t0 = static_cast<int64_t>(t) * kSampleTile;
  constexpr bool two = kTwo;
  const bool fast = t0 + kSampleTile <= V && aligned16<D>(row0, t0) && (!two || aligned16<D>(row1, t0));
  if (!fast) {
    out0 = wave_tile_ms_any<D>(row0, V, c, t);
    if (two) out1 = wave_tile_ms_any<D>(row1, V, c, t);
    return;
  }
  uint4 w0[kRuns], w1[kTwo ? kRuns : 1];
#pragma unroll
  for (int k = 0; k < kRuns; ++k) w0[k] = ld16<D>(row0, t0 + static_cast<int64_t>(k * kWave + lane) * kPer);
  if constexpr (kTwo) {
#pragma unroll
    for (int k = 0; k < kRuns; ++k) w1[k] = ld16<D>(row1, t0 + static_cast<int64_t>(k * kWave + lane) * kPer);
  }
  {
    float x[kRuns * kPer];
#pragma unroll
    for (int k = 0; k < kRuns; ++k) D::unpack(w0[k], x + k * kPer);
    MS acc{-INFINITY, 0.f};
    ms_fold<kRuns * kPer>(acc, x, c);
    out0 = wave_ms_dpp(acc);
  }
  if constexpr (kTwo) {
    float x[kRuns * kPer];
#pragma unroll
    for (int k = 0; k < kRuns; ++k) D::unpack(w1[k], x + k * kPer);
    MS acc{-INFINITY, 0.f};
    ms_fold<kRuns * kPer>(acc, x, c);
    out1 = wave_ms_dpp(acc);
  }
}

// Lane l's contiguous share [ta, tb) of ntiles tile sums for the tile search.
__device__ __forceinline__ void lane_tiles(int ntiles, int lane, int& ta, int& tb) {
  const int tpl = (ntiles + kWave - 1) / kWave;
  ta = min(lane * tpl, ntiles);
  tb = min(ta + tpl, ntiles);
}

struct TileHit {
  int tile;         // tile holding the target (or the last tile with weight)
  double base;      // running weight before that tile
  bool overshoot;   // no tile's running sum exceeded the target
};

// The tile holding `target`: the first tile of positive weight whose running
// sum exceeds it, else the last tile of positive weight.  ts[t * stride] is
// tile t's weight and `mine` the lane's own sum over lane_tiles (summed in
// order); returns false when no tile has weight.
__device__ __forceinline__ bool wave_find_tile(const double* ts, int stride, int ntiles, double mine,
                                               double target, TileHit& h) {
  const int lane = threadIdx.x & (kWave - 1);
  int ta, tb;
  lane_tiles(ntiles, lane, ta, tb);
  double run = wave_exclusive_from_inclusive(wave_incl_scan(mine));
  int hit = -1, lastpos = -1;
  double hit_base = 0.0;
  for (int t = ta; t < tb; ++t) {
    const double wt = ts[static_cast<int64_t>(t) * stride];
    if (wt > 0.0) {
      if (hit < 0 && run + wt > target) {
        hit = t;
        hit_base = run;
      }
      lastpos = t;
    }
    run += wt;
  }
  const uint64_t found = __ballot(hit >= 0);
  if (found) {
    const int src = __ffsll(static_cast<long long>(found)) - 1;
    h.tile = __builtin_amdgcn_readlane(hit, src);
    h.base = lane_value(hit_base, src);
    h.overshoot = false;
    return true;
  }
  const uint64_t any = __ballot(lastpos >= 0);
  if (!any) return false;
  h.tile = __builtin_amdgcn_readlane(lastpos, 63 - __clzll(static_cast<long long>(any)));
  h.base = 0.0;
  h.overshoot = true;
  return true;
}

// Bit i set: element e0 + i (i < kG) is one of the ids r.excl.
template <int kG>
__device__ __forceinline__ uint32_t run_excl_mask(const DrawRow& r, int64_t e0) {
  static_assert(kG <= 32, "one bit per element");
  uint32_t m = 0;
  for (int x = 0; x < r.nexcl; ++x) {
    const int64_t off = static_cast<int64_t>(r.excl[x]) - e0;
    if (off >= 0 && off < kG) m |= 1u << off;
  }
  return m;
}

// Weights of the kG contiguous elements [e0, e0 + kG) of the row (kG a
// multiple of 8), read in one round (16-byte vectors when aligned and
// complete); elements past the row's end weigh 0, and with kExcl the ids in
// r.excl too.  Each weight depends on its element alone, so any split of a
// tile into runs gives the same weights.
template <class DT, class DQ, int kG, bool kExcl = false>
__device__ __forceinline__ void run_weights(const DrawRow& r, int64_t V, int64_t e0, float (&wv)[kG]) {
  static_assert(kG % 8 == 0, "whole 8-element groups");
  constexpr int kTV = kG / DT::kPerVec, kQV = kG / DQ::kPerVec;
  uint4 tv[kTV], qv[kQV];
  const bool fast = e0 + kG <= V && aligned16<DT>(r.t, e0) && (!r.use_q || aligned16<DQ>(r.q, e0));
  if (fast) {
#pragma unroll
    for (int j = 0; j < kTV; ++j) tv[j] = ld16<DT>(r.t, e0 + j * DT::kPerVec);
    if (r.use_q) {
#pragma unroll
      for (int j = 0; j < kQV; ++j) qv[j] = ld16<DQ>(r.q, e0 + j * DQ::kPerVec);
    }
  }
#pragma unroll
  for (int g = 0; g < kG / 8; ++g) {
    float l[8], q[8];
    if (fast) {
      if (DT::kPerVec == 8) {
        DT::unpack(tv[g], l);
      } else {
        DT::unpack(tv[2 * g], l);
        DT::unpack(tv[2 * g + 1], l + 4);
      }
      if (r.use_q) {
        if (DQ::kPerVec == 8) {
          DQ::unpack(qv[g], q);
        } else {
          DQ::unpack(qv[2 * g], q);
          DQ::unpack(qv[2 * g + 1], q + 4);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = 0.f;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t e = e0 + 8 * g + j;
        const bool in = e < V;
        l[j] = in ? DT::at(r.t, e) : -INFINITY;
        q[j] = (in && r.use_q) ? DQ::at(r.q, e) : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) wv[8 * g + j] = draw_w(r, draw_p(r, l[j]), q[j]);
  }
  if constexpr (kExcl) {
    const uint32_t xm = run_excl_mask<kG>(r, e0);
#pragma unroll
    for (int i = 0; i < kG; ++i) wv[i] = ((xm >> i) & 1u) ? 0.f : wv[i];
  }
}

// The fp32 partial sum that lane Lx of a tile pass (wave_tile_sums over tile
// t, no draft row) forms, Lx being the lane whose runs hold id `extra`: its
// runs Lx, Lx + 64, ... of kPer elements, each summed pairwise, added in
// order from 0.  a: with the ids of r.excl weighing 0; b: with `extra` as well.
// The same element weights in the same order as the pass, so replacing a by
// b in a tile sum removes `extra` exactly up to fp64 rounding.  Valid in
// every lane; lanes [0, runs) do the loads.
template <class DT, class DQ>
__device__ __forceinline__ void lane_partial_excl(const DrawRow& r, int64_t V, int t, int extra, float& a,
                                                  float& b) {
  using L = TileRuns<DT, DQ>;
  constexpr int kPer = L::kPer;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t0 = static_cast<int64_t>(t) * kSampleTile;
  const int lx = static_cast<int>(((static_cast<int64_t>(extra) - t0) / kPer) % kWave);
  float pa = 0.f, pb = 0.f;
  if (lane < L::kRuns) {
    const int64_t e = t0 + static_cast<int64_t>(lane * kWave + lx) * kPer;
    float w[kPer], wb[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int64_t id = e + j;
      const float l = id < V ? DT::at(r.t, id) : -INFINITY;
      bool gone = false;
      for (int x = 0; x < r.nexcl; ++x) gone |= r.excl[x] == id;
      w[j] = gone ? 0.f : draw_w(r, draw_p(r, l), 0.f);
      wb[j] = id == extra ? 0.f : w[j];
    }
    pa = pairwise<kPer>(w);
    pb = pairwise<kPer>(wb);
  }
  float sa = 0.f, sb = 0.f;
#pragma unroll
  for (int k = 0; k < L::kRuns; ++k) {
    sa += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pa), k));
    sb += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pb), k));
  }
  a = sa;
  b = sb;
}

// The id inside tile h.tile.  Lane l of the tile's 64 lanes owns the 32
// contiguous elements [32 l, 32 l + 32), in four groups of 8: g_j is the
// pairwise fp32 sum of group j, the lane's weight (g_0 + g_1) + (g_2 + g_3)
// (its pairwise sum of 32), and the lanes' running bases are an fp64 scan.
// Inside group j the running weight starts from the fp32 sum of the groups
// before it (0, g_0, g_0 + g_1, (g_0 + g_1) + g_2) and adds the group's
// weights in order.  The id is the first element of positive weight where
// that running weight exceeds target - base (in fp32), else (or when h
// overshoots) the last element of positive weight.  wave_pick_in_tile does
// it in one wave, block_pick_in_tile over four waves, with identical results.
__device__ __forceinline__ float group_start(const float (&g)[4], int j) {
  const float g01 = g[0] + g[1];
  return j == 0 ? 0.f : (j == 1 ? g[0] : (j == 2 ? g01 : g01 + g[2]));
}

__device__ __forceinline__ void group_cross(const float* w, float start, float thr, bool overshoot, int idx0,
                                            int& first, int& lastw) {
  float lrun = start;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float wj = w[i];
    if (wj > 0.f) {
      if (first < 0 && !overshoot && lrun + wj > thr) first = idx0 + i;
      lastw = idx0 + i;
    }
    lrun += wj;
  }
}

// The lane's fp32 threshold: target minus the running weight of the lanes
// before it.
__device__ __forceinline__ float lane_threshold(const float (&g)[4], const TileHit& h, double target) {
  const float lw = (g[0] + g[1]) + (g[2] + g[3]);
  const double base = h.base + wave_exclusive_from_inclusive(wave_incl_scan(static_cast<double>(lw)));
  return static_cast<float>(target - base);
}

template <class DT, class DQ, bool kExcl = false>
__device__ __forceinline__ int wave_pick_in_tile(const DrawRow& r, int64_t V, const TileHit& h,
                                                 double target) {
  constexpr int kLane = kSampleTile / kWave;  // 32
  static_assert(kLane == 32, "four groups of 8 per lane");
  const int lane = threadIdx.x & (kWave - 1);
  float wv[kLane];
  run_weights<DT, DQ, kLane, kExcl>(r, V, static_cast<int64_t>(h.tile) * kSampleTile + lane * kLane, wv);
  float g[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) g[j] = pairwise<8>(wv + 8 * j);
  const float thr = lane_threshold(g, h, target);
  int first = -1, lastw = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) group_cross(wv + 8 * j, group_start(g, j), thr, h.overshoot, lane * kLane + 8 * j, first, lastw);
  int pick;
  const uint64_t found = __ballot(first >= 0);
  if (found) {
    pick = __builtin_amdgcn_readlane(first, __ffsll(static_cast<long long>(found)) - 1);
  } else {
    const uint64_t any = __ballot(lastw >= 0);
    pick = any ? __builtin_amdgcn_readlane(lastw, 63 - __clzll(static_cast<long long>(any))) : 0;
  }
  return static_cast<int>(static_cast<int64_t>(h.tile) * kSampleTile + pick);
}

// LDS of block_pick_in_tile: the groups' sums and each wave's candidates.
struct PickLds {
  float g[4][kWave];
  int first[4];
  int last[4];
};

// wave_pick_in_tile over waves 0..3 of the block, wave j taking group j of
// every lane's 32 elements (one 8-element run per thread).  Every thread of
// the block calls it (it holds two block barriers; waves past 3 only wait)
// with the same arguments; the id is returned in every thread.
template <class DT, class DQ, bool kExcl = false>
__device__ __forceinline__ int block_pick_in_tile(const DrawRow& r, int64_t V, const TileHit& h, double target,
                                                  PickLds& s) {
  const int lane = threadIdx.x & (kWave - 1), wid = static_cast<int>(threadIdx.x / kWave);
  const bool act = wid < 4;
  const int idx0 = lane * (kSampleTile / kWave) + 8 * wid;
  float wv[8];
  if (act) {
    run_weights<DT, DQ, 8, kExcl>(r, V, static_cast<int64_t>(h.tile) * kSampleTile + idx0, wv);
    s.g[wid][lane] = pairwise<8>(wv);
  }
  __syncthreads();
  if (act) {
    float g[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) g[j] = s.g[j][lane];
    const float thr = lane_threshold(g, h, target);
    int first = -1, lastw = -1;
    group_cross(wv, group_start(g, wid), thr, h.overshoot, idx0, first, lastw);
    const uint64_t found = __ballot(first >= 0), any = __ballot(lastw >= 0);
    const int f = found ? __builtin_amdgcn_readlane(first, __ffsll(static_cast<long long>(found)) - 1) : -1;
    const int l = any ? __builtin_amdgcn_readlane(lastw, 63 - __clzll(static_cast<long long>(any))) : -1;
    if (lane == 0) {
      s.first[wid] = f;
      s.last[wid] = l;
    }
  }
  __syncthreads();
  // the lowest crossing over the tile (index order is lane-major, then
  // group), else the highest element of positive weight
  int pick = -1, last = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int f = s.first[j];
    if (f >= 0 && (pick < 0 || f < pick)) pick = f;
    last = max(last, s.last[j]);
  }
  if (pick < 0) pick = last >= 0 ? last : 0;
  return static_cast<int>(static_cast<int64_t>(h.tile) * kSampleTile + pick);
}

// ---- greedy (T = 0): the argmax of a row ----

// Running argmax of one lane: the largest value, the lowest id among equal
// values (+0 and -0 are equal), and whether a NaN was seen.
struct ArgBest {
  float v;
  int32_t i;
  bool nan;
};

__device__ __forceinline__ void arg_update(ArgBest& s, float v, int32_t i) {
  s.nan |= (v != v);
  if (v > s.v || (v == s.v && i < s.i)) {
    s.v = v;
    s.i = i;
  }
}

// Order-preserving bits of a value (-0 -> +0): for a, b not NaN, a < b iff
// bits(a) < bits(b).
__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7fffffffu) == 0u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Fold tile t of a row into the lane's running argmax: lane l takes the
// 16-byte vectors l, l + 64, ... of the tile (element loads where the row is
// unaligned or the tile is cut by the row's end).
template <class D>
__device__ __forceinline__ void lane_tile_argmax(const void* row, int64_t V, int t, ArgBest& s) {
  constexpr int kPer = D::kPerVec;
  constexpr int kRuns = kSampleTile / (kWave * kPer);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t0 = static_cast<int64_t>(t) * kSampleTile;
  if (t0 + kSampleTile <= V && aligned16<D>(row, t0)) {
    uint4 w[kRuns];
#pragma unroll
    for (int k = 0; k < kRuns; ++k) w[k] = ld16<D>(row, t0 + static_cast<int64_t>(k * kWave + lane) * kPer);
    // the lane's largest value (fmaxf skips NaN, which only sets the flag),
    // then the first of its elements holding it: the lowest id, as its
    // elements ascend
    float x[kRuns][kPer];
    float m = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < kRuns; ++k) {
      D::unpack(w[k], x[k]);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        m = fmaxf(m, x[k][j]);
        nan |= x[k][j] != x[k][j];
      }
    }
    int32_t at = 0x7fffffff;
#pragma unroll
    for (int k = kRuns - 1; k >= 0; --k) {
      const int32_t e = static_cast<int32_t>(t0) + (k * kWave + lane) * kPer;
#pragma unroll
      for (int j = kPer - 1; j >= 0; --j) at = x[k][j] == m ? e + j : at;
    }
    s.nan |= nan;
    if (m > s.v || (m == s.v && at < s.i)) {
      s.v = m;
      s.i = at;
    }
  } else {
#pragma unroll 1
    for (int k = 0; k < kRuns; ++k) {
      const int64_t e = t0 + static_cast<int64_t>(k * kWave + lane) * kPer;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (e + j < V) arg_update(s, D::at(row, e + j), static_cast<int32_t>(e + j));
    }
  }
}

}  // namespace sv
