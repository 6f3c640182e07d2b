// Page-centroid arithmetic shared by the centroid kernel and the fused decode
// step, so that both produce the same bits: the S_p rows of a page-head tile
// are summed in fp32 as RG interleaved row groups (rows g, g+RG, g+2RG, ...),
// the groups are added in order, the sum is scaled by 1/S_p (exact for a
// power of two) and rounded once to the KV dtype.
#pragma once

#include "vx_device.h"
#include "vx_internal.h"

namespace vx {

template <typename T, int D>
struct CentroidShape {
  static constexpr int E = Vec16<T>::E;
  static constexpr int SEGS = D / E;                                   // 16-byte segments per row
  static constexpr int RG = (SEGS * 16 <= 1024) ? 16 : 1024 / SEGS;    // row groups
  static constexpr int THREADS = SEGS * RG;
};

// One lane computes segment `seg` of the centroid of a page-head tile alone.
template <typename T, int D>
__device__ __forceinline__ uint4 centroid_segment(const T* tile, int S_p, int seg) {
  using V = Vec16<T>;
  constexpr int E = V::E, RG = CentroidShape<T, D>::RG;
  float sum[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sum[e] = 0.f;
  for (int g = 0; g < RG; ++g) {
    float part[E];
#pragma unroll
    for (int e = 0; e < E; ++e) part[e] = 0.f;
    for (int t = g; t < S_p; t += RG) {
      float f[E];
      V::unpack(ld16(tile + (size_t)t * D + seg * E), f);
#pragma unroll
      for (int e = 0; e < E; ++e) part[e] += f[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) sum[e] += part[e];
  }
  const float inv = 1.0f / (float)S_p;
#pragma unroll
  for (int e = 0; e < E; ++e) sum[e] *= inv;
  return V::pack(sum);
}

// The centroid of one page-head tile computed inside a longer kernel of NT
// threads, in the order of the centroid kernel: load() issues each thread's
// rows early (thread t takes (row group, segment) pairs t, t + NT, ...),
// reduce() sums them per row group into LDS `red` [RG][D] later, and after a
// barrier finish() adds the groups in order for segment t < SEGS, scales and
// stores.  Pages of up to kMaxTileRows rows.

template <typename T, int D, int NT>
struct TileCentroid {
  using S = CentroidShape<T, D>;
  static constexpr int CP = (S::THREADS + NT - 1) / NT;               // pairs per thread
  static constexpr int CR = (kMaxTileRows + S::RG - 1) / S::RG;       // rows per pair
  uint4 rows[CP][CR];

  __device__ __forceinline__ void load(const T* tile, int S_p) {
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      const int pr = threadIdx.x + c * NT, g = pr / S::SEGS, sg = pr % S::SEGS;
#pragma unroll
      for (int j = 0; j < CR; ++j)
        if (pr < S::THREADS && g + j * S::RG < S_p)
          rows[c][j] = ld16(tile + (size_t)(g + j * S::RG) * D + sg * S::E);
    }
  }

  __device__ __forceinline__ void reduce(float* red, int S_p) const {
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      const int pr = threadIdx.x + c * NT, g = pr / S::SEGS, sg = pr % S::SEGS;
      if (pr < S::THREADS) {
        float part[S::E];
#pragma unroll
        for (int e = 0; e < S::E; ++e) part[e] = 0.f;
#pragma unroll
        for (int j = 0; j < CR; ++j) {
          if (g + j * S::RG < S_p) {
            float f[S::E];
            Vec16<T>::unpack(rows[c][j], f);
#pragma unroll
            for (int e = 0; e < S::E; ++e) part[e] += f[e];
          }
        }
#pragma unroll
        for (int e = 0; e < S::E; ++e) red[g * D + sg * S::E + e] = part[e];
      }
    }
  }

  static __device__ __forceinline__ void finish(const float* red, int S_p, T* cent_row, int t) {
    float sum[S::E];
#pragma unroll
    for (int e = 0; e < S::E; ++e) sum[e] = 0.f;
    for (int g = 0; g < S::RG; ++g)
#pragma unroll
      for (int e = 0; e < S::E; ++e) sum[e] += red[g * D + t * S::E + e];
    const float inv = 1.0f / (float)S_p;
#pragma unroll
    for (int e = 0; e < S::E; ++e) sum[e] *= inv;
    st16(cent_row + t * S::E, Vec16<T>::pack(sum));
  }
};

// The key bounds of one page-head tile (per-channel minimum and maximum,
// Quest's page summary) inside a longer kernel, with TileCentroid's row
// layout and load(): reduce() keeps each row group's minimum and maximum in
// LDS `red` [2][RG][D], finish() takes them over the groups for segment t
// and stores the two rows (minimum first).  Minimum and maximum are exact,
// so the rows equal the bounds kernel's in any order (but for the sign of a
// zero that ties with another zero).
template <typename T, int D, int NT>
struct TileBounds : TileCentroid<T, D, NT> {
  using Base = TileCentroid<T, D, NT>;
  using S = typename Base::S;

  __device__ __forceinline__ void reduce(float* red, int S_p) const {
#pragma unroll
    for (int c = 0; c < Base::CP; ++c) {
      const int pr = threadIdx.x + c * NT, g = pr / S::SEGS, sg = pr % S::SEGS;
      if (pr < S::THREADS) {
        float lo[S::E], hi[S::E];
#pragma unroll
        for (int e = 0; e < S::E; ++e) {
          lo[e] = INFINITY;
          hi[e] = -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < Base::CR; ++j) {
          if (g + j * S::RG < S_p) {
            float f[S::E];
            Vec16<T>::unpack(this->rows[c][j], f);
#pragma unroll
            for (int e = 0; e < S::E; ++e) {
              lo[e] = fminf(lo[e], f[e]);
              hi[e] = fmaxf(hi[e], f[e]);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < S::E; ++e) {
          red[g * D + sg * S::E + e] = lo[e];
          red[(S::RG + g) * D + sg * S::E + e] = hi[e];
        }
      }
    }
  }

  // bounds_row: the page-head's two summary rows [2][D]
  static __device__ __forceinline__ void finish(const float* red, int, T* bounds_row, int t) {
    float lo[S::E], hi[S::E];
#pragma unroll
    for (int e = 0; e < S::E; ++e) {
      lo[e] = INFINITY;
      hi[e] = -INFINITY;
    }
    for (int g = 0; g < S::RG; ++g)
#pragma unroll
      for (int e = 0; e < S::E; ++e) {
        lo[e] = fminf(lo[e], red[g * D + t * S::E + e]);
        hi[e] = fmaxf(hi[e], red[(S::RG + g) * D + t * S::E + e]);
      }
    st16(bounds_row + t * S::E, Vec16<T>::pack(lo));
    st16(bounds_row + D + t * S::E, Vec16<T>::pack(hi));
  }
};

// Part of the centroid rows of one page computed inside a longer kernel of NT
// threads, again in the centroid kernel's order: the block takes units
// [u0, u0 + nu) of the page's (KV head, 16-byte segment) pairs (unit u: head
// u / SEGS, segment u % SEGS), so that the blocks of a request can share a
// page without combining partial sums.  Thread t takes (unit, row group)
// pairs t, t + NT, ... (at most CP of them); load() issues their rows early,
// reduce() sums each pair into LDS `red` [nu * RG][E] later, and after a
// barrier finish() completes unit u0 + t for t < nu.
template <typename T, int D, int NT, int CP>
struct SegmentCentroid {
  using S = CentroidShape<T, D>;
  static constexpr int CR = (kMaxTileRows + S::RG - 1) / S::RG;       // rows per pair
  uint4 rows[CP][CR];

  // page: the page's K rows [H_kv][S_p][D]
  __device__ __forceinline__ void load(const T* page, int S_p, int u0, int nu) {
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      const int pr = threadIdx.x + c * NT;
      const int u = u0 + pr / S::RG, g = pr % S::RG;
      const int h = u / S::SEGS, sg = u % S::SEGS;
#pragma unroll
      for (int j = 0; j < CR; ++j)
        if (pr < nu * S::RG && g + j * S::RG < S_p)
          rows[c][j] = ld16(page + ((size_t)h * S_p + g + j * S::RG) * D + sg * S::E);
    }
  }

  __device__ __forceinline__ void reduce(float* red, int S_p, int nu) const {
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      const int pr = threadIdx.x + c * NT, g = pr % S::RG;
      if (pr < nu * S::RG) {
        float part[S::E];
#pragma unroll
        for (int e = 0; e < S::E; ++e) part[e] = 0.f;
#pragma unroll
        for (int j = 0; j < CR; ++j) {
          if (g + j * S::RG < S_p) {
            float f[S::E];
            Vec16<T>::unpack(rows[c][j], f);
#pragma unroll
            for (int e = 0; e < S::E; ++e) part[e] += f[e];
          }
        }
#pragma unroll
        for (int e = 0; e < S::E; ++e) red[pr * S::E + e] = part[e];
      }
    }
  }

  // cent: the page's centroid rows [H_kv][D]
  static __device__ __forceinline__ void finish(const float* red, int S_p, T* cent, int u0, int t) {
    const int u = u0 + t, h = u / S::SEGS, sg = u % S::SEGS;
    float sum[S::E];
#pragma unroll
    for (int e = 0; e < S::E; ++e) sum[e] = 0.f;
    for (int g = 0; g < S::RG; ++g)
#pragma unroll
      for (int e = 0; e < S::E; ++e) sum[e] += red[(t * S::RG + g) * S::E + e];
    const float inv = 1.0f / (float)S_p;
#pragma unroll
    for (int e = 0; e < S::E; ++e) sum[e] *= inv;
    st16(cent + (size_t)h * D + sg * S::E, Vec16<T>::pack(sum));
  }
};

}  // namespace vx
