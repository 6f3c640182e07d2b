// Page-centroid arithmetic shared by the centroid kernel and the fused decode
// step, so that both produce the same bits: the S_p rows of a page-head tile
// are summed in fp32 as RG interleaved row groups (rows g, g+RG, g+2RG, ...),
// the groups are added in order, the sum is scaled by 1/S_p (exact for a
// power of two) and rounded once to the KV dtype.
#pragma once

#include "vx_device.h"

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

}  // namespace vx
