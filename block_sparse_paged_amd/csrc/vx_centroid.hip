// K1: page centroids, the query-independent stage of block-top-k sparse
// attention (Vortex article, "A dual-stage programmable abstraction"; the
// vortex_torch README's "Quick Example" reduces a finished page's keys with a
// mean over its token rows into a centroid cache).
//
// One wave per (listed page, KV head).  The page-head tile is S_p rows of
// D elements, contiguous in HBM (S_p * D * e bytes: 4 KiB for 16 x 128 bf16).
// Lanes read 16-byte segments so each wave-load covers 1 KiB contiguously;
// column sums are kept in fp32 per lane, merged across lane groups with
// shuffles, scaled by 1/S_p (exact: S_p is a power of two) and rounded once.
#include "vx_device.h"
#include "vx_internal.h"

namespace vx {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(64) void centroid_kernel(CentroidArgs a) {
  using V = Vec16<T>;
  constexpr int E = V::E;
  constexpr int SEGS = D / E;               // 16-byte segments per row
  const int lane = threadIdx.x;
  const int i = blockIdx.x, h = blockIdx.y;
  const int page = a.ids[i];
  const size_t tile = ((size_t)page * a.H_kv + h) * (size_t)a.S_p * D;
  const T* kp = reinterpret_cast<const T*>(a.k) + tile;
  T* cp = reinterpret_cast<T*>(a.cent) + ((size_t)page * a.H_kv + h) * D;
  const float inv = 1.0f / (float)a.S_p;

  if constexpr (SEGS <= 64) {
    constexpr int R = 64 / SEGS;            // rows per wave-load
    const int seg = lane % SEGS, grp = lane / SEGS;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int t = grp; t < a.S_p; t += R) {
      float f[E];
      V::unpack(ld16(kp + (size_t)t * D + seg * E), f);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += f[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = across_groups_sum<SEGS>(acc[e]) * inv;
    if (grp == 0) st16(cp + seg * E, V::pack(acc));
  } else {
    for (int seg = lane; seg < SEGS; seg += 64) {
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = 0.f;
      for (int t = 0; t < a.S_p; ++t) {
        float f[E];
        V::unpack(ld16(kp + (size_t)t * D + seg * E), f);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += f[e];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= inv;
      st16(cp + seg * E, V::pack(acc));
    }
  }
}

template <typename T, int D>
hipError_t run(const CentroidArgs& a, hipStream_t s) {
  dim3 grid(a.n_ids, a.H_kv);
  hipLaunchKernelGGL((centroid_kernel<T, D>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_centroid(int dtype, const CentroidArgs& a, hipStream_t s) {
  if (dtype == 0) {
    switch (a.D) {
      case 64: return run<float, 64>(a, s);
      case 128: return run<float, 128>(a, s);
    }
  } else {
    switch (a.D) {
      case 64: return run<bf16_t, 64>(a, s);
      case 128: return run<bf16_t, 128>(a, s);
      case 576: return run<bf16_t, 576>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace vx
