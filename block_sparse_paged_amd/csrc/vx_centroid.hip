// K1: page centroids, the query-independent stage of block-top-k sparse
// attention (Vortex article, "A dual-stage programmable abstraction"; the
// vortex_torch README's "Quick Example" reduces a finished page's keys with a
// mean over its token rows into a centroid cache).
//
// One block per (listed page, KV head).  The page-head tile is S_p rows of
// D elements, contiguous in HBM (4 KiB for 16 x 128 bf16, 72 KiB for an MLA
// page).  Thread t reads 16-byte segment t % SEGS of rows t / SEGS,
// t / SEGS + RG, ..., all issued before the first is used, keeping fp32 sums;
// the RG row groups are then added in a fixed order through LDS, scaled by
// 1/S_p (exact: S_p is a power of two) and rounded once.
#include "vx_centroid.h"
#include "vx_internal.h"

namespace vx {
namespace {

constexpr int kMaxRowsPerThread = 8;

template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void centroid_kernel(CentroidArgs a) {
  using V = Vec16<T>;
  using S = CentroidShape<T, D>;
  constexpr int E = S::E, SEGS = S::SEGS, RG = S::RG;
  __shared__ float red[RG][SEGS * E];
  const int tid = threadIdx.x;
  const int seg = tid % SEGS, rg = tid / SEGS;
  int page;
  if (a.ids) {
    page = a.ids[blockIdx.x];
  } else {
    // the page that request blockIdx.x's latest token completed, if any
    const int b = blockIdx.x;
    int seq = a.seq_lens[b];
    seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
    if (seq == 0 || seq % a.S_p != 0) return;
    page = a.pt[(size_t)b * a.pt_stride + seq / a.S_p - 1];
  }
  const int h = blockIdx.y;
  const T* kp = reinterpret_cast<const T*>(a.k) + ((size_t)page * a.H_kv + h) * (size_t)a.S_p * D;

  uint4 buf[kMaxRowsPerThread];
#pragma unroll
  for (int j = 0; j < kMaxRowsPerThread; ++j) {
    const int t = rg + j * RG;
    if (t < a.S_p) buf[j] = ld16(kp + (size_t)t * D + seg * E);
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxRowsPerThread; ++j) {
    if (rg + j * RG < a.S_p) {
      float f[E];
      V::unpack(buf[j], f);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += f[e];
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[rg][seg * E + e] = acc[e];
  __syncthreads();
  if (tid < SEGS) {
    // same order as centroid_segment(): groups in order, then the scale
    const float inv = 1.0f / (float)a.S_p;
    float sum[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x = 0.f;
      for (int g = 0; g < RG; ++g) x += red[g][tid * E + e];
      sum[e] = x * inv;
    }
    T* cp = reinterpret_cast<T*>(a.cent) + ((size_t)page * a.H_kv + h) * D;
    st16(cp + tid * E, V::pack(sum));
  }
}

template <typename T, int D>
hipError_t run(const CentroidArgs& a, hipStream_t s) {
  using S = CentroidShape<T, D>;
  if (a.S_p > S::RG * kMaxRowsPerThread) return hipErrorInvalidValue;
  hipLaunchKernelGGL((centroid_kernel<T, D, S::THREADS>), dim3(a.n_ids, a.H_kv), dim3(S::THREADS),
                     0, s, a);
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
