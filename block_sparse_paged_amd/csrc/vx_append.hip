// K7: the write path beside the decode step.  New tokens' K/V rows go into
// their pages, and every page that the write fills gets its centroid, in the
// same kernel (Vortex article, section "A dual-stage programmable
// abstraction": the query-independent summaries are made while the cache is
// built; vortex_torch README, "Quick Example": the centroid of a page is
// computed once the page is full).  One decode token per request is an
// append; a prompt's tokens are a bulk prefill write with its centroids.
//
// One block per (touched page, KV head, request).  Thread (row group g,
// segment s) copies its new rows and, when the page becomes full, sums its
// rows g, g + RG, ... in order, new ones from the source registers and old
// ones from the cache, so no row is read back after it is written; the
// groups are then added in order and scaled, the summation order of the
// centroid kernel.
#include "vx_centroid.h"
#include "vx_internal.h"

namespace vx {
namespace {

template <typename T, int DQ, int NT>
__global__ __launch_bounds__(NT) void append_kernel(AppendArgs a) {
  using S = CentroidShape<T, DQ>;
  using V = Vec16<T>;
  static_assert(NT == S::THREADS, "one thread per (row group, segment)");
  constexpr int E = S::E, SEGS = S::SEGS, RG = S::RG;
  constexpr int CR = (kMaxTileRows + RG - 1) / RG;
  __shared__ float red[RG][SEGS * E];
  const int tid = threadIdx.x;
  const int seg = tid % SEGS, g = tid / SEGS;
  const int h = blockIdx.y, b = blockIdx.z;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_tokens ? a.max_tokens : L);
  int n = a.n_new[b];
  n = n < 0 ? 0 : (n > a.max_new ? a.max_new : n);
  n = n > L ? L : n;
  if (n == 0) return;
  const int first = L - n;                                  // first new position
  const int p = first / a.S_p + (int)blockIdx.x;
  if (p * a.S_p >= L) return;
  const int phys = a.pt[(size_t)b * a.pt_stride + p];
  const bool full = a.update && (p + 1) * a.S_p <= L;       // the write fills this page
  const int row0 = a.src_start[b] - first;                  // source row of position pos: row0 + pos

  T* kc = reinterpret_cast<T*>(a.k) + ((size_t)phys * a.H_kv + h) * (size_t)a.S_p * DQ;
  const T* ks = reinterpret_cast<const T*>(a.k_src);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  uint4 val[CR];
  bool have[CR];
#pragma unroll
  for (int j = 0; j < CR; ++j) {                            // all loads first
    const int t = g + j * RG, pos = p * a.S_p + t;
    const int row = row0 + pos;
    const bool is_new = t < a.S_p && pos >= first && pos < L && row >= 0 && row < a.n_src_rows;
    const bool is_old = t < a.S_p && full && !is_new;          // kept row (no source row)
    have[j] = is_new || is_old;
    if (is_new) val[j] = ld16(ks + ((size_t)row * a.H_kv + h) * DQ + seg * E);
    else if (is_old) val[j] = ld16(kc + (size_t)t * DQ + seg * E);
  }
#pragma unroll
  for (int j = 0; j < CR; ++j) {
    const int t = g + j * RG, pos = p * a.S_p + t;
    if (!have[j]) continue;
    const int row = row0 + pos;
    if (pos >= first && row >= 0 && row < a.n_src_rows) st16(kc + (size_t)t * DQ + seg * E, val[j]);
    if (full) {
      float f[E];
      V::unpack(val[j], f);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += f[e];
    }
  }

  // V rows of the new tokens (none when V is the leading part of K)
  if (a.v) {
    const int segs_v = a.Dv / E;
    T* vc = reinterpret_cast<T*>(a.v) + ((size_t)phys * a.H_kv + h) * (size_t)a.S_p * a.Dv;
    const T* vs = reinterpret_cast<const T*>(a.v_src);
    for (int i = tid; i < a.S_p * segs_v; i += NT) {
      const int t = i / segs_v, sv = i - t * segs_v, pos = p * a.S_p + t;
      const int row = row0 + pos;
      if (pos >= first && pos < L && row >= 0 && row < a.n_src_rows)
        st16(vc + (size_t)t * a.Dv + sv * E, ld16(vs + ((size_t)row * a.H_kv + h) * a.Dv + sv * E));
    }
  }

  if (!full) return;
#pragma unroll
  for (int e = 0; e < E; ++e) red[g][seg * E + e] = acc[e];
  __syncthreads();
  if (tid < SEGS) {
    float sum[E];
#pragma unroll
    for (int e = 0; e < E; ++e) sum[e] = 0.f;
    for (int gg = 0; gg < RG; ++gg)
#pragma unroll
      for (int e = 0; e < E; ++e) sum[e] += red[gg][tid * E + e];
    const float inv = 1.0f / (float)a.S_p;
#pragma unroll
    for (int e = 0; e < E; ++e) sum[e] *= inv;
    T* cp = reinterpret_cast<T*>(a.cent) + ((size_t)phys * a.H_kv + h) * DQ;
    st16(cp + tid * E, V::pack(sum));
  }
}

template <typename T, int DQ>
hipError_t run_append(const AppendArgs& a, int pages_per_req, hipStream_t s) {
  using S = CentroidShape<T, DQ>;
  if (a.S_p > kMaxTileRows || S::RG * ((kMaxTileRows + S::RG - 1) / S::RG) < a.S_p)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((append_kernel<T, DQ, S::THREADS>), dim3(pages_per_req, a.H_kv, a.B),
                     dim3(S::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int dtype, const AppendArgs& a, int pages_per_req, hipStream_t s) {
  if (dtype == 0) {
    if (a.Dq == 64) return run_append<float, 64>(a, pages_per_req, s);
    if (a.Dq == 128) return run_append<float, 128>(a, pages_per_req, s);
  } else {
    if (a.Dq == 64) return run_append<bf16_t, 64>(a, pages_per_req, s);
    if (a.Dq == 128) return run_append<bf16_t, 128>(a, pages_per_req, s);
    if (a.Dq == 576) return run_append<bf16_t, 576>(a, pages_per_req, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vx
