// Fused decode step of block-top-k sparse attention: one 512-thread block per
// (request, KV head) runs the whole query-dependent stage and the cache
// update of the page this step's token completed (Vortex article, "A
// dual-stage programmable abstraction"; vortex_torch README, "Quick Example"):
//
//   1. stage the request's page-table row and the head's group-mean query
//      in LDS;
//   2. score every candidate page's centroid (order-preserving keys in LDS);
//   3. select top-k + reserved pages (written to `sel` and kept in LDS);
//   4. attend over the selected pages (K/V loads start as soon as the list
//      exists: physical pages come from the staged row, no HBM round trip);
//   5. if the token completed a page, write that page's centroid row for
//      this head (the page is the last, reserved one, so no block of this
//      step reads it; its K tile was just streamed and sits in L2).
//
// Steps 2-3 and 4 are the code of vx_score_topk's per-(request, KV head)
// kernel and of vx_sparse_paged_decode's attention, and step 5 uses the
// summation order of vx_centroid_update, so the results equal those calls'.
// One launch replaces four, and the attention phase of each block overlaps
// the other blocks' scoring instead of waiting for a kernel boundary.
#include "vx_attend.h"
#include "vx_centroid.h"
#include "vx_select.h"

namespace vx {
namespace {

constexpr int kStepThreads = kNW * 64;

template <typename T, int D, int G, int HS, int PF>
__global__ __launch_bounds__(kStepThreads) void decode_step_kernel(StepArgs a) {
  extern __shared__ uint32_t dyn[];   // page row [max_pages], keys [max_pages], list [k_tot]
  __shared__ float qbar[D];
  __shared__ int hist[4 * 256];
  __shared__ int scan_tmp[kStepThreads / 64];
  __shared__ uint32_t bounds_tmp[2 * kStepThreads / 64];

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const ScoreArgs& s = a.s;
  int seq = s.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > s.max_tokens ? s.max_tokens : seq);
  const int SP = s.S_p;
  const int n_b = (seq + SP - 1) / SP;
  const int n_cand = max(n_b - a.n_bos - a.n_eos, 0);
  const bool scoring = n_cand > a.topk && a.topk > 0;
  int32_t* prow = reinterpret_cast<int32_t*>(dyn);
  uint32_t* keys = dyn + a.max_pages;
  int32_t* list = reinterpret_cast<int32_t*>(dyn + 2 * a.max_pages);

  const int32_t* ptb = s.pt + (size_t)b * s.pt_stride;
  for (int i = tid; i < n_b; i += kStepThreads) prow[i] = ptb[i];
  if (scoring) head_query_mean<T, D, kStepThreads>(s, b, h, qbar);
  for (int i = tid; i < 4 * 256; i += kStepThreads) hist[i] = 0;
  __syncthreads();

  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  if (scoring) score_head<T, D, kStepThreads>(s, h, n_cand, prow + a.n_bos, qbar, keys, kmax, kmin);
  block_key_bounds<kStepThreads>(kmax, kmin, bounds_tmp);
  const int count = select_pages<kStepThreads>(
      keys, n_cand, n_b, a.topk, a.n_bos, a.n_eos, a.k_tot,
      a.sel + ((size_t)b * s.H_kv + h) * a.k_tot, list, hist, scan_tmp, kmax, kmin);
  __syncthreads();

  auto page_at = [&](int idx, bool active) -> int2 {
    int logi = 0, phys = 0;
    if (active) {
      logi = list[idx];
      phys = prow[logi];
    }
    return make_int2(logi, phys);
  };
  attend_pages<T, D, G, HS, PF>(a.d, b, h, 0, 0, count, seq, page_at);

  if (a.update_completed && seq > 0 && seq % SP == 0) {
    constexpr int SEGS = CentroidShape<T, D>::SEGS;
    if (tid < SEGS) {
      const int phys = prow[n_b - 1];
      const T* tile = reinterpret_cast<const T*>(a.d.k) + ((size_t)phys * s.H_kv + h) * SP * D;
      T* cp = reinterpret_cast<T*>(a.cent) + ((size_t)phys * s.H_kv + h) * D;
      st16(cp + tid * Vec16<T>::E, centroid_segment<T, D>(tile, SP, tid));
    }
  }
}

template <typename T, int D, int G>
hipError_t run_step(const StepArgs& a, hipStream_t s) {
  constexpr int HS = attend_head_slices<G>(), PF = attend_prefetch<T, D>();
  const size_t lds = (2 * (size_t)a.max_pages + (size_t)a.k_tot) * sizeof(uint32_t);
  hipLaunchKernelGGL((decode_step_kernel<T, D, G, HS, PF>), dim3(a.s.H_kv, a.s.B),
                     dim3(kStepThreads), lds, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_step_g(int G, const StepArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return run_step<T, D, 1>(a, s);
    case 2: return run_step<T, D, 2>(a, s);
    case 4: return run_step<T, D, 4>(a, s);
    case 8: return run_step<T, D, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_step_supported(int dtype, int D, int G) {
  return (dtype == 0 || dtype == 1) && (D == 64 || D == 128) &&
         (G == 1 || G == 2 || G == 4 || G == 8);
}

hipError_t launch_decode_step(int dtype, int D, int G, const StepArgs& a, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return run_step_g<float, 64>(G, a, s);
    if (D == 128) return run_step_g<float, 128>(G, a, s);
  } else {
    if (D == 64) return run_step_g<bf16_t, 64>(G, a, s);
    if (D == 128) return run_step_g<bf16_t, 128>(G, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vx
