// Fused decode step of block-top-k sparse attention: one block per (request,
// KV head) runs the whole query-dependent stage and the cache
// update of the page this step's token completed (Vortex article, "A
// dual-stage programmable abstraction"; vortex_torch README, "Quick Example"):
//
//   1. stage the request's page-table row and the head's group-mean query
//      in LDS;
//   2. score every candidate page's centroid (order-preserving keys in LDS);
//   3. select top-k + reserved pages (kept in LDS; the row of `sel` is
//      stored at the end);
//   4. attend over the selected pages (K/V loads start as soon as the list
//      exists: physical pages come from the staged row, no HBM round trip);
//   5. if the token completed a page, write that page's centroid row (key
//      bounds: its minimum and maximum rows) for this head (the page is
//      the last, reserved one, so no score of this
//      step reads it).  Its K tile is loaded before the scoring loop and
//      reduced per row group after it, so the loads cost no extra round
//      trip; the row groups are added at the end.
//
// Steps 2-3 and 4 are the code of vx_score_topk's per-(request, KV head)
// kernel and of vx_sparse_paged_decode's attention, and step 5 uses the
// summation order of vx_centroid_update, so the selection and the centroids
// equal those calls' bit for bit; with 8-wave blocks the attention sums in
// the same order too.  One launch replaces four, and the attention phase of
// each block overlaps the other blocks' scoring instead of waiting for a
// kernel boundary.
//
// Blocks are 8 waves when there is about one (request, KV head) per CU, so
// each has the whole CU's memory parallelism; with two or more per CU they
// are 4 waves, so that two blocks share a CU and one's selection and merge
// (latency-bound, few loads in flight) overlap the other's streaming.  When
// the blocks take several rounds of the GPU, rows of blocks go to requests
// longest first (blocks start in about linear order), so that the long
// requests of a mixed batch do not start last and run alone at the end.
#include <type_traits>

#include "vx_attend.h"
#include "vx_centroid.h"
#include "vx_select.h"

namespace vx {
namespace {

// Request handled by block row r when rows go to requests in order of
// decreasing length, ties to the lower index: the request whose rank is r.
// len: LDS of roundup(B, 4) ints; pick: one LDS int.  Synchronises.
template <int NT>
__device__ __forceinline__ int longest_first_request(const int32_t* seq_lens, int B, int max_tokens, int r,
                                     int* len, int* pick) {
  const int tid = threadIdx.x;
  const int B4 = (B + 3) & ~3;
  for (int i = tid; i < B4; i += NT) {
    int L = -1;   // padding: shorter than any request
    if (i < B) {
      L = seq_lens[i];
      L = L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
    }
    len[i] = L;
  }
  __syncthreads();
  for (int j = tid; j < B; j += NT) {
    const int Lj = len[j];
    int rank = 0;
    for (int i = 0; i < B4; i += 4) {
      const int4 v = *reinterpret_cast<const int4*>(len + i);
      rank += (v.x > Lj || (v.x == Lj && i < j)) + (v.y > Lj || (v.y == Lj && i + 1 < j)) +
              (v.z > Lj || (v.z == Lj && i + 2 < j)) + (v.w > Lj || (v.w == Lj && i + 3 < j));
    }
    if (rank == r) *pick = j;
  }
  __syncthreads();
  return *pick;
}

// BOUNDS: the second summary rule (Quest's key bounds): the summary table
// holds two rows per (page, head), candidates are scored by the bound, and
// the completed page gets its bounds instead of its centroid.
template <typename T, int D, int G, int HS, int PF, int NW, bool BOUNDS>
__global__ __launch_bounds__(NW * 64) void decode_step_kernel(StepArgs a) {
  constexpr int NT = NW * 64;
  extern __shared__ __align__(16) uint32_t dyn[];   // page row, keys (each round4(max_pages)), list [k_tot]
  __shared__ float qbar[D];
  __shared__ SelectLds<NT> sl;
  // completed page: row-group sums (bounds: minima, then maxima)
  __shared__ float cred[(BOUNDS ? 2 : 1) * CentroidShape<T, D>::RG][D];

  __shared__ int pick;

  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const ScoreArgs& s = a.s;
  const int b = a.longest_first
                    ? longest_first_request<NT>(s.seq_lens, s.B, s.max_tokens, blockIdx.y,
                                                reinterpret_cast<int*>(dyn), &pick)
                    : blockIdx.y;
  // The first page-table entries (within the batch's page bound, which the
  // row holds) and the query are loaded before the request's length is
  // known, so the prologue costs one memory latency, not two.
  const int32_t* ptb = s.pt + (size_t)b * s.pt_stride;
  constexpr int kSpec = 4;
  int pv[kSpec];
#pragma unroll
  for (int j = 0; j < kSpec; ++j) {
    const int i = tid + j * NT;
    pv[j] = i < a.max_pages ? ptb[i] : 0;
  }
  head_query_mean<T, D, NT>(s, b, h, qbar);
  int seq = s.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > s.max_tokens ? s.max_tokens : seq);
  const int SP = s.S_p;
  const int n_b = (seq + SP - 1) / SP;
  const int n_cand = max(n_b - a.n_bos - a.n_eos, 0);
  const bool scoring = n_cand > a.topk && a.topk > 0;
  int32_t* prow = reinterpret_cast<int32_t*>(dyn);
  uint32_t* keys = dyn + round4(a.max_pages);
  int32_t* list = reinterpret_cast<int32_t*>(dyn + 2 * round4(a.max_pages));

#pragma unroll
  for (int j = 0; j < kSpec; ++j) {
    const int i = tid + j * NT;
    if (i < n_b) prow[i] = pv[j];
  }
  for (int i = tid + kSpec * NT; i < n_b; i += NT) prow[i] = ptb[i];
  select_init<NT>(sl);
  __syncthreads();

  // The page this step's token completed: its K tile rows are loaded now and
  // summed per row group after the scoring loop (the loads complete under
  // the scoring's), the groups are added at the end.
  using TC = std::conditional_t<BOUNDS, TileBounds<T, D, NT>, TileCentroid<T, D, NT>>;
  constexpr int RS = BOUNDS ? 2 : 1;           // summary rows per (page, head)
  const bool upd = a.update_completed && seq > 0 && seq % SP == 0;
  TC tc;
  if (upd) tc.load(reinterpret_cast<const T*>(a.d.k) + ((size_t)prow[n_b - 1] * s.H_kv + h) * SP * D, SP);

  if (scoring) score_head<T, D, NT, BOUNDS>(s, h, n_cand, prow + a.n_bos, qbar, keys, sl);
  if (upd) tc.reduce(&cred[0][0], SP);
  const int count = select_pages<NT>(keys, n_cand, n_b, a.topk, a.n_bos, a.n_eos, a.k_tot,
                                     nullptr, list, sl);
  __syncthreads();

  auto page_at = [&](int idx, bool active) -> int2 {
    int logi = 0, phys = 0;
    if (active) {
      logi = list[idx];
      phys = prow[logi];
    }
    return make_int2(logi, phys);
  };
  // the row of `sel` and the completed page's summary rows, by threads the
  // attention's merge leaves idle (stored late, so no barrier waits on them)
  int32_t* srow = a.sel + ((size_t)b * s.H_kv + h) * a.k_tot;
  auto epilogue = [&](int t, int nt) {
    for (int i = t; i < a.k_tot; i += nt) srow[i] = i < count ? list[i] : -1;
    if (upd && t < TC::S::SEGS)
      TC::finish(&cred[0][0], SP,
                 reinterpret_cast<T*>(a.cent) + ((size_t)prow[n_b - 1] * s.H_kv + h) * RS * D, t);
  };
  attend_pages<T, D, G, HS, PF, NW>(a.d, b, h, 0, 0, count, seq, page_at, epilogue);
}

template <typename T, int D, int G, int NW, bool BOUNDS>
hipError_t run_step(const StepArgs& a, hipStream_t s) {
  constexpr int HS = attend_head_slices<G>(), PF = attend_prefetch<T, D>();
  const size_t lds = step_dynamic_lds(a.max_pages, a.k_tot, a.longest_first ? a.s.B : 0);
  hipLaunchKernelGGL((decode_step_kernel<T, D, G, HS, PF, NW, BOUNDS>), dim3(a.s.H_kv, a.s.B),
                     dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t run_step_w(int waves, bool bounds, const StepArgs& a, hipStream_t s) {
  if (bounds) return waves == 4 ? run_step<T, D, G, 4, true>(a, s) : run_step<T, D, G, 8, true>(a, s);
  return waves == 4 ? run_step<T, D, G, 4, false>(a, s) : run_step<T, D, G, 8, false>(a, s);
}

template <typename T, int D>
hipError_t run_step_g(int G, int waves, bool bounds, const StepArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return run_step_w<T, D, 1>(waves, bounds, a, s);
    case 2: return run_step_w<T, D, 2>(waves, bounds, a, s);
    case 4: return run_step_w<T, D, 4>(waves, bounds, a, s);
    case 8: return run_step_w<T, D, 8>(waves, bounds, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t step_dynamic_lds(int max_pages, int k_tot, int ordered_batch) {
  const size_t main = 2 * (size_t)round4(max_pages) + (size_t)k_tot;
  const size_t order = ((size_t)ordered_batch + 3) & ~(size_t)3;
  return (main > order ? main : order) * sizeof(uint32_t);
}

bool decode_step_supported(int dtype, int D, int G) {
  return (dtype == 0 || dtype == 1) && (D == 64 || D == 128) &&
         (G == 1 || G == 2 || G == 4 || G == 8);
}

hipError_t launch_decode_step(int dtype, int D, int G, int waves, const StepArgs& a,
                              hipStream_t s, bool bounds) {
  if (waves != 4 && waves != 8) return hipErrorInvalidValue;
  if (dtype == 0) {
    if (D == 64) return run_step_g<float, 64>(G, waves, bounds, a, s);
    if (D == 128) return run_step_g<float, 128>(G, waves, bounds, a, s);
  } else {
    if (D == 64) return run_step_g<bf16_t, 64>(G, waves, bounds, a, s);
    if (D == 128) return run_step_g<bf16_t, 128>(G, waves, bounds, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vx
