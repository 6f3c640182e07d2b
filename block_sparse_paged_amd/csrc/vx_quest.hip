// K8 + K9: a second page-summary rule through the same pipeline.  The Vortex
// article (section "Speedups that scale to 229B parameters") names Quest as
// the other sparse-attention algorithm it serves; the rule, as the Quest
// paper states it (Tang et al., ICML 2024, section 3): a page is summarised
// by the per-channel minimum and maximum of its keys, and its criticality
// for a query q is sum_i max(q_i * min_i, q_i * max_i), an upper bound on
// q . k over the page's keys.  Selection and attention are the centroid
// pipeline's (K3, K4, K5); only the summary and the scores differ.  As for
// the centroids, q is the group mean of a KV head's query heads.
//
// K8 bounds_kernel: one block per listed page (or per request, for the page
//    its latest token completed); thread (KV head, 16-byte
//    segment) pairs read the page's rows, 16 loads in flight, keep the
//    channel minimum and maximum in fp32 (exact: both are key values) and
//    write them as two rows in the KV dtype.  Summary layout [P, H_kv, 2, D],
//    the minimum row first.
// K9 bound_score_kernel: the split scorer's layout (blocks over candidate
//    chunks of one request, rows r = page * H_kv + head, the H_kv row pairs
//    of a page contiguous); a lane reads the min and max segment of its row
//    (two 16-byte loads) and adds max(q*min, q*max) over its channels; the
//    row's lanes are then summed.  8 row pairs in flight per lane, the next
//    batch's pair u issued as this batch's pair u is consumed.
#include "vx_device.h"
#include "vx_internal.h"

namespace vx {
namespace {

constexpr int kBoundsThreads = 256;
constexpr int kBoundRows = 16;               // row loads in flight per thread
constexpr int kBoundScoreThreads = 512;
constexpr int kBoundPairs = 8;               // row pairs in flight per lane

template <typename T, int D>
__global__ __launch_bounds__(kBoundsThreads) void bounds_kernel(BoundsArgs a) {
  using V = Vec16<T>;
  constexpr int E = V::E, SEGS = D / E;
  int page;
  if (a.ids) {
    page = a.ids[blockIdx.x];
  } else {                                   // request blockIdx.x's completed page, if any
    int L = a.seq_lens[blockIdx.x];
    L = L < 0 ? 0 : (L > a.max_tokens ? a.max_tokens : L);
    if (L == 0 || L % a.S_p != 0) return;
    page = a.pt[(size_t)blockIdx.x * a.pt_stride + L / a.S_p - 1];
  }
  const T* kp = reinterpret_cast<const T*>(a.k) + (size_t)page * a.H_kv * a.S_p * D;
  T* bp = reinterpret_cast<T*>(a.bounds) + (size_t)page * a.H_kv * 2 * D;
  for (int i = threadIdx.x; i < a.H_kv * SEGS; i += kBoundsThreads) {
    const int h = i / SEGS, sg = i - h * SEGS;
    const T* src = kp + (size_t)h * a.S_p * D + sg * E;
    float lo[E], hi[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      lo[e] = INFINITY;
      hi[e] = -INFINITY;
    }
    for (int t0 = 0; t0 < a.S_p; t0 += kBoundRows) {
      uint4 r[kBoundRows];
#pragma unroll
      for (int j = 0; j < kBoundRows; ++j) r[j] = ld16(src + (size_t)min(t0 + j, a.S_p - 1) * D);
#pragma unroll
      for (int j = 0; j < kBoundRows; ++j) {
        float f[E];
        V::unpack(r[j], f);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          lo[e] = fminf(lo[e], f[e]);
          hi[e] = fmaxf(hi[e], f[e]);
        }
      }
    }
    st16(bp + (size_t)h * 2 * D + sg * E, V::pack(lo));
    st16(bp + (size_t)h * 2 * D + D + sg * E, V::pack(hi));
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kBoundScoreThreads) void bound_score_kernel(ScoreArgs a) {
  using V = Vec16<T>;
  constexpr int E = V::E;
  constexpr int LH = D / E;                  // lanes per row
  constexpr int R = 64 / LH;                 // rows per wave-load
  constexpr int NW = kBoundScoreThreads / 64;
  constexpr int STEP = NW * R;               // rows per block-wide wave-load
  constexpr int U = kBoundPairs;
  static_assert(LH * R == 64, "rows of at most 64 lanes");
  extern __shared__ float smem[];            // qbar [H_kv][D], then phys ids
  float* qbar = smem;
  int32_t* phys = reinterpret_cast<int32_t*>(smem + a.H_kv * D);

  const int b = blockIdx.y, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + a.S_p - 1) / a.S_p;
  const int n_cand = n_b - a.n_bos - a.n_eos;
  const int c0 = blockIdx.x * a.cand_per_block;
  if (c0 >= n_cand) return;
  const int nc = min(c0 + a.cand_per_block, n_cand) - c0;

  // group-mean query in fp32, G heads summed in order
  const int G = a.H_q / a.H_kv;
  const float invG = 1.0f / (float)G;
  const T* qb = reinterpret_cast<const T*>(a.q) + (size_t)b * a.H_q * D;
  for (int i = tid; i < a.H_kv * D; i += kBoundScoreThreads) {
    const int h = i / D, d = i - h * D;
    float s = 0.f;
    for (int g = 0; g < G; ++g) s += V::to_f32(qb[(size_t)(h * G + g) * D + d]);
    qbar[i] = s * invG;
  }
  const int32_t* ptb = a.pt + (size_t)b * a.pt_stride + a.n_bos;
  for (int i = tid; i < nc; i += kBoundScoreThreads) phys[i] = ptb[c0 + i];
  __syncthreads();

  const int rows = nc * a.H_kv;
  const int seg = lane % LH, grp = lane / LH;
  const int rw = wave * R + grp;             // this lane's first row
  const int nbat = rows > wave * R ? (rows - wave * R + STEP * U - 1) / (STEP * U) : 0;
  const T* bnd = reinterpret_cast<const T*>(a.cent);
  auto row_off = [&](int r) -> size_t {      // past the last row: the last row again
    const int rc = min(r, rows - 1);
    const int c = rc / a.H_kv, h = rc - c * a.H_kv;
    return ((size_t)phys[c] * a.H_kv + h) * 2 * D + seg * E;
  };
  float* out = a.scores + (size_t)b * a.H_kv * a.score_stride;
  // with H_kv dividing STEP every row of a lane has the same KV head, whose
  // query segment then stays in registers
  const bool fixed_head = STEP % a.H_kv == 0;
  float qr[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qr[e] = qbar[(rw % a.H_kv) * D + seg * E + e];
  uint4 lo[U], hi[U];
  if (nbat > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t o = row_off(rw + u * STEP);
      lo[u] = ld16(bnd + o);
      hi[u] = ld16(bnd + o + D);
    }
  }
  for (int k = 0; k < nbat; ++k) {
    const int r0 = rw + k * STEP * U;
    size_t nx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) nx[u] = row_off(r0 + STEP * U + u * STEP);
    float mine = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * STEP;
      const int rc = r < rows ? r : 0;
      const int h = rc - (rc / a.H_kv) * a.H_kv;
      float fl[E], fh[E];
      V::unpack(lo[u], fl);
      V::unpack(hi[u], fh);
      lo[u] = ld16(bnd + nx[u]);
      hi[u] = ld16(bnd + nx[u] + D);
      float acc = 0.f;
      if (fixed_head) {
#pragma unroll
        for (int e = 0; e < E; ++e) acc += fmaxf(qr[e] * fl[e], qr[e] * fh[e]);
      } else {
        const float* qh = qbar + h * D + seg * E;
#pragma unroll
        for (int e = 0; e < E; ++e) acc += fmaxf(qh[e] * fl[e], qh[e] * fh[e]);
      }
      acc = lane_group_sum<LH>(acc);
      if (seg == u) mine = acc;
    }
    // lane seg < U stores the row of its group's load seg
    const int r = r0 + seg * STEP;
    if (seg < U && r < rows) {
      const int c = r / a.H_kv, h = r - c * a.H_kv;
      out[(size_t)h * a.score_stride + c0 + c] = mine;
    }
  }
}

template <typename T, int D>
hipError_t run_bounds(const BoundsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bounds_kernel<T, D>), dim3(a.n_ids), dim3(kBoundsThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_bound_score(const ScoreArgs& a, int grid_x, hipStream_t s) {
  static_assert(D / Vec16<T>::E >= kBoundPairs, "a row has a lane for each pair it stores");
  const size_t lds = (size_t)a.H_kv * D * sizeof(float) + (size_t)a.cand_per_block * sizeof(int32_t);
  hipLaunchKernelGGL((bound_score_kernel<T, D>), dim3(grid_x, a.B), dim3(kBoundScoreThreads), lds,
                     s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_page_bounds(int dtype, const BoundsArgs& a, hipStream_t s) {
  if (a.n_ids == 0) return hipSuccess;
  if (dtype == 0) {
    if (a.D == 64) return run_bounds<float, 64>(a, s);
    if (a.D == 128) return run_bounds<float, 128>(a, s);
  } else {
    if (a.D == 64) return run_bounds<bf16_t, 64>(a, s);
    if (a.D == 128) return run_bounds<bf16_t, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bound_score(int dtype, const ScoreArgs& a, int grid_x, hipStream_t s) {
  if (dtype == 0) {
    if (a.D == 64) return run_bound_score<float, 64>(a, grid_x, s);
    if (a.D == 128) return run_bound_score<float, 128>(a, grid_x, s);
  } else {
    if (a.D == 64) return run_bound_score<bf16_t, 64>(a, grid_x, s);
    if (a.D == 128) return run_bound_score<bf16_t, 128>(a, grid_x, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vx
