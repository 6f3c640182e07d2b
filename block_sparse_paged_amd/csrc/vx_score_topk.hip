// K2 + K3: the query-dependent indexer of block-top-k sparse attention
// (vortex_torch README, "Quick Example": the query is averaged over heads,
// GeMV'd against the page centroids, and topK writes the page index
// structure; "Using Your Sparse Attention with SGLang": reserved first / last
// pages and the top-k value).
//
// Two schedules, chosen by the host planner:
//
// fused   one 512-thread block per (request, KV head) scores every candidate
//         page of that head and selects in the same block: the page table
//         slice is staged in LDS, each wave keeps 16 centroid-row loads in
//         flight, scores become order-preserving keys in LDS, and no score
//         touches HBM.  Used when there are enough (request, KV head) units
//         to fill the GPU and the candidate keys fit in LDS.
// split   K2 score_kernel: blocks over (candidate chunk, request) score all
//         KV heads of their pages (the H_kv rows of a page are contiguous, so
//         a wave-load reads 1 KiB of consecutive heads) into the workspace;
//         K3 topk_kernel: one block per (request, KV head) selects (in the
//         decode step the split decode kernels select instead).  Used when
//         few (request, KV head) units exist (long contexts, MLA's single
//         latent head).
//
// Selection (both schedules, vx_select.h): the k-th largest (key, page) pair
// from histograms of the key range in at most 1024 bins, each level
// narrowing the boundary bin's range by ten bits until that bin is taken
// whole (every wave locating the boundary bin itself), then the union with
// the reserved pages compacted in ascending page order with one block-wide
// scan.
#include <algorithm>

#include "vx_centroid.h"
#include "vx_select.h"

namespace vx {
namespace {

constexpr int kScoreThreads = 512;
constexpr int kTopkThreads = 512;
constexpr int kFusedThreads = 512;
constexpr int kSplitLoads = 8;      // wave-loads in flight per lane in the split scorer
// (KV head, segment, row group) triples of a completed page one scoring
// block takes at most (two per thread)
constexpr int kScoreCentroidPairs = 2 * kScoreThreads;

// ---------------------------------------------------------------- fused
template <typename T, int D, bool BOUNDS>
__global__ __launch_bounds__(kFusedThreads) void indexer_fused_kernel(ScoreArgs a, TopkArgs t) {
  extern __shared__ __align__(16) uint32_t dyn[];   // phys, keys: round4(max_cand) each
  __shared__ float qbar[D];
  __shared__ SelectLds<kFusedThreads> sl;

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + a.S_p - 1) / a.S_p;
  const int n_cand = max(n_b - a.n_bos - a.n_eos, 0);
  const bool scoring = n_cand > t.topk && t.topk > 0;
  int32_t* phys = reinterpret_cast<int32_t*>(dyn);
  uint32_t* keys = dyn + round4(a.score_stride);

  if (scoring) {
    head_query_mean<T, D, kFusedThreads>(a, b, h, qbar);
    const int32_t* ptb = a.pt + (size_t)b * a.pt_stride + a.n_bos;
    for (int i = tid; i < n_cand; i += kFusedThreads) phys[i] = ptb[i];
  }
  select_init<kFusedThreads>(sl);
  __syncthreads();

  if (scoring) score_head<T, D, kFusedThreads, BOUNDS>(a, h, n_cand, phys, qbar, keys, sl);
  select_pages<kFusedThreads>(keys, n_cand, n_b, t.topk, t.n_bos, t.n_eos, t.k_tot,
                              t.sel + ((size_t)b * t.H_kv + h) * t.k_tot, nullptr, sl, t.levels,
                              t.rnd ? t.rnd[(size_t)b * t.H_kv + h] : 0u);
}

// ---------------------------------------------------------------- split
// Order of a scoring block, so that HBM is busy as early as possible: the
// query rows, the block's page-table slice and the request length are
// loaded together; once the page ids are in LDS the first centroid loads
// are issued, and only then are the group-mean queries formed (their loads
// have long arrived) and the completed page's rows requested.
template <typename T, int D>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  using V = Vec16<T>;
  constexpr int E = V::E;
  constexpr int LH = D / E;                 // 16-byte segments per centroid row
  extern __shared__ float smem[];           // qbar [H_kv][D] then phys ids
  float* qbar = smem;
  int32_t* phys = reinterpret_cast<int32_t*>(smem + a.H_kv * D);

  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // group-mean query of every KV head, fp32: thread (chunk, head, segment)
  // sums eight query heads in order, the chunks' partials are then added in
  // chunk order.  Every load up to the first centroid batch is issued by
  // every thread (indices clamped, surplus values unused), so that the waits
  // for the query rows count the centroid loads behind them exactly.
  const int G = a.H_q / a.H_kv;
  const int NCH = (G + 7) / 8;
  const int QS = a.H_kv * LH;                 // (head, segment) pairs
  const T* qb = reinterpret_cast<const T*>(a.q) + (size_t)b * a.H_q * D;
  const float invG = 1.0f / (float)G;
  float* qpart = reinterpret_cast<float*>(phys + a.cand_per_block);   // [NCH][H_kv * D] when NCH > 1
  auto q_load = [&](int i, uint4* v) {
    i = min(i, QS * NCH - 1);
    const int ch = i / QS, hs = i - ch * QS;
    const int h = hs / LH, sg = hs - h * LH;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ld16(qb + (size_t)(h * G + min(ch * 8 + j, G - 1)) * D + sg * E);
  };
  auto q_store = [&](int i, const uint4* v) {
    const int ch = i / QS, hs = i - ch * QS;
    const int h = hs / LH, sg = hs - h * LH;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (ch * 8 + j < G) {
        float f[E];
        V::unpack(v[j], f);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += f[e];
      }
    }
    float* dst = NCH == 1 ? qbar : qpart + (size_t)ch * a.H_kv * D;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[h * D + sg * E + e] = NCH == 1 ? acc[e] * invG : acc[e];
  };
  uint4 qv[8];
  q_load(tid, qv);
  const int32_t* ptb = a.pt + (size_t)b * a.pt_stride + a.n_bos;
  const int c0 = blockIdx.x * a.cand_per_block;
  const int pv = ptb[max(min(c0 + tid, a.score_stride - a.n_bos - 1), 0)];   // used for tid < nc

  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + a.S_p - 1) / a.S_p;
  const int n_cand = n_b - a.n_bos - a.n_eos;
  // the completed page's centroid rows, shared by the request's blocks by
  // (KV head, segment) units: page id now, rows once the scoring loads are
  // issued, sums after the scoring
  using SC = SegmentCentroid<T, D, kScoreThreads, kScoreCentroidPairs / kScoreThreads>;
  const int n_units = a.H_kv * SC::S::SEGS;
  const int u0 = (int)((long long)blockIdx.x * n_units / gridDim.x);
  const int nu = (int)((long long)(blockIdx.x + 1) * n_units / gridDim.x) - u0;
  const bool upd = a.update_completed && nu > 0 && seq > 0 && seq % a.S_p == 0;
  const int cpage = upd ? a.pt[(size_t)b * a.pt_stride + n_b - 1] : 0;
  SC sc;
  auto centroid_load = [&]() {
    if (upd)
      sc.load(reinterpret_cast<const T*>(a.k) + (size_t)cpage * a.H_kv * a.S_p * D, a.S_p, u0, nu);
  };
  float* cred = smem + a.H_kv * D + a.cand_per_block + (NCH > 1 ? NCH * a.H_kv * D : 0);
  // staged scores [H_kv][nc]: the completed page's reduction reuses this LDS
  // only after the rows are written out
  float* sst = cred;
  auto centroid_done = [&]() {
    if (!upd) return;
    sc.reduce(cred, a.S_p, nu);
    __syncthreads();
    if (tid < nu)
      SC::finish(cred, a.S_p, reinterpret_cast<T*>(a.cent_out) + (size_t)cpage * a.H_kv * D, u0, tid);
  };
  if (c0 >= n_cand) {
    centroid_load();
    centroid_done();
    return;
  }
  const int c1 = min(c0 + a.cand_per_block, n_cand);
  const int nc = c1 - c0;
  if (tid < nc) phys[tid] = pv;
  for (int i = tid + kScoreThreads; i < nc; i += kScoreThreads) phys[i] = ptb[c0 + i];
  __syncthreads();

  // group-mean queries into qbar (every query load was issued first)
  auto q_finish = [&]() {
    if (tid < QS * NCH) q_store(tid, qv);
    for (int i = tid + kScoreThreads; i < QS * NCH; i += kScoreThreads) {
      q_load(i, qv);
      q_store(i, qv);
    }
    if (NCH > 1) {
      __syncthreads();
      for (int i = tid; i < a.H_kv * D; i += kScoreThreads) {
        float x = 0.f;
        for (int ch = 0; ch < NCH; ++ch) x += qpart[(size_t)ch * a.H_kv * D + i];
        qbar[i] = x * invG;
      }
    }
    __syncthreads();
  };

  const T* cent = reinterpret_cast<const T*>(a.cent);
  float* out = a.scores + (size_t)b * a.H_kv * a.score_stride;
  const int rows = nc * a.H_kv;
  // score of candidate c0 + c for KV head h: into LDS when staging (stores of
  // single words scattered over H_kv rows cost more than the final row copy)
  auto put = [&](int h, int c, float v) {
    if (LH <= 64 && a.stage_scores)
      sst[h * nc + c] = v;
    else
      out[(size_t)h * a.score_stride + c0 + c] = v;
  };

  if constexpr (LH <= 64) {
    // Rows r = c * H_kv + h (the H_kv rows of a page are contiguous), R per
    // wave-load, lane group grp taking rows wave * R + grp + STEP * j.  A
    // wave's rows come in batches of U wave-loads; load u of the next batch
    // is issued as soon as load u of this batch is consumed, so U loads stay
    // in flight per lane through the whole scoring (past the last row the
    // index is clamped to it: the surplus loads of the last batch hit the
    // cache).  Each lane keeps the sums of its group's loads seg, seg + LH,
    // ... and stores them after the batch.
    constexpr int R = 64 / LH;              // rows per wave-load
    constexpr int STEP = (kScoreThreads / 64) * R;   // rows per block-wide wave-load
    constexpr int U = kSplitLoads;
    constexpr int NS = (U + LH - 1) / LH;   // sums a lane stores per batch
    const int seg = lane % LH, grp = lane / LH;
    const int rw = wave * R + grp;          // this lane's first row
    const int nbat = rows > wave * R ? (rows - wave * R + STEP * U - 1) / (STEP * U) : 0;
    auto row_off = [&](int r) -> size_t {
      const int rc = min(r, rows - 1);
      const int c = rc / a.H_kv, h = rc - c * a.H_kv;
      return ((size_t)phys[c] * a.H_kv + h) * D + seg * E;
    };
    const T* cs = cent;
    uint4 buf[U];
    if (nbat > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) buf[u] = ld16(cs + row_off(rw + u * STEP));
    }
    q_finish();
    centroid_load();
    // with H_kv dividing STEP every row a lane touches has the same KV head,
    // so that head's query segment stays in registers
    const bool fixed_head = STEP % a.H_kv == 0;
    float qr[E];
    {
      const int h0 = rw % a.H_kv;
#pragma unroll
      for (int e = 0; e < E; ++e) qr[e] = qbar[h0 * D + seg * E + e];
    }
    for (int k = 0; k < nbat; ++k) {
      const int r0 = rw + k * STEP * U;     // this lane's row of load 0
      size_t nx[U];
#pragma unroll
      for (int u = 0; u < U; ++u) nx[u] = row_off(r0 + STEP * U + u * STEP);
      float mine[NS];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * STEP;
        float f[E];
        V::unpack(buf[u], f);
        buf[u] = ld16(cs + nx[u]);
        float acc = 0.f;
        if (fixed_head) {
#pragma unroll
          for (int e = 0; e < E; ++e) acc = fmaf(qr[e], f[e], acc);
        } else {
          const int rc = r < rows ? r : 0;
          const int h = rc - (rc / a.H_kv) * a.H_kv;
          const float* qh = qbar + h * D + seg * E;
#pragma unroll
          for (int e = 0; e < E; ++e) acc = fmaf(qh[e], f[e], acc);
        }
        acc = lane_group_sum<LH>(acc);
        if (seg == u % LH) mine[u / LH] = acc;
      }
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int u = seg + j * LH;
        const int r = r0 + u * STEP;
        if (u < U && r < rows) {
          const int c = r / a.H_kv, h = r - c * a.H_kv;
          put(h, c, mine[j]);
        }
      }
    }
  } else {
    // Rows of more than 64 segments (MLA: 72).  Eight rows form a tile of
    // 9 wave-loads: eight "head" loads of segments 0..63 of one row each and
    // one "tail" load of segments 64..71 of all eight rows.
    static_assert(LH > 64 && LH <= 72, "row width");
    constexpr int TL = LH - 64;             // tail segments per row (8)
    constexpr int RT = 64 / TL;             // rows per tile (8)
    struct Tile { uint4 hb[RT]; uint4 tb; };
    auto issue = [&](int r0, Tile& tl) {     // rows past the last are clamped to it
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int r = min(r0 + i, rows - 1);
        const int c = r / a.H_kv, h = r - c * a.H_kv;
        tl.hb[i] = ld16(cent + ((size_t)phys[c] * a.H_kv + h) * D + lane * E);
      }
      const int tr = min(r0 + lane / TL, rows - 1), tseg = 64 + lane % TL;
      const int c = tr / a.H_kv, h = tr - c * a.H_kv;
      tl.tb = ld16(cent + ((size_t)phys[c] * a.H_kv + h) * D + tseg * E);
    };
    // eight rows per tile, two tiles in flight per wave, both issued before
    // the queries are formed
    constexpr int NW = kScoreThreads / 64;
    Tile ta, tb;
    int r0 = wave * RT;
    if (r0 < rows) issue(r0, ta);
    if (r0 + NW * RT < rows) issue(r0 + NW * RT, tb);
    q_finish();
    centroid_load();
    // with one KV head (MLA) the query segments a lane needs stay in registers
    const bool one_head = a.H_kv == 1;
    float qh1[E], qt1[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      qh1[e] = qbar[lane * E + e];
      qt1[e] = qbar[(64 + lane % TL) * E + e];
    }
    auto consume = [&](int r0, const Tile& tl) {
      const int tr = r0 + lane / TL, tseg = 64 + lane % TL;
      float tp;
      {
        const int trc = tr < rows ? tr : 0;
        const int c = trc / a.H_kv, h = trc - c * a.H_kv;
        float f[E];
        V::unpack(tl.tb, f);
        const float* qh = qbar + h * D + tseg * E;
        tp = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) tp = fmaf(one_head ? qt1[e] : qh[e], f[e], tp);
        tp = row_sum<TL>(tp);               // sum over the TL lanes of one row
      }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int r = r0 + i;
        const int rc = r < rows ? r : 0;
        const int c = rc / a.H_kv, h = rc - c * a.H_kv;
        float f[E];
        V::unpack(tl.hb[i], f);
        const float* qh = qbar + h * D + lane * E;
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf(one_head ? qh1[e] : qh[e], f[e], acc);
        acc = lane_group_sum<64>(acc) +
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tp), i * TL));
        if (lane == 0 && r < rows) out[(size_t)h * a.score_stride + c0 + c] = acc;
      }
    };
    for (; r0 < rows; r0 += 2 * NW * RT) {
      const int r1 = r0 + NW * RT, r2 = r1 + NW * RT, r3 = r2 + NW * RT;
      consume(r0, ta);
      if (r2 < rows) issue(r2, ta);
      if (r1 < rows) consume(r1, tb);
      if (r3 < rows) issue(r3, tb);
    }
  }
  if (LH <= 64 && a.stage_scores) {
    __syncthreads();
    for (int i = tid; i < rows; i += kScoreThreads) {
      const int h = i / nc, c = i - h * nc;
      out[(size_t)h * a.score_stride + c0 + c] = sst[i];
    }
    __syncthreads();                        // sst is the centroid reduction's LDS
  }
  centroid_done();
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ __align__(16) uint32_t keys[];   // [round4(n_cand)]
  __shared__ SelectLds<kTopkThreads> sl;

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;                // b * H_kv + h
  const int b = bh / a.H_kv;
  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + a.S_p - 1) / a.S_p;
  const int n_cand = max(n_b - a.n_bos - a.n_eos, 0);
  select_init<kTopkThreads>(sl);
  __syncthreads();
  if (n_cand > a.topk && a.topk > 0) {
    // eight scores per thread in flight, then converted and counted
    const float* sc = a.scores + (size_t)bh * a.score_stride;
    for (int i0 = tid; i0 < n_cand; i0 += 8 * kTopkThreads) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + j * kTopkThreads;
        v[j] = i < n_cand ? sc[i] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + j * kTopkThreads;
        if (i < n_cand) {
          const uint32_t k = order_key(v[j]);
          keys[i] = k;
          select_count<kTopkThreads>(sl, k);
        }
      }
    }
  }
  select_pages<kTopkThreads>(keys, n_cand, n_b, a.topk, a.n_bos, a.n_eos, a.k_tot,
                             a.sel + (size_t)bh * a.k_tot, nullptr, sl, a.levels,
                             a.rnd ? a.rnd[bh] : 0u);
}

// LDS of the completed-page centroid share of the busiest scoring block.
template <typename T, int D>
size_t score_centroid_lds(int H_kv, int grid_x) {
  using S = CentroidShape<T, D>;
  const int per_block = (H_kv * S::SEGS + grid_x - 1) / grid_x;
  return (size_t)per_block * S::RG * S::E * sizeof(float);
}

// Largest staged score block (LDS): beyond it scores are stored directly.
constexpr size_t kScoreStageBytes = 32 * 1024;

template <typename T, int D>
hipError_t run_score(const ScoreArgs& a, int grid_x, hipStream_t s) {
  const int G = a.H_q / a.H_kv, nch = (G + 7) / 8;
  ScoreArgs b = a;
  const size_t stage = (size_t)a.H_kv * a.cand_per_block * sizeof(float);
  b.stage_scores = D / Vec16<T>::E <= 64 && stage <= kScoreStageBytes;
  const size_t tail = std::max(a.update_completed ? score_centroid_lds<T, D>(a.H_kv, grid_x) : 0,
                               b.stage_scores ? stage : 0);
  const size_t lds = (size_t)a.H_kv * D * sizeof(float) + (size_t)a.cand_per_block * sizeof(int32_t) +
                     (nch > 1 ? (size_t)nch * a.H_kv * D * sizeof(float) : 0) + tail;
  hipLaunchKernelGGL((score_kernel<T, D>), dim3(grid_x, a.B), dim3(kScoreThreads), lds, s, b);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_fused(const ScoreArgs& a, const TopkArgs& t, bool bounds, hipStream_t s) {
  const size_t lds = 2 * (size_t)round4(a.score_stride > 0 ? a.score_stride : 1) * sizeof(uint32_t);
  if (bounds)
    hipLaunchKernelGGL((indexer_fused_kernel<T, D, true>), dim3(a.H_kv, a.B), dim3(kFusedThreads),
                       lds, s, a, t);
  else
    hipLaunchKernelGGL((indexer_fused_kernel<T, D, false>), dim3(a.H_kv, a.B), dim3(kFusedThreads),
                       lds, s, a, t);
  return hipGetLastError();
}

}  // namespace

bool fused_indexer_supported(int dtype, int D) {
  return (dtype == 0 && (D == 64 || D == 128)) || (dtype == 1 && (D == 64 || D == 128));
}

template <typename T, int D>
bool centroid_share_fits(int H_kv, int grid_x) {
  using S = CentroidShape<T, D>;
  return (H_kv * S::SEGS + grid_x - 1) / grid_x * S::RG <= kScoreCentroidPairs;
}

bool score_centroid_fits(int dtype, int D, int H_kv, int grid_x) {
  if (grid_x < 1) return false;
  if (dtype == 0) {
    if (D == 64) return centroid_share_fits<float, 64>(H_kv, grid_x);
    if (D == 128) return centroid_share_fits<float, 128>(H_kv, grid_x);
  } else {
    if (D == 64) return centroid_share_fits<bf16_t, 64>(H_kv, grid_x);
    if (D == 128) return centroid_share_fits<bf16_t, 128>(H_kv, grid_x);
    if (D == 576) return centroid_share_fits<bf16_t, 576>(H_kv, grid_x);
  }
  return false;
}

hipError_t launch_score(int dtype, const ScoreArgs& a, int grid_x, hipStream_t s) {
  if (dtype == 0) {
    switch (a.D) {
      case 64: return run_score<float, 64>(a, grid_x, s);
      case 128: return run_score<float, 128>(a, grid_x, s);
    }
  } else {
    switch (a.D) {
      case 64: return run_score<bf16_t, 64>(a, grid_x, s);
      case 128: return run_score<bf16_t, 128>(a, grid_x, s);
      case 576: return run_score<bf16_t, 576>(a, grid_x, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_indexer_fused(int dtype, const ScoreArgs& a, const TopkArgs& t, hipStream_t s,
                                bool bounds) {
  if (dtype == 0) {
    switch (a.D) {
      case 64: return run_fused<float, 64>(a, t, bounds, s);
      case 128: return run_fused<float, 128>(a, t, bounds, s);
    }
  } else {
    switch (a.D) {
      case 64: return run_fused<bf16_t, 64>(a, t, bounds, s);
      case 128: return run_fused<bf16_t, 128>(a, t, bounds, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const TopkArgs& a, int max_cand, hipStream_t s) {
  const size_t lds = (size_t)round4(max_cand > 0 ? max_cand : 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_kernel, dim3(a.B * a.H_kv), dim3(kTopkThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace vx
