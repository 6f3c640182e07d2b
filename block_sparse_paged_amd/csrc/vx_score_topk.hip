// K2 + K3: the query-dependent indexer of block-top-k sparse attention
// (vortex_torch README, "Quick Example": the query is averaged over heads,
// GeMV'd against the page centroids, and topK writes the page index
// structure; "Using Your Sparse Attention with SGLang": reserved first / last
// pages and the top-k value).
//
// K2 score_kernel  - grid (candidate chunks, B), 4 waves per block.  The
//   group-mean queries of all KV heads of the request sit in LDS (fp32).
//   Centroid rows are gathered through the page table; for one page the H_kv
//   rows are contiguous (H_kv * D * e bytes), so a wave-load of 16 bytes per
//   lane reads 1 KiB of consecutive heads.  Each (page, head) dot product is
//   reduced across the lanes holding that row.  Scores go to the workspace
//   indexed by candidate number.
// K3 topk_kernel   - one 256-thread block per (request, KV head).  Scores are
//   mapped to order-preserving uint32 keys in LDS, the k-th largest key is
//   found by a 4-pass 8-bit radix select (LDS histograms), keys equal to the
//   threshold are taken lowest-index first via a block-wide scan, and the
//   union with the reserved pages is compacted in ascending page order.
#include "vx_device.h"
#include "vx_internal.h"

namespace vx {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  using V = Vec16<T>;
  constexpr int E = V::E;
  constexpr int LH = D / E;                 // 16-byte segments per centroid row
  extern __shared__ float smem[];           // qbar [H_kv][D] then phys ids
  float* qbar = smem;
  int32_t* phys = reinterpret_cast<int32_t*>(smem + a.H_kv * D);

  const int b = blockIdx.y;
  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + a.S_p - 1) / a.S_p;
  const int n_cand = n_b - a.n_bos - a.n_eos;
  const int c0 = blockIdx.x * a.cand_per_block;
  if (c0 >= n_cand) return;
  const int c1 = min(c0 + a.cand_per_block, n_cand);
  const int nc = c1 - c0;
  const int tid = threadIdx.x;

  // group-mean query of every KV head, fp32, summed in head order
  const int G = a.H_q / a.H_kv;
  const T* qb = reinterpret_cast<const T*>(a.q) + (size_t)b * a.H_q * D;
  const float invG = 1.0f / (float)G;
  for (int i = tid; i < a.H_kv * D; i += kScoreThreads) {
    const int h = i / D, d = i - h * D;
    float s = 0.f;
    for (int g = 0; g < G; ++g) s += V::to_f32(qb[(size_t)(h * G + g) * D + d]);
    qbar[i] = s * invG;
  }
  const int32_t* ptb = a.pt + (size_t)b * a.pt_stride + a.n_bos;
  for (int i = tid; i < nc; i += kScoreThreads) phys[i] = ptb[c0 + i];
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const T* cent = reinterpret_cast<const T*>(a.cent);
  float* out = a.scores + (size_t)b * a.H_kv * a.score_stride;
  const int rows = nc * a.H_kv;

  if constexpr (LH <= 64) {
    constexpr int R = 64 / LH;              // rows per wave-load
    constexpr int U = 4;                    // wave-loads in flight
    const int seg = lane % LH, grp = lane / LH;
    const int step = 4 * R;                 // rows advanced per wave-load by the block
    for (int r0 = wave * R; r0 < rows; r0 += step * U) {
      uint4 buf[U];
      int rr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * step + grp;
        rr[u] = r;
        if (r < rows) {
          const int c = r / a.H_kv, h = r - c * a.H_kv;
          buf[u] = ld16(cent + ((size_t)phys[c] * a.H_kv + h) * D + seg * E);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = rr[u];
        const int rc = r < rows ? r : 0;
        const int c = rc / a.H_kv, h = rc - c * a.H_kv;
        float f[E];
        V::unpack(r < rows ? buf[u] : make_uint4(0, 0, 0, 0), f);
        const float* qh = qbar + h * D + seg * E;
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf(qh[e], f[e], acc);
        acc = group_sum<LH>(acc);
        if (seg == 0 && r < rows) out[(size_t)h * a.score_stride + c0 + c] = acc;
      }
    }
  } else {
    // rows wider than a wave (MLA): one row per wave-step, full-wave reduce
    for (int r = wave; r < rows; r += 4) {
      const int c = r / a.H_kv, h = r - c * a.H_kv;
      const T* row = cent + ((size_t)phys[c] * a.H_kv + h) * D;
      const float* qh = qbar + h * D;
      float acc = 0.f;
      for (int seg = lane; seg < LH; seg += 64) {
        float f[E];
        V::unpack(ld16(row + seg * E), f);
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf(qh[seg * E + e], f[e], acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) out[(size_t)h * a.score_stride + c0 + c] = acc;
    }
  }
}

// Exclusive scan of one int per thread over a 256-thread block, in thread
// order.  `tmp` holds at least 4 ints of LDS.  Returns the block total too.
__device__ __forceinline__ int block_exclusive_scan(int x, int* tmp, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int inc = wave_inclusive_scan(x);
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const int t = tmp[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + inc - x;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);   // -0 and +0 are equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t keys[];        // [n_cand]
  __shared__ int hist[256];
  __shared__ int scan_tmp[4];
  __shared__ int pick[2];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;                // b * H_kv + h
  const int b = bh / a.H_kv;
  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + a.S_p - 1) / a.S_p;
  const int n_cand = max(n_b - a.n_bos - a.n_eos, 0);
  const bool all = n_cand <= a.topk;
  int32_t* out = a.sel + (size_t)bh * a.k_tot;

  uint32_t thr = 0xFFFFFFFFu;   // keys above thr are taken ...
  int take_eq = 0;              // ... and the first take_eq keys equal to thr
  const bool none = !all && a.topk == 0;
  if (!all && !none) {
    const float* sc = a.scores + (size_t)bh * a.score_stride;
    for (int i = tid; i < n_cand; i += kTopkThreads) keys[i] = order_key(sc[i]);
    uint32_t prefix = 0, mask = 0;
    int remaining = a.topk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n_cand; i += kTopkThreads) {
        const uint32_t k = keys[i];
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns bins 4l..4l+3; count keys in bins above each bin
        const int h0 = hist[4 * tid], h1 = hist[4 * tid + 1];
        const int h2 = hist[4 * tid + 2], h3 = hist[4 * tid + 3];
        const int own = h0 + h1 + h2 + h3;
        // exclusive suffix sum over lanes (higher lanes hold higher bins)
        int suf = own;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_down(suf, d, 64);
          if (tid + d < 64) suf += y;
        }
        int above = suf - own;              // keys in bins of higher lanes
        int digit = -1, above_d = 0;
        if (above + h3 >= remaining && above < remaining) { digit = 4 * tid + 3; above_d = above; }
        above += h3;
        if (digit < 0 && above + h2 >= remaining && above < remaining) { digit = 4 * tid + 2; above_d = above; }
        above += h2;
        if (digit < 0 && above + h1 >= remaining && above < remaining) { digit = 4 * tid + 1; above_d = above; }
        above += h1;
        if (digit < 0 && above + h0 >= remaining && above < remaining) { digit = 4 * tid; above_d = above; }
        if (digit >= 0) { pick[0] = digit; pick[1] = above_d; }
      }
      __syncthreads();
      prefix |= (uint32_t)pick[0] << shift;
      mask |= 0xFFu << shift;
      remaining -= pick[1];
      __syncthreads();
    }
    thr = prefix;
    take_eq = remaining;
  }

  // Thread tid owns logical pages [tid*per, tid*per + per).
  const int per = (n_b + kTopkThreads - 1) / kTopkThreads;
  const int p_lo = min(tid * per, n_b), p_hi = min(p_lo + per, n_b);
  // rank of equal-to-threshold candidates, in page order
  int n_eq = 0;
  if (!all && !none) {
    for (int p = p_lo; p < p_hi; ++p) {
      const int c = p - a.n_bos;
      if (c >= 0 && c < n_cand && keys[c] == thr) ++n_eq;
    }
  }
  int dummy;
  int eq_rank = block_exclusive_scan(n_eq, scan_tmp, &dummy);
  // which pages are taken, counted per thread
  const int eos_lo = n_b - a.n_eos;
  int n_take = 0;
  for (int p = p_lo; p < p_hi; ++p) {
    const int c = p - a.n_bos;
    bool take;
    if (p < a.n_bos || p >= eos_lo) {
      take = true;
    } else if (all || none) {
      take = all;
    } else {
      const uint32_t k = keys[c];
      take = k > thr || (k == thr && eq_rank < take_eq);
      if (k == thr) ++eq_rank;
    }
    n_take += take ? 1 : 0;
  }
  int total;
  int pos = block_exclusive_scan(n_take, scan_tmp, &total);
  // second pass writes the taken pages (recomputing the same decisions)
  eq_rank -= n_eq;
  for (int p = p_lo; p < p_hi; ++p) {
    const int c = p - a.n_bos;
    bool take;
    if (p < a.n_bos || p >= eos_lo) {
      take = true;
    } else if (all || none) {
      take = all;
    } else {
      const uint32_t k = keys[c];
      take = k > thr || (k == thr && eq_rank < take_eq);
      if (k == thr) ++eq_rank;
    }
    if (take) out[pos++] = p;
  }
  for (int i = total + tid; i < a.k_tot; i += kTopkThreads) out[i] = -1;
}

template <typename T, int D>
hipError_t run_score(const ScoreArgs& a, int grid_x, hipStream_t s) {
  const size_t lds = (size_t)a.H_kv * D * sizeof(float) + (size_t)a.cand_per_block * sizeof(int32_t);
  hipLaunchKernelGGL((score_kernel<T, D>), dim3(grid_x, a.B), dim3(kScoreThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

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

hipError_t launch_topk(const TopkArgs& a, int max_cand, hipStream_t s) {
  const size_t lds = (size_t)(max_cand > 0 ? max_cand : 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_kernel, dim3(a.B * a.H_kv), dim3(kTopkThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace vx
