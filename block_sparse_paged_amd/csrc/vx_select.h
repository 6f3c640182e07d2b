// Exact page selection shared by the indexer kernels and the fused decode
// step: order-preserving keys, an 8-bit radix select for the k-th largest
// key, index-ordered ranking of keys equal to it (ties go to the lower
// logical page), and the ascending union with the reserved first / last
// pages (vortex_torch README, "Quick Example" topK and "Using Your Sparse
// Attention with SGLang" reserved BOS / EOS pages).
#pragma once

#include "vx_device.h"
#include "vx_internal.h"

namespace vx {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);   // -0 and +0 are equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one int per thread over an NT-thread block, in thread
// order.  `tmp` holds NT/64 ints of LDS.  Also returns the block total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int* tmp, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int inc = wave_inclusive_scan(x);
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = tmp[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + inc - x;
}

// Selects and writes one (request, KV head) row of `sel` (and, when
// `lds_out` is given, the same list into LDS); returns the number of pages
// taken.
//   keys     LDS, n_cand order-preserving keys of candidates n_bos.. (in page order)
//   hist     LDS, 4*256 ints, zero on entry
// Keys and the zeroed histograms must be visible to every thread (the caller
// synchronises first).
//   kmax/kmin the largest / smallest key (bytes above the first byte in which
//            they differ are common to every key, so those passes are skipped)
template <int NT>
__device__ int select_pages(const uint32_t* keys, int n_cand, int n_b, int topk, int n_bos,
                            int n_eos, int k_tot, int32_t* out, int32_t* lds_out, int* hist,
                            int* scan_tmp, uint32_t kmax, uint32_t kmin) {
  const int tid = threadIdx.x, lane = tid & 63;
  const bool all = n_cand <= topk;
  const bool none = !all && topk == 0;
  uint32_t thr = 0, msk = 0;
  int take_eq = 0, cnt_eq = 0;
  if (!all && !none) {
    int remaining = topk;
    const uint32_t diff = kmax ^ kmin;
    const int hb = diff ? 31 - __builtin_clz(diff) : 0;
    const int first = 3 - hb / 8;
    msk = first ? (0xFFFFFFFFu << (32 - 8 * first)) : 0u;
    thr = kmax & msk;
    cnt_eq = n_cand;
    for (int pass = first; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      int* H = hist + 256 * pass;
      for (int i = tid; i < n_cand; i += NT) {
        const uint32_t k = keys[i];
        if ((k & msk) == thr) atomicAdd(&H[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      // every wave finds the bin where the count from the top crosses `remaining`
      const int h0 = H[4 * lane], h1 = H[4 * lane + 1], h2 = H[4 * lane + 2], h3 = H[4 * lane + 3];
      const int own = h0 + h1 + h2 + h3;
      int suf = own;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_down(suf, d, 64);
        if (lane + d < 64) suf += y;
      }
      int acc = suf - own, dsel = -1, above = 0, cnt = 0;
      if (acc < remaining && acc + h3 >= remaining) { dsel = 4 * lane + 3; above = acc; cnt = h3; }
      acc += h3;
      if (dsel < 0 && acc < remaining && acc + h2 >= remaining) { dsel = 4 * lane + 2; above = acc; cnt = h2; }
      acc += h2;
      if (dsel < 0 && acc < remaining && acc + h1 >= remaining) { dsel = 4 * lane + 1; above = acc; cnt = h1; }
      acc += h1;
      if (dsel < 0 && acc < remaining && acc + h0 >= remaining) { dsel = 4 * lane; above = acc; cnt = h0; }
      const unsigned long long found = __ballot(dsel >= 0);
      const int src = __builtin_ctzll(found);
      const int d = __builtin_amdgcn_readlane(dsel, src);
      above = __builtin_amdgcn_readlane(above, src);
      cnt = __builtin_amdgcn_readlane(cnt, src);
      remaining -= above;
      thr |= (uint32_t)d << shift;
      msk |= 0xFFu << shift;
      cnt_eq = cnt;
      if (remaining == cnt) break;    // the whole boundary bin is taken
    }
    take_eq = remaining;
  }
  const bool need_rank = !all && !none && take_eq < cnt_eq;

  // thread tid owns logical pages [p_lo, p_hi)
  const int per = (n_b + NT - 1) / NT;
  const int p_lo = min(tid * per, n_b), p_hi = min(p_lo + per, n_b);
  const int eos_lo = n_b - n_eos;
  int eq_rank = 0, dummy;
  if (need_rank) {
    int n_eq = 0;
    for (int p = max(p_lo, n_bos); p < min(p_hi, eos_lo); ++p) n_eq += (keys[p - n_bos] & msk) == thr;
    eq_rank = block_exclusive_scan<NT>(n_eq, scan_tmp, &dummy);
  }
  auto take = [&](int p, int& rank) -> bool {
    if (p < n_bos || p >= eos_lo) return true;
    if (all || none) return all;
    const uint32_t km = keys[p - n_bos] & msk;
    bool t = km > thr;
    if (km == thr) {
      t = !need_rank || rank < take_eq;
      ++rank;
    }
    return t;
  };
  int r = eq_rank, n_take = 0;
  for (int p = p_lo; p < p_hi; ++p) n_take += take(p, r) ? 1 : 0;
  int total;
  int pos = block_exclusive_scan<NT>(n_take, scan_tmp, &total);
  r = eq_rank;
  for (int p = p_lo; p < p_hi; ++p)
    if (take(p, r)) {
      out[pos] = p;
      if (lds_out) lds_out[pos] = p;
      ++pos;
    }
  for (int i = total + tid; i < k_tot; i += NT) out[i] = -1;
  return total;
}

// Block-wide max and min of per-thread key bounds (NT threads, LDS `tmp` of
// 2 * NT/64 words).  Synchronises.
template <int NT>
__device__ __forceinline__ void block_key_bounds(uint32_t& kmax, uint32_t& kmin, uint32_t* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, 64));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, m, 64));
  }
  if (lane == 0) {
    tmp[wave] = kmax;
    tmp[NT / 64 + wave] = kmin;
  }
  __syncthreads();
  kmax = 0u;
  kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    kmax = max(kmax, tmp[w]);
    kmin = min(kmin, tmp[NT / 64 + w]);
  }
}


// Group-mean query of KV head h of request b into LDS `qbar` (fp32, heads
// summed in order).  Every thread of the NT-thread block takes part.
template <typename T, int D, int NT>
__device__ __forceinline__ void head_query_mean(const ScoreArgs& a, int b, int h, float* qbar) {
  using V = Vec16<T>;
  constexpr int E = V::E, LH = D / E;
  const int G = a.H_q / a.H_kv;
  const T* qb = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.H_q + (size_t)h * G) * D;
  // one 16-byte segment per thread, eight heads' loads in flight, summed in order
  for (int sg = threadIdx.x; sg < LH; sg += NT) {
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int g0 = 0; g0 < G; g0 += 8) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (g0 + j < G) v[j] = ld16(qb + (size_t)(g0 + j) * D + sg * E);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (g0 + j < G) {
          float f[E];
          V::unpack(v[j], f);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] += f[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) qbar[sg * E + e] = acc[e] * (1.0f / (float)G);
  }
}

// Scores of candidates [0, n_cand) of KV head h into LDS `keys` as
// order-preserving keys; phys[c] is candidate c's physical page.  Rows are
// one head's centroid row (<= 64 lanes of 16 bytes); each wave keeps
// kScoreLoads wave-loads in flight.  Also tracks the thread's key bounds.
constexpr int kScoreLoads = 16;

template <typename T, int D, int NT>
__device__ __forceinline__ void score_head(const ScoreArgs& a, int h, int n_cand,
                                           const int32_t* phys, const float* qbar,
                                           uint32_t* keys, uint32_t& kmax, uint32_t& kmin) {
  using V = Vec16<T>;
  constexpr int E = V::E;
  constexpr int LH = D / E;                  // lanes per centroid row
  constexpr int R = 64 / LH;                 // rows per wave-load
  constexpr int NW = NT / 64;
  constexpr int U = kScoreLoads;
  static_assert(LH * R == 64, "rows of at most 64 lanes");
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seg = lane % LH, grp = lane / LH;
  float qr[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qr[e] = qbar[seg * E + e];
  const T* cent = reinterpret_cast<const T*>(a.cent);
  constexpr int STEP = NW * R;               // rows per block-wide wave-load
  for (int r0 = w * R; r0 < n_cand; r0 += STEP * U) {
    uint4 buf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = r0 + u * STEP + grp;
      buf[u] = c < n_cand ? ld16(cent + ((size_t)phys[c] * a.H_kv + h) * D + seg * E)
                          : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = r0 + u * STEP + grp;
      float f[E];
      V::unpack(buf[u], f);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc = fmaf(qr[e], f[e], acc);
      acc = lane_group_sum<LH>(acc);
      if (c < n_cand) {
        const uint32_t k = order_key(acc);
        kmax = max(kmax, k);
        kmin = min(kmin, k);
        if (seg == 0) keys[c] = k;
      }
    }
  }
}

}  // namespace vx
