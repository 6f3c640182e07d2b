// Exact page selection shared by the indexer kernels and the fused decode
// step (vortex_torch README, "Quick Example" topK, and "Using Your Sparse
// Attention with SGLang" reserved BOS / EOS pages): the top-k candidates by
// score, ties to the lower logical page, unioned with the reserved first /
// last pages and listed in ascending page order.
//
// Scores become order-preserving 32-bit keys.  The k-th largest (key, page)
// pair is located by histograms: level 0 counts the keys in 1024 fixed bins
// (the top ten key bits: sign, exponent and one mantissa bit, i.e. half an
// octave of score) and is filled by the caller while it computes the keys;
// each further level splits the boundary bin's key range into at most 1024
// equal bins, until the boundary bin is taken whole or holds one key value
// (then equal keys are taken in page order).  A candidate is taken iff
// (key, -page) >= the threshold pair.  Every step is a few dozen
// instructions per wave: this runs on each block's critical path.
#pragma once

#include <limits.h>

#include "vx_device.h"
#include "vx_internal.h"

namespace vx {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);   // -0 and +0 are equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelBits = 10;
constexpr int kSelBins = 1 << kSelBits;
constexpr int kSelShift0 = 32 - kSelBits;     // level-0 bin of a key: key >> 22

// Histogram slot of bin i: 4 words of padding after every 16 bins, so that
// 16-byte reads of 16 consecutive bins by consecutive lanes spread over all
// LDS banks.
__device__ __forceinline__ int sel_slot(int i) { return i + (i >> 4) * 4; }
constexpr int kSelHistWords = kSelBins + kSelBins / 4;


// LDS of one selection (NT threads): two histograms (levels alternate).
template <int NT>
struct SelectLds {
  alignas(16) int hist[2][kSelHistWords];
  int wsum[2][NT / 64];
  int misc[4];     // [0] tie threshold, [2] score_head's batch counter
};

static_assert(sizeof(SelectLds<512>) <= kSelectLdsBytes, "selection LDS bound");

// Clears both histograms; the caller synchronises before the keys (and their
// level-0 counts) are produced.
template <int NT>
__device__ __forceinline__ void select_init(SelectLds<NT>& S) {
  int* h = &S.hist[0][0];
  for (int i = threadIdx.x; i < 2 * kSelHistWords; i += NT) h[i] = 0;
  if (threadIdx.x == 0) S.misc[2] = 0;
}

// Level-0 count of one key (any thread, any time before select_pages).
template <int NT>
__device__ __forceinline__ void select_count(SelectLds<NT>& S, uint32_t key) {
  atomicAdd(&S.hist[0][sel_slot((int)(key >> kSelShift0))], 1);
}

// Exclusive scan of one int per thread over an NT-thread block, in thread
// order, through LDS `wsum` (NT/64 ints).  Also returns the block total.
// Synchronises once; `wsum` may not be reused before the next barrier.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int inc = wave_inclusive_scan(x);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = wsum[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  *total = tot;
  return base + inc - x;
}

// In a histogram of 1024 bins, the bin where the count from the top reaches
// `remaining` (1 <= remaining <= total): returns the bin, the count above it
// and its own count, the same in every lane.  Lane l first sums bins
// 16l .. 16l + 15 to find the crossing lane, then lanes 0..15 take one bin
// each of that lane, from the top down.
__device__ __forceinline__ void find_bin(const int* hist, int remaining, int& dsel, int& above,
                                         int& cnt) {
  const int lane = threadIdx.x & 63;
  const int4* hp = reinterpret_cast<const int4*>(hist + sel_slot(16 * lane));
  const int4 a = hp[0], b = hp[1], c = hp[2], d = hp[3];
  const int own = (a.x + a.y + a.z + a.w) + (b.x + b.y + b.z + b.w) +
                  (c.x + c.y + c.z + c.w) + (d.x + d.y + d.z + d.w);
  const int inc = wave_inclusive_scan(own);
  const int upper = __builtin_amdgcn_readlane(inc, 63) - inc;   // keys in lanes above
  const unsigned long long cross = __ballot(upper < remaining && upper + own >= remaining);
  const int L = __builtin_ctzll(cross);
  const int upL = __builtin_amdgcn_readlane(upper, L);
  const int j = lane & 15;
  const int hv = hist[sel_slot(16 * L + 15 - j)];
  const int incj = row_inclusive_scan(hv);                      // bins from the top down
  const unsigned long long hit =
      __ballot(lane < 16 && upL + incj - hv < remaining && upL + incj >= remaining);
  const int J = __builtin_ctzll(hit);
  dsel = 16 * L + 15 - J;
  above = upL + __builtin_amdgcn_readlane(incj - hv, J);
  cnt = __builtin_amdgcn_readlane(hv, J);
}

// Selects one (request, KV head)'s pages and returns how many were taken.
// The list goes to LDS `lds_out` when given (the caller writes the row of
// `sel` later, so that no barrier waits on those global stores), else to
// `out` (a row of k_tot entries, padded with -1).
//   keys   LDS, 16-byte aligned, readable up to roundup(n_cand, 4): the
//          order-preserving keys of candidates n_bos.. (in page order), each
//          counted by select_count; keys and counts visible to every thread
//   S      select_init()ed
// With max_levels > 0 the selection stops after that many histogram levels
// (the lossy radix top-k with early termination of the Vortex article,
// section "A dual-stage programmable abstraction"): when the boundary bin of
// the last level is not taken whole, its members are taken by rank in page
// order, cyclically from rank rnd mod (members), instead of by key.  This
// early stop applies when the keys are held in registers (n_cand <= NT *
// 4 * kSelRegChunks); larger inputs are selected exactly.
template <int NT>
__device__ __forceinline__ int select_pages(const uint32_t* keys, int n_cand, int n_b, int topk,
                                            int n_bos, int n_eos, int k_tot, int32_t* out,
                                            int32_t* lds_out, SelectLds<NT>& S, int max_levels = 0,
                                            uint32_t rnd = 0u) {
  const int tid = threadIdx.x;
  // Thread tid owns candidates [c0, c0 + 4 nch), nch a power of two, as nch
  // 16-byte chunks of keys.  Lanes 4a .. 4a+3 take their chunks starting at
  // chunk a mod nch, so that a wave's 16-byte reads spread over all LDS
  // banks.  Up to kSelRegChunks chunks are read once into registers and
  // serve every refinement pass and the compaction.
  int nch = 1;
  while (4 * nch * NT < n_cand) nch <<= 1;
  const int c0 = tid * 4 * nch;
  const int rot = ((tid & 63) >> 2) & (nch - 1);
  const bool in_regs = nch <= kSelRegChunks;
  uint4 kr[kSelRegChunks];
#pragma unroll
  for (int jj = 0; jj < kSelRegChunks; ++jj) kr[jj] = make_uint4(0u, 0u, 0u, 0u);
  auto reg_chunk = [&](int jj) { return c0 + 4 * ((jj + rot) & (nch - 1)); };

  // candidate c is taken iff keys[c] > thr_key || (keys[c] == thr_key && c <= thr_idx)
  uint32_t thr_key = 0u;
  int thr_idx = INT_MAX;                                  // all candidates
  // early stop: keys in [bin_lo, bin_hi] are taken by rank instead
  bool early = false;
  uint32_t bin_lo = 0u, bin_hi = 0u;
  int bin_take = 0, bin_n = 0, bin_r0 = 0;
  if (n_cand > topk && topk == 0) {
    thr_key = 0xFFFFFFFFu;                                // none of them
    thr_idx = -1;
  } else if (n_cand > topk) {
    __syncthreads();                   // keys and level-0 counts complete
    if (in_regs) {
#pragma unroll
      for (int jj = 0; jj < kSelRegChunks; ++jj) {
        const int c = reg_chunk(jj);
        if (jj < nch && c < n_cand) kr[jj] = *reinterpret_cast<const uint4*>(keys + c);
      }
    }
    int remaining = topk;              // still to take from keys in [lo, lo + span]
    uint32_t lo = 0u, span = 0xFFFFFFFFu;
    int shift = kSelShift0;
    for (int level = 0;; ++level) {
      int* H = S.hist[level & 1];
      if (level > 0) {
        if (level > 1) {               // this buffer held level - 2
          for (int i = tid; i < kSelHistWords; i += NT) H[i] = 0;
          __syncthreads();
        }
        auto count = [&](uint32_t k, int c) {
          if (c < n_cand && k - lo <= span) atomicAdd(&H[sel_slot((int)((k - lo) >> shift))], 1);
        };
        if (in_regs) {
#pragma unroll
          for (int jj = 0; jj < kSelRegChunks; ++jj) {
            if (jj < nch) {
              const int c = reg_chunk(jj);
              count(kr[jj].x, c);
              count(kr[jj].y, c + 1);
              count(kr[jj].z, c + 2);
              count(kr[jj].w, c + 3);
            }
          }
        } else {
          for (int i0 = tid; i0 < n_cand; i0 += 4 * NT) {
            uint32_t k[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) k[j] = keys[min(i0 + j * NT, n_cand - 1)];
#pragma unroll
            for (int j = 0; j < 4; ++j) count(k[j], i0 + j * NT);
          }
        }
        __syncthreads();
      }
      int dsel, above, cnt;
      find_bin(H, remaining, dsel, above, cnt);
      remaining -= above;
      lo += (uint32_t)dsel << shift;
      span = min(span - ((uint32_t)dsel << shift), (1u << shift) - 1u);
      if (remaining == cnt) {          // the whole bin is taken
        thr_key = lo;
        break;
      }
      if (max_levels > 0 && level + 1 >= max_levels && in_regs) {
        early = true;                  // keys above the bin, then members by rank
        bin_lo = lo;
        bin_hi = lo + span;
        bin_take = remaining;
        bin_n = cnt;
        bin_r0 = (int)(rnd % (uint32_t)cnt);
        if (bin_hi == 0xFFFFFFFFu) {   // no key lies above the bin
          thr_key = 0xFFFFFFFFu;
          thr_idx = -1;
        } else {                       // every key above the bin
          thr_key = bin_hi + 1u;
          thr_idx = INT_MAX;
        }
        break;
      }
      if (span == 0) {                 // cnt equal keys: the remaining-th in page order
        const int per = (n_cand + NT - 1) / NT;
        const int e0 = min(tid * per, n_cand), e1 = min(e0 + per, n_cand);
        int n_eq = 0;
        for (int i = e0; i < e1; ++i) n_eq += keys[i] == lo ? 1 : 0;
        int dummy;
        int r = block_exclusive_scan<NT>(n_eq, S.wsum[0], &dummy);
        if (r < remaining && r + n_eq >= remaining) {
          for (int i = e0; i < e1; ++i)
            if (keys[i] == lo && ++r == remaining) S.misc[0] = i;
        }
        __syncthreads();
        thr_key = lo;
        thr_idx = S.misc[0];
        break;
      }
      const int nb = 32 - __builtin_clz(span);
      shift = nb > kSelBits ? nb - kSelBits : 0;
    }
  }

  // Compaction in page order: reserved first pages, taken candidates, reserved
  // last pages.  Each thread's taken candidates become a bit mask (runs of
  // up to 64 candidates when the keys are not in registers: those runs are
  // read again to write them), then one block-wide scan places them.
  auto taken = [&](uint32_t k, int c) {
    return c < n_cand && (k > thr_key || (k == thr_key && c <= thr_idx));
  };
  const int per = 4 * nch;
  const int run = min(nch, 16);                 // chunks per run
  auto take_mask = [&](int s0) -> unsigned long long {   // from LDS: candidates c0 + s0 .. + 4 run
    const int rr = ((tid & 63) >> 2) & (run - 1);
    unsigned long long m = 0ull;
    for (int jj = 0; jj < run; ++jj) {
      const int j = (jj + rr) & (run - 1);
      const int c = c0 + s0 + 4 * j;
      if (c < n_cand) {
        const uint4 kv = *reinterpret_cast<const uint4*>(keys + c);
        m |= (unsigned long long)(taken(kv.x, c) | taken(kv.y, c + 1) << 1 |
                                  taken(kv.z, c + 2) << 2 | taken(kv.w, c + 3) << 3) << (4 * j);
      }
    }
    return m;
  };
  unsigned long long m0 = 0ull;
  int n_take = 0;
  if (in_regs) {
    unsigned long long mem = 0ull;      // early stop: members of the boundary bin
#pragma unroll
    for (int jj = 0; jj < kSelRegChunks; ++jj) {
      if (jj < nch) {
        const int c = reg_chunk(jj);
        const unsigned t = taken(kr[jj].x, c) | taken(kr[jj].y, c + 1) << 1 |
                           taken(kr[jj].z, c + 2) << 2 | taken(kr[jj].w, c + 3) << 3;
        m0 |= (unsigned long long)t << (c - c0);
        if (early) {
          auto in_bin = [&](uint32_t k, int cc) { return cc < n_cand && k >= bin_lo && k <= bin_hi; };
          const unsigned u = in_bin(kr[jj].x, c) | in_bin(kr[jj].y, c + 1) << 1 |
                             in_bin(kr[jj].z, c + 2) << 2 | in_bin(kr[jj].w, c + 3) << 3;
          mem |= (unsigned long long)u << (c - c0);
        }
      }
    }
    if (early) {
      // member of page-order rank rho is taken iff (rho - r0) mod n < take
      int mtot;
      int rho = block_exclusive_scan<NT>(__popcll(mem), S.wsum[0], &mtot);
      while (mem) {
        const int e = __builtin_ctzll(mem);
        if ((rho - bin_r0 + bin_n) % bin_n < bin_take) m0 |= 1ull << e;
        ++rho;
        mem &= mem - 1;
      }
    }
    n_take = __popcll(m0);
  } else {
    for (int s0 = 0; s0 < per && c0 + s0 < n_cand; s0 += 4 * run) {
      const unsigned long long m = take_mask(s0);
      if (s0 == 0) m0 = m;
      n_take += __popcll(m);
    }
  }
  int taken_all;
  int pos = block_exclusive_scan<NT>(n_take, S.wsum[1], &taken_all);
  const int n_lo = n_cand > 0 ? n_bos : n_b;           // no candidates: every page is reserved
  const int n_hi = n_cand > 0 ? n_eos : 0;
  const int total = n_lo + taken_all + n_hi;
  int32_t* dst = lds_out ? lds_out : out;
  pos += n_lo;
  for (int s0 = 0; s0 < per && c0 + s0 < n_cand; s0 += 4 * run) {
    unsigned long long m = s0 == 0 ? m0 : take_mask(s0);
    while (m) {
      dst[pos++] = n_bos + c0 + s0 + __builtin_ctzll(m);
      m &= m - 1;
    }
  }
  for (int i = tid; i < n_lo; i += NT) dst[i] = i;
  for (int i = tid; i < n_hi; i += NT) dst[n_lo + taken_all + i] = n_b - n_eos + i;
  if (!lds_out)
    for (int i = total + tid; i < k_tot; i += NT) out[i] = -1;
  return total;
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
// order-preserving keys, each counted into the selection's level-0
// histogram; phys[c] is candidate c's physical page.  Rows are one head's
// centroid row (<= 64 lanes of 16 bytes).  A wave takes batches of U
// wave-loads: each lane group reads U consecutive candidates' page ids from
// LDS at once, then issues all of its row loads (past the last candidate the
// index is clamped to it, so every load is unconditional and the rows are
// consumed as they arrive).  Waves start on batches 0 .. NW-1 and then take
// the next untaken batch, so that a wave whose loads return late does not
// hold up the end of the scoring (keys and counts do not depend on which
// wave computes them).  An 8-wave block has its CU alone and keeps 16
// loads per wave in flight.  Blocks of fewer waves share a CU with a block
// whose attention is a latency-bound chain of loads, and deeper queues slow
// that chain more than they speed the scoring: they keep 6.
constexpr int kScoreLoads = 16;
constexpr int kScoreLoadsShared = 6;

// BOUNDS: the summary is two rows per (page, head) [P, H_kv, 2, D] (the
// per-channel key minimum, then maximum) and the score is Quest's
// criticality sum_e max(q_e * min_e, q_e * max_e); both rows of a candidate
// are loaded together.
template <typename T, int D, int NT, bool BOUNDS = false>
__device__ __forceinline__ void score_head(const ScoreArgs& a, int h, int n_cand,
                                           const int32_t* phys, const float* qbar,
                                           uint32_t* keys, SelectLds<NT>& S) {
  using V = Vec16<T>;
  constexpr int E = V::E;
  constexpr int LH = D / E;                  // lanes per centroid row
  constexpr int R = 64 / LH;                 // rows per wave-load
  constexpr int NW = NT / 64;
  constexpr int U = NW >= 8 ? kScoreLoads : kScoreLoadsShared;
  constexpr int ROWS = R * U;                // rows per wave batch
  static_assert(LH * R == 64, "rows of at most 64 lanes");
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seg = lane % LH, grp = lane / LH;
  float qr[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qr[e] = qbar[seg * E + e];
  constexpr int RS = BOUNDS ? 2 : 1;         // summary rows per (page, head)
  const T* cent = reinterpret_cast<const T*>(a.cent) + (size_t)h * RS * D + seg * E;
  const size_t pstride = (size_t)a.H_kv * RS * D;
  const int last = n_cand - 1;
  for (int bi = w;;) {                       // batch bi: candidates [bi * ROWS, +ROWS)
    const int r0 = bi * ROWS;
    if (r0 >= n_cand) break;
    int next = 0;                            // the wave's next batch, taken from a counter
    if (lane == 0) next = atomicAdd(&S.misc[2], 1);
    const int c0 = r0 + grp * U;             // this lane group's first candidate
    int ph[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ph[u] = phys[min(c0 + u, last)];
    uint4 buf[U], hib[BOUNDS ? U : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      buf[u] = ld16(cent + (size_t)ph[u] * pstride);
      if constexpr (BOUNDS) hib[u] = ld16(cent + (size_t)ph[u] * pstride + D);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      float f[E];
      V::unpack(buf[u], f);
      float acc = 0.f;
      if constexpr (BOUNDS) {
        float fh[E];
        V::unpack(hib[u], fh);
#pragma unroll
        for (int e = 0; e < E; ++e) acc += fmaxf(qr[e] * f[e], qr[e] * fh[e]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf(qr[e], f[e], acc);
      }
      acc = lane_group_sum<LH>(acc);
      if (c < n_cand && seg == 0) {
        const uint32_t k = order_key(acc);
        keys[c] = k;
        select_count<NT>(S, k);
      }
    }
    bi = NW + __builtin_amdgcn_readfirstlane(next);
  }
}

}  // namespace vx
