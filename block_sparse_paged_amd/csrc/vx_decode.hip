// K4 + K5: split-K paged decode attention over a list of logical
// pages (the selected ones, or every page for the dense baseline).  The
// attention itself is the exact softmax attention the method runs after page
// selection (Vortex article, "A dual-stage programmable abstraction"); the
// split into page ranges with fp32 partials merged afterwards is this
// library's scheduling, not something the pages prescribe.
//
// K4: one block of 8 waves per (split, KV head, request) runs attend_pages()
// over its range of the page list.  A selection row of up to 64 pages is read
// once, one entry per lane, and its page ids are shuffled to the waves that
// need them; longer lists are read from memory per page.  In the fused form
// (indexer scores given) every split block selects its (request, KV head)'s
// pages from the scores itself, with the exact selection of the indexer
// kernels, instead of a separate top-k launch; split 0 writes the selection
// row.  The block writes the output directly when the plan has a single
// split, else fp32 partials.
// K5: merges the partials of each (request, query head).
#include "vx_attend.h"
#include "vx_select.h"

namespace vx {
namespace {

template <typename T, int D, int G, int HS, int PF, bool SELECT>
__global__ __launch_bounds__(kNW * 64) void decode_split_kernel(DecodeArgs a) {
  constexpr int NT = kNW * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  // with a selection to make, the first share of the scores row goes out
  // before the request length is known (entries past the request's
  // candidates are read and ignored)
  constexpr int kIn = 16;              // score loads in flight per thread
  float v0[kIn];
  if constexpr (SELECT) {
    const float* sc = a.scores + ((size_t)b * a.H_kv + h) * a.score_stride;
#pragma unroll
    for (int j = 0; j < kIn; ++j) v0[j] = sc[min(tid + j * NT, a.score_stride - 1)];
  }
  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + a.S_p - 1) / a.S_p;
  const int32_t* ptb = a.pt + (size_t)b * a.pt_stride;

  if constexpr (SELECT) {
    // the (request, KV head)'s selection, computed by every split block
    extern __shared__ __align__(16) uint32_t dyn[];   // keys [round4(score_stride)], list [k_tot]
    __shared__ SelectLds<NT> sl;
    uint32_t* keys = dyn;
    int32_t* list = reinterpret_cast<int32_t*>(dyn + round4(a.score_stride));
    const int n_cand = max(n_b - a.n_bos - a.n_eos, 0);
    select_init<NT>(sl);
    __syncthreads();
    if (n_cand > a.topk && a.topk > 0) {
      const float* sc = a.scores + ((size_t)b * a.H_kv + h) * a.score_stride;
      for (int i0 = tid; i0 < n_cand; i0 += kIn * NT) {
        float v[kIn];
#pragma unroll
        for (int j = 0; j < kIn; ++j) v[j] = i0 == tid ? v0[j] : sc[min(i0 + j * NT, n_cand - 1)];
#pragma unroll
        for (int j = 0; j < kIn; ++j) {
          const int i = i0 + j * NT;
          if (i < n_cand) {
            const uint32_t k = order_key(v[j]);
            keys[i] = k;
            select_count<NT>(sl, k);
          }
        }
      }
    }
    const int count = select_pages<NT>(keys, n_cand, n_b, a.topk, a.n_bos, a.n_eos, a.k_tot,
                                       nullptr, list, sl);
    __syncthreads();
    const int p0 = split * a.pages_per_split;
    const int p1 = min(p0 + a.pages_per_split, count);
    auto page_at = [&](int idx, bool active) -> int2 {
      int logi = 0, phys = 0;
      if (active) {
        logi = list[idx];
        phys = ptb[logi];
      }
      return make_int2(logi, phys);
    };
    int32_t* srow = a.sel_out + ((size_t)b * a.H_kv + h) * a.k_tot;
    auto epilogue = [&](int t, int nt) {
      if (split == 0)
        for (int i = t; i < a.k_tot; i += nt) srow[i] = i < count ? list[i] : -1;
    };
    attend_pages<T, D, G, HS, PF, kNW>(a, b, h, split, p0, p1, seq, page_at, epilogue);
  } else {
    // length of this request's page list (the selection ends at its first
    // entry outside [0, n_b))
    const int32_t* selrow = nullptr;
    int count = n_b, sel_l = 0;
    const bool sel_in_regs = a.sel && a.k_tot <= 64;
    if (a.sel) {
      selrow = a.sel + ((size_t)b * a.H_kv + h) * a.k_tot;
      count = a.k_tot;
      for (int base = 0; base < a.k_tot; base += 64) {
        const int i = base + lane;
        const int p = i < a.k_tot ? selrow[i] : 0;
        if (base == 0) sel_l = p;
        const unsigned long long bad = __ballot(i < a.k_tot && (p < 0 || p >= n_b));
        if (bad) { count = base + __builtin_ctzll(bad); break; }
      }
    }
    const int p0 = split * a.pages_per_split;
    const int p1 = min(p0 + a.pages_per_split, count);
    auto page_at = [&](int idx, bool active) -> int2 {
      const int from_regs = __shfl(sel_l, idx & 63, 64);
      int logi = idx, phys = 0;
      if (active) {
        if (selrow) logi = sel_in_regs ? from_regs : selrow[idx];
        phys = ptb[logi];
      }
      return make_int2(logi, phys);
    };
    attend_pages<T, D, G, HS, PF, kNW>(a, b, h, split, p0, p1, seq, page_at);
  }
}

// K4, dense work list: the dense decode of a batch whose requests differ in
// length ("workload planner for balanced GPU scheduling", Vortex article,
// "A dual-stage programmable abstraction").  Every request's pages are cut
// into chunks of pages_per_split pages; an item is one (request, chunk, KV
// head), all items but each request's last of equal size.  A fixed number of
// persistent blocks take items blockIdx.x, blockIdx.x + gridDim.x, ... in
// (request, chunk, head) order, so every block streams the same number of
// bytes to within one item, whatever the length mix.  Each block first
// forms the chunk offsets of every request itself (a block scan over the
// lengths), so the launch needs no host synchronisation, no counters and no
// cleared memory.  Chunk c of a request is its split c: the partials land in
// the split-K layout and combine_kernel merges each request's own chunks.
constexpr int kItemsMaxBatch = 2048;       // LDS: chunk offsets and lengths (16 KiB)
// Waves per work-list block.  Measured against 4-wave blocks (two resident
// per CU): the 8-wave block streams as fast on uniform batches and faster on
// mixed ones.
constexpr int kItemWaves = 8;

template <typename T, int D, int G, int HS, int PF, int NW>
__global__ __launch_bounds__(NW * 64) void decode_items_kernel(DecodeArgs a) {
  constexpr int NT = NW * 64;
  extern __shared__ int sh[];                // coff [B + 1], then seq [B]
  __shared__ int wsum[NT / 64];
  int* coff = sh;
  int* sq = sh + a.B + 1;
  const int tid = threadIdx.x;
  const int C = a.pages_per_split;
  int run = 0;
  for (int base = 0; base < a.B; base += NT) {
    const int i = base + tid;
    int n = 0;
    if (i < a.B) {
      int seq = a.seq_lens[i];
      seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
      sq[i] = seq;
      const int n_b = (seq + a.S_p - 1) / a.S_p;
      n = max((n_b + C - 1) / C, 1);           // an empty request still gets its (empty) item
    }
    int tot;
    const int ex = block_exclusive_scan<NT>(n, wsum, &tot);
    if (i < a.B) coff[i] = run + ex;
    run += tot;
    __syncthreads();                          // wsum is reused by the next round
  }
  if (tid == 0) coff[a.B] = run;
  __syncthreads();
  const int total = run * a.H_kv;
  int b = 0;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int cidx = item / a.H_kv, h = item - cidx * a.H_kv;
    while (coff[b + 1] <= cidx) ++b;           // items ascend, so b only moves forward
    const int chunk = cidx - coff[b];
    const int seq = sq[b];
    const int n_b = (seq + a.S_p - 1) / a.S_p;
    const int p0 = chunk * C, p1 = min(p0 + C, n_b);
    const int32_t* ptb = a.pt + (size_t)b * a.pt_stride;
    auto page_at = [&](int idx, bool active) -> int2 {
      return make_int2(idx, active ? ptb[idx] : 0);
    };
    attend_pages<T, D, G, HS, PF, NW>(a, b, h, chunk, p0, p1, seq, page_at);
    __syncthreads();                          // the merge's LDS is free for the next item
  }
}

// Splits row (b, .) of a combine merges: all n_split, or, for the work list,
// the chunks request b has.
__device__ __forceinline__ int combine_splits(const CombineArgs& a, size_t row) {
  if (!a.seq_lens) return a.n_split;
  const int b = (int)(row / a.H_q);
  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + a.S_p - 1) / a.S_p;
  return min(max((n_b + a.pages_per_split - 1) / a.pages_per_split, 1), a.n_split);
}

// K5: merge the splits of one (request, query head).  Splits with an empty
// page range have sum 0 and are skipped.  256 threads per row; each thread
// owns D_v/256 output dims (at least one) and keeps eight splits' loads in
// flight.
constexpr int kCombineThreads = 256;

template <typename T, int DV>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  constexpr int PER = (DV + kCombineThreads - 1) / kCombineThreads;
  __shared__ float w[1024];
  __shared__ float red[kCombineThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = blockIdx.x;            // b * H_q + hq
  const int n = combine_splits(a, row);
  const float* ml = a.part_ml + row * a.n_split * 2;
  float mx = -INFINITY;
  for (int i = tid; i < n; i += kCombineThreads)
    if (ml[2 * i + 1] > 0.f) mx = fmaxf(mx, ml[2 * i]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int v = 1; v < kCombineThreads / 64; ++v) mx = fmaxf(mx, red[v]);
  __syncthreads();
  float tot = 0.f;
  for (int i = tid; i < n; i += kCombineThreads) {
    const float li = ml[2 * i + 1];
    const float wi = li > 0.f ? exp2f(ml[2 * i] - mx) : 0.f;
    w[i] = wi;
    tot += wi * li;
  }
  tot = wave_sum(tot);
  if (lane == 0) red[wave] = tot;
  __syncthreads();
  tot = 0.f;
#pragma unroll
  for (int v = 0; v < kCombineThreads / 64; ++v) tot += red[v];
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  const float* po = a.part_o + row * a.n_split * DV;
  for (int i0 = 0; i0 < n; i0 += 8) {
    float x[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int d = j * kCombineThreads + tid;
        x[u][j] = (i0 + u < n && d < DV && w[i0 + u] != 0.f)
                      ? po[(size_t)(i0 + u) * DV + d] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + u < n) {
        const float wi = w[i0 + u];
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] = fmaf(wi, x[u][j], acc[j]);
      }
    }
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  T* op = reinterpret_cast<T*>(a.out) + row * DV;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int d = j * kCombineThreads + tid;
    if (d < DV) op[d] = Vec16<T>::from_f32(acc[j] * inv);
  }
  if (tid == 0 && a.lse) a.lse[row] = tot > 0.f ? (mx + __log2f(tot)) * kLn2 : -INFINITY;
}

// K5 for few splits (the sparse paths' usual case): one wave per row, so no
// block-wide reductions.  Lane i holds split i's (m, l); every partial-o load
// is issued before the weights are known.  A split with an empty page range
// has l = 0 and weight 0, and its slots are never folded in (not even
// multiplied by zero), so whatever they hold is ignored.  The maximum, the
// weights, their sum and the accumulation order are those of combine_kernel.
constexpr int kCombineFew = 8;

template <typename T, int DV>
__global__ __launch_bounds__(64) void combine_few_kernel(CombineArgs a) {
  constexpr int PD = DV / 64;               // output dims per lane
  static_assert(PD * 64 == DV, "rows of a multiple of 64 dims");
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;            // b * H_q + hq
  const int ns = a.n_split;                 // row stride of the partials
  const int n = combine_splits(a, row);     // splits this row merges
  const float2 mli = *reinterpret_cast<const float2*>(a.part_ml + (row * ns + min(lane, n - 1)) * 2);
  const float* po = a.part_o + row * ns * DV + lane * PD;
  float x[kCombineFew][PD];
#pragma unroll
  for (int i = 0; i < kCombineFew; ++i) {
    if (i < n) {
      const float* p = po + (size_t)i * DV;
      if constexpr (PD % 4 == 0) {
#pragma unroll
        for (int j = 0; j < PD; j += 4) {
          const float4 v = *reinterpret_cast<const float4*>(p + j);
          x[i][j] = v.x; x[i][j + 1] = v.y; x[i][j + 2] = v.z; x[i][j + 3] = v.w;
        }
      } else if constexpr (PD == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p);
        x[i][0] = v.x; x[i][1] = v.y;
      } else {
        x[i][0] = p[0];
      }
    }
  }
  const bool valid = lane < n && mli.y > 0.f;
  const float mx = wave_max(valid ? mli.x : -INFINITY);
  const float wl = valid ? exp2f(mli.x - mx) : 0.f;
  const float tot = wave_sum(lane < n ? wl * mli.y : 0.f);
  float acc[PD];
#pragma unroll
  for (int j = 0; j < PD; ++j) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < kCombineFew; ++i) {
    if (i < n) {
      const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
      if (wi != 0.f) {
#pragma unroll
        for (int j = 0; j < PD; ++j) acc[j] = fmaf(wi, x[i][j], acc[j]);
      }
    }
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  T* op = reinterpret_cast<T*>(a.out) + row * DV + lane * PD;
#pragma unroll
  for (int j = 0; j < PD; ++j) op[j] = Vec16<T>::from_f32(acc[j] * inv);
  if (lane == 0 && a.lse) a.lse[row] = tot > 0.f ? (mx + __log2f(tot)) * kLn2 : -INFINITY;
}

template <typename T, int D, int G>
hipError_t run_decode(const DecodeArgs& a, hipStream_t s) {
  constexpr int HS = attend_head_slices<G>(), PF = attend_prefetch<T, D>();
  dim3 grid(a.n_split, a.H_kv, a.B);
  if (a.scores) {
    const size_t lds = ((size_t)round4(a.score_stride) + (size_t)a.k_tot) * sizeof(uint32_t);
    hipLaunchKernelGGL((decode_split_kernel<T, D, G, HS, PF, true>), grid, dim3(kNW * 64), lds, s, a);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<T, D, G, HS, PF, false>), grid, dim3(kNW * 64), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t run_items(const DecodeArgs& a, int blocks, hipStream_t s) {
  constexpr int HS = attend_head_slices<G>(), PF = attend_prefetch<T, D>();
  const size_t lds = (2 * (size_t)a.B + 1) * sizeof(int);
  hipLaunchKernelGGL((decode_items_kernel<T, D, G, HS, PF, kItemWaves>), dim3(blocks),
                     dim3(kItemWaves * 64), lds, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_items_g(int G, const DecodeArgs& a, int blocks, hipStream_t s) {
  switch (G) {
    case 1: return run_items<T, D, 1>(a, blocks, s);
    case 2: return run_items<T, D, 2>(a, blocks, s);
    case 4: return run_items<T, D, 4>(a, blocks, s);
    case 8: return run_items<T, D, 8>(a, blocks, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t run_decode_g(int G, const DecodeArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return run_decode<T, D, 1>(a, s);
    case 2: return run_decode<T, D, 2>(a, s);
    case 4: return run_decode<T, D, 4>(a, s);
    case 8: return run_decode<T, D, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int DV>
hipError_t run_combine(const CombineArgs& a, hipStream_t s) {
  if (a.n_split <= kCombineFew)
    hipLaunchKernelGGL((combine_few_kernel<T, DV>), dim3(a.B * a.H_q), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<T, DV>), dim3(a.B * a.H_q), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(int dtype, int D, int G, const DecodeArgs& a, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return run_decode_g<float, 64>(G, a, s);
    if (D == 128) return run_decode_g<float, 128>(G, a, s);
  } else {
    if (D == 64) return run_decode_g<bf16_t, 64>(G, a, s);
    if (D == 128) return run_decode_g<bf16_t, 128>(G, a, s);
  }
  return hipErrorInvalidValue;
}

int decode_items_max_batch() { return kItemsMaxBatch; }

hipError_t launch_decode_items(int dtype, int D, int G, const DecodeArgs& a, int blocks,
                               hipStream_t s) {
  if (a.B > kItemsMaxBatch || a.B < 1 || blocks < 1 || a.pages_per_split < 1 || a.sel ||
      a.scores)
    return hipErrorInvalidValue;
  if (dtype == 0) {
    if (D == 64) return run_items_g<float, 64>(G, a, blocks, s);
    if (D == 128) return run_items_g<float, 128>(G, a, blocks, s);
  } else {
    if (D == 64) return run_items_g<bf16_t, 64>(G, a, blocks, s);
    if (D == 128) return run_items_g<bf16_t, 128>(G, a, blocks, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(int dtype, const CombineArgs& a, hipStream_t s) {
  if (a.n_split > 1024) return hipErrorInvalidValue;
  if (dtype == 0) {
    if (a.D_v == 64) return run_combine<float, 64>(a, s);
    if (a.D_v == 128) return run_combine<float, 128>(a, s);
  } else {
    if (a.D_v == 64) return run_combine<bf16_t, 64>(a, s);
    if (a.D_v == 128) return run_combine<bf16_t, 128>(a, s);
    if (a.D_v == 512) return run_combine<bf16_t, 512>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vx
