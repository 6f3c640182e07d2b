// K4 (MFMA): split-K paged decode for MLA-shaped attention: up to 32 query
// heads on one latent KV head, 576-dim keys (512 latent + 64 rotary) and
// values that are the first 512 dims of the same rows, 64-token pages.  The
// "rope-aware block-sparse attention for MLA" of the Vortex announcement
// (digg thread, post [4/6]) selects pages on the full 576-dim key and attends
// exactly over them; this kernel is the attention half.
//
// At ~60 flop per byte of KV this is past the fp32 VALU roofline, so both
// products run on gfx950 matrix cores (fp32 accumulation).  One 256-thread
// block per (split, request); 32-token tiles (36 KiB) staged HBM -> registers
// -> LDS, two tile buffers, the next tile's global loads in flight while the
// current one is computed; per tile, two barriers:
//   - S^T[32 tokens x 32 heads] = K Q^T in four quarters, one per wave: wave
//     w takes tokens 16(w & 1) .. +15 and heads 16(w >> 1) .. +15 over all
//     576 dims on mfma_f32_16x16x32_bf16 (18 k-steps), its query slice held in
//     registers, so no partial scores are exchanged;
//   - each wave forms the softmax weights of its quarter against the heads'
//     current reference maxima and writes them to LDS as bf16, with its per-
//     head maximum and weight sum; after the barrier every wave sees the
//     tile's maxima.  Only when a head's maximum passes its reference by
//     more than kLazyRescale (always on the first tile) are the references
//     raised, the weights recomputed and the running output rescaled (one
//     more barrier);
//   - O^T[dims x heads] += V^T P^T on mfma_f32_32x32x16_bf16: wave w owns V
//     dims 128w .. 128w+127 (4 tiles of 32); P^T is read from LDS already in
//     the B operand's token order; V^T is read from the K tile in LDS (so HBM
//     sees each 576-dim row once) with the transposing 64-bit LDS read.
//
// Given the split scorer's scores instead of a selection (the decode step),
// every split block first selects its request's pages itself, with the exact
// selection of the indexer kernels, in LDS that the tile buffers take over
// afterwards; split 0 writes the selection row.
#include "vx_device.h"
#include "vx_internal.h"
#include "vx_select.h"

namespace vx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDqk = 576, kDv = 512, kHeads = 32;
constexpr int kPage = 64;                    // tokens per page
constexpr int kT = 32;                       // tokens per tile
constexpr int kRowB = kDqk * 2;              // 1152 bytes per token row
constexpr int kLdsRow = kRowB + 16;          // padded LDS row stride (4 banks of shift per row)
constexpr int kTileB = kT * kLdsRow;         // one tile buffer
constexpr int kThreads = 256;
constexpr int kChunksPerRow = kRowB / 16;    // 72
constexpr int kLoads = kT * kChunksPerRow / kThreads;   // 9 x 16 B per thread per tile
constexpr int kKS = kDqk / 32;               // 18 k-steps of 32 dims (16x16x32 products)
constexpr int kPRow = 2 * kT + 16;           // bytes per head in the weight buffer (+ pad)
constexpr int kMaxPages = 128;               // pages per split (planner bound)
static_assert(kT * kChunksPerRow == kLoads * kThreads, "tile copy");
static_assert(kKS * 32 == kDqk, "k steps");

__device__ __forceinline__ float neg_inf() { return -INFINITY; }

// Selection scratch inside the tile buffer: keys [round4(n)], list [k_tot],
// then the histograms.
__host__ __device__ constexpr size_t mla_select_offset(int score_stride, int k_tot) {
  return (((size_t)round4(score_stride) + (size_t)k_tot) * 4 + 15) / 16 * 16;
}

template <bool SELECT>
__global__ __launch_bounds__(kThreads, 2) void decode_mla_kernel(DecodeArgs a) {
  __shared__ __align__(16) uint8_t ktile[2 * kTileB];
  __shared__ __align__(16) uint8_t pbuf[kHeads * kPRow];   // bf16 weights, B operand order
  __shared__ float smax[2][kHeads], ssum[2][kHeads];        // per token half and head
  __shared__ int page_phys[kMaxPages];
  __shared__ int page_logi[kMaxPages];
  __shared__ int s_count;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int hl = l & 31, hh = l >> 5;          // head (column) and k half of the 32x32 layouts
  const int th = w & 1, hq = w >> 1;           // this wave's token half and head half of S
  const int lr = l & 15, lg = l >> 4;          // 16x16 layouts: column and lane group
  const int split = blockIdx.x, b = blockIdx.y;
  const int G = a.H_q;                          // H_kv == 1

  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + kPage - 1) / kPage;
  const int32_t* selrow = a.sel ? a.sel + (size_t)b * a.k_tot : nullptr;
  if constexpr (SELECT) {
    // the request's pages from the indexer's scores (H_kv == 1)
    uint32_t* keys = reinterpret_cast<uint32_t*>(ktile);
    int32_t* list = reinterpret_cast<int32_t*>(keys + round4(a.score_stride));
    SelectLds<kThreads>& sl =
        *reinterpret_cast<SelectLds<kThreads>*>(ktile + mla_select_offset(a.score_stride, a.k_tot));
    const int n_cand = max(n_b - a.n_bos - a.n_eos, 0);
    select_init<kThreads>(sl);
    __syncthreads();
    if (n_cand > a.topk && a.topk > 0) {
      const float* sc = a.scores + (size_t)b * a.score_stride;
      constexpr int kIn = 8;
      for (int i0 = tid; i0 < n_cand; i0 += kIn * kThreads) {
        float v[kIn];
#pragma unroll
        for (int j = 0; j < kIn; ++j) v[j] = sc[min(i0 + j * kThreads, n_cand - 1)];
#pragma unroll
        for (int j = 0; j < kIn; ++j) {
          const int i = i0 + j * kThreads;
          if (i < n_cand) {
            const uint32_t k = order_key(v[j]);
            keys[i] = k;
            select_count<kThreads>(sl, k);
          }
        }
      }
    }
    const int count = select_pages<kThreads>(keys, n_cand, n_b, a.topk, a.n_bos, a.n_eos,
                                             a.k_tot, nullptr, list, sl);
    __syncthreads();
    if (split == 0) {
      int32_t* srow = a.sel_out + (size_t)b * a.k_tot;
      for (int i = tid; i < a.k_tot; i += kThreads) srow[i] = i < count ? list[i] : -1;
    }
    const int p0 = split * a.pages_per_split;
    const int p1 = min(p0 + a.pages_per_split, count);
    const int np = max(p1 - p0, 0);
    const int32_t* ptb = a.pt + (size_t)b * a.pt_stride;
    for (int i = tid; i < np; i += kThreads) {
      const int logi = list[p0 + i];
      page_logi[i] = logi;
      page_phys[i] = ptb[logi];
    }
    if (tid == 0) s_count = count;
  } else if (w == 0) {
    int count = n_b;
    if (selrow) {
      count = a.k_tot;
      for (int base = 0; base < a.k_tot; base += 64) {
        const int i = base + l;
        const int p = i < a.k_tot ? selrow[i] : 0;
        const unsigned long long bad = __ballot(i < a.k_tot && (p < 0 || p >= n_b));
        if (bad) { count = base + __builtin_ctzll(bad); break; }
      }
    }
    if (l == 0) s_count = count;
  }
  __syncthreads();
  const int count = s_count;
  const int p0 = split * a.pages_per_split;
  const int p1 = min(p0 + a.pages_per_split, count);
  const int np = max(p1 - p0, 0);
  if constexpr (!SELECT) {
    const int32_t* ptb = a.pt + (size_t)b * a.pt_stride;
    for (int i = tid; i < np; i += kThreads) {
      const int logi = selrow ? selrow[p0 + i] : p0 + i;
      page_logi[i] = logi;
      page_phys[i] = ptb[logi];
    }
  }

  // query slice as the B operand of S^T = K Q^T: head 16hq + lr, dims 32ks + 8lg ..
  bf16x8 qB[kKS];
  {
    const int head = 16 * hq + lr;
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) + ((size_t)b * a.H_q + head) * kDqk;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const uint4 v = head < G ? ld16(qp + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
      qB[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // o[dt][i] = O[head hl][dim 128w + 32dt + 8(i/4) + 4hh + i%4]
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  // reference maxima (log2 units) of head 16hq + lr (the S layout) and of
  // head hl (the O layout); the same values for the same head in every wave
  float m_s = neg_inf(), m_o = neg_inf();
  float lsum = 0.f;                              // of head hl

  __syncthreads();                               // page lists visible

  const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(a.k);
  const int n_tiles = np * (kPage / kT);
  uint4 regs[kLoads];
  auto load_tile = [&](int t) {
    const int j = t / (kPage / kT), half = t % (kPage / kT);
    const uint8_t* src = kbytes + ((size_t)page_phys[j] * kPage + half * kT) * kRowB;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) regs[r] = ld16(src + (size_t)(tid + r * kThreads) * 16);
  };
  if (n_tiles > 0) load_tile(0);

  // this lane's row / column in the transposing V reads: group g = l / 16 covers
  // dims 16(g % 2) .. of a 32-dim tile and the token half hh; lane 16g + 4j + c
  // supplies row 4hh + j (+8, +16 s) at dims 4c .. 4c+3
  const int tr_row = 4 * hh + ((l & 15) >> 2);
  const int tr_col = 16 * ((l >> 4) & 1) + 4 * (l & 3);
  // the weights this lane writes: S-layout head 16hq + lr, tokens 16th + 4lg ..
  // +3, at their place in the B operand's token order (within a 16-token slice,
  // k-half kh holds tokens 8(j/4) + 4kh + j%4, j = 0..7)
  uint8_t* pw = pbuf + (16 * hq + lr) * kPRow + 2 * (16 * th + 8 * (lg & 1) + 4 * (lg >> 1));

  for (int t = 0; t < n_tiles; ++t) {
    uint8_t* kt = ktile + (t & 1) * kTileB;
    // tile t into buffer t % 2: buffer (t - 1) % 2 may still be read (V of the
    // previous tile), this one was last read two tiles ago, before the
    // previous tile's second barrier
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + r * kThreads;
      const int row = c / kChunksPerRow, col = c - row * kChunksPerRow;
      st16(kt + row * kLdsRow + col * 16, regs[r]);
    }
    const int j = t / (kPage / kT), half = t % (kPage / kT);
    const int tok0 = page_logi[j] * kPage + half * kT;
    const bool tail = tok0 + kT > seq;
    if (tail) {
      // Rows at or past seq (the unwritten tail of the last page): their
      // scores are masked, but as V rows 0 * NaN would still reach O, so
      // each thread overwrites its own chunks of them with zeros (program
      // order within the thread makes the zeros win).
#pragma unroll
      for (int r = 0; r < kLoads; ++r) {
        const int c = tid + r * kThreads;
        const int row = c / kChunksPerRow, col = c - row * kChunksPerRow;
        if (tok0 + row >= seq) st16(kt + row * kLdsRow + col * 16, make_uint4(0u, 0u, 0u, 0u));
      }
    }
    __syncthreads();                             // (1) tile staged
    if (t + 1 < n_tiles) load_tile(t + 1);

    // ---- this wave's quarter of S^T: tokens 16th + 4lg + i, head 16hq + lr
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* krow = kt + (16 * th + lr) * kLdsRow + 16 * lg;
#pragma unroll
      for (int ks = 0; ks < kKS; ks += 2) {
        const bf16x8 k0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + 64 * ks));
        const bf16x8 k1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + 64 * ks + 64));
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qB[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qB[ks + 1], s1, 0, 0, 0);
      }
    }
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = s0[i] + s1[i];
    if (tail) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tok0 + 16 * th + 4 * lg + i >= seq) sv[i] = neg_inf();
    }
    // the quarter's maximum per head (16 tokens: 4 in the lane, 4 lane groups)
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    {
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                        false, false);
      mx = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                        false, false);
      mx = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    }
    mx *= a.scale_log2;          // the scale is positive: the maximum of the scaled scores
    // weights against the current reference (replaced below if it must grow)
    auto weights = [&](float ref) {
      const float neg_m = (ref == neg_inf()) ? 0.f : -ref;
      float ps = 0.f;
      s16x4 pv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(fmaf(sv[i], a.scale_log2, neg_m));
        ps += p;
        pv[i] = (short)f32_to_bf16(p);
      }
      *reinterpret_cast<s16x4*>(pw) = pv;
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ps), __float_as_uint(ps),
                                                        false, false);
      ps = __uint_as_float(x16[0]) + __uint_as_float(x16[1]);
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps),
                                                        false, false);
      ps = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);
      if (lg == 0) ssum[th][16 * hq + lr] = ps;
    };
    weights(m_s);
    if (lg == 0) smax[th][16 * hq + lr] = mx;
    __syncthreads();                             // (2) weights, maxima and sums of all quarters
    // the tile's maximum per head, in both layouts
    const float tmax_o = fmaxf(smax[0][hl], smax[1][hl]);
    const bool grow = __ballot(tmax_o > m_o + kLazyRescale) != 0ull;
    float alpha = 1.f;
    if (grow) {                                  // the same decision in every wave
      const float tmax_s = fmaxf(smax[0][16 * hq + lr], smax[1][16 * hq + lr]);
      const float mo_new = fmaxf(m_o, tmax_o);
      alpha = (mo_new == neg_inf()) ? 1.f : fast_exp2(m_o - mo_new);
      m_o = mo_new;
      m_s = fmaxf(m_s, tmax_s);
      weights(m_s);                              // nobody reads weights or sums before (2')
      __syncthreads();                           // (2') weights against the new references
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    }
    lsum = lsum * alpha + (ssum[0][hl] + ssum[1][hl]);

    // ---- O^T += V^T P^T over the tile's two 16-token slices
    s16x8 pk[2];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
      pk[sl] = *reinterpret_cast<const s16x8*>(pbuf + hl * kPRow + 2 * (16 * sl + 8 * hh));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x16 acc = o[dt];
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const uint8_t* vsrc = kt + (16 * sl + tr_row) * kLdsRow + 2 * (128 * w + 32 * dt + tr_col);
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vsrc));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vsrc + 8 * kLdsRow));
        const s16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv),
                                                      __builtin_bit_cast(bf16x8, pk[sl]), acc, 0, 0, 0);
      }
      o[dt] = acc;
    }
  }
  const float m = m_o;

  // ---- write: o[dt][i] is O[head hl][dim 128w + 32dt + 8(i/4) + 4hh + i%4]
  if (hl >= G) return;
  const size_t row = (size_t)b * a.H_q + hl;
  const bool direct = a.n_split == 1;
  if (direct) {
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    bf16_t* op = reinterpret_cast<bf16_t*>(a.out) + row * kDv;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        op[128 * w + 32 * dt + 8 * (i >> 2) + 4 * hh + (i & 3)] = f32_to_bf16(o[dt][i] * inv);
    if (w == 0 && hh == 0 && a.lse) a.lse[row] = lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : neg_inf();
  } else {
    const size_t prow = row * a.n_split + split;
    float* po = a.part_o + prow * kDv;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) po[128 * w + 32 * dt + 8 * (i >> 2) + 4 * hh + (i & 3)] = o[dt][i];
    if (w == 0 && hh == 0) {
      a.part_ml[prow * 2] = m;
      a.part_ml[prow * 2 + 1] = lsum;
    }
  }
}

}  // namespace

int mla_max_pages_per_split() { return kMaxPages; }

bool mla_select_fits(int score_stride, int k_tot) {
  return mla_select_offset(score_stride, k_tot) + sizeof(SelectLds<kThreads>) <= sizeof(uint8_t) *
                                                                                    kT * kLdsRow;
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t s) {
  if (a.pages_per_split > kMaxPages || a.S_p != kPage || a.H_kv != 1 || a.H_q > kHeads)
    return hipErrorInvalidValue;
  if (a.scores) {
    if (!mla_select_fits(a.score_stride, a.k_tot) || !a.sel_out) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_mla_kernel<true>), dim3(a.n_split, a.B), dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_mla_kernel<false>), dim3(a.n_split, a.B), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace vx
