// Exact softmax attention of one (request, KV head)'s query group over a list
// of logical pages, computed by one block of 8 waves (VALU path, D_qk = D_v =
// D).  Shared by the split-K decode kernel and the fused decode step.
//
// Lanes hold 16-byte segments of a token row: L = D*e/16 lanes per row,
// R = 64/L rows (tokens) per wave-load, so one wave-load reads 1 KiB of a
// page-head tile contiguously.  Each lane group of L lanes runs its own online
// softmax over the tokens it holds (per-token dot products reduced with DPP
// row moves), so nothing crosses lane groups inside the loop.  Waves take the
// list's pages round-robin with PF 16-token chunks of K and V in flight; with
// G = 8 the two halves of the query group go to different waves over the same
// pages (register pressure).  Lane groups merge with shuffles, waves through
// LDS; the block then writes the normalised output and lse, or fp32 partials
// (unnormalised sum, max in log2 units, denominator) for a later merge.
#pragma once

#include "vx_device.h"
#include "vx_internal.h"

namespace vx {

constexpr int kChunk = 16;   // tokens per softmax update
constexpr int kNW = 8;       // waves per attention block of the split-K decode

// page_at(idx) returns {logical page, physical page} of list entry idx; it is
// called by every lane (inactive lanes pass active = false and get ignored).
// NW is the block's wave count.
template <typename T, int D, int G, int HS, int PF, int NW, class PageAt, class Epi>
__device__ __forceinline__ void attend_pages_valu(const DecodeArgs& a, int b, int h, int split,
                                                  int p0, int p1, int seq, PageAt page_at,
                                                  Epi epi) {
  using V = Vec16<T>;
  constexpr int E = V::E;
  constexpr int L = D / E;          // lanes per token row
  constexpr int R = 64 / L;         // token rows per wave-load
  constexpr int NL = kChunk / R;    // wave-loads per chunk (K and V each)
  constexpr int HG = G / HS;        // query heads per wave
  constexpr int NWP = NW / HS;      // waves working on different pages
  static_assert(L * R == 64 && NL * R == kChunk && HG * HS == G, "layout");

  __shared__ float s_m[NW][HG], s_l[NW][HG];
  __shared__ float s_o[NW][HG][D];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int seg = lane % L, grp = lane / L;
  const int hs = w % HS, wp = w / HS;
  const int SP = a.S_p;
  const int hq0 = h * G + hs * HG;

  float q[HG][E];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.H_q + hq0) * D + seg * E;
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      V::unpack(ld16(qp + (size_t)g * D), q[g]);
#pragma unroll
      for (int e = 0; e < E; ++e) q[g][e] *= a.scale_log2;
    }
  }

  float o[HG][E], l[HG], m[HG];
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    l[g] = 0.f;
    m[g] = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.f;
  }

  const T* kbase = reinterpret_cast<const T*>(a.k);
  const T* vbase = reinterpret_cast<const T*>(a.v);
  const size_t tile_k = (size_t)SP * D;
  const size_t vtok = (size_t)a.v_stride_tok;
  const size_t tile_v = (size_t)SP * vtok;
  const int cpp = SP / kChunk;
  const int my_n = p1 > p0 + wp ? (p1 - p0 - wp + NWP - 1) / NWP : 0;

  for (int base = 0; base < my_n; base += 64) {
    const int nb = min(64, my_n - base);
    const int idx = p0 + wp + NWP * (base + lane);
    const int2 lp = page_at(idx, lane < nb);
    const int logi_l = lane < nb ? lp.x : 0, phys_l = lane < nb ? lp.y : 0;
    const int nch = nb * cpp;
    uint4 kb[PF][NL], vb[PF][NL];
    auto issue = [&](int c, uint4* kd, uint4* vd) {
      const int j = c / cpp, ch = c - j * cpp;
      const int phys = __builtin_amdgcn_readlane(phys_l, j);
      const T* kp = kbase + ((size_t)phys * a.H_kv + h) * tile_k + (size_t)(ch * kChunk) * D;
      const T* vp = vbase + ((size_t)phys * a.H_kv + h) * tile_v + (size_t)(ch * kChunk) * vtok;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int t = i * R + grp;
        kd[i] = ld16(kp + (size_t)t * D + seg * E);
        vd[i] = ld16(vp + (size_t)t * vtok + seg * E);
      }
    };
    auto process = [&](int c, const uint4* kd, const uint4* vd) {
      const int j = c / cpp, ch = c - j * cpp;
      const int logi = __builtin_amdgcn_readlane(logi_l, j);
      const int tok0 = logi * SP + ch * kChunk;
      float s[HG][NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float kf[E];
        V::unpack(kd[i], kf);
        const bool valid = tok0 + i * R + grp < seq;
#pragma unroll
        for (int g = 0; g < HG; ++g) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) acc = fmaf(q[g][e], kf[e], acc);
          acc = lane_group_sum<L>(acc);
          s[g][i] = valid ? acc : -INFINITY;
        }
      }
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        float mc = s[g][0];
#pragma unroll
        for (int i = 1; i < NL; ++i) mc = fmaxf(mc, s[g][i]);
        const float mn = fmaxf(m[g], mc);
        const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m[g] - mn);
        m[g] = mn;
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) o[g][e] *= alpha;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const float p = (mn == -INFINITY) ? 0.f : fast_exp2(s[g][i] - mn);
          s[g][i] = p;
          l[g] += p;
        }
      }
      if (tok0 + kChunk <= seq) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float vf[E];
          V::unpack(vd[i], vf);
#pragma unroll
          for (int g = 0; g < HG; ++g)
#pragma unroll
            for (int e = 0; e < E; ++e) o[g][e] = fmaf(s[g][i], vf[e], o[g][e]);
        }
      } else {
        // The chunk reaches past seq (the unwritten tail of the last page;
        // the same in every lane): those rows have weight 0, but 0 * NaN or
        // 0 * Inf would still reach the sum, so their values count as 0.
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const bool valid = tok0 + i * R + grp < seq;
          float vf[E];
          V::unpack(vd[i], vf);
#pragma unroll
          for (int e = 0; e < E; ++e) vf[e] = valid ? vf[e] : 0.f;
#pragma unroll
          for (int g = 0; g < HG; ++g)
#pragma unroll
            for (int e = 0; e < E; ++e) o[g][e] = fmaf(s[g][i], vf[e], o[g][e]);
        }
      }
    };
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (u < nch) issue(u, kb[u], vb[u]);
    for (int c0 = 0; c0 < nch; c0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int c = c0 + u;
        if (c < nch) {
          process(c, kb[u], vb[u]);
          if (c + PF < nch) issue(c + PF, kb[u], vb[u]);
        }
      }
    }
  }

  // merge the lane groups of this wave, then the waves of the block
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    const float mw = across_groups_max<L>(m[g]);
    const float sc = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - mw);
    const float lw = across_groups_sum<L>(l[g] * sc);
    float ow[E];
#pragma unroll
    for (int e = 0; e < E; ++e) ow[e] = across_groups_sum<L>(o[g][e] * sc);
    if (grp == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_o[w][g][seg * E + e] = ow[e];
      if (seg == 0) {
        s_m[w][g] = mw;
        s_l[w][g] = lw;
      }
    }
  }
  __syncthreads();
  if constexpr (G * D < NW * 64) {
    if (tid >= G * D) epi(tid - G * D, NW * 64 - G * D);
  }

  const bool direct = a.n_split == 1;
  for (int i = tid; i < G * D; i += NW * 64) {
    const int gg = i / D, d = i - gg * D;
    const int hs2 = gg / HG, g = gg - hs2 * HG;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NWP; ++v) M = fmaxf(M, s_m[v * HS + hs2][g]);
    float Ls = 0.f, Os = 0.f;
#pragma unroll
    for (int v = 0; v < NWP; ++v) {
      const int ww = v * HS + hs2;
      const float wt = (s_m[ww][g] == -INFINITY) ? 0.f : exp2f(s_m[ww][g] - M);
      Ls += wt * s_l[ww][g];
      Os += wt * s_o[ww][g][d];
    }
    const size_t row = (size_t)b * a.H_q + h * G + gg;
    if (direct) {
      T* op = reinterpret_cast<T*>(a.out) + row * D;
      op[d] = V::from_f32(Ls > 0.f ? Os / Ls : 0.f);
      if (d == 0 && a.lse) a.lse[row] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
    } else {
      const size_t prow = row * a.n_split + split;
      a.part_o[prow * D + d] = Os;
      if (d == 0) {
        a.part_ml[prow * 2] = M;
        a.part_ml[prow * 2 + 1] = Ls;
      }
    }
  }
  if constexpr (G * D >= NW * 64) epi(tid, NW * 64);
}

// ---------------------------------------------------------------- MFMA (bf16, G >= 2)
// The same attention with both products on matrix cores, for bf16 query
// groups of two or more heads (the VALU form issues about 8 G instructions
// per 16-byte segment of K/V and, from G = 4 on, runs out of issue slots).  Each wave takes the list's pages round-robin like the VALU
// form and runs one online softmax for all G heads over 16-token chunks:
//   S^T[16 tok x 16 heads] = K Q^T  on mfma_f32_16x16x32_bf16 (D/32 k-steps):
//     K rows come from HBM straight into the A operand (lane l: token l%16,
//     dims 32ks + 8(l/16) ..), the query is the B operand (head l%16 < G);
//     lane l receives S for tokens 4(l/16) .. +3 of head l%16;
//   per-head max and sum over the 16 tokens: 4 values in the lane, then the
//     16- and 32-lane swaps;
//   O^T[16 dims x 16 heads] += V^T P^T  on mfma_f32_16x16x16bf16_1k (D/16
//     dim tiles): P (rounded to bf16) is already in the B operand layout;
//     V^T comes from the chunk's rows, written to this wave's LDS buffer and
//     read back with the transposing 64-bit LDS read (lane 16g + i gets dim i
//     of tokens 4g .. 4g+3).
// Results: the same (m, l, o) per head as the VALU form, merged across waves
// the same way; only the rounding differs (P enters the product in bf16, the
// denominator sums the fp32 weights; MFMA summation order).
template <int D, int G, int NW, class PageAt, class Epi>
__device__ __forceinline__ void attend_pages_mfma(const DecodeArgs& a, int b, int h, int split,
                                                  int p0, int p1, int seq, PageAt page_at,
                                                  Epi epi) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int KS = D / 32;              // k-steps of S = K Q^T
  constexpr int DT = D / 16;              // dim tiles of O
  constexpr int PF = 2;                   // chunks of K and V in flight per wave
  constexpr int VROW = 2 * D + 32;        // LDS row stride of a V chunk (bytes)
  constexpr int VL = (16 * 2 * D) / (64 * 16);   // 16-byte V loads per lane per chunk
  static_assert(G >= 2 && G <= 16 && D % 32 == 0, "shape");
  static_assert(VL * 64 * 16 == 16 * 2 * D, "V chunk copy");
  constexpr int VBUF = 16 * VROW;
  constexpr int OBUF = G * D * 4;
  constexpr int WBUF = VBUF > OBUF ? VBUF : OBUF;   // V staging, later the wave's O
  __shared__ __align__(16) uint8_t s_w[NW][WBUF];
  __shared__ float s_m[NW][G], s_l[NW][G];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int lg = lane >> 4, lr = lane & 15;
  const int SP = a.S_p;
  uint8_t* vbuf = s_w[w];

  // query of head h*G + lr as the B operand (zero for lr >= G)
  bf16x8 qB[KS];
  {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) + ((size_t)b * a.H_q + h * G + lr) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = lr < G ? ld16(qp + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
      qB[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;            // of head lr, the same in its four lane groups

  const bf16_t* kbase = reinterpret_cast<const bf16_t*>(a.k);
  const bf16_t* vbase = reinterpret_cast<const bf16_t*>(a.v);
  const size_t vtok = (size_t)a.v_stride_tok;
  const size_t tile_k = (size_t)SP * D, tile_v = (size_t)SP * vtok;
  const int cpp = SP / kChunk;
  const int my_n = p1 > p0 + w ? (p1 - p0 - w + NW - 1) / NW : 0;
  // this lane's address of the transposing read (rows 4lg + lr/4, dims 4(lr%4) + 16dt)
  const int tr_off = (4 * lg + (lr >> 2)) * VROW + 8 * (lr & 3);

  for (int base = 0; base < my_n; base += 64) {
    const int nb = min(64, my_n - base);
    const int idx = p0 + w + NW * (base + lane);
    const int2 lp = page_at(idx, lane < nb);
    const int logi_l = lane < nb ? lp.x : 0, phys_l = lane < nb ? lp.y : 0;
    const int nch = nb * cpp;
    uint4 kb[PF][KS], vb[PF][VL];
    auto issue = [&](int c, uint4* kd, uint4* vd) {
      const int j = c / cpp, ch = c - j * cpp;
      const int phys = __builtin_amdgcn_readlane(phys_l, j);
      const bf16_t* kp = kbase + ((size_t)phys * a.H_kv + h) * tile_k + (size_t)(ch * kChunk + lr) * D;
      const bf16_t* vp = vbase + ((size_t)phys * a.H_kv + h) * tile_v + (size_t)(ch * kChunk) * vtok;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kd[ks] = ld16(kp + 32 * ks + 8 * lg);
#pragma unroll
      for (int r = 0; r < VL; ++r) {
        const int seg = r * 64 + lane, row = seg / (D / 8), col = seg % (D / 8);
        vd[r] = ld16(vp + (size_t)row * vtok + 8 * col);
      }
    };
    auto process = [&](int c, const uint4* kd, const uint4* vd) {
      const int j = c / cpp, ch = c - j * cpp;
      const int logi = __builtin_amdgcn_readlane(logi_l, j);
      const int tok0 = logi * SP + ch * kChunk;
      // V rows of the chunk into this wave's buffer
#pragma unroll
      for (int r = 0; r < VL; ++r) {
        const int seg = r * 64 + lane, row = seg / (D / 8), col = seg % (D / 8);
        st16(vbuf + row * VROW + 16 * col, vd[r]);
      }
      if (tok0 + kChunk > seq) {
        // Rows at or past seq (the unwritten tail of the last page) have
        // weight 0, but 0 * NaN would still reach O: each lane overwrites
        // its own segments of them with zeros (program order makes the
        // zeros win).
#pragma unroll
        for (int r = 0; r < VL; ++r) {
          const int seg = r * 64 + lane, row = seg / (D / 8), col = seg % (D / 8);
          if (tok0 + row >= seq) st16(vbuf + row * VROW + 16 * col, make_uint4(0u, 0u, 0u, 0u));
        }
      }
      // S^T = K Q^T
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kd[ks]), qB[ks], sc,
                                                    0, 0, 0);
      // raw scores; masked only where the chunk reaches past seq (the same
      // in every lane); the scale is positive, so the maximum is taken
      // before scaling
      float sv[4] = {sc[0], sc[1], sc[2], sc[3]};
      if (tok0 + kChunk > seq) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 4 * lg + i >= seq) sv[i] = -INFINITY;
      }
      float cm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      {
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(cm), __float_as_uint(cm),
                                                          false, false);
        cm = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(cm), __float_as_uint(cm),
                                                          false, false);
        cm = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      }
      cm *= a.scale_log2;
      // lazy reference (kLazyRescale): o and l are rescaled only when a
      // head's maximum passes its reference by more than the margin
      float alpha = 1.f;
      const bool grow = __ballot(cm > m + kLazyRescale) != 0ull;
      if (grow) {
        const float mn = fmaxf(m, cm);
        alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
        m = mn;
      }
      const float neg_m = (m == -INFINITY) ? 0.f : -m;
      s16x4 pB;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(fmaf(sv[i], a.scale_log2, neg_m));
        ps += p;                          // the denominator keeps fp32 weights
        pB[i] = (short)f32_to_bf16(p);
      }
      {
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ps), __float_as_uint(ps),
                                                          false, false);
        ps = __uint_as_float(x16[0]) + __uint_as_float(x16[1]);
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps),
                                                          false, false);
        ps = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);
      }
      l = grow ? l * alpha + ps : l + ps;
      if (grow) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[dt][i] *= alpha;
      }
      // the wave's V rows are in LDS before its transposing reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const s16x4 vA = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vbuf + tr_off + 32 * dt));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vA, pB, o[dt], 0, 0, 0);
      }
    };
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (u < nch) issue(u, kb[u], vb[u]);
    for (int c0 = 0; c0 < nch; c0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int c = c0 + u;
        if (c < nch) {
          process(c, kb[u], vb[u]);
          if (c + PF < nch) issue(c + PF, kb[u], vb[u]);
        }
      }
    }
  }

  // the wave's (m, l, o): o[dt][i] is O[head lr][dim 16dt + 4lg + i]
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* wo = reinterpret_cast<float*>(vbuf);     // [G][D]
  if (lr < G) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[lr * D + 16 * dt + 4 * lg + i] = o[dt][i];
    if (lg == 0) {
      s_m[w][lr] = m;
      s_l[w][lr] = l;
    }
  }
  __syncthreads();
  if constexpr (G * D < NW * 64) {
    if (tid >= G * D) epi(tid - G * D, NW * 64 - G * D);
  }

  const bool direct = a.n_split == 1;
  for (int i = tid; i < G * D; i += NW * 64) {
    const int gg = i / D, d = i - gg * D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, s_m[v][gg]);
    float Ls = 0.f, Os = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float wt = (s_m[v][gg] == -INFINITY) ? 0.f : exp2f(s_m[v][gg] - M);
      Ls += wt * s_l[v][gg];
      Os += wt * reinterpret_cast<const float*>(s_w[v])[gg * D + d];
    }
    const size_t row = (size_t)b * a.H_q + h * G + gg;
    if (direct) {
      bf16_t* op = reinterpret_cast<bf16_t*>(a.out) + row * D;
      op[d] = Vec16<bf16_t>::from_f32(Ls > 0.f ? Os / Ls : 0.f);
      if (d == 0 && a.lse) a.lse[row] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
    } else {
      const size_t prow = row * a.n_split + split;
      a.part_o[prow * D + d] = Os;
      if (d == 0) {
        a.part_ml[prow * 2] = M;
        a.part_ml[prow * 2 + 1] = Ls;
      }
    }
  }
  if constexpr (G * D >= NW * 64) epi(tid, NW * 64);
}

// Whether a shape takes the MFMA form: every bf16 query group of two or
// more heads.  From four heads on the VALU form runs out of issue slots; at
// two heads (the Qwen-like layer) the products are only 2 flop per byte, but
// the MFMA form still measured faster (fused step 46.2 -> 44.5 us), because it
// issues fewer instructions per 16-byte segment than the VALU form's G
// dot products and DPP reductions.
template <typename T, int D, int G>
constexpr bool attend_uses_mfma() {
  return sizeof(T) == 2 && G >= 2 && (D == 64 || D == 128);
}

// Work a caller hands to the attention's merge phase: epi(t, nt) runs once
// per thread t < nt of a thread group that is otherwise idle there (after
// the barrier that ends the page loop), or on every thread after the merge.
struct NoEpilogue {
  __device__ void operator()(int, int) const {}
};

template <typename T, int D, int G, int HS, int PF, int NW, class PageAt, class Epi = NoEpilogue>
__device__ __forceinline__ void attend_pages(const DecodeArgs& a, int b, int h, int split,
                                             int p0, int p1, int seq, PageAt page_at,
                                             Epi epi = Epi()) {
  if constexpr (attend_uses_mfma<T, D, G>())
    attend_pages_mfma<D, G, NW>(a, b, h, split, p0, p1, seq, page_at, epi);
  else
    attend_pages_valu<T, D, G, HS, PF, NW>(a, b, h, split, p0, p1, seq, page_at, epi);
}

// Chunks of K and V kept in flight per wave: two, or one where 32 lanes per
// row (fp32, D = 128) make a chunk of K and V 64 registers.
template <typename T, int D>
constexpr int attend_prefetch() {
  return (sizeof(T) == 4 && D == 128) ? 1 : 2;
}

// Query-head slices per wave group: the G = 8 group is split in two halves.
template <int G>
constexpr int attend_head_slices() {
  return G == 8 ? 2 : 1;
}

}  // namespace vx
