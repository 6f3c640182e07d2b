// K4 (VALU) + K5: split-K paged decode attention over a list of logical
// pages (the selected ones, or every page for the dense baseline).  The
// attention itself is the exact softmax attention the method runs after page
// selection (Vortex article, "A dual-stage programmable abstraction"); the
// split into page ranges with fp32 partials merged afterwards is this
// library's scheduling, not something the pages prescribe.
//
// One block of 8 waves per (split, KV head, request).  Lanes hold 16-byte
// segments of a token row: L = D*e/16 lanes per row, R = 64/L rows (tokens)
// per wave-load, so one wave-load reads 1 KiB of a page-head tile
// contiguously.  Each lane group of L lanes runs its own online softmax over
// the tokens it holds (per-token dot products reduced with DPP row moves, no
// LDS traffic), so nothing crosses lane groups inside the loop.  Waves take
// the split's pages round-robin and keep PF 16-token chunks of K and V in
// flight.  With G = 8 the two halves of the query group go to different
// waves over the same pages (register pressure).  Lane groups merge with
// shuffles and waves merge through LDS; the block writes the output directly
// when the request has a single split, else fp32 partials for K5.
#include "vx_device.h"
#include "vx_internal.h"

namespace vx {
namespace {

constexpr int kChunk = 16;   // tokens per softmax update
constexpr int kNW = 8;       // waves per block

template <typename T, int D, int G, int HS, int PF>
__global__ __launch_bounds__(kNW * 64) void decode_valu_kernel(DecodeArgs a) {
  using V = Vec16<T>;
  constexpr int E = V::E;
  constexpr int L = D / E;          // lanes per token row
  constexpr int R = 64 / L;         // token rows per wave-load
  constexpr int NL = kChunk / R;    // wave-loads per chunk (K and V each)
  constexpr int HG = G / HS;        // query heads per wave
  constexpr int NWP = kNW / HS;     // waves working on different pages
  static_assert(L * R == 64 && NL * R == kChunk && HG * HS == G, "layout");

  __shared__ float s_m[kNW][HG], s_l[kNW][HG];
  __shared__ float s_o[kNW][HG][D];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int seg = lane % L, grp = lane / L;
  const int hs = w % HS, wp = w / HS;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int SP = a.S_p;

  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + SP - 1) / SP;

  // length of this request's page list
  const int32_t* selrow = nullptr;
  int count = n_b;
  if (a.sel) {
    selrow = a.sel + ((size_t)b * a.H_kv + h) * a.k_tot;
    count = a.k_tot;
    for (int base = 0; base < a.k_tot; base += 64) {
      const int i = base + lane;
      const int p = i < a.k_tot ? selrow[i] : 0;
      const unsigned long long bad = __ballot(i < a.k_tot && (p < 0 || p >= n_b));
      if (bad) { count = base + __builtin_ctzll(bad); break; }
    }
  }
  const int p0 = split * a.pages_per_split;
  const int p1 = min(p0 + a.pages_per_split, count);
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
  const int32_t* ptb = a.pt + (size_t)b * a.pt_stride;
  const size_t tile_k = (size_t)SP * D;
  const size_t vtok = (size_t)a.v_stride_tok;
  const size_t tile_v = (size_t)SP * vtok;
  const int cpp = SP / kChunk;
  const int my_n = p1 > p0 + wp ? (p1 - p0 - wp + NWP - 1) / NWP : 0;

  for (int base = 0; base < my_n; base += 64) {
    const int nb = min(64, my_n - base);
    int logi_l = 0, phys_l = 0;
    if (lane < nb) {
      const int idx = p0 + wp + NWP * (base + lane);
      logi_l = selrow ? selrow[idx] : idx;
      phys_l = ptb[logi_l];
    }
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
        const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m[g] - mn);
        m[g] = mn;
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) o[g][e] *= alpha;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const float p = (mn == -INFINITY) ? 0.f : exp2f(s[g][i] - mn);
          s[g][i] = p;
          l[g] += p;
        }
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float vf[E];
        V::unpack(vd[i], vf);
#pragma unroll
        for (int g = 0; g < HG; ++g)
#pragma unroll
          for (int e = 0; e < E; ++e) o[g][e] = fmaf(s[g][i], vf[e], o[g][e]);
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

  const bool direct = a.n_split == 1;
  for (int i = tid; i < G * D; i += kNW * 64) {
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
}

// K5: merge the splits of one (request, query head).  Splits with an empty
// page range have sum 0 and are skipped.
template <typename T, int DV>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
  constexpr int PER = (DV + 63) / 64;
  __shared__ float w[1024];
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;            // b * H_q + hq
  const float* ml = a.part_ml + row * a.n_split * 2;
  float mx = -INFINITY;
  for (int i = lane; i < a.n_split; i += 64) {
    if (ml[2 * i + 1] > 0.f) mx = fmaxf(mx, ml[2 * i]);
  }
  mx = wave_max(mx);
  float tot = 0.f;
  for (int i = lane; i < a.n_split; i += 64) {
    const float li = ml[2 * i + 1];
    const float wi = li > 0.f ? exp2f(ml[2 * i] - mx) : 0.f;
    w[i] = wi;
    tot += wi * li;
  }
  tot = wave_sum(tot);
  __syncthreads();
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  const float* po = a.part_o + row * a.n_split * DV;
  for (int i = 0; i < a.n_split; ++i) {
    const float wi = w[i];
    if (wi == 0.f) continue;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = j * 64 + lane;
      if (d < DV) acc[j] = fmaf(wi, po[(size_t)i * DV + d], acc[j]);
    }
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  T* op = reinterpret_cast<T*>(a.out) + row * DV;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int d = j * 64 + lane;
    if (d < DV) op[d] = Vec16<T>::from_f32(acc[j] * inv);
  }
  if (lane == 0 && a.lse) a.lse[row] = tot > 0.f ? (mx + __log2f(tot)) * kLn2 : -INFINITY;
}

template <typename T, int D, int G, int HS, int PF>
hipError_t run_decode(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.H_kv, a.B);
  hipLaunchKernelGGL((decode_valu_kernel<T, D, G, HS, PF>), grid, dim3(kNW * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_decode_g(int G, const DecodeArgs& a, hipStream_t s) {
  // chunks in flight per wave: two, except where 32 lanes per row (fp32,
  // D = 128) make one chunk of K and V 64 registers
  constexpr int PF = (sizeof(T) == 4 && D == 128) ? 1 : 2;
  switch (G) {
    case 1: return run_decode<T, D, 1, 1, PF>(a, s);
    case 2: return run_decode<T, D, 2, 1, PF>(a, s);
    case 4: return run_decode<T, D, 4, 1, PF>(a, s);
    case 8: return run_decode<T, D, 8, 2, PF>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int DV>
hipError_t run_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<T, DV>), dim3(a.B * a.H_q), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_valu(int dtype, int D, int G, const DecodeArgs& a, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return run_decode_g<float, 64>(G, a, s);
    if (D == 128) return run_decode_g<float, 128>(G, a, s);
  } else {
    if (D == 64) return run_decode_g<bf16_t, 64>(G, a, s);
    if (D == 128) return run_decode_g<bf16_t, 128>(G, a, s);
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
