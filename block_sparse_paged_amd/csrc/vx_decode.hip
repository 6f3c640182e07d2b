// K4 (VALU) + K5: split-K paged decode attention over a list of logical
// pages (the selected ones, or every page for the dense baseline).  The
// attention itself is the exact softmax attention the method runs after page
// selection (Vortex article, "A dual-stage programmable abstraction"); the
// split into page ranges with fp32 partials merged afterwards is this
// library's scheduling, not something the pages prescribe.
//
// One wave per (split, KV head, request).  Lanes hold 16-byte segments of a
// token row: L = D*e/16 lanes per row, R = 64/L rows (tokens) per wave-load,
// so one wave-load reads 1 KiB of a page-head tile contiguously.  Per lane:
// the G query rows' segments (fp32, pre-scaled by sm_scale*log2 e), the
// running output segments for its token group, and per-group softmax sums.
// Dot products are reduced across the L lanes of a row; the running max is
// shared across the wave.  Pages are processed in 16-token chunks with the
// next chunk's K and V loads issued before the current chunk is consumed.
#include "vx_device.h"
#include "vx_internal.h"

namespace vx {
namespace {

constexpr int kChunk = 16;   // tokens per softmax update

template <typename T, int D, int G>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeArgs a) {
  using V = Vec16<T>;
  constexpr int E = V::E;
  constexpr int L = D / E;          // lanes per token row
  constexpr int R = 64 / L;         // token rows per wave-load
  constexpr int NL = kChunk / R;    // wave-loads per chunk (K and V each)
  static_assert(L * R == 64 && NL * R == kChunk, "layout");

  const int lane = threadIdx.x;
  const int seg = lane % L, grp = lane / L;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int SP = a.S_p;

  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + SP - 1) / SP;

  // number of pages in this request's list
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
  const bool direct = a.n_split == 1;
  const int hq0 = h * G;

  // query segments, pre-scaled
  float q[G][E];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.H_q + hq0) * D + seg * E;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      V::unpack(ld16(qp + (size_t)g * D), q[g]);
#pragma unroll
      for (int e = 0; e < E; ++e) q[g][e] *= a.scale_log2;
    }
  }

  float o[G][E], l[G], m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = 0.f;
    m[g] = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.f;
  }

  const T* kbase = reinterpret_cast<const T*>(a.k);
  const T* vbase = reinterpret_cast<const T*>(a.v);
  const int32_t* ptb = a.pt + (size_t)b * a.pt_stride;
  const size_t tile_k = (size_t)SP * D;                       // elements per page-head tile
  const size_t vtok = (size_t)a.v_stride_tok;                 // elements between V tokens
  const size_t tile_v = (size_t)SP * vtok;
  const int cpp = SP / kChunk;                                // chunks per page

  for (int base = p0; base < p1; base += 64) {
    const int np = min(64, p1 - base);
    int logi_l = 0, phys_l = 0;
    if (lane < np) {
      logi_l = selrow ? selrow[base + lane] : base + lane;
      phys_l = ptb[logi_l];
    }
    const int nchunks = np * cpp;
    uint4 kr[NL], vr[NL], kn[NL], vn[NL];
    auto issue = [&](int u, uint4* kd, uint4* vd) {
      const int j = u / cpp, c = u - j * cpp;
      const int phys = __builtin_amdgcn_readlane(phys_l, j);
      const T* kp = kbase + ((size_t)phys * a.H_kv + h) * tile_k + (size_t)(c * kChunk) * D;
      const T* vp = vbase + ((size_t)phys * a.H_kv + h) * tile_v + (size_t)(c * kChunk) * vtok;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int t = i * R + grp;
        kd[i] = ld16(kp + (size_t)t * D + seg * E);
        vd[i] = ld16(vp + (size_t)t * vtok + seg * E);
      }
    };
    issue(0, kr, vr);
    for (int u = 0; u < nchunks; ++u) {
      if (u + 1 < nchunks) issue(u + 1, kn, vn);
      const int j = u / cpp, c = u - j * cpp;
      const int logi = __builtin_amdgcn_readlane(logi_l, j);
      const int tok0 = logi * SP + c * kChunk;
      // logits of this lane's tokens
      float s[G][NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float kf[E];
        V::unpack(kr[i], kf);
        const bool valid = tok0 + i * R + grp < seq;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) acc = fmaf(q[g][e], kf[e], acc);
          acc = group_sum<L>(acc);
          s[g][i] = valid ? acc : -INFINITY;
        }
      }
      // online softmax update (log2 domain)
      float alpha[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mc = s[g][0];
#pragma unroll
        for (int i = 1; i < NL; ++i) mc = fmaxf(mc, s[g][i]);
        mc = across_groups_max<L>(mc);
        const float mn = fmaxf(m[g], mc);
        alpha[g] = (mn == -INFINITY) ? 1.f : exp2f(m[g] - mn);
        m[g] = mn;
        l[g] *= alpha[g];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const float p = (mn == -INFINITY) ? 0.f : exp2f(s[g][i] - mn);
          s[g][i] = p;
          l[g] += p;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) o[g][e] *= alpha[g];
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float vf[E];
        V::unpack(vr[i], vf);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < E; ++e) o[g][e] = fmaf(s[g][i], vf[e], o[g][e]);
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) { kr[i] = kn[i]; vr[i] = vn[i]; }
    }
  }

  // merge the token groups and write
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float lt = across_groups_sum<L>(l[g]);
    float ot[E];
#pragma unroll
    for (int e = 0; e < E; ++e) ot[e] = across_groups_sum<L>(o[g][e]);
    const int hq = hq0 + g;
    const size_t row = (size_t)b * a.H_q + hq;
    if (direct) {
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ot[e] *= inv;
      if (grp == 0) {
        T* op = reinterpret_cast<T*>(a.out) + row * D + seg * E;
        st16(op, V::pack(ot));
        if (seg == 0 && a.lse) a.lse[row] = lt > 0.f ? (m[g] + __log2f(lt)) * kLn2 : -INFINITY;
      }
    } else {
      const size_t prow = row * a.n_split + split;
      if (grp == 0) {
        float* po = a.part_o + prow * D + seg * E;
        st16(po, Vec16<float>::pack(ot));
        if (E == 8) st16(po + 4, Vec16<float>::pack(ot + 4));
        if (seg == 0) {
          a.part_ml[prow * 2] = m[g];
          a.part_ml[prow * 2 + 1] = lt;
        }
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

template <typename T, int D, int G>
hipError_t run_decode(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.H_kv, a.B);
  hipLaunchKernelGGL((decode_valu_kernel<T, D, G>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
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
