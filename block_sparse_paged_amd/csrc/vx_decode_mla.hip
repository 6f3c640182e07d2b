// K4 (MFMA): split-K paged decode for MLA-shaped attention: up to 32 query
// heads on one latent KV head, 576-dim keys (512 latent + 64 rotary) and
// values that are the first 512 dims of the same rows, 64-token pages.  The
// "rope-aware block-sparse attention for MLA" of the Vortex announcement
// (digg thread, post [4/6]) selects pages on the full 576-dim key and attends
// exactly over them; this kernel is the attention half.
//
// At ~60 flop per byte of KV this is past the fp32 VALU roofline, so both
// products run on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accum).
// One 256-thread block per (split, request).  Per 32-token tile (36 KiB):
//   - all threads copy the tile HBM -> registers -> LDS, the next tile's
//     global loads being in flight while the current one is computed;
//   - S^T = K Q^T: wave w owns tokens 16*(w&1).. and heads 16*(w>>1)..; the
//     query stays in registers as the MFMA B operand (18 k-steps of 32 dims);
//   - online softmax per head, the two token halves exchanging their maxima
//     and sums through LDS; P goes to LDS in bf16;
//   - O += P V: wave w owns V dims 128w..128w+127 (2 head tiles x 8 dim tiles
//     of 16x16 accumulators).  V is read from the K tile already in LDS, so
//     HBM sees each 576-dim row once.  The MFMA contracts over tokens: lane
//     group g takes tokens 8g .. 8g+7, read two rows of four at a time with
//     the transposing 64-bit LDS read; P is stored [head][token].
#include "vx_device.h"
#include "vx_internal.h"

namespace vx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDqk = 576, kDv = 512, kHeads = 32;
constexpr int kPage = 64;                    // tokens per page
constexpr int kT = 32;                       // tokens per tile
constexpr int kRowB = kDqk * 2;              // 1152 bytes per token row
constexpr int kLdsRow = kRowB + 32;          // padded LDS row stride (296 dwords)
constexpr int kThreads = 256;
constexpr int kChunksPerRow = kRowB / 16;    // 72
constexpr int kLoads = kT * kChunksPerRow / kThreads;   // 9 x 16 B per thread per tile
constexpr int kMaxPages = 256;               // pages per split (planner bound)
static_assert(kT * kChunksPerRow == kLoads * kThreads, "tile copy");

__device__ __forceinline__ float neg_inf() { return -INFINITY; }

__global__ __launch_bounds__(kThreads, 2) void decode_mla_kernel(DecodeArgs a) {
  __shared__ __align__(16) uint8_t ktile[kT * kLdsRow];
  __shared__ __align__(16) bf16_t ptile[kHeads * kT];   // [head][g][i] = P[head][4i+g]
  __shared__ float red_max[2][kHeads];
  __shared__ float red_sum[2][kHeads];
  __shared__ float m_state[2][kHeads];
  __shared__ float l_state[kHeads];
  __shared__ int page_phys[kMaxPages];
  __shared__ int page_logi[kMaxPages];
  __shared__ int s_count;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lg = l >> 4, lr = l & 15;          // lane group (k-block), row in group
  const int tw = w & 1, hw = w >> 1;
  const int split = blockIdx.x, b = blockIdx.y;
  const int G = a.H_q;                          // H_kv == 1

  int seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_tokens ? a.max_tokens : seq);
  const int n_b = (seq + kPage - 1) / kPage;
  const int32_t* selrow = a.sel ? a.sel + (size_t)b * a.k_tot : nullptr;
  if (w == 0) {
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
  if (tid < kHeads) {
    m_state[0][tid] = neg_inf();
    l_state[tid] = 0.f;
  }
  __syncthreads();
  const int count = s_count;
  const int p0 = split * a.pages_per_split;
  const int p1 = min(p0 + a.pages_per_split, count);
  const int np = max(p1 - p0, 0);
  const int32_t* ptb = a.pt + (size_t)b * a.pt_stride;
  for (int i = tid; i < np; i += kThreads) {
    const int logi = selrow ? selrow[p0 + i] : p0 + i;
    page_logi[i] = logi;
    page_phys[i] = ptb[logi];
  }

  // query as the B operand of S^T = K Q^T: head 16*hw + lr, dims 32*ks + 8*lg ..
  bf16x8 qB[kDqk / 32];
  {
    const int head = 16 * hw + lr;
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) + ((size_t)b * a.H_q + head) * kDqk;
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) {
      uint4 v = head < G ? ld16(qp + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
      qB[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[2][8];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

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

  int par = 0;
  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();                             // previous tile fully consumed
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + r * kThreads;
      const int row = c / kChunksPerRow, col = c - row * kChunksPerRow;
      st16(ktile + row * kLdsRow + col * 16, regs[r]);
    }
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(t + 1);

    const int j = t / (kPage / kT), half = t % (kPage / kT);
    const int tok0 = page_logi[j] * kPage + half * kT;

    // ---- S^T tile: tokens 16*tw + 4*lg + i, head 16*hw + lr
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* krow = ktile + (16 * tw + lr) * kLdsRow + 16 * lg;
#pragma unroll
      for (int ks = 0; ks < kDqk / 32; ++ks) {
        const bf16x8 kA = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + 64 * ks));
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, qB[ks], s, 0, 0, 0);
      }
    }
    const int head = 16 * hw + lr;
    float sv[4];
    float mx = neg_inf();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = tok0 + 16 * tw + 4 * lg + i;
      sv[i] = pos < seq ? s[i] * a.scale_log2 : neg_inf();
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (lg == 0) red_max[tw][head] = mx;
    __syncthreads();
    const float m_old = m_state[par][head];
    const float m_new = fmaxf(m_old, fmaxf(red_max[0][head], red_max[1][head]));
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = (m_new == neg_inf()) ? 0.f : exp2f(sv[i] - m_new);
      const bf16_t pb = f32_to_bf16(p);
      psum += Vec16<bf16_t>::to_f32(pb);
      ptile[head * kT + 16 * tw + 4 * lg + i] = pb;    // [head][token]
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    if (lg == 0) {
      red_sum[tw][head] = psum;
      if (tw == 0) m_state[par ^ 1][head] = m_new;
    }
    __syncthreads();
    if (tid < kHeads) {
      const float mo = m_state[par][tid], mn = m_state[par ^ 1][tid];
      const float alpha = (mn == neg_inf()) ? 1.f : exp2f(mo - mn);
      l_state[tid] = l_state[tid] * alpha + red_sum[0][tid] + red_sum[1][tid];
    }

    // ---- O += P V for dims 128*w .. 128*w + 127
    float alpha[2][4];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * ht + 4 * lg + i;
        const float mo = m_state[par][h], mn = m_state[par ^ 1][h];
        alpha[ht][i] = (mn == neg_inf()) ? 1.f : exp2f(mo - mn);
      }
    bf16x8 pA[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
      pA[ht] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(ptile + (16 * ht + lr) * kT + 8 * lg));
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      // V rows 8lg .. 8lg+7, dims 128w + 16dt .. +15, transposed by the LDS
      // read: lane 16g + i gets dim i of four rows supplied by lanes
      // 16g + 4j + c (row 8g + j (+4), dims 4c .. 4c+3)
      const uint8_t* vsrc = ktile + (8 * lg + (lr >> 2)) * kLdsRow + 2 * (128 * w + 16 * dt + 4 * (lr & 3));
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vsrc));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vsrc + 4 * kLdsRow));
      const s16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      const bf16x8 vB = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        f32x4 acc = o[ht][dt];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= alpha[ht][i];
        o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pA[ht], vB, acc, 0, 0, 0);
      }
    }
    par ^= 1;
  }
  __syncthreads();

  // ---- write: o[ht][dt][i] is O[head 16*ht + 4*lg + i][dim 128*w + 16*dt + lr]
  const bool direct = a.n_split == 1;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * ht + 4 * lg + i;
      if (h >= G) continue;
      const float m = m_state[par][h], lt = l_state[h];
      const size_t row = (size_t)b * a.H_q + h;
      if (direct) {
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        bf16_t* op = reinterpret_cast<bf16_t*>(a.out) + row * kDv;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) op[128 * w + 16 * dt + lr] = f32_to_bf16(o[ht][dt][i] * inv);
        if (w == 0 && lr == 0 && a.lse)
          a.lse[row] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : neg_inf();
      } else {
        const size_t prow = row * a.n_split + split;
        float* po = a.part_o + prow * kDv;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) po[128 * w + 16 * dt + lr] = o[ht][dt][i];
        if (w == 0 && lr == 0) {
          a.part_ml[prow * 2] = m;
          a.part_ml[prow * 2 + 1] = lt;
        }
      }
    }
}

}  // namespace

int mla_max_pages_per_split() { return kMaxPages; }

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t s) {
  if (a.pages_per_split > kMaxPages || a.S_p != kPage || a.H_kv != 1 || a.H_q > kHeads)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_mla_kernel, dim3(a.n_split, a.B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace vx
