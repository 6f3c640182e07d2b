// C-ABI entry points of libvx: argument validation (before any HIP call),
// launch planning, workspace layout and kernel dispatch.
//
// Planning ("workload planner for balanced GPU scheduling", Vortex article,
// "A dual-stage programmable abstraction") is a pure function of the shapes
// and of the GPU's compute-unit count (queried once per device): every
// (request, KV head) is cut into splits of whole pages so that the launch
// holds enough waves to keep every CU streaming, and the fp32 partials the
// splits produce stay a small fraction of the K/V bytes they replace.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "vx.h"
#include "vx_internal.h"

namespace {

using namespace vx;

constexpr int kDefaultCUs = 256;   // MI355X, when the device cannot be queried
// blocks per CU the planner aims for (split decode blocks are 8 waves, MLA
// blocks 4): one wave of resident blocks for the sparse step, several for
// the long dense stream so that unequal requests even out
constexpr int kSparseBlocksPerCU = 1;
constexpr int kFullBlocksPerCU = 16;
// MLA (4-wave blocks, two resident per CU): the sparse step takes one block
// per CU.  Its blocks select their pages themselves, so fewer, longer splits
// repeat less selection and leave the combine fewer partials (MLA step 70.9
// -> 68.1 us against two per CU); the dense stream keeps two per CU.
constexpr int kMlaSparseBlocksPerCU = 1;
constexpr int kMlaFullBlocksPerCU = 2;
constexpr int kMaxSplits = 1024;
constexpr int kMaxOrderedBatch = 512;
constexpr int kMaxCandidates = 16384;
constexpr int kFusedMaxPages = 6144;
            // page ids + keys in LDS: 48 KiB
constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

// Per-device properties, queried once per device (256 CUs / 64 KiB of LDS
// per block if a query fails).
struct DeviceProps {
  int cus = 0;
  size_t lds = 0;
};

const DeviceProps& device_props() {
  static DeviceProps cached[kMaxDevices];
  static const DeviceProps fallback{kDefaultCUs, 65536};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fallback;
  DeviceProps& p = cached[dev];
  if (!p.cus) {
    int v = 0;
    p.lds = (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
                 hipSuccess && v > 0)
                ? (size_t)v
                : 65536;
    v = 0;
    p.cus = (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                 hipSuccess && v > 0)
                ? v
                : kDefaultCUs;
  }
  return p;
}

// Largest LDS allocation one block may use on the current device.
size_t max_lds_per_block() { return device_props().lds; }
// Compute units of the current device.
int device_cus() { return device_props().cus; }

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }
int elem_bytes(int dtype) { return dtype == VX_F32 ? 4 : 2; }

bool is_mla(const vx_paged_kv* kv) { return kv->head_dim_qk == 576; }

vx_status check_kv(const vx_paged_kv* kv) {
  if (!kv) return VX_ERR_INVALID_ARGUMENT;
  if (kv->dtype != VX_F32 && kv->dtype != VX_BF16) return VX_ERR_INVALID_ARGUMENT;
  if (kv->num_pages < 1 || kv->page_size < 1 || kv->num_kv_heads < 1 ||
      kv->head_dim_qk < 1 || kv->head_dim_v < 1 || kv->reserved_ != 0)
    return VX_ERR_INVALID_ARGUMENT;
  if (kv->v_aliases_k != 0 && kv->v_aliases_k != 1) return VX_ERR_INVALID_ARGUMENT;
  if (kv->v_aliases_k) {
    if (kv->v_cache != nullptr || kv->head_dim_v > kv->head_dim_qk) return VX_ERR_INVALID_ARGUMENT;
  }
  if (kv->page_size != 16 && kv->page_size != 64) return VX_ERR_UNSUPPORTED;
  const int dq = kv->head_dim_qk, dv = kv->head_dim_v;
  if (dq == 576) {
    if (kv->dtype != VX_BF16 || dv != 512 || !kv->v_aliases_k || kv->num_kv_heads != 1 ||
        kv->page_size != 64)
      return VX_ERR_UNSUPPORTED;
  } else if (dq == 64 || dq == 128) {
    if (dv != dq) return VX_ERR_UNSUPPORTED;
  } else {
    return VX_ERR_UNSUPPORTED;
  }
  return VX_OK;
}

vx_status check_batch(const vx_paged_kv* kv, const vx_batch* bt) {
  if (!bt) return VX_ERR_INVALID_ARGUMENT;
  if (bt->batch < 0 || bt->num_q_heads < 1 || bt->max_pages_per_req < 1 || bt->max_seq_len < 1)
    return VX_ERR_INVALID_ARGUMENT;
  if (bt->num_q_heads % kv->num_kv_heads != 0) return VX_ERR_INVALID_ARGUMENT;
  if ((long long)bt->max_pages_per_req * kv->page_size < bt->max_seq_len)
    return VX_ERR_INVALID_ARGUMENT;
  const int G = bt->num_q_heads / kv->num_kv_heads;
  if (is_mla(kv)) {
    if (G > 32) return VX_ERR_UNSUPPORTED;
  } else if (G != 1 && G != 2 && G != 4 && G != 8) {
    return VX_ERR_UNSUPPORTED;
  }
  return VX_OK;
}

int max_pages_eff(const vx_paged_kv* kv, const vx_batch* bt) {
  return ceil_div(bt->max_seq_len, kv->page_size);
}

struct DecodePlan {
  int pages_per_split = 1;
  int n_split = 1;
  bool work_list = false;  // dense: persistent blocks over (request, chunk, KV head) items
  int blocks = 0;          // blocks of a work-list launch
  size_t part_o_bytes = 0, part_ml_bytes = 0;
  size_t ws_bytes() const { return part_o_bytes + part_ml_bytes; }
};

// Dense work list: pages per item, and blocks per CU.  One 8-wave block is
// resident per CU at a time (registers); four per CU in all still leave the
// dispatcher room to even out CUs that run at different speeds.  Items of
// 64 to 512 pages and 2 to 8 blocks per CU measured within 3% of each other
// (Qwen-like, heterogeneous and long-context dense decodes).
constexpr int kItemPages = 128;
constexpr int kItemBlocksPerCU = 4;

// Splits for `pages` pages per (request, KV head) on a GPU of `cus` compute
// units.  pps_hint > 0 asks for that many pages per split (still at least
// ceil(pages / kMaxSplits), and at most what the MLA kernel's page list
// holds).  A pure function of its arguments.
DecodePlan plan_decode(const vx_paged_kv* kv, const vx_batch* bt, int pages, bool sparse, int cus,
                       int pps_hint = 0) {
  DecodePlan p;
  const long long units = std::max(1LL, (long long)bt->batch * kv->num_kv_heads);
  const int G = bt->num_q_heads / kv->num_kv_heads;
  pages = std::max(pages, 1);
  cus = std::max(cus, 1);
  int pps;
  if (!sparse && !is_mla(kv) && bt->batch <= decode_items_max_batch()) {
    // dense: equal-size items over every request's pages, walked by a fixed
    // number of blocks, so a mixed-length batch streams evenly
    pps = std::max(pps_hint > 0 ? pps_hint : kItemPages, ceil_div(pages, kMaxSplits));
    p.work_list = true;
    p.pages_per_split = pps;
    p.n_split = ceil_div(pages, pps);
    const long long items = units * p.n_split;
    p.blocks = (int)std::min<long long>(items, (long long)cus * kItemBlocksPerCU);
  } else if (pps_hint > 0) {
    pps = pps_hint;
  } else if (is_mla(kv)) {
    const long long target = (long long)cus * (sparse ? kMlaSparseBlocksPerCU : kMlaFullBlocksPerCU);
    const int n_want = std::max(1, ceil_div(target, units));
    pps = ceil_div(pages, n_want);
    // partials: G rows of (D_v + 2) fp32, written and read once per split
    // (the reads mostly hit the on-package cache, hence the loose cap)
    const double kv_bytes = (double)pages * kv->page_size * kv->head_dim_qk * 2;
    while (ceil_div(pages, pps) > 1 &&
           (double)ceil_div(pages, pps) * G * (kv->head_dim_v + 2) * 8 > 0.6 * kv_bytes)
      ++pps;
  } else {
    const long long target = (long long)cus * (sparse ? kSparseBlocksPerCU : kFullBlocksPerCU);
    const int n_want = std::max(1, ceil_div(target, units));
    pps = ceil_div(pages, n_want);
    if (!sparse) pps = std::max(pps, 64);
    const double kv_bytes = (double)pages * kv->page_size *
                            (kv->head_dim_qk + kv->head_dim_v) * elem_bytes(kv->dtype);
    while (ceil_div(pages, pps) > 1 &&
           (double)ceil_div(pages, pps) * G * (kv->head_dim_v + 2) * 8 > 0.15 * kv_bytes)
      ++pps;
  }
  if (!p.work_list) {
    pps = std::max(pps, ceil_div(pages, kMaxSplits));
    if (is_mla(kv)) pps = std::min(pps, mla_max_pages_per_split());   // LDS page list
    p.pages_per_split = pps;
    p.n_split = ceil_div(pages, pps);
  }
  if (p.n_split > 1) {
    const size_t rows = (size_t)bt->batch * bt->num_q_heads * p.n_split;
    p.part_o_bytes = align_up(rows * kv->head_dim_v * sizeof(float));
    p.part_ml_bytes = align_up(rows * 2 * sizeof(float));
  }
  return p;
}

// Pages per (request, KV head) a decode call walks: the selection's length,
// or every page the batch can hold.
int decode_pages(const vx_paged_kv* kv, const vx_batch* bt, bool sparse, int k_tot) {
  return sparse ? k_tot : max_pages_eff(kv, bt);
}

size_t score_ws_bytes(const vx_paged_kv* kv, const vx_batch* bt) {
  return align_up((size_t)bt->batch * kv->num_kv_heads * max_pages_eff(kv, bt) * sizeof(float));
}

vx_status hip_status(hipError_t e) { return e == hipSuccess ? VX_OK : VX_ERR_HIP; }

// Selection done inside the split decode kernel from the indexer's scores
// (the fused step's fallback for few (request, KV head) units).
struct SelectInDecode {
  const float* scores;
  int32_t* sel_out;
  int32_t score_stride, topk, n_bos, n_eos;
  size_t ws_offset;        // partials start here in the workspace (after the scores)
};

vx_status run_decode(const vx_paged_kv* kv, const vx_batch* bt, const void* q,
                     const int32_t* sel, int32_t k_tot, float sm_scale, void* out, float* lse,
                     void* ws, size_t ws_bytes, hipStream_t stream,
                     const SelectInDecode* fs = nullptr, const DecodePlan* given = nullptr) {
  const bool sparse = sel != nullptr || fs != nullptr;
  const DecodePlan p =
      given ? *given : plan_decode(kv, bt, decode_pages(kv, bt, sparse, k_tot), sparse, device_cus());
  const size_t off = fs ? fs->ws_offset : 0;
  if (ws_bytes < off + p.ws_bytes()) return VX_ERR_WORKSPACE_TOO_SMALL;
  if (p.ws_bytes() > 0 && ws == nullptr) return VX_ERR_INVALID_ARGUMENT;
  if (bt->batch == 0) return VX_OK;
  ws = reinterpret_cast<char*>(ws) + off;

  DecodeArgs a{};
  a.q = q;
  a.k = kv->k_cache;
  a.v = kv->v_aliases_k ? kv->k_cache : kv->v_cache;
  a.pt = bt->page_table;
  a.seq_lens = bt->seq_lens;
  a.sel = sel;
  a.B = bt->batch;
  a.H_q = bt->num_q_heads;
  a.H_kv = kv->num_kv_heads;
  a.S_p = kv->page_size;
  a.pt_stride = bt->max_pages_per_req;
  a.k_tot = k_tot;
  a.max_tokens = bt->max_seq_len;   // validated <= max_pages_per_req * page_size
  a.pages_per_split = p.pages_per_split;
  a.n_split = p.n_split;
  a.v_stride_tok = kv->v_aliases_k ? kv->head_dim_qk : kv->head_dim_v;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  if (fs) {
    a.scores = fs->scores;
    a.sel_out = fs->sel_out;
    a.score_stride = fs->score_stride;
    a.topk = fs->topk;
    a.n_bos = fs->n_bos;
    a.n_eos = fs->n_eos;
  }
  if (p.n_split > 1) {
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.part_o_bytes);
  }
  a.work_list = p.work_list ? 1 : 0;
  const int G = bt->num_q_heads / kv->num_kv_heads;
  hipError_t e =
      p.work_list ? launch_decode_items(kv->dtype, kv->head_dim_qk, G, a, p.blocks, stream)
      : is_mla(kv) ? launch_decode_mla(a, stream)
                   : launch_decode_split(kv->dtype, kv->head_dim_qk, G, a, stream);
  if (e != hipSuccess) return VX_ERR_HIP;
  if (p.n_split > 1) {
    CombineArgs c{};
    if (p.work_list) {         // a request merges only the chunks it has
      c.seq_lens = bt->seq_lens;
      c.S_p = kv->page_size;
      c.pages_per_split = p.pages_per_split;
      c.max_tokens = bt->max_seq_len;
    }
    c.part_o = a.part_o;
    c.part_ml = a.part_ml;
    c.out = out;
    c.lse = lse;
    c.B = bt->batch;
    c.H_q = bt->num_q_heads;
    c.n_split = p.n_split;
    c.D_v = kv->head_dim_v;
    e = launch_combine(kv->dtype, c, stream);
  }
  return hip_status(e);
}

hipError_t launch_split_score(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                              int32_t n_bos, int32_t n_eos, float* scores, bool update_completed,
                              hipStream_t stream);
hipError_t launch_completed_centroids(const vx_paged_kv* kv, const vx_batch* batch,
                                      hipStream_t stream);

// The indexer.  With update_completed (the decode step) it also writes the
// centroids of the pages the batch's latest tokens completed: inside the
// split scorer when that runs, else with the centroid kernel first.
vx_status score_topk_impl(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                          int32_t topk, int32_t n_bos, int32_t n_eos, int32_t* sel,
                          void* workspace, size_t workspace_bytes, hipStream_t stream,
                          bool update_completed = false, int levels = 0,
                          const uint32_t* rnd = nullptr) {
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if ((st = check_batch(kv, batch)) != VX_OK) return st;
  if (topk < 0 || n_bos < 0 || n_eos < 1) return VX_ERR_INVALID_ARGUMENT;
  if ((long long)topk + n_bos + n_eos > 0x7fffffffLL) return VX_ERR_INVALID_ARGUMENT;
  if (batch->batch == 0) return VX_OK;
  if (!q || !sel || !kv->centroids || !batch->page_table || !batch->seq_lens)
    return VX_ERR_INVALID_ARGUMENT;
  const int mp = max_pages_eff(kv, batch);
  if (mp > kMaxCandidates) return VX_ERR_UNSUPPORTED;
  const size_t need = score_ws_bytes(kv, batch);
  if (workspace_bytes < need) return VX_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return VX_ERR_INVALID_ARGUMENT;
  const int k_tot = topk + n_bos + n_eos;
  // device-side lengths are clamped to this bound, which keeps every page
  // table read and score write in range even for out-of-contract lengths
  const int max_tokens = batch->max_seq_len;
  float* scores = reinterpret_cast<float*>(workspace);
  const int max_cand = std::max(mp - n_bos - n_eos, 0);
  const bool need_scores = max_cand > topk && topk > 0;   // else all or none are taken

  TopkArgs t{};
  t.scores = scores;
  t.seq_lens = batch->seq_lens;
  t.sel = sel;
  t.B = batch->batch;
  t.H_kv = kv->num_kv_heads;
  t.S_p = kv->page_size;
  t.score_stride = mp;
  t.max_tokens = max_tokens;
  t.topk = topk;
  t.n_bos = n_bos;
  t.n_eos = n_eos;
  t.k_tot = k_tot;
  t.levels = levels;
  t.rnd = rnd;

  // One block per (request, KV head) when there are enough of them to fill
  // the GPU (or the whole problem is tiny) and the candidate keys fit in LDS.
  const long long units = (long long)batch->batch * kv->num_kv_heads;
  if (fused_indexer_supported(kv->dtype, kv->head_dim_qk) && mp <= kFusedMaxPages &&
      (units >= device_cus() / 2 || units * mp <= 4096)) {
    ScoreArgs s{};
    s.q = q;
    s.cent = kv->centroids;
    s.pt = batch->page_table;
    s.seq_lens = batch->seq_lens;
    s.B = batch->batch;
    s.H_q = batch->num_q_heads;
    s.H_kv = kv->num_kv_heads;
    s.D = kv->head_dim_qk;
    s.S_p = kv->page_size;
    s.pt_stride = batch->max_pages_per_req;
    s.score_stride = mp;
    s.max_tokens = max_tokens;
    s.n_bos = n_bos;
    s.n_eos = n_eos;
    s.scores = scores;     // not read by the fused kernel
    if (update_completed && launch_completed_centroids(kv, batch, stream) != hipSuccess)
      return VX_ERR_HIP;
    return hip_status(launch_indexer_fused(kv->dtype, s, t, stream));
  }

  if (need_scores) {
    hipError_t e = launch_split_score(kv, batch, q, n_bos, n_eos, scores, update_completed, stream);
    if (e != hipSuccess) return VX_ERR_HIP;
  } else if (update_completed && launch_completed_centroids(kv, batch, stream) != hipSuccess) {
    return VX_ERR_HIP;
  }
  return hip_status(launch_topk(t, need_scores ? max_cand : 0, stream));
}

// The centroid kernel over the page each request's latest token completed.
hipError_t launch_completed_centroids(const vx_paged_kv* kv, const vx_batch* batch,
                                      hipStream_t stream) {
  CentroidArgs c{};
  c.k = kv->k_cache;
  c.cent = kv->centroids;
  c.ids = nullptr;
  c.pt = batch->page_table;
  c.seq_lens = batch->seq_lens;
  c.n_ids = batch->batch;
  c.H_kv = kv->num_kv_heads;
  c.S_p = kv->page_size;
  c.D = kv->head_dim_qk;
  c.pt_stride = batch->max_pages_per_req;
  c.max_tokens = batch->max_seq_len;
  return launch_centroid(kv->dtype, c, stream);
}

// The bounds kernel over the page each request's latest token completed.
hipError_t launch_completed_bounds(const vx_paged_kv* kv, const vx_batch* batch, void* bounds,
                                   hipStream_t stream) {
  BoundsArgs a{};
  a.k = kv->k_cache;
  a.bounds = bounds;
  a.ids = nullptr;
  a.pt = batch->page_table;
  a.seq_lens = batch->seq_lens;
  a.n_ids = batch->batch;
  a.H_kv = kv->num_kv_heads;
  a.S_p = kv->page_size;
  a.D = kv->head_dim_qk;
  a.pt_stride = batch->max_pages_per_req;
  a.max_tokens = batch->max_seq_len;
  return launch_page_bounds(kv->dtype, a, stream);
}

// The split indexer's scoring kernel alone: fp32 scores [B, H_kv, mp] into
// `scores`.  With update_completed it also writes the completed pages'
// centroids (in the kernel when each block's share of a page fits, else with
// the centroid kernel first).
// Candidates per block of a split scorer (K2, K9): about one 8-wave block
// per CU in all, each request's candidates cut into ceil(256 / B) chunks (a
// multiple of 8 pages, at least 32).
int split_score_chunk(const vx_batch* batch, int max_cand) {
  const int nblk = std::max(1, ceil_div(device_cus(), batch->batch));
  const int cpb = ceil_div(max_cand, nblk);
  return std::max(32, (cpb + 7) / 8 * 8);
}

hipError_t launch_split_score(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                              int32_t n_bos, int32_t n_eos, float* scores, bool update_completed,
                              hipStream_t stream) {
  const int mp = max_pages_eff(kv, batch);
  const int max_cand = std::max(mp - n_bos - n_eos, 0);
  {
    ScoreArgs s{};
    s.q = q;
    s.cent = kv->centroids;
    s.pt = batch->page_table;
    s.seq_lens = batch->seq_lens;
    s.scores = scores;
    s.B = batch->batch;
    s.H_q = batch->num_q_heads;
    s.H_kv = kv->num_kv_heads;
    s.D = kv->head_dim_qk;
    s.S_p = kv->page_size;
    s.pt_stride = batch->max_pages_per_req;
    s.score_stride = mp;
    s.max_tokens = batch->max_seq_len;
    s.n_bos = n_bos;
    s.n_eos = n_eos;
    const int cpb = split_score_chunk(batch, max_cand);
    s.cand_per_block = cpb;
    const int grid_x = ceil_div(max_cand, cpb);
    if (update_completed) {
      if (kv->page_size <= kMaxTileRows &&
          score_centroid_fits(kv->dtype, kv->head_dim_qk, kv->num_kv_heads, grid_x)) {
        s.k = kv->k_cache;
        s.cent_out = kv->centroids;
        s.update_completed = 1;
      } else {
        const hipError_t e = launch_completed_centroids(kv, batch, stream);
        if (e != hipSuccess) return e;
      }
    }
    return launch_score(kv->dtype, s, grid_x, stream);
  }
}

// The split scorer of the bound rule: fp32 scores [B, H_kv, mp] into `scores`.
hipError_t launch_split_bound_score(const vx_paged_kv* kv, const vx_batch* batch,
                                    const void* bounds, const void* q, int32_t n_bos,
                                    int32_t n_eos, float* scores, hipStream_t stream) {
  const int mp = max_pages_eff(kv, batch);
  const int max_cand = std::max(mp - n_bos - n_eos, 0);
  ScoreArgs s{};
  s.q = q;
  s.cent = bounds;
  s.pt = batch->page_table;
  s.seq_lens = batch->seq_lens;
  s.scores = scores;
  s.B = batch->batch;
  s.H_q = batch->num_q_heads;
  s.H_kv = kv->num_kv_heads;
  s.D = kv->head_dim_qk;
  s.S_p = kv->page_size;
  s.pt_stride = batch->max_pages_per_req;
  s.score_stride = mp;
  s.max_tokens = batch->max_seq_len;
  s.n_bos = n_bos;
  s.n_eos = n_eos;
  const int cpb = split_score_chunk(batch, max_cand);
  s.cand_per_block = cpb;
  return launch_bound_score(kv->dtype, s, ceil_div(max_cand, cpb), stream);
}

size_t step_ws_bytes(const vx_paged_kv* kv, const vx_batch* bt, int k_tot) {
  // the indexer's scores and the decode partials side by side (the decode
  // kernel may select from the scores while it writes partials)
  return align_up(score_ws_bytes(kv, bt)) + plan_decode(kv, bt, k_tot, true, device_cus()).ws_bytes();
}

// Dynamic LDS of the fused step kernel: staged page row and keys (one word
// per page each) and the selected list; plus its static arrays.
// LDS of an 8-wave attention block: per-wave partials (VALU form) or per-wave
// V staging / partials (MFMA form), whichever is larger.
size_t attention_lds_bytes(int D, int G) {
  const size_t att_valu = 8 * (size_t)G * (D + 2) * 4;
  const size_t att_mfma = 8 * std::max((size_t)16 * (2 * D + 32), (size_t)G * D * 4) + 2 * 8 * (size_t)G * 4;
  return std::max(att_valu, att_mfma);
}

size_t step_lds_bytes(int max_pages, int k_tot, int D, int G, int ordered_batch, bool bounds) {
  const size_t dyn = step_dynamic_lds(max_pages, k_tot, ordered_batch);
  const size_t stat = (size_t)D * 4 + kSelectLdsBytes + attention_lds_bytes(D, G) +
                      (bounds ? 32 : 16) * (size_t)D * 4 + 16;
  return dyn + stat;
}

// Host-side validation of vx_full_paged_decode / vx_sparse_decode_step
// (everything those calls check before their first HIP call).
vx_status full_decode_check(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                            float sm_scale, const void* out, const void* workspace,
                            size_t workspace_bytes) {
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if ((st = check_batch(kv, batch)) != VX_OK) return st;
  if (!(sm_scale > 0.f) || sm_scale == __builtin_inff()) return VX_ERR_INVALID_ARGUMENT;
  if (batch->batch == 0) return VX_OK;
  if (!q || !out || !kv->k_cache || (!kv->v_aliases_k && !kv->v_cache) || !batch->page_table ||
      !batch->seq_lens)
    return VX_ERR_INVALID_ARGUMENT;
  const DecodePlan p = plan_decode(kv, batch, max_pages_eff(kv, batch), false, device_cus());
  if (workspace_bytes < p.ws_bytes()) return VX_ERR_WORKSPACE_TOO_SMALL;
  if (p.ws_bytes() > 0 && !workspace) return VX_ERR_INVALID_ARGUMENT;
  return VX_OK;
}

// summary: the centroid table, or the key-bounds table of the bound rule.
vx_status step_check(const vx_paged_kv* kv, const vx_batch* batch, const void* summary,
                     const void* q, int32_t topk, int32_t n_bos, int32_t n_eos,
                     int32_t update_completed, float sm_scale, const int32_t* sel,
                     const void* out, const void* workspace, size_t workspace_bytes) {
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if ((st = check_batch(kv, batch)) != VX_OK) return st;
  if (topk < 0 || n_bos < 0 || n_eos < 1) return VX_ERR_INVALID_ARGUMENT;
  if ((long long)topk + n_bos + n_eos > 0x7fffffffLL) return VX_ERR_INVALID_ARGUMENT;
  if (update_completed != 0 && update_completed != 1) return VX_ERR_INVALID_ARGUMENT;
  if (!(sm_scale > 0.f) || sm_scale == __builtin_inff()) return VX_ERR_INVALID_ARGUMENT;
  if (batch->batch == 0) return VX_OK;
  if (!q || !sel || !out || !kv->k_cache || (!kv->v_aliases_k && !kv->v_cache) ||
      !summary || !batch->page_table || !batch->seq_lens)
    return VX_ERR_INVALID_ARGUMENT;
  if (max_pages_eff(kv, batch) > kMaxCandidates) return VX_ERR_UNSUPPORTED;
  if (workspace_bytes < step_ws_bytes(kv, batch, topk + n_bos + n_eos))
    return VX_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return VX_ERR_INVALID_ARGUMENT;
  return VX_OK;
}

// Workspace of vx_decode_layers: the larger of a step's and a dense call's.
size_t layers_ws_bytes(const vx_paged_kv* kv, const vx_batch* bt, int k_tot) {
  return std::max(step_ws_bytes(kv, bt, k_tot),
                  plan_decode(kv, bt, max_pages_eff(kv, bt), false, device_cus()).ws_bytes());
}

bool same_shape(const vx_paged_kv& a, const vx_paged_kv& b) {
  return a.dtype == b.dtype && a.page_size == b.page_size && a.num_kv_heads == b.num_kv_heads &&
         a.head_dim_qk == b.head_dim_qk && a.head_dim_v == b.head_dim_v &&
         a.v_aliases_k == b.v_aliases_k;
}

}  // namespace

extern "C" {

vx_status vx_centroid_update(const vx_paged_kv* kv, const int32_t* page_ids, int32_t n_ids,
                             hipStream_t stream) {
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if (n_ids < 0) return VX_ERR_INVALID_ARGUMENT;
  if (n_ids == 0) return VX_OK;
  if (!page_ids || !kv->k_cache || !kv->centroids) return VX_ERR_INVALID_ARGUMENT;
  CentroidArgs a{};
  a.k = kv->k_cache;
  a.cent = kv->centroids;
  a.ids = page_ids;
  a.pt = nullptr;
  a.seq_lens = nullptr;
  a.n_ids = n_ids;
  a.H_kv = kv->num_kv_heads;
  a.S_p = kv->page_size;
  a.D = kv->head_dim_qk;
  return hip_status(launch_centroid(kv->dtype, a, stream));
}

vx_status vx_append_kv(const vx_paged_kv* kv, const vx_batch* batch, const void* k_src,
                       const void* v_src, const int32_t* src_start, const int32_t* n_new,
                       int32_t n_src_rows, int32_t max_new, int32_t update_centroids,
                       hipStream_t stream) {
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if ((st = check_batch(kv, batch)) != VX_OK) return st;
  if (max_new < 0 || n_src_rows < 0) return VX_ERR_INVALID_ARGUMENT;
  if (update_centroids != 0 && update_centroids != 1) return VX_ERR_INVALID_ARGUMENT;
  if (batch->batch == 0 || max_new == 0) return VX_OK;
  if (!k_src || !src_start || !n_new || !kv->k_cache || !batch->page_table ||
      !batch->seq_lens || (update_centroids && !kv->centroids))
    return VX_ERR_INVALID_ARGUMENT;
  if (kv->v_aliases_k ? v_src != nullptr : (!v_src || !kv->v_cache))
    return VX_ERR_INVALID_ARGUMENT;
  AppendArgs a{};
  a.k = const_cast<void*>(kv->k_cache);
  a.v = kv->v_aliases_k ? nullptr : const_cast<void*>(kv->v_cache);
  a.cent = kv->centroids;
  a.k_src = k_src;
  a.v_src = v_src;
  a.src_start = src_start;
  a.n_new = n_new;
  a.pt = batch->page_table;
  a.seq_lens = batch->seq_lens;
  a.B = batch->batch;
  a.H_kv = kv->num_kv_heads;
  a.S_p = kv->page_size;
  a.Dq = kv->head_dim_qk;
  a.Dv = kv->head_dim_v;
  a.pt_stride = batch->max_pages_per_req;
  a.max_tokens = batch->max_seq_len;
  a.max_new = max_new;
  a.n_src_rows = n_src_rows;
  a.update = update_centroids;
  const long long pages = (long long)ceil_div(max_new, kv->page_size) + 1;
  if (pages > 0x7fffffffLL) return VX_ERR_INVALID_ARGUMENT;
  return hip_status(launch_append(kv->dtype, a, (int)pages, stream));
}

vx_status vx_bounds_update(const vx_paged_kv* kv, void* bounds, const int32_t* page_ids,
                           int32_t n_ids, hipStream_t stream) {
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if (n_ids < 0) return VX_ERR_INVALID_ARGUMENT;
  if (is_mla(kv)) return VX_ERR_UNSUPPORTED;
  if (n_ids == 0) return VX_OK;
  if (!bounds || !page_ids || !kv->k_cache) return VX_ERR_INVALID_ARGUMENT;
  BoundsArgs a{};
  a.k = kv->k_cache;
  a.bounds = bounds;
  a.ids = page_ids;
  a.n_ids = n_ids;
  a.H_kv = kv->num_kv_heads;
  a.S_p = kv->page_size;
  a.D = kv->head_dim_qk;
  return hip_status(launch_page_bounds(kv->dtype, a, stream));
}

vx_status vx_score_topk_bounds(const vx_paged_kv* kv, const vx_batch* batch, const void* bounds,
                               const void* q, int32_t topk, int32_t n_bos, int32_t n_eos,
                               int32_t* sel, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if ((st = check_batch(kv, batch)) != VX_OK) return st;
  if (topk < 0 || n_bos < 0 || n_eos < 1) return VX_ERR_INVALID_ARGUMENT;
  if ((long long)topk + n_bos + n_eos > 0x7fffffffLL) return VX_ERR_INVALID_ARGUMENT;
  if (is_mla(kv)) return VX_ERR_UNSUPPORTED;
  const int mp = max_pages_eff(kv, batch);
  if (mp > kMaxCandidates) return VX_ERR_UNSUPPORTED;
  if (batch->batch == 0) return VX_OK;
  if (!q || !sel || !bounds || !batch->page_table || !batch->seq_lens)
    return VX_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < score_ws_bytes(kv, batch)) return VX_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return VX_ERR_INVALID_ARGUMENT;
  const int k_tot = topk + n_bos + n_eos;
  const int max_cand = std::max(mp - n_bos - n_eos, 0);
  const bool need_scores = max_cand > topk && topk > 0;   // else all or none are taken
  float* scores = reinterpret_cast<float*>(workspace);
  TopkArgs t{};
  t.scores = scores;
  t.seq_lens = batch->seq_lens;
  t.sel = sel;
  t.B = batch->batch;
  t.H_kv = kv->num_kv_heads;
  t.S_p = kv->page_size;
  t.score_stride = mp;
  t.max_tokens = batch->max_seq_len;
  t.topk = topk;
  t.n_bos = n_bos;
  t.n_eos = n_eos;
  t.k_tot = k_tot;
  // as the centroid indexer: one block per (request, KV head) scoring and
  // selecting when such blocks fill the GPU, else the split scorer + K3
  const long long units = (long long)batch->batch * kv->num_kv_heads;
  if (fused_indexer_supported(kv->dtype, kv->head_dim_qk) && mp <= kFusedMaxPages &&
      (units >= device_cus() / 2 || units * mp <= 4096)) {
    ScoreArgs s{};
    s.q = q;
    s.cent = bounds;
    s.pt = batch->page_table;
    s.seq_lens = batch->seq_lens;
    s.B = batch->batch;
    s.H_q = batch->num_q_heads;
    s.H_kv = kv->num_kv_heads;
    s.D = kv->head_dim_qk;
    s.S_p = kv->page_size;
    s.pt_stride = batch->max_pages_per_req;
    s.score_stride = mp;
    s.max_tokens = batch->max_seq_len;
    s.n_bos = n_bos;
    s.n_eos = n_eos;
    s.scores = scores;     // not read by the fused kernel
    return hip_status(launch_indexer_fused(kv->dtype, s, t, stream, true));
  }
  if (need_scores &&
      launch_split_bound_score(kv, batch, bounds, q, n_bos, n_eos, scores, stream) != hipSuccess)
    return VX_ERR_HIP;
  return hip_status(launch_topk(t, need_scores ? max_cand : 0, stream));
}

vx_status vx_score_topk(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                        int32_t topk, int32_t n_bos, int32_t n_eos, int32_t* sel,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return score_topk_impl(kv, batch, q, topk, n_bos, n_eos, sel, workspace, workspace_bytes,
                         stream);
}

vx_status vx_score_topk_radix(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                              int32_t topk, int32_t n_bos, int32_t n_eos, int32_t levels,
                              const uint32_t* rnd, int32_t* sel, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if ((st = check_batch(kv, batch)) != VX_OK) return st;
  if (levels != 1 && levels != 2) return VX_ERR_INVALID_ARGUMENT;
  if (batch->batch > 0 && !rnd) return VX_ERR_INVALID_ARGUMENT;
  // the early stop works on candidates held in registers by 512-thread blocks
  if (max_pages_eff(kv, batch) - n_bos - n_eos > 4 * kSelRegChunks * 512) return VX_ERR_UNSUPPORTED;
  return score_topk_impl(kv, batch, q, topk, n_bos, n_eos, sel, workspace, workspace_bytes,
                         stream, false, levels, rnd);
}

vx_status vx_sparse_paged_decode(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                                 const int32_t* sel, int32_t k_tot, float sm_scale, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if ((st = check_batch(kv, batch)) != VX_OK) return st;
  if (k_tot < 1) return VX_ERR_INVALID_ARGUMENT;
  if (!(sm_scale > 0.f) || sm_scale == __builtin_inff()) return VX_ERR_INVALID_ARGUMENT;
  if (batch->batch == 0) return VX_OK;
  if (!q || !sel || !out || !kv->k_cache || (!kv->v_aliases_k && !kv->v_cache) ||
      !batch->page_table || !batch->seq_lens)
    return VX_ERR_INVALID_ARGUMENT;
  return run_decode(kv, batch, q, sel, k_tot, sm_scale, out, lse, workspace, workspace_bytes,
                    stream);
}

vx_status vx_full_paged_decode(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                               float sm_scale, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  const vx_status st = full_decode_check(kv, batch, q, sm_scale, out, workspace, workspace_bytes);
  if (st != VX_OK || batch->batch == 0) return st;
  return run_decode(kv, batch, q, nullptr, 0, sm_scale, out, lse, workspace, workspace_bytes,
                    stream);
}

}  // extern "C"

namespace {

// One decode step under the centroid rule or the bound rule (bounds: the
// key-bounds table [P, H_kv, 2, D]).
vx_status decode_step_impl(const vx_paged_kv* kv, const vx_batch* batch, bool use_bounds,
                           void* bounds, const void* q, int32_t topk, int32_t n_bos,
                           int32_t n_eos, int32_t update_completed, float sm_scale, int32_t* sel,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  void* summary = use_bounds ? bounds : kv->centroids;
  vx_status st = step_check(kv, batch, summary, q, topk, n_bos, n_eos, update_completed, sm_scale,
                            sel, out, workspace, workspace_bytes);
  if (st != VX_OK || batch->batch == 0) return st;
  if (use_bounds && is_mla(kv)) return VX_ERR_UNSUPPORTED;
  const int mp = max_pages_eff(kv, batch);
  const int k_tot = topk + n_bos + n_eos;
  const int G = batch->num_q_heads / kv->num_kv_heads;
  const long long units = (long long)batch->batch * kv->num_kv_heads;

  // One block per (request, KV head) runs the whole step when there are
  // enough of them to fill the GPU (or the problem is tiny) and its LDS fits.
  // With two or more units per CU: 4-wave blocks, two resident per CU, and
  // (up to 512 requests, where ranking them costs each block little) rows of
  // blocks taken longest request first.
  const int cus = device_cus();
  const int waves = units >= 2 * cus ? 4 : 8;
  const int ordered = (waves == 4 && batch->batch <= kMaxOrderedBatch) ? batch->batch : 0;
  if (!is_mla(kv) && decode_step_supported(kv->dtype, kv->head_dim_qk, G) &&
      (units >= cus / 2 || units * mp <= 4096) &&
      step_lds_bytes(mp, k_tot, kv->head_dim_qk, G, ordered, use_bounds) <= max_lds_per_block()) {
    StepArgs a{};
    DecodeArgs& d = a.d;
    d.q = q;
    d.k = kv->k_cache;
    d.v = kv->v_aliases_k ? kv->k_cache : kv->v_cache;
    d.pt = batch->page_table;
    d.seq_lens = batch->seq_lens;
    d.B = batch->batch;
    d.H_q = batch->num_q_heads;
    d.H_kv = kv->num_kv_heads;
    d.S_p = kv->page_size;
    d.pt_stride = batch->max_pages_per_req;
    d.k_tot = k_tot;
    d.max_tokens = batch->max_seq_len;
    d.pages_per_split = k_tot;
    d.n_split = 1;
    d.v_stride_tok = kv->v_aliases_k ? kv->head_dim_qk : kv->head_dim_v;
    d.scale_log2 = sm_scale * 1.4426950408889634f;
    d.out = out;
    d.lse = lse;
    ScoreArgs& sc = a.s;
    sc.q = q;
    sc.cent = summary;
    sc.pt = batch->page_table;
    sc.seq_lens = batch->seq_lens;
    sc.scores = reinterpret_cast<float*>(workspace);   // not read by the fused kernel
    sc.B = batch->batch;
    sc.H_q = batch->num_q_heads;
    sc.H_kv = kv->num_kv_heads;
    sc.D = kv->head_dim_qk;
    sc.S_p = kv->page_size;
    sc.pt_stride = batch->max_pages_per_req;
    sc.score_stride = mp;
    sc.max_tokens = batch->max_seq_len;
    sc.n_bos = n_bos;
    sc.n_eos = n_eos;
    a.sel = sel;
    a.cent = summary;
    a.topk = topk;
    a.n_bos = n_bos;
    a.n_eos = n_eos;
    a.k_tot = k_tot;
    a.max_pages = mp;
    a.update_completed = update_completed;
    a.longest_first = ordered > 0;
    return hip_status(
        launch_decode_step(kv->dtype, kv->head_dim_qk, G, waves, a, stream, use_bounds));
  }


  // Otherwise: the indexer (with the completed pages' centroids), then
  // attention.
  // The split scorer's scores are selected from inside the split decode
  // kernel, or the MLA decode kernel (no top-k launch), when its keys fit in
  // LDS beside the attention.
  const int max_cand = std::max(mp - n_bos - n_eos, 0);
  const bool split_scorer = !(fused_indexer_supported(kv->dtype, kv->head_dim_qk) &&
                              mp <= kFusedMaxPages &&
                              (units >= cus / 2 || units * mp <= 4096));
  const size_t sel_lds = (size_t)(round4(mp) + k_tot) * 4 + kSelectLdsBytes +
                         attention_lds_bytes(kv->head_dim_qk, G);
  const bool select_fits = is_mla(kv) ? mla_select_fits(mp, k_tot)
                                      : sel_lds <= max_lds_per_block();
  if (use_bounds) {
    // the completed pages' bounds first: the bound indexers do not write them
    if (update_completed && launch_completed_bounds(kv, batch, bounds, stream) != hipSuccess)
      return VX_ERR_HIP;
    if (split_scorer && max_cand > topk && topk > 0 && select_fits) {
      float* scores = reinterpret_cast<float*>(workspace);
      if (launch_split_bound_score(kv, batch, bounds, q, n_bos, n_eos, scores, stream) !=
          hipSuccess)
        return VX_ERR_HIP;
      SelectInDecode fs{scores, sel, mp, topk, n_bos, n_eos, align_up(score_ws_bytes(kv, batch))};
      return run_decode(kv, batch, q, nullptr, k_tot, sm_scale, out, lse, workspace,
                        workspace_bytes, stream, &fs);
    }
    st = vx_score_topk_bounds(kv, batch, bounds, q, topk, n_bos, n_eos, sel, workspace,
                              workspace_bytes, stream);
    if (st != VX_OK) return st;
    return run_decode(kv, batch, q, sel, k_tot, sm_scale, out, lse, workspace, workspace_bytes,
                      stream);
  }
  if (split_scorer && max_cand > topk && topk > 0 && select_fits) {
    float* scores = reinterpret_cast<float*>(workspace);
    if (launch_split_score(kv, batch, q, n_bos, n_eos, scores, update_completed != 0, stream) !=
        hipSuccess)
      return VX_ERR_HIP;
    SelectInDecode fs{scores, sel, mp, topk, n_bos, n_eos, align_up(score_ws_bytes(kv, batch))};
    return run_decode(kv, batch, q, nullptr, k_tot, sm_scale, out, lse, workspace,
                      workspace_bytes, stream, &fs);
  }
  st = score_topk_impl(kv, batch, q, topk, n_bos, n_eos, sel, workspace, workspace_bytes, stream,
                       update_completed != 0);
  if (st != VX_OK) return st;
  return run_decode(kv, batch, q, sel, k_tot, sm_scale, out, lse, workspace, workspace_bytes,
                    stream);
}

}  // namespace

extern "C" {

vx_status vx_sparse_decode_step(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                                int32_t topk, int32_t n_bos, int32_t n_eos,
                                int32_t update_completed, float sm_scale, int32_t* sel,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return decode_step_impl(kv, batch, false, nullptr, q, topk, n_bos, n_eos, update_completed, sm_scale,
                          sel, out, lse, workspace, workspace_bytes, stream);
}

vx_status vx_sparse_decode_step_bounds(const vx_paged_kv* kv, const vx_batch* batch,
                                       void* bounds, const void* q, int32_t topk, int32_t n_bos,
                                       int32_t n_eos, int32_t update_completed, float sm_scale,
                                       int32_t* sel, void* out, float* lse, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  return decode_step_impl(kv, batch, true, bounds, q, topk, n_bos, n_eos, update_completed, sm_scale,
                          sel, out, lse, workspace, workspace_bytes, stream);
}

vx_status vx_decode_layers(const vx_paged_kv* kv, const vx_batch* batch, const void* const* q,
                           int32_t n_layers, const uint8_t* dense, int32_t topk, int32_t n_bos,
                           int32_t n_eos, int32_t update_completed, float sm_scale,
                           int32_t* const* sel, void* const* out, float* const* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (n_layers < 0) return VX_ERR_INVALID_ARGUMENT;
  if (n_layers == 0) return VX_OK;
  if (!kv || !q || !out) return VX_ERR_INVALID_ARGUMENT;
  // every layer is checked before the first launch
  for (int l = 0; l < n_layers; ++l) {
    if (!same_shape(kv[l], kv[0])) return VX_ERR_INVALID_ARGUMENT;
    const bool is_dense = dense && dense[l];
    vx_status st;
    if (is_dense) {
      st = full_decode_check(&kv[l], batch, q[l], sm_scale, out[l], workspace, workspace_bytes);
    } else {
      if (!sel) return VX_ERR_INVALID_ARGUMENT;
      st = step_check(&kv[l], batch, kv[l].centroids, q[l], topk, n_bos, n_eos, update_completed,
                      sm_scale, sel[l], out[l], workspace, workspace_bytes);
    }
    if (st != VX_OK) return st;
  }
  for (int l = 0; l < n_layers; ++l) {
    float* lse_l = lse ? lse[l] : nullptr;
    const vx_status st =
        dense && dense[l]
            ? vx_full_paged_decode(&kv[l], batch, q[l], sm_scale, out[l], lse_l, workspace,
                                   workspace_bytes, stream)
            : vx_sparse_decode_step(&kv[l], batch, q[l], topk, n_bos, n_eos, update_completed,
                                    sm_scale, sel[l], out[l], lse_l, workspace, workspace_bytes,
                                    stream);
    if (st != VX_OK) return st;
  }
  return VX_OK;
}

vx_status vx_workspace_size(int32_t op, const vx_paged_kv* kv, const vx_batch* batch,
                            int32_t k_tot, size_t* bytes) {
  if (!bytes) return VX_ERR_INVALID_ARGUMENT;
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if ((st = check_batch(kv, batch)) != VX_OK) return st;
  switch (op) {
    case VX_OP_SCORE_TOPK:
      if (max_pages_eff(kv, batch) > kMaxCandidates) return VX_ERR_UNSUPPORTED;
      *bytes = score_ws_bytes(kv, batch);
      return VX_OK;
    case VX_OP_SPARSE_DECODE:
      if (k_tot < 1) return VX_ERR_INVALID_ARGUMENT;
      *bytes = plan_decode(kv, batch, k_tot, true, device_cus()).ws_bytes();
      return VX_OK;
    case VX_OP_FULL_DECODE:
      *bytes = plan_decode(kv, batch, max_pages_eff(kv, batch), false, device_cus()).ws_bytes();
      return VX_OK;
    case VX_OP_DECODE_STEP:
      if (max_pages_eff(kv, batch) > kMaxCandidates) return VX_ERR_UNSUPPORTED;
      if (k_tot < 1) return VX_ERR_INVALID_ARGUMENT;
      *bytes = step_ws_bytes(kv, batch, k_tot);
      return VX_OK;
    case VX_OP_DECODE_LAYERS:
      if (max_pages_eff(kv, batch) > kMaxCandidates) return VX_ERR_UNSUPPORTED;
      if (k_tot < 1) return VX_ERR_INVALID_ARGUMENT;
      *bytes = layers_ws_bytes(kv, batch, k_tot);
      return VX_OK;
  }
  return VX_ERR_INVALID_ARGUMENT;
}

vx_status vx_plan_decode(int32_t op, const vx_paged_kv* kv, const vx_batch* batch, int32_t k_tot,
                         int32_t num_cus, int32_t pages_per_split, vx_decode_plan* plan) {
  if (!plan) return VX_ERR_INVALID_ARGUMENT;
  vx_status st = check_kv(kv);
  if (st != VX_OK) return st;
  if ((st = check_batch(kv, batch)) != VX_OK) return st;
  if (op != VX_OP_SPARSE_DECODE && op != VX_OP_FULL_DECODE) return VX_ERR_INVALID_ARGUMENT;
  if (num_cus < 0 || pages_per_split < 0) return VX_ERR_INVALID_ARGUMENT;
  const bool sparse = op == VX_OP_SPARSE_DECODE;
  if (sparse && k_tot < 1) return VX_ERR_INVALID_ARGUMENT;
  const int cus = num_cus > 0 ? num_cus : device_cus();
  const DecodePlan p = plan_decode(kv, batch, decode_pages(kv, batch, sparse, k_tot), sparse, cus,
                                   pages_per_split);
  *plan = vx_decode_plan{};
  plan->op = op;
  plan->num_cus = cus;
  plan->pages_per_split = p.pages_per_split;
  plan->n_split = p.n_split;
  plan->work_list = p.work_list ? 1 : 0;
  plan->blocks = p.blocks;
  plan->workspace_bytes = p.ws_bytes();
  return VX_OK;
}

vx_status vx_paged_decode_planned(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                                  const int32_t* sel, int32_t k_tot, const vx_decode_plan* plan,
                                  float sm_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (!plan) return VX_ERR_INVALID_ARGUMENT;
  const bool sparse = plan->op == VX_OP_SPARSE_DECODE;
  vx_decode_plan again{};
  if (plan->num_cus < 1) return VX_ERR_INVALID_ARGUMENT;
  const vx_status st = vx_plan_decode(plan->op, kv, batch, k_tot, plan->num_cus,
                                      plan->pages_per_split, &again);
  if (st != VX_OK) return st;
  // the plan must be one vx_plan_decode made for these shapes
  if (again.num_cus != plan->num_cus || again.pages_per_split != plan->pages_per_split ||
      again.n_split != plan->n_split || again.work_list != plan->work_list ||
      again.blocks != plan->blocks || again.workspace_bytes != plan->workspace_bytes ||
      (sparse != (sel != nullptr)))
    return VX_ERR_INVALID_ARGUMENT;
  if (!(sm_scale > 0.f) || sm_scale == __builtin_inff()) return VX_ERR_INVALID_ARGUMENT;
  if (batch->batch == 0) return VX_OK;
  if (!q || !out || !kv->k_cache || (!kv->v_aliases_k && !kv->v_cache) || !batch->page_table ||
      !batch->seq_lens)
    return VX_ERR_INVALID_ARGUMENT;
  DecodePlan p;
  p.pages_per_split = plan->pages_per_split;
  p.n_split = plan->n_split;
  p.work_list = plan->work_list != 0;
  p.blocks = plan->blocks;
  if (p.n_split > 1) {
    const size_t rows = (size_t)batch->batch * batch->num_q_heads * p.n_split;
    p.part_o_bytes = align_up(rows * kv->head_dim_v * sizeof(float));
    p.part_ml_bytes = align_up(rows * 2 * sizeof(float));
  }
  return run_decode(kv, batch, q, sel, sparse ? k_tot : 0, sm_scale, out, lse, workspace,
                    workspace_bytes, stream, nullptr, &p);
}

const char* vx_status_string(vx_status status) {
  switch (status) {
    case VX_OK: return "ok";
    case VX_ERR_INVALID_ARGUMENT: return "invalid argument";
    case VX_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case VX_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case VX_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t vx_version(void) { return 100; }

}  // extern "C"
