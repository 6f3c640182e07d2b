// Internal interface between the C-ABI layer (vx_api.cpp) and the kernel
// translation units.  Launchers return hipErrorInvalidValue when no kernel
// instance matches the shape; the API layer validates shapes first.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace vx {

// Kernel argument blocks are passed by value.

struct CentroidArgs {
  const void* k;          // [P, H_kv, S_p, D]
  void* cent;             // [P, H_kv, D]
  const int32_t* ids;     // [n_ids] physical pages, or nullptr: one block row per request,
                          // updating the page its latest token completed (if any)
  const int32_t* pt;      // [B, pt_stride] (ids == nullptr)
  const int32_t* seq_lens;
  int32_t n_ids, H_kv, S_p, D;
  int32_t pt_stride, max_tokens;
};

// 16-byte chunks of keys a thread keeps in registers during a selection; the
// lossy radix top-k stops early only for candidates held that way.
constexpr int kSelRegChunks = 4;

// Most rows of a page-head tile whose centroid a longer kernel computes.
constexpr int kMaxTileRows = 64;

struct ScoreArgs {
  const void* q;          // [B, H_q, D]
  const void* cent;       // [P, H_kv, D]
  const int32_t* pt;      // [B, pt_stride]
  const int32_t* seq_lens;
  float* scores;          // [B, H_kv, score_stride], candidate-indexed
  int32_t B, H_q, H_kv, D, S_p, pt_stride, score_stride, max_tokens;
  int32_t n_bos, n_eos;
  int32_t cand_per_block;
  // split scorer only: when set, the blocks of each request also write the
  // centroid rows of the page its latest token completed, each block a share
  // of the (KV head, segment) units (that page is reserved, never a candidate)
  const void* k;          // [P, H_kv, S_p, D]
  void* cent_out;         // the centroid table, written
  int32_t update_completed;
  // split scorer only: when set, a block's scores are gathered in LDS and
  // written as whole rows at the end (set by the launcher when they fit)
  int32_t stage_scores;
};

struct TopkArgs {
  const float* scores;    // [B, H_kv, score_stride]
  const int32_t* seq_lens;
  int32_t* sel;           // [B, H_kv, k_tot]
  int32_t B, H_kv, S_p, score_stride, max_tokens;
  int32_t topk, n_bos, n_eos, k_tot;
  // lossy radix top-k: histogram levels before the early stop (0: exact) and
  // one random word per (request, KV head) [B, H_kv]
  int32_t levels;
  const uint32_t* rnd;
};

struct DecodeArgs {
  const void* q;          // [B, H_q, D_qk]
  const void* k;          // [P, H_kv, S_p, D_qk]
  const void* v;          // [P, H_kv, S_p, D_v] (may alias k)
  const int32_t* pt;      // [B, pt_stride]
  const int32_t* seq_lens;
  const int32_t* sel;     // [B, H_kv, k_tot] or nullptr for every page
  float* part_o;          // [B, H_q, n_split, D_v] fp32 (split mode)
  float* part_ml;         // [B, H_q, n_split, 2]  (max in log2 units, sum)
  void* out;              // [B, H_q, D_v] (direct mode)
  float* lse;             // [B, H_q] or nullptr (direct mode)
  int32_t B, H_q, H_kv, S_p, pt_stride, k_tot, max_tokens;
  int32_t pages_per_split, n_split;
  // work list (dense calls): the launch's blocks walk (request, chunk of
  // pages_per_split pages, KV head) items in turn instead of one block per
  // (split, KV head, request); chunk c of a request is its split c
  int32_t work_list;
  int32_t v_stride_tok;   // elements between consecutive tokens of V (D_qk when aliased)
  float scale_log2;       // sm_scale * log2(e)
  // Selection in the decode kernel (scores != nullptr): every split block of
  // a (request, KV head) selects its pages from the indexer's scores itself;
  // split 0 writes the row of sel_out.
  const float* scores;    // [B, H_kv, score_stride], candidate-indexed
  int32_t* sel_out;       // [B, H_kv, k_tot]
  int32_t score_stride, topk, n_bos, n_eos;
};

// One fused decode step per (request, KV head) block: completed-page
// centroid, indexer and attention over the selection.
// Upper bound of the LDS one block's page selection uses (static).
constexpr size_t kSelectLdsBytes = 12 * 1024;

struct StepArgs {
  DecodeArgs d;           // attention (n_split = 1; sel unused)
  ScoreArgs s;            // indexer (scores unused)
  int32_t* sel;           // [B, H_kv, k_tot]
  void* cent;             // centroid table, written for completed pages
  int32_t topk, n_bos, n_eos, k_tot;
  int32_t max_pages;      // page-table entries staged in LDS per request
  int32_t update_completed;
  int32_t longest_first;  // block row r takes the r-th longest request
};

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  void* out;
  float* lse;
  int32_t B, H_q, n_split, D_v;
  // when set, row (b, .) merges only the splits request b has:
  // ceil(ceil(seq / S_p) / pages_per_split), at least 1 (the others were
  // never written)
  const int32_t* seq_lens;
  int32_t S_p, pages_per_split, max_tokens;
};

hipError_t launch_centroid(int dtype, const CentroidArgs& a, hipStream_t s);

struct AppendArgs {
  void* k;                // [P, H_kv, S_p, Dq]
  void* v;                // [P, H_kv, S_p, Dv], or nullptr when V is the leading part of K
  void* cent;             // [P, H_kv, Dq]
  const void* k_src;      // [n_src_rows, H_kv, Dq]
  const void* v_src;      // [n_src_rows, H_kv, Dv] (v != nullptr)
  const int32_t* src_start;   // [B] source row of request b's first new token
  const int32_t* n_new;       // [B] new tokens of request b (its last ones)
  const int32_t* pt;          // [B, pt_stride]
  const int32_t* seq_lens;    // [B] lengths after the write
  int32_t B, H_kv, S_p, Dq, Dv, pt_stride, max_tokens, max_new, n_src_rows, update;
};
// grid x: pages a request's write can touch, ceil(max_new / S_p) + 1
hipError_t launch_append(int dtype, const AppendArgs& a, int pages_per_req, hipStream_t s);
hipError_t launch_score(int dtype, const ScoreArgs& a, int grid_x, hipStream_t s);
// Whether a split-scorer launch of grid_x blocks per request can also write
// the completed pages' centroids (each block's share of the page's rows fits).
bool score_centroid_fits(int dtype, int D, int H_kv, int grid_x);
hipError_t launch_topk(const TopkArgs& a, int max_cand, hipStream_t s);
// Page-bound (Quest) rule: the summary rows [P, H_kv, 2, D] (minimum row,
// then maximum row) of listed pages, and the split scorer of criticality,
// whose ScoreArgs::cent points at that summary table.
struct BoundsArgs {
  const void* k;          // [P, H_kv, S_p, D]
  void* bounds;           // [P, H_kv, 2, D]
  const int32_t* ids;     // [n_ids] physical pages, or nullptr: one block per request,
                          // for the page its latest token completed (if any)
  const int32_t* pt;      // [B, pt_stride] (ids == nullptr)
  const int32_t* seq_lens;
  int32_t n_ids, H_kv, S_p, D;
  int32_t pt_stride, max_tokens;
};
hipError_t launch_page_bounds(int dtype, const BoundsArgs& a, hipStream_t s);
hipError_t launch_bound_score(int dtype, const ScoreArgs& a, int grid_x, hipStream_t s);
// One block per (request, KV head) scores and selects (rows of <= 64 lanes);
// with bounds, a.cent is the key-bounds table and the score Quest's bound.
bool fused_indexer_supported(int dtype, int D);
hipError_t launch_indexer_fused(int dtype, const ScoreArgs& a, const TopkArgs& t, hipStream_t s,
                                bool bounds = false);
// D = D_qk = D_v for this path; G = H_q / H_kv.
hipError_t launch_decode_split(int dtype, int D, int G, const DecodeArgs& a, hipStream_t s);
// The dense work list: `blocks` persistent blocks over every (request,
// chunk, KV head) item (a.work_list set, a.sel and a.scores null).  LDS
// bound on B: decode_items_max_batch().
hipError_t launch_decode_items(int dtype, int D, int G, const DecodeArgs& a, int blocks,
                               hipStream_t s);
int decode_items_max_batch();
hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t s);
// Whether the MLA decode can select its pages itself (scores given) for this
// score row length and selection size.
bool mla_select_fits(int score_stride, int k_tot);
int mla_max_pages_per_split();
hipError_t launch_combine(int dtype, const CombineArgs& a, hipStream_t s);
bool decode_step_supported(int dtype, int D, int G);
// Entries rounded up to a multiple of 4 (16-byte aligned LDS arrays).
constexpr int round4(int n) { return (n + 3) & ~3; }
// Dynamic LDS bytes of a fused step block; ordered_batch = B when block rows
// go to requests longest first, else 0.
size_t step_dynamic_lds(int max_pages, int k_tot, int ordered_batch);
// waves: 4 or 8 per block (one block per (request, KV head)).  bounds: the
// key-bounds rule (a.s.cent and a.cent are the key-bounds table).
hipError_t launch_decode_step(int dtype, int D, int G, int waves, const StepArgs& a,
                              hipStream_t s, bool bounds = false);

}  // namespace vx
