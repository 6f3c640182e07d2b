/*
 * vx.h - C ABI of libvx: centroid-indexed block-top-k sparse decode attention
 * over a paged KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method (Vortex, "Efficient and Programmable Sparse Attention Serving
 * for AI Agents"; article section "A dual-stage programmable abstraction",
 * and the vortex_torch README section "Quick Example: Custom Sparse
 * Attention") runs in two stages:
 *   - query-independent: when a KV page fills up, the mean of its keys (its
 *     centroid) is stored in a per-page centroid table      -> vx_centroid_update
 *   - query-dependent, every decode step: the query is averaged over the
 *     query heads of each KV head, dotted with the centroids of the
 *     request's pages, and the top-k pages (plus reserved first and last
 *     pages) are chosen                                      -> vx_score_topk
 *     then exact attention runs over only those pages        -> vx_sparse_paged_decode
 * Full attention over every page is the baseline the method is measured
 * against, and what a skipped layer runs (README, "Using Your Sparse
 * Attention with SGLang")                                    -> vx_full_paged_decode
 * Around them: the whole step fused (vx_sparse_decode_step), every layer of
 * a step in one capturable call (vx_decode_layers), the write path with
 * centroids on completion (vx_append_kv), the lossy radix indexer
 * (vx_score_topk_radix) and a second summary rule, Quest's key bounds
 * (vx_bounds_update, vx_score_topk_bounds, vx_sparse_decode_step_bounds).
 *
 * Conventions shared by every call
 *   Pointers.   Every buffer pointer is a DEVICE pointer unless marked
 *               "host".  Structs are read on the host during the call
 *               only and are not retained.
 *   Ownership.  The caller owns every buffer.  The library never
 *               allocates or frees device memory and keeps no state across
 *               calls except cached device properties (compute-unit count,
 *               LDS per block) and, for vx_sparse_decode_step_static only,
 *               a static scratch array per GPU; calls are reentrant
 *               (overlapping static-step calls on one GPU share that
 *               scratch and race).
 *   Streams.    Work is enqueued on `stream` (NULL = the null stream);
 *               calls return after launch, never synchronise the host.
 *   Errors.     Arguments are validated on the host before any HIP call;
 *               on error nothing is launched and a vx_status is returned.
 *               A failed launch returns VX_ERR_HIP.  Device-side contract
 *               violations (page ids >= num_pages, seq_lens above
 *               max_seq_len or below 1, a page table that does not cover a
 *               sequence) are undefined behaviour.
 *   Determinism. Identical inputs give bit-identical outputs (fixed plan
 *               per shape, no floating-point atomics).
 *
 * Data layout in HBM (all row-major, contiguous):
 *   K pool       [P, H_kv, S_p, D_qk]   dtype     (head-major pages)
 *   V pool       [P, H_kv, S_p, D_v]    dtype     (or aliased into K, MLA)
 *   centroids    [P, H_kv, D_qk]        dtype     one row per page and KV head
 *   page_table   [B, max_pages] int32   physical page of logical page p
 *   seq_lens     [B] int32              tokens incl. the one being decoded
 *   q            [B, H_q, D_qk]         dtype     query head j uses KV head j / G
 *   sel          [B, H_kv, k_tot] int32 logical pages, ascending, -1 padded
 *   out          [B, H_q, D_v]          dtype
 *   lse          [B, H_q] float32       natural log of the softmax denominator
 *
 * Supported shapes (others return VX_ERR_UNSUPPORTED):
 *   dtype VX_F32 or VX_BF16, page_size 16 or 64, H_q = G * H_kv with
 *   G in {1, 2, 4, 8} for D_qk = D_v in {64, 128};
 *   MLA: VX_BF16, D_qk = 576, D_v = 512, v_aliases_k = 1, H_kv = 1,
 *   page_size 64, H_q <= 32.
 */
#ifndef VX_H
#define VX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VX_OK = 0,
  VX_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, negative size, inconsistent shape */
  VX_ERR_UNSUPPORTED = 2,        /* valid but not a shape/dtype this build handles  */
  VX_ERR_WORKSPACE_TOO_SMALL = 3,
  VX_ERR_HIP = 4                 /* a HIP runtime call or launch failed             */
} vx_status;

typedef enum { VX_F32 = 0, VX_BF16 = 1 } vx_dtype;

/* Operation ids for vx_workspace_size. */
typedef enum {
  VX_OP_SCORE_TOPK = 0,
  VX_OP_SPARSE_DECODE = 1,
  VX_OP_FULL_DECODE = 2,
  VX_OP_DECODE_STEP = 3,
  VX_OP_DECODE_LAYERS = 4
} vx_op;

/* The paged KV cache and its named centroid cache (the per-page summary
 * table the cache stage writes; README "Quick Example": one head_dim-wide
 * row per page). */
typedef struct {
  int32_t dtype;          /* vx_dtype of K, V, centroids, q and out           */
  int32_t num_pages;      /* P, physical pages in the pool                     */
  int32_t page_size;      /* S_p, tokens per page: 16 or 64                    */
  int32_t num_kv_heads;   /* H_kv                                              */
  int32_t head_dim_qk;    /* D_qk                                              */
  int32_t head_dim_v;     /* D_v                                               */
  int32_t v_aliases_k;    /* 1: V is K[..., :D_v] and v_cache must be NULL     */
  int32_t reserved_;      /* must be 0                                         */
  const void* k_cache;    /* [P, H_kv, S_p, D_qk]                              */
  const void* v_cache;    /* [P, H_kv, S_p, D_v], or NULL when v_aliases_k     */
  void* centroids;        /* [P, H_kv, D_qk]                                   */
} vx_paged_kv;

/* One decode batch: the page-table metadata of the article's section "The
 * friction of paged memory" (a logical sequence spread over physical pages). */
typedef struct {
  int32_t batch;              /* B; 0 is allowed: nothing is read or launched
                                 and the device pointers may be NULL            */
  int32_t num_q_heads;        /* H_q, a multiple of H_kv                         */
  int32_t max_pages_per_req;  /* row stride of page_table                        */
  int32_t max_seq_len;        /* host-side bound on every seq_lens[b], used to
                                 plan the launch; max_pages_per_req * page_size
                                 must be >= max_seq_len                         */
  const int32_t* page_table;  /* [B, max_pages_per_req]                          */
  const int32_t* seq_lens;    /* [B], each in [1, max_seq_len]                   */
} vx_batch;

/* Query-independent stage (article, "A dual-stage programmable
 * abstraction": centroids computed while the cache is built, stored and
 * reused across steps; README "Quick Example": CMean over the keys of a
 * page, run only when a page is finished).
 *
 * For each listed physical page p and KV head h:
 *   centroids[p, h, :] = round_to_dtype( (1/S_p) * sum_t K[p, h, t, :] )
 * summed in fp32 and rounded once (round to nearest even).
 *   page_ids  device int32 [n_ids], each in [0, num_pages); every listed page
 *             must hold S_p valid tokens.  Duplicates are allowed.
 *   n_ids     >= 0; 0 launches nothing.
 * Only kv->k_cache and kv->centroids are touched. */
vx_status vx_centroid_update(const vx_paged_kv* kv, const int32_t* page_ids,
                             int32_t n_ids, hipStream_t stream);

/* The write path beside the decode step: new tokens' K/V rows into their
 * pages, with the centroid of every page the write fills (article, "A
 * dual-stage programmable abstraction": summaries are made while the cache is
 * built; README "Quick Example": a page's centroid once it is full).  One
 * token per request is the decode append; many are a prefill write.
 *
 * For request b with L = seq_lens[b] (the length after the write) and
 * n = min(n_new[b], max_new, L) new tokens at positions L-n .. L-1:
 *   K[page_table[b, pos / S_p], h, pos % S_p, :] = k_src[src_start[b] + pos - (L-n), h, :]
 *   V likewise from v_src (skipped when v_aliases_k)
 * and, with update_centroids, for every page p whose last position lies in
 * [L-n, L): centroids[page_table[b, p], h, :] as vx_centroid_update writes it
 * (the same bits).  Rows outside [0, n_src_rows) are not read or written.
 *   k_src      device [n_src_rows, H_kv, D_qk], dtype
 *   v_src      device [n_src_rows, H_kv, D_v], dtype; NULL when v_aliases_k
 *   src_start  device int32 [B]; n_new device int32 [B]
 *   max_new    host bound on n_new (sets the launch); 0 launches nothing
 *   update_centroids  0 or 1
 * kv->k_cache and kv->v_cache are written (the rows above only), as is the
 * centroid table (its rows above only). */
vx_status vx_append_kv(const vx_paged_kv* kv, const vx_batch* batch, const void* k_src,
                       const void* v_src, const int32_t* src_start, const int32_t* n_new,
                       int32_t n_src_rows, int32_t max_new, int32_t update_centroids,
                       hipStream_t stream);

/* Query-dependent indexer (README "Quick Example": mean of the query over
 * heads, GeMV against the centroids, topK into the page index structure;
 * README "Using Your Sparse Attention with SGLang": top-k value and the
 * reserved BOS / EOS page counts).
 *
 * For request b with n_b = ceil(seq_lens[b] / S_p) logical pages and KV
 * head h:
 *   qbar      = mean of q[b, h*G : (h+1)*G, :]           (fp32)
 *   reserved  = pages [0, n_bos) and [n_b - n_eos, n_b)
 *   candidates= pages [n_bos, n_b - n_eos)   (all full pages, need centroids)
 *   score[p]  = dot(qbar, centroids[page_table[b, p], h, :])  (fp32)
 *   top       = the topk candidates of largest score, equal scores going
 *               to the lower logical page (all candidates if fewer)
 *   sel[b, h, :] = reserved U top, ascending, then -1 up to k_tot
 * with k_tot = topk + n_bos + n_eos.
 *   q          device [B, H_q, D_qk], dtype
 *   topk >= 0, n_bos >= 0, n_eos >= 1 (the last page may be partial and has
 *              no centroid, so it must be reserved)
 *   sel        device int32 [B, H_kv, k_tot], written completely
 *   workspace  device scratch of at least
 *              vx_workspace_size(VX_OP_SCORE_TOPK, ...) bytes; contents on
 *              entry do not matter.
 * Candidates per request are limited to 16384 pages (VX_ERR_UNSUPPORTED). */
vx_status vx_score_topk(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                        int32_t topk, int32_t n_bos, int32_t n_eos, int32_t* sel,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Lossy indexer: the "stochastic radix top-k" with early termination (Vortex
 * article, section "A dual-stage programmable abstraction": a lossy radix
 * top-k that stops early, trading a little exactness for indexing speed).
 * The pages give no further detail; this library's reading:
 *   keys      = order-preserving uint32 of the fp32 scores of vx_score_topk
 *               (-0 and +0 equal)
 *   level 0   = histogram of the top 10 key bits; level 1 (levels == 2)
 *               splits the boundary bin of level 0 by the next 10 bits.
 *   After `levels` levels, with A candidates in bins above the boundary bin
 *   and N in it (A < topk <= A + N): every candidate above it is taken, and
 *   of the bin's members, listed in ascending page order with ranks
 *   0 .. N-1, those with (rank - rnd[b, h] mod N) mod N < topk - A.  When
 *   the boundary bin is taken whole (A + N == topk) the result equals
 *   vx_score_topk's.  Reserved pages, output order and padding as there.
 *   levels     1 or 2 (VX_ERR_INVALID_ARGUMENT otherwise)
 *   rnd        device uint32 [B, H_kv]: one random word per (request, KV
 *              head), drawn by the caller (the "stochastic" part); read only
 * Candidates per request are limited to 8192 pages (VX_ERR_UNSUPPORTED).
 * Other arguments, workspace and errors as vx_score_topk. */
vx_status vx_score_topk_radix(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                              int32_t topk, int32_t n_bos, int32_t n_eos, int32_t levels,
                              const uint32_t* rnd, int32_t* sel, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* A second page-summary rule through the same pipeline: Quest's key bounds.
 * The Vortex article (section "Speedups that scale to 229B parameters")
 * names Quest as the other algorithm it serves without stating its rule;
 * the rule as the Quest paper gives it (Tang et al., ICML 2024, section 3):
 * a page is summarised by the per-channel minimum and maximum of its keys,
 * and its criticality for a query q is sum_i max(q_i * min_i, q_i * max_i),
 * an upper bound on q . k over the page.
 *
 * vx_bounds_update: for each listed physical page p and KV head h,
 *   bounds[p, h, 0, :] = min over t of K[p, h, t, :]
 *   bounds[p, h, 1, :] = max over t of K[p, h, t, :]     (exact, KV dtype)
 *   bounds     device [P, H_kv, 2, D_qk], dtype; only the listed rows written
 *   page_ids   device int32 [n_ids], each in [0, num_pages), full pages;
 *              n_ids >= 0 (0 launches nothing)
 *
 * vx_score_topk_bounds: vx_score_topk with the criticality above in place of
 * the centroid score (q is the group mean of the KV head's query heads, as
 * there); reserved pages, ties, order, padding, workspace
 * (VX_OP_SCORE_TOPK's size) and errors as vx_score_topk.  The selection
 * feeds vx_sparse_paged_decode unchanged.
 * Both: D_qk in {64, 128} (MLA shapes return VX_ERR_UNSUPPORTED). */
vx_status vx_bounds_update(const vx_paged_kv* kv, void* bounds, const int32_t* page_ids,
                           int32_t n_ids, hipStream_t stream);
vx_status vx_score_topk_bounds(const vx_paged_kv* kv, const vx_batch* batch, const void* bounds,
                               const void* q, int32_t topk, int32_t n_bos, int32_t n_eos,
                               int32_t* sel, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Sparse attention over the selected pages (article, "A dual-stage
 * programmable abstraction": after selecting the top-k blocks the system
 * performs the actual attention on them).
 *
 * For query head j of request b (KV head h = j / G), over the tokens
 * {(p, t) : p in sel[b, h, :], p >= 0, t < S_p, p*S_p + t < seq_lens[b]}:
 *   l_t = sm_scale * dot(q[b, j], K[page_table[b, p], h, t])
 *   out[b, j] = sum_t softmax(l)_t * V[page_table[b, p], h, t]
 *   lse[b, j] = log(sum_t exp(l_t))
 * Split-K flash decoding: each (request, KV head) is cut into splits of
 * whole pages whose fp32 partials (o, max, sum) are merged exactly.
 *   sel        device int32 [B, H_kv, k_tot] as written by vx_score_topk:
 *              valid entries are a prefix; the first negative entry ends it
 *   out        device [B, H_q, D_v], dtype
 *   lse        device float32 [B, H_q], or NULL
 *   workspace  at least vx_workspace_size(VX_OP_SPARSE_DECODE, ...) bytes
 * A request with no selected page gets out = 0 and lse = -inf. */
vx_status vx_sparse_paged_decode(const vx_paged_kv* kv, const vx_batch* batch,
                                 const void* q, const int32_t* sel, int32_t k_tot,
                                 float sm_scale, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Full paged attention over every page of every request: the baseline
 * (README, "Using Your Sparse Attention with SGLang": with sparsity off, or
 * for a skipped layer, full attention is used).  Same definition as
 * vx_sparse_paged_decode with sel = all n_b pages.  Scheduled as a work list
 * (the article's "workload planner for balanced GPU scheduling"): every
 * request's pages are cut into equal 128-page items that a fixed number of
 * blocks walk, so requests of mixed lengths stream evenly; the item offsets
 * come from seq_lens on the device, without a host synchronisation.
 *   workspace  at least vx_workspace_size(VX_OP_FULL_DECODE, ...) bytes */
vx_status vx_full_paged_decode(const vx_paged_kv* kv, const vx_batch* batch,
                               const void* q, float sm_scale, void* out, float* lse,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* One whole decode step, fused (Vortex article, "A dual-stage programmable
 * abstraction": the cache stage runs when a page is finished, the indexer and
 * the attention on every step).  Equivalent to, in order:
 *   - when update_completed == 1, vx_centroid_update on the page each
 *     request's newest token completed (logical page seq_lens[b]/S_p - 1 of
 *     requests with seq_lens[b] % S_p == 0);
 *   - vx_score_topk(kv, batch, q, topk, n_bos, n_eos, sel, ...);
 *   - vx_sparse_paged_decode(kv, batch, q, sel, topk + n_bos + n_eos,
 *     sm_scale, out, lse, ...).
 * The completed page is the last logical page, which is reserved
 * (n_eos >= 1), so its new centroid cannot change this step's selection.
 * When there are enough (request, KV head) pairs to fill the GPU, one kernel
 * does all of it, one block per pair; otherwise the three stages run as
 * separate launches.  sel and the centroids equal those calls' results bit
 * for bit; out and lse equal them up to the order of fp32 rounding (bit for
 * bit when vx_sparse_paged_decode would plan a single split).
 *   workspace  at least vx_workspace_size(VX_OP_DECODE_STEP, ..., k_tot) bytes
 * Arguments and errors as for the calls it stands for. */
vx_status vx_sparse_decode_step(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                                int32_t topk, int32_t n_bos, int32_t n_eos,
                                int32_t update_completed, float sm_scale, int32_t* sel,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* vx_sparse_decode_step under the key-bounds rule (Quest, section 3, as
 * for vx_score_topk_bounds above).  Equivalent to, in order:
 *   - when update_completed == 1, vx_bounds_update on the page each
 *     request's newest token completed;
 *   - vx_score_topk_bounds(kv, batch, bounds, q, topk, n_bos, n_eos, sel, ...);
 *   - vx_sparse_paged_decode(kv, batch, q, sel, topk + n_bos + n_eos, ...).
 * kv->centroids is not read.  Dispatch (one fused kernel or separate
 * launches), exactness and workspace (VX_OP_DECODE_STEP's size) as for
 * vx_sparse_decode_step; the bounds rows equal vx_bounds_update's (up to
 * the sign of a zero minimum or maximum that ties with another zero).
 *   bounds     device [P, H_kv, 2, D_qk], dtype (read; the completed pages'
 *              rows written)
 * D_qk in {64, 128}; MLA shapes return VX_ERR_UNSUPPORTED. */
vx_status vx_sparse_decode_step_bounds(const vx_paged_kv* kv, const vx_batch* batch,
                                       void* bounds, const void* q, int32_t topk, int32_t n_bos,
                                       int32_t n_eos, int32_t update_completed, float sm_scale,
                                       int32_t* sel, void* out, float* lse, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * vx_sparse_decode_step with its workspace taken from a library-owned static
 * device array of VX_STATIC_SCRATCH_BYTES (one per GPU, held until the
 * process ends) instead of an argument.  Same results as
 * vx_sparse_decode_step with a workspace of its own.
 *   - Allocates nothing (no hipMalloc / hipFree); the first call on a device
 *     looks the array's address up on that device.
 *   - Shapes whose VX_OP_DECODE_STEP workspace exceeds VX_STATIC_SCRATCH_BYTES
 *     return VX_ERR_WORKSPACE_TOO_SMALL with nothing launched.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (concurrent streams, or host threads) race and must be serialised
 *     by the caller.  The array's contents on entry do not matter.
 * Other arguments and errors as for vx_sparse_decode_step. */
#define VX_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
vx_status vx_sparse_decode_step_static(const vx_paged_kv* kv, const vx_batch* batch,
                                       const void* q, int32_t topk, int32_t n_bos, int32_t n_eos,
                                       int32_t update_completed, float sm_scale, int32_t* sel,
                                       void* out, float* lse, hipStream_t stream);

/* The attention layers of one decode step in one call (README, "Using
 * Your Sparse Attention with SGLang": with sparsity on, the layers listed as
 * skipped run full attention; the serving setting replays the step as a
 * captured graph).  For l = 0 .. n_layers-1, in order on `stream`:
 *   dense && dense[l]:  vx_full_paged_decode(&kv[l], batch, q[l], sm_scale,
 *                                            out[l], lse ? lse[l] : NULL, ...)
 *   otherwise:          vx_sparse_decode_step(&kv[l], batch, q[l], topk, n_bos,
 *                                             n_eos, update_completed, sm_scale,
 *                                             sel[l], out[l], lse ? lse[l] : NULL, ...)
 * Every layer shares `batch` (the same requests, page table and lengths) and
 * the shapes of kv[0] (dtype, page size, heads and head dims; each layer has
 * its own pools and centroid table), so every layer gets the same launch
 * plan; one workspace serves all of them, one layer after the other.
 *   kv         host array [n_layers] of caches
 *   q, out     host arrays [n_layers] of device pointers, as in the calls above
 *   dense      host uint8 [n_layers] (nonzero: full attention), or NULL (none)
 *   sel        host array [n_layers] of device pointers; entries of dense
 *              layers are not read (sel may be NULL when every layer is dense)
 *   lse        host array [n_layers] of device pointers (entries may be NULL),
 *              or NULL
 *   workspace  at least vx_workspace_size(VX_OP_DECODE_LAYERS, ..., k_tot) bytes
 * Every layer's arguments are checked before anything is launched.  No call
 * in it synchronises, allocates or clears memory with a memset, so the whole
 * call can be captured into a HIP graph and replayed (the graph then keeps
 * the device pointers, lengths bound and plan of the capture). */
vx_status vx_decode_layers(const vx_paged_kv* kv, const vx_batch* batch, const void* const* q,
                           int32_t n_layers, const uint8_t* dense, int32_t topk, int32_t n_bos,
                           int32_t n_eos, int32_t update_completed, float sm_scale,
                           int32_t* const* sel, void* const* out, float* const* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes the call `op` needs for these shapes (k_tot is read for
 * VX_OP_SPARSE_DECODE, VX_OP_DECODE_STEP and VX_OP_DECODE_LAYERS only).
 * Host-only; launches nothing.  The size depends on the shapes and on the
 * current device's compute-unit count (256 when it cannot be queried). */
vx_status vx_workspace_size(int32_t op, const vx_paged_kv* kv, const vx_batch* batch,
                            int32_t k_tot, size_t* bytes /* host */);

/* A decode launch plan (the article's "workload planner for balanced GPU
 * scheduling", section "A dual-stage programmable abstraction"): how
 * vx_sparse_paged_decode / vx_full_paged_decode cut each (request, KV head)'s
 * page list into splits of consecutive entries, merged afterwards.  Those
 * calls plan for the current device themselves; an explicit plan is for
 * callers that want a launch independent of the device (the same plan on GPUs
 * of different sizes, or a fixed split size).  The output does not depend on
 * the plan beyond the order of fp32 rounding. */
typedef struct {
  int32_t op;               /* VX_OP_SPARSE_DECODE or VX_OP_FULL_DECODE          */
  int32_t num_cus;          /* compute units the plan was made for               */
  int32_t pages_per_split;  /* list entries one split attends                    */
  int32_t n_split;          /* splits per (request, KV head); 1: direct output   */
  int32_t work_list;        /* 1: a fixed number of blocks walk the (request,
                               split, KV head) items of the whole batch, the
                               dense calls' balanced schedule; 0: one block per
                               (split, KV head, request)                       */
  int32_t blocks;           /* blocks of a work-list launch, else 0              */
  uint64_t workspace_bytes; /* workspace the planned call needs                  */
} vx_decode_plan;

/* Plans the decode call `op` for these shapes (k_tot read for
 * VX_OP_SPARSE_DECODE only) on a GPU of `num_cus` compute units (0: the
 * current device's), with `pages_per_split` pages per split (0: the
 * planner's choice; a given value is raised to ceil(pages / 1024) and, for
 * MLA shapes, capped at 256).  Dense plans of D_qk 64 / 128 with up to 2048
 * requests are work lists of pages_per_split-page items (128 by default);
 * other plans have one block per (split, KV head, request).  Host-only and a
 * pure function of its arguments (and, for num_cus 0, of the device's CU
 * count); writes *plan. */
vx_status vx_plan_decode(int32_t op, const vx_paged_kv* kv, const vx_batch* batch, int32_t k_tot,
                         int32_t num_cus, int32_t pages_per_split, vx_decode_plan* plan /* host */);

/* vx_sparse_paged_decode (sel given, plan->op VX_OP_SPARSE_DECODE) or
 * vx_full_paged_decode (sel NULL, plan->op VX_OP_FULL_DECODE) launched with
 * an explicit plan.  The plan must be what vx_plan_decode returns for these
 * shapes, its num_cus and its pages_per_split (VX_ERR_INVALID_ARGUMENT
 * otherwise); the workspace must hold plan->workspace_bytes.  Other
 * arguments and errors as for those calls. */
vx_status vx_paged_decode_planned(const vx_paged_kv* kv, const vx_batch* batch, const void* q,
                                  const int32_t* sel, int32_t k_tot, const vx_decode_plan* plan,
                                  float sm_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* vx_status_string(vx_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t vx_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VX_H */
