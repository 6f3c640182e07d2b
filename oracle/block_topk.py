"""fp64 CPU oracle: centroid-indexed block-top-k sparse decode attention over
a paged KV cache.

TEST INFRASTRUCTURE.  This module checks the GPU library; it is not part of
it.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it.  It shares no code with the HIP path and imports nothing
from the library package.

What it computes, and where the pages say so
--------------------------------------------
The method has two stages (Vortex article, section "A dual-stage
programmable abstraction"; vortex_torch README, "Quick Example: Custom
Sparse Attention"):

* query-independent, run while the cache is built and only for pages that
  are full: every page gets a centroid, the average of its keys, stored in a
  named cache with one head_dim-wide row per page (``CMean`` over the token
  axis in ``forward_cache``; ``create_cache`` returns a (1, head_dim) entry);
* query-dependent, run at every decode step: the query is averaged over the
  query heads of the single-request view (``forward_indexer``), dotted with
  the centroids (``GeMV``), the top-k pages are chosen (``topK``) and exact
  attention runs over only those pages.

The serving example fixes the parameters around it (README, "Using Your
Sparse Attention with SGLang"): 16-token pages, a top-k value, one reserved
page at the start and one at the end, and full attention when sparsity is
off or a layer is skipped.  Pages live in a paged pool reached through a page
table (article, "The friction of paged memory").

Readings where the pages are silent (all stated once more in the design
notes):
  * query head j belongs to KV head j // G (contiguous groups); the query
    mean is taken over the G query heads of one KV head, in fp64 (unrounded);
  * selection is per (request, KV head); reserved pages are the first
    ``n_bos`` and the last ``n_eos`` logical pages and are not candidates;
    top-k is taken among the candidates on top of them;
  * ties in score go to the lower logical page; the selection is emitted in
    ascending logical order, padded with -1;
  * the centroid is rounded once, to nearest-even, to the KV dtype;
  * scores are unscaled dot products;
  * the sequence length counts the token being decoded; only positions below
    it are attended; the softmax is natural-exp with scale ``sm_scale``;
  * MLA: V is the first ``head_dim_v`` dims of K.

Every pin of this module against something other than itself lives in the
test suite's oracle tests (closed forms, brute force, invariants, a textbook
library routine).  No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "round_to", "page_centroids", "request_centroids", "group_mean_query",
    "reserved_pages", "candidate_pages", "page_scores", "topk_pages",
    "select_pages", "selection_table", "attend", "gather_tokens",
    "decode_request", "sparse_decode_request", "merge_partials",
]

# (significand bits including the implicit one, exponent of the smallest
# normal number) of the binary formats the KV cache may be stored in.
_FORMATS = {"f32": (24, -126), "bf16": (8, -126)}


def round_to(x, dtype: str) -> np.ndarray:
    """Round fp64 values to the nearest ``dtype`` value, ties to even.

    Written from the definition of a binary floating-point format with p
    significand bits: the spacing of representable numbers around x is
    2**(e - p + 1) for |x| in [2**e, 2**(e+1)), never finer than the
    subnormal spacing.  The result is returned as fp64 (exactly
    representable in ``dtype``).  Overflow is not handled (not reachable
    with the inputs used here)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    p, emin = _FORMATS[dtype]
    _, e = np.frexp(x)              # x = m * 2**e with 0.5 <= |m| < 1
    q = np.maximum(e - p, emin - (p - 1))      # exponent of the spacing
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


# ---------------------------------------------------------------------------
# Query-independent stage
# ---------------------------------------------------------------------------
def page_centroids(k_pages, dtype: str) -> np.ndarray:
    """Centroid of each page: mean of its keys over the token axis.

    ``k_pages`` [n, H_kv, S_p, D] (any float dtype) -> [n, H_kv, D] fp64
    holding values exactly representable in ``dtype``.  The mean is taken in
    fp64 and rounded once.  Source: the cache stage's ``CMean`` over the
    token rows of each finished page, stored as one head_dim-wide row per
    page (README, "Quick Example"; article, "A dual-stage programmable
    abstraction": centroids are representative average points)."""
    k = np.asarray(k_pages, dtype=np.float64)
    return round_to(k.mean(axis=2), dtype)


def request_centroids(k_pages, seq_len: int, dtype: str) -> np.ndarray:
    """Centroids of one request's logical pages [n_b, H_kv, D]; pages that
    are not yet full (only the last can be) get NaN rows, because the cache
    stage runs only when a page is finished (README, "Quick Example")."""
    k = np.asarray(k_pages)
    n_b, _, S, _ = k.shape
    out = np.full((n_b, k.shape[1], k.shape[3]), np.nan)
    n_full = int(seq_len) // S
    if n_full:
        out[:n_full] = page_centroids(k[:n_full], dtype)
    return out


# ---------------------------------------------------------------------------
# Query-dependent stage: indexer
# ---------------------------------------------------------------------------
def group_mean_query(q, num_kv_heads: int) -> np.ndarray:
    """Mean query of each KV head's group: [H_q, D] -> [H_kv, D] fp64.

    The indexer averages the query over the heads of its single-request
    view (README, "Quick Example", ``forward_indexer``); with grouped KV
    heads the view of one KV head holds its G query heads, j // G == h."""
    q = np.asarray(q, dtype=np.float64)
    H_q, D = q.shape
    assert H_q % num_kv_heads == 0
    G = H_q // num_kv_heads
    return q.reshape(num_kv_heads, G, D).mean(axis=1)


def reserved_pages(n_pages: int, n_bos: int, n_eos: int) -> np.ndarray:
    """Logical pages always attended: the first n_bos and the last n_eos
    (README, "Using Your Sparse Attention with SGLang": reserved BOS / EOS
    page counts).  Overlaps collapse (set union); sorted ascending."""
    first = np.arange(min(n_bos, n_pages))
    last = np.arange(max(n_pages - n_eos, 0), n_pages)
    return np.union1d(first, last).astype(np.int64)


def candidate_pages(n_pages: int, n_bos: int, n_eos: int) -> np.ndarray:
    """Pages that compete in the top-k: those between the reserved ones."""
    return np.arange(n_bos, max(n_pages - n_eos, n_bos), dtype=np.int64)


def page_scores(qbar, centroids, pages) -> np.ndarray:
    """Score of each listed logical page for each KV head: the dot product of
    the group-mean query with the page's centroid row (README, "Quick
    Example": ``GeMV`` of the mean query against the centroid cache).
    ``qbar`` [H_kv, D], ``centroids`` [n_b, H_kv, D] -> [H_kv, len(pages)]."""
    qbar = np.asarray(qbar, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float64)[np.asarray(pages, dtype=np.int64)]
    return np.einsum("phd,hd->hp", c, qbar)


def topk_pages(scores, pages, k: int) -> np.ndarray:
    """The k listed pages with the largest scores; equal scores are ordered
    by lower page first.  All pages when there are at most k.  Returned in
    selection order (best first).  Source: ``topK`` over the scores
    (README, "Quick Example"); the tie rule is this library's reading."""
    scores = np.asarray(scores, dtype=np.float64)
    pages = np.asarray(pages, dtype=np.int64)
    if len(pages) <= k:
        return pages[np.lexsort((pages, -scores))]
    order = np.lexsort((pages, -scores))      # primary key: -score; then page
    return pages[order[:k]]


def select_pages(q, centroids, n_pages: int, topk: int, n_bos: int,
                 n_eos: int) -> list:
    """Selected logical pages per KV head (list of H_kv sorted int arrays):
    reserved pages united with the top-k candidates by centroid score.

    ``q`` [H_q, D] is one request's query; ``centroids`` [n_b, H_kv, D]."""
    H_kv = np.asarray(centroids).shape[1]
    qbar = group_mean_query(q, H_kv)
    res = reserved_pages(n_pages, n_bos, n_eos)
    cand = candidate_pages(n_pages, n_bos, n_eos)
    out = []
    if len(cand):
        s = page_scores(qbar, centroids, cand)
        assert np.all(np.isfinite(s)), "a candidate page has no centroid"
    for h in range(H_kv):
        top = topk_pages(s[h], cand, topk) if len(cand) else np.zeros(0, np.int64)
        out.append(np.union1d(res, top).astype(np.int64))
    return out


def selection_table(selected: list, k_tot: int) -> np.ndarray:
    """Pack per-head selections into int32 [H_kv, k_tot], ascending, -1 pad."""
    out = np.full((len(selected), k_tot), -1, dtype=np.int32)
    for h, s in enumerate(selected):
        assert len(s) <= k_tot
        out[h, :len(s)] = np.sort(s)
    return out


# ---------------------------------------------------------------------------
# Query-dependent stage: attention
# ---------------------------------------------------------------------------
def attend(q_rows, keys, values, sm_scale: float):
    """Softmax attention of G query rows over n keys/values, fp64.
    Returns o [G, D_v] and the natural-log sum of exponentials lse [G]."""
    q = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    logits = sm_scale * (q @ k.T)                     # [G, n]
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    s = w.sum(axis=1, keepdims=True)
    return (w @ v) / s, (m + np.log(s))[:, 0]


def gather_tokens(k_pages, v_pages, seq_len: int, pages, head: int,
                  v_dims: int | None = None):
    """Keys and values of KV head ``head`` at the positions < seq_len of the
    listed logical pages (ascending), as contiguous [n, D] arrays: the
    logical view over non-contiguous pages (article, "The friction of paged
    memory").  ``v_pages`` None means V is the first ``v_dims`` dims of K."""
    k_pages = np.asarray(k_pages)
    S = k_pages.shape[2]
    pages = np.sort(np.asarray(pages, dtype=np.int64))
    pos = (pages[:, None] * S + np.arange(S)[None, :]).reshape(-1)
    keep = pos < seq_len
    kk = np.asarray(k_pages[pages, head], dtype=np.float64).reshape(-1, k_pages.shape[3])
    if v_pages is None:
        vv = kk[:, :v_dims]
    else:
        v_pages = np.asarray(v_pages)
        vv = np.asarray(v_pages[pages, head], dtype=np.float64).reshape(-1, v_pages.shape[3])
    return kk[keep], vv[keep]


def decode_request(q, k_pages, v_pages, seq_len: int, sm_scale: float,
                   selected: list | None = None, v_dims: int | None = None):
    """Decode attention for one request.

    ``q`` [H_q, D_qk]; ``k_pages``/``v_pages`` the request's logical pages
    [n_b, H_kv, S_p, D]; ``selected`` per-KV-head logical pages, or None for
    every page (full attention, the baseline).  Returns o [H_q, D_v] and
    lse [H_q] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    H_q = q.shape[0]
    H_kv = np.asarray(k_pages).shape[1]
    G = H_q // H_kv
    n_b = -(-int(seq_len) // np.asarray(k_pages).shape[2])
    D_v = v_dims if v_pages is None else np.asarray(v_pages).shape[3]
    o = np.empty((H_q, D_v))
    lse = np.empty(H_q)
    for h in range(H_kv):
        pages = np.arange(n_b) if selected is None else selected[h]
        kk, vv = gather_tokens(k_pages, v_pages, seq_len, pages, h, v_dims)
        o[h * G:(h + 1) * G], lse[h * G:(h + 1) * G] = attend(
            q[h * G:(h + 1) * G], kk, vv, sm_scale)
    return o, lse


def sparse_decode_request(q, k_pages, v_pages, centroids, seq_len: int,
                          sm_scale: float, topk: int, n_bos: int, n_eos: int,
                          v_dims: int | None = None):
    """The whole query-dependent path for one request: group-mean query,
    centroid scores, top-k with reserved pages, attention over the selected
    pages.  Returns (selected per KV head, o, lse)."""
    S = np.asarray(k_pages).shape[2]
    n_b = -(-int(seq_len) // S)
    sel = select_pages(q, centroids[:n_b], n_b, topk, n_bos, n_eos)
    o, lse = decode_request(q, k_pages, v_pages, seq_len, sm_scale, sel, v_dims)
    return sel, o, lse


def merge_partials(outs, lses):
    """Combine attention results over disjoint key sets into the result over
    their union: o = sum_i e^(lse_i - lse) o_i, lse = log sum_i e^lse_i.
    ``outs`` [n, G, D_v], ``lses`` [n, G]."""
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    tot = w.sum(axis=0)
    return (w[:, :, None] * outs).sum(axis=0) / tot[:, None], m + np.log(tot)
