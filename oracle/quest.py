"""fp64 CPU oracle of a second page-summary rule through the same pipeline:
Quest's per-page key bounds.

TEST INFRASTRUCTURE.  This module checks the GPU library; it is not part of
it.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it.  It shares no code with the HIP path.

Where the rule comes from.  The Vortex article (section "Speedups that scale
to 229B parameters") names Quest as the second sparse-attention algorithm it
serves, next to block top-k, but does not state its rule.  The rule is taken
from the Quest paper (Tang et al., "Quest: Query-Aware Sparsity for
Efficient Long-Context LLM Inference", ICML 2024, section 3, "Query-aware
criticality estimation"), restated here:

* summary (query-independent, once per full page): for every channel i, the
  smallest and the largest key value over the page's tokens;
* criticality (query-dependent): for query q, the sum over channels of the
  larger of q_i * min_i and q_i * max_i.  It bounds from above the dot
  product of q with any key of the page, because each channel's term does;
* the top-k pages by criticality are attended exactly.

Readings that fit this pipeline (restated in the design notes):
  * the query is the group mean of the KV head's query heads, as for the
    centroid scores (one selection per (request, KV head)); with G = 1 it is
    the query head itself, as in the Quest paper;
  * the summary is stored in the KV dtype, [page, KV head, 2, D] with the
    minimum row first; min and max of representable values are
    representable, so no rounding is involved;
  * reserved pages, candidates, the tie rule and the output order are those
    of the centroid indexer.

Pins (test suite, tests/test_oracle_quest.py): the bound holds against every
key of the page (brute force); it is reached when all the page's keys are
equal, and when the query is non-negative it equals q . max; the summary is
numpy's own minimum / maximum; a hand-worked example in tests/golden.
"""

from __future__ import annotations

import numpy as np

from .block_topk import (candidate_pages, group_mean_query, reserved_pages,
                         topk_pages)

__all__ = ["page_bounds", "request_bounds", "bound_scores", "select_pages_quest",
           "quest_decode_request"]


def page_bounds(k_pages) -> np.ndarray:
    """Per-channel minimum and maximum of each page's keys.
    ``k_pages`` [n, H_kv, S_p, D] -> [n, H_kv, 2, D] fp64 (row 0 the
    minimum, row 1 the maximum)."""
    k = np.asarray(k_pages, dtype=np.float64)
    out = np.empty((k.shape[0], k.shape[1], 2, k.shape[3]))
    for p in range(k.shape[0]):
        for h in range(k.shape[1]):
            rows = k[p, h]                       # [S_p, D]
            lo = rows[0].copy()
            hi = rows[0].copy()
            for t in range(1, rows.shape[0]):    # channel by channel, token by token
                lo = np.where(rows[t] < lo, rows[t], lo)
                hi = np.where(rows[t] > hi, rows[t], hi)
            out[p, h, 0] = lo
            out[p, h, 1] = hi
    return out


def request_bounds(k_pages, seq_len: int) -> np.ndarray:
    """Bounds of one request's logical pages [n_b, H_kv, 2, D]; the page that
    is not yet full (only the last can be) gets NaN rows: like the centroid,
    the summary is made once a page is finished."""
    k = np.asarray(k_pages)
    n_b, H, S, D = k.shape
    out = np.full((n_b, H, 2, D), np.nan)
    n_full = int(seq_len) // S
    if n_full:
        out[:n_full] = page_bounds(k[:n_full])
    return out


def bound_scores(qbar, bounds, pages) -> np.ndarray:
    """Criticality of each listed logical page for each KV head:
    sum_i max(q_i * min_i, q_i * max_i).  ``qbar`` [H_kv, D], ``bounds``
    [n_b, H_kv, 2, D] -> [H_kv, len(pages)]."""
    qbar = np.asarray(qbar, dtype=np.float64)
    b = np.asarray(bounds, dtype=np.float64)[np.asarray(pages, dtype=np.int64)]
    lo = b[:, :, 0, :] * qbar[None]             # [n, H_kv, D]
    hi = b[:, :, 1, :] * qbar[None]
    return np.maximum(lo, hi).sum(axis=2).T


def select_pages_quest(q, bounds, n_pages: int, topk: int, n_bos: int, n_eos: int) -> list:
    """Selected logical pages per KV head (list of H_kv sorted int arrays):
    reserved pages united with the top-k candidates by criticality.
    ``q`` [H_q, D]; ``bounds`` [n_b, H_kv, 2, D]."""
    H_kv = np.asarray(bounds).shape[1]
    qbar = group_mean_query(q, H_kv)
    res = reserved_pages(n_pages, n_bos, n_eos)
    cand = candidate_pages(n_pages, n_bos, n_eos)
    out = []
    if len(cand):
        s = bound_scores(qbar, bounds, cand)
        assert np.all(np.isfinite(s)), "a candidate page has no summary"
    for h in range(H_kv):
        top = topk_pages(s[h], cand, topk) if len(cand) else np.zeros(0, np.int64)
        out.append(np.union1d(res, top).astype(np.int64))
    return out


def quest_decode_request(q, k_pages, v_pages, bounds, seq_len: int, sm_scale: float,
                         topk: int, n_bos: int, n_eos: int, v_dims: int | None = None):
    """Selection by criticality, then exact attention over the selected
    pages.  Returns (selected per KV head, o, lse)."""
    from .block_topk import decode_request
    S = np.asarray(k_pages).shape[2]
    n_b = -(-int(seq_len) // S)
    sel = select_pages_quest(q, bounds[:n_b], n_b, topk, n_bos, n_eos)
    o, lse = decode_request(q, k_pages, v_pages, seq_len, sm_scale, sel, v_dims)
    return sel, o, lse
