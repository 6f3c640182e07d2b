"""fp64 CPU oracle of the lossy indexer: the "stochastic radix top-k" with
early termination.

TEST INFRASTRUCTURE.  This module checks the GPU library; it is not part of
it.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it.  It shares no code with the HIP path.

What the pages say: the Vortex article (section "A dual-stage programmable
abstraction") names a stochastic radix top-k, a lossy variant that ends
early and gives up a little exactness for a faster indexing stage.  Nothing
more is given, so this is the plainest reading that fits those words:

* radix: the candidates' scores, as fp32 numbers, become order-preserving
  unsigned 32-bit keys (the IEEE-754 order of finite numbers, with -0 and +0
  equal); a level counts the keys of the current range in 1024 bins of their
  next 10 bits, from the top bit down, and finds the bin where the count
  from the top reaches the number still wanted;
* early termination: after ``levels`` levels (1 or 2) the search stops.
  Every candidate in a bin above the boundary bin is taken.  If the boundary
  bin is not taken whole, which of its members fill the remaining places is
  not decided by score;
* stochastic: those places go to the bin's members in ascending page order,
  cyclically from a random rank: with N members ranked 0 .. N-1 by page and
  a caller-drawn random 32-bit word r, the member of rank i is taken iff
  (i - r mod N) mod N < (places left).  The random words are inputs (one per
  request and KV head), so the GPU and this oracle need no shared generator.

When the boundary bin is taken whole (or all candidates fit in k) the result
is the exact top-k.  Reserved pages are handled as in the exact indexer.

Pins (test suite, oracle tests): the order-preserving key against Python's
own float ordering on special values and random floats; the result equals
the exact top-k whenever the boundary bin is taken whole; brute force over
every rotation on tiny hand-built inputs; invariants (exactly k taken, all
keys above the boundary bin taken, the members taken form one cyclic run of
ranks); a hand-worked example in ``tests/golden``.
"""

from __future__ import annotations

import numpy as np

from .block_topk import (candidate_pages, group_mean_query, page_scores,
                         reserved_pages)

__all__ = ["order_keys", "radix_boundary", "radix_topk_pages", "select_pages_radix"]

_BITS = 10               # key bits per level
_BINS = 1 << _BITS


def order_keys(scores_f32) -> np.ndarray:
    """Order-preserving uint32 keys of fp32 scores (as uint64 values): a > b
    as floats iff key(a) > key(b); -0 and +0 give the key of +0.  Negative
    numbers have all bits inverted, non-negative ones get the sign bit set."""
    f = np.asarray(scores_f32, dtype=np.float32)
    f = np.where(f == 0, np.float32(0.0), f).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    neg = (u >> 31) == 1
    return np.where(neg, (~u) & 0xFFFFFFFF, u | 0x80000000).astype(np.uint64)


def radix_boundary(keys, k: int, levels: int):
    """Run ``levels`` radix levels over ``keys`` (uint64 values < 2**32) for
    the k largest.  Returns (lo, hi, take, whole): the boundary bin's key
    range [lo, hi], the number of places left for its members, and whether
    the bin is taken whole.  Requires 0 < k < len(keys)."""
    keys = np.asarray(keys, dtype=np.uint64)
    assert 0 < k < len(keys) and levels >= 1
    lo, hi = 0, (1 << 32) - 1
    want = k
    for _ in range(levels):
        width = hi - lo + 1                       # a power of two
        shift = max(width.bit_length() - 1 - _BITS, 0)
        inside = keys[(keys >= lo) & (keys <= hi)]
        bins = ((inside - np.uint64(lo)) >> np.uint64(shift)).astype(np.int64)
        counts = np.bincount(bins, minlength=_BINS)
        above = 0
        for b in range(len(counts) - 1, -1, -1):  # from the top bin down
            if above + counts[b] >= want:
                break
            above += counts[b]
        want -= above
        lo = lo + (b << shift)
        hi = min(hi, lo + (1 << shift) - 1)
        if want == counts[b]:
            return lo, hi, want, True
    return lo, hi, want, False


def radix_topk_pages(scores_f32, pages, k: int, levels: int, rnd: int) -> np.ndarray:
    """The k pages the lossy radix top-k takes (sorted ascending).  All pages
    when there are at most k; none when k is 0."""
    pages = np.asarray(pages, dtype=np.int64)
    if len(pages) <= k:
        return np.sort(pages)
    if k == 0:
        return np.zeros(0, np.int64)
    keys = order_keys(scores_f32)
    lo, hi, take, whole = radix_boundary(keys, k, levels)
    above = pages[keys > hi]
    order = np.argsort(pages, kind="stable")
    members = pages[order][(keys[order] >= lo) & (keys[order] <= hi)]   # page order
    if whole:
        chosen = members
    else:
        n = len(members)
        r0 = int(rnd) % n
        rank = np.arange(n)
        chosen = members[(rank - r0) % n < take]
    out = np.sort(np.concatenate([above, chosen]))
    assert len(out) == k
    return out


def select_pages_radix(q, centroids, n_pages: int, topk: int, n_bos: int, n_eos: int,
                       levels: int, rnd_row) -> list:
    """Per KV head selection of the lossy indexer (list of H_kv sorted int
    arrays): reserved pages united with ``radix_topk_pages`` of the
    candidates, scored as by the exact indexer and rounded to fp32.
    ``q`` [H_q, D]; ``centroids`` [n_b, H_kv, D]; ``rnd_row`` [H_kv]."""
    H_kv = np.asarray(centroids).shape[1]
    qbar = group_mean_query(q, H_kv)
    res = reserved_pages(n_pages, n_bos, n_eos)
    cand = candidate_pages(n_pages, n_bos, n_eos)
    out = []
    if len(cand):
        s = page_scores(qbar, centroids, cand)
        assert np.all(np.isfinite(s)), "a candidate page has no centroid"
    for h in range(H_kv):
        if len(cand):
            top = radix_topk_pages(s[h].astype(np.float32), cand, topk, levels, int(rnd_row[h]))
        else:
            top = np.zeros(0, np.int64)
        out.append(np.union1d(res, top).astype(np.int64))
    return out
