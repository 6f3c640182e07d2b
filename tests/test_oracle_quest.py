"""Pins of the page-bound (Quest) oracle, oracle/quest.py, against things
other than itself: the bound's defining property checked by brute force
against every key, the cases where it is reached exactly, numpy's own
minimum / maximum for the summary, and a hand-worked example
(tests/golden/quest_example.json)."""

import json
import os

import numpy as np

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _pages(rng, n=6, H=2, S=16, D=8, scale=1.0):
    return rng.standard_normal((n, H, S, D)) * scale + rng.standard_normal((n, H, 1, D))


def test_summary_is_the_channel_min_and_max():
    rng = np.random.default_rng(1)
    k = _pages(rng)
    b = orc.page_bounds(k)
    assert np.array_equal(b[:, :, 0], k.min(axis=2))
    assert np.array_equal(b[:, :, 1], k.max(axis=2))


def test_bound_dominates_every_key_of_the_page():
    rng = np.random.default_rng(2)
    for trial in range(50):
        k = _pages(rng, n=5, H=3, S=int(rng.integers(1, 20)), D=int(rng.integers(1, 12)),
                   scale=10.0 ** rng.uniform(-2, 2))
        qbar = rng.standard_normal((3, k.shape[3])) * 10.0 ** rng.uniform(-2, 2)
        s = orc.bound_scores(qbar, orc.page_bounds(k), np.arange(5))        # [H, n]
        for p in range(5):
            for h in range(3):
                best = max(float(qbar[h] @ k[p, h, t]) for t in range(k.shape[2]))
                assert s[h, p] >= best - 1e-12 * (1 + abs(best))


def test_bound_is_reached_for_equal_keys_and_signed_queries():
    rng = np.random.default_rng(3)
    D = 16
    row = rng.standard_normal(D)
    k = np.broadcast_to(row, (1, 1, 16, D)).copy()               # every key equal
    q = rng.standard_normal((1, D))
    assert np.isclose(orc.bound_scores(q, orc.page_bounds(k), [0])[0, 0], q[0] @ row)
    k = _pages(rng, n=1, H=1, S=16, D=D)
    b = orc.page_bounds(k)
    qp = np.abs(rng.standard_normal((1, D)))                     # non-negative query
    assert np.isclose(orc.bound_scores(qp, b, [0])[0, 0], qp[0] @ k[0, 0].max(axis=0))
    assert np.isclose(orc.bound_scores(-qp, b, [0])[0, 0], -qp[0] @ k[0, 0].min(axis=0))


def test_partial_page_has_no_summary():
    rng = np.random.default_rng(4)
    k = _pages(rng, n=3, H=1, S=16, D=4)
    b = orc.request_bounds(k, 16 * 2 + 5)
    assert np.all(np.isfinite(b[:2])) and np.all(np.isnan(b[2]))


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "quest_example.json")))
    k = np.array(g["pages"])[:, None]                            # [5, 1, 3, 2]
    q = np.array(g["q"])
    assert np.array_equal(orc.group_mean_query(q, 1)[0], g["qbar"])
    b = orc.page_bounds(k)
    assert np.array_equal(b[1:4, 0], np.array(g["bounds_of_candidates"]))
    s = orc.bound_scores(np.array([g["qbar"]]), b, [1, 2, 3])[0]
    assert s.tolist() == g["criticality_of_candidates"]
    sel = orc.select_pages_quest(q, b, 5, g["topk"], 1, 1)
    assert sel[0].tolist() == g["selected"]


def test_selection_reserves_unites_and_orders():
    rng = np.random.default_rng(5)
    H_kv, G, D, n_b = 2, 4, 8, 30
    k = _pages(rng, n=n_b, H=H_kv, S=16, D=D)
    b = orc.page_bounds(k)
    q = rng.standard_normal((H_kv * G, D))
    for topk, bos, eos in ((5, 1, 1), (0, 1, 2), (40, 2, 1)):
        sel = orc.select_pages_quest(q, b, n_b, topk, bos, eos)
        for h in range(H_kv):
            assert set(range(bos)) | set(range(n_b - eos, n_b)) <= set(sel[h].tolist())
            assert len(sel[h]) == min(n_b, topk + bos + eos)
            assert np.all(np.diff(sel[h]) > 0)
    # top-k by criticality: every chosen candidate scores at least every other
    qbar = orc.group_mean_query(q, H_kv)
    sel = orc.select_pages_quest(q, b, n_b, 7, 1, 1)
    cand = np.arange(1, n_b - 1)
    s = orc.bound_scores(qbar, b, cand)
    for h in range(H_kv):
        chosen = [p for p in sel[h] if 1 <= p < n_b - 1]
        rest = [p for p in cand if p not in chosen]
        assert min(s[h, p - 1] for p in chosen) >= max(s[h, p - 1] for p in rest)


def _sdpa_fp64(q_rows, keys, values, sm_scale):
    """Textbook attention from torch's library routine, fp64 on the CPU."""
    import torch
    q = torch.from_numpy(np.asarray(q_rows, dtype=np.float64))[None, :, None, :]   # [1, G, 1, D]
    k = torch.from_numpy(np.asarray(keys, dtype=np.float64))[None, None].expand(1, q.shape[1], -1, -1)
    v = torch.from_numpy(np.asarray(values, dtype=np.float64))[None, None].expand(1, q.shape[1], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=sm_scale)
    lse = torch.logsumexp(sm_scale * (q[0, :, 0] @ k[0, 0].T), dim=-1)
    return o[0, :, 0].numpy(), lse.numpy()


def test_quest_decode_hand_worked_end_to_end():
    """The whole bound-rule path on the hand-worked example (its selection,
    pages 0, 1, 3 and 4, worked by hand in tests/golden/quest_example.json),
    with a partial last page: the output equals torch's scaled-dot-product
    attention over exactly the selected pages' tokens below seq_len."""
    g = json.load(open(os.path.join(GOLDEN, "quest_example.json")))
    k = np.array(g["pages"])[:, None]                            # [5, 1, 3, 2]
    rng = np.random.default_rng(6)
    v = rng.standard_normal((5, 1, 3, 4))
    q = np.array(g["q"])
    seq_len = 14                                                 # page 4 holds 2 tokens
    bounds = orc.request_bounds(k, seq_len)                      # page 4 is not full
    sel, o, lse = orc.quest_decode_request(q, k, v, bounds, seq_len, 0.5, g["topk"], 1, 1)
    assert sel[0].tolist() == g["selected"]
    toks = [(p, t) for p in g["selected"] for t in range(3) if 3 * p + t < seq_len]
    keys = np.array([k[p, 0, t] for p, t in toks])
    vals = np.array([v[p, 0, t] for p, t in toks])
    o_ref, lse_ref = _sdpa_fp64(q, keys, vals, 0.5)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_quest_decode_with_every_candidate_is_dense_attention():
    """With top-k at least the candidate count, the bound-rule path attends
    every page: its output is full attention over all tokens below seq_len,
    per KV head's query group (torch's routine, fp64)."""
    rng = np.random.default_rng(7)
    H_kv, G, S, D, L = 2, 3, 16, 8, 16 * 9 + 5
    n_b = -(-L // S)
    k = rng.standard_normal((n_b, H_kv, S, D))
    v = rng.standard_normal((n_b, H_kv, S, D))
    q = rng.standard_normal((H_kv * G, D))
    bounds = orc.request_bounds(k, L)
    sel, o, lse = orc.quest_decode_request(q, k, v, bounds, L, 0.3, n_b, 1, 1)
    for h in range(H_kv):
        assert sel[h].tolist() == list(range(n_b))
        keys = k[:, h].reshape(-1, D)[:L]
        vals = v[:, h].reshape(-1, D)[:L]
        o_ref, lse_ref = _sdpa_fp64(q[h * G:(h + 1) * G], keys, vals, 0.3)
        assert np.allclose(o[h * G:(h + 1) * G], o_ref, rtol=0, atol=1e-12)
        assert np.allclose(lse[h * G:(h + 1) * G], lse_ref, rtol=0, atol=1e-12)


def test_quest_decode_planted_ranking():
    """Pages whose keys are a constant row c_p * e_0 (the bound is exact:
    q . max = c_p q_0 for q_0 > 0): the path keeps the top-k pages by c_p
    and attends them only."""
    H_kv, S, D, n_b = 1, 4, 4, 12
    c = np.array([0.0, 5.0, -1.0, 7.0, 2.0, 9.0, 3.0, 6.5, -4.0, 1.0, 8.0, 0.0])
    k = np.zeros((n_b, H_kv, S, D))
    k[:, 0, :, 0] = c[:, None]
    v = np.arange(n_b * S * D, dtype=np.float64).reshape(n_b, H_kv, S, D)
    q = np.array([[1.0, 0.0, 0.0, 0.0], [3.0, 0.0, 0.0, 0.0]])     # group mean (2, 0, 0, 0)
    L = n_b * S
    sel, o, lse = orc.quest_decode_request(q, k, v, orc.request_bounds(k, L), L, 1.0, 3, 1, 1)
    assert sel[0].tolist() == [0, 3, 5, 10, 11]                  # top-3 of pages 1..10 by c_p
    toks = [(p, t) for p in (0, 3, 5, 10, 11) for t in range(S)]
    o_ref, lse_ref = _sdpa_fp64(q, np.array([k[p, 0, t] for p, t in toks]),
                                np.array([v[p, 0, t] for p, t in toks]), 1.0)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-9) and np.allclose(lse, lse_ref, rtol=0, atol=1e-12)
