"""Pins of the fp64 oracle against things other than itself: closed forms,
hand-worked examples, brute force, invariants and independent library
routines.  Each test names the part of the oracle it pins; together they are
chosen so that a plausible slip (mean over the wrong axis, a strided head
grouping, a reserved page counted as a candidate, a flipped tie rule, an
off-by-one in the last page, a dropped max-subtraction, a wrong merge
weight) fails at least one of them."""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle as orc


# ---------------------------------------------------------------- rounding
def test_round_to_f32_matches_numpy_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1e-45, 3e-39, -2.5e-40]])
    assert np.array_equal(orc.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


def test_round_to_bf16_matches_torch_on_f32_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(50000) * 10.0 ** rng.integers(-20, 20, 50000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.round_to(x.astype(np.float64), "bf16"), ref)


def test_round_to_bf16_ties_to_even():
    u = 2.0 ** -7                      # bf16 spacing in [1, 2)
    cases = {1 + u / 2: 1.0,           # midpoint, even neighbour below
             1 + 3 * u / 2: 1 + 2 * u, # midpoint, even neighbour above
             1 + u / 2 + 2 ** -30: 1 + u,
             -(1 + 3 * u / 2): -(1 + 2 * u)}
    for x, y in cases.items():
        assert orc.round_to(np.array([x]), "bf16")[0] == y


# ---------------------------------------------------------------- centroids
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S", [16, 64])
def test_centroid_closed_forms(dtype, S):
    D = 8
    const = np.full((1, 1, S, D), -1.75)                     # a constant page
    assert np.array_equal(orc.page_centroids(const, dtype), np.full((1, 1, D), -1.75))
    ramp = np.zeros((1, 1, S, D))                            # k_t = t * e_3
    ramp[0, 0, :, 3] = np.arange(S)
    want = np.zeros((1, 1, D))
    want[0, 0, 3] = (S - 1) / 2.0                            # 7.5 or 31.5: exact in bf16
    assert np.array_equal(orc.page_centroids(ramp, dtype), want)


def test_centroid_is_mean_over_tokens_per_head():
    rng = np.random.default_rng(2)
    k = rng.integers(-8, 8, size=(3, 2, 16, 4)).astype(np.float64)
    c = orc.page_centroids(k, "f32")
    for p, h, d in itertools.product(range(3), range(2), range(4)):
        # integer sums divided by 16 are exact in binary
        assert c[p, h, d] == sum(k[p, h, t, d] for t in range(16)) / 16


def test_centroid_rounds_once_to_kv_dtype():
    # mean exactly halfway between two bf16 values: ties to even
    S, u = 16, 2.0 ** -7
    k = np.full((1, 1, S, 1), 1.0)
    k[0, 0, :8, 0] = 1.0 + u           # mean = 1 + u/2
    assert orc.page_centroids(k, "bf16")[0, 0, 0] == 1.0
    assert orc.page_centroids(k, "f32")[0, 0, 0] == 1.0 + u / 2


def test_request_centroids_only_full_pages():
    k = np.ones((4, 1, 16, 2))
    c = orc.request_centroids(k, seq_len=50, dtype="f32")   # pages 0..2 full, 3 partial
    assert np.all(c[:3] == 1.0) and np.all(np.isnan(c[3]))
    c = orc.request_centroids(k, seq_len=64, dtype="f32")
    assert np.all(c == 1.0)


# ---------------------------------------------------------------- group mean
def test_group_mean_identity_and_contiguous_groups():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 5))
    assert np.array_equal(orc.group_mean_query(q, 4), q)                  # G = 1
    same = np.repeat(q[:1], 4, axis=0)
    assert np.allclose(orc.group_mean_query(same, 1), q[:1], rtol=0, atol=1e-15)
    a, b, c, d = np.eye(4)[:, :4]
    qb = orc.group_mean_query(np.stack([a, b, c, d]), 2)
    assert np.array_equal(qb, np.stack([(a + b) / 2, (c + d) / 2]))       # not (a+c)/2


# ---------------------------------------------------------------- reserved
@pytest.mark.parametrize("n,bos,eos,res,cand", [
    (10, 1, 1, [0, 9], list(range(1, 9))),
    (10, 2, 3, [0, 1, 7, 8, 9], list(range(2, 7))),
    (2, 1, 1, [0, 1], []),
    (1, 1, 1, [0], []),
    (3, 2, 2, [0, 1, 2], []),
])
def test_reserved_and_candidates(n, bos, eos, res, cand):
    assert orc.reserved_pages(n, bos, eos).tolist() == res
    assert orc.candidate_pages(n, bos, eos).tolist() == cand


# ---------------------------------------------------------------- scores / top-k
def test_scores_planted_axis():
    alpha = np.array([3.0, -1.0, 7.0, 0.5, 7.0, 2.0])
    cent = np.zeros((6, 1, 4))
    cent[:, 0, 0] = alpha
    qbar = np.array([[1.0, 9.0, 9.0, 9.0]])
    cent[:, 0, 1:] = 0.0
    assert np.array_equal(orc.page_scores(qbar, cent, np.arange(6))[0], alpha)


def _brute_topk(scores, pages, k):
    best = None
    for sub in itertools.combinations(range(len(pages)), k):
        key = (sum(scores[i] for i in sub), tuple(-pages[i] for i in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return sorted(pages[i] for i in best[1])


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(4)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(1, n + 1))
        s = rng.integers(-3, 4, size=n).astype(np.float64)   # many ties
        pages = np.sort(rng.choice(40, size=n, replace=False))
        got = sorted(orc.topk_pages(s, pages, k).tolist())
        assert got == _brute_topk(s, pages, k), (s, pages, k)


def test_topk_ties_go_to_lower_page():
    pages = np.arange(5, 15)
    assert sorted(orc.topk_pages(np.zeros(10), pages, 3).tolist()) == [5, 6, 7]
    s = np.array([1.0, 2.0, 2.0, 0.0, 2.0])
    assert sorted(orc.topk_pages(s, np.arange(5), 2).tolist()) == [1, 2]


def test_select_pages_invariants():
    rng = np.random.default_rng(5)
    for trial in range(50):
        H_kv, G, D = 2, 3, 6
        n_b = int(rng.integers(1, 40))
        topk, bos, eos = int(rng.integers(0, 10)), int(rng.integers(0, 3)), int(rng.integers(1, 3))
        cent = rng.standard_normal((n_b, H_kv, D))
        q = rng.standard_normal((H_kv * G, D))
        sel = orc.select_pages(q, cent, n_b, topk, bos, eos)
        res = set(orc.reserved_pages(n_b, bos, eos).tolist())
        cand = orc.candidate_pages(n_b, bos, eos)
        qbar = orc.group_mean_query(q, H_kv)
        for h in range(H_kv):
            s = set(sel[h].tolist())
            assert res <= s
            assert len(s) == min(n_b, topk + len(res)) if len(cand) > topk else len(s) == n_b
            chosen = [p for p in cand if p in s]
            other = [p for p in cand if p not in s]
            if chosen and other:
                sc = orc.page_scores(qbar, cent, np.arange(n_b))[h]
                assert min(sc[chosen]) >= max(sc[other])
            assert np.all(np.diff(sel[h]) > 0)


def test_selection_table_layout():
    t = orc.selection_table([np.array([4, 0, 9]), np.array([1])], 5)
    assert t.tolist() == [[0, 4, 9, -1, -1], [1, -1, -1, -1, -1]]


# ---------------------------------------------------------------- attention
def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(6)
    G, n, D, Dv = 4, 37, 16, 12
    q, k, v = rng.standard_normal((G, D)), rng.standard_normal((n, D)), rng.standard_normal((n, Dv))
    o, lse = orc.attend(q, k, v, 0.3)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.expand(1, 1, n, D), tv, scale=0.3)[0, 0].numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-13)
    ref_lse = torch.logsumexp(0.3 * torch.from_numpy(q) @ torch.from_numpy(k).T, dim=1).numpy()
    assert np.allclose(lse, ref_lse, rtol=0, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal((2, 8)), rng.standard_normal((1, 8)), rng.standard_normal((1, 5))
    o, lse = orc.attend(q, k, v, 0.5)                         # one key
    assert np.allclose(o, np.repeat(v, 2, 0), rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.5 * q @ k[0], rtol=0, atol=1e-14)
    kk = np.repeat(k, 9, axis=0)                              # equal keys
    vv = rng.standard_normal((9, 5))
    o, lse = orc.attend(q, kk, vv, 0.5)
    assert np.allclose(o, np.repeat(vv.mean(0)[None], 2, 0), rtol=0, atol=1e-14)
    assert np.allclose(lse, 0.5 * q @ k[0] + math.log(9), rtol=0, atol=1e-13)
    big = rng.standard_normal((6, 8)) * 0.01                  # one dominant logit
    big[3] = 50.0 * q[0] / np.linalg.norm(q[0])
    o, _ = orc.attend(q[:1], big, vv[:6], 1.0)
    assert np.allclose(o[0], vv[3], rtol=0, atol=1e-12)
    # large logits do not overflow (max is subtracted)
    o, lse = orc.attend(np.full((1, 2), 400.0), np.ones((3, 2)), np.eye(3), 1.0)
    assert np.allclose(o, 1 / 3, rtol=0, atol=1e-15) and np.isclose(lse[0], 800.0 + math.log(3), rtol=0, atol=1e-12)


def test_two_token_closed_form():
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [2.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, lse = orc.attend(q, k, v, 1.0)
    w1 = math.exp(2) / (1 + math.exp(2))
    assert np.allclose(o[0], [1 - w1, w1], rtol=0, atol=1e-15)
    assert math.isclose(lse[0], math.log(1 + math.exp(2)), rel_tol=1e-15)


def test_merge_partials_equals_whole():
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((3, 8)), rng.standard_normal((50, 8)), rng.standard_normal((50, 6))
    o, lse = orc.attend(q, k, v, 0.7)
    for cuts in ([25], [1, 2, 49], [10, 20, 30, 40]):
        parts = np.split(np.arange(50), cuts)
        res = [orc.attend(q, k[p], v[p], 0.7) for p in parts]
        mo, ml = orc.merge_partials([r[0] for r in res], [r[1] for r in res])
        assert np.allclose(mo, o, rtol=0, atol=1e-13) and np.allclose(ml, lse, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- paged decode
def _pool_and_table(rng, n_b, H, S, D, P):
    pool = rng.standard_normal((P, H, S, D))
    pt = rng.permutation(P)[:n_b]
    return pool, pt


def test_paged_decode_equals_contiguous_textbook():
    rng = np.random.default_rng(9)
    H_kv, G, S, D, L = 2, 2, 16, 8, 71
    n_b = -(-L // S)
    kp, pt = _pool_and_table(rng, n_b, H_kv, S, D, 20)
    vp = rng.standard_normal(kp.shape)
    q = rng.standard_normal((H_kv * G, D))
    o, lse = orc.decode_request(q, kp[pt], vp[pt], L, 0.25)
    for hq in range(H_kv * G):
        h = hq // G
        keys = np.concatenate([kp[pt[p], h] for p in range(n_b)])[:L]
        vals = np.concatenate([vp[pt[p], h] for p in range(n_b)])[:L]
        lg = 0.25 * keys @ q[hq]
        w = np.exp(lg - lg.max())
        assert np.allclose(o[hq], w @ vals / w.sum(), rtol=0, atol=1e-13)
        assert np.isclose(lse[hq], lg.max() + np.log(w.sum()), rtol=0, atol=1e-13)


def test_tokens_beyond_seq_len_are_ignored():
    rng = np.random.default_rng(10)
    kp = rng.standard_normal((4, 1, 16, 8))
    vp = rng.standard_normal((4, 1, 16, 8))
    q = rng.standard_normal((2, 8))
    o1, l1 = orc.decode_request(q, kp, vp, 50, 0.3)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[3, :, 2:] = 1e6
    vp2[3, :, 2:] = np.nan
    o2, l2 = orc.decode_request(q, kp2, vp2, 50, 0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_single_token_context():
    rng = np.random.default_rng(11)
    kp, vp = rng.standard_normal((1, 1, 16, 8)), rng.standard_normal((1, 1, 16, 8))
    q = rng.standard_normal((2, 8))
    o, lse = orc.decode_request(q, kp, vp, 1, 0.3)
    assert np.allclose(o, np.repeat(vp[0, 0, :1], 2, 0), rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.3 * q @ kp[0, 0, 0], rtol=0, atol=1e-14)


def test_mla_values_alias_keys():
    rng = np.random.default_rng(12)
    kp = rng.standard_normal((3, 1, 4, 10))
    q = rng.standard_normal((5, 10))
    o, lse = orc.decode_request(q, kp, None, 11, 0.2, v_dims=6)
    o2, lse2 = orc.decode_request(q, kp, np.ascontiguousarray(kp[..., :6]), 11, 0.2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_sparse_equals_dense_when_topk_covers_candidates():
    rng = np.random.default_rng(13)
    H_kv, G, S, D, L = 2, 4, 16, 8, 16 * 9 + 5
    n_b = -(-L // S)
    kp = rng.standard_normal((n_b, H_kv, S, D))
    vp = rng.standard_normal((n_b, H_kv, S, D))
    q = rng.standard_normal((H_kv * G, D))
    cent = orc.request_centroids(kp, L, "bf16")
    dense = orc.decode_request(q, kp, vp, L, 0.3)
    for topk in (n_b - 2, n_b, 100):
        sel, o, lse = orc.sparse_decode_request(q, kp, vp, cent, L, 0.3, topk, 1, 1)
        assert all(len(s) == n_b for s in sel)
        assert np.allclose(o, dense[0], rtol=0, atol=1e-12) and np.allclose(lse, dense[1], rtol=0, atol=1e-12)


def test_sparse_differs_from_dense_when_pages_dropped():
    rng = np.random.default_rng(14)
    kp = rng.standard_normal((12, 1, 16, 8))
    vp = rng.standard_normal((12, 1, 16, 8))
    q = rng.standard_normal((2, 8))
    cent = orc.request_centroids(kp, 190, "f32")
    sel, o, _ = orc.sparse_decode_request(q, kp, vp, cent, 190, 0.3, 3, 1, 1)
    assert len(sel[0]) == 5
    assert not np.allclose(o, orc.decode_request(q, kp, vp, 190, 0.3)[0])


def test_hand_worked_example():
    """One request, 2 query heads on 1 KV head, D = 2, 2-token pages, 7
    tokens (4 pages, the last holding one token), top-1 + 1 BOS + 1 EOS.

    keys by page: [1,0],[3,0] | [0,2],[0,4] | [2,2],[4,4] | [5,5]
    centroids of full pages: [2,0], [0,3], [3,3]; queries [1,0] and [1,2]
    give the mean query [1,1]; candidates are pages 1 and 2 with scores 3
    and 6, so page 2 wins and the selection is {0, 2, 3}.  Head 0 then sees
    logits (scale 1) 1, 3, 2, 4, 5 and head 1 sees 1, 3, 6, 12, 15."""
    keys = np.array([[1, 0], [3, 0], [0, 2], [0, 4], [2, 2], [4, 4], [5, 5], [0, 0]], float)
    vals = np.array([[1, 0], [0, 1], [9, 9], [9, 9], [2, 0], [0, 2], [1, 1], [7, 7]], float)
    kp = keys.reshape(4, 1, 2, 2)
    vp = vals.reshape(4, 1, 2, 2)
    q = np.array([[1.0, 0.0], [1.0, 2.0]])
    cent = orc.request_centroids(kp, 7, "f32")
    assert np.array_equal(cent[:3, 0], [[2, 0], [0, 3], [3, 3]]) and np.all(np.isnan(cent[3]))
    sel, o, lse = orc.sparse_decode_request(q, kp, vp, cent, 7, 1.0, 1, 1, 1)
    assert sel[0].tolist() == [0, 2, 3]
    used_v = np.array([[1, 0], [0, 1], [2, 0], [0, 2], [1, 1]], float)
    for hq, lg in enumerate(([1, 3, 2, 4, 5], [1, 3, 6, 12, 15])):
        e = [math.exp(x) for x in lg]
        z = sum(e)
        want = [sum(e[i] * used_v[i][d] for i in range(5)) / z for d in range(2)]
        assert np.allclose(o[hq], want, rtol=1e-14, atol=0)
        assert math.isclose(lse[hq], math.log(z), rel_tol=1e-15)


def test_selection_is_per_kv_head():
    # head 0's centroids favour page 1, head 1's favour page 2
    cent = np.zeros((4, 2, 1))
    cent[1, 0, 0], cent[2, 1, 0] = 5.0, 5.0
    cent[2, 0, 0], cent[1, 1, 0] = 1.0, 1.0
    q = np.ones((2, 1))
    sel = orc.select_pages(q, cent, 4, 1, 1, 1)
    assert sel[0].tolist() == [0, 1, 3] and sel[1].tolist() == [0, 2, 3]


def test_page_table_permutation_invariance():
    rng = np.random.default_rng(15)
    P, n_b, H, S, D, L = 30, 9, 2, 16, 8, 140
    pool = rng.standard_normal((P, H, S, D))
    vpool = rng.standard_normal((P, H, S, D))
    pt = rng.permutation(P)[:n_b]
    q = rng.standard_normal((4, D))
    a = orc.sparse_decode_request(q, pool[pt], vpool[pt],
                                  orc.request_centroids(pool[pt], L, "f32"), L, 0.3, 3, 1, 1)
    perm = rng.permutation(P)                 # move every physical page
    pool2 = np.empty_like(pool)
    vpool2 = np.empty_like(vpool)
    pool2[perm] = pool
    vpool2[perm] = vpool
    pt2 = perm[pt]
    b = orc.sparse_decode_request(q, pool2[pt2], vpool2[pt2],
                                  orc.request_centroids(pool2[pt2], L, "f32"), L, 0.3, 3, 1, 1)
    assert all(np.array_equal(x, y) for x, y in zip(a[0], b[0]))
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
