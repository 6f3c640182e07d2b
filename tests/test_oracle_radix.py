"""Pins of the lossy radix top-k oracle (oracle/radix_topk.py) against things
other than itself: Python's own float order, an independent closed form of
the boundary bin, brute force over every random start, the exact top-k, and
a hand-worked example (tests/golden/radix_topk_example.json)."""

import json
import os

import numpy as np
import pytest

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _special_floats(rng, n):
    x = np.concatenate([
        rng.standard_normal(n).astype(np.float32),
        (rng.standard_normal(n) * 1e-38).astype(np.float32),          # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0, 1.5, 2.0, 3.0,
                  np.finfo(np.float32).max, -np.finfo(np.float32).max,
                  np.finfo(np.float32).tiny, -np.finfo(np.float32).tiny], np.float32),
    ])
    return x


def test_order_keys_follow_float_order():
    rng = np.random.default_rng(1)
    x = _special_floats(rng, 3000)
    k = orc.order_keys(x)
    assert k.min() >= 0 and k.max() < 2 ** 32
    # pairwise on a sample: key order equals the float order, ties included
    i = rng.integers(0, len(x), 20000)
    j = rng.integers(0, len(x), 20000)
    for a, b in zip(i, j):
        fa, fb = float(x[a]), float(x[b])
        assert (k[a] > k[b]) == (fa > fb) and (k[a] == k[b]) == (fa == fb)
    assert orc.order_keys(np.float32(-0.0)) == orc.order_keys(np.float32(0.0))


def _prefix(keys, levels):
    return keys >> np.uint64(32 - 10 * levels)


@pytest.mark.parametrize("levels", [1, 2])
def test_boundary_is_the_bin_of_the_kth_largest_key(levels):
    """Closed form: after L levels the boundary bin is the 10L-bit prefix
    class of the k-th largest key; the places left are k minus the keys of
    larger prefix; the bin is taken whole iff all its members fit."""
    rng = np.random.default_rng(2 + levels)
    for trial in range(300):
        n = int(rng.integers(2, 400))
        k = int(rng.integers(1, n))
        scale = 10.0 ** rng.uniform(-3, 3)
        s = (rng.standard_normal(n) * scale + rng.uniform(-2, 2) * scale).astype(np.float32)
        if trial % 3 == 0:                       # many equal prefixes
            s = np.round(s * 8) / 8
        keys = orc.order_keys(s)
        lo, hi, take, whole = orc.radix_boundary(keys, k, levels)
        kth = np.sort(keys)[::-1][k - 1]
        for lev in range(1, levels + 1):        # the search stops at a whole bin
            shift = 32 - 10 * lev
            P = kth >> np.uint64(shift)
            pre = _prefix(keys, lev)
            above = int((pre > P).sum())
            members = int((pre == P).sum())
            if members == k - above or lev == levels:
                break
        assert lo == int(P) << shift and hi == lo + (1 << shift) - 1
        assert take == k - above
        assert whole == (members == take)


def test_whole_boundary_bin_gives_the_exact_topk():
    rng = np.random.default_rng(5)
    hits = 0
    for trial in range(400):
        n = int(rng.integers(5, 300))
        k = int(rng.integers(1, n))
        s = rng.standard_normal(n).astype(np.float32)
        pages = np.arange(3, 3 + n)
        keys = orc.order_keys(s)
        for levels in (1, 2):
            _, _, _, whole = orc.radix_boundary(keys, k, levels)
            if whole:
                hits += 1
                got = orc.radix_topk_pages(s, pages, k, levels, int(rng.integers(0, 2 ** 32)))
                want = np.sort(orc.topk_pages(s.astype(np.float64), pages, k))
                assert np.array_equal(got, want)
    assert hits > 100


def test_brute_force_every_random_start():
    """Tiny inputs: for every start r the members taken are the cyclic run of
    ranks r mod N .. in page order; over N consecutive starts every member is
    taken equally often (the fill does not favour any page)."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(4, 12))
        k = int(rng.integers(1, n))
        s = rng.choice(np.array([1.0, 1.1, 1.2, 1.3, 1.4, 2.5, 3.0, 0.5], np.float32), n)
        pages = rng.permutation(np.arange(10, 10 + n))
        keys = orc.order_keys(s)
        lo, hi, take, whole = orc.radix_boundary(keys, k, 1)
        members = np.sort(pages[(keys >= lo) & (keys <= hi)])
        above = set(pages[keys > hi].tolist())
        N = len(members)
        counts = {int(p): 0 for p in members}
        for r in range(N):
            got = orc.radix_topk_pages(s, pages, k, 1, r + N * int(rng.integers(0, 1000)))
            assert len(got) == k
            assert above <= set(got.tolist())
            chosen = [int(p) for p in got if int(p) not in above]
            want = [int(members[(r + i) % N]) for i in range(take)] if not whole else \
                [int(p) for p in members]
            assert sorted(chosen) == sorted(want)
            for p in chosen:
                counts[p] += 1
        if not whole:
            assert set(counts.values()) == {take}


def test_few_candidates_and_zero_k():
    s = np.array([3.0, 1.0, 2.0], np.float32)
    p = np.array([4, 5, 6])
    assert np.array_equal(orc.radix_topk_pages(s, p, 3, 1, 9), [4, 5, 6])
    assert np.array_equal(orc.radix_topk_pages(s, p, 5, 2, 9), [4, 5, 6])
    assert len(orc.radix_topk_pages(s, p, 0, 1, 9)) == 0


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "radix_topk_example.json")))
    s = np.array(g["scores"], np.float32)
    p = np.array(g["pages"])
    assert orc.radix_topk_pages(s, p, g["k"], 1, g["rnd"]).tolist() == g["levels_1"]["selected"]
    assert orc.radix_topk_pages(s, p, g["k"], 2, g["rnd"]).tolist() == g["levels_2"]["selected"]
    exact = np.sort(orc.topk_pages(s.astype(np.float64), p, g["k"])).tolist()
    assert exact == g["exact_top3"]
    key = int(orc.order_keys(np.float32(1.4)))
    assert (key >> 12) & 1023 == g["levels_2"]["level1_bin_of_1.4"]


def test_select_pages_radix_reserves_and_unites():
    rng = np.random.default_rng(11)
    H_kv, G, D, n_b = 2, 2, 8, 40
    cent = rng.standard_normal((n_b, H_kv, D))
    q = rng.standard_normal((H_kv * G, D))
    sel = orc.select_pages_radix(q, cent, n_b, 5, 1, 2, 1, [3, 4])
    for h in range(H_kv):
        assert {0, n_b - 2, n_b - 1} <= set(sel[h].tolist())
        assert len(sel[h]) == 5 + 3
        assert np.all(np.diff(sel[h]) > 0)
