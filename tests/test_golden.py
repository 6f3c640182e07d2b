"""Fixtures under tests/golden: the parameter values the pages print, and a
stored oracle result that guards the oracle against silent drift."""

import json
import os

import numpy as np

import oracle as orc
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_workloads_use_the_pages_serving_parameters():
    g = _load("pages_parameters.json")
    qwen = synth.WORKLOADS["qwen3_0p6b_b32_l32k"]
    assert qwen.page_size == g["page_size"]["value"]
    assert qwen.topk == g["topk_pages"]["value"]
    for w in synth.WORKLOADS.values():
        assert w.n_bos == g["reserved_bos_pages"]["value"]
        assert w.n_eos == g["reserved_eos_pages"]["value"]
        if w.structure != "mla":
            assert w.page_size == g["page_size"]["value"]


def test_centroid_row_is_head_dim_wide_per_page():
    g = _load("pages_parameters.json")
    assert g["centroid_cache_entry"]["value"][0] == 1
    k = np.zeros((5, 3, 16, 40))
    assert orc.page_centroids(k, "bf16").shape == (5, 3, 40)   # one row per page, per KV head


def test_oracle_matches_stored_golden():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_oracle_golden", os.path.join(GOLDEN, "make_oracle_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    got = mod.compute(mod.inputs())
    want = _load("oracle_small.json")
    assert got["selected"] == want["selected"]
    for key in ("centroids", "o", "lse", "o_dense", "lse_dense"):
        assert np.allclose(got[key], want[key], rtol=0, atol=1e-14), key
