"""Seeded input generators: determinism, page-table validity, the step
schedule of appended tokens, and the value structure of each workload."""

import numpy as np
import pytest
import torch

import synth


@pytest.mark.parametrize("name", list(synth.SMALL_WORKLOADS))
def test_same_seed_same_bytes(name):
    w = synth.get_workload(name)
    a, b = synth.build_layout(w), synth.build_layout(w)
    assert np.array_equal(a.page_table, b.page_table)
    ka, va = synth.make_kv_pool(w, a)
    kb, vb = synth.make_kv_pool(w, b)
    assert torch.equal(ka, kb) and (va is None or torch.equal(va, vb))
    assert torch.equal(synth.make_queries(w, a, 0), synth.make_queries(w, b, 0))
    if w.steps > 1:
        assert not torch.equal(synth.make_queries(w, a, 0), synth.make_queries(w, a, 1))


@pytest.mark.parametrize("name", list(synth.SMALL_WORKLOADS))
def test_page_table_is_injective_into_pool(name):
    w = synth.get_workload(name)
    lay = synth.build_layout(w)
    final = lay.seq_lens0 + w.steps - 1
    used = []
    for b in range(w.batch):
        n = -(-int(final[b]) // w.page_size)
        used.extend(lay.page_table[b, :n].tolist())
    assert len(used) == len(set(used))
    assert min(used) >= 0 and max(used) < lay.num_pages


def test_full_size_layouts_shapes():
    for name, w in synth.WORKLOADS.items():
        lay = synth.build_layout(w)
        if name == "qwen3_0p6b_b32_l32k":
            assert lay.num_pages == 65536 and lay.max_pages == 2048
        if name == "tiny_b1_l1k_f32":
            assert lay.num_pages == 128 and lay.max_pages == 64
        if name == "long_b8_l128k":
            assert lay.num_pages == 65536 and lay.max_pages == 8192
        if name == "mla_b64_l32k":
            assert lay.num_pages == 32768 and lay.max_pages == 512
        if name == "hetero_b128_l4k_64k":
            L = lay.seq_lens0
            assert L.min() >= 4096 and L.max() <= 65536 and len(L) == 128
            assert lay.max_pages == -(-(int(L.max()) + 31) // 16)


def test_append_schedule_and_completions():
    w = synth.SMALL_WORKLOADS["hetero_small"]
    lay = synth.build_layout(w)
    S = w.page_size
    done = set(synth.setup_full_pages(lay).tolist())
    for s in range(w.steps):
        L = synth.step_seq_lens(lay, s)
        for p in synth.completed_pages(lay, s).tolist():
            assert p not in done
            done.add(p)
        # after step s every page below L // S is complete
        want = set()
        for b in range(w.batch):
            want.update(lay.page_table[b, :L[b] // S].tolist())
        assert done == want


def test_page_offsets_make_page_means_informative():
    w = synth.SMALL_WORKLOADS["qwen3_small"]
    lay = synth.build_layout(w)
    K, _ = synth.make_kv_pool(w, lay)
    m = K.float().mean(dim=2)                     # [P, H, D]
    # per-page mean spread ~ sqrt(0.5^2 + 1/16) = 0.56, not 1/4
    assert 0.5 < float(m.std()) < 0.62


def test_clusters_structure():
    w = synth.SMALL_WORKLOADS["long_small"]
    lay = synth.build_layout(w)
    K, _ = synth.make_kv_pool(w, lay)
    m = K.float().mean(dim=2)[:, 0]               # page means of head 0, [P, D]
    # distance between page means: same cluster ~ sqrt(2*128*(0.1^2+1/16)) = 4.3,
    # different clusters ~ sqrt(2*128*(0.5^2+0.1^2+1/16)) = 9.1
    d = torch.cdist(m[:400], m[:400])
    near = (d < 6.5).float().sum(1) - 1           # same-cluster neighbours
    assert 400 / 8 * 0.6 < float(near.mean()) < 400 / 8 * 1.4


def test_mla_rope_part_is_a_rotation_of_gaussian_pairs():
    w = synth.SMALL_WORKLOADS["mla_small"]
    lay = synth.build_layout(w)
    K, V = synth.make_kv_pool(w, lay)
    assert V is None and K.shape[-1] == 576
    q = synth.make_queries(w, lay, 0)
    assert q.shape == (3, 32, 576)
    r = K[..., 512:].float()
    norms = (r[..., :32] ** 2 + r[..., 32:] ** 2)
    assert 1.7 < float(norms.mean()) < 2.3          # rotation keeps E|pair|^2 = 2
