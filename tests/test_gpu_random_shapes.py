"""GPU parity over seeded random shapes: dtype, head dim, KV heads, group
size, page size, batch, ragged lengths (down to one token), top-k and the
reserved first / last page counts all drawn per case (MLA cases: batch,
lengths, query heads, top-k and reserved pages; 16 more through the
bound-rule step).  Each case runs the
decode step (fused or split, whichever the shape gets), the separate
indexer, and the dense decode, and compares every request with the fp64
oracle: selections bit for bit, outputs and lse within the usual bars, the
completed pages' centroids within one unit in the last place."""

import numpy as np
import pytest
import torch

import oracle as orc
import synth
from tests import _harness as H

pytestmark = pytest.mark.gpu

N_CASES = 64
N_MLA_CASES = 8
N_BOUNDS_CASES = 16


@pytest.fixture(scope="module")
def vx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_paged_amd as m
    m.load_library()
    return m


def _draw(seed):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x5EED]))
    dtype = str(rng.choice(["bf16", "f32"]))
    D = int(rng.choice([64, 128]))
    H_kv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.choice([16, 64]))
    B = int(rng.integers(1, 41))
    lens = tuple(int(x) for x in rng.integers(1, 2500, size=B))
    topk = int(rng.integers(0, 61))
    n_bos = int(rng.integers(0, 3))
    n_eos = int(rng.integers(1, 4))
    return synth.Workload(name=f"random{seed}", batch=B, num_q_heads=H_kv * G, num_kv_heads=H_kv,
                          head_dim_qk=D, head_dim_v=D, page_size=S, dtype=dtype, topk=topk,
                          structure="page_offset", seed=300 + seed, seq_lens=lens, n_bos=n_bos,
                          n_eos=n_eos, spare_pages=4)


def _draw_mla(seed):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x3A1A]))
    B = int(rng.integers(1, 17))
    return synth.WORKLOADS["mla_b64_l32k"].with_(
        name=f"random_mla{seed}", batch=B, seq_len=None,
        seq_lens=tuple(int(x) for x in rng.integers(1, 9000, size=B)),
        num_q_heads=int(rng.choice([8, 16, 32])), topk=int(rng.integers(0, 41)),
        n_bos=int(rng.integers(0, 3)), n_eos=int(rng.integers(1, 3)), seed=400 + seed,
        spare_pages=4)


def _check(c, b, sel, out, lse, sparse):
    sel_ref, o_ref, lse_ref = H.oracle_request(c, b, sparse)
    if sparse:
        got = sel[b].cpu().numpy()
        assert np.array_equal(got, sel_ref), f"request {b}: selected pages differ"
    H.assert_close_out(H.to_f64(out[b]), o_ref, c.w.dtype, f"request {b} out")
    H.assert_close_lse(H.to_f64(lse[b]), lse_ref, c.w.dtype, f"request {b}")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(vx, seed):
    _run(vx, _draw(seed))


@pytest.mark.parametrize("seed", range(N_MLA_CASES))
def test_random_mla_shape(vx, seed):
    _run(vx, _draw_mla(seed))


def _run(vx, w):
    H.log(f"case {H.describe(w)} B={w.batch} bos={w.n_bos} eos={w.n_eos} "
          f"lens={min(w.seq_lens)}..{max(w.seq_lens)}")
    c = H.setup_case(vx, w)
    H.build_setup_centroids(vx, c)
    H.fix_gaps(c, range(w.batch))
    q = c.q_host.cuda()
    sel, out, lse = H.run_step(vx, c, q, update=True)
    sel_ix = H.run_indexer(vx, c, q)
    fo, fl = H.run_full(vx, c, q)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_ix), "the step's selection differs from vx_score_topk's"
    for b in range(w.batch):
        _check(c, b, sel, out, lse, sparse=True)
        _check(c, b, None, fo, fl, sparse=False)
    H.assert_centroids(c, np.concatenate([synth.setup_full_pages(c.layout),
                                          synth.completed_pages(c.layout, 0)]))


# ------------------------------------------------------- the bound rule
def _check_bounds_request(c, b, sel, out, lse):
    w = c.w
    want = H.oracle_selection(c, b, "bounds")
    got = sel[b].cpu().numpy()
    assert np.array_equal(got, want), f"request {b}: selected pages differ"
    k, v = c.request_pages(b)
    _, o_ref, lse_ref = orc.quest_decode_request(
        c.q_host[b].double().numpy(), k, v, c.oracle_bounds(b), int(c.L[b]), w.sm_scale, w.topk,
        w.n_bos, w.n_eos, v_dims=w.head_dim_v if v is None else None)
    H.assert_close_out(H.to_f64(out[b]), o_ref, w.dtype, f"request {b} out")
    H.assert_close_lse(H.to_f64(lse[b]), lse_ref, w.dtype, f"request {b}")


@pytest.mark.parametrize("seed", range(N_BOUNDS_CASES))
def test_random_shape_bounds(vx, seed):
    """The bound-rule step (Quest's key bounds) over random shapes: every
    request's selection and attention against the oracle, the selection
    equal to vx_score_topk_bounds', the completed pages' bounds exact."""
    w = _draw(1000 + seed)
    H.log(f"case {H.describe(w)} B={w.batch} bos={w.n_bos} eos={w.n_eos}")
    c = H.setup_case(vx, w)
    bounds = torch.zeros((c.layout.num_pages, w.num_kv_heads, 2, w.head_dim_qk),
                         dtype=w.torch_dtype, device="cuda")
    ids = synth.setup_full_pages(c.layout)
    if len(ids):
        vx.bounds_update(c.kv, bounds, torch.from_numpy(ids.astype(np.int32)).cuda())
    H.fix_gaps(c, range(w.batch), rule="bounds")
    q = c.q_host.cuda()
    bt = c.batch(vx)
    sel = torch.full((w.batch, w.num_kv_heads, w.k_tot), -7, dtype=torch.int32, device="cuda")
    out = torch.full((w.batch, w.num_q_heads, w.head_dim_v), float("nan"), dtype=w.torch_dtype,
                     device="cuda")
    lse = torch.full((w.batch, w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    vx.sparse_decode_step_bounds(c.kv, bt, bounds, q, w.topk, w.n_bos, w.n_eos, True, w.sm_scale,
                                 sel, out, lse, vx.alloc_workspace(vx.VX_OP_DECODE_STEP, c.kv, bt,
                                                                   w.k_tot))
    sel_ix = torch.full_like(sel, -7)
    vx.score_topk_bounds(c.kv, bt, bounds, q, w.topk, w.n_bos, w.n_eos, sel_ix,
                         vx.alloc_workspace(vx.VX_OP_SCORE_TOPK, c.kv, bt))
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_ix), "the step's selection differs from vx_score_topk_bounds'"
    for b in range(w.batch):
        _check_bounds_request(c, b, sel, out, lse)
    done = np.concatenate([ids, synth.completed_pages(c.layout, 0)])
    if len(done):
        idx = torch.from_numpy(done.astype(np.int64)).cuda()
        assert np.array_equal(H.to_f64(bounds[idx]), orc.page_bounds(H.to_f64(c.K[idx]))), \
            "page bounds differ"
