"""GPU parity of the second page-summary rule (Quest's key bounds) through
the same pipeline: vx_bounds_update against the oracle's per-channel
minimum and maximum (exact), vx_score_topk_bounds and the bound-rule decode
step against the oracle's selection by criticality (bit-exact on every
(request, KV head): query groups are redrawn until the k-th and (k+1)-th
criticalities differ by more than 1e-3 of the largest), and the attention
against the oracle's whole path (its own selection, then attention)."""

import numpy as np
import pytest
import torch

import synth
import oracle as orc
from tests import _harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_paged_amd as m
    m.load_library()
    return m


def _case(vx, w):
    H.log(f"case {H.describe(w)}")
    c = H.setup_case(vx, w)
    bounds = torch.zeros((c.layout.num_pages, w.num_kv_heads, 2, w.head_dim_qk),
                         dtype=w.torch_dtype, device="cuda")
    ids = np.concatenate([synth.setup_full_pages(c.layout), synth.completed_pages(c.layout, 0)])
    vx.bounds_update(c.kv, bounds, torch.from_numpy(ids.astype(np.int32)).cuda())
    return c, bounds, ids


def _check_request(c, b, sel_dev, out=None, lse=None):
    """Request b: the GPU selection equals the oracle's bit for bit; out and
    lse (when given) equal the oracle's quest_decode_request, which selects
    by criticality itself and attends over its own selection."""
    w = c.w
    want = H.oracle_selection(c, b, "bounds")
    got = sel_dev[b].cpu().numpy()
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert len(bad) == 0, f"request {b}: selected pages differ on KV heads {bad.tolist()}"
    if out is None:
        return
    k, v = c.request_pages(b)
    _, o_ref, lse_ref = orc.quest_decode_request(
        c.q_host[b].double().numpy(), k, v, c.oracle_bounds(b), int(c.L[b]), w.sm_scale, w.topk,
        w.n_bos, w.n_eos, v_dims=w.head_dim_v if v is None else None)
    H.assert_close_out(H.to_f64(out[b]), o_ref, w.dtype, f"request {b} out")
    H.assert_close_lse(H.to_f64(lse[b]), lse_ref, w.dtype, f"request {b}")


def _gap_fix(c, requests):
    n = H.fix_gaps(c, requests, rule="bounds")
    H.log(f"  {n} query groups redrawn for the criticality gap")


@pytest.mark.parametrize("name", ["qwen3_small", "long_small", "hetero_small", "tiny_b1_l1k_f32"])
def test_bounds_small(vx, name):
    w = synth.get_workload(name)
    c, bounds, ids = _case(vx, w)
    torch.cuda.synchronize()
    got = H.to_f64(bounds[torch.from_numpy(ids.astype(np.int64)).cuda()])
    want = orc.page_bounds(H.to_f64(c.K[torch.from_numpy(ids.astype(np.int64)).cuda()]))
    assert np.array_equal(got, want), "page bounds differ"
    _gap_fix(c, range(w.batch))
    bt = c.batch(vx)
    sel = torch.full((w.batch, w.num_kv_heads, w.k_tot), -7, dtype=torch.int32, device="cuda")
    ws = vx.alloc_workspace(vx.VX_OP_SCORE_TOPK, c.kv, bt)
    q = c.q_host.cuda()
    vx.score_topk_bounds(c.kv, bt, bounds, q, w.topk, w.n_bos, w.n_eos, sel, ws)
    out, lse = H.run_sparse(vx, c, q, sel)
    torch.cuda.synchronize()
    for b in range(w.batch):
        _check_request(c, b, sel, out, lse)


def test_bounds_full_size_sampled(vx):
    """The Qwen-like layer at full size (32 requests of 32768 tokens): the
    summary of every full page exact, every request's selection bit-exact,
    the attention of two sampled requests against the oracle's whole path."""
    w = synth.get_workload("qwen3_0p6b_b32_l32k")
    c, bounds, ids = _case(vx, w)
    H.prime_bounds_device(c, range(w.batch))
    _gap_fix(c, range(w.batch))
    bt = c.batch(vx)
    sel = torch.full((w.batch, w.num_kv_heads, w.k_tot), -7, dtype=torch.int32, device="cuda")
    ws = vx.alloc_workspace(vx.VX_OP_SCORE_TOPK, c.kv, bt)
    q = c.q_host.cuda()
    vx.score_topk_bounds(c.kv, bt, bounds, q, w.topk, w.n_bos, w.n_eos, sel, ws)
    out, lse = H.run_sparse(vx, c, q, sel)
    torch.cuda.synchronize()
    for b in range(w.batch):
        phys = torch.from_numpy(c.layout.page_table[b, :int(c.L[b]) // w.page_size].astype(np.int64)).cuda()
        assert torch.equal(bounds[phys, :, 0], c.K[phys].amin(dim=2))
        assert torch.equal(bounds[phys, :, 1], c.K[phys].amax(dim=2))
        assert c.n_pages(b) > w.k_tot
        _check_request(c, b, sel)
    for b in (0, w.batch - 1):
        H.log(f"  request {b}")
        _check_request(c, b, sel, out, lse)


def test_bounds_rejects_mla(vx):
    w = synth.get_workload("mla_small")
    c = H.setup_case(vx, w)
    bounds = torch.zeros((c.layout.num_pages, 1, 2, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vx.VxError) as e:
        vx.bounds_update(c.kv, bounds, torch.zeros(1, dtype=torch.int32, device="cuda"))
    assert e.value.status == vx.VX_ERR_UNSUPPORTED


@pytest.mark.parametrize("topk,bos,eos", [(4, 1, 1), (0, 1, 1), (3, 0, 2)])
@pytest.mark.parametrize("dtype,D,G,S", [("f32", 64, 1, 16), ("bf16", 128, 8, 16),
                                         ("bf16", 64, 4, 64), ("f32", 128, 2, 16)])
def test_bounds_edge_lengths(vx, dtype, D, G, S, topk, bos, eos):
    """Ragged and tiny requests (fewer candidates than k, none at all, a
    partial last page) through the bound indexer and the attention."""
    lens = (1, S - 1, S, S + 1, S * 6, S * 6 + 1, S * 9 + 3)
    w = synth.Workload(name="edges", batch=len(lens), num_q_heads=2 * G, num_kv_heads=2,
                       head_dim_qk=D, head_dim_v=D, page_size=S, dtype=dtype, topk=topk,
                       structure="page_offset", seed=81, seq_lens=lens, n_bos=bos, n_eos=eos,
                       spare_pages=5)
    c, bounds, ids = _case(vx, w)
    _gap_fix(c, range(w.batch))
    bt = c.batch(vx)
    sel = torch.full((w.batch, w.num_kv_heads, w.k_tot), -7, dtype=torch.int32, device="cuda")
    ws = vx.alloc_workspace(vx.VX_OP_SCORE_TOPK, c.kv, bt)
    q = c.q_host.cuda()
    vx.score_topk_bounds(c.kv, bt, bounds, q, w.topk, w.n_bos, w.n_eos, sel, ws)
    out, lse = H.run_sparse(vx, c, q, sel)
    torch.cuda.synchronize()
    for b in range(w.batch):
        _check_request(c, b, sel, out, lse)


# ------------------------------------------------------- the step, bound rule
def _setup_bounds(vx, c):
    """Bounds of the pages full before step 0's token only."""
    w = c.w
    bounds = torch.zeros((c.layout.num_pages, w.num_kv_heads, 2, w.head_dim_qk),
                         dtype=w.torch_dtype, device="cuda")
    ids = synth.setup_full_pages(c.layout)
    if len(ids):
        vx.bounds_update(c.kv, bounds, torch.from_numpy(ids.astype(np.int32)).cuda())
    return bounds


def _run_step_bounds(vx, c, bounds, q, update=True):
    w = c.w
    bt = c.batch(vx)
    sel = torch.full((w.batch, w.num_kv_heads, w.k_tot), -7, dtype=torch.int32, device="cuda")
    out = torch.full((w.batch, w.num_q_heads, w.head_dim_v), float("nan"), dtype=w.torch_dtype,
                     device="cuda")
    lse = torch.full((w.batch, w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    ws = vx.alloc_workspace(vx.VX_OP_DECODE_STEP, c.kv, bt, w.k_tot)
    vx.sparse_decode_step_bounds(c.kv, bt, bounds, q, w.topk, w.n_bos, w.n_eos, update,
                                 w.sm_scale, sel, out, lse, ws)
    return sel, out, lse


def _assert_bounds(c, bounds, ids):
    idx = torch.from_numpy(np.asarray(ids).astype(np.int64)).cuda()
    assert np.array_equal(H.to_f64(bounds[idx]), orc.page_bounds(H.to_f64(c.K[idx]))), \
        "page bounds differ"


@pytest.mark.parametrize("name", ["qwen3_small", "long_small", "hetero_small", "tiny_b1_l1k_f32"])
def test_step_bounds_equals_separate_calls(vx, name):
    """vx_sparse_decode_step_bounds == bounds of the completed pages +
    vx_score_topk_bounds + vx_sparse_paged_decode, and matches the oracle."""
    w = synth.get_workload(name)
    H.log(f"case {H.describe(w)}")
    c = H.setup_case(vx, w)
    bounds = _setup_bounds(vx, c)
    _gap_fix(c, range(w.batch))
    q = c.q_host.cuda()
    before = bounds.clone()
    done = synth.completed_pages(c.layout, 0)
    if len(done):
        vx.bounds_update(c.kv, bounds, torch.from_numpy(done.astype(np.int32)).cuda())
    bt = c.batch(vx)
    sel1 = torch.full((w.batch, w.num_kv_heads, w.k_tot), -7, dtype=torch.int32, device="cuda")
    vx.score_topk_bounds(c.kv, bt, bounds, q, w.topk, w.n_bos, w.n_eos, sel1,
                         vx.alloc_workspace(vx.VX_OP_SCORE_TOPK, c.kv, bt))
    out1, lse1 = H.run_sparse(vx, c, q, sel1)
    after = bounds.clone()
    bounds.copy_(before)
    sel2, out2, lse2 = _run_step_bounds(vx, c, bounds, q)
    torch.cuda.synchronize()
    assert torch.equal(sel1, sel2)
    assert torch.equal(after, bounds)
    if H.single_split(vx, c):
        assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    else:
        assert (out1.float() - out2.float()).abs().max().item() <= (1e-5 if w.dtype == "f32" else 1e-2)
    for b in range(w.batch):
        _check_request(c, b, sel2, out2, lse2)
    _assert_bounds(c, bounds, np.concatenate([synth.setup_full_pages(c.layout), done]))


@pytest.mark.parametrize("topk,bos,eos", [(4, 1, 1), (0, 1, 1), (3, 0, 2)])
@pytest.mark.parametrize("dtype,D,G,S", [("f32", 64, 1, 16), ("bf16", 128, 8, 16),
                                         ("bf16", 64, 4, 64), ("f32", 128, 2, 16)])
def test_step_bounds_edge_lengths(vx, dtype, D, G, S, topk, bos, eos):
    """Ragged and tiny requests through the bound-rule step (one fused
    kernel here): selection, attention and the completed pages' bounds."""
    lens = (1, S - 1, S, S + 1, S * 6, S * 6 + 1, S * 9 + 3)
    w = synth.Workload(name="edges", batch=len(lens), num_q_heads=2 * G, num_kv_heads=2,
                       head_dim_qk=D, head_dim_v=D, page_size=S, dtype=dtype, topk=topk,
                       structure="page_offset", seed=82, seq_lens=lens, n_bos=bos, n_eos=eos,
                       spare_pages=5)
    H.log(f"case {H.describe(w)} lens={lens} bos={bos} eos={eos}")
    c = H.setup_case(vx, w)
    bounds = _setup_bounds(vx, c)
    _gap_fix(c, range(w.batch))
    q = c.q_host.cuda()
    sel, out, lse = _run_step_bounds(vx, c, bounds, q)
    torch.cuda.synchronize()
    for b in range(w.batch):
        _check_request(c, b, sel, out, lse)
    _assert_bounds(c, bounds, np.concatenate([synth.setup_full_pages(c.layout),
                                              synth.completed_pages(c.layout, 0)]))


def test_step_bounds_many_units(vx):
    """Two or more units per CU: the bound-rule step's 4-wave blocks, taken
    longest request first, against the bound indexer and the oracle."""
    batch, H_kv, G = 80, 8, 2
    rng = np.random.default_rng(batch)
    seq_lens = tuple(int(x) for x in rng.choice((1, 15, 16, 17, 200, 513, 1600), size=batch))
    w = synth.Workload(name="many_units", batch=batch, num_q_heads=H_kv * G, num_kv_heads=H_kv,
                       head_dim_qk=128, head_dim_v=128, page_size=16, dtype="bf16", topk=6,
                       structure="page_offset", seed=83, seq_lens=seq_lens, spare_pages=4)
    H.log(f"case {H.describe(w)}")
    c = H.setup_case(vx, w)
    bounds = _setup_bounds(vx, c)
    _gap_fix(c, range(w.batch))
    q = c.q_host.cuda()
    sel, out, lse = _run_step_bounds(vx, c, bounds, q)
    bt = c.batch(vx)
    sel1 = torch.full_like(sel, -7)
    vx.score_topk_bounds(c.kv, bt, bounds, q, w.topk, w.n_bos, w.n_eos, sel1,
                         vx.alloc_workspace(vx.VX_OP_SCORE_TOPK, c.kv, bt))
    torch.cuda.synchronize()
    assert torch.equal(sel, sel1)
    for b in range(w.batch):
        _check_request(c, b, sel, out, lse)
    _assert_bounds(c, bounds, np.concatenate([synth.setup_full_pages(c.layout),
                                              synth.completed_pages(c.layout, 0)]))


def test_step_bounds_full_size_sampled(vx):
    """The Qwen-like layer at full size through the bound-rule step: the
    completed pages' bounds exact, every request's selection bit-exact, two
    sampled requests' attention against the oracle's whole path."""
    w = synth.get_workload("qwen3_0p6b_b32_l32k")
    H.log(f"case {H.describe(w)}")
    c = H.setup_case(vx, w)
    bounds = _setup_bounds(vx, c)
    H.prime_bounds_device(c, range(w.batch))
    _gap_fix(c, range(w.batch))
    q = c.q_host.cuda()
    sel, out, lse = _run_step_bounds(vx, c, bounds, q)
    torch.cuda.synchronize()
    for b in range(w.batch):
        _check_request(c, b, sel)
    for b in (0, w.batch - 1):
        H.log(f"  request {b}")
        _check_request(c, b, sel, out, lse)
    done = synth.completed_pages(c.layout, 0)
    if len(done):
        _assert_bounds(c, bounds, done)


@pytest.mark.parametrize("name", ["qwen3_small", "long_small", "hetero_small"])
def test_device_bounds_shortcut(vx, name):
    """The full-size tests take oracle key bounds from minima and maxima
    taken on the device: on the small workloads they equal
    orc.request_bounds on the host bit for bit."""
    w = synth.get_workload(name)
    c = H.setup_case(vx, w)
    fast = H.Case(**{**c.__dict__, "_oracle_cent": {}, "_oracle_bounds": {}})
    H.prime_bounds_device(fast, range(w.batch))
    for b in range(w.batch):
        want, got = c.oracle_bounds(b), fast.oracle_bounds(b)
        assert np.array_equal(np.isnan(got), np.isnan(want))
        m = ~np.isnan(want)
        assert np.array_equal(got[m], want[m]), f"request {b}"


def test_step_bounds_rejects_mla(vx):
    w = synth.get_workload("mla_small")
    c = H.setup_case(vx, w)
    bounds = torch.zeros((c.layout.num_pages, 1, 2, 576), dtype=torch.bfloat16, device="cuda")
    bt = c.batch(vx)
    sel = torch.empty((w.batch, 1, w.k_tot), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim_v), dtype=torch.bfloat16, device="cuda")
    ws = vx.alloc_workspace(vx.VX_OP_DECODE_STEP, c.kv, bt, w.k_tot)
    with pytest.raises(vx.VxError) as e:
        vx.sparse_decode_step_bounds(c.kv, bt, bounds, c.q_host.cuda(), w.topk, w.n_bos,
                                     w.n_eos, True, w.sm_scale, sel, out, None, ws)
    assert e.value.status == vx.VX_ERR_UNSUPPORTED
