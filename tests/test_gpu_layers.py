"""GPU tests of vx_decode_layers (the attention layers of one decode step
in one call, the layers listed as dense running full attention) and of that
call captured into a HIP graph.  Each layer equals the single-layer call it
stands for bit for bit, a sparse layer matches the oracle, and every replay
of the captured graph equals an eager call on the same inputs (replays with
the program's own eager work and synchronisation between them)."""

import numpy as np
import pytest
import torch

import synth
from tests import _harness as H
from tests.test_gpu_parity import _check_request, _mla_guard

pytestmark = pytest.mark.gpu

N_LAYERS = 3
DENSE = [True, False, False]          # layer 0 full attention, as a skipped layer


@pytest.fixture(scope="module")
def vx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_paged_amd as m
    m.load_library()
    return m


def _layers(vx, name):
    """N_LAYERS cases over one page layout (one batch), each with its own
    K/V pools, centroid table and queries (seeds differ by layer)."""
    w = synth.get_workload(name)
    _mla_guard(vx, w)
    lay = synth.build_layout(w)
    pt = torch.from_numpy(lay.page_table).cuda()
    sl = torch.from_numpy(synth.step_seq_lens(lay, 0).astype(np.int32)).cuda()
    cases = []
    for l in range(N_LAYERS):
        wl = w.with_(seed=w.seed + 7919 * l)
        K, V = synth.make_kv_pool(wl, lay, device="cuda")
        cent = torch.zeros((lay.num_pages, w.num_kv_heads, w.head_dim_qk), dtype=w.torch_dtype,
                           device="cuda")
        kv = vx.PagedKV(k_cache=K, v_cache=V, centroids=cent, head_dim_v=w.head_dim_v)
        c = H.Case(w=wl, layout=lay, K=K, V=V, cent=cent, pt=pt, seq_lens=sl, kv=kv)
        c.attempts = np.zeros((w.batch, w.num_kv_heads), dtype=np.int64)
        c.q_host = synth.make_queries(wl, lay, 0)
        H.build_setup_centroids(vx, c)
        H.fix_gaps(c, range(w.batch))
        cases.append(c)
    H.log(f"case {H.describe(w)} x {N_LAYERS} layers, dense {DENSE}")
    return w, cases


def _buffers(w):
    sels = [torch.full((w.batch, w.num_kv_heads, w.k_tot), -7, dtype=torch.int32, device="cuda")
            for _ in range(N_LAYERS)]
    outs = [torch.full((w.batch, w.num_q_heads, w.head_dim_v), float("nan"), dtype=w.torch_dtype,
                       device="cuda") for _ in range(N_LAYERS)]
    lses = [torch.full((w.batch, w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
            for _ in range(N_LAYERS)]
    return sels, outs, lses


def _call(vx, w, cases, qs, bufs, ws, stream=None):
    sels, outs, lses = bufs
    return vx.prepare_decode_layers([c.kv for c in cases], cases[0].batch(vx), qs, DENSE, w.topk,
                                    w.n_bos, w.n_eos, True, w.sm_scale, sels, outs, lses, ws,
                                    stream)


@pytest.mark.parametrize("name", ["qwen3_small", "long_small", "mla_small", "tiny_b1_l1k_f32"])
def test_decode_layers_equals_single_calls(vx, name):
    w, cases = _layers(vx, name)
    qs = [c.q_host.cuda() for c in cases]
    before = [c.cent.clone() for c in cases]
    ref = []
    for l, c in enumerate(cases):
        if DENSE[l]:
            out, lse = H.run_full(vx, c, qs[l])
            ref.append((None, out, lse))
        else:
            ref.append(H.run_step(vx, c, qs[l], update=True))
    torch.cuda.synchronize()
    after = [c.cent.clone() for c in cases]
    for c, b in zip(cases, before):
        c.cent.copy_(b)
    bt = cases[0].batch(vx)
    ws = vx.alloc_workspace(vx.VX_OP_DECODE_LAYERS, cases[0].kv, bt, w.k_tot)
    bufs = _buffers(w)
    _call(vx, w, cases, qs, bufs, ws)()
    torch.cuda.synchronize()
    sels, outs, lses = bufs
    for l in range(N_LAYERS):
        sel_r, out_r, lse_r = ref[l]
        assert torch.equal(outs[l], out_r) and torch.equal(lses[l], lse_r), f"layer {l} output"
        if DENSE[l]:
            assert torch.equal(sels[l], torch.full_like(sels[l], -7)), "dense layer wrote sel"
            assert torch.equal(cases[l].cent, before[l]), "dense layer wrote centroids"
        else:
            assert torch.equal(sels[l], sel_r), f"layer {l} selection"
            assert torch.equal(cases[l].cent, after[l]), f"layer {l} centroid table"
    last = cases[-1]
    for b in H.sample_requests(w.batch):
        _check_request(vx, last, b, sels[-1], outs[-1], lses[-1])
    for b in H.sample_requests(w.batch, 1):
        _check_request(vx, cases[0], b, None, outs[0], lses[0], sparse=False)


@pytest.mark.parametrize("name", ["qwen3_small", "long_small", "mla_small", "tiny_b1_l1k_f32"])
def test_decode_layers_graph_replays(vx, name):
    """Capture once, then three rounds of: new queries written into the
    captured buffers, replay, an eager call on the same inputs into other
    buffers; every replay must equal its eager call bit for bit."""
    w, cases = _layers(vx, name)
    qs = [c.q_host.cuda() for c in cases]
    bt = cases[0].batch(vx)
    ws_g = vx.alloc_workspace(vx.VX_OP_DECODE_LAYERS, cases[0].kv, bt, w.k_tot)
    ws_e = vx.alloc_workspace(vx.VX_OP_DECODE_LAYERS, cases[0].kv, bt, w.k_tot)
    bufs_g, bufs_e = _buffers(w), _buffers(w)
    graph = vx.capture_graph(lambda s: _call(vx, w, cases, qs, bufs_g, ws_g, s))
    gen = torch.Generator(device="cuda").manual_seed(int(w.seed) + 1)
    for rep in range(3):
        for q in qs:
            q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype))
        graph.replay()
        torch.cuda.synchronize()
        _call(vx, w, cases, qs, bufs_e, ws_e)()
        torch.cuda.synchronize()
        for l in range(N_LAYERS):
            for what, g, e in zip(("sel", "out", "lse"), (b[l] for b in bufs_g),
                                  (b[l] for b in bufs_e)):
                assert torch.equal(g, e), f"replay {rep} layer {l} {what}"
        H.log(f"  replay {rep} equal")
