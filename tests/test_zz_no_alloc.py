"""The no-allocation decode step: vx_sparse_decode_step_static (workspace in
the library's static device scratch) called through the C ABI gives what
vx_sparse_decode_step gives with a workspace of its own, bit for bit, on two
calls in a row, the second with a smaller batch; over the fused step, the
split scorer with selection in the split decode, and the MLA path."""

import ctypes

import pytest
import torch

import synth
from tests import _harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_paged_amd as m
    m.load_library()
    return m


def _static_call(vx, c, bt, q, sel, out, lse):
    """vx_sparse_decode_step_static straight through ctypes."""
    w = c.w
    kvs, bs = c.kv.struct(), bt.struct()
    st = vx.load_library().vx_sparse_decode_step_static(
        ctypes.byref(kvs), ctypes.byref(bs), ctypes.c_void_p(q.data_ptr()), w.topk, w.n_bos,
        w.n_eos, 1, ctypes.c_float(w.sm_scale), ctypes.c_void_p(sel.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == vx.VX_OK, vx.status_string(st)


def _outputs(w, B):
    sel = torch.full((B, w.num_kv_heads, w.k_tot), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, w.num_q_heads, w.head_dim_v), float("nan"), dtype=w.torch_dtype,
                     device="cuda")
    lse = torch.full((B, w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    return sel, out, lse


def _reference(vx, c, bt, q):
    w = c.w
    B = bt.page_table.shape[0]
    sel, out, lse = _outputs(w, B)
    ws = vx.alloc_workspace(vx.VX_OP_DECODE_STEP, c.kv, bt, w.k_tot)
    vx.sparse_decode_step(c.kv, bt, q, w.topk, w.n_bos, w.n_eos, True, w.sm_scale, sel, out,
                          lse, ws)
    return sel, out, lse


@pytest.mark.parametrize("name", ["qwen3_small", "long_small", "mla_small", "tiny_b1_l1k_f32"])
def test_static_step_equals_step(vx, name):
    w = synth.get_workload(name)
    H.log(f"case {H.describe(w)}")
    c = H.setup_case(vx, w)
    H.build_setup_centroids(vx, c)
    q = c.q_host.cuda()
    bt = c.batch(vx)
    need = vx.workspace_size(vx.VX_OP_DECODE_STEP, c.kv, bt, w.k_tot)
    assert 0 < need <= vx.STATIC_SCRATCH_BYTES
    cent0 = c.cent.clone()
    # first call: the whole batch
    ref = _reference(vx, c, bt, q)
    cent_ref = c.cent.clone()
    c.cent.copy_(cent0)
    got = _outputs(w, w.batch)
    _static_call(vx, c, bt, q, *got)
    torch.cuda.synchronize()
    assert torch.equal(c.cent, cent_ref), "completed-page centroids differ"
    for x, y, what in zip(ref, got, ("sel", "out", "lse")):
        assert torch.equal(x, y), f"full batch: {what} differs"
    # second call in a row: a smaller batch (the last request alone, shorter)
    b = w.batch - 1
    L = max(int(c.L[b]) - 3 * w.page_size - 1, 1)
    small = vx.Batch(page_table=c.pt[b:b + 1].contiguous(),
                     seq_lens=torch.tensor([L], dtype=torch.int32, device="cuda"),
                     num_q_heads=w.num_q_heads, max_seq_len=L)
    assert vx.workspace_size(vx.VX_OP_DECODE_STEP, c.kv, small, w.k_tot) <= need
    q1 = q[b:b + 1].contiguous()
    ref1 = _reference(vx, c, small, q1)
    got1 = _outputs(w, 1)
    _static_call(vx, c, small, q1, *got1)
    torch.cuda.synchronize()
    for x, y, what in zip(ref1, got1, ("sel", "out", "lse")):
        assert torch.equal(x, y), f"smaller batch: {what} differs"
    assert not torch.isnan(got1[1].float()).any()


def test_static_step_rejects_shapes_beyond_scratch(vx):
    """Shapes whose workspace exceeds the static scratch are refused with
    nothing launched; an empty batch launches nothing either."""
    w = synth.SMALL_WORKLOADS["qwen3_small"]
    c = H.setup_case(vx, w)
    big = vx.Batch(page_table=c.pt, seq_lens=c.seq_lens, num_q_heads=w.num_q_heads,
                   max_seq_len=c.pt.shape[1] * w.page_size)
    kvs = c.kv.struct()
    bs = big.struct()
    bs.batch = 4096
    bs.max_pages_per_req = 16384
    bs.max_seq_len = 16384 * 16
    lib = vx.load_library()
    st = lib.vx_sparse_decode_step_static(ctypes.byref(kvs), ctypes.byref(bs), None, w.topk,
                                          w.n_bos, w.n_eos, 1, ctypes.c_float(0.1), None, None,
                                          None, None)
    assert st == vx.VX_ERR_WORKSPACE_TOO_SMALL
    bs.batch = 0
    st = lib.vx_sparse_decode_step_static(ctypes.byref(kvs), ctypes.byref(bs), None, w.topk,
                                          w.n_bos, w.n_eos, 1, ctypes.c_float(0.1), None, None,
                                          None, None)
    assert st == vx.VX_OK
