"""GPU tests of vx_append_kv, the write path beside the decode step: new
tokens' K/V rows land in their pages bit for bit, and the pages the write
fills get the centroid vx_centroid_update computes (the same bits) and the
oracle's rounded mean (within one bf16 ulp)."""

import numpy as np
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


def _case(vx, dtype, D, S, lens, seed, mla=False, H_kv=2):
    if mla:
        w = synth.Workload(name="append_mla", batch=len(lens), num_q_heads=32, num_kv_heads=1,
                           head_dim_qk=576, head_dim_v=512, page_size=64, dtype="bf16", topk=4,
                           structure="mla", seed=seed, seq_lens=lens, spare_pages=3,
                           v_aliases_k=True)
    else:
        w = synth.Workload(name="append", batch=len(lens), num_q_heads=2 * H_kv, num_kv_heads=H_kv,
                           head_dim_qk=D, head_dim_v=D, page_size=S, dtype=dtype, topk=4,
                           structure="page_offset", seed=seed, seq_lens=lens, spare_pages=3)
    H.log(f"case {H.describe(w)} lens={lens}")
    return w, H.setup_case(vx, w)


def _expected(c, n_new, src_start, k_src, v_src, max_new):
    """The pool after the write (torch indexing on the device), and the
    physical pages the write fills."""
    w = c.w
    K, V = c.K.clone(), None if c.V is None else c.V.clone()
    L = c.L
    filled = []
    for b in range(w.batch):
        n = min(int(n_new[b]), max_new, int(L[b]))
        first = int(L[b]) - n
        for pos in range(first, int(L[b])):
            row = int(src_start[b]) + pos - first
            if not 0 <= row < k_src.shape[0]:
                continue
            page = int(c.pt[b, pos // w.page_size])
            K[page, :, pos % w.page_size] = k_src[row]
            if V is not None and v_src is not None:
                V[page, :, pos % w.page_size] = v_src[row]
        for p in range(first // w.page_size, -(-int(L[b]) // w.page_size)):
            if (p + 1) * w.page_size <= int(L[b]):
                filled.append(int(c.pt[b, p]))
    return K, V, np.array(sorted(set(filled)), dtype=np.int64)


def _run_and_check(vx, c, n_new, src_start, k_src, v_src, max_new, update=True):
    w = c.w
    K_want, V_want, filled = _expected(c, n_new, src_start, k_src, v_src, max_new)
    sentinel = torch.full_like(c.cent, -3.0)
    c.cent.copy_(sentinel)
    bt = c.batch(vx)
    vx.append_kv(c.kv, bt, k_src, v_src,
                 torch.tensor(src_start, dtype=torch.int32, device="cuda"),
                 torch.tensor(n_new, dtype=torch.int32, device="cuda"), max_new, update)
    torch.cuda.synchronize()
    assert torch.equal(c.K, K_want), "K rows differ"
    if c.V is not None:
        assert torch.equal(c.V, V_want), "V rows differ"
    touched = torch.zeros(c.cent.shape[0], dtype=torch.bool, device="cuda")
    if update and len(filled):
        idx = torch.from_numpy(filled).cuda()
        touched[idx] = True
        got = c.cent[idx].clone()
        c.cent[idx] = -3.0
        vx.centroid_update(c.kv, idx.to(torch.int32))          # the same rows, K1
        torch.cuda.synchronize()
        assert torch.equal(got, c.cent[idx]), "centroids differ from vx_centroid_update"
        H.assert_centroids(c, filled)
    assert torch.equal(c.cent[~touched], sentinel[~touched]), "other centroid rows changed"
    H.log(f"  {len(filled)} pages filled")
    return filled


def _src(w, rows, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    k = torch.randn((rows, w.num_kv_heads, w.head_dim_qk), generator=g, device="cuda")
    v = None
    if w.structure != "mla":
        v = torch.randn((rows, w.num_kv_heads, w.head_dim_v), generator=g, device="cuda")
        v = v.to(w.torch_dtype)
    return k.to(w.torch_dtype), v


@pytest.mark.parametrize("dtype,D,S", [("bf16", 128, 16), ("f32", 64, 16), ("bf16", 64, 64)])
def test_append_one_token_per_request(vx, dtype, D, S):
    """The decode append: each request's last token; the ones that end on a
    page boundary fill their page."""
    lens = (S, S + 1, 3 * S, 3 * S - 1, 1, 5 * S, 2 * S + 7)
    w, c = _case(vx, dtype, D, S, lens, seed=91)
    k_src, v_src = _src(w, w.batch, 92)
    filled = _run_and_check(vx, c, [1] * w.batch, list(range(w.batch)), k_src, v_src, 1)
    assert len(filled) == sum(1 for L in lens if L % S == 0)


@pytest.mark.parametrize("dtype,D,S", [("bf16", 128, 16), ("f32", 128, 16)])
def test_prefill_write_fills_every_full_page(vx, dtype, D, S):
    """A prompt written whole: every position comes from the source and every
    full page gets its centroid."""
    lens = (S * 20 + 3, S * 7, 5, S * 33)
    w, c = _case(vx, dtype, D, S, lens, seed=93)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    k_src, v_src = _src(w, int(sum(lens)), 94)
    filled = _run_and_check(vx, c, list(lens), starts, k_src, v_src, max(lens))
    assert len(filled) == sum(L // S for L in lens)


def test_partial_writes_clamps_and_no_update(vx):
    """Writes of 0..40 tokens from scattered source rows, n_new above the
    host bound (clamped to it), a source range running past the last row (not
    written), and the same without centroid updates (table untouched)."""
    S = 16
    lens = (S * 9 + 5, S * 4, S * 2, S * 6 + 15, S * 3, 40)
    w, c = _case(vx, "bf16", 128, S, lens, seed=95)
    n_new = [17, 0, 40, 31, 50, 40]
    starts = [3, 70, 20, 100, 140, 170]
    k_src, v_src = _src(w, 190, 96)      # request 5's rows 170..209 run past 190
    _run_and_check(vx, c, n_new, starts, k_src, v_src, 40)
    w, c = _case(vx, "bf16", 128, S, lens, seed=95)
    _run_and_check(vx, c, n_new, starts, k_src, v_src, 40, update=False)


def test_append_mla_latent_rows(vx):
    """MLA: 576-dim rows in 64-token pages, V the leading 512 dims of K (no
    V source)."""
    lens = (64 * 3, 64 * 2 + 1, 64 * 5, 63)
    w, c = _case(vx, "bf16", 576, 64, lens, seed=97, mla=True)
    k_src, _ = _src(w, w.batch, 98)
    filled = _run_and_check(vx, c, [1] * w.batch, list(range(w.batch)), k_src, None, 1)
    assert len(filled) == 2
    lens2 = (64 * 3 + 10, 64 * 2, 100, 64)
    w, c = _case(vx, "bf16", 576, 64, lens2, seed=99, mla=True)
    starts = np.concatenate([[0], np.cumsum(lens2)[:-1]]).tolist()
    k_src, _ = _src(w, int(sum(lens2)), 100)
    _run_and_check(vx, c, list(lens2), starts, k_src, None, max(lens2))


@pytest.mark.parametrize("seed", range(16))
def test_append_random_shapes(vx, seed):
    """Seeded random writes: dtype, head dim, page size, KV heads, lengths,
    tokens per request (none to several pages), the host bound, source rows
    (some running past the source), with and without centroid updates."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xA99E]))
    dtype = str(rng.choice(["bf16", "f32"]))
    D = int(rng.choice([64, 128]))
    S = int(rng.choice([16, 64]))
    H_kv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 25))
    lens = tuple(int(x) for x in rng.integers(1, 1500, size=B))
    n_new = [int(x) for x in rng.integers(0, 3 * S + 1, size=B)]
    max_new = int(rng.integers(1, 3 * S + 1))
    rows = int(sum(min(n, max_new) for n in n_new)) + 8
    starts = [int(x) for x in rng.integers(0, rows, size=B)]
    update = bool(rng.integers(0, 4))                       # mostly with centroids
    w, c = _case(vx, dtype, D, S, lens, seed=500 + seed, H_kv=H_kv)
    k_src, v_src = _src(w, rows, 600 + seed)
    _run_and_check(vx, c, n_new, starts, k_src, v_src, max_new, update=update)


def test_append_arguments(vx):
    w, c = _case(vx, "bf16", 128, 16, (32, 20), seed=101)
    bt = c.batch(vx)
    k_src, v_src = _src(w, 2, 102)
    z = torch.zeros(2, dtype=torch.int32, device="cuda")
    for args, why in (((k_src, None, z, z, 1, True), "V source missing"),
                      ((k_src, v_src, z, z, -1, True), "negative bound")):
        with pytest.raises(vx.VxError) as e:
            vx.append_kv(c.kv, bt, *args)
        assert e.value.status == vx.VX_ERR_INVALID_ARGUMENT, why
