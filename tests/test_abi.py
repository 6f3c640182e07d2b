"""The C ABI on the host: the library loads, exports every function the
header declares, and rejects invalid arguments before any HIP call (nothing
here launches a kernel, so it runs without a GPU)."""

import ctypes
import os
import re

import pytest

import block_sparse_paged_amd as vx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000                      # never dereferenced: validation fails first


def header_functions():
    with open(os.path.join(ROOT, "include", "vx.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vx_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return vx.load_library()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(vx.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert vx.status_string(0) == "ok"
    assert "workspace" in vx.status_string(3)
    assert vx.status_string(99) == "unknown status"
    assert vx.version() >= 100


def kv_struct(**kw):
    d = dict(dtype=vx.VX_BF16, num_pages=64, page_size=16, num_kv_heads=8, head_dim_qk=128,
             head_dim_v=128, v_aliases_k=0, reserved_=0, k_cache=FAKE, v_cache=FAKE,
             centroids=FAKE)
    d.update(kw)
    return vx.PagedKVStruct(**d)


def batch_struct(**kw):
    d = dict(batch=4, num_q_heads=16, max_pages_per_req=64, max_seq_len=1024,
             page_table=FAKE, seq_lens=FAKE)
    d.update(kw)
    return vx.BatchStruct(**d)


def ws_size(lib, op, kv, bt, k_tot=32):
    out = ctypes.c_size_t(0)
    st = lib.vx_workspace_size(op, ctypes.byref(kv), ctypes.byref(bt), k_tot, ctypes.byref(out))
    return st, out.value


BAD_KV = [
    (dict(dtype=7), vx.VX_ERR_INVALID_ARGUMENT),
    (dict(num_pages=0), vx.VX_ERR_INVALID_ARGUMENT),
    (dict(num_kv_heads=0), vx.VX_ERR_INVALID_ARGUMENT),
    (dict(reserved_=1), vx.VX_ERR_INVALID_ARGUMENT),
    (dict(page_size=32), vx.VX_ERR_UNSUPPORTED),
    (dict(head_dim_qk=96, head_dim_v=96), vx.VX_ERR_UNSUPPORTED),
    (dict(head_dim_v=64), vx.VX_ERR_UNSUPPORTED),
    (dict(v_aliases_k=1), vx.VX_ERR_INVALID_ARGUMENT),            # v_cache must be NULL
    (dict(v_aliases_k=2), vx.VX_ERR_INVALID_ARGUMENT),
    (dict(head_dim_qk=576, head_dim_v=512, v_aliases_k=1, v_cache=None, num_kv_heads=1,
          page_size=64, dtype=vx.VX_F32), vx.VX_ERR_UNSUPPORTED),
]

BAD_BATCH = [
    (dict(batch=-1), vx.VX_ERR_INVALID_ARGUMENT),
    (dict(num_q_heads=12), vx.VX_ERR_INVALID_ARGUMENT),           # not a multiple of H_kv
    (dict(num_q_heads=24), vx.VX_ERR_UNSUPPORTED),                # G = 3
    (dict(max_seq_len=0), vx.VX_ERR_INVALID_ARGUMENT),
    (dict(max_pages_per_req=0), vx.VX_ERR_INVALID_ARGUMENT),
    (dict(max_seq_len=1025), vx.VX_ERR_INVALID_ARGUMENT),         # 64 pages * 16 < 1025
]


@pytest.mark.parametrize("kw,want", BAD_KV)
def test_bad_kv_rejected_everywhere(lib, kw, want):
    kv, bt = kv_struct(**kw), batch_struct()
    r = ctypes.byref
    assert lib.vx_centroid_update(r(kv), FAKE, 4, None) == want
    assert lib.vx_score_topk(r(kv), r(bt), FAKE, 30, 1, 1, FAKE, FAKE, 1 << 30, None) == want
    assert lib.vx_sparse_paged_decode(r(kv), r(bt), FAKE, FAKE, 32, 0.1, FAKE, FAKE, FAKE,
                                      1 << 30, None) == want
    assert lib.vx_full_paged_decode(r(kv), r(bt), FAKE, 0.1, FAKE, FAKE, FAKE, 1 << 30,
                                    None) == want
    assert ws_size(lib, vx.VX_OP_FULL_DECODE, kv, bt)[0] == want
    assert lib.vx_sparse_decode_step(r(kv), r(bt), FAKE, 30, 1, 1, 1, 0.1, FAKE, FAKE, FAKE,
                                     FAKE, 1 << 30, None) == want


@pytest.mark.parametrize("kw,want", BAD_BATCH)
def test_bad_batch_rejected(lib, kw, want):
    kv, bt = kv_struct(), batch_struct(**kw)
    r = ctypes.byref
    assert lib.vx_score_topk(r(kv), r(bt), FAKE, 30, 1, 1, FAKE, FAKE, 1 << 30, None) == want
    assert lib.vx_sparse_paged_decode(r(kv), r(bt), FAKE, FAKE, 32, 0.1, FAKE, FAKE, FAKE,
                                      1 << 30, None) == want
    assert lib.vx_full_paged_decode(r(kv), r(bt), FAKE, 0.1, FAKE, FAKE, FAKE, 1 << 30,
                                    None) == want
    assert lib.vx_sparse_decode_step(r(kv), r(bt), FAKE, 30, 1, 1, 1, 0.1, FAKE, FAKE, FAKE,
                                     FAKE, 1 << 30, None) == want
    for op in (0, 1, 2, 3):
        assert ws_size(lib, op, kv, bt)[0] == want


def test_null_pointers_rejected(lib):
    r = ctypes.byref
    kv, bt = kv_struct(), batch_struct()
    assert lib.vx_centroid_update(None, FAKE, 1, None) == vx.VX_ERR_INVALID_ARGUMENT
    assert lib.vx_centroid_update(r(kv), None, 1, None) == vx.VX_ERR_INVALID_ARGUMENT
    assert lib.vx_centroid_update(r(kv_struct(centroids=None)), FAKE, 1, None) == 1
    assert lib.vx_score_topk(r(kv), None, FAKE, 30, 1, 1, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.vx_score_topk(r(kv), r(bt), None, 30, 1, 1, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.vx_score_topk(r(kv), r(bt), FAKE, 30, 1, 1, None, FAKE, 1 << 30, None) == 1
    assert lib.vx_score_topk(r(kv), r(bt), FAKE, 30, 1, 1, FAKE, None, 1 << 30, None) == 1
    assert lib.vx_score_topk(r(kv), r(batch_struct(page_table=None)), FAKE, 30, 1, 1, FAKE,
                             FAKE, 1 << 30, None) == 1
    assert lib.vx_sparse_paged_decode(r(kv), r(bt), FAKE, None, 32, 0.1, FAKE, FAKE, FAKE,
                                      1 << 30, None) == 1
    assert lib.vx_sparse_paged_decode(r(kv), r(bt), FAKE, FAKE, 32, 0.1, None, FAKE, FAKE,
                                      1 << 30, None) == 1
    assert lib.vx_full_paged_decode(r(kv_struct(v_cache=None)), r(bt), FAKE, 0.1, FAKE,
                                    FAKE, FAKE, 1 << 30, None) == 1
    assert lib.vx_workspace_size(0, r(kv), r(bt), 32, None) == 1


def test_scalar_arguments_rejected(lib):
    r = ctypes.byref
    kv, bt = kv_struct(), batch_struct()
    for topk, bos, eos in ((-1, 1, 1), (30, -1, 1), (30, 1, 0)):
        assert lib.vx_score_topk(r(kv), r(bt), FAKE, topk, bos, eos, FAKE, FAKE, 1 << 30,
                                 None) == vx.VX_ERR_INVALID_ARGUMENT
    assert lib.vx_centroid_update(r(kv), FAKE, -1, None) == vx.VX_ERR_INVALID_ARGUMENT
    assert lib.vx_centroid_update(r(kv), None, 0, None) == vx.VX_OK      # nothing to do
    for k_tot in (0, -3):
        assert lib.vx_sparse_paged_decode(r(kv), r(bt), FAKE, FAKE, k_tot, 0.1, FAKE, FAKE,
                                          FAKE, 1 << 30, None) == 1
    for scale in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.vx_full_paged_decode(r(kv), r(bt), FAKE, scale, FAKE, FAKE, FAKE, 1 << 30,
                                        None) == 1
    step = lib.vx_sparse_decode_step
    for topk, bos, eos, upd, scale in ((-1, 1, 1, 1, 0.1), (30, -1, 1, 1, 0.1), (30, 1, 0, 1, 0.1),
                                       (30, 1, 1, 2, 0.1), (30, 1, 1, 1, 0.0),
                                       (30, 1, 1, 1, float("nan"))):
        assert step(r(kv), r(bt), FAKE, topk, bos, eos, upd, scale, FAKE, FAKE, FAKE, FAKE,
                    1 << 30, None) == vx.VX_ERR_INVALID_ARGUMENT
    for nulls in ((None, FAKE, FAKE), (FAKE, None, FAKE), (FAKE, FAKE, None)):
        assert step(r(kv), r(bt), nulls[0], 30, 1, 1, 1, 0.1, nulls[1], nulls[2], FAKE, FAKE,
                    1 << 30, None) == vx.VX_ERR_INVALID_ARGUMENT
    assert step(r(kv_struct(centroids=None)), r(bt), FAKE, 30, 1, 1, 1, 0.1, FAKE, FAKE, FAKE,
                FAKE, 1 << 30, None) == vx.VX_ERR_INVALID_ARGUMENT
    assert step(r(kv), r(batch_struct(batch=0)), None, 30, 1, 1, 1, 0.1, None, None, None, None,
                0, None) == vx.VX_OK
    st, need = ws_size(lib, vx.VX_OP_DECODE_STEP, kv, bt, 32)
    assert st == 0 and need >= ws_size(lib, vx.VX_OP_SCORE_TOPK, kv, bt)[1]
    assert step(r(kv), r(bt), FAKE, 30, 1, 1, 1, 0.1, FAKE, FAKE, FAKE, FAKE, need - 1,
                None) == vx.VX_ERR_WORKSPACE_TOO_SMALL
    assert lib.vx_workspace_size(9, r(kv), r(bt), 32, r(ctypes.c_size_t())) == 1


def test_workspace_too_small_rejected(lib):
    r = ctypes.byref
    kv = kv_struct()
    bt = batch_struct(batch=64, max_pages_per_req=2048, max_seq_len=32768)
    st, need = ws_size(lib, vx.VX_OP_SCORE_TOPK, kv, bt)
    assert st == 0 and need >= 64 * 8 * 2048 * 4
    assert lib.vx_score_topk(r(kv), r(bt), FAKE, 30, 1, 1, FAKE, FAKE, need - 1, None) == 3
    st, need = ws_size(lib, vx.VX_OP_FULL_DECODE, kv, bt)
    assert st == 0 and need > 0
    assert lib.vx_full_paged_decode(r(kv), r(bt), FAKE, 0.1, FAKE, FAKE, FAKE, need - 1,
                                    None) == 3
    st, need = ws_size(lib, vx.VX_OP_SPARSE_DECODE, kv, bt, 32)
    assert st == 0
    if need:
        assert lib.vx_sparse_paged_decode(r(kv), r(bt), FAKE, FAKE, 32, 0.1, FAKE, FAKE, FAKE,
                                          need - 1, None) == 3


def test_empty_batch_launches_nothing(lib):
    r = ctypes.byref
    kv, bt = kv_struct(), batch_struct(batch=0)
    assert lib.vx_score_topk(r(kv), r(bt), FAKE, 30, 1, 1, FAKE, FAKE, 1 << 30, None) == 0
    assert lib.vx_sparse_paged_decode(r(kv), r(bt), FAKE, FAKE, 32, 0.1, FAKE, FAKE, FAKE,
                                      1 << 30, None) == 0
    assert lib.vx_full_paged_decode(r(kv), r(bt), FAKE, 0.1, FAKE, FAKE, FAKE, 1 << 30,
                                    None) == 0


def test_too_many_candidates_unsupported(lib):
    kv = kv_struct()
    bt = batch_struct(max_pages_per_req=20000, max_seq_len=20000 * 16)
    assert ws_size(lib, vx.VX_OP_SCORE_TOPK, kv, bt)[0] == vx.VX_ERR_UNSUPPORTED


def test_workspace_monotone_in_shapes(lib):
    kv = kv_struct()
    prev = 0
    for B in (1, 4, 16, 64, 256):
        bt = batch_struct(batch=B, max_pages_per_req=4096, max_seq_len=65536)
        st, n = ws_size(lib, vx.VX_OP_SCORE_TOPK, kv, bt)
        assert st == 0 and n >= prev
        prev = n
    for op, kt in ((vx.VX_OP_SPARSE_DECODE, 66), (vx.VX_OP_FULL_DECODE, 0)):
        sizes = []
        for L in (1024, 8192, 65536):
            bt = batch_struct(batch=32, max_pages_per_req=4096, max_seq_len=L)
            st, n = ws_size(lib, op, kv, bt, kt)
            assert st == 0
            sizes.append(n)
        assert sizes == sorted(sizes) or op == vx.VX_OP_SPARSE_DECODE


def plan(lib, op, kv, bt, k_tot=0, cus=0, pps=0):
    p = vx.DecodePlanStruct()
    st = lib.vx_plan_decode(op, ctypes.byref(kv), ctypes.byref(bt), k_tot, cus, pps,
                            ctypes.byref(p))
    return st, p


@pytest.mark.parametrize("cus", [256, 32])
def test_plan_is_a_function_of_shapes_and_cus(lib, cus):
    """The planner on the host, for a full MI355X (256 CUs) and a 32-CU
    partition: sparse splits aim at one 8-wave block per CU, dense ones at
    16 per CU (at least 64 pages each), partials within 15% of the K/V bytes
    they replace, and the workspace holds exactly the partials."""
    kv = kv_struct()
    # long context: 8 requests x 8 KV heads, 258 selected pages each
    bt = batch_struct(batch=8, num_q_heads=64, max_pages_per_req=8192, max_seq_len=131072)
    st, p = plan(lib, vx.VX_OP_SPARSE_DECODE, kv, bt, 258, cus)
    assert st == 0 and p.num_cus == cus and p.op == vx.VX_OP_SPARSE_DECODE
    want = -(-258 // -(-cus // 64))                      # ceil(258 / ceil(cus / 64 units))
    assert p.pages_per_split == want and p.n_split == -(-258 // want)
    rows = 8 * 64 * p.n_split
    assert p.workspace_bytes == (0 if p.n_split == 1 else
                                 -(-rows * 128 * 4 // 256) * 256 + -(-rows * 2 * 4 // 256) * 256)
    # Qwen-like: 256 units, one split per unit on either GPU
    bt2 = batch_struct(batch=32, num_q_heads=16, max_pages_per_req=2048, max_seq_len=32768)
    st, p = plan(lib, vx.VX_OP_SPARSE_DECODE, kv, bt2, 32, cus)
    assert st == 0 and p.n_split == 1 and p.workspace_bytes == 0
    # dense: the work list of 128-page items (16 per request and KV head),
    # walked by four blocks per CU
    st, p = plan(lib, vx.VX_OP_FULL_DECODE, kv, bt2, 0, cus)
    assert st == 0 and p.work_list == 1 and p.pages_per_split == 128 and p.n_split == 16
    assert p.blocks == min(32 * 8 * 16, 4 * cus)
    rows = 32 * 16 * 16
    assert p.workspace_bytes == -(-rows * 128 * 4 // 256) * 256 + -(-rows * 2 * 4 // 256) * 256
    # the same shapes always give the same plan
    assert plan(lib, vx.VX_OP_FULL_DECODE, kv, bt2, 0, cus)[1].pages_per_split == p.pages_per_split


def test_plan_with_a_fixed_split_size(lib):
    kv = kv_struct()
    bt = batch_struct(batch=2, max_pages_per_req=256, max_seq_len=4096)
    st, p1 = plan(lib, vx.VX_OP_SPARSE_DECODE, kv, bt, 32, 256, 1)
    assert st == 0 and p1.pages_per_split == 1 and p1.n_split == 32
    assert p1.workspace_bytes >= 2 * 16 * 32 * 128 * 4                 # 32 splits of fp32 partials
    st, p2 = plan(lib, vx.VX_OP_SPARSE_DECODE, kv, bt, 32, 256, 1000)
    assert st == 0 and p2.n_split == 1 and p2.workspace_bytes == 0     # one split: direct output
    st, p3 = plan(lib, vx.VX_OP_FULL_DECODE, kv, bt, 0, 256, 0)
    assert st == 0 and p3.pages_per_split == 128 and p3.work_list == 1 and p3.n_split == 2
    st, p4 = plan(lib, vx.VX_OP_FULL_DECODE, kv, bt, 0, 256, 7)       # a fixed item size
    assert st == 0 and p4.pages_per_split == 7 and p4.n_split == 37 and p4.blocks == 2 * 8 * 37
    big = batch_struct(batch=4096, max_pages_per_req=64, max_seq_len=1024)
    st, p5 = plan(lib, vx.VX_OP_FULL_DECODE, kv, big, 0, 256, 0)
    assert st == 0 and p5.work_list == 0                                # beyond the list's batch bound
    r = ctypes.byref
    for bad in ((vx.VX_OP_SCORE_TOPK, 32, 256, 0), (vx.VX_OP_SPARSE_DECODE, 0, 256, 0),
                (vx.VX_OP_SPARSE_DECODE, 32, -1, 0), (vx.VX_OP_SPARSE_DECODE, 32, 256, -2)):
        assert plan(lib, bad[0], kv, bt, bad[1], bad[2], bad[3])[0] == vx.VX_ERR_INVALID_ARGUMENT
    assert lib.vx_plan_decode(vx.VX_OP_FULL_DECODE, r(kv), r(bt), 0, 256, 0,
                              None) == vx.VX_ERR_INVALID_ARGUMENT
    # a planned call checks its plan against the planner before launching anything
    run = lib.vx_paged_decode_planned
    forged = vx.DecodePlanStruct.from_buffer_copy(p1)
    forged.n_split = 7
    assert run(r(kv), r(bt), FAKE, FAKE, 32, r(forged), 0.1, FAKE, FAKE, FAKE, 1 << 30,
               None) == vx.VX_ERR_INVALID_ARGUMENT
    assert run(r(kv), r(bt), FAKE, None, 32, r(p1), 0.1, FAKE, FAKE, FAKE, 1 << 30,
               None) == vx.VX_ERR_INVALID_ARGUMENT                     # sparse plan, no sel
    assert run(r(kv), r(bt), FAKE, FAKE, 32, r(p1), 0.1, FAKE, FAKE, FAKE, p1.workspace_bytes - 1,
               None) == vx.VX_ERR_WORKSPACE_TOO_SMALL
    empty = batch_struct(batch=0)
    st, p0 = plan(lib, vx.VX_OP_SPARSE_DECODE, kv, empty, 32, 256, 1)
    assert st == 0 and p0.workspace_bytes == 0
    assert run(r(kv), r(empty), None, FAKE, 32, r(p0), 0.1, None, None, None, 0, None) == vx.VX_OK
    assert run(r(kv), r(empty), None, FAKE, 32, r(p1), 0.1, None, None, None, 0,
               None) == vx.VX_ERR_INVALID_ARGUMENT                     # planned for 2 requests


def test_radix_and_append_arguments_rejected(lib):
    r = ctypes.byref
    kv, bt = kv_struct(), batch_struct()
    radix = lib.vx_score_topk_radix
    for levels in (0, 3, -1):
        assert radix(r(kv), r(bt), FAKE, 30, 1, 1, levels, FAKE, FAKE, FAKE, 1 << 30,
                     None) == vx.VX_ERR_INVALID_ARGUMENT
    assert radix(r(kv), r(bt), FAKE, 30, 1, 1, 1, None, FAKE, FAKE, 1 << 30,
                 None) == vx.VX_ERR_INVALID_ARGUMENT                  # no random words
    big = batch_struct(max_pages_per_req=9000, max_seq_len=9000 * 16)
    assert radix(r(kv), r(big), FAKE, 30, 1, 1, 2, FAKE, FAKE, FAKE, 1 << 30,
                 None) == vx.VX_ERR_UNSUPPORTED                       # > 8192 candidates
    assert radix(r(kv), r(batch_struct(batch=0)), None, 30, 1, 1, 1, None, None, None, 0,
                 None) == vx.VX_OK
    app = lib.vx_append_kv
    for k_src, v_src, rows, max_new, upd in ((None, FAKE, 8, 1, 1), (FAKE, None, 8, 1, 1),
                                             (FAKE, FAKE, -1, 1, 1), (FAKE, FAKE, 8, -1, 1),
                                             (FAKE, FAKE, 8, 1, 2)):
        assert app(r(kv), r(bt), k_src, v_src, FAKE, FAKE, rows, max_new, upd,
                   None) == vx.VX_ERR_INVALID_ARGUMENT
    assert app(r(kv), r(bt), FAKE, FAKE, None, FAKE, 8, 1, 1, None) == vx.VX_ERR_INVALID_ARGUMENT
    assert app(r(kv_struct(centroids=None)), r(bt), FAKE, FAKE, FAKE, FAKE, 8, 1, 1,
               None) == vx.VX_ERR_INVALID_ARGUMENT                    # centroids to update
    mla = kv_struct(head_dim_qk=576, head_dim_v=512, num_kv_heads=1, page_size=64,
                    v_aliases_k=1, v_cache=None)
    mbt = batch_struct(num_q_heads=32, max_seq_len=64 * 64)
    assert app(r(mla), r(mbt), FAKE, FAKE, FAKE, FAKE, 8, 1, 1,
               None) == vx.VX_ERR_INVALID_ARGUMENT                    # V is part of K
    assert app(r(kv), r(bt), FAKE, FAKE, FAKE, FAKE, 8, 0, 1, None) == vx.VX_OK      # nothing new
    assert app(r(kv), r(batch_struct(batch=0)), None, None, None, None, 0, 5, 1,
               None) == vx.VX_OK


def test_decode_layers_arguments_rejected(lib):
    """Every layer is checked before anything is launched: a bad argument in
    any layer returns its status (with FAKE device pointers a launch would
    fault, so a pass here also shows that none happened)."""
    r = ctypes.byref
    fn = lib.vx_decode_layers
    n = 3
    kvs = (vx.PagedKVStruct * n)(*[kv_struct() for _ in range(n)])
    bt = batch_struct()
    VPA = ctypes.c_void_p * n
    qs, outs, sels = VPA(FAKE, FAKE, FAKE), VPA(FAKE, FAKE, FAKE), VPA(FAKE, FAKE, FAKE)
    dense = (ctypes.c_uint8 * n)(1, 0, 0)
    st, need = ws_size(lib, vx.VX_OP_DECODE_LAYERS, kvs[0], bt, 32)
    assert st == 0
    st_step = ws_size(lib, vx.VX_OP_DECODE_STEP, kvs[0], bt, 32)[1]
    st_full = ws_size(lib, vx.VX_OP_FULL_DECODE, kvs[0], bt, 32)[1]
    assert need == max(st_step, st_full)

    def call(kv_arr=kvs, batch=bt, q=qs, layers=n, dn=dense, topk=30, sl=sels, out=outs,
             ws_bytes=need, scale=0.1):
        return fn(kv_arr, r(batch), q, layers, dn, topk, 1, 1, 1, scale, sl, out, None, FAKE,
                  ws_bytes, None)

    assert call(layers=-1) == vx.VX_ERR_INVALID_ARGUMENT
    assert call(layers=0, q=None, out=None, sl=None) == vx.VX_OK
    assert call(q=None) == vx.VX_ERR_INVALID_ARGUMENT
    assert call(sl=None) == vx.VX_ERR_INVALID_ARGUMENT              # layers 1, 2 are sparse
    assert call(ws_bytes=need - 1) == vx.VX_ERR_WORKSPACE_TOO_SMALL
    assert call(topk=-1) == vx.VX_ERR_INVALID_ARGUMENT
    assert call(scale=0.0) == vx.VX_ERR_INVALID_ARGUMENT
    odd = (vx.PagedKVStruct * n)(kv_struct(), kv_struct(), kv_struct(head_dim_qk=64, head_dim_v=64))
    assert call(kv_arr=odd) == vx.VX_ERR_INVALID_ARGUMENT          # shapes differ between layers
    bad_last = (vx.PagedKVStruct * n)(kv_struct(), kv_struct(), kv_struct(centroids=None))
    assert call(kv_arr=bad_last) == vx.VX_ERR_INVALID_ARGUMENT      # the last layer's table
    late_null = VPA(FAKE, FAKE, None)
    assert call(out=late_null) == vx.VX_ERR_INVALID_ARGUMENT
    big = batch_struct(batch=64, max_pages_per_req=2048, max_seq_len=32768)
    full_big = ws_size(lib, vx.VX_OP_FULL_DECODE, kvs[0], big, 32)[1]
    assert full_big > 0
    all_dense = (ctypes.c_uint8 * n)(1, 1, 1)
    assert call(batch=big, dn=all_dense, sl=None,
                ws_bytes=full_big - 1) == vx.VX_ERR_WORKSPACE_TOO_SMALL
    assert call(batch=batch_struct(batch=0)) == vx.VX_OK


def test_bounds_arguments_rejected(lib):
    r = ctypes.byref
    kv, bt = kv_struct(), batch_struct()
    upd, score = lib.vx_bounds_update, lib.vx_score_topk_bounds
    assert upd(r(kv), FAKE, FAKE, -1, None) == vx.VX_ERR_INVALID_ARGUMENT
    assert upd(r(kv), None, FAKE, 4, None) == vx.VX_ERR_INVALID_ARGUMENT
    assert upd(r(kv), FAKE, None, 4, None) == vx.VX_ERR_INVALID_ARGUMENT
    assert upd(r(kv), None, None, 0, None) == vx.VX_OK                   # nothing to do
    mla = kv_struct(head_dim_qk=576, head_dim_v=512, num_kv_heads=1, page_size=64,
                    v_aliases_k=1, v_cache=None)
    assert upd(r(mla), FAKE, FAKE, 4, None) == vx.VX_ERR_UNSUPPORTED
    need = ws_size(lib, vx.VX_OP_SCORE_TOPK, kv, bt)[1]
    for args, want in (((FAKE, FAKE, 30, 1, 0, FAKE, FAKE, need), vx.VX_ERR_INVALID_ARGUMENT),
                       ((FAKE, FAKE, -1, 1, 1, FAKE, FAKE, need), vx.VX_ERR_INVALID_ARGUMENT),
                       ((None, FAKE, 30, 1, 1, FAKE, FAKE, need), vx.VX_ERR_INVALID_ARGUMENT),
                       ((FAKE, None, 30, 1, 1, FAKE, FAKE, need), vx.VX_ERR_INVALID_ARGUMENT),
                       ((FAKE, FAKE, 30, 1, 1, FAKE, FAKE, need - 1), vx.VX_ERR_WORKSPACE_TOO_SMALL)):
        assert score(r(kv), r(bt), *args, None) == want
    mbt = batch_struct(num_q_heads=32, max_seq_len=64 * 64)
    assert score(r(mla), r(mbt), FAKE, FAKE, 30, 1, 1, FAKE, FAKE, 1 << 30,
                 None) == vx.VX_ERR_UNSUPPORTED
    assert score(r(kv), r(batch_struct(batch=0)), None, None, 30, 1, 1, None, None, 0,
                 None) == vx.VX_OK


def test_step_bounds_arguments_rejected(lib):
    """vx_sparse_decode_step_bounds checks as vx_sparse_decode_step, with the
    bounds table in place of the centroid table (which it does not read)."""
    r = ctypes.byref
    step = lib.vx_sparse_decode_step_bounds
    kv, bt = kv_struct(), batch_struct()
    need = ws_size(lib, vx.VX_OP_DECODE_STEP, kv, bt, 32)[1]
    good = dict(bounds=FAKE, q=FAKE, topk=30, bos=1, eos=1, upd=1, scale=0.1, sel=FAKE, out=FAKE,
                ws=FAKE, ws_bytes=need)

    def call(kv=kv, bt=bt, **kw):
        a = dict(good, **kw)
        return step(r(kv), r(bt), a["bounds"], a["q"], a["topk"], a["bos"], a["eos"], a["upd"],
                    a["scale"], a["sel"], a["out"], None, a["ws"], a["ws_bytes"], None)

    assert call(bounds=None) == vx.VX_ERR_INVALID_ARGUMENT
    assert call(q=None) == vx.VX_ERR_INVALID_ARGUMENT
    assert call(eos=0) == vx.VX_ERR_INVALID_ARGUMENT
    assert call(upd=2) == vx.VX_ERR_INVALID_ARGUMENT
    assert call(scale=0.0) == vx.VX_ERR_INVALID_ARGUMENT
    assert call(ws_bytes=need - 1) == vx.VX_ERR_WORKSPACE_TOO_SMALL
    assert call(bt=batch_struct(max_pages_per_req=20000, max_seq_len=16 * 20000),
                ws_bytes=1 << 40) == vx.VX_ERR_UNSUPPORTED        # more pages than it selects from
    mla = kv_struct(head_dim_qk=576, head_dim_v=512, num_kv_heads=1, page_size=64,
                    v_aliases_k=1, v_cache=None)
    assert call(kv=mla, bt=batch_struct(num_q_heads=32, max_seq_len=64 * 64),
                ws_bytes=1 << 40) == vx.VX_ERR_UNSUPPORTED
    assert call(kv=kv_struct(centroids=None), bounds=None) == vx.VX_ERR_INVALID_ARGUMENT
    assert call(bt=batch_struct(batch=0), bounds=None, q=None, sel=None, out=None,
                ws=None) == vx.VX_OK


def test_static_step_refuses_shapes_beyond_its_scratch(lib):
    """vx_sparse_decode_step_static checks the shapes' workspace against its
    static scratch (VX_STATIC_SCRATCH_BYTES) on the host, before any HIP
    call: too large is VX_ERR_WORKSPACE_TOO_SMALL, an empty batch is a
    no-op, invalid arguments are rejected as vx_sparse_decode_step rejects
    them."""
    r = ctypes.byref
    kv = kv_struct()
    big = batch_struct(batch=4096, max_pages_per_req=16384, max_seq_len=16384 * 16)
    st, need = ws_size(lib, vx.VX_OP_DECODE_STEP, kv, big, 32)
    assert st == 0 and need > vx.STATIC_SCRATCH_BYTES
    step = lib.vx_sparse_decode_step_static
    assert step(r(kv), r(big), FAKE, 30, 1, 1, 1, 0.1, FAKE, FAKE, FAKE,
                None) == vx.VX_ERR_WORKSPACE_TOO_SMALL
    assert step(r(kv), r(batch_struct(batch=0)), None, 30, 1, 1, 1, 0.1, None, None, None,
                None) == vx.VX_OK
    for topk, bos, eos in ((-1, 1, 1), (30, -1, 1), (30, 1, 0)):
        assert step(r(kv), r(batch_struct()), FAKE, topk, bos, eos, 1, 0.1, FAKE, FAKE, FAKE,
                    None) == vx.VX_ERR_INVALID_ARGUMENT


def test_binding_rejects_mismatched_tensors():
    """The binding checks dtypes, shapes and contiguity before building the
    C structs (no GPU needed): an int64 page table would otherwise be read as
    int32 halves, a wrong-dtype query as the cache dtype, and so on."""
    import torch
    P, H, S, D, B, Hq = 8, 2, 16, 64, 3, 4
    k = torch.zeros((P, H, S, D), dtype=torch.bfloat16)
    v = torch.zeros((P, H, S, D), dtype=torch.bfloat16)
    cent = torch.zeros((P, H, D), dtype=torch.bfloat16)
    kv = vx.PagedKV(k_cache=k, v_cache=v, centroids=cent)
    pt = torch.zeros((B, 4), dtype=torch.int32)
    sl = torch.ones(B, dtype=torch.int32)
    bt = vx.Batch(page_table=pt, seq_lens=sl, num_q_heads=Hq, max_seq_len=64)
    kv.struct()
    bt.struct()
    bad = [
        lambda: vx.Batch(page_table=pt.long(), seq_lens=sl, num_q_heads=Hq, max_seq_len=64).struct(),
        lambda: vx.Batch(page_table=pt, seq_lens=sl.long(), num_q_heads=Hq, max_seq_len=64).struct(),
        lambda: vx.Batch(page_table=pt, seq_lens=sl[:2], num_q_heads=Hq, max_seq_len=64).struct(),
        lambda: vx.Batch(page_table=pt.t(), seq_lens=torch.ones(4, dtype=torch.int32), num_q_heads=Hq,
                         max_seq_len=64).struct(),
        lambda: vx.PagedKV(k_cache=k, v_cache=v, centroids=cent.float()).struct(),
        lambda: vx.PagedKV(k_cache=k, v_cache=v, centroids=cent[:4]).struct(),
        lambda: vx.PagedKV(k_cache=k, v_cache=v.float(), centroids=cent).struct(),
        lambda: vx.PagedKV(k_cache=k.half(), v_cache=None, centroids=None).struct(),
        lambda: vx._args(kv, bt, q=torch.zeros((B, Hq, D), dtype=torch.float32)),
        lambda: vx._args(kv, bt, q=torch.zeros((B, Hq + 1, D), dtype=torch.bfloat16)),
        lambda: vx._args(kv, bt, out=torch.zeros((B, Hq, D + 1), dtype=torch.bfloat16)),
        lambda: vx._args(kv, bt, sel=torch.zeros((B, H + 1, 5), dtype=torch.int32)),
        lambda: vx._args(kv, bt, sel=torch.zeros((B, H, 5), dtype=torch.int64)),
        lambda: vx._args(kv, bt, lse=torch.zeros((B, Hq), dtype=torch.bfloat16)),
        lambda: vx._args(kv, bt, q=torch.zeros((B, D, Hq), dtype=torch.bfloat16).transpose(1, 2)),
    ]
    for i, f in enumerate(bad):
        with pytest.raises(ValueError):
            f()
    vx._args(kv, bt, q=torch.zeros((B, Hq, D), dtype=torch.bfloat16),
             out=torch.zeros((B, Hq, D), dtype=torch.bfloat16),
             sel=torch.zeros((B, H, 5), dtype=torch.int32), lse=torch.zeros((B, Hq)))
