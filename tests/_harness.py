"""Test plumbing shared by the GPU parity tests: sets up a workload on the
device through the library's binding, draws queries whose k-th / (k+1)-th
page-score gap is large enough for the selected set to be unique, and runs
the fp64 oracle request by request on the same bytes.

The gap rule: for every (request, KV head) whose candidate count exceeds k,
the fp64 oracle scores must satisfy  s_(k) - s_(k+1) > 1e-3 * max|s|  over
the candidates.  Groups that fail are redrawn (attempt 1, 2, ...) from the
seeded generator.  The margin dwarfs the fp32 scoring error and a one-ulp
bf16 centroid disagreement, so any set mismatch is a bug.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle as orc
import synth

GAP_REL = 1e-3
MAX_ATTEMPTS = 1000


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 7)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


@dataclass
class Case:
    w: synth.Workload
    layout: synth.PageLayout
    K: torch.Tensor
    V: torch.Tensor | None
    cent: torch.Tensor
    pt: torch.Tensor
    seq_lens: torch.Tensor
    kv: object
    step: int = 0
    q_host: torch.Tensor | None = None          # [B, H_q, D] in the workload dtype
    attempts: np.ndarray | None = None
    _oracle_cent: dict = field(default_factory=dict)
    _oracle_bounds: dict = field(default_factory=dict)

    @property
    def L(self) -> np.ndarray:
        return synth.step_seq_lens(self.layout, self.step)

    def batch(self, vx):
        return vx.Batch(page_table=self.pt, seq_lens=self.seq_lens,
                        num_q_heads=self.w.num_q_heads,
                        max_seq_len=int(self.layout.seq_lens0.max()) + self.w.steps - 1)

    def n_pages(self, b: int) -> int:
        return -(-int(self.L[b]) // self.w.page_size)

    def request_pages(self, b: int):
        """Logical view of request b's pages on the host (fp64): K, V."""
        n = -(-int(self.layout.seq_lens0[b] + self.w.steps - 1) // self.w.page_size)
        idx = self.pt[b, :n].long()
        k = to_f64(self.K[idx])
        v = None if self.V is None else to_f64(self.V[idx])
        return k, v

    def oracle_centroids(self, b: int, k_pages=None) -> np.ndarray:
        """Oracle centroids of request b's logical pages at the current step."""
        key = (b, int(self.L[b]) // self.w.page_size)
        if key not in self._oracle_cent:
            if k_pages is None:
                k_pages, _ = self.request_pages(b)
            self._oracle_cent[key] = orc.request_centroids(k_pages, int(self.L[b]), self.w.dtype)
        return self._oracle_cent[key]

    def oracle_bounds(self, b: int) -> np.ndarray:
        """Oracle key bounds [n_b, H_kv, 2, D] of request b at the current step."""
        key = (b, int(self.L[b]) // self.w.page_size)
        if key not in self._oracle_bounds:
            k_pages, _ = self.request_pages(b)
            n_b = self.n_pages(b)
            self._oracle_bounds[key] = orc.request_bounds(k_pages, int(self.L[b]))[:n_b]
        return self._oracle_bounds[key]


def setup_case(vx, w: synth.Workload, device="cuda") -> Case:
    lay = synth.build_layout(w)
    K, V = synth.make_kv_pool(w, lay, device=device)
    cent = torch.zeros((lay.num_pages, w.num_kv_heads, w.head_dim_qk), dtype=w.torch_dtype,
                       device=device)
    pt = torch.from_numpy(lay.page_table).to(device)
    sl = torch.from_numpy(synth.step_seq_lens(lay, 0).astype(np.int32)).to(device)
    kv = vx.PagedKV(k_cache=K, v_cache=V, centroids=cent, head_dim_v=w.head_dim_v)
    c = Case(w=w, layout=lay, K=K, V=V, cent=cent, pt=pt, seq_lens=sl, kv=kv)
    c.attempts = np.zeros((w.batch, w.num_kv_heads), dtype=np.int64)
    c.q_host = synth.make_queries(w, lay, 0)
    return c


def set_step(c: Case, step: int):
    c.step = step
    c.seq_lens.copy_(torch.from_numpy(synth.step_seq_lens(c.layout, step).astype(np.int32)))
    c.attempts[:] = 0
    c.q_host = synth.make_queries(c.w, c.layout, step)


def page_sums_fp64(c: Case, b: int) -> np.ndarray:
    """Sum over each full page's tokens of request b's keys, in fp64 on the
    device: [n_full, H_kv, D].  For bf16 keys the sum of 16 or 64 values is
    exact in fp64 (each has an 8-bit significand; the exponents of the values
    drawn here span far fewer than the 41 binades that would take), so it
    equals the sum numpy forms for the oracle's mean, whatever the order."""
    n_full = int(c.L[b]) // c.w.page_size
    idx = c.pt[b, :n_full].long()
    return c.K[idx].double().sum(dim=2).cpu().numpy()


def prime_centroids_device(c: Case, requests):
    """Fill the oracle-centroid cache of the listed requests from exact fp64
    page sums formed on the device (bf16 only, see page_sums_fp64), divided
    by the page size and rounded by the oracle's own round_to.  Equal bit for
    bit to orc.request_centroids (pinned by test_device_centroid_shortcut);
    used where the oracle's host pass over every page of a full-size batch
    would take minutes."""
    w = c.w
    assert w.dtype == "bf16", "exact fp64 page sums need bf16 keys"
    for b in requests:
        key = (b, int(c.L[b]) // w.page_size)
        if key in c._oracle_cent:
            continue
        n_b = c.n_pages(b)
        out = np.full((n_b, w.num_kv_heads, w.head_dim_qk), np.nan)
        n_full = int(c.L[b]) // w.page_size
        if n_full:
            out[:n_full] = orc.round_to(page_sums_fp64(c, b) / w.page_size, w.dtype)
        c._oracle_cent[key] = out


def prime_bounds_device(c: Case, requests):
    """Fill the oracle-bounds cache of the listed requests with per-channel
    minima and maxima taken on the device.  Minimum and maximum are exact in
    any order, so these equal orc.request_bounds (pinned by
    test_device_bounds_shortcut)."""
    w = c.w
    for b in requests:
        key = (b, int(c.L[b]) // w.page_size)
        if key in c._oracle_bounds:
            continue
        n_b = c.n_pages(b)
        out = np.full((n_b, w.num_kv_heads, 2, w.head_dim_qk), np.nan)
        n_full = int(c.L[b]) // w.page_size
        if n_full:
            kk = c.K[c.pt[b, :n_full].long()]
            out[:n_full, :, 0] = kk.amin(dim=2).double().cpu().numpy()
            out[:n_full, :, 1] = kk.amax(dim=2).double().cpu().numpy()
        c._oracle_bounds[key] = out


def gap_ok(scores: np.ndarray, k: int) -> bool:
    if len(scores) <= k or k == 0:
        return True
    s = np.sort(scores)[::-1]
    return (s[k - 1] - s[k]) > GAP_REL * np.max(np.abs(scores))


def fix_gaps(c: Case, requests, rule: str = "centroid") -> int:
    """Redraw query groups of the listed requests until every group's score
    gap is wide enough.  ``rule`` "centroid" scores by the oracle centroids,
    "bounds" by Quest's criticality over the oracle key bounds.  Returns the
    number of redraws."""
    w = c.w
    G = w.group
    redraws = 0
    for b in requests:
        n_b = c.n_pages(b)
        cand = orc.candidate_pages(n_b, w.n_bos, w.n_eos)
        if len(cand) <= w.topk:
            continue
        summ = c.oracle_centroids(b) if rule == "centroid" else c.oracle_bounds(b)
        for h in range(w.num_kv_heads):
            while True:
                q = c.q_host[b, h * G:(h + 1) * G].to(torch.float64).numpy()
                qbar = orc.group_mean_query(q, 1)
                if rule == "centroid":
                    s = orc.page_scores(qbar, summ[:, h:h + 1], cand)[0]
                else:
                    s = orc.bound_scores(qbar, summ[:, h:h + 1], cand)[0]
                if gap_ok(s, w.topk):
                    break
                c.attempts[b, h] += 1
                redraws += 1
                if c.attempts[b, h] > MAX_ATTEMPTS:
                    raise RuntimeError(f"no query draw with a score gap for ({b},{h})")
                g = synth.draw_query_group(w, c.layout, c.step, b, h, int(c.attempts[b, h]))
                c.q_host[b, h * G:(h + 1) * G] = torch.from_numpy(g).to(w.torch_dtype)
    return redraws


def oracle_selection(c: Case, b: int, rule: str = "centroid") -> np.ndarray:
    """The oracle's selection table [H_kv, k_tot] of request b."""
    w = c.w
    n_b = c.n_pages(b)
    q = c.q_host[b].to(torch.float64).numpy()
    if rule == "centroid":
        sel = orc.select_pages(q, c.oracle_centroids(b)[:n_b], n_b, w.topk, w.n_bos, w.n_eos)
    else:
        sel = orc.select_pages_quest(q, c.oracle_bounds(b), n_b, w.topk, w.n_bos, w.n_eos)
    return orc.selection_table(sel, w.k_tot)


def assert_all_selections(c: Case, sel_dev: torch.Tensor, rule: str = "centroid"):
    """Every (request, KV head) row of the GPU selection equals the oracle's,
    bit for bit."""
    got = sel_dev.cpu().numpy()
    for b in range(c.w.batch):
        want = oracle_selection(c, b, rule)
        bad = np.nonzero((got[b] != want).any(axis=1))[0]
        assert len(bad) == 0, f"request {b}: selected pages differ on KV heads {bad.tolist()}"


def oracle_request(c: Case, b: int, sparse: bool = True):
    """(selection table [H_kv, k_tot] or None, o [H_q, D_v], lse [H_q])."""
    w = c.w
    k, v = c.request_pages(b)
    q = c.q_host[b].to(torch.float64).numpy()
    L = int(c.L[b])
    vd = w.head_dim_v if v is None else None
    if sparse:
        cent = c.oracle_centroids(b, k)
        sel, o, lse = orc.sparse_decode_request(q, k, v, cent, L, w.sm_scale, w.topk,
                                                w.n_bos, w.n_eos, v_dims=vd)
        return orc.selection_table(sel, w.k_tot), o, lse
    o, lse = orc.decode_request(q, k, v, L, w.sm_scale, None, v_dims=vd)
    return None, o, lse


def out_tolerance(dtype: str):
    """(max-abs, relative L2) bounds for outputs; lse bound."""
    if dtype == "f32":
        return 1e-4, 1e-5, 1e-4
    return 2e-2, 1e-2, 1e-3


def assert_close_out(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    ma, rel, _ = out_tolerance(dtype)
    d = np.abs(got - want)
    err = float(d.max()) if d.size else 0.0
    r = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    assert err <= ma and r <= rel, f"{what}: max|d|={err:.3g} (<= {ma}), rel={r:.3g} (<= {rel})"


def assert_close_lse(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    tol = out_tolerance(dtype)[2]
    d = float(np.max(np.abs(got - want)))
    assert d <= tol, f"{what}: lse max|d|={d:.3g} (<= {tol})"


def assert_centroids(c: Case, pages_phys: np.ndarray):
    """GPU centroid rows of the listed physical pages vs the oracle."""
    if len(pages_phys) == 0:
        return
    idx = torch.from_numpy(pages_phys.astype(np.int64)).to(c.K.device)
    got = to_f64(c.cent[idx])
    kp = to_f64(c.K[idx])
    want = orc.page_centroids(kp, c.w.dtype)
    if c.w.dtype == "bf16":
        tol = np.maximum(bf16_ulp(want), 2.0 ** -20)
    else:
        tol = 2e-6 * np.abs(kp).mean(axis=2) + 2.0 ** -24 * np.abs(want)
    bad = np.abs(got - want) > tol
    assert not bad.any(), f"{int(bad.sum())} centroid elements off by more than the bound"


def run_indexer(vx, c: Case, q_dev: torch.Tensor, ws=None):
    w = c.w
    bt = c.batch(vx)
    sel = torch.empty((w.batch, w.num_kv_heads, w.k_tot), dtype=torch.int32, device=q_dev.device)
    if ws is None:
        ws = vx.alloc_workspace(vx.VX_OP_SCORE_TOPK, c.kv, bt)
    vx.score_topk(c.kv, bt, q_dev, w.topk, w.n_bos, w.n_eos, sel, ws)
    return sel


def run_sparse(vx, c: Case, q_dev, sel, ws=None):
    w = c.w
    bt = c.batch(vx)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim_v), dtype=w.torch_dtype,
                      device=q_dev.device)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=q_dev.device)
    if ws is None:
        ws = vx.alloc_workspace(vx.VX_OP_SPARSE_DECODE, c.kv, bt, w.k_tot)
    vx.sparse_paged_decode(c.kv, bt, q_dev, sel, w.sm_scale, out, lse, ws)
    return out, lse


def run_full(vx, c: Case, q_dev, ws=None):
    w = c.w
    bt = c.batch(vx)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim_v), dtype=w.torch_dtype,
                      device=q_dev.device)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=q_dev.device)
    if ws is None:
        ws = vx.alloc_workspace(vx.VX_OP_FULL_DECODE, c.kv, bt)
    vx.full_paged_decode(c.kv, bt, q_dev, w.sm_scale, out, lse, ws)
    return out, lse


def run_step(vx, c: Case, q_dev, update: bool = True, ws=None):
    """vx_sparse_decode_step: returns (sel, out, lse)."""
    w = c.w
    bt = c.batch(vx)
    # sentinels: a row the call fails to write shows up in the comparison
    sel = torch.full((w.batch, w.num_kv_heads, w.k_tot), -7, dtype=torch.int32,
                     device=q_dev.device)
    out = torch.full((w.batch, w.num_q_heads, w.head_dim_v), float("nan"), dtype=w.torch_dtype,
                     device=q_dev.device)
    lse = torch.full((w.batch, w.num_q_heads), float("nan"), dtype=torch.float32,
                     device=q_dev.device)
    if ws is None:
        ws = vx.alloc_workspace(vx.VX_OP_DECODE_STEP, c.kv, bt, w.k_tot)
    vx.sparse_decode_step(c.kv, bt, q_dev, w.topk, w.n_bos, w.n_eos, update, w.sm_scale, sel,
                          out, lse, ws)
    return sel, out, lse


def single_split(vx, c: Case) -> bool:
    """Whether vx_sparse_paged_decode plans one split for this case."""
    return vx.workspace_size(vx.VX_OP_SPARSE_DECODE, c.kv, c.batch(vx), c.w.k_tot) == 0


def build_setup_centroids(vx, c: Case):
    """Centroids of the pages full before step 0's token only."""
    ids = synth.setup_full_pages(c.layout)
    if len(ids):
        vx.centroid_update(c.kv, torch.from_numpy(ids.astype(np.int32)).to(c.K.device))


def build_centroids(vx, c: Case):
    """Bulk centroids of every page full before step 0, then step 0's completions."""
    ids = np.concatenate([synth.setup_full_pages(c.layout), synth.completed_pages(c.layout, 0)])
    t = torch.from_numpy(ids.astype(np.int32)).to(c.K.device)
    vx.centroid_update(c.kv, t)
    return ids


def sample_requests(B: int, n: int = 3):
    if B <= n:
        return list(range(B))
    return sorted({0, B - 1, *range(B // n, B - 1, max(1, B // n))})[:n + 1]


def describe(w) -> str:
    return (f"{w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
            f"D={w.head_dim_qk}/{w.head_dim_v} Sp={w.page_size} {w.dtype} k={w.topk}")


def log(msg: str):
    print(msg, flush=True)


__all__ = [n for n in dir() if not n.startswith("_")] + ["math"]
