"""Workload definitions and seeded generators.

The five full-size workloads follow the evaluation setting of the Vortex
pages (decode over a paged KV cache with 16-token pages, top-k pages plus one
reserved first and one reserved last page; vortex_torch README, "Using Your
Sparse Attention with SGLang"), at the shapes of the models the pages name
(Qwen3-0.6B in the README; an MLA model with one shared latent KV head, digg
thread post [4/6]).  The pages' evaluation suites and trained weights are not
used: every value here is synthetic and seeded.

Position semantics used throughout: at decode step ``s`` request ``b`` holds
``L0[b] + s`` tokens, the last of which (position ``L0[b] + s - 1``) is the
token being decoded; its K/V are already in the pool.  The K/V of every
position a run will ever reach are generated up front, so "appending" a token
moves the sequence length and nothing else.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np
import torch

# Pages are generated this many at a time so that the random stream is the
# same whatever the pool size's factorisation.
_GEN_CHUNK_PAGES = 2048

# Number of Gaussian clusters of page means in the "clusters" structure.
_N_CLUSTERS = 8

# Dims of the positional (rotary) part of an MLA key: the last 64 of 576.
_MLA_ROPE_DIMS = 64
_ROPE_BASE = 10000.0


@dataclass(frozen=True)
class Workload:
    """Shapes, structure and seed of one synthetic decode workload."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    dtype: str                     # "f32" | "bf16"
    topk: int
    structure: str                 # "gauss" | "page_offset" | "clusters" | "mla"
    seed: int
    n_bos: int = 1
    n_eos: int = 1
    seq_len: Optional[int] = None                    # same length for every request
    seq_lens: Optional[Sequence[int]] = None         # explicit per-request lengths
    seq_len_range: Optional[tuple] = None            # inclusive uniform integer range
    steps: int = 1                 # decode steps; each after the first appends a token
    pool_pages: Optional[int] = None   # explicit pool size (else exact fit + spare)
    spare_pages: int = 0               # extra free pages beyond what the run needs
    v_aliases_k: bool = False          # MLA: V is the first head_dim_v dims of K
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def k_tot(self) -> int:
        return self.topk + self.n_bos + self.n_eos

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim_qk)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# --------------------------------------------------------------------------
# The five full-size workloads (seeds 101..105).
# --------------------------------------------------------------------------
WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="tiny_b1_l1k_f32",
            description="batch 1, 2 query heads on 1 KV head, head_dim 64, fp32, "
                        "16-token pages, 1024 tokens in a 128-page pool; N(0,1)",
            batch=1, num_q_heads=2, num_kv_heads=1, head_dim_qk=64, head_dim_v=64,
            page_size=16, dtype="f32", topk=8, structure="gauss", seed=101,
            seq_len=1024, pool_pages=128,
        ),
        Workload(
            name="qwen3_0p6b_b32_l32k",
            description="Qwen3-0.6B-like attention layer: batch 32, 16 query / 8 KV "
                        "heads, head_dim 128, bf16, 16-token pages, 32768 tokens per "
                        "request over a shuffled 65536-page pool; per-page mean "
                        "offsets (std 0.5)",
            batch=32, num_q_heads=16, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
            page_size=16, dtype="bf16", topk=30, structure="page_offset", seed=102,
            seq_len=32768,
        ),
        Workload(
            name="hetero_b128_l4k_64k",
            description="heterogeneous batch: 128 requests, lengths uniform in "
                        "[4096, 65536], 32 query / 8 KV heads, head_dim 128, bf16, "
                        "16-token pages; 32 decode steps each appending one token",
            batch=128, num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
            page_size=16, dtype="bf16", topk=64, structure="page_offset", seed=103,
            seq_len_range=(4096, 65536), steps=32, spare_pages=128,
        ),
        Workload(
            name="long_b8_l128k",
            description="long context: batch 8, 131072 tokens (8192 pages), 64 query "
                        "/ 8 KV heads, head_dim 128, bf16, 16-token pages; page means "
                        "from 8 Gaussian clusters per KV head",
            batch=8, num_q_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
            page_size=16, dtype="bf16", topk=256, structure="clusters", seed=104,
            seq_len=131072,
        ),
        Workload(
            name="mla_b64_l32k",
            description="MLA-style: batch 64, 32768 tokens, 32 query heads on one "
                        "latent KV head (512 latent + 64 rotary dims = 576-dim key, "
                        "value = the 512 latent dims), bf16, 64-token pages",
            batch=64, num_q_heads=32, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
            page_size=64, dtype="bf16", topk=32, structure="mla", seed=105,
            seq_len=32768, v_aliases_k=True,
        ),
    ]
}

# Reduced variants: same structure, small enough for the oracle to finish in
# seconds, with several pages per split and a partial last page.
SMALL_WORKLOADS = {
    w.name: w
    for w in [
        WORKLOADS["tiny_b1_l1k_f32"],
        WORKLOADS["qwen3_0p6b_b32_l32k"].with_(
            name="qwen3_small", batch=3, seq_lens=(3001, 1000, 517), seq_len=None,
            seed=202),
        WORKLOADS["hetero_b128_l4k_64k"].with_(
            name="hetero_small", batch=6, seq_len_range=(300, 2200), steps=20,
            spare_pages=6, seed=203),
        WORKLOADS["long_b8_l128k"].with_(
            name="long_small", batch=2, seq_len=8200, seed=204),
        WORKLOADS["mla_b64_l32k"].with_(
            name="mla_small", batch=3, seq_lens=(3000, 2113, 4096), seq_len=None,
            seed=205),
    ]
}


def get_workload(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in SMALL_WORKLOADS:
        return SMALL_WORKLOADS[name]
    raise KeyError(f"unknown workload {name!r}")


# --------------------------------------------------------------------------
# Page layout: sequence lengths, page table, pool size, completions per step.
# --------------------------------------------------------------------------
@dataclass
class PageLayout:
    workload: Workload
    seq_lens0: np.ndarray          # int64 [B]: tokens at step 0 (incl. the decoded one)
    page_table: np.ndarray         # int32 [B, max_pages]; unused entries are 0
    num_pages: int                 # physical pool size P
    max_pages: int                 # page-table row width
    phys_to_logical: np.ndarray = field(repr=False, default=None)  # int64 [P], -1 if free

    @property
    def steps(self) -> int:
        return self.workload.steps


def _initial_seq_lens(w: Workload) -> np.ndarray:
    if w.seq_lens is not None:
        assert len(w.seq_lens) == w.batch
        return np.asarray(w.seq_lens, dtype=np.int64)
    if w.seq_len is not None:
        return np.full(w.batch, w.seq_len, dtype=np.int64)
    lo, hi = w.seq_len_range
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 0x5E9]))
    return rng.integers(lo, hi, size=w.batch, endpoint=True).astype(np.int64)


def _pages(n_tokens: int, page_size: int) -> int:
    return -(-int(n_tokens) // page_size)


def build_layout(w: Workload) -> PageLayout:
    """Sequence lengths and a page table over a seeded shuffled pool.

    Request b first receives ceil(L0[b] / S_p) pages, taken in order from a
    seeded permutation of the pool; what remains of the permutation is the
    free list.  At each later step a request whose new token starts a page
    pops the next free page (requests in index order).
    """
    S = w.page_size
    L0 = _initial_seq_lens(w)
    final = L0 + (w.steps - 1)
    need = np.array([_pages(x, S) for x in final], dtype=np.int64)
    max_pages = int(need.max())
    total_needed = int(need.sum())
    if w.pool_pages is not None:
        P = int(w.pool_pages)
    else:
        P = total_needed + int(w.spare_pages)
    if P < total_needed:
        raise ValueError(f"pool of {P} pages cannot hold {total_needed}")
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 0xA11C]))
    perm = rng.permutation(P).astype(np.int64)
    pt = np.zeros((w.batch, max_pages), dtype=np.int32)
    cursor = 0
    n_live = np.zeros(w.batch, dtype=np.int64)
    for b in range(w.batch):
        n0 = _pages(L0[b], S)
        pt[b, :n0] = perm[cursor:cursor + n0]
        cursor += n0
        n_live[b] = n0
    for s in range(1, w.steps):
        for b in range(w.batch):
            pos = L0[b] + s - 1          # position of the token decoded at step s
            if pos % S == 0:
                pt[b, n_live[b]] = perm[cursor]
                cursor += 1
                n_live[b] += 1
    assert np.array_equal(n_live, need)
    p2l = np.full(P, -1, dtype=np.int64)
    for b in range(w.batch):
        p2l[pt[b, :need[b]]] = np.arange(need[b])
    return PageLayout(workload=w, seq_lens0=L0, page_table=pt, num_pages=P,
                      max_pages=max_pages, phys_to_logical=p2l)


def step_seq_lens(layout: PageLayout, step: int) -> np.ndarray:
    """Tokens per request at decode step ``step`` (int64 [B])."""
    assert 0 <= step < layout.steps
    return layout.seq_lens0 + step


def completed_pages(layout: PageLayout, step: int) -> np.ndarray:
    """Physical ids of the pages that the token decoded at ``step`` fills up."""
    S = layout.workload.page_size
    L = step_seq_lens(layout, step)
    out = []
    for b in range(layout.workload.batch):
        if L[b] % S == 0:
            out.append(layout.page_table[b, L[b] // S - 1])
    return np.asarray(out, dtype=np.int32)


def setup_full_pages(layout: PageLayout) -> np.ndarray:
    """Physical ids of the pages already full before step 0's token arrives."""
    S = layout.workload.page_size
    out = []
    for b in range(layout.workload.batch):
        n_full = (int(layout.seq_lens0[b]) - 1) // S
        out.extend(layout.page_table[b, :n_full].tolist())
    return np.asarray(out, dtype=np.int32)


# --------------------------------------------------------------------------
# Rotary tables (input structure of the MLA workload only).
# --------------------------------------------------------------------------
def rope_tables(positions, dims: int = _MLA_ROPE_DIMS, base: float = _ROPE_BASE):
    """cos/sin [len(positions), dims/2] in fp64 for NeoX-style rotate-half
    rotary; an int argument n means positions 0..n-1."""
    if np.isscalar(positions):
        positions = np.arange(int(positions))
    half = dims // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / dims)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _rotate(x, cos, sin):
    """Rotate-half on the last axis of x (numpy or torch), half = x.shape[-1]/2."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    if isinstance(x, torch.Tensor):
        return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


# --------------------------------------------------------------------------
# KV pool.
# --------------------------------------------------------------------------
def make_kv_pool(w: Workload, layout: PageLayout, device="cpu"):
    """K and V pools [P, H_kv, S_p, D] in the workload dtype, drawn in
    physical-page order from a torch generator seeded with the workload seed.
    For MLA the V pool is None (V is the first head_dim_v dims of K)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(w.seed))
    P, H, S = layout.num_pages, w.num_kv_heads, w.page_size
    dt = w.torch_dtype
    K = torch.empty((P, H, S, w.head_dim_qk), dtype=dt, device=dev)
    V = None if w.v_aliases_k else torch.empty((P, H, S, w.head_dim_v), dtype=dt, device=dev)

    centres = None
    if w.structure == "clusters":
        centres = {
            "k": 0.5 * torch.randn((_N_CLUSTERS, H, w.head_dim_qk), generator=gen,
                                   device=dev, dtype=torch.float32),
            "v": 0.5 * torch.randn((_N_CLUSTERS, H, w.head_dim_v), generator=gen,
                                   device=dev, dtype=torch.float32),
        }
    cos_t = sin_t = None
    if w.structure == "mla":
        cos, sin = rope_tables(layout.max_pages * S)
        cos_t = torch.from_numpy(cos.astype(np.float32)).to(dev)
        sin_t = torch.from_numpy(sin.astype(np.float32)).to(dev)
        p2l = torch.from_numpy(np.maximum(layout.phys_to_logical, 0)).to(dev)

    def draw(n, D, which):
        x = torch.randn((n, H, S, D), generator=gen, device=dev, dtype=torch.float32)
        if w.structure == "page_offset":
            x += 0.5 * torch.randn((n, H, 1, D), generator=gen, device=dev,
                                   dtype=torch.float32)
        elif w.structure == "clusters":
            cid = torch.randint(0, _N_CLUSTERS, (n, H), generator=gen, device=dev)
            jitter = 0.1 * torch.randn((n, H, D), generator=gen, device=dev,
                                       dtype=torch.float32)
            heads = torch.arange(H, device=dev)[None, :].expand(n, H)
            mean = centres[which][cid, heads] + jitter
            x += mean[:, :, None, :]
        return x

    for p0 in range(0, P, _GEN_CHUNK_PAGES):
        n = min(_GEN_CHUNK_PAGES, P - p0)
        xk = draw(n, w.head_dim_qk, "k")
        if w.structure == "mla":
            r = _MLA_ROPE_DIMS
            pos = (p2l[p0:p0 + n, None] * S
                   + torch.arange(S, device=dev)[None, :])        # [n, S]
            c = cos_t[pos][:, None, :, :]                          # [n, 1, S, r/2]
            s_ = sin_t[pos][:, None, :, :]
            xk[..., -r:] = _rotate(xk[..., -r:], c, s_)
        K[p0:p0 + n] = xk.to(dt)
        if V is not None:
            V[p0:p0 + n] = draw(n, w.head_dim_v, "v").to(dt)
    return K, V


# --------------------------------------------------------------------------
# Queries (host side, numpy; one seed per (step, request, KV head, attempt)).
# --------------------------------------------------------------------------
def draw_query_group(w: Workload, layout: PageLayout, step: int, b: int, h: int,
                     attempt: int = 0) -> np.ndarray:
    """The G query rows of KV head h of request b at ``step`` (float32 [G, D]).

    Attempt 0 is the default draw; a caller that needs to redraw a group
    (for instance to keep a margin between the k-th and (k+1)-th page score)
    asks for attempt 1, 2, ...  MLA queries get the rotary part applied at
    the position of the decoded token."""
    ss = np.random.SeedSequence([w.seed, 0x0, step, b, h, attempt])
    rng = np.random.default_rng(ss)
    x = rng.standard_normal((w.group, w.head_dim_qk))
    if w.structure == "mla":
        r = _MLA_ROPE_DIMS
        pos = int(step_seq_lens(layout, step)[b]) - 1
        cos, sin = rope_tables([pos])
        x[:, -r:] = _rotate(x[:, -r:], cos[0], sin[0])
    return x.astype(np.float32)


def make_queries(w: Workload, layout: PageLayout, step: int = 0,
                 attempts: Optional[np.ndarray] = None) -> torch.Tensor:
    """Q [B, H_q, D_qk] as a CPU tensor in the workload dtype.

    ``attempts`` (int [B, H_kv], optional) picks the draw per group."""
    G = w.group
    q = np.empty((w.batch, w.num_q_heads, w.head_dim_qk), dtype=np.float32)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            a = 0 if attempts is None else int(attempts[b, h])
            q[b, h * G:(h + 1) * G] = draw_query_group(w, layout, step, b, h, a)
    return torch.from_numpy(q).to(w.torch_dtype)
