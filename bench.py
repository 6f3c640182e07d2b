#!/usr/bin/env python3
"""Benchmark of block-top-k sparse paged decode on one MI355X.

One step = one decode query per request through one attention layer, in one
call of vx_sparse_decode_step: the centroid of the page this step's token
completes, the indexer (group-mean query, centroid scores through the page
table, exact top-k with the reserved first / last pages) and attention over
the selected pages.  Steps cycle over several independent layers (separate
KV pools and centroid tables of the same shape), so a step's working set is
not still sitting in the 256 MB on-package cache from the previous visit.
After the timed steps the same work is run once more as separate calls
(vx_centroid_update, vx_score_topk, vx_sparse_paged_decode) for a per-stage
breakdown, then the dense paged decode over every page for the speedup.  All
inputs are synthetic and seeded.

The headline is the heterogeneous batch (128 requests of 4k-64k tokens, the
largest workload); every other workload is timed after it (sparse step and
dense decode) into the line's "configs" map.

Prints one JSON line on stdout.  Progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--only]
"""

import argparse
import gc
import json
import math
import os
import re
import sys
import time

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
MALL_BYTES = 256 << 20           # on-package cache the layer rotation has to defeat
METRIC = "sparse decode queries/s + achieved HBM GB/s (% peak) + speedup vs dense paged"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- traffic
_ROOT = os.path.dirname(os.path.abspath(__file__))


def _source_sha256():
    """Hash of the kernel sources and the C header (names and bytes)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(_ROOT, "block_sparse_paged_amd", "csrc", "*")))
    files.append(os.path.join(_ROOT, "include", "vx.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per step of this workload from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE record (copy-calibrated), or None when there is
    none or the kernel sources changed since the counters were taken."""
    path = os.path.join(_ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != _source_sha256():
        return None
    w = rec.get("workloads", {}).get(workload)
    return int(w["hbm_bytes_per_step"]) if w else None


# ---------------------------------------------------------------- bytes
def _pages(L, S):
    return -(-int(L) // S)


def indexer_bytes(w, L):
    """Bytes the indexer must move for one request of length L: candidate
    centroid rows, page-table entries, the query and the selection."""
    n_b = _pages(L, w.page_size)
    n_c = max(n_b - w.n_bos - w.n_eos, 0)
    e = w.elem_bytes
    return (n_c * w.num_kv_heads * w.head_dim_qk * e + 4 * n_b
            + w.num_q_heads * w.head_dim_qk * e + 4 * w.num_kv_heads * w.k_tot)


def attention_bytes(w, L, dense=False):
    """Bytes attention must move for one request: K/V of the attended
    tokens (MLA reads each 576-dim row once), q, o, and the selection and
    page-table entries it walks."""
    S, e = w.page_size, w.elem_bytes
    n_b = _pages(L, S)
    row = w.head_dim_qk * e if w.v_aliases_k else (w.head_dim_qk + w.head_dim_v) * e
    qo = w.num_q_heads * (w.head_dim_qk + w.head_dim_v) * e
    if dense:
        return int(L) * w.num_kv_heads * row + 4 * n_b + qo
    pages = min(n_b, w.k_tot)
    tokens = min(pages * S, int(L))
    return tokens * w.num_kv_heads * row + qo + 8 * w.num_kv_heads * pages


def centroid_bytes(w, n_pages):
    e = w.elem_bytes
    return n_pages * (w.num_kv_heads * w.head_dim_qk * e * (w.page_size + 1) + 4)


# ---------------------------------------------------------------- cpu baseline
def host_cores():
    """Host cores this process may use: the affinity mask, capped by
    OMP_NUM_THREADS when the environment sets a smaller share."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and 0 < int(env) < n:
        n = int(env)
    return n


def cpu_baseline(w, lay, layer, seconds, max_requests):
    """The fp64 oracle's sparse step, timed on the host on a sample of
    requests of layer 0, with the BLAS thread pool on every host core this
    process may use."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle as orc
    import synth

    L = synth.step_seq_lens(lay, 0)
    reqs = list(range(min(w.batch, max_requests)))
    data = []
    for b in reqs:
        n = _pages(L[b], w.page_size)
        idx = layer["pt"][b, :n].long()
        k = layer["K"][idx].float().cpu().numpy()
        v = None if layer["V"] is None else layer["V"][idx].float().cpu().numpy()
        q = layer["q"][b].float().cpu().numpy()
        data.append((b, k, v, q))
    cores = host_cores()
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        cents = [orc.request_centroids(k, int(L[b]) - (1 if L[b] % w.page_size == 0 else 0),
                                       w.dtype) for b, k, v, q in data]
        setup_s = time.perf_counter() - t0
        vd = w.head_dim_v if w.v_aliases_k else None
        done = 0
        t0 = time.perf_counter()
        while True:
            for (b, k, v, q), cent in zip(data, cents):
                Lb = int(L[b])
                if Lb % w.page_size == 0:          # the page this token completes
                    p = Lb // w.page_size - 1
                    cent[p] = orc.page_centroids(k[p:p + 1], w.dtype)[0]
                orc.sparse_decode_request(q, k, v, cent, Lb, w.sm_scale, w.topk, w.n_bos,
                                          w.n_eos, v_dims=vd)
                done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {
        "value": done / el, "unit": "queries/s", "cores": cores, "kind": "oracle",
        "sample": (f"{w.name}: {len(reqs)} of {w.batch} requests of layer 0 at step 0, "
                   f"{done // len(reqs)} passes ({done} sparse decode queries: completed-page "
                   f"centroid, group-mean query, centroid scores, exact top-k, attention over "
                   f"the selected pages), fp64 numpy with {cores} BLAS threads "
                   f"(affinity {len(os.sched_getaffinity(0))} cores), {el:.1f} s"),
        "setup_centroids_s": setup_s,
    }


def run_workload(args, name, full):
    """Sets up one workload's layers and times its decode step (and, with
    ``full``, every other section).  Returns the measurements; the workload's
    device memory is released before returning."""
    import numpy as np
    import torch
    import block_sparse_paged_amd as vx
    import synth

    w = synth.get_workload(name)
    lay = synth.build_layout(w)
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: {w.description}")

    T = w.steps
    L_steps = [synth.step_seq_lens(lay, s) for s in range(T)]
    step_bytes = [sum(indexer_bytes(w, L) + attention_bytes(w, L) for L in Ls)
                  + centroid_bytes(w, len(synth.completed_pages(lay, s)))
                  for s, Ls in enumerate(L_steps)]
    mean_step_bytes = float(np.mean(step_bytes))
    pool_bytes = lay.num_pages * w.num_kv_heads * w.page_size * w.elem_bytes * (
        w.head_dim_qk + (0 if w.v_aliases_k else w.head_dim_v))
    n_layers = args.layers or max(2, math.ceil(3 * MALL_BYTES / mean_step_bytes) + 1)
    n_layers = max(1, min(n_layers, 16, int((48 << 30) // max(pool_bytes, 1))))
    log(f"step bytes {mean_step_bytes / 1e6:.1f} MB, pool {pool_bytes / 1e9:.2f} GB, "
        f"{n_layers} layers")

    pt = torch.from_numpy(lay.page_table).to(dev)
    max_len = int(lay.seq_lens0.max()) + T - 1
    seq_dev = [torch.from_numpy(L.astype(np.int32)).to(dev) for L in L_steps]
    batches = [vx.Batch(page_table=pt, seq_lens=s, num_q_heads=w.num_q_heads, max_seq_len=max_len)
               for s in seq_dev]
    done_ids = [torch.from_numpy(synth.completed_pages(lay, s)).to(dev) for s in range(T)]
    setup_ids = torch.from_numpy(synth.setup_full_pages(lay)).to(dev)

    layers = []
    for i in range(n_layers):
        wl = w.with_(seed=w.seed + 7919 * i)
        K, V = synth.make_kv_pool(wl, lay, device=dev)
        cent = torch.zeros((lay.num_pages, w.num_kv_heads, w.head_dim_qk), dtype=w.torch_dtype,
                           device=dev)
        kv = vx.PagedKV(k_cache=K, v_cache=V, centroids=cent, head_dim_v=w.head_dim_v)
        vx.centroid_update(kv, setup_ids)              # cache construction (setup)
        qs = [synth.make_queries(wl, lay, s).to(dev) for s in range(T)]
        layers.append({"K": K, "V": V, "kv": kv, "q": qs[0], "qs": qs, "pt": pt})
        log(f"layer {i} ready")
    torch.cuda.synchronize()

    sel = torch.empty((w.batch, w.num_kv_heads, w.k_tot), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim_v), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    kv0 = layers[0]["kv"]
    ws_step = vx.alloc_workspace(vx.VX_OP_DECODE_STEP, kv0, batches[0], w.k_tot)
    ws_idx = vx.alloc_workspace(vx.VX_OP_SCORE_TOPK, kv0, batches[0])
    ws_dec = vx.alloc_workspace(vx.VX_OP_SPARSE_DECODE, kv0, batches[0], w.k_tot)
    ws_full = vx.alloc_workspace(vx.VX_OP_FULL_DECODE, kv0, batches[0])
    stream = torch.cuda.current_stream()

    # prepared calls per (layer, step of the schedule)
    calls = []
    for li, lay_i in enumerate(layers):
        per = []
        for s in range(T):
            kv, bt, q = lay_i["kv"], batches[s], lay_i["qs"][s]
            c_step = vx.prepare_sparse_decode_step(kv, bt, q, w.topk, w.n_bos, w.n_eos, True,
                                                   w.sm_scale, sel, out, lse, ws_step, stream)
            c_upd = (vx.prepare_centroid_update(kv, done_ids[s], stream)
                     if done_ids[s].numel() else None)
            c_idx = vx.prepare_score_topk(kv, bt, q, w.topk, w.n_bos, w.n_eos, sel, ws_idx, stream)
            c_dec = vx.prepare_sparse_paged_decode(kv, bt, q, sel, w.sm_scale, out, lse, ws_dec,
                                                   stream)
            c_full = vx.prepare_full_paged_decode(kv, bt, q, w.sm_scale, out, lse, ws_full, stream)
            per.append({"step": c_step, "upd": c_upd, "idx": c_idx, "dec": c_dec, "full": c_full})
        calls.append(per)

    K_steps, W_steps = args.steps, args.warmup
    nL = n_layers

    def schedule(i):
        return calls[i % nL][i % T]

    # ---------------- timed sparse steps (fused entry point)
    for i in range(W_steps):
        schedule(i)["step"]()
    torch.cuda.synchronize()
    log(f"warmup {W_steps} steps done")
    # the timed region: K back-to-back launches, events only at its two ends
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K_steps):
        schedule(W_steps + i)["step"]()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = ev0.elapsed_time(ev1)
    log(f"timed {K_steps} sparse steps: {wall * 1e3:.2f} ms wall, {region_ms:.2f} ms on the stream")
    # host cost of one launch: a short burst from an idle queue, timed on the
    # host before any wait (a long run blocks once the runtime's limit of
    # launches in flight is reached, which measures the GPU instead)
    n_host = 16
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_host):
        schedule(i)["step"]()
    enqueue = (time.perf_counter() - t0) * K_steps / n_host
    torch.cuda.synchronize()
    # per-launch spread, from a second pass with events around every launch
    # (each event pair adds a few microseconds, so this pass is not the headline)
    n_ev = max(K_steps // 4, 1)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ev)]
    for i in range(n_ev):
        c = schedule(W_steps + i)
        ev[i][0].record(stream)
        c["step"]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    ms_per_step = wall * 1e3 / K_steps
    qps = w.batch * K_steps / wall

    sched = [(W_steps + i) % T for i in range(K_steps)]
    b_upd = np.mean([centroid_bytes(w, len(synth.completed_pages(lay, s))) for s in sched])
    b_idx = np.mean([sum(indexer_bytes(w, L) for L in L_steps[s]) for s in sched])
    b_dec = np.mean([sum(attention_bytes(w, L) for L in L_steps[s]) for s in sched])
    b_step = b_upd + b_idx + b_dec
    call_ms = region_ms / K_steps    # average launch duration over the timed region
    achieved = b_step / (call_ms * 1e-3) / 1e9
    step_gbps = b_step / (ms_per_step * 1e-3) / 1e9

    # ---------------- the same work as separate calls (per-stage breakdown)
    n_sep = max(K_steps // 2, 1)
    for i in range(min(W_steps, 8)):
        c = schedule(i)
        if c["upd"]:
            c["upd"]()
        c["idx"]()
        c["dec"]()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_sep)]
    t1 = time.perf_counter()
    for i in range(n_sep):
        c = schedule(W_steps + i)
        e = evs[i]
        e[0].record(stream)
        if c["upd"]:
            c["upd"]()
        e[1].record(stream)
        c["idx"]()
        e[2].record(stream)
        c["dec"]()
        e[3].record(stream)
    torch.cuda.synchronize()
    sep_wall = time.perf_counter() - t1
    seg = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])
    separate = {
        "ms_per_step": sep_wall * 1e3 / n_sep,
        "queries_per_s": w.batch * n_sep / sep_wall,
        "calls": {k: {"bytes_per_call": int(bb), "avg_ms": float(seg[:, j].mean()),
                      "gbps": bb / (seg[:, j].mean() * 1e-3) / 1e9 if seg[:, j].mean() > 0 else None}
                  for j, (k, bb) in enumerate((("vx_centroid_update", b_upd),
                                                ("vx_score_topk", b_idx),
                                                ("vx_sparse_paged_decode", b_dec)))},
    }
    log(f"separate calls: {separate['ms_per_step']:.4f} ms/step")

    # ---------------- lossy radix top-k against the exact indexer
    radix = None
    if not args.no_radix:
        rng = np.random.default_rng(w.seed + 17)
        rnd = torch.from_numpy(rng.integers(0, 2 ** 32, size=w.batch * w.num_kv_heads,
                                            dtype=np.uint64).astype(np.uint32).view(np.int32)).to(dev)
        sel_r = torch.empty_like(sel)

        def time_calls(pick):
            for i in range(min(W_steps, 8)):
                pick(i)()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n_sep):
                pick(W_steps + i)()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n_sep

        def recall(step_i):
            """Mean over (request, KV head) of |lossy top-k & exact top-k| / |exact top-k|
            (reserved pages, in both, left out)."""
            s_ = step_i % T
            e_tab, r_tab = sel.cpu().numpy(), sel_r.cpu().numpy()
            vals = []
            for b in range(w.batch):
                n_b = -(-int(L_steps[s_][b]) // w.page_size)
                res = set(range(min(w.n_bos, n_b))) | set(range(max(n_b - w.n_eos, 0), n_b))
                for h in range(w.num_kv_heads):
                    E = set(e_tab[b, h][e_tab[b, h] >= 0].tolist()) - res
                    R = set(r_tab[b, h][r_tab[b, h] >= 0].tolist()) - res
                    if E:
                        vals.append(len(E & R) / len(E))
            return float(np.mean(vals)), float(np.mean(np.array(vals) < 1.0))

        radix = {"exact_indexer_ms": time_calls(lambda i: schedule(i)["idx"]), "levels": {}}
        for levels in (1, 2):
            prep = {}

            def pick(i, levels=levels, prep=prep):
                key = (i % nL, i % T)
                if key not in prep:
                    kv, bt, q = layers[key[0]]["kv"], batches[key[1]], layers[key[0]]["qs"][key[1]]
                    prep[key] = vx.prepare_score_topk_radix(kv, bt, q, w.topk, w.n_bos, w.n_eos,
                                                            levels, rnd, sel_r, ws_idx, stream)
                return prep[key]
            ms = time_calls(pick)
            rec, frac = [], []
            for i in range(min(nL * T, 8)):
                schedule(i)["idx"]()
                pick(i)()
                torch.cuda.synchronize()
                r_, f_ = recall(i)
                rec.append(r_)
                frac.append(f_)
            radix["levels"][str(levels)] = {
                "avg_ms": ms, "speedup_vs_exact": radix["exact_indexer_ms"] / ms,
                "recall_at_k": float(np.mean(rec)),
                "units_not_exact": float(np.mean(frac))}
        log(f"radix top-k: {radix}")

    # ---------------- the write path: vx_append_kv (rows rewritten with their own
    # values, so the layers stay as they are)
    append = None
    if not args.no_append:
        lay0, s0 = layers[0], 0
        L0 = np.asarray(L_steps[s0], dtype=np.int64)
        e = 2 if w.dtype == "bf16" else 4
        K0 = lay0["K"]
        V0 = lay0["V"]
        append = {}
        for n in (1, 64):
            pos = np.concatenate([np.arange(max(int(Lb) - n, 0), int(Lb)) for Lb in L0])
            req = np.concatenate([np.full(min(n, int(Lb)), b) for b, Lb in enumerate(L0)])
            pages = torch.from_numpy(lay.page_table[req, pos // w.page_size].astype(np.int64)).to(dev)
            slots = torch.from_numpy((pos % w.page_size).astype(np.int64)).to(dev)
            k_src = K0[pages, :, slots].contiguous()
            v_src = None if V0 is None else V0[pages, :, slots].contiguous()
            n_req = np.minimum(n, L0)
            starts = torch.from_numpy(np.concatenate([[0], np.cumsum(n_req)[:-1]]).astype(np.int32)).to(dev)
            n_new = torch.from_numpy(n_req.astype(np.int32)).to(dev)
            call = vx.prepare_append_kv(lay0["kv"], batches[s0], k_src, v_src, starts, n_new, n,
                                        True, stream)
            # algorithmic bytes: new rows read and written; each filled page's
            # old rows read and its centroid row written
            dv = 0 if V0 is None else w.head_dim_v
            b_rows = 2 * len(pos) * w.num_kv_heads * (w.head_dim_qk + dv) * e
            b_cent = 0
            for Lb, nb in zip(L0, n_req):
                first = int(Lb) - int(nb)
                for p_ in range(first // w.page_size, int(Lb) // w.page_size):
                    old = max(first - p_ * w.page_size, 0)
                    b_cent += w.num_kv_heads * w.head_dim_qk * e * (old + 1)
            for _ in range(5):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 200
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            append["decode_1_token" if n == 1 else f"write_{n}_tokens"] = {
                "tokens_per_request": n, "avg_ms": ms, "bytes": int(b_rows + b_cent),
                "gbps": (b_rows + b_cent) / (ms * 1e-3) / 1e9}
        log(f"append: {append}")

    # ---------------- the second summary rule: per-page key bounds (Quest's
    # criticality) against the centroid indexer, same steps and layers
    bounds_sec = None
    if not args.no_bounds and not w.v_aliases_k:
        setup_bnd = [torch.zeros((lay.num_pages, w.num_kv_heads, 2, w.head_dim_qk),
                                 dtype=w.torch_dtype, device=dev) for _ in layers]
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for tab, lay_i in zip(setup_bnd, layers):        # cache construction (setup)
            vx.bounds_update(lay_i["kv"], tab, setup_ids, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        build_ms = e0.elapsed_time(e1) / len(setup_bnd)
        sel_b = torch.empty_like(sel)
        prep_b = {}

        def pick_b(i):
            key = (i % nL, i % T)
            if key not in prep_b:
                kv, bt, q = layers[key[0]]["kv"], batches[key[1]], layers[key[0]]["qs"][key[1]]
                prep_b[key] = vx.prepare_score_topk_bounds(kv, bt, setup_bnd[key[0]], q, w.topk,
                                                           w.n_bos, w.n_eos, sel_b, ws_idx, stream)
            return prep_b[key]

        def time_pick(pick):
            for i in range(min(W_steps, 8)):
                pick(i)()
            torch.cuda.synchronize()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for i in range(n_sep):
                pick(W_steps + i)()
            a1.record(stream)
            torch.cuda.synchronize()
            return a0.elapsed_time(a1) / n_sep

        ms_c = time_pick(lambda i: schedule(i)["idx"])
        ms_b = time_pick(pick_b)
        # the whole step under the bound rule (vx_sparse_decode_step_bounds,
        # with the completed pages' bounds), beside the centroid rule's step
        prep_s = {}

        def pick_s(i):
            key = (i % nL, i % T)
            if key not in prep_s:
                kv, bt, q = layers[key[0]]["kv"], batches[key[1]], layers[key[0]]["qs"][key[1]]
                prep_s[key] = vx.prepare_sparse_decode_step_bounds(
                    kv, bt, setup_bnd[key[0]], q, w.topk, w.n_bos, w.n_eos, True, w.sm_scale,
                    sel_b, out, lse, ws_step, stream)
            return prep_s[key]

        ms_sc = time_pick(lambda i: schedule(i)["step"])
        ms_sb = time_pick(pick_s)
        overlap = []
        for i in range(min(nL * T, 8)):
            schedule(i)["idx"]()
            pick_b(i)()
            torch.cuda.synchronize()
            s_ = i % T
            e_tab, b_tab = sel.cpu().numpy(), sel_b.cpu().numpy()
            for bq in range(w.batch):
                n_b = -(-int(L_steps[s_][bq]) // w.page_size)
                res = set(range(min(w.n_bos, n_b))) | set(range(max(n_b - w.n_eos, 0), n_b))
                for h in range(w.num_kv_heads):
                    E = set(e_tab[bq, h][e_tab[bq, h] >= 0].tolist()) - res
                    Bs = set(b_tab[bq, h][b_tab[bq, h] >= 0].tolist()) - res
                    if E:
                        overlap.append(len(E & Bs) / len(E))
        # the indexer's bytes with two summary rows per candidate instead of one
        rows = np.mean([sum(max(-(-int(Lb) // w.page_size) - w.n_bos - w.n_eos, 0) for Lb in L_steps[s])
                        for s in sched]) * w.num_kv_heads * w.head_dim_qk * w.elem_bytes
        b_bnd = b_idx + rows
        b_sb = b_step + rows
        bounds_sec = {"indexer_ms": ms_b, "centroid_indexer_ms": ms_c, "bytes_per_call": int(b_bnd),
                      "gbps": b_bnd / (ms_b * 1e-3) / 1e9,
                      "step_ms": ms_sb, "centroid_step_ms": ms_sc, "step_bytes": int(b_sb),
                      "step_gbps": b_sb / (ms_sb * 1e-3) / 1e9,
                      "setup_build_ms_per_layer": build_ms,
                      "overlap_with_centroid_topk": float(np.mean(overlap))}
        log(f"page bounds: {bounds_sec}")

    # ---------------- every layer in one call (vx_decode_layers), eager and as a
    # captured graph replayed; all layers sparse, then layer 0 dense (a skipped
    # layer); step 0's batch throughout
    graph = None
    if not args.no_graph:
        s0 = 0
        sels_l = [torch.empty_like(sel) for _ in range(nL)]
        outs_l = [torch.empty_like(out) for _ in range(nL)]
        lses_l = [torch.empty_like(lse) for _ in range(nL)]
        ws_l = vx.alloc_workspace(vx.VX_OP_DECODE_LAYERS, kv0, batches[s0], w.k_tot)
        kvs_l = [lay_i["kv"] for lay_i in layers]
        qs_l = [lay_i["qs"][s0] for lay_i in layers]

        def make(dense_mask, st):
            return vx.prepare_decode_layers(kvs_l, batches[s0], qs_l, dense_mask, w.topk, w.n_bos,
                                            w.n_eos, True, w.sm_scale, sels_l, outs_l, lses_l,
                                            ws_l, st)

        def time_reps(fn, reps):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t_ = time.perf_counter()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps, (time.perf_counter() - t_) * 1e3 / reps

        graph = {"layers": nL}
        reps = max(8, min(200, K_steps // nL))
        for tag, mask in (("all_sparse", [False] * nL), ("layer0_dense", [True] + [False] * (nL - 1))):
            if tag == "layer0_dense" and args.no_dense:
                continue
            r_ = reps if tag == "all_sparse" else max(4, reps // 8)
            eager = make(mask, stream)
            e_ms, e_wall = time_reps(eager, r_)
            g = vx.capture_graph(lambda st, mask=mask: make(mask, st))
            g_ms, g_wall = time_reps(g.replay, r_)
            graph[tag] = {"eager_ms_per_pass": e_wall, "graph_ms_per_pass": g_wall,
                          "eager_stream_ms": e_ms, "graph_stream_ms": g_ms,
                          "eager_us_per_layer": e_wall * 1e3 / nL,
                          "graph_us_per_layer": g_wall * 1e3 / nL}
            del g
        log(f"layers: {graph}")

    # ---------------- dense comparator
    dense = None
    if not args.no_dense:
        nd = args.dense_steps
        for i in range(min(4, nd)):
            schedule(i)["full"]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t1 = time.perf_counter()
        e0.record(stream)
        for i in range(nd):
            schedule(W_steps + i)["full"]()
        e1.record(stream)
        torch.cuda.synchronize()
        dwall = time.perf_counter() - t1
        dms = e0.elapsed_time(e1) / nd
        dbytes = np.mean([sum(attention_bytes(w, L, dense=True) for L in L_steps[(W_steps + i) % T])
                          for i in range(nd)])
        dense = {"queries_per_s": w.batch * nd / dwall, "ms_per_step": dwall * 1e3 / nd,
                 "avg_call_ms": dms, "bytes_per_step": int(dbytes),
                 "gbps": dbytes / (dms * 1e-3) / 1e9,
                 "pct_peak": 100.0 * dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        log(f"dense: {dense['ms_per_step']:.3f} ms/step")

    res = {
        "w": w, "lay": lay, "layer0": {"K": layers[0]["K"], "V": layers[0]["V"],
                                       "q": layers[0]["qs"][0], "pt": pt},
        "qps": qps, "ms_per_step": ms_per_step, "max_len": max_len, "n_layers": n_layers,
        "step_gbps": step_gbps, "achieved": achieved, "call_ms": call_ms, "b_step": b_step,
        "step_ms": step_ms, "enqueue": enqueue, "separate": separate, "radix": radix,
        "append": append, "bounds": bounds_sec, "graph": graph, "dense": dense,
        "steps": K_steps,
    }
    return res


def calibrate():
    """Plain streams of known size, timed with events on the current stream:
    device copies of 1 and 4 GiB (read + write), a gather of 64Ki random
    4 KiB pages (the access shape of a page-table walk) and a read-only sum
    of 4 GiB of bf16.  Under rocprofv3 --pmc their FETCH_SIZE / WRITE_SIZE
    per dispatch give the counters' scale; timed alone they give the GPU's
    streaming ceiling."""
    import torch
    out = {}
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for gib in (1, 4):
        n = gib << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        ms = timed(lambda: dst.copy_(src), 5)
        out[f"copy_{gib}GiB"] = {"read_bytes": n, "write_bytes": n, "ms": ms,
                                 "gbps": 2 * n / (ms * 1e-3) / 1e9}
        del src, dst
    pages = 65536
    pool = torch.ones((4 * pages, 2048), dtype=torch.bfloat16, device="cuda")
    idx = torch.randperm(4 * pages, device="cuda")[:pages]
    dst = torch.empty((pages, 2048), dtype=torch.bfloat16, device="cuda")
    ms = timed(lambda: torch.index_select(pool, 0, idx, out=dst), 5)
    nb = pages * 4096
    out["gather_64Ki_4KiB_pages"] = {"read_bytes": nb + 8 * pages, "write_bytes": nb, "ms": ms,
                                     "gbps": (2 * nb + 8 * pages) / (ms * 1e-3) / 1e9}
    del pool, dst, idx
    x = torch.ones(2 << 30, dtype=torch.bfloat16, device="cuda")
    ms = timed(lambda: torch.sum(x, dtype=torch.float32), 5)
    out["read_sum_4GiB"] = {"read_bytes": 4 << 30, "write_bytes": 4, "ms": ms,
                            "gbps": (4 << 30) / (ms * 1e-3) / 1e9}
    torch.cuda.synchronize()
    return out


def _short_kernel(name):
    """Kernel name without namespaces, return type and parameter list."""
    name = name.replace("(anonymous namespace)::", "").replace("void ", "", 1)
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    name = re.sub(r"\b(vx|at::native)::", "", name[:cut]).strip()
    return name if len(name) <= 90 else name[:87] + "..."


def summarize_trace(db_path):
    """Markdown table of a rocprofv3 --kernel-trace results database: one row
    per (kernel, grid, block, LDS) in first-launch order with the launch count
    and the average / median / minimum duration."""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = db.execute(
        "select s.display_name, d.grid_size_x, d.grid_size_y, d.grid_size_z, d.workgroup_size_x,"
        " d.group_segment_size, d.end - d.start from rocpd_kernel_dispatch d join"
        " rocpd_info_kernel_symbol s on d.kernel_id = s.id order by d.start")
    stats = {}
    for name, gx, gy, gz, wg, lds, dur in rows:
        stats.setdefault((_short_kernel(name), f"{gx // wg}x{gy}x{gz}", wg, lds), []).append(dur)
    out = ["| kernel | grid (blocks) | block | LDS B | launches | avg us | median us | min us |",
           "|---|---|---|---|---|---|---|---|"]
    for (n, g, wg, lds), d in stats.items():
        d.sort()
        out.append(f"| `{n}` | {g} | {wg} | {lds} | {len(d)} | {sum(d) / len(d) / 1e3:.2f} | "
                   f"{d[len(d) // 2] / 1e3:.2f} | {d[0] / 1e3:.2f} |")
    return "\n".join(out)


def summarize_counters(csv_dir, pattern):
    """Per-dispatch values of one rocprofv3 --pmc counter (csv output under
    csv_dir) for kernels whose name matches the regular expression pattern:
    {kernel: {"grid", "block", "dispatches", "median", "min", "max",
    "values"}} in first-dispatch order, values in KiB as the counter reports
    them (summed over the counter's instances per dispatch)."""
    import csv
    import glob
    per = {}
    for f in sorted(glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"),
                              recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = _short_kernel(r["Kernel_Name"])
                if not re.search(pattern, name):
                    continue
                key = (name, r.get("Grid_Size", r.get("Grid_Size_X")),
                       r.get("Workgroup_Size", r.get("Workgroup_Size_X")))
                d = per.setdefault(key, {})
                did = int(r["Dispatch_Id"])
                d[did] = d.get(did, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, grid, block), d in sorted(per.items(), key=lambda kv: min(kv[1])):
        vals = [d[k] for k in sorted(d)]
        srt = sorted(vals)
        out[f"{name} grid={grid} block={block}"] = {
            "dispatches": len(vals), "median": srt[len(srt) // 2], "min": srt[0],
            "max": srt[-1], "values": vals if len(vals) <= 16 else None}
    return out


def config_entry(r):
    """One workload's line in the per-workload map."""
    d = r["dense"]
    e = {
        "queries_per_s": r["qps"], "ms_per_step": r["ms_per_step"],
        "algorithmic_bytes_per_step": int(r["b_step"]),
        "launch_ms_avg_over_timed_region": r["call_ms"],
        "achieved_gbps": r["achieved"], "frac": r["achieved"] / HBM_PEAK_GBPS,
        "dense_ms_per_step": d["ms_per_step"] if d else None,
        "dense_call_ms": d["avg_call_ms"] if d else None,
        "dense_gbps": d["gbps"] if d else None,
        "dense_frac": d["gbps"] / HBM_PEAK_GBPS if d else None,
        "speedup_vs_dense": (d["ms_per_step"] / r["ms_per_step"]) if d else None,
        "traffic_bytes_per_step": measured_traffic(r["w"].name),
        "steps": r["steps"],
    }
    return e


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="hetero_b128_l4k_64k",
                    help="the headline workload (every section is timed on it)")
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload only (no per-workload map)")
    ap.add_argument("--config-steps", type=int, default=200,
                    help="timed steps of each other workload in the map")
    ap.add_argument("--config-warmup", type=int, default=20)
    ap.add_argument("--config-dense-steps", type=int, default=20)
    ap.add_argument("--layers", type=int, default=0,
                    help="distinct KV pools cycled over (0: enough to defeat the 256 MB cache)")
    ap.add_argument("--dense-steps", type=int, default=40)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-requests", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-append", action="store_true",
                    help="skip timing the write path (vx_append_kv)")
    ap.add_argument("--no-bounds", action="store_true",
                    help="skip the second summary rule (per-page key bounds)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the multi-layer call, eager and as a replayed graph")
    ap.add_argument("--no-radix", action="store_true",
                    help="skip the lossy radix top-k (vx_score_topk_radix) comparison")
    ap.add_argument("--calibrate", action="store_true",
                    help="only time plain streams of known size (copies, a page gather, a "
                         "read-only sum): the streaming ceiling, and the references that "
                         "scale rocprofv3's HBM counters")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="print a markdown table of a rocprofv3 kernel-trace database and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print per-kernel values of a rocprofv3 --pmc csv run and exit")
    ap.add_argument("--kernels", default=".",
                    help="regular expression on kernel names for --summarize-counters")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters, args.kernels), indent=1))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this library "
              f"has no multi-GPU path: each GPU would run its own shard independently)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import block_sparse_paged_amd as vx
    import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.calibrate:
        print(json.dumps(calibrate()), flush=True)
        return
    vx.load_library()
    names = [args.workload]
    if not args.only:
        names += [n for n in synth.WORKLOADS if n != args.workload]
    configs = {}
    head = None
    cpu = None
    for i, name in enumerate(names):
        full = i == 0
        sub = args if full else argparse.Namespace(**{
            **vars(args), "no_radix": True, "no_append": True, "no_bounds": True,
            "no_graph": True, "steps": args.config_steps, "warmup": args.config_warmup,
            "dense_steps": args.config_dense_steps, "layers": 0})
        r = run_workload(sub, name, full)
        configs[name] = config_entry(r)
        if full:
            head = {k: v for k, v in r.items() if k != "layer0"}
            if not args.no_cpu_baseline:
                log("timing the oracle on the host")
                cpu = cpu_baseline(r["w"], r["lay"], r["layer0"], args.cpu_seconds,
                                   args.cpu_requests)
        del r
        gc.collect()
        torch.cuda.empty_cache()

    w, r = head["w"], head
    dense = r["dense"]
    line = {
        "metric": METRIC,
        "value": r["qps"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": int(r["max_len"]),
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim_qk": w.head_dim_qk, "head_dim_v": w.head_dim_v,
                   "page_size": w.page_size, "topk": w.topk, "n_bos": w.n_bos,
                   "n_eos": w.n_eos, "layers_cycled": r["n_layers"]},
        "achieved_gbps": r["step_gbps"],
        "pct_peak": 100.0 * r["step_gbps"] / HBM_PEAK_GBPS,
        "speedup_vs_dense": (dense["ms_per_step"] / r["ms_per_step"]) if dense else None,
        "roofline": {"bound": "hbm", "kernel": "vx_sparse_decode_step",
                     "achieved": r["achieved"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": r["achieved"] / HBM_PEAK_GBPS, "traffic": measured_traffic(w.name),
                     "traffic_unit": "HBM bytes per step (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)"},
        "cpu_baseline": cpu,
        "algorithmic_bytes_per_step": int(r["b_step"]),
        "launch_ms_avg_over_timed_region": r["call_ms"],
        "launch_ms_p10_p50_p90_with_events": [float(np.percentile(r["step_ms"], p))
                                              for p in (10, 50, 90)],
        "host_enqueue_us_per_step": r["enqueue"] * 1e6 / args.steps,
        "separate_calls": r["separate"],
        "radix_topk": r["radix"],
        "append_kv": r["append"],
        "page_bounds": r["bounds"],
        "decode_layers": r["graph"],
        "dense": dense,
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
