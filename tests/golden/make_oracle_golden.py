"""Writes oracle_small.json: the oracle's outputs on one small seeded
request.  It calls only the oracle (and numpy for the inputs).  The stored
file guards the oracle against silent drift; it is not an independent pin.

    python tests/golden/make_oracle_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle as orc  # noqa: E402


def inputs():
    rng = np.random.default_rng(20261203)
    H_q, H_kv, D, S, L = 4, 2, 8, 4, 23
    n_b = -(-L // S)
    k = orc.round_to(rng.standard_normal((n_b, H_kv, S, D)), "bf16")
    v = orc.round_to(rng.standard_normal((n_b, H_kv, S, D)), "bf16")
    q = orc.round_to(rng.standard_normal((H_q, D)), "bf16")
    return dict(q=q, k=k, v=v, seq_len=L, topk=2, n_bos=1, n_eos=1, sm_scale=0.125)


def compute(x):
    cent = orc.request_centroids(x["k"], x["seq_len"], "bf16")
    sel, o, lse = orc.sparse_decode_request(x["q"], x["k"], x["v"], cent, x["seq_len"],
                                            x["sm_scale"], x["topk"], x["n_bos"], x["n_eos"])
    od, lsed = orc.decode_request(x["q"], x["k"], x["v"], x["seq_len"], x["sm_scale"])
    return {"centroids": np.nan_to_num(cent, nan=0.0).tolist(),
            "selected": [s.tolist() for s in sel],
            "o": o.tolist(), "lse": lse.tolist(), "o_dense": od.tolist(),
            "lse_dense": lsed.tolist()}


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(compute(inputs()), f, indent=1)
