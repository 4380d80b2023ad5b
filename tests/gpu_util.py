"""Shared helpers of the GPU parity tests: run the oracle on chosen units.

Only test code uses this module.  It moves the seeded inputs (drawn by
``workloads``) to the host for the oracle; it never feeds the oracle anything
the GPU path computed.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import seer_oracle as O

TOL = {"bf16": 2e-3, "f32": 1e-5}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def unit_kv(case, b: int, g: int, n_tokens: int):
    """(T, d) float64 keys and values of unit (b, g) covering n_tokens tokens."""
    wl = case.wl
    S = wl.block_size
    n = O.block_count(n_tokens, S)
    if case.page_table is None:
        k = f64(case.k[b, g, : n * S])
        v = f64(case.v[b, g, : n * S])
        return k, v
    pages = case.page_table[b, :n].long()
    kp = f64(case.k[pages][:, g])          # (n, S, d)
    vp = f64(case.v[pages][:, g])
    table = np.arange(n)[None]
    k = O.gather_paged(kp[:, None], table, 0, n)[0]
    v = O.gather_paged(vp[:, None], table, 0, n)[0]
    return k, v


def oracle_unit(case, b: int, g: int, q: torch.Tensor, L: int, *, sel=None, dense=False,
                top_k=None, keep=None):
    """Pooling, scores, selection and attention of one unit, all in the oracle."""
    wl = case.wl
    S, G, d = wl.block_size, wl.group, wl.head_dim
    k, v = unit_kv(case, b, g, L)
    p32, p64, open_sum = O.pool_keys(k, L, S)
    qg = f64(q[b, g * G:(g + 1) * G])
    s = O.gate_scores(qg, p32, d)
    n = O.block_count(L, S)
    if dense:
        chosen = np.arange(n)
    elif sel is not None:
        chosen = np.sort(np.asarray(sel))
    else:
        if top_k is not None:
            kk = O.clamp_count(top_k, n)
        else:
            kk = O.keep_count(n, *keep)
        chosen = O.select_top_blocks(s, kk)
    toks = O.selected_tokens(chosen, L, S)
    outs, lses = [], []
    for h in range(G):
        o, l, _ = O.attend(qg[h], k, v, toks)
        outs.append(o)
        lses.append(l)
    return dict(pooled=p32, pooled64=p64, open_sum=open_sum, scores=s, sel=chosen,
                out=np.stack(outs), lse=np.array(lses))
