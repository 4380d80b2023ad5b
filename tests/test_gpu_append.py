"""The decode step with the pooling append folded in (seer_gated_sparse_decode_append).

Each case runs the same inputs twice: the one-call step (append + gate + decode)
and the reference sequence of separate calls (seer_block_pool_keys, then the
gate kernels, then the attention and combine), and requires every output --
pooled table, open sums, scores, ids, counts, out, lse -- to be bit-identical;
the reference sequence itself is held to the oracle by the other parity tests,
and a sampled unit of every case is checked against the oracle here as well.
"""

import numpy as np
import pytest
import torch

from block_sparse_attention_29_amd import seer
from oracle import seer_oracle as O
from tests.gpu_util import TOL, f64, unit_kv
from tests.test_gpu_parity import SMALL, state_for
from workloads import WORKLOADS, make_case

pytestmark = pytest.mark.gpu

OUTS = ("pooled", "open_sum", "scores", "sel_idx", "sel_cnt", "out", "lse")

CASES = {
    # 1026-block tables: the score kernel (with the append) over (unit,
    # 256-block chunk), the select kernel, then attention
    "long_1026": WORKLOADS["long_131k"].with_(batch=1, context=131072, decode_steps=256),
    # tables of at most 256 blocks, one unit per workgroup: the gate inside
    # the attention kernel, the append as its own launch
    "long_small": SMALL["long_small"].with_(decode_steps=300),
    # more units than workgroups: the one-launch gate kernel with the append,
    # then attention
    "paged": SMALL["paged_small"].with_(batch=48, variable_context=(1, 600)),
}


def run(case, lens_old, lens_new, q, *, rule=None, ref=False):
    st = state_for(case, **(rule or {}))
    st.build_pool(lens_old)
    if ref:
        st.append(lens_old, lens_new)
        st.step_unfused(q, lens_new)
    else:
        st.step_append(q, lens_old, lens_new)
    torch.cuda.synchronize()
    return st


def check_oracle_unit(st, case, q, lens_new, b, g):
    wl = case.wl
    S, d, G = wl.block_size, wl.head_dim, wl.group
    L = int(lens_new[b])
    k, v = unit_kv(case, b, g, L)
    p32 = O.pool_keys(k, L, S)[0]
    qg = f64(q[b, g * G:(g + 1) * G])
    s = O.gate_scores(qg, p32, d)
    n = O.block_count(L, S)
    kk = O.clamp_count(wl.top_k, n) if wl.top_k is not None else O.keep_count(n, *wl.keep)
    sel = O.select_top_blocks(s, kk)
    u = b * wl.num_kv_heads + g
    assert np.array_equal(st.sel_idx[u, :int(st.sel_cnt[u])].cpu().numpy(), sel)
    toks = O.selected_tokens(sel, L, S)
    for h in range(G):
        o, _, _ = O.attend(qg[h], k, v, toks)
        assert np.abs(st.out[b, g * G + h].cpu().double().numpy() - o).max() <= TOL[wl.dtype]


@pytest.mark.parametrize("step", [1, 5, 127, 300], ids=["1tok", "5tok", "127tok", "300tok"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_append_step_equals_separate_calls(name, step):
    """Appends of 1 token (the decode loop), a few, and many (crossing one or
    two block boundaries, so that the open block continues in one score
    workgroup and the last block is opened by the append) -- bit-identical to
    the separate append, gate and attention calls."""
    wl = CASES[name]
    print(f"[case] append step {name} +{step}", flush=True)
    case = make_case(wl, "cuda")
    q = case.q[0] if wl.decode_steps else case.q
    if wl.variable_context:
        lens_old = torch.clamp(case.lens - step, min=1)
        lens_new = case.lens
    else:
        lens_old = case.lens.clone()
        lens_new = case.lens + min(step, wl.decode_steps)
    a = run(case, lens_old, lens_new, q)
    r = run(case, lens_old, lens_new, q, ref=True)
    for attr in OUTS:
        assert torch.equal(getattr(a, attr), getattr(r, attr)), attr
    check_oracle_unit(a, case, q, lens_new.tolist(), 0, 0)
    check_oracle_unit(a, case, q, lens_new.tolist(), wl.batch - 1, wl.num_kv_heads - 1)


def test_append_with_a_unified_rule():
    """A rule the score kernels do not take (unified): the append runs as its
    own launch, with the same results."""
    wl = CASES["long_small"]
    case = make_case(wl, "cuda")
    q = case.q[0]
    lens_new = case.lens + 3
    a = run(case, case.lens, lens_new, q, rule=dict(unified=True))
    r = run(case, case.lens, lens_new, q, rule=dict(unified=True), ref=True)
    for attr in OUTS:
        assert torch.equal(getattr(a, attr), getattr(r, attr)), attr
