"""GPU parity of the learned gate (seer_learned_gate_select) against the oracle.

Bars as for the parameter-free gate: block ids and kept counts bit-exact,
scores within 1e-12 of the unit's largest score, outputs of the decode that
follows within the dtype's tolerance.  The weights are seeded and untrained.
"""

import zlib

import numpy as np
import pytest
import torch

from oracle import seer_oracle as O
from tests.gpu_util import TOL, f64, unit_kv
from tests.test_gpu_parity import SMALL, state_for, units_of
from workloads import WORKLOADS, make_case, make_gate_weights

pytestmark = pytest.mark.gpu


def run_learned(case, seed=7, q=None, **rule):
    wl = case.wl
    w = make_gate_weights(wl.num_kv_heads, wl.head_dim, seed=seed)
    st = state_for(case, gate_weights=w.to("cuda"), **rule)
    st.build_pool(case.lens)
    st.step(case.q if q is None else q, case.lens)
    torch.cuda.synchronize()
    return st, w


def check_learned_unit(st, case, w, b, g, *, q=None, rule=None, tag=""):
    wl = case.wl
    rule = rule or {}
    S, d, G = wl.block_size, wl.head_dim, wl.group
    L = int(case.lens[b])
    n = O.block_count(L, S)
    k, v = unit_kv(case, b, g, L)
    p32 = O.pool_keys(k, L, S)[0]
    qq = case.q if q is None else q
    qg = f64(qq[b, g * G:(g + 1) * G])
    s = O.learned_gate_scores(qg, p32, w.w1[g].numpy(), w.w1_scale[g].numpy(),
                              w.b1[g].numpy(), w.wq[g].numpy())
    if "threshold" in rule:
        sel = O.select_blocks(s, threshold=rule["threshold"],
                              force_first=rule.get("force_first", False),
                              force_last=rule.get("force_last", False), k_max=st.k_max)
    else:
        kk = O.clamp_count(wl.top_k, n) if wl.top_k is not None else O.keep_count(n, *wl.keep)
        sel = O.select_blocks(s, k=kk, force_first=rule.get("force_first", False),
                              force_last=rule.get("force_last", False), k_max=st.k_max)
    u = b * wl.num_kv_heads + g
    got_s = st.scores.view(-1, wl.max_blocks)[u, :n].cpu().numpy()
    assert np.abs(got_s - s).max() <= 1e-12 * max(np.abs(s).max(), 1e-300), f"{tag} scores {b},{g}"
    cnt = int(st.sel_cnt[u])
    ids = st.sel_idx[u].cpu().numpy()
    assert cnt == len(sel), f"{tag} count {b},{g}: {cnt} vs {len(sel)}"
    assert np.array_equal(ids[:cnt], sel), f"{tag} ids {b},{g}"
    assert (ids[cnt:] == -1).all()
    toks = O.selected_tokens(sel, L, S)
    out = st.out[b, g * G:(g + 1) * G].cpu().double().numpy()
    for h in range(G):
        o, _, _ = O.attend(qg[h], k, v, toks)
        assert np.abs(out[h] - o).max() <= TOL[wl.dtype], f"{tag} out {b},{g},{h}"
    return s, sel


@pytest.mark.parametrize("name", sorted(SMALL))
def test_learned_gate_small(name):
    wl = SMALL[name]
    print(f"[case] learned gate {name}", flush=True)
    case = make_case(wl, "cuda")
    st, w = run_learned(case, seed=zlib.crc32(name.encode()) % 1000)
    for (b, g) in units_of(wl):
        check_learned_unit(st, case, w, b, g, tag=name)


@pytest.mark.parametrize("rule", [dict(threshold=0.0), dict(threshold=0.0, force_first=True),
                                  dict(force_first=True, force_last=True)],
                         ids=["threshold_0", "threshold_forced", "forced"])
@pytest.mark.parametrize("name", ["planted_b2", "paged_small"])
def test_learned_gate_rules(name, rule):
    wl = SMALL[name]
    print(f"[case] learned gate {name} {rule}", flush=True)
    case = make_case(wl, "cuda")
    st, w = run_learned(case, **rule)
    for (b, g) in units_of(wl):
        check_learned_unit(st, case, w, b, g, rule=rule, tag=name)


def test_learned_gate_ties_and_zero_query():
    """All-zero keys give every block the same score (alpha = 1, int8 image 0):
    the lowest ids win.  A zero query gives u = 0 and all-zero scores."""
    wl = SMALL["planted_b2"]
    case = make_case(wl, "cuda")
    case.k.zero_()
    st, w = run_learned(case)
    for (b, g) in units_of(wl):
        s, sel = check_learned_unit(st, case, w, b, g, tag="zero keys")
        assert np.all(s == s[0]) and sel.tolist() == list(range(len(sel)))
    case = make_case(wl, "cuda")
    q0 = torch.zeros_like(case.q)
    st, w = run_learned(case, q=q0)
    for (b, g) in units_of(wl):
        s, sel = check_learned_unit(st, case, w, b, g, q=q0, tag="zero query")
        assert np.all(s == 0.0) and sel.tolist() == list(range(len(sel)))


def test_learned_gate_wide_table():
    """8192 blocks per sequence: the largest table the library takes."""
    wl = WORKLOADS["tiny_1k"].with_(dtype="bf16", head_dim=128, num_q_heads=4, num_kv_heads=1,
                                    block_size=64, context=8192 * 64 - 37,
                                    top_k=40)
    print("[case] learned gate, 8192 blocks", flush=True)
    case = make_case(wl, "cuda")
    st, w = run_learned(case)
    check_learned_unit(st, case, w, 0, 0, tag="wide")


@pytest.mark.parametrize("name", ["budget_32k", "sparse90_32k"])
def test_learned_gate_full_size(name):
    wl = WORKLOADS[name]
    print(f"[case] learned gate full size {name}", flush=True)
    case = make_case(wl, "cuda")
    st, w = run_learned(case)
    for (b, g) in units_of(wl, limit=6, seed=3):
        check_learned_unit(st, case, w, b, g, tag=name)
