"""GPU parity of several new query tokens per sequence (seer_multi_gate_select,
seer_multi_sparse_decode) against the oracle.

Bars as for one token: block ids and kept counts bit-exact, scores within
1e-12 of the unit's largest, outputs and log-sum-exps within the dtype's
tolerance; a token that sees no key gets 0 and -inf exactly.
"""

import numpy as np
import pytest
import torch

from oracle import seer_oracle as O
from tests.gpu_util import TOL, f64, unit_kv
from tests.test_gpu_parity import SMALL, state_for, units_of
from workloads import WORKLOADS, make_case

pytestmark = pytest.mark.gpu

CASES = {
    "planted_b2_t4": SMALL["planted_b2"].with_(query_tokens=4),            # G4: 16 rows
    "bf16_d64_g8_t2": SMALL["bf16_d64_g8"].with_(query_tokens=2),         # G8: 16 rows
    "tiny_f32_t3": SMALL["tiny_1k"].with_(query_tokens=3),                # fp32 d64: 12 rows
    "f32_d128_g1_t5": SMALL["f32_d128_s128_g1"].with_(query_tokens=5),    # fp32 d128: 5 rows
    "paged_g5_t2": SMALL["paged_small"].with_(query_tokens=2),            # paged, G5: 10 rows
    "g3_keep_t5": SMALL["bf16_g3_keep"].with_(query_tokens=5),            # G3: 15 rows
}


def run_multi(case, dense=False, **kw):
    wl = case.wl
    st = state_for(case, query_tokens=wl.query_tokens, **kw)
    st.build_pool(case.lens)
    if dense:
        st.attend(case.q, case.lens, dense=True)
    else:
        st.step(case.q, case.lens)
    torch.cuda.synchronize()
    return st


def check_multi_unit(st, case, b, g, *, dense=False, sel=None, tag=""):
    wl = case.wl
    S, d, G, T = wl.block_size, wl.head_dim, wl.group, wl.query_tokens
    L = int(case.lens[b])
    n = O.block_count(L, S)
    k, v = unit_kv(case, b, g, L)
    qt = f64(case.q[b, :, g * G:(g + 1) * G])                       # (T, G, d)
    u = b * wl.num_kv_heads + g
    if dense:
        chosen = np.arange(n)
    elif sel is not None:
        chosen = np.asarray(sel)
    else:
        p32 = O.pool_keys(k, L, S)[0]
        s = O.gate_scores_tokens(qt, p32, d)
        kk = O.clamp_count(wl.top_k, n) if wl.top_k is not None else O.keep_count(n, *wl.keep)
        chosen = O.select_top_blocks(s, kk)
        got_s = st.scores.view(-1, wl.max_blocks)[u, :n].cpu().numpy()
        assert np.abs(got_s - s).max() <= 1e-12 * max(np.abs(s).max(), 1e-300), f"{tag} scores {b},{g}"
        cnt = int(st.sel_cnt[u])
        ids = st.sel_idx[u].cpu().numpy()
        assert cnt == len(chosen) and np.array_equal(ids[:cnt], chosen), f"{tag} ids {b},{g}"
    out, lse = O.attend_tokens(qt, k, v, chosen, L, S)
    got_o = st.out[b, :, g * G:(g + 1) * G].cpu().double().numpy()
    got_l = st.lse[b, :, g * G:(g + 1) * G].cpu().double().numpy()
    tol = TOL[wl.dtype]
    assert np.abs(got_o - out).max() <= tol, f"{tag} out {b},{g}: {np.abs(got_o - out).max()}"
    fin = np.isfinite(lse)
    assert np.array_equal(np.isfinite(got_l), fin), f"{tag} lse finiteness {b},{g}"
    assert np.abs(got_l[fin] - lse[fin]).max(initial=0.0) <= tol, f"{tag} lse {b},{g}"
    assert np.all(got_l[~fin] == -np.inf) and np.all(got_o[~fin] == 0.0)


@pytest.mark.parametrize("name", sorted(CASES))
def test_multi_token_small(name):
    wl = CASES[name]
    print(f"[case] multi-token {name}", flush=True)
    case = make_case(wl, "cuda")
    st = run_multi(case)
    for (b, g) in units_of(wl):
        check_multi_unit(st, case, b, g, tag=name)


@pytest.mark.parametrize("name", ["planted_b2_t4", "tiny_f32_t3", "paged_g5_t2"])
def test_multi_token_dense(name):
    wl = CASES[name]
    case = make_case(wl, "cuda")
    st = run_multi(case, dense=True)
    for (b, g) in units_of(wl):
        check_multi_unit(st, case, b, g, dense=True, tag=name + " dense")


@pytest.mark.parametrize("name", ["paged_g5_t2", "planted_b2_t4"])
def test_multi_token_nan_poison(name):
    """Unused cache slots hold NaN: never read into a result."""
    wl = CASES[name]
    case = make_case(wl, "cuda", poison=True)
    st = run_multi(case)
    assert torch.isfinite(st.out).all()
    for (b, g) in units_of(wl, limit=3):
        check_multi_unit(st, case, b, g, tag=name + " poison")


def test_multi_token_causal_edge():
    """Kept block = the last one only; the first tokens sit before it and see
    nothing (0, -inf), the later ones see 1 and 2 keys."""
    wl = SMALL["tiny_1k"].with_(context=5 * 64 + 2, query_tokens=4, top_k=1)
    case = make_case(wl, "cuda")
    st = state_for(case, query_tokens=4)
    sel = torch.tensor([[5]], dtype=torch.int32, device="cuda")
    cnt = torch.tensor([1], dtype=torch.int32, device="cuda")
    st.attend(case.q, case.lens, sel_idx=sel, sel_cnt=cnt, k_max=1)
    torch.cuda.synchronize()
    check_multi_unit(st, case, 0, 0, sel=[5], tag="causal edge")
    assert torch.all(st.lse[0, :2] == -float("inf")) and torch.all(st.out[0, :2] == 0)
    assert torch.all(torch.isfinite(st.lse[0, 2:]))


def test_multi_token_two_stages():
    """seer_multi_sparse_decode_partial then _combine on one workspace gives
    the bits of seer_multi_sparse_decode."""
    from block_sparse_attention_29_amd import seer
    wl = CASES["planted_b2_t4"]
    case = make_case(wl, "cuda")
    st = run_multi(case)
    T = wl.query_tokens
    out = torch.full_like(st.out, float("nan"))
    lse = torch.full_like(st.lse, float("nan"))
    seer.multi_sparse_decode_partial(st.shape, T, case.q, st.kv, case.lens, st.sel_idx,
                                     st.sel_cnt, st.k_max, st.workspace)
    seer.multi_sparse_decode_combine(st.shape, T, out, lse, st.workspace)
    torch.cuda.synchronize()
    assert torch.equal(out, st.out) and torch.equal(lse, st.lse)


def test_query_shape_checked():
    """The binding refuses a query whose element count is not [B][T][Hq][d]."""
    from block_sparse_attention_29_amd import seer
    wl = CASES["planted_b2_t4"]
    case = make_case(wl, "cuda")
    st = run_multi(case)
    one = state_for(case)                   # one query token per sequence
    with pytest.raises(ValueError):
        seer.gate_select(one.shape, case.q, st.pooled, case.lens, one.rule, one.k_max,
                         one.scores, one.sel_idx, one.sel_cnt)
    with pytest.raises(ValueError):
        seer.multi_sparse_decode_partial(st.shape, 2, case.q, st.kv, case.lens, st.sel_idx,
                                         st.sel_cnt, st.k_max, st.workspace)


@pytest.mark.parametrize("name", sorted(CASES) + ["spec4_32k"])
def test_multi_gated_equals_separate_calls_bitwise(name):
    """The multi-token step with the gate fused into the attention kernel
    writes exactly what the gate call followed by the attention calls writes
    (scores, ids, counts, out, lse); the fused kernel is forced."""
    wl = CASES[name] if name in CASES else WORKLOADS[name].with_(batch=2)
    print(f"[case] multi gated vs separate {name}", flush=True)
    case = make_case(wl, "cuda")
    fused = state_for(case, query_tokens=wl.query_tokens, fuse=True)
    sep = state_for(case, query_tokens=wl.query_tokens)
    for st in (fused, sep):
        st.build_pool(case.lens)
    fused.step(case.q, case.lens)
    sep.step_unfused(case.q, case.lens)
    torch.cuda.synchronize()
    for attr in ("scores", "sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(fused, attr), getattr(sep, attr)), attr


@pytest.mark.parametrize("rule", [dict(force_first=True), dict(force_first=True, force_last=True)],
                         ids=["first", "both"])
def test_multi_gated_forced_blocks(rule):
    """Forced blocks in the fused multi-token gate: bitwise the separate calls,
    and the oracle's selection."""
    wl = CASES["paged_g5_t2"]
    case = make_case(wl, "cuda")
    fused = state_for(case, query_tokens=wl.query_tokens, fuse=True, **rule)
    sep = state_for(case, query_tokens=wl.query_tokens, **rule)
    for st in (fused, sep):
        st.build_pool(case.lens)
    fused.step(case.q, case.lens)
    sep.step_unfused(case.q, case.lens)
    torch.cuda.synchronize()
    for attr in ("scores", "sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(fused, attr), getattr(sep, attr)), attr


def test_multi_fusion_policy():
    """Several tokens follow the single-token rule: fused at 4 tokens of
    sparse90_32k's shape, not with more units than workgroups."""
    from block_sparse_attention_29_amd import seer
    from tests.test_gpu_parity import DT
    for name, want in [("spec4_32k", True), ("paged_var", False)]:
        wl = WORKLOADS[name]
        T = 4 if name == "spec4_32k" else 2
        shape = seer.make_shape(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                wl.block_size, wl.max_blocks, DT[wl.dtype])
        k_max = seer.keep_blocks(wl.max_blocks, *wl.keep)
        rule = seer.make_select(keep=wl.keep)
        assert seer.gated_decode_is_fused(shape, rule, k_max, T) == want, name
