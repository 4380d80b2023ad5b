"""A sequence of length 0 inside a batch, on every decode path: its units get
an empty selection (count 0, ids -1), output 0 and log-sum-exp -inf; the other
sequences match the oracle as usual (paged storage, so the page table of the
empty sequence is never followed).
"""

import numpy as np
import pytest
import torch

from oracle import seer_oracle as O
from tests.gpu_util import TOL, f64, unit_kv
from tests.test_gpu_learned_gate import check_learned_unit
from tests.test_gpu_multi_token import check_multi_unit
from tests.test_gpu_parity import SMALL, check_unit, state_for, units_of
from workloads import make_case, make_gate_weights

pytestmark = pytest.mark.gpu

EMPTY = 1  # the sequence given length 0


def zero_case(tokens=1):
    wl = SMALL["paged_small"].with_(query_tokens=tokens)
    case = make_case(wl, "cuda")
    case.lens[EMPTY] = 0
    torch.cuda.synchronize()
    return case


def check_empty(st, case):
    wl = case.wl
    for g in range(wl.num_kv_heads):
        u = EMPTY * wl.num_kv_heads + g
        assert int(st.sel_cnt[u]) == 0
        assert (st.sel_idx[u] == -1).all()
    assert (st.out[EMPTY] == 0).all()
    assert (st.lse[EMPTY] == -float("inf")).all()


@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_zero_length_one_token(mode):
    case = zero_case()
    print(f"[case] zero length, one token, {mode}", flush=True)
    st = state_for(case, fuse=True)
    st.build_pool(case.lens)
    (st.step if mode == "fused" else st.step_unfused)(case.q, case.lens)
    torch.cuda.synchronize()
    check_empty(st, case)
    lens = case.lens.tolist()
    for (b, g) in units_of(case.wl):
        if b != EMPTY:
            check_unit(st, case, case.q, lens, b, g, tag=f"zero-length {mode}")


@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_zero_length_tokens(mode):
    case = zero_case(tokens=2)
    print(f"[case] zero length, 2 tokens, {mode}", flush=True)
    st = state_for(case, query_tokens=2, fuse=True)
    st.build_pool(case.lens)
    (st.step if mode == "fused" else st.step_unfused)(case.q, case.lens)
    torch.cuda.synchronize()
    check_empty(st, case)
    for (b, g) in units_of(case.wl):
        if b != EMPTY:
            check_multi_unit(st, case, b, g, tag=f"zero-length tokens {mode}")


def test_zero_length_learned_gate():
    case = zero_case()
    print("[case] zero length, learned gate", flush=True)
    w = make_gate_weights(case.wl.num_kv_heads, case.wl.head_dim, seed=11)
    st = state_for(case, gate_weights=w.to("cuda"))
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    check_empty(st, case)
    for (b, g) in units_of(case.wl):
        if b != EMPTY:
            check_learned_unit(st, case, w, b, g, tag="zero-length learned")


def test_zero_length_dense():
    case = zero_case()
    st = state_for(case)
    st.build_pool(case.lens)
    st.attend(case.q, case.lens, dense=True)
    torch.cuda.synchronize()
    assert (st.out[EMPTY] == 0).all() and (st.lse[EMPTY] == -float("inf")).all()
    wl = case.wl
    S, G = wl.block_size, wl.group
    for (b, g) in units_of(wl):
        if b == EMPTY:
            continue
        L = int(case.lens[b])
        k, v = unit_kv(case, b, g, L)
        toks = O.selected_tokens(np.arange(O.block_count(L, S)), L, S)
        for h in range(G):
            o, _, _ = O.attend(f64(case.q[b, g * G + h]), k, v, toks)
            got = st.out[b, g * G + h].cpu().double().numpy()
            assert np.abs(got - o).max() <= TOL[wl.dtype]


def long_table_case():
    """Paged, 313-block tables (more than one 256-block score chunk), 40 units
    (at most one per attention workgroup): sequence 1 empty, sequence 2 of 79
    blocks, sequence 3 of 5 blocks, the others of 258..313 blocks."""
    from workloads import WORKLOADS
    wl = WORKLOADS["paged_var"].with_(batch=5, variable_context=(16500, 20000))
    case = make_case(wl, "cuda")
    case.lens[EMPTY] = 0
    case.lens[2] = 5000
    case.lens[3] = 300
    torch.cuda.synchronize()
    return case


def test_zero_and_short_lengths_long_table():
    """The score-kernel-then-select path with an empty sequence and sequences
    far shorter than the table: empty selections, out 0 and lse -inf for the
    empty one, the oracle for the others, and bitwise the separate calls."""
    from block_sparse_attention_29_amd import seer
    case = long_table_case()
    print("[case] zero and short lengths, 313-block paged tables", flush=True)
    st, sep = state_for(case), state_for(case)
    assert seer.gated_decode_path(st.shape, st.rule, st.k_max) == 2
    for s in (st, sep):
        s.build_pool(case.lens)
    st.step(case.q, case.lens)
    sep.step_unfused(case.q, case.lens)
    torch.cuda.synchronize()
    check_empty(st, case)
    lens = case.lens.tolist()
    for (b, g) in units_of(case.wl):
        if b != EMPTY:
            check_unit(st, case, case.q, lens, b, g, tag="long table")
    for attr in ("sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(st, attr), getattr(sep, attr)), attr
    U, NB = case.wl.batch * case.wl.num_kv_heads, case.wl.max_blocks
    for u in range(U):   # the scores of every unit's valid blocks
        n = O.block_count(lens[u // case.wl.num_kv_heads], case.wl.block_size)
        assert torch.equal(st.scores.view(U, NB)[u, :n], sep.scores.view(U, NB)[u, :n])


def test_zero_and_short_lengths_long_table_learned():
    """The learned gate's one-call step on the same batch (its gate splits
    each unit over several workgroups, so the attention kernel selects)."""
    case = long_table_case()
    print("[case] zero and short lengths, 313-block tables, learned gate", flush=True)
    w = make_gate_weights(case.wl.num_kv_heads, case.wl.head_dim, seed=13)
    st = state_for(case, gate_weights=w.to("cuda"))
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    check_empty(st, case)
    for (b, g) in units_of(case.wl):
        if b != EMPTY:
            check_learned_unit(st, case, w, b, g, tag="long table learned")
