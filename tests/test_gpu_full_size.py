"""GPU parity at the full sizes of the workloads, on every (sequence, KV head).

Bars as in test_gpu_parity: pooled keys and open sums bit-exact, scores within
1e-12 of the unit's largest, block ids and kept counts bit-exact, outputs and
log-sum-exps within max-abs 2e-3 (bf16 inputs) of the fp64 oracle -- here for
every unit of planted_8k, budget_32k, sparse90_32k, paged_var and spec4_32k,
for all 32 units of long_131k at 20 of its 256 decode steps, and for the dense
decode at the 32K shape on a slice of the batch.

Each test also prints the oracle's reporting extras over the units it
checked: the smallest boundary gap (s_k - s_k+1) / std(s), and how many
units' selections from the unrounded fp64 block means equal the stored-table
selections (reported, not gated).
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import seer_oracle as O
from tests.gpu_util import TOL, f64, oracle_unit
from tests.test_gpu_parity import check_unit, state_for
from tests.test_gpu_multi_token import check_multi_unit
from workloads import WORKLOADS, make_case

pytestmark = pytest.mark.gpu


class Snapshot:
    """The outputs of a decode state, copied to the host once."""

    def __init__(self, st):
        for a in ("pooled", "open_sum", "scores", "sel_idx", "sel_cnt", "out", "lse"):
            setattr(self, a, getattr(st, a).cpu())


def host_case(case):
    """The same inputs on the host (one copy each), for the oracle."""
    mv = lambda t: None if t is None else t.cpu()
    return dataclasses.replace(case, q=mv(case.q), k=mv(case.k), v=mv(case.v),
                               lens=mv(case.lens), page_table=mv(case.page_table),
                               top_k=mv(case.top_k), planted=mv(case.planted))


def report(name, gaps, pure_equal, n_units):
    print(f"[report] {name}: {n_units} units checked; smallest boundary gap "
          f"{min(gaps):.3g} std; pure-fp64 selection equal on {pure_equal}/{n_units}",
          flush=True)


def kept_count(wl, L):
    n = O.block_count(L, wl.block_size)
    return O.clamp_count(wl.top_k, n) if wl.top_k is not None else O.keep_count(n, *wl.keep)


@pytest.mark.parametrize("name", ["planted_8k", "budget_32k", "sparse90_32k", "paged_var"])
def test_full_size_every_unit(name):
    wl = WORKLOADS[name]
    print(f"[case] full size {name}, every unit", flush=True)
    case = make_case(wl, "cuda")
    st = state_for(case)
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    snap, hc = Snapshot(st), host_case(case)
    del st, case
    lens = hc.lens.tolist()
    gaps, pure = [], 0
    units = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    for (b, g) in units:
        ref = check_unit(snap, hc, hc.q, lens, b, g, tag=name)
        k = kept_count(wl, lens[b])
        gaps.append(O.boundary_gap(ref["scores"], k))
        qg = f64(hc.q[b, g * wl.group:(g + 1) * wl.group])
        pure += int(np.array_equal(O.pure_selection(qg, ref["pooled64"], wl.head_dim, k),
                                   ref["sel"]))
    if hc.planted is not None:
        sel = snap.sel_idx.numpy()
        pl = hc.planted.view(len(units), -1).numpy()
        for u in range(len(units)):
            assert set(pl[u].tolist()) <= set(sel[u].tolist()), f"planted blocks of unit {u}"
    report(name, gaps, pure, len(units))


def test_full_size_multi_token_every_unit():
    wl = WORKLOADS["spec4_32k"]
    print("[case] full size spec4_32k, every unit", flush=True)
    case = make_case(wl, "cuda")
    st = state_for(case, query_tokens=wl.query_tokens)
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    snap, hc = Snapshot(st), host_case(case)
    del st, case
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            check_multi_unit(snap, hc, b, g, tag="spec4_32k")


def test_dense_full_shape_slice():
    """Dense decode (every block kept) at the full 32K shape -- the speedup's
    denominator -- against the oracle's dense attention on the first, a middle
    and the last sequence, every KV head."""
    wl = WORKLOADS["sparse90_32k"]
    print("[case] dense decode at 16 x 32K, 3 sequences x 8 KV heads", flush=True)
    case = make_case(wl, "cuda")
    st = state_for(case)
    st.attend(case.q, case.lens, dense=True)
    torch.cuda.synchronize()
    snap, hc = Snapshot(st), host_case(case)
    del st, case
    G = wl.group
    for b in (0, wl.batch // 2, wl.batch - 1):
        L = int(hc.lens[b])
        for g in range(wl.num_kv_heads):
            ref = oracle_unit(hc, b, g, hc.q, L, dense=True)
            out = snap.out[b, g * G:(g + 1) * G].double().numpy()
            lse = snap.lse[b, g * G:(g + 1) * G].double().numpy()
            assert np.abs(out - ref["out"]).max() <= TOL[wl.dtype], f"dense out {b},{g}"
            assert np.abs(lse - ref["lse"]).max() <= TOL[wl.dtype], f"dense lse {b},{g}"


def test_long_decode_loop_every_unit():
    """256 decode steps at 131K context (pooling append, gate, sparse decode):
    all 32 units checked at 20 steps spread over the loop, including the steps
    that fill block 1024 and open block 1025; the oracle's pooled tables
    follow by its own incremental append (pinned equal to a rebuild)."""
    wl = WORKLOADS["long_131k"]
    print("[case] long decode loop, every unit at 20 steps", flush=True)
    case = make_case(wl, "cuda")
    st = state_for(case)
    S, d, G, Hkv = wl.block_size, wl.head_dim, wl.group, wl.num_kv_heads
    L0 = wl.context
    lens = torch.full((wl.batch,), L0, dtype=torch.int32, device="cuda")
    st.build_pool(lens)
    hc = host_case(case)
    units = [(b, g) for b in range(wl.batch) for g in range(Hkv)]
    # the oracle's state per unit: keys/values (fp32 holds bf16 exactly), pooled, open sum
    kv32, pool = {}, {}
    for (b, g) in units:
        k32 = hc.k[b, g].float().numpy()
        v32 = hc.v[b, g].float().numpy()
        kv32[(b, g)] = (k32, v32)
        p32, _, osum = O.pool_keys(k32[:L0].astype(np.float64), L0, S)
        pool[(b, g)] = (p32, osum, L0)
    check_steps = sorted(set(range(0, 256, 16)) | {1, 127, 128, 255})
    assert len(check_steps) >= 16
    gaps = []
    for i in range(wl.decode_steps):
        new = lens + 1
        q = case.q[i]
        st.step_append(q, lens, new)       # pooling append inside the gate's score launch
        lens = new
        if i not in check_steps:
            continue
        torch.cuda.synchronize()
        snap = Snapshot(st)
        L = L0 + i + 1
        qh = f64(q)
        for (b, g) in units:
            u = b * Hkv + g
            k32, v32 = kv32[(b, g)]
            p32, osum, Lp = pool[(b, g)]
            p32, osum = O.pool_keys_append(p32, osum, k32[:L].astype(np.float64), Lp, L, S)
            pool[(b, g)] = (p32, osum, L)
            n = O.block_count(L, S)
            got_p = snap.pooled.view(-1, d, wl.max_blocks)[u, :, :n].t().contiguous().numpy()
            assert np.array_equal(got_p.view(np.uint32), p32.view(np.uint32)), f"step{i} pooled {b},{g}"
            got_open = snap.open_sum.view(-1, d)[u].numpy()
            assert np.array_equal(got_open.view(np.uint64), osum.view(np.uint64)), f"step{i} open {b},{g}"
            qg = qh[b, g * G:(g + 1) * G]
            s = O.gate_scores(qg, p32, d)
            got_s = snap.scores.view(-1, wl.max_blocks)[u, :n].numpy()
            assert np.abs(got_s - s).max() <= 1e-12 * np.abs(s).max(), f"step{i} scores {b},{g}"
            k = O.keep_count(n, *wl.keep)
            sel = O.select_top_blocks(s, k)
            gaps.append(O.boundary_gap(s, k))
            cnt = int(snap.sel_cnt[u])
            ids = snap.sel_idx[u].numpy()
            assert cnt == k and np.array_equal(ids[:cnt], sel), f"step{i} ids {b},{g}"
            toks = O.selected_tokens(sel, L, S)
            kk, vv = k32[toks].astype(np.float64), v32[toks].astype(np.float64)
            rows = np.arange(len(toks))
            for h in range(G):
                o, lse, _ = O.attend(qg[h], kk, vv, rows)
                got_o = snap.out[b, g * G + h].double().numpy()
                assert np.abs(got_o - o).max() <= TOL[wl.dtype], f"step{i} out {b},{g},{h}"
                assert abs(float(snap.lse[b, g * G + h]) - lse) <= TOL[wl.dtype], f"step{i} lse"
        print(f"[step] {i}: {len(units)} units match", flush=True)
    print(f"[report] long_131k: {len(gaps)} unit-steps checked; smallest boundary gap "
          f"{min(gaps):.3g} std", flush=True)
    torch.cuda.synchronize()
    fresh = state_for(case)
    fresh.build_pool(lens)
    torch.cuda.synchronize()
    assert torch.equal(st.pooled, fresh.pooled)
    assert torch.equal(st.open_sum, fresh.open_sum)
