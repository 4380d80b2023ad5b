"""GPU parity of the learned gate (seer_learned_gate_select) against the oracle.

The oracle evaluates the gate network in fp64 on the stored fp32 pooled keys.
The kernel runs the first layer on int8 MFMA over a five-limb image of each
block's keys (block exponent e_j: the smallest integer with
127 * 2^e_j >= max_i |P_ji|), which holds every key to within 2^(e_j - 29);
so its scores carry a stated error bound

    |s_gpu_j - s_j| <= 2^(e_j - 29) * sum_m |u_m| beta_m ||W1_m||_1
                       + 1e-12 * (rounding scale of the fp64 steps),

u = Wq qbar.  Bars: scores within that bound; block ids and counts bit-exact
wherever the oracle's selection margin (the smallest change of a score that
could change the selection) exceeds twice the largest bound of the unit;
below that the kernel's ids must be the selection its own in-bound scores
make.  Outputs of the decode that follows within the dtype's tolerance of the
oracle's attention over the kernel's selection.  The weights are seeded and
untrained.
"""

import zlib

import numpy as np
import pytest
import torch

from block_sparse_attention_29_amd.pipeline import DecodeState
from oracle import seer_oracle as O
from tests.gpu_util import TOL, f64, unit_kv
from tests.test_gpu_parity import SMALL, state_for, units_of
from workloads import WORKLOADS, make_case, make_gate_weights

pytestmark = pytest.mark.gpu

LIMB_BITS = 29   # 2^(e - 29): the five-limb image's resolution relative to 2^e


def run_learned(case, seed=7, q=None, **rule):
    wl = case.wl
    w = make_gate_weights(wl.num_kv_heads, wl.head_dim, seed=seed)
    st = state_for(case, gate_weights=w.to("cuda"), **rule)
    st.build_pool(case.lens)
    st.step(case.q if q is None else q, case.lens)
    torch.cuda.synchronize()
    return st, w


def block_exponents(p32):
    """e_j: the smallest integer with 127 * 2^e_j >= max_i |P_ji| (0 for a zero block)."""
    amax = np.abs(p32.astype(np.float64)).max(axis=1)
    e = np.zeros(len(amax), dtype=np.int64)
    nz = amax > 0
    e[nz] = np.ceil(np.log2(amax[nz] / 127.0)).astype(np.int64)
    # guard the log against rounding: step to the smallest exponent that fits
    e[nz] -= (127.0 * np.ldexp(1.0, e[nz] - 1) >= amax[nz]).astype(np.int64)
    e[nz] += (127.0 * np.ldexp(1.0, e[nz]) < amax[nz]).astype(np.int64)
    return e


def score_bound(qg, p32, w, g):
    """Per-block bound on |s_gpu - s_oracle| (module docstring)."""
    w1 = w.w1[g].numpy().astype(np.float64)
    beta = w.w1_scale[g].numpy().astype(np.float64)
    b1 = w.b1[g].numpy().astype(np.float64)
    u = w.wq[g].numpy().astype(np.float64) @ qg.sum(axis=0)
    l1 = np.abs(w1).sum(axis=1)
    lim = np.ldexp(1.0, block_exponents(p32) - LIMB_BITS) * float(np.sum(np.abs(u) * beta * l1))
    amax = np.abs(p32.astype(np.float64)).max(axis=1)
    rnd = 1e-12 * (np.abs(u) * (beta * l1 * amax[:, None] + np.abs(b1))).sum(axis=1)
    return lim + rnd


def selection_margin(s, rule, kk, k_max):
    """The smallest change of one score that could change the oracle's
    selection under the rule (inf when nothing can)."""
    n = len(s)
    forced = set()
    if rule.get("force_first"):
        forced.add(0)
    if rule.get("force_last"):
        forced.add(n - 1)
    rest = np.array(sorted(set(range(n)) - forced), dtype=np.int64)
    if len(rest) == 0:
        return float("inf")
    rs = np.sort(s[rest])[::-1]
    cap = min(n, k_max)
    margin = float("inf")
    if "threshold" in rule:
        margin = float(np.min(np.abs(rs - rule["threshold"])))
        above = int(np.sum(rs > rule["threshold"]))
        count = min(max(1, len(forced) + above), cap)
    else:
        count = max(1, min(max(kk, len(forced)), cap))
    kr = count - min(count, len(forced))
    if 0 < kr < len(rs):
        margin = min(margin, float(rs[kr - 1] - rs[kr]))
    if kr == 0 and "threshold" in rule and len(forced) == 0:
        margin = min(margin, float(rs[0] - rs[1]) if len(rs) > 1 else margin)
    return margin


def oracle_select(s, rule, kk, k_max):
    if "threshold" in rule:
        return O.select_blocks(s, threshold=rule["threshold"],
                               force_first=rule.get("force_first", False),
                               force_last=rule.get("force_last", False), k_max=k_max)
    return O.select_blocks(s, k=kk, force_first=rule.get("force_first", False),
                           force_last=rule.get("force_last", False), k_max=k_max)


MARGINS = []   # (margin / bound) of every checked unit, for the report


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
    bound = score_bound(qg, p32, w, g)
    kk = O.clamp_count(wl.top_k, n) if wl.top_k is not None else O.keep_count(n, *wl.keep)
    sel = oracle_select(s, rule, kk, st.k_max)
    u = b * wl.num_kv_heads + g
    got_s = st.scores.view(-1, wl.max_blocks)[u, :n].cpu().numpy()
    err = np.abs(got_s - s)
    assert np.all(err <= bound), f"{tag} scores {b},{g}: worst {(err / bound).max():.3g} x bound"
    cnt = int(st.sel_cnt[u])
    ids = st.sel_idx[u].cpu().numpy()
    margin = selection_margin(s, rule, kk, st.k_max)
    if bound.max() > 0:   # a zero query scores every block 0 with a zero bound
        MARGINS.append(margin / bound.max())
    if margin > 2.0 * bound.max():
        assert cnt == len(sel), f"{tag} count {b},{g}: {cnt} vs {len(sel)}"
        assert np.array_equal(ids[:cnt], sel), f"{tag} ids {b},{g}"
    else:
        own = oracle_select(got_s, rule, kk, st.k_max)
        print(f"[near tie] {tag} unit {b},{g}: margin {margin:.3g}, bound {bound.max():.3g}",
              flush=True)
        assert cnt == len(own) and np.array_equal(ids[:cnt], own), f"{tag} own ids {b},{g}"
        sel = own
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
    """All-zero keys give every block the same score (every limb 0): the
    lowest ids win.  A zero query gives u = 0 and all-zero scores."""
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


def test_learned_gate_fine_key_bits_decide():
    """fp32 keys, one unit: the best block is copied twice with 2^-18 added to
    and taken from dimension 0 of every key.  The three blocks' scores differ
    by far less than a 7-bit image of the keys resolves but by far more than
    the kernel's bound, so the top-2 among them must come out exactly as the
    oracle's."""
    wl = WORKLOADS["tiny_1k"].with_(head_dim=128, context=2048, top_k=2)
    case = make_case(wl, "cuda")
    S, L = wl.block_size, wl.context
    w = make_gate_weights(1, wl.head_dim, seed=11)
    k = f64(case.k[0, 0, :L])
    s = O.learned_gate_scores(f64(case.q[0]), O.pool_keys(k, L, S)[0], w.w1[0].numpy(),
                              w.w1_scale[0].numpy(), w.b1[0].numpy(), w.wq[0].numpy())
    top = int(np.argmax(s))
    dsts = [j for j in range(O.block_count(L, S)) if j != top][:2]
    for dst, sign in zip(dsts, (1.0, -1.0)):
        case.k[0, 0, dst * S:(dst + 1) * S] = case.k[0, 0, top * S:(top + 1) * S]
        case.k[0, 0, dst * S:(dst + 1) * S, 0] += sign * 2.0 ** -18
    st, _ = run_learned(case, seed=11)
    s2, sel = check_learned_unit(st, case, w, 0, 0, tag="fine bits")
    lead = sorted([top, *dsts], key=lambda j: -s2[j])
    assert abs(s2[lead[0]] - s2[lead[2]]) < 1e-4 * abs(s2[top])      # three near-equal blocks
    assert sel.tolist() == sorted(lead[:2])


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
    """Every unit of the full-size workloads."""
    wl = WORKLOADS[name]
    print(f"[case] learned gate full size {name}", flush=True)
    case = make_case(wl, "cuda")
    st, w = run_learned(case)
    MARGINS.clear()
    for (b, g) in units_of(wl):
        check_learned_unit(st, case, w, b, g, tag=name)
    print(f"[report] {name}: smallest selection margin / score bound over "
          f"{len(MARGINS)} units = {min(MARGINS, default=float('inf')):.3g}", flush=True)


def test_learned_gate_split_equals_one_launch():
    """With fewer units than CUs a unit's chunks are scored by several
    workgroups and selected by a second launch; with as many units as CUs by
    one workgroup in one launch.  The same sequences gated both ways (a batch
    of 32, 256 units, and its first 8 sequences, 64 units) give bit-identical
    scores, ids and counts."""
    wl = WORKLOADS["planted_8k"].with_(batch=32)
    print("[case] learned gate split vs one launch, planted_8k shape, 32 and 8 sequences",
          flush=True)
    case = make_case(wl, "cuda")
    w = make_gate_weights(wl.num_kv_heads, wl.head_dim, seed=7).to("cuda")
    full = state_for(case, gate_weights=w)
    full.build_pool(case.lens)
    full.select(case.q, case.lens)
    part_b = 8
    part = DecodeState(batch=part_b, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                       head_dim=wl.head_dim, block_size=wl.block_size, max_blocks=wl.max_blocks,
                       dtype=torch.bfloat16, k=case.k[:part_b], v=case.v[:part_b], keep=wl.keep,
                       gate_weights=w)
    lens = case.lens[:part_b].contiguous()
    part.build_pool(lens)
    part.select(case.q[:part_b].contiguous(), lens)
    torch.cuda.synchronize()
    U = part_b * wl.num_kv_heads
    NB = wl.max_blocks
    s_full = full.scores.view(-1, NB)[:U].cpu()
    s_part = part.scores.view(-1, NB).cpu()
    n = (wl.context + wl.block_size - 1) // wl.block_size
    assert torch.equal(s_full[:, :n].view(torch.int64), s_part[:, :n].view(torch.int64))
    assert torch.equal(full.sel_cnt[:U].cpu(), part.sel_cnt.cpu())
    assert torch.equal(full.sel_idx.view(-1, full.k_max)[:U].cpu(),
                       part.sel_idx.view(-1, part.k_max).cpu())


@pytest.mark.parametrize("rule", [dict(), dict(force_first=True, force_last=True),
                                  dict(threshold=0.0)], ids=["topk", "forced", "threshold"])
@pytest.mark.parametrize("name", ["planted_8k", "sparse90_32k"])
def test_learned_step_equals_separate_calls(name, rule):
    """The learned gate's one-call step (its score launch, then the attention
    kernel selecting from those scores where the gate splits units over
    workgroups) writes exactly what the gate call followed by the attention
    call writes: scores, ids, counts, out, lse."""
    wl = WORKLOADS[name].with_(batch=4)
    print(f"[case] learned step vs separate calls, {name}, {rule}", flush=True)
    case = make_case(wl, "cuda")
    w = make_gate_weights(wl.num_kv_heads, wl.head_dim, seed=5).to("cuda")
    one, sep = state_for(case, gate_weights=w, **rule), state_for(case, gate_weights=w, **rule)
    for st in (one, sep):
        st.build_pool(case.lens)
    one.step(case.q, case.lens)
    sep.step_unfused(case.q, case.lens)
    torch.cuda.synchronize()
    for attr in ("scores", "sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(one, attr), getattr(sep, attr)), attr
