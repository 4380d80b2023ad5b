"""GPU parity of the libseer kernels against the fp64 oracle (run on an MI355X).

Bars: pooled keys, open sums, block ids and kept counts are bit-exact; gate
scores agree to 1e-12 of the unit's largest score; outputs and log-sum-exps
agree to max-abs 2e-3 for bf16 inputs and 1e-5 for fp32 inputs.
"""

import numpy as np
import pytest
import torch

from block_sparse_attention_29_amd import seer
from block_sparse_attention_29_amd.pipeline import DecodeState
from oracle import seer_oracle as O
from tests.gpu_util import TOL, f64, oracle_unit, unit_kv
from workloads import WORKLOADS, make_case

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def state_for(case, **kw):
    wl = case.wl
    return DecodeState(batch=wl.batch, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                       head_dim=wl.head_dim, block_size=wl.block_size, max_blocks=wl.max_blocks,
                       dtype=DT[wl.dtype], k=case.k, v=case.v, page_table=case.page_table,
                       keep=wl.keep, top_k=case.top_k, **kw)


def gpu_pooled(st, wl, b, g, n):
    D, NB = wl.head_dim, wl.max_blocks
    u = b * wl.num_kv_heads + g
    t = st.pooled.view(-1, D, NB)[u, :, :n]
    return t.t().contiguous().cpu().numpy()


def units_of(wl, limit=None, seed=0):
    all_u = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    if limit is None or limit >= len(all_u):
        return all_u
    rng = np.random.default_rng(seed)
    idx = sorted(rng.choice(len(all_u), size=limit, replace=False).tolist())
    # always include the first and the last unit
    return sorted(set([all_u[0], all_u[-1]] + [all_u[i] for i in idx]))


def check_unit(st, case, q, lens_host, b, g, *, sel_only=False, tag=""):
    wl = case.wl
    L = int(lens_host[b])
    n = O.block_count(L, wl.block_size)
    ref = oracle_unit(case, b, g, q, L, keep=wl.keep, top_k=wl.top_k)
    u = b * wl.num_kv_heads + g
    # pooled keys: bit-exact
    got_p = gpu_pooled(st, wl, b, g, n)
    assert np.array_equal(got_p.view(np.uint32), ref["pooled"].view(np.uint32)), f"{tag} pooled {b},{g}"
    # scores
    got_s = st.scores.view(-1, wl.max_blocks)[u, :n].cpu().numpy()
    scale = max(np.abs(ref["scores"]).max(), 1e-300)
    assert np.abs(got_s - ref["scores"]).max() <= 1e-12 * scale, f"{tag} scores {b},{g}"
    # selection: bit-exact ids and count
    cnt = int(st.sel_cnt[u])
    ids = st.sel_idx[u].cpu().numpy()
    assert cnt == len(ref["sel"]), f"{tag} count {b},{g}: {cnt} vs {len(ref['sel'])}"
    assert np.array_equal(ids[:cnt], ref["sel"]), f"{tag} ids {b},{g}"
    assert (ids[cnt:] == -1).all()
    if sel_only:
        return ref
    G = wl.group
    out = st.out[b, g * G:(g + 1) * G].cpu().double().numpy()
    lse = st.lse[b, g * G:(g + 1) * G].cpu().double().numpy()
    tol = TOL[wl.dtype]
    assert np.abs(out - ref["out"]).max() <= tol, f"{tag} out {b},{g}: {np.abs(out - ref['out']).max()}"
    assert np.abs(lse - ref["lse"]).max() <= tol, f"{tag} lse {b},{g}"
    return ref


# ------------------------------------------------------------------ small configs

SMALL = {
    "tiny_1k": WORKLOADS["tiny_1k"],
    "planted_b2": WORKLOADS["planted_8k"].with_(batch=2),
    "paged_small": WORKLOADS["paged_var"].with_(batch=5, variable_context=(1, 700)),
    "long_small": WORKLOADS["long_131k"].with_(batch=2, context=3000, decode_steps=0),
    "f32_d128_s128_g1": WORKLOADS["tiny_1k"].with_(num_q_heads=2, num_kv_heads=2, head_dim=128,
                                                  block_size=128, context=1300, top_k=3),
    "bf16_d64_g8": WORKLOADS["tiny_1k"].with_(dtype="bf16", num_q_heads=16, num_kv_heads=2,
                                              context=777, top_k=5),
    "bf16_g3_keep": WORKLOADS["planted_8k"].with_(batch=3, num_q_heads=6, num_kv_heads=2,
                                                 context=641, planted_fraction=None,
                                                 keep=(3, 10)),
    "f32_g5_paged": WORKLOADS["paged_var"].with_(dtype="f32", batch=3, num_q_heads=10,
                                                num_kv_heads=2, variable_context=(60, 400)),
}


COMBINE = {"unit": seer.SEER_COMBINE_PER_UNIT, "head": seer.SEER_COMBINE_PER_HEAD}


@pytest.mark.parametrize("combine", sorted(COMBINE))
@pytest.mark.parametrize("name", sorted(SMALL))
def test_full_chain_small(name, combine):
    """The whole step against the oracle, with the combine run per unit and
    per query head on every shape."""
    wl = SMALL[name]
    print(f"[case] full chain {name} combine per {combine}", flush=True)
    case = make_case(wl, "cuda")
    st = state_for(case, combine=COMBINE[combine])
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    lens = case.lens.tolist()
    for (b, g) in units_of(wl):
        check_unit(st, case, case.q, lens, b, g, tag=name)


FEW_UNITS = {
    # one 32K sequence on 8 KV heads, 4K budget: 1024 tiles on 1024 waves, so
    # every unit merges ~128 one-tile records (per head: two chunks of 64)
    "budget_b1": WORKLOADS["budget_32k"].with_(batch=1),
    # one 8K sequence at 90% sparsity: fewer tiles than waves, so empty waves
    # sit between the records of a unit
    "planted_b1": WORKLOADS["planted_8k"].with_(batch=1),
}


COMBINE_CASES = sorted(SMALL) + ["budget_b1", "planted_b1", "budget_b2"]


@pytest.mark.parametrize("name", COMBINE_CASES)
def test_combine_modes_bitwise(name):
    """The merge per unit and per query head run the same fp32 operations in
    the same record order, so on one set of partial records they give the
    same bits: shapes with few records per unit (one-shot merges), and with
    ~64 and ~128 records per unit (two-pass merges), some with empty waves
    between a unit's records."""
    wl = SMALL.get(name) or FEW_UNITS.get(name) or WORKLOADS["budget_32k"].with_(batch=2)
    print(f"[case] combine modes {name}", flush=True)
    case = make_case(wl, "cuda")
    st = state_for(case)
    st.build_pool(case.lens)
    seer.gated_sparse_decode(st.shape, case.q, st.kv, case.lens, st.pooled, st.rule, st.k_max,
                             st.scores, st.sel_idx, st.sel_cnt, None, None, st.workspace)
    outs = []
    for mode in (seer.SEER_COMBINE_PER_UNIT, seer.SEER_COMBINE_PER_HEAD):
        st.out.fill_(float("nan"))
        st.lse.fill_(float("nan"))
        seer.sparse_decode_combine(st.shape, st.out, st.lse, st.workspace, mode)
        torch.cuda.synchronize()
        outs.append((st.out.clone(), st.lse.clone()))
    (o0, l0), (o1, l1) = outs
    bad = (o0.view(torch.int32) != o1.view(torch.int32)).sum().item()
    assert bad == 0, f"{bad} output elements differ"
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))




@pytest.mark.parametrize("combine", sorted(COMBINE))
@pytest.mark.parametrize("name", sorted(FEW_UNITS))
def test_few_long_units(name, combine):
    """Units with many partial records, merged per unit and per query head."""
    wl = FEW_UNITS[name]
    print(f"[case] few long units {name} combine per {combine}", flush=True)
    case = make_case(wl, "cuda")
    st = state_for(case, combine=COMBINE[combine])
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    lens = case.lens.tolist()
    for (b, g) in units_of(wl):
        check_unit(st, case, case.q, lens, b, g, tag=name)


@pytest.mark.parametrize("name", ["tiny_1k", "paged_small", "bf16_d64_g8"])
def test_dense_matches_oracle(name):
    wl = SMALL[name]
    case = make_case(wl, "cuda")
    st = state_for(case)
    st.attend(case.q, case.lens, dense=True)
    torch.cuda.synchronize()
    G = wl.group
    for (b, g) in units_of(wl):
        L = int(case.lens[b])
        ref = oracle_unit(case, b, g, case.q, L, dense=True)
        out = st.out[b, g * G:(g + 1) * G].cpu().double().numpy()
        lse = st.lse[b, g * G:(g + 1) * G].cpu().double().numpy()
        assert np.abs(out - ref["out"]).max() <= TOL[wl.dtype]
        assert np.abs(lse - ref["lse"]).max() <= TOL[wl.dtype]


def test_decode_with_oracle_selection():
    """Attention fed the oracle's ids (random subsets, any order) matches the oracle."""
    wl = SMALL["planted_b2"]
    case = make_case(wl, "cuda")
    st = state_for(case)
    rng = np.random.default_rng(3)
    U = wl.batch * wl.num_kv_heads
    n = O.block_count(wl.context, wl.block_size)
    k_max = 20
    sel = np.full((U, k_max), -1, np.int32)
    cnt = np.zeros(U, np.int32)
    chosen = {}
    for u in range(U):
        c = int(rng.integers(1, k_max + 1))
        ids = rng.choice(n, size=c, replace=False)
        sel[u, :c] = ids          # deliberately unsorted
        cnt[u] = c
        chosen[u] = ids
    st.attend(case.q, case.lens, sel_idx=torch.from_numpy(sel).cuda(),
              sel_cnt=torch.from_numpy(cnt).cuda(), k_max=k_max)
    torch.cuda.synchronize()
    G = wl.group
    for u in range(U):
        b, g = divmod(u, wl.num_kv_heads)
        ref = oracle_unit(case, b, g, case.q, wl.context, sel=chosen[u])
        out = st.out[b, g * G:(g + 1) * G].cpu().double().numpy()
        assert np.abs(out - ref["out"]).max() <= TOL["bf16"]


@pytest.mark.parametrize("fuse", [True, None], ids=["forced", "auto"])
@pytest.mark.parametrize("name", sorted(SMALL) + ["budget_32k", "long_131k", "paged_var"])
def test_gated_equals_separate_calls_bitwise(name, fuse):
    """The gated call writes exactly what the gate call followed by the
    attention call writes: scores, ids, counts, out, lse -- with the fused
    kernel forced, also where the call would not choose it (more than 256
    blocks per unit, more units than workgroups), and on the library's own
    choice."""
    wl = SMALL[name] if name in SMALL else WORKLOADS[name].with_(batch=2)
    if name == "paged_var":
        wl = WORKLOADS[name].with_(batch=48)     # 384 units on 256 workgroups
    print(f"[case] gated vs separate {name}", flush=True)
    case = make_case(wl, "cuda")
    q = case.q[0] if wl.decode_steps else case.q
    fused, sep = state_for(case, fuse=fuse), state_for(case)
    for st in (fused, sep):
        st.build_pool(case.lens)
    fused.step(q, case.lens)
    sep.step_unfused(q, case.lens)
    torch.cuda.synchronize()
    for attr in ("scores", "sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(fused, attr), getattr(sep, attr)), attr


def test_max_units():
    """SEER_MAX_UNITS (sequence, KV head) pairs: 1024 paged sequences of 1..700
    tokens on 8 KV heads.  Waves cross many units and most units hold one or two
    partial records.  Every unit's kept count follows the keep rule, sampled
    units match the oracle, and the fused call (forced: its workgroups gate
    32 units each) equals the separate calls bitwise."""
    wl = WORKLOADS["paged_var"].with_(batch=1024, num_q_heads=16, num_kv_heads=8, head_dim=64,
                                      variable_context=(1, 700), keep=(1, 4))
    assert wl.batch * wl.num_kv_heads == 8192          # SEER_MAX_UNITS
    print("[case] max units: 1024 x 8 units", flush=True)
    case = make_case(wl, "cuda")
    sep = state_for(case, fuse=False)
    sep.build_pool(case.lens)
    sep.step(case.q, case.lens)
    torch.cuda.synchronize()
    lens = case.lens.tolist()
    want = [O.clamp_count(O.keep_count(O.block_count(L, wl.block_size), 1, 4),
                          O.block_count(L, wl.block_size)) for L in lens]
    got = sep.sel_cnt.view(wl.batch, wl.num_kv_heads).cpu().numpy()
    assert (got == np.array(want)[:, None]).all()
    for (b, g) in units_of(wl, limit=12, seed=7):
        check_unit(sep, case, case.q, lens, b, g, tag="max units")
    fused = state_for(case, fuse=True)
    fused.build_pool(case.lens)
    fused.step(case.q, case.lens)
    torch.cuda.synchronize()
    for attr in ("scores", "sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(fused, attr), getattr(sep, attr)), attr


def test_gated_with_a_wide_block_table():
    """8192 blocks per sequence (the largest table): the gated call (fused
    kernel forced) matches the separate calls and the oracle (its key buffer
    alone is 64 KiB of LDS)."""
    S, d, NB, L = 64, 64, 8192, 3000
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8192)
    k = torch.zeros(1, 1, NB * S, d, device="cuda")
    v = torch.zeros_like(k)
    k[0, 0, :L] = torch.randn(L, d, generator=gen, device="cuda")
    v[0, 0, :L] = torch.randn(L, d, generator=gen, device="cuda")
    q = torch.randn(1, 4, d, generator=gen, device="cuda")
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    top_k = torch.tensor([7], dtype=torch.int32, device="cuda")
    sts = [DecodeState(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=d, block_size=S,
                       max_blocks=NB, dtype=torch.float32, k=k, v=v, k_max=16, top_k=top_k,
                       fuse=True)
           for _ in range(2)]
    for st in sts:
        st.build_pool(lens)
    sts[0].step(q, lens)
    sts[1].step_unfused(q, lens)
    torch.cuda.synchronize()
    for attr in ("scores", "sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(sts[0], attr), getattr(sts[1], attr)), attr
    kk, vv = f64(k[0, 0, :L]), f64(v[0, 0, :L])
    p32, _, _ = O.pool_keys(kk, L, S)
    qg = f64(q[0])
    s = O.gate_scores(qg, p32, d)
    sel = O.select_top_blocks(s, O.clamp_count(7, O.block_count(L, S)))
    assert np.array_equal(sts[0].sel_idx[0, :7].cpu().numpy(), sel)
    toks = O.selected_tokens(sel, L, S)
    for h in range(4):
        o, lse, _ = O.attend(qg[h], kk, vv, toks)
        assert np.abs(sts[0].out[0, h].cpu().double().numpy() - o).max() <= TOL["f32"]


def test_paged_equals_contiguous_bitwise():
    wl = SMALL["paged_small"]
    case = make_case(wl, "cuda")
    flat = wl.with_(paged=False)
    case_c = make_case(flat, "cuda")
    # same draws: the paged pools hold exactly the contiguous rows
    st_p, st_c = state_for(case), state_for(case_c)
    for st, c in ((st_p, case), (st_c, case_c)):
        st.build_pool(c.lens)
        st.step(c.q, c.lens)
    torch.cuda.synchronize()
    assert torch.equal(st_p.pooled, st_c.pooled)
    assert torch.equal(st_p.sel_idx, st_c.sel_idx)
    assert torch.equal(st_p.out, st_c.out) and torch.equal(st_p.lse, st_c.lse)


@pytest.mark.parametrize("name", ["paged_small", "long_small", "tiny_1k"])
def test_nan_poison_never_reaches_outputs(name):
    wl = SMALL[name]
    clean, dirty = make_case(wl, "cuda"), make_case(wl, "cuda", poison=True)
    outs = []
    for c in (clean, dirty):
        st = state_for(c)
        st.out.fill_(float("nan"))
        st.lse.fill_(float("nan"))
        st.build_pool(c.lens)
        st.step(c.q, c.lens)
        torch.cuda.synchronize()
        assert torch.isfinite(st.out).all() and torch.isfinite(st.lse).all()
        outs.append((st.pooled.clone(), st.sel_idx.clone(), st.out.clone(), st.lse.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_repeatable_bitwise():
    wl = SMALL["paged_small"]
    case = make_case(wl, "cuda")
    st = state_for(case)
    st.build_pool(case.lens)
    ref = None
    for _ in range(10):
        st.step(case.q, case.lens)
        cur = (st.sel_idx.clone(), st.out.clone(), st.lse.clone())
        if ref is None:
            ref = cur
        else:
            for a, b in zip(ref, cur):
                assert torch.equal(a, b)


def test_split_stages_equal_fused():
    wl = SMALL["bf16_g3_keep"]
    case = make_case(wl, "cuda")
    st = state_for(case)
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    out1, lse1 = st.out.clone(), st.lse.clone()
    st.out.zero_()
    seer.sparse_decode_partial(st.shape, case.q, st.kv, case.lens, st.sel_idx, st.sel_cnt,
                               st.k_max, st.workspace)
    seer.sparse_decode_combine(st.shape, st.out, st.lse, st.workspace)
    torch.cuda.synchronize()
    assert torch.equal(out1, st.out) and torch.equal(lse1, st.lse)


# ------------------------------------------------------------------ edge shapes

EDGE = [
    # (name, overrides): lengths 1, S+1, k = 1, k = n, G = 1, d/S/dtype corners
    ("len1", dict(context=1, top_k=1)),
    ("len_s_plus_1", dict(context=65, top_k=1)),
    ("k1", dict(context=1000, top_k=1)),
    ("k_all", dict(context=1000, top_k=16)),
    ("k_over", dict(context=1000, top_k=99)),
    ("g1_bf16", dict(dtype="bf16", num_q_heads=1, num_kv_heads=1, context=513, top_k=2)),
    ("d128_s128_bf16", dict(dtype="bf16", head_dim=128, block_size=128, context=1025, top_k=3)),
    ("d64_s128_f32", dict(block_size=128, context=1000, top_k=2)),
    ("g8_d128_f32", dict(num_q_heads=8, head_dim=128, context=700, top_k=4)),
]


@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(name, kw):
    wl = WORKLOADS["tiny_1k"].with_(**kw)
    print(f"[case] edge {name}", flush=True)
    case = make_case(wl, "cuda")
    st = state_for(case, k_max=min(wl.max_blocks, max(1, wl.top_k)))
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    for (b, g) in units_of(wl):
        check_unit(st, case, case.q, case.lens.tolist(), b, g, tag=name)


@pytest.mark.parametrize("context", [2048, 32768, 32769, 40000])
def test_ties_and_zero_query(context):
    """Duplicated blocks and a zero query: ties go to the lower block id (block
    counts 32 and 512 take the rank-counting selection, 513 and 625 the radix
    selection)."""
    wl = WORKLOADS["planted_8k"].with_(batch=1, planted_fraction=None, context=context)
    print(f"[case] ties context {context}", flush=True)
    case = make_case(wl, "cuda")
    S = wl.block_size
    # blocks 5 and 20 identical (keys and values), and block 7 == block 3
    for dst, src in ((20, 5), (7, 3)):
        case.k[:, :, dst * S:(dst + 1) * S] = case.k[:, :, src * S:(src + 1) * S]
        case.v[:, :, dst * S:(dst + 1) * S] = case.v[:, :, src * S:(src + 1) * S]
    case.q[:, :8] = 0          # KV heads 0 and 1 see a zero query: scores all zero
    st = state_for(case)
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    for g in range(wl.num_kv_heads):
        ref = check_unit(st, case, case.q, case.lens.tolist(), 0, g, tag="ties")
        if g < 2:
            assert list(ref["sel"]) == list(range(len(ref["sel"])))


# ------------------------------------------------------------------ pooling

def test_incremental_pooling_bitwise():
    wl = WORKLOADS["long_131k"].with_(batch=3, context=200, decode_steps=700)
    case = make_case(wl, "cuda")
    st = state_for(case)
    L0 = wl.context
    lens = torch.full((wl.batch,), L0, dtype=torch.int32, device="cuda")
    st.build_pool(lens)
    steps = [1, 1, 55, 1, 127, 128, 1, 200, 1, 1, 180]
    cur = L0
    for inc in steps:
        new = torch.full_like(lens, cur + inc)
        st.append(lens, new)
        lens, cur = new, cur + inc
    torch.cuda.synchronize()
    fresh = state_for(case)
    fresh.build_pool(lens)
    torch.cuda.synchronize()
    assert torch.equal(st.pooled, fresh.pooled)
    assert torch.equal(st.open_sum, fresh.open_sum)
    for b in range(wl.batch):
        for g in (0, wl.num_kv_heads - 1):
            k, _ = unit_kv(case, b, g, cur)
            p32, _, open_sum = O.pool_keys(k, cur, wl.block_size)
            n = O.block_count(cur, wl.block_size)
            assert np.array_equal(gpu_pooled(st, wl, b, g, n).view(np.uint32), p32.view(np.uint32))
            u = b * wl.num_kv_heads + g
            got_open = st.open_sum.view(-1, wl.head_dim)[u].cpu().numpy()
            assert np.array_equal(got_open.view(np.uint64), open_sum.view(np.uint64))


# ------------------------------------------------------------------ graphs

def test_graph_replay_matches_eager():
    """A captured decode step replays bit-identically, with eager work in between."""
    wl = SMALL["paged_small"]
    case = make_case(wl, "cuda")
    st = state_for(case)
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    ref = (st.sel_idx.clone(), st.sel_cnt.clone(), st.out.clone(), st.lse.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.step(case.q, case.lens)
    for _ in range(3):
        st.out.zero_()
        st.lse.zero_()
        st.sel_idx.fill_(-7)
        st.sel_cnt.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (st.sel_idx, st.sel_cnt, st.out, st.lse)):
            assert torch.equal(a, b)


# ------------------------------------------------------------------ selection rules

RULES = [
    ("force_first", dict(force_first=True)),
    ("force_both", dict(force_first=True, force_last=True)),
    ("threshold_0", dict(threshold=0.0)),
    ("threshold_1", dict(threshold=1.0)),
    ("threshold_forced", dict(threshold=1.5, force_last=True)),
    ("unified", dict(unified=True)),
    ("unified_forced", dict(unified=True, force_first=True, force_last=True)),
    ("unified_threshold", dict(unified=True, threshold=0.0)),
]


@pytest.mark.parametrize("wname", ["planted_b2", "paged_small", "bf16_d64_g8"])
@pytest.mark.parametrize("rname,rule", RULES, ids=[r[0] for r in RULES])
def test_selection_rules(wname, rname, rule):
    """Forced blocks, the threshold gate and the cross-head unified selection:
    ids and counts bit-exact, scores and outputs against the oracle."""
    wl = SMALL[wname]
    print(f"[case] rule {rname} on {wname}", flush=True)
    case = make_case(wl, "cuda")
    st = state_for(case, **rule)
    st.build_pool(case.lens)
    st.step(case.q, case.lens)
    torch.cuda.synchronize()
    S, d, G, Hkv = wl.block_size, wl.head_dim, wl.group, wl.num_kv_heads
    lens = case.lens.tolist()
    for b in range(wl.batch):
        L = lens[b]
        n = O.block_count(L, S)
        kv = [unit_kv(case, b, g, L) for g in range(Hkv)]
        pooled = [O.pool_keys(k, L, S)[0] for k, _ in kv]
        qb = f64(case.q[b])
        if rule.get("unified"):
            s_all = [O.gate_scores_unified(qb, pooled, d)] * Hkv
        else:
            s_all = [O.gate_scores(qb[g * G:(g + 1) * G], pooled[g], d) for g in range(Hkv)]
        for g in range(Hkv):
            u = b * Hkv + g
            s = s_all[g]
            if "threshold" in rule:
                sel = O.select_blocks(s, threshold=rule["threshold"],
                                      force_first=rule.get("force_first", False),
                                      force_last=rule.get("force_last", False), k_max=st.k_max)
            else:
                k = (O.clamp_count(wl.top_k, n) if wl.top_k is not None
                     else O.keep_count(n, *wl.keep))
                sel = O.select_blocks(s, k=k, force_first=rule.get("force_first", False),
                                      force_last=rule.get("force_last", False), k_max=st.k_max)
            cnt = int(st.sel_cnt[u])
            ids = st.sel_idx[u].cpu().numpy()
            assert cnt == len(sel), f"{rname} count {b},{g}"
            assert np.array_equal(ids[:cnt], sel), f"{rname} ids {b},{g}"
            assert (ids[cnt:] == -1).all()
            got_s = st.scores.view(-1, wl.max_blocks)[u, :n].cpu().numpy()
            assert np.abs(got_s - s).max() <= 1e-12 * max(np.abs(s).max(), 1e-300)
            toks = O.selected_tokens(sel, L, S)
            out = st.out[b, g * G:(g + 1) * G].cpu().double().numpy()
            for h in range(G):
                o, lse, _ = O.attend(qb[g * G + h], kv[g][0], kv[g][1], toks)
                assert np.abs(out[h] - o).max() <= TOL[wl.dtype], f"{rname} out {b},{g},{h}"


@pytest.mark.parametrize("rule", [dict(force_first=True), dict(force_first=True, force_last=True)],
                         ids=["first", "both"])
def test_fused_forced_blocks_equal_separate_calls(rule):
    wl = SMALL["paged_small"]
    case = make_case(wl, "cuda")
    fused, sep = state_for(case, fuse=True, **rule), state_for(case, **rule)
    for st in (fused, sep):
        st.build_pool(case.lens)
    fused.step(case.q, case.lens)
    sep.step_unfused(case.q, case.lens)
    torch.cuda.synchronize()
    for attr in ("scores", "sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(fused, attr), getattr(sep, attr)), attr


@pytest.mark.parametrize("name,want", [("sparse90_32k", 1), ("budget_32k", 1),
                                       ("planted_8k", 1), ("tiny_1k", 1),
                                       ("long_131k", 2), ("paged_var", 0)])
def test_fusion_policy(name, want):
    """The gate is fused while each workgroup gates about one unit in one
    pass (at most one unit per workgroup, at most 256 blocks per unit: 1);
    with longer tables and at most one unit per workgroup the score kernel
    scores and the attention kernel selects (2); never for a threshold or
    unified rule; the rule's fuse field forces either way."""
    wl = WORKLOADS[name]
    shape = seer.make_shape(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                            wl.block_size, wl.max_blocks, DT[wl.dtype])
    k_max = wl.top_k if wl.top_k else seer.keep_blocks(wl.max_blocks, *wl.keep)
    top_k = (None if wl.keep else
             torch.full((wl.batch,), wl.top_k, dtype=torch.int32, device="cuda"))

    def rule(fuse=None):
        return seer.make_select(keep=wl.keep, top_k=top_k, fuse=fuse)

    assert seer.gated_decode_path(shape, rule(), k_max) == want
    assert seer.gated_decode_is_fused(shape, rule(), k_max) == (want != 0)
    thr = seer.make_select(threshold=0.0, fuse=True)
    assert seer.gated_decode_path(shape, thr, k_max) == 0
    assert seer.gated_decode_path(shape, seer.make_select(keep=wl.keep, top_k=top_k,
                                                          unified=True), k_max) == 0
    assert seer.gated_decode_path(shape, rule(False), k_max) == 0
    assert seer.gated_decode_path(shape, rule(True), k_max) == 1   # these all fit in LDS


@pytest.mark.parametrize("rule", [dict(), dict(force_first=True),
                                  dict(force_first=True, force_last=True)],
                         ids=["plain", "first", "both"])
def test_given_scores_path_equals_separate_calls(rule):
    """Tables longer than one score chunk, with at most one unit per
    workgroup: the score kernel scores and the attention kernel's workgroups
    select from those scores.  Scores, ids, counts, out and lse equal the gate
    kernels followed by the attention kernel bitwise, forced blocks
    included, and the selections match the oracle."""
    wl = WORKLOADS["long_131k"].with_(batch=2)
    print(f"[case] given-scores path, long table, rule {rule}", flush=True)
    case = make_case(wl, "cuda")
    given, sep = state_for(case, **rule), state_for(case, **rule)
    assert seer.gated_decode_path(given.shape, given.rule, given.k_max) == 2
    q = case.q[0]
    for st in (given, sep):
        st.build_pool(case.lens)
    given.step(q, case.lens)
    sep.step_unfused(q, case.lens)
    torch.cuda.synchronize()
    for attr in ("scores", "sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(given, attr), getattr(sep, attr)), attr
    S, d, G = wl.block_size, wl.head_dim, wl.group
    lens = case.lens.tolist()
    for (b, g) in [(0, 0), (1, wl.num_kv_heads - 1)]:
        L = lens[b]
        n = O.block_count(L, S)
        k, _ = unit_kv(case, b, g, L)
        s = O.gate_scores(f64(q[b, g * G:(g + 1) * G]), O.pool_keys(k, L, S)[0], d)
        sel = O.select_blocks(s, k=O.keep_count(n, *wl.keep),
                              force_first=rule.get("force_first", False),
                              force_last=rule.get("force_last", False), k_max=given.k_max)
        u = b * wl.num_kv_heads + g
        cnt = int(given.sel_cnt[u])
        assert cnt == len(sel) and np.array_equal(given.sel_idx[u].cpu().numpy()[:cnt], sel)


def test_usage_example():
    """The decode loop as the documentation shows it: build the pooled table,
    step, write the next token's K/V, append, step again; the second step
    equals a step on a state built from scratch at the new lengths."""
    torch.manual_seed(3)
    B, Hq, Hkv, d, S, NB = 2, 8, 2, 128, 64, 20
    k = torch.randn(B, Hkv, NB * S, d, device="cuda").to(torch.bfloat16)
    v = torch.randn(B, Hkv, NB * S, d, device="cuda").to(torch.bfloat16)
    lens = torch.tensor([700, 1111], dtype=torch.int32, device="cuda")
    q = torch.randn(B, Hq, d, device="cuda").to(torch.bfloat16)
    kw = dict(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, block_size=S,
              max_blocks=NB, dtype=torch.bfloat16, k=k, v=v, keep=(1, 10))
    st = DecodeState(**kw)
    st.build_pool(lens)
    out, lse = st.step(q, lens)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    st.append(lens, lens + 1)
    st.step(q, lens + 1)
    fresh = DecodeState(**kw)
    fresh.build_pool(lens + 1)
    fresh.step(q, lens + 1)
    torch.cuda.synchronize()
    for attr in ("pooled", "scores", "sel_idx", "sel_cnt", "out", "lse"):
        assert torch.equal(getattr(st, attr), getattr(fresh, attr)), attr
