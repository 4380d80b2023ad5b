"""Pins of the fp64 oracle to the pages' definitions and to mathematics.

Every check here compares the oracle with something other than itself: a
hand-worked case (tests/golden/hand_cases.json), a closed form, an invariant,
brute force, or a library routine (torch's scaled_dot_product_attention and
logsumexp in fp64 on the CPU, Python's sorted).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import seer_oracle as O
from workloads import WORKLOADS, make_case

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


# ---------------------------------------------------------------- kept counts

def test_keep_counts_hand_table():
    for c in GOLD["keep_counts"]["cases"]:
        n = c["n"]
        if "top_k" in c:
            got = O.clamp_count(c["top_k"], n)
        elif "keep" in c:
            got = O.keep_count(n, *c["keep"])
        else:
            got = O.budget_count(n, c["budget_tokens"], c["block_size"])
        assert got == c["expected"], c


@pytest.mark.parametrize("frac", [(1, 10), (1, 20), (1, 4), (3, 10), (7, 8), (1, 1)])
def test_keep_count_is_smallest_cover(frac):
    a, b = frac
    f = Fraction(a, b)
    for n in range(1, 2049):
        k = O.keep_count(n, a, b)
        assert 1 <= k <= n
        assert Fraction(k, n) >= f or k == n
        if k > 1:
            assert Fraction(k - 1, n) < f


def test_block_partition():
    for S in (64, 128):
        for L in (1, 2, S - 1, S, S + 1, 5 * S, 5 * S + 7, 1024 * S + 1):
            n = O.block_count(L, S)
            ranges = [O.block_range(j, L, S) for j in range(n)]
            assert ranges[0][0] == 0 and ranges[-1][1] == L
            assert all(ranges[i][1] == ranges[i + 1][0] for i in range(n - 1))
            assert all(1 <= hi - lo <= S for lo, hi in ranges)
            assert all(hi - lo == S for lo, hi in ranges[:-1])


# ---------------------------------------------------------------- pooling

def test_pool_hand_mean_partial_block():
    c = GOLD["pool_mean_partial_block"]
    keys = np.array(c["keys"], dtype=np.float64)
    p32, p64, open_sum = O.pool_keys(keys, c["length"], c["block_size"])
    assert np.array_equal(p64, np.array(c["expected_pooled"], dtype=np.float64))
    assert np.array_equal(p32, np.array(c["expected_pooled"], dtype=np.float32))
    assert np.array_equal(open_sum, np.array([60.0, -12.0]))


def test_pool_sequential_order():
    c = GOLD["pool_sequential_fp64"]
    col = np.array(c["keys_col0"], dtype=np.float64)
    keys = np.stack([col, np.ones_like(col)], axis=1)
    _, p64, _ = O.pool_keys(keys, c["length"], c["block_size"])
    assert p64[0, 0] == c["expected_pooled_col0"]
    assert p64[0, 1] == 1.0


def test_pool_fp32_round_to_nearest_even():
    for c in GOLD["pool_fp32_rne"]["cases"]:
        keys = np.array(c["keys"], dtype=np.float64)[:, None]
        p32, p64, _ = O.pool_keys(keys, 2, 2)
        assert p64[0, 0] == c["expected_fp64_mean"]
        assert p32.dtype == np.float32 and float(p32[0, 0]) == c["expected_fp32"]


def test_pool_identical_rows_give_that_row():
    rng = np.random.default_rng(1)
    d, S = 16, 64
    for L in (1, 7, 64, 65, 200):
        n = O.block_count(L, S)
        rows = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
        keys = np.repeat(rows, S, axis=0)
        p32, p64, _ = O.pool_keys(keys, L, S)
        # a block of c identical rows x sums to c*x exactly only when exact; use
        # small dyadic rows so every sum is exact
        small = np.round(rows * 8) / 8
        p32s, p64s, _ = O.pool_keys(np.repeat(small, S, axis=0), L, S)
        assert np.array_equal(p64s, small)
        assert np.allclose(p64, rows, rtol=1e-15, atol=0)


def test_pool_incremental_equals_rebuild_bitwise():
    rng = np.random.default_rng(2)
    d, S = 8, 16
    keys = rng.standard_t(3, size=(200, d)).astype(np.float32).astype(np.float64)
    L0 = 37
    p32, _, acc = O.pool_keys(keys, L0, S)
    L = L0
    for step in (1, 1, 10, 11, 1, 16, 31, 1, 60):
        p32, acc = O.pool_keys_append(p32, acc, keys, L, L + step, S)
        L += step
        r32, _, racc = O.pool_keys(keys, L, S)
        assert p32.shape == r32.shape
        assert np.array_equal(p32.view(np.uint32), r32.view(np.uint32))
        assert np.array_equal(acc.view(np.uint64), racc.view(np.uint64))


# ---------------------------------------------------------------- gate scores

def test_gate_scores_hand_case():
    c = GOLD["gate_scores_group_sum"]
    s = O.gate_scores(np.array(c["q_group"], float), np.array(c["pooled"], np.float32), c["head_dim"])
    assert np.array_equal(s, np.array(c["expected_scores"]))


def test_gate_scores_group_mapping_through_decode_step():
    c = GOLD["gqa_group_mapping"]
    d = c["head_dim"]
    q = np.array(c["q"], float)[None]
    k = np.zeros((1, c["num_kv_heads"], 2, d))
    v = np.zeros_like(k)
    pooled = [[np.zeros((2, d), np.float32), np.array(c["pooled_kv1"], np.float32)]]
    res = O.decode_step(q, k, v, [2], 1, pooled=pooled, top_k=[1])
    assert np.array_equal(res["scores"][(0, 1)], np.array(c["expected_scores_kv1"]))
    assert list(res["sel"][(0, 1)]) == [0]


def test_gate_scores_zero_query_and_linearity():
    rng = np.random.default_rng(3)
    P = rng.standard_normal((50, 32)).astype(np.float32)
    q = rng.standard_normal((4, 32))
    assert np.array_equal(O.gate_scores(np.zeros((4, 32)), P, 32), np.zeros(50))
    assert np.array_equal(O.gate_scores(2.0 * q, P, 32), 2.0 * O.gate_scores(q, P, 32))
    # G = 1 is a plain dot product over sqrt(d); 1/sqrt(64) = 1/8 exactly
    s = O.gate_scores(q[:1], P, 64)
    assert np.allclose(s * 8.0, P.astype(float) @ q[0], rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------- selection

def _brute_select(s, k):
    order = sorted(range(len(s)), key=lambda j: (-(s[j] + 0.0), j))
    return sorted(order[:k])


def test_select_matches_full_sort_brute_force():
    rng = np.random.default_rng(4)
    for trial in range(300):
        n = int(rng.integers(1, 80))
        k = int(rng.integers(1, n + 1))
        if trial % 3 == 0:
            s = rng.integers(-3, 4, size=n).astype(float)      # many ties
        else:
            s = rng.standard_normal(n)
        got = O.select_top_blocks(s, k)
        assert list(got) == _brute_select(list(s), k)
        assert all(got[i] < got[i + 1] for i in range(len(got) - 1))


def test_select_special_cases():
    assert list(O.select_top_blocks(np.zeros(10), 3)) == [0, 1, 2]
    assert list(O.select_top_blocks(np.array([-0.0, 0.0, -0.0]), 1)) == [0]
    assert list(O.select_top_blocks(np.array([0.0, -0.0]), 1)) == [0]
    assert list(O.select_top_blocks(np.arange(7.0), 7)) == list(range(7))
    assert list(O.select_top_blocks(np.array([1.0, 5.0, 3.0, 5.0]), 1)) == [1]
    assert list(O.select_top_blocks(np.array([1.0, 5.0, 3.0, 5.0]), 3)) == [1, 2, 3]


def test_duplicate_block_loses_to_lower_twin():
    rng = np.random.default_rng(5)
    P = rng.standard_normal((20, 16)).astype(np.float32)
    q = rng.standard_normal((2, 16))
    s = O.gate_scores(q, P, 16)
    top = int(np.argmax(s))
    P2 = P.copy()
    P2[19] = P2[top]
    s2 = O.gate_scores(q, P2, 16)
    assert s2[19] == s2[top]
    assert list(O.select_top_blocks(s2, 1)) == [top]


# ---------------------------------------------------------------- attention

def _sdpa_dense(q, k, v, L, G):
    """torch's fp64 scaled_dot_product_attention over the first L keys."""
    qt = torch.from_numpy(q)[:, :, None, :]                     # B, Hq, 1, d
    kt = torch.from_numpy(k[:, :, :L]).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v[:, :, :L]).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, :, 0].numpy()


@pytest.mark.parametrize("G,L,S,d", [(4, 1000, 64, 64), (5, 130, 64, 32), (1, 129, 128, 16), (8, 17, 16, 8)])
def test_dense_equals_sdpa_and_logsumexp(G, L, S, d):
    rng = np.random.default_rng(6)
    B, Hkv = 2, 2
    Hq = G * Hkv
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, L + 5, d))
    v = rng.standard_normal((B, Hkv, L + 5, d))
    res = O.decode_step(q, k, v, [L, L], S, dense=True)
    ref = _sdpa_dense(q, k, v, L, G)
    assert np.allclose(res["out"], ref, rtol=0, atol=1e-12)
    kt = torch.from_numpy(k[:, :, :L]).repeat_interleave(G, dim=1)
    logits = torch.einsum("bhd,bhtd->bht", torch.from_numpy(q), kt) / math.sqrt(d)
    assert np.allclose(res["lse"], torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_gather_equals_masked_brute_force():
    rng = np.random.default_rng(7)
    for trial in range(40):
        S = int(rng.choice([4, 8]))
        L = int(rng.integers(1, 60))
        d = 8
        n = O.block_count(L, S)
        k = int(rng.integers(1, n + 1))
        sel = np.sort(rng.choice(n, size=k, replace=False))
        keys = rng.standard_normal((n * S, d))
        vals = rng.standard_normal((n * S, d))
        q = rng.standard_normal(d)
        toks = O.selected_tokens(sel, L, S)
        mask = np.zeros(n * S, bool)
        mask[toks] = True
        o1, l1, w = O.attend(q, keys, vals, toks)
        o2, l2 = O.attend_masked(q, keys, vals, mask)
        assert np.allclose(o1, o2, rtol=0, atol=1e-13)
        assert abs(l1 - l2) < 1e-13
        assert abs(w.sum() - 1.0) < 1e-12 and (w >= 0).all()
        # the partial last block contributes only its valid tokens
        assert toks.max() < L


def test_attention_order_invariance():
    rng = np.random.default_rng(8)
    L, S, d = 500, 32, 16
    keys = rng.standard_normal((L, d))
    vals = rng.standard_normal((L, d))
    q = rng.standard_normal(d)
    sel = np.array([0, 3, 7, 15])
    o1, l1, _ = O.attend(q, keys, vals, O.selected_tokens(sel, L, S))
    o2, l2, _ = O.attend(q, keys, vals, O.selected_tokens(sel[::-1], L, S))
    assert np.allclose(o1, o2, rtol=0, atol=1e-14) and abs(l1 - l2) < 1e-13


def test_attention_closed_forms():
    c = GOLD["attention_two_tokens"]
    e = math.e
    o, l, w = O.attend(np.array(c["q"], float), np.array(c["keys"], float),
                       np.array(c["values"], float), np.array([0, 1]))
    assert np.allclose(o, [e / (e + 1), 1 / (e + 1), 0, 0], rtol=0, atol=1e-15)
    assert abs(l - math.log(e + 1)) < 1e-15
    rng = np.random.default_rng(9)
    keys = rng.standard_normal((10, 4))
    vals = rng.standard_normal((10, 4))
    q = rng.standard_normal(4)
    # one token: the output is its value, the lse its logit
    o, l, _ = O.attend(q, keys, vals, np.array([3]))
    assert np.array_equal(o, vals[3]) and abs(l - keys[3] @ q / 2.0) < 1e-15
    # constant values: the output is that constant
    o, _, _ = O.attend(q, keys, np.tile(vals[:1], (10, 1)), np.arange(10))
    assert np.allclose(o, vals[0], rtol=0, atol=1e-14)
    # equal keys: uniform weights, the output is the mean value
    o, _, w = O.attend(q, np.tile(keys[:1], (10, 1)), vals, np.arange(10))
    assert np.allclose(w, 0.1, rtol=0, atol=1e-16) and np.allclose(o, vals.mean(0), atol=1e-14)


# ---------------------------------------------------------------- paging

def test_paged_gather_round_trip_and_poison():
    rng = np.random.default_rng(10)
    B, Hkv, S, d = 3, 2, 8, 4
    lens = [17, 8, 30]
    nb = [O.block_count(x, S) for x in lens]
    kc = rng.standard_normal((B, Hkv, 4 * S, d))
    perm = rng.permutation(sum(nb))
    pool = np.full((sum(nb), Hkv, S, d), np.nan)
    table = -np.ones((B, 4), int)
    nxt = 0
    for b in range(B):
        for j in range(nb[b]):
            table[b, j] = perm[nxt]
            pool[perm[nxt]] = kc[b, :, j * S:(j + 1) * S]
            nxt += 1
    for b in range(B):
        g = O.gather_paged(pool, table, b, nb[b])
        assert np.array_equal(g, kc[b, :, : nb[b] * S])
    # NaN past the length never reaches the output
    kp = kc.copy()
    vp = rng.standard_normal(kc.shape)
    q = rng.standard_normal((B, 2 * Hkv, d))
    base = O.decode_step(q, kp, vp, lens, S, top_k=[2, 2, 2])
    for b in range(B):
        kp[b, :, lens[b]:] = np.nan
        vp[b, :, lens[b]:] = np.nan
    pois = O.decode_step(q, kp, vp, lens, S, top_k=[2, 2, 2])
    assert np.array_equal(base["out"], pois["out"])


# ---------------------------------------------------------------- workloads

def _np(t):
    return t.double().numpy()


def test_planted_blocks_are_selected():
    """Planted blocks (about 16 standard deviations above the rest) are kept."""
    wl = WORKLOADS["planted_8k"].with_(batch=1)
    c = make_case(wl)
    res = O.decode_step(_np(c.q), _np(c.k), _np(c.v), c.lens.tolist(), wl.block_size, keep=wl.keep)
    for g in range(wl.num_kv_heads):
        sel = set(res["sel"][(0, g)].tolist())
        assert len(sel) == 13
        assert set(c.planted[0, g].tolist()) <= sel


def test_tiny_workload_selection_and_dense_limit():
    wl = WORKLOADS["tiny_1k"]
    c = make_case(wl)
    q, k, v = _np(c.q), _np(c.k), _np(c.v)
    res = O.decode_step(q, k, v, c.lens.tolist(), wl.block_size, top_k=c.top_k.tolist())
    assert len(res["sel"][(0, 0)]) == 4
    full = O.decode_step(q, k, v, c.lens.tolist(), wl.block_size, top_k=[16])
    ref = _sdpa_dense(q, k, v, 1024, 4)
    assert np.allclose(full["out"], ref, rtol=0, atol=1e-12)


def test_generator_is_deterministic():
    wl = WORKLOADS["paged_var"].with_(batch=3, variable_context=(100, 300))
    a = make_case(wl)
    b = make_case(wl)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.lens, b.lens), (a.page_table, b.page_table)):
        assert torch.equal(x, y)


def test_pool_signed_zero_sum_of_valid_keys_only():
    """A block whose valid keys are all -0.0 pools to -0.0: only valid keys are summed."""
    keys = np.zeros((8, 2))
    keys[4:6] = -0.0
    p32, p64, _ = O.pool_keys(keys, 6, 4)
    assert np.signbit(p64[1]).all() and np.signbit(p32[1]).all()
    assert not np.signbit(p64[0]).any()


# ------------------------------------------------------------------ selection rules

def _rule_brute_force(s, k, forced, cap):
    """Direct check of the top-k-with-forced-blocks definition."""
    n = len(s)
    count = max(1, min(max(k, len(forced)), cap))
    chosen = list(forced[:count])
    others = [j for j in range(n) if j not in forced]
    while len(chosen) < count:
        best = None
        for j in others:
            if j in chosen:
                continue
            if best is None or s[j] > s[best] or (s[j] == s[best] and j < best):
                best = j
        chosen.append(best)
    return sorted(chosen)


def test_select_blocks_reduces_to_plain_top_k():
    rng = np.random.default_rng(41)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        s = np.round(rng.standard_normal(n), 1)          # many ties
        k = int(rng.integers(1, n + 1))
        assert np.array_equal(O.select_blocks(s, k=k), O.select_top_blocks(s, k))


def test_select_blocks_forced_brute_force():
    rng = np.random.default_rng(42)
    for _ in range(300):
        n = int(rng.integers(1, 30))
        s = np.round(rng.standard_normal(n), 1)
        k = int(rng.integers(1, n + 1))
        ff, fl = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        cap = int(rng.integers(1, n + 1))
        forced = ([0] if ff else []) + ([n - 1] if fl and not (ff and n == 1) else [])
        got = O.select_blocks(s, k=k, force_first=ff, force_last=fl, k_max=cap)
        assert list(got) == _rule_brute_force(s, k, forced, cap)
        for f in forced[: len(got)]:
            assert f in got


def test_threshold_zero_is_the_sigmoid_gate():
    """The pages' hard gate keeps sigmoid(s / T) > 0.5; with tau = 0 the rule
    keeps exactly those blocks, whatever the temperature T > 0."""
    rng = np.random.default_rng(43)
    for T in (0.05, 1.0, 20.0):
        for _ in range(50):
            s = rng.standard_normal(64) * 3
            gate = 1.0 / (1.0 + np.exp(-s / T)) > 0.5
            if not gate.any():
                continue
            assert np.array_equal(O.select_blocks(s, threshold=0.0), np.nonzero(gate)[0])


def test_threshold_edges():
    s = np.array([-1.0, -0.5, -2.0, -0.5])
    assert list(O.select_blocks(s, threshold=0.0)) == [1]        # none above: the best block
    s = np.array([3.0, 1.0, 2.0, 5.0, 4.0])
    assert list(O.select_blocks(s, threshold=0.0, k_max=2)) == [3, 4]   # capped: the best two
    assert list(O.select_blocks(s, threshold=2.5)) == [0, 3, 4]
    # forced blocks count towards the threshold set and survive the cap first
    assert list(O.select_blocks(s, threshold=2.5, force_first=True, force_last=True,
                                k_max=3)) == [0, 3, 4]
    assert list(O.select_blocks(np.array([-0.0, 0.0, 1.0]), threshold=0.0)) == [2]


def test_unified_scores_pins():
    rng = np.random.default_rng(44)
    d, n, Hkv, G = 16, 12, 3, 2
    q = rng.standard_normal((Hkv * G, d))
    P = [rng.standard_normal((n, d)).astype(np.float32).astype(np.float64) for _ in range(Hkv)]
    # one KV head: the per-head gate score
    assert np.array_equal(O.gate_scores_unified(q[:G], P[:1], d), O.gate_scores(q[:G], P[0], d))
    # scaling the query by 2 doubles every score exactly
    assert np.array_equal(O.gate_scores_unified(2 * q, P, d), 2 * O.gate_scores_unified(q, P, d))
    # the sum of the per-head scores (equal up to the order of the additions)
    per = sum(O.gate_scores(q[g * G:(g + 1) * G], P[g], d) for g in range(Hkv))
    assert np.allclose(O.gate_scores_unified(q, P, d), per, rtol=1e-14, atol=1e-14)
    # reordering the KV heads (with their query groups) changes nothing but rounding
    perm = [2, 0, 1]
    qp = np.concatenate([q[g * G:(g + 1) * G] for g in perm])
    assert np.allclose(O.gate_scores_unified(qp, [P[g] for g in perm], d),
                       O.gate_scores_unified(q, P, d), rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- learned gate

def _gate_weights(rng, H, d):
    w1 = rng.integers(-127, 128, size=(H, d)).astype(np.int8)
    beta = (rng.uniform(0.5, 1.5, size=H) / (127.0 * math.sqrt(d))).astype(np.float32)
    b1 = rng.normal(0.0, 0.05, size=H).astype(np.float32)
    wq = (rng.normal(0.0, 1.0, size=(H, d)) / math.sqrt(d)).astype(np.float32)
    return w1, beta, b1, wq


def test_learned_gate_hand_case():
    """The network on two blocks, worked by hand in exact rational arithmetic
    (tests/golden): the scores depend on key bits far below a 7-bit image of
    the block, and those bits decide the top-1 block."""
    c = GOLD["learned_gate_network"]
    p = np.array(c["pooled"], dtype=np.float64)
    p32 = p.astype(np.float32)
    assert np.array_equal(p32.astype(np.float64), p)          # the stored values are fp32
    s = O.learned_gate_scores(np.array(c["q_group"]), p32, np.array(c["w1"], dtype=np.int8),
                              np.array(c["w1_scale"], dtype=np.float32),
                              np.array(c["b1"], dtype=np.float32),
                              np.array(c["wq"], dtype=np.float32))
    want = np.array([float(x) for x in c["expected_scores"]])
    assert np.array_equal(s, want)                             # short dyadic values: exact
    assert O.select_top_blocks(s, 1).tolist() == c["expected_top1"]


def test_learned_gate_hidden_permutation_invariance():
    rng = np.random.default_rng(12)
    H, d, n = 256, 64, 40
    w1, beta, b1, wq = _gate_weights(rng, H, d)
    p = rng.normal(size=(n, d)).astype(np.float32)
    qg = rng.normal(size=(4, d))
    s = O.learned_gate_scores(qg, p, w1, beta, b1, wq)
    perm = rng.permutation(H)
    s2 = O.learned_gate_scores(qg, p, w1[perm], beta[perm], b1[perm], wq[perm])
    assert np.allclose(s, s2, rtol=1e-12, atol=1e-12 * np.abs(s).max())


def test_learned_gate_homogeneity():
    rng = np.random.default_rng(13)
    H, d, n = 256, 128, 33
    w1, beta, b1, wq = _gate_weights(rng, H, d)
    p = rng.normal(size=(n, d)).astype(np.float32)
    qg = rng.normal(size=(4, d))
    s = O.learned_gate_scores(qg, p, w1, beta, b1, wq)
    # the query enters linearly (through u only): 2q gives exactly 2s
    assert np.array_equal(O.learned_gate_scores(2.0 * qg, p, w1, beta, b1, wq), 2.0 * s)
    # without a bias the network is positively homogeneous in the keys; a
    # power-of-two factor scales every fp64 step exactly
    zb = np.zeros_like(b1)
    s0 = O.learned_gate_scores(qg, p, w1, beta, zb, wq)
    assert np.array_equal(O.learned_gate_scores(qg, p * np.float32(4.0), w1, beta, zb, wq), 4.0 * s0)
    # and a negative factor moves every unit to the other side of the ReLU
    neg = O.learned_gate_scores(qg, -p, w1, beta, zb, wq)
    both = O.learned_gate_scores(qg, p, w1, beta, zb, wq) - neg
    lin = O.gate_scores((((wq.astype(np.float64) @ qg.sum(axis=0)) * beta.astype(np.float64))
                         @ w1.astype(np.float64))[None, :], p, d) * math.sqrt(d)
    assert np.allclose(both, lin, rtol=0, atol=1e-11 * np.abs(lin).max())


def test_learned_gate_bias_saturation():
    rng = np.random.default_rng(14)
    H, d, n = 256, 64, 50
    w1, beta, _, wq = _gate_weights(rng, H, d)
    p = rng.normal(size=(n, d)).astype(np.float32)
    qg = rng.normal(size=(2, d))
    s = O.learned_gate_scores(qg, p, w1, beta, np.full(H, -1e30, dtype=np.float32), wq)
    assert np.all(s == 0.0)
    assert O.select_top_blocks(s, 7).tolist() == list(range(7))


def test_learned_gate_reduces_to_the_linear_gate():
    """With every hidden unit active the network is linear: s_j equals the
    parameter-free gate on the same fp32 keys with the effective query
    w = sum_m u_m beta_m W1_m (times sqrt(d), undoing that gate's scale),
    plus the constant u . b1."""
    rng = np.random.default_rng(15)
    H, d, n = 256, 128, 64
    w1, beta, _, wq = _gate_weights(rng, H, d)
    p = rng.normal(size=(n, d)).astype(np.float32)
    qg = rng.normal(size=(4, d))
    zmax = (beta[None, :].astype(np.float64)
            * np.abs(p.astype(np.float64) @ w1.astype(np.float64).T)).max()
    b1 = np.full(H, np.float32(2.0 * zmax + 1.0), dtype=np.float32)     # every z_jm > 0
    s = O.learned_gate_scores(qg, p, w1, beta, b1, wq)
    u = wq.astype(np.float64) @ qg.sum(axis=0)
    w = (u * beta.astype(np.float64)) @ w1.astype(np.float64)
    c = float(u @ b1.astype(np.float64))
    lin = O.gate_scores(w[None, :], p, d) * math.sqrt(d)
    assert np.allclose(s - c, lin, rtol=0, atol=1e-9 * (abs(c) + np.abs(lin).max()))
    assert not np.allclose(lin, 0.0)


def test_learned_gate_one_unit_by_brute_force():
    """Random small networks against a scalar loop over units and dimensions
    (exact fractions for the first layer, so no rounding order is shared)."""
    from fractions import Fraction
    rng = np.random.default_rng(16)
    for _ in range(5):
        H, d, n = 7, 5, 6
        w1 = rng.integers(-127, 128, size=(H, d)).astype(np.int8)
        beta = rng.uniform(0.1, 2.0, size=H).astype(np.float32)
        b1 = rng.normal(size=H).astype(np.float32)
        wq = rng.normal(size=(H, d)).astype(np.float32)
        p = rng.normal(size=(n, d)).astype(np.float32)
        qg = rng.normal(size=(3, d))
        s = O.learned_gate_scores(qg, p, w1, beta, b1, wq)
        qbar = [sum(Fraction(float(qg[h, i])) for h in range(3)) for i in range(d)]
        for j in range(n):
            tot = Fraction(0)
            for m in range(H):
                z = Fraction(float(beta[m])) * sum(int(w1[m, i]) * Fraction(float(p[j, i]))
                                                   for i in range(d)) + Fraction(float(b1[m]))
                um = sum(Fraction(float(wq[m, i])) * qbar[i] for i in range(d))
                tot += um * max(z, Fraction(0))
            assert abs(s[j] - float(tot)) <= 1e-12 * max(1.0, abs(float(tot)))


# ---------------------------------------------------------------- reporting

def test_boundary_gap_hand_case():
    c = GOLD["boundary_gap"]
    assert O.boundary_gap(np.array(c["scores"]), c["k"]) == pytest.approx(c["expected"], rel=1e-15)


def test_boundary_gap_properties():
    rng = np.random.default_rng(31)
    s = rng.normal(size=100)
    g = O.boundary_gap(s, 10)
    # invariant to a positive affine change of the scores, order-free
    assert O.boundary_gap(3.0 * s - 7.0, 10) == pytest.approx(g, rel=1e-12)
    assert O.boundary_gap(rng.permutation(s), 10) == g
    # by brute force: the k-th minus the (k+1)-th largest over the std
    srt = sorted(s.tolist(), reverse=True)
    assert g == pytest.approx((srt[9] - srt[10]) / np.std(s), rel=1e-12)
    assert O.boundary_gap(s, 100) == float("inf") and O.boundary_gap(s, 150) == float("inf")
    t = s.copy()
    t[np.argsort(-t)[10]] = t[np.argsort(-t)[9]]          # tie at the boundary
    assert O.boundary_gap(t, 10) == 0.0
    assert O.boundary_gap(np.full(8, 2.5), 3) == 0.0


def test_pure_selection_hand_case():
    c = GOLD["pure_selection_rounding_tie"]
    S = c["block_size"]
    keys = np.array(c["keys_col0"])[:, None]
    p32, p64, _ = O.pool_keys(keys, len(keys), S)
    q = np.array(c["q"])
    assert p32[0, 0] == p32[1, 0] and p64[1, 0] > p64[0, 0]
    assert O.select_top_blocks(O.gate_scores(q, p32, 1), c["k"]).tolist() == c["expected_selection"]
    assert O.pure_selection(q, p64, 1, c["k"]).tolist() == c["expected_pure_selection"]


def test_pure_selection_equals_stored_when_means_are_fp32():
    """Blocks whose means are fp32 values (here: identical rows) give the same
    selection from the stored and the unrounded table."""
    rng = np.random.default_rng(32)
    S, d, n = 8, 16, 30
    rows = rng.normal(size=(n, d)).astype(np.float32).astype(np.float64)
    keys = np.repeat(rows, S, axis=0)
    p32, p64, _ = O.pool_keys(keys, n * S, S)
    assert np.array_equal(p32.astype(np.float64), p64)
    q = rng.normal(size=(4, d))
    assert np.array_equal(O.pure_selection(q, p64, d, 7),
                          O.select_top_blocks(O.gate_scores(q, p32, d), 7))


# ---------------------------------------------------------------- several query tokens

def test_gate_scores_tokens_reduce_to_the_head_sum():
    rng = np.random.default_rng(21)
    q = rng.normal(size=(3, 4, 64))
    p = rng.normal(size=(30, 64)).astype(np.float32)
    s = O.gate_scores_tokens(q, p, 64)
    # the T x G query rows act as T*G heads of one group (same order of addition)
    assert np.array_equal(s, O.gate_scores(q.reshape(12, 64), p, 64))
    assert np.array_equal(O.gate_scores_tokens(q[:1], p, 64), O.gate_scores(q[0], p, 64))
    assert np.array_equal(O.gate_scores_tokens(2.0 * q, p, 64), 2.0 * s)


def test_attend_tokens_single_token_and_causal_truncation():
    rng = np.random.default_rng(22)
    S, d, L, T, G = 16, 32, 150, 5, 3
    k = rng.normal(size=(L, d))
    v = rng.normal(size=(L, d))
    q = rng.normal(size=(T, G, d))
    sel = [0, 3, 7, 8, 9]
    out, lse = O.attend_tokens(q, k, v, sel, L, S)
    # T = 1 is the single-token decode
    o1, l1 = O.attend_tokens(q[-1:], k, v, sel, L, S)
    toks = O.selected_tokens(sel, L, S)
    for h in range(G):
        o, l, _ = O.attend(q[-1, h], k, v, toks)
        assert np.allclose(o1[0, h], o) and np.isclose(l1[0, h], l)
    # token t is the single-token decode of the sequence cut after its own position
    for t in range(T):
        cut = O.selected_tokens(sel, L - T + 1 + t, S)
        for h in range(G):
            o, l, _ = O.attend(q[t, h], k, v, cut)
            assert np.allclose(out[t, h], o, rtol=0, atol=1e-12) and np.isclose(lse[t, h], l)


def test_attend_tokens_equals_the_causal_masked_form():
    """The gather form against softmax over every key with a -inf mask that is
    block-selected AND causal (the mask form of the pages' Step 4)."""
    rng = np.random.default_rng(23)
    S, d, L, T, G = 8, 16, 61, 4, 2
    k = rng.normal(size=(L, d))
    v = rng.normal(size=(L, d))
    q = rng.normal(size=(T, G, d))
    sel = [1, 5, 7]                            # block 7 holds the last tokens 56..60
    out, lse = O.attend_tokens(q, k, v, sel, L, S)
    pos = np.arange(L)
    for t in range(T):
        mask = np.isin(pos // S, sel) & (pos <= L - T + t)
        for h in range(G):
            o, l = O.attend_masked(q[t, h], k, v, mask)
            assert np.allclose(out[t, h], o, rtol=0, atol=1e-12) and np.isclose(lse[t, h], l)


def test_attend_tokens_nothing_visible():
    """A token whose kept blocks all lie after it sees nothing: 0 and -inf."""
    rng = np.random.default_rng(24)
    S, d, L, T = 8, 8, 20, 3                   # tokens at 17, 18, 19; block 2 = 16..19
    k = rng.normal(size=(L, d))
    v = rng.normal(size=(L, d))
    q = rng.normal(size=(T, 1, d))
    out, lse = O.attend_tokens(q, k, v, [2], L, S)
    assert np.all(np.isfinite(lse))            # block 2 starts at 16 <= 17
    out, lse = O.attend_tokens(q, k, v, [2], 17, S)   # tokens at 14, 15, 16
    assert lse[0, 0] == -np.inf and lse[1, 0] == -np.inf and np.isfinite(lse[2, 0])
    assert np.all(out[0] == 0.0) and np.all(out[1] == 0.0)
