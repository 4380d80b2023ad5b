"""Plain fp64 CPU oracle for gated block-sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the library never does, and it
shares no code with the GPU path.

What it computes (one decode step, one attention layer, one new query token per
sequence, grouped-query attention with G = Hq / Hkv query heads per KV head):

* keys are cut into blocks of S tokens and each block is summarised by the
  mean of its keys; the new query token is used as it is, not pooled
  ("SeerAttention-R: Sparse Attention Adaptation for Long Reasoning",
  Abstract and AI Summary: keys pooled per block, query pooling removed for
  autoregressive decoding; block sizes 64/128);
* each block gets a gate score against the query, one selection is made per KV
  head and the top-scoring blocks are kept ("Sparse Attention Reasoning",
  Step 1: top-k selection of the gate's scores, k from the sparsity);
* exact softmax attention then runs over the tokens of the kept blocks only,
  which is softmax(QK^T / sqrt(d)) with every other key masked to -inf
  ("Sparse Attention Reasoning", Step 4: masked sparse attention).

Readings taken where the pages leave a step open (the pages describe a learned
gate but give no weights or internals):

* pooled key of block j = mean of the keys of its valid tokens, summed in
  fp64 in token order, then divided by the token count c_j (c_j < S for a
  partial last block), and stored rounded to fp32 (round to nearest even);
* gate score of block j for KV head g = sum over the group's query heads h of
  q_h . P_j / sqrt(d), evaluated in fp64 on the stored fp32 pooled keys;
* kept count: k = max(1, min(n, ceil(n * a / b))) for a kept fraction a/b
  (90% sparsity keeps 1/10), exact integer arithmetic; or an explicit count
  (a token budget B gives B // S), clamped to [1, n];
* order: score descending, ties to the lower block index, -0 equal to +0;
  the kept block ids are reported in ascending order;
* the new token's key and value are in the cache (its length includes it);
* a second, learned gate (``learned_gate_scores``) is the pages' gate network
  (Linear(d, 256), ReLU, Linear(256, 1)) applied to each block's stored fp32
  pooled key, with the second layer's weights a projection of the group's
  query so that the query stays unpooled; its weights are given (seeded,
  untrained; the first layer stored int8 with per-row scales), and every step
  runs in fp64 on the exact values;
* reporting only (nothing is gated on them): the selection the gate would
  make from the unrounded fp64 block means (``pure_selection``) and the gap
  between the last kept and the first dropped score in units of the scores'
  standard deviation (``boundary_gap``);
* several new query tokens per sequence (T, speculative or chunked decode):
  token t sits at position length-T+t and sees the kept positions up to its
  own (causal), and one selection per KV head serves all T tokens, scored
  with the query summed over the tokens and the group's heads.

Every function works on one (sequence, KV head) unless its name says otherwise.
Inputs are float64 arrays holding the exact values of the stored tensors.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# Blocks and kept counts
# --------------------------------------------------------------------------

def block_count(length: int, block_size: int) -> int:
    """Number of blocks that hold ``length`` tokens (the last one may be partial)."""
    return -(-int(length) // int(block_size))


def block_range(j: int, length: int, block_size: int) -> tuple:
    """Token positions [lo, hi) of block j of a sequence of ``length`` tokens."""
    lo = j * block_size
    return lo, min(lo + block_size, int(length))


def keep_count(n_blocks: int, keep_num: int, keep_den: int) -> int:
    """Blocks kept at kept fraction keep_num/keep_den of ``n_blocks``.

    The smallest count whose share of the blocks reaches the kept fraction, at
    least one and at most all blocks ("Sparse Attention Reasoning", Step 1,
    keeps the top (1 - sparsity) fraction with at least one kept; the ceiling
    here, computed on integers, is the reading that keeps a 90%-sparse
    selection from dropping below 10% of the blocks).
    """
    k = -(-int(n_blocks) * int(keep_num) // int(keep_den))
    return max(1, min(int(n_blocks), k))


def budget_count(n_blocks: int, budget_tokens: int, block_size: int) -> int:
    """Blocks kept under a token budget ("SeerAttention-R", Abstract: 4K budget)."""
    return max(1, min(int(n_blocks), int(budget_tokens) // int(block_size)))


def clamp_count(k: int, n_blocks: int) -> int:
    return max(1, min(int(n_blocks), int(k)))


# --------------------------------------------------------------------------
# Key pooling
# --------------------------------------------------------------------------

def pool_keys(keys: np.ndarray, length: int, block_size: int):
    """Block means of one (sequence, KV head)'s keys.

    keys: (T, d) float64, rows past ``length`` are ignored.
    Returns (pooled32 (n, d) float32, pooled64 (n, d) float64, open_sum (d,)
    float64) where open_sum is the fp64 sum of the last block's keys (the block
    that the next appended token continues, unless that block is full).
    The sum runs over the block's tokens in order, one fp64 add per token.
    """
    n = block_count(length, block_size)
    d = keys.shape[1]
    L = int(length)
    counts = np.array([block_range(j, L, block_size)[1] - j * block_size for j in range(n)])
    kb = np.zeros((n * block_size, d), dtype=np.float64)
    kb[:L] = keys[:L]
    kb = kb.reshape(n, block_size, d)
    # Token by token within every block at once: position 0, then 1, 2, ...
    acc = kb[:, 0].copy()
    for pos in range(1, block_size):
        valid = (pos < counts)[:, None]
        acc = np.where(valid, acc + kb[:, pos], acc)
    pooled64 = acc / counts[:, None]
    return pooled64.astype(np.float32), pooled64, acc[n - 1].copy()


def pool_keys_append(pooled32: np.ndarray, open_sum: np.ndarray, keys: np.ndarray,
                     old_length: int, new_length: int, block_size: int):
    """Appends tokens old_length..new_length-1 to a pooled table.

    The running fp64 sum of the open block restarts when a token opens a new
    block; after each token the mean of its block is rewritten.  Returns the
    updated (pooled32 (n_new, d), open_sum).  Equal, bit for bit, to
    ``pool_keys`` on new_length tokens, since both add the same fp64 values in
    the same order.
    """
    n_new = block_count(new_length, block_size)
    d = keys.shape[1]
    out = np.zeros((n_new, d), dtype=np.float32)
    out[: pooled32.shape[0]] = pooled32[:n_new]
    acc = open_sum.copy()
    for t in range(int(old_length), int(new_length)):
        j, pos = divmod(t, block_size)
        acc = keys[t].copy() if pos == 0 else acc + keys[t]
        out[j] = (acc / (pos + 1)).astype(np.float32)
    return out, acc


# --------------------------------------------------------------------------
# Gate scores and selection
# --------------------------------------------------------------------------

def gate_scores(q_group: np.ndarray, pooled: np.ndarray, head_dim: int) -> np.ndarray:
    """s_j = sum_h q_h . P_j / sqrt(d) for one KV head.

    q_group: (G, d) float64, the group's query heads; pooled: (n, d), the
    stored pooled keys (their exact values are used in fp64).
    """
    p = np.asarray(pooled, dtype=np.float64)
    s = np.zeros(p.shape[0], dtype=np.float64)
    for h in range(q_group.shape[0]):
        s = s + p @ q_group[h]
    return s / np.sqrt(float(head_dim))


def select_top_blocks(scores: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k highest-scoring blocks, in ascending order.

    Order: score descending, ties to the lower block id; -0.0 and +0.0 are the
    same score.  Scores must be finite.
    """
    s = np.asarray(scores, dtype=np.float64) + 0.0       # -0.0 + 0.0 is +0.0
    ids = np.arange(s.shape[0])
    order = np.lexsort((ids, -s))
    return np.sort(order[: int(k)])


def gate_scores_unified(q_seq: np.ndarray, pooled_heads: Sequence[np.ndarray],
                        head_dim: int) -> np.ndarray:
    """One score per block for a whole sequence: the KV heads' gate scores
    summed, s_j = sum_g sum_{h in group(g)} q_h . P_{g,j} / sqrt(d).

    q_seq: (Hq, d) float64, all query heads of the sequence (head h belongs to
    KV head h // G); pooled_heads[g]: (n, d), KV head g's stored pooled keys.
    The cross-head selection of the LessIsMore abstract (author page "Shijie
    Cao"): one ranking for every head of a layer instead of one per head.
    """
    Hkv = len(pooled_heads)
    G = q_seq.shape[0] // Hkv
    n = np.asarray(pooled_heads[0]).shape[0]
    s = np.zeros(n, dtype=np.float64)
    for g in range(Hkv):
        p = np.asarray(pooled_heads[g], dtype=np.float64)
        for h in range(g * G, (g + 1) * G):
            s = s + p @ q_seq[h]
    return s / np.sqrt(float(head_dim))


def select_blocks(scores: np.ndarray, *, k: Optional[int] = None,
                  threshold: Optional[float] = None, force_first: bool = False,
                  force_last: bool = False, k_max: Optional[int] = None) -> np.ndarray:
    """Kept block ids (ascending) of one selection under the general rule.

    Forced blocks F: block 0 when ``force_first`` (an attention sink) and the
    newest block n-1 when ``force_last`` (the recent context the LessIsMore
    abstract keeps); they are kept whatever their score.
    Top-k (``k`` given): the count is raised to |F| if smaller and capped at
    min(n, k_max); the kept set is F plus the best other blocks by
    (score desc, id asc) up to that count.
    Threshold (``threshold`` = tau given): the hard gate of "Sparse Attention
    Reasoning" (Step 1, the selection with a temperature keeps
    sigmoid(s / T) > 0.5, i.e. s > 0 for any T > 0), generalised to s > tau:
    the kept set is F plus every other block with s_j > tau; past k_max
    blocks, F plus the best of them up to k_max; if empty, the single best
    block.
    """
    s = np.asarray(scores, dtype=np.float64) + 0.0       # -0.0 + 0.0 is +0.0
    n = s.shape[0]
    cap = n if k_max is None else min(n, int(k_max))
    forced = []
    if force_first:
        forced.append(0)
    if force_last and (n - 1) not in forced:
        forced.append(n - 1)
    rest = np.array([j for j in range(n) if j not in forced], dtype=np.int64)
    ranked = rest[np.lexsort((rest, -s[rest]))] if len(rest) else rest
    if threshold is None:
        count = max(int(k), len(forced))
    else:
        count = len(forced) + int(np.sum(s[rest] > float(threshold)))
    count = max(1, min(count, cap))
    kept = forced[:count] + list(ranked[: count - min(count, len(forced))])
    return np.sort(np.array(kept, dtype=np.int64))


# --------------------------------------------------------------------------
# Learned gate (the gate network's shape, with given weights)
# --------------------------------------------------------------------------

GATE_HIDDEN = 256  # hidden width of the gate network ("Sparse Attention Reasoning", Step 1)


def learned_gate_scores(q_group: np.ndarray, pooled32: np.ndarray, w1: np.ndarray,
                        w1_scale: np.ndarray, b1: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """Gate scores of one KV head from a two-layer gate network.

    The network is the gate of "Sparse Attention Reasoning" (Step 1:
    Linear(hidden, 256), ReLU, Linear(256, 1)) applied to each block's pooled
    key, hidden = d; the second layer's weights are a projection of the
    group's query, u = Wq qbar, so that the score depends on the unpooled
    decode query ("SeerAttention-R", Abstract: a learned gate, query pooling
    removed):

        z_jm = beta_m * (W1_m . P_j) + b1_m,   h_jm = max(z_jm, 0),
        s_j  = sum_m u_m h_jm,                 u_m = Wq_m . qbar,  qbar = sum_h q_h,

    evaluated in fp64 on the exact values of the stored fp32 pooled keys P
    (pooled32 (n, d)), W1 (H, d) int8 with row scales beta = w1_scale (H,),
    b1 (H,), Wq (H, d) and q_group (G, d).
    """
    p = np.asarray(pooled32, dtype=np.float32).astype(np.float64)
    w = np.asarray(w1, dtype=np.int8).astype(np.float64)
    z = (p @ w.T) * np.asarray(w1_scale, dtype=np.float64)[None, :] \
        + np.asarray(b1, dtype=np.float64)[None, :]
    h = np.maximum(z, 0.0)
    qbar = np.asarray(q_group, dtype=np.float64).sum(axis=0)
    u = np.asarray(wq, dtype=np.float64) @ qbar
    return h @ u


# --------------------------------------------------------------------------
# Reporting: selection from unrounded block means, boundary gap
# --------------------------------------------------------------------------

def pure_selection(q_group: np.ndarray, pooled64: np.ndarray, head_dim: int, k: int) -> np.ndarray:
    """The top-k selection the gate would make from the unrounded fp64 block
    means (``pool_keys``'s second result) instead of the stored fp32 ones.

    Reported beside the selection, never required to equal it: the stored
    table is fp32, and blocks whose means differ by less than fp32 resolution
    tie there (the lower id wins) while they are ordered here.
    """
    return select_top_blocks(gate_scores(q_group, pooled64, head_dim), k)


def boundary_gap(scores: np.ndarray, k: int) -> float:
    """(s_(k) - s_(k+1)) / std(s): the gap between the k-th and the (k+1)-th
    largest score, in units of the scores' standard deviation (population,
    ddof = 0).  +inf when every block is kept (k >= n); 0 for a tie at the
    boundary or when all scores are equal.  The smaller it is, the smaller a
    perturbation of the scores that could change the selection.
    """
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    k = int(k)
    if k >= s.shape[0]:
        return float("inf")
    sd = float(np.std(s))
    if sd == 0.0:
        return 0.0
    return float((s[k - 1] - s[k]) / sd)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def selected_tokens(sel: Sequence[int], length: int, block_size: int) -> np.ndarray:
    """Valid token positions of the selected blocks."""
    parts = [np.arange(*block_range(int(j), length, block_size)) for j in sel]
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts)


def attend(q_head: np.ndarray, keys: np.ndarray, values: np.ndarray,
           tokens: np.ndarray, scale: Optional[float] = None):
    """Softmax attention of one query head over the given token positions.

    Returns (out (d,), lse, weights (len(tokens),)); lse is the natural log of
    sum_t exp(l_t) with l_t = (q . k_t) / sqrt(d) (or times ``scale``).
    """
    kk = keys[tokens]
    logits = kk @ q_head
    logits = logits / np.sqrt(float(q_head.shape[0])) if scale is None else logits * scale
    m = logits.max()
    e = np.exp(logits - m)
    z = e.sum()
    w = e / z
    return w @ values[tokens], m + np.log(z), w


def attend_masked(q_head: np.ndarray, keys: np.ndarray, values: np.ndarray,
                  token_mask: np.ndarray, scale: Optional[float] = None):
    """The same attention written as in "Sparse Attention Reasoning", Step 4.

    Scores against every key, keys outside the mask set to -inf, softmax over
    all keys, weights times all values.  Returns (out (d,), lse).
    """
    logits = keys @ q_head
    logits = logits / np.sqrt(float(q_head.shape[0])) if scale is None else logits * scale
    masked = np.where(token_mask, logits, -np.inf)
    m = masked.max()
    e = np.exp(masked - m)
    w = e / e.sum()
    vv = np.where(token_mask[:, None], values, 0.0)     # masked rows carry weight 0
    return w @ vv, m + np.log(e.sum())


# --------------------------------------------------------------------------
# Several new query tokens per sequence (speculative or chunked decode)
# --------------------------------------------------------------------------

def gate_scores_tokens(q_tokens: np.ndarray, pooled: np.ndarray, head_dim: int) -> np.ndarray:
    """Gate scores shared by the T new query tokens of one KV head: the query
    summed over the tokens and the group's heads (token-major),
    s_j = sum_t sum_h q_{t,h} . P_j / sqrt(d).

    q_tokens: (T, G, d) float64; pooled: (n, d).  The query tokens are pooled
    for the gate only, as SeerAttention pools queries before "-R" removes the
    pooling for single-token decoding ("SeerAttention-R", Abstract).
    """
    p = np.asarray(pooled, dtype=np.float64)
    s = np.zeros(p.shape[0], dtype=np.float64)
    for t in range(q_tokens.shape[0]):
        for h in range(q_tokens.shape[1]):
            s = s + p @ q_tokens[t, h]
    return s / np.sqrt(float(head_dim))


def attend_tokens(q_tokens: np.ndarray, keys: np.ndarray, values: np.ndarray,
                  sel: Sequence[int], length: int, block_size: int,
                  scale: Optional[float] = None):
    """Causal attention of T new tokens over the kept blocks of one KV head.

    The new tokens sit at positions length-T .. length-1 (their keys and
    values are in the cache); token t sees the kept positions p <= length-T+t
    ("Sparse Attention Reasoning", Step 4, with query_len = T and the causal
    mask of autoregressive decoding).  q_tokens: (T, G, d).  Returns out
    (T, G, d) and lse (T, G); a token that sees no key gets 0 and -inf.
    """
    T, G, d = q_tokens.shape
    toks = selected_tokens(sel, length, block_size)
    out = np.zeros((T, G, d))
    lse = np.full((T, G), -np.inf)
    for t in range(T):
        vis = toks[toks <= length - T + t]
        if len(vis) == 0:
            continue
        for h in range(G):
            o, l, _ = attend(q_tokens[t, h], keys, values, vis, scale)
            out[t, h] = o
            lse[t, h] = l
    return out, lse


# --------------------------------------------------------------------------
# Paged caches
# --------------------------------------------------------------------------

def gather_paged(pool: np.ndarray, page_table: np.ndarray, b: int, n_blocks: int) -> np.ndarray:
    """Contiguous (Hkv, n_blocks * S, d) view of sequence b from a paged pool.

    pool: (num_pages, Hkv, S, d); page_table: (B, max_blocks) page ids.
    """
    pages = [pool[int(page_table[b, j])] for j in range(n_blocks)]
    return np.concatenate(pages, axis=1)


# --------------------------------------------------------------------------
# One decode step for a batch
# --------------------------------------------------------------------------

def decode_step(q: np.ndarray, k: np.ndarray, v: np.ndarray, lens: Sequence[int],
                block_size: int, *, top_k: Optional[Sequence[int]] = None,
                keep: Optional[tuple] = None, pooled: Optional[list] = None,
                selection: Optional[list] = None, dense: bool = False,
                scale: Optional[float] = None, units: Optional[list] = None):
    """Gate, select and attend for every (sequence, KV head).

    q: (B, Hq, d); k, v: (B, Hkv, T, d) (a paged cache is gathered first);
    lens: tokens per sequence including the new one.  The kept count comes
    from ``top_k`` (explicit, clamped to [1, n]) or ``keep`` = (a, b).
    ``pooled[b][g]`` may hold a prebuilt fp32 pooled table; ``selection[b][g]``
    may fix the kept blocks; ``dense`` keeps every block.  ``units`` limits
    the work to a list of (b, g) pairs.

    Returns a dict with, per (b, g): ``sel`` (ascending ids), ``scores``
    (fp64), ``pooled`` (fp32); and ``out`` (B, Hq, d), ``lse`` (B, Hq) filled
    for the heads of the computed units (NaN elsewhere).
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    res_sel, res_scores, res_pool = {}, {}, {}
    todo = units if units is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for (b, g) in todo:
        L = int(lens[b])
        n = block_count(L, block_size)
        if pooled is not None:
            p32 = pooled[b][g]
        else:
            p32, _, _ = pool_keys(k[b, g], L, block_size)
        res_pool[(b, g)] = p32
        qg = q[b, g * G:(g + 1) * G]
        s = gate_scores(qg, p32, d)
        res_scores[(b, g)] = s
        if dense:
            sel = np.arange(n)
        elif selection is not None:
            sel = np.sort(np.asarray(selection[b][g], dtype=np.int64))
        else:
            if top_k is not None:
                kk = clamp_count(int(top_k[b]), n)
            else:
                kk = keep_count(n, keep[0], keep[1])
            sel = select_top_blocks(s, kk)
        res_sel[(b, g)] = sel
        toks = selected_tokens(sel, L, block_size)
        for h in range(g * G, (g + 1) * G):
            o, l, _ = attend(q[b, h], k[b, g], v[b, g], toks, scale)
            out[b, h] = o
            lse[b, h] = l
    return {"sel": res_sel, "scores": res_scores, "pooled": res_pool, "out": out, "lse": lse}
