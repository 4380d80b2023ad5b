"""Benchmark of gated block-sparse decode on one MI355X.

Workload (default ``sparse90_32k``): 16 sequences of 32768 tokens, 32 query /
8 KV heads, head_dim 128, 128-token blocks, 90% sparsity (26 of 256 blocks kept
per KV head), bf16 KV cache.  A step = gate scores + top-k selection + sparse
decode (split-KV partials, then their log-sum-exp combine) for one attention
layer, as two launches: the attention kernel with the gate fused in, then the
combine; the pooled-key table is built once beforehand (after prefill).  For a
workload with an incremental decode loop (``long_131k``) a step also appends
the new token to the pooled table, and the timed loop runs every decode step
of the loop, the context growing by one token per step.  The timed loop cycles
through ``--layers`` independent caches (one per attention layer of a model),
so no step finds its KV bytes in the 256 MB last-level cache.

Timed regions are replays of HIP graphs captured from the library's launches
(as a serving loop would run them), bracketed by events on the launch stream.

Prints one JSON line per workload (``--workload all``: every workload).
``value`` is decode tokens/s for one attention layer (sequences x steps /
time); ``roofline`` reports the fused gate + partial-decode kernel's
algorithmic bytes per launch (pooled table, kept K/V rows, query) over its mean
launch time (HIP events on the launch stream) against the 8 TB/s HBM peak;
``unfused`` times the same step as three launches (gate kernel, partial,
combine); ``dense`` times the same step with every block kept;
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + achieved HBM GB/s (% of peak), 90% sparsity, 32K ctx"
HBM_PEAK_GBPS = 8000.0
# Measured HBM bytes per launch of the fused kernel (rocprofv3 FETCH_SIZE and
# WRITE_SIZE, calibrated on a plain copy), valid only for the kernel sources
# whose digest the file records.
KERNEL_SOURCES = ["block_sparse_attention_29_amd/csrc/sparse_decode.hip",
                  "block_sparse_attention_29_amd/csrc/multi_decode.hip",
                  "block_sparse_attention_29_amd/csrc/decode_common.h",
                  "block_sparse_attention_29_amd/csrc/gate_phase.h",
                  "block_sparse_attention_29_amd/csrc/seer_device.h",
                  "block_sparse_attention_29_amd/csrc/seer_kernels.h",
                  "block_sparse_attention_29_amd/csrc/select_device.h",
                  "block_sparse_attention_29_amd/build.py"]


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"decode_partial_{workload}_hbm_traffic.txt")


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """Counter-measured bytes per fused launch, or None when the counters were
    taken on other kernel sources (or another workload)."""
    try:
        fields = {}
        with open(traffic_file(workload)) as f:
            for line in f:
                if ":" in line and not line.startswith((" ", "|", "#")):
                    key, val = line.split(":", 1)
                    fields[key.strip()] = val.strip()
        if fields.get("workload") != workload:
            return None
        if fields.get("source_sha256") != kernel_source_digest():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="timed steps (a workload with a decode loop runs its whole loop)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="sparse90_32k", help="a workload name, or 'all'")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--dense-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-learned-gate", action="store_true",
                    help="skip the learned gate network's step")
    ap.add_argument("--no-multi-token", action="store_true",
                    help="skip the step with several query tokens per sequence")
    ap.add_argument("--cpu-sample-seqs", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle processes for the CPU baseline (0: the host cores this "
                         "process may run on, at most 16)")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle check of the timed step")
    ap.add_argument("--parity-units", type=int, default=8)
    ap.add_argument("--fuse", choices=["auto", "always", "never"], default="auto",
                    help="where the step selects: the library's choice (auto), inside the "
                         "attention kernel whenever the rule allows (always), or in the gate "
                         "kernel first (never)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the decode path runs on one GPU; sharding it over "
                                   "several GPUs (by sequence or KV head) is not implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from block_sparse_attention_29_amd import seer
    from workloads import WORKLOADS

    torch.cuda.set_device(torch.device("cuda:0"))
    seer.load()
    names = list(WORKLOADS) if args.workload == "all" else [args.workload]
    for name in names:
        line = run_workload(WORKLOADS[name], args)
        print(json.dumps(line), flush=True)
        torch.cuda.empty_cache()

    if args.copy_calibration:
        dev = torch.device("cuda:0")
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


def run_workload(wl, args):
    import torch

    from block_sparse_attention_29_amd import seer
    from block_sparse_attention_29_amd.pipeline import DecodeState
    from workloads import make_case

    dev = torch.device("cuda:0")
    DT = {"f32": torch.float32, "bf16": torch.bfloat16}[wl.dtype]
    loop = wl.decode_steps > 0
    L0 = wl.context
    S, d = wl.block_size, wl.head_dim
    T = wl.query_tokens        # new query tokens per sequence per step

    # one case per layer: the same shape, independent draws
    states, cases = [], []
    for layer in range(args.layers):
        case = make_case(wl.with_(seed=wl.seed + 1000 * layer), dev)
        st = DecodeState(batch=wl.batch, num_q_heads=wl.num_q_heads,
                         num_kv_heads=wl.num_kv_heads, head_dim=d, block_size=S,
                         max_blocks=wl.max_blocks, dtype=DT, k=case.k, v=case.v,
                         page_table=case.page_table, keep=wl.keep, top_k=case.top_k,
                         query_tokens=T, fuse=args.fuse)
        st.build_pool(case.lens)
        states.append(st)
        cases.append(case)
        torch.cuda.synchronize()
        log(f"{wl.name}: layer {layer} ready")

    n_layers = args.layers
    if loop:
        # lens of every decode step of the loop (step i holds L0 + i + 1 tokens)
        lens_seq = [torch.full((wl.batch,), L0 + i, dtype=torch.int32, device=dev)
                    for i in range(wl.decode_steps + 1)]
        n_steps = wl.decode_steps * n_layers          # model steps x layers
    else:
        n_steps = args.steps

    def layer_of(i):
        return states[i % n_layers], cases[i % n_layers]

    def step(i, fused=True):
        st, case = layer_of(i)
        if loop:
            s = i // n_layers                         # decode step of the loop
            q, lens = case.q[s], lens_seq[s + 1]
            if fused:                                 # append, gate and decode in one call
                st.step_append(q, lens_seq[s], lens)
            else:
                st.append(lens_seq[s], lens)
                st.step_unfused(q, lens)
            return
        q, lens = case.q, case.lens
        if fused:
            st.step(q, lens)
        else:
            st.step_unfused(q, lens)

    def step_unfused(i):
        step(i, fused=False)

    def q_lens(i):
        st, case = layer_of(i)
        if loop:
            s = i // n_layers
            return case.q[s], lens_seq[s + 1]
        return case.q, case.lens

    # does the step select inside the attention kernel for this shape?
    # (2: the score kernel scores first and the attention kernel selects)
    path = seer.gated_decode_path(states[0].shape, states[0].rule, states[0].k_max, T)
    fused = path != 0

    def partial_only(i):
        """The step's dominant kernel alone (no combine): the fused gate +
        partial-decode kernel (with long tables the gate's score kernel and
        the attention kernel that selects from its scores, both), else the
        partial kernel (several query tokens: the multi-token one) on the
        selection the step made."""
        st, case = layer_of(i)
        q, lens = q_lens(i)
        if T > 1 and fused:
            seer.multi_gated_sparse_decode(st.shape, T, q, st.kv, lens, st.pooled, st.rule,
                                           st.k_max, st.scores, st.sel_idx, st.sel_cnt, None,
                                           None, st.workspace)
        elif T > 1:
            seer.multi_sparse_decode_partial(st.shape, T, q, st.kv, lens, st.sel_idx, st.sel_cnt,
                                             st.k_max, st.workspace)
        elif fused:
            seer.gated_sparse_decode(st.shape, q, st.kv, lens, st.pooled, st.rule, st.k_max,
                                     st.scores, st.sel_idx, st.sel_cnt, None, None, st.workspace)
        else:
            seer.sparse_decode_partial(st.shape, q, st.kv, lens, st.sel_idx, st.sel_cnt,
                                       st.k_max, st.workspace)

    def dense_step(i):
        st, case = layer_of(i)
        q, lens = q_lens(i)
        st.attend(q, lens, dense=True)

    def capture(fn, n):
        """One HIP graph of n consecutive calls of fn (launch gaps off the host)."""
        for i in range(min(n, 2 * n_layers)):        # eager warm-up before capture
            fn(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n):
                fn(i)
        torch.cuda.synchronize()
        return graph

    def timed(graph, reps=1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream()
        torch.cuda.synchronize()
        e0.record(cur)
        for _ in range(reps):
            graph.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def reset_pools():
        """A decode loop's pooled tables back to the prefill state."""
        for st, case in zip(states, cases):
            st.build_pool(case.lens)
        torch.cuda.synchronize()

    # ---- whole-step timing: all steps in one graph, warm-up steps before ----
    g_steps = capture(step, n_steps)
    if loop:
        reset_pools()
        timed(g_steps)                                # one warm-up pass of the loop
        reset_pools()
    elif args.warmup > 0:
        g_warm = capture(step, args.warmup)
        timed(g_warm)
    wall0 = time.perf_counter()
    ms_total = timed(g_steps)
    wall = time.perf_counter() - wall0
    ms_per_step = ms_total / n_steps
    tokens_per_s = wl.batch * T * n_steps / (ms_total / 1e3)
    # spread: five more replays of the same graph (a decode loop restarts from
    # the prefill state each time), per-step means
    reps = []
    for _ in range(5):
        if loop:
            reset_pools()
        reps.append(timed(g_steps) / n_steps)
    reps.sort()
    spread = {"replays": len(reps), "p10_ms": reps[0] + 0.4 * (reps[1] - reps[0]),
              "p50_ms": reps[2], "p90_ms": reps[3] + 0.6 * (reps[4] - reps[3])}
    del g_steps

    # ---- correctness of the timed step: one more step on layer 0, compared
    # with the fp64 oracle on sampled units ----
    parity = None
    if not args.no_parity:
        if loop:
            s_last = wl.decode_steps - 1
            q_chk, lens_chk = cases[0].q[s_last], lens_seq[s_last + 1]
        else:
            q_chk, lens_chk = cases[0].q, cases[0].lens
        states[0].step(q_chk, lens_chk)
        torch.cuda.synchronize()
        parity = check_parity(wl, states[0], cases[0], q_chk, lens_chk, args.parity_units)
        log(f"{wl.name}: parity {parity}")

    # ---- the same steps as three launches (gate kernel, partial, combine);
    # several query tokens have no fused gate, so their step is already that ----
    unfused_ms = None
    if T == 1:
        if loop:
            reset_pools()
        g_unf = capture(step_unfused, n_steps)
        if loop:
            reset_pools()
        unfused_ms = timed(g_unf) / n_steps
        del g_unf
        if loop:
            reset_pools()

    # ---- fused-kernel timing: back-to-back launches in one graph, events
    # around it on the launch stream ----
    n_k = 8 * n_layers if loop else max(4 * n_layers, n_steps // 2)
    if not fused:
        # the partial kernel runs on each layer's selection for the lengths it
        # is timed at (a decode loop's steps moved the lengths on)
        for i in range(n_layers):
            st, case = layer_of(i)
            q, lens = q_lens(i)
            st.select(q, lens)
        torch.cuda.synchronize()
    g_part = capture(partial_only, n_k)
    timed(g_part)
    k_ms = timed(g_part, 3) / (3 * n_k)

    # algorithmic bytes of one fused launch (layer 0, the selection it just
    # made): the pooled table, valid K/V tokens of the kept blocks, the query
    st0 = states[0]
    q0, lens0 = q_lens(0)
    torch.cuda.synchronize()
    e = wl.elem_bytes
    sel = st0.sel_idx.cpu().numpy()
    cnt = st0.sel_cnt.cpu().numpy()
    lens = lens0.cpu().numpy()
    tokens = 0
    for u in range(sel.shape[0]):
        L = int(lens[u // wl.num_kv_heads])
        for j in sel[u, : cnt[u]]:
            tokens += min(S, L - int(j) * S)
    kv_bytes = tokens * d * e * 2
    q_bytes = wl.batch * T * wl.num_q_heads * d * e
    blocks = int(sum(-(-int(L) // S) for L in lens))
    pooled_bytes = blocks * wl.num_kv_heads * d * 4
    # the fused kernel reads the pooled table; a partial kernel runs on a
    # selection made before it
    k_bytes = kv_bytes + q_bytes + (pooled_bytes if fused else 0)
    achieved = k_bytes / (k_ms * 1e-3) / 1e9
    step_gbps = k_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- dense decode at the same shape (speedup denominator) ----
    dense = None
    if args.dense_steps > 0:
        n_d = n_layers if loop else args.dense_steps
        g_dense = capture(dense_step, n_d)
        timed(g_dense)
        dense_ms = timed(g_dense) / n_d
        dense_bytes = int(lens.sum()) * wl.num_kv_heads * d * e * 2 + q_bytes
        dense = {"ms_per_step": dense_ms,
                 "tokens_per_s": wl.batch * T / (dense_ms * 1e-3),
                 "hbm_gbps": dense_bytes / (dense_ms * 1e-3) / 1e9,
                 "speedup_sparse_vs_dense": dense_ms / ms_per_step}
    log(f"{wl.name}: gpu timing done: {ms_per_step:.4f} ms/step")

    # ---- the learned gate network (seeded, untrained weights): its gate kernel,
    # then the partial and combine kernels on its selection ----
    learned = None
    if not loop and not args.no_learned_gate and T == 1:
        from workloads import make_gate_weights
        for layer, st in enumerate(states):
            st.gate_weights = make_gate_weights(wl.num_kv_heads, d, seed=wl.seed + 77 + layer).to(dev)

        def learned_gate_only(i):
            st, case = layer_of(i)
            q, lens_i = q_lens(i)
            st.select(q, lens_i)

        g_l = capture(step, n_steps)
        timed(g_l)
        l_ms = timed(g_l) / n_steps
        del g_l
        g_lg = capture(learned_gate_only, n_k)
        timed(g_lg)
        lg_ms = timed(g_lg, 3) / (3 * n_k)
        del g_lg
        for st in states:
            st.gate_weights = None
        H = 256
        # algorithmic bytes of one gate launch: pooled table, query, each KV
        # head's weights once; int8 operations of its first layer
        lg_bytes = pooled_bytes + q_bytes + wl.num_kv_heads * H * (d + 4 * d + 8)
        lg_ops = 2 * blocks * wl.num_kv_heads * H * d
        learned = {"ms_per_step": l_ms, "tokens_per_s": wl.batch / (l_ms * 1e-3),
                   "speedup_vs_dense": (dense["ms_per_step"] / l_ms) if dense else None,
                   "gate_kernel": f"learned_gate_kernel<{wl.dtype},{d}>",
                   "gate_launch_ms": lg_ms, "gate_bytes": lg_bytes,
                   "gate_hbm_gbps": lg_bytes / (lg_ms * 1e-3) / 1e9,
                   "gate_int8_tops": lg_ops / (lg_ms * 1e-3) / 1e12,
                   "weights": "seeded, untrained"}
        log(f"{wl.name}: learned gate step {l_ms:.4f} ms, gate kernel {lg_ms * 1e3:.2f} us")

    # ---- several new query tokens per sequence: the same layers' K/V, 4 query
    # tokens (16 query rows per KV head when G = 4), one selection per KV head ----
    multi = None
    TQ = 16 // wl.group if wl.group <= 16 else 0
    TQ = min(TQ, 4)
    if not loop and not args.no_multi_token and TQ > 1 and T == 1:
        gen = torch.Generator(device=dev)
        gen.manual_seed(wl.seed + 4242)
        mstates = []
        for st, case in zip(states, cases):
            ms = DecodeState(batch=wl.batch, num_q_heads=wl.num_q_heads,
                             num_kv_heads=wl.num_kv_heads, head_dim=d, block_size=S,
                             max_blocks=wl.max_blocks, dtype=DT, k=case.k, v=case.v,
                             page_table=case.page_table, keep=wl.keep, top_k=case.top_k,
                             query_tokens=TQ)
            ms.build_pool(case.lens)
            qm = torch.randn((wl.batch, TQ, wl.num_q_heads, d), generator=gen,
                             device=dev).to(DT)
            mstates.append((ms, qm, case))

        def mstep(i):
            ms, qm, case = mstates[i % n_layers]
            ms.step(qm, case.lens)

        def mdecode(i):
            ms, qm, case = mstates[i % n_layers]
            ms.attend(qm, case.lens)

        g_m = capture(mstep, n_steps)
        timed(g_m)
        m_ms = timed(g_m) / n_steps
        del g_m
        def mpartial(i):
            ms, qm, case = mstates[i % n_layers]
            seer.multi_sparse_decode_partial(ms.shape, TQ, qm, ms.kv, case.lens, ms.sel_idx,
                                             ms.sel_cnt, ms.k_max, ms.workspace)

        g_md = capture(mdecode, n_k)
        timed(g_md)
        md_ms = timed(g_md, 3) / (3 * n_k)
        del g_md
        g_mp = capture(mpartial, n_k)
        timed(g_mp)
        mp_ms = timed(g_mp, 3) / (3 * n_k)
        del g_mp
        ms0 = mstates[0][0]
        m_fused = seer.gated_decode_is_fused(ms0.shape, ms0.rule, ms0.k_max, TQ)
        mf_ms = None
        if m_fused:
            def mfused(i):
                ms, qm, case = mstates[i % n_layers]
                seer.multi_gated_sparse_decode(ms.shape, TQ, qm, ms.kv, case.lens, ms.pooled,
                                               ms.rule, ms.k_max, ms.scores, ms.sel_idx,
                                               ms.sel_cnt, None, None, ms.workspace)

            g_mf = capture(mfused, n_k)
            timed(g_mf)
            mf_ms = timed(g_mf, 3) / (3 * n_k)
            del g_mf
        msel = ms0.sel_idx.cpu().numpy()
        mcnt = ms0.sel_cnt.cpu().numpy()
        mtok = 0
        for u in range(msel.shape[0]):
            L = int(lens[u // wl.num_kv_heads])
            for j in msel[u, : mcnt[u]]:
                mtok += min(S, L - int(j) * S)
        m_bytes = mtok * d * e * 2 + wl.batch * TQ * wl.num_q_heads * d * e
        multi = {"workload": f"{wl.name} K/V with {TQ} new query tokens per sequence",
                 "query_tokens": TQ, "ms_per_step": m_ms,
                 "tokens_per_s": wl.batch * TQ / (m_ms * 1e-3),
                 "tokens_per_s_vs_one_token": (wl.batch * TQ / m_ms) / (wl.batch / ms_per_step),
                 "attend_ms": md_ms, "attend_bytes": m_bytes,
                 "attend_hbm_gbps": m_bytes / (md_ms * 1e-3) / 1e9,
                 "partial_launch_ms": mp_ms,
                 "partial_hbm_gbps": m_bytes / (mp_ms * 1e-3) / 1e9,
                 "gate_fused": m_fused,
                 "fused_launch_ms": mf_ms,
                 "fused_hbm_gbps": ((m_bytes + pooled_bytes) / (mf_ms * 1e-3) / 1e9
                                    if mf_ms else None),
                 "kernels": (f"decode_multi_kernel<{wl.dtype},{d},gated>, " if m_fused else
                             f"gate_unit_kernel, decode_multi_kernel<{wl.dtype},{d}>, ")
                            + f"decode_multi_combine_kernel<{d}>"}
        del mstates
        log(f"{wl.name}: {TQ}-token step {m_ms:.4f} ms")

    # ---- CPU baseline: the fp64 oracle on a bounded sample ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, cases[0], min(args.cpu_sample_seqs, wl.batch), args.cpu_seconds,
                           args.cpu_workers)

    kept = cnt[cnt > 0]
    config = {"workload": wl.name, "batch": wl.batch, "q_heads": wl.num_q_heads,
              "kv_heads": wl.num_kv_heads, "head_dim": d, "block_size": S,
              "context": list(wl.variable_context) if wl.variable_context else wl.context,
              "kept_blocks": [int(kept.min()), int(kept.max())] if len(kept) else [0, 0],
              "blocks_max": int(-(-int(lens.max()) // S)),
              "query_tokens": T, "paged": wl.paged, "decode_loop_steps": wl.decode_steps,
              "layers_cycled": n_layers}
    G = wl.group
    return {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": n_steps if loop else args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": config,
        "step_spread": spread,
        "step_hbm_gbps": step_gbps,
        "step_pct_hbm_peak": 100.0 * step_gbps / HBM_PEAK_GBPS,
        "gate_fused": fused,
        "gate_path": ["gate kernels first", "scores and selection in the attention kernel",
                      "score kernel, then selection in the attention kernel"][path],
        "unfused": None if unfused_ms is None else {
            "ms_per_step": unfused_ms, "speedup_fused_vs_unfused": unfused_ms / ms_per_step},
        "roofline": {"bound": "hbm",
                     "kernel": (("gate_score_kernel + " if path == 2 else "")
                                + (f"decode_multi_kernel<{wl.dtype},{d}" if T > 1 else
                                   f"decode_partial_kernel<{wl.dtype},{d},{G}")
                                + (",gated from scores>" if path == 2 else
                                   ",gated>" if fused else ">")),
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(wl.name),
                     "bytes_per_launch": k_bytes, "launch_ms": k_ms},
        "dense": dense,
        "learned_gate": learned,
        "multi_token": multi,
        "parity": parity,
        "cpu_baseline": cpu,
        "wall_s_timed_region": wall,
    }


def check_parity(wl, st, case, q, lens, n_units):
    """The step's outputs against the fp64 oracle on n_units sampled units
    (the first, the last and a seeded sample): max-abs error of out and lse,
    how many selections are bit-exact, the smallest boundary gap
    (s_k - s_k+1) / std(s), and how often the selection from the unrounded
    fp64 block means agrees."""
    import numpy as np

    from oracle import seer_oracle as O

    S, d, G, T = wl.block_size, wl.head_dim, wl.group, wl.query_tokens
    Hkv = wl.num_kv_heads
    U = wl.batch * Hkv
    rng = np.random.default_rng(12345)
    pick = sorted(set([0, U - 1] + rng.choice(U, size=min(U, n_units), replace=False).tolist()))
    lens_h = lens.cpu().numpy()
    sel_idx, sel_cnt = st.sel_idx.cpu().numpy(), st.sel_cnt.cpu().numpy()
    out, lse = st.out.cpu().double().numpy(), st.lse.cpu().double().numpy()
    qh = q.cpu().double().numpy()
    err_o = err_l = 0.0
    exact = pure = 0
    gaps = []
    for u in pick:
        b, g = divmod(u, Hkv)
        L = int(lens_h[b])
        n = O.block_count(L, S)
        if case.page_table is None:
            k = case.k[b, g, :n * S].double().cpu().numpy()
            v = case.v[b, g, :n * S].double().cpu().numpy()
        else:
            pages = case.page_table[b, :n].long()
            k = case.k[pages][:, g].reshape(-1, d).double().cpu().numpy()
            v = case.v[pages][:, g].reshape(-1, d).double().cpu().numpy()
        p32, p64, _ = O.pool_keys(k, L, S)
        kk = O.clamp_count(wl.top_k, n) if wl.top_k else O.keep_count(n, *wl.keep)
        if T > 1:
            qt = qh[b, :, g * G:(g + 1) * G]
            s = O.gate_scores_tokens(qt, p32, d)
            s_pure = O.gate_scores_tokens(qt, p64, d)
        else:
            qg = qh[b, g * G:(g + 1) * G]
            s = O.gate_scores(qg, p32, d)
            s_pure = O.gate_scores(qg, p64, d)
        sel = O.select_top_blocks(s, kk)
        exact += int(sel_cnt[u] == len(sel) and np.array_equal(sel_idx[u, :sel_cnt[u]], sel))
        pure += int(np.array_equal(O.select_top_blocks(s_pure, kk), sel))
        gaps.append(O.boundary_gap(s, kk))
        if T > 1:
            o_ref, l_ref = O.attend_tokens(qt, k, v, sel, L, S)
            o_got = out[b, :, g * G:(g + 1) * G]
            l_got = lse[b, :, g * G:(g + 1) * G]
        else:
            toks = O.selected_tokens(sel, L, S)
            o_ref = np.stack([O.attend(qg[h], k, v, toks)[0] for h in range(G)])
            l_ref = np.array([O.attend(qg[h], k, v, toks)[1] for h in range(G)])
            o_got = out[b, g * G:(g + 1) * G]
            l_got = lse[b, g * G:(g + 1) * G]
        err_o = max(err_o, float(np.abs(o_got - o_ref).max()))
        fin = np.isfinite(l_ref)
        err_l = max(err_l, float(np.abs(l_got[fin] - l_ref[fin]).max(initial=0.0)))
    return {"units_checked": len(pick), "max_abs_err_out": err_o, "max_abs_err_lse": err_l,
            "tolerance": 2e-3 if wl.dtype == "bf16" else 1e-5,
            "selection_bit_exact": f"{exact}/{len(pick)}",
            "gap_min_std": float(min(gaps)),
            "pure_fp64_selection_equal": f"{pure}/{len(pick)}"}


def _cpu_worker(job):
    """One oracle process of the CPU baseline: loads its units' inputs from
    the .npy files the parent wrote, builds their pooled tables (setup), then
    repeats the oracle's step over them for `seconds`.  Returns
    (repetitions, seconds, units)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import seer_oracle as O

    folder, units, spec, seconds = job
    S, d, G, TQ, loop, top_k, keep = spec
    data = []
    for u in units:
        z = np.load(os.path.join(folder, f"unit{u}.npz"))
        k = z["k"].astype(np.float64)
        v = z["v"].astype(np.float64)
        L = int(z["L"])
        p32, _, osum = O.pool_keys(k, L, S)
        data.append((k, v, p32, osum, z["q"], L))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        reps = 0
        while True:
            for (k, v, p32, osum, qg, L) in data:
                if loop:     # append the new token, then decode at L + 1
                    p32, _ = O.pool_keys_append(p32, osum.copy(), k, L, L + 1, S)
                    L = L + 1
                s = O.gate_scores_tokens(qg, p32, d) if TQ > 1 else O.gate_scores(qg, p32, d)
                n = O.block_count(L, S)
                kk = O.clamp_count(top_k, n) if top_k else O.keep_count(n, *keep)
                sel = O.select_top_blocks(s, kk)
                if TQ > 1:
                    O.attend_tokens(qg, k, v, sel, L, S)
                else:
                    toks = O.selected_tokens(sel, L, S)
                    for h in range(G):
                        O.attend(qg[h], k, v, toks)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return reps, el, len(units)


def cpu_baseline(wl, case, n_seqs, seconds, workers):
    """Times the fp64 oracle's step (pool append for a decode loop, gate,
    selection, attention) on the host cores: one process per core, the
    (sequence, KV head) units of the first n_seqs sequences dealt out to
    them; throughput is the units all processes finish per second, scaled to
    the whole batch."""
    import multiprocessing as mp
    import shutil
    import tempfile

    S, d, G, TQ = wl.block_size, wl.head_dim, wl.group, wl.query_tokens
    lens = case.lens.cpu().numpy()
    loop = wl.decode_steps > 0
    units = [(b, g) for b in range(n_seqs) for g in range(wl.num_kv_heads)]
    if workers <= 0:
        workers = min(16, len(os.sched_getaffinity(0)))
    workers = max(1, min(workers, len(units)))
    folder = tempfile.mkdtemp(prefix="seer_cpu_")
    try:
        import numpy as np
        for i, (b, g) in enumerate(units):
            L = int(lens[b])
            T = L + (1 if loop else 0)
            if case.page_table is None:
                k = case.k[b, g, :T].float().cpu().numpy()
                v = case.v[b, g, :T].float().cpu().numpy()
            else:
                n = -(-T // S)
                pages = case.page_table[b, :n].long()
                k = case.k[pages][:, g].reshape(-1, d)[:T].float().cpu().numpy()
                v = case.v[pages][:, g].reshape(-1, d)[:T].float().cpu().numpy()
            qsrc = case.q[0] if loop else case.q
            if TQ > 1:  # [B][TQ][Hq][d]: the group's heads of every token
                qg = qsrc[b, :, g * G:(g + 1) * G].double().cpu().numpy()
            else:
                qg = qsrc[b, g * G:(g + 1) * G].double().cpu().numpy()
            np.savez(os.path.join(folder, f"unit{i}.npz"), k=k, v=v, q=qg, L=np.int64(L))
        spec = (S, d, G, TQ, loop, wl.top_k, wl.keep)
        jobs = [(folder, list(range(w, len(units), workers)), spec, seconds)
                for w in range(workers)]
        with mp.get_context("spawn").Pool(workers) as pool:
            res = pool.map(_cpu_worker, jobs)
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    units_per_s = sum(reps * nu / el for reps, el, nu in res)
    steps_per_s = units_per_s / wl.num_kv_heads          # one step = every KV head of a sequence
    reps_min = min(r for r, _, _ in res)
    return {"value": steps_per_s * TQ, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{n_seqs} of {wl.batch} sequences ({len(units)} (sequence, KV head) "
                      f"units{f', {TQ} query tokens each' if TQ > 1 else ''}) dealt to "
                      f"{workers} oracle processes of one thread each; "
                      f"{'pool append + ' if loop else ''}gate + top-k + attention in fp64 "
                      f"NumPy repeated for {seconds:.0f} s per process (at least {reps_min} "
                      f"passes each), units per second summed over the processes and "
                      f"scaled to tokens/s of the full batch; pooled tables built beforehand"}


if __name__ == "__main__":
    main()
