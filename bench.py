"""Benchmark of one gated block-sparse decode step on one MI355X.

Workload (default): 16 sequences of 32768 tokens, 32 query / 8 KV heads,
head_dim 128, 128-token blocks, 90% sparsity (26 of 256 blocks kept per KV
head), bf16 KV cache.  A step = gate scores + top-k selection + sparse decode
(partial + log-sum-exp combine) for one attention layer; the pooled-key table
is built once beforehand (after prefill).  The timed loop cycles through
``--layers`` independent caches (one per attention layer of a model), so no
step finds its KV bytes in the 256 MB last-level cache.

Timed regions are replays of HIP graphs captured from the library's launches
(as a serving loop would run them), bracketed by events on the launch stream.

Prints one JSON line.  ``value`` is decode tokens/s (sequences x steps / time);
``roofline`` reports the partial-decode kernel's algorithmic bytes per launch
over its mean launch time (HIP events on the launch stream) against the 8 TB/s
HBM peak; ``dense`` times the same step with every block kept; ``cpu_baseline``
times the fp64 oracle on a bounded sample of the same workload.
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
# Measured HBM bytes per launch of the partial kernel (rocprofv3 FETCH_SIZE and
# WRITE_SIZE, calibrated on a plain copy), valid only for the kernel sources
# whose digest the file records.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partial_sparse90_32k_hbm_traffic.txt")
KERNEL_SOURCES = ["block_sparse_attention_29_amd/csrc/sparse_decode.hip",
                  "block_sparse_attention_29_amd/csrc/seer_device.h",
                  "block_sparse_attention_29_amd/csrc/seer_kernels.h",
                  "block_sparse_attention_29_amd/build.py"]


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """Counter-measured bytes per partial launch, or None when the counters were
    taken on other kernel sources (or another workload)."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="sparse90_32k")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--dense-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=2)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU sharding is "
                                   "described in DESIGN.md but not implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_attention_29_amd import seer
    from block_sparse_attention_29_amd.pipeline import DecodeState
    from workloads import WORKLOADS, make_case

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seer.load()
    DT = {"f32": torch.float32, "bf16": torch.bfloat16}[wl.dtype]

    # one case per layer: the same shape, independent draws
    states, cases = [], []
    for layer in range(args.layers):
        case = make_case(wl.with_(seed=wl.seed + 1000 * layer), dev)
        st = DecodeState(batch=wl.batch, num_q_heads=wl.num_q_heads,
                         num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim,
                         block_size=wl.block_size, max_blocks=wl.max_blocks, dtype=DT,
                         k=case.k, v=case.v, page_table=case.page_table, keep=wl.keep,
                         top_k=case.top_k)
        st.build_pool(case.lens)
        states.append(st)
        cases.append(case)
        torch.cuda.synchronize()
        print(f"[bench] layer {layer} ready", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()

    def step(i):
        st, case = states[i % args.layers], cases[i % args.layers]
        st.select(case.q, case.lens)
        seer.sparse_decode_partial(st.shape, case.q, st.kv, case.lens, st.sel_idx, st.sel_cnt,
                                   st.k_max, st.workspace)
        seer.sparse_decode_combine(st.shape, st.out, st.lse, st.workspace)

    def partial_only(i):
        st, case = states[i % args.layers], cases[i % args.layers]
        seer.sparse_decode_partial(st.shape, case.q, st.kv, case.lens, st.sel_idx, st.sel_cnt,
                                   st.k_max, st.workspace)

    def dense_step(i):
        st, case = states[i % args.layers], cases[i % args.layers]
        st.attend(case.q, case.lens, dense=True)

    def capture(fn, n):
        """One HIP graph of n consecutive calls of fn (launch gaps off the host)."""
        for i in range(min(n, 2 * args.layers)):   # eager warm-up before capture
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

    # ---- whole-step timing: K steps in one graph, W warm-up steps before ----
    g_steps = capture(step, args.steps)
    if args.warmup > 0:
        g_warm = capture(step, args.warmup)
        timed(g_warm)
    wall0 = time.perf_counter()
    ms_total = timed(g_steps)
    wall = time.perf_counter() - wall0
    ms_per_step = ms_total / args.steps
    tokens_per_s = wl.batch * args.steps / (ms_total / 1e3)

    # ---- partial-kernel timing: back-to-back launches in one graph, events
    # around it on the launch stream (selections computed beforehand) ----
    for i in range(args.layers):
        states[i].select(cases[i].q, cases[i].lens)
    n_k = max(4 * args.layers, args.steps // 2)
    g_part = capture(partial_only, n_k)
    timed(g_part)
    k_ms = timed(g_part, 3) / (3 * n_k)

    # algorithmic bytes of one partial launch (layer 0): valid K/V tokens of the
    # kept blocks (bf16 K and V rows) plus the query
    st0, case0 = states[0], cases[0]
    torch.cuda.synchronize()
    e = 2 if wl.dtype == "bf16" else 4
    S, d = wl.block_size, wl.head_dim
    sel = st0.sel_idx.cpu().numpy()
    cnt = st0.sel_cnt.cpu().numpy()
    lens = case0.lens.cpu().numpy()
    tokens = 0
    for u in range(sel.shape[0]):
        L = int(lens[u // wl.num_kv_heads])
        for j in sel[u, : cnt[u]]:
            tokens += min(S, L - int(j) * S)
    kv_bytes = tokens * d * e * 2
    q_bytes = wl.batch * wl.num_q_heads * d * e
    k_bytes = kv_bytes + q_bytes
    achieved = k_bytes / (k_ms * 1e-3) / 1e9

    # whole-step algorithmic bytes: + pooled-key table read by the gate
    pooled_bytes = int(sum(-(-int(L) // S) for L in lens)) * wl.num_kv_heads * d * 4
    step_bytes = k_bytes + pooled_bytes
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- dense decode at the same shape (speedup denominator) ----
    dense = None
    if args.dense_steps > 0:
        g_dense = capture(dense_step, args.dense_steps)
        timed(g_dense)
        dense_ms = timed(g_dense) / args.dense_steps
        dense_bytes = int(lens.sum()) * wl.num_kv_heads * d * e * 2 + q_bytes
        dense = {"ms_per_step": dense_ms,
                 "tokens_per_s": wl.batch / (dense_ms * 1e-3),
                 "hbm_gbps": dense_bytes / (dense_ms * 1e-3) / 1e9,
                 "speedup_sparse_vs_dense": dense_ms / ms_per_step}

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    print(f"[bench] gpu timing done: {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)
    # ---- CPU baseline: the fp64 oracle on a bounded sample ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, cases[0], states[0], args.cpu_sample_seqs)

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.num_q_heads,
                   "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "context": wl.context, "block_size": wl.block_size,
                   "kept_blocks": int(cnt.max()), "blocks": int(-(-wl.context // S)),
                   "layers_cycled": args.layers},
        "step_hbm_gbps": step_gbps,
        "step_pct_hbm_peak": 100.0 * step_gbps / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "kernel": "decode_partial_kernel<bf16,128,4>",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(wl.name),
                     "bytes_per_launch": k_bytes, "launch_ms": k_ms},
        "dense": dense,
        "cpu_baseline": cpu,
        "wall_s_timed_region": wall,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, case, st, n_seqs):
    """Times the fp64 oracle's gate + selection + attention for n_seqs sequences."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import seer_oracle as O

    S, d, G = wl.block_size, wl.head_dim, wl.group
    lens = case.lens.cpu().numpy()
    units = [(b, g) for b in range(n_seqs) for g in range(wl.num_kv_heads)]
    # inputs on the host, pooled tables built with the oracle (setup, untimed)
    data = {}
    for (b, g) in units:
        L = int(lens[b])
        k = case.k[b, g, :L].double().cpu().numpy()
        v = case.v[b, g, :L].double().cpu().numpy()
        p32, _, _ = O.pool_keys(k, L, S)
        qg = case.q[b, g * G:(g + 1) * G].double().cpu().numpy()
        data[(b, g)] = (k, v, p32, qg, L)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        reps = 0
        while True:
            for (b, g), (k, v, p32, qg, L) in data.items():
                s = O.gate_scores(qg, p32, d)
                n = O.block_count(L, S)
                kk = O.clamp_count(wl.top_k, n) if wl.top_k else O.keep_count(n, *wl.keep)
                sel = O.select_top_blocks(s, kk)
                toks = O.selected_tokens(sel, L, S)
                for h in range(G):
                    O.attend(qg[h], k, v, toks)
            reps += 1
            el = time.perf_counter() - t0
            if el >= 10.0 or reps >= 1000:
                break
    sec_per_step = el / reps * (wl.batch / n_seqs)   # scaled to the full batch
    return {"value": wl.batch / sec_per_step, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_seqs} of {wl.batch} sequences (all {wl.num_kv_heads} KV heads), "
                      f"gate+top-k+attention in fp64 NumPy, {reps} repetitions in {el:.1f} s, "
                      f"scaled to the full batch; pooled tables built beforehand"}


if __name__ == "__main__":
    main()
