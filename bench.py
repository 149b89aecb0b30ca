#!/usr/bin/env python3
"""Throughput of the DSA path (indexer -> top-k -> sparse MQA attention) on one
MI355X, printed as one JSON line.

A step is one dsa_forward call over one batch of synthetic inputs already
resident in HBM. The default workload is the 128K-context decode batch:
64 sequences x 131072 keys, indexer dim 128 in fp8 e4m3fn with clustered
keys, top_k 2048, 16 query heads on one shared K/V set. value = queries/s.

The roofline object covers the slowest of the three stages, timed alone with
HIP events on the stream it runs on; cpu_baseline times the CPU oracle on a
bounded sample of the same inputs (rank 0, one GPU only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"hbm": 8000.0, "fp8": 5000.0, "bf16": 2500.0}  # GB/s, TFLOP/s (dense)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Sources of the kernels behind each stage (decode rows use decode.hip's
# threshold / filter / select kernels).
KERNEL_SOURCES = {
    ("prefill", "indexer"): ["prefill.hip", "frag.h"],
    ("prefill", "topk"): ["prefill.hip", "topk_common.h"],
    ("prefill", "attn"): ["attn.hip"],
    ("decode", "indexer"): ["decode.hip", "frag.h"],
    ("decode", "topk"): ["decode.hip", "topk_common.h"],
    ("decode", "attn"): ["attn.hip"],
    ("prefill", "project"): ["project.hip"],
    ("decode", "project"): ["project.hip"],
}


def source_hash(mode, stage):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[(mode, stage)]:
        with open(os.path.join(ROOT, "dsa_top_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stage_work(w, stage, seed=0):
    """Algorithmic work of one launch of `stage` on workload w:
    (bound, amount, unit, peak)."""
    es = 1 if w.idx_dtype == "fp8" else 2
    if stage == "project":
        # read the hidden rows once per projection and both weights, write the
        # q rows and the new k rows
        rows = w.batch * w.n_q
        b = 2 * rows * w.d_model * 2 + 2 * w.d_idx * w.d_model * 2 + 2 * rows * w.d_idx * es
        return "hbm", b / 1e9, "GB/s", PEAK["hbm"]
    pairs = w.n_causal_pairs(seed)
    if stage == "indexer":
        if w.mode == "decode":
            # stream the indexer row of every key in a query's range once
            # (+ the query rows)
            b = pairs * w.d_idx * es + w.batch * w.n_q * w.d_idx * es
            return "hbm", b / 1e9, "GB/s", PEAK["hbm"]
        f = 2.0 * w.d_idx * pairs
        return "mfma", f / 1e12, "TFLOP/s", PEAK[w.idx_dtype]
    if stage == "topk":
        # read each candidate score once, write the index lists
        b = 4 * pairs + 4 * w.batch * w.n_q * w.top_k
        return "hbm", b / 1e9, "GB/s", PEAK["hbm"]
    if w.mode == "prefill":
        # many causal rows over a K/V table of tens of MB that the key-range
        # schedule keeps in the L2s: the gathered bytes are mostly cache hits,
        # so the roofline is the bf16 MFMA work, 2 x 2 x 128 flop per (selected
        # key, head) for Q.K and P.V
        f = 4.0 * 128 * w.n_selected(seed) * w.n_heads
        return "mfma", f / 1e12, "TFLOP/s", PEAK["bf16"]
    # attention: gather each selected K and V row once, read Q, write O
    b = w.n_selected(seed) * 2 * 128 * 2 + 2 * w.batch * w.n_q * w.n_heads * 128 * 2
    return "hbm", b / 1e9, "GB/s", PEAK["hbm"]


def gather_bytes(w, seed=0):
    """Algorithmic K/V gather bytes of one step (each selected row once)."""
    return w.n_selected(seed) * 2 * 128 * 2


def calib_copy(nbytes=1 << 30, reps=5):
    """A plain device copy of known size (for scaling PMC byte counters)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": nbytes, "reps": reps}))


def project_oracle(oracle, x, wname, r0, r1, w):
    """The oracle's indexer projection of hidden rows [r0, r1) with weight
    x[wname], as a torch fp8 / bf16 tensor [r1 - r0, d_idx]."""
    import torch
    dt = "fp8" if w.idx_dtype == "fp8" else "bf16"
    raw = oracle.index_project(x["X"][r0:r1], x[wname], dt)
    tdt = torch.float8_e4m3fn if dt == "fp8" else torch.bfloat16
    return torch.from_numpy(raw.view(np.uint8 if dt == "fp8" else np.int16)).view(tdt)


def cpu_baseline(w, x, target_s=12.0, seed=0):
    """Time the oracle on a bounded sample of the workload's queries."""
    import oracle
    if w.mode == "decode":
        # one decode row per sequence: sample sequences
        pos = w.positions(seed)

        def run(nseq):
            if not w.ragged:
                xs = {k: v[:nseq] for k, v in x.items()}
                q_idx, k_idx = xs["q_idx"], xs["k_idx"]
                if w.d_model:
                    # the front-end: each sequence's query and its new key row
                    q_idx = project_oracle(oracle, x, "W_q", 0, nseq, w).reshape(nseq, 1, -1)
                    k_idx = k_idx.clone()
                    k_idx[:, w.q_pos0] = project_oracle(oracle, x, "W_k", 0, nseq, w)
                oracle.forward(q_idx, k_idx, xs["Q"], xs["K"], xs["V"], w.q_pos0, w.top_k,
                               tau=w.tau)
                return nseq
            xs = {k: v[:nseq] for k, v in x.items()}  # each sequence at its own position
            oracle.forward(xs["q_idx"], xs["k_idx"], xs["Q"], xs["K"], xs["V"], 0, w.top_k,
                           seq_pos=pos[:nseq])
            return nseq
        nthreads = oracle.num_threads()
        probe = min(w.batch, nthreads)
        t0 = time.perf_counter()
        run(probe)
        tp = time.perf_counter() - t0
        n = probe
        if tp < target_s:
            n = int(min(w.batch, max(probe, probe * target_s / max(tp, 1e-3))))
            n = max(probe, n // probe * probe)
        # a whole batch that runs faster than the target is run again (at
        # most 64 passes) so that the rate rests on seconds of CPU work
        t0 = time.perf_counter()
        q, reps = 0, 0
        while True:
            q += run(n)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= target_s or reps >= 64:
                break
        sample = "%d of %d sequences (one decode query each), all stages, %d pass%s" % (
            n, w.batch, reps, "" if reps == 1 else "es")
    else:
        # prefill: groups of query rows at 64 strided positions; further
        # sweeps (at most 16) start at other offsets until target_s is timed
        nthreads = oracle.num_threads()
        step = max(1, w.n_q // 64)
        t0 = time.perf_counter()
        q, sweeps, done = 0, 0, False
        for off in range(0, step, max(1, step // 16)):
            sweeps += 1
            for r in range(off, w.n_q, step):
                r1 = min(r + nthreads, w.n_q)
                if w.d_model:
                    # the front-end's work per query: its own q and k rows
                    project_oracle(oracle, x, "W_q", r, r1, w)
                    project_oracle(oracle, x, "W_k", r, r1, w)
                oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], w.q_pos0,
                               w.top_k, r, r1, tau=w.tau)
                q += r1 - r
                if time.perf_counter() - t0 > target_s:
                    done = True
                    break
            if done or sweeps >= 16:
                break
        dt = time.perf_counter() - t0
        sample = ("%d query rows (of the prefill's %d; repeats counted) in %d strided sweep%s, "
                  "all stages" % (q, w.n_q, sweeps, "" if sweeps == 1 else "s"))
    return {"value": q / dt, "unit": "queries/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample, "seconds": round(dt, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_128k_clustered")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tau", type=float, default=None,
                    help="threshold-mode selection at this tau (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true",
                    help="skip the per-stage timing loops")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timing (1 GiB flush before each step)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (PMC byte scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU only: this path runs on a single "
                         "MI355X with no sharding or collectives (asked for %d GPUs)\n"
                         % max(args.gpus, world))
        sys.exit(2)

    import torch
    if args.calib_copy:
        calib_copy()
        return

    import dsa_top_token_amd as dsa
    from dsa_top_token_amd import synth

    w = synth.WORKLOADS[args.workload]
    if args.tau is not None:
        w = w.replace(tau=args.tau)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = synth.make_inputs(w, seed=args.seed)  # canonical CPU draw
    d = {k: v.to(dev) for k, v in x.items()}
    p = dsa.make_problem(w.batch, w.n_q, w.n_k, w.q_pos0, w.d_idx, w.idx_dtype, w.top_k,
                         w.n_heads)
    fwd = dsa.Forward(p, dev)
    # a ragged batch: each sequence's query position (device int32 [B])
    sp = (torch.tensor(w.positions(args.seed), dtype=torch.int32, device=dev)
          if w.ragged else None)
    pages = None
    if w.page_size:
        # k_idx, K and V moved into shuffled page pools (on the device)
        table, n_pages = w.page_pool(args.seed)
        per = w.n_k // w.page_size
        perm = table.reshape(-1).to(dev).long()
        for name in ("k_idx", "K", "V"):
            t = d[name]
            pool = torch.zeros((n_pages, w.page_size) + tuple(t.shape[2:]), dtype=t.dtype,
                               device=dev)
            pool[perm] = t.reshape((w.batch * per, w.page_size) + tuple(t.shape[2:]))
            d[name] = pool
        d["table"] = table.to(dev)
        pages = dsa.make_pages(d["table"], w.page_size, n_pages)
    O = torch.empty_like(d["Q"])
    idx = torch.empty((w.batch, w.n_q, w.top_k), dtype=torch.int32, device=dev)
    lse = torch.empty((w.batch, w.n_q, w.n_heads), dtype=torch.float32, device=dev)

    project = None
    if w.d_model:
        if w.ragged or w.page_size:
            raise SystemExit("the projection front-end runs on the contiguous layout")
        # the indexer projection front-end: q_idx from every query row's hidden
        # state; k_idx rows for the same tokens (decode: appended at each
        # sequence's position; prefill: every key row)
        rows = w.batch * w.n_q
        proj = dsa.Projection(rows, w.d_model, w.d_idx, dev)
        q_flat = d["q_idx"].view(rows, w.d_idx)
        k_flat = d["k_idx"].view(w.batch * w.n_k, w.d_idx)
        krows = None
        if w.mode == "decode":
            krows = torch.tensor([b * w.n_k + p for b, p in enumerate(w.positions(args.seed))],
                                 dtype=torch.int32, device=dev)

        def project():
            proj(d["X"], d["W_q"], q_flat)
            proj(d["X"], d["W_k"], k_flat, krows)

    def step():
        if project:
            project()
        fwd(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], O, idx, lse, seq_pos=sp, pages=pages,
            tau=w.tau)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    queries = w.batch * w.n_q
    value = queries / (ms / 1e3)

    # The same steps from a cold cache: a 1 GiB buffer (four times the
    # 256 MB MALL) is written before each step, and HIP events on the step's
    # stream time the step alone. Back-to-back steps over an input set under
    # 1 GiB (decode_32k: 100 MB of k_idx) can be served from the MALL.
    cold = None
    if not args.no_cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evs:
            flush.fill_(1)
            e0.record()
            step()
            e1.record()
        torch.cuda.synchronize()
        cms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
        cold = {"ms_per_step": round(cms, 4), "value": round(queries / (cms / 1e3), 2),
                "protocol": "1 GiB buffer written before each step; step timed with HIP events"}
        del flush

    # Per-stage device time of the same forward call, from HIP events that
    # dsa_forward_timed records on this stream between the stage kernels.
    stages = {}
    roof = None
    if not args.no_stages:
        names = ("indexer", "topk", "attn")
        tot = [0.0, 0.0, 0.0]
        n_rep = max(3, args.steps)
        slabs = 1
        for _ in range(n_rep):
            ms3, slabs = fwd.timed(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], O, idx, lse,
                                   seq_pos=sp, pages=pages, tau=w.tau)
            tot = [a + b for a, b in zip(tot, ms3)]
        stages = {n: t / n_rep for n, t in zip(names, tot)}
        if project:
            # the projections run on torch's current stream: time them with its events
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n_rep):
                project()
            e1.record()
            e1.synchronize()
            stages["project"] = e0.elapsed_time(e1) / n_rep
        dom = max(stages, key=stages.get)
        bound, amount, unit, peak = stage_work(w, dom, args.seed)
        achieved = amount / (stages[dom] / 1e3)
        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            rec = json.load(open(TRAFFIC_FILE)).get("%s/%s" % (w.name, dom))
            if rec and rec.get("source_sha256_16") == source_hash(w.mode, dom):
                traffic = rec.get("bytes_per_step")
        roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                "stage_ms": round(stages[dom], 4), "launches_per_step": slabs}
        if dom == "attn":
            # context: the gather rate of the selected K/V rows (cache hits count)
            roof["gather_GBps"] = round(gather_bytes(w, args.seed) / 1e9 / (stages[dom] / 1e3), 1)
        if "indexer" in stages and w.mode == "prefill":
            ib, ia, iu, ip = stage_work(w, "indexer", args.seed)
            tk = stages["indexer"] + stages.get("topk", 0.0)
            roof["indexer_mfma"] = {"achieved": round(ia / (stages["indexer"] / 1e3), 2),
                                    "with_topk": round(ia / (tk / 1e3), 2), "peak": ip,
                                    "unit": iu, "frac": round(ia / (stages["indexer"] / 1e3) / ip, 4),
                                    "frac_with_topk": round(ia / (tk / 1e3) / ip, 4)}

    # Selection statistics of the last forward call (the last slab's rows for
    # a many-row problem): how many candidates the sampled threshold let
    # through, and how many rows a fallback recomputed.
    sel = None
    try:
        st = dsa.selection_stats(p, fwd.ws, fwd.ws_bytes, sp)
        if st[0] > 0 and st[1] >= 0:
            sel = {"rows": st[0], "mean_candidates": round(st[1] / st[0], 1),
                   "candidates_per_top_k": round(st[1] / st[0] / w.top_k, 3),
                   "fallback_rows": st[2], "overflow_rows": st[3]}
    except Exception as exc:  # statistics are diagnostics; never fail the bench
        sel = {"error": str(exc)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, x, seed=args.seed)

    out = {
        "metric": "queries/sec (indexer+top-k+sparse attn) at 128K ctx; % of fp8 MFMA / HBM peak",
        "value": round(value, 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8" if w.idx_dtype == "fp8" else "bf16") + "+bf16",
        "data": "synthetic (seeded integer indexer inputs, N(0,1) bf16 Q/K/V)",
        "config": {"workload": w.name, "mode": w.mode, "batch": w.batch, "n_q": w.n_q,
                   "n_k": w.n_k, "d_idx": w.d_idx, "idx_dtype": w.idx_dtype,
                   "top_k": w.top_k, "n_heads": w.n_heads, "clustered_keys": w.clustered,
                   "parallelism": "single GPU"},
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "roofline": roof,
        "cold_cache": cold,
        "selection": sel,
        "cpu_baseline": cpu,
    }
    if w.ragged:
        pos = w.positions(args.seed)
        out["config"]["ragged"] = {"positions": "seeded, uniform in [n_k/8, n_k-1]",
                                   "mean_len": round(sum(p + 1 for p in pos) / len(pos), 1)}
    if w.d_model:
        out["config"]["projection"] = {"d_model": w.d_model, "front_end": "q_idx and new k_idx "
                                       "rows projected from bf16 hidden states each step"}
        out["data"] += "; integer hidden states and sparse {-1,0,1} projection weights"
    if w.tau is not None:
        kept = (idx >= 0).sum(-1).float()
        out["config"]["threshold"] = {"tau": w.tau, "kept_mean": round(float(kept.mean()), 1),
                                      "kept_min": int(kept.min()), "kept_max": int(kept.max())}
    if w.page_size:
        out["config"]["paged"] = {"page_size": w.page_size, "pool": "shuffled, 16 spare pages"}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
