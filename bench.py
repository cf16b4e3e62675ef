"""Benchmark of one Twilight sparse decode step on one MI355X.

A step is the whole hot path for one decode layer: Quest page selection, the int4 weight
estimate, top-p with compaction, and sparse decode over the kept tokens (the
select-then-prune pipeline of the Twilight pages, atlas.scime.ai summary "Approach").
Inputs are synthetic and already resident in HBM. To keep the 256 MB Infinity Cache and
the L2 from serving a step out of cache, consecutive steps rotate over independent layer
replicas (distinct buffers), as consecutive layers of a real decode do.

Prints ONE JSON line. `value` is candidate tokens per second: sum over (sequence, KV head)
of the candidate count, divided by the step time, with the steps of the layer replicas
captured back to back in one hipGraph as a decode loop runs them (single-step graphs are
reported beside it).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn µs/decode step & candidate tokens/s at 1 GPU; % of HBM peak"
HBM_PEAK = 8.0e12            # MI355X HBM3E, bytes/s
PAGE = 16


# the kernels behind each call of the step, in launch order
CALL_KERNELS = {
    "quest_page_scores": ("quest_score_kernel",),
    "quest_top_pages": ("quest_select_kernel",),
    "twilight_estimate_topp": ("estimate_logits_kernel", "topp_kernel"),
    "twilight_sparse_decode": ("sparse_decode_kernel", "decode_merge_kernel"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--p", type=float, default=None)
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip the dense and Quest-only comparison steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for scaling HBM "
                         "traffic counters) and exit")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, five times: HBM counters read on it give
    the factor between counter bytes and real bytes (it reads and writes COPY_BYTES)."""
    import torch
    src = torch.randint(0, 255, (COPY_BYTES,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "repeats": 5}))


def stream_bandwidth(stream, nbytes=1 << 30, repeats=5):
    """Measured HBM bandwidth of a plain device copy of `nbytes` (it reads and writes
    nbytes), timed with events on `stream`: the practical streaming ceiling that the
    roofline fraction is also reported against, beside the 8 TB/s specification."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(repeats):
            dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) * 1e-3 / repeats
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / secs


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel_call, config_id, p):
    """HBM bytes per launch of a call's kernels from the committed counter summary, or None
    when there is none, it was taken on another workload, or a kernel source changed since
    the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("config_id") != config_id or rec.get("p") is None or abs(rec["p"] - p) > 1e-9:
        return None
    entry = rec.get("calls", {}).get(kernel_call)
    if not entry:
        return None
    for src, digest in entry.get("sources", {}).items():
        path = os.path.join(ROOT, src)
        if not os.path.exists(path) or source_digest(path) != digest:
            return None
    return entry.get("bytes_per_launch")


def stage_bytes(c, buf, d):
    """Algorithmic bytes per stage (each byte the method must move counted once)."""
    import torch
    B, Hq, Hkv = c.B, c.Hq, c.Hkv
    G = Hq // Hkv
    seq = c.seq_lens.cpu().numpy().astype(np.int64)
    pages = -(-seq // PAGE)
    stride = c.cand_stride_pages
    if c.budget is not None:
        sel_count = buf.sel_count.cpu().numpy().astype(np.int64)          # [B, Hkv]
        sel = buf.sel_pages.cpu().numpy().astype(np.int64)
        cand = np.zeros((B, Hkv), np.int64)
        for b in range(B):
            for g in range(Hkv):
                pg = sel[b, g, :sel_count[b, g]]
                cand[b, g] = int(np.minimum(seq[b] - pg * PAGE, PAGE).clip(0).sum())
    else:
        sel_count = None
        cand = np.repeat(seq[:, None], Hkv, axis=1)
    kept = buf.kept_count.cpu().numpy().astype(np.int64)
    qo = B * Hq * d * 2
    out = {}
    if c.budget is not None:
        # the two halves of quest_select_pages as separate calls: bounds and q in, one fp64
        # score per page out; those scores in, the selected page ids out
        score_bytes = int(pages.sum() * Hkv * 8)
        out["quest_page_scores"] = int(pages.sum() * Hkv * (2 * d * 2) + qo + score_bytes)
        out["quest_top_pages"] = int(score_bytes + sel_count.sum() * 4)
    int4_row = d // 2 + (d // 32) * 4
    # the estimate's logits are written once and read once by the top-p
    out["twilight_estimate_topp"] = int(cand.sum() * int4_row + cand.sum() * G * 8 + qo +
                                        kept.sum() * 4)
    out["twilight_sparse_decode"] = int(kept.sum() * (2 * d * 2 + 4) + 2 * qo)
    return out, int(cand.sum()), int(kept.sum())


def time_baselines(reps, bufs, stream, steps, warmup, twilight_us):
    """Dense and Quest-only decode steps on the same kernels, timed like the Twilight step
    (the layer replicas' steps in one hipGraph): dense = twilight_sparse_decode over every
    token; Quest-only = quest_select_pages + twilight_sparse_decode over every token of the
    selected pages."""
    import torch
    import adaptive_top_sparse_amd as twl
    from adaptive_top_sparse_amd import pipeline
    out = {"twilight_us": twilight_us}
    modes = ["dense"] + (["quest"] if reps[0].budget is not None else [])
    for mode in modes:
        runs, keep = [], []
        for c, buf in zip(reps, bufs):
            kept, count, stride = pipeline.baseline_kept(c, buf, mode)
            lay = c.layout()
            ws = torch.zeros(twl.twilight_workspace_size(lay, stride // twl.PAGE_SIZE),
                             dtype=torch.uint8, device=c.q.device)
            o = torch.empty_like(buf.out)
            keep.append((kept, count, ws, o))

            def run(c=c, buf=buf, kept=kept, count=count, ws=ws, o=o, stride=stride, lay=lay):
                if mode == "quest":
                    twl.quest_select_pages(lay, c.q, c.page_minmax, c.budget, buf.sel_pages,
                                           buf.sel_count, ws, stream=stream)
                twl.twilight_sparse_decode(lay, c.q, c.k_cache, c.v_cache, kept, count, stride,
                                           pipeline.default_sm_scale(c.d), o, ws, stream=stream)
            runs.append(run)
        us = layers_us(runs, stream, steps, warmup)
        name = "dense_us" if mode == "dense" else "quest_only_us"
        out[name] = us
        out["speedup_vs_" + ("dense" if mode == "dense" else "quest")] = us / twilight_us
        del runs, keep
    out["note"] = ("same decode kernel; Quest-only token lists expanded once outside the "
                   "timed region (fixed q)")
    return out


def time_append_and_layers(reps, bufs, p, stream, steps, warmup, layers=32):
    """Two views of a real decode loop: the step with its per-token cache maintenance first
    (quantize the newest token, recompute its page's bounds), timed like the plain step (the
    layer replicas' steps in one hipGraph), and one graph of `layers` such steps over the
    rotating replicas (a whole model's attention layers), reported per layer."""
    import torch
    from adaptive_top_sparse_amd import pipeline
    R = len(reps)
    step_us = layers_us([lambda r=r: pipeline.run_step(reps[r], bufs[r], p, stream=stream,
                                                       append=True) for r in range(R)],
                        stream, steps, warmup)
    big = torch.cuda.CUDAGraph()
    with torch.cuda.graph(big, stream=stream):
        for i in range(layers):
            pipeline.run_step(reps[i % R], bufs[i % R], p, stream=stream, append=True)
    with torch.cuda.stream(stream):
        big.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_big = max(1, steps // layers)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(n_big):
            big.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    layer_us = e0.elapsed_time(e1) / (n_big * layers) * 1e3
    return {"append_step_us": step_us, "layers": layers,
            "whole_model_graph_us_per_layer": layer_us}


def time_headwise(reps, bufs, p, stream, steps, warmup):
    """The step with head-wise top-p and decode (a kept set per query head instead of one per
    KV-head group), timed like the group-wise step over the same replicas, with the kept
    token-heads of both modes (a group-wise kept token counts once per query head)."""
    from adaptive_top_sparse_amd import pipeline
    hbufs = [pipeline.alloc_step(c, headwise=True) for c in reps]
    us = layers_us([lambda c=c, hb=hb: pipeline.run_step(c, hb, p, stream=stream, headwise=True)
                    for c, hb in zip(reps, hbufs)], stream, steps, warmup)
    G = reps[0].Hq // reps[0].Hkv
    return {"headwise_step_us": us,
            "kept_token_heads_headwise": int(hbufs[0].kept_count.sum().item()),
            "kept_token_heads_groupwise": int(bufs[0].kept_count.sum().item()) * G}


def layers_us(runs, stream, steps, warmup):
    """Device time per step of `runs` (one callable per layer replica, each enqueueing one
    step on `stream`), captured back to back in one hipGraph as a decode loop runs them and
    replayed until about `steps` steps have run."""
    import torch
    with torch.cuda.stream(stream):
        for run in runs:
            run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for run in runs:
            run()
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup // len(runs))):
            g.replay()
    torch.cuda.synchronize()
    n = max(1, steps // len(runs))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(n):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (n * len(runs)) * 1e3


def time_two_bit(w, p, stream, steps, warmup, replicas, buf4):
    """The 2-bit key cache the pages ablate (4-bit keeps the estimated weights more stable):
    the step on its own layer replicas (timed like the 4-bit step), and the stability of
    both widths' kept sets on the first replica, measured against the exact weights
    (softmax of q.k on the fp16 keys over the same candidates, fp64, group mean): the exact
    mass each kept set captures (p is the target) and the overlap of the two sets."""
    import torch
    from adaptive_top_sparse_amd import pipeline
    s = w.spec
    base = pipeline.upload(w, key_bits=2)
    base.build_caches()
    torch.cuda.synchronize()
    # replicas while they fit beside the 4-bit ones (two already defeat the 256 MB
    # Infinity Cache when a layer's caches are larger than it)
    rep_bytes = sum(t.numel() * t.element_size() for t in vars(base).values()
                    if isinstance(t, torch.Tensor))
    fit = int(torch.cuda.mem_get_info()[0] * 0.6 // max(1, rep_bytes))
    replicas = max(2, min(replicas, fit + 1))
    reps = [base] + [base.clone() for _ in range(replicas - 1)]
    bufs = [pipeline.alloc_step(r) for r in reps]
    us = layers_us([lambda c=c, b=b: pipeline.run_step(c, b, p, stream=stream)
                    for c, b in zip(reps, bufs)], stream, steps, warmup)
    k2, c2 = bufs[0].kept.cpu().numpy(), bufs[0].kept_count.cpu().numpy()
    k4, c4 = buf4.kept.cpu().numpy(), buf4.kept_count.cpu().numpy()
    sel = None if buf4.sel_pages is None else buf4.sel_pages.cpu().numpy()
    sel_n = None if buf4.sel_count is None else buf4.sel_count.cpu().numpy()
    del bufs, reps, base
    torch.cuda.empty_cache()
    G = s.G
    sm = pipeline.default_sm_scale(s.d)
    m2, m4, jac = [], [], []
    for b in range(s.B):
        n = int(w.seq_lens[b])
        if n == 0:
            continue
        for g in range(s.Hkv):
            if sel is None:
                toks = np.arange(n)
            else:
                pages = sel[b, g, :sel_n[b, g]].astype(np.int64)
                toks = (pages[:, None] * 16 + np.arange(16)).reshape(-1)
                toks = toks[toks < n]
            q = w.q[b, g * G:(g + 1) * G].astype(np.float64)
            lg = float(sm) * (q @ w.k[b][g][toks].astype(np.float64).T)
            e = np.exp(lg - lg.max(1, keepdims=True))
            Wx = (e / e.sum(1, keepdims=True)).mean(0)
            a = k2[b, g, :c2[b, g]]
            c = k4[b, g, :c4[b, g]]
            m2.append(float(Wx[np.searchsorted(toks, a)].sum()))
            m4.append(float(Wx[np.searchsorted(toks, c)].sum()))
            jac.append(len(np.intersect1d(a, c)) / max(1, len(np.union1d(a, c))))
    return {"step_us": us, "layer_replicas": replicas,
            "estimate_bytes_per_token": s.d // 4 + (s.d // 32) * 4,
            "kept_2bit": int(c2.sum()), "kept_4bit": int(c4.sum()),
            "exact_mass_kept_2bit": float(np.mean(m2)), "exact_mass_kept_4bit": float(np.mean(m4)),
            "exact_mass_kept_2bit_min": float(np.min(m2)),
            "exact_mass_kept_4bit_min": float(np.min(m4)),
            "kept_set_jaccard_2bit_vs_4bit": float(np.mean(jac))}


def cpu_info():
    """Host CPU model name and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return model, usable


def _oracle_unit_prep(w, units):
    """Per (sequence, KV head) unit, the quantized keys and page bounds the step reads
    (cache maintenance, done before timing, as on the GPU)."""
    import oracle
    prep = {}
    for b, g in units:
        k = w.k[b][g]
        codes, scale, zero = oracle.quantize_keys(k)
        lo, hi = oracle.page_bounds(k) if w.budget is not None else (None, None)
        prep[(b, g)] = (codes, scale, zero, lo, hi)
    return prep


def _oracle_unit_step(w, p, b, g, prep, sm):
    """One unit of a decode step in the oracle: Quest select, estimate, top-p, attention.
    Returns its candidate count."""
    import oracle
    G = w.spec.G
    codes, scale, zero, lo, hi = prep
    qg = w.q[b, g * G:(g + 1) * G]
    n = int(w.seq_lens[b])
    if n == 0:
        return 0
    if w.budget is not None:
        sel = oracle.quest_select(qg, lo, hi, w.budget)
        n_slots = w.budget * PAGE
        tok = np.repeat(sel.astype(np.int64), PAGE) * PAGE + np.tile(np.arange(PAGE), len(sel))
        valid = np.zeros(n_slots, bool)
        valid[:tok.size] = tok < n
    else:
        sel = None
        n_slots = -(-n // PAGE) * PAGE
        valid = np.arange(n_slots) < n
    wts = oracle.estimate_weights(qg, codes, scale, zero, n, sel, n_slots, sm)
    kept, _ = oracle.topp_select(wts, valid, p, sel)
    oracle.sparse_attention(qg, w.k[b][g], w.v[b][g], kept, sm)
    return int(valid.sum())


def cpu_baseline(w, p, seconds, max_threads=16):
    """The fp64 oracle on whole decode steps of the same workload (every (sequence, KV head)
    unit of the step: Quest select, estimate, top-p, attention; the cache is quantized
    beforehand, as on the GPU), timed on the host cores, first single-threaded, then with
    one thread per unit across the cores this process may use (at most `max_threads`; the
    oracle's C functions release the interpreter lock, so the threads run in parallel).
    Each variant repeats whole steps until `seconds` have passed (at least one step); on
    the large batched workloads a bounded sample of the step's units is timed instead, as
    the sample field says."""
    import concurrent.futures
    s = w.spec
    sm = float(np.float32(1.0 / math.sqrt(s.d)))
    model, usable = cpu_info()
    units = [(b, g) for b in range(s.B) for g in range(s.Hkv)]
    # about one second of single-threaded work per unit sample keeps the default run short
    sample = units
    if len(units) > 64:
        rng = np.random.default_rng(0)
        sample = [units[i] for i in sorted(rng.choice(len(units), 64, replace=False))]
    # one unit per thread at a time: more threads than units would sit idle
    threads = max(1, min(max_threads, usable, len(sample)))
    prep = _oracle_unit_prep(w, sample)

    def one_step(pool):
        if pool is None:
            return sum(_oracle_unit_step(w, p, b, g, prep[(b, g)], sm) for b, g in sample)
        futs = [pool.submit(_oracle_unit_step, w, p, b, g, prep[(b, g)], sm) for b, g in sample]
        return sum(f.result() for f in futs)

    res = {}
    for name, nthr in (("single", 1), ("multi", threads)):
        pool = concurrent.futures.ThreadPoolExecutor(nthr) if nthr > 1 else None
        cand, steps = 0, 0
        t0 = time.perf_counter()
        while True:
            cand += one_step(pool)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds / 2:
                break
        if pool is not None:
            pool.shutdown()
        res[name] = {"value": cand / el, "threads": nthr, "steps": steps, "seconds": el,
                     "step_ms": el / steps * 1e3}
    scope = ("every (sequence, KV head) unit of the step" if sample is units else
             f"{len(sample)} of the step's {len(units)} (sequence, KV head) units, seeded choice")
    return {"value": res["multi"]["value"], "unit": "candidate tokens/s",
            "cores": res["multi"]["threads"], "kind": "oracle",
            "sample": f"{res['multi']['steps']} passes over {scope} (Quest select, estimate, "
                      f"top-p, attention), fp64 oracle, one thread per unit on "
                      f"{res['multi']['threads']} threads, {res['multi']['seconds']:.1f} s; "
                      f"cache quantization excluded",
            "single_thread": {"value": res["single"]["value"], "cores": 1,
                              "steps": res["single"]["steps"],
                              "step_ms": res["single"]["step_ms"]},
            "multi_thread_step_ms": res["multi"]["step_ms"],
            "cpu_model": model, "usable_cores": usable, "units_per_step": len(sample)}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the hot path "
              "is a single-GPU kernel library with no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import adaptive_top_sparse_amd as twl
    from adaptive_top_sparse_amd import pipeline, workloads

    torch.cuda.set_device(0)
    spec = workloads.SPECS[args.config]
    p = args.p if args.p is not None else spec.ps[len(spec.ps) // 2]
    t_gen = time.perf_counter()
    w = workloads.make_workload(args.config)
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] generated config {args.config} ({spec.name}) in {t_gen:.1f} s", file=sys.stderr,
          flush=True)
    base = pipeline.upload(w)
    stream = torch.cuda.Stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # cache maintenance (prefill-time quantization and page bounds), timed once
    with torch.cuda.stream(stream):
        ev0.record(stream)
        base.build_caches(stream=stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    build_ms = ev0.elapsed_time(ev1)
    reps = [base] + [base.clone() for _ in range(args.replicas - 1)]
    bufs = [pipeline.alloc_step(r) for r in reps]
    torch.cuda.synchronize()
    print(f"[bench] {len(reps)} layer replicas resident; warming up", file=sys.stderr, flush=True)

    def step(i):
        pipeline.run_step(reps[i % len(reps)], bufs[i % len(reps)], p, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    # plain launches, with events around every ABI call to time the stages: the Quest
    # selector as its two halves (page scores, then top pages; the step's single
    # quest_select_pages call runs the same two kernels), the fused estimate + top-p as one
    names = (["quest_page_scores", "quest_top_pages"] if base.budget is not None else []) + [
        "twilight_estimate_topp", "twilight_sparse_decode"]
    stage_map = {"quest_page_scores": ("quest_scores",), "quest_top_pages": ("quest_top",),
                 "twilight_estimate_topp": ("estimate", "topp"),
                 "twilight_sparse_decode": ("decode",)}
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_plain0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            r = i % len(reps)
            evs[i][0].record(stream)
            for j, nm in enumerate(names):
                pipeline.run_step(reps[r], bufs[r], p, stream=stream, stages=stage_map[nm])
                evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    t_plain = (time.perf_counter() - t_plain0) / args.steps
    stage_ms = {nm: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
                for j, nm in enumerate(names)}
    plain_ms = float(np.mean([evs[i][0].elapsed_time(evs[i][-1]) for i in range(args.steps)]))

    # each call alone: one graph of back-to-back launches over the replicas, captured in step
    # order (so every call reads what the previous call of its replica wrote), replayed
    # between two events; this is the per-launch duration the roofline uses (plain launches
    # above leave the GPU waiting on the host between calls)
    call_ms = {}
    for nm in names:
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg, stream=stream):
            for r in range(len(reps)):
                pipeline.run_step(reps[r], bufs[r], p, stream=stream, stages=stage_map[nm])
        with torch.cuda.stream(stream):
            cg.replay()
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_rep = max(1, args.steps // len(reps))
        with torch.cuda.stream(stream):
            c0.record(stream)
            for _ in range(n_rep):
                cg.replay()
            c1.record(stream)
        torch.cuda.synchronize()
        call_ms[nm] = c0.elapsed_time(c1) / (n_rep * len(reps))
        del cg

    # hipGraph, as a decode loop runs the path: the steps of all R layer replicas captured
    # back to back in one graph (the way a model's whole decode step is captured), so that
    # the time is the stages' device time and not R graph launches. K steps are K // R
    # replays of it and K % R single-step graphs (one captured step per replica, replayed in
    # rotation, also timed alone below).
    R = len(reps)
    graphs = []
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            pipeline.run_step(reps[r], bufs[r], p, stream=stream)
        graphs.append(g)
    layers = torch.cuda.CUDAGraph()
    with torch.cuda.graph(layers, stream=stream):
        for r in range(R):
            pipeline.run_step(reps[r], bufs[r], p, stream=stream)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            graphs[i % R].replay()
        layers.replay()
    torch.cuda.synchronize()
    n_layers, n_rest = divmod(args.steps, R)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g0.record(stream)
        for _ in range(n_layers):
            layers.replay()
        for i in range(n_rest):
            graphs[i].replay()
        g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / args.steps

    # one graph launch per step: the same steps, each its own graph
    with torch.cuda.stream(stream):
        g0.record(stream)
        for i in range(args.steps):
            graphs[i % R].replay()
        g1.record(stream)
    torch.cuda.synchronize()
    single_graph_ms = g0.elapsed_time(g1) / args.steps

    # the distribution of step times: one event between consecutive R-step replays (each
    # replay's time over R), and one between consecutive single-step replays (each recorded
    # event adds a little to the step it closes)
    n_dist = max(20, args.steps // R)
    lev = [torch.cuda.Event(enable_timing=True) for _ in range(n_dist + 1)]
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with torch.cuda.stream(stream):
        lev[0].record(stream)
        for i in range(n_dist):
            layers.replay()
            lev[i + 1].record(stream)
        sev[0].record(stream)
        for i in range(args.steps):
            graphs[i % R].replay()
            sev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step_us = np.array([lev[i].elapsed_time(lev[i + 1]) * 1e3 / R for i in range(n_dist)])
    per_single_us = np.array([sev[i].elapsed_time(sev[i + 1]) * 1e3 for i in range(args.steps)])
    del layers

    # the pruner and the sparse decode (stages a2-a5) alone, on the selection the step made:
    # one graph of the fused estimate + top-p call and the decode call for every replica in
    # turn (back-to-back launches, as each call alone is timed above)
    a25 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(a25, stream=stream):
        for r in range(len(reps)):
            pipeline.run_step(reps[r], bufs[r], p, stream=stream,
                              stages=("estimate", "topp", "decode"))
    with torch.cuda.stream(stream):
        a25.replay()
    torch.cuda.synchronize()
    n_rep = max(1, args.steps // len(reps))
    with torch.cuda.stream(stream):
        g0.record(stream)
        for _ in range(n_rep):
            a25.replay()
        g1.record(stream)
    torch.cuda.synchronize()
    a25_ms = g0.elapsed_time(g1) / (n_rep * len(reps))
    del a25

    per_stage_bytes, cand, kept = stage_bytes(base, bufs[0], base.d)
    step_bytes = sum(per_stage_bytes.values())
    stream_bw = stream_bandwidth(stream)

    def roof(call):
        achieved = per_stage_bytes[call] / (call_ms[call] * 1e-3)
        return {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": achieved / HBM_PEAK,
                "traffic": measured_traffic(call, args.config, p), "kernel": call,
                "kernels": list(CALL_KERNELS[call]),
                "bytes_per_launch": per_stage_bytes[call], "avg_launch_us": call_ms[call] * 1e3,
                "measured_stream": stream_bw / 1e9,
                "frac_of_measured_stream": achieved / stream_bw}

    # the roofline is reported for the call that takes the most device time per step (each
    # call of the step timed alone, as back-to-back launches in a graph), and for the Quest
    # page scorer, the kernel that moves the most bytes, when the workload has one
    dom = max(call_ms, key=lambda k: call_ms[k])
    roofline = roof(dom)
    roofline["chosen_by"] = "device time per step"
    a25_bytes = per_stage_bytes["twilight_estimate_topp"] + per_stage_bytes["twilight_sparse_decode"]
    a25_rate = a25_bytes / (a25_ms * 1e-3)
    step_s = graph_ms * 1e-3
    res = {
        "metric": METRIC,
        "value": cand / step_s,
        "unit": "candidate tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": graph_ms,
        "us_per_step": graph_ms * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}: B={spec.B}, Hq={spec.Hq}, Hkv={spec.Hkv}, "
                               f"head_dim={spec.d}, n={spec.n or spec.n_range}, "
                               f"Quest budget={w.budget} pages, p={p}",
                   "config_id": args.config, "p": p, "layer_replicas": len(reps),
                   "launch": f"hipGraph of {len(reps)} steps, one per layer replica"},
        "step_us_median": float(np.median(per_step_us)),
        "step_us_p90": float(np.percentile(per_step_us, 90)),
        "single_step_graph": {
            "us_per_step": single_graph_ms * 1e3,
            "us_median": float(np.median(per_single_us)),
            "us_p90": float(np.percentile(per_single_us, 90)),
            "note": "one graph launch per step; the difference to us_per_step is graph-launch "
                    "time between steps, not stage device time"},
        "hbm_frac_step": step_bytes / step_s / HBM_PEAK,
        "step_bytes": step_bytes,
        "pruner_and_decode": {
            "stages": "estimate + top-p + compaction + sparse decode (a2-a5)",
            "calls": ["twilight_estimate_topp", "twilight_sparse_decode"],
            "us": a25_ms * 1e3, "bytes": a25_bytes, "achieved_GBps": a25_rate / 1e9,
            "frac": a25_rate / HBM_PEAK, "frac_of_measured_stream": a25_rate / stream_bw,
            "us_at_70pct_of_peak": a25_bytes / (0.7 * HBM_PEAK) * 1e6},
        "roofline_scorer": roof("quest_page_scores") if "quest_page_scores" in call_ms else None,
        "candidates": cand,
        "kept": kept,
        "plain_launch_us_per_step": plain_ms * 1e3,
        "host_us_per_plain_step": t_plain * 1e6,
        "stage_us_plain": {k: v * 1e3 for k, v in stage_ms.items()},
        "call_us_graph": {k: v * 1e3 for k, v in call_ms.items()},
        "stage_bytes": per_stage_bytes,
        "cache_build_ms": build_ms,
        "roofline": roofline,
        "baselines": None,
        "decode_loop": None,
        "headwise": None,
        "key_bits_2": None,
        "cpu_baseline": None,
    }
    if not args.no_baselines:
        print("[bench] timing the dense and Quest-only steps", file=sys.stderr, flush=True)
        res["baselines"] = time_baselines(reps, bufs, stream, args.steps, args.warmup,
                                          graph_ms * 1e3)
        print("[bench] timing the step with per-token cache maintenance", file=sys.stderr,
              flush=True)
        res["decode_loop"] = time_append_and_layers(reps, bufs, p, stream, args.steps,
                                                    args.warmup)
        if reps[0].Hq != reps[0].Hkv:
            print("[bench] timing the head-wise step", file=sys.stderr, flush=True)
            res["headwise"] = time_headwise(reps, bufs, p, stream, args.steps, args.warmup)
        print("[bench] timing the 2-bit key cache variant", file=sys.stderr, flush=True)
        res["key_bits_2"] = time_two_bit(w, p, stream, args.steps, args.warmup, len(reps),
                                         bufs[0])
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, p, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
