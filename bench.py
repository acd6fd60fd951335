"""Benchmark of the CommunityKV decode hot path on one MI355X.

A step is one pass of the whole path -- centroid scoring, budgeted selection with
sinks and compaction, sparse attention, local update -- for every sequence of the
batch (and every layer for the 36-layer ragged workload).  Default workload: one
Qwen3-8B-shaped attention layer, 4 sequences x 131072 tokens, 32 query / 8 KV
heads, d = 128, bf16 K/V, query-group graphs with ~2048 communities per KV head,
budget 4096 tokens + 4 sinks.

Timing protocol (cold): before every timed step the script reads through a
1 GiB scrub buffer (a reduction, so the caches end up holding clean scrub data)
so that neither the 4 MB L2s nor the 256 MB MALL hold the previous step's
centroids, lists or KV rows; the step itself is bracketed by HIP events on the
stream the kernels run on (launch gaps included), and each kernel carries its own
start / stop events bound to its execution.  `value` = tokens (decode tokens of
all sequences) / sum of the bracketed step times; the roofline uses the bound
kernel duration.  `--warm` drops the scrub (back-to-back steps); without it a
short back-to-back pass follows the cold passes and is reported as `warm`.
Inputs are resident in HBM before timing starts.

Besides the step, one run also reports: the dense baseline on the same cache,
the centroid rebuild and drift, the graph-granularity sweep (group, per query
head, per layer: step time and graph memory), the prefill edge kernel against
the bf16 MFMA peak, and the fp64 oracle on the host cores (all threads and one).

Prints ONE JSON line.  `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_long_context_centroid_amd import binding as Bd  # noqa: E402
from sparse_long_context_centroid_amd import inputs as I  # noqa: E402

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(layer: Bd.DecodeLayer, idx_len: np.ndarray, elem: int):
    """Algorithmic bytes of one step of one layer, per kernel: what the method has
    to move (centroids, scores, member/index lists, the selected K/V rows -- for
    per-head graphs the union of the rows of a KV head's lists -- q and out, the
    candidate centroids and the appended row); workspace partials not counted."""
    d = layer.d
    cd = layer.cdim                       # centroid row: d, or Hkv*d for the layer graph
    C = int(layer.num_comms_host.sum())
    Bq = layer.B * layer.Hq * d * elem
    score = C * (cd * 4 + 4 + 4) + Bq
    ntok = int(idx_len.sum())
    select = C * (4 + 4) + ntok * (4 + 4)
    if layer.gpk > 1:
        lists = layer.index_list.cpu().numpy()
        rows = 0
        for kv in range(layer.B * layer.Hkv):
            gs = range(kv * layer.gpk, (kv + 1) * layer.gpk)
            rows += len(np.unique(np.concatenate([lists[g, :idx_len[g]] for g in gs])))
        entries = ntok
    elif layer.gpk == 0:
        rows = entries = ntok * layer.Hkv  # every KV head reads the layer's one list
    else:
        rows = entries = ntok
    attn = rows * 2 * d * elem + entries * 4 + Bq
    upd = layer.NG * (layer.M * cd * 4 + layer.M * 4 + cd * 4 * 2) + \
        layer.B * layer.Hkv * 2 * d * elem * 2
    merge = layer.B * layer.Hq * d * 4
    return dict(score=score, select=select, attn_update=attn + upd, merge=merge), attn


KERNELS = ["score", "select", "attn_update", "merge"]

# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries of the attention launch, per workload
PMC_FILES = {
    "qwen3-8b-layer-b4-ctx128k-group": "attn_kernel_b4_ctx128k_pmc_traffic.txt",
    "qwen3-8b-36layer-ragged16-ctx8k-128k-paged": "attn_kernel_ragged16_36layer_pmc_traffic.txt",
    "qwen3-8b-layer-b4-ctx128k-perhead": "attn_kernel_b4_ctx128k_perhead_pmc_traffic.txt",
}
ATTN_SOURCES = ["attn.hip", "update_rule.h", "ckv_device.h", "ckv_internal.h"]


def measured_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (calibrated against a plain copy), or None when there is no
    summary for this workload or the attention kernel's sources changed since the
    counters were taken."""
    import hashlib
    name = PMC_FILES.get(workload)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if path is None or not os.path.exists(path):
        return None
    txt = open(path).read()
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, "sparse_long_context_centroid_amd", "csrc", f), "rb").read())
    traffic = sha = None
    for line in txt.splitlines():
        if line.startswith("roofline traffic of"):
            traffic = int(line.rsplit(":", 1)[1])
        elif line.startswith("source-sha256"):
            sha = line.rsplit(":", 1)[1].strip()
    return traffic if sha == h.hexdigest() else None


class Timed:
    """One layer's fused decode step (ckv_decode_step, 4 kernels) on torch's current
    stream: a pair of events around the whole step (launch gaps included) and the
    library's per-kernel start / stop events (kernel execution only)."""

    def __init__(self, layer):
        self.layer = layer
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
        self.step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def run(self, q, kn, vn, scale, per_kernel: bool):
        self.step_ev[0].record()
        self.layer.step_fused(q, kn, vn, scale, events=self.ev if per_kernel else None)
        self.step_ev[1].record()

    def step_ms(self):
        return self.step_ev[0].elapsed_time(self.step_ev[1])

    def times_ms(self):
        return [self.ev[2 * i].elapsed_time(self.ev[2 * i + 1]) for i in range(4)]


def dense_baseline(layers, qkv, wl, scrub, args, elem):
    """The same layers through ckv_dense_decode_attn (attention over every cached
    token, no selection), same cold protocol, on the state the sparse steps left."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    outs = [torch.empty_like(l.out) for l in layers]
    T = qkv[0][0].shape[0]
    ms = []
    for t in range(min(args.steps, 10) + 2):
        tot = 0.0
        for lay, (q, _, _), o in zip(layers, qkv, outs):
            if not args.warm:
                scrub_sum = scrub.sum()
            ev[0].record()
            lay.dense(q[T - 1], wl.scale, out=o)
            ev[1].record()
            torch.cuda.synchronize()
            tot += ev[0].elapsed_time(ev[1])
        if t >= 2:
            ms.append(tot)
    n = np.concatenate([l.seq_len.cpu().numpy() for l in layers]).astype(np.float64)
    kv_bytes = float(n.sum()) * layers[0].Hkv * 2 * layers[0].d * elem
    step_ms = float(np.mean(ms))
    return dict(ms_per_step=step_ms, tokens_per_s=wl.B / (step_ms / 1e3),
                kv_bytes_per_step=kv_bytes, gbs=kv_bytes / (step_ms / 1e3) / 1e9,
                steps=len(ms))


def rebuild_timing(layers, scrub, args, elem):
    """Maintenance path: centroids recomputed from the member lists (every member
    key read once) and the drift of the running means from them, per layer, cold."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ms_r, ms_d, worst = [], [], 0.0
    for t in range(4):
        for lay in layers:
            ref = torch.empty_like(lay.centroids)
            if not args.warm:
                scrub_sum = scrub.sum()
            ev[0].record()
            lay.rebuild(out=ref)
            ev[1].record()
            dr = lay.drift(ref)
            ev[2].record()
            torch.cuda.synchronize()
            if t >= 1:
                ms_r.append(ev[0].elapsed_time(ev[1]))
                ms_d.append(ev[1].elapsed_time(ev[2]))
                worst = max(worst, float(dr.max().item()))
    lay = layers[0]
    members = int(lay.comm_size.sum().item())
    by = members * (lay.d * elem + 4 + 4) + lay.centroids.numel() * 4
    mr = float(np.mean(ms_r))
    return dict(ms_per_layer=mr, gbs=by / (mr / 1e3) / 1e9, bytes_per_layer=by,
                drift_ms_per_layer=float(np.mean(ms_d)), max_drift=worst)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def edges_timing(wl, args):
    """Prefill-side producer of the graph: per-query top-8 direct edges and their
    co-attention pairs of one layer's prefill of one sequence at the workload's
    longest context (ckv_prefill_edges), kernel-bound events, warm (the prefill's
    Q and K outgrow the caches anyway).  Algorithmic work: q.k for every causal,
    non-sink (query head, query, key) triple, 2 d flops each."""
    n = int(wl.seq_len0.max())
    pf = I.make_prefill(9000 + wl.seed, B=1, n=n, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, S=wl.S,
                        device="cuda")
    topk = 8
    NG = wl.Hkv * wl.gpk
    dims = Bd.ckv_dims(1, wl.Hq, wl.Hkv, wl.d, wl.gpk, 64, wl.S, I.DT_BF16)
    idx = torch.empty((NG, n, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((NG, n, topk), dtype=torch.float32, device="cuda")
    pr = torch.empty((NG, n, topk * (topk - 1) // 2, 2), dtype=torch.int32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms = []
    for t in range(5):
        Bd.ckv_prefill_edges(dims, pf.q, pf.k, n, topk, pf.scale, idx, sc, pr, events=ev)
        torch.cuda.synchronize()
        if t >= 2:
            ms.append(ev[0].elapsed_time(ev[1]))
    m = max(n - wl.S, 0)
    flops = 2.0 * wl.d * wl.Hq * (m * (m - 1) / 2 + 0.0)
    mean = float(np.mean(ms))
    tf = flops / (mean / 1e3) / 1e12
    return dict(kernel="edges_kernel", prefill_tokens=n, topk=topk, ms_per_layer=mean,
                flops_per_layer=flops, tflops=tf, peak_tflops=MFMA_BF16_PEAK_TFLOPS,
                frac_mfma_bf16=tf / MFMA_BF16_PEAK_TFLOPS,
                prefill_tokens_per_s=n / (mean / 1e3))


def graph_bytes(L, cdim: int) -> dict:
    """Memory the graphs of one layer keep beside the KV cache: centroids as
    allocated (Cmax padding) and as used (communities in use), the member pool
    (with its append slack), and the three per-community int32 arrays."""
    NG, Cmax = L.comm_start.shape
    C = int(np.asarray(L.num_comms).sum())
    cent_alloc = NG * Cmax * cdim * 4
    cent_used = C * cdim * 4
    members = int(L.members.size) * 4
    percomm_alloc = 3 * NG * Cmax * 4
    return dict(graphs=NG, communities=C, centroid_bytes=cent_alloc,
                centroid_bytes_used=cent_used, member_bytes=members,
                per_community_bytes=percomm_alloc,
                total=cent_alloc + members + percomm_alloc,
                total_used=cent_used + members + 3 * C * 4)


def granularity_sweep(spec, args, scrub, elem):
    """The same workload (layer 0) with one graph per KV head (group), per query
    head, and per layer: step time under the cold protocol, the speed-up over dense
    attention on the same cache, and the graphs' memory next to the KV cache."""
    dev = "cuda:0"
    K = max(3, min(args.steps, 20))
    W = 3
    out = []
    dense_ms = None
    for mode in ("group", "head", "layer"):
        sp = I.granularity_spec(spec, mode)
        wl = I.make_workload(sp, args.seed, device=dev, steps=W + K, layers=1)
        lay = build_layers(wl, int(wl.S + wl.budget.max()))[0]
        tm = Timed(lay)
        L = wl.layers[0]
        ms = []
        for t in range(W + K):
            if not args.warm:
                scrub_sum = scrub.sum()
            tm.run(L.q[t], L.k_new[t], L.v_new[t], wl.scale, per_kernel=False)
            torch.cuda.synchronize()
            if t >= W:
                ms.append(tm.step_ms())
        if int(lay.err.item()):
            raise SystemExit(f"device error flag during the {mode} sweep")
        if dense_ms is None:
            # dense attention reads every cached token: the same for every granularity
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            dm = []
            o = torch.empty_like(lay.out)
            for t in range(5):
                if not args.warm:
                    scrub_sum = scrub.sum()
                ev[0].record()
                lay.dense(L.q[W + K - 1], wl.scale, out=o)
                ev[1].record()
                torch.cuda.synchronize()
                if t >= 2:
                    dm.append(ev[0].elapsed_time(ev[1]))
            dense_ms = float(np.mean(dm))
        n = wl.seq_len0.astype(np.float64)
        kv_bytes = float(n.sum()) * wl.Hkv * 2 * wl.d * elem
        gb = graph_bytes(L, wl.Hkv * wl.d if wl.gpk == 0 else wl.d)
        step = float(np.mean(ms))
        out.append(dict(graphs=mode, workload=sp.name, graphs_per_layer=gb["graphs"],
                        ms_per_step=step, tokens_per_s=wl.B / (step / 1e3),
                        speedup_vs_dense=dense_ms / step, dense_ms_per_step=dense_ms,
                        mean_index_len=float(lay.index_len.float().mean().item()),
                        graph_bytes=gb, kv_bytes=kv_bytes,
                        graph_overhead_vs_kv=gb["total"] / kv_bytes,
                        graph_overhead_vs_kv_used=gb["total_used"] / kv_bytes))
        log(f"[bench] granularity {mode}: {step * 1e3:.1f} us/step, "
            f"{dense_ms / step:.2f}x dense, graphs {gb['total'] / 1e6:.1f} MB = "
            f"{100 * gb['total'] / kv_bytes:.2f}% of KV")
        del lay, tm, wl, L
        torch.cuda.empty_cache()
    return out


def build_layers(wl, index_stride):
    layers = []
    for li in range(len(wl.layers)):
        lay = Bd.decode_layer_from_workload(wl, li, index_stride=index_stride)
        lay.num_comms_host = wl.layers[li].num_comms.astype(np.int64)
        layers.append(lay)
    return layers


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> tuple:
    """Threads for the oracle: every CPU this process may run on, capped by the
    host's declared CPU share for this job (OMP_NUM_THREADS when it is set)."""
    aff = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return (min(aff, int(cap)) if cap.isdigit() and int(cap) > 0 else aff), aff


def cpu_baseline(wl, seconds: float, threads: int):
    """The fp64 oracle on the host cores.  One-layer workloads: the first decode
    steps of the layer, as many as fit in `seconds`.  Multi-layer workloads: one
    whole decode step, the layers streamed one at a time (each layer's host copy
    is made outside the timed region), the per-layer times summed."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import helpers as H  # test infrastructure: host copies for the oracle
    max_len = int(wl.S + wl.budget.max())
    layers = len(wl.layers)
    if layers > 1:
        total = 0.0
        for li in range(layers):
            st = H.oracle_state(wl, li, threads=threads)
            q, kn, vn = H.step_inputs(wl, li, 0)
            t0 = time.perf_counter()
            st.step(q, kn, vn, wl.budget, wl.scale, wl.M, max_len)
            total += time.perf_counter() - t0
            del st
        return dict(value=wl.B / total, unit="tokens/s", cores=threads, kind="oracle",
                    sample=f"one decode step of all {layers} layers x {wl.B} sequences, layers "
                           f"streamed one at a time (host copies untimed), fp64 C oracle, "
                           f"{threads} threads over graphs", seconds=total)
    st = H.oracle_state(wl, 0, threads=threads)
    done = 0
    t0 = time.perf_counter()
    while done < wl.steps:
        q, kn, vn = H.step_inputs(wl, 0, done)
        st.step(q, kn, vn, wl.budget, wl.scale, wl.M, max_len)
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=wl.B * done / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{done} decode steps x {wl.B} sequences of the layer (the whole step), "
                       f"fp64 C oracle, {threads} threads over graphs", seconds=dt)


def update_cost_vs_context(args, scrub, contexts=(8192, 131072), steps=24):
    """The local update alone (ckv_local_update, one launch) on the 4-sequence
    Qwen3-8B layer shape at two context lengths: its cost is set by the candidate
    count and d, not by n.  Each timed call follows a cold-cache scrub; HIP events
    bracket the single launch on its stream.  The candidates come from the same
    step's score and selection (untimed)."""
    out = {}
    for n in contexts:
        wl = I.make_workload(3, args.seed, device="cuda:0", context=n, steps=steps, layers=1)
        lay = build_layers(wl, int(wl.S + wl.budget.max()))[0]
        L = wl.layers[0]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        us = []
        for t in range(steps):
            lay.score(L.q[t], wl.scale)
            lay.select()
            if not args.warm:
                scrub_sum = scrub.sum()
            ev[0].record()
            lay.update(L.k_new[t], L.v_new[t])
            ev[1].record()
            torch.cuda.synchronize()
            if t >= 4:
                us.append(ev[0].elapsed_time(ev[1]) * 1e3)
        if int(lay.err.item()):
            raise SystemExit("device error flag during the update timing")
        out[str(n)] = dict(us_median=float(np.median(us)), us_mean=float(np.mean(us)),
                           graphs=lay.NG, communities_per_graph=float(L.num_comms.mean()),
                           calls=len(us))
        del lay, wl, L
        torch.cuda.empty_cache()
    a, b = (out[str(c)]["us_median"] for c in contexts)
    out["ratio_long_over_short"] = b / a
    out["what"] = ("ckv_local_update alone (candidates from the same step), 4 sequences x 8 KV "
                   "heads, M = 8, d = 128; event pair around the launch after a cache scrub")
    return out


def four_call_step(args, scrub, steps=24):
    """One decode step of the 4 x 128K workload through the four separate C-ABI
    calls (ckv_score_centroids, ckv_select, ckv_sparse_decode_attn, ckv_local_update:
    5 launches, the update after the attention instead of inside its launch), beside
    the fused ckv_decode_step on the same state.  Cold protocol: a scrub before each
    step, one pair of events around the calls."""
    wl = I.make_workload(3, args.seed, device="cuda:0", steps=2 * steps, layers=1)
    lay = build_layers(wl, int(wl.S + wl.budget.max()))[0]
    L = wl.layers[0]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    res = {}
    for name, fn, base in (("four_calls", lay.step, 0), ("fused", lay.step_fused, steps)):
        us = []
        for t in range(base, base + steps):
            if not args.warm:
                scrub_sum = scrub.sum()
            ev[0].record()
            fn(L.q[t], L.k_new[t], L.v_new[t], wl.scale)
            ev[1].record()
            torch.cuda.synchronize()
            if t - base >= 4:
                us.append(ev[0].elapsed_time(ev[1]) * 1e3)
        res[name] = dict(us_median=float(np.median(us)), us_mean=float(np.mean(us)),
                         steps=len(us))
    if int(lay.err.item()):
        raise SystemExit("device error flag during the four-call timing")
    del lay, wl, L
    torch.cuda.empty_cache()
    res["what"] = ("one 4 x 128K decode step: the four C-ABI calls in turn against "
                   "ckv_decode_step, each after a cache scrub, events around the calls")
    return res


def measure(spec, args, scrub, *, extras: bool):
    """Generate `spec` on the GPU and time its fused decode step.  Passes, in order:
    warmup; K steps bracketed by a pair of events each (value); K steps with the
    per-kernel events (kernel times, roofline); without --warm, up to 20
    back-to-back steps without the scrub, the host reading results after each; up
    to 20 steps queued back to back without the scrub or any host wait, one pair of
    events around them all; then the configuration's remaining decode steps,
    untimed, so that every step the configuration runs is run.
    With `extras`: centroid rebuild, the dense baseline, the granularity sweep and
    the prefill edges as well."""
    dev = "cuda:0"
    KW = 0 if args.warm else min(args.steps, 20)
    KQ = min(args.steps, 20)
    b_warm = args.warmup + 2 * args.steps
    b_queued = b_warm + KW
    T_timed = b_queued + KQ
    T = max(T_timed, spec.steps)
    t0 = time.perf_counter()
    wl = I.make_workload(spec, args.seed, device=dev, steps=T,
                         layers=args.layers if extras else None)
    torch.cuda.synchronize()
    log(f"[bench] workload {spec.name}: {len(wl.layers)} layer(s), B={wl.B}, "
        f"n={wl.seq_len0.tolist()[:4]}..., Cmax={wl.Cmax}, {T} steps, generated in "
        f"{time.perf_counter() - t0:.1f}s")
    index_stride = int(wl.S + wl.budget.max())
    cpu = None
    if not args.no_cpu_baseline:
        threads, aff = oracle_threads()
        t1 = time.perf_counter()
        cpu = cpu_baseline(wl, args.cpu_seconds, threads)
        cpu["affinity_cpus"] = aff
        cpu["threads_rule"] = "min(len(sched_getaffinity), OMP_NUM_THREADS when set)"
        if len(wl.layers) == 1:
            one = cpu_baseline(wl, max(2.0, args.cpu_seconds / 5), 1)
            cpu["value_1_thread"] = one["value"]
            cpu["sample_1_thread"] = one["sample"]
        cpu["cpu_model"] = cpu_model()
        log(f"[bench] cpu baseline {cpu['value']:.2f} tokens/s on {threads} threads "
            f"({time.perf_counter() - t1:.1f}s)")
    layers = build_layers(wl, index_stride)
    timers = [Timed(l) for l in layers]
    elem = 2 if wl.dtype == I.DT_BF16 else 4
    qkv = [(L.q, L.k_new, L.v_new) for L in wl.layers]
    kernel_ms = np.zeros(4)
    kernel_bytes = {k: 0 for k in KERNELS}
    attn_only_bytes = 0
    step_ms, step_ms_instr, step_ms_warm = [], [], []
    value_bytes = 0
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    # the timed passes keep the host out of the measured spans: garbage collection is
    # off, and in the cold passes every layer's scrub and step of a decode step are
    # queued before the host waits, so the GPU never waits for a launch between a
    # step's events (the events are read, and the list lengths counted, afterwards)
    queued_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    queued_ms = None
    gc.collect()
    gc.disable()
    for t in range(T):
        phase = 0 if t < args.warmup else (1 if t < args.warmup + args.steps else (
            2 if t < b_warm else (3 if t < b_queued else (5 if t < T_timed else 4))))
        tot = 0.0
        queued = []
        if phase == 5 and t == b_queued:
            queued_ev[0].record()
        for li, (tm, (q, kn, vn)) in enumerate(zip(timers, qkv)):
            if not args.warm and phase in (1, 2):
                scrub_sum = scrub.sum()               # cold caches, outside the events
            tm.run(q[t], kn[t], vn[t], wl.scale, per_kernel=phase == 2)
            if phase in (4, 5):
                continue
            if phase == 3:
                # warm: back to back, the host waits and reads after every step
                torch.cuda.synchronize()
                tot += tm.step_ms()
                continue
            if phase:
                queued.append(tm)
            else:
                torch.cuda.synchronize()
        if queued:
            torch.cuda.synchronize()
        for tm in queued:
            tot += tm.step_ms()
            idx_len = tm.layer.index_len.cpu().numpy()
            by, ab = step_bytes(tm.layer, idx_len, elem)
            if phase == 1:
                value_bytes += sum(by.values())
            else:
                kernel_ms += np.array(tm.times_ms())
                for k, v in by.items():
                    kernel_bytes[k] += v
                attn_only_bytes += ab
        if phase == 5 and t == T_timed - 1:
            queued_ev[1].record()
            torch.cuda.synchronize()
            queued_ms = queued_ev[0].elapsed_time(queued_ev[1]) / KQ
        if phase == 1:
            step_ms.append(tot)
        elif phase == 2:
            step_ms_instr.append(tot)
        elif phase == 3:
            step_ms_warm.append(tot)
        if t == 0 or (t + 1) % 25 == 0:
            log(f"[bench] step {t + 1}/{T}")
    torch.cuda.synchronize()
    gc.enable()
    wall = time.perf_counter() - wall0
    err = max(int(l.err.item()) for l in layers)
    if err:
        raise SystemExit(f"device error flag {err} during the benchmark")
    K = args.steps
    nl = len(layers)
    total_ms = float(np.sum(step_ms))
    per_kernel = {n: dict(ms_per_launch=kernel_ms[i] / (K * nl),
                          gbs=kernel_bytes[n] / (kernel_ms[i] / 1e3) / 1e9 if kernel_ms[i] else None)
                  for i, n in enumerate(KERNELS)}
    attn_gbs = per_kernel["attn_update"]["gbs"]
    path_gbs = value_bytes / (total_ms / 1e3) / 1e9
    r = {
        "workload": spec.name,
        "value": wl.B * K / (total_ms / 1e3),
        "ms_per_step": total_ms / K,
        "ms_per_step_median": float(np.median(step_ms)),
        "config": {
            "workload": spec.name, "batch": wl.B, "layers": nl,
            "context": int(wl.seq_len0.max()) if not spec.ragged else "8K-128K ragged",
            "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.d,
            "graphs": "per-head" if wl.gpk > 1 else ("per-layer" if wl.gpk == 0 else "query-group"),
            "budget": int(wl.budget.max()) if not spec.ragged else "5% of context",
            "sinks": wl.S, "n_cand": wl.M, "kv_dtype": "bf16" if elem == 2 else "fp32",
            "score_arith": "fp64", "attn_arith": "fp32", "steps_run": T,
            "protocol": "warm (back-to-back)" if args.warm else
            f"cold ({args.scrub_mib} MiB scrub before each layer's step, outside the events)",
        },
        "dtype": "bf16" if elem == 2 else "fp32",
        "path_gbs": path_gbs,
        "path_frac_hbm": path_gbs / HBM_PEAK_GBS,
        "path_frac_target": 0.60,
        "path_target_met": path_gbs / HBM_PEAK_GBS >= 0.60,
        "bytes_per_step": value_bytes / K,
        "ms_per_step_with_kernel_events": float(np.mean(step_ms_instr)),
        "warm": ({"ms_per_step": float(np.mean(step_ms_warm)),
                  "tokens_per_s": wl.B / (float(np.mean(step_ms_warm)) / 1e3),
                  "steps": len(step_ms_warm),
                  "protocol": "back-to-back steps, no scrub; the host synchronises and reads "
                              "results after every step, so its launch latency is exposed"}
                 if step_ms_warm else None),
        "warm_queued": ({"ms_per_step": queued_ms, "tokens_per_s": wl.B / (queued_ms / 1e3),
                         "steps": KQ,
                         "protocol": "steps queued back to back with no scrub and no host wait "
                                     "between them (a decode loop that does not read results "
                                     "every step); one pair of events around all of them"}
                        if queued_ms else None),
        "kernels": per_kernel,
        "attn_share_of_attn_update_bytes": attn_only_bytes / kernel_bytes["attn_update"],
        "wall_s_timed_loop": wall,
        "roofline": {
            "kernel": "attn_kernel (indexed split-K flash-decode partials + local update)",
            "bound": "hbm", "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": attn_gbs / HBM_PEAK_GBS if attn_gbs else None,
            "traffic": measured_traffic(spec.name),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_launch": kernel_bytes["attn_update"] / (K * nl),
        },
        "cpu_baseline": cpu,
    }
    if extras and not args.no_rebuild:
        r["centroid_rebuild"] = rebuild_timing(layers, scrub, args, elem)
    if not args.no_dense:
        dense = dense_baseline(layers, qkv, wl, scrub, args, elem)
        dense["sparse_speedup"] = dense["ms_per_step"] / (total_ms / K)
        r["dense_baseline"] = dense
    if extras and not args.no_edges:
        r["prefill_edges"] = edges_timing(wl, args)
    del layers, timers, qkv, wl
    torch.cuda.empty_cache()
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--graphs", choices=("config", "group", "head", "layer"), default="config",
                    help="graph granularity of the timed workload (default: the config's own)")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scrub-mib", type=int, default=1024)
    ap.add_argument("--warm", action="store_true", help="no cache scrub between steps")
    ap.add_argument("--no-rebuild", action="store_true",
                    help="skip timing the centroid rebuild from the member lists")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-attention baseline (every cached token)")
    ap.add_argument("--no-granularity", action="store_true",
                    help="skip the graph-granularity sweep (group / per-head / per-layer)")
    ap.add_argument("--no-edges", action="store_true",
                    help="skip the prefill edge-extraction measurement")
    ap.add_argument("--no-update-timing", action="store_true",
                    help="skip timing the local update alone at 8K and 128K contexts")
    ap.add_argument("--no-config4", action="store_true",
                    help="skip the 36-layer ragged paged workload measured after the main one")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before timing, run a plain device copy of this many MiB three times "
                         "(a known-size kernel to calibrate hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU only (asked for --gpus {args.gpus}); "
              "there is no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    Bd.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    spec = I.CONFIGS[args.config]
    if args.graphs != "config":
        spec = I.granularity_spec(spec, args.graphs)
    scrub = torch.empty(args.scrub_mib << 18, dtype=torch.float32, device=dev).fill_(0.0)
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    main_r = measure(spec, args, scrub, extras=True)
    res = {
        "metric": "sparse decode attention tokens/s + achieved HBM GB/s at 128K, Qwen3-8B shape",
        "value": main_r["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["ms_per_step"],
        "ms_per_step_median": main_r["ms_per_step_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_r["dtype"],
        "data": "synthetic",
    }
    for k, v in main_r.items():
        if k not in res and k not in ("workload",):
            res[k] = v
    if not args.no_update_timing:
        res["update_cost_vs_context"] = update_cost_vs_context(args, scrub)
        u = res["update_cost_vs_context"]
        log(f"[bench] local update alone: {u['8192']['us_median']:.2f} us at 8K, "
            f"{u['131072']['us_median']:.2f} us at 128K")
        if args.config == 3:
            res["four_call_step"] = f4 = four_call_step(args, scrub)
            log(f"[bench] four C-ABI calls {f4['four_calls']['us_median']:.2f} us per step, "
                f"fused {f4['fused']['us_median']:.2f} us")
    if not args.no_granularity:
        res["granularity_sweep"] = granularity_sweep(spec, args, scrub, 2 if spec.dtype == I.DT_BF16 else 4)
    if args.config != 4 and not args.no_config4:
        c4 = measure(I.CONFIGS[4], args, scrub, extras=False)
        res["config4"] = {k: v for k, v in c4.items() if k not in ("dtype",)}
        log(f"[bench] {c4['workload']}: {c4['ms_per_step']:.3f} ms per 36-layer step, "
            f"{c4['value']:.0f} tokens/s, path {c4['path_frac_hbm']:.3f} of HBM peak")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
