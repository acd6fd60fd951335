"""Seeded synthetic workloads for the CommunityKV decode step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scoring, selection, attention or update).  Both the HIP
path and the fp64 oracle consume exactly the bytes it produces.

What stands in for what (the pages evaluate trained models on long-context
suites; no weights or datasets are used here):

* Communities stand in for the Leiden partition of the prefill token graph
  (rit.work post "CommunityKV long-context decoding", section on the token graph):
  each community has a Gaussian centre, its keys are centre + 0.3 noise, and its
  members sit in Markov-scattered spans of the context.
* Positions 0..S-1 are the attention sinks; they belong to no community.
* The initial centroid of a community is the fp64 mean of its stored member keys,
  rounded to fp32 -- the centre the off-path partitioning step would hand over.
* Each decode step draws a query that lies near two centres, and a new key/value
  whose label continues the Markov chain of the context.

Bulk keys/values are generated with torch on the requested device (the GPU for
the real sizes); the structure (labels, CSR) is drawn with numpy on the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

PAGE_SIZE = 16
DT_F32 = 0
DT_BF16 = 1


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    """Shape of one workload (one decode layer unless `layers` > 1)."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int                  # tokens in cache at the first step (cfg 0-3)
    per_head_graphs: bool         # one graph per query head instead of per KV head
    budget: int                   # token budget (sinks not counted); -1: 5% of context
    steps: int                    # decode steps the configuration runs
    dtype: int                    # DT_BF16 or DT_F32 for q/K/V
    num_sinks: int = 4
    n_cand: int = 8
    markov_labels: int = 0        # >0: labels from a literal Markov chain over this many centres
    ragged: bool = False          # contexts uniform in [ctx_lo, ctx_hi] per sequence
    ctx_lo: int = 0
    ctx_hi: int = 0
    layers: int = 1
    shuffled_pages: bool = False
    layer_graph: bool = False     # one graph per layer, shared by all heads
    mean_comm_size: float = 64.0  # mean of the geometric community sizes


def granularity_spec(base: ConfigSpec, mode: str) -> ConfigSpec:
    """The same workload with another graph granularity: "group" (one graph per KV
    head), "head" (one per query head) or "layer" (one per layer)."""
    if mode not in ("group", "head", "layer"):
        raise ValueError(mode)
    stem = base.name.rsplit("-", 1)[0] if base.name.endswith(("-group", "-perhead")) else base.name
    tag = {"group": "group", "head": "perhead", "layer": "layergraph"}[mode]
    return dataclasses.replace(base, name=f"{stem}-{tag}", per_head_graphs=mode == "head",
                               layer_graph=mode == "layer")


CONFIGS: List[ConfigSpec] = [
    ConfigSpec("tiny-fp32-d64-ctx2048", 1, 4, 1, 64, 2048, False, 256, 1, DT_F32,
               markov_labels=32),
    ConfigSpec("qwen3-8b-layer-ctx32k-group", 1, 32, 8, 128, 32768, False, 2048, 64, DT_BF16),
    ConfigSpec("qwen3-8b-layer-ctx32k-perhead", 1, 32, 8, 128, 32768, True, 2048, 64, DT_BF16),
    ConfigSpec("qwen3-8b-layer-b4-ctx128k-group", 4, 32, 8, 128, 131072, False, 4096, 256, DT_BF16),
    ConfigSpec("qwen3-8b-36layer-ragged16-ctx8k-128k-paged", 16, 32, 8, 128, 0, False, -1, 10,
               DT_BF16, ragged=True, ctx_lo=8192, ctx_hi=131072, layers=36, shuffled_pages=True),
]


def torch_dtype(dt: int):
    return torch.bfloat16 if dt == DT_BF16 else torch.float32


@dataclasses.dataclass
class Layer:
    """One layer's graph state and KV pool."""
    centroids: torch.Tensor       # [NG, Cmax, d] fp32, natural row layout ([B, Cmax, Hkv*d]
                                  # for the layer graph: one centroid per KV head, in order)
    num_comms: np.ndarray         # [NG] int32
    comm_start: np.ndarray        # [NG, Cmax] int32, offset into `members`
    comm_size: np.ndarray         # [NG, Cmax] int32
    comm_cap: np.ndarray          # [NG, Cmax] int32
    members: np.ndarray           # [pool] int32 token positions (-1 = free slot)
    k_pages: torch.Tensor         # [num_pages, Hkv, page_size, d]
    v_pages: torch.Tensor
    base_labels: List[np.ndarray]  # per (b, kvh): label of every position (-1 = sink)
    centres: List[np.ndarray]      # per (b, kvh): [C, d] fp32 generating centres
    # per-step inputs, raw dtype, on the workload's device
    q: torch.Tensor               # [T, B, Hq, d]
    k_new: torch.Tensor           # [T, B, Hkv, d]
    v_new: torch.Tensor           # [T, B, Hkv, d]
    step_labels: np.ndarray       # [T, B, Hkv] generating label of each new token


@dataclasses.dataclass
class Workload:
    spec: ConfigSpec
    seed: int
    B: int
    Hq: int
    Hkv: int
    d: int
    gpk: int                      # graphs per KV head (1 or Hq/Hkv; 0: one per layer)
    S: int
    M: int
    dtype: int
    Cmax: int
    steps: int
    page_size: int
    max_pages: int
    num_pages: int
    page_table: torch.Tensor      # [B, max_pages] int32
    seq_len0: np.ndarray          # [B] int32 tokens at the first step
    budget: np.ndarray            # [B] int32
    scale: float
    layers: List[Layer]
    device: str

    @property
    def NG(self) -> int:
        return self.B if self.gpk == 0 else self.B * self.Hkv * self.gpk


def _ss(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, *key]))


def _torch_gen(device: str, seed: int, *key: int) -> torch.Generator:
    s = np.random.SeedSequence([seed, *key]).generate_state(2, dtype=np.uint32)
    g = torch.Generator(device=device)
    g.manual_seed(int(s[0]) << 32 | int(s[1]))
    return g


def geometric_partition(rng: np.random.Generator, N: int, mean_size: float = 64.0,
                        stay: float = 0.7):
    """Labels for N non-sink positions: community sizes ~ Geometric(1/mean_size)
    (the last one truncated so they sum to N), each community cut into runs whose
    lengths are those of a Markov chain with stay probability `stay`, and all runs
    shuffled over the positions.  Returns (labels[N], C)."""
    if N <= 0:
        return np.zeros(0, np.int32), 0
    est = int(N / mean_size * 1.3) + 16
    sizes = rng.geometric(1.0 / mean_size, size=est)
    while sizes.sum() < N:
        sizes = np.concatenate([sizes, rng.geometric(1.0 / mean_size, size=est)])
    cs = np.cumsum(sizes)
    C = int(np.searchsorted(cs, N)) + 1
    sizes = sizes[:C].copy()
    sizes[-1] -= int(cs[C - 1] - N)
    comm_of_tok = np.repeat(np.arange(C, dtype=np.int64), sizes)
    first = np.zeros(N, bool)
    first[np.concatenate([[0], np.cumsum(sizes)[:-1]])] = True
    brk = rng.random(N) < (1.0 - stay)
    starts = first | brk
    run_id = np.cumsum(starts) - 1
    R = int(run_id[-1]) + 1
    run_len = np.bincount(run_id, minlength=R)
    run_comm = comm_of_tok[starts]
    order = rng.permutation(R)
    labels = np.repeat(run_comm[order], run_len[order]).astype(np.int32)
    return labels, C


def markov_labels(rng: np.random.Generator, N: int, C: int, stay: float = 0.7):
    """Labels from a literal Markov chain: keep the previous label with probability
    `stay`, else draw uniformly over C labels."""
    lab = np.empty(N, np.int32)
    cur = int(rng.integers(C))
    u = rng.random(N)
    draws = rng.integers(0, C, size=N)
    for i in range(N):
        if i > 0 and u[i] >= stay:
            cur = int(draws[i])
        lab[i] = cur
    return lab


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def make_workload(cfg: int | ConfigSpec, seed: Optional[int] = None, *, device: str = "cpu",
                  context: Optional[int] = None, batch: Optional[int] = None,
                  steps: Optional[int] = None, layers: Optional[int] = None,
                  budget: Optional[int] = None, contexts: Optional[List[int]] = None,
                  n_cand: Optional[int] = None, slack: Optional[int] = None,
                  page_size: Optional[int] = None) -> Workload:
    """Build a seeded workload.  Overrides shrink a configuration for tests while
    keeping its structure (same recipe, fewer tokens/sequences/steps); page_size
    (a power of two, default PAGE_SIZE) sets the tokens per page of the KV pools."""
    spec = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    cfg_id = CONFIGS.index(spec) if spec in CONFIGS else 99
    if seed is None:
        seed = 1000 + cfg_id
    B = batch if batch is not None else spec.batch
    T = steps if steps is not None else spec.steps
    L = layers if layers is not None else spec.layers
    S = spec.num_sinks
    M = n_cand if n_cand is not None else spec.n_cand
    d = spec.head_dim
    Hq, Hkv = spec.num_q_heads, spec.num_kv_heads
    G = Hq // Hkv
    gpk = G if spec.per_head_graphs else (0 if spec.layer_graph else 1)
    slack = T if slack is None else slack
    rng0 = _ss(seed, 0)
    if contexts is not None:
        ns = np.asarray(contexts, np.int64)
        B = len(ns)
    elif spec.ragged:
        lo, hi = spec.ctx_lo, spec.ctx_hi
        if context is not None:       # shrink the whole range proportionally
            lo, hi = max(S + 1, context * lo // hi), context
        ns = rng0.integers(lo, hi + 1, size=B)
    else:
        ns = np.full(B, context if context is not None else spec.context, np.int64)
    if budget is not None:
        bud = np.full(B, budget, np.int64)
    elif spec.budget < 0:
        bud = ns // 20
    else:
        bud = np.full(B, spec.budget, np.int64)

    ps = PAGE_SIZE if page_size is None else int(page_size)
    if ps < 1 or ps & (ps - 1):
        raise ValueError(f"page_size {ps} is not a power of two")
    pages_per_seq = [(int(n) + T + ps - 1) // ps for n in ns]
    max_pages = max(pages_per_seq)
    num_pages = int(sum(pages_per_seq))
    page_table = np.full((B, max_pages), -1, np.int32)
    if spec.shuffled_pages:
        perm = rng0.permutation(num_pages).astype(np.int32)
    else:
        perm = np.arange(num_pages, dtype=np.int32)
    off = 0
    for b in range(B):
        page_table[b, :pages_per_seq[b]] = perm[off:off + pages_per_seq[b]]
        off += pages_per_seq[b]
    tdt = torch_dtype(spec.dtype)

    layer_objs = []
    for li in range(L):
        layer_objs.append(_make_layer(spec, seed, li, B, ns, T, slack, S, M, d, Hq, Hkv, G,
                                      gpk, page_table, num_pages, tdt, device, ps))
    # one community stride for every layer: pad each layer's per-community arrays
    # to the largest (padding columns are empty communities past num_comms)
    Cmax = max(lo.centroids.shape[1] for lo in layer_objs)
    for lo in layer_objs:
        _pad_communities(lo, Cmax)
    return Workload(spec=spec, seed=seed, B=B, Hq=Hq, Hkv=Hkv, d=d, gpk=gpk, S=S, M=M,
                    dtype=spec.dtype, Cmax=Cmax, steps=T, page_size=ps, max_pages=max_pages,
                    num_pages=num_pages,
                    page_table=torch.from_numpy(page_table).to(device),
                    seq_len0=ns.astype(np.int32), budget=bud.astype(np.int32),
                    scale=float(np.float32(1.0 / math.sqrt(d))), layers=layer_objs,
                    device=device)


def _pad_communities(layer: Layer, Cmax: int) -> None:
    c0 = layer.centroids.shape[1]
    if c0 == Cmax:
        return
    pad = Cmax - c0
    layer.centroids = torch.cat(
        [layer.centroids, layer.centroids.new_zeros((layer.centroids.shape[0], pad,
                                                     layer.centroids.shape[2]))], dim=1)
    for name in ("comm_start", "comm_size", "comm_cap"):
        a = getattr(layer, name)
        setattr(layer, name, np.concatenate([a, np.zeros((a.shape[0], pad), a.dtype)], axis=1))


def _make_layer(spec, seed, li, B, ns, T, slack, S, M, d, Hq, Hkv, G, gpk, page_table,
                num_pages, tdt, device, ps=PAGE_SIZE) -> Layer:
    layer = gpk == 0
    NG = B if layer else B * Hkv * gpk
    gps = 1 if layer else Hkv * gpk           # graphs per sequence
    cd = Hkv * d if layer else d              # centroid row length
    # --- structure: per (b, kvh) base labels, per graph member lists -------------
    base_labels, centres, graph_labels = [], [], []
    Cs = []
    for b in range(B):
        n = int(ns[b])
        if layer:
            # one partition of the sequence, one centre per community and KV head
            rng = _ss(seed, 1, li, b, 0)
            N = max(n - S, 0)
            if spec.markov_labels:
                C = spec.markov_labels
                lab = markov_labels(rng, N, C)
            else:
                lab, C = geometric_partition(rng, N, spec.mean_comm_size)
            full = np.full(n, -1, np.int32)
            full[min(S, n):] = lab
            for kvh in range(Hkv):
                base_labels.append(full)
                centres.append(_ss(seed, 8, li, b, kvh).standard_normal((max(C, 1), d))
                               .astype(np.float32))
            graph_labels.append(lab)
            Cs.append(C)
            continue
        for kvh in range(Hkv):
            rng = _ss(seed, 1, li, b, kvh)
            N = max(n - S, 0)
            if spec.markov_labels:
                C = spec.markov_labels
                lab = markov_labels(rng, N, C)
            else:
                lab, C = geometric_partition(rng, N, spec.mean_comm_size)
            full = np.full(n, -1, np.int32)
            full[min(S, n):] = lab
            base_labels.append(full)
            centres.append(rng.standard_normal((max(C, 1), d)).astype(np.float32))
            for j in range(gpk):
                if gpk > 1:
                    rj = _ss(seed, 2, li, b, kvh, j)
                    lj = lab.copy()
                    mv = rj.random(N) < 0.25
                    lj[mv] = rj.integers(0, C, size=int(mv.sum()))
                else:
                    lj = lab
                graph_labels.append(lj)
                Cs.append(C)
    Cmax = _round_up(max(max(Cs), 1), 64)
    num_comms = np.asarray(Cs, np.int32)
    comm_start = np.zeros((NG, Cmax), np.int32)
    comm_size = np.zeros((NG, Cmax), np.int32)
    comm_cap = np.zeros((NG, Cmax), np.int32)
    pools = []
    off = 0
    for g in range(NG):
        b = g // gps
        lj = graph_labels[g]
        C = Cs[g]
        size = np.bincount(lj, minlength=C).astype(np.int32) if C else np.zeros(0, np.int32)
        cap = size + slack
        start = off + np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
        pool = np.full(int(cap.sum()), -1, np.int32)
        pos = np.argsort(lj, kind="stable").astype(np.int64) + min(S, int(ns[b]))
        sorted_lab = lj[np.argsort(lj, kind="stable")]
        within = np.arange(len(lj)) - np.concatenate([[0], np.cumsum(size)[:-1]])[sorted_lab] \
            if len(lj) else np.zeros(0, np.int64)
        pool[(start[sorted_lab] - off + within).astype(np.int64)] = pos
        comm_start[g, :C] = start
        comm_size[g, :C] = size
        comm_cap[g, :C] = cap
        pools.append(pool)
        off += len(pool)
        assert off < 2**31
    members = np.concatenate(pools) if pools else np.zeros(0, np.int32)

    # --- bulk keys / values on the device, written into the paged pool ----------
    k_pages = torch.zeros((num_pages, Hkv, ps, d), dtype=tdt, device=device)
    v_pages = torch.zeros_like(k_pages)
    centroids = torch.zeros((NG, Cmax, cd), dtype=torch.float32, device=device)
    for b in range(B):
        n = int(ns[b])
        npg = (n + ps - 1) // ps
        pt = torch.from_numpy(page_table[b, :npg].astype(np.int64)).to(device)
        gk = _torch_gen(device, seed, 3, li, b)
        kl = torch.empty((Hkv, npg * ps, d), dtype=torch.float32, device=device)
        vl = torch.randn((Hkv, npg * ps, d), generator=gk, device=device)
        for kvh in range(Hkv):
            lab = torch.from_numpy(base_labels[b * Hkv + kvh].astype(np.int64)).to(device)
            cen = torch.from_numpy(centres[b * Hkv + kvh]).to(device)
            noise = torch.randn((n, d), generator=gk, device=device)
            sink = lab < 0
            rows = torch.where(sink[:, None], noise, cen[lab.clamp(min=0)] + 0.3 * noise)
            kl[kvh, :n] = rows
            kl[kvh, n:] = 0
            vl[kvh, n:] = 0
        kb = kl.to(tdt)
        vb = vl.to(tdt)
        # logical [Hkv, pos, d] -> physical pages [page, Hkv, slot, d]
        k_pages[pt] = kb.view(Hkv, npg, ps, d).permute(1, 0, 2, 3)
        v_pages[pt] = vb.view(Hkv, npg, ps, d).permute(1, 0, 2, 3)
        # initial centroids: fp64 mean of the stored member keys, rounded to fp32
        for kvh in range(Hkv):
            k64 = kb[kvh, :n].to(torch.float64)
            if layer:
                C = Cs[b]
                if C == 0:
                    continue
                lab = torch.from_numpy(graph_labels[b].astype(np.int64)).to(device)
                ssum = torch.zeros((C, d), dtype=torch.float64, device=device)
                ssum.index_add_(0, lab, k64[min(S, n):])
                cnt = torch.from_numpy(comm_size[b, :C].astype(np.float64)).to(device)
                centroids[b, :C, kvh * d:(kvh + 1) * d] = \
                    (ssum / cnt.clamp(min=1)[:, None]).to(torch.float32)
                continue
            for j in range(gpk):
                g = (b * Hkv + kvh) * gpk + j
                C = Cs[g]
                if C == 0:
                    continue
                lab = torch.from_numpy(graph_labels[g].astype(np.int64)).to(device)
                ssum = torch.zeros((C, d), dtype=torch.float64, device=device)
                ssum.index_add_(0, lab, k64[min(S, n):])
                cnt = torch.from_numpy(comm_size[g, :C].astype(np.float64)).to(device)
                mean = ssum / cnt.clamp(min=1)[:, None]
                centroids[g, :C] = mean.to(torch.float32)

    # --- per-step inputs ---------------------------------------------------------
    q = np.zeros((T, B, Hq, d), np.float32)
    kn = np.zeros((T, B, Hkv, d), np.float32)
    vn = np.zeros((T, B, Hkv, d), np.float32)
    zl = np.zeros((T, B, Hkv), np.int32)
    for b in range(B):
        if layer:
            # one label sequence per sequence, shared by its KV heads
            rz = _ss(seed, 9, li, b)
            lab = base_labels[b * Hkv]
            C = centres[b * Hkv].shape[0]
            z = int(lab[-1]) if len(lab) and lab[-1] >= 0 else int(rz.integers(C))
            for t in range(T):
                if rz.random() >= 0.7:
                    z = int(rz.integers(C))
                zl[t, b, :] = z
            for kvh in range(Hkv):
                rng = _ss(seed, 4, li, b, kvh)
                cen = centres[b * Hkv + kvh]
                for t in range(T):
                    z = int(zl[t, b, kvh])
                    kn[t, b, kvh] = cen[z] + 0.3 * rng.standard_normal(d)
                    vn[t, b, kvh] = rng.standard_normal(d)
                    for j in range(G):
                        other = int(rng.integers(C - 1)) if C > 1 else 0
                        if C > 1 and other >= z:
                            other += 1
                        q[t, b, kvh * G + j] = cen[z] + cen[other] + 0.3 * rng.standard_normal(d)
            continue
        for kvh in range(Hkv):
            rng = _ss(seed, 4, li, b, kvh)
            lab = base_labels[b * Hkv + kvh]
            cen = centres[b * Hkv + kvh]
            C = cen.shape[0]
            z = int(lab[-1]) if len(lab) and lab[-1] >= 0 else int(rng.integers(C))
            for t in range(T):
                if rng.random() >= 0.7:
                    z = int(rng.integers(C))
                zl[t, b, kvh] = z
                kn[t, b, kvh] = cen[z] + 0.3 * rng.standard_normal(d)
                vn[t, b, kvh] = rng.standard_normal(d)
                for j in range(G):
                    other = int(rng.integers(C - 1)) if C > 1 else 0
                    if C > 1 and other >= z:
                        other += 1
                    q[t, b, kvh * G + j] = cen[z] + cen[other] + 0.3 * rng.standard_normal(d)
    return Layer(centroids=centroids, num_comms=num_comms, comm_start=comm_start,
                 comm_size=comm_size, comm_cap=comm_cap, members=members,
                 k_pages=k_pages, v_pages=v_pages, base_labels=base_labels, centres=centres,
                 q=torch.from_numpy(q).to(tdt).to(device),
                 k_new=torch.from_numpy(kn).to(tdt).to(device),
                 v_new=torch.from_numpy(vn).to(tdt).to(device), step_labels=zl)


@dataclasses.dataclass
class Prefill:
    """Prefill queries and keys of one layer (bf16, contiguous)."""
    q: torch.Tensor      # [B, n, Hq, d]
    k: torch.Tensor      # [B, n, Hkv, d]
    S: int
    scale: float


def make_prefill(seed: int, *, B: int, n: int, Hq: int, Hkv: int, d: int, S: int = 4,
                 device: str = "cpu", mean_size: float = 64.0) -> Prefill:
    """Seeded prefill Q/K with the community structure of the decode workloads.

    Per (sequence, KV head): positions S.. carry Markov-scattered community labels
    with geometric sizes (mean `mean_size`), each community a Gaussian centre;
    a key is its community's centre + 0.3 noise (sinks: plain N(0, 1)).  The query
    of head h at position i lies between the centre of its own position's
    community and that of a uniformly drawn community, + 0.3 noise (a sink
    position's own term is a random centre).  Bulk values are drawn with torch on
    `device`."""
    G = Hq // Hkv
    q = torch.empty((B, n, Hq, d), dtype=torch.bfloat16, device=device)
    k = torch.empty((B, n, Hkv, d), dtype=torch.bfloat16, device=device)
    for b in range(B):
        for kvh in range(Hkv):
            rng = _ss(seed, 5, b, kvh)
            N = max(n - S, 0)
            lab, C = geometric_partition(rng, N, mean_size)
            C = max(C, 1)
            full = np.concatenate([rng.integers(0, C, size=min(S, n)), lab]).astype(np.int64)
            other = rng.integers(0, C, size=(n, G)).astype(np.int64)
            cen = torch.from_numpy(rng.standard_normal((C, d)).astype(np.float32)).to(device)
            gk = _torch_gen(device, seed, 6, b, kvh)
            lab_t = torch.from_numpy(full).to(device)
            kn = torch.randn((n, d), generator=gk, device=device)
            rows = cen[lab_t] + 0.3 * kn
            rows[:min(S, n)] = kn[:min(S, n)]
            k[b, :, kvh] = rows.to(torch.bfloat16)
            oth = torch.from_numpy(other).to(device)
            qn = torch.randn((n, G, d), generator=gk, device=device)
            qq = 0.5 * (cen[lab_t][:, None, :] + cen[oth]) + 0.3 * qn
            q[b, :, kvh * G:(kvh + 1) * G] = qq.to(torch.bfloat16)
    return Prefill(q=q, k=k, S=S, scale=float(np.float32(1.0 / math.sqrt(d))))
