"""Seeded random sweep of small decode workloads through the whole path, against
the fp64 oracle: graph granularity (per KV head, per query head, per layer),
dtype, head_dim, group size, batch with ragged contexts, shuffled pages, sink
count, budget (0, small, beyond the context), candidate count and steps are drawn
per case; both the four calls and the fused step are exercised.  Every case
prints its parameters before it runs.  CKV_RANDOM_CASES sets the number of cases
(256 by default; a longer sweep draws the same first 256 and more)."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from gpu_parity import run_parity
from sparse_long_context_centroid_amd import binding as Bd
from sparse_long_context_centroid_amd import inputs as I

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("CKV_RANDOM_CASES", "256"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bd.load()


def _draw(case: int):
    r = np.random.default_rng(90_000 + case)
    d = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.choice([1, 2, 4])) if G < 8 else int(r.choice([1, 2]))
    mode = str(r.choice(["group", "head", "layer"]))
    dtype = int(r.choice([I.DT_BF16, I.DT_F32]))
    B = int(r.integers(1, 4))
    S = int(r.choice([0, 1, 4, 7]))
    contexts = [int(x) for x in r.integers(max(S, 1), 3000, size=B)]
    steps = int(r.integers(1, 4))
    budget = int(r.choice([0, 64, 300, 1 << 20]))
    M = int(r.choice([1, 3, 8, 16]))
    if mode == "layer" and Hkv * d * (8 + 4 * M) + 16 * M > 65536:
        M = 8
    spec = I.ConfigSpec(f"random-{case}", B, Hkv * G, Hkv, d, max(contexts), mode == "head",
                        budget, steps, dtype, num_sinks=S, n_cand=M,
                        shuffled_pages=bool(r.integers(2)), layer_graph=mode == "layer")
    return spec, contexts, bool(r.integers(2))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_workload_matches_oracle(case):
    spec, contexts, fused = _draw(case)
    print(f"\n[case] random {case}: {spec} contexts={contexts} fused={fused}", flush=True)
    wl = I.make_workload(spec, 31_000 + case, device="cuda", contexts=contexts)
    index_stride = int(wl.S + min(int(wl.budget.max()), max(contexts) + spec.steps))
    run_parity(wl, fused=fused, index_stride=max(index_stride, 1))
