"""GPU parity of the indexed attention (ckv_sparse_decode_attn) on logits that
stress the online softmax, against the fp64 oracle, for bf16 and fp32 K/V.

The attention kernel keeps one softmax reference per head for a wave and rescales
its sums only when a logit passes that reference by more than 2^8.  These cases
make the logits span hundreds of log2 units along the index list: rising (a new
reference at almost every 16-row group of every wave), falling (no rescale after
the first group), one spike far above the rest (every other weight underflows) and
a wide random spread.  The K rows are t_j * u plus noise for a unit direction u
and the queries lie along u, so the logit of list entry j follows t_j.  The graphs
of a case have list lengths 700, 193, 17 and 1 (several workgroups, ragged
16-row groups, a lone entry), over a shuffled page table.  Acceptance as for every
attention output: max-abs <= 2e-3 and relative L2 <= 1e-3 per head.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import ckv_oracle as O
from sparse_long_context_centroid_amd import binding as Bd

pytestmark = pytest.mark.gpu

B, HKV, G, D, PAGE, N = 2, 2, 4, 128, 16, 4096
HQ = HKV * G
LENS = [700, 193, 17, 1]  # one list per (sequence, KV head) graph
STRIDE = 704


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bd.load()


def _dev_type(x: np.ndarray, dt: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.bfloat16) if dt == "bf16" else t


def _raw(t: torch.Tensor) -> np.ndarray:
    """Stored values as the oracle takes them (bf16 as uint16 bit patterns)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def _logit_profile(mode: str, L: int, rng) -> np.ndarray:
    j = np.arange(L, dtype=np.float64)
    if mode == "rising":
        return -150.0 + 300.0 * j / max(L - 1, 1)
    if mode == "falling":
        return 150.0 - 300.0 * j / max(L - 1, 1)
    if mode == "spike":
        t = rng.normal(0.0, 1.0, L)
        t[L // 2] = 200.0
        return t
    assert mode == "wide"
    return rng.normal(0.0, 40.0, L)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["rising", "falling", "spike", "wide"])
def test_attention_extreme_logits_match_oracle(mode, dt):
    print(f"\n[case] attention softmax stress: {mode} {dt}", flush=True)
    rng = np.random.default_rng({"rising": 1, "falling": 2, "spike": 3, "wide": 4}[mode])
    scale = 1.0 / np.sqrt(D)
    u = rng.normal(size=D)
    u /= np.linalg.norm(u)
    # logical K / V per (sequence, KV head), queries along u
    K = rng.normal(0.0, 0.05, (B, HKV, N, D))
    V = rng.normal(0.0, 1.0, (B, HKV, N, D))
    q = 8.0 * u[None, None, :] + rng.normal(0.0, 0.05, (B, HQ, D))
    idx = np.zeros((B * HKV, STRIDE), np.int32)
    for g in range(B * HKV):
        b, kvh = divmod(g, HKV)
        L = LENS[g]
        pos = rng.permutation(N)[:L]
        idx[g, :L] = pos
        # logit of entry j ~ scale * 8 * t_j
        K[b, kvh, pos] += _logit_profile(mode, L, rng)[:, None] * u[None, :]
    Kt, Vt, qt = _dev_type(K, dt), _dev_type(V, dt), _dev_type(q, dt)
    # paged cache: page p of sequence b at a shuffled physical page
    pages_per_seq = N // PAGE
    perm = rng.permutation(B * pages_per_seq).astype(np.int32)
    page_table = perm.reshape(B, pages_per_seq)
    kp = torch.empty((B * pages_per_seq, HKV, PAGE, D), dtype=Kt.dtype)
    vp = torch.empty_like(kp)
    for b in range(B):
        for p in range(pages_per_seq):
            kp[page_table[b, p]] = Kt[b, :, p * PAGE:(p + 1) * PAGE]
            vp[page_table[b, p]] = Vt[b, :, p * PAGE:(p + 1) * PAGE]
    dev = torch.device("cuda")
    kd, vd = kp.to(dev), vp.to(dev)
    pt = torch.from_numpy(page_table).to(dev)
    seq_len = torch.full((B,), N, dtype=torch.int32, device=dev)
    dims = Bd.make_dims(B, HQ, HKV, D, 1, 64, 0,
                        Bd.CKV_DT_BF16 if dt == "bf16" else Bd.CKV_DT_F32)
    kv = Bd.make_kv(kd, vd, pt, PAGE, seq_len)
    il = torch.from_numpy(idx).to(dev)
    ilen = torch.tensor(LENS, dtype=torch.int32, device=dev)
    out = torch.zeros((B, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(Bd.ckv_workspace_size(dims, STRIDE), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    Bd.ckv_sparse_decode_attn(dims, qt.to(dev), kv, il, ilen, float(scale), out, ws, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = out.cpu().numpy().astype(np.float64)
    Kr, Vr, qr = _raw(Kt), _raw(Vt), _raw(qt)
    for b in range(B):
        for h in range(HQ):
            kvh = h // G
            g = b * HKV + kvh
            ref = O.attend(qr[b, h], Kr[b, kvh], Vr[b, kvh], idx[g, :LENS[g]], float(scale))
            diff = got[b, h] - ref
            rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30)
            assert np.abs(diff).max() <= 2e-3, (mode, b, h, np.abs(diff).max())
            assert rel <= 1e-3, (mode, b, h, rel)
