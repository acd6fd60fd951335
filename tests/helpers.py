"""Test-side glue: turn a generated workload into the oracle's host arrays and
compare results.  Layout conversions only; no arithmetic of the method."""
from __future__ import annotations

import numpy as np
import torch

from oracle import ckv_oracle as O


def raw_np(t: torch.Tensor) -> np.ndarray:
    """Stored bytes of a bf16/fp32 tensor as numpy (bf16 -> uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    assert t.dtype == torch.float32
    return t.numpy()


def logical_kv(wl, layer):
    """[B, Hkv, max_pages*PAGE, d] raw K and V in token order, through the page table
    (a gather of whole pages where the pages live, then one copy to the host;
    unmapped pages read as zeros)."""
    pt = wl.page_table
    kp, vp = layer.k_pages, layer.v_pages
    pt = pt.to(kp.device).long()
    B, P = pt.shape
    ps = wl.page_size
    mapped = (pt >= 0)
    sel = pt.clamp(min=0).reshape(-1)

    def gather(pool):
        g = pool.index_select(0, sel).reshape(B, P, wl.Hkv, ps, wl.d)
        if not bool(mapped.all()):
            g = torch.where(mapped.reshape(B, P, 1, 1, 1), g, torch.zeros_like(g))
        return raw_np(g.permute(0, 2, 1, 3, 4).reshape(B, wl.Hkv, P * ps, wl.d))

    return gather(kp), gather(vp)


def oracle_state(wl, li=0, threads=None) -> O.OracleState:
    L = wl.layers[li]
    K, V = logical_kv(wl, L)
    return O.OracleState(B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, gpk=wl.gpk, S=wl.S,
                         centroids=L.centroids.cpu().numpy(), num_comms=L.num_comms,
                         comm_start=L.comm_start, comm_size=L.comm_size,
                         comm_cap=L.comm_cap, members=L.members, K=K, V=V,
                         seq_len=wl.seq_len0, threads=threads)


def step_inputs(wl, li, t):
    L = wl.layers[li]
    return raw_np(L.q[t]), raw_np(L.k_new[t]), raw_np(L.v_new[t])


def max_index_len(wl) -> int:
    return int(wl.S + wl.budget.max())
