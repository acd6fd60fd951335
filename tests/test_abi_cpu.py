"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, sizes workspaces, and rejects bad arguments before any HIP call.
No call here passes validation, so nothing is ever launched."""
from __future__ import annotations

import ctypes as C
import os
import re

import pytest

from sparse_long_context_centroid_amd import binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ckv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(Bd.LIB_PATH):
        from sparse_long_context_centroid_amd import build
        build.build()
    return Bd.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ckv_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    decl = _declared()
    assert set(decl) == set(Bd.EXPORTED), decl
    out = os.popen(f"nm -D --defined-only {Bd.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (ckv_\w+)", out))
    assert set(decl) <= exported
    # nothing else leaks out of the library's C++ internals
    assert not re.search(r"\bT _ZN3ckv", out)


def dims(**kw):
    d = dict(B=1, Hq=32, Hkv=8, d=128, gpk=1, Cmax=2048, S=4, dtype=Bd.CKV_DT_BF16)
    d.update(kw)
    return Bd.make_dims(d["B"], d["Hq"], d["Hkv"], d["d"], d["gpk"], d["Cmax"], d["S"],
                        d["dtype"])


def test_workspace_sizes(lib):
    ok = dims(B=4)
    # partials NG*G*splits*(d+2) fp32; 4100 entries at 192 per split -> 22 splits
    ng, g, splits = 32, 4, (4100 + 191) // 192
    assert lib.ckv_workspace_size(C.byref(ok), 4100) == ng * g * splits * (128 + 2) * 4
    assert lib.ckv_workspace_size(C.byref(dims(d=96)), 4100) == 0
    assert lib.ckv_workspace_size(C.byref(ok), 0) == 0
    assert lib.ckv_workspace_size(None, 16) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), -2), (dict(Hq=30), -1), (dict(Hq=48, Hkv=4), -2), (dict(gpk=2), -1),
    (dict(Cmax=100), -1), (dict(Cmax=8256), -2), (dict(dtype=7), -2), (dict(B=0), -1),
    (dict(S=-1), -1),
])
def test_bad_dims_rejected(lib, kw, status):
    d = dims(**kw)
    fake = C.c_void_p(0x1000)
    g = Bd.ckv_graphs(fake, fake, fake, fake, fake, fake)
    r = lib.ckv_score_centroids(C.byref(d), fake, C.byref(g), 0.1, fake, None)
    assert r == status


def test_null_pointers_and_small_workspace(lib):
    d = dims()
    fake = C.c_void_p(0x1000)
    g = Bd.ckv_graphs(None, fake, fake, fake, fake, fake)           # centroids missing
    assert lib.ckv_score_centroids(C.byref(d), fake, C.byref(g), 0.1, fake, None) == -1
    g = Bd.ckv_graphs(fake, fake, fake, None, fake, fake)           # sizes missing
    assert lib.ckv_score_centroids(C.byref(d), fake, C.byref(g), 0.1, fake, None) == -1
    g = Bd.ckv_graphs(fake, fake, fake, fake, fake, fake)
    assert lib.ckv_score_centroids(C.byref(d), None, C.byref(g), 0.1, fake, None) == -1
    kv = Bd.ckv_kv(fake, fake, fake, 16, 8, 8, fake)
    assert lib.ckv_sparse_decode_attn(C.byref(d), fake, C.byref(kv), fake, 2052, fake, 0.1,
                                      fake, fake, 64, fake, None) == -3
    kv_bad = Bd.ckv_kv(fake, fake, fake, 12, 8, 8, fake)             # page size not 2^k
    assert lib.ckv_sparse_decode_attn(C.byref(d), fake, C.byref(kv_bad), fake, 2052, fake,
                                      0.1, fake, fake, 1 << 30, fake, None) == -1
    # select: n_cand out of range
    assert lib.ckv_select(C.byref(d), fake, C.byref(g), fake, fake, 0, fake, 2052, fake, None,
                          fake, None, fake, None) == -1
    assert lib.ckv_select(C.byref(d), fake, C.byref(g), fake, fake, 17, fake, 2052, fake, None,
                          fake, None, fake, None) == -1
    assert lib.ckv_local_update(C.byref(d), fake, None, fake, 8, C.byref(g), C.byref(kv), fake,
                                fake, None) == -1
    big = Bd.ckv_kv(fake, fake, fake, 16, 8, 1 << 24, fake)          # 32-bit row index overflow
    assert lib.ckv_sparse_decode_attn(C.byref(d), fake, C.byref(big), fake, 2052, fake, 0.1,
                                      fake, fake, 1 << 30, fake, None) == -2
    # fused step: workspace too small, n_cand out of range
    assert lib.ckv_decode_step(C.byref(d), fake, fake, fake, C.byref(g), C.byref(kv), fake, 8,
                               0.1, fake, fake, 2052, fake, None, fake, None, fake, fake, fake,
                               64, fake, None, None) == -3
    assert lib.ckv_decode_step(C.byref(d), fake, fake, fake, C.byref(g), C.byref(kv), fake, 0,
                               0.1, fake, fake, 2052, fake, None, fake, None, fake, fake, fake,
                               1 << 30, fake, None, None) == -1


def test_empty_member_pool_passes_validation(lib):
    """A null member pool (no community has a slot) is a valid graph set: the calls
    that take graphs reach the next check -- here a workspace that is too small, or
    a candidate count out of range -- instead of rejecting the pool."""
    d = dims()
    fake = C.c_void_p(0x1000)
    g = Bd.ckv_graphs(fake, fake, fake, fake, fake, None)
    kv = Bd.ckv_kv(fake, fake, fake, 16, 8, 8, fake)
    assert lib.ckv_decode_step(C.byref(d), fake, fake, fake, C.byref(g), C.byref(kv), fake, 8,
                               0.1, fake, fake, 2052, fake, None, fake, None, fake, fake, fake,
                               64, fake, None, None) == -3
    assert lib.ckv_select(C.byref(d), fake, C.byref(g), fake, fake, 0, fake, 2052, fake, None,
                          fake, None, fake, None) == -1
    assert lib.ckv_local_update(C.byref(d), fake, fake, fake, 0, C.byref(g), C.byref(kv), fake,
                                fake, None) == -1


def test_noalloc_step_refuses_oversized_scratch(lib):
    """ckv_decode_step_noalloc checks the step's scratch against its array's size
    before touching the device: 512 graphs x 86 splits need more than it holds."""
    d = dims(B=64)
    fake = C.c_void_p(0x1000)
    g = Bd.ckv_graphs(fake, fake, fake, fake, fake, fake)
    kv = Bd.ckv_kv(fake, fake, fake, 16, 8, 8, fake)
    assert lib.ckv_workspace_size(C.byref(d), 16388) > 32 << 20
    assert lib.ckv_decode_step_noalloc(C.byref(d), fake, fake, fake, C.byref(g), C.byref(kv),
                                       fake, 8, 0.1, fake, fake, 16388, fake, None, fake, None,
                                       fake, fake, fake, None, None) == -3
    assert lib.ckv_decode_step_noalloc(C.byref(dims(d=96)), fake, fake, fake, C.byref(g),
                                       C.byref(kv), fake, 8, 0.1, fake, fake, 16388, fake, None,
                                       fake, None, fake, fake, fake, None, None) == -2


def test_dense_entry_points_validate(lib):
    d = dims(B=4)
    fake = C.c_void_p(0x1000)
    kv = Bd.ckv_kv(fake, fake, fake, 16, 8208, 8208 * 4, fake)
    # 32 KV heads x 4 query heads, pieces of 11 chunks of 192 tokens -> 63 pieces
    assert lib.ckv_dense_workspace_size(C.byref(d), C.byref(kv)) == 32 * 4 * 63 * 130 * 4
    assert lib.ckv_dense_workspace_size(C.byref(d), None) == 0
    assert lib.ckv_dense_decode_attn(C.byref(d), None, C.byref(kv), 0.1, fake, fake, 1 << 30,
                                     fake, None) == -1
    assert lib.ckv_dense_decode_attn(C.byref(d), fake, C.byref(kv), 0.1, fake, fake, 64,
                                     fake, None) == -3
    kv_bad = Bd.ckv_kv(fake, fake, fake, 12, 8, 8, fake)
    assert lib.ckv_dense_decode_attn(C.byref(d), fake, C.byref(kv_bad), 0.1, fake, fake,
                                     1 << 30, fake, None) == -1


def test_prefill_edges_validate(lib):
    d = dims()
    fake = C.c_void_p(0x1000)
    nan = float("nan")
    # null buffers, empty prefill, topk outside 1..8, non-finite scale
    assert lib.ckv_prefill_edges(C.byref(d), None, fake, 64, 8, 0.1, fake, fake, None, None,
                                 None) == -1
    assert lib.ckv_prefill_edges(C.byref(d), fake, fake, 64, 8, 0.1, None, fake, None, None,
                                 None) == -1
    assert lib.ckv_prefill_edges(C.byref(d), fake, fake, 0, 8, 0.1, fake, fake, None, None,
                                 None) == -1
    for topk in (0, 9):
        assert lib.ckv_prefill_edges(C.byref(d), fake, fake, 64, topk, 0.1, fake, fake, None,
                                     None, None) == -1
    assert lib.ckv_prefill_edges(C.byref(d), fake, fake, 64, 8, nan, fake, fake, None, None,
                                 None) == -1
    # fp32 operands are not built for the matrix-core kernel
    f32 = dims(dtype=0)
    assert lib.ckv_prefill_edges(C.byref(f32), fake, fake, 64, 8, 0.1, fake, fake, None, None,
                                 None) == -2


def test_layer_graph_dims(lib):
    """graphs_per_kv = 0 (one graph per layer): the attention workspace is the group
    graph's (the one list feeds every KV head's G query heads); the update refuses
    candidate rows that do not fit its LDS stage; the prefill edges refuse it."""
    lay, grp = dims(B=4, gpk=0), dims(B=4, gpk=1)
    assert lib.ckv_workspace_size(C.byref(lay), 4100) == lib.ckv_workspace_size(C.byref(grp), 4100)
    fake = C.c_void_p(0x1000)
    g = Bd.ckv_graphs(fake, fake, fake, fake, fake, fake)
    kv = Bd.ckv_kv(fake, fake, fake, 16, 8, 8, fake)
    # 8 KV heads x d 128: 16 candidate rows of 1028 floats + 1024 floats > 64 KiB
    assert lib.ckv_local_update(C.byref(lay), fake, fake, fake, 16, C.byref(g), C.byref(kv),
                                fake, fake, None) == -2
    assert lib.ckv_decode_step(C.byref(lay), fake, fake, fake, C.byref(g), C.byref(kv), fake, 16,
                               0.1, fake, fake, 2052, fake, None, fake, None, fake, fake, fake,
                               1 << 30, fake, None, None) == -2
    assert lib.ckv_prefill_edges(C.byref(lay), fake, fake, 64, 8, 0.1, fake, fake, None, None,
                                 None) == -2


def test_status_strings(lib):
    for s, txt in [(0, "ok"), (-1, "invalid argument"), (-2, "unsupported configuration"),
                   (-3, "workspace missing or too small"), (-4, "HIP launch failed")]:
        assert lib.ckv_status_string(s).decode() == txt
