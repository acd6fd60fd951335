"""Host logic of the ctypes binding, without a GPU: the fused-step call marshals a
layer's own buffers once and reuses them while the same objects stay in place, and
marshals afresh when one of them is replaced.  A stand-in library records the
arguments each call would pass to ckv_decode_step."""
from __future__ import annotations

import ctypes as C

import pytest
import torch

from sparse_long_context_centroid_amd import binding as Bd


class _FakeLib:
    def __init__(self):
        self.calls = []

    def ckv_decode_step(self, *args):
        self.calls.append(args)
        return Bd.CKV_OK


@pytest.fixture
def fake(monkeypatch):
    lib = _FakeLib()
    monkeypatch.setattr(Bd, "load", lambda *a, **k: lib)
    # pointers stand for the tensors they come from (no device memory here)
    monkeypatch.setattr(Bd, "_ptr", lambda t: None if t is None else ("ptr", id(t)))
    monkeypatch.setattr(Bd, "_stream", lambda s=None: "stream")
    return lib


def _layer():
    lay = object.__new__(Bd.DecodeLayer)
    lay.dims = Bd.make_dims(1, 4, 1, 64, 1, 64, 4, Bd.CKV_DT_F32)
    lay.graphs = Bd.ckv_graphs()
    lay.kv = Bd.ckv_kv()
    lay.M = 8
    i32 = dict(dtype=torch.int32)
    lay.budget = torch.zeros(1, **i32)
    lay.scores = torch.zeros(1, 64)
    lay.index_list = torch.zeros(1, 300, **i32)
    lay.index_len = torch.zeros(1, **i32)
    lay.num_selected = torch.zeros(1, **i32)
    lay.cand = torch.zeros(1, 8, **i32)
    lay.selected = torch.zeros(1, 64, dtype=torch.uint8)
    lay.assigned = torch.zeros(1, **i32)
    lay.out = torch.zeros(1, 4, 64)
    lay.ws = torch.zeros(4096, dtype=torch.uint8)
    lay.err = torch.zeros(1, **i32)
    return lay


def test_fused_step_arguments_follow_the_layer(fake):
    lay = _layer()
    q, kn, vn = torch.zeros(4, 64), torch.zeros(1, 64), torch.zeros(1, 64)
    lay.step_fused(q, kn, vn, 0.125)
    lay.step_fused(q, kn, vn, 0.25)
    a, b = fake.calls
    assert len(a) == 23 and len(b) == 23
    # the per-call arguments: q, k_new, v_new, the scale, the stream
    assert a[1:4] == (("ptr", id(q)), ("ptr", id(kn)), ("ptr", id(vn)))
    assert (a[8], b[8]) == (0.125, 0.25) and a[22] == "stream"
    # the layer's own arguments, in ckv_decode_step's order, reused as the same objects
    assert a[9] == ("ptr", id(lay.scores)) and a[10] == ("ptr", id(lay.index_list))
    assert a[11] == 300 and a[7] == 8
    assert a[17] == ("ptr", id(lay.out)) and a[18] == ("ptr", id(lay.ws))
    assert a[19] == lay.ws.numel() and a[20] == ("ptr", id(lay.err)) and a[21] is None
    assert all(x is y for x, y in zip(a[4:8], b[4:8])) and all(x is y for x, y in zip(a[9:22], b[9:22]))
    # a replaced buffer is marshalled afresh (and the others stay what they were)
    old_out = lay.out
    lay.out = torch.zeros(1, 4, 64)
    lay.index_list = torch.zeros(1, 500, dtype=torch.int32)
    lay.step_fused(q, kn, vn, 0.25)
    c = fake.calls[-1]
    assert c[17] == ("ptr", id(lay.out)) and c[17] != ("ptr", id(old_out))
    assert c[10] == ("ptr", id(lay.index_list)) and c[11] == 500
    assert c[9] == a[9] and c[18] == a[18]
    # so is a replaced struct (a byref of the new one)
    lay.kv = Bd.ckv_kv()
    lay.step_fused(q, kn, vn, 0.25)
    d = fake.calls[-1]
    assert d[5] is not c[5]
    assert C.addressof(d[5]._obj) == C.addressof(lay.kv)


def test_fused_step_with_events_takes_the_marshalling_path(fake, monkeypatch):
    lay = _layer()
    seen = {}
    monkeypatch.setattr(Bd, "ckv_decode_step", lambda *a, **k: seen.update(events=k["events"]))
    ev = ["e"] * 8
    lay.step_fused(torch.zeros(4, 64), torch.zeros(1, 64), torch.zeros(1, 64), 1.0, events=ev)
    assert seen["events"] is ev and not fake.calls
