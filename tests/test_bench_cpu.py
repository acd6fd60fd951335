"""bench.py's command-line contract that needs no GPU: more than one GPU is refused
with a message (this path runs on one GPU), and the options parse."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_help_lists_the_measurement_switches():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--gpus", "--config", "--graphs", "--no-granularity",
                 "--no-edges", "--no-dense", "--no-rebuild", "--warm", "--copy-mib"):
        assert flag in r.stdout, flag


def _fake_layer(gpk, index_list=None):
    import types
    import numpy as np
    Hkv, Hq, d, B = 2, 8, 128, 1
    NG = B if gpk == 0 else B * Hkv * gpk
    return types.SimpleNamespace(d=d, cdim=Hkv * d if gpk == 0 else d, B=B, Hq=Hq, Hkv=Hkv,
                                 gpk=gpk, NG=NG, M=8, index_list=index_list,
                                 num_comms_host=np.arange(10, 10 + 10 * NG, 10, dtype=np.int64))


def test_step_bytes_count_what_the_method_moves():
    """The algorithmic bytes behind the roofline figures, on small hand-made layers:
    centroids, sizes and scores per community; list entries; each selected K/V row
    once per KV head (for per-head graphs the union of a KV head's lists, whatever
    the overlap); the update's candidate rows and appended row; q and out."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import bench
    Bq = 1 * 8 * 128 * 2                                # q, bf16
    merge = 1 * 8 * 128 * 4                             # out, fp32
    upd_kv = 1 * 2 * 2 * 128 * 2 * 2                    # k_new, v_new read and written
    # group graphs: 2 graphs of 10 and 20 communities, lists of 100 and 50 entries
    lay = _fake_layer(1)
    by, attn = bench.step_bytes(lay, np.array([100, 50]), 2)
    assert by["score"] == 30 * (128 * 4 + 4 + 4) + Bq
    assert by["select"] == 30 * 8 + 150 * 8
    assert attn == 150 * 2 * 128 * 2 + 150 * 4 + Bq
    assert by["attn_update"] == attn + 2 * (8 * 128 * 4 + 8 * 4 + 128 * 4 * 2) + upd_kv
    assert by["merge"] == merge
    # per-head graphs: 4 lists per KV head that overlap; rows count once per KV head
    lists = torch.full((8, 4), -1, dtype=torch.int32)
    rows = [[0, 1, 2], [1, 2, 3], [5], [], [7, 8], [8], [9], [7]]
    for g, r in enumerate(rows):
        lists[g, :len(r)] = torch.tensor(r, dtype=torch.int32)
    lens = np.array([len(r) for r in rows])
    lay = _fake_layer(4, lists)
    _, attn = bench.step_bytes(lay, lens, 2)
    union = len({0, 1, 2, 3, 5}) + len({7, 8, 9})
    assert attn == union * 2 * 128 * 2 + int(lens.sum()) * 4 + Bq
    # the layer graph: one list per sequence, read by each of the 2 KV heads
    lay = _fake_layer(0)
    by, attn = bench.step_bytes(lay, np.array([40]), 2)
    assert by["score"] == 10 * (2 * 128 * 4 + 4 + 4) + Bq
    assert attn == 40 * 2 * (2 * 128 * 2 + 4) + Bq
