"""Host logic of bench.py that needs no GPU: the schedule figures computed
from a traced step, on a hand-made trace whose answers follow by hand."""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _task(op, layer, level):
    t = np.zeros(12, np.int32)
    t[0], t[1], t[11] = op, layer, level
    t[6] = t[8] = t[10] = -1
    return t


def test_schedule_from_trace_by_hand():
    # 4 workgroups (w and w + 2 share a compute unit), a 6-layer model (middle
    # layers 1-4): a down tile of layer 1 (level 9), a QKV tile of layer 2
    # (level 10), two attention tiles (level 11), and a claim task that spans
    # one of them (ignored)
    tasks = np.stack([_task(8, 1, 9), _task(1, 2, 10), _task(2, 2, 11), _task(2, 2, 11), _task(11, 2, 11)])
    us = 100  # ticks per microsecond
    rows = [  # task, workgroup, start, end of wait, end (microseconds)
        (0, 0, 0, 1, 3),
        (1, 1, 0, 3, 5),
        (2, 2, 1, 5, 8),
        (3, 3, 0, 6, 7),
        (4, 3, 0, 0, 7),
    ]
    tr = np.zeros((len(rows), 8), np.uint64)
    for i, (t, w, a, b, c) in enumerate(rows):
        tr[i, 0] = t | (w << 32)
        tr[i, 1], tr[i, 2], tr[i, 7] = 1000 + a * us, 1000 + b * us, 1000 + c * us
    s = bench.schedule_from_trace(tr, tasks, 6)
    assert s["traced_step_us"] == 8.0 and s["n_wg"] == 4
    assert s["wait_stall_frac"] == round(14 / 32, 4)      # 1 + 3 + 4 + 6 of 4 x 8 workgroup-us
    assert s["busy_wg_frac"] == 0.25                       # 2 + 2 + 3 + 1 of 32
    assert s["busy_cu_frac"] == 0.5                        # unit 0: [1,3] + [5,8]; unit 1: [3,5] + [6,7]; of 2 x 8
    assert s["level_us"] == {"qkv": 2.0, "attention": 3.0}
