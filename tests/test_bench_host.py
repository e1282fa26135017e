"""Host-side logic of the benchmark (no GPU): the one-GPU guard and the wait
for a round's result words in pinned memory."""
import os
import subprocess
import sys
import threading
import time

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


class _Stream:
    def __init__(self):
        self.syncs = 0

    def synchronize(self):
        self.syncs += 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_wait_returns_once_every_entry_has_arrived():
    res = np.full(7, bench.PENDING, dtype=np.int32)

    def writer():
        # entries arrive one at a time, in no particular order
        for i in (3, 0, 6, 1, 5, 2, 4):
            time.sleep(0.002)
            res[i] = i - 1        # -1 is a legitimate committed value
    t = threading.Thread(target=writer)
    t.start()
    s = _Stream()
    bench.wait_result(res, s, spin_s=5.0)
    t.join()
    assert not (res == bench.PENDING).any()
    assert s.syncs == 0


def test_wait_falls_back_to_a_sync_and_fails_if_an_entry_never_arrives():
    res = np.full(5, bench.PENDING, dtype=np.int32)
    res[:4] = 1
    s = _Stream()
    with pytest.raises(RuntimeError):
        bench.wait_result(res, s, spin_s=0.05)
    assert s.syncs == 1
