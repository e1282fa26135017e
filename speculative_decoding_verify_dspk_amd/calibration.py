"""Verify-cost curve measurement and its on-disk cache, for the cap policy.

The cap that maximises expected committed tokens per unit time depends on
the measured cost of a verify round at each width on this device, ROCm
release and weight format ("mlx-dspark 0.7.0", "Tuning": measured once,
cached on disk; "mlx-dspark" wiki summary, "Design decisions": keyed by
device and library versions, so that an upgrade or another format
invalidates the entry).  The curve feeds ``binding.CapController``.
"""
from __future__ import annotations

import json
import os


def cache_key(model: str, bits: int, device: str | None = None, rocm: str | None = None) -> str:
    """Key of a cached curve: device name, ROCm (HIP) version, weight format, model shape."""
    if device is None or rocm is None:
        import torch
        device = device or torch.cuda.get_device_name(0)
        rocm = rocm or str(torch.version.hip)
    return f"{device}|rocm {rocm}|{bits}-bit|{model}"


def measure_verify_curve(stack, widths, reps: int = 10, stream=None) -> list[float]:
    """Median device time (us) of one verify pass -- every projection of the
    stack's layers plus the vocabulary head with argmax -- at each width, on
    weight copy 0, launched like a serving loop (arguments marshalled once)."""
    import numpy as np
    import torch
    stream = stream or torch.cuda.current_stream()
    out = []
    for m in widths:
        layers, head = stack.prepare_round(m, 0, stream=stream)
        times = []
        for r in range(reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for f in layers:
                f()
            head()
            e1.record(stream)
            e1.synchronize()
            if r >= 2:                      # two warm-up passes per width
                times.append(e0.elapsed_time(e1) * 1e3)
        out.append(float(np.median(times)))
    return out


def load_or_measure(path: str, key: str, measure) -> list[float]:
    """The curve cached under ``key`` in the JSON file ``path``, or
    ``measure()`` stored there first."""
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    if key in data:
        return [float(x) for x in data[key]]
    curve = [float(x) for x in measure()]
    data[key] = curve
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    os.replace(tmp, path)
    return curve
