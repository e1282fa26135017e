"""The allocation-free projection entry point (dspk_qgemm_verify_grouped_noalloc).

Two calls in a row through the C ABI, the second smaller than the first, each
compared bit for bit with dspk_qgemm_verify_grouped on the same inputs (a
caller workspace) and with the oracle within the contract tolerance.  A third
call repeats the first, so the scratch left by the smaller call is reused.
"""
import numpy as np
import pytest

import oracle
from speculative_decoding_verify_dspk_amd import binding, inputs
from gpuutil import assert_rows_close, dev_act, torch

pytestmark = pytest.mark.gpu


def _case(ns, k, m, bits, tag):
    ws_ = [inputs.make_qweight(n, k, bits, "noalloc", tag, i) for i, n in enumerate(ns)]
    x = inputs.make_activations(m, k, "noalloc", tag)
    return ws_, [binding.DeviceQWeight.upload(w) for w in ws_], x


def _run(ws_, dws, x, m, noalloc):
    t = torch()
    ys = [t.full((m, w.n), float("nan"), dtype=t.float32, device="cuda") for w in ws_]
    xd = dev_act(x)
    if noalloc:
        binding.qgemm_verify_grouped_noalloc(dws, xd, m, ys)
    else:
        need = sum(binding.qgemm_workspace_bytes(w.n, w.k, m) for w in ws_)
        binding.qgemm_verify_grouped(dws, xd, m, ys, binding.alloc_workspace(need))
    t.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


def test_noalloc_matches_workspace_call_twice_then_smaller():
    t = torch()
    big = _case((4096, 1024, 1024), 2560, 16, 8, "big")        # Qwen3-4B q/k/v, grouped
    small = _case((300,), 512, 3, 4, "small")                   # one small 4-bit weight
    for label, (ws_, dws, x), m in (("first", big, 16), ("second", small, 3), ("third", big, 16)):
        print(f"noalloc {label}: n={[w.n for w in ws_]} k={ws_[0].k} m={m}", flush=True)
        got = _run(ws_, dws, x, m, noalloc=True)
        want = _run(ws_, dws, x, m, noalloc=False)
        for w, a, b in zip(ws_, got, want):
            assert np.array_equal(a, b), f"{label}: differs from the workspace call (n={w.n})"
            ref = oracle.qlinear(x, w.codes, w.scales, w.biases, w.bits, w.n, w.k)
            assert_rows_close(a, ref, what=f"{label} n={w.n}")
    t.cuda.synchronize()


def test_noalloc_rejects_calls_beyond_its_scratch():
    from speculative_decoding_verify_dspk_amd.binding import DspkError
    t = torch()
    w, dw, x = None, None, inputs.make_activations(2, 64, "noalloc", "big-n")
    n = 4096 * 64 + 1      # one column past 4096 blocks
    desc = binding.TiledDesc(n, 64, 8, 64, 0x1000)   # never read: the size check comes first
    y = t.empty((2, n), dtype=t.float32, device="cuda")

    class _W:
        pass
    fake = _W()
    fake.desc = desc
    with pytest.raises(DspkError) as e:
        binding.qgemm_verify_grouped_noalloc([fake], dev_act(x), 2, [y])
    assert e.value.code == -2
