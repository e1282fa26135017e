"""GPU parity of dspk_qgemm_prefill (the wide-row projection) against the
oracle's x . deq(W)^T (through the C ABI).

Tolerance: per-row normwise relative error <= 2e-3 (the contract), as for the
verify projection.  Shapes: ragged rows (not a multiple of the 128-row block)
and columns (not a multiple of 64, an odd number of 64-column blocks), the
smallest K, a short last K unit, padded leading dimensions, bf16 output,
every weight format; at a full projection shape with 2048 rows, sampled rows.
"""
import numpy as np
import pytest

import oracle
from speculative_decoding_verify_dspk_amd import binding, inputs
from gpuutil import assert_rows_close, dev_u16, torch

pytestmark = pytest.mark.gpu


def run_prefill(w, x_bits, m, ldx=None, ldy=None, out_bf16=False, dw=None, workspace=None):
    t = torch()
    dw = dw or binding.DeviceQWeight.upload(w)
    k = w.k
    ldx = ldx or k
    xp = np.zeros((m, ldx), np.uint16)
    xp[:, :k] = x_bits
    x = dev_u16(xp)
    ldy = ldy or w.n
    y = t.full((m, ldy), -7, dtype=t.int16 if out_bf16 else t.float32, device="cuda")
    binding.qgemm_prefill(dw, x, m, y, workspace=workspace)
    t.cuda.synchronize()
    r = y.cpu().numpy()
    assert (r[:, w.n:] == -7).all(), "columns past n were written"
    r = r[:, :w.n]
    if out_bf16:
        r = inputs.bf16_bits_to_f32(np.ascontiguousarray(r).view(np.uint16))
    return r


@pytest.mark.parametrize("bits", [8, 4, 3, 2, 16])
@pytest.mark.parametrize("n,k,m", [
    (64, 64, 1), (37, 320, 130), (200, 1024, 300), (130, 2560, 129), (520, 4160, 64), (1000, 512, 257),
])
def test_prefill_matches_oracle(bits, n, k, m):
    print(f"prefill bits={bits} n={n} k={k} m={m}", flush=True)
    w = inputs.make_qweight(n, k, bits, "prefill", n, k)
    x = inputs.make_activations(m, k, "prefill", m, k)
    ref = oracle.qlinear(x, w.codes, w.scales, w.biases, bits, n, k)
    worst = assert_rows_close(run_prefill(w, x, m), ref, what=f"bits={bits} n={n} k={k} m={m}")
    print(f"  worst row normwise error {worst:.2e}")


def test_prefill_padded_strides_and_bf16_output():
    n, k, m = 300, 640, 200
    w = inputs.make_qweight(n, k, 8, "prefill-ld")
    x = inputs.make_activations(m, k, "prefill-ld")
    ref = oracle.qlinear(x, w.codes, w.scales, w.biases, 8, n, k)
    assert_rows_close(run_prefill(w, x, m, ldx=k + 24, ldy=n + 5), ref, what="padded")
    got = run_prefill(w, x, m, out_bf16=True)
    # bf16 output: the fp32 result rounded once (<= 2^-9 relative per element)
    assert_rows_close(got, ref, rtol=2e-3 + 2 ** -8, what="bf16 out", design=None)   # rounded to bf16


def test_prefill_deterministic():
    t = torch()
    n, k, m = 700, 2560, 300
    w = inputs.make_qweight(n, k, 4, "prefill-det")
    x = inputs.make_activations(m, k, "prefill-det")
    dw = binding.DeviceQWeight.upload(w)
    a = run_prefill(w, x, m, dw=dw)
    b = run_prefill(w, x, m, dw=dw)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("bits,n,k", [
    (8, 9728, 2560), (4, 9728, 2560), (16, 9728, 2560),     # gate: 128-row blocks
    (8, 1024, 2560), (4, 2560, 9728),                       # k/v and down: 64-row blocks
])
def test_prefill_full_shape_sampled_rows(bits, n, k):
    """Qwen3-4B projections over 2048 prompt rows on the device, with the
    row block chosen automatically; the oracle recomputes 12 sampled rows in
    full."""
    t = torch()
    m = 2048
    print(f"prefill full shape bits={bits} n={n} k={k}", flush=True)
    w = inputs.make_qweight(n, k, bits, "prefill-full")
    x = inputs.make_activations(m, k, "prefill-full")
    got = run_prefill(w, x, m)
    rows = np.unique(np.concatenate([[0, 127, 128, m - 1], np.random.default_rng(3).integers(0, m, 8)]))
    ref = oracle.qlinear(x[rows], w.codes, w.scales, w.biases, bits, n, k)
    assert_rows_close(got[rows], ref, what=f"bits={bits} sampled rows")
    assert np.isfinite(got).all()


@pytest.mark.parametrize("bits", [8, 4, 3, 2, 16])
def test_prefill_row_blocks_identical(bits):
    """64-row and 128-row output blocks walk K in the same order, so forcing
    either gives bit-identical results (ragged rows and columns, a short last
    K unit); both match the oracle."""
    n, k, m = 200, 1088, 300
    print(f"prefill row blocks bits={bits}", flush=True)
    w = inputs.make_qweight(n, k, bits, "prefill-blocks")
    x = inputs.make_activations(m, k, "prefill-blocks")
    dw = binding.DeviceQWeight.upload(w)
    prev = binding.set_prefill_block_rows(64)
    try:
        a = run_prefill(w, x, m, dw=dw)
        binding.set_prefill_block_rows(128)
        b = run_prefill(w, x, m, dw=dw)
    finally:
        binding.set_prefill_block_rows(prev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ref = oracle.qlinear(x, w.codes, w.scales, w.biases, bits, n, k)
    assert_rows_close(a, ref, what=f"bits={bits} row blocks")


def _workspace(n, k, m, bits):
    need = binding.prefill_workspace_bytes(n, k, m, bits)
    assert need > 0, "this shape is expected to split K"
    return binding.alloc_workspace(need)


@pytest.mark.parametrize("bits", [8, 4, 3, 2, 16])
@pytest.mark.parametrize("n,k,m", [(200, 4160, 300), (130, 4096, 129), (64, 4096, 1), (520, 8256, 64)])
def test_prefill_split_k_matches_oracle(bits, n, k, m):
    """With a workspace, launches with few output blocks split K over up to
    four workgroups and the last arrival adds the partial blocks in split
    order: matches the oracle, deterministic, and the counters are left
    zero (the same buffer serves the next call)."""
    print(f"prefill split-K bits={bits} n={n} k={k} m={m}", flush=True)
    w = inputs.make_qweight(n, k, bits, "prefill-split", n, k)
    x = inputs.make_activations(m, k, "prefill-split", m, k)
    dw = binding.DeviceQWeight.upload(w)
    ws = _workspace(n, k, m, bits)
    a = run_prefill(w, x, m, dw=dw, workspace=ws)
    b = run_prefill(w, x, m, dw=dw, workspace=ws)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ref = oracle.qlinear(x, w.codes, w.scales, w.biases, bits, n, k)
    assert_rows_close(a, ref, what=f"split-K bits={bits} n={n} k={k} m={m}")


def test_prefill_split_k_workspace_shared_across_shapes():
    """One zero-filled buffer, sized for the largest call, serves calls of
    different shapes in a row (each leaves its arrival counters zero); bf16
    output included."""
    shapes = [(200, 2176, 300, 8), (130, 4096, 129, 4), (64, 1024, 1, 16), (200, 2176, 300, 8)]
    ws = binding.alloc_workspace(max(binding.prefill_workspace_bytes(n, k, m, b) for n, k, m, b in shapes))
    for i, (n, k, m, bits) in enumerate(shapes):
        w = inputs.make_qweight(n, k, bits, "prefill-share", i)
        x = inputs.make_activations(m, k, "prefill-share", i)
        ref = oracle.qlinear(x, w.codes, w.scales, w.biases, bits, n, k)
        assert_rows_close(run_prefill(w, x, m, workspace=ws), ref, what=f"shared workspace call {i}")
        got = run_prefill(w, x, m, workspace=ws, out_bf16=True)
        assert_rows_close(got, ref, rtol=2e-3 + 2 ** -8, what=f"shared workspace call {i}, bf16 out", design=None)


def test_prefill_split_k_counters_stay_put_across_block_counts():
    """Calls of 40, 60 and again 40 split output blocks share one buffer:
    the arrival counters sit at a place that does not depend on the call,
    so a call with more blocks never counts on the partial sums an earlier
    call with fewer blocks left behind (a counter region sized per call
    overlapped them)."""
    k, m, bits = 2176, 300, 8
    ns = (1000, 1500, 1000)
    ws = binding.alloc_workspace(max(binding.prefill_workspace_bytes(n, k, m, bits) for n in ns))
    for i, n in enumerate(ns):
        w = inputs.make_qweight(n, k, bits, "prefill-ctr", n)
        x = inputs.make_activations(m, k, "prefill-ctr", i)
        ref = oracle.qlinear(x, w.codes, w.scales, w.biases, bits, n, k)
        assert_rows_close(run_prefill(w, x, m, workspace=ws), ref, what=f"call {i} (n={n})")


@pytest.mark.parametrize("bits,n,k", [(8, 2560, 4096), (16, 2560, 9728), (3, 2560, 9728), (4, 2560, 9728)])
def test_prefill_split_k_full_shape_sampled_rows(bits, n, k):
    """Qwen3-4B o and down projections over 2048 rows with a workspace: 320
    128-row output blocks, K split three ways; the oracle recomputes sampled
    rows."""
    m = 2048
    print(f"prefill split-K full shape bits={bits} n={n} k={k}", flush=True)
    w = inputs.make_qweight(n, k, bits, "prefill-split-full")
    x = inputs.make_activations(m, k, "prefill-split-full")
    got = run_prefill(w, x, m, workspace=_workspace(n, k, m, bits))
    rows = np.unique(np.concatenate([[0, 127, 128, m - 1], np.random.default_rng(5).integers(0, m, 8)]))
    ref = oracle.qlinear(x[rows], w.codes, w.scales, w.biases, bits, n, k)
    assert_rows_close(got[rows], ref, what=f"split-K bits={bits} sampled rows")
    assert np.isfinite(got).all()


def test_prefill_rejects_bad_arguments():
    t = torch()
    w = inputs.make_qweight(64, 128, 8, "prefill-bad")
    dw = binding.DeviceQWeight.upload(w)
    x = t.zeros((4, 128), dtype=t.int16, device="cuda")
    y = t.zeros((4, 64), dtype=t.float32, device="cuda")
    with pytest.raises(binding.DspkError):
        binding.qgemm_prefill(dw, x, 0, y)
    with pytest.raises(binding.DspkError):
        binding.qgemm_prefill(dw, t.zeros((4, 120), dtype=t.int16, device="cuda"), 4, y)   # ldx < k
    with pytest.raises(binding.DspkError):
        binding.qgemm_prefill(dw, t.zeros((4, 132), dtype=t.int16, device="cuda"), 4, y)   # ldx % 8
    # a workspace shorter than the K split needs
    w2 = inputs.make_qweight(64, 2048, 8, "prefill-bad-ws")
    dw2 = binding.DeviceQWeight.upload(w2)
    x2 = t.zeros((4, 2048), dtype=t.int16, device="cuda")
    need = binding.prefill_workspace_bytes(64, 2048, 4, 8)
    assert need > 0
    with pytest.raises(binding.DspkError):
        binding.qgemm_prefill(dw2, x2, 4, y, workspace=binding.alloc_workspace(need)[: need - 1])
