"""GPU parity at the full shapes where a workgroup walks several quads.

A projection launch is a list of quads (64 columns x four K units, one per
wave); each persistent workgroup takes a contiguous range of them.  With at
most one quad per workgroup a range is a single piece; with more, a range
crosses block boundaries, carries split pieces at both ends, cycles the LDS
sum slots and (for the head) folds many tiles into its argmax keys.  The
2/3/4-bit kernels run three workgroups per CU (768 on 256 CUs) and the
17..32-row kernels two or three, so these paths are reached only by the
large shapes below -- which are the shapes of the 9B-, 4B- and 27B-shaped
workloads:

* the 151936 x 4096 vocabulary head at 2, 3 and 4 bits (9496 quads) with
  full logits, and at 4 bits with 24 rows;
* 12288 x 4096 gate/up grouped (1536 quads) and 4096 x 12288 down at 2, 3 and
  4 bits, 8 and 17 rows;
* 4-bit K = 2560: a block's last quad holds two units, so waves 2 and 3 skip
  it -- gate/up 9728 x 2560 grouped (912 quads) and the 151936 x 2560 head
  (7122 quads);
* bf16 at 17..32 rows: the 151936 x 2560 head and a 4096 x 4096 projection
  at 24 rows (1024 quads on 512 workgroups).

Each weight is generated once per module; the oracle's logits for a head are
computed once for all the row sets that use it.
"""
import functools

import numpy as np
import pytest

import oracle
from speculative_decoding_verify_dspk_amd import binding, inputs
from gpuutil import (assert_argmax_parity, assert_rows_close, dev_act, oracle_logits_chunked, run_lmhead,
                     run_qgemm, torch)

pytestmark = pytest.mark.gpu

V = 151936


@functools.lru_cache(maxsize=None)
def _weight(n, k, bits, *labels):
    w = inputs.make_qweight(n, k, bits, "multiquad", *labels)
    return w, binding.DeviceQWeight.upload(w)


@functools.lru_cache(maxsize=None)
def _head_case(bits, hidden, rows):
    """The head, activation rows for every width in `rows`, and the oracle's
    logits of all of them (one pass over the weight)."""
    w, dw = _weight(V, hidden, bits, "head")
    xs = {m: inputs.make_activations(m, hidden, "multiquad", "head", bits, m) for m in rows}
    stacked = np.concatenate([xs[m] for m in rows])
    print(f"oracle logits of the {V}x{hidden} {bits}-bit head for {stacked.shape[0]} rows", flush=True)
    z = oracle_logits_chunked(w, stacked, chunk=8192)
    zs, r0 = {}, 0
    for m in rows:
        zs[m] = z[r0:r0 + m]
        r0 += m
    return w, dw, xs, zs


@pytest.mark.parametrize("bits,hidden,m", [(4, 4096, 8), (4, 4096, 24), (3, 4096, 8), (2, 4096, 8),
                                           (4, 2560, 8), (16, 2560, 20)])
def test_head_full_vocabulary_multi_quad(bits, hidden, m):
    rows = {4: (8, 24)}.get(bits, (m,)) if hidden == 4096 else (m,)
    w, dw, xs, zs = _head_case(bits, hidden, rows)
    print(f"head bits={bits} {V}x{hidden} m={m}", flush=True)
    ids, z = run_lmhead(w, xs[m], m, dw=dw)
    worst = assert_rows_close(z, zs[m], what=f"{bits}-bit head logits")
    print(f"  worst row normwise error {worst:.2e}")
    assert_argmax_parity(ids, zs[m], what=f"{bits}-bit head h={hidden} m={m}")
    ids2, _ = run_lmhead(w, xs[m], m, want_logits=False, dw=dw)
    assert np.array_equal(ids, ids2)


def _grouped(ws, dws, x, m):
    t = torch()
    ys = [t.empty((m, w.n), dtype=t.float32, device="cuda") for w in ws]
    need = sum(binding.qgemm_workspace_bytes(w.n, w.k, m) for w in ws)
    binding.qgemm_verify_grouped(dws, dev_act(x), m, ys, binding.alloc_workspace(need))
    t.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


@pytest.mark.parametrize("bits", [4, 3, 2])
@pytest.mark.parametrize("m", [8, 17])
def test_gate_up_grouped_and_down_multi_quad(bits, m):
    F, H = 12288, 4096
    gate, dg = _weight(F, H, bits, "gate")
    up, du = _weight(F, H, bits, "up")
    down, dd = _weight(H, F, bits, "down")
    x = inputs.make_activations(m, H, "multiquad", "mlp", bits, m)
    print(f"gate/up bits={bits} m={m}", flush=True)
    yg, yu = _grouped([gate, up], [dg, du], x, m)
    for name, w, y in (("gate", gate, yg), ("up", up, yu)):
        ref = oracle.qlinear(x, w.codes, w.scales, w.biases, bits, w.n, w.k)
        worst = assert_rows_close(y, ref, what=f"{name} bits={bits} m={m}")
        print(f"  {name} worst row normwise error {worst:.2e}")
    xd = inputs.make_activations(m, F, "multiquad", "down", bits, m)
    print(f"down bits={bits} m={m}", flush=True)
    yd = run_qgemm(down, xd, m, dw=dd)
    ref = oracle.qlinear(xd, down.codes, down.scales, down.biases, bits, H, F)
    worst = assert_rows_close(yd, ref, what=f"down bits={bits} m={m}")
    print(f"  down worst row normwise error {worst:.2e}")


@pytest.mark.parametrize("m", [8, 16, 17])
def test_4bit_skipped_last_quad_with_multi_quad_ranges(m):
    """K = 2560 at 4 bits: ten units per block, so a block's last quad has two
    and waves 2, 3 skip it -- combined with ranges of several quads."""
    F, H = 9728, 2560
    gate, dg = _weight(F, H, 4, "g2560")
    up, du = _weight(F, H, 4, "u2560")
    x = inputs.make_activations(m, H, "multiquad", "skip", m)
    yg, yu = _grouped([gate, up], [dg, du], x, m)
    for w, y in ((gate, yg), (up, yu)):
        ref = oracle.qlinear(x, w.codes, w.scales, w.biases, 4, w.n, w.k)
        assert_rows_close(y, ref, what=f"4-bit K=2560 n={w.n} m={m}")


def test_bf16_projection_two_row_tiles_multi_quad():
    m, n, k = 24, 4096, 4096
    w, dw = _weight(n, k, 16, "bf16proj")
    x = inputs.make_activations(m, k, "multiquad", "bf16proj")
    y = run_qgemm(w, x, m, dw=dw)
    ref = oracle.qlinear(x, w.codes, None, None, 16, n, k)
    worst = assert_rows_close(y, ref, what="bf16 24 rows")
    print(f"  bf16 24-row worst row normwise error {worst:.2e}")
