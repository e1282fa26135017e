"""GPU parity of dspk_qgemm_verify against the oracle (through the C ABI).

Tolerance: per-row normwise relative error <= 2e-3 (the contract); the exact
factoring of the kernel is expected to land near 1e-6, which is printed.
Shapes span several 64-column blocks and K splits, ragged N, the smallest K,
M = 1 .. 32 (one and two 16-row MFMA tiles), all three weight formats, and at
the full projection shapes the benchmark times, sampled columns.
"""
import numpy as np
import pytest

import oracle
from speculative_decoding_verify_dspk_amd import binding, inputs
from gpuutil import (assert_rows_close, dev_act, oracle_columns, run_qgemm, torch)

pytestmark = pytest.mark.gpu


def _case(bits, n, k, m, tag="qgemm"):
    w = inputs.make_qweight(n, k, bits, tag)
    x = inputs.make_activations(m, k, tag, bits)
    return w, x


@pytest.mark.parametrize("bits", [8, 4, 3, 2, 16])
@pytest.mark.parametrize("n,k,m", [
    (2048, 2048, 6),      # the single-linear workload (anchor + 5 drafts)
    (64, 64, 1), (37, 64, 3), (1000, 320, 16), (130, 1024, 24), (96, 512, 32),
    (1024, 9728, 16),     # long K, narrow N: K split across workgroups
    (200, 2560, 17), (4096, 2560, 1), (520, 4160, 12),
])
def test_qgemm_matches_oracle(bits, n, k, m):
    print(f"qgemm bits={bits} n={n} k={k} m={m}", flush=True)
    w, x = _case(bits, n, k, m)
    ref = oracle.qlinear(x, w.codes, w.scales, w.biases, bits, n, k)
    got = run_qgemm(w, x, m)
    worst = assert_rows_close(got, ref, what=f"bits={bits} n={n} k={k} m={m}")
    print(f"  worst row normwise error {worst:.2e}")


@pytest.mark.parametrize("m", list(range(1, 33)))
def test_qgemm_every_row_count(m):
    w, x = _case(8, 300, 1024, m, "rows")
    ref = oracle.qlinear(x, w.codes, w.scales, w.biases, 8, 300, 1024)
    assert_rows_close(run_qgemm(w, x, m), ref, what=f"m={m}")


def test_qgemm_deterministic_and_grouped_equal():
    t = torch()
    k, m = 2560, 16
    ws_ = [inputs.make_qweight(n, k, 8, "grp", n) for n in (4096, 1024, 1024)]
    x = inputs.make_activations(m, k, "grp")
    dws = [binding.DeviceQWeight.upload(w) for w in ws_]
    xd = dev_act(x)
    sep = []
    for w, dw in zip(ws_, dws):
        outs = []
        for _ in range(2):
            y = t.empty((m, w.n), dtype=t.float32, device="cuda")
            wsp = binding.alloc_workspace(binding.qgemm_workspace_bytes(w.n, k, m))
            binding.qgemm_verify(dw, xd, m, y, wsp)
            outs.append(y)
        t.cuda.synchronize()
        assert t.equal(outs[0], outs[1]), "two runs differ"
        sep.append(outs[0])
    ys = [t.empty((m, w.n), dtype=t.float32, device="cuda") for w in ws_]
    need = sum(binding.qgemm_workspace_bytes(w.n, k, m) for w in ws_)
    wsp = binding.alloc_workspace(need)
    first = None
    for _ in range(3):   # the workspace is reused: its counters must come back to zero
        for y in ys:
            y.fill_(float("nan"))
        binding.qgemm_verify_grouped(dws, xd, m, ys, wsp)
        t.cuda.synchronize()
        if first is None:
            first = [y.clone() for y in ys]
        for a, b in zip(first, ys):
            assert t.equal(a, b), "grouped call not deterministic"
    # the grouped launch splits K differently, so it agrees with the separate
    # calls to rounding, and each agrees with the oracle
    for w, a, b in zip(ws_, sep, ys):
        ref = oracle.qlinear(x, w.codes, w.scales, w.biases, 8, w.n, k)
        assert_rows_close(a.cpu().numpy(), ref, what=f"separate n={w.n}")
        assert_rows_close(b.cpu().numpy(), ref, what=f"grouped n={w.n}")


def test_qgemm_bf16_output_is_rounded_fp32():
    w, x = _case(8, 777, 1024, 7, "bf16out")
    f = run_qgemm(w, x, 7)
    b = run_qgemm(w, x, 7, out_bf16=True)
    assert np.array_equal(b, inputs.f32_to_bf16_bits(f))


def test_qgemm_padded_rows_and_strided_output():
    """ldx > k and ldy > n: the padding columns of each activation row are
    never read (NaN there would show) and only n entries of each output row
    are written."""
    t = torch()
    w, x = _case(8, 300, 512, 5, "strided")
    xc = dev_act(x, ld=512 + 24)
    xc[:, 512:] = 0x7fc0             # NaN bf16 bit pattern in the padding columns
    dw = binding.DeviceQWeight.upload(w)
    y = t.full((5, 300 + 12), 123.0, dtype=t.float32, device="cuda")
    binding.qgemm_verify(dw, xc, 5, y, binding.alloc_workspace(binding.qgemm_workspace_bytes(300, 512, 5)))
    t.cuda.synchronize()
    yy = y.cpu().numpy()
    assert (yy[:, 300:] == 123.0).all()
    ref = oracle.qlinear(x, w.codes, w.scales, w.biases, 8, 300, 512)
    assert_rows_close(yy[:, :300], ref, what="strided")


SHAPES_FULL = {
    # one Qwen3-4B-shaped layer
    "qwen3-4b": [("q", 4096, 2560), ("k", 1024, 2560), ("o", 2560, 4096), ("gate", 9728, 2560),
                 ("down", 2560, 9728)],
    # one 27B-shaped layer
    "dense-27b": [("q", 5120, 5120), ("k", 1024, 5120), ("gate", 17408, 5120), ("down", 5120, 17408)],
}


@pytest.mark.parametrize("model,m", [("qwen3-4b", 1), ("qwen3-4b", 8), ("qwen3-4b", 16), ("dense-27b", 17)])
def test_qgemm_full_shapes_sampled(model, m):
    """Full-size projections in the benchmark's launch configuration; the oracle
    computes 192 sampled output columns (first, last and random ones)."""
    g = np.random.default_rng(7)
    for name, n, k in SHAPES_FULL[model]:
        print(f"full {model} {name} n={n} k={k} m={m}", flush=True)
        w = inputs.make_qweight(n, k, 8, model, 0, name)
        x = inputs.make_activations(m, k, model, name)
        got = run_qgemm(w, x, m)
        cols = np.unique(np.concatenate([[0, 1, 63, 64, n - 1], g.choice(n, 187, replace=False)]))
        ref = oracle_columns(w, x, cols)
        assert_rows_close(got[:, cols], ref, what=f"full {model} {name} m={m} (sampled columns)")


def _tiles_by_definition(w) -> np.ndarray:
    """The tiled layout written out from its definition in the packing source:
    64-column blocks, units of KU K elements, S 1 KiB slots of one 16-byte
    piece per lane (S = 8; 4 for 2-bit, 6 for 3-bit), then (scale | bias <<
    16) dwords.  2/3-bit pieces are built from the ground-truth codes."""
    bits, n, k = w.bits, w.n, w.k
    ku = {8: 128, 4: 256, 3: 256, 2: 256, 16: 64}[bits]
    ns = {2: 4, 3: 6}.get(bits, 8)
    gs = ku // 64
    nst, nb = -(-k // ku), -(-n // 64)
    unit = 1024 * ns + (0 if bits == 16 else 256 * gs)
    out = np.zeros(nb * nst * unit, np.uint8)
    if bits in (2, 3):
        q = np.zeros((n, nst * ku), np.uint32)
        q[:, :k] = w.codes_u8
    else:
        rowb = np.ascontiguousarray(w.codes).view(np.uint8).reshape(n, k * bits // 8)

    def put_dwords(dst, dwords):
        out[dst:dst + 4 * len(dwords)] = np.array(dwords, dtype=np.uint32).view(np.uint8)

    for b in range(nb):
        for u in range(nst):
            base = (b * nst + u) * unit
            for lane in range(64):
                c, j = lane % 16, lane // 16
                for t in range(4):
                    col = 64 * b + 16 * t + c
                    if col >= n:
                        continue
                    if bits in (2, 3):
                        # the lane's 16 codes of group g: K = ku*u + 64*g + 16*j + e
                        grp = [q[col, ku * u + 64 * g + 16 * j: ku * u + 64 * g + 16 * j + 16] for g in range(4)]
                        lo = [sum(int(cd & 3) << (2 * e) for e, cd in enumerate(grp[g])) for g in range(4)]
                        put_dwords(base + 1024 * t + 16 * lane, lo)
                        if bits == 3:
                            for p in range(2):
                                d = 0
                                for r in range(2):
                                    for e, cd in enumerate(grp[2 * p + r]):
                                        bit = int(cd) >> 2
                                        d |= bit << (8 * r + e if e < 8 else 16 + 8 * r + e - 8)
                                put_dwords(base + 1024 * (4 + t // 2) + 16 * lane + 4 * (2 * (t % 2) + p), [d])
                        continue
                    for hi in range(2):
                        i = 4 * hi + t
                        dst = base + 1024 * i + 16 * lane
                        if bits == 8:
                            k0 = ku * u + 64 * hi + 16 * j
                            if k0 < k:
                                out[dst:dst + 16] = rowb[col, k0:k0 + 16]
                        elif bits == 4:
                            for half in range(2):
                                k0 = ku * u + 64 * (2 * hi + half) + 16 * j
                                if k0 < k:
                                    out[dst + 8 * half:dst + 8 * half + 8] = rowb[col, k0 // 2:k0 // 2 + 8]
                        else:
                            k0 = ku * u + 16 * j + 8 * hi
                            if k0 < k:
                                out[dst:dst + 16] = rowb[col, 2 * k0:2 * k0 + 16]
            if bits == 16:
                continue
            for c in range(16):
                for g in range(gs):
                    for t in range(4):
                        col, gk = 64 * b + 16 * t + c, gs * u + g
                        if col < n and gk < k // 64:
                            d = int(w.scales[col, gk]) | (int(w.biases[col, gk]) << 16)
                            put_dwords(base + 1024 * ns + 16 * gs * c + 4 * (4 * g + t), [d])
    return out


@pytest.mark.parametrize("bits", [8, 4, 3, 2, 16])
@pytest.mark.parametrize("n,k", [(37, 320), (130, 1024), (64, 64)])
def test_pack_layout_matches_definition(bits, n, k):
    """dspk_qweight_pack is a pure byte permutation: bit-exact against the
    layout written out on the host, including the zero padding."""
    w = inputs.make_qweight(n, k, bits, "pack", n, k)
    dw = binding.DeviceQWeight.upload(w)
    got = dw.tiles.cpu().numpy()
    assert np.array_equal(got, _tiles_by_definition(w))


@pytest.fixture
def variant():
    """Force a projection decomposition for one test, then restore it."""
    prev = binding.set_projection_variant(binding.VARIANT_AUTO)
    yield binding.set_projection_variant
    binding.set_projection_variant(prev)


@pytest.mark.parametrize("which", ["streamk", "slab"])
@pytest.mark.parametrize("bits", [8, 4, 3, 2, 16])
@pytest.mark.parametrize("n,k,m", [
    (2560, 4096, 8),      # Qwen3-4B o
    (2560, 9728, 4),      # Qwen3-4B down: long K, 160 tiles
    (1000, 320, 16),      # ragged N, short last unit
    (37, 64, 3),          # a single partial tile
    (520, 4160, 17),      # two row tiles, K not a multiple of any unit
    (200, 2560, 32),
])
def test_qgemm_both_decompositions_match_oracle(variant, which, bits, n, k, m):
    """Each projection decomposition (stream-K, slab), forced, against the oracle."""
    variant(binding.VARIANT_STREAMK if which == "streamk" else binding.VARIANT_SLAB)
    print(f"{which} bits={bits} n={n} k={k} m={m}", flush=True)
    w, x = _case(bits, n, k, m, "variants")
    ref = oracle.qlinear(x, w.codes, w.scales, w.biases, bits, n, k)
    got = run_qgemm(w, x, m)
    worst = assert_rows_close(got, ref, what=f"{which} bits={bits} n={n} k={k} m={m}")
    print(f"  worst row normwise error {worst:.2e}")


@pytest.mark.parametrize("bits", [8, 16, 4])
@pytest.mark.parametrize("n,k", [(19456, 2560), (24576, 1024)])
@pytest.mark.parametrize("m", [1, 5])
def test_slab_resident_wave_counts(variant, bits, n, k, m):
    """Forced slab launches of 4.75 and 6 tiles per CU on a 256-CU device (the
    Qwen3-4B- and 9B-shaped gate/up widths), which run as five 3-wave and
    eight 2-wave workgroups per CU; the oracle computes sampled columns."""
    variant(binding.VARIANT_SLAB)
    print(f"slab bits={bits} n={n} k={k} m={m}", flush=True)
    g = np.random.default_rng(n + k + m + bits)
    w = inputs.make_qweight(n, k, bits, "slab-waves", n, k)
    x = inputs.make_activations(m, k, "slab-waves", n, k, m)
    got = run_qgemm(w, x, m)
    cols = np.unique(np.concatenate([[0, 15, 16, 63, 64, n - 1], g.choice(n, 186, replace=False)]))
    ref = oracle_columns(w, x, cols)
    assert_rows_close(got[:, cols], ref, what=f"slab bits={bits} n={n} k={k} m={m} (sampled columns)")


@pytest.mark.parametrize("bits", [8, 16])
@pytest.mark.parametrize("m", [3, 16])
def test_slab_multi_tile_workgroups_ragged_grouped(variant, bits, m):
    """Forced slab launch of a grouped call with ragged widths, 1180 tiles:
    five tiles per workgroup on a 256-CU device, so workgroups straddle the
    two weights and hold tiles past each weight's last column (which stage
    and wait but store nothing).  Both outputs against the oracle on sampled
    columns (each weight's first and last columns included), deterministic,
    columns past n untouched."""
    t = torch()
    variant(binding.VARIANT_SLAB)
    k = 2560
    print(f"slab multi-tile bits={bits} m={m}", flush=True)
    ws_ = [inputs.make_qweight(n, k, bits, "slab-multi", n, m) for n in (9800, 9000)]
    x = inputs.make_activations(m, k, "slab-multi", m)
    dws = [binding.DeviceQWeight.upload(w) for w in ws_]
    xd = dev_act(x)
    runs = []
    for _ in range(2):
        ys = [t.full((m, w.n + 8), -7.0, dtype=t.float32, device="cuda") for w in ws_]
        binding.qgemm_verify_grouped(dws, xd, m, ys, binding.alloc_workspace(
            sum(binding.qgemm_workspace_bytes(w.n, k, m) for w in ws_)))
        t.cuda.synchronize()
        runs.append([y.cpu().numpy() for y in ys])
    for a, b in zip(*runs):
        assert np.array_equal(a, b)
    g = np.random.default_rng(bits + m)
    for w, y in zip(ws_, runs[0]):
        assert (y[:, w.n:] == -7.0).all(), "columns past n were written"
        cols = np.unique(np.concatenate([[0, 15, 16, w.n - 41, w.n - 9, w.n - 8, w.n - 1],
                                         g.choice(w.n, 120, replace=False)]))
        ref = oracle_columns(w, x, cols)
        assert_rows_close(y[:, cols], ref, what=f"slab multi-tile bits={bits} n={w.n} m={m} (sampled columns)")


def test_slab_grouped_and_deterministic(variant):
    """The slab kernel on a grouped q/k/v call (the automatic choice at this
    size): deterministic, and each weight agrees with the oracle."""
    t = torch()
    variant(binding.VARIANT_AUTO)
    k, m = 2560, 8
    ws_ = [inputs.make_qweight(n, k, 8, "slabgrp", n) for n in (4096, 1024, 1024)]
    x = inputs.make_activations(m, k, "slabgrp")
    dws = [binding.DeviceQWeight.upload(w) for w in ws_]
    xd = dev_act(x)
    runs = []
    for _ in range(2):
        ys = [t.full((m, w.n), float("nan"), dtype=t.float32, device="cuda") for w in ws_]
        binding.qgemm_verify_grouped(dws, xd, m, ys, binding.alloc_workspace(
            sum(binding.qgemm_workspace_bytes(w.n, k, m) for w in ws_)))
        t.cuda.synchronize()
        runs.append([y.cpu().numpy() for y in ys])
    for a, b in zip(*runs):
        assert np.array_equal(a, b)
    for w, y in zip(ws_, runs[0]):
        assert_rows_close(y, oracle.qlinear(x, w.codes, w.scales, w.biases, 8, w.n, k), what=f"slab n={w.n}")


@pytest.mark.parametrize("n,k", [(2560, 4096), (2560, 9728), (1000, 320), (37, 64), (9728, 2560), (520, 4160)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_qgemm_dot_product_variant_matches_oracle(variant, n, k, m):
    """The vector-ALU (bf16 dot2) form of the slab kernel, forced: 8-bit
    weights at 1..4 rows, against the oracle."""
    variant(binding.VARIANT_DOT)
    w, x = _case(8, n, k, m, "dotvariant")
    ref = oracle.qlinear(x, w.codes, w.scales, w.biases, 8, n, k)
    got = run_qgemm(w, x, m)
    worst = assert_rows_close(got, ref, what=f"dot n={n} k={k} m={m}")
    print(f"dot n={n} k={k} m={m}: worst row normwise error {worst:.2e}")
