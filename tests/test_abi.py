"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libdspk.so loads and exports every function include/dspk.h declares;
* argument validation rejects bad calls before touching the device, with the
  documented error code and a message;
* the oracle and the HIP path share no code: neither imports the other.
"""
import ctypes
import os
import re
import subprocess

import pytest

from speculative_decoding_verify_dspk_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EINVAL, EUNSUPPORTED = -1, -2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from speculative_decoding_verify_dspk_amd import build
        build.build()
    return binding.lib()


def test_exports_every_header_symbol(lib):
    names = binding.header_symbols()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dspk_\w+)", out))
    assert set(names) <= exported
    assert lib.dspk_version() >= 100


def test_prefill_block_rows_setting(lib):
    assert binding.set_prefill_block_rows(64) == 0
    assert binding.set_prefill_block_rows(128) == 64
    with pytest.raises(binding.DspkError):
        binding.set_prefill_block_rows(96)
    assert binding.set_prefill_block_rows(0) == 128


def _desc(n=64, k=128, bits=8, group=64, tiles=0x10000):
    return binding.TiledDesc(n, k, bits, group, tiles)


def _src(n=64, k=128, bits=8, group=64, codes=0x10000, scales=0x20000, biases=0x30000):
    return binding.QWeightDesc(n, k, bits, group, codes, scales, biases)


# pointers below are never dereferenced: every call fails validation first
X, Y, WS = 0x40000, 0x50000, 0x60000


@pytest.mark.parametrize("mutate,code", [
    (dict(bits=5), EUNSUPPORTED), (dict(bits=1), EUNSUPPORTED), (dict(group=32), EUNSUPPORTED),
    (dict(k=100), EINVAL), (dict(k=0), EINVAL), (dict(n=0), EINVAL),
    (dict(tiles=0), EINVAL), (dict(tiles=0x10010), EINVAL),      # NULL, not 256-byte aligned
])
def test_qgemm_rejects_bad_weight(lib, mutate, code):
    d = _desc(**mutate)
    rc = lib.dspk_qgemm_verify(ctypes.byref(d), X, 128, 4, Y, 0, 64, WS, 1 << 20, None)
    assert rc == code
    assert lib.dspk_last_error().decode().startswith("dspk_qgemm_verify")


@pytest.mark.parametrize("mutate,code", [
    (dict(bits=6), EUNSUPPORTED), (dict(group=32), EUNSUPPORTED), (dict(k=100), EINVAL), (dict(n=0), EINVAL),
    (dict(codes=0), EINVAL), (dict(codes=0x10004), EINVAL), (dict(scales=0), EINVAL), (dict(biases=0x30001), EINVAL),
    (dict(bits=16), EINVAL),   # bf16 weights must not carry scales/biases
])
def test_pack_rejects_bad_weight(lib, mutate, code):
    d = _src(**mutate)
    assert lib.dspk_qweight_pack(ctypes.byref(d), WS, 1 << 30, None) == code
    assert lib.dspk_last_error().decode().startswith("dspk_qweight_pack")


def test_pack_sizes_and_rejects_bad_destination(lib):
    # whole units of 64 columns x (128 | 256 | 64) K elements: 8 KiB of codes plus 4 * KU bytes of
    # scale/bias dwords for the quantised formats
    assert lib.dspk_tiled_bytes(151936, 2560, 8) == 2374 * 20 * 8704 == 151936 * 2560 * 17 // 16
    assert lib.dspk_tiled_bytes(151936, 2560, 4) == 2374 * 10 * 9216 == 151936 * 2560 * 9 // 16
    assert lib.dspk_tiled_bytes(4096, 4096, 16) == 64 * 64 * 8192 == 4096 * 4096 * 2
    assert lib.dspk_tiled_bytes(37, 320, 8) == 1 * 3 * 8704                  # ragged N and K padded
    assert lib.dspk_tiled_bytes(37, 320, 4) == 1 * 2 * 9216
    assert lib.dspk_tiled_bytes(0, 64, 8) == 0 and lib.dspk_tiled_bytes(64, 100, 8) == 0
    assert lib.dspk_tiled_bytes(151936, 2560, 2) == 2374 * 10 * 5120 == 151936 * 2560 * 5 // 16
    assert lib.dspk_tiled_bytes(151936, 2560, 3) == 2374 * 10 * 7168 == 151936 * 2560 * 7 // 16
    assert lib.dspk_tiled_bytes(64, 64, 5) == 0
    d = _src(n=64, k=128)
    need = lib.dspk_tiled_bytes(64, 128, 8)
    assert lib.dspk_qweight_pack(ctypes.byref(d), WS, need - 1, None) == EINVAL
    assert lib.dspk_qweight_pack(ctypes.byref(d), WS + 16, need, None) == EINVAL
    assert lib.dspk_qweight_pack(ctypes.byref(d), None, need, None) == EINVAL


@pytest.mark.parametrize("args,code", [
    (dict(m=0), EINVAL), (dict(m=33), EINVAL),
    (dict(ldx=120), EINVAL),                   # row-major rows: ldx >= k ...
    (dict(ldx=132), EINVAL),                   # ... and a multiple of 8 (16-byte aligned rows)
    (dict(ldx=1 << 26, m=32), EUNSUPPORTED),   # rows spanning 2 GiB
    (dict(x=0), EINVAL), (dict(x=X + 8), EINVAL), (dict(ldy=32), EINVAL), (dict(dt=7), EINVAL),
    (dict(y=0), EINVAL),
])
def test_qgemm_rejects_bad_rows(lib, args, code):
    a = dict(x=X, ldx=128, m=4, y=Y, dt=0, ldy=64)
    a.update(args)
    d = _desc()
    rc = lib.dspk_qgemm_verify(ctypes.byref(d), a["x"], a["ldx"], a["m"], a["y"], a["dt"], a["ldy"],
                               WS, 1 << 20, None)
    assert rc == code


def test_qgemm_workspace_contract(lib):
    # every call needs a workspace (arrival counters and split partial sums)
    for n, k, m in ((151936, 2560, 16), (1024, 9728, 16), (64, 64, 1), (4096, 4096, 32)):
        need = lib.dspk_qgemm_workspace_bytes(n, k, m)
        assert need > 256 and need % 256 == 0
    assert lib.dspk_qgemm_workspace_bytes(0, 64, 1) == 0
    need = lib.dspk_qgemm_workspace_bytes(1024, 9728, 16)
    d = _desc(n=1024, k=9728)
    rc = lib.dspk_qgemm_verify(ctypes.byref(d), X, 9728, 16, Y, 0, 1024, WS, 256, None)
    assert rc == EINVAL and "workspace" in lib.dspk_last_error().decode()
    rc = lib.dspk_qgemm_verify(ctypes.byref(d), X, 9728, 16, Y, 0, 1024, WS + 16, need, None)
    assert rc == EINVAL


def test_workspace_for_m_rows_serves_every_narrower_width(lib):
    # one buffer follows a varying draft length: the size queried at the
    # widest width is enough at every width below it (narrower launches run
    # more workgroups, so this is not automatic)
    for n, k in ((151936, 5120), (5120, 17408), (1024, 5120), (2560, 9728)):
        for m in (1, 8, 16, 17, 24, 32):
            big = lib.dspk_qgemm_workspace_bytes(n, k, m)
            assert all(lib.dspk_qgemm_workspace_bytes(n, k, mm) <= big for mm in range(1, m + 1))
    for v in (151936, 8192, 1000):
        for m in (1, 16, 17, 32):
            big = lib.dspk_lmhead_workspace_bytes(v, m)
            assert all(lib.dspk_lmhead_workspace_bytes(v, mm) <= big for mm in range(1, m + 1))


def test_workspace_offsets_do_not_depend_on_the_call(lib):
    # the counters and keys sit at fixed offsets (the partial-sum region is
    # sized for the largest grid), so one buffer serves any projection or head
    # call: the size depends on the column count only
    for n in (1, 64, 1000, 9728, 151936):
        sizes = {lib.dspk_qgemm_workspace_bytes(n, k, m) for k in (64, 2560, 17408) for m in (1, 16, 17, 32)}
        sizes |= {lib.dspk_lmhead_workspace_bytes(n, m) for m in (1, 8, 32)}
        assert len(sizes) == 1, (n, sizes)
    # 16 bytes of counters per 64 columns on top of a fixed part
    a, b = lib.dspk_qgemm_workspace_bytes(64 * 1024, 64, 1), lib.dspk_qgemm_workspace_bytes(64 * 2048, 64, 1)
    assert b - a == 16 * 1024


def test_grouped_rejects_mismatch(lib):
    ds = (binding.TiledDesc * 2)(_desc(k=128), _desc(k=256))
    ys = (ctypes.c_void_p * 2)(Y, Y)
    ld = (ctypes.c_int64 * 2)(64, 64)
    assert lib.dspk_qgemm_verify_grouped(2, ds, X, 256, 4, ys, 0, ld, WS, 1 << 20, None) == EINVAL
    assert lib.dspk_qgemm_verify_grouped(0, ds, X, 256, 4, ys, 0, ld, WS, 1 << 20, None) == EINVAL
    assert lib.dspk_qgemm_verify_grouped(5, ds, X, 256, 4, ys, 0, ld, WS, 1 << 20, None) == EINVAL


def test_lmhead_rejects(lib):
    d = _desc(n=1000, k=128)
    assert lib.dspk_lmhead_argmax(ctypes.byref(d), X, 128, 4, Y, None, 0, None, 0, None) == EINVAL
    assert lib.dspk_lmhead_argmax(ctypes.byref(d), X, 128, 4, Y, Y, 999, WS, 4096, None) == EINVAL
    need = lib.dspk_lmhead_workspace_bytes(1000, 4)
    assert need >= 256 + 4 * 32 * 8
    assert lib.dspk_lmhead_argmax(ctypes.byref(d), X, 128, 4, Y, None, 0, WS, need - 8, None) == EINVAL
    assert lib.dspk_lmhead_argmax(ctypes.byref(d), X, 128, 40, Y, None, 0, WS, 1 << 20, None) == EINVAL


def test_fused_head_accept_rejects(lib):
    d = _desc(n=1000, k=128)
    need = lib.dspk_lmhead_workspace_bytes(1000, 32)
    f = lib.dspk_lmhead_argmax_accept_greedy
    # rows: b * m_rows must lie in 1..32
    assert f(ctypes.byref(d), X, 128, 0, 4, Y, None, 0, X, Y, Y, WS, need, None) == EINVAL
    assert f(ctypes.byref(d), X, 128, 4, 9, Y, None, 0, X, Y, Y, WS, need, None) == EINVAL
    assert f(ctypes.byref(d), X, 128, 1, 33, Y, None, 0, X, Y, Y, WS, need, None) == EINVAL
    # acceptance pointers
    assert f(ctypes.byref(d), X, 128, 2, 4, Y, None, 0, None, Y, Y, WS, need, None) == EINVAL
    assert f(ctypes.byref(d), X, 128, 2, 4, Y, None, 0, X, None, Y, WS, need, None) == EINVAL
    assert f(ctypes.byref(d), X, 128, 2, 4, Y, None, 0, X, Y, None, WS, need, None) == EINVAL
    # the head's own checks still apply (workspace too small)
    assert f(ctypes.byref(d), X, 128, 2, 4, Y, None, 0, X, Y, Y, WS, 64, None) == EINVAL
    assert "workspace" in lib.dspk_last_error().decode()


def test_accept_rejects(lib):
    assert lib.dspk_accept_greedy(X, X, 0, 4, Y, Y, None) == EINVAL
    assert lib.dspk_accept_greedy(X, X, 1, 33, Y, Y, None) == EINVAL
    assert lib.dspk_accept_greedy(X, None, 1, 4, Y, Y, None) == EINVAL
    need = lib.dspk_sample_workspace_bytes(151936, 17)
    assert need > 0
    ok = dict(z=X, ldz=1000, q=X, ldq=1000, d=X, u=X, rows=4, v=1000, T=1.0, ws=WS, wsb=need)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.dspk_accept_sample(a["z"], a["ldz"], a["q"], a["ldq"], a["d"], a["u"], a["rows"], a["v"],
                                      a["T"], Y, Y, a["ws"], a["wsb"], None)
    assert call(T=0.0) == EINVAL
    assert call(T=float("nan")) == EINVAL
    assert call(T=float("inf")) == EINVAL
    assert call(rows=1) == EINVAL
    assert call(rows=33) == EINVAL
    assert call(ldz=999) == EINVAL
    assert call(wsb=16) == EINVAL
    assert call(z=X + 2) == EINVAL


def test_accept_sample_ex_rejects(lib):
    need = lib.dspk_sample_workspace_bytes(1000, 4)

    def call(params=True, counts=None, **kw):
        sp = binding.sample_params(**{**dict(temperature=1.0), **kw})
        return lib.dspk_accept_sample_ex(X, 1000, X, 1000, X, X, 4, 1000, ctypes.byref(sp) if params else None,
                                         counts, Y, Y, WS, need, None)
    assert call(params=False) == EINVAL
    assert call(temperature=0.0) == EINVAL
    assert call(temperature=float("inf")) == EINVAL
    assert call(top_k=-1) == EINVAL
    assert call(top_p=0.0) == EINVAL
    assert call(top_p=1.5) == EINVAL
    assert call(top_p=float("nan")) == EINVAL
    assert call(presence=float("nan")) == EINVAL
    assert call(frequency=float("inf")) == EINVAL
    assert call(counts=X + 2) == EINVAL
    # the truncation records live in the same workspace query
    assert lib.dspk_sample_workspace_bytes(151936, 32) > lib.dspk_sample_workspace_bytes(151936, 2)


def _imports(path):
    src = open(path).read()
    return set(re.findall(r"^\s*(?:from|import)\s+([\w\.]+)", src, re.M))


def test_oracle_and_hip_path_are_independent():
    pkg = os.path.join(ROOT, "speculative_decoding_verify_dspk_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            p = os.path.join(dirpath, f)
            if f.endswith(".py"):
                assert not any(m.split(".")[0] == "oracle" for m in _imports(p)), p
            if f.endswith((".hip", ".cpp", ".h")):
                assert "oracle" not in open(p).read().lower(), p
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            mods = _imports(os.path.join(ROOT, "oracle", f))
            assert not any(m.startswith("speculative_decoding_verify_dspk_amd") for m in mods), f
