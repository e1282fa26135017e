"""Thin ctypes binding of libdspk.so (argument marshalling only).

Every function takes torch tensors that live in HIP device memory, passes their
addresses and sizes to the C entry point of the same name, and raises
``DspkError`` on a non-zero return.  No arithmetic of the verify pass happens
here; the library must be built (``python -m
speculative_decoding_verify_dspk_amd.build``) -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

from . import inputs

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdspk.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dspk.h")

DSPK_F32, DSPK_BF16 = 0, 1
MAX_ROWS = 32
MAX_GROUPED = 4


class DspkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dspk error {code}: {msg}")
        self.code = code


class QWeightDesc(ctypes.Structure):
    """dspk_qweight: a weight in the interchange layout (input of the packing)."""
    _fields_ = [("n", c_int32), ("k", c_int32), ("bits", c_int32), ("group", c_int32),
                ("codes", c_void_p), ("scales", c_void_p), ("biases", c_void_p)]


class TiledDesc(ctypes.Structure):
    """dspk_tiled_weight: a weight in the library's tiled layout."""
    _fields_ = [("n", c_int32), ("k", c_int32), ("bits", c_int32), ("group", c_int32), ("tiles", c_void_p)]


class CapControllerDesc(ctypes.Structure):
    """dspk_cap_controller (host struct)."""
    _fields_ = [("verify_us", ctypes.c_double * MAX_ROWS), ("draft_us", ctypes.c_double * MAX_ROWS),
                ("n", c_int32), ("decay", ctypes.c_double), ("hits", ctypes.c_double),
                ("trials", ctypes.c_double), ("probe_every", c_int32), ("probe_cap", c_int32),
                ("parked_rounds", c_int32)]


class SampleParamsDesc(ctypes.Structure):
    """dspk_sample_params (host struct)."""
    _fields_ = [("temperature", c_float), ("top_k", c_int32), ("top_p", c_float),
                ("presence_penalty", c_float), ("frequency_penalty", c_float)]


def sample_params(temperature: float, top_k: int = 0, top_p: float = 1.0, presence: float = 0.0,
                  frequency: float = 0.0) -> SampleParamsDesc:
    return SampleParamsDesc(float(temperature), int(top_k), float(top_p), float(presence), float(frequency))


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libdspk.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m speculative_decoding_verify_dspk_amd.build`")
    # torch first: the library needs the HIP runtime under the soname
    # libamdhip64.so.7, and torch's ROCm wheel brings its own copy under that
    # name.  With torch loaded, the library binds to that same runtime, so the
    # streams and device pointers this binding passes (torch's) are valid in
    # it.  Loaded the other way round, the process would hold two HIP/HSA
    # runtimes and the one initialised second finds no device.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sig = {
        "dspk_version": (c_int32, []),
        "dspk_set_projection_variant": (c_int32, [c_int32]),
        "dspk_set_prefill_block_rows": (c_int32, [c_int32]),
        "dspk_last_error": (ctypes.c_char_p, []),
        "dspk_tiled_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "dspk_qweight_pack": (c_int32, [P(QWeightDesc), c_void_p, c_size_t, c_void_p]),
        "dspk_qgemm_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "dspk_qgemm_verify": (c_int32, [P(TiledDesc), c_void_p, c_int64, c_int32, c_void_p, c_int32,
                                        c_int64, c_void_p, c_size_t, c_void_p]),
        "dspk_qgemm_verify_grouped": (c_int32, [c_int32, P(TiledDesc), c_void_p, c_int64, c_int32,
                                                P(c_void_p), c_int32, P(c_int64), c_void_p, c_size_t,
                                                c_void_p]),
        "dspk_qgemm_verify_grouped_noalloc": (c_int32, [c_int32, P(TiledDesc), c_void_p, c_int64, c_int32,
                                                        P(c_void_p), c_int32, P(c_int64), c_void_p]),
        "dspk_qgemm_prefill": (c_int32, [P(TiledDesc), c_void_p, c_int64, c_int32, c_void_p, c_int32, c_int64,
                                         c_void_p, c_size_t, c_void_p]),
        "dspk_prefill_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
        "dspk_lmhead_workspace_bytes": (c_size_t, [c_int32, c_int32]),
        "dspk_lmhead_argmax": (c_int32, [P(TiledDesc), c_void_p, c_int64, c_int32, c_void_p, c_void_p,
                                         c_int64, c_void_p, c_size_t, c_void_p]),
        "dspk_lmhead_argmax_accept_greedy": (c_int32, [P(TiledDesc), c_void_p, c_int64, c_int32, c_int32,
                                                       c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                                       c_void_p, c_void_p, c_size_t, c_void_p]),
        "dspk_accept_greedy": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                         c_void_p]),
        "dspk_sample_workspace_bytes": (c_size_t, [c_int32, c_int32]),
        "dspk_accept_sample": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int32,
                                         c_int32, c_float, c_void_p, c_void_p, c_void_p, c_size_t,
                                         c_void_p]),
        "dspk_accept_sample_ex": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int32,
                                            c_int32, P(SampleParamsDesc), c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_size_t, c_void_p]),
        "dspk_choose_cap": (c_int32, [P(ctypes.c_double), P(ctypes.c_double), c_int32, ctypes.c_double,
                                      P(ctypes.c_double)]),
        "dspk_cap_init": (c_int32, [P(CapControllerDesc), P(ctypes.c_double), P(ctypes.c_double), c_int32,
                                    ctypes.c_double, ctypes.c_double, c_int32, c_int32]),
        "dspk_cap_next": (c_int32, [P(CapControllerDesc)]),
        "dspk_cap_observe": (c_int32, [P(CapControllerDesc), c_int32, c_int32]),
        "dspk_cap_alpha": (ctypes.c_double, [P(CapControllerDesc)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _LIB = L
    return L


def header_symbols() -> list[str]:
    """Names of the functions include/dspk.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dspk_[a-z_0-9]+)\s*\(", text)))


def _check(rc: int) -> None:
    if rc != 0:
        raise DspkError(rc, lib().dspk_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _rows(t, name: str) -> int:
    """Leading dimension of a row-major 2-D tensor (unit column stride)."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name}: expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _acts(t, name: str) -> int:
    """Leading dimension of row-major bf16 activation rows [rows][ld] (int16 bit
    patterns or bfloat16): unit column stride, ld % 8 == 0."""
    if t.element_size() != 2:
        raise ValueError(f"{name}: expected bf16 activations (2-byte elements)")
    ld = _rows(t, name)
    if ld % 8:
        raise ValueError(f"{name}: leading dimension {ld} must be a multiple of 8")
    return ld


# ---------------------------------------------------------------- weights
class DeviceQWeight:
    """A weight matrix in device memory, in the library's tiled layout, plus
    its C descriptor.  Built from the interchange layout (packed codes,
    row-major fp16 scales/biases [n][k/64]) by dspk_qweight_pack."""

    def __init__(self, n: int, k: int, bits: int, codes, scales=None, biases=None, stream=None):
        import torch
        self.n, self.k, self.bits = n, k, bits
        src = QWeightDesc(n, k, bits, 64, codes.data_ptr(),
                          None if scales is None else scales.data_ptr(),
                          None if biases is None else biases.data_ptr())
        nbytes = tiled_bytes(n, k, bits)
        if nbytes == 0:
            raise ValueError(f"invalid weight shape n={n} k={k} bits={bits}")
        self.tiles = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
        _check(lib().dspk_qweight_pack(ctypes.byref(src), self.tiles.data_ptr(), nbytes, _stream(stream)))
        self.desc = TiledDesc(n, k, bits, 64, self.tiles.data_ptr())

    @classmethod
    def upload(cls, w: inputs.QWeight, device="cuda"):
        import torch
        codes = torch.from_numpy(np.ascontiguousarray(w.codes.view(np.int32) if w.bits != 16
                                                      else w.codes.view(np.int16))).to(device)
        sc = bi = None
        if w.bits != 16:
            sc = torch.from_numpy(np.ascontiguousarray(w.scales.view(np.int16))).to(device)
            bi = torch.from_numpy(np.ascontiguousarray(w.biases.view(np.int16))).to(device)
        out = cls(w.n, w.k, w.bits, codes, sc, bi)
        torch.cuda.current_stream().synchronize()      # the sources may be freed now
        return out

    @property
    def nbytes(self) -> int:
        """Algorithmic bytes of the weight (codes plus fp16 scale and bias per group)."""
        return inputs.weight_bytes(self.n, self.k, self.bits)


def tiled_bytes(n: int, k: int, bits: int) -> int:
    return lib().dspk_tiled_bytes(n, k, bits)


# ------------------------------------------------------------ cap policy
def _doubles(xs):
    return None if xs is None else (ctypes.c_double * len(xs))(*[float(x) for x in xs])


def choose_cap(verify_us, draft_us, alpha: float) -> tuple[int, float]:
    """(cap, expected tokens per us) for a measured verify curve (width 1..n)."""
    rate = ctypes.c_double(0.0)
    cap = lib().dspk_choose_cap(_doubles(verify_us), _doubles(draft_us), len(verify_us), float(alpha),
                                ctypes.byref(rate))
    if cap < 0:
        raise DspkError(cap, "dspk_choose_cap: invalid curve or alpha")
    return cap, rate.value


class CapController:
    """The library's cap controller (host struct owned here)."""

    def __init__(self, verify_us, draft_us=None, decay: float = 0.9, prior_alpha: float = 0.5,
                 probe_every: int = 8, probe_cap: int = 1):
        self.st = CapControllerDesc()
        _check(lib().dspk_cap_init(ctypes.byref(self.st), _doubles(verify_us), _doubles(draft_us),
                                   len(verify_us), decay, prior_alpha, probe_every, probe_cap))

    def next_cap(self) -> int:
        return lib().dspk_cap_next(ctypes.byref(self.st))

    def observe(self, drafted: int, accepted: int) -> None:
        _check(lib().dspk_cap_observe(ctypes.byref(self.st), drafted, accepted))

    def alpha(self) -> float:
        return lib().dspk_cap_alpha(ctypes.byref(self.st))


# ------------------------------------------------------- prepared launches
_CARG = type(ctypes.byref(ctypes.c_int()))


class Prepared:
    """One entry-point call with every argument already marshalled: calling it
    is a single foreign call (no Python-side conversion), for rounds that
    repeat the same launches with the same buffers."""

    def __init__(self, name: str, *args):
        self.name = name
        self.fn = getattr(lib(), name)
        conv = []
        for t, a in zip(self.fn.argtypes, args):
            if a is None or isinstance(a, (ctypes._SimpleCData, ctypes.Array, _CARG)):
                conv.append(a)                   # NULL, or already a ctypes object
            else:
                conv.append(t(a))                # plain int / float -> its C type, once
        self.args = tuple(conv)
        self.keep = args            # descriptors and arrays the pointers refer to

    def __call__(self) -> None:
        rc = self.fn(*self.args)
        if rc != 0:
            _check(rc)


def prepare_qgemm(w: DeviceQWeight, x, m: int, y, workspace, stream=None) -> Prepared:
    dt = DSPK_BF16 if y.element_size() == 2 else DSPK_F32
    return Prepared("dspk_qgemm_verify", ctypes.byref(w.desc), x.data_ptr(), _acts(x, "x"), m, y.data_ptr(), dt,
                    _rows(y, "y"), workspace.data_ptr(), workspace.numel(), _stream(stream))


def prepare_qgemm_grouped(ws: list, x, m: int, ys: list, workspace, stream=None) -> Prepared:
    cnt = len(ws)
    descs = (TiledDesc * cnt)(*[w.desc for w in ws])
    yptr = (c_void_p * cnt)(*[y.data_ptr() for y in ys])
    ldy = (c_int64 * cnt)(*[_rows(y, "y") for y in ys])
    dt = DSPK_BF16 if ys[0].element_size() == 2 else DSPK_F32
    return Prepared("dspk_qgemm_verify_grouped", cnt, descs, x.data_ptr(), _acts(x, "x"), m, yptr, dt, ldy,
                    workspace.data_ptr(), workspace.numel(), _stream(stream))


def prepare_lmhead(w: DeviceQWeight, h, m: int, argmax, logits, workspace, stream=None) -> Prepared:
    return Prepared("dspk_lmhead_argmax", ctypes.byref(w.desc), h.data_ptr(), _acts(h, "h"), m, argmax.data_ptr(),
                    _ptr(logits), 0 if logits is None else _rows(logits, "logits"), workspace.data_ptr(),
                    workspace.numel(), _stream(stream))


def prepare_lmhead_accept_greedy(w: DeviceQWeight, h, b: int, m_rows: int, argmax, logits, draft_ids, accept_len,
                                 committed, workspace, stream=None) -> Prepared:
    return Prepared("dspk_lmhead_argmax_accept_greedy", ctypes.byref(w.desc), h.data_ptr(), _acts(h, "h"), b,
                    m_rows, argmax.data_ptr(), _ptr(logits), 0 if logits is None else _rows(logits, "logits"),
                    _ptr(draft_ids), accept_len.data_ptr(), committed.data_ptr(), workspace.data_ptr(),
                    workspace.numel(), _stream(stream))


def prepare_accept_greedy(target_ids, draft_ids, b: int, m_rows: int, accept_len, committed,
                          stream=None) -> Prepared:
    return Prepared("dspk_accept_greedy", target_ids.data_ptr(), _ptr(draft_ids), b, m_rows, accept_len.data_ptr(),
                    committed.data_ptr(), _stream(stream))


def prepare_accept_sample(logits, q, draft_ids, uniforms, m_rows: int, v: int, temperature: float, accept_len,
                          committed, workspace, stream=None) -> Prepared:
    return Prepared("dspk_accept_sample", logits.data_ptr(), _rows(logits, "logits"), q.data_ptr(), _rows(q, "q"),
                    draft_ids.data_ptr(), uniforms.data_ptr(), m_rows, v, float(temperature),
                    accept_len.data_ptr(), committed.data_ptr(), workspace.data_ptr(), workspace.numel(),
                    _stream(stream))


def prepare_accept_sample_ex(logits, q, draft_ids, uniforms, m_rows: int, v: int, params: SampleParamsDesc,
                             counts, accept_len, committed, workspace, stream=None) -> Prepared:
    return Prepared("dspk_accept_sample_ex", logits.data_ptr(), _rows(logits, "logits"), q.data_ptr(),
                    _rows(q, "q"), draft_ids.data_ptr(), uniforms.data_ptr(), m_rows, v, ctypes.byref(params),
                    _ptr(counts), accept_len.data_ptr(), committed.data_ptr(), workspace.data_ptr(),
                    workspace.numel(), _stream(stream))


# ------------------------------------------------------------ entry points
def version() -> int:
    return lib().dspk_version()


VARIANT_AUTO, VARIANT_STREAMK, VARIANT_SLAB, VARIANT_DOT = 0, 1, 2, 3


def set_projection_variant(variant: int) -> int:
    """Process-wide projection decomposition; returns the previous setting."""
    prev = lib().dspk_set_projection_variant(int(variant))
    if prev < 0:
        _check(prev)
    return prev


def set_prefill_block_rows(rows: int) -> int:
    """Process-wide prefill row block (0 automatic, 64, 128); returns the
    previous setting."""
    prev = lib().dspk_set_prefill_block_rows(int(rows))
    if prev < 0:
        _check(prev)
    return prev


def qgemm_workspace_bytes(n: int, k: int, m: int) -> int:
    return lib().dspk_qgemm_workspace_bytes(n, k, m)


def lmhead_workspace_bytes(v: int, m: int) -> int:
    return lib().dspk_lmhead_workspace_bytes(v, m)


def sample_workspace_bytes(v: int, m_rows: int) -> int:
    return lib().dspk_sample_workspace_bytes(v, m_rows)


def alloc_workspace(nbytes: int, device="cuda"):
    """Zero-filled workspace (the library keeps it zeroed between calls)."""
    import torch
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def qgemm_verify(w: DeviceQWeight, x, m: int, y, workspace=None, stream=None) -> None:
    """x: row-major bf16 activation rows [>= m][ldx]."""
    ldx, ldy = _acts(x, "x"), _rows(y, "y")
    dt = DSPK_BF16 if y.element_size() == 2 else DSPK_F32
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(lib().dspk_qgemm_verify(ctypes.byref(w.desc), x.data_ptr(), ldx, m, y.data_ptr(), dt, ldy,
                                   _ptr(workspace), ws_bytes, _stream(stream)))


def qgemm_verify_grouped(ws: list, x, m: int, ys: list, workspace=None, stream=None) -> None:
    cnt = len(ws)
    descs = (TiledDesc * cnt)(*[w.desc for w in ws])
    yptr = (c_void_p * cnt)(*[y.data_ptr() for y in ys])
    ldy = (c_int64 * cnt)(*[_rows(y, "y") for y in ys])
    dt = DSPK_BF16 if ys[0].element_size() == 2 else DSPK_F32
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(lib().dspk_qgemm_verify_grouped(cnt, descs, x.data_ptr(), _acts(x, "x"), m, yptr, dt, ldy,
                                           _ptr(workspace), ws_bytes, _stream(stream)))


def qgemm_verify_grouped_noalloc(ws: list, x, m: int, ys: list, stream=None) -> None:
    """The grouped projection on the library's own per-GPU scratch (no workspace)."""
    cnt = len(ws)
    descs = (TiledDesc * cnt)(*[w.desc for w in ws])
    yptr = (c_void_p * cnt)(*[y.data_ptr() for y in ys])
    ldy = (c_int64 * cnt)(*[_rows(y, "y") for y in ys])
    dt = DSPK_BF16 if ys[0].element_size() == 2 else DSPK_F32
    _check(lib().dspk_qgemm_verify_grouped_noalloc(cnt, descs, x.data_ptr(), _acts(x, "x"), m, yptr, dt, ldy,
                                                   _stream(stream)))


def prefill_workspace_bytes(n: int, k: int, m: int, bits: int) -> int:
    return lib().dspk_prefill_workspace_bytes(n, k, m, bits)


def qgemm_prefill(w: DeviceQWeight, x, m: int, y, workspace=None, stream=None) -> None:
    """x: ROW-major bf16 activations [m][ldx] (int16 bit patterns or bfloat16).
    workspace: None, or a zero-filled buffer of prefill_workspace_bytes."""
    dt = DSPK_BF16 if y.element_size() == 2 else DSPK_F32
    _check(lib().dspk_qgemm_prefill(ctypes.byref(w.desc), x.data_ptr(), _rows(x, "x"), m, y.data_ptr(), dt,
                                    _rows(y, "y"), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                    _stream(stream)))


def prepare_qgemm_prefill(w: DeviceQWeight, x, m: int, y, workspace=None, stream=None) -> Prepared:
    dt = DSPK_BF16 if y.element_size() == 2 else DSPK_F32
    return Prepared("dspk_qgemm_prefill", ctypes.byref(w.desc), x.data_ptr(), _rows(x, "x"), m, y.data_ptr(), dt,
                    _rows(y, "y"), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                    _stream(stream))


def lmhead_argmax(w: DeviceQWeight, h, m: int, argmax, logits=None, workspace=None, stream=None) -> None:
    ldl = 0 if logits is None else _rows(logits, "logits")
    _check(lib().dspk_lmhead_argmax(ctypes.byref(w.desc), h.data_ptr(), _acts(h, "h"), m, argmax.data_ptr(),
                                    _ptr(logits), ldl, _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), _stream(stream)))


def lmhead_argmax_accept_greedy(w: DeviceQWeight, h, b: int, m_rows: int, argmax, draft_ids, accept_len, committed,
                                logits=None, workspace=None, stream=None) -> None:
    ldl = 0 if logits is None else _rows(logits, "logits")
    _check(lib().dspk_lmhead_argmax_accept_greedy(ctypes.byref(w.desc), h.data_ptr(), _acts(h, "h"), b, m_rows,
                                                  argmax.data_ptr(), _ptr(logits), ldl, _ptr(draft_ids),
                                                  accept_len.data_ptr(), committed.data_ptr(), _ptr(workspace),
                                                  0 if workspace is None else workspace.numel(), _stream(stream)))


def accept_greedy(target_ids, draft_ids, b: int, m_rows: int, accept_len, committed, stream=None) -> None:
    _check(lib().dspk_accept_greedy(target_ids.data_ptr(), _ptr(draft_ids), b, m_rows, accept_len.data_ptr(),
                                    committed.data_ptr(), _stream(stream)))


def accept_sample(logits, q, draft_ids, uniforms, m_rows: int, v: int, temperature: float, accept_len,
                  committed, workspace=None, stream=None) -> None:
    _check(lib().dspk_accept_sample(logits.data_ptr(), _rows(logits, "logits"), q.data_ptr(), _rows(q, "q"),
                                    draft_ids.data_ptr(), uniforms.data_ptr(), m_rows, v, float(temperature),
                                    accept_len.data_ptr(), committed.data_ptr(), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), _stream(stream)))


def accept_sample_ex(logits, q, draft_ids, uniforms, m_rows: int, v: int, params: SampleParamsDesc, counts=None,
                     accept_len=None, committed=None, workspace=None, stream=None) -> None:
    """Speculative sampling over penalised, top-k/top-p truncated
    distributions; ``params`` from sample_params(), ``counts`` an int32 [v]
    device tensor of history counts or None."""
    _check(lib().dspk_accept_sample_ex(logits.data_ptr(), _rows(logits, "logits"), q.data_ptr(), _rows(q, "q"),
                                       draft_ids.data_ptr(), uniforms.data_ptr(), m_rows, v, ctypes.byref(params),
                                       _ptr(counts), accept_len.data_ptr(), committed.data_ptr(), _ptr(workspace),
                                       0 if workspace is None else workspace.numel(), _stream(stream)))
