"""The pins catch plausible mistakes: each test plants one mistake in the
oracle (on the CPU, through monkeypatching) and checks that a pin fails."""
import json
import os
import types

import numpy as np
import pytest

import oracle
from oracle import dspk_oracle
from speculative_decoding_verify_dspk_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _sample_golden_passes():
    for c in json.load(open(GOLDEN))["sample"]:
        alen, com = dspk_oracle.accept_sample(np.array(c["z"], np.float64), np.array(c["q"]),
                                              np.array(c["d"]), np.array(c["u"]), c["T"])
        if alen != c["accept_len"] or list(com) != c["committed"]:
            return False
    return True


def test_baseline_passes():
    assert _sample_golden_passes()


def test_inclusive_vs_strict_cdf_mistake_is_caught(monkeypatch):
    def bad(weights, threshold):
        c = np.cumsum(np.asarray(weights, np.float64))
        hit = np.nonzero(c >= threshold)[0]
        return int(hit[0]) if hit.size else len(c) - 1
    monkeypatch.setattr(dspk_oracle, "inverse_cdf", bad)
    assert not _sample_golden_passes()


def test_temperature_multiplied_is_caught(monkeypatch):
    def bad(z, temperature):
        a = np.asarray(z, np.float64) * float(temperature)
        e = np.exp(a - a.max())
        return e / e.sum()
    monkeypatch.setattr(dspk_oracle, "softmax_t", bad)
    assert not _sample_golden_passes()


def test_residual_sign_flip_is_caught(monkeypatch):
    proxy = types.SimpleNamespace(**{k: getattr(np, k) for k in dir(np) if not k.startswith("__")})
    proxy.maximum = lambda a, b: np.maximum(a, -b)     # max(0, q - p) instead of max(0, p - q)
    monkeypatch.setattr(dspk_oracle, "np", proxy)
    assert not _sample_golden_passes()


def test_msb_first_unpack_is_caught():
    w = inputs.make_qweight(4, 128, 4, "mutant")
    per = 8
    words = np.asarray(w.codes, np.uint32)
    bad = np.empty((4, 128), np.int64)
    for slot in range(per):
        bad[:, slot::per] = (words >> np.uint32(4 * (per - 1 - slot))) & np.uint32(15)
    assert not np.array_equal(bad, w.codes_u8)
    assert np.array_equal(oracle.unpack_codes(w.codes, 4, 128), w.codes_u8)


def test_dropped_bias_and_wrong_group_index_are_caught(monkeypatch):
    n, k = 9, 320
    w = inputs.make_qweight(n, k, 8, "ones-pin")
    x = np.full((1, k), 0x3F80, np.uint16)
    good = oracle.qlinear(x, w.codes, w.scales, w.biases, 8, n, k)

    def no_bias(codes, scales, biases, bits, n_, k_):
        q = dspk_oracle.unpack_codes(codes, bits, k_).astype(np.float64)
        s = dspk_oracle.decode_fp16(scales).reshape(n_, k_ // 64)
        return s[:, np.arange(k_) // 64] * q

    def wrong_group(codes, scales, biases, bits, n_, k_):
        q = dspk_oracle.unpack_codes(codes, bits, k_).astype(np.float64)
        s = dspk_oracle.decode_fp16(scales).reshape(n_, k_ // 64)
        b = dspk_oracle.decode_fp16(biases).reshape(n_, k_ // 64)
        g = np.arange(k_) % (k_ // 64)
        return s[:, g] * q + b[:, g]

    for mutant in (no_bias, wrong_group):
        monkeypatch.setattr(dspk_oracle, "dequantize", mutant)
        bad = dspk_oracle.qlinear(x, w.codes, w.scales, w.biases, 8, n, k)
        assert not np.allclose(bad, good, rtol=1e-6)


def test_row_draft_misalignment_is_caught():
    """Comparing draft j with row j+1 instead of row j breaks the golden cases."""
    def bad(t, d):
        t = np.atleast_2d(t)
        d = np.atleast_2d(d)
        a = 0
        while a < t.shape[1] - 1 and d[0, a] == t[0, a + 1]:
            a += 1
        return a + 1
    c = json.load(open(GOLDEN))["greedy"][0]
    assert bad(np.array(c["t"]), np.array(c["d"])) != c["accept_len"]


def _penalty_golden_passes():
    for c in json.load(open(GOLDEN))["penalties"]:
        got = dspk_oracle.penalized_logits(np.array(c["z"], np.float64), c["counts"], np.array(c["d"], np.int64),
                                           c["presence"], c["frequency"])
        if not np.array_equal(got, np.array(c["expected"], np.float64)):
            return False
    return True


def test_penalty_pins_pass_and_catch_mistakes(monkeypatch):
    """Frequency applied as an indicator, and a row counting its own draft,
    both fail the hand-worked penalty cases."""
    assert _penalty_golden_passes()
    real = dspk_oracle.penalized_logits

    def freq_as_indicator(logits, counts, draft_ids, presence, frequency):
        z = np.asarray(logits, np.float64)
        c = np.zeros(z.shape[1]) if counts is None else np.asarray(counts, np.float64).copy()
        d = np.asarray(draft_ids, np.int64).ravel()
        out = np.empty_like(z)
        for j in range(z.shape[0]):
            out[j] = z[j] - presence * (c > 0) - frequency * (c > 0)
            if j < z.shape[0] - 1:
                c[d[j]] += 1
        return out
    monkeypatch.setattr(dspk_oracle, "penalized_logits", freq_as_indicator)
    assert not _penalty_golden_passes()

    def counts_own_draft(logits, counts, draft_ids, presence, frequency):
        z = np.asarray(logits, np.float64)
        c = np.zeros(z.shape[1]) if counts is None else np.asarray(counts, np.float64).copy()
        d = np.asarray(draft_ids, np.int64).ravel()
        out = np.empty_like(z)
        for j in range(z.shape[0]):
            if j < z.shape[0] - 1:
                c[d[j]] += 1
            out[j] = z[j] - presence * (c > 0) - frequency * c
        return out
    monkeypatch.setattr(dspk_oracle, "penalized_logits", counts_own_draft)
    assert not _penalty_golden_passes()
    monkeypatch.setattr(dspk_oracle, "penalized_logits", real)
