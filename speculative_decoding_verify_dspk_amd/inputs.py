"""Seeded synthetic inputs for the verify pass.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests.  It holds no arithmetic of the verify method itself (no
dequantisation, no matmul, no argmax, no acceptance rule): it only draws random
numbers, rounds them to the storage formats and packs integer codes into words.

Storage formats (the pages say only that the target's weights are quantised in
groups -- "mlx-dspark" wiki summary, "Key techniques"; the format below is the
plain affine group format):

* codes: unsigned integers 0 .. 2**bits - 1, each output row's K codes one
  LSB-first bit stream in uint32 words (32/bits codes per word for 2, 4 and
  8 bits; 3-bit codes may straddle words);
* scales, biases: IEEE binary16 bit patterns, row-major ``[N][K/64]``;
* activations: bfloat16 bit patterns, row-major ``[M][K]``;
* uniforms for stochastic acceptance: float32 values k / 2**24.

Every generator takes an explicit seed; seeds are derived from readable labels
with a stable hash, so a label such as ``("qwen3-4b", 0, "gate", "codes")``
always yields the same tensor.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np

GROUP = 64


# --------------------------------------------------------------------------- seeds
def seed_of(*labels) -> int:
    """Stable 64-bit seed from a tuple of labels (str/int)."""
    h = 0
    for lab in labels:
        data = str(lab).encode()
        h = (h * 1000003) ^ zlib.crc32(data) ^ (zlib.adler32(data) << 32)
        h &= (1 << 64) - 1
    return h


def rng(*labels) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_of(*labels)))


# --------------------------------------------------------------- format rounding
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    NaN inputs become a quiet NaN; infinities are kept.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32) & 0xFFFF
    nan = np.isnan(f)
    r = np.where(nan, (u >> 16).astype(np.uint32) | 0x0040, r)
    return r.astype(np.uint16)


def f32_to_fp16_bits(a) -> np.ndarray:
    """Round to IEEE binary16 (numpy's conversion, nearest-even); return uint16 bits."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------- packing
def pack_codes(codes_u8: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes ``[N][K]`` into ``uint32[N][K*bits/32]``: each row an
    LSB-first bit stream (code k at stream bits bits*k ..), 32 stream bits per
    little-endian word.  For 2, 4 and 8 bits that is 32/bits codes per word."""
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    c = np.asarray(codes_u8, dtype=np.uint64)
    n, k = c.shape
    if (k * bits) % 32:
        raise ValueError("K * bits must be a multiple of 32")
    if c.max(initial=0) >= (1 << bits):
        raise ValueError("code out of range")
    if 32 % bits == 0:
        # no code straddles a word: word w holds codes w*per .. w*per + per-1,
        # code i of the word at bits bits*i ..
        per = 32 // bits
        cw = c.reshape(n, k // per, per)
        words = np.zeros((n, k // per), dtype=np.uint64)
        for i in range(per):
            words |= cw[:, :, i] << np.uint64(bits * i)
        return words.astype(np.uint32)
    words = np.zeros((n, k * bits // 32), dtype=np.uint64)
    pos = np.arange(k, dtype=np.int64) * bits
    w, off = pos // 32, (pos % 32).astype(np.uint64)
    for i in range(k):
        words[:, w[i]] |= (c[:, i] << off[i]) & np.uint64(0xffffffff)
        if off[i] + bits > 32:                       # the code's high bits start the next word
            words[:, w[i] + 1] |= c[:, i] >> (np.uint64(32) - off[i])
    return words.astype(np.uint32)


# ----------------------------------------------------------------- weights, acts
@dataclass
class QWeight:
    """One weight matrix in storage format (host arrays)."""
    n: int
    k: int
    bits: int
    codes: np.ndarray            # uint32 [N][K*bits/32] (bits 2/3/4/8) or uint16 bf16 [N][K] (bits 16)
    scales: np.ndarray | None    # uint16 fp16 [N][K/64]
    biases: np.ndarray | None    # uint16 fp16 [N][K/64]
    codes_u8: np.ndarray | None  # uint8 [N][K] ground-truth codes (quantised formats)

    @property
    def nbytes(self) -> int:
        b = self.codes.nbytes
        if self.scales is not None:
            b += self.scales.nbytes + self.biases.nbytes
        return b


def make_qweight(n: int, k: int, bits: int, *labels,
                 scale_lo: float = 0.001, scale_hi: float = 0.01,
                 bias_std: float = 0.1, keep_codes: bool = True) -> QWeight:
    """Affine group-quantised weight with the distributions of the workloads:
    codes uniform over 0..2**bits-1, scales U(scale_lo, scale_hi) and biases
    N(0, bias_std) rounded to fp16.  ``bits == 16`` gives the unquantised bf16
    control: values N(0.7, 0.45) in bf16 (close to the mean and spread of the
    8-bit weights above), no scales or biases."""
    if k % GROUP:
        raise ValueError("K must be a multiple of 64")
    g = rng(*labels, n, k, bits)
    if bits == 16:
        w = g.normal(0.7, 0.45, size=(n, k)).astype(np.float32)
        return QWeight(n, k, 16, f32_to_bf16_bits(w), None, None, None)
    codes = g.integers(0, 1 << bits, size=(n, k), dtype=np.uint8)
    scales = f32_to_fp16_bits(g.uniform(scale_lo, scale_hi, size=(n, k // GROUP)))
    biases = f32_to_fp16_bits(g.normal(0.0, bias_std, size=(n, k // GROUP)))
    return QWeight(n, k, bits, pack_codes(codes, bits), scales, biases,
                   codes if keep_codes else None)


def make_activations(m: int, k: int, *labels, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns ``[M][K]`` drawn N(0, std)."""
    g = rng(*labels, m, k, "act")
    return f32_to_bf16_bits(g.normal(0.0, std, size=(m, k)).astype(np.float32))


def make_uniforms(count: int, *labels) -> np.ndarray:
    """float32 uniforms k / 2**24, k uniform over [0, 2**24): exact in fp32/fp64, < 1."""
    g = rng(*labels, count, "uniform")
    return (g.integers(0, 1 << 24, size=count).astype(np.float64) / float(1 << 24)).astype(np.float32)


# -------------------------------------------------------------------- draft ids
def drafts_first_equal(target_ids: np.ndarray, n_equal: int, vocab: int, *labels) -> np.ndarray:
    """Draft ids for one request: the first ``n_equal`` copy the given target ids,
    the rest are uniform over [0, vocab) (an accidental match is allowed)."""
    t = np.asarray(target_ids, dtype=np.int64)
    m = t.shape[0] - 1
    g = rng(*labels, "drafts-first-equal", m, vocab)
    d = g.integers(0, vocab, size=m).astype(np.int32)
    d[:n_equal] = t[:n_equal]
    return d


def drafts_match_rate(target_ids: np.ndarray, alpha: float, vocab: int, *labels) -> np.ndarray:
    """Draft ids ``[B][M-1]`` with an independent per-position match rate.

    Position j matches (d_j = t_j) with probability alpha[b]; otherwise d_j is
    uniform over the vocabulary minus t_j.  ``target_ids`` is ``[B][M]``.
    """
    t = np.atleast_2d(np.asarray(target_ids, dtype=np.int64))
    bsz, mrows = t.shape
    alpha = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (bsz,))
    g = rng(*labels, "drafts-match-rate", bsz, mrows, vocab)
    d = np.empty((bsz, mrows - 1), dtype=np.int32)
    for b in range(bsz):
        hit = g.random(mrows - 1) < alpha[b]
        other = g.integers(0, vocab - 1, size=mrows - 1)
        other = other + (other >= t[b, :mrows - 1])      # skip t_j: uniform over V \ {t_j}
        d[b] = np.where(hit, t[b, :mrows - 1], other)
    return d


# -------------------------------------------------------- synthetic drafter side
def draft_distribution(target_logits: np.ndarray, temperature: float,
                       noise_std: float, *labels) -> tuple[np.ndarray, np.ndarray]:
    """Stand-in for a drafter: q_j = softmax((z_j + eps_j) / T), eps ~ N(0, noise_std),
    for the first M-1 rows of ``target_logits`` ``[M][V]``; d_j drawn from q_j with
    numpy's categorical sampler.  Returns (q float32 [M-1][V], d int32 [M-1]).

    This is the drafter's side of the round, not the verify method: it only
    produces the proposal the verify pass then judges.
    """
    z = np.asarray(target_logits, dtype=np.float64)
    mrows, v = z.shape
    g = rng(*labels, "draft-q", mrows, v)
    noisy = (z[:mrows - 1] + g.normal(0.0, noise_std, size=(mrows - 1, v))) / temperature
    noisy -= noisy.max(axis=1, keepdims=True)
    e = np.exp(noisy)
    q = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    d = np.empty(mrows - 1, dtype=np.int32)
    for j in range(mrows - 1):
        pj = q[j].astype(np.float64)
        d[j] = g.choice(v, p=pj / pj.sum())
    return q, d


# ------------------------------------------------------- workload shape tables
# Projection shapes (N out, K in) of the synthetic decoder layers.
def history_counts(vocab: int, length: int, *labels) -> np.ndarray:
    """Token counts of a seeded synthetic history of ``length`` tokens
    (Zipf-like token frequencies, as text has), int32 [vocab]."""
    g = rng("history", vocab, length, *labels)
    ranks = np.minimum(g.zipf(1.2, size=length), vocab) - 1
    ids = g.permutation(vocab)[ranks]
    return np.bincount(ids, minlength=vocab).astype(np.int32)


LAYER_SHAPES = {
    # Qwen3-4B: hidden 2560, 32 q heads x 128, 8 kv heads x 128, intermediate 9728
    "qwen3-4b": dict(hidden=2560, q=4096, kv=1024, inter=9728, vocab=151936),
    # Ornith-1.0-9B-shaped dense layer: hidden 4096, intermediate 12288
    "ornith-9b": dict(hidden=4096, q=4096, kv=1024, inter=12288, vocab=151936),
    # Qwen3-8B-shaped layer (same dense shapes as above)
    "qwen3-8b": dict(hidden=4096, q=4096, kv=1024, inter=12288, vocab=151936),
    # 27B-shaped dense layer: hidden 5120, 40 q heads x 128, intermediate 17408
    "dense-27b": dict(hidden=5120, q=5120, kv=1024, inter=17408, vocab=151936),
}


def layer_projections(model: str):
    """[(name, N, K, input)] for one layer; ``input`` names which of the four
    independent activation tensors the projection reads (q/k/v share the
    attention input, gate/up share the MLP input)."""
    s = LAYER_SHAPES[model]
    h, q, kv, f = s["hidden"], s["q"], s["kv"], s["inter"]
    return [
        ("q", q, h, "attn_in"), ("k", kv, h, "attn_in"), ("v", kv, h, "attn_in"),
        ("o", h, q, "o_in"),
        ("gate", f, h, "mlp_in"), ("up", f, h, "mlp_in"),
        ("down", h, f, "down_in"),
    ]


def weight_bytes(n: int, k: int, bits: int) -> int:
    """Algorithmic bytes of one weight matrix in storage format."""
    if bits == 16:
        return n * k * 2
    return n * k * bits // 8 + 2 * 2 * n * (k // GROUP)


# ------------------------------------------------- device-side bulk generators
def device_generator(*labels):
    """torch CUDA generator seeded from labels (for multi-GB weight stacks)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed_of(*labels) & ((1 << 63) - 1))
    return g


def make_qweight_device(n: int, k: int, bits: int, *labels):
    """Same distributions as ``make_qweight``, drawn on the GPU with torch's
    generator: uniform random 32-bit words are exactly LSB-first packed words of
    independent uniform codes; scales U(0.001, 0.01) and biases N(0, 0.1) are
    rounded to fp16; the bf16 control is N(0.7, 0.45).  Returns
    (codes, scales, biases) device tensors (int32 / int16 / int16 bit
    patterns) in the interchange layout: scales and biases row-major [N][K/64]."""
    import torch
    g = device_generator(*labels, n, k, bits)
    if bits == 16:
        w = torch.empty((n, k), dtype=torch.float32, device="cuda").normal_(0.7, 0.45, generator=g)
        return w.to(torch.bfloat16).view(torch.int16), None, None
    words = torch.randint(-(1 << 31), 1 << 31, (n, k * bits // 32), dtype=torch.int64, device="cuda",
                          generator=g).to(torch.int32)
    sc = torch.empty((n, k // GROUP), dtype=torch.float32, device="cuda").uniform_(0.001, 0.01, generator=g)
    bi = torch.empty((n, k // GROUP), dtype=torch.float32, device="cuda").normal_(0.0, 0.1, generator=g)
    return words, sc.to(torch.float16).view(torch.int16), bi.to(torch.float16).view(torch.int16)


def make_activations_rowmajor_device(m: int, k: int, *labels):
    """bf16 N(0, 1) rows on the GPU (int16 bit patterns), row-major [m][k]:
    the prefill projection's layout."""
    import torch
    g = device_generator(*labels, m, k)
    a = torch.empty((m, k), dtype=torch.float32, device="cuda").normal_(0.0, 1.0, generator=g)
    return a.to(torch.bfloat16).view(torch.int16)


def make_activations_device(m: int, k: int, *labels):
    """bf16 N(0, 1) rows on the GPU (int16 bit patterns), row-major ``[M][K]``:
    the layout every projection call reads."""
    import torch
    g = device_generator(*labels, m, k, "act")
    x = torch.empty((m, k), dtype=torch.float32, device="cuda").normal_(0.0, 1.0, generator=g)
    return x.to(torch.bfloat16).view(torch.int16)
