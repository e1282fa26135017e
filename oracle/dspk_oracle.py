"""Plain, slow fp64 CPU oracle of the speculative-decoding verify pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP library (no kernels, headers, helpers or tables) and never
imports it; the only module both sides use is the seeded input generator, which
holds none of the method's arithmetic.

What it computes, and the passages it follows (pages quoted by title):

* "mlx-dspark" wiki summary, section "Architecture", first bullet: one
  target pass evaluates the anchor and all m drafts; every draft is checked
  against what the target itself predicts at its position and the drafts are
  kept up to the first failed check.  Greedy checks reproduce plain decoding;
  at temperature > 0 the Leviathan/Chen min(1, p/q) test keeps the output an
  exact sample of the target.
* Same page, "Key techniques" (auto-calibration bullet): a round commits
  1 + sum p^i tokens in expectation, i.e. the accepted drafts plus one token of
  the target's own; "Design decisions": a miss costs a plain one-token forward.
* Same page, "Key techniques" (custom kernels bullet): the verify kernel
  dequantises each weight group once and reuses it for every row -- the
  arithmetic is the plain dequantise-then-matmul below.
* "mlx-dspark 0.7.0" project page, "How it works": the output matches plain
  decoding except where rounding breaks a tie; with temperature > 0 the
  committed tokens are an exact sample of the target at temperature T.
* "mlx-dspark releases", v0.0.2 notes: the sampling path was validated to give
  exactly the target's output distribution.

* "mlx-dspark 0.7.0", "Tuning" and "The Apple-Silicon speedup ceiling"; wiki
  summary "Key techniques" (auto-calibration) and "Design decisions": the
  draft cap is chosen from measured verify/drafter cost curves and a live
  acceptance estimate, maximising expected committed tokens per unit time,
  and speculation parks (with probe rounds) when it would lose.

Readings where the pages are silent (quantisation format, packing, tie rule,
the extra committed token, strictness of the accept test, residual with zero
mass, inverse-CDF rule) are listed in the design notes and restated at each
function below.

Every function works in float64 on exactly the values the storage formats hold
(bf16 activations, fp16 scales/biases, integer codes), so the matmul result is
exact up to fp64 rounding (relative error of order K * 2**-53).
"""
from __future__ import annotations

import numpy as np

GROUP = 64


# ------------------------------------------------------------------ decoders
def decode_fp16(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact): the upper half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):     # signalling-NaN patterns widen to NaN
        return u.view(np.float32).astype(np.float64)


# ------------------------------------------------------------- O1: unpacking
def unpack_codes(codes, bits: int, k: int) -> np.ndarray:
    """Integer codes ``[N][K]`` from packed words ``uint32[N][K*bits/32]``.

    Reading of the (unstated) packing: each row is one LSB-first bit stream
    stored in little-endian uint32 words -- bit i of the row is bit i % 32 of
    word i // 32 -- and code k occupies stream bits bits*k .. bits*k + bits-1,
    lowest bit first.  For 2, 4 and 8 bits that is 32/bits codes per word;
    3-bit codes may straddle two words.
    """
    if bits not in (2, 3, 4, 8):
        raise ValueError("unpack_codes: bits must be 2, 3, 4 or 8")
    words = np.ascontiguousarray(codes, dtype="<u4")
    n = words.shape[0]
    if words.shape[1] * 32 != k * bits:
        raise ValueError("unpack_codes: packed width does not match K")
    # the row's bit stream, bit i at column i: the words' little-endian bytes,
    # each byte's bits lowest first
    stream = np.unpackbits(words.view(np.uint8), axis=1, bitorder="little")
    q = np.zeros((n, k), dtype=np.int64)
    for b in range(bits):
        q |= stream[:, b::bits][:, :k].astype(np.int64) << b
    return q


# --------------------------------------------------------------- O2: dequant
def dequantize(codes, scales, biases, bits: int, n: int, k: int) -> np.ndarray:
    """Weight matrix ``W[N][K]`` in float64.

    Affine group quantisation (reading of "quantized" / "weight group" in the
    wiki summary's "Key techniques"): w[n,k] = s[n, k//64] * q[n,k] + b[n, k//64]
    with fp16 scale s and bias b per 64-wide group along K.  ``bits == 16`` is
    the unquantised bf16 control: ``codes`` holds bf16 bit patterns [N][K].
    """
    if bits == 16:
        return decode_bf16(codes).reshape(n, k)
    if k % GROUP:
        raise ValueError("dequantize: K must be a multiple of 64")
    q = unpack_codes(codes, bits, k).astype(np.float64)
    s = decode_fp16(scales).reshape(n, k // GROUP)
    b = decode_fp16(biases).reshape(n, k // GROUP)
    g = np.arange(k) // GROUP
    return s[:, g] * q + b[:, g]


# ---------------------------------------------------------------- O3: linear
def qlinear(x_bf16, codes, scales, biases, bits: int, n: int, k: int) -> np.ndarray:
    """Verify-pass projection y[M][N] = x[M][K] . W[N][K]^T in float64.

    The M rows are the anchor plus the drafts ("mlx-dspark" wiki summary,
    "Architecture"): every row goes through the same dequantised weights.
    """
    x = decode_bf16(x_bf16)
    x = x.reshape(-1, k)
    w = dequantize(codes, scales, biases, bits, n, k)
    return x @ w.T


# ------------------------------------------------------ O4: argmax and margin
def argmax_lowest(z) -> tuple[np.ndarray, np.ndarray]:
    """Per-row argmax with the lowest index on ties, and the top-2 margin.

    The target's greedy token is the argmax of its own logits.  The project page
    ("mlx-dspark 0.7.0", "How it works") allows the output to differ from plain
    decoding only where floating-point rounding breaks a tie, and leaves the tie
    rule open -- the reading taken is the lowest index.  A NaN counts as
    the maximum (the first NaN wins), so a row holding a NaN never reports a
    finite token silently.

    margin[m] = z[m, t] - max over v != t of z[m, v]  (NaN if the row holds a
    NaN; +inf when V == 1).
    """
    z = np.asarray(z, dtype=np.float64)
    t = np.argmax(z, axis=1)
    rows = np.arange(z.shape[0])
    top = z[rows, t]
    if z.shape[1] == 1:
        return t.astype(np.int32), np.full(z.shape[0], np.inf)
    rest = z.copy()
    rest[rows, t] = -np.inf
    margin = top - rest.max(axis=1)
    margin[np.isnan(z).any(axis=1)] = np.nan
    return t.astype(np.int32), margin


def lmhead_argmax(h_bf16, codes, scales, biases, bits: int, v: int, hdim: int):
    """Target logits z[M][V] = h . W_lm^T, their argmax and top-2 margin."""
    z = qlinear(h_bf16, codes, scales, biases, bits, v, hdim)
    t, margin = argmax_lowest(z)
    return z, t, margin


# -------------------------------------------------------- O5: greedy accept
def accept_greedy(target_ids, draft_ids) -> tuple[np.ndarray, np.ndarray]:
    """Longest accepted prefix plus the target's own token, per request.

    target_ids ``[B][M]``: row j's greedy token (row 0 reads the anchor, row j
    reads draft j-1).  draft_ids ``[B][M-1]``.  Draft j is accepted while it
    equals row j's token; at the first mismatch (or after all M-1 drafts) the
    target's token of that row is committed ("Architecture": commit the longest
    accepted prefix; "Key techniques": 1 + sum p^i tokens per round).

    Returns accept_len ``[B]`` = number of committed tokens (accepted drafts
    + 1, so 1..M) and committed ``[B][M]`` padded with -1.
    """
    t = np.atleast_2d(np.asarray(target_ids, dtype=np.int64))
    d = np.atleast_2d(np.asarray(draft_ids, dtype=np.int64))
    bsz, m_rows = t.shape
    if d.shape != (bsz, m_rows - 1):
        raise ValueError("accept_greedy: draft_ids must be [B][M-1]")
    accept_len = np.zeros(bsz, dtype=np.int32)
    committed = np.full((bsz, m_rows), -1, dtype=np.int32)
    for b in range(bsz):
        a = 0
        while a < m_rows - 1 and d[b, a] == t[b, a]:
            a += 1
        committed[b, :a] = d[b, :a]
        committed[b, a] = t[b, a]
        accept_len[b] = a + 1
    return accept_len, committed


def sequential_greedy(target_ids, draft_ids) -> list[int]:
    """What plain one-token-at-a-time greedy decoding emits from the same rows.

    Decoding emits row j's token; row j+1 was computed on input d_j, so it is
    a valid next step only while the emitted token equals d_j.  Emission stops
    after the first token that differs from its draft, or after the last row.
    Independent formulation of the invariant "greedy output equals plain
    decoding" ("Architecture", "How it works").
    """
    t = list(np.asarray(target_ids, dtype=np.int64).ravel())
    d = list(np.asarray(draft_ids, dtype=np.int64).ravel())
    out = []
    for j, tok in enumerate(t):
        out.append(int(tok))
        if j == len(t) - 1 or tok != d[j]:
            break
    return out


# ---------------------------------------------------- O6: stochastic accept
def softmax_t(z, temperature: float) -> np.ndarray:
    """p = softmax(z / T) in float64 with max-subtraction (one row)."""
    a = np.asarray(z, dtype=np.float64) / float(temperature)
    a = a - a.max()
    e = np.exp(a)
    return e / e.sum()


def inverse_cdf(weights, threshold: float) -> int:
    """Index-order inverse CDF on non-negative weights.

    Reading: inclusive prefix sums C_v in index order; the sample is the first
    v with C_v > threshold (threshold = u * total).  If rounding leaves no such
    v, the last v with positive weight is taken.
    """
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    hit = np.nonzero(c > threshold)[0]
    if hit.size:
        return int(hit[0])
    pos = np.nonzero(w > 0)[0]
    return int(pos[-1]) if pos.size else w.size - 1


def accept_sample(logits, q, draft_ids, uniforms, temperature: float):
    """Leviathan/Chen speculative sampling over one verify block.

    logits ``[M][V]`` (row j is the target's distribution after input j),
    q ``[M-1][V]`` the drafter's distributions, draft_ids ``[M-1]``, uniforms
    ``[M]``: u_j decides draft j, u_{M-1} is the single final draw.

    p_j = softmax(z_j / T).  For j = 0 .. M-2: accept d_j iff
    u_j * q_j(d_j) < p_j(d_j)  (equals u_j < min(1, p/q) for q > 0; q(d) = 0
    with p(d) > 0 accepts).  At the first reject j, sample from the residual
    r = max(0, p_j - q_j) with threshold u_{M-1} * sum(r); if the residual has no
    mass (possible only through rounding), sample from p_j instead.  If every
    draft is accepted, sample the bonus token from p_{M-1}
    ("Architecture": exact sample via min(1, p/q); "How it works": exact sample
    from the target at temperature T; v0.0.2 release notes: validated to equal
    the target's distribution).

    Data faults -- T <= 0 or non-finite, a non-finite logit, a non-finite or
    negative q, a uniform outside [0, 1), a draft id outside [0, V) -- return
    accept_len = -1 and all -1 committed ids.

    Returns (accept_len = committed count 1..M, committed ``[M]`` padded -1).
    """
    z = np.asarray(logits, dtype=np.float64)
    m_rows, v = z.shape
    qq = np.asarray(q, dtype=np.float64).reshape(m_rows - 1, v)
    d = np.asarray(draft_ids, dtype=np.int64).ravel()
    u = np.asarray(uniforms, dtype=np.float64).ravel()
    committed = np.full(m_rows, -1, dtype=np.int32)
    bad = (not np.isfinite(temperature) or temperature <= 0
           or not np.isfinite(z).all()
           or not np.isfinite(qq).all() or (qq < 0).any()
           or not np.isfinite(u).all() or (u < 0).any() or (u >= 1).any()
           or (d < 0).any() or (d >= v).any())
    if bad:
        return -1, committed
    final_u = u[m_rows - 1]
    for j in range(m_rows - 1):
        p = softmax_t(z[j], temperature)
        if u[j] * qq[j, d[j]] < p[d[j]]:
            committed[j] = d[j]
            continue
        r = np.maximum(0.0, p - qq[j])
        mass = r.sum()
        if not mass > 0:
            r = p
            mass = p.sum()
        committed[j] = inverse_cdf(r, final_u * mass)
        return j + 1, committed
    p = softmax_t(z[m_rows - 1], temperature)
    committed[m_rows - 1] = inverse_cdf(p, final_u * p.sum())
    return m_rows, committed


# ------------------------------------------------------------ cap policy
def expected_committed(cap: int, alpha: float) -> float:
    """Expected tokens committed by a round that drafts ``cap`` tokens with
    per-position acceptance alpha: 1 + sum_{i=1..cap} alpha^i ("mlx-dspark"
    wiki summary, "Key techniques", auto-calibration bullet)."""
    return float(sum(alpha ** i for i in range(cap + 1)))


def choose_cap(verify_us, draft_us, alpha: float) -> tuple[int, float]:
    """The cap c in 0..n-1 with the most expected tokens per microsecond,
    a round costing the verify pass at width c + 1 plus the drafter's time
    at cap c (none at c = 0) ("mlx-dspark 0.7.0", "The Apple-Silicon
    speedup ceiling": tok/s = A / (drafter + overhead + slope * C); "Tuning":
    the cap is chosen from the measured curves).  Ties keep the smaller cap;
    cap 0 means speculation is parked.  Returns (cap, tokens per us).

    A narrower verify can always run as a wider one (the extra rows are
    padding and change no commit), so the verify cost of width w is taken as
    the least measured cost at width w or above: measurement noise that
    makes a wider pass look cheaper than a narrower one cannot, by itself,
    select a longer cap."""
    n = len(verify_us)
    best, best_rate = 0, None
    for c in range(n):
        verify = min(float(t) for t in verify_us[c:])
        cost = verify + (float(draft_us[c]) if (draft_us is not None and c > 0) else 0.0)
        rate = expected_committed(c, alpha) / cost
        if best_rate is None or rate > best_rate:
            best, best_rate = c, rate
    return best, best_rate


class CapController:
    """Cap per round from the curves and a live acceptance estimate: an
    exponentially weighted count of accepted over tested draft positions (a
    round accepting a of d drafts tested a positions, plus the first reject
    when a < d); the prior counts as one tested position.  While the best cap
    is 0 (parked), every probe_every-th round drafts probe_cap tokens
    ("mlx-dspark 0.7.0", "Tuning": parks speculation with periodic probe
    rounds)."""

    def __init__(self, verify_us, draft_us, decay: float, prior_alpha: float, probe_every: int, probe_cap: int):
        self.verify_us, self.draft_us = list(verify_us), (None if draft_us is None else list(draft_us))
        self.decay = decay
        self.hits, self.trials = prior_alpha, 1.0
        self.probe_every, self.probe_cap = probe_every, probe_cap
        self.parked_rounds = 0

    def alpha(self) -> float:
        return self.hits / self.trials

    def observe(self, drafted: int, accepted: int) -> None:
        if drafted == 0:
            return
        tested = accepted + (1 if accepted < drafted else 0)
        self.hits = self.decay * self.hits + accepted
        self.trials = self.decay * self.trials + tested

    def next_cap(self) -> int:
        cap, _ = choose_cap(self.verify_us, self.draft_us, self.alpha())
        if cap > 0:
            self.parked_rounds = 0
            return cap
        self.parked_rounds += 1
        if self.parked_rounds >= self.probe_every:
            self.parked_rounds = 0
            return self.probe_cap
        return 0


# -------------------------------------------- truncated / penalised sampling
def penalized_logits(logits, counts, draft_ids, presence: float, frequency: float) -> np.ndarray:
    """Target logits with presence/frequency penalties, row by row
    ("mlx-dspark releases", v0.2.0 notes: the penalties act on the target
    logits, and the committed tokens are those one-token decoding of the
    penalised target would give).  Row j is reached only when drafts 0..j-1
    were accepted, so its token counts are the history's plus those drafts:
        c_j(v) = counts[v] + #{i < j : d_i = v}
        z'_j(v) = z_j(v) - presence * [c_j(v) > 0] - frequency * c_j(v)
    (the OpenAI definition the pages name)."""
    z = np.asarray(logits, dtype=np.float64)
    m_rows, v = z.shape
    c = np.zeros(v, dtype=np.float64) if counts is None else np.asarray(counts, dtype=np.float64).copy()
    d = np.asarray(draft_ids, dtype=np.int64).ravel()
    out = np.empty_like(z)
    for j in range(m_rows):
        out[j] = z[j] - presence * (c > 0) - frequency * c
        if j < m_rows - 1 and 0 <= d[j] < v:
            c[d[j]] += 1
    return out


def truncate(prob, top_k: int, top_p: float) -> np.ndarray:
    """Keep-mask of top-k then top-p truncation of one distribution
    ("mlx-dspark releases", v0.1.0 notes: when the draft and the target are
    cut down by the same top-k / top-p filter, speculative sampling stays an
    exact sample of the filtered target).  Reading: order the entries by probability, larger first, ties by
    the smaller index; top-k keeps the first k (k <= 0: all); top-p then keeps
    an entry iff the mass of the kept entries before it is below
    top_p * (mass kept by top-k) -- the smallest leading set whose mass
    reaches top_p of the top-k distribution (top_p >= 1: all)."""
    w = np.asarray(prob, dtype=np.float64)
    v = w.size
    order = np.lexsort((np.arange(v), -w))       # by -w, then index
    keep = np.zeros(v, dtype=bool)
    kk = v if top_k <= 0 else min(top_k, v)
    kept = order[:kk]
    if top_p < 1.0:
        target = top_p * w[kept].sum()
        excl = np.concatenate([[0.0], np.cumsum(w[kept])[:-1]])
        kept = kept[excl < target]
    keep[kept] = True
    return keep


def accept_sample_filtered(logits, q, draft_ids, uniforms, temperature: float, top_k: int = 0,
                           top_p: float = 1.0, counts=None, presence: float = 0.0,
                           frequency: float = 0.0):
    """Speculative sampling over the penalised, truncated target.

    p_j = truncate(softmax(z'_j / T)) renormalised, z' the penalised logits;
    q~_j = truncate(q_j) renormalised with the same top-k/top-p (the draft
    was drawn from q~_j).  Then the rule of accept_sample: accept d_j iff
    u_j * q~_j(d_j) < p~_j(d_j); at the first reject sample the residual
    max(0, p~_j - q~_j) (p~_j if it has no mass); else the bonus from p~_{M-1}.
    Without truncation q is used as supplied, as in accept_sample; truncation
    is off when top_p == 1 and top_k keeps everything (top_k <= 0, or
    top_k >= v: every entry would be kept).  Faults as accept_sample, plus
    top_p outside (0, 1],
    negative penalties' counts, and counts < 0."""
    z = np.asarray(logits, dtype=np.float64)
    m_rows, v = z.shape
    qq = np.asarray(q, dtype=np.float64).reshape(m_rows - 1, v)
    d = np.asarray(draft_ids, dtype=np.int64).ravel()
    u = np.asarray(uniforms, dtype=np.float64).ravel()
    committed = np.full(m_rows, -1, dtype=np.int32)
    bad = (not np.isfinite(temperature) or temperature <= 0 or not (0 < top_p <= 1)
           or not np.isfinite(z).all()
           or not np.isfinite(qq).all() or (qq < 0).any()
           or not np.isfinite(u).all() or (u < 0).any() or (u >= 1).any()
           or (d < 0).any() or (d >= v).any()
           or (counts is not None and (np.asarray(counts) < 0).any()))
    if bad:
        return -1, committed
    trunc = (0 < top_k < v) or top_p < 1.0
    zp = penalized_logits(z, counts, d, presence, frequency)

    def target(j):
        p = softmax_t(zp[j], temperature)
        if trunc:
            p = np.where(truncate(p, top_k, top_p), p, 0.0)
            p = p / p.sum()
        return p

    def draft(j):
        if not trunc:
            return qq[j]
        w = np.where(truncate(qq[j], top_k, top_p), qq[j], 0.0)
        s = w.sum()
        return w / s if s > 0 else w

    final_u = u[m_rows - 1]
    for j in range(m_rows - 1):
        p, qj = target(j), draft(j)
        if u[j] * qj[d[j]] < p[d[j]]:
            committed[j] = d[j]
            continue
        r = np.maximum(0.0, p - qj)
        mass = r.sum()
        if not mass > 0:
            r = p
            mass = p.sum()
        committed[j] = inverse_cdf(r, final_u * mass)
        return j + 1, committed
    p = target(m_rows - 1)
    committed[m_rows - 1] = inverse_cdf(p, final_u * p.sum())
    return m_rows, committed
