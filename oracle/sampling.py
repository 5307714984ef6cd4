"""CPU oracle of the stochastic (rejection-sampling) verify -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the HIP library and its binding never do, and it shares no code
with them.  Plain numpy in float64, one sequence and one position at a time.

What it computes.  "Architecture and acceleration of an end-to-end OCR expert
model", section 6.1, states the property this step must keep: the draft /
verify loop with rejection sampling leaves the distribution of the output
exactly that of the target model decoding on its own; section 7 gives the
loop (keep the agreeing prefix, let the target resample at the first
disagreement).  The pages give no formula for the sampled case.  The rule here
is the standard speculative-sampling one (Leviathan, Kalman and Matias, "Fast
Inference from Transformers via Speculative Decoding", 2023; Chen et al.,
"Accelerating Large Language Model Decoding with Speculative Sampling", 2023),
restated:

  p_j = softmax(logits_j / tau) is the target's distribution after position j
  (j = 0 .. K), q_i the draft's distribution that draft d_i was drawn from
  (i = 1 .. K).  Draft d_i is kept while u_i * q_i(d_i) < p_{i-1}(d_i), i.e.
  with probability min(1, p/q).  At the first draft that fails (index a + 1),
  the target's token is drawn from the residual distribution proportional to
  max(0, p_a - q_{a+1}); when all K drafts are kept the bonus token is drawn
  from p_K.  accepted_len = a, next_tok = that draw, the context grows by a + 1.

Readings where the pages and papers leave a step open (the same ones the GPU
path implements):
  - the acceptance uniforms u [B][K] are inputs;
  - draws from a categorical distribution use the Gumbel-max construction
    (the index of the largest log-weight plus an independent standard Gumbel
    variable is distributed as the normalised weights), with the Gumbel noise
    of (sequence b, position j, vocabulary entry v) taken from the
    counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
    "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): key = the 64-bit
    seed (low word first), counter = (v // 4, j, b, offset), output word v % 4;
    a 32-bit word w becomes the uniform ((w >> 9) + 0.5) * 2**-23, which lies
    in (0, 1) and is exact in fp32, and the noise is -log(-log(uniform));
  - ties go to the lower vocabulary index;
  - a residual with no positive entry (possible only through rounding when
    p_a and q_{a+1} agree) falls back to a draw from p_a with the same noise;
  - the two integer decisions (keep a draft; the largest key) are taken after
    rounding the deciding values to fp32, the precision the GPU decides in.
"""
from __future__ import annotations

import numpy as np

_MASK = np.uint64(0xFFFFFFFF)
_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds.  counter: integer array [..., 4], key:
    [..., 2] (32-bit values); returns uint64 array [..., 4] of 32-bit words.
    Each round multiplies words 0 and 2 by the two round constants (full
    64-bit products), and outputs (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1),
    hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); the key is bumped by the two Weyl
    constants before every round after the first."""
    c = np.asarray(counter, dtype=np.uint64) & _MASK
    k = np.asarray(key, dtype=np.uint64) & _MASK
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0            # both factors < 2**32: exact in uint64
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _MASK,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _MASK)
    return np.stack([c0, c1, c2, c3], axis=-1)


def uniform_from_word(w):
    """32-bit word -> ((w >> 9) + 0.5) * 2**-23 in (0, 1), float64 (exact)."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel_noise(seed: int, offset: int, b: int, j: int, V: int):
    """Standard Gumbel noise for vocabulary entries 0..V-1 of (sequence b,
    position j), from the counter (v // 4, j, b, offset) and key seed."""
    v = np.arange(V, dtype=np.uint64)
    ctr = np.zeros((V, 4), np.uint64)
    ctr[:, 0] = v >> np.uint64(2)
    ctr[:, 1] = j
    ctr[:, 2] = b
    ctr[:, 3] = offset & 0xFFFFFFFF
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], np.uint64)
    words = philox4x32_10(ctr, key)
    w = words[np.arange(V), (v & np.uint64(3)).astype(np.int64)]
    u = uniform_from_word(w)
    return -np.log(-np.log(u))


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def gumbel_argmax(logw, noise):
    """Index of the largest fp32-rounded key logw + noise over the entries with
    finite logw (lowest index on ties), and the gap between the two largest
    keys; (-1, inf) when no entry is finite."""
    ok = np.isfinite(logw)
    if not ok.any():
        return -1, np.inf
    key = np.full(logw.shape, -np.inf, np.float32)
    key[ok] = _f32(logw[ok] + noise[ok])
    best = int(np.argmax(key))                    # numpy: first maximum
    top = np.partition(np.asarray(key[ok], np.float64), -2)[-2:] if ok.sum() > 1 else None
    gap = np.inf if top is None else float(top[1] - top[0])
    return best, gap


def log_softmax(z):
    z = np.asarray(z, dtype=np.float64)
    m = z.max()
    return z - (m + np.log(np.exp(z - m).sum()))


def _certain(key_lo, key_hi, best):
    """The entry `best` wins for every choice of keys inside [key_lo, key_hi]."""
    if best < 0:
        return bool(np.all(key_hi == -np.inf))
    others = np.delete(key_hi, best)
    return bool(key_lo[best] > (others.max() if others.size else -np.inf))


def sampled_verify(logits, drafts, q, u, tau: float, seed: int, offset: int,
                   delta: float = 0.0, key_slack: float = 0.0) -> dict:
    """Stochastic verify for a batch.

    logits [B][K+1][V] target logits (before the temperature), drafts [B][K]
    int, q [B][K][V] the draft distributions, u [B][K] acceptance uniforms in
    [0, 1).  Returns accepted [B], next_tok [B], and for choosing a check set:
    accept_margin [B] (smallest |p - u q| over the deciding comparisons,
    relative to p + u q) and key_gap [B] (gap between the two largest keys of
    the final draw), plus the row ("row") and kind ("residual", "bonus",
    "fallback") of the final draw.  With delta > 0 it also reports whether the
    outcome is certain when every target probability may be off by a
    relative delta and every key by key_slack: accept_certain [B] (every
    acceptance comparison keeps its side) and draw_certain [B] (the final
    draw keeps its winner)."""
    logits = np.asarray(logits, dtype=np.float64)
    B, K1, V = logits.shape
    K = K1 - 1
    drafts = np.asarray(drafts).reshape(B, K)
    q = np.asarray(q, dtype=np.float64).reshape(B, K, V)
    u = np.asarray(u, dtype=np.float64).reshape(B, K)
    out = {"accepted": np.zeros(B, np.int32), "next_tok": np.zeros(B, np.int32),
           "accept_margin": np.full(B, np.inf), "key_gap": np.zeros(B),
           "row": np.zeros(B, np.int32), "kind": [""] * B,
           "accept_certain": np.ones(B, bool), "draw_certain": np.ones(B, bool)}
    for b in range(B):
        logp = np.stack([log_softmax(logits[b, j] / tau) for j in range(K1)])
        a = K
        for i in range(1, K + 1):
            d = int(drafts[b, i - 1])
            p = float(np.exp(logp[i - 1, d]))
            uq = float(u[b, i - 1] * q[b, i - 1, d])
            den = p + uq
            if den > 0:
                out["accept_margin"][b] = min(out["accept_margin"][b], abs(p - uq) / den)
            kept = bool(_f32(uq) < _f32(p))
            if kept and not p * (1 - delta) > uq * (1 + 1e-6):
                out["accept_certain"][b] = False
            if not kept and not p * (1 + delta) < uq * (1 - 1e-6):
                out["accept_certain"][b] = False
            if not kept:
                a = i - 1
                break
        g = gumbel_noise(seed, offset, b, a, V)
        kind = "bonus"
        if a < K:
            r = np.exp(logp[a]) - q[b, a]
            with np.errstate(divide="ignore"):
                logr = np.where(r > 0, np.log(np.where(r > 0, r, 1.0)), -np.inf)
            tok, gap = gumbel_argmax(logr, g)
            kind = "residual"
            if tok < 0:
                tok, gap = gumbel_argmax(logp[a], g)
                kind = "fallback"
        else:
            tok, gap = gumbel_argmax(logp[a], g)
        if delta > 0 or key_slack > 0:
            if a < K:
                pa = np.exp(logp[a])
                with np.errstate(divide="ignore", invalid="ignore"):
                    r_lo, r_hi = pa * (1 - delta) - q[b, a], pa * (1 + delta) - q[b, a]
                    k_lo = np.where(r_lo > 0, np.log(np.maximum(r_lo, 1e-300)) + g - key_slack, -np.inf)
                    k_hi = np.where(r_hi > 0, np.log(np.maximum(r_hi, 1e-300)) + g + key_slack, -np.inf)
                if kind == "fallback":
                    sure = bool(np.all(r_hi <= 0))
                    w = np.log1p(delta) + key_slack
                    sure = sure and _certain(logp[a] + g - w, logp[a] + g + w, tok)
                else:
                    sure = _certain(k_lo, k_hi, tok)
            else:
                w = np.log1p(delta) + key_slack
                sure = _certain(logp[a] + g - w, logp[a] + g + w, tok)
            out["draw_certain"][b] = sure
        out["accepted"][b] = a
        out["next_tok"][b] = tok
        out["key_gap"][b] = gap
        out["row"][b] = a
        out["kind"][b] = kind
    return out
