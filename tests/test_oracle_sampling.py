"""Pins of the stochastic-verify oracle (oracle/sampling.py) to things other
than itself: the generator's published known-answer vectors, the exactness of
Gumbel-max sampling, and the lossless property of speculative sampling
(output distribution = the target's), checked by chi-square tests over many
seeded trials, plus closed-form acceptance rates and special cases that reduce
to known behaviour.  All on the CPU; every trial is seeded, so the outcomes
are fixed."""
import numpy as np
import pytest
import scipy.stats

from oracle import sampling as S


# ------------------------------------------------------------- generator
@pytest.mark.parametrize("ctr,key,want", [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
])
def test_philox_known_answers(ctr, key, want):
    """Known-answer vectors published with the Random123 library for
    Philox4x32-10 (Salmon et al., SC 2011)."""
    got = S.philox4x32_10(np.array(ctr, np.uint64), np.array(key, np.uint64))
    assert [int(x) for x in got] == want


def test_uniform_grid_and_range():
    w = np.array([0, 1 << 9, 0xFFFFFFFF, 0x80000000], np.uint64)
    u = S.uniform_from_word(w)
    assert u[0] == 0.5 * 2.0 ** -23 and u[1] == 1.5 * 2.0 ** -23
    assert u[2] == 1.0 - 0.5 * 2.0 ** -23 and u[3] == 0.5 + 0.5 * 2.0 ** -23
    assert np.all(u.astype(np.float32).astype(np.float64) == u)    # exact in fp32
    noise = S.gumbel_noise(seed=7, offset=0, b=0, j=0, V=200_000)
    # standard Gumbel: mean = Euler-Mascheroni constant, variance = pi^2 / 6
    assert abs(noise.mean() - np.euler_gamma) < 0.01
    assert abs(noise.var() - np.pi ** 2 / 6) < 0.03


def test_gumbel_noise_streams_are_distinct():
    a = S.gumbel_noise(1, 0, 0, 0, 64)
    for args in [(2, 0, 0, 0), (1, 1, 0, 0), (1, 0, 1, 0), (1, 0, 0, 1)]:
        assert not np.array_equal(a, S.gumbel_noise(*args, 64))
    # the four words of one counter serve four consecutive entries
    w = S.philox4x32_10(np.array([0, 0, 0, 0], np.uint64),
                        np.array([1, 0], np.uint64))
    assert np.array_equal(a[:4], -np.log(-np.log(S.uniform_from_word(w))))


def _chi2_pvalue(counts, probs):
    counts = np.asarray(counts, np.float64)
    exp = np.asarray(probs, np.float64) * counts.sum()
    keep = exp > 0
    assert counts[~keep].sum() == 0, "a draw landed on a zero-probability entry"
    return scipy.stats.chisquare(counts[keep], exp[keep]).pvalue


# ------------------------------------------------------------- sampling
def test_gumbel_argmax_samples_the_distribution():
    p = np.array([0.05, 0.3, 0.0, 0.15, 0.4, 0.1])
    logw = np.where(p > 0, np.log(np.where(p > 0, p, 1)), -np.inf)
    counts = np.zeros(6)
    for n in range(20000):
        tok, _ = S.gumbel_argmax(logw, S.gumbel_noise(3, n, 0, 0, 6))
        counts[tok] += 1
    assert _chi2_pvalue(counts, p) > 1e-3


def _trials(N, V, K, logits_fn, q, tau, seed, rng):
    """Run N independent single-sequence verify steps with d_i ~ q_i; returns
    per-trial (accepted, next_tok, drafts)."""
    drafts = np.zeros((N, K), np.int64)
    logits = np.zeros((N, K + 1, V))
    for n in range(N):
        for i in range(K):
            drafts[n, i] = rng.choice(V, p=q[i])
        logits[n] = logits_fn(drafts[n])
    u = rng.random((N, K))
    qq = np.broadcast_to(q, (N, K, V))
    out = S.sampled_verify(logits, drafts, qq, u, tau, seed, offset=5)
    return out["accepted"], out["next_tok"], drafts


def test_first_token_is_distributed_as_the_target():
    """Lossless property (OCR explainer section 6.1): the first token a step
    emits -- the first draft if kept, else the residual draw -- follows the
    target's p_0 whatever the draft distribution."""
    V, K, tau = 5, 1, 0.8
    L0 = np.array([0.3, -1.0, 1.2, 0.0, 0.5])
    q = np.array([[0.5, 0.2, 0.05, 0.05, 0.2]])
    rng = np.random.default_rng(11)
    N = 20000
    a, nt, d = _trials(N, V, K, lambda dr: np.stack([L0, np.zeros(V)]), q, tau, 99, rng)
    first = np.where(a >= 1, d[:, 0], nt)
    p0 = np.exp(S.log_softmax(L0 / tau))
    assert _chi2_pvalue(np.bincount(first, minlength=V), p0) > 1e-3
    # closed form: P(keep d_1) = sum_v min(p_0(v), q_1(v))
    acc = np.minimum(p0, q[0]).sum()
    assert abs((a == 1).mean() - acc) < 4 * np.sqrt(acc * (1 - acc) / N)


def test_second_token_given_first_is_distributed_as_the_target():
    """With K = 2 and the target's second distribution depending on the first
    token, the second emitted token given a kept first draft x follows
    p_1(. | x)."""
    V, K, tau = 4, 2, 1.0
    L0 = np.array([0.2, 0.9, -0.4, 0.1])
    L1 = np.array([[1.0, 0.0, -1.0, 0.5], [-0.5, 0.8, 0.3, 0.0],
                   [0.0, 0.0, 1.5, -1.0], [0.4, -0.2, 0.1, 0.9]])
    q = np.array([[0.4, 0.3, 0.2, 0.1], [0.1, 0.2, 0.3, 0.4]])
    rng = np.random.default_rng(12)

    def logits_fn(dr):
        return np.stack([L0, L1[dr[0]], np.zeros(V)])

    a, nt, d = _trials(24000, V, K, logits_fn, q, tau, 7, rng)
    kept = a >= 1
    second = np.where(a >= 2, d[:, 1], nt)
    stat, dof = 0.0, 0
    for x in range(V):
        sel = kept & (d[:, 0] == x)
        counts = np.bincount(second[sel], minlength=V).astype(np.float64)
        exp = np.exp(S.log_softmax(L1[x] / tau)) * counts.sum()
        stat += ((counts - exp) ** 2 / exp).sum()
        dof += V - 1
    assert scipy.stats.chi2.sf(stat, dof) > 1e-3


def test_residual_draw_follows_normalised_positive_part():
    """Force a rejection (u close to 1, q(d) > p(d)): the target's token is
    drawn from max(0, p - q) normalised."""
    V = 6
    L0 = np.array([0.5, 0.1, -0.3, 0.8, 0.0, -1.0])
    p = np.exp(S.log_softmax(L0))
    q = np.array([0.02, 0.5, 0.08, 0.1, 0.2, 0.1])
    d = 1                                   # q(d) = 0.5 > p(d)
    N = 20000
    logits = np.broadcast_to(np.stack([L0, np.zeros(V)]), (N, 2, V))
    out = {"next_tok": np.zeros(N, np.int64)}
    res = np.maximum(p - q, 0)
    for n0 in range(0, N, 5000):
        o = S.sampled_verify(logits[n0:n0 + 5000], np.full((5000, 1), d),
                             np.broadcast_to(q, (5000, 1, V)), np.full((5000, 1), 0.999999),
                             1.0, seed=n0 + 1, offset=3)
        assert np.all(o["accepted"] == 0)
        out["next_tok"][n0:n0 + 5000] = o["next_tok"]
    counts = np.bincount(out["next_tok"], minlength=V)
    assert counts[d] == 0 and counts[1] == 0
    assert _chi2_pvalue(counts, res / res.sum()) > 1e-3


def test_draft_equal_to_target_is_always_kept():
    """q = p: u q < p for every u in [0, 1), so every draft is kept and the
    bonus token follows p_K."""
    V, K = 7, 3
    rng = np.random.default_rng(5)
    L = rng.normal(size=(K + 1, V))
    N = 6000
    tau = 1.3
    q = np.exp(np.stack([S.log_softmax(L[j] / tau) for j in range(K)]))
    d = np.stack([[rng.choice(V, p=q[i]) for i in range(K)] for _ in range(N)])
    out = S.sampled_verify(np.broadcast_to(L, (N, K + 1, V)), d,
                           np.broadcast_to(q, (N, K, V)), rng.random((N, K)), tau, 17, 0)
    assert np.all(out["accepted"] == K)
    pK = np.exp(S.log_softmax(L[K] / tau))
    assert _chi2_pvalue(np.bincount(out["next_tok"], minlength=V), pK) > 1e-3


def test_certain_draft_is_kept_with_target_probability():
    """q_1 one-hot on d: kept with probability p_0(d); a rejected d is never
    the residual draw."""
    V, N = 5, 20000
    L0 = np.array([0.0, 1.0, -0.5, 0.2, 0.7])
    p0 = np.exp(S.log_softmax(L0))
    d = 4
    q = np.zeros((1, V))
    q[0, d] = 1.0
    rng = np.random.default_rng(8)
    out = S.sampled_verify(np.broadcast_to(np.stack([L0, np.zeros(V)]), (N, 2, V)),
                           np.full((N, 1), d), np.broadcast_to(q, (N, 1, V)),
                           rng.random((N, 1)), 1.0, 23, 0)
    rate = (out["accepted"] == 1).mean()
    assert abs(rate - p0[d]) < 4 * np.sqrt(p0[d] * (1 - p0[d]) / N)
    rej = out["accepted"] == 0
    assert not np.any(out["next_tok"][rej] == d)


def test_low_temperature_reduces_to_greedy(oracle_mod):
    """tau -> 0 turns p_j into the one-hot of the greedy token, so the sampled
    verify keeps exactly the drafts greedy verification keeps and ends on the
    greedy token (checked against the greedy oracle's acceptance)."""
    V, K, B = 50, 4, 40
    rng = np.random.default_rng(9)
    L = rng.normal(size=(B, K + 1, V))
    g = L.argmax(-1)
    drafts = np.where(rng.random((B, K)) < 0.7, g[:, :K], rng.integers(0, V, (B, K)))
    q = rng.dirichlet(np.ones(V), size=(B, K))
    out = S.sampled_verify(L, drafts, q, rng.random((B, K)), 1e-4, 31, 0)
    for b in range(B):
        a, n = oracle_mod.accept(g[b].astype(np.int32), drafts[b].astype(np.int32))
        assert out["accepted"][b] == a
        assert out["next_tok"][b] == g[b, a]
