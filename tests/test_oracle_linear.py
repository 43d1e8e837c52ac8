"""Pins of the linear speculative-sampling oracle (oracle/linear.py).

What the method fixes independently of the oracle's code: with the drafted
token drawn from the draft distribution p, the emitted token of a position is
distributed exactly as the target distribution q (the guarantee of
speculative sampling), the acceptance probability is sum_x min(p(x), q(x)),
p = q always accepts, a token q gives no mass is never accepted or emitted,
and the uniform extremes decide as the closed forms say.  p and q are the
exact laws w / R of the vocabulary oracle's integer weights (pinned in
test_oracle_vocab.py); chi-square tests at p < 1e-4.
"""
import numpy as np
import pytest
from scipy.stats import chisquare, norm

from oracle import weight_constants, weights
from oracle.linear import verify_linear_sample

U64 = np.uint64


def _law(row, T):
    c, a = weight_constants(T)
    w = weights(row, row.max(), c, a).astype(np.float64)
    return w / w.sum()


def _setup(V, T, seed, trials):
    rng = np.random.default_rng(seed)
    q_row = rng.normal(0, 1.5, V).astype(np.float32)
    p_row = rng.normal(0, 1.5, V).astype(np.float32)
    p = _law(p_row, T)
    x = rng.choice(V, size=trials, p=p).astype(np.int32)      # drafted tokens ~ p
    tl = np.broadcast_to(np.stack([q_row, q_row]), (trials, 2, V)).copy()
    dl = np.broadcast_to(p_row, (trials, 1, V)).copy()
    u = rng.integers(0, 2 ** 63, size=(trials, 2, 2), dtype=np.int64).astype(np.uint64) * U64(2)
    u += rng.integers(0, 2, size=(trials, 2, 2)).astype(np.uint64)
    return q_row, p_row, x, tl, dl, u


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_emitted_token_follows_target_law(T):
    V, trials = 8, 40000
    q_row, p_row, x, tl, dl, u = _setup(V, T, 5, trials)
    r = verify_linear_sample(tl, dl, x[:, None], T, u)
    first = r["out_tokens"][:, 0]
    q = _law(q_row, T)
    counts = np.bincount(first, minlength=V)
    assert chisquare(counts, q * trials).pvalue > 1e-4
    # acceptance probability sum_x min(p, q)
    p = _law(p_row, T)
    pa = np.minimum(p, q).sum()
    acc = (r["accept_len"] == 1).mean()
    z = (acc - pa) / np.sqrt(pa * (1 - pa) / trials)
    assert abs(z) < norm.isf(1e-4 / 2)


def test_equal_laws_accept_everything():
    rng = np.random.default_rng(6)
    B, D, V = 200, 3, 32
    rows = rng.normal(0, 2, (B, D + 1, V)).astype(np.float32)
    u = rng.integers(0, 2 ** 63, size=(B, D + 1, 2), dtype=np.int64).astype(np.uint64)
    x = np.stack([[int(np.argmax(rows[b, k])) for k in range(D)] for b in range(B)])
    r = verify_linear_sample(rows, rows[:, :D].copy(), x, 0.8, u)
    assert np.all(r["accept_len"] == D)
    assert np.array_equal(r["out_tokens"][:, :D], x)
    assert np.all(r["bonus"] >= 0) and np.all(r["out_tokens"][:, D] == r["bonus"])


def test_zero_target_mass_is_never_accepted_or_emitted():
    V, T = 16, 1.0
    rng = np.random.default_rng(7)
    q_row = rng.normal(0, 1, V).astype(np.float32)
    q_row[3] = -200.0                    # weight 0 under the target
    p_row = np.zeros(V, dtype=np.float32)
    p_row[3] = 5.0                       # the draft likes token 3
    n = 300
    u = rng.integers(0, 2 ** 63, size=(n, 2, 2), dtype=np.int64).astype(np.uint64)
    tl = np.broadcast_to(np.stack([q_row, q_row]), (n, 2, V)).copy()
    dl = np.broadcast_to(p_row, (n, 1, V)).copy()
    r = verify_linear_sample(tl, dl, np.full((n, 1), 3), T, u)
    assert np.all(r["accept_len"] == 0)
    assert not np.any(r["bonus"] == 3)
    # the residual only emits tokens where q > p
    q, p = _law(q_row, T), _law(p_row, T)
    assert np.all(q[r["bonus"]] > p[r["bonus"]])


def test_uniform_extremes():
    V = 4
    row = np.array([1.0, 0.5, 0.0, -1.0], dtype=np.float32)
    top = np.uint64(2 ** 64 - 1)
    # q == p: u = 0 and u = 2^64 - 1 both accept (floor(u A / 2^64) < A)
    for u0 in (np.uint64(0), top):
        u = np.array([[[u0, 0], [0, 0]]], dtype=np.uint64)
        r = verify_linear_sample(row[None, None].repeat(2, 1), row[None, None], [[1]], 1.0, u)
        assert r["accept_len"][0] == 1
    # q(x) slightly below p(x): u = 0 accepts, u = 2^64 - 1 rejects
    q_row = row.copy()
    q_row[1] -= 0.01
    for u0, want in ((np.uint64(0), 1), (top, 0)):
        u = np.array([[[u0, 0], [0, 0]]], dtype=np.uint64)
        r = verify_linear_sample(np.stack([q_row, q_row])[None], row[None, None], [[1]], 1.0, u)
        assert r["accept_len"][0] == want
    # a rejection with u1 = 0 emits the first token of positive residual weight
    u = np.array([[[top, 0], [0, 0]]], dtype=np.uint64)
    r = verify_linear_sample(np.stack([q_row, q_row])[None], row[None, None], [[1]], 1.0, u)
    q, p = _law(q_row, 1.0), _law(row, 1.0)
    assert r["bonus"][0] == int(np.nonzero(q > p)[0][0])
