"""Pins of the oracle's vocabulary reduction and its integer softmax weights (CPU only).

  * argmax: a plain Python scan that keeps the first maximum (lowest id);
    rows with planted ties;
  * lse: scipy's logsumexp;
  * weights: w(m) = 2^32 exactly at the row maximum; 0 below 2^-32 of it;
    monotone in the logit; within 2e-6 relative of the exact 2^32 * 2^(y) for
    y = (l - m) log2(e) / T evaluated in high precision (this is what makes
    w/R the temperature-T softmax of "Dissecting DDTree's Tree-Parallel
    Evaluation Strategy", Section 3);
  * the Taylor constants equal the correctly rounded fp32 values of
    (ln 2)^n / n!, computed here with 50-digit decimals;
  * R equals the Python-integer sum of per-token weights computed one by one.
"""
import decimal
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import vocab_reduce, weight_constants, weights
from workloads import f32_to_bf16_bits


def _exact_f32(dec: decimal.Decimal) -> np.float32:
    """Correctly rounded fp32 of a decimal, via a bracketing search on fp32 neighbours."""
    f = np.float32(float(dec))
    lo = np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(f, np.float32(np.inf))
    cands = [lo, f, hi]
    errs = [abs(decimal.Decimal(float(c)) - dec) for c in cands]
    best = min(range(3), key=lambda i: errs[i])
    assert sorted(errs)[0] != sorted(errs)[1]          # never a midpoint
    return cands[best]


def test_taylor_constants_correctly_rounded():
    decimal.getcontext().prec = 50
    ln2 = decimal.Decimal(2).ln()
    _, a = weight_constants(1.0)
    for n in range(7):
        exact = ln2 ** n / math.factorial(n)
        assert a[n] == _exact_f32(exact), n


@pytest.mark.parametrize("T", [0.7, 1.0, 0.3, 2.5])
def test_weights_close_to_exact_softmax(T):
    rng = np.random.default_rng(int(T * 10))
    c, a = weight_constants(T)
    l = (rng.standard_normal(20000) * 4).astype(np.float32)
    m = l.max()
    w = weights(l, m, c, a)
    assert int(w[np.argmax(l)]) == 2 ** 32
    decimal.getcontext().prec = 40
    for i in rng.choice(len(l), 400, replace=False):
        y = (float(l[i]) - float(m)) * (1 / math.log(2)) / float(np.float32(T))
        exact = 2.0 ** (32 + y)
        if y < -31.5:
            assert int(w[i]) <= 2
            continue
        if exact < 2 ** 20:
            assert abs(int(w[i]) - exact) <= 1 + 2e-6 * exact
        else:
            assert abs(int(w[i]) / exact - 1) < 2e-6
    order = np.argsort(l, kind="stable")
    assert np.all(np.diff(w[order].astype(np.float64)) >= 0)            # monotone


def test_weights_cutoff_and_extremes():
    c, a = weight_constants(1.0)
    m = np.float32(10.0)
    far = np.float32(10.0 - 40.0 / float(c))
    assert int(weights(np.array([far], np.float32), m, c, a)[0]) == 0
    assert int(weights(np.array([m], np.float32), m, c, a)[0]) == 2 ** 32
    # total over a row is below 2^50 for V = 163840 (sums stay exact in uint64)
    assert 163840 * 2 ** 33 < 2 ** 64


def test_argmax_first_index_and_ties():
    rng = np.random.default_rng(11)
    B, N, V = 2, 5, 300
    x = rng.standard_normal((B, N, V)).astype(np.float32)
    x[0, 1, [17, 40, 299]] = 9.0                       # three-way tie
    x[1, 2, [0, 5]] = 9.0
    x[0, 3, 100] = -0.0
    x[0, 3, :] = np.where(np.arange(V) == 100, -0.0, -1.0)
    x[0, 3, 200] = 0.0                                  # -0 and +0 tie: first wins
    res = vocab_reduce(x, np.array([5, 4]), 0.0)
    for b in range(B):
        for n in range(N):
            if n >= [5, 4][b]:
                assert res["argmax"][b, n] == -1
                continue
            best, bi = None, -1
            for v in range(V):
                if best is None or x[b, n, v] > best:
                    best, bi = x[b, n, v], v
            assert res["argmax"][b, n] == bi
            assert res["maxv"][b, n] == best
    assert res["argmax"][0, 1] == 17 and res["argmax"][1, 2] == 0 and res["argmax"][0, 3] == 100
    assert np.signbit(res["maxv"][0, 3]) == False                      # written as +0.0


def test_lse_and_R_against_independent_sums():
    rng = np.random.default_rng(12)
    B, N, V = 1, 3, 257
    xb = f32_to_bf16_bits((rng.standard_normal((B, N, V)) * 3).astype(np.float32))
    res = vocab_reduce(xb, np.array([3]), 0.7, dtype="bf16")
    c, a = weight_constants(0.7)
    for n in range(N):
        row = (xb[0, n].astype(np.uint32) << 16).view(np.float32)
        assert abs(res["lse"][0, n] - logsumexp(row.astype(np.float64))) < 1e-12
        m = row.max()
        total = 0
        for v in range(V):
            total += int(weights(row[v:v + 1], m, c, a)[0])
        assert int(res["R"][0, n]) == total


def test_block_sums_partition_R():
    """R_blocks[k] is the exact sum over tokens [k*R_BLOCK, (k+1)*R_BLOCK) and the
    blocks add up to R (checked with Python integers, token by token)."""
    from oracle.vocab import R_BLOCK
    rng = np.random.default_rng(13)
    B, N, V = 1, 2, 2 * R_BLOCK + 1000
    xb = f32_to_bf16_bits((rng.standard_normal((B, N, V)) * 3).astype(np.float32))
    res = vocab_reduce(xb, np.array([1]), 1.0, dtype="bf16")
    c, a = weight_constants(1.0)
    row = (xb[0, 0].astype(np.uint32) << 16).view(np.float32)
    w = [int(x) for x in weights(row, row.max(), c, a)]
    nb = res["R_blocks"].shape[2]
    assert nb == 3
    for k in range(nb):
        assert int(res["R_blocks"][0, 0, k]) == sum(w[k * R_BLOCK:(k + 1) * R_BLOCK])
    assert sum(int(x) for x in res["R_blocks"][0, 0]) == int(res["R"][0, 0])
    assert not res["R_blocks"][0, 1].any()          # padding row
