"""Pins of the draft top-K oracle (oracle/topk.py) against what the definition
fixes independently of its code: closed forms (a constant row, two tokens, one
dominant logit), brute force over tiny rows with ties (Python sorting and
math.fsum), normalisation of the full distribution, shift invariance."""
import itertools
import math

import numpy as np
import pytest

from oracle.topk import draft_topk, topk_row


def test_constant_row_closed_form():
    # every token has probability 1/V: log-prob -ln V, ties broken by id
    for V in (1, 7, 1024, 163840):
        K = min(V, 8)
        tok, lp = topk_row(np.full(V, 2.5, dtype=np.float32), K)
        assert tok.tolist() == list(range(K))
        assert np.all(lp == np.float32(-math.log(V)))


def test_two_tokens_closed_form():
    rng = np.random.default_rng(1)
    for _ in range(50):
        a, b = rng.normal(0, 5, 2).astype(np.float32)
        tok, lp = topk_row(np.array([a, b], dtype=np.float32), 2)
        hi, lo = (0, 1) if (a > b or a == b) else (1, 0)
        d = abs(float(a) - float(b))
        assert tok.tolist() == [hi, lo]
        assert lp[0] == np.float32(-math.log1p(math.exp(-d)))
        assert lp[1] == np.float32(-d - math.log1p(math.exp(-d)))


def test_dominant_logit():
    # one logit far above the rest: its log-prob is 0, the others -gap exactly
    x = np.zeros(4096, dtype=np.float32)
    x[1234] = 1e4
    tok, lp = topk_row(x, 3)
    assert tok.tolist() == [1234, 0, 1]
    assert lp[0] == 0.0 and lp[1] == np.float32(-1e4) and lp[2] == np.float32(-1e4)


@pytest.mark.parametrize("V", [1, 2, 3, 5, 6])
def test_brute_force_tiny_rows_with_ties(V):
    # small integer logits: plenty of ties; order by sorting (value desc, id asc)
    # and log-probs from math.fsum of the explicit exponentials
    for vals in itertools.islice(itertools.product(range(-2, 3), repeat=V), 400):
        x = np.array(vals, dtype=np.float32)
        want = sorted(range(V), key=lambda i: (-vals[i], i))
        z = math.fsum(math.exp(v) for v in vals)
        for K in range(1, V + 1):
            tok, lp = topk_row(x, K)
            assert tok.tolist() == want[:K]
            ref = np.array([math.log(math.exp(vals[i]) / z) for i in want[:K]])
            # one rounding to fp32: within half an fp32 ulp of the exact value
            ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
            assert np.all(np.abs(lp.astype(np.float64) - ref) <= 0.5 * ulp + 1e-12)


def test_full_distribution_normalised_and_topk_not_renormalised():
    rng = np.random.default_rng(2)
    x = rng.normal(0, 3, 4096).astype(np.float32)
    tok, lp = topk_row(x, 4096)
    assert sorted(tok.tolist()) == list(range(4096))
    assert abs(math.fsum(math.exp(float(v)) for v in lp) - 1.0) < 1e-5
    tok8, lp8 = topk_row(x, 8)
    assert np.array_equal(tok8, tok[:8]) and np.array_equal(lp8, lp[:8])
    mass = math.fsum(math.exp(float(v)) for v in lp8)
    assert 0.0 < mass < 0.999


def test_shift_invariance_and_shape():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 3, (2, 3, 500)).astype(np.float32)
    tok, lp = draft_topk(x, 4)
    tok2, lp2 = draft_topk(x + np.float32(64.0), 4)
    assert tok.shape == (2, 3, 4) and lp.dtype == np.float32
    assert np.array_equal(tok, tok2)
    assert np.abs(lp.astype(np.float64) - lp2).max() < 1e-5
    assert np.all(np.diff(lp, axis=-1) <= 0) and np.all(lp <= 0)
    for b in range(2):
        for d in range(3):
            assert len(set(tok[b, d].tolist())) == 4


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        topk_row(np.zeros(4, dtype=np.float32), 5)
    with pytest.raises(ValueError):
        topk_row(np.zeros(4, dtype=np.float32), 0)
