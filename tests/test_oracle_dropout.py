"""Pins for the dropout oracle (oracle/dropout.py), none of them a retyped formula.

* Philox4x32-10 against the known-answer vectors published with the generator
  (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC '11, and the
  Random123 distribution's known-answer tests).
* p = 0 reduces to plain attention (pinned by tests/test_oracle.py).
* The gradients against central differences with the mask held fixed by the seed.
* A pure-Python brute force of the masked forward on a tiny head.
* Unbiasedness: the mean of the dropout forward over many seeds approaches the
  undropped O (fails if the keep-scale factor is missing or misplaced).
* Keep-rate statistics, seed / offset / head / row / column decorrelation, and the
  row-term identity rowsum(P * dP) = rowsum(dO * O) that lets kernels keep their
  undropped row term.
"""
import math

import numpy as np
import pytest

from oracle import (attention_backward, attention_backward_dropout, attention_backward_dropout_batched,
                    attention_forward, attention_forward_dropout, attention_forward_dropout_batched,
                    dropout_keep_mask, keep_scale, keep_threshold, philox4x32_10)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def rand_head(seed, n, d, scale_qk=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((n, d)) * scale_qk, r.standard_normal((n, d)) * scale_qk, r.standard_normal((n, d)),
            r.standard_normal((n, d)))


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    got = philox4x32_10(*ctr, *key)
    assert tuple(int(x) for x in got) == want


def test_philox_vectorised_equals_scalar_calls():
    c0 = np.array([0, 1, 7, 0xFFFFFFFF], dtype=np.int64)
    vec = philox4x32_10(c0, 5, 9, 3, 11, 13)
    for t, c in enumerate(c0):
        sc = philox4x32_10(int(c), 5, 9, 3, 11, 13)
        assert [int(w[t]) for w in vec] == [int(w) for w in sc]


def test_keep_threshold_values():
    assert keep_threshold(0.0) == 0 and keep_scale(0.0) == 1.0
    assert keep_threshold(0.5) == 1 << 15 and keep_scale(0.5) == 2.0
    assert keep_threshold(0.25) == 1 << 14
    assert keep_threshold(0.1) == 6553 and keep_scale(0.1) == 65536 / (65536 - 6553)
    assert keep_threshold(2 ** -17) == 0          # rounds down to "keep everything"
    assert keep_threshold(1 - 2 ** -40) == 0xFFFF
    for bad in (-0.1, 1.0, 1.5):
        with pytest.raises(ValueError):
            keep_threshold(bad)


def test_mask_follows_the_counter_layout():
    """Element (i, j) of head bh is 16-bit half (j mod 2) of word ((j mod 8) div 2) of
    Philox(j div 8, i, bh, offset; seed lo, seed hi), low half first."""
    seed, off, bh, p = 0x1234_5678_9ABC_DEF0, 3, 5, 0.3
    rows = [0, 2, 9]
    m = dropout_keep_mask(bh, rows, 21, p, seed, off)
    t = keep_threshold(p)
    for a, i in enumerate(rows):
        for j in range(21):
            w = int(philox4x32_10(j // 8, i, bh, off, seed & 0xFFFFFFFF, seed >> 32)[(j % 8) // 2])
            draw = (w & 0xFFFF) if j % 2 == 0 else (w >> 16)
            assert bool(m[a, j]) == (draw >= t)


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_plain_attention(causal):
    q, k, v, do = rand_head(3, 70, 8)
    o0, l0 = attention_forward(q, k, v, 0.4, causal)
    o1, l1 = attention_forward_dropout(q, k, v, 0.4, causal, 0.0, seed=99)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(l1, l0)
    g0 = attention_backward(q, k, v, do, 0.4, causal)
    g1 = attention_backward_dropout(q, k, v, do, 0.4, causal, 0.0, seed=99)
    for a, b in zip(g0, g1):
        np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_forward_matches_brute_force(causal):
    """Pure-Python loops: softmax over the visible keys, then keep / scale each probability."""
    q, k, v, _ = rand_head(4, 9, 3)
    scale, p, seed = 0.8, 0.35, 77
    o, lse = attention_forward_dropout(q, k, v, scale, causal, p, seed)
    mask = dropout_keep_mask(0, np.arange(9), 9, p, seed)
    assert 0 < mask.sum() < mask.size
    for i in range(9):
        keys = [j for j in range(9) if not causal or j <= i]
        s = [scale * sum(q[i, t] * k[j, t] for t in range(3)) for j in keys]
        z = sum(math.exp(x) for x in s)
        w = [math.exp(x) / z * (65536 / (65536 - math.floor(p * 65536)) if mask[i, j] else 0.0)
             for x, j in zip(s, keys)]
        for c in range(3):
            assert abs(o[i, c] - sum(w[a] * v[j, c] for a, j in enumerate(keys))) < 1e-13
        assert abs(lse[i] - math.log(z)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_gradients_match_central_differences(causal):
    n, d, scale, p, seed = 7, 3, 0.6, 0.4, 2024
    q, k, v, do = rand_head(5, n, d)
    g = attention_backward_dropout(q, k, v, do, scale, causal, p, seed)
    h = 1e-6

    def loss():
        return float(np.sum(attention_forward_dropout(q, k, v, scale, causal, p, seed)[0] * do))

    for x, gx in zip((q, k, v), g):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss()
            x[idx] = old - h
            lm = loss()
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        assert np.linalg.norm(fd - gx) <= 1e-6 * np.linalg.norm(gx)


@pytest.mark.parametrize("causal", [False, True])
def test_rowterm_identity_and_invariants(causal):
    q, k, v, do = rand_head(6, 50, 8, scale_qk=1.5)
    scale, p = 0.3, 0.2
    dq, dk, dv, t = attention_backward_dropout(q, k, v, do, scale, causal, p, 5, return_rowterm=True)
    o, _ = attention_forward_dropout(q, k, v, scale, causal, p, 5)
    np.testing.assert_allclose(t, np.sum(do * o, axis=1), rtol=1e-10, atol=1e-12)
    # rows of dS still sum to zero, so sum_j dK_j = 0; <Q, dQ> = <K, dK>
    np.testing.assert_allclose(dk.sum(axis=0), np.zeros(8), atol=1e-11)
    a, b = float(np.sum(q * dq)), float(np.sum(k * dk))
    assert abs(a - b) <= 1e-10 * max(1.0, abs(a))


def test_unbiased_over_seeds():
    """E[O_dropout] = O: the mean over S seeds sits within a few standard errors of O."""
    q, k, v, _ = rand_head(7, 12, 4)
    scale, p, S = 0.5, 0.5, 3000
    o_ref, _ = attention_forward(q, k, v, scale, False)
    runs = np.stack([attention_forward_dropout(q, k, v, scale, False, p, seed=s)[0] for s in range(S)])
    se = runs.std(axis=0) / math.sqrt(S)
    z = np.abs(runs.mean(axis=0) - o_ref) / np.maximum(se, 1e-12)
    assert z.max() < 5.0, z.max()
    # without the keep-scale factor the mean would be (1-p) O: far outside that band
    assert np.abs(runs.mean(axis=0) * (1 - p) - o_ref).max() > 10 * se.max()


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_rate_and_decorrelation(p):
    n = 256
    m = dropout_keep_mask(3, np.arange(n), n, p, seed=0xDEADBEEF12345)
    sigma = math.sqrt(p * (1 - p) / m.size)
    assert abs(m.mean() - (1 - p)) < 5 * sigma
    # each residue class of j (the eight draws of one Philox call) keeps at the same rate
    for r in range(8):
        sub = m[:, r::8]
        assert abs(sub.mean() - (1 - p)) < 5 * math.sqrt(p * (1 - p) / sub.size)
    # other heads, seeds, offsets and the transposed coordinates give different masks that agree
    # only at the rate of independent draws: P(equal) = p^2 + (1-p)^2
    agree = p * p + (1 - p) ** 2
    tol = 5 * math.sqrt(agree * (1 - agree) / m.size)
    for other in (dropout_keep_mask(4, np.arange(n), n, p, seed=0xDEADBEEF12345),
                  dropout_keep_mask(3, np.arange(n), n, p, seed=0xDEADBEEF12346),
                  dropout_keep_mask(3, np.arange(n), n, p, seed=0xDEADBEEF12345 + (1 << 32)),
                  dropout_keep_mask(3, np.arange(n), n, p, seed=0xDEADBEEF12345, offset=1),
                  m.T):
        assert abs((other == m).mean() - agree) < tol


def test_batched_uses_flat_head_index():
    r = np.random.default_rng(8)
    q, k, v, do = (r.standard_normal((2, 3, 20, 4)) for _ in range(4))
    o, lse = attention_forward_dropout_batched(q, k, v, 0.5, True, 0.3, 41, offset=2)
    g = attention_backward_dropout_batched(q, k, v, do, 0.5, True, 0.3, 41, offset=2)
    for b in range(2):
        for h in range(3):
            o1, l1 = attention_forward_dropout(q[b, h], k[b, h], v[b, h], 0.5, True, 0.3, 41, 2, bh=b * 3 + h)
            np.testing.assert_array_equal(o[b, h], o1)
            np.testing.assert_array_equal(lse[b, h], l1)
            g1 = attention_backward_dropout(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True, 0.3, 41, 2, bh=b * 3 + h)
            for a, c in zip(g, g1):
                np.testing.assert_array_equal(a[b, h], c)
