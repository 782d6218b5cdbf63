"""Pins for the fp64 oracle, checked against closed forms, invariants, finite
differences and brute force -- never against the oracle's own formula retyped.

Each plausible mistake in oracle/attention.py (a dropped scale, a transposed
operand, a wrong sign in the softmax backward, an off-by-one causal mask, a
log2 LSE, a missing max subtraction) fails at least one test here.
"""
import math

import numpy as np
import pytest

from oracle import (attention_backward, attention_backward_batched, attention_backward_jacobian,
                    attention_backward_key_rows,
                    attention_forward, attention_forward_batched, blockwise_attention_forward,
                    online_softmax_stats, score_matrix, softmax_rows)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rng(seed):
    return np.random.default_rng(seed)


def rand_head(seed, n, d, scale_qk=1.0):
    r = rng(seed)
    q = r.standard_normal((n, d)) * scale_qk
    k = r.standard_normal((n, d)) * scale_qk
    v = r.standard_normal((n, d))
    do = r.standard_normal((n, d))
    return q, k, v, do


def loss(q, k, v, do, scale, causal):
    o, _ = attention_forward(q, k, v, scale, causal)
    return float(np.sum(o * do))


# --------------------------------------------------------------------------- brute force
def brute_attention(q, k, v, scale, causal):
    """Pure-Python loops over scalars (tiny inputs only)."""
    n, d = len(q), len(q[0])
    out, lse = [], []
    for i in range(n):
        keys = [j for j in range(n) if (not causal or j <= i)]
        s = [scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        z = sum(math.exp(x) for x in s)
        w = [math.exp(x) / z for x in s]
        out.append([sum(w[a] * v[j][c] for a, j in enumerate(keys)) for c in range(len(v[0]))])
        lse.append(math.log(z))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_brute_force(causal):
    q, k, v, _ = rand_head(1, 6, 3)
    scale = 0.7
    o, lse = attention_forward(q, k, v, scale, causal)
    ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(o, ob, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------- closed forms
def test_two_key_sigmoid_closed_form():
    # one query, two keys: P = (sigmoid(s0 - s1), sigmoid(s1 - s0)), lse = log(e^s0 + e^s1)
    q = np.array([[1.0, 2.0]])
    k = np.array([[0.5, 0.25], [-1.0, 0.75]])
    v = np.array([[1.0, 2.0], [3.0, -1.0]])
    scale = 0.3
    s0 = scale * (1.0 * 0.5 + 2.0 * 0.25)
    s1 = scale * (1.0 * -1.0 + 2.0 * 0.75)
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    p1 = 1.0 - p0
    o, lse = attention_forward(q, k, v, scale, False)
    np.testing.assert_allclose(o[0], [p0 * 1 + p1 * 3, p0 * 2 - p1 * 1], rtol=1e-14)
    assert abs(lse[0] - math.log(math.exp(s0) + math.exp(s1))) < 1e-14


def test_huge_logits_do_not_overflow():
    # scores (1000, 999): a softmax without max subtraction overflows; the answer is a sigmoid of 1
    q = np.array([[1.0]])
    k = np.array([[1000.0], [999.0]])
    v = np.array([[1.0], [0.0]])
    o, lse = attention_forward(q, k, v, 1.0, False)
    assert abs(o[0, 0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-14
    assert abs(lse[0] - (1000.0 + math.log(1.0 + math.exp(-1.0)))) < 1e-12


@pytest.mark.parametrize("n,d", [(7, 4), (33, 8)])
def test_zero_query_closed_forms(n, d):
    _, k, v, do = rand_head(2, n, d)
    q = np.zeros((n, d))
    # non-causal: P = 1/N, O = column mean of V, lse = ln N
    o, lse = attention_forward(q, k, v, 0.5, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, np.full(n, math.log(n)), rtol=1e-14)
    _, _, dv = attention_backward(q, k, v, do, 0.5, False)
    np.testing.assert_allclose(dv, np.broadcast_to(do.sum(axis=0) / n, dv.shape), rtol=1e-12, atol=1e-13)
    # causal: P_ij = 1/(i+1) for j <= i, O_i = mean(V_0..V_i), lse_i = ln(i+1)
    o, lse = attention_forward(q, k, v, 0.5, True)
    want = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), rtol=1e-14, atol=1e-15)
    _, _, dv = attention_backward(q, k, v, do, 0.5, True)
    w = do / np.arange(1, n + 1)[:, None]                     # dO_i / (i+1)
    want_dv = np.cumsum(w[::-1], axis=0)[::-1]                 # sum over i >= j
    np.testing.assert_allclose(dv, want_dv, rtol=1e-12, atol=1e-13)


def test_causal_row_zero():
    q, k, v, _ = rand_head(3, 9, 5)
    scale = 0.37
    o, lse = attention_forward(q, k, v, scale, True)
    np.testing.assert_array_equal(o[0], v[0])
    assert abs(lse[0] - scale * float(q[0] @ k[0])) < 1e-14


def test_single_key_gives_v():
    q, k, v, _ = rand_head(4, 1, 6)
    o, lse = attention_forward(q, k, v, 0.2, False)
    np.testing.assert_array_equal(o, v)
    assert abs(lse[0] - 0.2 * float(q[0] @ k[0])) < 1e-14


# --------------------------------------------------------------------------- softmax invariants
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    q, k, _, _ = rand_head(5, 50, 16, scale_qk=3.0)
    p, _ = softmax_rows(score_matrix(q, k, 0.25, causal))
    np.testing.assert_allclose(p.sum(axis=1), np.ones(50), atol=1e-14)
    assert np.all(p >= 0)
    if causal:
        assert np.all(np.triu(p, 1) == 0.0)
        assert np.all(np.diag(p) > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_and_shifted_v(causal):
    q, k, v, _ = rand_head(6, 20, 8)
    c = rng(7).standard_normal(8)
    o, _ = attention_forward(q, k, np.broadcast_to(c, v.shape), 0.3, causal)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=1e-13, atol=1e-13)
    o1, _ = attention_forward(q, k, v, 0.3, causal)
    o2, _ = attention_forward(q, k, v + c, 0.3, causal)
    np.testing.assert_allclose(o2, o1 + c, rtol=1e-12, atol=1e-12)


def test_permutation_equivariance():
    q, k, v, do = rand_head(8, 24, 8)
    perm = rng(9).permutation(24)
    o1, l1 = attention_forward(q, k, v, 0.4, False)
    o2, l2 = attention_forward(q, k[perm], v[perm], 0.4, False)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)
    o3, _ = attention_forward(q[perm], k, v, 0.4, False)
    np.testing.assert_allclose(o3, o1[perm], rtol=1e-13, atol=1e-14)
    dq1, dk1, dv1 = attention_backward(q, k, v, do, 0.4, False)
    dq2, dk2, dv2 = attention_backward(q, k[perm], v[perm], do, 0.4, False)
    np.testing.assert_allclose(dq2, dq1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk2, dk1[perm], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv2, dv1[perm], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    q, k, v, do = rand_head(10, 16, 6)
    a = rng(11).standard_normal(6)
    scale = 0.45
    o1, l1 = attention_forward(q, k, v, scale, causal)
    o2, l2 = attention_forward(q, k + a, v, scale, causal)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + scale * (q @ a), rtol=1e-12, atol=1e-12)
    dq1, dk1, _ = attention_backward(q, k, v, do, scale, causal)
    dq2, dk2, _ = attention_backward(q, k + a, v, do, scale, causal)
    np.testing.assert_allclose(dq2, dq1, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk2, dk1, rtol=1e-10, atol=1e-11)


# --------------------------------------------------------------------------- gradients
@pytest.mark.parametrize("n,d", [(5, 3), (8, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences(n, d, causal):
    q, k, v, do = rand_head(12 + n + d, n, d)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss(q, k, v, do, scale, causal)
            x[idx] = old - h
            lm = loss(q, k, v, do, scale, causal)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(fd - g) / np.linalg.norm(g)
        assert err <= 1e-6, err


@pytest.mark.parametrize("causal", [False, True])
def test_key_row_gradients_match_central_differences(causal):
    """dK and dV of selected key rows (the large-N parity reference) against central
    differences of L = sum(dO * O) in those rows only, on chunks smaller than the rows."""
    n, d = 9, 4
    q, k, v, do = rand_head(71, n, d, scale_qk=1.5)
    scale = 0.6
    keys = [8, 2, 5]
    dk, dv = attention_backward_key_rows(q, k, v, do, scale, causal, keys, row_chunk=2, workers=2)
    h = 1e-6
    for x, g in ((k, dk), (v, dv)):
        fd = np.zeros_like(g)
        for a, j in enumerate(keys):
            for c in range(d):
                old = x[j, c]
                x[j, c] = old + h
                lp = loss(q, k, v, do, scale, causal)
                x[j, c] = old - h
                lm = loss(q, k, v, do, scale, causal)
                x[j, c] = old
                fd[a, c] = (lp - lm) / (2 * h)
        err = np.linalg.norm(fd - g) / np.linalg.norm(fd)
        assert err <= 1e-6, err


def test_key_row_gradients_skip_rows_that_cannot_see_the_keys():
    """Under the causal mask the key-row gradients of keys near the end use only the query
    rows from the first sampled key on; the result must not depend on the rows before it
    (changing them leaves the sampled dK, dV unchanged) and matches the full backward's."""
    n, d = 40, 6
    q, k, v, do = rand_head(72, n, d)
    keys = [39, 37, 31]
    dk, dv = attention_backward_key_rows(q, k, v, do, 0.4, True, keys, row_chunk=7)
    q2, do2 = q.copy(), do.copy()
    q2[:31] += 3.0
    do2[:31] *= -2.0
    dk2, dv2 = attention_backward_key_rows(q2, k, v, do2, 0.4, True, keys, row_chunk=5)
    np.testing.assert_allclose(dk2, dk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv2, dv, rtol=1e-12, atol=1e-13)
    _, fk, fv = attention_backward(q, k, v, do, 0.4, True)
    np.testing.assert_allclose(dk, fk[keys], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, fv[keys], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_closed_form_backward_equals_literal_jacobian(causal):
    q, k, v, do = rand_head(20, 40, 8, scale_qk=2.0)
    a = attention_backward(q, k, v, do, 0.35, causal)
    b = attention_backward_jacobian(q, k, v, do, 0.35, causal)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    q, k, v, do = rand_head(21, 64, 16, scale_qk=1.5)
    scale = 0.25
    dq, dk, dv, rowterm = attention_backward(q, k, v, do, scale, causal, return_rowterm=True)
    # rows of dS sum to zero  =>  sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0
    np.testing.assert_allclose(dk.sum(axis=0), np.zeros(16), atol=1e-11)
    # <Q, dQ> == <K, dK> (both equal sum dS * S over unmasked entries)
    a, b = float(np.sum(q * dq)), float(np.sum(k * dk))
    assert abs(a - b) <= 1e-10 * max(1.0, abs(a))
    # rowsum(P * dP) == rowsum(dO * O): the identity a kernel may use for its row term
    o, _ = attention_forward(q, k, v, scale, causal)
    np.testing.assert_allclose(rowterm, np.sum(do * o, axis=1), rtol=1e-10, atol=1e-12)
    # dV is linear in dO and sums like P^T dO: columns of P sum over queries
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-10, atol=1e-11)


# --------------------------------------------------------------------------- online softmax
def partitions(n, r):
    yield [n]
    yield [1] * n
    for bs in (160, 64, 7, 3):
        full, tail = divmod(n, bs)
        yield [bs] * full + ([tail] if tail else [])
    cuts = sorted(r.choice(np.arange(1, n), size=min(6, n - 1), replace=False).tolist())
    yield np.diff([0] + cuts + [n]).tolist()


def test_online_softmax_stats_match_full_row():
    r = rng(30)
    for n in (1, 5, 161, 700):
        s = r.standard_normal(n) * 20.0
        want = float(np.max(s)) + math.log(float(np.sum(np.exp(s - np.max(s)))))
        for parts in partitions(n, r):
            blocks = np.split(s, np.cumsum(parts)[:-1])
            m, l = online_softmax_stats(blocks)
            assert abs((m + math.log(l)) - want) <= 1e-12 * max(1.0, abs(want))
            assert m == float(np.max(s))
            m2, l2 = online_softmax_stats(blocks[::-1])          # any merge order
            assert abs(l2 - l) <= 1e-12 * l and m2 == m


def test_online_softmax_skips_fully_masked_blocks():
    s = np.array([-np.inf, -np.inf, 1.0, 2.0, -np.inf])
    m, l = online_softmax_stats([s[:2], s[2:4], s[4:]])
    assert m == 2.0 and abs(l - (1.0 + math.exp(-1.0))) < 1e-15


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 37, 300])
def test_blockwise_forward_matches_plain(causal, n):
    q, k, v, _ = rand_head(31 + n, n, 16, scale_qk=3.0)
    o, lse = attention_forward(q, k, v, 0.25, causal)
    for parts in partitions(n, rng(n)):
        ob, lb = blockwise_attention_forward(q, k, v, 0.25, causal, parts)
        np.testing.assert_allclose(ob, o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lb, lse, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- plumbing
def test_row_chunking_is_exact():
    q, k, v, do = rand_head(40, 130, 8)
    a = attention_forward(q, k, v, 0.3, True, row_chunk=1000)
    b = attention_forward(q, k, v, 0.3, True, row_chunk=17)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    ga = attention_backward(q, k, v, do, 0.3, True, row_chunk=1000)
    gb = attention_backward(q, k, v, do, 0.3, True, row_chunk=17)
    np.testing.assert_array_equal(ga[0], gb[0])
    for x, y in zip(ga[1:], gb[1:]):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


def test_batched_equals_per_head_and_heads_subset():
    r = rng(41)
    q, k, v, do = (r.standard_normal((2, 3, 20, 4)) for _ in range(4))
    o, lse = attention_forward_batched(q, k, v, 0.5, True, workers=3)
    dq, dk, dv = attention_backward_batched(q, k, v, do, 0.5, True, workers=2)
    for b in range(2):
        for h in range(3):
            oo, ll = attention_forward(q[b, h], k[b, h], v[b, h], 0.5, True)
            np.testing.assert_array_equal(o[b, h], oo)
            np.testing.assert_array_equal(lse[b, h], ll)
            g = attention_backward(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            np.testing.assert_array_equal(dq[b, h], g[0])
            np.testing.assert_array_equal(dk[b, h], g[1])
            np.testing.assert_array_equal(dv[b, h], g[2])
    o2, _ = attention_forward_batched(q, k, v, 0.5, True, heads=[4])
    assert np.isnan(o2[0, 0]).all() and np.array_equal(o2[1, 1], o[1, 1])
