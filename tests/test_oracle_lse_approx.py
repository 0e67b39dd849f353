"""Pins for the oracle's LSE approximation (CPU only).

The coarse keys are pinned to brute-force means and to their identity with
four non-overlapping fine kernels; the estimate to a closed form on constant
keys (which also fixes the coarse visibility rule and the count correction);
the selection to its invariance for one head per group, where any per-row
normaliser leaves the ranking unchanged; and the fallback to the exact LSE
for queries that see no coarse kernel.
"""
import math

import numpy as np
import pytest

from oracle import (Problem, coarse_lse, coarse_visible, compress_k, compress_k2,
                    n_coarse_kernels, n_kernels, select_blocks, selection_scores)


def _int_keys(rng, n, h_kv, d):
    # small integers: every sum and every mean by a power of two is exact
    return rng.integers(-8, 9, size=(1, n, h_kv, d)).astype(np.float64)


def test_coarse_keys_brute_force_means():
    rng = np.random.default_rng(1)
    prob = Problem(G=1, h_kv=2, d=4, io="f32", lse_approx=True)
    n = 700
    K = _int_keys(rng, n, 2, 4)
    Kc2 = compress_k2(K, prob)
    n_c2 = (n - 128) // 64 + 1
    assert Kc2.shape == (1, 2, n_c2, 4) and n_coarse_kernels(n, prob) == n_c2
    for j in range(n_c2):
        for g in range(2):
            want = K[0, 64 * j: 64 * j + 128, g, :].sum(axis=0) / 128.0
            np.testing.assert_array_equal(Kc2[0, g, j], want)
    # a coarse kernel is the mean of the four fine kernels that tile it
    Kc1 = compress_k(K, prob)
    for j in range(n_c2):
        quad = Kc1[0, :, [4 * j, 4 * j + 2, 4 * j + 4, 4 * j + 6], :].mean(axis=0)
        np.testing.assert_array_equal(Kc2[0, :, j], quad)


def test_too_short_for_a_coarse_kernel():
    prob = Problem(G=1, h_kv=1, d=4, lse_approx=True)
    assert n_coarse_kernels(127, prob) == 0
    assert n_coarse_kernels(128, prob) == 1
    assert n_coarse_kernels(191, prob) == 1
    assert n_coarse_kernels(192, prob) == 2
    assert compress_k2(np.zeros((1, 100, 1, 4)), prob).shape == (1, 1, 0, 4)


@pytest.mark.parametrize("p", [126, 127, 190, 191, 255, 1000, 4095])
def test_constant_keys_closed_form(p):
    # Every key equal: z is the same for every kernel of a head, so the
    # estimate is z + ln(n_C2 visible) + ln(s_C2/s_C1) and every visible fine
    # kernel scores 1 / (4 n2) per head, G / (4 n2) after the group sum.
    # Without a visible coarse kernel the exact LSE gives 1 / n1 per head.
    rng = np.random.default_rng(p)
    G, d = 4, 8
    prob = Problem(G=G, h_kv=1, d=d, io="f32", lse_approx=True)
    n_kv = p + 1
    k_row = rng.standard_normal(d).astype(np.float32).astype(np.float64)   # exact in f32
    K = np.tile(k_row, (1, n_kv, 1, 1))
    Q = rng.standard_normal((1, G, d))
    Kc1 = compress_k(K, prob)[0]
    Kc2 = compress_k2(K, prob)[0]
    lse, S_shared, S_cmp = selection_scores(Q, Kc1, np.array([p]), n_kv, prob, Kc2=Kc2)
    n1 = (p - 31) // 16 + 1
    n2 = (p - 127) // 64 + 1 if p >= 127 else 0
    z = (Q[0] @ K[0, 0, 0]) / math.sqrt(d)
    if n2 > 0:
        np.testing.assert_allclose(lse[0], z + math.log(n2) + math.log(4.0), rtol=0, atol=1e-12)
        want = G / (4.0 * n2)
    else:
        np.testing.assert_allclose(lse[0], z + math.log(n1), rtol=0, atol=1e-12)
        want = G / float(n1)
    np.testing.assert_allclose(S_shared[0, 0, :n1], want, rtol=1e-12)
    causal = S_cmp[0, 0, :p // 64 + 1]
    np.testing.assert_allclose(causal[np.isfinite(causal)], want, rtol=1e-12)


def test_coarse_visibility_rule():
    prob = Problem(G=1, h_kv=1, d=4, lse_approx=True)
    # coarse kernel j covers tokens 64j .. 64j+127
    assert not coarse_visible(0, 126, prob) and coarse_visible(0, 127, prob)
    assert not coarse_visible(3, 318, prob) and coarse_visible(3, 319, prob)
    est = coarse_lse(np.ones((2, 1, 4)), np.ones((1, 5, 4)), np.array([126, 127]), prob)
    assert np.isnan(est[0, 0]) and np.isfinite(est[1, 0])


def test_one_head_per_group_selects_as_the_exact_lse():
    # With G = 1 the normaliser is one number per row: S^cmp is scaled by
    # exp(lse - lse~) and the top-k order is unchanged.
    rng = np.random.default_rng(5)
    d, n_kv = 16, 3000
    exact = Problem(G=1, h_kv=2, d=d, io="f32", k=5)
    approx = Problem(G=1, h_kv=2, d=d, io="f32", k=5, lse_approx=True)
    K = rng.standard_normal((1, n_kv, 2, d))
    Q = rng.standard_normal((40, 2, d))
    pos = np.sort(rng.choice(n_kv, size=40, replace=False))
    Kc1 = compress_k(K, exact)[0]
    Kc2 = compress_k2(K, approx)[0]
    lse_e, _, S_e = selection_scores(Q, Kc1, pos, n_kv, exact)
    lse_a, _, S_a = selection_scores(Q, Kc1, pos, n_kv, approx, Kc2=Kc2)
    for r, p in enumerate(pos):
        for g in range(2):
            f = math.exp(lse_e[r, g] - lse_a[r, g]) if np.isfinite(lse_e[r, g]) else 1.0
            fin = np.isfinite(S_e[r, g])
            np.testing.assert_array_equal(fin, np.isfinite(S_a[r, g]))
            np.testing.assert_allclose(S_a[r, g][fin], S_e[r, g][fin] * f, rtol=1e-10)
            np.testing.assert_array_equal(select_blocks(S_a[r, g], int(p), approx),
                                          select_blocks(S_e[r, g], int(p), exact))


def test_early_rows_fall_back_to_the_exact_lse():
    rng = np.random.default_rng(6)
    d = 8
    exact = Problem(G=4, h_kv=1, d=d, io="f32")
    approx = Problem(G=4, h_kv=1, d=d, io="f32", lse_approx=True)
    n_kv = 400
    K = rng.standard_normal((1, n_kv, 1, d))
    Q = rng.standard_normal((n_kv, 4, d))
    pos = np.arange(n_kv)
    Kc1 = compress_k(K, exact)[0]
    Kc2 = compress_k2(K, approx)[0]
    lse_e, _, S_e = selection_scores(Q, Kc1, pos, n_kv, exact)
    lse_a, _, S_a = selection_scores(Q, Kc1, pos, n_kv, approx, Kc2=Kc2)
    np.testing.assert_array_equal(lse_a[:127], lse_e[:127])
    np.testing.assert_array_equal(S_a[:127], S_e[:127])
    assert not np.allclose(lse_a[127:], lse_e[127:])
    # the estimate sums fewer, smoother terms: it stays within a few nats here
    assert np.abs(lse_a[127:] - lse_e[127:]).max() < 3.0
    assert n_kernels(n_kv, 32, 16) == Kc1.shape[1]
