"""Pins for the oracle's varlen / paged-cache decode (CPU only).

The page gather is pinned to a closed form (pool entries that encode their
own page and row).  The varlen composition is pinned by causality, which the
method fixes: the output of the query at position p depends only on tokens
0..p, so a sequence of length L decoded on its own must give exactly the
row at position L-1 of the prefill of any longer sequence with the same
prefix (including its block set).  Paging is pinned by invariance: any page
placement of the same tokens gives the same result.
"""
import numpy as np
import pytest

from oracle import Problem, decode_varlen, forward_rows, gather_paged


def test_gather_paged_closed_form():
    B = 16
    pool = np.zeros((5, B, 1, 2))
    for pg in range(5):
        for r in range(B):
            pool[pg, r] = 1000 * pg + r
    table = np.array([3, 0, 4, 1])
    rows = gather_paged(pool, table, 50, B)
    assert rows.shape == (50, 1, 2)
    for u in range(50):
        assert rows[u, 0, 0] == 1000 * table[u // B] + u % B


def _seq(rng, n, prob):
    Q = rng.standard_normal((n, prob.h_q, prob.d))
    K = rng.standard_normal((n, prob.h_kv, prob.d))
    V = rng.standard_normal((n, prob.h_kv, prob.d))
    return Q, K, V


@pytest.mark.parametrize("lse_approx", [False, True])
def test_decode_of_a_prefix_equals_the_prefill_row(lse_approx):
    rng = np.random.default_rng(5)
    prob = Problem(G=2, h_kv=2, d=8, B=16, l_C1=8, s_C1=4, k=3, io="f32",
                   lse_approx=lse_approx)
    n_full = 700
    Q, K, V = _seq(rng, n_full, prob)
    lens = [9, 64, 65, 211, 700]           # below one kernel, block edges, ragged
    full = forward_rows(Q, K, V, np.array([L - 1 for L in lens]), prob, mode="sparse")
    Qb = np.stack([Q[L - 1: L] for L in lens])                      # [b, 1, h_q, d]
    Kb = np.zeros((len(lens), n_full, prob.h_kv, prob.d))
    Vb = np.zeros_like(Kb)
    for i, L in enumerate(lens):
        Kb[i, :L], Vb[i, :L] = K[:L], V[:L]
        Kb[i, L:], Vb[i, L:] = 1e3, -1e3                            # beyond the sequence
    out = decode_varlen(Qb, Kb, Vb, lens, prob, mode="sparse")
    for i, L in enumerate(lens):
        for g in range(prob.h_kv):
            np.testing.assert_array_equal(out[i]["sets"][0][g], full["sets"][i][g])
        np.testing.assert_allclose(out[i]["O64"][0], full["O64"][i], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out[i]["lse"][0], full["lse"][i], rtol=1e-12)


def test_paging_does_not_change_the_result():
    rng = np.random.default_rng(6)
    prob = Problem(G=2, h_kv=1, d=8, B=16, l_C1=8, s_C1=4, k=2, io="f32")
    lens = [40, 130, 17]
    n_q = 2
    max_blocks = 9
    seqs = [_seq(rng, L, prob) for L in lens]
    Qb = np.stack([s[0][L - n_q:] for s, L in zip(seqs, lens)])
    Kc = np.zeros((3, max_blocks * 16, 1, 8))
    Vc = np.zeros_like(Kc)
    for i, ((_, K, V), L) in enumerate(zip(seqs, lens)):
        Kc[i, :L], Vc[i, :L] = K, V
    # scatter into a shuffled pool of pages
    n_pages = 3 * max_blocks + 4
    order = rng.permutation(n_pages)
    table = order[: 3 * max_blocks].reshape(3, max_blocks)
    Kp = rng.standard_normal((n_pages, 16, 1, 8))
    Vp = rng.standard_normal((n_pages, 16, 1, 8))
    for i in range(3):
        for j in range(max_blocks):
            Kp[table[i, j]] = Kc[i, 16 * j: 16 * j + 16]
            Vp[table[i, j]] = Vc[i, 16 * j: 16 * j + 16]
    a = decode_varlen(Qb, Kc, Vc, lens, prob)
    b = decode_varlen(Qb, Kp, Vp, lens, prob, block_table=table)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x["O64"], y["O64"])
        np.testing.assert_array_equal(x["lse"], y["lse"])
        for r in range(n_q):
            np.testing.assert_array_equal(x["sets"][r][0], y["sets"][r][0])
