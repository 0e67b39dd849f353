"""Pins for the oracle's block selection (CPU only).

S^C1 is pinned to torch's scaled_dot_product_attention (its probabilities are
read out with identity values), the max-pool to a hand-written golden file and
to a second, sliding-window formulation, top-k to closed forms, a golden row
and brute-force enumeration of subsets.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import (Problem, dense_switch, kernel_visible, kernels_of_block, max_pool_blocks,
                    n_kernels, select_blocks, selection_scores)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "window":
                out.setdefault("window", {})[int(vals[0])] = [int(v) for v in vals[1:]]
            else:
                out[key] = vals
    return out


def test_visibility_brute_force():
    prob = Problem(G=1, h_kv=1, d=4)
    for p in range(0, 400):
        for j in range(0, 30):
            toks = range(16 * j, 16 * j + 32)
            assert bool(kernel_visible(j, p, prob)) == all(t <= p for t in toks)


def test_maxpool_golden_windows_and_values():
    gd = _read_golden("maxpool_window.txt")
    prob = Problem(G=1, h_kv=1, d=4)
    n_kv = int(gd["n_kv"][0])
    n_c1 = n_kernels(n_kv, prob.l_C1, prob.s_C1)
    S = np.array([float(v) for v in gd["S_shared"]])
    assert n_c1 == S.size
    n_blk = -(-n_kv // prob.B)
    for blk, win in gd["window"].items():
        assert kernels_of_block(blk, n_c1, prob) == win
    for key, p in (("S_cmp_p207", 207), ("S_cmp_p120", 120)):
        vis = kernel_visible(np.arange(n_c1), p, prob)[None, :]
        got = max_pool_blocks(S[None, :], vis, n_blk, prob)[0]
        want = np.array([float(v) for v in gd[key]])
        np.testing.assert_array_equal(got, want)


def test_maxpool_equals_padded_sliding_window():
    # Second formulation: pad one kernel on the left (floor((l_C1-1)/s_C1) = 1),
    # then the pages' max-pool with length l=5 and stride s=4.
    rng = np.random.default_rng(3)
    prob = Problem(G=1, h_kv=1, d=4)
    for n_kv in (64, 100, 208, 1000, 1024):
        n_c1 = n_kernels(n_kv, 32, 16)
        n_blk = -(-n_kv // 64)
        S = rng.random((5, n_c1))
        vis = np.ones((5, n_c1), bool)
        got = max_pool_blocks(S, vis, n_blk, prob)
        pad = (prob.l_C1 - 1) // prob.s_C1
        padded = np.concatenate([np.full((5, pad), -np.inf), S, np.full((5, 8), -np.inf)], axis=1)
        want = np.stack([padded[:, i * prob.s: i * prob.s + prob.l].max(axis=1)
                         for i in range(n_blk)], axis=1)
        np.testing.assert_array_equal(got, want)


def _rand_selection_case(rng, n_kv=700, G=4, h_kv=2, d=16, R=6):
    prob = Problem(G=G, h_kv=h_kv, d=d, io="f32")
    n_c1 = n_kernels(n_kv, 32, 16)
    Q = rng.standard_normal((R, G * h_kv, d)) * 2
    Kc1 = rng.standard_normal((h_kv, n_c1, d))
    pos = rng.integers(0, n_kv, R)
    pos[0], pos[1] = 0, 31          # no visible kernel / exactly one
    return prob, Q, Kc1, pos, n_kv


def test_scores_match_torch_sdpa_probabilities():
    # softmax(scale Q K^C1^T) with the visibility mask, read out of torch SDPA
    # by using the identity matrix as values; then summed over the group.
    rng = np.random.default_rng(4)
    prob, Q, Kc1, pos, n_kv = _rand_selection_case(rng)
    lse, S_sh, _ = selection_scores(Q, Kc1, pos, n_kv, prob)
    n_c1 = Kc1.shape[1]
    eye = torch.eye(n_c1, dtype=torch.float64)
    for r, p in enumerate(pos):
        vis = torch.from_numpy(kernel_visible(np.arange(n_c1), p, prob))
        for g in range(prob.h_kv):
            if not bool(vis.any()):
                assert np.all(S_sh[r, g] == 0)
                assert np.all(np.isneginf(lse[r, g * prob.G:(g + 1) * prob.G]))
                continue
            q = torch.from_numpy(Q[r, g * prob.G:(g + 1) * prob.G])[None]      # [1, G, d]
            k = torch.from_numpy(Kc1[g])[None]                                 # [1, n_c1, d]
            P = torch.nn.functional.scaled_dot_product_attention(
                q, k, eye[None], attn_mask=vis[None, None, :].expand(1, prob.G, n_c1))
            np.testing.assert_allclose(S_sh[r, g], P[0].sum(0).numpy(), rtol=1e-12, atol=1e-15)


def test_scores_invariants():
    rng = np.random.default_rng(5)
    prob, Q, Kc1, pos, n_kv = _rand_selection_case(rng)
    lse, S_sh, S_cmp = selection_scores(Q, Kc1, pos, n_kv, prob)
    n_c1 = Kc1.shape[1]
    for r, p in enumerate(pos):
        nv = int(kernel_visible(np.arange(n_c1), p, prob).sum())
        for g in range(prob.h_kv):
            assert S_sh[r, g].sum() == pytest.approx(prob.G if nv else 0.0, rel=1e-12)
            # invisible kernels carry no score
            assert np.all(S_sh[r, g, nv:] == 0)
    # Q = 0: uniform softmax -> S^shared = G/|V(p)| and lse = log|V(p)|
    lse0, S0, C0 = selection_scores(np.zeros_like(Q), Kc1, pos, n_kv, prob)
    for r, p in enumerate(pos):
        nv = int(kernel_visible(np.arange(n_c1), p, prob).sum())
        if nv:
            np.testing.assert_allclose(S0[r, :, :nv], prob.G / nv, rtol=1e-13)
            np.testing.assert_allclose(lse0[r], math.log(nv), rtol=1e-13)


def test_scores_head_permutation_and_planted_kernel():
    rng = np.random.default_rng(6)
    prob, Q, Kc1, pos, n_kv = _rand_selection_case(rng)
    _, S_sh, S_cmp = selection_scores(Q, Kc1, pos, n_kv, prob)
    perm = np.concatenate([rng.permutation(prob.G) + g * prob.G for g in range(prob.h_kv)])
    _, S_sh2, S_cmp2 = selection_scores(Q[:, perm], Kc1, pos, n_kv, prob)
    np.testing.assert_allclose(S_sh2, S_sh, rtol=1e-12, atol=1e-15)
    # planted kernel: every head of group 1 sees kernel 7 with a huge logit
    Kp = Kc1.copy()
    q = Q[-1, prob.G:2 * prob.G]
    Kp[1, 7] = 50.0 * q.sum(0) / np.linalg.norm(q.sum(0))
    Qp = Q.copy()
    Qp[-1, prob.G:2 * prob.G] = q.sum(0) / np.linalg.norm(q.sum(0)) * 10
    p = np.array([n_kv - 1])
    _, S3, C3 = selection_scores(Qp[-1:], Kp, p, n_kv, prob)
    assert S3[0, 1, 7] == pytest.approx(prob.G, rel=1e-9)
    blk = int(np.argmax(C3[0, 1, :-2]))
    assert 7 in kernels_of_block(blk, Kc1.shape[1], prob)


def test_topk_golden_row():
    gd = _read_golden("topk_row.txt")
    prob = Problem(G=1, h_kv=1, d=4, k=3)
    row = np.array([float(v) for v in gd["S_cmp"]])
    got = select_blocks(row, 586, prob)
    np.testing.assert_array_equal(got, [int(v) for v in gd["I"]])


def test_topk_all_ties_closed_form():
    # Q = 0 makes every score equal: top-k = the k lowest-index candidates.
    prob = Problem(G=1, h_kv=1, d=4, k=16)
    for p in (0, 63, 64, 200, 1100, 4095, 70000):
        b_p = p // 64
        row = np.full(b_p + 1, 0.25)
        got = select_blocks(row, p, prob)
        local = set(range(max(0, b_p - 1), b_p + 1))
        cand = [b for b in range(1, b_p + 1) if b not in local]
        want = sorted({0} & set(range(b_p + 1)) | local | set(cand[:16]))
        np.testing.assert_array_equal(got, want)
        assert got.size == min(b_p + 1, prob.budget)


def test_topk_brute_force_subsets():
    # The selected top-k is the unique k-subset of the candidates in which
    # every member beats every non-member under (score desc, index asc).
    rng = np.random.default_rng(7)
    prob = Problem(G=1, h_kv=1, d=4, k=3)
    for _ in range(60):
        b_p = int(rng.integers(0, 10))
        p = b_p * 64 + int(rng.integers(0, 64))
        row = rng.integers(0, 4, b_p + 1).astype(float) / 4      # many exact ties
        got = set(select_blocks(row, p, prob).tolist())
        init, local = {0}, set(range(max(0, b_p - 1), b_p + 1))
        cand = [b for b in range(b_p + 1) if b not in init | local]
        kk = min(3, len(cand))
        wins = []
        for sub in itertools.combinations(cand, kk):
            rest = [c for c in cand if c not in sub]
            if all((row[a] > row[c]) or (row[a] == row[c] and a < c) for a in sub for c in rest):
                wins.append(set(sub))
        assert len(wins) == 1
        assert got == (init & set(range(b_p + 1))) | local | wins[0]


def test_topk_k_zero_keeps_init_and_local_only():
    # k = 0 leaves the union of the initial and local blocks, whatever the scores
    prob = Problem(G=1, h_kv=1, d=4, k=0)
    rng = np.random.default_rng(9)
    for p in (0, 64, 130, 5000):
        b_p = p // 64
        got = select_blocks(rng.random(b_p + 1), p, prob)
        want = sorted({0} | set(range(max(0, b_p - 1), b_p + 1)))
        np.testing.assert_array_equal(got, want)


def test_topk_planted_block_and_init_local_always_in():
    rng = np.random.default_rng(8)
    prob = Problem(G=1, h_kv=1, d=4, k=16)
    for _ in range(50):
        p = int(rng.integers(0, 5000))
        b_p = p // 64
        row = rng.random(b_p + 1)
        row[0] = row[b_p] = -np.inf        # init/local need no score
        if b_p >= 4:
            star = int(rng.integers(1, b_p - 1))
            row[star] = 10.0
        got = set(select_blocks(row, p, prob).tolist())
        assert 0 in got and b_p in got and max(0, b_p - 1) in got
        if b_p >= 4:
            assert star in got
        assert len(got) == min(b_p + 1, prob.budget)


def test_dense_switch_threshold():
    prob = Problem(G=16, h_kv=2, d=128, k=64)
    assert dense_switch(4096, prob)              # 64 blocks <= 67
    assert dense_switch(67 * 64, prob)
    assert not dense_switch(67 * 64 + 1, prob)
    prob16 = Problem(G=16, h_kv=2, d=128, k=16)
    assert dense_switch(19 * 64, prob16) and not dense_switch(19 * 64 + 1, prob16)
