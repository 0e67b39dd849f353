"""Pins for the oracle's attention and the whole forward path (CPU only).

Dense attention is pinned to torch's scaled_dot_product_attention (causal,
fp64); sparse attention to the same routine with a boolean mask built from the
selected block sets; the log-sum-exp to torch.logsumexp of masked logits.
"""
import numpy as np
import pytest
import torch

from oracle import Problem, attended_tokens, forward_rows, round_to_io
from synth import CONFIGS, make_inputs


def _sdpa(Q, K, V, mask, prob):
    """torch SDPA in fp64 with GQA by repeating K/V per group.  Q [n, h_q, d]."""
    q = torch.from_numpy(Q).permute(1, 0, 2)                          # [h_q, n, d]
    k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(prob.G, 0)
    v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(prob.G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()


def _rand(rng, n, prob):
    Q = round_to_io(rng.standard_normal((n, prob.h_q, prob.d)), prob.io)
    K = round_to_io(rng.standard_normal((n, prob.h_kv, prob.d)), prob.io)
    V = round_to_io(rng.standard_normal((n, prob.h_kv, prob.d)), prob.io)
    return Q, K, V


def test_dense_matches_torch_causal_sdpa():
    rng = np.random.default_rng(10)
    prob = Problem(G=4, h_kv=2, d=16, io="f32")
    n = 300
    Q, K, V = _rand(rng, n, prob)
    out = forward_rows(Q, K, V, np.arange(n), prob, mode="dense")
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    ref = _sdpa(Q, K, V, mask, prob)
    np.testing.assert_allclose(out["O64"], ref, rtol=0, atol=1e-12)


def test_sparse_matches_sdpa_with_block_mask_and_lse():
    rng = np.random.default_rng(11)
    prob = Problem(G=4, h_kv=2, d=16, io="f32", k=2)
    n = 640                                  # 10 blocks > budget 5: really sparse
    Q, K, V = _rand(rng, n, prob)
    rows = np.arange(n)
    out = forward_rows(Q, K, V, rows, prob, mode="sparse")
    assert out["mode"] == "sparse"
    for g in range(prob.h_kv):
        mask = torch.zeros(n, n, dtype=torch.bool)
        for p in rows:
            toks = attended_tokens(out["sets"][p][g], int(p), prob)
            mask[p, toks] = True
        sl = slice(g * prob.G, (g + 1) * prob.G)
        ref = _sdpa(Q[:, sl], K[:, g:g + 1], V[:, g:g + 1], mask,
                    Problem(G=prob.G, h_kv=1, d=prob.d, io="f32"))
        np.testing.assert_allclose(out["O64"][:, sl], ref, rtol=0, atol=1e-12)
        # lse against torch.logsumexp of the masked logits
        z = torch.einsum("nhd,md->nhm", torch.from_numpy(Q[:, sl]),
                         torch.from_numpy(K[:, g])) * prob.sm_scale
        z = z.masked_fill(~mask[:, None, :], float("-inf"))
        np.testing.assert_allclose(out["lse"][:, sl], torch.logsumexp(z, -1).numpy(),
                                   rtol=1e-13, atol=1e-13)


def test_sparse_equals_dense_when_budget_covers_everything():
    rng = np.random.default_rng(12)
    prob = Problem(G=4, h_kv=2, d=16, io="f32", k=8)
    n = 11 * 64                              # 11 blocks <= budget 11
    Q, K, V = _rand(rng, n, prob)
    rows = np.arange(0, n, 7)
    sp = forward_rows(Q, K, V, rows, prob, mode="sparse")
    de = forward_rows(Q, K, V, rows, prob, mode="dense")
    assert forward_rows(Q, K, V, rows[:1], prob)["mode"] == "dense"
    np.testing.assert_allclose(sp["O64"], de["O64"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sp["lse"], de["lse"], rtol=0, atol=1e-12)


def test_rows_within_budget_equal_dense_rows():
    # a query whose causal prefix has <= budget blocks attends to all of it
    rng = np.random.default_rng(13)
    prob = Problem(G=4, h_kv=2, d=16, io="f32", k=2)
    n = 1000
    Q, K, V = _rand(rng, n, prob)
    rows = np.array([0, 5, 63, 64, 200, 319])           # b_p <= 4 -> b_p+1 <= 5
    sp = forward_rows(Q, K, V, rows, prob, mode="sparse")
    de = forward_rows(Q, K, V, rows, prob, mode="dense")
    np.testing.assert_allclose(sp["O64"], de["O64"], rtol=0, atol=1e-12)


def test_local_blocks_cover_sliding_window():
    # coverage rule: with w = (N_local-1)*B, N_local >= ceil(w/B)+1 holds and
    # every token in [p-w+1, p] is attended
    rng = np.random.default_rng(14)
    for N_local in (1, 2, 3):
        prob = Problem(G=4, h_kv=1, d=8, io="f32", k=1, N_local=N_local)
        w = (N_local - 1) * prob.B
        assert N_local >= -(-w // prob.B) + 1
        n = 900
        Q, K, V = _rand(rng, n, prob)
        rows = rng.integers(0, n, 40)
        out = forward_rows(Q, K, V, rows, prob, mode="sparse")
        for r, p in enumerate(rows):
            toks = set(attended_tokens(out["sets"][r][0], int(p), prob).tolist())
            assert set(range(max(0, p - w + 1), p + 1)) <= toks


def test_group_shared_selection_and_softmax_normalisation():
    rng = np.random.default_rng(15)
    prob = Problem(G=4, h_kv=2, d=16, io="f32", k=2)
    n = 700
    Q, K, V = _rand(rng, n, prob)
    rows = rng.integers(0, n, 20)
    out = forward_rows(Q, K, V, rows, prob, mode="sparse")
    for r, p in enumerate(rows):
        for g in range(prob.h_kv):
            toks = attended_tokens(out["sets"][r][g], int(p), prob)
            for h in range(g * prob.G, (g + 1) * prob.G):
                z = Q[p, h] @ K[toks, g].T * prob.sm_scale
                assert np.exp(z - out["lse"][r, h]).sum() == pytest.approx(1.0, rel=1e-13)


def test_tiny_config_end_to_end_smoke():
    cfg = CONFIGS["tiny"]
    x = make_inputs(cfg, n_kv=640)
    prob = Problem(G=cfg.G, h_kv=cfg.h_kv, d=cfg.d, io=cfg.io, k=cfg.k)
    Q = x["q"][0].double().numpy()
    K = x["k"][0].double().numpy()
    V = x["v"][0].double().numpy()
    out = forward_rows(Q, K, V, np.array([0, 100, 639]), prob)
    assert out["mode"] == "sparse"
    assert all(len(s) == min(p // 64 + 1, prob.budget)
               for s, p in zip([o[0] for o in out["sets"]], [0, 100, 639]))
