"""Pins for the oracle's attention backward (CPU only): central finite
differences of the oracle's own forward, torch autograd of a masked dense
softmax attention built independently from the same key sets, and torch's
scaled_dot_product_attention backward for the dense causal case (fp64)."""
import numpy as np
import torch

from oracle import Problem, attended_tokens, attention_rows, attention_rows_backward


def _random_sets(rng, n_kv, rows, prob, k_blocks=3):
    """Causal block sets in the method's shape: init, local, random others."""
    sets = []
    for p in rows:
        b_p = p // prob.B
        cand = [b for b in range(1, max(1, b_p - 1))]
        top = rng.choice(cand, size=min(k_blocks, len(cand)), replace=False).tolist() if cand else []
        blocks = sorted({0} | set(range(max(0, b_p - 1), b_p + 1)) | set(top))
        sets.append([attended_tokens(np.array(blocks), int(p), prob) for _ in range(prob.h_kv)])
    return sets


def test_finite_differences():
    rng = np.random.default_rng(1)
    prob = Problem(G=2, h_kv=2, d=8, B=16, io="f32")
    n_kv = 90
    rows = np.array([5, 17, 40, 63, 89])
    Q = rng.standard_normal((len(rows), prob.h_q, prob.d))
    K = rng.standard_normal((n_kv, prob.h_kv, prob.d))
    V = rng.standard_normal((n_kv, prob.h_kv, prob.d))
    W = rng.standard_normal((len(rows), prob.h_q, prob.d))
    sets = _random_sets(rng, n_kv, rows, prob)

    def loss(Q_, K_, V_):
        O, _ = attention_rows(Q_, K_, V_, sets, prob)
        return float((O * W).sum())

    dQ, dK, dV = attention_rows_backward(Q, K, V, sets, W, prob)
    eps = 1e-6
    for X, dX in ((Q, dQ), (K, dK), (V, dV)):
        for idx in [tuple(rng.integers(0, s) for s in X.shape) for _ in range(25)]:
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = [Xp if X is Y else Y for Y in (Q, K, V)]
            args_m = [Xm if X is Y else Y for Y in (Q, K, V)]
            num = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(num - dX[idx]) <= 1e-6 * max(1.0, abs(num)), (idx, num, dX[idx])


def test_matches_torch_autograd_of_a_masked_dense_attention():
    rng = np.random.default_rng(2)
    prob = Problem(G=4, h_kv=2, d=16, B=32, io="f32")
    n_kv = 300
    rows = np.sort(rng.choice(n_kv, size=30, replace=False))
    Q = rng.standard_normal((len(rows), prob.h_q, prob.d))
    K = rng.standard_normal((n_kv, prob.h_kv, prob.d))
    V = rng.standard_normal((n_kv, prob.h_kv, prob.d))
    dO = rng.standard_normal((len(rows), prob.h_q, prob.d))
    sets = _random_sets(rng, n_kv, rows, prob)
    dQ, dK, dV = attention_rows_backward(Q, K, V, sets, dO, prob)

    Qt = torch.tensor(Q, requires_grad=True)
    Kt = torch.tensor(K, requires_grad=True)
    Vt = torch.tensor(V, requires_grad=True)
    mask = torch.zeros((len(rows), prob.h_kv, n_kv), dtype=torch.bool)
    for r in range(len(rows)):
        for g in range(prob.h_kv):
            mask[r, g, torch.tensor(sets[r][g], dtype=torch.long)] = True
    heads = torch.arange(prob.h_q) // prob.G
    Kh, Vh = Kt[:, heads, :], Vt[:, heads, :]                      # [n_kv, h_q, d]
    z = torch.einsum("rhd,nhd->rhn", Qt, Kh) / np.sqrt(prob.d)
    z = z.masked_fill(~mask[:, heads, :], float("-inf"))
    O = torch.einsum("rhn,nhd->rhd", torch.softmax(z, dim=-1), Vh)
    (O * torch.tensor(dO)).sum().backward()
    np.testing.assert_allclose(dQ, Qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, Kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, Vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_dense_causal_matches_sdpa_backward():
    rng = np.random.default_rng(3)
    prob = Problem(G=2, h_kv=1, d=8, B=16, io="f32")
    n = 70
    Q = rng.standard_normal((n, prob.h_q, prob.d))
    K = rng.standard_normal((n, prob.h_kv, prob.d))
    V = rng.standard_normal((n, prob.h_kv, prob.d))
    dO = rng.standard_normal((n, prob.h_q, prob.d))
    sets = [[np.arange(p + 1)] for p in range(n)]
    dQ, dK, dV = attention_rows_backward(Q, K, V, sets, dO, prob)
    Qt = torch.tensor(Q.transpose(1, 0, 2)[None], requires_grad=True)        # [1, h, n, d]
    Kt = torch.tensor(K.transpose(1, 0, 2)[None], requires_grad=True)
    Vt = torch.tensor(V.transpose(1, 0, 2)[None], requires_grad=True)
    Ke, Ve = Kt.expand(1, prob.h_q, n, prob.d), Vt.expand(1, prob.h_q, n, prob.d)
    O = torch.nn.functional.scaled_dot_product_attention(Qt, Ke, Ve, is_causal=True)
    (O * torch.tensor(dO.transpose(1, 0, 2)[None])).sum().backward()
    np.testing.assert_allclose(dQ, Qt.grad[0].numpy().transpose(1, 0, 2), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dK, Kt.grad[0].numpy().transpose(1, 0, 2), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dV, Vt.grad[0].numpy().transpose(1, 0, 2), rtol=1e-9, atol=1e-12)


def test_keys_outside_every_set_get_no_gradient():
    rng = np.random.default_rng(4)
    prob = Problem(G=2, h_kv=1, d=8, B=16, io="f32")
    n_kv = 128
    rows = np.array([100, 127])
    sets = [[attended_tokens(np.array([0, 5, 6, 7]), int(p), prob)] for p in rows]
    Q = rng.standard_normal((2, prob.h_q, prob.d))
    K = rng.standard_normal((n_kv, 1, prob.d))
    V = rng.standard_normal((n_kv, 1, prob.d))
    dO = rng.standard_normal((2, prob.h_q, prob.d))
    _, dK, dV = attention_rows_backward(Q, K, V, sets, dO, prob)
    outside = np.ones(n_kv, bool)
    outside[np.concatenate([s[0] for s in sets])] = False
    assert not dK[outside].any() and not dV[outside].any()
    assert dK[~outside].any() and dV[~outside].any()
