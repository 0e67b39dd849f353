"""GPU parity of the attention backward (dQ, dK, dV with the selected sets
held fixed) against the fp64 oracle, through the C ABI.

Bars: the gradients are fp32 outputs of bf16 products (P and dZ enter the
matrix unit in bf16, relative rounding 2^-9); measured against the oracle's
fp64 gradients on the same inputs and the GPU's own block sets,
  * the largest error relative to the largest gradient entry of the tensor
    must stay below 2e-2 for bf16 I/O (1e-4 for fp32 I/O), and
  * row by row (the d features of one key's dK / dV, or of one token-head's
    dQ), the largest error must stay below the bar times max(1, the row's
    largest entry): an absolute bar (the bar of O) on rows whose entries are
    at most 1 and a relative one on larger rows, so that a row of small
    gradients in a tensor with large ones cannot hide a large error behind
    the normalisation by the tensor's largest entry.  (The error of an
    entry follows the sum of its terms, not its own size: block 0 is
    attended by every query, so the entries of its dK / dV rows sum
    thousands of terms and reach ~20, and one of them that cancels to ~0
    still carries the row's ~2^-9 relative rounding.)
"""
import numpy as np
import pytest
import torch

import oracle as orc
import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import gpu_set, problems, to_f64

pytestmark = pytest.mark.gpu

BAR = {"bf16": 2e-2, "f32": 1e-4}


def _say(*a):
    print(*a, flush=True)


def _grad_out(shape, dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=gen).to(dtype)


def _rel_err(got, ref):
    scale = max(float(np.abs(ref).max()), 1e-30)
    return float(np.abs(got - ref).max()) / scale


def _mixed_err(got, ref):
    """max over rows (last axis) of max|got - ref| / max(1, max|ref|)."""
    err = np.abs(got - ref).max(axis=-1)
    return float((err / np.maximum(1.0, np.abs(ref).max(axis=-1))).max())


def _check(cfg, lp, op, x, q0, dense, seed):
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    dO = _grad_out(Q.shape, Q.dtype, seed).to(dev)
    if dense:
        O, lse = tbs.dense_attn(lp, Q, K, V)
        dQ, dK, dV = tbs.dense_attn_bwd(lp, Q, K, V, O, lse, dO)
    else:
        Kc1 = tbs.compress_k(lp, K)
        S = tbs.block_scores(lp, Q, Kc1)
        idx, n_sel = tbs.topk_select(lp, S)
        O, lse = tbs.sparse_attn(lp, Q, K, V, idx, n_sel)
        dQ, dK, dV = tbs.sparse_attn_bwd(lp, Q, K, V, idx, n_sel, O, lse, dO)
    torch.cuda.synchronize()
    res = {"idx": None if dense else idx.cpu(), "n_sel": None if dense else n_sel.cpu()}
    n_kv = K.shape[1]
    worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    worst_abs = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    worst_mixed = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    biggest = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for b in range(lp.batch):
        pos = q0 + np.arange(lp.n_q)
        if dense:
            sets = [[np.arange(p // op.B + 1) for _ in range(op.h_kv)] for p in pos]
        else:
            sets = [[gpu_set(res, b, g, t) for g in range(op.h_kv)] for t in range(lp.n_q)]
        token_sets = [[orc.attended_tokens(sets[r][g], int(p), op) for g in range(op.h_kv)]
                      for r, p in enumerate(pos)]
        rQ, rK, rV = orc.attention_rows_backward(to_f64(x["q"][b]), to_f64(x["k"][b]),
                                                 to_f64(x["v"][b]), token_sets,
                                                 to_f64(dO[b].cpu()), op)
        gQ = dQ[b].cpu().double().numpy()
        gK = dK[b, :n_kv].cpu().double().numpy()
        gV = dV[b, :n_kv].cpu().double().numpy()
        worst["dQ"] = max(worst["dQ"], _rel_err(gQ, rQ))
        worst["dK"] = max(worst["dK"], _rel_err(gK, rK))
        worst["dV"] = max(worst["dV"], _rel_err(gV, rV))
        for name, got, ref in (("dQ", gQ, rQ), ("dK", gK, rK), ("dV", gV, rV)):
            worst_abs[name] = max(worst_abs[name], float(np.abs(got - ref).max()))
            worst_mixed[name] = max(worst_mixed[name], _mixed_err(got, ref))
            biggest[name] = max(biggest[name], float(np.abs(ref).max()))
    _say("relative errors", worst, "row errors / max(1, row max |ref|)", worst_mixed,
         "max-abs errors", worst_abs, "largest entries", biggest)
    for k, v in worst.items():
        assert v <= BAR[op.io], (k, v)
    for k, v in worst_mixed.items():
        assert v <= BAR[op.io], (k, "row", v)
    return worst


@pytest.mark.parametrize("n_kv,batch", [(1300, 1), (2085, 2)])
def test_bf16_sparse_backward(n_kv, batch):
    cfg = CONFIGS["prefill32k"]
    _say(f"case: bf16 sparse backward n_kv={n_kv} batch={batch}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=60 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    _check(cfg, lp, op, x, 0, False, seed=n_kv)


def test_bf16_sparse_backward_query_offset():
    # queries 1700..2499 of a 2500-key sequence: dK / dV get the contributions
    # of these queries only
    cfg = CONFIGS["prefill32k"]
    n_kv, q0 = 2500, 1700
    _say("case: bf16 sparse backward, q offset", n_kv, q0)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=61)
    xq = dict(x)
    xq["q"] = x["q"][:, q0:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=1, n_q=n_kv - q0, q_pos0=q0)
    _check(cfg, lp, op, xq, q0, False, seed=62)


def test_bf16_sparse_backward_several_token_windows():
    # 4300 query tokens: three windows of the dK / dV kernel (2048 tokens
    # each, the last one ragged), block 0 selected by every token of every
    # window
    cfg = CONFIGS["prefill32k"]
    n_kv = 4300
    _say("case: bf16 sparse backward, 3 windows", n_kv)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=63)
    lp, op = problems(cfg, n_kv=n_kv, batch=1)
    _check(cfg, lp, op, x, 0, False, seed=64)


@pytest.mark.parametrize("n_kv,batch", [(1000, 2), (64, 1)])
def test_bf16_dense_backward(n_kv, batch):
    cfg = CONFIGS["dense_switch"]
    _say(f"case: bf16 dense backward n_kv={n_kv} batch={batch}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=65 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    _check(cfg, lp, op, x, 0, True, seed=66)


def test_fp32_tiny_sparse_backward_generic_kernel():
    cfg = CONFIGS["tiny"]
    _say("case: fp32 tiny sparse backward")
    x = make_inputs(cfg)
    lp, op = problems(cfg)
    _check(cfg, lp, op, x, 0, False, seed=67)


def test_bf16_sparse_backward_generic_kernel():
    # G = 8, d = 64: the generic backward with bf16 loads
    import dataclasses
    cfg = dataclasses.replace(CONFIGS["prefill32k"], name="g8d64", h_q=32, h_kv=4, d=64, k=8,
                              n_needles=8)
    _say("case: bf16 G=8 d=64 sparse backward")
    x = make_inputs(cfg, n_kv=1100, batch=1, seed=69)
    lp, op = problems(cfg, n_kv=1100, batch=1)
    _check(cfg, lp, op, x, 0, False, seed=70)


def test_backward_is_repeatable():
    # dQ bitwise; dK / dV to fp32 accumulation-order rounding
    cfg = CONFIGS["prefill32k"]
    n_kv = 2100
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=68)
    lp, _ = problems(cfg, n_kv=n_kv, batch=1)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    dO = _grad_out(Q.shape, Q.dtype, 69).to(dev)
    Kc1 = tbs.compress_k(lp, K)
    idx, n_sel = tbs.topk_select(lp, tbs.block_scores(lp, Q, Kc1))
    O, lse = tbs.sparse_attn(lp, Q, K, V, idx, n_sel)
    r1 = tbs.sparse_attn_bwd(lp, Q, K, V, idx, n_sel, O, lse, dO)
    r1 = [t.clone() for t in r1]
    r2 = tbs.sparse_attn_bwd(lp, Q, K, V, idx, n_sel, O, lse, dO)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0])
    for a_, b_ in zip(r1[1:], r2[1:]):
        torch.testing.assert_close(a_, b_, rtol=1e-5, atol=1e-6)
