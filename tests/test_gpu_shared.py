"""S^shared, the optional output of infv2_block_scores, against the fp64
oracle on every kernel that forms it: the fast prefill sweep, the exact pass
(tiles with extreme logits, and the LSE approximation's tiles that keep the
exact LSE), the decode split pool, the LSE approximation's prefill and decode
sweeps, and the fp64 generic kernel.

Bars: 0 exactly for the kernels a token does not see; relative 1e-5 against
the oracle elsewhere (the bar of S^cmp).  S^cmp from the same call must be
bitwise the S^cmp of a call without S^shared, and bitwise the max-pool of
the returned S^shared over the visible kernels of each block -- except on
the LSE approximation's decode sweep, which recomputes the kernel before each
256-kernel chunk with a plain fp32 dot product instead of reading it from the
previous chunk's MFMA result: there the two agree to 1e-6 relative."""
import numpy as np
import pytest
import torch

import oracle as orc
import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import problems, to_f64

pytestmark = pytest.mark.gpu
REL = 1e-5


def _say(*a):
    print(*a, flush=True)


def _run(lp, q, k):
    dev = torch.device("cuda:0")
    Q, K = q.to(dev), k.to(dev)
    Kc1 = tbs.compress_k(lp, K)
    Kc2 = tbs.compress_k2(lp, K) if lp.lse_approx else None
    shape = (lp.batch, lp.h_kv, lp.n_q, tbs.n_kernels(lp))
    S_sh = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    S_with = tbs.block_scores(lp, Q, Kc1, Kc2=Kc2, S_shared=S_sh)
    S_without = tbs.block_scores(lp, Q, Kc1, Kc2=Kc2)
    torch.cuda.synchronize()
    return S_without.cpu(), S_with.cpu(), S_sh.cpu()


def _check(lp, op, x, rows_per_b, S_without, S_with, S_sh, pool_rel=0.0):
    n_kv, q0 = lp.n_kv, lp.q_pos0
    n_c1, n_blk = tbs.n_kernels(lp), tbs.n_blocks(lp)
    assert S_sh.shape[-1] == n_c1
    worst = 0.0
    for b, rows in rows_per_b.items():
        rows = np.asarray(rows, dtype=np.int64)
        Q, K = to_f64(x["q"][b]), to_f64(x["k"][b])
        pos = q0 + rows
        Kc1 = orc.compress_k(K[None], op)[0]
        Kc2 = orc.compress_k2(K[None], op)[0] if op.lse_approx else None
        _, sh_ref, _ = orc.selection_scores(Q[rows], Kc1, pos, n_kv, op, Kc2=Kc2)
        vis = orc.kernel_visible(np.arange(n_c1)[None, :], pos[:, None], op)
        for g in range(lp.h_kv):
            got = S_sh[b, g, rows].double().numpy()
            ref = sh_ref[:, g, :]
            assert not np.isnan(got).any(), f"S^shared not written (b={b}, g={g})"
            assert np.all(got[~vis] == 0.0), f"non-zero S^shared past the visible kernels"
            if vis.any():
                err = np.abs(got[vis] - ref[vis]) / np.maximum(np.abs(ref[vis]), 1e-30)
                worst = max(worst, float(err.max()))
            pooled = orc.max_pool_blocks(got, vis, n_blk, op)
            for r, p in enumerate(pos):
                b_p = int(p) // op.B
                s_with = S_with[b, g, rows[r], :b_p + 1].double().numpy()
                s_without = S_without[b, g, rows[r], :b_p + 1].double().numpy()
                assert np.array_equal(s_with, s_without), f"S^cmp changed at p={p}"
                pool = pooled[r, :b_p + 1]
                if pool_rel == 0.0:
                    assert np.array_equal(s_with, pool), \
                        f"S^cmp is not the max-pool of S^shared at p={p}"
                else:
                    assert np.array_equal(np.isneginf(s_with), np.isneginf(pool))
                    fin = ~np.isneginf(pool)
                    d = np.abs(s_with[fin] - pool[fin]) / np.abs(pool[fin])
                    assert d.max(initial=0.0) <= pool_rel, f"max-pool differs at p={p}"
    assert worst <= REL, f"S^shared relative error {worst:.3e}"
    return worst


def test_generic_fp32_tiny():
    cfg = CONFIGS["tiny"]
    _say("case: S^shared tiny fp32 (generic kernel)")
    x = make_inputs(cfg)
    lp, op = problems(cfg)
    res = _run(lp, x["q"], x["k"])
    _say("max rel", _check(lp, op, x, {0: np.arange(cfg.n_q)}, *res))


@pytest.mark.parametrize("n_kv,batch", [(1300, 2), (2085, 1)])
def test_bf16_prefill(n_kv, batch):
    cfg = CONFIGS["prefill32k"]
    _say(f"case: S^shared bf16 prefill n_kv={n_kv} batch={batch}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=31 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    res = _run(lp, x["q"], x["k"])
    rows = {b: np.arange(n_kv) for b in range(batch)}
    _say("max rel", _check(lp, op, x, rows, *res))


def test_bf16_prefill_q_offset():
    cfg = CONFIGS["prefill32k"]
    n_kv, q0 = 2500, 1700
    _say("case: S^shared chunked prefill", n_kv, q0)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=77)
    xq = dict(x)
    xq["q"] = x["q"][:, q0:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=1, n_q=n_kv - q0, q_pos0=q0)
    res = _run(lp, xq["q"], x["k"])
    _say("max rel", _check(lp, op, xq, {0: np.arange(n_kv - q0)}, *res))


def test_bf16_prefill_extreme_logits_exact_pass():
    # as in the selection parity test: one head with 64x larger queries, and
    # one block of 64x larger keys, send tiles to the exact pass
    cfg = CONFIGS["prefill32k"]
    n_kv, batch = 1500, 2
    _say("case: S^shared extreme logits", n_kv, batch)
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=5)
    x["q"][0, :, 5, :] *= 64
    x["k"][1, 1200:1264, 1, :] *= 64
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    res = _run(lp, x["q"], x["k"])
    rows = {b: np.arange(n_kv) for b in range(batch)}
    _say("max rel", _check(lp, op, x, rows, *res))


@pytest.mark.parametrize("n_kv,batch", [(4129, 3), (33, 1)])
def test_bf16_decode_split(n_kv, batch):
    cfg = CONFIGS["decode"]
    _say(f"case: S^shared decode n_kv={n_kv} batch={batch}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=41 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    res = _run(lp, x["q"], x["k"])
    _say("max rel", _check(lp, op, x, {b: np.array([0]) for b in range(batch)}, *res))


def test_bf16_split_four_query_tokens():
    # the split path serves up to 4 query tokens
    cfg = CONFIGS["prefill32k"]
    n_kv = 3001
    _say("case: S^shared split, 4 tokens", n_kv)
    x = make_inputs(cfg, n_kv=n_kv, batch=2, seed=13)
    xq = dict(x)
    xq["q"] = x["q"][:, n_kv - 4:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=2, n_q=4, q_pos0=n_kv - 4)
    res = _run(lp, xq["q"], x["k"])
    _say("max rel", _check(lp, op, xq, {b: np.arange(4) for b in range(2)}, *res))


def test_lse_approx_prefill():
    cfg = CONFIGS["prefill32k"]
    n_kv = 2085
    _say("case: S^shared LSE approximation prefill", n_kv)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=55)
    lp, op = problems(cfg, n_kv=n_kv, batch=1, lse_approx=True)
    res = _run(lp, x["q"], x["k"])
    _say("max rel", _check(lp, op, x, {0: np.arange(n_kv)}, *res))


@pytest.mark.parametrize("n_kv", [4129, 100])
def test_lse_approx_decode(n_kv):
    # 100 keys: the token sees fine kernels but no coarse kernel (exact LSE)
    cfg = CONFIGS["decode"]
    _say("case: S^shared LSE approximation decode", n_kv)
    x = make_inputs(cfg, n_kv=n_kv, batch=2, seed=60 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=2, lse_approx=True)
    res = _run(lp, x["q"], x["k"])
    _say("max rel", _check(lp, op, x, {b: np.array([0]) for b in range(2)}, *res,
                           pool_rel=1e-6))
