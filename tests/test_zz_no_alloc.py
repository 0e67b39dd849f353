"""infv2_sparse_attn_noalloc (the entry point for callers that cannot
allocate: its workspace is the library's static per-GPU scratch) against
infv2_sparse_attn with a caller workspace, through the C ABI: the same
kernels, so O and LSE must be bitwise equal.  Two calls in a row on each
path (decode split-KV partials, prefill fragment packs), the second with a
smaller input, so the second reuses scratch the first filled."""
import numpy as np
import pytest
import torch

import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import problems

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _case(cfg, n_kv, batch, n_q, seed):
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=seed)
    q0 = n_kv - n_q
    lp, _ = problems(cfg, n_kv=n_kv, batch=batch, n_q=n_q, q_pos0=q0)
    dev = torch.device("cuda:0")
    if x["q"].shape[1] == n_q:
        qh = x["q"]
    else:
        qh = x["q"][:, q0:].contiguous()
    Q, K, V = qh.to(dev), x["k"].to(dev), x["v"].to(dev)
    Kc1 = tbs.compress_k(lp, K)
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1)
    return lp, Q, K, V, idx, n_sel


@pytest.mark.parametrize("name,sizes", [
    ("decode", [(40000, 6, 1), (9000, 3, 1)]),          # split-KV partials in the scratch
    ("prefill32k", [(2085, 2, 2085), (1300, 1, 1300)]),  # fragment packs in the scratch
])
def test_noalloc_equals_sparse_attn(name, sizes):
    cfg = CONFIGS[name]
    for i, (n_kv, batch, n_q) in enumerate(sizes):
        _say(f"case: noalloc {name} call {i}: n_kv={n_kv} batch={batch} n_q={n_q}")
        lp, Q, K, V, idx, n_sel = _case(cfg, n_kv, batch, n_q, seed=500 + i)
        assert 0 < tbs.sparse_attn_workspace(lp) <= tbs.NOALLOC_SCRATCH_BYTES
        O_ref, lse_ref = tbs.sparse_attn(lp, Q, K, V, idx, n_sel)
        O = torch.full_like(O_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        tbs.sparse_attn_noalloc(lp, Q, K, V, idx, n_sel, O, lse)
        torch.cuda.synchronize()
        assert torch.equal(O, O_ref), i
        assert torch.equal(lse, lse_ref), i


def test_noalloc_refuses_a_problem_past_the_scratch():
    cfg = CONFIGS["prefill32k"]
    lp, _ = problems(cfg, n_kv=40000, batch=1)
    assert tbs.sparse_attn_workspace(lp) > tbs.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    e = lp._ext()
    Q = torch.zeros(e.q, dtype=torch.bfloat16, device=dev)
    K = torch.zeros(e.kv, dtype=torch.bfloat16, device=dev)
    idx = torch.zeros(e.rows * e.budget, dtype=torch.int32, device=dev)
    n_sel = torch.zeros(e.rows, dtype=torch.int32, device=dev)
    with pytest.raises(tbs.Infv2Error, match="static scratch"):
        tbs.sparse_attn_noalloc(lp, Q, K, K, idx, n_sel, torch.empty_like(Q))
