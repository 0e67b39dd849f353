"""GPU parity of the LSE approximation (coarse kernels estimate the stage-1
softmax normaliser) against the fp64 oracle in the same mode, through the C
ABI: the fast prefill kernel, the exact kernel it hands early or extreme
tiles to, the generic fp64 kernel, and the one-sweep decode path."""
import numpy as np
import pytest
import torch

import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import check_compress, check_rows, problems, run_gpu_sparse, sample_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_tiny_fp32_generic_kernel():
    cfg = CONFIGS["tiny"]
    _say("case: approx tiny fp32", cfg.n_kv)
    x = make_inputs(cfg)
    lp, op = problems(cfg, lse_approx=True)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    check_compress(res, x["k"], op)
    _say(check_rows(res, x, op, 0, {0: np.arange(cfg.n_q)}))


@pytest.mark.parametrize("n_kv,batch", [(2085, 2), (1300, 1)])
def test_bf16_prefill_every_row(n_kv, batch):
    # rows 31..126 see fine kernels but no coarse one: their tiles take the
    # exact kernel with the exact LSE; every later row the coarse estimate
    cfg = CONFIGS["prefill32k"]
    _say(f"case: approx prefill n_kv={n_kv} batch={batch}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=40 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch, lse_approx=True)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    check_compress(res, x["k"], op)
    _say(check_rows(res, x, op, 0, {b: np.arange(n_kv) for b in range(batch)}))


def test_bf16_chunked_prefill_offset_across_the_first_coarse_kernel():
    # queries 100..1499: the first tile mixes rows without and with a coarse
    # kernel (position 127)
    cfg = CONFIGS["prefill32k"]
    n_kv, q0 = 1500, 100
    _say("case: approx chunked prefill", n_kv, q0)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=41)
    xq = dict(x)
    xq["q"] = x["q"][:, q0:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=1, n_q=n_kv - q0, q_pos0=q0, lse_approx=True)
    res = run_gpu_sparse(lp, xq["q"], x["k"], x["v"])
    _say(check_rows(res, xq, op, q0, {0: np.arange(n_kv - q0)}))


def test_bf16_prefill_extreme_logits():
    # large per-head spreads send tiles to the exact kernel (bad sums); its
    # approximate path must agree with the oracle too
    cfg = CONFIGS["prefill32k"]
    n_kv, batch = 1500, 2
    _say("case: approx extreme logits", n_kv)
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=42)
    x["q"][0, :, 5, :] *= 64
    lp, op = problems(cfg, n_kv=n_kv, batch=batch, lse_approx=True)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    _say(check_rows(res, x, op, 0, {b: np.arange(n_kv) for b in range(batch)}))


def test_bf16_prefill_32k_sampled_rows():
    cfg = CONFIGS["prefill32k"]
    _say("case: approx prefill 32k sampled rows")
    x = make_inputs(cfg)
    lp, op = problems(cfg, lse_approx=True)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    rows = sample_rows(cfg.n_q, 48, np.random.default_rng(3), must=(0, 126, 127, 128, cfg.n_q - 1))
    _say(check_rows(res, x, op, 0, {0: rows}))


@pytest.mark.parametrize("n_kv,batch", [(4129, 3), (128, 2), (100, 1), (33, 1)])
def test_bf16_decode(n_kv, batch):
    cfg = CONFIGS["decode"]
    _say(f"case: approx decode n_kv={n_kv} batch={batch}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=43 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch, lse_approx=True)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    check_compress(res, x["k"], op)
    _say(check_rows(res, x, op, n_kv - 1, {b: np.array([0]) for b in range(batch)}))


def test_bf16_decode_rows_across_the_first_coarse_kernel():
    # four query rows at positions 125..128: the first two keep the exact LSE
    cfg = CONFIGS["prefill32k"]
    n_kv, n_q = 129, 4
    _say("case: approx few rows across position 127")
    x = make_inputs(cfg, n_kv=n_kv, batch=2, seed=44)
    xq = dict(x)
    xq["q"] = x["q"][:, n_kv - n_q:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=2, n_q=n_q, q_pos0=n_kv - n_q, lse_approx=True)
    res = run_gpu_sparse(lp, xq["q"], x["k"], x["v"])
    _say(check_rows(res, xq, op, n_kv - n_q, {b: np.arange(n_q) for b in range(2)}))


def test_bf16_decode_full_cache_sampled():
    cfg = CONFIGS["decode"]
    _say("case: approx decode 16 x 128k (2 sequences checked)")
    x = make_inputs(cfg)
    lp, op = problems(cfg, lse_approx=True)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    _say(check_rows(res, x, op, cfg.n_kv - 1, {b: np.array([0]) for b in (0, 15)}))


@pytest.mark.parametrize("n_kv,n_q", [(131072, 1), (20000, 3), (130, 4)])
def test_fused_selection_equals_two_calls(n_kv, n_q):
    cfg = CONFIGS["prefill32k"]
    _say(f"case: approx select_blocks n_kv={n_kv} n_q={n_q}")
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(n_kv)
    K = torch.randn((2, n_kv, cfg.h_kv, cfg.d), generator=gen).to(torch.bfloat16).to(dev)
    Q = torch.randn((2, n_q, cfg.h_q, cfg.d), generator=gen).to(torch.bfloat16).to(dev)
    lp, _ = problems(cfg, n_kv=n_kv, batch=2, n_q=n_q, q_pos0=n_kv - n_q, lse_approx=True)
    Kc1, Kc2 = tbs.compress_k(lp, K), tbs.compress_k2(lp, K)
    S = tbs.block_scores(lp, Q, Kc1, Kc2=Kc2)
    idx_ref, n_ref = tbs.topk_select(lp, S)
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1, Kc2=Kc2)
    S2 = torch.full_like(S, float("nan"))
    idx2, n_sel2 = tbs.select_blocks(lp, Q, Kc1, S_cmp=S2, Kc2=Kc2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref) and torch.equal(n_sel, n_ref)
    assert torch.equal(idx2, idx_ref) and torch.equal(n_sel2, n_ref)
    b_last = (n_kv - 1) // 64
    assert torch.equal(torch.nan_to_num(S2[..., :b_last + 1]), torch.nan_to_num(S[..., :b_last + 1]))


def test_approximation_selects_close_to_the_exact_lse():
    # the estimate changes each head's weight in the group sum, so a few
    # selections may move; on these inputs about 99% of the entries stay
    cfg = CONFIGS["prefill32k"]
    n_kv = 8192
    _say("case: approx vs exact overlap", n_kv)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=45)
    lp_e, _ = problems(cfg, n_kv=n_kv, batch=1)
    lp_a, _ = problems(cfg, n_kv=n_kv, batch=1, lse_approx=True)
    dev = torch.device("cuda:0")
    Q, K = x["q"].to(dev), x["k"].to(dev)
    Kc1, Kc2 = tbs.compress_k(lp_e, K), tbs.compress_k2(lp_a, K)
    idx_e, n_e = tbs.topk_select(lp_e, tbs.block_scores(lp_e, Q, Kc1))
    idx_a, n_a = tbs.topk_select(lp_a, tbs.block_scores(lp_a, Q, Kc1, Kc2=Kc2))
    torch.cuda.synchronize()
    assert torch.equal(n_e, n_a)
    same = (idx_e == idx_a).float().mean().item()
    _say(f"fraction of equal idx entries: {same:.4f}")
    assert same > 0.9
