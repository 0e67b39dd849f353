"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle, at
sizes the oracle finishes in seconds that span several tiles and a ragged
tail, plus the degenerate cases of the method."""
import numpy as np
import pytest
import torch

import oracle as orc
import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import (check_compress, check_rows, problems, run_gpu_dense, run_gpu_sparse,
                    sample_rows)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_tiny_fp32_config_full():
    cfg = CONFIGS["tiny"]
    _say("case: tiny fp32 full", cfg)
    x = make_inputs(cfg)
    lp, op = problems(cfg)
    assert not tbs.use_dense(lp)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    check_compress(res, x["k"], op)
    rep = check_rows(res, x, op, lp.q_pos0, {0: np.arange(cfg.n_q)})
    _say(rep)


@pytest.mark.parametrize("n_kv,batch", [(2085, 2), (1217, 1), (1300, 1)])
def test_bf16_sparse_prefill_ragged(n_kv, batch):
    cfg = CONFIGS["prefill32k"]
    _say(f"case: bf16 sparse prefill n_kv={n_kv} batch={batch}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=7 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    assert not tbs.use_dense(lp)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    check_compress(res, x["k"], op)
    rows = {b: np.arange(n_kv) for b in range(batch)}
    rep = check_rows(res, x, op, 0, rows)
    _say(rep)


def test_bf16_chunked_prefill_q_offset():
    # queries 1700..2499 of a 2500-key sequence (q_pos0 > 0, ragged tiles)
    cfg = CONFIGS["prefill32k"]
    n_kv, q0 = 2500, 1700
    _say("case: chunked prefill", n_kv, q0)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=99)
    xq = dict(x)
    xq["q"] = x["q"][:, q0:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=1, n_q=n_kv - q0, q_pos0=q0)
    res = run_gpu_sparse(lp, xq["q"], x["k"], x["v"])
    rep = check_rows(res, xq, op, q0, {0: np.arange(n_kv - q0)})
    _say(rep)


@pytest.mark.parametrize("n_kv,batch", [(1000, 2), (64, 1), (1, 1)])
def test_bf16_dense_attention(n_kv, batch):
    cfg = CONFIGS["dense_switch"]
    _say(f"case: bf16 dense n_kv={n_kv} batch={batch}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=5 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    res = run_gpu_dense(lp, x["q"], x["k"], x["v"])
    rep = check_rows(res, x, op, 0, {b: np.arange(n_kv) for b in range(batch)}, dense=True)
    _say(rep)


def test_bf16_dense_attention_unaligned_q_offset():
    # queries 437..999: 16-token query tiles straddle 64-key blocks
    cfg = CONFIGS["dense_switch"]
    n_kv, q0 = 1000, 437
    _say("case: bf16 dense, q_pos0", q0)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=31)
    xq = dict(x)
    xq["q"] = x["q"][:, q0:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=1, n_q=n_kv - q0, q_pos0=q0)
    res = run_gpu_dense(lp, xq["q"], x["k"], x["v"])
    rep = check_rows(res, xq, op, q0, {0: np.arange(n_kv - q0)}, dense=True)
    _say(rep)


def test_fp32_dense_attention():
    cfg = CONFIGS["tiny"]
    x = make_inputs(cfg, n_kv=700, seed=3)
    lp, op = problems(cfg, n_kv=700)
    res = run_gpu_dense(lp, x["q"], x["k"], x["v"])
    check_rows(res, x, op, 0, {0: np.arange(700)}, dense=True)


def test_sparse_path_equals_dense_when_budget_covers_all_blocks():
    # the dense-switch configuration's rule on a shorter sequence: k=64 covers
    # all 40 blocks, so the sparse kernels must reproduce dense attention
    cfg = CONFIGS["dense_switch"]
    n_kv = 2560
    _say("case: sparse == dense, n_kv", n_kv)
    x = make_inputs(cfg, n_kv=n_kv, batch=2, seed=11)
    lp, op = problems(cfg, n_kv=n_kv, batch=2)
    assert tbs.use_dense(lp)
    sp = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    de = run_gpu_dense(lp, x["q"], x["k"], x["v"])
    for b in range(2):
        for g in range(lp.h_kv):
            for t in range(0, n_kv, 97):
                n = int(sp["n_sel"][b, g, t])
                assert n == t // 64 + 1
                assert sp["idx"][b, g, t, :n].tolist() == list(range(n))
    diff = (sp["O"].double() - de["O"].double()).abs().max().item()
    assert diff <= 2e-2
    rows = {b: np.arange(0, n_kv, 5) for b in range(2)}
    check_rows(sp, x, op, 0, rows)
    check_rows(de, x, op, 0, rows, dense=True)


@pytest.mark.parametrize("n_kv,batch", [(4129, 3), (2048, 2), (33, 1)])
def test_bf16_decode_step(n_kv, batch):
    cfg = CONFIGS["decode"]
    _say(f"case: decode n_kv={n_kv} batch={batch}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=21 + n_kv)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    check_compress(res, x["k"], op)
    rep = check_rows(res, x, op, n_kv - 1, {b: np.array([0]) for b in range(batch)})
    _say(rep)


def test_decode_incremental_compress_append():
    # K^C1 built for L-1 tokens, then the step appends the kernel completed by
    # the new token; the result must equal a full recompute bit for bit.
    cfg = CONFIGS["decode"]
    L = 32 + 16 * 40          # (L - 32) % 16 == 0: the new token completes a kernel
    x = make_inputs(cfg, n_kv=L, batch=2, seed=5)
    dev = torch.device("cuda:0")
    K = x["k"].to(dev)
    lp_prev, _ = problems(cfg, n_kv=L - 1, batch=2)
    lp, op = problems(cfg, n_kv=L, batch=2)
    n_prev, n_now = tbs.n_kernels(lp_prev), tbs.n_kernels(lp)
    assert n_now == n_prev + 1
    lp.c1_cap = lp_prev.c1_cap = n_now + 8
    lp_prev.kv_cap = L                 # the cache tensor holds L rows per sequence
    Kc1 = torch.zeros((2, lp.h_kv, n_now + 8, lp.d), dtype=K.dtype, device=dev)
    tbs.compress_k(lp_prev, K, Kc1)
    tbs.compress_k(lp, K, Kc1, c1_begin=n_prev, c1_end=n_now)
    torch.cuda.synchronize()
    ref = orc.compress_k(x["k"].double().numpy(), op)
    np.testing.assert_array_equal(Kc1[:, :, :n_now].cpu().double().numpy(), ref)


def test_deterministic_bitwise():
    cfg = CONFIGS["prefill32k"]
    x = make_inputs(cfg, n_kv=3000, batch=1, seed=17)
    lp, _ = problems(cfg, n_kv=3000, batch=1)
    r1 = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    r2 = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    for key in ("Kc1", "idx", "n_sel", "O", "lse"):
        assert torch.equal(r1[key], r2[key]), key
    b_last = (3000 - 1) // 64
    s1, s2 = r1["S_cmp"][..., :b_last + 1], r2["S_cmp"][..., :b_last + 1]
    assert torch.equal(torch.nan_to_num(s1), torch.nan_to_num(s2))


def test_all_equal_scores_pick_lowest_blocks():
    # Q = 0 makes every S^cmp equal: top-k must be the lowest-index candidates
    cfg = CONFIGS["prefill32k"]
    n_kv = 1600
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=1)
    x["q"].zero_()
    lp, op = problems(cfg, n_kv=n_kv, batch=1)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    for t in (0, 63, 64, 500, 1200, 1599):
        b_p = t // 64
        local = set(range(max(0, b_p - 1), b_p + 1))
        cand = [c for c in range(1, b_p + 1) if c not in local]
        want = sorted({0} | local | set(cand[:16]))
        for g in range(lp.h_kv):
            n = int(res["n_sel"][0, g, t])
            assert res["idx"][0, g, t, :n].tolist() == want
    check_rows(res, x, op, 0, {0: np.arange(0, n_kv, 13)})


def test_extreme_logits_take_exact_pass():
    # Sequence 0: head 5 of group 0 has 64x larger queries, so the other heads'
    # sums fall far below the token-wide exponent reference (underflow risk).
    # Sequence 1: keys of one late block are 64x larger, so later logits
    # overflow the first chunk's reference.  Both send tiles to the exact
    # selection pass; results must still match the oracle everywhere.
    cfg = CONFIGS["prefill32k"]
    n_kv, batch = 1500, 2
    _say("case: extreme logits", n_kv, batch)
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=5)
    x["q"][0, :, 5, :] *= 64
    x["k"][1, 1200:1264, 1, :] *= 64
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    check_compress(res, x["k"], op)
    rep = check_rows(res, x, op, 0, {b: np.arange(n_kv) for b in range(batch)})
    _say(rep)


@pytest.mark.parametrize("n_kv,lean", [(2600, False), (2600, True), (70000, False)])
def test_prefill_pipeline_matches_one_shot(n_kv, lean):
    # the two-stream range pipeline computes every row exactly as the one-shot
    # path: O and LSE bitwise equal, and both match the oracle (lean: the
    # streamed top-k selection, no S^cmp buffers; 70000 keys = 1094 blocks:
    # the attention splits the keys into ranges, in the one-shot call and in
    # every range call alike)
    cfg = CONFIGS["prefill32k"]
    _say("case: prefill pipeline, n_kv", n_kv, "lean", lean)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=23)
    lp, op = problems(cfg, n_kv=n_kv, batch=1)
    ref = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    Kc1 = torch.empty((1, lp.h_kv, tbs.n_kernels(lp), lp.d), dtype=Q.dtype, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((1, lp.h_q, lp.n_q), dtype=torch.float32, device=dev)
    pipe = tbs.PrefillPipeline(lp, 3, lean=lean)
    if n_kv == 2600:
        assert [c["r0"] for c in pipe.chunks] == [0, 896, 1728]
    for _ in range(2):                  # a second run reuses every buffer
        pipe.run(Q, K, V, Kc1, O, lse)
    torch.cuda.synchronize()
    assert torch.equal(O.cpu(), ref["O"])
    assert torch.equal(lse.cpu(), ref["lse"])
    assert torch.equal(Kc1.cpu(), ref["Kc1"])
    cuts = [c["r0"] for c in pipe.chunks[1:]]
    rows = sample_rows(n_kv, 40 if n_kv < 10000 else 12, np.random.default_rng(3),
                       must=(0, n_kv - 1, *cuts, *(r - 1 for r in cuts)))
    res = dict(ref, O=O.cpu(), lse=lse.cpu())
    _say(check_rows(res, x, op, 0, {0: rows}))


def test_k_zero_selects_init_and_local_blocks_only():
    cfg = CONFIGS["decode"]
    n_kv, batch = 4000, 2
    _say("case: decode k=0", n_kv, batch)
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=31)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch, k=0)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    b_p = (n_kv - 1) // 64
    for b in range(batch):
        for g in range(lp.h_kv):
            n = int(res["n_sel"][b, g, 0])
            assert res["idx"][b, g, 0, :n].tolist() == [0, b_p - 1, b_p]
    rep = check_rows(res, x, op, n_kv - 1, {b: np.array([0]) for b in range(batch)})
    _say(rep)


# From 1024 key blocks (65536 keys) on, the sparse prefill attention splits
# the keys into ranges of 128 blocks (8192 keys): a token whose blocks span
# several ranges is attended range by range and its partial results merged.
# These sizes span nine ranges; the rows sampled include the range edges, a
# tile that straddles one, and the split threshold.
RANGE_KEYS = 128 * 64
RANGE_EDGE_ROWS = (0, 63, 64, RANGE_KEYS - 65, RANGE_KEYS - 2, RANGE_KEYS - 1, RANGE_KEYS,
                   RANGE_KEYS + 1, RANGE_KEYS + 63, RANGE_KEYS + 64, 2 * RANGE_KEYS - 1,
                   2 * RANGE_KEYS, 2 * RANGE_KEYS + 63, 5 * RANGE_KEYS - 1, 5 * RANGE_KEYS,
                   65535, 65536, 65537)


@pytest.mark.parametrize("n_kv,batch,q0", [
    (70000, 1, 0),         # nine ranges
    (66000, 2, 0),         # two sequences
    (70000, 1, 60005),     # a query offset that is not a multiple of the tile
])
def test_bf16_sparse_prefill_key_ranges(n_kv, batch, q0):
    cfg = CONFIGS["prefill32k"]
    _say(f"case: key ranges n_kv={n_kv} batch={batch} q0={q0}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=31 + n_kv + q0)
    xq = dict(x)
    xq["q"] = x["q"][:, q0:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=batch, n_q=n_kv - q0, q_pos0=q0)
    res = run_gpu_sparse(lp, xq["q"], x["k"], x["v"])
    rng = np.random.default_rng(n_kv + batch)
    n_q = n_kv - q0
    must = tuple(t - q0 for t in RANGE_EDGE_ROWS) + (n_q - 1, n_q - 64)
    rows = {b: sample_rows(n_q, 30, rng, must=must) for b in range(batch)}
    rep = check_rows(res, xq, op, q0, rows)
    _say(rep)
