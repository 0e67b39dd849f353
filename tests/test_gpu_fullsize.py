"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (same calls, same shapes), on outputs the oracle computes one by one:
K^C1 everywhere (bit-exact), and the selection, S^cmp, O and LSE of sampled
query rows that include the edge rows (first tokens, block boundaries, the
last token)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as orc
import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs, paged_cache, varlen_lengths

from parity import (check_compress, check_rows, gpu_set, problems, run_gpu_dense,
                    run_gpu_sparse, sample_rows, to_f64)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


EDGE_ROWS = (0, 1, 30, 31, 32, 47, 63, 64, 65, 127, 128, 1215, 1216, 1217, 4095, 4096)


@pytest.mark.parametrize("name,n_rows", [("prefill32k", 48), ("prefill128k", 40)])
def test_prefill_full_size(name, n_rows):
    cfg = CONFIGS[name]
    _say(f"case: {name} full size")
    x = make_inputs(cfg)
    lp, op = problems(cfg)
    assert not tbs.use_dense(lp)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    Kc1_ref = check_compress(res, x["k"], op)
    rng = np.random.default_rng(2024)
    rows = sample_rows(cfg.n_q, n_rows, rng, must=EDGE_ROWS + (cfg.n_q - 1, cfg.n_q - 64))
    rep = check_rows(res, x, op, 0, {0: rows}, Kc1_ref=Kc1_ref)
    _say(rep)


def test_decode_full_size():
    cfg = CONFIGS["decode"]
    _say("case: decode full size (16 x 131072 cache)")
    x = make_inputs(cfg)
    lp, op = problems(cfg)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    # K^C1 of the cache before this step, then the kernel the new token completes
    prev, _ = problems(cfg, n_kv=cfg.n_kv - 1, n_q=1, q_pos0=cfg.n_kv - 2)
    prev.kv_cap = cfg.n_kv
    n_prev, n_now = tbs.n_kernels(prev), tbs.n_kernels(lp)
    assert n_now == n_prev + 1 == 8191
    lp.c1_cap = prev.c1_cap = n_now
    Kc1 = torch.empty((cfg.batch, cfg.h_kv, n_now, cfg.d), dtype=K.dtype, device=dev)
    tbs.compress_k(prev, K, Kc1)
    # the step exactly as bench.py launches it: the append fused into the
    # selection (the new kernel formed inside the score sweep; scores and
    # top-k in one call, S^cmp not stored) with a preallocated workspace,
    # then the attention; the appended row is NaN beforehand
    ws_s = torch.empty(max(tbs.select_blocks_workspace(lp), tbs.block_scores_workspace(lp), 16),
                       dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(tbs.sparse_attn_workspace(lp), 16), dtype=torch.uint8, device=dev)
    bud = tbs.budget(lp)
    idx = torch.empty((cfg.batch, cfg.h_kv, 1, bud), dtype=torch.int32, device=dev)
    n_sel = torch.empty((cfg.batch, cfg.h_kv, 1), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((cfg.batch, lp.h_q, 1), dtype=torch.float32, device=dev)
    Kc1[:, :, n_prev:n_now] = float("nan")
    tbs.select_blocks_append(lp, Q, K, Kc1, n_prev, n_now, idx, n_sel, ws_s)
    tbs.sparse_attn(lp, Q, K, V, idx, n_sel, O, lse, ws_a)
    # S^cmp for the score check, and the two-call selection, bitwise the same
    S = tbs.block_scores(lp, Q, Kc1)
    idx2, n_sel2 = tbs.topk_select(lp, S)
    # the one-call step (infv2_decode_step, the list merge inside the
    # attention launch), on its own copy of the cache's K^C1: bitwise the same
    # Kc1, sets, O and LSE; its outputs are the ones checked below
    Kc1_s = Kc1.clone()
    Kc1_s[:, :, n_prev:n_now] = float("nan")
    ws_d = torch.empty(tbs.decode_step_workspace(lp), dtype=torch.uint8, device=dev)
    idx_s = torch.full_like(idx, 12345)
    n_sel_s = torch.full_like(n_sel, -7)
    O_s = torch.full_like(O, float("nan"))
    lse_s = torch.full_like(lse, float("nan"))
    tbs.decode_step(lp, Q, K, V, Kc1_s, n_prev, n_now, idx_s, n_sel_s, O_s, lse_s, ws_d)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(n_sel, n_sel2)
    assert torch.equal(Kc1_s, Kc1) and torch.equal(idx_s, idx) and torch.equal(n_sel_s, n_sel)
    assert torch.equal(O_s.view(torch.int16), O.view(torch.int16))
    assert torch.equal(lse_s.view(torch.int32), lse.view(torch.int32))
    res = dict(Kc1=Kc1_s.cpu(), S_cmp=S.cpu(), idx=idx_s.cpu(), n_sel=n_sel_s.cpu(),
               O=O_s.cpu(), lse=lse_s.cpu())
    del Q, K, V
    Kc1_ref = check_compress(res, x["k"], op)
    rep = check_rows(res, x, op, cfg.n_kv - 1, {b: np.array([0]) for b in range(cfg.batch)},
                     Kc1_ref=Kc1_ref)
    # the planted needles are close to the query direction: most are selected
    picked = sum(len(set(res["idx"][b, g, 0, :int(res["n_sel"][b, g, 0])].tolist())
                     & set(x["needles"][b].tolist()))
                 for b in range(cfg.batch) for g in range(cfg.h_kv))
    _say(rep, "needles selected:", picked, "of", cfg.batch * cfg.h_kv * x["needles"].shape[1])


def test_prefill_lean_selection_full_size():
    # the memory-lean prefill selection (the top-k streamed through the
    # score sweep, S^cmp never stored) at 32k, against the oracle's sets on
    # sampled rows with the edges, not only against the two-call path
    cfg = CONFIGS["prefill32k"]
    _say("case: lean streamed top-k, prefill32k full size")
    x = make_inputs(cfg)
    lp, op = problems(cfg)
    dev = torch.device("cuda:0")
    Q, K = x["q"].to(dev), x["k"].to(dev)
    Kc1 = tbs.compress_k(lp, K)
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1)
    torch.cuda.synchronize()
    res = dict(Kc1=Kc1.cpu(), idx=idx.cpu(), n_sel=n_sel.cpu())
    del Q, K, Kc1
    Kc1_ref = check_compress(res, x["k"], op)
    rng = np.random.default_rng(77)
    rows = sample_rows(cfg.n_q, 40, rng, must=EDGE_ROWS + (cfg.n_q - 1, cfg.n_q - 64))
    rep = check_rows(res, x, op, 0, {0: rows}, Kc1_ref=Kc1_ref, check_scores=False,
                     check_outputs=False)
    _say(rep)


def test_decode_varlen_paged_full_size():
    # the serving bench's step: 16 sequences with seeded lengths up to 131072
    # (the first at full length), pages in a shuffled pool, the new token
    # completing or not a kernel per sequence
    cfg = CONFIGS["decode"]
    lens = varlen_lengths(cfg.batch, cfg.n_kv, seed=cfg.seed + 100, must=(cfg.n_kv,))
    _say("case: varlen paged decode full size, lengths", lens.tolist())
    x = make_inputs(cfg)
    lp, op = problems(cfg, q_pos0=0)
    dev = torch.device("cuda:0")
    kp, vp, table = paged_cache(x["k"], x["v"], lens, cfg.B, cfg.seed + 101)
    Q, K, V, table = x["q"].to(dev), kp.to(dev), vp.to(dev), table.to(dev)
    del kp, vp
    seq = torch.tensor(lens, device=dev)
    Kc1 = torch.empty((cfg.batch, cfg.h_kv, tbs.n_kernels(lp), cfg.d), dtype=K.dtype, device=dev)
    tbs.compress_k_varlen(lp, K, seq - 1, Kc1, block_table=table)       # before this step
    tbs.compress_k_varlen(lp, K, seq, Kc1, block_table=table, last_n=1)
    idx, n_sel = tbs.select_blocks_varlen(lp, Q, Kc1, seq)
    O, lse = tbs.sparse_attn_varlen(lp, Q, K, V, seq, idx, n_sel, block_table=table)
    torch.cuda.synchronize()
    idx, n_sel, O, lse, Kc1 = idx.cpu(), n_sel.cpu(), O.cpu(), lse.cpu(), Kc1.cpu()
    del K, V
    # every sequence: bitwise equal to the one-sequence calls on its own rows
    for i, L in enumerate(int(v) for v in lens):
        p1 = tbs.Problem(batch=1, n_q=1, n_kv=L, q_pos0=L - 1, h_kv=cfg.h_kv, G=cfg.G, d=cfg.d,
                         k=cfg.k)
        Ki = x["k"][i:i + 1, :L].to(dev)
        Vi = x["v"][i:i + 1, :L].to(dev)
        K1 = tbs.compress_k(p1, Ki)
        i1, n1 = tbs.select_blocks(p1, Q[i:i + 1], K1)
        O1, l1 = tbs.sparse_attn(p1, Q[i:i + 1], Ki, Vi, i1, n1)
        torch.cuda.synchronize()
        n_c1 = tbs.n_kernels(p1)
        assert torch.equal(K1.cpu()[0, :, :n_c1], Kc1[i, :, :n_c1]), i
        assert torch.equal(i1.cpu()[0], idx[i]) and torch.equal(n1.cpu()[0], n_sel[i]), i
        assert torch.equal(O1.cpu()[0], O[i]) and torch.equal(l1.cpu()[0], lse[i]), i
        del Ki, Vi, K1
    # the oracle on four sequences (the longest, the shortest, two others)
    order = np.argsort(lens)
    for i in sorted({0, int(order[0]), int(order[len(lens) // 2]), int(order[-2])}):
        L = int(lens[i])
        res_i = dict(idx=idx[i:i + 1], n_sel=n_sel[i:i + 1], O=O[i:i + 1], lse=lse[i:i + 1])
        x_i = dict(q=x["q"][i:i + 1], k=x["k"][i:i + 1, :L], v=x["v"][i:i + 1, :L])
        Kc1_ref = orc.compress_k(to_f64(x_i["k"]), op)[0]
        np.testing.assert_array_equal(to_f64(Kc1[i, :, :Kc1_ref.shape[1]]), Kc1_ref)
        rep = check_rows(res_i, x_i, op, L - 1, {0: np.array([0])}, check_scores=False,
                         Kc1_ref={0: Kc1_ref})
        _say("sequence", i, "length", L, rep)


def test_dense_switch_full_size():
    cfg = CONFIGS["dense_switch"]
    _say("case: dense switch full size (8 x 4096)")
    x = make_inputs(cfg)
    lp, op = problems(cfg)
    assert tbs.use_dense(lp)
    de = run_gpu_dense(lp, x["q"], x["k"], x["v"])
    sp = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    # the sparse path's selection is every causal block, so it equals dense
    nsel = sp["n_sel"].numpy()
    want = (np.arange(cfg.n_q) // 64 + 1)[None, None, :]
    assert np.array_equal(nsel, np.broadcast_to(want, nsel.shape))
    assert (sp["O"].double() - de["O"].double()).abs().max().item() <= 2e-2
    rng = np.random.default_rng(7)
    rows = {b: sample_rows(cfg.n_q, 24, rng, must=(0, 63, 64, 4095)) for b in (0, 3, 7)}
    check_rows(de, x, op, 0, rows, dense=True)
    check_rows(sp, x, op, 0, rows)


@pytest.mark.parametrize("batch", [1, 2])
def test_backward_full_size_prefill32k(batch):
    # the bench's backward call (32k, bf16, the stash path); dQ on sampled
    # query rows (edges included), dK / dV on the keys of two sampled blocks
    # against the oracle's backward over exactly the rows whose GPU sets hold
    # those blocks (every other row adds nothing to their gradients).  Batch 1
    # is the bench's launch; at either batch the dZ stash of the whole
    # sequence does not fit the workspace budget, so the backward runs query
    # chunk by chunk.  At batch 2 the second sequence is the one checked.
    cfg = dataclasses.replace(CONFIGS["prefill32k"], batch=batch)
    sb = batch - 1
    _say(f"case: backward full size (prefill32k, batch {batch})")
    x = make_inputs(cfg)
    lp, op = problems(cfg)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    gen = torch.Generator().manual_seed(321)
    dO_cpu = torch.randn(Q.shape, generator=gen).to(Q.dtype)
    dO = dO_cpu.to(dev)
    Kc1 = tbs.compress_k(lp, K)
    idx, n_sel = tbs.topk_select(lp, tbs.block_scores(lp, Q, Kc1))
    O, lse = tbs.sparse_attn(lp, Q, K, V, idx, n_sel)
    dQ, dK, dV = tbs.sparse_attn_bwd(lp, Q, K, V, idx, n_sel, O, lse, dO)
    torch.cuda.synchronize()
    res = dict(idx=idx.cpu(), n_sel=n_sel.cpu())
    # 2 KB of dZ per selected block of every (query, group) row
    whole_stash = cfg.batch * lp.h_kv * cfg.n_q * (lp.N_init + lp.N_local + lp.k) * 2048
    ws = tbs.sparse_attn_bwd_workspace(lp)
    _say("workspace bytes:", ws, "a whole-sequence stash:", whole_stash)
    assert ws <= 1 << 30
    assert ws < whole_stash              # the stash holds part of the queries
    q_rows = np.array(sorted({0, 1, 63, 64, 65, 1215, 1216, 4096, 20000, cfg.n_q - 64,
                              cfg.n_q - 1} | set(np.random.default_rng(9).choice(cfg.n_q, 8,
                                                                               replace=False).tolist())))
    blocks = (100, 317)
    idx_np = res["idx"][sb].numpy()                                  # [h_kv, n_q, budget]
    hit = np.zeros(cfg.n_q, bool)
    for blk in blocks:
        hit |= (idx_np == blk).any(axis=-1).any(axis=0)
    k_rows = np.nonzero(hit)[0]
    rows = np.union1d(q_rows, k_rows)
    _say("rows:", len(rows), "of which attend the sampled blocks:", len(k_rows))
    gQ = dQ[sb].cpu()
    key_idx = np.concatenate([np.arange(blk * cfg.B, (blk + 1) * cfg.B) for blk in blocks])
    gK = dK[sb, key_idx].cpu().double().numpy()
    gV = dV[sb, key_idx].cpu().double().numpy()
    del Q, K, V, O, lse, dO, dQ, dK, dV, Kc1
    token_sets = [[orc.attended_tokens(gpu_set(res, sb, g, int(t)), int(t), op)
                   for g in range(op.h_kv)] for t in rows]
    rQ, rK, rV = orc.attention_rows_backward(to_f64(x["q"][sb, rows]), to_f64(x["k"][sb]),
                                             to_f64(x["v"][sb]), token_sets,
                                             to_f64(dO_cpu[sb, rows]), op)
    pos = {int(t): i for i, t in enumerate(rows)}
    sel = [pos[int(t)] for t in q_rows]
    err, err_abs, err_mixed, big = {}, {}, {}, {}
    got_q = gQ[q_rows].double().numpy()
    for name, got, ref in (("dQ", got_q, rQ[sel]), ("dK", gK, rK[key_idx]),
                           ("dV", gV, rV[key_idx])):
        err_abs[name] = float(np.abs(got - ref).max())
        big[name] = float(np.abs(ref).max())
        err[name] = err_abs[name] / big[name]
        row_err = np.abs(got - ref).max(axis=-1)
        err_mixed[name] = float((row_err / np.maximum(1.0, np.abs(ref).max(axis=-1))).max())
    _say("relative errors", err, "row errors / max(1, row max |ref|)", err_mixed,
         "max-abs errors", err_abs, "largest entries", big)
    for k, v in err.items():
        assert v <= 2e-2, (k, v)
    # row by row: absolute 2e-2 (the bar of O) on rows up to 1, relative above
    for k, v in err_mixed.items():
        assert v <= 2e-2, (k, "row", v)
