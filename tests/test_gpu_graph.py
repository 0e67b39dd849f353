"""A decode step captured in a HIP graph and replayed several times, with
eager work and synchronisations in between, gives the eager result bit for
bit on every replay (the library issues no memset and allocates nothing)."""
import numpy as np
import pytest
import torch

import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import check_rows, problems

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replay_matches_eager():
    cfg = CONFIGS["decode"]
    n_kv, batch = 5000, 4
    print("case: decode graph replay", n_kv, batch, flush=True)
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=77)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    n_c1, n_blk, bud = tbs.n_kernels(lp), tbs.n_blocks(lp), tbs.budget(lp)
    Kc1 = tbs.compress_k(lp, K)
    S = torch.empty((batch, lp.h_kv, 1, n_blk), dtype=torch.float32, device=dev)
    idx = torch.empty((batch, lp.h_kv, 1, bud), dtype=torch.int32, device=dev)
    nsel = torch.empty((batch, lp.h_kv, 1), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((batch, lp.h_q, 1), dtype=torch.float32, device=dev)
    ws_s = torch.empty(tbs.block_scores_workspace(lp), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(tbs.sparse_attn_workspace(lp), dtype=torch.uint8, device=dev)

    def step():
        tbs.compress_k(lp, K, Kc1, c1_begin=n_c1 - 1, c1_end=n_c1)
        tbs.block_scores(lp, Q, Kc1, S, ws_s)
        tbs.topk_select(lp, S, idx, nsel)
        tbs.sparse_attn(lp, Q, K, V, idx, nsel, O, lse, ws_a)

    step()
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in dict(idx=idx, nsel=nsel, O=O, lse=lse).items()}
    res = dict(Kc1=Kc1.cpu(), S_cmp=S.cpu(), idx=idx.cpu(), n_sel=nsel.cpu(), O=O.cpu(),
               lse=lse.cpu())
    check_rows(res, x, op, n_kv - 1, {b: np.array([0]) for b in range(batch)})

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (O, lse, idx, nsel):
            t.zero_()                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, t in dict(idx=idx, nsel=nsel, O=O, lse=lse).items():
            assert torch.equal(t, ref[k]), f"replay {rep}: {k} differs"


def test_fused_selection_graph_replay_matches_eager():
    # the fused selection's row counters are reset by a kernel of the same
    # call, so replays need no memset between them
    cfg = CONFIGS["decode"]
    n_kv, batch = 20000, 3
    print("case: fused selection graph replay", n_kv, batch, flush=True)
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=78)
    lp, _ = problems(cfg, n_kv=n_kv, batch=batch)
    dev = torch.device("cuda:0")
    Q, K = x["q"].to(dev), x["k"].to(dev)
    Kc1 = tbs.compress_k(lp, K)
    bud = tbs.budget(lp)
    idx = torch.empty((batch, lp.h_kv, 1, bud), dtype=torch.int32, device=dev)
    nsel = torch.empty((batch, lp.h_kv, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(tbs.select_blocks_workspace(lp), dtype=torch.uint8, device=dev)
    S = tbs.block_scores(lp, Q, Kc1)
    idx_ref, nsel_ref = tbs.topk_select(lp, S)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tbs.select_blocks(lp, Q, Kc1, None, idx, nsel, ws)
    for rep in range(4):
        idx.zero_()
        nsel.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref), f"replay {rep}: idx differs"
        assert torch.equal(nsel, nsel_ref), f"replay {rep}: n_sel differs"


def test_varlen_paged_decode_step_graph_replay_matches_eager():
    # the serving step the bench times: append, varlen selection, paged
    # attention; the lengths change between replays through the device array
    from synth import paged_cache
    cfg = CONFIGS["decode"]
    lens = np.array([1, 700, 3001, 5000], np.int32)
    b, n_max = len(lens), int(lens.max())
    print("case: varlen paged decode graph replay", lens.tolist(), flush=True)
    x = make_inputs(cfg, n_kv=n_max, batch=b, seed=79)
    lp, _ = problems(cfg, n_kv=n_max, batch=b, q_pos0=0)
    dev = torch.device("cuda:0")
    kp, vp, table = paged_cache(x["k"], x["v"], lens, cfg.B, 80)
    Q, K, V, table = x["q"].to(dev), kp.to(dev), vp.to(dev), table.to(dev)
    seq = torch.tensor(lens, device=dev)
    Kc1 = torch.zeros((b, lp.h_kv, tbs.n_kernels(lp), lp.d), dtype=torch.bfloat16, device=dev)
    tbs.compress_k_varlen(lp, K, seq - 1, Kc1, block_table=table)
    idx = torch.empty((b, lp.h_kv, 1, tbs.budget(lp)), dtype=torch.int32, device=dev)
    nsel = torch.empty((b, lp.h_kv, 1), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((b, lp.h_q, 1), dtype=torch.float32, device=dev)
    ws_s = torch.empty(tbs.select_blocks_varlen_workspace(lp), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(tbs.sparse_attn_varlen_workspace(lp), dtype=torch.uint8, device=dev)

    def step():
        tbs.compress_k_varlen(lp, K, seq, Kc1, block_table=table, last_n=1)
        tbs.select_blocks_varlen(lp, Q, Kc1, seq, idx, nsel, ws_s)
        tbs.sparse_attn_varlen(lp, Q, K, V, seq, idx, nsel, block_table=table, O=O, lse=lse,
                               ws=ws_a)

    def eager_for(lengths):
        seq.copy_(torch.tensor(lengths, device=dev))
        step()
        torch.cuda.synchronize()
        return {k: t.clone() for k, t in dict(idx=idx, nsel=nsel, O=O, lse=lse, Kc1=Kc1).items()}

    other = np.minimum(lens + 16, n_max).astype(np.int32)
    ref_a, ref_b = eager_for(lens), eager_for(other)
    seq.copy_(torch.tensor(lens, device=dev))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        lengths, ref = (lens, ref_a) if rep % 2 == 0 else (other, ref_b)
        for t in (O, lse, idx, nsel):
            t.zero_()                     # eager work between replays
        seq.copy_(torch.tensor(lengths, device=dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("idx", "nsel", "O", "lse"):
            assert torch.equal(dict(idx=idx, nsel=nsel, O=O, lse=lse)[k], ref[k]), \
                f"replay {rep}: {k} differs"


def test_two_call_decode_step_graph_replay_matches_eager():
    # the bench's decode step (the append inside the selection, then the
    # attention) captured once; the appended K^C1 row is cleared to NaN
    # between replays so that every replay must form it again
    cfg = CONFIGS["decode"]
    n_kv, batch = 9000, 3
    print("case: two-call decode graph replay", n_kv, batch, flush=True)
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=79)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    n_c1, bud = tbs.n_kernels(lp), tbs.budget(lp)
    Kc1 = tbs.compress_k(lp, K)
    Kc1_ref = Kc1.clone()
    idx = torch.empty((batch, lp.h_kv, 1, bud), dtype=torch.int32, device=dev)
    nsel = torch.empty((batch, lp.h_kv, 1), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((batch, lp.h_q, 1), dtype=torch.float32, device=dev)
    ws_s = torch.empty(max(tbs.select_blocks_workspace(lp), 16), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(tbs.sparse_attn_workspace(lp), 16), dtype=torch.uint8, device=dev)

    def step():
        tbs.select_blocks_append(lp, Q, K, Kc1, n_c1 - 1, n_c1, idx, nsel, ws_s)
        tbs.sparse_attn(lp, Q, K, V, idx, nsel, O, lse, ws_a)

    Kc1[:, :, n_c1 - 1] = float("nan")
    step()
    torch.cuda.synchronize()
    assert torch.equal(Kc1, Kc1_ref)
    ref = {k: t.clone() for k, t in dict(idx=idx, nsel=nsel, O=O, lse=lse).items()}
    res = dict(Kc1=Kc1.cpu(), idx=idx.cpu(), n_sel=nsel.cpu(), O=O.cpu(), lse=lse.cpu())
    check_rows(res, x, op, n_kv - 1, {b: np.array([0]) for b in range(batch)},
               check_scores=False)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (O, lse, idx, nsel):
            t.zero_()                     # eager work between replays
        Kc1[:, :, n_c1 - 1] = float("nan")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Kc1, Kc1_ref), f"replay {rep}: Kc1 differs"
        for k, t in dict(idx=idx, nsel=nsel, O=O, lse=lse).items():
            assert torch.equal(t, ref[k]), f"replay {rep}: {k} differs"


def test_one_call_decode_step_graph_replay_matches_eager():
    # infv2_decode_step captured once and replayed: the appended K^C1 row is
    # cleared to NaN and the outputs zeroed between replays, so every replay
    # must form the row, merge the lists and attend again
    cfg = CONFIGS["decode"]
    n_kv, batch = 9000, 3
    print("case: one-call decode graph replay", n_kv, batch, flush=True)
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=83)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    n_c1, bud = tbs.n_kernels(lp), tbs.budget(lp)
    Kc1 = tbs.compress_k(lp, K)
    Kc1_ref = Kc1.clone()
    idx = torch.empty((batch, lp.h_kv, 1, bud), dtype=torch.int32, device=dev)
    nsel = torch.empty((batch, lp.h_kv, 1), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((batch, lp.h_q, 1), dtype=torch.float32, device=dev)
    ws = torch.empty(tbs.decode_step_workspace(lp), dtype=torch.uint8, device=dev)

    def step():
        tbs.decode_step(lp, Q, K, V, Kc1, n_c1 - 1, n_c1, idx, nsel, O, lse, ws)

    Kc1[:, :, n_c1 - 1] = float("nan")
    step()
    torch.cuda.synchronize()
    assert torch.equal(Kc1, Kc1_ref)
    ref = {k: t.clone() for k, t in dict(idx=idx, nsel=nsel, O=O, lse=lse).items()}
    res = dict(Kc1=Kc1.cpu(), idx=idx.cpu(), n_sel=nsel.cpu(), O=O.cpu(), lse=lse.cpu())
    check_rows(res, x, op, n_kv - 1, {b: np.array([0]) for b in range(batch)},
               check_scores=False)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (O, lse, idx, nsel):
            t.zero_()                     # eager work between replays
        Kc1[:, :, n_c1 - 1] = float("nan")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Kc1, Kc1_ref), f"replay {rep}: Kc1 differs"
        for k, t in dict(idx=idx, nsel=nsel, O=O, lse=lse).items():
            assert torch.equal(t, ref[k]), f"replay {rep}: {k} differs"
