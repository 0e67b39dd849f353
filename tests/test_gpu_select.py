"""infv2_select_blocks (scores + top-k in one call) against the two separate
calls, bitwise, and against the fp64 oracle on decode steps.  Decode shapes
take the fused pooling/top-k kernel; prefill shapes take the two-kernel
fallback inside the same entry point."""
import numpy as np
import pytest
import torch

import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import check_compress, check_rows, problems

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _selection_inputs(cfg, n_kv, batch, n_q, seed, k=None):
    """Keys from the config's generator; the last n_q positions query them
    (decode configs hold one query row, extra rows are seeded normals)."""
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=seed)
    q0 = n_kv - n_q
    lp, op = problems(cfg, n_kv=n_kv, batch=batch, n_q=n_q, q_pos0=q0, k=k)
    dev = torch.device("cuda:0")
    if x["q"].shape[1] == n_q:
        qh = x["q"]
    elif x["q"].shape[1] == n_kv:
        qh = x["q"][:, q0:].contiguous()
    else:
        gen = torch.Generator().manual_seed(seed)
        qh = torch.randn((batch, n_q) + tuple(x["q"].shape[2:]), generator=gen)
        qh = qh.to(x["q"].dtype)
    Q = qh.to(dev)
    K = x["k"].to(dev)
    Kc1 = tbs.compress_k(lp, K)
    return x, lp, op, Q, Kc1


def _separate(lp, Q, Kc1):
    S = tbs.block_scores(lp, Q, Kc1)
    idx, n_sel = tbs.topk_select(lp, S)
    return S, idx, n_sel


@pytest.mark.parametrize("n_kv,batch,n_q,k", [
    (131072, 2, 1, 16),     # 32 chunks of 64 blocks per row
    (131072, 1, 4, 32),     # k = 32: 32 x 32 candidate keys
    (40000, 3, 2, 16),      # ragged last chunk
    (5000, 2, 3, 16),       # fewer chunks (2) than k: several keys per list
    (600, 2, 1, 16),        # one chunk, 10 blocks: fewer candidates than k
    (100, 1, 4, 16),        # early tokens with no candidate at all
    (33, 1, 1, 16),         # one kernel
    (20, 1, 1, 16),         # no kernel yet
    (70000, 2, 1, 8),
    (70000, 1, 1, 0),       # k = 0: init and local blocks only
])
def test_fused_selection_equals_separate_calls(n_kv, batch, n_q, k):
    cfg = CONFIGS["decode"]
    _say(f"case: fused selection n_kv={n_kv} batch={batch} n_q={n_q} k={k}")
    x, lp, op, Q, Kc1 = _selection_inputs(cfg, n_kv, batch, n_q, seed=3 + n_kv + k, k=k)
    S_ref, idx_ref, n_ref = _separate(lp, Q, Kc1)
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1)
    S2 = torch.full_like(S_ref, float("nan"))
    idx2, n_sel2 = tbs.select_blocks(lp, Q, Kc1, S_cmp=S2)
    torch.cuda.synchronize()
    assert torch.equal(n_sel, n_ref)
    assert torch.equal(idx, idx_ref)
    assert torch.equal(n_sel2, n_ref) and torch.equal(idx2, idx_ref)
    b_last = (n_kv - 1) // lp.B
    assert torch.equal(torch.nan_to_num(S2[..., :b_last + 1]),
                       torch.nan_to_num(S_ref[..., :b_last + 1]))


def test_fused_selection_ties_pick_lowest_blocks():
    # Q = 0: every candidate scores the same, so the k lowest candidates win
    cfg = CONFIGS["decode"]
    n_kv, n_q = 20000, 2
    _say("case: fused selection ties", n_kv)
    x, lp, op, Q, Kc1 = _selection_inputs(cfg, n_kv, 1, n_q, seed=11)
    Q.zero_()
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1)
    _, idx_ref, n_ref = _separate(lp, Q, Kc1)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref) and torch.equal(n_sel, n_ref)
    for t in range(n_q):
        b_p = (n_kv - n_q + t) // lp.B
        want = [0] + list(range(1, 1 + lp.k)) + [b_p - 1, b_p]
        for g in range(lp.h_kv):
            n = int(n_sel[0, g, t])
            assert idx[0, g, t, :n].tolist() == want


def test_fused_selection_matches_oracle_decode():
    cfg = CONFIGS["decode"]
    n_kv, batch = 9000, 2
    _say("case: fused selection vs oracle", n_kv, batch)
    x, lp, op, Q, Kc1 = _selection_inputs(cfg, n_kv, batch, 1, seed=77)
    S = torch.full((batch, lp.h_kv, 1, tbs.n_blocks(lp)), float("nan"), device=Q.device)
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1, S_cmp=S)
    torch.cuda.synchronize()
    res = dict(Kc1=Kc1.cpu(), S_cmp=S.cpu(), idx=idx.cpu(), n_sel=n_sel.cpu())
    check_compress(res, x["k"], op)
    rep = check_rows(res, x, op, n_kv - 1, {b: np.array([0]) for b in range(batch)},
                     check_outputs=False)
    _say(rep)


@pytest.mark.parametrize("n_kv,batch,n_q,k,approx", [
    (2300, 1, 2300, 16, False),    # ragged last tile
    (3000, 2, 3000, 32, False),
    (2100, 1, 1333, 8, False),     # query offset 767, ragged
    (1500, 1, 1500, 0, False),     # init and local only
    (700, 1, 700, 16, False),      # fewer candidates than k for most rows
    (2300, 2, 2300, 16, True),     # LSE approximation (early tiles: exact kernel)
    (1800, 1, 1700, 16, True),
])
def test_prefill_streamed_topk_equals_separate_calls(n_kv, batch, n_q, k, approx):
    # the prefill selection streams the top-k through the score sweep; idx,
    # n_sel and (when asked for) S^cmp equal the two-call path bit for bit
    cfg = CONFIGS["prefill32k"]
    _say(f"case: prefill select_blocks n_kv={n_kv} batch={batch} n_q={n_q} k={k} approx={approx}")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=8 + n_kv + k)
    q0 = n_kv - n_q
    lp, _ = problems(cfg, n_kv=n_kv, batch=batch, n_q=n_q, q_pos0=q0, k=k, lse_approx=approx)
    dev = torch.device("cuda:0")
    Q = x["q"][:, q0:].contiguous().to(dev)
    K = x["k"].to(dev)
    Kc1 = tbs.compress_k(lp, K)
    Kc2 = tbs.compress_k2(lp, K) if approx else None
    S_ref = tbs.block_scores(lp, Q, Kc1, Kc2=Kc2)
    idx_ref, n_ref = tbs.topk_select(lp, S_ref)
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1, Kc2=Kc2)
    S2 = torch.full_like(S_ref, float("nan"))
    idx2, n_sel2 = tbs.select_blocks(lp, Q, Kc1, S_cmp=S2, Kc2=Kc2)
    torch.cuda.synchronize()
    assert torch.equal(n_sel, n_ref)
    assert torch.equal(idx, idx_ref)
    assert torch.equal(idx2, idx_ref) and torch.equal(n_sel2, n_ref)
    for t in (0, n_q // 2, n_q - 1):
        b_p = (q0 + t) // 64
        assert torch.equal(torch.nan_to_num(S2[:, :, t, :b_p + 1]),
                           torch.nan_to_num(S_ref[:, :, t, :b_p + 1]))


def test_prefill_streamed_topk_extreme_logits_take_exact_kernel():
    cfg = CONFIGS["prefill32k"]
    n_kv, batch = 1500, 2
    _say("case: prefill select_blocks extreme logits")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=5)
    x["q"][0, :, 5, :] *= 64
    x["k"][1, 1200:1264, 1, :] *= 64
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    dev = torch.device("cuda:0")
    Q, K = x["q"].to(dev), x["k"].to(dev)
    Kc1 = tbs.compress_k(lp, K)
    S_ref = tbs.block_scores(lp, Q, Kc1)
    idx_ref, n_ref = tbs.topk_select(lp, S_ref)
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref) and torch.equal(n_sel, n_ref)


def test_prefill_streamed_topk_all_ties():
    # Q = 0: every candidate ties; the lowest k candidates win
    cfg = CONFIGS["prefill32k"]
    n_kv = 1600
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=1)
    x["q"].zero_()
    lp, _ = problems(cfg, n_kv=n_kv, batch=1)
    dev = torch.device("cuda:0")
    Q, K = x["q"].to(dev), x["k"].to(dev)
    Kc1 = tbs.compress_k(lp, K)
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1)
    torch.cuda.synchronize()
    for t in (0, 63, 64, 500, 1200, 1599):
        b_p = t // 64
        local = set(range(max(0, b_p - 1), b_p + 1))
        cand = [c for c in range(1, b_p + 1) if c not in local]
        want = sorted({0} | local | set(cand[:16]))
        for g in range(lp.h_kv):
            n = int(n_sel[0, g, t])
            assert idx[0, g, t, :n].tolist() == want
            assert (idx[0, g, t, n:] == -1).all()


def test_fused_selection_repeated_calls_share_workspace():
    # the row counters live in the workspace and are reset by each call
    cfg = CONFIGS["decode"]
    dev = torch.device("cuda:0")
    _say("case: fused selection workspace reuse")
    ws = None
    for n_kv in (30000, 12000, 30000):
        x, lp, op, Q, Kc1 = _selection_inputs(cfg, n_kv, 2, 1, seed=n_kv)
        need = tbs.select_blocks_workspace(lp)
        if ws is None:
            ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=dev)
        assert need <= ws.numel()
        _, idx_ref, n_ref = _separate(lp, Q, Kc1)
        idx, n_sel = tbs.select_blocks(lp, Q, Kc1, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref) and torch.equal(n_sel, n_ref)


@pytest.mark.parametrize("n_kv", [262144, 300001])
def test_decode_at_and_past_the_longest_fused_selection(n_kv):
    # 262144 keys: 16383 kernels in 64 chunks of 256, the most the fused
    # decode selection takes; 300001 keys: past it, select_blocks runs the
    # scores and the general top-k kernel (4688 blocks, re-read from memory)
    cfg = CONFIGS["decode"]
    _say("case: decode selection and attention at", n_kv)
    x, lp, op, Q, Kc1 = _selection_inputs(cfg, n_kv, 2, 1, seed=90)
    S = torch.full((2, lp.h_kv, 1, tbs.n_blocks(lp)), float("nan"), device=Q.device)
    idx, n_sel = tbs.select_blocks(lp, Q, Kc1, S_cmp=S)
    K, V = x["k"].to(Q.device), x["v"].to(Q.device)
    O, lse = tbs.sparse_attn(lp, Q, K, V, idx, n_sel)
    torch.cuda.synchronize()
    res = dict(Kc1=Kc1.cpu(), S_cmp=S.cpu(), idx=idx.cpu(), n_sel=n_sel.cpu(), O=O.cpu(),
               lse=lse.cpu())
    del K, V
    check_compress(res, x["k"], op)
    _say(check_rows(res, x, op, n_kv - 1, {b: np.array([0]) for b in range(2)}))


@pytest.mark.parametrize("n_kv,batch,n_q,c1_back", [
    (5000, 3, 1, 1),        # the decode step: the newest kernel
    (4130, 2, 2, 7),        # several kernels across a 256-kernel chunk edge, two query rows
    (131072, 16, 1, 1),     # the bench's decode launch (16 x 131072)
    (999, 1, 1, 0),         # nothing to append
])
def test_select_blocks_append_equals_compress_then_select(n_kv, batch, n_q, c1_back):
    # infv2_select_blocks_append forms the appended K^C1 rows inside the
    # logits sweep: Kc1, idx and n_sel must be bitwise those of compress_k on
    # the same rows followed by select_blocks; the rows are NaN beforehand so
    # a read of the stale rows would show
    cfg = CONFIGS["decode"]
    _say(f"case: select_blocks_append n_kv={n_kv} batch={batch} n_q={n_q} rows back={c1_back}")
    x, lp, op, Q, Kc1_ref = _selection_inputs(cfg, n_kv, batch, n_q, seed=41)
    K = x["k"].to(Q.device)
    n_c1 = tbs.n_kernels(lp)
    c1_begin, c1_end = n_c1 - c1_back, n_c1
    idx_ref, ns_ref = tbs.select_blocks(lp, Q, Kc1_ref)
    Kc1 = Kc1_ref.clone()
    Kc1[:, :, c1_begin:c1_end] = float("nan")
    idx, ns = tbs.select_blocks_append(lp, Q, K, Kc1, c1_begin, c1_end)
    torch.cuda.synchronize()
    assert torch.equal(Kc1.cpu(), Kc1_ref.cpu())
    assert torch.equal(idx.cpu(), idx_ref.cpu())
    assert torch.equal(ns.cpu(), ns_ref.cpu())
    if n_kv <= 5000:
        # and the appended rows against the oracle's exact mean
        res = dict(Kc1=Kc1.cpu(), idx=idx.cpu(), n_sel=ns.cpu())
        check_compress(res, x["k"], op)


def test_select_blocks_append_refuses_other_shapes():
    cfg = CONFIGS["prefill32k"]
    lp, _ = problems(cfg, n_kv=2000, batch=1)           # a prefill shape
    dev = torch.device("cuda:0")
    e = lp._ext()
    Q = torch.zeros(e.q, dtype=torch.bfloat16, device=dev)
    K = torch.zeros(e.kv, dtype=torch.bfloat16, device=dev)
    Kc1 = torch.zeros(e.kc1, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tbs.Infv2Error, match="decode shapes"):
        tbs.select_blocks_append(lp, Q, K, Kc1, 0, 1)
    dcfg = CONFIGS["decode"]
    dp, _ = problems(dcfg, n_kv=3000, batch=1)
    n_c1 = tbs.n_kernels(dp)
    e = dp._ext()
    Q = torch.zeros(e.q, dtype=torch.bfloat16, device=dev)
    K = torch.zeros(e.kv, dtype=torch.bfloat16, device=dev)
    Kc1 = torch.zeros(e.kc1, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tbs.Infv2Error, match="c1_begin"):
        tbs.select_blocks_append(dp, Q, K, Kc1, n_c1 - 1, n_c1 + 1)


@pytest.mark.parametrize("n_kv,batch,n_q,k,c1_back", [
    (131072, 16, 1, 16, 1),  # the bench's decode step (16 x 131072)
    (131072, 1, 4, 32, 1),   # k = 32: 32 x 32 candidate keys, four query rows
    (40000, 3, 2, 16, 3),    # ragged last chunk, kernels across a chunk edge
    (5000, 2, 3, 16, 1),     # fewer chunks than k: several keys per list
    (600, 2, 1, 16, 1),      # one chunk, 10 blocks: fewer candidates than k
    (100, 1, 4, 16, 1),      # early tokens with no candidate at all
    (33, 1, 1, 16, 1),       # one kernel
    (20, 1, 1, 16, 0),       # no kernel yet, nothing to append
    (70000, 1, 1, 0, 1),     # k = 0: init and local blocks only
])
def test_decode_step_equals_append_then_attention(n_kv, batch, n_q, k, c1_back):
    # infv2_decode_step merges the candidate lists inside the attention's
    # split workgroups: Kc1, idx, n_sel, O and LSE must be bitwise those of
    # select_blocks_append followed by sparse_attn (the appended rows are NaN
    # beforehand in both); small shapes also against the oracle
    cfg = CONFIGS["decode"]
    _say(f"case: decode_step n_kv={n_kv} batch={batch} n_q={n_q} k={k} rows back={c1_back}")
    x, lp, op, Q, Kc1_ref = _selection_inputs(cfg, n_kv, batch, n_q, seed=53, k=k)
    K, V = x["k"].to(Q.device), x["v"].to(Q.device)
    n_c1 = tbs.n_kernels(lp)
    c1_begin, c1_end = max(n_c1 - c1_back, 0), n_c1
    Kc1_a = Kc1_ref.clone()
    Kc1_a[:, :, c1_begin:c1_end] = float("nan")
    idx_r, ns_r = tbs.select_blocks_append(lp, Q, K, Kc1_a, c1_begin, c1_end)
    O_r, lse_r = tbs.sparse_attn(lp, Q, K, V, idx_r, ns_r)
    Kc1_b = Kc1_ref.clone()
    Kc1_b[:, :, c1_begin:c1_end] = float("nan")
    # outputs prefilled with garbage: every element must be written
    idx = torch.full_like(idx_r, 12345)
    ns = torch.full_like(ns_r, -7)
    O = torch.full_like(O_r, float("nan"))
    lse = torch.full_like(lse_r, float("nan"))
    tbs.decode_step(lp, Q, K, V, Kc1_b, c1_begin, c1_end, idx, ns, O, lse)
    torch.cuda.synchronize()
    assert torch.equal(Kc1_b.cpu(), Kc1_a.cpu())
    assert torch.equal(idx.cpu(), idx_r.cpu())
    assert torch.equal(ns.cpu(), ns_r.cpu())
    assert torch.equal(O.cpu().view(torch.int16), O_r.cpu().view(torch.int16))
    assert torch.equal(lse.cpu().view(torch.int32), lse_r.cpu().view(torch.int32))
    if n_kv <= 5000 and k > 0:
        q0 = n_kv - n_q
        xq = dict(x, q=Q.cpu())
        res = dict(Kc1=Kc1_b.cpu(), idx=idx.cpu(), n_sel=ns.cpu(), O=O.cpu(), lse=lse.cpu())
        rep = check_rows(res, xq, op, q0, {b: np.arange(n_q) for b in range(batch)},
                         check_scores=False)
        _say(rep)


def test_decode_step_refuses_other_shapes():
    cfg = CONFIGS["prefill32k"]
    lp, _ = problems(cfg, n_kv=2000, batch=1)           # a prefill shape
    dev = torch.device("cuda:0")
    e = lp._ext()
    Q = torch.zeros(e.q, dtype=torch.bfloat16, device=dev)
    K = torch.zeros(e.kv, dtype=torch.bfloat16, device=dev)
    Kc1 = torch.zeros(e.kc1, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tbs.Infv2Error, match="decode shapes"):
        tbs.decode_step(lp, Q, K, K, Kc1, 0, 1)


@pytest.mark.parametrize("n_kv", [40000, 131072])
def test_decode_step_all_ties(n_kv):
    # Q = 0: every block scores the same, so the set is init, the lowest
    # candidate blocks and local; far more than 64 keys reach the merge's
    # bound, which takes the ranking path
    cfg = CONFIGS["decode"]
    _say(f"case: decode_step all ties n_kv={n_kv}")
    x, lp, op, Q, Kc1 = _selection_inputs(cfg, n_kv, 2, 1, seed=57)
    Q = torch.zeros_like(Q)
    K, V = x["k"].to(Q.device), x["v"].to(Q.device)
    n_c1 = tbs.n_kernels(lp)
    Kc1_a = Kc1.clone()
    idx_r, ns_r = tbs.select_blocks_append(lp, Q, K, Kc1_a, n_c1 - 1, n_c1)
    O_r, lse_r = tbs.sparse_attn(lp, Q, K, V, idx_r, ns_r)
    Kc1_b = Kc1.clone()
    idx, ns, O, lse = tbs.decode_step(lp, Q, K, V, Kc1_b, n_c1 - 1, n_c1)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), idx_r.cpu()) and torch.equal(ns.cpu(), ns_r.cpu())
    assert torch.equal(O.cpu().view(torch.int16), O_r.cpu().view(torch.int16))
    b_p = (n_kv - 1) // lp.B
    want = list(range(lp.N_init + lp.k)) + [b_p - 1, b_p]
    assert idx[0, 0, 0, :int(ns[0, 0, 0])].cpu().tolist() == want
