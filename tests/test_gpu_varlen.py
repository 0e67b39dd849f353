"""GPU parity of the varlen / paged-cache decode calls through the C ABI.

Each sequence of a batch has its own cache length (some below one kernel,
some on block and kernel edges, ragged ones) and its K/V pages sit in a
seeded random order in a shared pool.  Checked per sequence:
  * K^C1 / K^C2 written by infv2_compress_k_varlen: bit-exact against the
    oracle (and an appended kernel equals a full rebuild);
  * idx, n_sel: bit-exact against the oracle's sets (exemption rule of
    parity.py), O and LSE against the oracle's attention over those sets
    (bars of parity.py);
  * the same rows through the ordinary one-sequence calls
    (infv2_compress_k, infv2_select_blocks, infv2_sparse_attn): idx, O and
    LSE bitwise equal -- the varlen calls run the same kernels and only move
    positions and rows.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs, paged_cache

from parity import check_rows, problems, to_f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _run(lens, n_q=1, lse_approx=False, paged=True, seed=80):
    cfg = CONFIGS["decode"]
    b, n_max = len(lens), int(max(lens))
    x = make_inputs(cfg, n_kv=n_max, batch=b, seed=seed)
    if n_q > 1:
        gen = torch.Generator().manual_seed(seed + 1)
        x["q"] = torch.randn((b, n_q, cfg.h_q, cfg.d), generator=gen).to(torch.bfloat16)
    lp, op = problems(cfg, n_kv=n_max, batch=b, n_q=n_q, q_pos0=0, lse_approx=lse_approx)
    seq = torch.tensor(np.asarray(lens, np.int32), device=DEV)
    Q = x["q"].to(DEV)
    if paged:
        kp, vp, table = paged_cache(x["k"], x["v"], lens, cfg.B, seed + 2)
        K, V, table = kp.to(DEV), vp.to(DEV), table.to(DEV)
    else:
        K, V, table = x["k"].to(DEV), x["v"].to(DEV), None
    n_c1, n_c2 = tbs.n_kernels(lp), tbs.n_coarse_kernels(lp)
    Kc1 = torch.zeros((b, cfg.h_kv, max(n_c1, 1), cfg.d), dtype=torch.bfloat16, device=DEV)
    tbs.compress_k_varlen(lp, K, seq, Kc1, block_table=table)
    Kc2 = None
    if lse_approx:
        Kc2 = torch.zeros((b, cfg.h_kv, max(n_c2, 1), cfg.d), dtype=torch.bfloat16, device=DEV)
        tbs.compress_k_varlen(lp, K, seq, Kc2, block_table=table, coarse=True)
    idx, n_sel = tbs.select_blocks_varlen(lp, Q, Kc1, seq, Kc2=Kc2)
    O, lse = tbs.sparse_attn_varlen(lp, Q, K, V, seq, idx, n_sel, block_table=table)
    torch.cuda.synchronize()
    return dict(x=x, lp=lp, op=op, Kc1=Kc1.cpu(), Kc2=None if Kc2 is None else Kc2.cpu(),
                idx=idx.cpu(), n_sel=n_sel.cpu(), O=O.cpu(), lse=lse.cpu())


def _check_against_oracle(r, lens, n_q):
    op, x = r["op"], r["x"]
    exempt = 0
    for i, L in enumerate(lens):
        L = int(L)
        k_i = x["k"][i:i + 1, :L]
        n_c1 = orc.n_kernels(L, op.l_C1, op.s_C1)
        ref = orc.compress_k(to_f64(k_i), op)[0]
        np.testing.assert_array_equal(to_f64(r["Kc1"][i, :, :n_c1]), ref)
        if r["Kc2"] is not None:
            n_c2 = orc.n_coarse_kernels(L, op)
            np.testing.assert_array_equal(to_f64(r["Kc2"][i, :, :n_c2]),
                                          orc.compress_k2(to_f64(k_i), op)[0])
        res_i = dict(idx=r["idx"][i:i + 1], n_sel=r["n_sel"][i:i + 1], O=r["O"][i:i + 1],
                     lse=r["lse"][i:i + 1])
        x_i = dict(q=x["q"][i:i + 1], k=k_i, v=x["v"][i:i + 1, :L])
        rep = check_rows(res_i, x_i, op, L - n_q, {0: np.arange(n_q)}, check_scores=False,
                         Kc1_ref={0: ref})
        exempt += rep["exempt"]
    return exempt


def _check_against_one_sequence_calls(r, lens, n_q):
    x, lp = r["x"], r["lp"]
    for i, L in enumerate(lens):
        L = int(L)
        p1 = tbs.Problem(batch=1, n_q=n_q, n_kv=L, q_pos0=L - n_q, h_kv=lp.h_kv, G=lp.G, d=lp.d,
                         k=lp.k, lse_approx=lp.lse_approx)
        Q = x["q"][i:i + 1].to(DEV)
        K = x["k"][i:i + 1, :L].contiguous().to(DEV)
        V = x["v"][i:i + 1, :L].contiguous().to(DEV)
        Kc1 = tbs.compress_k(p1, K)
        Kc2 = tbs.compress_k2(p1, K) if lp.lse_approx else None
        idx, n_sel = tbs.select_blocks(p1, Q, Kc1, Kc2=Kc2)
        O, lse = tbs.sparse_attn(p1, Q, K, V, idx, n_sel)
        torch.cuda.synchronize()
        assert torch.equal(idx.cpu()[0], r["idx"][i]), (i, L)
        assert torch.equal(n_sel.cpu()[0], r["n_sel"][i]), (i, L)
        assert torch.equal(O.cpu()[0], r["O"][i]), (i, L)
        assert torch.equal(lse.cpu()[0], r["lse"][i]), (i, L)


EDGE_LENS = [1, 31, 32, 33, 64, 127, 128, 129, 1000, 1216, 1217, 2049, 4129, 3000]


@pytest.mark.parametrize("paged", [True, False])
def test_varlen_decode_edge_lengths(paged):
    _say(f"case: varlen decode, paged={paged}, lens={EDGE_LENS}")
    r = _run(EDGE_LENS, paged=paged)
    ex = _check_against_oracle(r, EDGE_LENS, 1)
    _check_against_one_sequence_calls(r, EDGE_LENS, 1)
    _say("exempt sets:", ex)


def test_varlen_decode_lse_approx():
    lens = [1, 100, 127, 128, 191, 192, 1000, 4129]
    _say(f"case: varlen decode, LSE approximation, lens={lens}")
    r = _run(lens, lse_approx=True, seed=81)
    _check_against_oracle(r, lens, 1)
    _check_against_one_sequence_calls(r, lens, 1)


def test_varlen_two_query_tokens():
    lens = [2, 40, 65, 1300, 2085]
    _say(f"case: varlen, n_q=2, lens={lens}")
    r = _run(lens, n_q=2, seed=82)
    _check_against_oracle(r, lens, 2)
    _check_against_one_sequence_calls(r, lens, 2)


def test_compress_append_one_kernel_matches_full_build():
    # lengths that each complete a kernel at this step; Kc1 first holds the
    # kernels of length L-1, then the step appends the new one
    cfg = CONFIGS["decode"]
    lens = np.array([32, 48, 1024 + 32, 4000], np.int32)    # (L - 32) % 16 == 0
    b, n_max = len(lens), int(lens.max())
    x = make_inputs(cfg, n_kv=n_max, batch=b, seed=83)
    lp, _ = problems(cfg, n_kv=n_max, batch=b, q_pos0=0)
    kp, vp, table = paged_cache(x["k"], x["v"], lens, cfg.B, 84)
    K, table = kp.to(DEV), table.to(DEV)
    Kc1 = torch.zeros((b, cfg.h_kv, tbs.n_kernels(lp), cfg.d), dtype=torch.bfloat16, device=DEV)
    tbs.compress_k_varlen(lp, K, torch.tensor(lens - 1, device=DEV), Kc1, block_table=table)
    tbs.compress_k_varlen(lp, K, torch.tensor(lens, device=DEV), Kc1, block_table=table,
                          last_n=1)
    full = torch.zeros_like(Kc1)
    tbs.compress_k_varlen(lp, K, torch.tensor(lens, device=DEV), full, block_table=table)
    torch.cuda.synchronize()
    for i, L in enumerate(lens):
        n_c1 = (int(L) - 32) // 16 + 1
        assert torch.equal(Kc1[i, :, :n_c1].cpu(), full[i, :, :n_c1].cpu()), i


def test_out_of_range_lengths_are_clamped_not_read_past_the_buffers():
    # entries below n_q or above n_kv act as n_q / n_kv
    lens = [5, 700, 1000]
    r_ref = _run(lens, seed=85)
    cfg = CONFIGS["decode"]
    x = r_ref["x"]
    lp = r_ref["lp"]
    Q = x["q"].to(DEV)
    kp, vp, table = paged_cache(x["k"], x["v"], lens, cfg.B, 87)
    K, V, table = kp.to(DEV), vp.to(DEV), table.to(DEV)
    bad = torch.tensor([-7, 700, 10 ** 9], dtype=torch.int32, device=DEV)   # -> 1, 700, 1000
    Kc1 = torch.zeros((3, cfg.h_kv, tbs.n_kernels(lp), cfg.d), dtype=torch.bfloat16, device=DEV)
    tbs.compress_k_varlen(lp, K, bad, Kc1, block_table=table)
    idx, n_sel = tbs.select_blocks_varlen(lp, Q, Kc1, bad)
    O, lse = tbs.sparse_attn_varlen(lp, Q, K, V, bad, idx, n_sel, block_table=table)
    torch.cuda.synchronize()
    good = _run([1, 700, 1000], seed=85)
    assert torch.equal(idx.cpu(), good["idx"]) and torch.equal(O.cpu(), good["O"])
