"""Block-sparse attention on hand-made block lists: every length from one
entry (the token's own block alone) to the budget, mixed across the tokens a
wave takes in turn, so that the attention kernels' entry sequences start,
change token and end at every parity -- the two-token kernel (lists of at
most 64 entries), the one-token kernel (longer lists) and the key-range
kernel (from 1024 blocks on) -- against the oracle's attention over the same
sets.  The lists obey the sparse_attn contract: ascending, distinct, causal,
the last entry the token's own block."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as orc
import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import TOL, problems, sample_rows, to_f64

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _hand_lists(batch, h_kv, n_q, q_pos0, B, budget, rng):
    """(idx [batch][h_kv][n_q][budget] padded -1, n_sel): row r's length
    cycles through 1, the cap, 2 and a random length (cap = min(budget,
    b_p + 1)), its other blocks drawn without replacement below b_p."""
    idx = np.full((batch, h_kv, n_q, budget), -1, np.int32)
    n_sel = np.zeros((batch, h_kv, n_q), np.int32)
    r = 0
    for b in range(batch):
        for g in range(h_kv):
            for t in range(n_q):
                b_p = (q_pos0 + t) // B
                cap = min(budget, b_p + 1)
                mode = (r + t // 2) % 4
                L = (1, cap, min(2, cap), int(rng.integers(1, cap + 1)))[mode]
                rest = rng.choice(b_p, size=L - 1, replace=False) if L > 1 else np.zeros(0, int)
                blocks = np.sort(np.append(rest, b_p)).astype(np.int32)
                idx[b, g, t, :L] = blocks
                n_sel[b, g, t] = L
                r += 1
    return idx, n_sel


# (keys, query tokens at the end of the sequence, batch, k): the two-token
# kernel at a ragged size, the key-range kernel (1094 blocks) and the
# one-token kernel (budget 103 > 64)
CASES = [(4130, 4130, 2, 16, "two-token"), (70001, 384, 1, 16, "key-range"),
         (8192, 640, 1, 100, "one-token, long lists")]


@pytest.mark.parametrize("n_kv,n_q,batch,k,kind", CASES)
def test_sparse_attn_hand_made_lists(n_kv, n_q, batch, k, kind):
    cfg = dataclasses.replace(CONFIGS["prefill32k"], batch=batch)
    _say(f"case: hand-made lists, {kind}: n_kv={n_kv} n_q={n_q} batch={batch} k={k}")
    q_pos0 = n_kv - n_q
    lp, op = problems(cfg, n_kv=n_kv, batch=batch, n_q=n_q, q_pos0=q_pos0, k=k)
    budget = tbs.budget(lp)
    if kind == "one-token, long lists":
        assert budget > 64
    x = make_inputs(cfg, n_kv=n_kv, batch=batch)
    q = x["q"][:, q_pos0:].contiguous()
    rng = np.random.default_rng(11)
    idx_np, n_np = _hand_lists(batch, cfg.h_kv, n_q, q_pos0, cfg.B, budget, rng)
    dev = torch.device("cuda:0")
    idx = torch.from_numpy(idx_np).to(dev)
    n_sel = torch.from_numpy(n_np).to(dev)
    O, lse = tbs.sparse_attn(lp, q.to(dev), x["k"].to(dev), x["v"].to(dev), idx, n_sel)
    torch.cuda.synchronize()
    O, lse = O.cpu(), lse.cpu()
    tol = TOL[op.io]
    worst_o = worst_l = 0.0
    for b in range(batch):
        rows = sample_rows(n_q, 160, rng, must=(0, 1, 2, 3, 63, 64, n_q - 2, n_q - 1))
        Qr = to_f64(q[b, rows])
        K = to_f64(x["k"][b])
        V = to_f64(x["v"][b])
        sets = [[orc.attended_tokens(idx_np[b, g, t, :n_np[b, g, t]], q_pos0 + int(t), op)
                 for g in range(cfg.h_kv)] for t in rows]
        O64, lse_ref = orc.attention_rows(Qr, K, V, sets, op)
        err_o = float(np.abs(to_f64(O[b, rows]) - orc.round_to_io(O64, op.io)).max())
        err_l = float(np.abs(to_f64(lse[b][:, rows]).T - lse_ref).max())
        worst_o, worst_l = max(worst_o, err_o), max(worst_l, err_l)
        assert err_o <= tol["o"], f"batch {b}: O max-abs {err_o:.3e} > {tol['o']}"
        assert err_l <= tol["lse"], f"batch {b}: LSE max-abs {err_l:.3e} > {tol['lse']}"
    _say(f"max |dO| {worst_o:.3e}, max |dLSE| {worst_l:.3e}")
