"""Buffers with spare capacity: K/V caches of kv_cap > n_kv rows and K^C1
buffers of c1_cap > n_C1 rows whose unused rows hold NaN.  Nothing past
n_kv / n_C1 may be read into a result: every output must equal, bit for bit,
the one computed from tightly sized buffers."""
import dataclasses

import pytest
import torch

import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import problems

pytestmark = pytest.mark.gpu


def _path(lp, Q, K, V, Kc1=None):
    Kc1 = tbs.compress_k(lp, K, Kc1)
    S = tbs.block_scores(lp, Q, Kc1)
    idx, n_sel = tbs.topk_select(lp, S)
    O, lse = tbs.sparse_attn(lp, Q, K, V, idx, n_sel)
    idx2, n_sel2 = tbs.select_blocks(lp, Q, Kc1)
    torch.cuda.synchronize()
    n_c1 = tbs.n_kernels(lp)
    return dict(Kc1=Kc1[:, :, :n_c1].cpu(), idx=idx.cpu(), n_sel=n_sel.cpu(), O=O.cpu(),
                lse=lse.cpu(), idx2=idx2.cpu(), n_sel2=n_sel2.cpu())


def _padded(t, rows, dim=1):
    shape = list(t.shape)
    shape[dim] = rows
    out = torch.full(shape, float("nan"), dtype=t.dtype, device=t.device)
    out.narrow(dim, 0, t.shape[dim]).copy_(t)
    return out


@pytest.mark.parametrize("name,n_kv,batch,n_q", [("decode", 5000, 3, 1), ("prefill32k", 1500, 2, None),
                                                 ("prefill32k", 4000, 2, 3), ("tiny", 700, 1, None)])
def test_spare_capacity_is_never_read(name, n_kv, batch, n_q):
    cfg = CONFIGS[name]
    print(f"case: spare capacity {name} n_kv={n_kv} batch={batch} n_q={n_q}", flush=True)
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=500 + n_kv)
    q = x["q"] if n_q is None or x["q"].shape[1] == n_q else x["q"][:, n_kv - n_q:].contiguous()
    nq = q.shape[1]
    lp, _ = problems(cfg, n_kv=n_kv, batch=batch, n_q=nq, q_pos0=n_kv - nq)
    dev = torch.device("cuda:0")
    Q, K, V = q.to(dev), x["k"].to(dev), x["v"].to(dev)
    tight = _path(lp, Q, K, V)
    n_c1 = tbs.n_kernels(lp)
    lw = dataclasses.replace(lp, kv_cap=n_kv + 333, c1_cap=n_c1 + 17)
    Kw, Vw = _padded(K, n_kv + 333), _padded(V, n_kv + 333)
    Kc1w = torch.full((batch, lp.h_kv, n_c1 + 17, lp.d), float("nan"), dtype=K.dtype, device=dev)
    wide = _path(lw, Q, Kw, Vw, Kc1w)
    for key in tight:
        assert torch.equal(tight[key], wide[key]), key
