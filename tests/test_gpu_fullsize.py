"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (same calls, same shapes), on outputs the oracle computes one by one:
K^C1 everywhere (bit-exact), and the selection, S^cmp, O and LSE of sampled
query rows that include the edge rows (first tokens, block boundaries, the
last token)."""
import numpy as np
import pytest
import torch

import oracle as orc
import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import check_compress, check_rows, problems, run_gpu_dense, run_gpu_sparse, sample_rows

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
    tbs.compress_k(lp, K, Kc1, c1_begin=n_prev, c1_end=n_now)
    S = tbs.block_scores(lp, Q, Kc1)
    idx, n_sel = tbs.topk_select(lp, S)
    O, lse = tbs.sparse_attn(lp, Q, K, V, idx, n_sel)
    torch.cuda.synchronize()
    res = dict(Kc1=Kc1.cpu(), S_cmp=S.cpu(), idx=idx.cpu(), n_sel=n_sel.cpu(), O=O.cpu(),
               lse=lse.cpu())
    del Q, K, V
    Kc1_ref = check_compress(res, x["k"], op)
    rep = check_rows(res, x, op, cfg.n_kv - 1, {b: np.array([0]) for b in range(cfg.batch)},
                     Kc1_ref=Kc1_ref)
    # the planted needles are close to the query direction: most are selected
    picked = sum(len(set(res["idx"][b, g, 0, :int(res["n_sel"][b, g, 0])].tolist())
                     & set(x["needles"][b].tolist()))
                 for b in range(cfg.batch) for g in range(cfg.h_kv))
    _say(rep, "needles selected:", picked, "of", cfg.batch * cfg.h_kv * x["needles"].shape[1])


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
