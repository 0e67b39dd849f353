"""Parity helpers: run the HIP path through the C ABI and compare it with the
fp64 oracle on the same seeded inputs.

Bars (written here once, used by every GPU test):
  * K^C1: bit-exact.
  * block sets: bit-exact per (token, group), except that a GPU/oracle
    difference is accepted when every block in the symmetric difference has
    an oracle S^cmp within 1e-6 (relative) of the oracle's k-th selected
    score -- the GPU's fp32 scores cannot order blocks closer than that.
    Accepted differences are counted and reported.
  * O and LSE: the oracle's attention over the GPU's accepted sets;
    max-abs 2e-2 (bf16 I/O) / 1e-4 (fp32 I/O) for O, 1e-3 / 1e-5 for LSE.
  * S^cmp (diagnostic): relative 1e-5; -inf exactly where the oracle has it.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as orc
import trainable_block_sparse_amd as tbs

TOL = {"bf16": dict(o=2e-2, lse=1e-3), "f32": dict(o=1e-4, lse=1e-5)}
EXEMPT_REL = 1e-6


def problems(cfg, n_kv=None, batch=None, n_q=None, q_pos0=None, k=None, lse_approx=False):
    """(library Problem, oracle Problem) for a config variant."""
    n_kv = cfg.n_kv if n_kv is None else n_kv
    batch = cfg.batch if batch is None else batch
    if n_q is None:
        n_q = 1 if cfg.decode else n_kv
    if q_pos0 is None:
        q_pos0 = n_kv - n_q
    k = cfg.k if k is None else k
    lp = tbs.Problem(batch=batch, n_q=n_q, n_kv=n_kv, h_kv=cfg.h_kv, G=cfg.G, d=cfg.d,
                     q_pos0=q_pos0, B=cfg.B, l_C1=cfg.l_C1, s_C1=cfg.s_C1, l=cfg.l, s=cfg.s,
                     k=k, N_init=cfg.N_init, N_local=cfg.N_local, dtype=cfg.io,
                     lse_approx=lse_approx)
    op = orc.Problem(G=cfg.G, h_kv=cfg.h_kv, d=cfg.d, B=cfg.B, l_C1=cfg.l_C1, s_C1=cfg.s_C1,
                     l=cfg.l, s=cfg.s, k=k, N_init=cfg.N_init, N_local=cfg.N_local, io=cfg.io,
                     lse_approx=lse_approx)
    return lp, op


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def run_gpu_sparse(lp, q, k, v):
    """The sparse path through the C ABI, every intermediate kept (with the
    LSE approximation, the coarse keys too)."""
    dev = torch.device("cuda:0")
    Q, K, V = q.to(dev), k.to(dev), v.to(dev)
    Kc1 = tbs.compress_k(lp, K)
    Kc2 = tbs.compress_k2(lp, K) if lp.lse_approx else None
    S = tbs.block_scores(lp, Q, Kc1, Kc2=Kc2)
    idx, n_sel = tbs.topk_select(lp, S)
    O, lse = tbs.sparse_attn(lp, Q, K, V, idx, n_sel)
    torch.cuda.synchronize()
    out = dict(Kc1=Kc1.cpu(), S_cmp=S.cpu(), idx=idx.cpu(), n_sel=n_sel.cpu(), O=O.cpu(),
               lse=lse.cpu())
    if Kc2 is not None:
        out["Kc2"] = Kc2.cpu()
    return out


def run_gpu_dense(lp, q, k, v):
    dev = torch.device("cuda:0")
    O, lse = tbs.dense_attn(lp, q.to(dev), k.to(dev), v.to(dev))
    torch.cuda.synchronize()
    return dict(O=O.cpu(), lse=lse.cpu())


def gpu_set(res, b, g, t):
    n = int(res["n_sel"][b, g, t])
    s = res["idx"][b, g, t, :n].numpy().astype(np.int64)
    pad = res["idx"][b, g, t, n:].numpy()
    assert np.all(pad == -1), "idx padding must be -1"
    assert np.all(np.diff(s) > 0), "idx must be strictly ascending"
    return s


def compare_sets(gpu, ref, S_cmp_ref, p, op):
    """Returns 'equal' or 'exempt'; raises AssertionError otherwise."""
    if np.array_equal(gpu, ref):
        return "equal"
    b_p = p // op.B
    init = set(range(min(op.N_init, b_p + 1)))
    local = set(range(max(0, b_p - op.N_local + 1), b_p + 1))
    top = [blk for blk in ref if blk not in init and blk not in local]
    assert top, f"sets differ with no top-k part: gpu={gpu} ref={ref}"
    kth = min(S_cmp_ref[blk] for blk in top)
    diff = set(gpu.tolist()) ^ set(ref.tolist())
    assert not (diff & (init | local)), f"init/local block missing: {diff}"
    for blk in diff:
        gap = abs(S_cmp_ref[blk] - kth)
        assert gap <= EXEMPT_REL * abs(kth), (
            f"p={p}: block {blk} differs (gpu={gpu.tolist()} ref={ref.tolist()}), "
            f"score {S_cmp_ref[blk]!r} vs k-th {kth!r}, rel gap {gap / abs(kth):.3e}")
    assert len(gpu) == len(ref)
    return "exempt"


def check_compress(res, k_cpu, op):
    """K^C1 (and K^C2 when the result holds it) bit-exact against the oracle;
    returns the oracle's K^C1 per sequence ({b: [h_kv, n_C1, d]})."""
    n_c1 = orc.n_kernels(k_cpu.shape[1], op.l_C1, op.s_C1)
    ref = orc.compress_k(to_f64(k_cpu), op)
    got = to_f64(res["Kc1"][:, :, :n_c1])
    np.testing.assert_array_equal(got, ref)
    if "Kc2" in res:
        n_c2 = orc.n_coarse_kernels(k_cpu.shape[1], op)
        ref2 = orc.compress_k2(to_f64(k_cpu), op)
        np.testing.assert_array_equal(to_f64(res["Kc2"][:, :, :n_c2]), ref2)
    return {b: ref[b] for b in range(ref.shape[0])}


def check_rows(res, x, op, q_pos0, rows_per_b, dense=False, check_scores=True,
               Kc1_ref=None, check_outputs=True):
    """Selection, S^cmp and (unless check_outputs is false) O and LSE for the
    listed rows of each sequence.  Returns a small report dict."""
    tol = TOL[op.io]
    n_kv = x["k"].shape[1]
    report = dict(rows=0, exempt=0, max_o=0.0, max_lse=0.0, max_scmp_rel=0.0)
    for b, rows in rows_per_b.items():
        rows = np.asarray(rows, dtype=np.int64)
        Q = to_f64(x["q"][b])
        K = to_f64(x["k"][b])
        V = to_f64(x["v"][b])
        pos = q_pos0 + rows
        if dense:
            sets = [[np.arange(p // op.B + 1) for _ in range(op.h_kv)] for p in pos]
        else:
            Kc1 = orc.compress_k(K[None], op)[0] if Kc1_ref is None else Kc1_ref[b]
            Kc2 = orc.compress_k2(K[None], op)[0] if op.lse_approx else None
            _, _, S_ref = orc.selection_scores(Q[rows], Kc1, pos, n_kv, op, Kc2=Kc2)
            sets = []
            for r, (t, p) in enumerate(zip(rows, pos)):
                row_sets = []
                b_p = int(p) // op.B
                for g in range(op.h_kv):
                    ref = orc.select_blocks(S_ref[r, g], int(p), op)
                    got = gpu_set(res, b, g, int(t))
                    if compare_sets(got, ref, S_ref[r, g], int(p), op) == "exempt":
                        report["exempt"] += 1
                    row_sets.append(got)
                    if check_scores:
                        s_gpu = res["S_cmp"][b, g, t, :b_p + 1].double().numpy()
                        s_ref = S_ref[r, g, :b_p + 1]
                        inf_ref = np.isneginf(s_ref)
                        assert np.array_equal(np.isneginf(s_gpu), inf_ref), \
                            f"-inf pattern differs at row {t} group {g}"
                        fin = ~inf_ref
                        if fin.any():
                            rel = np.abs(s_gpu[fin] - s_ref[fin]) / np.abs(s_ref[fin])
                            report["max_scmp_rel"] = max(report["max_scmp_rel"], float(rel.max()))
                sets.append(row_sets)
        report["rows"] += len(rows)
        if not check_outputs:
            continue
        token_sets = [[orc.attended_tokens(sets[r][g], int(p), op) for g in range(op.h_kv)]
                      for r, p in enumerate(pos)]
        O64, lse = orc.attention_rows(Q[rows], K, V, token_sets, op)
        O_ref = orc.round_to_io(O64, op.io)
        O_gpu = to_f64(res["O"][b, rows])
        lse_gpu = to_f64(res["lse"][b][:, rows]).T
        err_o = float(np.abs(O_gpu - O_ref).max())
        err_l = float(np.abs(lse_gpu - lse).max())
        report["max_o"] = max(report["max_o"], err_o)
        report["max_lse"] = max(report["max_lse"], err_l)
        assert err_o <= tol["o"], f"O max-abs {err_o:.3e} > {tol['o']}"
        assert err_l <= tol["lse"], f"LSE max-abs {err_l:.3e} > {tol['lse']}"
    if check_scores and not dense:
        assert report["max_scmp_rel"] <= 1e-5, report
    return report


def sample_rows(n_q, count, rng, must=()):
    """Spread-out sample of query rows, always including the listed ones."""
    base = set(int(t) for t in must if 0 <= t < n_q)
    base |= set(rng.choice(n_q, size=min(count, n_q), replace=False).tolist())
    return np.array(sorted(base), dtype=np.int64)
