"""GPU parity on shapes off the workloads' own: bf16 I/O through the generic
kernels (another group size and head dimension, a block of 128 tokens), fp32
I/O at the workloads' group shape, and short query runs against a long cache
(more tokens than the decode path takes, one ragged selection tile).  The
bars are those of tests/parity.py."""
import dataclasses

import numpy as np
import pytest

import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import check_compress, check_rows, problems, run_gpu_sparse, sample_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _variant(base, **kw):
    return dataclasses.replace(CONFIGS[base], **kw)


def _full(cfg, n_kv, batch, seed):
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=seed)
    lp, op = problems(cfg, n_kv=n_kv, batch=batch)
    assert not tbs.use_dense(lp)
    res = run_gpu_sparse(lp, x["q"], x["k"], x["v"])
    check_compress(res, x["k"], op)
    return check_rows(res, x, op, 0, {b: np.arange(n_kv) for b in range(batch)})


def test_bf16_generic_group_and_head_size():
    # G = 8, d = 64, h_kv = 4: every selection and attention kernel is the
    # generic one, with bf16 loads and a single rounding of O
    cfg = _variant("prefill32k", name="g8d64", h_q=32, h_kv=4, d=64, k=8, n_needles=8)
    _say("case: bf16 G=8 d=64 h_kv=4")
    _say(_full(cfg, 1500, 2, seed=301))


def test_bf16_block_of_128_tokens():
    # B = 128: 8 kernels start in a block and 9 intersect it (l = 9, s = 8)
    cfg = _variant("prefill32k", name="b128", B=128, l=9, s=8, k=6, n_needles=6)
    _say("case: bf16 B=128")
    _say(_full(cfg, 2000, 1, seed=302))


def test_fp32_at_the_workload_group_shape():
    cfg = _variant("prefill32k", name="f32g16", io="f32", k=8, n_needles=8)
    _say("case: fp32 G=16 d=128")
    _say(_full(cfg, 900, 1, seed=303))


@pytest.mark.parametrize("n_q", [5, 17])
def test_bf16_short_query_run_on_a_long_cache(n_q):
    # n_q > 4 takes the prefill kernels; the selection tile of 16 tokens is ragged
    cfg = CONFIGS["prefill32k"]
    n_kv, batch = 9000, 2
    _say(f"case: bf16 {n_q} queries on {n_kv} keys")
    x = make_inputs(cfg, n_kv=n_kv, batch=batch, seed=310 + n_q)
    xq = dict(x)
    xq["q"] = x["q"][:, n_kv - n_q:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=batch, n_q=n_q, q_pos0=n_kv - n_q)
    res = run_gpu_sparse(lp, xq["q"], x["k"], x["v"])
    _say(check_rows(res, xq, op, n_kv - n_q, {b: np.arange(n_q) for b in range(batch)}))


def test_bf16_long_prefill_chunk_sampled():
    # 6000 queries from position 3000 of 9000 keys: many selection tiles, a
    # ragged last tile, rows sampled including both ends
    cfg = CONFIGS["prefill32k"]
    n_kv, q0 = 9000, 3000
    _say("case: bf16 prefill chunk", q0, n_kv)
    x = make_inputs(cfg, n_kv=n_kv, batch=1, seed=320)
    xq = dict(x)
    xq["q"] = x["q"][:, q0:].contiguous()
    lp, op = problems(cfg, n_kv=n_kv, batch=1, n_q=n_kv - q0, q_pos0=q0)
    res = run_gpu_sparse(lp, xq["q"], x["k"], x["v"])
    rows = sample_rows(n_kv - q0, 300, np.random.default_rng(5), must=(0, 15, 16, 5999))
    _say(check_rows(res, xq, op, q0, {0: rows}))
