"""The Python binding refuses buffers the kernels cannot use -- host tensors,
wrong dtypes, strided views, short buffers -- before anything is enqueued,
and its buffer extents follow the library's own size helpers (CPU only)."""
import pytest
import torch

import trainable_block_sparse_amd as tbs


def _prob(**kw):
    base = dict(batch=2, n_q=300, n_kv=300, h_kv=2, G=16, d=128, k=16)
    base.update(kw)
    return tbs.Problem(**base)


@pytest.mark.parametrize("kw", [dict(), dict(n_kv=31, n_q=31), dict(n_kv=32, n_q=1, q_pos0=31),
                                dict(n_kv=131072, n_q=1, q_pos0=131071, batch=16),
                                dict(n_kv=4096, n_q=4096, k=64, B=64),
                                dict(dtype="f32", G=4, d=64, n_kv=2048, n_q=2048, k=4),
                                dict(n_kv=1000, n_q=1000, kv_cap=1500, c1_cap=99, c2_cap=20)])
def test_extents_follow_the_library(kw):
    p = _prob(**kw)
    e = p._ext()
    assert e.n_c1 == tbs.n_kernels(p)
    assert e.n_blk == tbs.n_blocks(p)
    assert e.budget == tbs.budget(p)
    n_c2 = tbs.n_coarse_kernels(p)
    assert e.n_c2 == n_c2
    assert e.kc2 == p.batch * p.h_kv * (p.c2_cap or n_c2) * p.d
    assert e.kc1 == p.batch * p.h_kv * (p.c1_cap or e.n_c1) * p.d
    assert e.kv == p.batch * (p.kv_cap or p.n_kv) * p.h_kv * p.d
    assert e.q == p.batch * p.n_q * p.h_q * p.d
    assert e.io == (torch.bfloat16 if p.dtype == "bf16" else torch.float32)


def test_arg_checks_in_order():
    good = torch.zeros(64, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="torch.Tensor"):
        tbs._arg([0] * 64, "Q", torch.bfloat16, 64)
    with pytest.raises(TypeError, match="float32"):
        tbs._arg(good, "S_cmp", torch.float32, 64)
    with pytest.raises(ValueError, match="contiguous"):
        tbs._arg(torch.zeros(8, 16, dtype=torch.bfloat16).t(), "K", torch.bfloat16, 64)
    with pytest.raises(ValueError, match="needs 65"):
        tbs._arg(good, "K", torch.bfloat16, 65)
    with pytest.raises(ValueError, match="GPU tensor"):
        tbs._arg(good, "K", torch.bfloat16, 64)
    with pytest.raises(ValueError, match="required"):
        tbs._arg(None, "K", torch.bfloat16, 64)
    assert tbs._arg(None, "lse", torch.float32, 64, optional=True) is None
    with pytest.raises(ValueError, match="GPU tensor"):
        tbs._ws(torch.zeros(16, dtype=torch.uint8))


def test_wrappers_refuse_host_tensors_before_any_launch():
    p = _prob()
    e = p._ext()
    Q = torch.zeros(e.q, dtype=torch.bfloat16).view(p.batch, p.n_q, p.h_q, p.d)
    K = torch.zeros(e.kv, dtype=torch.bfloat16).view(p.batch, p.n_kv, p.h_kv, p.d)
    idx = torch.zeros(e.rows * e.budget, dtype=torch.int32)
    n_sel = torch.zeros(e.rows, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        tbs.compress_k(p, K)
    with pytest.raises(ValueError, match="GPU tensor"):
        tbs.sparse_attn(p, Q, K, K, idx, n_sel)
    with pytest.raises(ValueError, match="GPU tensor"):
        tbs.dense_attn(p, Q, K, K)
    with pytest.raises(ValueError, match="GPU tensor"):
        tbs.topk_select(p, torch.zeros(e.rows * e.n_blk), idx, n_sel)


def test_paged_pool_shape_is_checked():
    p = _prob(batch=2, n_q=1, n_kv=4096, q_pos0=4095)
    e = p._ext()
    pool = torch.zeros(10, 32, p.h_kv, p.d, dtype=torch.bfloat16)     # pages of 32 rows, B = 64
    table = torch.zeros(2, 64, dtype=torch.int32)
    with pytest.raises(ValueError, match="pool"):
        tbs._cache(p, e, pool, pool, table)
    pool = torch.zeros(10, 64, p.h_kv, p.d, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="block_table"):
        tbs._cache(p, e, pool, pool, torch.zeros(1, 64, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU tensor"):
        tbs._cache(p, e, pool, pool, table)


def test_cached_struct_follows_field_changes():
    p = _prob(n_kv=4096, n_q=4096)
    assert p._c().n_kv == 4096 and p._ext().n_c1 == tbs.n_kernels(p)
    p.n_kv = p.n_q = 1000
    p.c1_cap = 77
    assert p._c().n_kv == 1000 and p._c().c1_cap == 77
    assert p._ext().n_c1 == tbs.n_kernels(p) == 61
    assert p._ext().kc1 == p.batch * p.h_kv * 77 * p.d


def test_replace_builds_a_fresh_struct():
    import dataclasses
    p = _prob(n_kv=4096, n_q=4096)
    p._c()
    r = dataclasses.replace(p, n_q=64, q_pos0=100, n_kv=164)
    assert r._c().n_q == 64 and r._c().q_pos0 == 100 and p._c().n_q == 4096
