"""The C ABI library loads, exports every declared symbol, and its host-side
validation rejects bad arguments without touching a device (CPU only)."""
import ctypes
import os
import re

import pytest

import trainable_block_sparse_amd as tbs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "infv2.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(infv2_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tbs.LIB_PATH):
        from trainable_block_sparse_amd.build import build
        build()
    return tbs.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(tbs.EXPORTED)


def _prob(**kw):
    base = dict(batch=1, n_q=4096, n_kv=4096, h_kv=2, G=16, d=128, k=16)
    base.update(kw)
    return tbs.Problem(**base)


def _status(L, p):
    return L.infv2_check_problem(ctypes.byref(p.to_c()))


def test_derived_sizes(L):
    p = _prob(n_kv=131072, n_q=1, q_pos0=131071)
    assert tbs.n_kernels(p) == 8191
    assert tbs.n_blocks(p) == 2048
    assert tbs.budget(p) == 19
    assert tbs.n_kernels(_prob(n_kv=31, n_q=31)) == 0
    assert tbs.n_kernels(_prob(n_kv=32, n_q=32)) == 1
    assert tbs.n_coarse_kernels(_prob(n_kv=127, n_q=127)) == 0
    assert tbs.n_coarse_kernels(_prob(n_kv=128, n_q=128)) == 1
    assert tbs.n_coarse_kernels(_prob(n_kv=131072, n_q=1, q_pos0=131071)) == 2047


def test_dense_switch_rule(L):
    assert tbs.use_dense(_prob(k=64))                  # 64 blocks <= 67
    assert not tbs.use_dense(_prob(k=16))              # 64 blocks > 19
    assert tbs.use_dense(_prob(n_kv=19 * 64, n_q=19 * 64))
    assert not tbs.use_dense(_prob(n_kv=19 * 64 + 1, n_q=19 * 64 + 1))


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(n_q=4097), tbs.INFV2_E_ARG),                 # q_pos0 + n_q > n_kv
    (dict(q_pos0=-1), tbs.INFV2_E_ARG),
    (dict(l=4), tbs.INFV2_E_ARG),                      # max-pool length must be 5
    (dict(s=5), tbs.INFV2_E_ARG),
    (dict(B=60), tbs.INFV2_E_ARG),                     # B not a multiple of s_C1
    (dict(N_local=0), tbs.INFV2_E_ARG),
    (dict(scale=-1.0), tbs.INFV2_E_ARG),
    (dict(kv_cap=100), tbs.INFV2_E_ARG),
    (dict(lse_approx=True), 0),
    (dict(lse_approx=True, c2_cap=10), tbs.INFV2_E_ARG),                 # < n_C2 = 63
    (dict(l_C1=24, l=5, s=4), tbs.INFV2_E_UNSUPPORTED),  # not a power of two
    (dict(d=260), tbs.INFV2_E_UNSUPPORTED),
    (dict(dtype="f32", G=4, d=64), 0),
    (dict(dtype="f32", G=4, d=64, n_kv=131072, n_q=131072), tbs.INFV2_E_UNSUPPORTED),
])
def test_check_problem(L, kw, status):
    assert _status(L, _prob(**kw)) == status


def test_calls_reject_null_and_misaligned_pointers_before_any_launch(L):
    p = _prob()
    pc = ctypes.byref(p.to_c())
    assert L.infv2_compress_k(pc, None, None, 0, 1, None) == tbs.INFV2_E_ARG
    assert b"NULL" in L.infv2_last_error()
    assert L.infv2_compress_k(pc, 16, 17, 0, 1, None) == tbs.INFV2_E_ARG
    assert b"aligned" in L.infv2_last_error()
    assert L.infv2_compress_k(pc, 16, 32, 0, 10 ** 6, None) == tbs.INFV2_E_ARG
    assert L.infv2_topk_select(pc, None, 16, 16, None) == tbs.INFV2_E_ARG
    assert L.infv2_block_scores(pc, 16, 16, None, None, None, None, 0, None) == tbs.INFV2_E_ARG
    # the optional S^shared output must be aligned like every other buffer
    assert L.infv2_block_scores(pc, 16, 16, None, 16, 20, None, 0, None) == tbs.INFV2_E_ARG
    assert b"S_shared" in L.infv2_last_error()
    assert L.infv2_select_blocks(pc, 16, 16, None, None, None, 16, None, 0, None) \
        == tbs.INFV2_E_ARG
    assert L.infv2_select_blocks(pc, 16, 16, None, 17, 16, 16, None, 0, None) == tbs.INFV2_E_ARG
    assert L.infv2_compress_k2(pc, 16, None, 0, 1, None) == tbs.INFV2_E_ARG
    # the LSE approximation needs the coarse keys
    pa = _prob(lse_approx=True)
    pac = ctypes.byref(pa.to_c())
    assert L.infv2_block_scores(pac, 16, 16, None, 16, None, None, 0, None) == tbs.INFV2_E_ARG
    assert b"Kc2" in L.infv2_last_error()
    assert L.infv2_compress_k2(pac, 16, 32, 0, tbs.n_coarse_kernels(pa) + 1, None) \
        == tbs.INFV2_E_ARG
    assert L.infv2_sparse_attn(pc, 16, 16, 16, 16, 16, None, None, None, 0, None) == tbs.INFV2_E_ARG
    assert L.infv2_dense_attn(pc, 16, 16, 16, 16, None, None, 0, None) == tbs.INFV2_E_ARG
    assert L.infv2_check_problem(None) == tbs.INFV2_E_ARG


def test_workspace_sizes_and_errors(L):
    dec = _prob(batch=16, n_q=1, q_pos0=131071, n_kv=131072)
    pc = ctypes.byref(dec.to_c())
    need = L.infv2_block_scores_workspace(pc)
    assert need >= 16 * 2 * 16 * 8191 * 4
    assert L.infv2_block_scores(pc, 16, 16, None, 16, None, 16, need - 1, None) \
        == tbs.INFV2_E_WORKSPACE
    need_a = L.infv2_sparse_attn_workspace(pc)
    assert need_a >= 16 * 2 * 19 * 16 * 128 * 4
    assert L.infv2_sparse_attn(pc, 16, 16, 16, 16, 16, 16, None, 16, 0, None) \
        == tbs.INFV2_E_WORKSPACE
    # fused selection: the scores' workspace, then 16 candidate keys per
    # chunk of 64 blocks and row
    need_s = L.infv2_select_blocks_workspace(pc, 0)
    assert need_s == L.infv2_select_blocks_workspace(pc, 1)
    assert need_s >= need + 16 * 2 * 32 * 16 * 8
    assert L.infv2_select_blocks(pc, 16, 16, None, None, 16, 16, 16, need_s - 1, None) \
        == tbs.INFV2_E_WORKSPACE
    # the approximation's split path keeps only the coarse partials: 8 chunks
    # of 256 coarse kernels x 16 heads x (max, sum) per row
    dec_a = _prob(batch=16, n_q=1, q_pos0=131071, n_kv=131072, lse_approx=True)
    assert tbs.n_coarse_kernels(dec_a) == 2047
    assert L.infv2_block_scores_workspace(ctypes.byref(dec_a.to_c())) == 16 * 2 * 8 * 16 * 8
    pre = _prob(n_q=32768, n_kv=32768)
    assert L.infv2_block_scores_workspace(ctypes.byref(pre.to_c())) == 0
    # prefill selection streams the top-k: one mark per 16-token tile
    assert L.infv2_select_blocks_workspace(ctypes.byref(pre.to_c()), 0) == 2 * 2048 * 4
    assert L.infv2_select_blocks_workspace(ctypes.byref(pre.to_c()), 1) == 2 * 2048 * 4
    # shapes without a fused path keep S^cmp in the workspace
    pre64 = _prob(n_q=32768, n_kv=32768, k=64)
    assert L.infv2_select_blocks_workspace(ctypes.byref(pre64.to_c()), 1) == 0
    assert L.infv2_select_blocks_workspace(ctypes.byref(pre64.to_c()), 0) == 2 * 32768 * 512 * 4
    # packed K and V: 2 tensors x h_kv x (blocks x B) keys x d x 2 bytes
    assert L.infv2_dense_attn_workspace(ctypes.byref(pre.to_c())) == 2 * 2 * 32768 * 128 * 2
    for s in (0, -1, -2, -3, -4, 7):
        assert L.infv2_status_string(s)


def test_varlen_calls_validate_before_any_launch(L):
    dec = _prob(batch=4, n_q=1, q_pos0=0, n_kv=131072)
    pc = ctypes.byref(dec.to_c())
    # workspaces: the fused decode selection's and the split attention's
    assert L.infv2_select_blocks_varlen_workspace(pc) == L.infv2_select_blocks_workspace(pc, 0)
    assert L.infv2_sparse_attn_varlen_workspace(pc) == L.infv2_sparse_attn_workspace(pc)
    ws = L.infv2_select_blocks_varlen_workspace(pc)
    # seq_lens is required
    assert L.infv2_select_blocks_varlen(pc, 16, 16, None, None, 16, 16, 16, ws, None) \
        == tbs.INFV2_E_ARG
    assert b"seq_lens" in L.infv2_last_error()
    assert L.infv2_select_blocks_varlen(pc, 16, 16, None, 16, 16, 16, 16, ws - 1, None) \
        == tbs.INFV2_E_WORKSPACE
    # a page table must cover ceil(n_kv / B) = 2048 blocks
    assert L.infv2_sparse_attn_varlen(pc, 16, 16, 16, 16, 2047, 10, 16, 16, 16, 16, None, 16,
                                      1 << 30, None) == tbs.INFV2_E_ARG
    assert b"max_blocks" in L.infv2_last_error()
    assert L.infv2_compress_k_varlen(pc, 16, 16, 2048, 0, 16, 16, 0, 1, None) == tbs.INFV2_E_ARG
    assert L.infv2_compress_k_varlen(pc, 16, None, 0, 0, 16, 16, 2, 1, None) == tbs.INFV2_E_ARG
    # prefill shapes and other dtypes have no varlen kernels
    pre = ctypes.byref(_prob(n_q=4096, n_kv=4096).to_c())
    assert L.infv2_select_blocks_varlen(pre, 16, 16, None, 16, 16, 16, 16, 1 << 30, None) \
        == tbs.INFV2_E_UNSUPPORTED
    f32 = ctypes.byref(_prob(dtype="f32", G=4, d=64, n_q=1, n_kv=4096).to_c())
    assert L.infv2_sparse_attn_varlen(f32, 16, 16, 16, None, 0, 0, 16, 16, 16, 16, None, 16,
                                      1 << 30, None) == tbs.INFV2_E_UNSUPPORTED


def test_batches_beyond_one_launch_are_refused(L):
    # the batch (times up to 4 query tokens) rides in a grid dimension of at
    # most 65535 workgroups
    assert _status(L, _prob(batch=16383, n_q=4, n_kv=4096, q_pos0=4092)) == tbs.INFV2_OK
    assert _status(L, _prob(batch=16384, n_q=4, n_kv=4096, q_pos0=4092)) \
        == tbs.INFV2_E_UNSUPPORTED
    assert b"65535" in L.infv2_last_error()
    assert _status(L, _prob(batch=65535, n_q=1, n_kv=4096, q_pos0=4095)) == tbs.INFV2_OK
    assert _status(L, _prob(batch=65536, n_q=1, n_kv=4096, q_pos0=4095)) \
        == tbs.INFV2_E_UNSUPPORTED
    assert _status(L, _prob(batch=65536, n_q=1, n_kv=4096, q_pos0=4095, dtype="f32", G=4,
                            d=64)) == tbs.INFV2_E_UNSUPPORTED


def test_error_messages_are_per_thread(L):
    # each thread sees the message of its own last failing call, while the
    # other threads fail in other ways at the same time
    import threading
    barrier = threading.Barrier(4)
    out = {}

    def worker(i):
        p = ctypes.byref(_prob(n_kv=4096 + 64 * i, n_q=4096 + 64 * i).to_c())
        barrier.wait()
        for _ in range(200):
            if i % 2:
                st = L.infv2_compress_k(p, None, 16, 0, 1, None)      # NULL K
                want = b"NULL"
            else:
                st = L.infv2_compress_k(p, 16, 17, 0, 1, None)        # misaligned Kc1
                want = b"aligned"
            msg = L.infv2_last_error()
            if st != tbs.INFV2_E_ARG or want not in msg:
                out[i] = (st, msg)
                return
        out[i] = "ok"

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert out == {i: "ok" for i in range(4)}, out


def test_noalloc_refuses_problems_past_its_scratch(L):
    # the size check comes before any device call: a problem whose workspace
    # exceeds the static scratch is refused, with the sizes in the message
    p = _prob(n_kv=131072, n_q=131072)
    assert tbs.sparse_attn_workspace(p) > tbs.NOALLOC_SCRATCH_BYTES
    one = ctypes.c_void_p(256)
    st = L.infv2_sparse_attn_noalloc(ctypes.byref(p.to_c()), one, one, one, one, one, one, None,
                                     None)
    assert st == tbs.INFV2_E_WORKSPACE
    assert "static scratch" in L.infv2_last_error().decode()
    st = L.infv2_sparse_attn_noalloc(ctypes.byref(p.to_c()), None, one, one, one, one, one, None,
                                     None)
    assert st == tbs.INFV2_E_ARG


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define INFV2_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m, "INFV2_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == tbs.NOALLOC_SCRATCH_BYTES


def test_backward_refuses_grids_past_65535_before_any_launch(L):
    # the fast backward's dK/dV grid takes the key blocks in y and batch x
    # h_kv in z: larger problems are refused up front, nothing enqueued
    one = ctypes.c_void_p(256)
    p = _prob(n_kv=65536 * 64 + 64, n_q=1, q_pos0=65536 * 64 + 63)      # 65537 blocks
    st = L.infv2_sparse_attn_bwd(ctypes.byref(p.to_c()), one, one, one, one, one, one, one,
                                 one, one, one, one, one, ctypes.c_size_t(1 << 62), None)
    assert st == tbs.INFV2_E_UNSUPPORTED
    assert "65535" in L.infv2_last_error().decode()
    p = _prob(batch=40000, h_kv=2, n_kv=256, n_q=256)                    # batch x h_kv = 80000
    st = L.infv2_dense_attn_bwd(ctypes.byref(p.to_c()), one, one, one, one, one, one, one,
                                one, one, one, ctypes.c_size_t(1 << 62), None)
    assert st == tbs.INFV2_E_UNSUPPORTED


def test_select_blocks_append_validates_before_any_launch(L):
    # shape, range, pointer and workspace errors are returned before anything
    # is enqueued (no GPU is needed to reach them)
    one = ctypes.c_void_p(256)
    big = ctypes.c_size_t(1 << 62)
    pre = _prob()                                                        # prefill shape
    st = L.infv2_select_blocks_append(ctypes.byref(pre.to_c()), one, one, one, 0, 1, one, one,
                                      one, big, None)
    assert st == tbs.INFV2_E_UNSUPPORTED
    assert "decode shapes" in L.infv2_last_error().decode()
    dec = _prob(n_kv=131072, n_q=1, q_pos0=131071)
    dc = ctypes.byref(dec.to_c())
    n_c1 = tbs.n_kernels(dec)
    assert L.infv2_select_blocks_append(dc, one, one, one, n_c1, n_c1 + 1, one, one, one, big,
                                        None) == tbs.INFV2_E_ARG
    assert "c1_begin" in L.infv2_last_error().decode()
    assert L.infv2_select_blocks_append(dc, one, one, one, 5, 4, one, one, one, big,
                                        None) == tbs.INFV2_E_ARG
    assert L.infv2_select_blocks_append(dc, one, None, one, n_c1 - 1, n_c1, one, one, one, big,
                                        None) == tbs.INFV2_E_ARG
    assert L.infv2_select_blocks_append(dc, one, one, one, n_c1 - 1, n_c1, one, one, one,
                                        ctypes.c_size_t(16), None) == tbs.INFV2_E_WORKSPACE
    approx = _prob(n_kv=131072, n_q=1, q_pos0=131071, lse_approx=True)
    assert L.infv2_select_blocks_append(ctypes.byref(approx.to_c()), one, one, one, 0, 1, one,
                                        one, one, big, None) == tbs.INFV2_E_UNSUPPORTED
