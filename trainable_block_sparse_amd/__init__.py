"""Thin Python binding of libinfv2 (the C ABI in include/infv2.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libinfv2.so.  torch supplies device memory and the current HIP stream.  The
library must have been built (``python -m trainable_block_sparse_amd.build``);
importing a function without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import dataclasses
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# INFV2_LIB names another build of the same library (the host-ASan build of
# the CPU tests); by default the package's own libinfv2.so.
LIB_PATH = os.environ.get("INFV2_LIB") or os.path.join(_PKG, "libinfv2.so")

INFV2_OK, INFV2_E_ARG, INFV2_E_UNSUPPORTED, INFV2_E_WORKSPACE, INFV2_E_HIP = 0, -1, -2, -3, -4
INFV2_BF16, INFV2_F32 = 0, 1
EXPORTED = (
    "infv2_n_kernels", "infv2_n_coarse_kernels", "infv2_n_blocks", "infv2_budget",
    "infv2_use_dense", "infv2_check_problem", "infv2_compress_k", "infv2_compress_k2",
    "infv2_block_scores_workspace",
    "infv2_block_scores", "infv2_topk_select", "infv2_select_blocks_workspace",
    "infv2_select_blocks", "infv2_select_blocks_append", "infv2_decode_step_workspace",
    "infv2_decode_step", "infv2_sparse_attn_workspace",
    "infv2_sparse_attn", "infv2_dense_attn_workspace", "infv2_dense_attn",
    "infv2_sparse_attn_bwd_workspace", "infv2_sparse_attn_bwd",
    "infv2_dense_attn_bwd_workspace", "infv2_dense_attn_bwd",
    "infv2_compress_k_varlen", "infv2_select_blocks_varlen_workspace",
    "infv2_select_blocks_varlen", "infv2_sparse_attn_varlen_workspace",
    "infv2_sparse_attn_varlen",
    "infv2_sparse_attn_noalloc",
    "infv2_status_string", "infv2_last_error", "infv2_build_id",
)
# static scratch of infv2_sparse_attn_noalloc (INFV2_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("q_pos0", ctypes.c_int32),
        ("n_kv", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("G", ctypes.c_int32),
        ("d", ctypes.c_int32), ("B", ctypes.c_int32), ("l_C1", ctypes.c_int32),
        ("s_C1", ctypes.c_int32), ("l", ctypes.c_int32), ("s", ctypes.c_int32),
        ("k", ctypes.c_int32), ("N_init", ctypes.c_int32), ("N_local", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("kv_cap", ctypes.c_int64),
        ("c1_cap", ctypes.c_int64), ("c2_cap", ctypes.c_int64), ("lse_approx", ctypes.c_int32),
    ]


@dataclass
class Problem:
    """One attention-layer call in the pages' notation (mirrors infv2_problem)."""
    batch: int
    n_q: int
    n_kv: int
    h_kv: int
    G: int
    d: int
    q_pos0: int = 0
    B: int = 64
    l_C1: int = 32
    s_C1: int = 16
    l: int = 5
    s: int = 4
    k: int = 16
    N_init: int = 1
    N_local: int = 2
    dtype: str = "bf16"
    scale: float = 0.0
    kv_cap: int = 0
    c1_cap: int = 0
    c2_cap: int = 0
    lse_approx: bool = False

    @property
    def h_q(self) -> int:
        return self.G * self.h_kv

    def to_c(self) -> _Problem:
        return _Problem(self.batch, self.n_q, self.q_pos0, self.n_kv, self.h_kv, self.G, self.d,
                        self.B, self.l_C1, self.s_C1, self.l, self.s, self.k, self.N_init,
                        self.N_local, INFV2_BF16 if self.dtype == "bf16" else INFV2_F32,
                        self.scale, self.kv_cap, self.c1_cap, self.c2_cap, int(self.lse_approx))

    # The C struct and the buffer extents are built once and kept until a
    # field changes (the calls below take them on every launch).
    def __setattr__(self, name, value):
        object.__setattr__(self, name, value)
        self.__dict__.pop("_cached", None)

    def _c(self) -> _Problem:
        c = self.__dict__.get("_cached")
        if c is None:
            cs = self.to_c()
            c = self.__dict__["_cached"] = (cs, _Ext(self, cs))
        return c[0]

    def _ext(self) -> "_Ext":
        self._c()
        return self.__dict__["_cached"][1]


class Infv2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"infv2 status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libinfv2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run "
                               "`python -m trainable_block_sparse_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(_Problem)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "infv2_n_kernels": (i32, [P]), "infv2_n_coarse_kernels": (i32, [P]),
            "infv2_n_blocks": (i32, [P]),
            "infv2_budget": (i32, [P]), "infv2_use_dense": (ctypes.c_int, [P]),
            "infv2_check_problem": (ctypes.c_int, [P]),
            "infv2_compress_k": (ctypes.c_int, [P, vp, vp, i32, i32, vp]),
            "infv2_compress_k2": (ctypes.c_int, [P, vp, vp, i32, i32, vp]),
            "infv2_block_scores_workspace": (sz, [P]),
            "infv2_block_scores": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, sz, vp]),
            "infv2_topk_select": (ctypes.c_int, [P, vp, vp, vp, vp]),
            "infv2_select_blocks_workspace": (sz, [P, ctypes.c_int]),
            "infv2_select_blocks": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "infv2_select_blocks_append": (ctypes.c_int,
                                           [P, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]),
            "infv2_decode_step_workspace": (sz, [P]),
            "infv2_decode_step": (ctypes.c_int,
                                  [P, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "infv2_sparse_attn_workspace": (sz, [P]),
            "infv2_sparse_attn": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "infv2_sparse_attn_noalloc": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp]),
            "infv2_dense_attn_workspace": (sz, [P]),
            "infv2_dense_attn": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, sz, vp]),
            "infv2_sparse_attn_bwd_workspace": (sz, [P]),
            "infv2_sparse_attn_bwd": (ctypes.c_int, [P] + [vp] * 12 + [sz, vp]),
            "infv2_dense_attn_bwd_workspace": (sz, [P]),
            "infv2_dense_attn_bwd": (ctypes.c_int, [P] + [vp] * 10 + [sz, vp]),
            "infv2_compress_k_varlen": (ctypes.c_int, [P, vp, vp, i32, i32, vp, vp, i32, i32, vp]),
            "infv2_select_blocks_varlen_workspace": (sz, [P]),
            "infv2_select_blocks_varlen": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "infv2_sparse_attn_varlen_workspace": (sz, [P]),
            "infv2_sparse_attn_varlen": (ctypes.c_int, [P, vp, vp, vp, vp, i32, i32] + [vp] * 6
                                         + [sz, vp]),
            "infv2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "infv2_last_error": (ctypes.c_char_p, []),
            "infv2_build_id": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def build_id() -> str:
    """Source hash the loaded library was compiled from (infv2_build_id)."""
    return lib().infv2_build_id().decode()


def library_info() -> dict:
    """The loaded library's path and build id, and whether that id is the
    hash of the library sources in this tree (the library is current)."""
    from .build import source_hash
    cur = source_hash()
    bid = build_id()
    return {"path": os.path.relpath(LIB_PATH, os.path.dirname(_PKG)), "build_id": bid,
            "source_hash": cur, "built_from_these_sources": bid == cur}


def _check(status: int) -> None:
    if status != INFV2_OK:
        raise Infv2Error(status, lib().infv2_last_error().decode())


class _Ext:
    """Element counts of every buffer of one problem (the layouts of
    include/infv2.h), for the checks below."""
    __slots__ = ("io", "q", "kv", "kc1", "kc2", "n_c1", "n_c2", "n_blk", "rows", "budget",
                 "lse", "kv_rows")

    def __init__(self, prob: "Problem", c: _Problem):
        # the sizes come from the library's own helpers (one copy of the rules)
        self.io = torch.bfloat16 if prob.dtype == "bf16" else torch.float32
        L, ref = lib(), ctypes.byref(c)
        n_kv = prob.n_kv
        self.n_c1 = max(L.infv2_n_kernels(ref), 0)
        self.n_c2 = n_c2 = max(L.infv2_n_coarse_kernels(ref), 0)
        self.n_blk = max(L.infv2_n_blocks(ref), 0)
        self.budget = max(L.infv2_budget(ref), 0)
        h_q = prob.G * prob.h_kv
        self.kv_rows = prob.kv_cap or n_kv
        self.q = prob.batch * prob.n_q * h_q * prob.d
        self.kv = prob.batch * self.kv_rows * prob.h_kv * prob.d
        self.kc1 = prob.batch * prob.h_kv * (prob.c1_cap or self.n_c1) * prob.d
        self.kc2 = prob.batch * prob.h_kv * (prob.c2_cap or n_c2) * prob.d
        self.rows = prob.batch * prob.h_kv * prob.n_q
        self.lse = prob.batch * h_q * prob.n_q


def _arg(t, name: str, dtype, numel: int, optional: bool = False):
    """Device pointer of `t` once the kernels can use it: a contiguous GPU
    tensor of `dtype` that holds at least `numel` elements.  A host tensor,
    a strided view or a short buffer raises here instead of reaching a kernel."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if (not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != dtype
            or not t.is_contiguous() or t.numel() < numel):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor, not {type(t).__name__}")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype} (it is {t.dtype})")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() < numel:
            raise ValueError(f"{name} holds {t.numel()} elements; the problem needs {numel}")
        raise ValueError(f"{name} must be a GPU tensor (it is on {t.device})")
    return t.data_ptr()


def _ws(ws):
    """(pointer, size in bytes) of a workspace tensor of any dtype."""
    if ws is None:
        return None, 0
    if not isinstance(ws, torch.Tensor) or ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous GPU tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# --- derived sizes ----------------------------------------------------------

def n_kernels(prob: Problem) -> int:
    return lib().infv2_n_kernels(ctypes.byref(prob._c()))


def n_coarse_kernels(prob: Problem) -> int:
    return lib().infv2_n_coarse_kernels(ctypes.byref(prob._c()))


def n_blocks(prob: Problem) -> int:
    return lib().infv2_n_blocks(ctypes.byref(prob._c()))


def budget(prob: Problem) -> int:
    return lib().infv2_budget(ctypes.byref(prob._c()))


def use_dense(prob: Problem) -> bool:
    r = lib().infv2_use_dense(ctypes.byref(prob._c()))
    if r < 0:
        _check(lib().infv2_check_problem(ctypes.byref(prob._c())))
    return r == 1


def check_problem(prob: Problem) -> None:
    _check(lib().infv2_check_problem(ctypes.byref(prob._c())))


def _torch_dtype(prob: Problem):
    return torch.bfloat16 if prob.dtype == "bf16" else torch.float32


# --- the five calls -----------------------------------------------------------

def compress_k(prob: Problem, K: torch.Tensor, Kc1: torch.Tensor | None = None,
               c1_begin: int = 0, c1_end: int | None = None, stream=None) -> torch.Tensor:
    """K [b, kv_cap, h_kv, d] -> K^C1 [b, h_kv, c1_cap, d] (rows c1_begin..c1_end-1)."""
    e = prob._ext()
    if Kc1 is None:
        cap = prob.c1_cap or e.n_c1
        Kc1 = torch.empty((prob.batch, prob.h_kv, max(cap, 1), prob.d), dtype=K.dtype,
                          device=K.device)
    c1_end = e.n_c1 if c1_end is None else c1_end
    _check(lib().infv2_compress_k(ctypes.byref(prob._c()), _arg(K, "K", e.io, e.kv),
                                  _arg(Kc1, "Kc1", e.io, e.kc1), c1_begin, c1_end,
                                  _stream(stream)))
    return Kc1


def compress_k2(prob: Problem, K: torch.Tensor, Kc2: torch.Tensor | None = None,
                c2_begin: int = 0, c2_end: int | None = None, stream=None) -> torch.Tensor:
    """K [b, kv_cap, h_kv, d] -> K^C2 [b, h_kv, c2_cap, d] (rows c2_begin..c2_end-1),
    the coarse keys of the LSE approximation."""
    e = prob._ext()
    if Kc2 is None:
        cap = prob.c2_cap or e.n_c2
        Kc2 = torch.empty((prob.batch, prob.h_kv, max(cap, 1), prob.d), dtype=K.dtype,
                          device=K.device)
    c2_end = e.n_c2 if c2_end is None else c2_end
    _check(lib().infv2_compress_k2(ctypes.byref(prob._c()), _arg(K, "K", e.io, e.kv),
                                   _arg(Kc2, "Kc2", e.io, e.kc2), c2_begin, c2_end,
                                   _stream(stream)))
    return Kc2


def block_scores_workspace(prob: Problem) -> int:
    return lib().infv2_block_scores_workspace(ctypes.byref(prob._c()))


def block_scores(prob: Problem, Q: torch.Tensor, Kc1: torch.Tensor,
                 S_cmp: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                 stream=None, Kc2: torch.Tensor | None = None,
                 S_shared: torch.Tensor | None = None) -> torch.Tensor:
    """Q, K^C1 (and K^C2 with prob.lse_approx) -> S^cmp [b, h_kv, n_q, n_blk]
    fp32 (blocks after floor(p/B) untouched).  S_shared, when given
    ([b, h_kv, n_q, n_C1] fp32), also receives S^shared (0 where a kernel is
    not visible)."""
    if S_cmp is None:
        S_cmp = torch.full((prob.batch, prob.h_kv, prob.n_q, n_blocks(prob)), float("nan"),
                           dtype=torch.float32, device=Q.device)
    if ws is None and (need := block_scores_workspace(prob)):
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    e = prob._ext()
    ws_p, ws_n = _ws(ws)
    _check(lib().infv2_block_scores(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                    _arg(Kc1, "Kc1", e.io, e.kc1, optional=True),
                                    _arg(Kc2, "Kc2", e.io, e.kc2, optional=True),
                                    _arg(S_cmp, "S_cmp", torch.float32, e.rows * e.n_blk),
                                    _arg(S_shared, "S_shared", torch.float32, e.rows * e.n_c1,
                                         optional=True),
                                    ws_p, ws_n, _stream(stream)))
    return S_cmp


def topk_select(prob: Problem, S_cmp: torch.Tensor, idx: torch.Tensor | None = None,
                n_sel: torch.Tensor | None = None, stream=None):
    """S^cmp -> (idx [b, h_kv, n_q, budget] int32 ascending / -1, n_sel [b, h_kv, n_q])."""
    if idx is None:
        idx = torch.empty((prob.batch, prob.h_kv, prob.n_q, budget(prob)), dtype=torch.int32,
                          device=S_cmp.device)
    if n_sel is None:
        n_sel = torch.empty((prob.batch, prob.h_kv, prob.n_q), dtype=torch.int32,
                            device=S_cmp.device)
    e = prob._ext()
    _check(lib().infv2_topk_select(ctypes.byref(prob._c()),
                                   _arg(S_cmp, "S_cmp", torch.float32, e.rows * e.n_blk),
                                   _arg(idx, "idx", torch.int32, e.rows * e.budget),
                                   _arg(n_sel, "n_sel", torch.int32, e.rows), _stream(stream)))
    return idx, n_sel


def select_blocks_workspace(prob: Problem, with_scores: bool = False) -> int:
    return lib().infv2_select_blocks_workspace(ctypes.byref(prob._c()), int(bool(with_scores)))


def select_blocks(prob: Problem, Q: torch.Tensor, Kc1: torch.Tensor,
                  S_cmp: torch.Tensor | None = None, idx: torch.Tensor | None = None,
                  n_sel: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                  stream=None, Kc2: torch.Tensor | None = None):
    """Q, K^C1 (and K^C2 with prob.lse_approx) -> (idx, n_sel) as block_scores
    + topk_select; S^cmp is written only when a tensor is passed for it."""
    if idx is None:
        idx = torch.empty((prob.batch, prob.h_kv, prob.n_q, budget(prob)), dtype=torch.int32,
                          device=Q.device)
    if n_sel is None:
        n_sel = torch.empty((prob.batch, prob.h_kv, prob.n_q), dtype=torch.int32,
                            device=Q.device)
    if ws is None and (need := select_blocks_workspace(prob, S_cmp is not None)):
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    e = prob._ext()
    ws_p, ws_n = _ws(ws)
    _check(lib().infv2_select_blocks(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                     _arg(Kc1, "Kc1", e.io, e.kc1, optional=True),
                                     _arg(Kc2, "Kc2", e.io, e.kc2, optional=True),
                                     _arg(S_cmp, "S_cmp", torch.float32, e.rows * e.n_blk,
                                          optional=True),
                                     _arg(idx, "idx", torch.int32, e.rows * e.budget),
                                     _arg(n_sel, "n_sel", torch.int32, e.rows), ws_p, ws_n,
                                     _stream(stream)))
    return idx, n_sel


def select_blocks_append(prob: Problem, Q: torch.Tensor, K: torch.Tensor, Kc1: torch.Tensor,
                         c1_begin: int, c1_end: int, idx: torch.Tensor | None = None,
                         n_sel: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                         stream=None):
    """Decode: K^C1 rows c1_begin..c1_end-1 formed from K and written to Kc1
    inside the selection's score sweep, then (idx, n_sel) as select_blocks
    (bitwise compress_k(c1_begin, c1_end) followed by select_blocks)."""
    if idx is None:
        idx = torch.empty((prob.batch, prob.h_kv, prob.n_q, budget(prob)), dtype=torch.int32,
                          device=Q.device)
    if n_sel is None:
        n_sel = torch.empty((prob.batch, prob.h_kv, prob.n_q), dtype=torch.int32,
                            device=Q.device)
    if ws is None and (need := select_blocks_workspace(prob, False)):
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    e = prob._ext()
    ws_p, ws_n = _ws(ws)
    _check(lib().infv2_select_blocks_append(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                            _arg(K, "K", e.io, e.kv),
                                            _arg(Kc1, "Kc1", e.io, e.kc1), c1_begin, c1_end,
                                            _arg(idx, "idx", torch.int32, e.rows * e.budget),
                                            _arg(n_sel, "n_sel", torch.int32, e.rows), ws_p,
                                            ws_n, _stream(stream)))
    return idx, n_sel


def decode_step_workspace(prob: Problem) -> int:
    return lib().infv2_decode_step_workspace(ctypes.byref(prob._c()))


def decode_step(prob: Problem, Q, K, V, Kc1, c1_begin: int, c1_end: int, idx=None, n_sel=None,
                O=None, lse=None, ws=None, want_lse: bool = True, stream=None):
    """The decode step in one call (infv2_decode_step): K^C1 rows
    c1_begin..c1_end-1 appended, the selection, and the attention, with the
    selection's list merge inside the attention launch -> (idx, n_sel, O, lse),
    bitwise select_blocks_append followed by sparse_attn."""
    if idx is None:
        idx = torch.empty((prob.batch, prob.h_kv, prob.n_q, budget(prob)), dtype=torch.int32,
                          device=Q.device)
    if n_sel is None:
        n_sel = torch.empty((prob.batch, prob.h_kv, prob.n_q), dtype=torch.int32,
                            device=Q.device)
    if O is None:
        O = torch.empty_like(Q)
    if lse is None and want_lse:
        lse = torch.empty((prob.batch, prob.h_q, prob.n_q), dtype=torch.float32, device=Q.device)
    if ws is None:
        ws = torch.empty(max(decode_step_workspace(prob), 1), dtype=torch.uint8, device=Q.device)
    e = prob._ext()
    ws_p, ws_n = _ws(ws)
    _check(lib().infv2_decode_step(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                   _arg(K, "K", e.io, e.kv), _arg(V, "V", e.io, e.kv),
                                   _arg(Kc1, "Kc1", e.io, e.kc1), c1_begin, c1_end,
                                   _arg(idx, "idx", torch.int32, e.rows * e.budget),
                                   _arg(n_sel, "n_sel", torch.int32, e.rows),
                                   _arg(O, "O", e.io, e.q),
                                   _arg(lse, "lse", torch.float32, e.lse, optional=True),
                                   ws_p, ws_n, _stream(stream)))
    return idx, n_sel, O, lse


def sparse_attn_workspace(prob: Problem) -> int:
    return lib().infv2_sparse_attn_workspace(ctypes.byref(prob._c()))


def sparse_attn(prob: Problem, Q, K, V, idx, n_sel, O=None, lse=None, ws=None,
                want_lse: bool = True, stream=None):
    """Attention over the selected blocks -> (O [b, n_q, h_q, d], lse [b, h_q, n_q])."""
    if O is None:
        O = torch.empty_like(Q)
    if lse is None and want_lse:
        lse = torch.empty((prob.batch, prob.h_q, prob.n_q), dtype=torch.float32, device=Q.device)
    if ws is None and (need := sparse_attn_workspace(prob)):
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    e = prob._ext()
    ws_p, ws_n = _ws(ws)
    _check(lib().infv2_sparse_attn(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                   _arg(K, "K", e.io, e.kv), _arg(V, "V", e.io, e.kv),
                                   _arg(idx, "idx", torch.int32, e.rows * e.budget),
                                   _arg(n_sel, "n_sel", torch.int32, e.rows),
                                   _arg(O, "O", e.io, e.q),
                                   _arg(lse, "lse", torch.float32, e.lse, optional=True),
                                   ws_p, ws_n, _stream(stream)))
    return O, lse


def sparse_attn_noalloc(prob: Problem, Q, K, V, idx, n_sel, O, lse=None, stream=None):
    """sparse_attn with the library's static per-GPU scratch as its workspace
    (infv2_sparse_attn_noalloc): nothing is allocated, O (and lse, optional)
    are the caller's.  Calls that overlap on one GPU race on the scratch."""
    e = prob._ext()
    _check(lib().infv2_sparse_attn_noalloc(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                           _arg(K, "K", e.io, e.kv), _arg(V, "V", e.io, e.kv),
                                           _arg(idx, "idx", torch.int32, e.rows * e.budget),
                                           _arg(n_sel, "n_sel", torch.int32, e.rows),
                                           _arg(O, "O", e.io, e.q),
                                           _arg(lse, "lse", torch.float32, e.lse, optional=True),
                                           _stream(stream)))
    return O, lse


def dense_attn_workspace(prob: Problem) -> int:
    return lib().infv2_dense_attn_workspace(ctypes.byref(prob._c()))


def dense_attn(prob: Problem, Q, K, V, O=None, lse=None, ws=None, want_lse: bool = True,
               stream=None):
    """Dense causal attention -> (O, lse)."""
    if O is None:
        O = torch.empty_like(Q)
    if lse is None and want_lse:
        lse = torch.empty((prob.batch, prob.h_q, prob.n_q), dtype=torch.float32, device=Q.device)
    if ws is None and (need := dense_attn_workspace(prob)):
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    e = prob._ext()
    ws_p, ws_n = _ws(ws)
    _check(lib().infv2_dense_attn(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                  _arg(K, "K", e.io, e.kv), _arg(V, "V", e.io, e.kv),
                                  _arg(O, "O", e.io, e.q),
                                  _arg(lse, "lse", torch.float32, e.lse, optional=True),
                                  ws_p, ws_n, _stream(stream)))
    return O, lse


# --- varlen batches / paged cache (decode shapes) ---------------------------

def _cache(prob: Problem, e: _Ext, K, V, block_table):
    """(K, V, block_table pointers, max_blocks, n_pages): a contiguous cache
    [batch, kv_cap, h_kv, d], or page pools [n_pages, B, h_kv, d] (V may be
    None for the key-only calls) with a table [batch, max_blocks]."""
    if block_table is None:
        return (_arg(K, "K", e.io, e.kv), _arg(V, "V", e.io, e.kv, optional=True), None, 0, 0)
    if not isinstance(K, torch.Tensor) or K.dim() != 4 or \
            tuple(K.shape[1:]) != (prob.B, prob.h_kv, prob.d):
        raise ValueError("a paged K must be a pool [n_pages, B, h_kv, d]")
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2 or \
            block_table.shape[0] < prob.batch:
        raise ValueError("block_table must be [batch, max_blocks]")
    n_pages, mb = K.shape[0], block_table.shape[1]
    pool = n_pages * prob.B * prob.h_kv * prob.d
    return (_arg(K, "K", e.io, pool), _arg(V, "V", e.io, pool, optional=True),
            _arg(block_table, "block_table", torch.int32, prob.batch * mb), mb, n_pages)


def compress_k_varlen(prob: Problem, K: torch.Tensor, seq_lens: torch.Tensor, Kc: torch.Tensor,
                      block_table: torch.Tensor | None = None, coarse: bool = False,
                      last_n: int = 0, stream=None) -> torch.Tensor:
    """Each sequence's last `last_n` complete kernels (all when last_n <= 0)
    of K^C1 (coarse=False) or K^C2 (coarse=True) into Kc [b, h_kv, cap, d];
    K is a page pool [n_pages, B, h_kv, d] when block_table is given."""
    e = prob._ext()
    k_p, _, bt, mb, npg = _cache(prob, e, K, None, block_table)
    _check(lib().infv2_compress_k_varlen(ctypes.byref(prob._c()), k_p, bt, mb, npg,
                                         _arg(seq_lens, "seq_lens", torch.int32, prob.batch),
                                         _arg(Kc, "Kc", e.io, e.kc2 if coarse else e.kc1),
                                         int(bool(coarse)), last_n, _stream(stream)))
    return Kc


def select_blocks_varlen_workspace(prob: Problem) -> int:
    return lib().infv2_select_blocks_varlen_workspace(ctypes.byref(prob._c()))


def select_blocks_varlen(prob: Problem, Q, Kc1, seq_lens, idx=None, n_sel=None, ws=None,
                         stream=None, Kc2=None):
    """(idx, n_sel) of a varlen decode batch (sequence i: seq_lens[i] keys)."""
    if idx is None:
        idx = torch.empty((prob.batch, prob.h_kv, prob.n_q, budget(prob)), dtype=torch.int32,
                          device=Q.device)
    if n_sel is None:
        n_sel = torch.empty((prob.batch, prob.h_kv, prob.n_q), dtype=torch.int32,
                            device=Q.device)
    if ws is None:
        ws = torch.empty(max(select_blocks_varlen_workspace(prob), 16), dtype=torch.uint8,
                         device=Q.device)
    e = prob._ext()
    ws_p, ws_n = _ws(ws)
    _check(lib().infv2_select_blocks_varlen(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                            _arg(Kc1, "Kc1", e.io, e.kc1, optional=True),
                                            _arg(Kc2, "Kc2", e.io, e.kc2, optional=True),
                                            _arg(seq_lens, "seq_lens", torch.int32, prob.batch),
                                            _arg(idx, "idx", torch.int32, e.rows * e.budget),
                                            _arg(n_sel, "n_sel", torch.int32, e.rows),
                                            ws_p, ws_n, _stream(stream)))
    return idx, n_sel


def sparse_attn_varlen_workspace(prob: Problem) -> int:
    return lib().infv2_sparse_attn_varlen_workspace(ctypes.byref(prob._c()))


def sparse_attn_varlen(prob: Problem, Q, K, V, seq_lens, idx, n_sel, block_table=None, O=None,
                       lse=None, ws=None, want_lse: bool = True, stream=None):
    """Sparse attention of a varlen decode batch -> (O, lse); K, V are page
    pools [n_pages, B, h_kv, d] when block_table [b, max_blocks] is given."""
    if O is None:
        O = torch.empty_like(Q)
    if lse is None and want_lse:
        lse = torch.empty((prob.batch, prob.h_q, prob.n_q), dtype=torch.float32, device=Q.device)
    if ws is None:
        ws = torch.empty(max(sparse_attn_varlen_workspace(prob), 16), dtype=torch.uint8,
                         device=Q.device)
    e = prob._ext()
    if V is None:
        raise ValueError("V is required")
    k_p, v_p, bt, mb, npg = _cache(prob, e, K, V, block_table)
    ws_p, ws_n = _ws(ws)
    _check(lib().infv2_sparse_attn_varlen(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                          k_p, v_p, bt, mb, npg,
                                          _arg(seq_lens, "seq_lens", torch.int32, prob.batch),
                                          _arg(idx, "idx", torch.int32, e.rows * e.budget),
                                          _arg(n_sel, "n_sel", torch.int32, e.rows),
                                          _arg(O, "O", e.io, e.q),
                                          _arg(lse, "lse", torch.float32, e.lse, optional=True),
                                          ws_p, ws_n, _stream(stream)))
    return O, lse


def _bwd_outputs(prob: Problem, Q, K, dQ, dK, dV):
    kv_rows = prob.kv_cap or prob.n_kv
    if dQ is None:
        dQ = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    if dK is None:
        dK = torch.empty((prob.batch, kv_rows, prob.h_kv, prob.d), dtype=torch.float32,
                         device=K.device)
    if dV is None:
        dV = torch.empty_like(dK)
    return dQ, dK, dV


def sparse_attn_bwd_workspace(prob: Problem) -> int:
    return lib().infv2_sparse_attn_bwd_workspace(ctypes.byref(prob._c()))


def sparse_attn_bwd(prob: Problem, Q, K, V, idx, n_sel, O, lse, dO, dQ=None, dK=None,
                    dV=None, ws=None, stream=None):
    """Gradients (dQ, dK, dV) in fp32 of the block-sparse attention with the
    selected sets held fixed."""
    dQ, dK, dV = _bwd_outputs(prob, Q, K, dQ, dK, dV)
    if ws is None and (need := sparse_attn_bwd_workspace(prob)):
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    e = prob._ext()
    ws_p, ws_n = _ws(ws)
    f32 = torch.float32
    _check(lib().infv2_sparse_attn_bwd(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                       _arg(K, "K", e.io, e.kv), _arg(V, "V", e.io, e.kv),
                                       _arg(idx, "idx", torch.int32, e.rows * e.budget),
                                       _arg(n_sel, "n_sel", torch.int32, e.rows),
                                       _arg(O, "O", e.io, e.q), _arg(lse, "lse", f32, e.lse),
                                       _arg(dO, "dO", e.io, e.q), _arg(dQ, "dQ", f32, e.q),
                                       _arg(dK, "dK", f32, e.kv), _arg(dV, "dV", f32, e.kv),
                                       ws_p, ws_n, _stream(stream)))
    return dQ, dK, dV


def dense_attn_bwd_workspace(prob: Problem) -> int:
    return lib().infv2_dense_attn_bwd_workspace(ctypes.byref(prob._c()))


def dense_attn_bwd(prob: Problem, Q, K, V, O, lse, dO, dQ=None, dK=None, dV=None, ws=None,
                   stream=None):
    """Gradients (dQ, dK, dV) in fp32 of dense causal attention."""
    dQ, dK, dV = _bwd_outputs(prob, Q, K, dQ, dK, dV)
    if ws is None and (need := dense_attn_bwd_workspace(prob)):
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    e = prob._ext()
    ws_p, ws_n = _ws(ws)
    f32 = torch.float32
    _check(lib().infv2_dense_attn_bwd(ctypes.byref(prob._c()), _arg(Q, "Q", e.io, e.q),
                                      _arg(K, "K", e.io, e.kv), _arg(V, "V", e.io, e.kv),
                                      _arg(O, "O", e.io, e.q), _arg(lse, "lse", f32, e.lse),
                                      _arg(dO, "dO", e.io, e.q), _arg(dQ, "dQ", f32, e.q),
                                      _arg(dK, "dK", f32, e.kv), _arg(dV, "dV", f32, e.kv),
                                      ws_p, ws_n, _stream(stream)))
    return dQ, dK, dV


def forward(prob: Problem, Q, K, V, Kc1=None, mode: str = "auto", stream=None,
            Kc2=None) -> dict:
    """Whole forward path: the dense switch, else compress -> scores -> top-k ->
    sparse attention (with prob.lse_approx the coarse keys are compressed too).
    Returns a dict of the intermediate and final tensors."""
    if mode == "auto":
        mode = "dense" if use_dense(prob) else "sparse"
    out = {"mode": mode}
    if mode == "dense":
        out["O"], out["lse"] = dense_attn(prob, Q, K, V, stream=stream)
        return out
    if Kc1 is None:
        Kc1 = compress_k(prob, K, stream=stream)
    if prob.lse_approx and Kc2 is None:
        Kc2 = compress_k2(prob, K, stream=stream)
    S_cmp = block_scores(prob, Q, Kc1, stream=stream, Kc2=Kc2)
    idx, n_sel = topk_select(prob, S_cmp, stream=stream)
    O, lse = sparse_attn(prob, Q, K, V, idx, n_sel, stream=stream)
    out.update(Kc1=Kc1, Kc2=Kc2, S_cmp=S_cmp, idx=idx, n_sel=n_sel, O=O, lse=lse)
    return out


class PrefillPipeline:
    """Sparse prefill of one sequence as a two-stream pipeline over query chunks.

    The query rows are split into ``n_chunks`` ranges on 64-token boundaries.
    The selection of range i+1 (compressed scores and top-k: bound by the
    matrix unit) is enqueued on one stream while the block-sparse attention of
    range i (bound by the K/V gather) runs on another; an event per range
    orders the two.  Each range is an ordinary call of the C ABI with
    q_pos0/n_q of that range (the selection with n_kv of the range, the
    attention with the whole sequence's n_kv, so that the library takes the
    same attention plan for every range as for the one-shot call: from 1024
    blocks on it splits the keys into ranges, which rounds differently), so
    every output row is computed exactly as in the one-shot path (bitwise the
    same O and LSE).  Buffers and workspaces
    are allocated once here; ``run`` allocates nothing.  With ``lean`` the
    selection streams the top-k through the score sweep (select_blocks), so
    no S^cmp buffer is held (2.1 GB at 128k); the two-call selection is
    faster on MI355X and is the default.
    """

    def __init__(self, prob: Problem, n_chunks: int, device=None, lean: bool = False):
        if prob.batch != 1:
            raise ValueError("PrefillPipeline takes one sequence (batch == 1)")
        if use_dense(prob):
            raise ValueError("the dense switch applies: use dense_attn")
        device = device or torch.device("cuda", torch.cuda.current_device())
        self.prob = prob
        self.lean = lean
        n_q = prob.n_q
        kv_cap = prob.kv_cap or prob.n_kv
        self.n_c1 = n_kernels(prob)
        c1_cap = prob.c1_cap or self.n_c1
        c2_cap = prob.c2_cap or n_coarse_kernels(prob)
        cuts = sorted({0, n_q} | {min(n_q, round(n_q * i / n_chunks / prob.B) * prob.B)
                                  for i in range(1, n_chunks)})
        self.chunks = []
        for r0, r1 in zip(cuts[:-1], cuts[1:]):
            p = dataclasses.replace(prob, n_q=r1 - r0, q_pos0=prob.q_pos0 + r0,
                                    n_kv=prob.q_pos0 + r1, kv_cap=kv_cap, c1_cap=c1_cap,
                                    c2_cap=c2_cap)
            p_att = dataclasses.replace(p, n_kv=prob.n_kv)
            ws_bytes = select_blocks_workspace(p) if lean else block_scores_workspace(p)
            self.chunks.append(dict(
                p=p, p_att=p_att, r0=r0, r1=r1,
                S=None if lean else torch.empty((1, p.h_kv, p.n_q, n_blocks(p)),
                                                dtype=torch.float32, device=device),
                idx=torch.empty((1, p.h_kv, p.n_q, budget(p)), dtype=torch.int32, device=device),
                n_sel=torch.empty((1, p.h_kv, p.n_q), dtype=torch.int32, device=device),
                lse=torch.empty((1, p.h_q, p.n_q), dtype=torch.float32, device=device),
                ws_s=torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=device),
                ws_a=torch.empty(max(sparse_attn_workspace(p_att), 16), dtype=torch.uint8,
                                 device=device),
                ready=torch.cuda.Event()))
        self.sel_stream = torch.cuda.Stream(device=device)
        self.att_stream = torch.cuda.Stream(device=device)
        self.done = torch.cuda.Event()

    def run(self, Q, K, V, Kc1, O, lse=None, attn_events=None, Kc2=None):
        """Enqueue one prefill: compress (K^C1, and K^C2 into ``Kc2`` with the
        LSE approximation), then per range selection and attention.
        Both streams first wait for the caller's current stream; the caller's
        stream then waits for the end.  With ``attn_events`` (a list of
        (start, end) timing-event pairs, one per range) the attention launches
        are bracketed on the attention stream."""
        caller = torch.cuda.current_stream()
        self.sel_stream.wait_stream(caller)
        self.att_stream.wait_stream(caller)
        prob, s_sel, s_att = self.prob, self.sel_stream, self.att_stream
        # the previous run's attention has consumed every range's idx/n_sel
        s_sel.wait_event(self.done)
        compress_k(prob, K, Kc1, stream=s_sel)
        if prob.lse_approx:
            if Kc2 is None:
                raise ValueError("the LSE approximation needs a K^C2 buffer (Kc2)")
            compress_k2(prob, K, Kc2, stream=s_sel)
        for c in self.chunks:
            p = c["p"]
            q = Q[:, c["r0"]:c["r1"]]
            if self.lean:
                select_blocks(p, q, Kc1, None, c["idx"], c["n_sel"], c["ws_s"], stream=s_sel,
                              Kc2=Kc2)
            else:
                block_scores(p, q, Kc1, c["S"], c["ws_s"], stream=s_sel, Kc2=Kc2)
                topk_select(p, c["S"], c["idx"], c["n_sel"], stream=s_sel)
            c["ready"].record(s_sel)
        for i, c in enumerate(self.chunks):
            s_att.wait_event(c["ready"])
            if attn_events is not None:
                attn_events[i][0].record(s_att)
            sparse_attn(c["p_att"], Q[:, c["r0"]:c["r1"]], K, V, c["idx"], c["n_sel"],
                        O[:, c["r0"]:c["r1"]], c["lse"], c["ws_a"], stream=s_att)
            if attn_events is not None:
                attn_events[i][1].record(s_att)
            if lse is not None:
                with torch.cuda.stream(s_att):
                    lse[:, :, c["r0"]:c["r1"]].copy_(c["lse"])
        self.done.record(s_att)
        caller.wait_stream(s_att)
        caller.wait_stream(s_sel)
        return O, lse
