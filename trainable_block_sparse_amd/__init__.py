"""Thin Python binding of libinfv2 (the C ABI in include/infv2.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libinfv2.so.  torch supplies device memory and the current HIP stream.  The
library must have been built (``python -m trainable_block_sparse_amd.build``);
importing a function without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libinfv2.so")

INFV2_OK, INFV2_E_ARG, INFV2_E_UNSUPPORTED, INFV2_E_WORKSPACE, INFV2_E_HIP = 0, -1, -2, -3, -4
INFV2_BF16, INFV2_F32 = 0, 1
EXPORTED = (
    "infv2_n_kernels", "infv2_n_blocks", "infv2_budget", "infv2_use_dense",
    "infv2_check_problem", "infv2_compress_k", "infv2_block_scores_workspace",
    "infv2_block_scores", "infv2_topk_select", "infv2_sparse_attn_workspace",
    "infv2_sparse_attn", "infv2_dense_attn_workspace", "infv2_dense_attn",
    "infv2_status_string", "infv2_last_error",
)


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("q_pos0", ctypes.c_int32),
        ("n_kv", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("G", ctypes.c_int32),
        ("d", ctypes.c_int32), ("B", ctypes.c_int32), ("l_C1", ctypes.c_int32),
        ("s_C1", ctypes.c_int32), ("l", ctypes.c_int32), ("s", ctypes.c_int32),
        ("k", ctypes.c_int32), ("N_init", ctypes.c_int32), ("N_local", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("kv_cap", ctypes.c_int64),
        ("c1_cap", ctypes.c_int64),
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

    @property
    def h_q(self) -> int:
        return self.G * self.h_kv

    def to_c(self) -> _Problem:
        return _Problem(self.batch, self.n_q, self.q_pos0, self.n_kv, self.h_kv, self.G, self.d,
                        self.B, self.l_C1, self.s_C1, self.l, self.s, self.k, self.N_init,
                        self.N_local, INFV2_BF16 if self.dtype == "bf16" else INFV2_F32,
                        self.scale, self.kv_cap, self.c1_cap)


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
            "infv2_n_kernels": (i32, [P]), "infv2_n_blocks": (i32, [P]),
            "infv2_budget": (i32, [P]), "infv2_use_dense": (ctypes.c_int, [P]),
            "infv2_check_problem": (ctypes.c_int, [P]),
            "infv2_compress_k": (ctypes.c_int, [P, vp, vp, i32, i32, vp]),
            "infv2_block_scores_workspace": (sz, [P]),
            "infv2_block_scores": (ctypes.c_int, [P, vp, vp, vp, vp, sz, vp]),
            "infv2_topk_select": (ctypes.c_int, [P, vp, vp, vp, vp]),
            "infv2_sparse_attn_workspace": (sz, [P]),
            "infv2_sparse_attn": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "infv2_dense_attn_workspace": (sz, [P]),
            "infv2_dense_attn": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, sz, vp]),
            "infv2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "infv2_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != INFV2_OK:
        raise Infv2Error(status, lib().infv2_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# --- derived sizes ----------------------------------------------------------

def n_kernels(prob: Problem) -> int:
    return lib().infv2_n_kernels(ctypes.byref(prob.to_c()))


def n_blocks(prob: Problem) -> int:
    return lib().infv2_n_blocks(ctypes.byref(prob.to_c()))


def budget(prob: Problem) -> int:
    return lib().infv2_budget(ctypes.byref(prob.to_c()))


def use_dense(prob: Problem) -> bool:
    r = lib().infv2_use_dense(ctypes.byref(prob.to_c()))
    if r < 0:
        _check(lib().infv2_check_problem(ctypes.byref(prob.to_c())))
    return r == 1


def check_problem(prob: Problem) -> None:
    _check(lib().infv2_check_problem(ctypes.byref(prob.to_c())))


def _torch_dtype(prob: Problem):
    return torch.bfloat16 if prob.dtype == "bf16" else torch.float32


# --- the five calls -----------------------------------------------------------

def compress_k(prob: Problem, K: torch.Tensor, Kc1: torch.Tensor | None = None,
               c1_begin: int = 0, c1_end: int | None = None, stream=None) -> torch.Tensor:
    """K [b, kv_cap, h_kv, d] -> K^C1 [b, h_kv, c1_cap, d] (rows c1_begin..c1_end-1)."""
    n_c1 = n_kernels(prob)
    if Kc1 is None:
        cap = prob.c1_cap or n_c1
        Kc1 = torch.empty((prob.batch, prob.h_kv, max(cap, 1), prob.d), dtype=K.dtype,
                          device=K.device)
    c1_end = n_c1 if c1_end is None else c1_end
    _check(lib().infv2_compress_k(ctypes.byref(prob.to_c()), _ptr(K), _ptr(Kc1), c1_begin, c1_end,
                                  _stream(stream)))
    return Kc1


def block_scores_workspace(prob: Problem) -> int:
    return lib().infv2_block_scores_workspace(ctypes.byref(prob.to_c()))


def block_scores(prob: Problem, Q: torch.Tensor, Kc1: torch.Tensor,
                 S_cmp: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Q, K^C1 -> S^cmp [b, h_kv, n_q, n_blk] fp32 (blocks after floor(p/B) untouched)."""
    if S_cmp is None:
        S_cmp = torch.full((prob.batch, prob.h_kv, prob.n_q, n_blocks(prob)), float("nan"),
                           dtype=torch.float32, device=Q.device)
    need = block_scores_workspace(prob)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    _check(lib().infv2_block_scores(ctypes.byref(prob.to_c()), _ptr(Q), _ptr(Kc1), _ptr(S_cmp),
                                    _ptr(ws), ws.numel() if ws is not None else 0,
                                    _stream(stream)))
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
    _check(lib().infv2_topk_select(ctypes.byref(prob.to_c()), _ptr(S_cmp), _ptr(idx), _ptr(n_sel),
                                   _stream(stream)))
    return idx, n_sel


def sparse_attn_workspace(prob: Problem) -> int:
    return lib().infv2_sparse_attn_workspace(ctypes.byref(prob.to_c()))


def sparse_attn(prob: Problem, Q, K, V, idx, n_sel, O=None, lse=None, ws=None,
                want_lse: bool = True, stream=None):
    """Attention over the selected blocks -> (O [b, n_q, h_q, d], lse [b, h_q, n_q])."""
    if O is None:
        O = torch.empty_like(Q)
    if lse is None and want_lse:
        lse = torch.empty((prob.batch, prob.h_q, prob.n_q), dtype=torch.float32, device=Q.device)
    need = sparse_attn_workspace(prob)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    _check(lib().infv2_sparse_attn(ctypes.byref(prob.to_c()), _ptr(Q), _ptr(K), _ptr(V),
                                   _ptr(idx), _ptr(n_sel), _ptr(O), _ptr(lse), _ptr(ws),
                                   ws.numel() if ws is not None else 0, _stream(stream)))
    return O, lse


def dense_attn_workspace(prob: Problem) -> int:
    return lib().infv2_dense_attn_workspace(ctypes.byref(prob.to_c()))


def dense_attn(prob: Problem, Q, K, V, O=None, lse=None, ws=None, want_lse: bool = True,
               stream=None):
    """Dense causal attention -> (O, lse)."""
    if O is None:
        O = torch.empty_like(Q)
    if lse is None and want_lse:
        lse = torch.empty((prob.batch, prob.h_q, prob.n_q), dtype=torch.float32, device=Q.device)
    need = dense_attn_workspace(prob)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    _check(lib().infv2_dense_attn(ctypes.byref(prob.to_c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                  _ptr(lse), _ptr(ws), ws.numel() if ws is not None else 0,
                                  _stream(stream)))
    return O, lse


def forward(prob: Problem, Q, K, V, Kc1=None, mode: str = "auto", stream=None) -> dict:
    """Whole forward path: the dense switch, else compress -> scores -> top-k ->
    sparse attention.  Returns a dict of the intermediate and final tensors."""
    if mode == "auto":
        mode = "dense" if use_dense(prob) else "sparse"
    out = {"mode": mode}
    if mode == "dense":
        out["O"], out["lse"] = dense_attn(prob, Q, K, V, stream=stream)
        return out
    if Kc1 is None:
        Kc1 = compress_k(prob, K, stream=stream)
    S_cmp = block_scores(prob, Q, Kc1, stream=stream)
    idx, n_sel = topk_select(prob, S_cmp, stream=stream)
    O, lse = sparse_attn(prob, Q, K, V, idx, n_sel, stream=stream)
    out.update(Kc1=Kc1, S_cmp=S_cmp, idx=idx, n_sel=n_sel, O=O, lse=lse)
    return out
