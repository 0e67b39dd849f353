"""Seeded synthetic Q/K/V with planted needle blocks.

Recipe (stated once, used by the tests and the bench):
  * numpy ``Generator(PCG64(seed))``; Q [b, n_q, h_q, d], then K, then V
    [b, n_kv, h_kv, d], each ``standard_normal`` in float32;
  * per sequence, ``n_needles`` needle blocks (fewer if a shortened variant
    has fewer blocks) drawn without replacement, uniformly from blocks
    [N_init, n_blk - N_local);
  * per sequence and KV group g, the mean query direction
    u_g = normalise(sum over tokens t and heads h of group g of Q[t, h, :])
    is added, times 0.5, to every K row of each needle block;
  * the arrays are then cast to the I/O dtype (torch's bf16 cast rounds to
    nearest even); fp32 configs stay fp32.
Decode workloads draw the whole cache the same way and the single query of
each sequence from the same generator (Q is drawn first).
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Config

_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def needle_blocks(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """[batch, n_needles] needle block ids per sequence (sorted)."""
    lo, hi = cfg.N_init, cfg.n_blk - cfg.N_local
    count = max(0, min(cfg.n_needles, hi - lo))   # shortened variants have fewer blocks
    out = np.zeros((cfg.batch, count), dtype=np.int64)
    for b in range(cfg.batch):
        if count:
            out[b] = np.sort(rng.choice(np.arange(lo, hi), size=count, replace=False))
    return out


def make_inputs(cfg: Config, seed: int | None = None, n_kv: int | None = None,
                batch: int | None = None):
    """Return dict(q, k, v) as contiguous CPU torch tensors in the I/O dtype,
    plus ``needles`` [batch, n_needles].

    ``n_kv`` and ``batch`` override the config (tests use smaller variants).
    """
    from dataclasses import replace
    seed = cfg.seed if seed is None else seed
    n_kv = cfg.n_kv if n_kv is None else n_kv
    if batch is not None and batch != cfg.batch:
        cfg = replace(cfg, batch=batch)
    n_q = 1 if cfg.decode else n_kv
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((cfg.batch, n_q, cfg.h_q, cfg.d), dtype=np.float32)
    k = rng.standard_normal((cfg.batch, n_kv, cfg.h_kv, cfg.d), dtype=np.float32)
    v = rng.standard_normal((cfg.batch, n_kv, cfg.h_kv, cfg.d), dtype=np.float32)
    sub = cfg if n_kv == cfg.n_kv else _with_nkv(cfg, n_kv)
    needles = needle_blocks(sub, rng)
    G = cfg.G
    for b in range(cfg.batch):
        for g in range(cfg.h_kv):
            u = q[b, :, g * G:(g + 1) * G, :].astype(np.float64).sum(axis=(0, 1))
            nrm = np.linalg.norm(u)
            if nrm == 0.0:
                continue
            shift = (0.5 * u / nrm).astype(np.float32)
            for blk in needles[b]:
                k[b, blk * cfg.B:(blk + 1) * cfg.B, g, :] += shift
    dt = _TORCH_DT[cfg.io]
    return {
        "q": torch.from_numpy(q).to(dt).contiguous(),
        "k": torch.from_numpy(k).to(dt).contiguous(),
        "v": torch.from_numpy(v).to(dt).contiguous(),
        "needles": needles,
    }


def _with_nkv(cfg: Config, n_kv: int) -> Config:
    from dataclasses import replace
    return replace(cfg, n_kv=n_kv, n_q=(1 if cfg.decode else n_kv))


def varlen_lengths(batch: int, max_len: int, seed: int, must=()) -> np.ndarray:
    """Seeded cache lengths of a varlen decode batch: the listed lengths first,
    the rest uniform on [1, max_len]; int32 [batch]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = list(must)[:batch]
    lens += rng.integers(1, max_len + 1, size=batch - len(lens)).tolist()
    return np.asarray(lens, dtype=np.int32)


def paged_cache(k: torch.Tensor, v: torch.Tensor, lengths, B: int, seed: int,
                extra_pages: int = 3):
    """The same tokens in a paged layout: pools [n_pages, B, h_kv, d] and a
    page table [batch, max_blocks] int32 with the pages of all sequences in a
    seeded random order (pages past a sequence's length hold its zero-padded
    rows; the pool also has `extra_pages` random pages no table points to).
    k, v: contiguous [batch, kv_cap, h_kv, d] CPU tensors.  Layout only."""
    b, cap, h_kv, d = k.shape
    max_blocks = (cap + B - 1) // B
    rng = np.random.Generator(np.random.PCG64(seed))
    n_pages = b * max_blocks + extra_pages
    order = rng.permutation(n_pages)
    table = order[: b * max_blocks].reshape(b, max_blocks).astype(np.int32)
    kp = torch.empty((n_pages, B, h_kv, d), dtype=k.dtype)
    vp = torch.empty((n_pages, B, h_kv, d), dtype=v.dtype)
    spare = torch.from_numpy(order[b * max_blocks:].astype(np.int64))
    kp[spare] = torch.from_numpy(rng.standard_normal((extra_pages, B, h_kv, d), dtype=np.float32)).to(k.dtype)
    vp[spare] = torch.from_numpy(rng.standard_normal((extra_pages, B, h_kv, d), dtype=np.float32)).to(v.dtype)
    pad = max_blocks * B - cap
    kf = torch.nn.functional.pad(k, (0, 0, 0, 0, 0, pad)) if pad else k
    vf = torch.nn.functional.pad(v, (0, 0, 0, 0, 0, pad)) if pad else v
    idx = torch.from_numpy(table.reshape(-1).astype(np.int64))
    kp[idx] = kf.reshape(b * max_blocks, B, h_kv, d)
    vp[idx] = vf.reshape(b * max_blocks, B, h_kv, d)
    return kp.contiguous(), vp.contiguous(), torch.from_numpy(table)
