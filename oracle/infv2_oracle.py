"""InfLLM-V2 dense-sparse switchable attention, forward path: plain fp64 CPU oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never imports it, and it imports nothing from the GPU library: the two share no
code.  It is deliberately slow and literal: numpy fp64, one library primitive
per step (a matmul, a sort, a sum), no blocking, fusion or reordering beyond
what each definition states.  Loops over query rows only bound memory.

Sources (cited by tag in the docstrings below):

[KD2]  papernotes.org note "InfLLM-V2: Dense-Sparse Switchable Attention for
       Seamless Short-to-Long Adaptation", section 方法详解 > 关键设计 2 (key design
       2): attended set I(i) = I_init u I_local(i) u I_topk(i), top-k over the
       remaining blocks by S^cmp; local blocks cover the sliding window when
       N_local >= ceil(w/B)+1.
[KD3]  same page, 关键设计 3 (key design 3): stage 1 mean-pools K with kernel
       length l_C1 and stride s_C1 into K^C1 and takes S^C1 = Softmax(Q K^C1^T);
       stage 2 sums S^C1 over the G heads of a GQA group (S^shared); stage 3
       max-pools S^shared with length l and stride s into S^cmp;
       l_C1 = B/2, s_C1 = B/4, l = 5, s = 4.
[KD4]  same page, 关键设计 4 (key design 4): the softmax normaliser is an exact
       log-sum-exp taken in a first pass; the method's result is the plain
       softmax.  Its LSE approximation estimates that normaliser from coarser
       kernels with s_C2 = 4 s_C1 and l_C2 = 4 l_C1, cutting the selection's
       cost from 2x to 1.25x of one pass.
[BLOG-LSE] OpenBMB blog (below), 高效Top-K实现: the coarse kernels are much
       longer than the ordinary ones; the LSE is taken between the query and
       the coarse kernels, at a fraction s_C1/s_C2 of the original cost.
[FLOW] same page, 整体框架 (overall framework) flowchart: short inputs take
       dense attention, long inputs the sparse path.
[APPA] paperlayer.ai summary of arXiv 2509.24663v1, "A IMPLEMENTATION DETAIL":
       attention restricted to the key blocks in the visible set; the kernel
       returns O and the log-sum-exp.
[BLOG-KERNEL] OpenBMB blog "技术Blog-4 | 新一代InfLLM：可训练的稀疏注意力机制",
       section 动态上下文块选择 > 语义核 (semantic kernels): kernels overlap so that
       every segment lies inside a complete kernel; keys only; a block's score
       is the maximum over the kernels that intersect it; initial and local
       blocks get an infinite score; inputs shorter than the selected budget
       degrade to dense attention.
[BLOG-SHARE] same blog, Top-K块共享 (top-k sharing): the heads of one group
       share one block selection.
[BLOG-TRAIN] same blog, 可训练稀疏注意力的设计原则 (design principles of trainable
       sparse attention): the top-k selection is not differentiable; the kernels
       are parameter-free mean-pools, optimised only through the token-level
       keys, so training differentiates the block-sparse attention with the
       selected sets held fixed.
[BLOG-TOPK] same blog, 高效Top-K实现 (efficient top-k): softmax per kernel,
       aggregate over the head group, then top-k per query token.
[BLOG-GRAN] same blog, 查询和键值词元的不同粒度 (query and key-value tokens at
       different granularity): selection is made per query token, which is
       what lets decoding (one new token per sequence) use the sparse path.

Readings where the pages are silent or ambiguous are tagged READING-<n>; the
ones this module follows (the others concern the tests' exemption rule, the
inputs and the GPU kernels' own sweeps):
 1 scale 1/sqrt(d) in both softmaxes          8 dense switch: ceil(n/B) <= N_init+N_local+k
 2 a kernel is visible when its last token <= p 9 top-k ties go to the lower block index
 3 group SUM (not mean) over the G heads       11 K^C1 and O rounded once (RNE) to the I/O dtype
 4 max-pool window = kernels intersecting block 12 no visible kernel -> lse and S^cmp are -inf
 5 partial kernels at the end are excluded      13 decode: cache length L includes the new token
 6 top-k is in addition to init and local     16 LSE approximation: coarse keys are the
 7 local = the N_local blocks ending at the        exact mean (one rounding) of l_C2 keys at
   query's own block                               stride s_C2, visible by READING-2; the
                                                   estimate is log sum over visible coarse
                                                   kernels of exp(z2) + ln(s_C2/s_C1); with
                                                   no visible coarse kernel the exact LSE
                                                17 backward: the sets I(p) are constants;
                                                   gradients of the sparse attention only
                                                18 varlen batch / paged cache: each sequence
                                                   is its own problem of its own length;
                                                   a page table only says where its key
                                                   rows are stored

Parity: every function below is pinned by ``tests/test_oracle_*.py`` against
closed forms, invariants, library special cases (torch SDPA, torch's bf16
cast), brute force on tiny inputs and the hand-written golden file
``tests/golden/maxpool_window.txt``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

__all__ = [
    "Problem", "round_to_bf16", "round_to_io", "n_kernels", "kernel_visible",
    "kernels_of_block", "compress_k", "selection_scores", "max_pool_blocks", "select_blocks",
    "attention_rows", "dense_switch", "forward_rows", "attended_tokens", "compress_k2",
    "n_coarse_kernels", "coarse_visible", "coarse_lse", "attention_rows_backward",
    "gather_paged", "decode_varlen",
]

# --------------------------------------------------------------------------
# Problem description (the oracle's own; the library has its own struct)
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Problem:
    """Hyper-parameters in the pages' notation ([KD2], [KD3])."""
    G: int            # query heads per KV group
    h_kv: int         # KV heads (groups)
    d: int            # head dimension
    B: int = 64       # KV block size
    l_C1: int = 32    # stage-1 kernel length
    s_C1: int = 16    # stage-1 kernel stride
    l: int = 5        # stage-3 max-pool length (in kernels)
    s: int = 4        # stage-3 max-pool stride (in kernels)
    k: int = 16       # top-k blocks
    N_init: int = 1
    N_local: int = 2
    io: str = "bf16"  # "bf16" or "f32": dtype of Q, K, V, K^C1 and O
    scale: float | None = None  # None -> 1/sqrt(d)  (READING-1)
    lse_approx: bool = False    # estimate the normaliser from coarse kernels ([KD4])

    @property
    def l_C2(self) -> int:
        """Coarse kernel length, 4 l_C1 ([KD4])."""
        return 4 * self.l_C1

    @property
    def s_C2(self) -> int:
        """Coarse kernel stride, 4 s_C1 ([KD4])."""
        return 4 * self.s_C1

    @property
    def h_q(self) -> int:
        return self.G * self.h_kv

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d) if self.scale is None else float(self.scale)

    @property
    def budget(self) -> int:
        """Largest |I(p)|: N_init + N_local + k blocks ([KD2], READING-6)."""
        return self.N_init + self.N_local + self.k


# --------------------------------------------------------------------------
# Rounding (own implementation; single rounding straight from fp64)
# --------------------------------------------------------------------------

_BF16_P, _F32_P = 8, 24          # significant bits
_EMIN = -126                     # smallest normal exponent (bf16 and fp32)
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(x) -> np.ndarray:
    """Nearest bf16 value of each fp64 input, ties to even, in ONE rounding.

    bf16 has 8 significant bits and fp32's exponent range.  For |x| >= 2^-126
    the spacing of bf16 values around x is 2^(e-8) with x = m*2^e, 0.5<=|m|<1;
    below that the spacing is the subnormal quantum 2^-133.  ``np.rint``
    rounds half to even.  Never goes through fp32 (which would round twice).
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)
    q = np.maximum(e - _BF16_P, _EMIN - _BF16_P + 1)      # quantum exponent
    r = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    over = np.abs(r) > _BF16_MAX
    r[over] = np.copysign(np.inf, r[over])
    out[fin] = r
    return out


def round_to_io(x, io: str) -> np.ndarray:
    """Round fp64 values once (RNE) to the I/O dtype (READING-11)."""
    if io == "bf16":
        return round_to_bf16(x)
    if io == "f32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(io)


def _round_fraction(fr: Fraction, io: str) -> float:
    """Nearest value of the I/O format to an exact rational, ties to even."""
    p = _BF16_P if io == "bf16" else _F32_P
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                      # now 2^e <= a < 2^(e+1)
    e = max(e, _EMIN)
    quantum = Fraction(2) ** (e - p + 1)
    n, rem = divmod(a, quantum)     # a = n*quantum + rem, 0 <= rem < quantum
    half = quantum / 2
    if rem > half or (rem == half and n % 2 == 1):
        n += 1
    val = float(n * quantum)
    if io == "bf16" and val > _BF16_MAX:
        val = math.inf
    return sign * val


# --------------------------------------------------------------------------
# Stage 1: K^C1 = mean-pooled keys ([KD3] stage 1, [BLOG-KERNEL])
# --------------------------------------------------------------------------


def n_kernels(n_kv: int, l_C1: int, s_C1: int) -> int:
    """Number of COMPLETE stage-1 kernels over n_kv keys (READING-5)."""
    return 0 if n_kv < l_C1 else (n_kv - l_C1) // s_C1 + 1


def compress_k(K, prob: Problem) -> np.ndarray:
    """K^C1[b, g, j, :] = mean over u < l_C1 of K[b, j*s_C1 + u, g, :].

    K: [b, n_kv, h_kv, d] (values already exact in the I/O dtype).
    Returns [b, h_kv, n_C1, d] fp64 holding I/O-dtype values: the exact mean,
    rounded once (READING-11).  The sum is taken in fp64 term by term; an
    error-free TwoSum step shows whether every partial sum was exact.  Where
    it was not, that element is redone in exact rational arithmetic.
    """
    return _mean_pool_keys(K, prob.l_C1, prob.s_C1, prob.io)


def n_coarse_kernels(n_kv: int, prob: Problem) -> int:
    """Number of complete coarse kernels (length l_C2, stride s_C2) over n_kv
    keys ([KD4], READING-5, READING-16)."""
    return n_kernels(n_kv, prob.l_C2, prob.s_C2)


def compress_k2(K, prob: Problem) -> np.ndarray:
    """Coarse keys for the LSE approximation ([KD4], [BLOG-LSE], READING-16):
    K^C2[b, g, j, :] = mean over u < l_C2 of K[b, j*s_C2 + u, g, :], the exact
    mean rounded once to the I/O dtype, as for K^C1.
    Returns [b, h_kv, n_C2, d]."""
    return _mean_pool_keys(K, prob.l_C2, prob.s_C2, prob.io)


def _mean_pool_keys(K, lc: int, sc: int, io: str) -> np.ndarray:
    K = np.asarray(K, dtype=np.float64)
    b, n, h_kv, d = K.shape
    n_c1 = n_kernels(n, lc, sc)
    out = np.zeros((b, h_kv, n_c1, d))
    pow2 = (lc & (lc - 1)) == 0
    for j in range(n_c1):
        seg = K[:, j * sc: j * sc + lc]                 # [b, l_C1, h_kv, d]
        s = np.zeros((b, h_kv, d))
        inexact = np.zeros((b, h_kv, d), dtype=bool)
        for u in range(lc):
            x = seg[:, u]
            t = s + x
            bp = t - s
            err = (s - (t - bp)) + (x - bp)             # TwoSum error term
            inexact |= err != 0
            s = t
        mean = round_to_io(s / lc, io) if pow2 else np.zeros_like(s)
        redo = inexact if pow2 else np.ones_like(inexact)
        for bi, g, di in zip(*np.nonzero(redo)):
            exact = sum(Fraction(float(v)) for v in seg[bi, :, g, di])
            mean[bi, g, di] = _round_fraction(exact / lc, io)
        out[:, :, j, :] = mean
    return out


# --------------------------------------------------------------------------
# Stages 2-3: compressed scores, group sum, max-pool ([KD3], [KD4], [BLOG-*])
# --------------------------------------------------------------------------


def kernel_visible(j, p, prob: Problem):
    """Kernel j is causal for query position p when its LAST token is <= p
    (READING-2).  Works elementwise on arrays."""
    return np.asarray(j) * prob.s_C1 + prob.l_C1 - 1 <= np.asarray(p)


def kernels_of_block(blk: int, n_c1: int, prob: Problem) -> list[int]:
    """Kernels whose token span [j*s_C1, j*s_C1+l_C1-1] intersects block
    [blk*B, blk*B+B-1] ([BLOG-KERNEL]: a block's score is the maximum over
    the kernels that intersect it; READING-4)."""
    lo_tok, hi_tok = blk * prob.B, blk * prob.B + prob.B - 1
    return [j for j in range(n_c1)
            if j * prob.s_C1 <= hi_tok and j * prob.s_C1 + prob.l_C1 - 1 >= lo_tok]


def coarse_visible(j2, p, prob: Problem):
    """Coarse kernel j2 is causal for position p when its last token is <= p
    (READING-2 applied to the coarse kernels, READING-16)."""
    return np.asarray(j2) * prob.s_C2 + prob.l_C2 - 1 <= np.asarray(p)


def coarse_lse(Qrows, Kc2, q_pos, prob: Problem) -> np.ndarray:
    """The LSE approximation's estimate of the fine normaliser ([KD4],
    [BLOG-LSE], READING-16), per row and query head:
        lse~[h] = log sum_{j2 visible} exp(scale * Q[p, h] . K^C2[g(h), j2])
                  + ln(s_C2 / s_C1),
    NaN where no coarse kernel is visible (the caller then takes the exact
    LSE).  Qrows: [R, h_q, d]; Kc2: [h_kv, n_C2, d]; q_pos: [R]."""
    Qrows = np.asarray(Qrows, np.float64)
    Kc2 = np.asarray(Kc2, np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    R = Qrows.shape[0]
    n_c2 = Kc2.shape[1]
    G = prob.G
    vis = coarse_visible(np.arange(n_c2)[None, :], q_pos[:, None], prob)   # [R, n_C2]
    out = np.full((R, prob.h_q), np.nan)
    for g in range(prob.h_kv):
        z = (Qrows[:, g * G:(g + 1) * G, :] @ Kc2[g].T) * prob.sm_scale    # [R, G, n_C2]
        zm = np.where(vis[:, None, :], z, -np.inf)
        mx = zm.max(axis=2, keepdims=True) if n_c2 else np.full((R, G, 1), -np.inf)
        has = np.isfinite(mx)
        safe_mx = np.where(has, mx, 0.0)
        ssum = np.exp(zm - safe_mx).sum(axis=2, keepdims=True)
        est = safe_mx + np.log(np.where(has, ssum, 1.0)) + math.log(prob.s_C2 / prob.s_C1)
        out[:, g * G:(g + 1) * G] = np.where(has, est, np.nan)[:, :, 0]
    return out


def selection_scores(Qrows, Kc1, q_pos, n_kv: int, prob: Problem, Kc2=None):
    """Selection scores for a set of query rows of ONE sequence.

    Qrows: [R, h_q, d]; Kc1: [h_kv, n_C1, d]; q_pos: [R] absolute positions.
    Returns (lse [R, h_q], S_shared [R, h_kv, n_C1], S_cmp [R, h_kv, n_blk]).

    z[h, j]       = scale * Q[p, h] . K^C1[g(h), j]        (READING-1)
    lse[h]        = log sum_{j visible} exp(z[h, j])       ([KD4]: exact LSE)
                    or, when prob.lse_approx (Kc2 [h_kv, n_C2, d] given), the
                    coarse estimate coarse_lse() where it exists (READING-16)
    S^C1[h, j]    = exp(z[h, j] - lse[h]) on visible j     ([KD3] stage 1)
    S^shared[g,j] = sum over the G heads h of group g      ([KD3] stage 2, READING-3)
    S^cmp[g, blk] = max over visible kernels intersecting blk of S^shared
                    (-inf if there is none)                 ([KD3] stage 3, READING-4/12)
    """
    Qrows = np.asarray(Qrows, np.float64)
    Kc1 = np.asarray(Kc1, np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    R = Qrows.shape[0]
    n_c1 = Kc1.shape[1]
    n_blk = -(-n_kv // prob.B)
    G = prob.G
    vis = kernel_visible(np.arange(n_c1)[None, :], q_pos[:, None], prob)   # [R, n_C1]
    if prob.lse_approx:
        if Kc2 is None:
            raise ValueError("lse_approx needs the coarse keys Kc2")
        est = coarse_lse(Qrows, Kc2, q_pos, prob)                           # [R, h_q]
    lse = np.full((R, prob.h_q), -np.inf)
    S_shared = np.zeros((R, prob.h_kv, n_c1))
    S_cmp = np.full((R, prob.h_kv, n_blk), -np.inf)
    for g in range(prob.h_kv):
        z = (Qrows[:, g * G:(g + 1) * G, :] @ Kc1[g].T) * prob.sm_scale    # [R, G, n_C1]
        zm = np.where(vis[:, None, :], z, -np.inf)
        mx = zm.max(axis=2, keepdims=True) if n_c1 else np.full((R, G, 1), -np.inf)
        has = np.isfinite(mx)
        safe_mx = np.where(has, mx, 0.0)
        ssum = np.exp(zm - safe_mx).sum(axis=2, keepdims=True)
        lse_g = np.where(has, safe_mx + np.log(np.where(has, ssum, 1.0)), -np.inf)
        if prob.lse_approx:
            e = est[:, g * G:(g + 1) * G, None]
            lse_g = np.where(np.isnan(e), lse_g, e)
        lse[:, g * G:(g + 1) * G] = lse_g[:, :, 0]
        s_c1 = np.where(vis[:, None, :], np.exp(zm - np.where(has, lse_g, 0.0)), 0.0)
        S_shared[:, g, :] = s_c1.sum(axis=1)
        S_cmp[:, g, :] = max_pool_blocks(S_shared[:, g, :], vis, n_blk, prob)
    return lse, S_shared, S_cmp


def max_pool_blocks(S_shared, vis, n_blk: int, prob: Problem) -> np.ndarray:
    """S^cmp[r, blk] = max over the visible kernels that intersect block blk
    of S^shared[r, j]; -inf where there is none ([KD3] stage 3, [BLOG-KERNEL],
    READING-4, READING-12).  S_shared, vis: [R, n_C1]."""
    S_shared = np.asarray(S_shared, np.float64)
    R, n_c1 = S_shared.shape
    out = np.full((R, n_blk), -np.inf)
    for blk in range(n_blk):
        win = kernels_of_block(blk, n_c1, prob)
        if not win:
            continue
        w = np.array(win)
        out[:, blk] = np.where(vis[:, w], S_shared[:, w], -np.inf).max(axis=1)
    return out


def select_blocks(S_cmp_row, p: int, prob: Problem) -> np.ndarray:
    """I(p) = I_init u I_local(p) u top-k(p), ascending ([KD2], [BLOG-KERNEL]).

    b_p = floor(p/B); I_init = {0..N_init-1}; I_local = {b_p-N_local+1..b_p}
    (READING-7); candidates C = {0..b_p} minus both; top-k = the first
    min(k, |C|) candidates ordered by (S^cmp descending, block ascending)
    (READING-6, READING-9).  Only causal blocks are ever candidates.
    """
    b_p = p // prob.B
    init = set(range(min(prob.N_init, b_p + 1)))
    local = set(range(max(0, b_p - prob.N_local + 1), b_p + 1))
    cand = np.array([blk for blk in range(b_p + 1) if blk not in init and blk not in local],
                    dtype=np.int64)
    top: list[int] = []
    if cand.size:
        sc = np.asarray(S_cmp_row, np.float64)[cand]
        order = np.lexsort((cand, -sc))          # primary -score, then index
        top = cand[order[:min(prob.k, cand.size)]].tolist()
    return np.array(sorted(init | local | set(top)), dtype=np.int64)


def dense_switch(n_kv: int, prob: Problem) -> bool:
    """True when the whole causal context fits in the block budget, so the
    sparse path IS dense attention ([FLOW], [BLOG-KERNEL], READING-8)."""
    return -(-n_kv // prob.B) <= prob.budget


# --------------------------------------------------------------------------
# Attention over the attended tokens ([APPA])
# --------------------------------------------------------------------------


def attended_tokens(blocks, p: int, prob: Problem) -> np.ndarray:
    """T(p) = {t <= p : floor(t/B) in I(p)} ([APPA]: only visible blocks)."""
    toks = [np.arange(blk * prob.B, min(blk * prob.B + prob.B, p + 1)) for blk in blocks]
    toks = [t for t in toks if t.size]
    return np.concatenate(toks) if toks else np.zeros(0, np.int64)


def attention_rows(Qrows, K, V, token_sets, prob: Problem):
    """Softmax attention of each query row over its own key set.

    Qrows: [R, h_q, d]; K, V: [n_kv, h_kv, d]; token_sets[r][g]: key positions
    for row r and group g (shared by the G heads of the group, [BLOG-SHARE]).
    O[r, h] = sum_t softmax_t(scale * q.k_t) v_t, lse[r, h] = log sum_t exp(.)
    Returns (O fp64 unrounded [R, h_q, d], lse [R, h_q]).
    """
    Qrows = np.asarray(Qrows, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    R = Qrows.shape[0]
    G = prob.G
    O = np.zeros((R, prob.h_q, prob.d))
    lse = np.full((R, prob.h_q), -np.inf)
    for r in range(R):
        for g in range(prob.h_kv):
            T = np.asarray(token_sets[r][g], dtype=np.int64)
            if T.size == 0:
                continue
            z = (Qrows[r, g * G:(g + 1) * G] @ K[T, g].T) * prob.sm_scale   # [G, |T|]
            mx = z.max(axis=1, keepdims=True)
            e = np.exp(z - mx)
            ssum = e.sum(axis=1, keepdims=True)
            O[r, g * G:(g + 1) * G] = (e / ssum) @ V[T, g]
            lse[r, g * G:(g + 1) * G] = (mx + np.log(ssum))[:, 0]
    return O, lse

def attention_rows_backward(Qrows, K, V, token_sets, dO, prob: Problem, q_index=None):
    """Gradients of the block-sparse attention with the selected sets held
    fixed ([BLOG-TRAIN], READING-17), for the rows of one sequence.

    Qrows, dO: [R, h_q, d]; K, V: [n_kv, h_kv, d]; token_sets[r][g] as for
    attention_rows.  For each row and head, with z_t = scale * q . k_t over
    t in T(p), P = softmax(z) and O = sum_t P_t v_t:
        dP_t = dO . v_t,   D = sum_t P_t dP_t (= dO . O),   dZ_t = P_t (dP_t - D)
        dq   = scale * sum_t dZ_t k_t
        dk_t += scale * dZ_t q,   dv_t += P_t dO
    dK and dV sum over every row given (rows of other queries add nothing).
    Returns (dQ [R, h_q, d], dK [n_kv, h_kv, d], dV [n_kv, h_kv, d]) in fp64.
    """
    Qrows = np.asarray(Qrows, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    R = Qrows.shape[0]
    G = prob.G
    sc = prob.sm_scale
    dQ = np.zeros_like(Qrows)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for r in range(R):
        for g in range(prob.h_kv):
            T = np.asarray(token_sets[r][g], dtype=np.int64)
            if T.size == 0:
                continue
            q = Qrows[r, g * G:(g + 1) * G]                  # [G, d]
            do = dO[r, g * G:(g + 1) * G]                    # [G, d]
            Kt, Vt = K[T, g], V[T, g]                        # [|T|, d]
            z = (q @ Kt.T) * sc                              # [G, |T|]
            e = np.exp(z - z.max(axis=1, keepdims=True))
            P = e / e.sum(axis=1, keepdims=True)
            dP = do @ Vt.T                                   # [G, |T|]
            Dr = (P * dP).sum(axis=1, keepdims=True)
            dZ = P * (dP - Dr)
            dQ[r, g * G:(g + 1) * G] = sc * (dZ @ Kt)
            np.add.at(dK[:, g], T, sc * (dZ.T @ q))
            np.add.at(dV[:, g], T, P.T @ do)
    return dQ, dK, dV


# --------------------------------------------------------------------------
# Whole forward path for selected query rows of one sequence
# --------------------------------------------------------------------------


def forward_rows(Q, K, V, rows, prob: Problem, q_pos0: int = 0, Kc1=None,
                 mode: str = "auto", Kc2=None):
    """Forward path for query rows ``rows`` (indices into Q's token axis).

    Q: [n_q, h_q, d]; K, V: [n_kv, h_kv, d] (one sequence, I/O-dtype values).
    Query row t sits at absolute position p = q_pos0 + t.
    mode: "auto" (dense when dense_switch), "sparse" or "dense".
    Returns a dict: Kc1, lse_sel, S_shared, S_cmp, sets [R][h_kv] (block
    lists), O (rounded to the I/O dtype), O64 (unrounded), lse, mode.
    """
    K = np.asarray(K, np.float64)
    n_kv = K.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    q_pos = q_pos0 + rows
    Qrows = np.asarray(Q, np.float64)[rows]
    if mode == "auto":
        mode = "dense" if dense_switch(n_kv, prob) else "sparse"
    out = {"mode": mode}
    if mode == "dense":
        sets = [[np.arange(p // prob.B + 1) for _ in range(prob.h_kv)] for p in q_pos]
    else:
        if Kc1 is None:
            Kc1 = compress_k(K[None], prob)[0]
        if prob.lse_approx and Kc2 is None:
            Kc2 = compress_k2(K[None], prob)[0]
        lse_sel, S_shared, S_cmp = selection_scores(Qrows, Kc1, q_pos, n_kv, prob, Kc2=Kc2)
        sets = [[select_blocks(S_cmp[r, g], int(p), prob) for g in range(prob.h_kv)]
                for r, p in enumerate(q_pos)]
        out.update(Kc1=Kc1, lse_sel=lse_sel, S_shared=S_shared, S_cmp=S_cmp)
    token_sets = [[attended_tokens(sets[r][g], int(p), prob) for g in range(prob.h_kv)]
                  for r, p in enumerate(q_pos)]
    O64, lse = attention_rows(Qrows, K, V, token_sets, prob)
    out.update(sets=sets, O64=O64, O=round_to_io(O64, prob.io), lse=lse)
    return out


# --------------------------------------------------------------------------
# Varlen batches and paged caches (serving decode)
# --------------------------------------------------------------------------


def gather_paged(pool, table_row, n_tokens: int, B: int) -> np.ndarray:
    """The first n_tokens token rows of one sequence kept in a paged cache
    (READING-18): token u lives in page table_row[u // B], row u % B.  Pure
    indexing, no arithmetic.  pool: [n_pages, B, ...]."""
    pool = np.asarray(pool)
    u = np.arange(n_tokens)
    pages = np.asarray(table_row)[u // B]
    return pool[pages, u % B]


def decode_varlen(Q, K, V, seq_lens, prob: Problem, block_table=None, mode: str = "auto"):
    """A varlen batch ([BLOG-GRAN], READING-18): sequence i holds seq_lens[i]
    tokens and its n_q = Q.shape[1] query tokens are its last ones; each
    sequence is the problem of forward_rows on its own keys, with
    q_pos0 = seq_lens[i] - n_q.

    Q: [b, n_q, h_q, d].  K, V: [b, kv_cap, h_kv, d] (contiguous) or, with
    block_table [b, max_blocks], page pools [n_pages, B, h_kv, d].
    Returns one forward_rows dict per sequence."""
    Q = np.asarray(Q)
    n_q = Q.shape[1]
    out = []
    for i, L in enumerate(int(x) for x in seq_lens):
        if block_table is None:
            Ki, Vi = np.asarray(K)[i, :L], np.asarray(V)[i, :L]
        else:
            Ki = gather_paged(K, block_table[i], L, prob.B)
            Vi = gather_paged(V, block_table[i], L, prob.B)
        out.append(forward_rows(Q[i], Ki, Vi, np.arange(n_q), prob, q_pos0=L - n_q, mode=mode))
    return out
