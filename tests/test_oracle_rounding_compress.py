"""Pins for the oracle's rounding and stage-1 compression (CPU only).

Rounding is pinned to torch's own fp32->bf16 cast (round to nearest even) and to
an exact-rational brute force; K^C1 to a closed form and to exact rational means.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import Problem, compress_k, n_kernels, round_to_bf16, round_to_io
from oracle.infv2_oracle import _round_fraction


def _bf16_neighbours_nearest(fr: Fraction) -> float:
    """Brute force: nearest bf16 to an exact rational, ties to the even bit
    pattern, by testing the bf16 values around a first guess."""
    guess = torch.tensor([float(fr)], dtype=torch.float32).to(torch.bfloat16)
    bits = int(guess.view(torch.int16).item()) & 0xFFFF
    best = None
    for db in (-2, -1, 0, 1, 2):
        b = (bits + db) & 0xFFFF
        val = torch.tensor([b if b < 0x8000 else b - 0x10000], dtype=torch.int16) \
            .view(torch.bfloat16).float().item()
        if not np.isfinite(val):
            continue
        dist = abs(Fraction(val) - fr)
        key = (dist, b & 1)
        if best is None or key < best[0]:
            best = (key, val)
    return best[1]


def test_bf16_matches_torch_cast_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(50000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-38).astype(np.float32),     # subnormal range
        (rng.standard_normal(5000) * 1e37).astype(np.float32),      # near the top
        np.array([0.0, -0.0, 3.3895314e38, -3.3895314e38, 1.0, 1.00390625], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = round_to_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_single_rounding_not_double():
    # 1 + 2^-8 + 2^-40 lies above the midpoint between 1 and 1+2^-7: direct
    # rounding goes up.  Going through fp32 first would drop 2^-40, land on the
    # midpoint and round to even (1.0).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert round_to_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    # exact midpoints round to even
    assert round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_rational_rounding_agrees_with_fp64_rounding():
    rng = np.random.default_rng(1)
    xs = rng.standard_normal(400) * np.exp(rng.uniform(-30, 30, 400))
    for x in xs:
        fr = Fraction(float(x))
        assert _round_fraction(fr, "bf16") == round_to_bf16(np.array([x]))[0]
        assert _round_fraction(fr, "f32") == float(np.float32(x))
        assert _round_fraction(fr, "bf16") == _bf16_neighbours_nearest(fr)


def test_n_kernels_counts_complete_kernels_only():
    # kernel j spans [16j, 16j+31]; it is complete when 16j+31 <= n-1
    for n in range(0, 300):
        brute = sum(1 for j in range(0, 40) if 16 * j + 31 <= n - 1)
        assert n_kernels(n, 32, 16) == brute


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_compress_closed_form_ramp(io):
    # K[t] = t * e0 -> K^C1[j] = mean_{u<32}(16j+u) = 16j + 15.5, rounded once.
    n = 256
    prob = Problem(G=1, h_kv=1, d=4, io=io)
    K = np.zeros((1, n, 1, 4))
    K[0, :, 0, 0] = np.arange(n)
    kc = compress_k(K, prob)
    n_c1 = n_kernels(n, 32, 16)
    exact = torch.tensor([16.0 * j + 15.5 for j in range(n_c1)], dtype=torch.float32)
    ref = exact.to(torch.bfloat16).double().numpy() if io == "bf16" else exact.double().numpy()
    np.testing.assert_array_equal(kc[0, 0, :, 0], ref)
    assert np.all(kc[0, 0, :, 1:] == 0)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_compress_matches_exact_rational_mean(io):
    rng = np.random.default_rng(2)
    n, h_kv, d = 80, 2, 3
    prob = Problem(G=1, h_kv=h_kv, d=d, io=io)
    K = round_to_io(rng.standard_normal((1, n, h_kv, d)) * 3, io)
    kc = compress_k(K, prob)
    for j in range(n_kernels(n, 32, 16)):
        for g in range(h_kv):
            for di in range(d):
                fr = sum(Fraction(float(v)) for v in K[0, 16 * j:16 * j + 32, g, di]) / 32
                want = _bf16_neighbours_nearest(fr) if io == "bf16" else float(np.float32(float(fr)))
                if io == "f32":
                    # float(fr) is the nearest fp64; confirm no tie ambiguity by
                    # also checking the exact-rational rounder
                    assert want == _round_fraction(fr, "f32")
                assert kc[0, g, j, di] == want


def test_compress_inexact_fp64_sum_is_redone_exactly():
    # fp32 inputs 1, 2^-24 and 2^-80 in one kernel: the fp64 running sum drops
    # 2^-80, which would land (1+2^-24)/32 exactly on an fp32 midpoint and
    # round down to even.  The exact value lies above it: round up.
    prob = Problem(G=1, h_kv=1, d=1, io="f32")
    K = np.zeros((1, 32, 1, 1))
    K[0, 0, 0, 0] = 1.0
    K[0, 1, 0, 0] = 2.0 ** -24
    K[0, 2, 0, 0] = 2.0 ** -80
    kc = compress_k(K, prob)
    assert kc[0, 0, 0, 0] == (1.0 + 2.0 ** -23) / 32
