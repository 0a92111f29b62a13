"""Pins for the oracle's BF16 contracting ragged dot (CPU only).

    dW[g][n][k] = sum_{m in [start_g, end_g)} bf16(A[n][m]) * bf16(B[k][m])

(ROCm blog "Group-GEMM in XLA", the "Contracting" ragged dot and Table 7's
wgrad classes, bfloat16 throughout.)  Compared with things other than the
oracle itself:
  - the bf16 decoder against torch's bfloat16 -> float64 conversion for all
    65,536 bit patterns, and the format's closed forms;
  - exact rational brute force on tiny random problems (unaligned, empty and
    one-token groups), where fp64 accumulation is exact;
  - the XLA blog's small ragged-dot example, rounded to bf16, in its
    weight-gradient form;
  - the MXFP8 weight-gradient oracle, on operands whose decoded MXFP8 values
    are exactly representable in bf16 (the two definitions must then agree
    bit for bit);
  - a rank-one closed form, padding garbage and empty experts, and the
    point evaluator against the full tensor.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def bits_of(x):
    """fp64/fp32 values -> bf16 bit patterns (torch's round-to-nearest-even)."""
    return torch.tensor(np.asarray(x, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_decode_all_patterns():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(1, -1)
    got = oracle.decode_bf16_plane(allbits)[0]
    ref = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()[0]
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    # NaN exactly where the exponent field is 255 and the fraction is not 0
    e = (allbits[0] >> 7) & 0xFF
    f = allbits[0] & 0x7F
    assert (nan == ((e == 0xFF) & (f != 0))).all()
    # closed forms
    assert oracle.bf16(0x3F80) == 1.0 and oracle.bf16(0xBF80) == -1.0
    assert oracle.bf16(0x0001) == 2.0 ** -133 and oracle.bf16(0x0080) == 2.0 ** -126
    assert oracle.bf16(0x7F7F) == (2 - 2.0 ** -7) * 2.0 ** 127
    assert oracle.bf16(0x7F80) == float("inf") and oracle.bf16(0xFF80) == float("-inf")
    assert np.signbit(oracle.bf16(0x8000)) and oracle.bf16(0x8000) == 0.0


def bf16_fraction(b):
    return Fraction(float(oracle.bf16(int(b))))


def random_bf16(rng, shape, emin=-4, emax=4):
    """bf16 values with exponents in [emin, emax] (and some zeros): every sum
    of products of a small problem is then exact in fp64."""
    mant = rng.integers(128, 256, shape)
    ex = rng.integers(emin, emax + 1, shape)
    v = mant.astype(np.float64) / 128.0 * np.exp2(ex) * rng.choice([-1.0, 1.0], shape)
    v[rng.random(shape) < 0.1] = 0.0
    return bits_of(v)


def exact_wgrad(A, B, sizes):
    N, M = A.shape
    K = B.shape[0]
    Af = [[bf16_fraction(A[n, m]) for m in range(M)] for n in range(N)]
    Bf = [[bf16_fraction(B[k, m]) for m in range(M)] for k in range(K)]
    out, s = [], 0
    for L in sizes:
        out.append([[sum((Af[n][m] * Bf[k][m] for m in range(s, s + L)), Fraction(0)) for k in range(K)]
                    for n in range(N)])
        s += L
    return out


@pytest.mark.parametrize("seed", range(4))
def test_bf16_brute_force_exact(seed):
    rng = np.random.default_rng(7100 + seed)
    E, N, K, M = 4, 5, 3, 45
    sizes = [[7, 0, 1, 30], [0, 0, 0, 45], [13, 17, 5, 3], [1, 1, 1, 1]][seed]
    A = random_bf16(rng, (N, M))
    B = random_bf16(rng, (K, M))
    offs = np.cumsum(sizes).astype(np.int32)
    got = oracle.bf16_wgrad_f64(A, B, offs)
    ex = exact_wgrad(A, B, sizes)
    for g in range(E):
        for n in range(N):
            for k in range(K):
                assert Fraction(got[g, n, k]) == ex[g][n][k], (g, n, k)


def test_bf16_xla_example_wgrad_form(golden_dir):
    """The XLA blog's ragged_dot example (lhs (5, 4), rhs (2, 4, 3), group sizes
    [3, 2]), rounded to bf16: dW[g] = Y[g]^T lhs[g] with Y the forward output,
    also rounded to bf16, as the bf16 wgrad classes see it."""
    with open(os.path.join(golden_dir, "xla_ragged_dot_example.json")) as f:
        ex = json.load(f)
    lhs = np.array([[float(v) for v in row] for row in ex["lhs"]])
    rhs = np.array([[[float(v) for v in row] for row in w] for w in ex["rhs"]])
    sizes = ex["group_sizes"]
    gid = np.repeat(np.arange(len(sizes)), sizes)
    lb = bits_of(lhs)
    rb = bits_of(rhs)
    # forward in exact rationals from the bf16 inputs, then rounded to bf16
    Y = np.array([[float(sum(bf16_fraction(lb[m, k]) * bf16_fraction(rb[gid[m], k, n]) for k in range(4)))
                   for n in range(3)] for m in range(5)])
    yb = bits_of(Y)
    got = oracle.bf16_wgrad_f64(np.ascontiguousarray(yb.T), np.ascontiguousarray(lb.T),
                                np.cumsum(sizes).astype(np.int32))
    exact = exact_wgrad(np.ascontiguousarray(yb.T), np.ascontiguousarray(lb.T), sizes)
    for g in range(2):
        for n in range(3):
            for k in range(4):
                assert Fraction(got[g, n, k]) == exact[g][n][k]
    # and close to the unrounded fp64 weight gradient (bf16 keeps 8 bits)
    ref = np.stack([Y[gid == g].T @ lhs[gid == g] for g in range(2)])
    np.testing.assert_allclose(got, ref, rtol=2 ** -5, atol=2 ** -6)


def test_bf16_equals_mxfp8_oracle_on_shared_values():
    """MXFP8 values e4m3 * 2^(s-127) with s in 118..136 are exact in bf16
    (3 fraction bits, exponents far inside bf16's range): encoding each decoded
    value as bf16 must reproduce the MXFP8 oracle's weight gradient bit for bit."""
    rng = np.random.default_rng(7200)
    E, N, K, M = 3, 6, 5, 128
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    A = rng.choice(codes, (N, M))
    B = rng.choice(codes, (K, M))
    sA = rng.integers(118, 137, (N, M // 32)).astype(np.uint8)
    sB = rng.integers(118, 137, (K, M // 32)).astype(np.uint8)
    offs = np.array([32, 32, 96], np.int32)
    mx = oracle.wgrad_f64(A, sA, B, sB, offs)
    Ab = bits_of(oracle.decode_plane(A, sA))
    Bb = bits_of(oracle.decode_plane(B, sB))
    np.testing.assert_array_equal(oracle.decode_bf16_plane(Ab), oracle.decode_plane(A, sA))  # exact encoding
    np.testing.assert_array_equal(oracle.bf16_wgrad_f64(Ab, Bb, offs), mx)


def test_bf16_rank_one_closed_form():
    """A[n][m] = a_n, B[k][m] = b_k on every token: dW[g][n][k] = a_n b_k len_g exactly."""
    rng = np.random.default_rng(7300)
    N, K, M = 7, 9, 300
    a = bits_of(rng.normal(0, 1, N))
    b = bits_of(rng.normal(0, 3, K))
    A = np.repeat(a[:, None], M, axis=1)
    B = np.repeat(b[:, None], M, axis=1)
    sizes = np.array([0, 1, 64, 235])
    got = oracle.bf16_wgrad_f64(A, B, np.cumsum(sizes).astype(np.int32))
    av = oracle.decode_bf16_plane(a[None])[0]
    bv = oracle.decode_bf16_plane(b[None])[0]
    for g, L in enumerate(sizes):
        np.testing.assert_array_equal(got[g], np.outer(av, bv) * L)
    assert not np.signbit(got[0]).any() and (got[0] == 0).all()


def test_bf16_padding_garbage_ignored():
    rng = np.random.default_rng(7400)
    N, K, M = 4, 6, 96
    A = random_bf16(rng, (N, M))
    B = random_bf16(rng, (K, M))
    offs = np.array([16, 48, 80], np.int32)
    base = oracle.bf16_wgrad_f64(A, B, offs)
    A2, B2 = A.copy(), B.copy()
    A2[:, 80:] = 0x7FC0  # NaN
    B2[:, 80:] = 0x7F80  # +inf
    np.testing.assert_array_equal(oracle.bf16_wgrad_f64(A2, B2, offs), base)
    assert np.isfinite(base).all()


def test_bf16_points_match_full():
    cfg = W.make_bf16(5, 40, 24, 320, [64, 0, 100, 48, 92], seed=7500)
    A = cfg["A"].view(torch.int16).numpy().view(np.uint16)
    B = cfg["B"].view(torch.int16).numpy().view(np.uint16)
    offs = cfg["offs"].numpy()
    full = oracle.bf16_wgrad_f64(A, B, offs)
    rng = np.random.default_rng(7501)
    g = rng.integers(0, 5, 300)
    n = rng.integers(0, 40, 300)
    k = rng.integers(0, 24, 300)
    np.testing.assert_array_equal(oracle.bf16_wgrad_points(A, B, offs, g, n, k), full[g, n, k])


def test_bf16_against_float64_matmul():
    """Each expert's slab equals the fp64 matrix product of its decoded token
    slices (a library routine; different summation order, so to fp64 rounding)."""
    cfg = W.make_bf16(3, 33, 17, 256, [100, 0, 120], seed=7600, std=(1.0, 0.5))
    A = cfg["A"].view(torch.int16).numpy().view(np.uint16)
    B = cfg["B"].view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_wgrad_f64(A, B, cfg["offs"].numpy())
    Ad = cfg["A"].to(torch.float64).numpy()
    Bd = cfg["B"].to(torch.float64).numpy()
    for g, (s, e) in enumerate([(0, 100), (100, 100), (100, 220)]):
        np.testing.assert_allclose(got[g], Ad[:, s:e] @ Bd[:, s:e].T, rtol=1e-12, atol=1e-12)


def test_bf16_rejects_malformed_offs():
    A = np.zeros((2, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.bf16_wgrad_f64(A, A, np.array([4, 2], np.int32))  # decreasing
    with pytest.raises(ValueError):
        oracle.bf16_wgrad_f64(A, A, np.array([4, 9], np.int32))  # past M
    oracle.bf16_wgrad_f64(A, A, np.array([3, 3, 5], np.int32))  # unaligned is fine
