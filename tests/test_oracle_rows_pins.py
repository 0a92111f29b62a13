"""Pins for the oracle's row-ragged grouped GEMM (forward / data gradient), CPU only.

    out[m][n] = sum_{c < C} dec(X[m][c], sX[m][c/32]) * dec(W[g][n][c], sW[g][n][c/32]),
    m in [start_g, end_g)

Every check compares the oracle with something other than itself:
  - exact rational brute force on tiny random problems (row boundaries at any
    row, empty experts, padding rows), with the exact decoder of
    test_oracle_pins (written from the OCP E4M3FN / E8M0 definitions);
  - the XLA blog's ragged_dot example (inputs printed on the page) in its
    forward form, computed exactly here;
  - invariants: a single expert is a dense product (numpy), a +1 weight-scale
    exponent doubles exactly the rows of that expert, splitting an expert into
    two with the same weights changes nothing, garbage past the last expert is
    never read, and one expert covering the contraction in the weight-gradient
    oracle (pinned on its own) gives the same numbers;
  - the selected-point evaluator against the full one.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from test_oracle_pins import E4M3_Q, FINITE_CODES


def exact_rows(X, sX, W, sW, offs):
    """out as exact rationals (None for rows past the last expert)."""
    M, C = X.shape
    E, Nw, _ = W.shape
    out = [[None] * Nw for _ in range(M)]
    start = 0
    for g in range(E):
        end = int(offs[g])
        for m in range(start, end):
            for n in range(Nw):
                acc = Fraction(0)
                for c in range(C):
                    a = E4M3_Q[X[m, c]] * Fraction(2) ** (int(sX[m, c // 32]) - 127)
                    b = E4M3_Q[W[g, n, c]] * Fraction(2) ** (int(sW[g, n, c // 32]) - 127)
                    acc += a * b
                out[m][n] = acc
        start = end
    return out


def rand_rows(rng, E, M, C, Nw, scale_lo=110, scale_hi=144, empty_prob=0.25):
    X = rng.choice(FINITE_CODES, (M, C))
    W = rng.choice(FINITE_CODES, (E, Nw, C))
    sX = rng.integers(scale_lo, scale_hi + 1, (M, C // 32)).astype(np.uint8)
    sW = rng.integers(scale_lo, scale_hi + 1, (E, Nw, C // 32)).astype(np.uint8)
    cuts = np.sort(rng.integers(0, M + 1, E))  # any row boundary, padding rows after the last
    for g in range(1, E):
        if rng.random() < empty_prob:
            cuts[g] = cuts[g - 1]
    return X, sX, W, sW, np.sort(cuts).astype(np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_rows_brute_force_exact(seed):
    rng = np.random.default_rng(9100 + seed)
    E = int(rng.integers(1, 4))
    M = int(rng.integers(1, 24))
    C = 32 * int(rng.integers(1, 4))
    Nw = int(rng.integers(1, 6))
    X, sX, W, sW, offs = rand_rows(rng, E, M, C, Nw)
    got = oracle.rows_f64(X, sX, W, sW, offs)
    ref = exact_rows(X, sX, W, sW, offs)
    for m in range(M):
        for n in range(Nw):
            if ref[m][n] is None:
                assert np.isnan(got[m, n]), (m, n)
                continue
            g = int(np.searchsorted(offs, m, side="right"))
            absum = sum(abs(E4M3_Q[X[m, c]] * E4M3_Q[W[g, n, c]]) *
                        Fraction(2) ** (int(sX[m, c // 32]) + int(sW[g, n, c // 32]) - 254) for c in range(C))
            assert abs(Fraction(got[m, n]) - ref[m][n]) <= C * Fraction(1, 2 ** 53) * absum


def test_rows_xla_ragged_dot_forward_example(golden_dir):
    with open(os.path.join(golden_dir, "xla_ragged_dot_example.json")) as f:
        ex = json.load(f)
    lhs = [[Fraction(v) for v in row] for row in ex["lhs"]]  # [5, 4]: tokens x contraction
    rhs = [[[Fraction(v) for v in row] for row in w] for w in ex["rhs"]]  # [2, 4, 3]: expert, contraction, out
    sizes = ex["group_sizes"]
    Mtok, C, Nw = len(lhs), len(lhs[0]), len(rhs[0][0])
    gid = [g for g, s in enumerate(sizes) for _ in range(s)]
    exact = [[sum(lhs[m][c] * rhs[gid[m]][c][n] for c in range(C)) for n in range(Nw)] for m in range(Mtok)]
    # contraction-contiguous weights: Wd[g][n][c] = rhs[g][c][n]
    Xd = np.array([[float(v) for v in r] for r in lhs])
    Wd = np.array([[[float(rhs[g][c][n]) for c in range(C)] for n in range(Nw)] for g in range(len(sizes))])
    start, end = oracle.windows(np.cumsum(sizes).astype(np.int32), Mtok, align=1)
    got = oracle.rows_contract_f64(Xd, Wd, start, end)
    for m in range(Mtok):
        for n in range(Nw):
            assert abs(Fraction(got[m, n]) - exact[m][n]) <= Fraction(1, 10 ** 14)
    np.testing.assert_allclose(got, [[2.05, 1.5, 0.1], [0.3, 1.05, 0.52], [2.1, 2.1, 1.1], [0.34, 0.34, 0.34],
                                     [0.7, 0.7, 0.7]], rtol=0, atol=1e-14)


@pytest.fixture(scope="module")
def mid_rows():
    rng = np.random.default_rng(9200)
    M, C, Nw, E = 200, 160, 24, 4
    X = rng.choice(FINITE_CODES, (M, C))
    W = rng.choice(FINITE_CODES, (E, Nw, C))
    sX = rng.integers(118, 136, (M, C // 32)).astype(np.uint8)
    sW = rng.integers(118, 136, (E, Nw, C // 32)).astype(np.uint8)
    offs = np.array([37, 37, 120, 181], np.int32)  # an empty expert, unaligned ends, 19 padding rows
    return X, sX, W, sW, offs


def test_rows_single_expert_is_dense_matmul():
    rng = np.random.default_rng(9300)
    M, C, Nw = 48, 96, 16
    X = rng.choice(FINITE_CODES, (M, C))
    W = rng.choice(FINITE_CODES, (1, Nw, C))
    sX = rng.integers(120, 134, (M, C // 32)).astype(np.uint8)
    sW = rng.integers(120, 134, (1, Nw, C // 32)).astype(np.uint8)
    got = oracle.rows_f64(X, sX, W, sW, np.array([M], np.int32))
    Xd = oracle.decode_plane(X, sX)
    Wd = oracle.decode_plane(W[0], sW[0])
    np.testing.assert_allclose(got, Xd @ Wd.T, rtol=1e-13, atol=1e-300)


def test_rows_weight_scale_shift_doubles_exactly(mid_rows):
    X, sX, W, sW, offs = mid_rows
    base = oracle.rows_f64(X, sX, W, sW, offs)
    sW2 = sW.copy()
    sW2[2] += 1
    got = oracle.rows_f64(X, sX, W, sW2, offs)
    g2 = slice(int(offs[1]), int(offs[2]))
    np.testing.assert_array_equal(got[g2], 2.0 * base[g2])
    rest = np.ones(X.shape[0], bool)
    rest[g2] = False
    np.testing.assert_array_equal(got[rest], base[rest])


def test_rows_expert_split_with_same_weights(mid_rows):
    X, sX, W, sW, offs = mid_rows
    base = oracle.rows_f64(X, sX, W, sW, offs)
    # expert 3 (rows 120..180) split at row 150 into two experts with its weights
    W2 = np.concatenate([W, W[3:4]], 0)
    sW2 = np.concatenate([sW, sW[3:4]], 0)
    offs2 = np.array([37, 37, 120, 150, 181], np.int32)
    got = oracle.rows_f64(X, sX, W2, sW2, offs2)
    np.testing.assert_array_equal(got, base)


def test_rows_padding_garbage_ignored(mid_rows):
    X, sX, W, sW, offs = mid_rows
    base = oracle.rows_f64(X, sX, W, sW, offs)
    X2, sX2 = X.copy(), sX.copy()
    X2[int(offs[-1]):] = 0x7F  # NaN codes
    sX2[int(offs[-1]):] = 0xFF  # NaN scales
    got = oracle.rows_f64(X2, sX2, W, sW, offs)
    np.testing.assert_array_equal(got, base)
    assert np.isnan(got[int(offs[-1]):]).all()


def test_rows_matches_weight_gradient_oracle_on_one_expert():
    """One expert covering the whole contraction: the weight-gradient oracle
    with A = X [M rows, C tokens], B = W[0] [Nw rows, C tokens] computes the
    same sums (its own pins are independent of this function)."""
    rng = np.random.default_rng(9400)
    M, C, Nw = 20, 128, 12
    X = rng.choice(FINITE_CODES, (M, C))
    W = rng.choice(FINITE_CODES, (1, Nw, C))
    sX = rng.integers(120, 134, (M, C // 32)).astype(np.uint8)
    sW = rng.integers(120, 134, (1, Nw, C // 32)).astype(np.uint8)
    got = oracle.rows_f64(X, sX, W, sW, np.array([M], np.int32))
    dw = oracle.wgrad_f64(X, sX, W[0], sW[0], np.array([C], np.int32))
    np.testing.assert_array_equal(got, dw[0])


def test_rows_points_match_full(mid_rows):
    X, sX, W, sW, offs = mid_rows
    full = oracle.rows_f64(X, sX, W, sW, offs)
    rng = np.random.default_rng(9500)
    m = rng.integers(0, X.shape[0], 300)
    n = rng.integers(0, W.shape[1], 300)
    pts = oracle.rows_points(X, sX, W, sW, offs, m, n)
    np.testing.assert_array_equal(np.isnan(pts), np.isnan(full[m, n]))
    ok = ~np.isnan(pts)
    np.testing.assert_array_equal(pts[ok], full[m, n][ok])


def test_rows_malformed_offs_rejected(mid_rows):
    X, sX, W, sW, _ = mid_rows
    for bad in ([50, 40, 100, 120], [10, 20, 30, 201]):  # decreasing, past M
        with pytest.raises(ValueError):
            oracle.rows_f64(X, sX, W, sW, np.array(bad, np.int32))
