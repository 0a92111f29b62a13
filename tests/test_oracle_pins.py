"""Pins for the oracle's weight-gradient contraction (CPU only).

Every check here compares the oracle with something other than itself:
  - a hand-computed two-expert case (tests/golden/hand_two_expert.json);
  - exact rational brute force on tiny random problems, with this file's own
    decoder written from the OCP E4M3FN / E8M0 definitions;
  - invariants of the definition (empty expert, exact doubling under a +1
    scale exponent, single-block linearity, single expert = dense product via
    numpy, operand swap = transpose, expert split = sum, padding garbage
    ignored);
  - the XLA blog's ragged_dot example (inputs printed on the page) in its
    weight-gradient form, computed exactly here, plus the adjoint identity;
  - the XLA blog's group-lookup table (Table 2).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

# ----------------------------------------------------------------------------
# an independent exact decoder (rationals), from the format definitions
# ----------------------------------------------------------------------------


def _e4m3_q(code):
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    assert not (e == 0xF and m == 0x7)
    if e == 0:
        return s * Fraction(m, 512)
    return s * Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


E4M3_Q = [None if (c & 0x7F) == 0x7F else _e4m3_q(c) for c in range(256)]
FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def exact_wgrad(A, sA, B, sB, offs):
    """dW as exact rationals, straight from the definition."""
    N, M = A.shape
    K = B.shape[0]
    E = len(offs)
    out = [[[Fraction(0)] * K for _ in range(N)] for _ in range(E)]
    start = 0
    for g in range(E):
        end = int(offs[g])
        for n in range(N):
            for k in range(K):
                acc = Fraction(0)
                for m in range(start, end):
                    a = E4M3_Q[A[n, m]] * Fraction(2) ** (int(sA[n, m // 32]) - 127)
                    b = E4M3_Q[B[k, m]] * Fraction(2) ** (int(sB[k, m // 32]) - 127)
                    acc += a * b
                out[g][n][k] = acc
        start = end
    return out


def rand_problem(rng, E, N, K, M, scale_lo=110, scale_hi=144, empty_prob=0.25):
    A = rng.choice(FINITE_CODES, (N, M))
    B = rng.choice(FINITE_CODES, (K, M))
    sA = rng.integers(scale_lo, scale_hi + 1, (N, M // 32)).astype(np.uint8)
    sB = rng.integers(scale_lo, scale_hi + 1, (K, M // 32)).astype(np.uint8)
    # random 32-aligned cumulative ends with possible empties and unused padding
    units = M // 32
    cuts = np.sort(rng.integers(0, units + 1, E))
    for g in range(E):
        if rng.random() < empty_prob and g > 0:
            cuts[g] = cuts[g - 1]
    offs = (np.sort(cuts) * 32).astype(np.int32)
    return A, sA, B, sB, offs


# ----------------------------------------------------------------------------
# hand-computed case
# ----------------------------------------------------------------------------


def _load_hand(golden_dir):
    with open(os.path.join(golden_dir, "hand_two_expert.json")) as f:
        h = json.load(f)
    M = h["M"]

    def rows(spec, nrows):
        out = np.zeros((nrows, M), np.uint8)
        for r, row in enumerate(spec):
            for lo, hi, code in row["codes"]:
                out[r, lo:hi] = int(code, 16)
        return out

    A = rows(h["A_rows"], h["N"])
    B = rows(h["B_rows"], h["K"])
    sA = np.array(h["sA"], np.uint8)
    sB = np.array(h["sB"], np.uint8)
    offs = np.array(h["offs"], np.int32)
    return h, A, sA, B, sB, offs


def test_hand_computed_case(golden_dir):
    h, A, sA, B, sB, offs = _load_hand(golden_dir)
    out = oracle.wgrad_f64(A, sA, B, sB, offs)
    assert out.tolist() == h["expected"]
    bits = oracle.to_bf16_bits(out)
    assert [[["0x%04X" % int(x) for x in r] for r in g] for g in bits] == h["expected_bf16"]
    # points path agrees
    g, n, k = np.meshgrid(np.arange(2), np.arange(2), np.arange(1), indexing="ij")
    pts = oracle.wgrad_points(A, sA, B, sB, offs, g.ravel(), n.ravel(), k.ravel())
    assert pts.tolist() == out.ravel().tolist()


# ----------------------------------------------------------------------------
# exact brute force
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_exact(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(1, 5))
    N = int(rng.integers(1, 9))
    K = int(rng.integers(1, 9))
    M = 32 * int(rng.integers(1, 9))
    A, sA, B, sB, offs = rand_problem(rng, E, N, K, M)
    got = oracle.wgrad_f64(A, sA, B, sB, offs)
    ref = exact_wgrad(A, sA, B, sB, offs)
    start = 0
    for g in range(E):
        length = int(offs[g]) - start
        for n in range(N):
            for k in range(K):
                r = ref[g][n][k]
                # bound on fp64 accumulation error: len * 2^-53 * sum |terms|
                absum = sum(abs(E4M3_Q[A[n, m]] * E4M3_Q[B[k, m]]) *
                            Fraction(2) ** (int(sA[n, m // 32]) + int(sB[k, m // 32]) - 254)
                            for m in range(start, int(offs[g])))
                assert abs(Fraction(got[g, n, k]) - r) <= length * Fraction(1, 2 ** 53) * absum
        start = int(offs[g])


def test_points_match_full():
    rng = np.random.default_rng(5)
    A, sA, B, sB, offs = rand_problem(rng, 3, 6, 5, 256, empty_prob=0.0)
    full = oracle.wgrad_f64(A, sA, B, sB, offs)
    g, n, k = [x.ravel() for x in np.meshgrid(np.arange(3), np.arange(6), np.arange(5), indexing="ij")]
    pts = oracle.wgrad_points(A, sA, B, sB, offs, g, n, k)
    np.testing.assert_array_equal(pts, full.ravel())


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------


@pytest.fixture(scope="module")
def mid_problem():
    rng = np.random.default_rng(2024)
    E, N, K, M = 4, 24, 20, 512
    A = rng.choice(FINITE_CODES, (N, M))
    B = rng.choice(FINITE_CODES, (K, M))
    sA = rng.integers(118, 136, (N, M // 32)).astype(np.uint8)
    sB = rng.integers(118, 136, (K, M // 32)).astype(np.uint8)
    offs = np.array([96, 96, 256, 448], np.int32)  # one empty expert, 64 tokens of padding
    return A, sA, B, sB, offs


def test_empty_expert_is_exact_zero(mid_problem):
    A, sA, B, sB, offs = mid_problem
    out = oracle.wgrad_f64(A, sA, B, sB, offs)
    assert (out[1] == 0).all() and not np.signbit(out[1]).any()
    assert (out[0] != 0).any() and (out[2] != 0).any()


def test_scale_exponent_shift_doubles_exactly(mid_problem):
    A, sA, B, sB, offs = mid_problem
    base = oracle.wgrad_f64(A, sA, B, sB, offs)
    g, lo, hi = 2, 96, 256  # expert 2 owns blocks 3..7
    sA2 = sA.copy()
    sA2[:, lo // 32:hi // 32] += 1
    out = oracle.wgrad_f64(A, sA2, B, sB, offs)
    np.testing.assert_array_equal(out[g], 2.0 * base[g])
    for h in (0, 1, 3):
        np.testing.assert_array_equal(out[h], base[h])
    # the same holds on the B side
    sB2 = sB.copy()
    sB2[:, lo // 32:hi // 32] += 1
    out = oracle.wgrad_f64(A, sA, B, sB2, offs)
    np.testing.assert_array_equal(out[g], 2.0 * base[g])


def test_single_block_linearity(mid_problem):
    A, sA, B, sB, offs = mid_problem
    base = oracle.wgrad_f64(A, sA, B, sB, offs)
    n, blk, g = 7, 5, 2  # block 5 = tokens [160,192) lies in expert 2
    sA2 = sA.copy()
    sA2[n, blk] += 1
    out = oracle.wgrad_f64(A, sA2, B, sB, offs)
    # contribution of that block to row n, from an independent fp64 evaluation
    a = np.array([float(E4M3_Q[c]) for c in A[n, 32 * blk:32 * blk + 32]]) * 2.0 ** (int(sA[n, blk]) - 127)
    contrib = np.array([sum(a[i] * float(E4M3_Q[B[k, 32 * blk + i]]) * 2.0 ** (int(sB[k, blk]) - 127)
                            for i in range(32)) for k in range(B.shape[0])])
    diff = out[g, n] - base[g, n]
    np.testing.assert_allclose(diff, contrib, rtol=0, atol=4 * np.finfo(float).eps * np.abs(base[g, n]).max() + 1e-300)
    mask = np.ones(out.shape, bool)
    mask[g, n] = False
    np.testing.assert_array_equal(out[mask], base[mask])


def _decode_indep(q, s):
    lut = np.array([np.nan if v is None else float(v) for v in E4M3_Q])
    rows, M = q.shape
    return lut[q] * np.exp2(np.repeat(s.astype(np.float64), 32, axis=1) - 127.0)


def test_single_expert_is_dense_matmul():
    rng = np.random.default_rng(11)
    N, K, M = 40, 36, 640
    A = rng.choice(FINITE_CODES, (N, M))
    B = rng.choice(FINITE_CODES, (K, M))
    sA = rng.integers(120, 134, (N, M // 32)).astype(np.uint8)
    sB = rng.integers(120, 134, (K, M // 32)).astype(np.uint8)
    out = oracle.wgrad_f64(A, sA, B, sB, np.array([M], np.int32))
    Ad, Bd = _decode_indep(A, sA), _decode_indep(B, sB)
    ref = Ad @ Bd.T
    bound = M * np.finfo(float).eps * (np.abs(Ad) @ np.abs(Bd).T)
    assert (np.abs(out[0] - ref) <= bound).all()


def test_operand_swap_is_transpose(mid_problem):
    A, sA, B, sB, offs = mid_problem
    out = oracle.wgrad_f64(A, sA, B, sB, offs)
    sw = oracle.wgrad_f64(B, sB, A, sA, offs)
    np.testing.assert_array_equal(sw, out.transpose(0, 2, 1))


def test_expert_split_sums(mid_problem):
    A, sA, B, sB, offs = mid_problem
    out = oracle.wgrad_f64(A, sA, B, sB, offs)
    # split expert 2 ([96,256)) at 160 into two adjacent experts
    offs2 = np.array([96, 96, 160, 256, 448], np.int32)
    out2 = oracle.wgrad_f64(A, sA, B, sB, offs2)
    ref = out[2]
    got = out2[2] + out2[3]
    tol = 8 * np.finfo(float).eps * (np.abs(out2[2]) + np.abs(out2[3]) + np.abs(ref)).max()
    assert np.abs(got - ref).max() <= tol
    np.testing.assert_array_equal(out2[4], out[3])


def test_padding_garbage_ignored(mid_problem):
    A, sA, B, sB, offs = mid_problem
    out = oracle.wgrad_f64(A, sA, B, sB, offs)
    A2, B2, sA2, sB2 = A.copy(), B.copy(), sA.copy(), sB.copy()
    used = int(offs[-1])
    A2[:, used:] = 0x7F  # E4M3 NaN
    B2[:, used:] = 0xFF
    sA2[:, used // 32:] = 0xFF  # E8M0 NaN
    sB2[:, used // 32:] = 0xFF
    out2 = oracle.wgrad_f64(A2, sA2, B2, sB2, offs)
    np.testing.assert_array_equal(out2, out)
    assert np.isfinite(out2).all()


def test_malformed_offs_rejected():
    A = np.zeros((2, 64), np.uint8)
    s = np.full((2, 2), 127, np.uint8)
    for bad in ([64, 32], [16, 64], [32, 96]):  # decreasing, unaligned, past M
        with pytest.raises(ValueError):
            oracle.wgrad_f64(A, s, A, s, np.array(bad, np.int32))


# ----------------------------------------------------------------------------
# the XLA blog's worked examples
# ----------------------------------------------------------------------------


def _dec(x):
    return Fraction(x)


def test_xla_ragged_dot_example_wgrad_form(golden_dir):
    with open(os.path.join(golden_dir, "xla_ragged_dot_example.json")) as f:
        ex = json.load(f)
    lhs = [[_dec(v) for v in row] for row in ex["lhs"]]  # [5, 4] tokens x features
    rhs = [[[_dec(v) for v in row] for row in w] for w in ex["rhs"]]  # [2, 4, 3]
    sizes = ex["group_sizes"]
    Mtok, Kf, Nf = len(lhs), len(lhs[0]), len(rhs[0][0])
    # forward ragged_dot, exactly: Y[m] = lhs[m] @ rhs[g(m)]
    gid = [g for g, s in enumerate(sizes) for _ in range(s)]
    Y = [[sum(lhs[m][k] * rhs[gid[m]][k][n] for k in range(Kf)) for n in range(Nf)] for m in range(Mtok)]
    assert [[float(v) for v in r] for r in Y] == [[2.05, 1.5, 0.1], [0.3, 1.05, 0.52], [2.1, 2.1, 1.1],
                                                  [0.34, 0.34, 0.34], [0.7, 0.7, 0.7]]
    # weight-gradient form with dY = Y and X = lhs: dW[g] = Y[g]^T lhs[g], [3, 4]
    offs = np.cumsum(sizes).astype(np.int32)
    start, end = oracle.windows(offs, Mtok, align=1)
    assert start.tolist() == [0, 3] and end.tolist() == [3, 5]
    At = np.array([[float(Y[m][n]) for m in range(Mtok)] for n in range(Nf)])  # Y^T [3, 5]
    Bt = np.array([[float(lhs[m][k]) for m in range(Mtok)] for k in range(Kf)])  # lhs^T [4, 5]
    got = oracle.ragged_contract_f64(At, Bt, start, end)
    exact = [[[sum(Y[m][n] * lhs[m][k] for m in range(s, e)) for k in range(Kf)] for n in range(Nf)]
             for s, e in zip(start.tolist(), end.tolist())]
    for g in range(2):
        for n in range(Nf):
            for k in range(Kf):
                assert abs(Fraction(got[g, n, k]) - exact[g][n][k]) <= Fraction(1, 10 ** 14)
    np.testing.assert_allclose(got[0], [[4.21, 3.425, 2.25, 4.15], [3.81, 3.9, 2.625, 3.6], [1.304, 1.67, 1.36, 1.2]],
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[1], [[0.384, 0.418, 0.452, 0.486]] * 3, rtol=0, atol=1e-13)
    # adjoint identity: sum_g <dW[g], rhs[g]^T> = <Y, Y>
    lhs_side = sum(got[g, n, k] * float(rhs[g][k][n]) for g in range(2) for n in range(Nf) for k in range(Kf))
    yy = sum(v * v for r in Y for v in r)
    assert float(yy) == pytest.approx(19.7722, abs=1e-12)
    assert lhs_side == pytest.approx(float(yy), abs=1e-12)


def test_xla_group_lookup_table2(golden_dir):
    with open(os.path.join(golden_dir, "xla_group_lookup_table2.json")) as f:
        t = json.load(f)
    offs = np.cumsum(t["group_sizes"]).astype(np.int32)
    start, end = oracle.windows(offs, int(offs[-1]), align=1)
    for row in t["rows"]:
        rs = row["pid_m"] * t["block_m"]
        assert rs == row["row_start"]
        g = max(i for i in range(len(start)) if start[i] <= rs)
        assert start[g] <= rs < end[g]
        assert g == row["group"] and start[g] == row["group_start_row"]
