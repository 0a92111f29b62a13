"""Pins for the oracle's token-axis MXFP8 quantiser (CPU only).

    s        = clamp(floor(log2 amax) - 8 + 127, 0, 254)   (127 when amax = 0)
    q[h][m]  = E4M3FN_RNE_sat(x[m][h] / 2^(s - 127))         (0 past `used`)

Compared with things other than the oracle itself:
  - an exact rational re-implementation here (scale from the exact binary
    exponent, E4M3 rounding by enumerating the exact code values, ties to the
    even code), on random bf16 blocks that include constructed ties,
    saturation-range values, subnormal-range values and zeros;
  - the input generator's quantiser (workloads.quantize_rows, a separate
    torch implementation used only to make test inputs), transposed;
  - closed forms (a power-of-two amax, an all-zero block, padding tokens) and
    the sign symmetry;
  - the format's error bound on dequantisation.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from test_oracle_pins import E4M3_Q

# the non-negative finite codes 0x00..0x7E as exact rationals
POS = [(c, E4M3_Q[c]) for c in range(0x7F)]


def bf16_value(bits):
    return Fraction(np.array([int(bits) << 16], np.uint32).view(np.float32)[0].item())


def floor_log2(f):
    """floor(log2 f) for a positive rational, exactly."""
    e = f.numerator.bit_length() - f.denominator.bit_length()
    while Fraction(2) ** e > f:
        e -= 1
    while Fraction(2) ** (e + 1) <= f:
        e += 1
    return e


def rne_e4m3(y):
    a = abs(y)
    if a > 448:
        c = 0x7E
    else:
        best = None
        for c_, v in POS:
            d = abs(v - a)
            if best is None or d < best[0] or (d == best[0] and c_ % 2 == 0 and best[1] % 2 == 1):
                best = (d, c_)
        c = best[1]
    return (c | 0x80) if (y < 0 and c != 0) else c


def exact_quantize(bits, used):
    M, H = bits.shape
    q = np.zeros((H, M), np.uint8)
    s = np.zeros((H, M // 32), np.uint8)
    for h in range(H):
        for b in range(M // 32):
            vals = [bf16_value(bits[m, h]) if m < used else Fraction(0) for m in range(32 * b, 32 * b + 32)]
            amax = max(abs(v) for v in vals)
            sb = 127 if amax == 0 else min(max(floor_log2(amax) - 8 + 127, 0), 254)
            s[h, b] = sb
            for i, v in enumerate(vals):
                m = 32 * b + i
                q[h, m] = rne_e4m3(v / Fraction(2) ** (sb - 127)) if m < used else 0
    return q, s


def bf16_bits_of(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def tricky_block(rng, amax_exp):
    """32 bf16 values around 2^amax_exp: exact E4M3 grid midpoints (ties),
    values in [448, 512) after scaling, tiny values, zeros and -0."""
    sc = 2.0 ** (amax_exp - 8)
    grid = np.array([float(v) for _, v in POS])
    mids = (grid[1:] + grid[:-1]) / 2  # exact ties between neighbouring codes
    vals = list(rng.choice(mids, 12) * sc)
    vals += list(rng.uniform(448, 511.9, 4) * sc)  # saturation range
    vals += list(rng.uniform(0, 2 ** -9, 4) * sc)  # below the smallest subnormal code
    vals += [0.0, -0.0]
    vals += list(rng.normal(0, 64, 32 - len(vals) - 1) * sc)
    vals += [2.0 ** amax_exp * 1.5]  # keeps amax in [2^e, 2^(e+1))
    vals = np.array(vals, np.float64)
    vals *= rng.choice([-1.0, 1.0], vals.shape)
    rng.shuffle(vals)
    return vals


@pytest.mark.parametrize("seed", range(4))
def test_quantizer_exact_rational(seed):
    rng = np.random.default_rng(9600 + seed)
    M, H = 96, 5
    x = np.zeros((M, H))
    for h in range(H):
        for b in range(M // 32):
            x[32 * b:32 * b + 32, h] = tricky_block(rng, int(rng.integers(-20, 20)))
    bits = bf16_bits_of(x)
    used = 80  # the last block is half padding
    q, s = oracle.quantize_tokens(bits, used=used)
    eq, es = exact_quantize(bits, used)
    np.testing.assert_array_equal(s, es)
    np.testing.assert_array_equal(q, eq)


def test_quantizer_matches_input_generator():
    """workloads.quantize_rows (torch, fp64 frexp/ldexp/round) quantises rows
    along their last axis; the oracle quantises x [M, H] along M and
    transposes: the two must give the same bytes."""
    g = torch.Generator().manual_seed(9700)
    x = torch.randn((256, 48), generator=g) * torch.exp2(torch.randint(-12, 12, (1, 48), generator=g).float())
    xb = x.to(torch.bfloat16)
    q, s = oracle.quantize_tokens(xb.view(torch.int16).numpy().view(np.uint16))
    wq, ws = W.quantize_rows(xb.to(torch.float64).t().contiguous())
    np.testing.assert_array_equal(q, wq.numpy())
    np.testing.assert_array_equal(s, ws.numpy())


def test_quantizer_closed_forms():
    M, H = 64, 4
    x = np.zeros((M, H), np.float32)
    x[:32, 0] = 3.0 * 2.0 ** -10
    x[5, 0] = 2.0 ** 7            # amax = 2^7 exactly -> scale byte 7 + 119, element 2^8 -> code 0x78
    x[:32, 2] = -1.0              # amax 1 -> byte 119, elements -256 -> 0xF8
    x[:, 3] = 7.0                 # tokens past `used` (= 32) become 0 and do not count
    q, s = oracle.quantize_tokens(bf16_bits_of(x), used=32)
    assert s[0, 0] == 126 and q[0, 5] == 0x78
    assert s[1, 0] == 127 and (q[1, :32] == 0).all()        # all-zero block
    assert s[2, 0] == 119 and (q[2, :32] == 0xF8).all()
    assert (q[:, 32:] == 0).all() and (s[:, 1] == 127).all()  # padding block
    # 7 = 1.75 * 2^2: byte 2 - 8 + 127, element 7 * 2^6 = 448, the largest code
    assert s[3, 0] == 121 and (q[3, :32] == 0x7E).all()


def test_quantizer_sign_symmetry():
    rng = np.random.default_rng(9800)
    x = rng.normal(0, 1, (128, 8)).astype(np.float32)
    q1, s1 = oracle.quantize_tokens(bf16_bits_of(x))
    q2, s2 = oracle.quantize_tokens(bf16_bits_of(-x))
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(q2, np.where(q1 == 0, 0, q1 ^ 0x80))


def test_quantizer_error_bound():
    """Within a block, an element at least 2^-6 of the block's power-of-two
    scale of 2^8 (the E4M3 normal range) dequantises to within 2^-4 relative
    (3 mantissa bits, round to nearest); saturation only clips values that
    scale to more than 448, by at most 512/448."""
    rng = np.random.default_rng(9900)
    x = rng.normal(0, 1, (256, 16)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (1, 16))).astype(np.float32)
    bits = bf16_bits_of(x)
    xv = bits.astype(np.uint32) << 16
    xv = xv.view(np.float32).astype(np.float64)
    q, s = oracle.quantize_tokens(bits)
    dec = np.vectorize(oracle.e4m3)(q) * np.exp2(s.astype(np.float64) - 127).repeat(32, axis=1)
    ref = xv.T
    scale = np.exp2(s.astype(np.float64) - 127).repeat(32, axis=1)
    y = np.abs(ref) / scale
    sat = y > 448
    normal = (y >= 2.0 ** -6) & ~sat
    err = np.abs(dec - ref)
    assert (err[normal] <= 2.0 ** -4 * np.abs(ref[normal])).all()
    assert (y < 512).all()
    np.testing.assert_array_equal(dec[sat], np.sign(ref[sat]) * 448 * scale[sat])
