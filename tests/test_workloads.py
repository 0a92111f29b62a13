"""Host-side checks of the seeded input generators (CPU only).

The generators hold no contraction arithmetic; these tests check that the
routings have the stated structure (sums, 32-token alignment, skew bands,
empty experts, Zipf start parity) and that the MXFP8 encoder follows its
recipe (scale from the exact binary exponent of the block amax, round-half-even
E4M3 codes, saturation at 448).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W


@pytest.mark.parametrize("name", sorted(W.CONFIGS))
def test_routing_structure(name):
    c = W.CONFIGS[name]
    sizes, _ = W.routing_sizes(name)
    assert sizes.shape == (c["E"],)
    assert sizes.sum() == c["M"]
    assert (sizes % 32 == 0).all() and (sizes >= 0).all()
    offs = W.offs_from_sizes(sizes)
    assert offs.dtype == np.int32 and offs[-1] == c["M"]
    assert (np.diff(offs) >= 0).all()
    r = c["routing"]
    skew = sizes.max() / (c["M"] / c["E"])
    if r[0] == "dirichlet":
        assert r[2][0] <= skew <= r[2][1]
        assert (sizes == 0).sum() == r[3]
    if r[0] == "ramp":
        assert skew == pytest.approx(r[1], rel=0.02)
        assert (sizes % r[2] == 0).all()
    if r[0] == "balanced":
        assert (sizes == c["M"] // c["E"]).all()


def test_routing_reproducible():
    a, sa = W.routing_sizes("16b_24k")
    b, sb = W.routing_sizes("16b_24k")
    assert sa == sb and (a == b).all()


def test_zipf_starts_odd_multiples_of_32():
    sizes, _ = W.routing_sizes("671b_down_zipf")
    assert (sizes == 0).sum() == 4
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    live = [int(s) for s, n in zip(starts, sizes) if n > 0]
    assert live[0] == 0
    for s in live[1:]:
        assert s % 64 == 32  # odd multiple of 32, never 64- or 128-aligned
    assert sizes.max() / (131072 / 32) > 8  # heavy Zipf head


def test_tiny_config():
    cfg = W.make_config("tiny")
    assert cfg["offs"].tolist() == [96, 96, 256, 512]
    assert cfg["A"].shape == (128, 512) and cfg["sA"].shape == (128, 16)
    assert cfg["B"].shape == (256, 512) and cfg["sB"].shape == (256, 16)
    cfg2 = W.make_config("tiny")
    assert torch.equal(cfg["A"], cfg2["A"]) and torch.equal(cfg["sB"], cfg2["sB"])


def _e4m3_value(code):
    s = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 15, code & 7
    return s * (Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7))


def test_encoder_round_half_even_exhaustive_grid():
    # every finite positive E4M3 value, the midpoints between neighbours, and
    # points just off the midpoints
    vals = sorted({_e4m3_value(c) for c in range(0x7F)})
    pts, want = [], []
    for i, v in enumerate(vals):
        pts.append(v)
        want.append(v)
        if i + 1 < len(vals):
            mid = (v + vals[i + 1]) / 2
            lo_code = vals.index(v)
            even = v if lo_code % 2 == 0 else vals[i + 1]  # codes are ordered like values
            pts += [mid, mid - Fraction(1, 2 ** 20), mid + Fraction(1, 2 ** 20)]
            want += [even, v, vals[i + 1]]
    y = torch.tensor([float(p) for p in pts], dtype=torch.float64)
    codes = W.e4m3_encode_rne(y)
    got = [_e4m3_value(int(c)) for c in codes]
    assert got == want
    codes_neg = W.e4m3_encode_rne(-y)
    for c, w in zip(codes_neg.tolist(), want):
        assert _e4m3_value(c) == -w or (w == 0 and c == 0)


def test_quantize_block_scale_and_saturation():
    rows = torch.tensor([
        [1.0] * 32,                       # amax 1 -> byte 119, 1.0 -> 256 -> 0x78
        [511.0] + [0.0] * 31,             # amax 511 -> byte 127, saturates to 448 (0x7E)
        [0.0] * 32,                       # amax 0 -> byte 127, all-zero codes
        [3.0] + [-2.0 ** -20] * 31,       # amax 3 -> byte 120
    ], dtype=torch.float32)
    q, s = W.quantize_rows(rows)
    assert s[:, 0].tolist() == [119, 127, 127, 120]
    assert q[0, 0] == 0x78 and q[1, 0] == 0x7E and (q[2] == 0).all()
    # 3.0 / 2^-7 = 384 = 1.5 * 2^8 -> exponent field 15, mantissa 4
    assert q[3, 0] == (15 << 3 | 4)


def test_quantize_roundtrip_error_bound():
    g = torch.Generator().manual_seed(3)
    x = torch.randn((8, 256), generator=g)
    q, s = W.quantize_rows(x)
    lut = np.array([float(_e4m3_value(c)) if (c & 0x7F) != 0x7F else np.nan for c in range(256)])
    dec = lut[q.numpy()] * np.exp2(np.repeat(s.numpy().astype(np.float64), 32, axis=1) - 127)
    xb = x.numpy().astype(np.float64)
    blk_amax = np.repeat(np.abs(xb).reshape(8, 8, 32).max(-1), 32, axis=1)
    # relative error of E4M3 is <= 2^-4 for normals; saturation clips the top of each block to 448/512
    err = np.abs(dec - xb)
    assert (err <= np.maximum(np.abs(xb) * 2.0 ** -4, blk_amax * 2.0 ** -9) + blk_amax * (1 - 448 / 512) + 1e-12).all()
    assert np.isfinite(dec).all()


def test_useful_flops_and_bytes():
    cfg = dict(sizes=np.array([100 * 32, 0, 50 * 32]), N=1408, K=2048, E=3)
    assert W.useful_flops(cfg) == 2.0 * 4800 * 1408 * 2048
    assert W.algorithmic_bytes(cfg) == pytest.approx(4800 * 3456 * (1 + 1 / 32) + 2 * 3 * 1408 * 2048 + 12)


def test_bf16_workload_recipe():
    """The named bf16 workloads keep their base workload's shape and routing;
    values are std * N(0, 1) rounded once to bf16, deterministic per seed."""
    cfg = W.make_bf16_config("16b_1k_bf16")
    base = W.CONFIGS["16b_1k"]
    assert (cfg["E"], cfg["N"], cfg["K"], cfg["M"]) == (base["E"], base["N"], base["K"], base["M"])
    sizes, _ = W.routing_sizes("16b_1k")
    np.testing.assert_array_equal(cfg["sizes"], sizes)
    np.testing.assert_array_equal(cfg["offs"].numpy(), W.offs_from_sizes(sizes))
    assert cfg["A"].dtype == torch.bfloat16 and cfg["A"].shape == (1408, 8192) and cfg["B"].shape == (2048, 8192)
    again = W.make_bf16_config("16b_1k_bf16")
    assert torch.equal(cfg["A"].view(torch.int16), again["A"].view(torch.int16))
    assert abs(float(cfg["A"].float().std()) - 1.0) < 0.01 and abs(float(cfg["B"].float().std()) - 0.5) < 0.01
    bf = dict(sizes=np.array([100, 0, 60]), N=1408, K=2048, E=3)
    assert W.bf16_algorithmic_bytes(bf) == 160 * 3456 * 2 + 2 * 3 * 1408 * 2048 + 12
