"""Short tiles of the weight gradient (needs an MI355X).

When N % 256 == 128 the last 384 rows along N are computed as two tiles of 192
rows (96 rows, three 32-row blocks per wave) instead of a whole tile and one
whose upper half lies past N.  These cases put short tiles through both
scheduling paths (one workgroup per tile, column mode; a launch with half
tiles keeps whole ones), both scale paths (the caller's planes and the
pre-shuffled bands, whose band of a short tile starts at its own first row),
ragged and empty experts and partial K tiles; in the exact-arithmetic regime
the GPU's bf16 must equal RNE(oracle) bit for bit, elsewhere the tolerance
holds over the whole output.
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle
import workloads as W
from helpers import ENTRIES, bf16_bits, check_close, host, run_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda"
EXACT_CODES = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x3C, 0xBC, 0x40, 0xC0], np.uint8)  # 0, +-.5, +-1, +-1.5, +-2


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def exact_cfg(rng, E, N, K, M, sizes):
    A = rng.choice(EXACT_CODES, (N, M))
    B = rng.choice(EXACT_CODES, (K, M))
    sA = rng.integers(126, 129, (N, M // 32)).astype(np.uint8)
    sB = rng.integers(126, 129, (K, M // 32)).astype(np.uint8)
    offs = np.cumsum(sizes).astype(np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return dict(E=E, N=N, K=K, M=M, A=t(A), sA=t(sA), B=t(B), sB=t(sB), offs=t(offs), sizes=np.asarray(sizes))


EXACT_CASES = [
    # E, N, K, M, sizes: every window at most 1,024 tokens (exact partial sums)
    (3, 384, 528, 2048, [96, 1024, 544]),        # two short tiles only, partial K tile
    (4, 640, 256, 1920, [0, 992, 160, 736]),     # one whole tile and two short ones, an empty expert
    (2, 1408, 272, 1536, [512, 1024]),           # the 16B expert width
]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("case", range(len(EXACT_CASES)))
def test_short_tiles_exact_bitwise(case, entry):
    E, N, K, M, sizes = EXACT_CASES[case]
    cfg = exact_cfg(np.random.default_rng(600 + case), E, N, K, M, sizes)
    say("short tiles, exact regime case %d [%s]: E=%d N=%d K=%d M=%d" % (case, entry, E, N, K, M))
    bits = bf16_bits(run_gpu(cfg, entry=entry))
    ref = oracle.wgrad_f64(*host(cfg))
    np.testing.assert_array_equal(bits, oracle.to_bf16_bits(ref))


def test_width_with_short_tiles_in_a_half_tile_launch():
    """A launch whose last round runs as half tiles, on a width that would
    have short tiles: such a launch keeps whole 256-row tiles (a short tile
    cannot be halved), the last of them half past N.  Exact regime, both
    entry points, bitwise."""
    E, N, K, M = 40, 640, 768, 20480
    rng = np.random.default_rng(611)
    sizes = 32 * rng.integers(0, 33, E)
    sizes[rng.choice(E, 3, replace=False)] = 0
    while sizes.sum() > M:
        sizes[np.argmax(sizes)] -= 32
    cfg = exact_cfg(rng, E, N, K, M, sizes)
    say("short tiles in the half-tile round: %d tiles as halves" % mxw.tail_split(E, M, N, K))
    ref = oracle.to_bf16_bits(oracle.wgrad_f64(*host(cfg)))
    for entry in ENTRIES:
        bits = bf16_bits(run_gpu(cfg, entry=entry))
        np.testing.assert_array_equal(bits, ref)


def test_short_tiles_column_mode_and_shuffled_bands():
    """Column mode on a width with short tiles (their regions are the last
    band's) and the pre-shuffled scale bands: whole output within tolerance,
    bitwise repeat, and the entry point without a workspace on the same
    problem within tolerance."""
    E, N, K, M, sizes = 3, 640, 1024, 49152, [16384, 0, 24576]
    assert mxw.columns(E, M, N, K) > 0 and mxw.scale_shuffle(E, M)
    cfg = W.make_random(E, N, K, M, sizes, seed=612, device=DEV)
    ref = oracle.wgrad_f64(*host(cfg))
    say("short tiles, column mode: E=%d N=%d K=%d M=%d" % (E, N, K, M))
    a = bf16_bits(run_gpu(cfg, entry="ws"))
    check_close(a, ref, what="short tiles, column mode")
    assert (a[1] == 0).all()
    b = bf16_bits(run_gpu(cfg, entry="ws"))
    np.testing.assert_array_equal(a, b)
    c = bf16_bits(run_gpu(cfg, entry="plain"))
    check_close(c, ref, what="short tiles, one workgroup per tile")


def test_short_tiles_shuffled_and_direct_scales_bitwise_equal():
    """Long experts (M >= 4096 E) make the workspace entry pre-shuffle the
    scales of each tile's band (a short tile's band starts at its own first
    row); the entry without one reads the caller's planes, whose rows are not
    a whole number of dwords here (M % 128 != 0), a dword early.  One
    workgroup per tile in both, the same MFMA sequence: identical bits, NaN
    scales in the padding included."""
    E, N, K, M = 2, 1408, 1024, 8192 + 160
    sizes = [4096] * E
    assert mxw.columns(E, M, N, K) == 0 and mxw.scale_shuffle(E, M)
    cfg = W.make_random(E, N, K, M, sizes, seed=613, device=DEV)
    cfg["sA"][:, 8192 // 32:] = 0xFF
    cfg["sB"][:, 8192 // 32:] = 0xFF
    say("short tiles, scale paths: N=%d K=%d M=%d" % (N, K, M))
    shuf = bf16_bits(run_gpu(cfg, entry="ws"))
    direct = bf16_bits(run_gpu(cfg, entry="plain"))
    np.testing.assert_array_equal(shuf, direct)
    check_close(shuf, oracle.wgrad_f64(*host(cfg)), what="short tiles, shuffled scales")


def test_short_tiles_bf16_exact_bitwise():
    """The bf16 weight gradient on a width with short tiles: small integers
    times powers of two, all partial sums exact, so bit for bit."""
    E, N, K, M, sizes = 3, 640, 272, 1536, [224, 0, 1296]
    rng = np.random.default_rng(614)
    vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 1.5, -1.5, 2.0, -2.0], np.float32)
    A = torch.from_numpy(rng.choice(vals, (N, M))).to(torch.bfloat16).to(DEV)
    B = torch.from_numpy(rng.choice(vals, (K, M))).to(torch.bfloat16).to(DEV)
    offs = torch.from_numpy(np.cumsum(sizes).astype(np.int32)).to(DEV)
    a16 = A.view(torch.int16).cpu().numpy().view(np.uint16)
    b16 = B.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.to_bf16_bits(oracle.bf16_wgrad_f64(a16, b16, offs.cpu().numpy()))
    for plain in (False, True):
        out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
        out.view(torch.int16).fill_(0x7FC0)
        say("short tiles, bf16 exact [%s]" % ("plain" if plain else "ws"))
        mxw.wgrad_bf16(A, B, offs, out=out, plain=plain)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_bits(out), ref)
