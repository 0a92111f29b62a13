"""GPU parity of the row-ragged grouped GEMM (forward / data gradient) against
the CPU oracle (needs an MI355X).

Each case NaN-poisons the output, runs the C-ABI library through the Python
binding, and compares every row that belongs to an expert with the oracle to
the same tolerance as the weight gradient; rows past the last expert must keep
their poison (they are never written).  Every case covers the whole output,
the full-size workloads (the benchmark's launch configuration) included.
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle
import workloads as W
from helpers import BF16_NAN, bf16_bits, bf16_to_f64, check_close

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def run_rows(cfg):
    out = torch.empty((cfg["R"], cfg["N"]), dtype=torch.bfloat16, device=cfg["A"].device)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.fwd(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out)
    torch.cuda.synchronize()
    return bf16_bits(out)


def host_rows(cfg):
    return tuple(cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs"))


def full_compare_rows(cfg, what):
    say("%s: launch E=%d R=%d C=%d N=%d" % (what, cfg["E"], cfg["R"], cfg["C"], cfg["N"]))
    bits = run_rows(cfg)
    ref = oracle.rows_f64(*host_rows(cfg))
    used = int(np.asarray(cfg["sizes"]).sum())
    stats = check_close(bits[:used], ref[:used], what=what)
    assert (bits[used:] == BF16_NAN).all(), "%s: a row past the last expert was written" % what
    return bits, ref, stats


ROWS_CASES = [
    # E, R, C, N, sizes (sum <= R; rows after them are padding)
    (3, 700, 256, 272, [300, 0, 290]),          # unaligned row boundaries, empty expert, partial N tile, padding
    (1, 16, 32, 16, [16]),                      # the smallest problem
    (4, 1100, 160, 512, [1, 255, 257, 513]),    # whole-tile scale blocks, 5-byte scale rows; 1-row and tile-straddling experts
    (2, 600, 512, 256, [512, 88]),              # whole-tile scale blocks, dword-aligned scale rows
    (5, 1024, 1408, 336, [200, 0, 0, 600, 224]),  # the 16B down-projection width as C
    (6, 520, 2048, 1408, [100, 32, 0, 200, 96, 64]),  # 16B gate/up widths (C % 512 == 0: grouped scale loads)
    (3, 520, 1440, 272, [0, 260, 200]),         # whole-tile scale blocks, 45-byte scale rows (odd)
    (2, 600, 1504, 128, [300, 257]),            # the largest C with whole-tile scale blocks
    (2, 300, 1568, 160, [150, 100]),            # C % 128 != 0 above it: the paired scale path
    (3, 400, 1664, 144, [130, 0, 200]),         # C % 128 == 0, C % 512 != 0: 16-byte groups from 4-byte-aligned rows
]


@pytest.mark.parametrize("case", range(len(ROWS_CASES)))
def test_rows_ragged_shapes(case):
    E, R, C, N, sizes = ROWS_CASES[case]
    cfg = W.make_rows(E, R, C, N, sizes, seed=800 + case, device=DEV)
    bits, ref, stats = full_compare_rows(cfg, "rows case %d" % case)
    print("rows case %d max_rel %.3e" % (case, stats["max_rel"]))


def test_rows_bitwise_repeat():
    cfg = W.make_rows(4, 1100, 160, 512, [1, 255, 257, 513], seed=810, device=DEV)
    say("rows repeat: launch twice")
    a = run_rows(cfg)
    b = run_rows(cfg)
    np.testing.assert_array_equal(a, b)


def test_rows_exact_regime_bitwise():
    """Codes in {0, +-.5, +-1, +-1.5, +-2} and scale bytes 126..128 keep every
    partial sum exact in FP32: the bf16 output equals the oracle rounded once."""
    rng = np.random.default_rng(820)
    E, R, C, N = 3, 600, 512, 272
    codes = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x3C, 0xBC, 0x40, 0xC0], np.uint8)
    A = rng.choice(codes, (R, C))
    B = rng.choice(codes, (E, N, C))
    sA = rng.integers(126, 129, (R, C // 32)).astype(np.uint8)
    sB = rng.integers(126, 129, (E, N, C // 32)).astype(np.uint8)
    sizes = np.array([257, 0, 300])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    cfg = dict(E=E, R=R, C=C, N=N, A=t(A), sA=t(sA), B=t(B), sB=t(sB),
               offs=t(np.cumsum(sizes).astype(np.int32)), sizes=sizes)
    say("rows exact regime: launch")
    bits = run_rows(cfg)
    ref = oracle.rows_f64(A, sA, B, sB, np.cumsum(sizes).astype(np.int32))
    used = int(sizes.sum())
    np.testing.assert_array_equal(bits[:used], oracle.to_bf16_bits(ref[:used]))


def test_rows_padding_garbage_ignored():
    cfg = W.make_rows(3, 700, 256, 272, [300, 0, 290], seed=830, device=DEV)
    say("rows padding garbage: two launches")
    base = run_rows(cfg)
    used = int(np.asarray(cfg["sizes"]).sum())
    cfg["A"][used:] = 0x7F   # NaN codes
    cfg["sA"][used:] = 0xFF  # NaN scales
    np.testing.assert_array_equal(run_rows(cfg), base)


def test_rows_nan_inside_windows():
    """A NaN code in a live row, a NaN scale in a live expert's weight block
    and a negative-NaN code in another live row give NaN at exactly the
    oracle's positions (two output rows and one output column of expert 2's
    rows); the same values in a row past offs[E-1] and in an empty expert's
    weights change nothing; everything else finite and within tolerance."""
    cfg = W.make_rows(3, 700, 256, 272, [300, 0, 290], seed=831, device=DEV)
    used = 590
    cfg["A"][17, 40] = 0x7F
    cfg["sB"][2, 100, 3] = 0xFF
    cfg["A"][450, 200] = 0xFF
    cfg["A"][600, 5] = 0x7F      # past the last expert's rows
    cfg["sB"][1, 50, 0] = 0xFF   # expert 1 has no rows
    say("rows NaN inside windows: launch")
    bits = run_rows(cfg)
    ref = oracle.rows_f64(*host_rows(cfg))[:used]
    got = bf16_to_f64(bits[:used])
    gn, rn = np.isnan(got), np.isnan(ref)
    assert rn.sum() == 272 + 290 + 272 - 1
    np.testing.assert_array_equal(gn, rn)
    check_close(np.where(rn, 0, bits[:used]).astype(np.uint16), np.where(rn, 0.0, ref), what="rows NaN case")
    assert (bits[used:] == BF16_NAN).all()


def test_rows_all_experts_empty():
    cfg = W.make_rows(4, 256, 256, 256, [0, 0, 0, 0], seed=840, device=DEV)
    say("rows all empty: launch")
    assert (run_rows(cfg) == BF16_NAN).all()


@pytest.mark.slow
@pytest.mark.parametrize("name", ["16b_fwd", "16b_fwd_down"])
def test_rows_full_size_whole_output(name):
    """The 16B gate/up and down widths at full size (196,608 routed rows), in
    the benchmark's launch configuration: every row of every expert against
    the oracle (rms over the whole reference), rows past the last expert
    never written."""
    cfg = W.make_rows_config(name, device=DEV)
    say("%s: launch R=%d C=%d N=%d (whole output)" % (name, cfg["R"], cfg["C"], cfg["N"]))
    bits = run_rows(cfg)
    used = int(np.asarray(cfg["sizes"]).sum())
    say("%s: oracle on %d x %d outputs" % (name, used, cfg["N"]))
    ref = oracle.rows_f64(*host_rows(cfg))
    st = check_close(bits[:used], ref[:used], what=name)
    print("%s whole output max_rel %.3e" % (name, st["max_rel"]))
    assert (bits[used:] == BF16_NAN).all()


@pytest.mark.parametrize("offs_list,exact", [
    ([600, 300, 1000], ((0, 300, 0), (600, 1000, 2))),   # decreasing: windows [0,600), [600,600), [300,1000)
    ([-5, 700, 5000], ((0, 700, 1), (700, 1200, 2))),     # negative and past R: clamped to [0, R]
])
def test_rows_malformed_offs(offs_list, exact):
    """Malformed offs: the call returns, nothing outside out is written, rows
    past every clamped window keep their poison, and rows that one expert's
    clamped window alone covers equal the oracle for that expert."""
    E, R, C, N = 3, 1200, 256, 272
    cfg = W.make_rows(E, R, C, N, [400, 400, 400], seed=870, device=DEV)
    offs = torch.tensor(offs_list, dtype=torch.int32, device=DEV)
    guard = 4096
    big = torch.empty(R * N + 2 * guard, dtype=torch.bfloat16, device=DEV)
    big.view(torch.int16).fill_(BF16_NAN)
    out = big[guard:guard + R * N].view(R, N)
    say("rows malformed offs %s" % offs_list)
    mxw.fwd(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], offs, out=out)
    torch.cuda.synchronize()
    gb = bf16_bits(big)
    assert (gb[:guard] == BF16_NAN).all() and (gb[-guard:] == BF16_NAN).all(), "store outside out"
    bits = bf16_bits(out)
    clamp = [min(max(v, 0), R) for v in offs_list]
    hi = max(clamp)
    assert (bits[hi:] == BF16_NAN).all(), "a row past every window was written"
    A, sA, B, sB, _ = host_rows(cfg)
    for lo, up, g in exact:
        # expert g alone, as the only expert of a well-formed call over rows [0, up)
        ref = oracle.rows_f64(A[:up], sA[:up], B[g:g + 1], sB[g:g + 1], np.array([up], np.int32))
        check_close(bits[lo:up], ref[lo:up], what="rows malformed offs %s rows %d..%d" % (offs_list, lo, up))
