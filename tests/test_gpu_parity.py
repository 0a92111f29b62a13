"""GPU parity: the HIP path against the CPU oracle (needs an MI355X).

Every case runs the C-ABI library through the Python binding on seeded inputs
that the oracle also consumes, with the output NaN-poisoned before the launch so
that a skipped store shows, through both weight-gradient entry points
(mxfp8_wgrad_grouped_ws with a workspace, mxfp8_wgrad_grouped without).
Cases here are compared element by element over the whole output; the
full-size workloads are in test_gpu_full.py.
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle
import workloads as W
from helpers import ENTRIES, bf16_bits, bf16_to_f64, check_close, host, run_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda"

BF16_NAN_I16 = 0x7FC0
EXACT_CODES = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x3C, 0xBC, 0x40, 0xC0], np.uint8)  # 0, +-.5, +-1, +-1.5, +-2


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def full_compare(cfg, what, entries=ENTRIES):
    """Both entry points (or `entries`) against one oracle run, whole output.
    Returns {entry: (bits, stats)} and the reference."""
    ref = oracle.wgrad_f64(*host(cfg))
    res = {}
    for entry in entries:
        say("%s [%s]: launch E=%d N=%d K=%d M=%d" % (what, entry, cfg["E"], cfg["N"], cfg["K"], cfg["M"]))
        bits = bf16_bits(run_gpu(cfg, entry=entry))
        stats = check_close(bits, ref, what="%s [%s]" % (what, entry))
        for g in range(cfg["E"]):
            if int(cfg["sizes"][g]) == 0:
                assert (bits[g] == 0).all(), "%s [%s]: empty expert %d not exact +0" % (what, entry, g)
        res[entry] = (bits, stats)
    return res, ref


def from_numpy(A, sA, B, sB, offs, sizes, device=DEV):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    N, M = A.shape
    return dict(E=len(offs), N=N, K=B.shape[0], M=M, A=t(A), sA=t(sA), B=t(B), sB=t(sB),
                offs=t(np.asarray(offs, np.int32)), sizes=np.asarray(sizes))


# ----------------------------------------------------------------------------
# small cases, whole output
# ----------------------------------------------------------------------------


def test_tiny_config():
    cfg = W.make_config("tiny", device=DEV)
    res, ref = full_compare(cfg, "tiny")
    for entry, (bits, stats) in res.items():
        print("tiny [%s] max_rel %.3e" % (entry, stats["max_rel"]))
        assert stats["max_rel"] < 2 ** -7
    np.testing.assert_array_equal(res["ws"][0], res["plain"][0])  # no column mode: the same kernel


def test_hand_case_embedded(golden_dir):
    """The hand-computed two-expert case, zero-padded into a 16 x 16 output."""
    import json, os
    h = json.load(open(os.path.join(golden_dir, "hand_two_expert.json")))
    N = K = 16
    M = h["M"]
    A = np.zeros((N, M), np.uint8)
    B = np.zeros((K, M), np.uint8)
    sA = np.full((N, M // 32), 127, np.uint8)
    sB = np.full((K, M // 32), 127, np.uint8)
    for r, row in enumerate(h["A_rows"]):
        for lo, hi, code in row["codes"]:
            A[r, lo:hi] = int(code, 16)
    for r, row in enumerate(h["B_rows"]):
        for lo, hi, code in row["codes"]:
            B[r, lo:hi] = int(code, 16)
    sA[:2] = np.array(h["sA"], np.uint8)
    sB[:1] = np.array(h["sB"], np.uint8)
    cfg = from_numpy(A, sA, B, sB, h["offs"], [32, 64])
    want = np.zeros((2, N, K), np.uint16)
    for g in range(2):
        for n in range(2):
            want[g, n, 0] = int(h["expected_bf16"][g][n][0], 16)
    for entry in ENTRIES:
        say("hand case [%s]" % entry)
        bits = bf16_bits(run_gpu(cfg, entry=entry))
        np.testing.assert_array_equal(bits, want)


RAGGED_CASES = [
    # E, N, K, M, sizes (sum <= M; the rest is padding)
    (3, 272, 528, 1024, [96, 0, 800]),          # partial N and K tiles, empty expert, padding
    (5, 256, 256, 1056, [32, 160, 64, 352, 416]),  # M % 128 != 0 (scale rows read a dword early), short groups
    (2, 512, 256, 2048, [1888, 160]),           # long group, tail step inside the last 128 tokens
    (4, 144, 400, 640, [0, 0, 608, 0]),         # only one live expert, odd start
    (1, 16, 16, 32, [32]),                      # the smallest problem
    (6, 256, 768, 4096, [64, 1184, 0, 32, 2400, 224]),
]


@pytest.mark.parametrize("case", range(len(RAGGED_CASES)))
def test_ragged_shapes(case):
    E, N, K, M, sizes = RAGGED_CASES[case]
    cfg = W.make_random(E, N, K, M, sizes, seed=500 + case, device=DEV)
    full_compare(cfg, "ragged case %d" % case)


COLUMN_CASES = [
    # E, N, K, M, sizes: long experts on few tiles -> column mode, with regions
    # cut across many columns (several partial tiles per region)
    (1, 272, 528, 8192, [8192]),                   # one region spread over every column
    (2, 512, 768, 16416, [8992, 7392]),            # M % 512 != 0 (dword scale path), padding
    (3, 1040, 272, 24576, [12000, 0, 9600]),       # empty expert, partial tiles, 4-row and 1-row bands
    (8, 1408, 2048, 65536, [12000, 4000, 9600, 0, 11200, 8000, 6400, 14336]),  # 16B shape
]


@pytest.mark.parametrize("case", range(len(COLUMN_CASES)))
def test_column_mode_cases(case):
    """Column mode of the workspace entry (one workgroup per CU, regions split
    between columns and summed through FP32 partials), whole output, plus
    bitwise repeat; the same problem through the entry point without a
    workspace (one workgroup per tile)."""
    E, N, K, M, sizes = COLUMN_CASES[case]
    assert mxw.columns(E, M, N, K) > 0, "case does not select column mode"
    cfg = W.make_random(E, N, K, M, sizes, seed=700 + case, device=DEV)
    res, ref = full_compare(cfg, "column case %d" % case)
    for entry, (bits, stats) in res.items():
        print("column case %d [%s] max_rel %.3e" % (case, entry, stats["max_rel"]))
    again = bf16_bits(run_gpu(cfg))
    np.testing.assert_array_equal(again, res["ws"][0])


def test_mode_selection():
    """The shapes the benchmark and parity cases rely on pick the mode the
    design expects: column mode for the 16B shape at 24k tokens/expert, one
    workgroup per tile for 1k tokens/expert and for the 671B shapes."""
    assert mxw.columns(8, 196608, 1408, 2048) > 0
    assert mxw.columns(8, 8192, 1408, 2048) == 0
    assert mxw.columns(32, 262144, 4096, 7168) == 0
    assert mxw.columns(32, 262144, 7168, 2048) == 0


def test_16b_1k_full():
    """The 16B expert shape at 1,024 tokens/expert, whole output."""
    cfg = W.make_config("16b_1k", device=DEV)
    res, ref = full_compare(cfg, "16b_1k")
    for entry, (bits, stats) in res.items():
        print("16b_1k [%s] max_rel %.3e" % (entry, stats["max_rel"]))
    np.testing.assert_array_equal(res["ws"][0], res["plain"][0])  # one workgroup per tile in both


def _exact_problem(rng, E, N, K, M, sizes):
    A = rng.choice(EXACT_CODES, (N, M))
    B = rng.choice(EXACT_CODES, (K, M))
    sA = rng.integers(126, 129, (N, M // 32)).astype(np.uint8)
    sB = rng.integers(126, 129, (K, M // 32)).astype(np.uint8)
    offs = np.cumsum(sizes).astype(np.int32)
    return A, sA, B, sB, offs


@pytest.mark.parametrize("entry", ENTRIES)
def test_exact_regime_bitwise(entry):
    """All partial sums exactly representable in FP32: GPU bf16 == RNE(oracle)
    bit for bit, whatever the MFMA's summation order.  A misplaced scale or
    lane shows as whole wrong rows."""
    rng = np.random.default_rng(77)
    sizes = [96, 0, 448, 1024, 32, 160]
    A, sA, B, sB, offs = _exact_problem(rng, 6, 272, 528, 1920, sizes)
    cfg = from_numpy(A, sA, B, sB, offs, sizes)
    say("exact regime [%s]" % entry)
    bits = bf16_bits(run_gpu(cfg, entry=entry))
    ref = oracle.wgrad_f64(A, sA, B, sB, offs)
    np.testing.assert_array_equal(bits, oracle.to_bf16_bits(ref))


# 320 tiles on a 256-CU device at 512 tokens per expert on average: the last
# 64 tiles of the longest-first dealing run as two half tiles each
TAIL_SHAPE = (40, 512, 1024, 20480)


def _tail_sizes(rng, E, M):
    sizes = 32 * rng.integers(0, 33, E)  # 0 .. 1,024 tokens, ragged
    sizes[rng.choice(E, 3, replace=False)] = 0
    while sizes.sum() > M:
        sizes[np.argmax(sizes)] -= 32
    return sizes


@pytest.mark.parametrize("entry", ENTRIES)
def test_tail_split_halves(entry):
    """A launch whose last round of tiles runs as half tiles (each covering
    the even or the odd 32-row blocks of a tile's 256 rows), with ragged and
    empty experts: in the exact-arithmetic regime GPU bf16 == RNE(oracle)
    bit for bit, and on normal values within the tolerance.  The halves
    compute every element as the whole tile would, so nothing else changes."""
    E, N, K, M = TAIL_SHAPE
    assert mxw.tail_split(E, M, N, K) > 0 or torch.cuda.get_device_properties(0).multi_processor_count >= 320
    rng = np.random.default_rng(91)
    sizes = _tail_sizes(rng, E, M)
    A, sA, B, sB, offs = _exact_problem(rng, E, N, K, M, sizes)
    say("tail split, exact regime [%s]: %d tiles as halves" % (entry, mxw.tail_split(E, M, N, K)))
    bits = bf16_bits(run_gpu(from_numpy(A, sA, B, sB, offs, sizes), entry=entry))
    np.testing.assert_array_equal(bits, oracle.to_bf16_bits(oracle.wgrad_f64(A, sA, B, sB, offs)))
    cfg = W.make_random(E, N, K, M, _tail_sizes(rng, E, M), seed=92, device=DEV)
    say("tail split, normal values [%s]" % entry)
    got = bf16_bits(run_gpu(cfg, entry=entry))
    check_close(got, oracle.wgrad_f64(*host(cfg)), what="tail split [%s]" % entry)


@pytest.mark.parametrize("entry", ENTRIES)
def test_bitwise_repeat(entry):
    cfg = W.make_random(4, 528, 784, 3072, [1056, 0, 992, 960], seed=31, device=DEV)
    say("bitwise repeat [%s]" % entry)
    a = bf16_bits(run_gpu(cfg, entry=entry))
    b = bf16_bits(run_gpu(cfg, entry=entry))
    c = bf16_bits(run_gpu(cfg, poison=False, entry=entry))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


@pytest.mark.parametrize("entry", ENTRIES)
def test_padding_garbage_ignored(entry):
    """NaN codes and 0xFF scales past offs[E-1] never reach the result (bitwise)."""
    sizes = [160, 0, 288, 96]
    cfg = W.make_random(4, 272, 272, 1024, sizes, seed=9, device=DEV)
    used = int(np.sum(sizes))
    say("padding garbage [%s]" % entry)
    clean = bf16_bits(run_gpu(cfg, entry=entry))
    for key, val in (("A", 0x7F), ("B", 0xFF)):
        cfg[key][:, used:] = val
    for key in ("sA", "sB"):
        cfg[key][:, used // 32:] = 0xFF
    dirty = bf16_bits(run_gpu(cfg, entry=entry))
    np.testing.assert_array_equal(dirty, clean)


NAN_CASES = {
    # E, N, K, M, sizes, NaN code inside, NaN scale inside (B row, block), a second NaN code inside,
    # garbage just past offs[E-1] (token)
    "per_tile": (3, 272, 528, 1024, [96, 0, 800], (5, 10), (300, 5), (9, 500), 900),
    "column": (2, 512, 768, 16416, [8992, 7392], (5, 10), (300, 400), (9, 9500), 16400),
}


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("case", sorted(NAN_CASES))
def test_nan_inside_windows(case, entry):
    """A NaN code (0x7F, 0xFF) or a NaN scale (0xFF) in a live sub-block makes
    exactly the outputs that contract over it NaN, as the oracle (IEEE fp64)
    does: the element's row (or column) of its expert, nothing else.  The same
    values in the 128-token pair just past offs[E-1] (loaded, then masked)
    change nothing.  NaN positions must match the oracle's exactly; every
    other element must be finite and within the tolerance.  (The column case
    also carries NaN through the FP32 partial tiles of a cut region.)"""
    E, N, K, M, sizes, a_in, sb_in, a_in2, past = NAN_CASES[case]
    cfg = W.make_random(E, N, K, M, sizes, seed=4242, device=DEV)
    if case == "column":
        assert mxw.columns(E, M, N, K) > 0
    cfg["A"][a_in] = 0x7F
    cfg["sB"][sb_in] = 0xFF
    cfg["A"][a_in2] = 0xFF
    cfg["A"][7, past] = 0x7F
    cfg["sB"][301, past // 32] = 0xFF
    say("NaN inside windows [%s, %s]" % (case, entry))
    bits = bf16_bits(run_gpu(cfg, entry=entry))
    ref = oracle.wgrad_f64(*host(cfg))
    gn, rn = np.isnan(bf16_to_f64(bits)), np.isnan(ref)
    assert rn.sum() == K + N + K - 1  # a row, a column and a row; one element shared
    np.testing.assert_array_equal(gn, rn)
    check_close(np.where(rn, 0, bits).astype(np.uint16), np.where(rn, 0.0, ref), what="NaN case %s" % case)


@pytest.mark.parametrize("entry", ENTRIES)
def test_scale_shift_doubles_bitwise(entry):
    """+1 on every scale exponent of one expert's blocks doubles that expert's
    output exactly (power-of-two scaling commutes with FP32 sums and bf16
    rounding) and leaves the others unchanged."""
    sizes = [192, 416, 96, 320]
    cfg = W.make_random(4, 400, 272, 1024, sizes, seed=17, device=DEV)
    say("scale shift [%s]" % entry)
    base = bf16_bits(run_gpu(cfg, entry=entry)).astype(np.uint32)
    lo, hi = 192, 192 + 416  # expert 1
    cfg["sA"][:, lo // 32:hi // 32] += 1
    shifted = bf16_bits(run_gpu(cfg, entry=entry)).astype(np.uint32)
    nonzero = (base[1] & 0x7FFF) != 0
    # doubling a bf16 = +1 in the exponent field (no overflow/underflow here)
    np.testing.assert_array_equal(shifted[1][nonzero], base[1][nonzero] + 0x80)
    np.testing.assert_array_equal(shifted[1][~nonzero], base[1][~nonzero])
    for g in (0, 2, 3):
        np.testing.assert_array_equal(shifted[g], base[g])


@pytest.mark.parametrize("entry", ENTRIES)
def test_out_fully_overwritten_and_empty_zero(entry):
    cfg = W.make_random(3, 256, 512, 512, [0, 512, 0], seed=3, device=DEV)
    say("empty experts [%s]" % entry)
    out = torch.empty((3, 256, 512), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(0x7FC0)
    mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, plain=(entry == "plain"))
    torch.cuda.synchronize()
    bits = bf16_bits(out)
    assert (bits[0] == 0).all() and (bits[2] == 0).all()
    assert np.isfinite(bits[1].astype(np.uint32)).all() and (bits[1] != 0x7FC0).all()


@pytest.mark.parametrize("entry", ENTRIES)
def test_no_tokens(entry):
    """M = 0: every expert is empty and the output is exact +0 (the kernel
    writes it; no operand byte is read)."""
    E, N, K = 3, 272, 528
    e = lambda *shape: torch.empty(shape, dtype=torch.uint8, device=DEV)
    offs = torch.zeros(E, dtype=torch.int32, device=DEV)
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN_I16)
    say("no tokens [%s]" % entry)
    mxw.wgrad(e(N, 0), e(N, 0), e(K, 0), e(K, 0), offs, out=out, plain=(entry == "plain"))
    torch.cuda.synchronize()
    assert (bf16_bits(out) == 0).all()


@pytest.mark.parametrize("entry", ENTRIES)
def test_all_experts_empty(entry):
    cfg = W.make_random(2, 256, 256, 64, [0, 0], seed=1, device=DEV)
    say("all experts empty [%s]" % entry)
    bits = bf16_bits(run_gpu(cfg, entry=entry))
    assert (bits == 0).all()
