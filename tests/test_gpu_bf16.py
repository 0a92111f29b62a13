"""GPU parity of the BF16 contracting ragged dot (the weight gradient on bf16
operands) against the CPU oracle (needs an MI355X).

Same bar as the MXFP8 path: every element within 2^-7 |ref| + 2^-10 rms(ref)
(FP32 accumulation of exact bf16 products, one bf16 rounding of the result),
bit-exact where every partial sum is exact in FP32, bitwise reproducible.
Small cases cover the whole output (NaN-poisoned first); the full-size
workloads are checked on seeded sample points plus the edges of partial tiles.
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle
import workloads as W
from helpers import BF16_NAN, bf16_bits, bf16_to_f64, check_close, tile_pairs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_bf16(cfg, out=None, plain=False):
    E, N, K = cfg["E"], cfg["N"], cfg["K"]
    if out is None:
        out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.wgrad_bf16(cfg["A"], cfg["B"], cfg["offs"], out=out, plain=plain)
    torch.cuda.synchronize()
    return out


def oracle_full(cfg):
    return oracle.bf16_wgrad_f64(u16(cfg["A"]), u16(cfg["B"]), cfg["offs"].cpu().numpy())


BF16_CASES = [
    # E, N, K, M, sizes (multiples of 16, sum <= M)
    (4, 128, 256, 512, [96, 0, 160, 256]),          # the tiny shape, head/tail-masked windows
    (3, 272, 528, 1024, [16, 0, 800]),              # partial N and K tiles, a 16-token expert
    (5, 144, 160, 2048, [48, 208, 0, 1104, 672]),   # boundaries on odd multiples of 16
    (1, 16, 16, 64, [64]),                          # the smallest problem
    (2, 512, 768, 16416, [8992, 7392]),             # long experts: column mode
    (6, 1408, 2048, 768, [128, 0, 96, 32, 256, 64]),  # the 16B widths, short experts
]


@pytest.mark.parametrize("case", range(len(BF16_CASES)))
def test_bf16_ragged_shapes(case):
    E, N, K, M, sizes = BF16_CASES[case]
    cfg = W.make_bf16(E, N, K, M, sizes, seed=2600 + case, device=DEV, std=(1.0, 0.5))
    say("bf16 case %d: E=%d N=%d K=%d M=%d columns(2M)=%d" % (case, E, N, K, M, mxw.columns(E, 2 * M, N, K)))
    ref = oracle_full(cfg)
    for plain in (False, True):
        bits = bf16_bits(run_bf16(cfg, plain=plain))
        stats = check_close(bits, ref, what="bf16 case %d plain=%s" % (case, plain))
        for g in range(E):
            if sizes[g] == 0:
                assert (bits[g] == 0).all()
        print("bf16 case %d plain=%s max_rel %.3e" % (case, plain, stats["max_rel"]))


def test_bf16_column_mode_selected():
    # the column-mode case above really runs in column mode, the others do not
    assert mxw.columns(2, 2 * 16416, 512, 768) > 0
    assert mxw.columns(3, 2 * 1024, 272, 528) == 0


def test_bf16_exact_regime_bitwise():
    """Values in {0, +-0.5, +-1, +-1.5, +-2}: every FP32 partial sum is exact, so
    the output is the oracle's exact result rounded once to bf16, bit for bit."""
    rng = np.random.default_rng(2700)
    E, N, K, M = 3, 272, 528, 1536
    vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 1.5, -1.5, 2.0, -2.0])
    A = torch.from_numpy(rng.choice(vals, (N, M))).to(torch.bfloat16).to(DEV)
    B = torch.from_numpy(rng.choice(vals, (K, M))).to(torch.bfloat16).to(DEV)
    sizes = np.array([400, 0, 1088])
    cfg = dict(E=E, N=N, K=K, M=M, A=A, B=B, offs=torch.from_numpy(np.cumsum(sizes).astype(np.int32)).to(DEV))
    say("bf16 exact regime")
    bits = bf16_bits(run_bf16(cfg))
    np.testing.assert_array_equal(bits, oracle.to_bf16_bits(oracle_full(cfg)))


def test_bf16_bitwise_repeat_and_padding_garbage():
    cfg = W.make_bf16(3, 272, 528, 1024, [96, 0, 800], seed=2800, device=DEV)
    say("bf16 repeat / padding garbage")
    a = bf16_bits(run_bf16(cfg))
    b = bf16_bits(run_bf16(cfg))
    np.testing.assert_array_equal(a, b)
    cfg["A"].view(torch.int16)[:, 896:] = 0x7FC0  # NaN past the last expert
    cfg["B"].view(torch.int16)[:, 896:] = 0x7F80  # +inf
    np.testing.assert_array_equal(bf16_bits(run_bf16(cfg)), a)


@pytest.mark.parametrize("plain", [False, True])
def test_bf16_nan_and_inf_inside_windows(plain):
    """bf16 NaN and -inf values in live tokens: NaN where the oracle (IEEE
    fp64) has NaN, +-inf where it has +-inf (a row of expert 0, a column and
    a row of expert 2), the same values just past offs[E-1] change nothing,
    everything else finite and within tolerance."""
    cfg = W.make_bf16(3, 272, 528, 1024, [96, 0, 800], seed=2801, device=DEV)
    a16, b16 = cfg["A"].view(torch.int16), cfg["B"].view(torch.int16)
    a16[5, 10] = 0x7FC0     # NaN, expert 0
    b16[300, 200] = -128    # 0xFF80 = -inf, expert 2
    a16[9, 500] = 0x7FC0    # NaN, expert 2
    a16[7, 900] = 0x7FC0    # past offs[E-1] = 896
    b16[301, 950] = 0x7F80  # +inf, past
    say("bf16 NaN / inf inside windows [plain=%s]" % plain)
    bits = bf16_bits(run_bf16(cfg, plain=plain))
    u16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.bf16_wgrad_f64(u16(cfg["A"]), u16(cfg["B"]), cfg["offs"].cpu().numpy())
    got = bf16_to_f64(bits)
    bad = ~np.isfinite(ref)
    assert bad.sum() == 528 + 272 + 528 - 1
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
    check_close(np.where(bad, 0, bits).astype(np.uint16), np.where(bad, 0.0, ref), what="bf16 NaN/inf case")


def test_bf16_all_experts_empty():
    cfg = W.make_bf16(2, 256, 256, 64, [0, 0], seed=2900, device=DEV)
    say("bf16 all experts empty")
    assert (bf16_bits(run_bf16(cfg)) == 0).all()


def test_bf16_agrees_with_mxfp8_path_on_shared_values():
    """MXFP8 operands whose decoded values are exact in bf16, fed to both GPU
    paths: the same exact values reach the MFMAs, so both outputs meet the
    tolerance against the one oracle result (the summation orders differ)."""
    cfg = W.make_random(3, 272, 528, 1024, [96, 0, 800], seed=3000, device=DEV)
    A8, sA, B8, sB, offs = (cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs"))
    ref = oracle.wgrad_f64(A8, sA, B8, sB, offs)
    Ab = torch.from_numpy(oracle.decode_plane(A8, sA)).to(torch.bfloat16).to(DEV)
    Bb = torch.from_numpy(oracle.decode_plane(B8, sB)).to(torch.bfloat16).to(DEV)
    assert (oracle.decode_bf16_plane(u16(Ab)) == oracle.decode_plane(A8, sA)).all()  # exact
    say("bf16 vs mxfp8 on shared values")
    bcfg = dict(E=3, N=272, K=528, M=1024, A=Ab, B=Bb, offs=cfg["offs"])
    check_close(bf16_bits(run_bf16(bcfg)), ref, what="bf16 path")
    out8 = mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"])
    torch.cuda.synchronize()
    check_close(bf16_bits(out8), ref, what="mxfp8 path")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["16b_bf16", "16b_1k_bf16"])
def test_bf16_full_size_tiles(name):
    """The 16B shape at full size in the benchmark's launch configuration (the
    workspace entry; column mode at 24,576 tokens per expert): 12 whole
    (tn, tk) output-tile pairs (the four corner pairs plus seeded ones), every
    expert's tile of each, against the oracle run on those tiles' rows."""
    cfg = W.make_bf16_config(name, device=DEV)
    E, N, K, M = cfg["E"], cfg["N"], cfg["K"], cfg["M"]
    say("%s: launch E=%d N=%d K=%d M=%d columns(2M)=%d" % (name, E, N, K, M, mxw.columns(E, 2 * M, N, K)))
    out = run_bf16(cfg)
    assert torch.isfinite(out.float()).all().item()
    bits = bf16_bits(out)
    A, B, offs = u16(cfg["A"]), u16(cfg["B"]), cfg["offs"].cpu().numpy()
    pairs = tile_pairs(cfg, 12, 3)
    say("%s: oracle on %d tile pairs x %d experts" % (name, len(pairs), E))
    refs = {}
    for tn, tk in pairs:
        n0, k0 = 256 * tn, 256 * tk
        refs[(tn, tk)] = oracle.bf16_wgrad_f64(np.ascontiguousarray(A[n0:n0 + 256]),
                                               np.ascontiguousarray(B[k0:k0 + 256]), offs)
    rms = float(np.sqrt(np.mean(np.concatenate([r.ravel() for r in refs.values()]) ** 2)))
    worst = 0.0
    for (tn, tk), r in refs.items():
        n0, k0 = 256 * tn, 256 * tk
        st = check_close(bits[:, n0:n0 + r.shape[1], k0:k0 + r.shape[2]], r, rms=rms,
                         what="%s tile (%d, %d)" % (name, tn, tk))
        worst = max(worst, st["max_rel"])
    print("%s: %d whole tiles, max_rel %.3e" % (name, len(pairs) * E, worst))
