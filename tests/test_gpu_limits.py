"""The largest sizes the C ABI accepts (needs an MI355X).

M = MXW_MAX_TOKENS (2^23) E4M3 tokens makes every operand row 8 MiB long, so a
whole 256-row tile's rows sit up to 255 x 8 MiB into its buffer range and its
token offsets reach 2^23 - 128: the largest offsets the 32-bit buffer
arithmetic meets.  One expert spans almost all tokens (checked at sampled
outputs, each a fresh 8-million-term fp64 sum by the oracle), a short one ends
2,048 tokens before M (checked whole), the first is empty, and the padding
holds NaN codes and 0xFF scales.  Both entry points (column mode with the
scale pre-shuffle, and one workgroup per tile).  The bf16 weight gradient is
checked the same way at its own maximum, 2^22 tokens (8 MiB rows); the weight
gradient at the largest widths (N = K = 65,536: 196,608 workgroups, 8 GiB of
output per expert); the row-ragged GEMM at the largest row count (2^23); and
the quantiser at the largest token count and hidden width.
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle
import workloads as W
from helpers import ENTRIES, bf16_bits, check_close, run_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAX_TOKENS = 8 * 1024 * 1024  # MXW_MAX_TOKENS


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def rows_to_host(t, rows):
    return t[torch.as_tensor(rows, device=t.device)].cpu().numpy()


@pytest.fixture(scope="module")
def big():
    N = K = 256
    M = MAX_TOKENS
    sizes = [0, M - 4096, 2048]  # the last 2,048 tokens are padding
    say("max tokens: generating E=3 N=%d K=%d M=%d" % (N, K, M))
    cfg = W.make_random(3, N, K, M, sizes, seed=8800, device=DEV)
    cfg["A"][:, M - 2048:] = 0x7F  # NaN codes and scales past the last expert
    cfg["sA"][:, (M - 2048) // 32:] = 0xFF
    cfg["sB"][:, (M - 2048) // 32:] = 0xFF
    torch.cuda.synchronize()
    yield cfg
    del cfg
    torch.cuda.empty_cache()


@pytest.mark.parametrize("entry", ENTRIES)
def test_max_tokens_wgrad(big, entry):
    cfg = big
    N, K, M = cfg["N"], cfg["K"], cfg["M"]
    offs = cfg["offs"].cpu().numpy()
    say("max tokens [%s]: launch (columns %d)" % (entry, mxw.columns(3, M, N, K) if entry == "ws" else 0))
    bits = bf16_bits(run_gpu(cfg, entry=entry))
    assert (bits[0] == 0).all(), "empty expert not exact +0"
    # expert 2 whole: the oracle on its own slab of tokens
    lo, hi = int(offs[1]), int(offs[2])
    sl = lambda t, div=1: np.ascontiguousarray(t[:, lo // div:hi // div].cpu().numpy())
    ref2 = oracle.wgrad_f64(sl(cfg["A"]), sl(cfg["sA"], 32), sl(cfg["B"]), sl(cfg["sB"], 32),
                            np.array([hi - lo], np.int32))[0]
    check_close(bits[2], ref2, what="max tokens, short expert [%s]" % entry)
    # expert 1 at sampled outputs (corners and the last row/column included)
    rng = np.random.default_rng(8801)
    n = np.concatenate([[0, 255, 255, 0, 128], rng.integers(0, N, 11)])
    k = np.concatenate([[0, 255, 0, 255, 127], rng.integers(0, K, 11)])
    un, inv_n = np.unique(n, return_inverse=True)
    uk, inv_k = np.unique(k, return_inverse=True)
    say("max tokens [%s]: oracle at %d sampled outputs of the 8M-token expert" % (entry, len(n)))
    ref1 = oracle.wgrad_points(rows_to_host(cfg["A"], un), rows_to_host(cfg["sA"], un),
                               rows_to_host(cfg["B"], uk), rows_to_host(cfg["sB"], uk), offs,
                               np.ones(len(n), np.int32), inv_n.astype(np.int32), inv_k.astype(np.int32))
    got1 = bits[1][n, k]
    check_close(got1, ref1, rms=float(np.sqrt(np.mean(ref1 ** 2))), what="max tokens, long expert [%s]" % entry)


def test_max_tokens_bf16():
    N = K = 256
    M = MAX_TOKENS // 2
    sizes = [M - 4096, 2048]
    say("bf16 max tokens: generating E=2 N=%d K=%d M=%d" % (N, K, M))
    g = torch.Generator(device=DEV)
    g.manual_seed(8810)
    A = torch.randn((N, M), generator=g, device=DEV).to(torch.bfloat16)
    B = torch.randn((K, M), generator=g, device=DEV).to(torch.bfloat16)
    A[:, M - 2048:] = float("nan")
    offs_np = np.cumsum(sizes).astype(np.int32)
    offs = torch.from_numpy(offs_np).to(DEV)
    ref1_slab = lambda t: np.ascontiguousarray(t[:, offs_np[0]:offs_np[1]].view(torch.int16).cpu().numpy().view(np.uint16))
    ref_short = oracle.bf16_wgrad_f64(ref1_slab(A), ref1_slab(B), np.array([2048], np.int32))[0]
    rng = np.random.default_rng(8811)
    n = np.concatenate([[0, 255, 255, 0], rng.integers(0, N, 8)])
    k = np.concatenate([[0, 255, 0, 255], rng.integers(0, K, 8)])
    un, inv_n = np.unique(n, return_inverse=True)
    uk, inv_k = np.unique(k, return_inverse=True)
    h16 = lambda t, rows: rows_to_host(t.view(torch.int16), rows).view(np.uint16)
    ref_long = oracle.bf16_wgrad_points(h16(A, un), h16(B, uk), offs_np, np.zeros(len(n), np.int32),
                                        inv_n.astype(np.int32), inv_k.astype(np.int32))
    for plain in (False, True):
        out = torch.empty((2, N, K), dtype=torch.bfloat16, device=DEV)
        out.view(torch.int16).fill_(0x7FC0)
        say("bf16 max tokens [%s]: launch" % ("plain" if plain else "ws"))
        mxw.wgrad_bf16(A, B, offs, out=out, plain=plain)
        torch.cuda.synchronize()
        bits = bf16_bits(out)
        check_close(bits[1], ref_short, what="bf16 max tokens, short expert")
        check_close(bits[0][n, k], ref_long, rms=float(np.sqrt(np.mean(ref_long ** 2))),
                    what="bf16 max tokens, long expert")
    del A, B
    torch.cuda.empty_cache()


def test_max_width_wgrad():
    """N = K = 65,536, the largest widths: 256 x 256 tiles per expert (65,536
    workgroups) and an 8 GiB bf16 output per expert.  Sampled outputs against
    the oracle (the last tile's last row and column included), and no NaN
    poison left anywhere.  Short windows, so both entry points run one
    workgroup per tile."""
    N = K = 65536
    M = 96
    sizes = [32, 0, 64]
    cfg = W.make_random(3, N, K, M, sizes, seed=8820, device=DEV)
    offs = cfg["offs"].cpu().numpy()
    rng = np.random.default_rng(8821)
    g = np.concatenate([[0, 2, 2, 0], rng.choice([0, 2], 12)])
    n = np.concatenate([[0, N - 1, N - 1, 0], rng.integers(0, N, 12)])
    k = np.concatenate([[0, K - 1, 0, K - 1], rng.integers(0, K, 12)])
    ref = oracle.wgrad_points(cfg["A"].cpu().numpy(), cfg["sA"].cpu().numpy(), cfg["B"].cpu().numpy(),
                              cfg["sB"].cpu().numpy(), offs, g.astype(np.int32), n.astype(np.int32),
                              k.astype(np.int32))
    for entry in ENTRIES:
        out = torch.empty((3, N, K), dtype=torch.bfloat16, device=DEV)
        out.view(torch.int16).fill_(0x7FC0)
        say("max widths [%s]: launch, %d workgroups" % (entry, mxw.grid_size(3, N, K)))
        mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, plain=(entry == "plain"))
        torch.cuda.synchronize()
        assert not torch.isnan(out).any().item(), "NaN poison left in the output"
        assert (out[1].view(torch.int16) == 0).all().item(), "empty expert not exact +0"
        idx = torch.as_tensor(np.stack([g, n, k]), device=DEV)
        got = out[idx[0], idx[1], idx[2]].view(torch.int16).cpu().numpy().view(np.uint16)
        check_close(got, ref, rms=float(np.sqrt(np.mean(ref ** 2))), what="max widths [%s]" % entry)
        del out
        torch.cuda.empty_cache()


def test_max_rows_fwd():
    """The row-ragged GEMM at R = MXW_MAX_ROWS (2^23) rows: row offsets up to
    2^23 x C in the operand and the output, the last expert ending 1,000 rows
    before R (rows past it keep their NaN poison).  Sampled rows against the
    oracle, the last live row included."""
    R, C, N = 8 * 1024 * 1024, 64, 32
    sizes = [R - 5000, 0, 4000]
    cfg = W.make_rows(3, R, C, N, sizes, seed=8830, device=DEV)
    offs = cfg["offs"].cpu().numpy()
    out = torch.empty((R, N), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(0x7FC0)
    say("max rows: launch R=%d C=%d N=%d" % (R, C, N))
    mxw.fwd(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out)
    torch.cuda.synchronize()
    used = int(offs[-1])
    assert torch.isnan(out[used:].float()).all().item(), "rows past the last expert were written"
    assert not torch.isnan(out[:used].float()).any().item(), "a live row was not written"
    rng = np.random.default_rng(8831)
    m = np.concatenate([[0, R - 5001, R - 5000, used - 1], rng.integers(0, used, 12)])
    nn = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, 12)])
    ref = oracle.rows_points(cfg["A"].cpu().numpy(), cfg["sA"].cpu().numpy(), cfg["B"].cpu().numpy(),
                             cfg["sB"].cpu().numpy(), offs, m.astype(np.int32), nn.astype(np.int32))
    idx = torch.as_tensor(np.stack([m, nn]), device=DEV)
    got = out[idx[0], idx[1]].view(torch.int16).cpu().numpy().view(np.uint16)
    check_close(got, ref, rms=float(np.sqrt(np.mean(ref ** 2))), what="max rows")


@pytest.mark.parametrize("M,H", [(MAX_TOKENS, 64), (4096, 65536)])
def test_quantize_limits(M, H):
    """The quantiser at the largest token count (2^23: 8 MiB code rows) and
    the largest hidden width (65,536), with offs ending 4,096 tokens before M
    and NaN in those padding tokens: codes and scales of the first 16 hidden
    columns (and, at the largest width, the last 16) equal the oracle's
    byte for byte."""
    g = torch.Generator(device=DEV)
    g.manual_seed(8840 + H)
    x = torch.randn((M, H), generator=g, device=DEV).to(torch.bfloat16)
    used = M - 4096 if M > 8192 else M - 512
    x[used:] = float("nan")
    offs = torch.tensor([used // 2, used], dtype=torch.int32, device=DEV)
    say("quantiser limits: M=%d H=%d used=%d" % (M, H, used))
    q, s = mxw.quantize_tokens(x, offs)
    torch.cuda.synchronize()
    for c0 in sorted({0, H - 16}):
        xs = x[:, c0:c0 + 16].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        rq, rs = oracle.quantize_tokens(xs, used=used)
        np.testing.assert_array_equal(q[c0:c0 + 16].cpu().numpy(), rq)
        np.testing.assert_array_equal(s[c0:c0 + 16].cpu().numpy(), rs)
    del x, q, s
    torch.cuda.empty_cache()
