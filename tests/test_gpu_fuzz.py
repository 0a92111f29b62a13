"""Seeded random shapes for every entry point against the oracle (needs an
MI355X).  Shapes, routings, empty experts, unaligned row boundaries and
padding garbage are drawn from fixed seeds; every case prints its parameters
before it launches.  The weight-gradient cases include shapes that select
column mode (long experts on few tiles).
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle
import workloads as W
from helpers import BF16_NAN, bf16_bits, check_close

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def random_sizes(rng, E, total, unit, empty_prob=0.2):
    """E sizes, multiples of `unit`, summing to at most `total`."""
    w = rng.dirichlet(np.full(E, 1.0))
    w[rng.random(E) < empty_prob] = 0.0
    if w.sum() == 0:
        w[0] = 1.0
    units = int(total * rng.uniform(0.7, 1.0)) // unit
    s = np.floor(w / w.sum() * units).astype(np.int64) * unit
    return s


@pytest.mark.parametrize("seed", range(24))
def test_wgrad_random_shapes(seed):
    rng = np.random.default_rng(2000 + seed)
    if seed % 3 == 0:  # column mode: long experts, few tiles
        E = int(rng.integers(1, 4))
        N = 16 * int(rng.integers(1, 33))
        K = 16 * int(rng.integers(1, 49))
        M = 32 * int(rng.integers(8192 * E // 32 + 1, 8192 * E // 32 + 400))
    else:
        E = int(rng.integers(1, 41))
        N = 16 * int(rng.integers(1, 50))
        K = 16 * int(rng.integers(1, 50))
        M = 32 * int(rng.integers(1, 120))
    sizes = random_sizes(rng, E, M, 32)
    cfg = W.make_random(E, N, K, M, sizes, seed=2100 + seed, device=DEV)
    used = int(sizes.sum())
    cfg["A"][:, used:] = 0x7F  # NaN codes past the last expert
    cfg["sB"][:, used // 32:] = 0xFF
    plain = bool(seed % 2)
    # every fourth workspace case reads row-padded operands (ld = M + 32 k)
    ld = M + 32 * int(rng.integers(1, 9)) if (not plain and seed % 4 == 2) else M
    say("wgrad fuzz %d: E=%d N=%d K=%d M=%d ld=%d used=%d columns=%d plain=%s" % (
        seed, E, N, K, M, ld, used, mxw.columns(E, M, N, K), plain))
    ops = {k: cfg[k] for k in ("A", "sA", "B", "sB")}
    if ld != M:
        for k, div in (("A", 1), ("B", 1), ("sA", 32), ("sB", 32)):
            buf = torch.full((cfg[k].shape[0], ld // div), 0x7F, dtype=torch.uint8, device=DEV)
            buf[:, :M // div] = cfg[k]
            ops[k] = buf[:, :M // div]
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.wgrad(ops["A"], ops["sA"], ops["B"], ops["sB"], cfg["offs"], out=out, plain=plain)
    torch.cuda.synchronize()
    bits = bf16_bits(out)
    ref = oracle.wgrad_f64(*(cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs")))
    check_close(bits, ref, what="wgrad fuzz %d" % seed)
    for g in range(E):
        if sizes[g] == 0:
            assert (bits[g] == 0).all()


@pytest.mark.parametrize("seed", range(10))
def test_fwd_random_shapes(seed):
    rng = np.random.default_rng(2200 + seed)
    E = int(rng.integers(1, 21))
    R = int(rng.integers(1, 3000))
    C = 32 * int(rng.integers(1, 40))
    N = 16 * int(rng.integers(1, 40))
    sizes = random_sizes(rng, E, R, 1)
    cfg = W.make_rows(E, R, C, N, sizes, seed=2300 + seed, device=DEV)
    used = int(sizes.sum())
    cfg["A"][used:] = 0x7F
    say("fwd fuzz %d: E=%d R=%d C=%d N=%d used=%d" % (seed, E, R, C, N, used))
    out = torch.empty((R, N), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.fwd(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out)
    torch.cuda.synchronize()
    bits = bf16_bits(out)
    ref = oracle.rows_f64(*(cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs")))
    check_close(bits[:used], ref[:used], what="fwd fuzz %d" % seed)
    assert (bits[used:] == BF16_NAN).all()


@pytest.mark.parametrize("seed", range(12))
def test_quantize_random_shapes(seed):
    """Random shapes and padding, with row strides (multiples of 256 tokens,
    those plus 128, M plus a random multiple of 32) and scale-plane offsets
    (0, 8, 4 or 1 bytes into its buffer) such that the 8-byte, 4-byte and
    byte scale stores all run; the padding columns and the
    bytes around the scale plane keep their poison."""
    rng = np.random.default_rng(2400 + seed)
    M = 32 * int(rng.integers(1, 200))
    H = 16 * int(rng.integers(1, 80))
    used = 32 * int(rng.integers(0, M // 32 + 1))
    # seeds 0-3: ld a multiple of 256; 4-7: a multiple of 256 plus 128; 8-11: M plus a random pad
    pad = 32 * int(rng.integers(0, 9))
    ld = [-(-M // 256) * 256, -(-M // 256) * 256 + 128, M + pad][(seed // 4) % 3]
    soff = [0, 8, 4, 1][seed % 4]
    g = torch.Generator().manual_seed(2500 + seed)
    x = (torch.randn((M, H), generator=g) * torch.exp2(torch.randint(-30, 30, (1, H), generator=g).float()))
    x = x.to(torch.bfloat16)
    x[used:] = float("nan")
    say("quant fuzz %d: M=%d H=%d used=%d ld=%d s offset %d" % (seed, M, H, used, ld, soff))
    qbuf = torch.full((H, ld), 0xAA, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((H * (ld // 32) + 16,), 0xAA, dtype=torch.uint8, device=DEV)
    splane = sbuf[soff:soff + H * (ld // 32)].view(H, ld // 32)
    q, s = mxw.quantize_tokens(x.to(DEV), torch.tensor([used], dtype=torch.int32, device=DEV),
                               q=qbuf[:, :M], s=splane[:, :M // 32], ld=ld)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_tokens(x.view(torch.int16).numpy().view(np.uint16), used=used)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    assert (qbuf[:, M:] == 0xAA).all().item(), "codes written past M"
    assert (splane[:, M // 32:] == 0xAA).all().item(), "scales written past M / 32"
    sh = sbuf.cpu().numpy()
    assert (sh[:soff] == 0xAA).all() and (sh[soff + H * (ld // 32):] == 0xAA).all(), "bytes around s written"


@pytest.mark.parametrize("seed", range(8))
def test_bf16_wgrad_random_shapes(seed):
    rng = np.random.default_rng(2600 + seed)
    if seed % 4 == 0:  # column mode: long experts, few tiles
        E = int(rng.integers(1, 4))
        N = 16 * int(rng.integers(1, 33))
        K = 16 * int(rng.integers(1, 49))
        M = 16 * int(rng.integers(4096 * E // 16 + 1, 4096 * E // 16 + 400))
    else:
        E = int(rng.integers(1, 41))
        N = 16 * int(rng.integers(1, 50))
        K = 16 * int(rng.integers(1, 50))
        M = 16 * int(rng.integers(1, 200))
    sizes = random_sizes(rng, E, M, 16)
    cfg = W.make_bf16(E, N, K, M, sizes, seed=2700 + seed, device=DEV)
    used = int(sizes.sum())
    cfg["A"].view(torch.int16)[:, used:] = 0x7FC0  # NaN past the last expert
    cfg["B"].view(torch.int16)[:, used:] = -128    # 0xFF80, -inf
    say("bf16 fuzz %d: E=%d N=%d K=%d M=%d used=%d columns(2M)=%d" % (seed, E, N, K, M, used,
                                                                       mxw.columns(E, 2 * M, N, K)))
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.wgrad_bf16(cfg["A"], cfg["B"], cfg["offs"], out=out, plain=bool(seed % 2))
    torch.cuda.synchronize()
    bits = bf16_bits(out)
    u16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.bf16_wgrad_f64(u16(cfg["A"]), u16(cfg["B"]), cfg["offs"].cpu().numpy())
    check_close(bits, ref, what="bf16 fuzz %d" % seed)
    for g in range(E):
        if sizes[g] == 0:
            assert (bits[g] == 0).all()
