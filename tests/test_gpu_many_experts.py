"""Expert counts above one wavefront (needs an MI355X).

The schedulers scan the experts 64 at a time (longest-first ranking, column
mode's compact lists and cost prefix, the row-ragged GEMM's tile prefix and
expert lookup). These cases use up to the 256-expert maximum, with many empty
experts, and compare every output with the oracle.
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


def sizes_for(rng, E, total, unit, empty=0.3):
    w = rng.random(E) ** 3
    w[rng.random(E) < empty] = 0.0
    w[0] = max(w[0], 0.5)
    s = np.floor(w / w.sum() * (total // unit)).astype(np.int64) * unit
    return s


def u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("entry", ["ws", "plain"])
@pytest.mark.parametrize("E,N,K,M,mode", [
    (256, 16, 48, 16384, "per_tile"),
    (130, 32, 16, 8192, "per_tile"),
    (70, 16, 16, 8192 * 70, "column"),
])
def test_wgrad_many_experts(E, N, K, M, mode, entry):
    rng = np.random.default_rng(4000 + E)
    sizes = sizes_for(rng, E, M, 32)
    cfg = W.make_random(E, N, K, M, sizes, seed=4100 + E, device=DEV)
    ncol = mxw.columns(E, M, N, K)
    assert (ncol > 0) == (mode == "column")
    say("wgrad many experts [%s]: E=%d N=%d K=%d M=%d columns=%d empty=%d" % (
        entry, E, N, K, M, 0 if entry == "plain" else ncol, int((sizes == 0).sum())))
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, plain=(entry == "plain"))
    torch.cuda.synchronize()
    bits = bf16_bits(out)
    ref = oracle.wgrad_f64(*(cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs")))
    check_close(bits, ref, what="wgrad E=%d" % E)
    assert (bits[sizes == 0] == 0).all()


@pytest.mark.parametrize("entry", ["ws", "plain"])
def test_bf16_wgrad_256_experts(entry):
    E, N, K, M = 256, 16, 32, 8192
    rng = np.random.default_rng(4200)
    sizes = sizes_for(rng, E, M, 16)
    cfg = W.make_bf16(E, N, K, M, sizes, seed=4201, device=DEV)
    say("bf16 wgrad 256 experts: M=%d" % M)
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.wgrad_bf16(cfg["A"], cfg["B"], cfg["offs"], out=out, plain=(entry == "plain"))
    torch.cuda.synchronize()
    bits = bf16_bits(out)
    ref = oracle.bf16_wgrad_f64(u16(cfg["A"]), u16(cfg["B"]), cfg["offs"].cpu().numpy())
    check_close(bits, ref, what="bf16 wgrad E=256 [%s]" % entry)
    assert (bits[sizes == 0] == 0).all()


def test_rows_256_experts():
    E, R, C, N = 256, 3000, 64, 32
    rng = np.random.default_rng(4300)
    sizes = sizes_for(rng, E, R - 100, 1)
    cfg = W.make_rows(E, R, C, N, sizes, seed=4301, device=DEV)
    used = int(sizes.sum())
    say("rows 256 experts: R=%d used=%d" % (R, used))
    out = torch.empty((R, N), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.fwd(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out)
    torch.cuda.synchronize()
    bits = bf16_bits(out)
    ref = oracle.rows_f64(*(cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs")))
    check_close(bits[:used], ref[:used], what="rows E=256")
    assert (bits[used:] == BF16_NAN).all()


def test_quantize_256_experts_offs():
    E, M, H = 256, 2048, 64
    offs = torch.tensor(np.minimum(np.arange(1, E + 1) * 8, 1600).astype(np.int32) // 32 * 32, device=DEV)
    g = torch.Generator().manual_seed(4400)
    x = torch.randn((M, H), generator=g).to(torch.bfloat16)
    x[1600:] = float("nan")
    say("quantise with 256-expert offs")
    q, s = mxw.quantize_tokens(x.to(DEV), offs)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_tokens(x.view(torch.int16).numpy().view(np.uint16), used=int(offs[-1]))
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("E,live", [
    (65, {64: 777}),
    (130, {0: 300, 63: 513, 64: 256, 127: 1, 128: 700, 129: 17}),
    (256, {255: 1000}),
    (256, {0: 5, 64: 600, 128: 257, 192: 3, 255: 511}),
])
def test_rows_chunk_boundaries(E, live):
    """The row-ragged GEMM's tile prefix runs in 64-expert chunks (a scan per
    chunk plus the carry) and its expert lookup takes the last hit over the
    chunks: live experts only on either side of the chunk edges, several of
    them spanning more than one 256-row tile, every other expert empty."""
    sizes = np.zeros(E, np.int64)
    for g, n in live.items():
        sizes[g] = n
    used = int(sizes.sum())
    R, C, N = used + 64, 64, 48
    cfg = W.make_rows(E, R, C, N, sizes, seed=4500 + E + len(live), device=DEV)
    say("rows chunk edges: E=%d live=%s R=%d" % (E, sorted(live), R))
    out = torch.empty((R, N), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.fwd(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out)
    torch.cuda.synchronize()
    bits = bf16_bits(out)
    ref = oracle.rows_f64(*(cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs")))
    check_close(bits[:used], ref[:used], what="rows chunk edges E=%d" % E)
    assert (bits[used:] == BF16_NAN).all()


def test_wgrad_column_mode_chunk_boundaries():
    """Column mode's compact lists and cost prefix are built by 64-lane scans
    with a carry: the live experts sit at 63, 64 and 69 (one long window
    starting at an odd multiple of 32), the rest are empty."""
    E, N, K = 70, 16, 16
    M = 8192 * E
    sizes = np.zeros(E, np.int64)
    sizes[0] = 32
    sizes[63] = 8192 * 20 + 32
    sizes[64] = 8192 * 30 + 160
    sizes[69] = 8192 * 10
    assert mxw.columns(E, M, N, K) > 0
    cfg = W.make_random(E, N, K, M, sizes, seed=4600, device=DEV)
    ref = oracle.wgrad_f64(*(cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs")))
    for entry in ("ws", "plain"):
        say("wgrad column-mode chunk edges [%s]: E=%d M=%d" % (entry, E, M))
        out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
        out.view(torch.int16).fill_(BF16_NAN)
        mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, plain=(entry == "plain"))
        torch.cuda.synchronize()
        bits = bf16_bits(out)
        check_close(bits, ref, what="column-mode chunk edges [%s]" % entry)
        assert (bits[sizes == 0] == 0).all()
