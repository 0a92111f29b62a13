"""GPU parity of the token-axis MXFP8 quantiser against the CPU oracle (needs
an MI355X).  Codes and scales are bytes: every case compares them bit for
bit.  The full-size cases check a seeded subset of hidden columns against the
oracle, all columns against the input generator's separate quantiser, and run
the quantised operands through the weight gradient end to end.
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle
import workloads as W
from test_oracle_quant_pins import tricky_block

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def to_bits(x):
    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_quant(x, offs=None):
    q = torch.full((x.shape[1], x.shape[0]), 0xAA, dtype=torch.uint8, device=DEV)  # poison
    s = torch.full((x.shape[1], x.shape[0] // 32), 0xAA, dtype=torch.uint8, device=DEV)
    mxw.quantize_tokens(x, offs, q=q, s=s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


QUANT_CASES = [
    # M, H, used (None = all), value kind
    (128, 128, None, "normal"),
    (96, 144, 64, "normal"),        # M % 128 != 0, H % 128 != 0, padding tokens
    (1024, 1408, 1000 // 32 * 32, "wide"),  # the 16B hidden width, wide per-block ranges
    (32, 16, None, "tricky"),       # the smallest shapes, with ties / saturation / subnormals
    (640, 272, None, "tricky"),
    (256, 64, 0, "normal"),         # every token is padding
]


def make_x(M, H, kind, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        x = torch.randn((M, H), generator=g)
    elif kind == "wide":
        x = torch.randn((M, H), generator=g) * torch.exp2(torch.randint(-40, 40, (M // 32, 1, H), generator=g)
                                                          .float()).repeat_interleave(32, 0).reshape(M, H)
    else:
        rng = np.random.default_rng(seed)
        xs = np.zeros((M, H))
        for h in range(H):
            for b in range(M // 32):
                xs[32 * b:32 * b + 32, h] = tricky_block(rng, int(rng.integers(-60, 60)))
        x = torch.from_numpy(xs)
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("case", range(len(QUANT_CASES)))
def test_quantize_matches_oracle_bitwise(case):
    M, H, used, kind = QUANT_CASES[case]
    x = make_x(M, H, kind, 1000 + case)
    if used is not None:
        x[used:] = float("nan")  # garbage past the last expert
    offs = None if used is None else torch.tensor([used // 2 // 32 * 32, used], dtype=torch.int32, device=DEV)
    say("quant case %d: M=%d H=%d used=%s %s" % (case, M, H, used, kind))
    q, s = run_quant(x.to(DEV), offs)
    rq, rs = oracle.quantize_tokens(to_bits(x), used=used)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)


def test_quantize_repeat_and_offs_none_equal_full():
    x = make_x(512, 256, "normal", 1100).to(DEV)
    say("quant repeat")
    a = run_quant(x)
    b = run_quant(x, torch.tensor([512], dtype=torch.int32, device=DEV))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.slow
def test_quantize_full_size_and_end_to_end():
    """16B shapes: dY [196608, 1408] and X [196608, 2048] quantised on the GPU
    equal the input generator's operands (the benchmark's inputs) byte for byte,
    a seeded subset of hidden columns equals the oracle, and the weight gradient
    of the GPU-quantised operands equals the one of the generator's."""
    cfg = W.make_config("16b_24k", device=DEV)
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    g = torch.Generator(device=DEV)
    g.manual_seed(1200)
    dy = (torch.randn((M, N), generator=g, device=DEV)).to(torch.bfloat16)
    xx = (0.5 * torch.randn((M, K), generator=g, device=DEV)).to(torch.bfloat16)
    say("quant full size: dY [%d, %d], X [%d, %d]" % (M, N, M, K))
    qa, sa = mxw.quantize_tokens(dy, cfg["offs"])
    qb, sb = mxw.quantize_tokens(xx, cfg["offs"])
    torch.cuda.synchronize()
    # against the generator's quantiser (whole planes)
    for name, qq, ss, src in (("dY", qa, sa, dy), ("X", qb, sb, xx)):
        wq, ws = W.quantize_rows(src.t().contiguous())
        assert torch.equal(qq, wq), name
        assert torch.equal(ss, ws), name
    # against the oracle on seeded hidden columns
    rng = np.random.default_rng(1201)
    cols = np.sort(rng.choice(N, 12, replace=False))
    rq, rs = oracle.quantize_tokens(to_bits(dy[:, torch.from_numpy(cols).to(DEV)]), used=int(cfg["offs"][-1]))
    np.testing.assert_array_equal(qa[torch.from_numpy(cols).to(DEV)].cpu().numpy(), rq)
    np.testing.assert_array_equal(sa[torch.from_numpy(cols).to(DEV)].cpu().numpy(), rs)
    # end to end: identical operands give identical weight gradients
    say("quant end to end: two weight-gradient launches")
    w1 = mxw.wgrad(qa, sa, qb, sb, cfg["offs"])
    wq_a, ws_a = W.quantize_rows(dy.t().contiguous())
    wq_b, ws_b = W.quantize_rows(xx.t().contiguous())
    w2 = mxw.wgrad(wq_a, ws_a, wq_b, ws_b, cfg["offs"])
    torch.cuda.synchronize()
    assert torch.equal(w1.view(torch.int16), w2.view(torch.int16))


STRIDE_CASES = [
    # M, H, ld - M, byte offset of s in its buffer
    (640, 272, 128, 0),   # ld % 256 == 0, s 8-byte aligned: one 8-byte scale store per row and whole tile
    (640, 272, 128, 4),   # s only 4-byte aligned: two 4-byte stores
    (640, 272, 256, 0),   # ld % 256 == 128 (rows M + 128 tokens apart at M % 256 == 0): two 4-byte stores
    (640, 272, 32, 0),    # ld / 32 odd: scale rows start at any byte, byte stores
    (640, 272, 0, 1),     # s itself not aligned, byte stores
    (608, 80, 64, 3),     # a partial last token tile as well
    (1024, 64, 0, 0),     # whole tiles only, the 8-byte stores throughout
]


@pytest.mark.parametrize("case", range(len(STRIDE_CASES)))
def test_quantize_row_stride_and_scale_alignment(case):
    """Codes and scales written into [H, ld] / [H, ld/32] rows, the scale
    plane at any byte offset: every byte equals the oracle's, and the padding
    columns and the bytes around the scale plane keep their poison."""
    M, H, pad, soff = STRIDE_CASES[case]
    ld = M + pad
    x = make_x(M, H, "normal", 1300 + case)
    used = M - 32
    x[used:] = float("nan")
    offs = torch.tensor([used // 64 * 32, used], dtype=torch.int32, device=DEV)
    say("quant strides: M=%d H=%d ld=%d s offset %d" % (M, H, ld, soff))
    qbuf = torch.full((H, ld), 0xAA, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((H * (ld // 32) + 8,), 0xAA, dtype=torch.uint8, device=DEV)
    s = sbuf[soff:soff + H * (ld // 32)].view(H, ld // 32)[:, :M // 32]
    q, s2 = mxw.quantize_tokens(x.to(DEV), offs, q=qbuf[:, :M], s=s, ld=ld)
    torch.cuda.synchronize()
    assert s2.data_ptr() == s.data_ptr()
    rq, rs = oracle.quantize_tokens(to_bits(x), used=used)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    qh = qbuf.cpu().numpy()
    assert (qh[:, M:] == 0xAA).all(), "codes written past M"
    sh = sbuf.cpu().numpy()
    plane = sh[soff:soff + H * (ld // 32)].reshape(H, ld // 32)
    assert (plane[:, M // 32:] == 0xAA).all(), "scales written past M / 32"
    assert (sh[:soff] == 0xAA).all() and (sh[soff + H * (ld // 32):] == 0xAA).all(), "bytes around s written"
