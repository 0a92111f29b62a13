"""The weight gradient's two scale paths (needs an MI355X).

With long experts (M >= 4096 E) or scale rows that are not 16-byte aligned
(M % 512 != 0) the library first rewrites the scale planes so that each
workgroup's scale loads read consecutive bytes; otherwise the K-loop reads the
caller's planes directly.  Both feed the same scale bytes to the same MFMA
sequence, so on one problem they must give identical bits.
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


def run(cfg, offs):
    E = offs.shape[0]
    out = torch.empty((E, cfg["N"], cfg["K"]), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], offs, out=out)
    torch.cuda.synchronize()
    return out


def test_shuffled_and_direct_scales_bitwise_equal():
    """E = 1 with M = 8192 takes the shuffled path (M >= 4096 E); the same
    operands with a second, empty expert take the direct one.  N x K is large
    enough that both run one workgroup per tile."""
    N, K, M = 8192, 8448, 8192
    cfg = W.make_random(1, N, K, M, [8192 - 96], seed=3100, device=DEV)
    cfg["A"][:, 8192 - 96:] = 0x7F  # NaN codes and scales in the padding
    cfg["sA"][:, (8192 - 96) // 32:] = 0xFF
    assert mxw.columns(1, M, N, K) == 0 and mxw.columns(2, M, N, K) == 0
    say("scale paths: E=1 (shuffled) vs E=2 (direct), N=%d K=%d M=%d" % (N, K, M))
    one = run(cfg, cfg["offs"])
    two = run(cfg, torch.cat([cfg["offs"], cfg["offs"]]))
    assert torch.equal(one[0].view(torch.int16), two[0].view(torch.int16))
    assert (two[1].view(torch.int16) == 0).all().item()
    assert torch.isfinite(one.float()).all().item()


@pytest.mark.parametrize("E,N,K,M,sizes", [
    (2, 272, 528, 8224, [4000, 4128]),          # M / 32 = 257 bytes per scale row (odd), M % 512 != 0
    (3, 144, 400, 12320, [0, 5000 // 32 * 32, 6112]),  # padding tokens with NaN scales, an empty expert
    (1, 16, 48, 4128, [4096]),                  # the smallest tiles, M % 512 == 32
])
def test_shuffled_scales_odd_strides(E, N, K, M, sizes):
    cfg = W.make_random(E, N, K, M, sizes, seed=3200 + M, device=DEV)
    used = int(np.sum(sizes))
    cfg["sA"][:, used // 32:] = 0xFF
    cfg["sB"][:, used // 32:] = 0xFF
    cfg["B"][:, used:] = 0xFF
    say("shuffled scales: E=%d N=%d K=%d M=%d used=%d" % (E, N, K, M, used))
    bits = bf16_bits(run(cfg, cfg["offs"]))
    ref = oracle.wgrad_f64(*(cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs")))
    check_close(bits, ref, what="shuffled scales M=%d" % M)
    for g in range(E):
        if sizes[g] == 0:
            assert (bits[g] == 0).all()
