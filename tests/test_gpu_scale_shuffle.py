"""The weight gradient's scale paths (needs an MI355X).

With a workspace, long experts (M >= 4096 E) make the library first rewrite
the scale planes so that each workgroup's scale loads read consecutive bytes;
otherwise, and always without a workspace, the K-loop reads the caller's planes
directly, 16 bytes of 8 K-steps per row (from 16-byte or 4-byte aligned rows,
or, when rows are not a whole number of dwords, from the dword boundary below
each row's group, every scale word then joined from two dwords).  All feed the same scale bytes to the same
MFMA sequence, so on one problem they must give identical bits.
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


def run(cfg, offs, plain=False):
    E = offs.shape[0]
    out = torch.empty((E, cfg["N"], cfg["K"]), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], offs, out=out, plain=plain)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M", [8192, 8192 + 128, 8192 + 160])
def test_shuffled_and_direct_scales_bitwise_equal(M):
    """E = 1 with M >= 4096 takes the shuffled path with a workspace; without
    one the same problem reads the caller's planes (16-byte groups: from
    16-byte or only 4-byte aligned rows when M % 128 == 0, otherwise read a
    dword early).  N x K is large enough that
    the workspace entry runs one workgroup per tile too."""
    N, K = 8192, 8448
    used = 8192 - 96
    cfg = W.make_random(1, N, K, M, [used], seed=3100, device=DEV)
    cfg["A"][:, used:] = 0x7F  # NaN codes and scales in the padding
    cfg["sA"][:, used // 32:] = 0xFF
    assert mxw.columns(1, M, N, K) == 0 and mxw.scale_shuffle(1, M)
    say("scale paths: shuffled (workspace) vs direct (none), N=%d K=%d M=%d" % (N, K, M))
    shuf = run(cfg, cfg["offs"])
    direct = run(cfg, cfg["offs"], plain=True)
    assert torch.equal(shuf.view(torch.int16), direct.view(torch.int16))
    assert torch.isfinite(shuf.float()).all().item()


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
