"""The no-allocation entry point (needs an MI355X).

mxfp8_wgrad_grouped_noalloc is mxfp8_wgrad_grouped_ws on the library's static
device scratch: the same plan and kernels, so on every call its output must
equal the workspace entry's bit for bit (and both match the oracle).  Two calls
in a row, the second with a smaller input, show that the scratch's leftover
contents from the first call do not leak into the second.  A shape whose
workspace exceeds the scratch is rejected on the host before any launch.
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle
import workloads as W
from helpers import BF16_NAN, bf16_bits, check_close, host

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCRATCH_BYTES = 160 * 1024 * 1024  # MXW_SCRATCH_BYTES
P = 0x10000  # a fake device address: the rejected call never reaches a launch


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def call_noalloc(cfg):
    E, N, K, M = cfg["E"], cfg["N"], cfg["K"], cfg["M"]
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    torch.cuda.synchronize()
    rc = mxw.mxfp8_wgrad_grouped_noalloc(*(cfg[k].data_ptr() for k in ("A", "sA", "B", "sB", "offs")),
                                         E, M, N, K, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, mxw.strerror(rc)
    torch.cuda.synchronize()
    return bf16_bits(out)


def call_ws(cfg):
    E, N, K, M = cfg["E"], cfg["N"], cfg["K"], cfg["M"]
    need = mxw.workspace_size(E, M, N, K)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(BF16_NAN)
    torch.cuda.synchronize()
    rc = mxw.mxfp8_wgrad_grouped_ws(*(cfg[k].data_ptr() for k in ("A", "sA", "B", "sB", "offs")),
                                    E, M, N, K, out.data_ptr(), ws.data_ptr(), need,
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 0, mxw.strerror(rc)
    torch.cuda.synchronize()
    return bf16_bits(out)


def test_noalloc_matches_workspace_entry_two_calls():
    big = W.make_random(8, 1408, 2048, 65536, [12000, 4000, 9600, 0, 11200, 8000, 6400, 14336], seed=5000,
                        device=DEV)
    small = W.make_random(2, 512, 768, 16416, [8992, 7392], seed=5001, device=DEV)
    for cfg in (big, small):
        E, N, K, M = cfg["E"], cfg["N"], cfg["K"], cfg["M"]
        need = mxw.workspace_size(E, M, N, K)
        assert 0 < need <= SCRATCH_BYTES and mxw.columns(E, M, N, K) > 0
    for name, cfg in (("first call (column mode, 135 MiB of scratch)", big),
                      ("second call, smaller (column mode)", small)):
        say("noalloc %s: E=%d N=%d K=%d M=%d" % (name, cfg["E"], cfg["N"], cfg["K"], cfg["M"]))
        got = call_noalloc(cfg)
        want = call_ws(cfg)
        np.testing.assert_array_equal(got, want)
        check_close(got, oracle.wgrad_f64(*host(cfg)), what="noalloc " + name)


def test_noalloc_headline_shape():
    cfg = W.make_config("16b_24k", device=DEV)
    assert mxw.workspace_size(cfg["E"], cfg["M"], cfg["N"], cfg["K"]) <= SCRATCH_BYTES
    say("noalloc 16b_24k")
    np.testing.assert_array_equal(call_noalloc(cfg), call_ws(cfg))


def test_noalloc_rejects_beyond_scratch():
    E, M, N, K = 1, 65536, 65536, 65536  # 512 bands x 128 groups x 4 KiB of shuffled scales
    assert mxw.workspace_size(E, M, N, K) > SCRATCH_BYTES
    say("noalloc rejection (host check, nothing launched)")
    rc = mxw.mxfp8_wgrad_grouped_noalloc(P, P, P, P, P, E, M, N, K, P, torch.cuda.current_stream().cuda_stream)
    assert rc == -7
    assert "scratch" in mxw.strerror(rc)
