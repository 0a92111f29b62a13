"""The three entry points inside a captured HIP graph (needs an MI355X).

None of them records a memset or allocates per call; column mode's workspace is
allocated by the first column-mode call on a device, so each case makes one
eager call before capturing.  Every replay, with eager work and synchronisation
between replays, must equal the eager result bit for bit.
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def replay_check(fn, outs, name, replays=3):
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    for o in outs:
        o.zero_()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(replays):
        for o in outs:
            o.fill_(0x7F if o.dtype == torch.uint8 else float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), "%s: replay %d differs" % (name, r)


@pytest.mark.parametrize("mode", ["per_tile", "column"])
def test_wgrad_graph_replay(mode):
    if mode == "column":
        cfg = W.make_random(2, 512, 768, 16416, [8992, 7392], seed=1300, device=DEV)
        assert mxw.columns(cfg["E"], cfg["M"], cfg["N"], cfg["K"]) > 0
    else:
        cfg = W.make_random(3, 272, 528, 1024, [96, 0, 800], seed=1301, device=DEV)
        assert mxw.columns(cfg["E"], cfg["M"], cfg["N"], cfg["K"]) == 0
    out = torch.empty((cfg["E"], cfg["N"], cfg["K"]), dtype=torch.bfloat16, device=DEV)
    say("graph wgrad %s" % mode)
    replay_check(lambda: mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out), [out],
                 "wgrad " + mode)


def test_fwd_graph_replay():
    cfg = W.make_rows(4, 1100, 160, 512, [1, 255, 257, 587], seed=1302, device=DEV)  # every row written
    out = torch.zeros((cfg["R"], cfg["N"]), dtype=torch.bfloat16, device=DEV)
    say("graph fwd")
    replay_check(lambda: mxw.fwd(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out), [out], "fwd")


def test_quantize_graph_replay():
    x = torch.randn((640, 272), device=DEV).to(torch.bfloat16)
    offs = torch.tensor([320, 608], dtype=torch.int32, device=DEV)
    q = torch.empty((272, 640), dtype=torch.uint8, device=DEV)
    s = torch.empty((272, 20), dtype=torch.uint8, device=DEV)
    say("graph quantize")
    replay_check(lambda: mxw.quantize_tokens(x, offs, q=q, s=s), [q, s], "quantize")


@pytest.mark.parametrize("mode", ["per_tile", "column"])
def test_bf16_graph_replay(mode):
    if mode == "column":
        cfg = W.make_bf16(2, 512, 768, 16416, [8992, 7392], seed=1303, device=DEV)
        assert mxw.columns(cfg["E"], 2 * cfg["M"], cfg["N"], cfg["K"]) > 0
    else:
        cfg = W.make_bf16(3, 272, 528, 1024, [96, 0, 800], seed=1304, device=DEV)
        assert mxw.columns(cfg["E"], 2 * cfg["M"], cfg["N"], cfg["K"]) == 0
    out = torch.empty((cfg["E"], cfg["N"], cfg["K"]), dtype=torch.bfloat16, device=DEV)
    say("graph bf16 wgrad %s" % mode)
    replay_check(lambda: mxw.wgrad_bf16(cfg["A"], cfg["B"], cfg["offs"], out=out), [out], "bf16 wgrad " + mode)


def test_wgrad_graph_survives_scale_workspace_growth():
    """A graph captured on a shape that uses the scale pre-shuffle keeps
    replaying correctly after a larger call has replaced the device's scale
    workspace (replaced buffers stay allocated)."""
    small = W.make_random(2, 272, 528, 8224, [4000, 4128], seed=1305, device=DEV)
    assert mxw.scale_shuffle(2, 8224)
    out = torch.empty((2, 272, 528), dtype=torch.bfloat16, device=DEV)
    fn = lambda: mxw.wgrad(small["A"], small["sA"], small["B"], small["sB"], small["offs"], out=out)
    say("graph + scale workspace growth: capture on the small shape")
    fn()
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # a larger call: (4 + 4) bands x 128 groups x 4 KiB of shuffled scales
    big = W.make_random(4, 1024, 1024, 65536, [16384, 0, 30000 // 32 * 32, 18944], seed=1306, device=DEV)
    assert mxw.scale_shuffle(4, 65536)
    say("graph + scale workspace growth: larger eager call, then replays")
    ob = mxw.wgrad(big["A"], big["sA"], big["B"], big["sB"], big["offs"])
    torch.cuda.synchronize()
    assert torch.isfinite(ob.float()).all().item()
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "replay %d after growth differs" % r
    # the small shape eagerly (now on the larger buffer) gives the same bits
    fn()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
