"""The entry points inside a captured HIP graph (needs an MI355X).

None of them records a memset, allocates or synchronises; the workspace
entries' workspace comes from torch's allocator (inside the capture, its graph
pool).  Every replay, with eager work and synchronisation between replays,
must equal the eager result bit for bit.  (A fresh process whose first library
calls are captured is in test_gpu_boundary.py.)
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


@pytest.mark.parametrize("plain", [False, True])
@pytest.mark.parametrize("mode", ["per_tile", "column"])
def test_wgrad_graph_replay(mode, plain):
    if mode == "column":
        cfg = W.make_random(2, 512, 768, 16416, [8992, 7392], seed=1300, device=DEV)
        assert mxw.columns(cfg["E"], cfg["M"], cfg["N"], cfg["K"]) > 0
    else:
        cfg = W.make_random(3, 272, 528, 1024, [96, 0, 800], seed=1301, device=DEV)
        assert mxw.columns(cfg["E"], cfg["M"], cfg["N"], cfg["K"]) == 0
    out = torch.empty((cfg["E"], cfg["N"], cfg["K"]), dtype=torch.bfloat16, device=DEV)
    say("graph wgrad %s plain=%s" % (mode, plain))
    replay_check(lambda: mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, plain=plain),
                 [out], "wgrad %s plain=%s" % (mode, plain))


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


@pytest.mark.parametrize("plain", [False, True])
@pytest.mark.parametrize("mode", ["per_tile", "column"])
def test_bf16_graph_replay(mode, plain):
    if mode == "column":
        cfg = W.make_bf16(2, 512, 768, 16416, [8992, 7392], seed=1303, device=DEV)
        assert mxw.columns(cfg["E"], 2 * cfg["M"], cfg["N"], cfg["K"]) > 0
    else:
        cfg = W.make_bf16(3, 272, 528, 1024, [96, 0, 800], seed=1304, device=DEV)
        assert mxw.columns(cfg["E"], 2 * cfg["M"], cfg["N"], cfg["K"]) == 0
    out = torch.empty((cfg["E"], cfg["N"], cfg["K"]), dtype=torch.bfloat16, device=DEV)
    say("graph bf16 wgrad %s plain=%s" % (mode, plain))
    replay_check(lambda: mxw.wgrad_bf16(cfg["A"], cfg["B"], cfg["offs"], out=out, plain=plain), [out],
                 "bf16 wgrad %s plain=%s" % (mode, plain))
