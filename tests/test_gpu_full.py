"""Full-size parity on whole output tiles (needs an MI355X).

The benchmark's workloads at full size, in the launch configuration bench.py
times (mxfp8_wgrad_grouped_ws with its workspace; the 16B production shape
then runs in column mode), against the oracle on whole 256 x 256 output tiles:

  * 16b_24k (the headline): the whole [8, 1408, 2048] output, so every tile
    of every region that column mode cuts between columns (three or more
    pieces included) is checked, with rms over the whole reference;
  * the other 16B routings (skew 1.2x, 1.7x, balanced, linear ramp), both
    671B shapes and the Zipf ragged-edge stress: 12 (tn, tk) tile pairs each,
    the four corner pairs (first and last tiles of every expert, the partial
    last N tile at 16B) plus seeded random pairs, every expert's tile of each
    pair: 96 to 384 whole tiles per workload; the 256-expert stress at the
    16B shape: the four corner pairs, 1,024 whole tiles; the 16B down
    projection (N = 2048, K = 1408: column mode with 8-row bands of regions);
  * the entry point without a workspace on the headline shape, the same way.

Every element must be finite (no skipped store) and empty experts exact +0;
the tolerance is |gpu - ref| <= 2^-7 |ref| + 2^-10 rms(ref) with rms over the
computed tiles (the whole output for 16b_24k).  The oracle runs on the host
cores (OpenMP), reading the A and B rows of a tile over all tokens.
"""
import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import workloads as W
from helpers import bf16_bits, check_close, host, oracle_tiles, run_gpu, tile_pairs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print("[gpu-case] " + msg, flush=True)


def check_tiles(cfg, name, entry, pairs):
    say("%s [%s]: launch E=%d N=%d K=%d M=%d (columns %d)" % (
        name, entry, cfg["E"], cfg["N"], cfg["K"], cfg["M"],
        0 if entry == "plain" else mxw.columns(cfg["E"], cfg["M"], cfg["N"], cfg["K"])))
    out = run_gpu(cfg, entry=entry)
    assert torch.isfinite(out.float()).all().item(), "%s: non-finite output (skipped store?)" % name
    for g in range(cfg["E"]):
        if int(cfg["sizes"][g]) == 0:
            assert (out[g].view(torch.int16) == 0).all().item(), "%s: empty expert %d not +0" % (name, g)
    bits = bf16_bits(out)
    del out
    say("%s [%s]: oracle on %d tile pairs x %d experts" % (name, entry, len(pairs), cfg["E"]))
    ref = oracle_tiles(host(cfg), pairs)
    rms = float(np.sqrt(np.mean(np.concatenate([r.ravel() for r in ref.values()]) ** 2)))
    worst = 0.0
    for (tn, tk), r in ref.items():
        n0, k0 = 256 * tn, 256 * tk
        got = bits[:, n0:n0 + r.shape[1], k0:k0 + r.shape[2]]
        st = check_close(got, r, rms=rms, what="%s [%s] tile (%d, %d)" % (name, entry, tn, tk))
        worst = max(worst, st["max_rel"])
    print("%s [%s]: %d whole tiles, rms %.4g, max_rel %.3e" % (name, entry, len(pairs) * cfg["E"], rms, worst))
    return bits


def test_16b_24k_whole_output():
    cfg = W.make_config("16b_24k", device=DEV)
    assert mxw.columns(cfg["E"], cfg["M"], cfg["N"], cfg["K"]) > 0
    pairs = tile_pairs(cfg, 10 ** 6, 0)
    assert len(pairs) == 48
    a = check_tiles(cfg, "16b_24k", "ws", pairs)
    say("16b_24k: bitwise repeat")
    b = bf16_bits(run_gpu(cfg, poison=False))
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("name", ["16b_24k_skew1.2", "16b_24k_skew1.7", "16b_24k_balanced", "16b_24k_ramp",
                                  "671b_gateup", "671b_down", "671b_down_zipf", "16b_256e", "16b_down"])
def test_full_size_tiles(name):
    cfg = W.make_config(name, device=DEV)
    check_tiles(cfg, name, "ws", tile_pairs(cfg, 4 if cfg["E"] > 64 else 12, 17))


def test_16b_24k_plain_entry_tiles():
    cfg = W.make_config("16b_24k", device=DEV)
    check_tiles(cfg, "16b_24k", "plain", tile_pairs(cfg, 12, 23))


def test_16b_24k_bitwise_many_calls():
    """Bitwise reproducibility at the headline configuration under load: 48
    calls of the workspace entry (column mode, arrival counters, partial tiles,
    the scale pre-shuffle) back to back on one stream, no synchronisation in
    between, into four rotating outputs that are compared with the first call
    on the GPU as they come; then 12 calls of the entry without a workspace
    the same way."""
    cfg = W.make_config("16b_24k", device=DEV)
    E, N, K, M = cfg["E"], cfg["N"], cfg["K"], cfg["M"]
    args = [cfg[k] for k in ("A", "sA", "B", "sB", "offs")]
    for plain, calls in ((False, 48), (True, 12)):
        tag = "plain" if plain else "ws"
        say("16b_24k [%s]: %d calls back to back, each against the first" % (tag, calls))
        first = mxw.wgrad(*args, plain=plain)
        outs = [torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV) for _ in range(4)]
        diffs = torch.zeros(calls, dtype=torch.int64, device=DEV)
        for c in range(calls):
            o = outs[c % 4]
            o.view(torch.int16).fill_(0x7FC0)
            mxw.wgrad(*args, out=o, plain=plain)
            diffs[c] = (o.view(torch.int16) != first.view(torch.int16)).sum()
        torch.cuda.synchronize()
        d = diffs.cpu().numpy()
        assert (d == 0).all(), "%s: calls %s differ from the first (%s elements)" % (tag, np.nonzero(d)[0], d[d != 0])
