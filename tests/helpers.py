"""Shared test helpers: running the HIP path and comparing it with the oracle.

Tolerance (per element, floating-point result): |gpu - ref| <= 2^-7 |ref| +
2^-10 rms(ref), with rms over the whole [E, N, K] reference (over the computed
whole tiles where a full-size case checks a subset of tiles).  The 2^-7 term covers the
one bf16 rounding of the output (half an ulp is <= 2^-8 relative) plus FP32
accumulation-order differences; the rms term absorbs cancellation near zero.
"""
import numpy as np
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle

REL_TOL = 2.0 ** -7
RMS_TOL = 2.0 ** -10
BF16_NAN = 0x7FC0


def bf16_bits(t):
    """uint16 numpy array of the bf16 bit patterns of a (device) bf16 tensor."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


ENTRIES = ["ws", "plain"]  # mxfp8_wgrad_grouped_ws (workspace), mxfp8_wgrad_grouped (none)


def run_gpu(cfg, poison=True, out=None, entry="ws", offs=None):
    """Run the HIP path on the config's device tensors through one of the two
    entry points; out is NaN-poisoned first."""
    E, N, K = cfg["E"], cfg["N"], cfg["K"]
    dev = cfg["A"].device
    offs = cfg["offs"] if offs is None else offs
    if out is None:
        out = torch.empty((offs.shape[0], N, K), dtype=torch.bfloat16, device=dev)
    if poison:
        out.view(torch.int16).fill_(BF16_NAN)
    mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], offs, out=out, plain=(entry == "plain"))
    torch.cuda.synchronize(dev)
    return out


def tile_pairs(cfg, count, seed):
    """Seeded (tn, tk) output-tile pairs: the four corner tiles (first and
    last tiles of every expert, the partial last N and K tiles) plus random
    ones, `count` in all (every pair when there are fewer)."""
    tN, tK = -(-cfg["N"] // 256), -(-cfg["K"] // 256)
    allp = [(a, b) for a in range(tN) for b in range(tK)]
    if count >= len(allp):
        return allp
    pick = []
    for p in [(0, 0), (tN - 1, tK - 1), (tN - 1, 0), (0, tK - 1)]:
        if p not in pick:
            pick.append(p)
    rng = np.random.default_rng(seed)
    rest = [p for p in allp if p not in pick]
    for i in rng.permutation(len(rest))[:count - len(pick)]:
        pick.append(rest[i])
    return pick


def oracle_tiles(host_ops, pairs):
    """The oracle's fp64 result on whole 256 x 256 output tiles: for each
    (tn, tk), every expert's tile, from the same definition run on the A rows
    and B rows of that tile (all tokens).  Returns {(tn, tk): [E, rows, cols]}."""
    A, sA, B, sB, offs = host_ops
    res = {}
    for tn, tk in pairs:
        n0, k0 = 256 * tn, 256 * tk
        res[(tn, tk)] = oracle.wgrad_f64(np.ascontiguousarray(A[n0:n0 + 256]), np.ascontiguousarray(sA[n0:n0 + 256]),
                                         np.ascontiguousarray(B[k0:k0 + 256]), np.ascontiguousarray(sB[k0:k0 + 256]),
                                         offs)
    return res


def host(cfg):
    """numpy copies of the operands for the oracle."""
    return (cfg["A"].cpu().numpy(), cfg["sA"].cpu().numpy(), cfg["B"].cpu().numpy(), cfg["sB"].cpu().numpy(),
            cfg["offs"].cpu().numpy())


def check_close(got_bits, ref, rms=None, what=""):
    """Assert the benchmark spec's tolerance element by element; returns stats."""
    got = bf16_to_f64(np.asarray(got_bits))
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), "%s: non-finite output (skipped store or NaN leak)" % what
    if rms is None:
        rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(got - ref)
    tol = REL_TOL * np.abs(ref) + RMS_TOL * rms
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:8]
        raise AssertionError("%s: %d of %d elements outside tolerance; first %s; got %s ref %s" % (
            what, int(bad.sum()), bad.size, idx.tolist(), got[bad][:8].tolist(), ref[bad][:8].tolist()))
    # relative error where the value is not tiny next to the tensor's rms
    big = np.abs(ref) >= 0.125 * rms
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    return dict(max_abs=float(err.max()) if err.size else 0.0, max_rel=max_rel, rms=rms)
