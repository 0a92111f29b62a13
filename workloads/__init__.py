"""Seeded synthetic workloads for the MXFP8 ragged weight-gradient grouped GEMM.

This module only *makes inputs*: routings (per-expert token counts and their
cumulative ends ``offs``), operand values, and their MXFP8 encoding (E4M3 codes
plus one E8M0 scale byte per 32 tokens).  It holds none of the contraction's
arithmetic and no decoder, and it is shared by the GPU path's tests/benchmark
and by the oracle's tests alike: both sides consume exactly the bytes it
produces.

Shapes and distributions follow the blog post "Ragged MXFP8 Weight Gradients:
A FlyDSL Grouped GEMM on MI355X": the DeepSeek-V3 "16B" expert shape (N=1408,
K=2048, 8 local experts) and the "671B" shapes (N=4096/K=7168 and
N=7168/K=2048, 32 experts) of section 2; unequal groups with the busiest
expert at 1.2-1.7x the mean and possibly empty experts (section 1); group
boundaries on 32-token multiples (sections 1 and 7).  The pages' own routings
are not public, so seeded Dirichlet / Zipf draws stand in for them.  The
balanced control splits tokens evenly with the remainder on the first experts
(XLA blog, "Fixing group_sizes Deterministically"); the linear-ramp control is
the blog's results-table routing (section 7: linear ramp, busiest 1.5x the
mean, groups rounded to 256 tokens).

Quantisation recipe (input generation only, excluded from the timed operator
as in the blog's section 7): per row and per 32-token block,
    scale byte  = clamp(floor(log2(amax)) - 8 + 127, 0, 254)   (amax = 0 -> 127)
    element     = round-half-even(x / 2^(byte - 127)) to OCP E4M3FN,
                  saturated to +-448.
floor(log2) is taken exactly from the binary exponent (frexp), and saturation
is applied before encoding, so no library overflow behaviour is relied on.

Values are drawn with ``torch`` on the requested device from a seeded
generator; a workload is therefore defined by (name, seed, device type).  The
GPU tests and the benchmark generate on the GPU and copy to the host whatever
the oracle needs.
"""
import math

import numpy as np
import torch

# name -> shape/routing recipe.  "values": (std_A, std_B) or "wide" (per-block
# amax log-uniform over 2^-6..2^6).
CONFIGS = {
    # tiny ragged case: one head-masked start, one empty expert, one tail end
    "tiny": dict(E=4, N=128, K=256, M=512, routing=("fixed", [96, 0, 160, 256]), values=(1.0, 1.0), cid=1),
    # 16B expert shape, mean 1,024 tokens/expert, busiest ~1.5x
    "16b_1k": dict(E=8, N=1408, K=2048, M=8192, routing=("dirichlet", 8.0, (1.45, 1.55), 0), values=(1.0, 0.5), cid=2),
    # 16B expert shape at production token count (headline), busiest ~1.5x
    "16b_24k": dict(E=8, N=1408, K=2048, M=196608, routing=("dirichlet", 8.0, (1.45, 1.55), 0), values=(1.0, 0.5), cid=3),
    # same shape, milder and stronger skews, and the two controls
    "16b_24k_skew1.2": dict(E=8, N=1408, K=2048, M=196608, routing=("dirichlet", 32.0, (1.15, 1.25), 0), values=(1.0, 0.5), cid=31),
    "16b_24k_skew1.7": dict(E=8, N=1408, K=2048, M=196608, routing=("dirichlet", 4.0, (1.65, 1.75), 0), values=(1.0, 0.5), cid=32),
    "16b_24k_balanced": dict(E=8, N=1408, K=2048, M=196608, routing=("balanced",), values=(1.0, 0.5), cid=33),
    "16b_24k_ramp": dict(E=8, N=1408, K=2048, M=196608, routing=("ramp", 1.5, 256), values=(1.0, 0.5), cid=34),
    # 671B gate/up and down shapes: mean 8,192 tokens/expert, one empty expert
    "671b_gateup": dict(E=32, N=4096, K=7168, M=262144, routing=("dirichlet", 16.0, (1.55, 1.70), 1), values=(1.0, 1.0), cid=41),
    "671b_down": dict(E=32, N=7168, K=2048, M=262144, routing=("dirichlet", 16.0, (1.55, 1.70), 1), values=(1.0, 1.0), cid=42),
    # ragged-edge stress at the 671B down shape: Zipf routing, 4 empty
    # experts, every non-first group start an odd multiple of 32
    "671b_down_zipf": dict(E=32, N=7168, K=2048, M=131072, routing=("zipf", 1.1, 4), values="wide", cid=5),
    # the 16B down projection's weight gradient (not a configuration of the
    # pages, which measure gate/up): N = hidden 2048, K = intermediate 1408
    "16b_down": dict(E=8, N=2048, K=1408, M=196608, routing=("dirichlet", 8.0, (1.45, 1.55), 0), values=(1.0, 0.5),
                     cid=62),
    # many-expert stress (not a configuration of the pages): 256 experts of the
    # 16B expert shape on one GPU, mean 1,024 tokens/expert, busiest ~1.8x
    "16b_256e": dict(E=256, N=1408, K=2048, M=262144, routing=("dirichlet", 8.0, (1.45, 1.8), 0), values=(1.0, 0.5),
                     cid=61),
}


# --------------------------------------------------------------------------
# routings
# --------------------------------------------------------------------------
def round_to_units(weights, total, unit=32):
    """Integer sizes, multiples of `unit`, summing exactly to `total`, by
    largest remainder (ties -> lower index)."""
    w = np.asarray(weights, np.float64)
    units = total // unit
    if units * unit != total:
        raise ValueError("total must be a multiple of unit")
    if w.sum() <= 0:
        raise ValueError("weights must have positive sum")
    share = w / w.sum() * units
    base = np.floor(share).astype(np.int64)
    rem = units - int(base.sum())
    frac = share - base
    order = sorted(range(len(w)), key=lambda i: (-frac[i], i))
    for i in order[:rem]:
        base[i] += 1
    return base * unit


def balanced_sizes(E, M):
    """Even split, remainder one extra on the first experts (XLA blog)."""
    base = M // E
    gs = np.full(E, base, np.int64)
    gs[: M - base * E] += 1
    return gs


def dirichlet_sizes(E, M, alpha, band, n_empty, cid, max_attempts=100000):
    """Dirichlet(alpha) shares rounded to 32-token units; redraw (seed 1000*cid + j)
    until busiest/mean lies in `band`, the mean taken over all E experts.
    With n_empty > 0, that many experts (seeded choice) get zero tokens and the
    rest share M.  Returns (sizes, seed_used)."""
    for j in range(max_attempts):
        seed = 1000 * cid + j
        rng = np.random.default_rng(seed)
        empty = rng.choice(E, size=n_empty, replace=False) if n_empty else np.array([], np.int64)
        live = np.array([g for g in range(E) if g not in set(empty.tolist())])
        p = rng.dirichlet(np.full(len(live), alpha))
        sizes = np.zeros(E, np.int64)
        sizes[live] = round_to_units(p, M, 32)
        skew = sizes.max() / (M / E)
        if band[0] <= skew <= band[1] and (sizes[live] > 0).all():
            return sizes, seed
    raise RuntimeError("no Dirichlet draw in band")


def ramp_sizes(E, M, busiest, unit):
    """Linear ramp from (2 - busiest) to busiest times the mean, each rounded to
    `unit` tokens, the rounding residue put on the largest group."""
    mean = M / E
    w = np.linspace(2.0 - busiest, busiest, E) * mean
    sizes = (np.round(w / unit) * unit).astype(np.int64)
    sizes[-1] += M - sizes.sum()
    if (sizes < 0).any() or sizes.sum() != M:
        raise RuntimeError("ramp rounding failed")
    return sizes


def zipf_sizes(E, M, s, n_empty, cid):
    """Zipf(s) weights over the non-empty experts (rank order from a seeded
    permutation), rounded to 32 tokens, then moved +-32 between neighbours so
    that the first non-empty length is 32 mod 64, middle ones 0 mod 64 and the
    last 32 mod 64: every non-empty group after the first then starts at an
    odd multiple of 32."""
    seed = 1000 * cid
    rng = np.random.default_rng(seed)
    empty = set(rng.choice(E, size=n_empty, replace=False).tolist())
    live = [g for g in range(E) if g not in empty]
    ranks = rng.permutation(len(live)) + 1
    w = ranks.astype(np.float64) ** (-s)
    sz = round_to_units(w, M, 32)
    # alignment fix-up, walking the live experts in index order
    L = len(live)
    for i in range(L - 1):
        want = 32 if i == 0 else 0
        if sz[i] % 64 != want:
            # move 32 tokens to or from the next live group (keep both >= 32)
            if sz[i] >= 64 + 32 or sz[i + 1] < 64:
                sz[i] -= 32
                sz[i + 1] += 32
            else:
                sz[i] += 32
                sz[i + 1] -= 32
    sizes = np.zeros(E, np.int64)
    sizes[live] = sz
    return sizes, seed


def routing_sizes(name):
    """Per-expert token counts for a named workload, plus the routing seed."""
    c = CONFIGS[name]
    kind = c["routing"][0]
    E, M = c["E"], c["M"]
    if kind == "fixed":
        sizes = np.array(c["routing"][1], np.int64)
        if sizes.sum() != M:
            raise ValueError("fixed sizes must sum to M")
        return sizes, None
    if kind == "balanced":
        return balanced_sizes(E, M), None
    if kind == "ramp":
        return ramp_sizes(E, M, c["routing"][1], c["routing"][2]), None
    if kind == "dirichlet":
        _, alpha, band, n_empty = c["routing"]
        return dirichlet_sizes(E, M, alpha, band, n_empty, c["cid"])
    if kind == "zipf":
        _, s, n_empty = c["routing"]
        return zipf_sizes(E, M, s, n_empty, c["cid"])
    raise ValueError(kind)


def offs_from_sizes(sizes):
    """Cumulative ends (int32): offs[g] = sum(sizes[:g+1])."""
    return np.cumsum(np.asarray(sizes, np.int64)).astype(np.int32)


# --------------------------------------------------------------------------
# MXFP8 encoding (input generation only)
# --------------------------------------------------------------------------
def mx_scale_bytes(amax):
    """E8M0 byte per block: clamp(floor(log2 amax) - 8 + 127, 0, 254); 127 for
    amax == 0.  floor(log2) from the binary exponent, exactly."""
    _, ex = torch.frexp(amax.to(torch.float64))  # amax = f * 2^ex, f in [0.5, 1)
    b = (ex.to(torch.int64) - 1) - 8 + 127
    b = torch.clamp(b, 0, 254)
    b = torch.where(amax == 0, torch.full_like(b, 127), b)
    return b.to(torch.uint8)


def pow2(k):
    """2**k as float64, exactly, for integer tensors k in [-1022, 1023]: built
    from the exponent field.  (torch.ldexp and torch.pow(2, k) round on some
    devices: on the GPU they are not exact for integer k.)"""
    k = k.to(torch.int64)
    return ((k + 1023) << 52).view(torch.float64)


def e4m3_encode_rne(y):
    """Encode float64 values (already within +-448) to OCP E4M3FN codes,
    round-half-even.  Returns uint8 codes."""
    a = y.abs()
    _, ex = torch.frexp(a)
    fl = ex.to(torch.int64) - 1  # floor(log2 a) for a > 0
    qexp = torch.where(fl < -6, torch.full_like(fl, -9), fl - 3)  # grid spacing exponent
    q = torch.round(a * pow2(-qexp))  # half-to-even
    v = q * pow2(qexp)  # representable magnitude
    # code from the exact value
    sub = v < 2.0 ** -6
    code_sub = (v * 512.0).to(torch.int64)
    _, ev = torch.frexp(torch.where(sub, torch.ones_like(v), v))
    e_field = ev.to(torch.int64) - 1 + 7
    mant = (v * pow2(-(ev.to(torch.int64) - 1)) * 8.0 - 8.0).to(torch.int64)
    code_norm = (e_field << 3) | mant
    code = torch.where(sub, code_sub, code_norm)
    code = torch.where(y < 0, code | 0x80, code)
    code = torch.where(v == 0, torch.zeros_like(code), code)
    return code.to(torch.uint8)


def quantize_rows(x):
    """MXFP8-quantise x [rows, M] (M % 32 == 0) along the token axis.
    Returns (codes uint8 [rows, M], scales uint8 [rows, M/32])."""
    rows, M = x.shape
    if M % 32:
        raise ValueError("M must be a multiple of 32")
    xb = x.to(torch.float64).reshape(rows, M // 32, 32)
    amax = xb.abs().amax(dim=-1)
    sb = mx_scale_bytes(amax)
    y = xb * pow2(127 - sb.to(torch.int64)).unsqueeze(-1)
    y = torch.clamp(y, -448.0, 448.0)
    codes = e4m3_encode_rne(y).reshape(rows, M)
    return codes, sb


def _gen_values(rows, M, mode, std, gen, device, chunk_rows):
    """Yield (r0, x chunk fp32) row chunks of the operand values."""
    for r0 in range(0, rows, chunk_rows):
        r = min(chunk_rows, rows - r0)
        z = torch.randn((r, M), generator=gen, device=device, dtype=torch.float32)
        if mode == "wide":
            zb = z.reshape(r, M // 32, 32)
            u = torch.rand((r, M // 32, 1), generator=gen, device=device, dtype=torch.float32) * 12.0 - 6.0
            amax = zb.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
            z = (zb / amax * torch.exp2(u)).reshape(r, M)
        else:
            z = z * std
        yield r0, z


def make_operand(rows, M, mode, std, seed, device="cpu", chunk_rows=None):
    """Quantised operand (codes [rows, M], scales [rows, M/32]) on `device`."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    if chunk_rows is None:
        chunk_rows = max(1, min(rows, (1 << 24) // max(M, 1)))
    q = torch.empty((rows, M), dtype=torch.uint8, device=device)
    s = torch.empty((rows, M // 32), dtype=torch.uint8, device=device)
    for r0, x in _gen_values(rows, M, mode, std, gen, device, chunk_rows):
        cq, cs = quantize_rows(x)
        q[r0:r0 + x.shape[0]] = cq
        s[r0:r0 + x.shape[0]] = cs
    return q, s


def make_config(name, device="cpu", seed=None):
    """Build a named workload.  Returns a dict with A, sA, B, sB (uint8 torch
    tensors on `device`), offs (int32 torch tensor on `device`), the sizes and
    the shape/seed metadata."""
    c = CONFIGS[name]
    E, N, K, M = c["E"], c["N"], c["K"], c["M"]
    sizes, rseed = routing_sizes(name)
    offs = offs_from_sizes(sizes)
    vseed = 1000 * c["cid"] + 999 if seed is None else int(seed)
    if c["values"] == "wide":
        mode, sa_std, sb_std = "wide", 1.0, 1.0
    else:
        mode, (sa_std, sb_std) = "normal", c["values"]
    A, sA = make_operand(N, M, mode, sa_std, vseed, device)
    B, sB = make_operand(K, M, mode, sb_std, vseed + 1, device)
    return dict(name=name, E=E, N=N, K=K, M=M, A=A, sA=sA, B=B, sB=sB,
                offs=torch.from_numpy(offs).to(device), sizes=sizes,
                routing_seed=rseed, value_seed=vseed,
                skew=float(sizes.max() / (M / E)))


def make_random(E, N, K, M, sizes, seed, device="cpu", mode="normal", std=(1.0, 1.0)):
    """A custom-shaped workload (for parity cases that are not named configs)."""
    sizes = np.asarray(sizes, np.int64)
    if sizes.shape != (E,) or sizes.sum() > M:
        raise ValueError("sizes must be [E] with sum <= M")
    offs = offs_from_sizes(sizes)
    A, sA = make_operand(N, M, mode, std[0], seed, device)
    B, sB = make_operand(K, M, mode, std[1], seed + 1, device)
    return dict(name="custom", E=E, N=N, K=K, M=M, A=A, sA=sA, B=B, sB=sB,
                offs=torch.from_numpy(offs).to(device), sizes=sizes, routing_seed=None, value_seed=seed,
                skew=float(sizes.max() / max(M / E, 1)))


def useful_flops(cfg):
    """2 * M_used * N * K with M_used = offs[E-1] (masked/padded work excluded)."""
    return 2.0 * float(np.asarray(cfg["sizes"]).sum()) * cfg["N"] * cfg["K"]


def algorithmic_bytes(cfg):
    """Bytes the method must move: each routed token's (N+K) E4M3 bytes and
    (N+K)/32 scale bytes read once, the bf16 output written once, offs read."""
    mu = float(np.asarray(cfg["sizes"]).sum())
    N, K, E = cfg["N"], cfg["K"], cfg["E"]
    return mu * (N + K) * (1.0 + 1.0 / 32.0) + 2.0 * E * N * K + 4.0 * E


# --------------------------------------------------------------------------
# Row-ragged grouped GEMM (forward / data gradient of the same layer)
# --------------------------------------------------------------------------
# (base routing, C = contraction, N = output columns): the forward gate/up
# GEMM of a workload contracts over its K (hidden) and produces N columns,
# the forward down GEMM contracts over N and produces K.
ROWS_CONFIGS = {
    "16b_fwd": dict(base="16b_24k", C="K", N="N"),
    "16b_fwd_down": dict(base="16b_24k", C="N", N="K"),
    "16b_1k_fwd": dict(base="16b_1k", C="K", N="N"),
    "671b_fwd": dict(base="671b_gateup", C="K", N="N"),
}


def make_rows(E, R, C, N, sizes, seed, device="cpu", mode="normal", std=(1.0, 1.0)):
    """A row-ragged problem: A [R, C] and B [E, N, C] quantised along C,
    offs from `sizes` (any row counts, sum <= R)."""
    sizes = np.asarray(sizes, np.int64)
    if sizes.shape != (E,) or sizes.sum() > R:
        raise ValueError("sizes must be [E] with sum <= R")
    A, sA = make_operand(R, C, mode, std[0], seed, device)
    B, sB = make_operand(E * N, C, mode, std[1], seed + 1, device)
    return dict(name="custom_rows", E=E, R=R, C=C, N=N, A=A, sA=sA, B=B.reshape(E, N, C),
                sB=sB.reshape(E, N, C // 32), offs=torch.from_numpy(offs_from_sizes(sizes)).to(device),
                sizes=sizes, value_seed=seed)


def make_rows_config(name, device="cpu", seed=None):
    """A named row-ragged workload: the routing of its base workload, rows =
    that workload's tokens."""
    rc = ROWS_CONFIGS[name]
    c = CONFIGS[rc["base"]]
    sizes, rseed = routing_sizes(rc["base"])
    vseed = 1000 * c["cid"] + 777 if seed is None else int(seed)
    mode, std = ("wide", (1.0, 1.0)) if c["values"] == "wide" else ("normal", c["values"])
    cfg = make_rows(c["E"], c["M"], c[rc["C"]], c[rc["N"]], sizes, vseed, device, mode, std)
    cfg.update(name=name, routing_seed=rseed)
    return cfg


def rows_useful_flops(cfg):
    """2 * rows_used * C * N (rows past the last expert excluded)."""
    return 2.0 * float(np.asarray(cfg["sizes"]).sum()) * cfg["C"] * cfg["N"]


def rows_algorithmic_bytes(cfg):
    """Each routed row's C codes + C/32 scales read once, each expert's
    [N, C] operand + scales read once, the bf16 rows written once, offs."""
    mu = float(np.asarray(cfg["sizes"]).sum())
    C, N, E = cfg["C"], cfg["N"], cfg["E"]
    return mu * C * (1.0 + 1.0 / 32.0) + E * N * C * (1.0 + 1.0 / 32.0) + 2.0 * mu * N + 4.0 * E


# --------------------------------------------------------------------------
# BF16 contracting ragged dot (the same weight gradient on bf16 operands)
# --------------------------------------------------------------------------
# The XLA blog's wgrad classes (Table 7) are bfloat16; these workloads take a
# named MXFP8 workload's shape and routing and draw the same value
# distributions, rounded once to bf16 (round-to-nearest-even), stored
# token-contiguous like the MXFP8 operands: A = dY^T [N, M], B = X^T [K, M].
BF16_CONFIGS = {
    "16b_bf16": "16b_24k",
    "16b_1k_bf16": "16b_1k",
    "671b_bf16": "671b_gateup",
}


def make_bf16_operand(rows, M, std, seed, device="cpu", chunk_rows=None):
    """bf16 operand [rows, M]: std * N(0, 1) rounded to bf16, on `device`."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    if chunk_rows is None:
        chunk_rows = max(1, min(rows, (1 << 24) // max(M, 1)))
    x = torch.empty((rows, M), dtype=torch.bfloat16, device=device)
    for r0, z in _gen_values(rows, M, "normal", std, gen, device, chunk_rows):
        x[r0:r0 + z.shape[0]] = z.to(torch.bfloat16)
    return x


def make_bf16(E, N, K, M, sizes, seed, device="cpu", std=(1.0, 1.0)):
    """A custom-shaped bf16 problem: A [N, M], B [K, M] (torch.bfloat16) and offs."""
    sizes = np.asarray(sizes, np.int64)
    if sizes.shape != (E,) or sizes.sum() > M:
        raise ValueError("sizes must be [E] with sum <= M")
    A = make_bf16_operand(N, M, std[0], seed, device)
    B = make_bf16_operand(K, M, std[1], seed + 1, device)
    return dict(name="custom_bf16", E=E, N=N, K=K, M=M, A=A, B=B,
                offs=torch.from_numpy(offs_from_sizes(sizes)).to(device), sizes=sizes,
                routing_seed=None, value_seed=seed, skew=float(sizes.max() / max(M / E, 1)))


def make_bf16_config(name, device="cpu", seed=None):
    """A named bf16 workload: the shape, routing and value spread of its base
    MXFP8 workload, value seed 1000 * cid + 998."""
    base = BF16_CONFIGS[name]
    c = CONFIGS[base]
    E, N, K, M = c["E"], c["N"], c["K"], c["M"]
    sizes, rseed = routing_sizes(base)
    vseed = 1000 * c["cid"] + 998 if seed is None else int(seed)
    sa_std, sb_std = c["values"]
    cfg = make_bf16(E, N, K, M, sizes, vseed, device, (sa_std, sb_std))
    cfg.update(name=name, base=base, routing_seed=rseed, skew=float(sizes.max() / (M / E)))
    return cfg


def bf16_algorithmic_bytes(cfg):
    """Each routed token's (N + K) bf16 values read once, the bf16 output
    written once, offs read."""
    mu = float(np.asarray(cfg["sizes"]).sum())
    N, K, E = cfg["N"], cfg["K"], cfg["E"]
    return mu * (N + K) * 2.0 + 2.0 * E * N * K + 4.0 * E
