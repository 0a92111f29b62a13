"""Benchmark: MXFP8 ragged weight-gradient grouped GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one call of the whole hot path (windows from offs, tile
scheduling, masked head/tail staging, scale relayout, block-scaled MFMA
contraction, bf16 epilogue) on seeded synthetic inputs already resident in
HBM.  The headline times mxfp8_wgrad_grouped_ws with a workspace allocated
once beforehand: at the default workload a call is two kernels, the scale
pre-shuffle and the main kernel in column mode, and the time is the whole
call's.  The line also carries `plain_entry`: the same problem through
mxfp8_wgrad_grouped, the entry point that takes no workspace (one kernel, one
workgroup per output tile, scales read from the caller's planes).

Timing method (stated in the line as `timing`): W untimed warm-up steps, then
an untimed pre-run of back-to-back steps for about 2 s so that clocks and
power reach the state they keep under sustained load, a synchronisation, then
exactly K steps between HIP events on the launch stream.  `sustained` adds two
further passes of >= 3 s (>= 1 s for the small workloads) with an event every
8 steps, reporting the mean and median time per step of each pass.

The default workload is the DeepSeek-V3 16B expert shape at production token
count (E=8, N=1408, K=2048, 24,576 tokens/expert,
Dirichlet routing with the busiest expert ~1.5x the mean): the shape the
blog "Ragged MXFP8 Weight Gradients: A FlyDSL Grouped GEMM on MI355X" quotes
2,174 TFLOP/s at (sections 5.6 and 7).

Prints ONE JSON line: TFLOP/s of useful work (2 * M_used * N * K), the
MFMA-roofline fraction of the kernel (HIP events on the launch stream), the
HBM traffic measured by rocprofv3 counters (when the committed counter
summary matches this kernel source), and the CPU oracle timed on the host
cores on a bounded sample of the same workload.

The row-ragged grouped GEMM of the same layer (forward / data gradient,
mxfp8_grouped_fwd) is measured the same way with --workload 16b_fwd,
16b_fwd_down, 16b_1k_fwd or 671b_fwd (rows = the base workload's routed
tokens; useful work 2 * rows * C * N).

The token-axis quantiser (mxfp8_quantize_tokens) is measured with
--workload 16b_quant (or 671b_quant): one step quantises the base workload's
dY [M, N] and X [M, K] (bf16, seeded) into its two MXFP8 operands; the metric
is algorithmic HBM GB/s (2 bytes read, 1 + 1/32 bytes written per element)
against the 8 TB/s HBM roof.

The same weight gradient on bf16 operands (bf16_wgrad_grouped, the XLA blog's
contracting ragged dot) is measured with --workload 16b_bf16, 16b_1k_bf16 or
671b_bf16 (the base workload's shape and routing), against the 2.5 PFLOP/s
dense BF16 MFMA peak, with torch._grouped_mm timed on the same operands.

For the weight-gradient workloads the line also carries `bf16_context`: the
same ragged problem in bf16 through torch._grouped_mm (dY^T [N, M] and X
[M, K], contraction ragged by the same offs, hipBLASLt on ROCm), timed the same
way in the same process, as the pages' "x BF16" comparison (context, not the
metric).

The weight-gradient line also carries `padded_rows`: the same call on the same
values stored with rows M + 128 tokens apart (the layout the quantiser writes
when given a row stride; --ld-pad N times that layout as the headline).

The weight-gradient line also carries `cold_caches`: 30 calls each timed alone
after a 1 GiB write that evicts the L2s and the Infinity Cache, beside the same
per-call timing without it (the pages saw no difference between the two).

The weight-gradient line also carries `graph_replay`: the same call captured
20 times into one HIP graph and replayed back to back, the device-side time
per call without the host's per-call argument marshalling (what bounds the
tiny workload).

The weight-gradient lines also carry `power`: socket power, joules per step and
the mean shader clock over the first sustained pass (amdsmi, read-only), and
the clock-normalised roofline fraction TFLOP/s / (peak x clock / 2.4 GHz).

Extra modes (profiling helpers, same file so profiles run committed code):
    --no-cpu             skip the oracle leg (for profiler runs)
    --no-power           skip the power sampling
    --no-sustained / --no-plain / --no-padded / --no-cold / --no-graph / --no-bf16   skip those legs
    --prerun S           seconds of untimed pre-run (0 for counter runs)
    --entry plain        time mxfp8_wgrad_grouped (no workspace) as the headline
    --ld-pad N           store the operands with rows M + N tokens apart
    --copy-calibration   run a plain 1 GiB device copy (counter calibration)
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 wgrad TFLOP/s (2·M·N·K) at 16B/671B shapes; % of MXFP8 MFMA peak"
PEAK_TFLOPS = 5000.0  # MI355X dense FP8 / MXFP8 MFMA peak
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA peak
PAGES_TFLOPS_16B = 2174.0  # the blog's shipping kernel at the 16B ragged shape, MI355X
KERNEL_SRC = os.path.join(ROOT, "mxfp8_ragged_grouped_amd", "csrc", "mxfp8_wgrad.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    if it was taken on another kernel source or workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get("workloads", {}).get(workload)
    if not entry or entry.get("kernel_sha") != kernel_sha():
        return None
    return entry.get("hbm_bytes_per_launch")


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}))


def note(msg):
    """A progress line on stderr (stdout carries only the JSON line)."""
    print("bench: " + msg, file=sys.stderr, flush=True)


def cpu_baseline(cfg, A, sA, B, sB, offs, budget_s=25.0):
    """Time the oracle on a bounded sample of the workload: every s-th row of A
    and of B (1/s^2 of the outputs, every routed token of every expert).  A
    stride-8 probe picks the smallest s in (1, 2, 4, 8) whose estimated time
    stays within budget_s; only the run at that stride is reported."""
    import oracle

    used = float(np.sum(cfg["sizes"]))

    def run(stride):
        A_s, sA_s = np.ascontiguousarray(A[::stride]), np.ascontiguousarray(sA[::stride])
        B_s, sB_s = np.ascontiguousarray(B[::stride]), np.ascontiguousarray(sB[::stride])
        t0 = time.perf_counter()
        oracle.wgrad_f64(A_s, sA_s, B_s, sB_s, offs)
        return time.perf_counter() - t0, A_s.shape[0], B_s.shape[0]

    t_probe = run(8)[0]
    stride = next(s for s in (1, 2, 4, 8) if t_probe * (8 // s) ** 2 <= budget_s or s == 8)
    dt, na, nb = run(stride)
    flops = 2.0 * used * na * nb
    res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": "%s: %s of A and of B (%d x %d of %d x %d outputs per expert, all %d routed "
                     "tokens), fp64, %.1f s" % (cfg["name"], {1: "every row", 2: "every 2nd row", 4: "every 4th row",
                                                               8: "every 8th row"}[stride], na, nb,
                                               cfg["N"], cfg["K"], int(used), dt)}
    if float(cfg["M"]) / cfg["E"] < 8192:
        # the small workloads: a run on one core as well, at the smallest
        # stride (not below the one above) whose estimate stays within budget_s
        threads = oracle.max_threads()
        est1 = lambda s: t_probe * threads * (8 // s) ** 2
        s1 = next((s for s in (1, 2, 4, 8) if s >= stride and est1(s) <= budget_s), None)
        if s1 is not None:
            oracle.set_threads(1)
            try:
                dt1, na1, nb1 = run(s1)
            finally:
                oracle.set_threads(threads)
            res["single_core"] = {"value": 2.0 * used * na1 * nb1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                                  "seconds": round(dt1, 2), "stride": s1}
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_rows(cfg, A, sA, B, sB, offs, budget_s=20.0):
    """Time the oracle on seeded sample points of the row-ragged GEMM (each a
    full C-term dot product); a 2,000-point probe sizes the sample to about
    budget_s."""
    import oracle

    used = int(np.sum(cfg["sizes"]))
    rng = np.random.default_rng(11)

    def run(npts):
        m = rng.integers(0, used, npts)
        n = rng.integers(0, cfg["N"], npts).astype(np.int32)
        t0 = time.perf_counter()
        oracle.rows_points(A, sA, B, sB, offs, m, n)
        return time.perf_counter() - t0

    t_probe = run(2000)
    npts = int(max(2000, min(4_000_000, 2000 * budget_s / max(t_probe, 1e-6))))
    dt = run(npts)
    return {"value": 2.0 * cfg["C"] * npts / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "sample": "%s: %d seeded (row, column) outputs of %d x %d, each a %d-term fp64 dot "
                                        "product, %.1f s" % (cfg["name"], npts, used, cfg["N"], cfg["C"], dt)}


def bench_rows(args):
    import torch

    import mxfp8_ragged_grouped_amd as mxw
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.make_rows_config(args.workload, device=dev)
    E, R, C, N = cfg["E"], cfg["R"], cfg["C"], cfg["N"]
    out = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        mxw.fwd(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, stream=stream)

    ms, wall = time_steps(step, args, stream)
    tflops = W.rows_useful_flops(cfg) / (ms * 1e-3) / 1e12
    res = {
        "metric": "MXFP8 row-ragged grouped GEMM TFLOP/s (2·rows·C·N), forward / data gradient",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8(e4m3,e8m0/32)->fp32acc->bf16",
        "data": "synthetic (seeded routing of the base workload, N(0,1) values, MXFP8-quantised along C)",
        "config": {"workload": args.workload, "E": E, "R": R, "C": C, "N": N,
                   "rows_used": int(np.sum(cfg["sizes"])), "routing_seed": cfg["routing_seed"],
                   "value_seed": cfg["value_seed"], "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_TFLOPS, 4), "traffic": load_traffic(args.workload)},
        "hbm_gbps_algorithmic": round(W.rows_algorithmic_bytes(cfg) / (ms * 1e-3) / 1e9, 1),
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline_rows(cfg, *(cfg[k].cpu().numpy() for k in ("A", "sA", "B", "sB", "offs")))
    print(json.dumps(res))


def cpu_baseline_bf16(cfg, A, B, offs, budget_s=25.0):
    """The bf16 oracle on a bounded sample, chosen as for the MXFP8 weight
    gradient: every s-th row of A and of B, all routed tokens."""
    import oracle

    used = float(np.sum(cfg["sizes"]))

    def run(stride):
        A_s, B_s = np.ascontiguousarray(A[::stride]), np.ascontiguousarray(B[::stride])
        t0 = time.perf_counter()
        oracle.bf16_wgrad_f64(A_s, B_s, offs)
        return time.perf_counter() - t0, A_s.shape[0], B_s.shape[0]

    t_probe = run(8)[0]
    stride = next(s for s in (1, 2, 4, 8) if t_probe * (8 // s) ** 2 <= budget_s or s == 8)
    dt, na, nb = run(stride)
    return {"value": 2.0 * used * na * nb / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "sample": "%s: %s of A and of B (%d x %d of %d x %d outputs per expert, all "
                                        "%d routed tokens), fp64, %.1f s" % (
                                            cfg["name"], {1: "every row", 2: "every 2nd row", 4: "every 4th row",
                                                          8: "every 8th row"}[stride], na, nb, cfg["N"], cfg["K"],
                                            int(used), dt)}


def bench_bf16(args):
    """BF16 contracting ragged dot (bf16_wgrad_grouped) on a named bf16
    workload, with torch._grouped_mm on the very same operands beside it."""
    import torch

    import mxfp8_ragged_grouped_amd as mxw
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.make_bf16_config(args.workload, device=dev)
    E, N, K, M = cfg["E"], cfg["N"], cfg["K"], cfg["M"]
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws = torch.empty(max(mxw.bf16_workspace_size(E, M, N, K), 1), dtype=torch.uint8, device=dev)
    plain = args.entry == "plain"

    def step():
        mxw.wgrad_bf16(cfg["A"], cfg["B"], cfg["offs"], out=out, stream=stream, workspace=ws, plain=plain)

    ms, wall = time_steps(step, args, stream)
    flops = W.useful_flops(cfg)
    tflops_of = lambda t_ms: flops / (t_ms * 1e-3) / 1e12
    tflops = tflops_of(ms)
    res = {
        "metric": "BF16 contracting ragged dot (weight gradient) TFLOP/s (2·M·N·K); % of BF16 MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->fp32acc->bf16",
        "data": "synthetic (the base workload's seeded routing, N(0,1) values rounded to bf16, token-contiguous)",
        "config": {"workload": args.workload, "base": cfg["base"], "E": E, "N": N, "K": K, "M": M,
                   "busiest_over_mean": round(cfg["skew"], 3), "routing_seed": cfg["routing_seed"],
                   "value_seed": cfg["value_seed"], "columns": 0 if plain else mxw.columns(E, 2 * M, N, K),
                   "entry": "bf16_wgrad_grouped" if plain else "bf16_wgrad_grouped_ws",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic(args.workload + ("_plain" if plain else ""))},
        "hbm_gbps_algorithmic": round(W.bf16_algorithmic_bytes(cfg) / (ms * 1e-3) / 1e9, 1),
        "wall_s_timed": round(wall, 3),
        "timing": "%d untimed warm-up steps, an untimed ~%g s back-to-back pre-run, a synchronisation, then exactly "
                  "%d steps between HIP events on the launch stream" % (args.warmup, args.prerun, args.steps),
    }
    if not args.no_sustained:
        sus = sustained_leg(step, ms, stream, 1.0 if M // E < 8192 else 3.0, tflops_of_ms=tflops_of,
                            peak=PEAK_BF16_TFLOPS, power=not args.no_power)
        if "power" in sus:
            res["power"] = sus.pop("power")
        res["sustained"] = sus
    if not args.no_bf16:
        # the same operands through torch._grouped_mm (X as a contiguous [M, K])
        xb = cfg["B"].t().contiguous()
        try:
            tms, _ = time_steps(lambda: torch._grouped_mm(cfg["A"], xb, offs=cfg["offs"]), args, stream)
            ttf = flops / (tms * 1e-3) / 1e12
            res["torch_grouped_mm"] = {"value": round(ttf, 1), "unit": "TFLOP/s", "ms": round(tms, 4),
                                       "ours_over_torch": round(tflops / ttf, 3),
                                       "what": "torch._grouped_mm(A [N, M], X [M, K], offs) on the same bf16 "
                                               "values, same steps/warmup, same stream, this process"}
        except Exception as ex:  # not every build has a grouped GEMM for this layout
            res["torch_grouped_mm"] = {"value": None, "error": str(ex)[:200]}
        del xb
    if not args.no_cpu:
        u16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        res["cpu_baseline"] = cpu_baseline_bf16(cfg, u16(cfg["A"]), u16(cfg["B"]), cfg["offs"].cpu().numpy())
    print(json.dumps(res))


QUANT_WORKLOADS = {"16b_quant": "16b_24k", "671b_quant": "671b_gateup"}
HBM_PEAK_GBS = 8000.0


def bench_quant(args):
    import torch

    import mxfp8_ragged_grouped_amd as mxw
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = QUANT_WORKLOADS[args.workload]
    c = W.CONFIGS[base]
    M, N, K = c["M"], c["N"], c["K"]
    offs = torch.from_numpy(W.offs_from_sizes(W.routing_sizes(base)[0])).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(1000 * c["cid"] + 555)
    dy = torch.randn((M, N), generator=g, device=dev).to(torch.bfloat16)
    xx = (0.5 * torch.randn((M, K), generator=g, device=dev)).to(torch.bfloat16)
    qa = torch.empty((N, M), dtype=torch.uint8, device=dev)
    sa = torch.empty((N, M // 32), dtype=torch.uint8, device=dev)
    qb = torch.empty((K, M), dtype=torch.uint8, device=dev)
    sb = torch.empty((K, M // 32), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        mxw.quantize_tokens(dy, offs, q=qa, s=sa, stream=stream)
        mxw.quantize_tokens(xx, offs, q=qb, s=sb, stream=stream)

    ms, wall = time_steps(step, args, stream)
    per_launch = load_traffic(args.workload)  # mean of the dY and X launches
    elems = float(M) * (N + K)
    alg_bytes = elems * (2.0 + 1.0 + 1.0 / 32.0)
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "MXFP8 token-axis quantiser HBM GB/s (algorithmic bytes: 2 read + 1 + 1/32 written per element)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->e4m3+e8m0/32", "data": "synthetic (seeded N(0,1) bf16 dY and 0.5 N(0,1) X)",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "elements": int(elems),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if per_launch is None else 2 * per_launch},  # per step (two launches)
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu:
        import oracle
        cols = 192
        x_s = dy[:, :cols].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        oracle.quantize_tokens(x_s, used=int(offs[-1]))
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(M * cols * 3.03125 / dt / 1e9, 4), "unit": "GB/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": "%s: the first %d of %d hidden columns of dY (%d x %d elements), %.1f s"
                                         % (args.workload, cols, N, M, cols, dt)}
    print(json.dumps(res))


def bf16_context(cfg, ours_tflops, args, stream):
    """torch._grouped_mm on bf16 operands of the same shape and offs."""
    import torch

    dev = cfg["A"].device
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    a = torch.randn((N, M), generator=g, device=dev).to(torch.bfloat16)  # dY^T, contiguous
    b = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)  # X
    offs = cfg["offs"]
    try:
        ms, _ = time_steps(lambda: torch._grouped_mm(a, b, offs=offs), args, stream)
    except Exception as ex:  # not every build has a grouped GEMM for this layout
        return {"value": None, "error": str(ex)[:200]}
    finally:
        del a, b
    import workloads as W
    tf = W.useful_flops(cfg) / (ms * 1e-3) / 1e12
    return {"value": round(tf, 1), "unit": "TFLOP/s", "ms": round(ms, 4),
            "mxfp8_over_bf16": round(ours_tflops / tf, 3),
            "what": "torch._grouped_mm(dY^T bf16 [N, M], X bf16 [M, K], offs) -> [E, N, K], same steps/warmup, "
                    "same stream, this process",
            "comparable_to_pages": False,
            "note": "the blog's ~900 TFLOP/s BF16 comparator is its own library GEMM with its library versions; "
                    "torch._grouped_mm on this image takes another path, so this ratio is not the pages' "
                    "'x BF16' figure"}


class _Power:
    """Socket power and shader clock sampled while the GPU runs (amdsmi,
    read-only).  A sampler thread polls the energy accumulator and the GPU
    metrics table every 20 ms.  The accumulator advances about once a second,
    so power is taken between its first and last updates inside the busy
    window (energy difference over the firmware timestamps), and the clock is
    the mean of the current-GFX-clock readings in that window."""

    def __init__(self):
        import threading
        import torch
        self.error = None
        self.samples = []
        self.stop = threading.Event()
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
        except Exception as ex:  # no amdsmi on this host
            self.error = "amdsmi unavailable: %s" % str(ex)[:120]
            return
        try:
            props = torch.cuda.get_device_properties(torch.cuda.current_device())
            want = "%04x:%02x:%02x" % (getattr(props, "pci_domain_id", 0), getattr(props, "pci_bus_id", 0),
                                       getattr(props, "pci_device_id", 0))
            hs = amdsmi.amdsmi_get_processor_handles()
            self.h = next((x for x in hs if amdsmi.amdsmi_get_gpu_device_bdf(x).lower().startswith(want)), None)
            if self.h is None:
                self.error = "no amdsmi handle for PCI %s" % want
                return
            self.limit_w = amdsmi.amdsmi_get_power_info(self.h).get("power_limit")
        except Exception as ex:
            self.error = str(ex)[:200]
            return
        self.th = threading.Thread(target=self._run, daemon=True)
        self.th.start()

    def _run(self):
        a = self.amdsmi
        while not self.stop.is_set():
            t = time.perf_counter()
            try:
                e = a.amdsmi_get_energy_count(self.h)
                gm = a.amdsmi_get_gpu_metrics_info(self.h)
                self.samples.append((t, e["energy_accumulator"], e["timestamp"], e["counter_resolution"],
                                     gm.get("current_gfxclk"), gm.get("current_socket_power")))
            except Exception:
                pass
            self.stop.wait(0.02)

    def finish(self, t0, t1, sustained_ms, tflops=None, peak=None):
        if self.error:
            return {"error": self.error}
        self.stop.set()
        self.th.join()
        try:
            win = [x for x in self.samples if t0 + 0.3 <= x[0] <= t1]  # skip the ramp-up
            edges = [x for i, x in enumerate(win) if i == 0 or x[1] != win[i - 1][1]]
            if len(edges) < 3:
                return {"error": "too few energy-counter updates in the busy window (%d)" % len(edges)}
            a, b = edges[1], edges[-1]  # first and last update seen inside the window
            joules = (b[1] - a[1]) * a[3] * 1e-6
            secs = (b[2] - a[2]) * 1e-9
            watts = joules / secs
            clks = [x[4] for x in win if isinstance(x[4], (int, float)) and x[4] > 0]
            clk = sum(clks) / len(clks) if clks else None
            lim = self.limit_w
            res = {"avg_socket_w": round(watts, 1), "joules_per_step": round(watts * sustained_ms * 1e-3, 4),
                   "gfxclk_mhz_mean": round(clk, 1) if clk else None,
                   "power_limit_w": round(lim / 1e6, 1) if isinstance(lim, (int, float)) else None,
                   "window_s": round(secs, 3),
                   "how": "amdsmi energy accumulator between its first and last update in the first sustained "
                          "pass; clock = mean current GFX clock over it; joules = power x that pass's mean time "
                          "per step"}
            if clk and tflops and peak:
                # the peak scales with the shader clock (quoted at 2.4 GHz)
                res["clock_normalised_frac"] = round(tflops / (peak * clk / 2400.0), 4)
            return res
        except Exception as ex:
            return {"error": str(ex)[:200]}
        finally:
            try:
                self.amdsmi.amdsmi_shut_down()
            except Exception:
                pass


def _estimate_ms(step, stream, n=8):
    """Rough time per step from a short burst (sizes the untimed pre-run)."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    return max(a.elapsed_time(b) / n, 1e-3)


def padded_rows(cfg, ld):
    """The operands copied into row-strided storage ([rows, ld] buffers whose
    first M columns hold the values; the rest never read), as [:, :M] views."""
    import torch
    c = dict(cfg)
    M = cfg["M"]
    for k, div in (("A", 1), ("B", 1), ("sA", 32), ("sB", 32)):
        t = cfg[k]
        buf = torch.zeros((t.shape[0], ld // div), dtype=t.dtype, device=t.device)
        buf[:, :M // div] = t
        c[k] = buf[:, :M // div]
    return c


def time_steps(step, args, stream, prerun_s=None):
    """W untimed warm-up steps; an untimed pre-run of back-to-back steps for
    about prerun_s seconds, so that the timed steps run at the clock and power
    the chip keeps under sustained load (a short window straight after a few
    warm-up steps catches the clock still ramping); a synchronisation; then
    exactly K steps between HIP events on `stream`.  Returns (ms per step,
    wall seconds of the timed region)."""
    import torch

    if prerun_s is None:
        prerun_s = args.prerun
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if prerun_s > 0:
        est = _estimate_ms(step, stream)
        for _ in range(int(prerun_s * 1e3 / est)):
            step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / args.steps, time.perf_counter() - t0


def sustained_leg(step, ms_per_step, stream, seconds, passes=2, chunk=8, tflops_of_ms=None, peak=None, power=True):
    """`passes` back-to-back runs of about `seconds` each, with a HIP event on
    `stream` every `chunk` steps: per pass, the mean and median time per step
    over its chunks.  The socket power and clock are sampled over the first
    pass (when power is true)."""
    import torch

    out = {"passes": [], "chunk_steps": chunk, "seconds_per_pass": seconds}
    pw = None
    for k in range(passes):
        nch = max(2, int(seconds * 1e3 / (ms_per_step * chunk)))
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nch + 1)]
        torch.cuda.synchronize()
        if k == 0 and power:
            pw = _Power()
        t0 = time.perf_counter()
        evs[0].record(stream)
        for c in range(nch):
            for _ in range(chunk):
                step()
            evs[c + 1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        per = np.array([evs[c].elapsed_time(evs[c + 1]) / chunk for c in range(nch)])
        rec = {"steps": nch * chunk, "seconds": round(float(per.sum() * chunk / 1e3), 3),
               "mean_ms": round(float(per.mean()), 5), "median_ms": round(float(np.median(per)), 5)}
        if tflops_of_ms:
            rec["mean_tflops"] = round(tflops_of_ms(rec["mean_ms"]), 2)
        out["passes"].append(rec)
        if k == 0 and pw is not None:
            out["power"] = pw.finish(t0, t1, rec["mean_ms"], rec.get("mean_tflops"), peak)
    return out


def cold_leg(step, stream, calls=30, flush_bytes=1 << 30):
    """Cold caches: each call timed alone (HIP events around the call only,
    on the launch stream) right after a write of flush_bytes, more than the
    eight XCD L2s (4 MB each) and the 256 MB Infinity Cache hold together, so
    the call starts with none of its operands cached; beside it the same
    per-call timing without the flush.  The pages report no difference
    between cold and warm caches for their kernel."""
    import torch

    buf = torch.empty(flush_bytes, dtype=torch.uint8, device=stream.device)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]

    def run(flush):
        with torch.cuda.stream(stream):
            for i, (a, b) in enumerate(evs):
                if flush:
                    buf.fill_(i & 0xFF)
                a.record(stream)
                step()
                b.record(stream)
        stream.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    run(False)  # warm the code paths once
    warm, cold = run(False), run(True)
    del buf
    return {"calls": calls, "flush_bytes": flush_bytes,
            "cold_median_ms": round(float(np.median(cold)), 5), "cold_mean_ms": round(float(cold.mean()), 5),
            "warm_median_ms": round(float(np.median(warm)), 5), "warm_mean_ms": round(float(warm.mean()), 5),
            "cold_over_warm": round(float(np.median(cold) / np.median(warm)), 4),
            "what": "each call timed alone between HIP events, after a write of flush_bytes (evicts the L2s and "
                    "the Infinity Cache) or without it"}


def graph_leg(make_step, stream, calls=20, seconds=1.0):
    """The call captured `calls` times into one HIP graph (on a capture
    stream, with the workspace allocated beforehand: the entry points record
    only kernel launches) and the graph replayed back to back for about
    `seconds`: the device-side time per call without the host's per-call
    argument marshalling, which is what bounds the tiny workload."""
    import torch

    cap = torch.cuda.Stream(device=stream.device)
    cap.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        step = make_step(cap)
        step()  # one eager call on the capture stream first
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            for _ in range(calls):
                step()
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        t0 = time.time()
        g.replay()
        torch.cuda.synchronize()
        one = max(time.time() - t0, 1e-6)
        reps = max(2, int(seconds / one))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (reps * calls)
    del g
    return {"calls_per_graph": calls, "replays": reps, "ms_per_call": round(ms, 6),
            "what": "the same call captured %d times into one HIP graph, replayed back to back (HIP events on the "
                    "launch stream): device-side time per call without the host's per-call overhead" % calls}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="16b_24k")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bf16 torch._grouped_mm context leg")
    ap.add_argument("--no-power", action="store_true", help="skip the power / energy / clock sampling")
    ap.add_argument("--no-sustained", action="store_true", help="skip the two sustained passes (and power)")
    ap.add_argument("--prerun", type=float, default=2.0,
                    help="seconds of untimed back-to-back steps before the timed ones (0 for counter runs)")
    ap.add_argument("--no-plain", action="store_true", help="skip timing the entry point without a workspace")
    ap.add_argument("--no-padded", action="store_true", help="skip timing the row-padded layout")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache per-call timing")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--ld-pad", type=int, default=0,
                    help="store the operands with rows M + LD_PAD tokens apart (a multiple of 32) for the headline")
    ap.add_argument("--entry", choices=("ws", "plain"), default="ws",
                    help="weight-gradient entry point of the headline: mxfp8_wgrad_grouped_ws (default) or "
                         "mxfp8_wgrad_grouped")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (each expert-parallel rank "
              "runs the same kernel on its own experts; see the sharding paragraph of the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    import mxfp8_ragged_grouped_amd as mxw
    import workloads as W

    if args.workload in W.ROWS_CONFIGS:
        bench_rows(args)
        return
    if args.workload in QUANT_WORKLOADS:
        bench_quant(args)
        return
    if args.workload in W.BF16_CONFIGS:
        bench_bf16(args)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.make_config(args.workload, device=dev)
    E, N, K, M = cfg["E"], cfg["N"], cfg["K"], cfg["M"]
    if args.ld_pad:
        if args.entry == "plain":
            sys.exit("--ld-pad needs the workspace entry (the entry without one takes contiguous operands)")
        cfg = padded_rows(cfg, M + args.ld_pad)
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    ld = cfg["A"].stride(0)
    ws_bytes = mxw.workspace_size(E, M, N, K, ld)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    plain_first = args.entry == "plain"

    def step_ws():
        mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, stream=stream, workspace=ws)

    def step_plain():
        mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, stream=stream, plain=True)

    step = step_plain if plain_first else step_ws
    ms, wall = time_steps(step, args, stream)

    flops = W.useful_flops(cfg)
    tflops_of = lambda t_ms: flops / (t_ms * 1e-3) / 1e12
    tflops = tflops_of(ms)
    alg_bytes = W.algorithmic_bytes(cfg)
    traffic = load_traffic(args.workload)
    small = M // E < 8192  # the small-token workloads: 1 s sustained passes

    if plain_first:
        kernels = 1
        timed = "the whole call of mxfp8_wgrad_grouped (one kernel, wgrad_kernel)"
    else:
        kernels = 2 if mxw.scale_shuffle(E, M) else 1
        timed = ("the whole call of mxfp8_wgrad_grouped_ws (%s); traffic is wgrad_kernel's" %
                 ("scale_shuffle_kernel then wgrad_kernel" if kernels == 2 else "wgrad_kernel"))
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / PAGES_TFLOPS_16B, 4) if args.workload == "16b_24k" else None,
        "dtype": "mxfp8(e4m3,e8m0/32)->fp32acc->bf16",
        "data": "synthetic (seeded Dirichlet routing, N(0,1) values, MXFP8-quantised along tokens)",
        "config": {"workload": args.workload, "E": E, "N": N, "K": K, "M": M,
                   "tokens_per_expert_mean": M // E, "busiest_over_mean": round(cfg["skew"], 3),
                   "routing_seed": cfg["routing_seed"], "value_seed": cfg["value_seed"],
                   "entry": "mxfp8_wgrad_grouped" if plain_first else "mxfp8_wgrad_grouped_ws",
                   "row_stride_tokens": ld,
                   "workspace_bytes": 0 if plain_first else ws_bytes,
                   "columns": 0 if plain_first else mxw.columns(E, M, N, K),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_TFLOPS, 4),
                     "traffic": load_traffic(args.workload + "_plain") if plain_first else (
                         load_traffic("%s_ld%d" % (args.workload, args.ld_pad)) if args.ld_pad else traffic),
                     "kernels_per_call": kernels, "timed": timed},
        "hbm_gbps_algorithmic": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
        "wall_s_timed": round(wall, 3),
        "timing": "%d untimed warm-up steps, an untimed ~%g s back-to-back pre-run (steady clock and power), a "
                  "synchronisation, then exactly %d steps between HIP events on the launch stream" % (
                      args.warmup, args.prerun, args.steps),
    }
    if args.workload == "16b_24k":
        res["baseline_note"] = ("vs_baseline = value / 2,174 TFLOP/s, the blog's kernel at the 16B ragged shape on "
                                "MI355X (their routing: linear ramp / ragged draw at 1.5x; ours: seeded Dirichlet "
                                "at %.2fx)" % cfg["skew"])
    note("%s: %.4f ms per step; sustained passes" % (args.workload, ms))
    if not args.no_sustained:
        sus = sustained_leg(step, ms, stream, 1.0 if small else 3.0, tflops_of_ms=tflops_of, peak=PEAK_TFLOPS,
                            power=not args.no_power)
        if "power" in sus:
            res["power"] = sus.pop("power")
        res["sustained"] = sus
    note("padded rows, the entry without a workspace, cold caches, graph replay")
    if not args.no_padded and not plain_first and not args.ld_pad:
        # the same operands in row-padded storage (ld = M + 128 tokens: the
        # layout mxfp8_quantize_tokens writes with ld), the same entry point
        pc = padded_rows(cfg, M + 128)
        pws = torch.empty(max(mxw.workspace_size(E, M, N, K, M + 128), 1), dtype=torch.uint8, device=dev)
        step_pad = lambda: mxw.wgrad(pc["A"], pc["sA"], pc["B"], pc["sB"], pc["offs"], out=out, stream=stream,
                                     workspace=pws)
        pdms, _ = time_steps(step_pad, args, stream, prerun_s=min(args.prerun, 1.0))
        res["padded_rows"] = {"row_stride_tokens": M + 128, "ms_per_step": round(pdms, 5),
                              "tflops": round(tflops_of(pdms), 2), "frac": round(tflops_of(pdms) / PEAK_TFLOPS, 4),
                              "traffic": load_traffic("%s_ld128" % args.workload),
                              "what": "the same call on the same values stored with rows M + 128 tokens apart (no "
                                      "multiple-of-64 KiB row stride, so the lines a tile reads at once spread over "
                                      "the L2 sets), same timing method, this process; a layout choice of the "
                                      "operands' producer, not the headline's layout"}
        del pc, pws
    if not args.no_plain and not plain_first:
        pms, _ = time_steps(step_plain, args, stream, prerun_s=min(args.prerun, 1.0))
        ptf = tflops_of(pms)
        res["plain_entry"] = {"entry": "mxfp8_wgrad_grouped", "ms_per_step": round(pms, 5),
                              "tflops": round(ptf, 2), "frac": round(ptf / PEAK_TFLOPS, 4),
                              "what": "the entry point without a workspace (one workgroup per output tile, scales "
                                      "from the caller's planes), same timing method, this process"}
    if not args.no_cold:
        res["cold_caches"] = cold_leg(step, stream)
    if not args.no_graph:
        def make_step(st):
            if plain_first:
                return lambda: mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, stream=st,
                                         plain=True)
            return lambda: mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, stream=st,
                                     workspace=ws)
        gr = graph_leg(make_step, stream, seconds=1.0 if small else 2.0)
        gr["tflops"] = round(tflops_of(gr["ms_per_call"]), 2)
        res["graph_replay"] = gr
    if not args.no_bf16:
        note("torch bf16 grouped GEMM on the same problem")
        res["bf16_context"] = bf16_context(cfg, tflops, args, stream)
    if not args.no_cpu:
        note("CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(cfg, cfg["A"].cpu().numpy(), cfg["sA"].cpu().numpy(),
                                           cfg["B"].cpu().numpy(), cfg["sB"].cpu().numpy(),
                                           cfg["offs"].cpu().numpy())
    print(json.dumps(res))


if __name__ == "__main__":
    main()
