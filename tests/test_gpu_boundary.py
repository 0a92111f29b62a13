"""The C-ABI boundary of the weight gradient (needs an MI355X).

mxfp8_wgrad_grouped allocates nothing, keeps no state and synchronises
nothing; mxfp8_wgrad_grouped_ws does the same with a caller-owned workspace.
These tests check what that promises:

  * a fresh process whose very first library calls are made under HIP-graph
    capture (both entry points, column mode included) replays correctly;
  * two different problems enqueued on two streams at once, each with its own
    workspace, both match the oracle and their own sequential results bit for
    bit;
  * the workspace query and the workspace errors (missing, short, misaligned);
  * the blog's copy-based check (section 7): with garbage in the padding, the
    ragged call equals the same call on operands copied down to the experts'
    real token width, bitwise (the entry point without a workspace always;
    the workspace entry when both widths take the same schedule);
  * without a workspace an expert's bits depend on its own window only;
  * malformed offs (decreasing, past M, negative, not 32-aligned) return,
    write nothing outside out, and give the clamped windows' results.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import mxfp8_ragged_grouped_amd as mxw
import oracle
import workloads as W
from helpers import BF16_NAN, ENTRIES, bf16_bits, check_close, host, run_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(msg):
    print("[gpu-case] " + msg, flush=True)


FIRST_CALL_CHILD = r'''
import sys
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[1] + "/tests")
import numpy as np, torch
import mxfp8_ragged_grouped_amd as mxw, oracle, workloads as W
from helpers import bf16_bits, check_close, host
dev = "cuda"
cases = [("column", W.make_random(2, 512, 768, 16416, [8992, 7392], seed=1400, device=dev)),
         ("per_tile", W.make_random(3, 272, 528, 1024, [96, 0, 800], seed=1401, device=dev))]
torch.cuda.synchronize()
graphs = []
s = torch.cuda.Stream()
s.wait_stream(torch.cuda.current_stream())
for name, cfg in cases:
    for plain in (False, True):
        out = torch.full((cfg["E"], cfg["N"], cfg["K"]), float("nan"), dtype=torch.bfloat16, device=dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], out=out, plain=plain)
        graphs.append((name, plain, cfg, out, g))
torch.cuda.current_stream().wait_stream(s)
torch.cuda.synchronize()
print("captured %d graphs before any eager library call" % len(graphs), flush=True)
for name, plain, cfg, out, g in graphs:
    ref = oracle.wgrad_f64(*host(cfg))
    first = None
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bits = bf16_bits(out)
        check_close(bits, ref, what="%s plain=%s replay %d" % (name, plain, r))
        if first is None:
            first = bits
        assert (bits == first).all(), "%s plain=%s: replay %d differs" % (name, plain, r)
    eager = mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], cfg["offs"], plain=plain)
    torch.cuda.synchronize()
    assert (bf16_bits(eager) == first).all(), "%s plain=%s: eager differs from the replays" % (name, plain)
    print("ok %s plain=%s" % (name, plain), flush=True)
print("FIRST_CALL_OK", flush=True)
'''


def test_graph_capture_as_first_call():
    """A fresh process captures both entry points (column mode and one
    workgroup per tile) before making any eager library call."""
    say("first call under graph capture (child process)")
    r = subprocess.run([sys.executable, "-c", FIRST_CALL_CHILD, ROOT], capture_output=True, text=True, timeout=110)
    print(r.stdout[-3000:])
    print(r.stderr[-3000:])
    assert r.returncode == 0 and "FIRST_CALL_OK" in r.stdout


def test_two_streams_at_once():
    """Two different shapes (one in column mode) on two streams, enqueued
    alternately with no synchronisation between them; each stream has its own
    workspace from torch's allocator."""
    ca = W.make_random(8, 1408, 2048, 65536, [12000, 4000, 9600, 0, 11200, 8000, 6400, 14336], seed=1500,
                       device=DEV)
    cb = W.make_random(2, 512, 768, 16416, [8992, 7392], seed=1501, device=DEV)
    assert mxw.columns(8, 65536, 1408, 2048) > 0 and mxw.columns(2, 16416, 512, 768) > 0
    say("two streams: sequential references")
    seq_a = bf16_bits(run_gpu(ca))
    seq_b = bf16_bits(run_gpu(cb))
    seq_bp = bf16_bits(run_gpu(cb, entry="plain"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    oa = torch.empty((8, 1408, 2048), dtype=torch.bfloat16, device=DEV)
    ob = torch.empty((2, 512, 768), dtype=torch.bfloat16, device=DEV)
    obp = torch.empty((2, 512, 768), dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    say("two streams: 4 rounds interleaved")
    for _ in range(4):
        mxw.wgrad(ca["A"], ca["sA"], ca["B"], ca["sB"], ca["offs"], out=oa, stream=s1)
        mxw.wgrad(cb["A"], cb["sA"], cb["B"], cb["sB"], cb["offs"], out=ob, stream=s2)
        mxw.wgrad(cb["A"], cb["sA"], cb["B"], cb["sB"], cb["offs"], out=obp, stream=s2, plain=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(oa), seq_a)
    np.testing.assert_array_equal(bf16_bits(ob), seq_b)
    np.testing.assert_array_equal(bf16_bits(obp), seq_bp)
    check_close(seq_a, oracle.wgrad_f64(*host(ca)), what="stream 1")
    refb = oracle.wgrad_f64(*host(cb))
    check_close(seq_b, refb, what="stream 2 (workspace)")
    check_close(seq_bp, refb, what="stream 2 (no workspace)")


def test_workspace_query_and_errors():
    E, N, K = 8, 1408, 2048
    # 16 columns x 2 x 16 partial tiles of 256 KiB + counters, and the shuffled scales
    cols = mxw.columns(E, 196608, N, K)
    want = 4096 + cols * 2 * 16 * 256 * 1024 + (6 + 8) * 384 * 4096
    assert mxw.workspace_size(E, 196608, N, K) == want
    assert mxw.workspace_size(E, 8192, N, K) == 0              # 1,024 tokens/expert: no workspace used
    assert mxw.workspace_size(32, 262144, 4096, 7168) == (16 + 28) * 512 * 4096  # shuffled scales only
    assert mxw.bf16_workspace_size(E, 196608, N, K) == 4096 + cols * 2 * 16 * 256 * 1024
    cfg = W.make_random(2, 512, 768, 16416, [8992, 7392], seed=1600, device=DEV)
    need = mxw.workspace_size(2, 16416, 512, 768)
    assert need > 0
    ws = torch.empty(need + 256, dtype=torch.uint8, device=DEV)
    out = torch.empty((2, 512, 768), dtype=torch.bfloat16, device=DEV)
    args = [cfg[k].data_ptr() for k in ("A", "sA", "B", "sB", "offs")] + [2, 16416, 512, 768, out.data_ptr()]
    stream = torch.cuda.current_stream().cuda_stream
    say("workspace errors (nothing launched)")
    assert mxw.mxfp8_wgrad_grouped_ws(*args, 0, 0, stream) == -6
    assert mxw.mxfp8_wgrad_grouped_ws(*args, ws.data_ptr(), need - 1, stream) == -6
    assert mxw.mxfp8_wgrad_grouped_ws(*args, ws.data_ptr() + 16, need, stream) == -6
    assert mxw.mxfp8_wgrad_grouped_ws(*args, ws.data_ptr() + 256, need, stream) == 0
    torch.cuda.synchronize()
    check_close(bf16_bits(out), oracle.wgrad_f64(*host(cfg)), what="workspace at an offset")
    # a shape that needs none accepts a NULL workspace
    small = W.make_random(3, 272, 528, 1024, [96, 0, 800], seed=1601, device=DEV)
    o2 = torch.empty((3, 272, 528), dtype=torch.bfloat16, device=DEV)
    a2 = [small[k].data_ptr() for k in ("A", "sA", "B", "sB", "offs")] + [3, 1024, 272, 528, o2.data_ptr()]
    assert mxw.workspace_size(3, 1024, 272, 528) == 0
    assert mxw.mxfp8_wgrad_grouped_ws(*a2, 0, 0, stream) == 0
    torch.cuda.synchronize()
    check_close(bf16_bits(o2), oracle.wgrad_f64(*host(small)), what="no workspace needed")


def copy_down(cfg, used):
    """The operands cut down to the experts' real token width `used`."""
    c = dict(cfg)
    for k in ("A", "B"):
        c[k] = cfg[k][:, :used].contiguous()
    for k in ("sA", "sB"):
        c[k] = cfg[k][:, :used // 32].contiguous()
    c["M"] = used
    return c


@pytest.mark.parametrize("entry,E,N,K,M,sizes", [
    ("plain", 4, 272, 528, 2048, [160, 0, 928, 96]),          # aligned rows padded -> 1,184 (paired scale path)
    ("plain", 3, 1040, 272, 26624, [12000, 0, 9600]),        # long experts, one workgroup per tile
    ("ws", 4, 272, 528, 2048, [160, 0, 928, 96]),            # no column mode at either width
    ("ws", 2, 512, 768, 20480, [8992, 7392]),                # column mode at both widths: the same cuts
])
def test_copy_down_bitwise(entry, E, N, K, M, sizes):
    """Blog section 7's check: NaN codes and 0xFF scales in the padding, and
    the call equals the same call on copies cut to offs[E-1] tokens, bit for
    bit.  (The workspace entry's column mode cuts by the cost of the experts'
    windows, which does not change here; when the cut-down width switches the
    mode the two differ only within the FP32 summation tolerance, which the
    oracle comparisons cover.)"""
    cfg = W.make_random(E, N, K, M, sizes, seed=1700 + M + E, device=DEV)
    used = int(np.sum(sizes))
    cfg["A"][:, used:] = 0x7F
    cfg["B"][:, used:] = 0xFF
    cfg["sA"][:, used // 32:] = 0xFF
    cfg["sB"][:, used // 32:] = 0xFF
    if entry == "ws":
        assert (mxw.columns(E, M, N, K) > 0) == (mxw.columns(E, used, N, K) > 0)
    say("copy-down [%s] E=%d M=%d -> %d" % (entry, E, M, used))
    padded = bf16_bits(run_gpu(cfg, entry=entry))
    cut = bf16_bits(run_gpu(copy_down(cfg, used), entry=entry))
    np.testing.assert_array_equal(padded, cut)
    check_close(cut, oracle.wgrad_f64(*host(copy_down(cfg, used))), what="copy-down [%s]" % entry)


def test_plain_bits_depend_on_own_window_only():
    """Without a workspace an expert's output is one workgroup's sum over its
    own window: shrinking the last expert (more padding) or making M larger
    leaves every other expert's bits unchanged."""
    sizes = [4000, 1216, 9600, 2560]
    cfg = W.make_random(4, 528, 784, 20480, sizes, seed=1800, device=DEV)
    say("own-window bits (no workspace)")
    base = bf16_bits(run_gpu(cfg, entry="plain"))
    short = torch.tensor(np.cumsum([4000, 1216, 9600, 640]), dtype=torch.int32, device=DEV)
    other = bf16_bits(run_gpu(cfg, entry="plain", offs=short))
    np.testing.assert_array_equal(other[:3], base[:3])
    wide = dict(cfg)
    for k in ("A", "B"):
        wide[k] = torch.cat([cfg[k], torch.full_like(cfg[k][:, :4096], 0x7F)], dim=1).contiguous()
    for k in ("sA", "sB"):
        wide[k] = torch.cat([cfg[k], torch.full_like(cfg[k][:, :128], 0xFF)], dim=1).contiguous()
    wide["M"] = cfg["M"] + 4096
    np.testing.assert_array_equal(bf16_bits(run_gpu(wide, entry="plain")), base)


def expert_ref(hops, start, end):
    """The oracle for one expert whose window is [start, end)."""
    A, sA, B, sB, _ = hops
    if end <= start:
        return np.zeros((A.shape[0], B.shape[0]))
    if start == 0:
        return oracle.wgrad_f64(A, sA, B, sB, np.array([end], np.int32))[0]
    return oracle.wgrad_f64(A, sA, B, sB, np.array([start, end], np.int32))[1]


MALFORMED = [
    # (E, N, K, M, offs): windows are [clamp(offs[g-1]), max(clamp(offs[g]), clamp(offs[g-1])))
    # with clamp to [0, M] (start 0 for the first expert)
    (4, 272, 528, 2048, [1024, 512, 1536, 2048]),      # decreasing: expert 1 empty, expert 2 = [512, 1536)
    (4, 272, 528, 2048, [256, 1024, 4096, 9999]),      # past M: clamped to M
    (4, 272, 528, 2048, [-64, 256, 2048, 1024]),       # negative, then decreasing at the end
    (4, 272, 528, 2048, [100, 300, 300, 2000]),        # not multiples of 32: values unspecified, bounds only
    (4, 272, 528, 20480, [8192, 4096, 30000, 1 << 30]),  # scale pre-shuffle with a workspace
    (2, 512, 768, 16416, [8992, 4000]),                # column mode with a workspace; decreasing
    (2, 512, 768, 16416, [-32, 40000]),                # column mode; negative and past M
    (2, 512, 768, 16416, [5000, 16000]),               # column mode; not multiples of 32
]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("case", range(len(MALFORMED)))
def test_malformed_offs(entry, case):
    """Malformed offs give unspecified values but no access outside the
    operands and out: the call returns, the poison around out survives, every
    element of out is written, and (for 32-aligned values) each expert equals
    the oracle on its clamped window."""
    E, N, K, M, offs_list = MALFORMED[case]
    cfg = W.make_random(E, N, K, M, [M // E // 32 * 32] * E, seed=1900 + case, device=DEV)
    offs = torch.tensor(offs_list, dtype=torch.int32, device=DEV)
    guard = 4096  # bf16 elements of poison on each side of out
    big = torch.empty(E * N * K + 2 * guard, dtype=torch.bfloat16, device=DEV)
    big.view(torch.int16).fill_(BF16_NAN)
    out = big[guard:guard + E * N * K].view(E, N, K)
    say("malformed offs %s M=%d [%s]" % (offs_list, M, entry))
    mxw.wgrad(cfg["A"], cfg["sA"], cfg["B"], cfg["sB"], offs, out=out, plain=(entry == "plain"))
    torch.cuda.synchronize()
    gb = bf16_bits(big)
    assert (gb[:guard] == BF16_NAN).all() and (gb[-guard:] == BF16_NAN).all(), "store outside out"
    bits = bf16_bits(out)
    assert not (bits == BF16_NAN).any(), "an output left unwritten"
    if any(v % 32 for v in offs_list):
        return
    hops = host(cfg)
    clamp = [min(max(v, 0), M) for v in offs_list]
    for g in range(E):
        start = clamp[g - 1] if g else 0
        end = max(clamp[g], start)
        if end == start:
            assert (bits[g] == 0).all(), "expert %d with an empty clamped window not +0" % g
        else:
            check_close(bits[g], expert_ref(hops, start, end), what="malformed offs %s expert %d" % (offs_list, g))


def strided(cfg, ld, fill=0x7F):
    """The operands copied into row-strided storage: [rows, ld] buffers (the
    padding columns hold NaN codes / 0xFF scales) and their [:, :M] views."""
    c = dict(cfg)
    M = cfg["M"]
    for k in ("A", "B"):
        t = cfg[k]
        buf = torch.full((t.shape[0], ld), fill, dtype=torch.uint8, device=t.device)
        buf[:, :M] = t
        c[k] = buf[:, :M]
    for k in ("sA", "sB"):
        t = cfg[k]
        buf = torch.full((t.shape[0], ld // 32), 0xFF, dtype=torch.uint8, device=t.device)
        buf[:, :M // 32] = t
        c[k] = buf[:, :M // 32]
    return c


@pytest.mark.parametrize("E,N,K,M,sizes,pad", [
    (8, 1408, 2048, 65536, [12000, 4000, 9600, 0, 11200, 8000, 6400, 14336], 128),  # column mode
    (3, 272, 528, 2048, [160, 0, 1856], 128),        # short experts: direct scales -> pre-shuffle (ld % 512)
    (3, 272, 528, 2048, [160, 0, 1856], 512),        # ld % 512 == 0: direct 16-byte scale groups
    (4, 528, 784, 20480, [4000, 1216, 9600, 2560], 4224),  # long experts, one workgroup per tile
])
def test_row_stride_bitwise(E, N, K, M, sizes, pad):
    """The workspace entry (and the no-allocation one) on padded rows
    (ld = M + pad) gives the bits of the contiguous call: the same schedule
    and the same scale bytes, whichever scale path the stride selects."""
    cfg = W.make_random(E, N, K, M, sizes, seed=2000 + pad + M, device=DEV)
    ld = M + pad
    say("row stride: E=%d N=%d K=%d M=%d ld=%d" % (E, N, K, M, ld))
    base = bf16_bits(run_gpu(cfg))
    sc = strided(cfg, ld)
    assert sc["A"].stride(0) == ld and sc["sA"].stride(0) == ld // 32
    np.testing.assert_array_equal(bf16_bits(run_gpu(sc)), base)
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device=DEV)
    rc = mxw.mxfp8_wgrad_grouped_noalloc(*(sc[k].data_ptr() for k in ("A", "sA", "B", "sB", "offs")), E, M, N, K,
                                         out.data_ptr(), torch.cuda.current_stream().cuda_stream, ld=ld)
    assert rc == 0, mxw.strerror(rc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(out), base)
    with pytest.raises(ValueError):
        mxw.wgrad(sc["A"], sc["sA"], sc["B"], sc["sB"], sc["offs"], plain=True)
    check_close(base, oracle.wgrad_f64(*host(cfg)), what="row stride %d" % ld)


def test_quantize_padded_rows_end_to_end():
    """The quantiser writing padded rows (ld = M + 128): the [H, M] codes and
    scales equal the contiguous ones bit for bit, the padding columns keep
    their poison, and the weight gradient of the padded operands equals the
    contiguous one bit for bit."""
    E, N, K, M = 4, 400, 528, 8192
    sizes = [2048, 0, 3584, 2368]
    offs = torch.tensor(np.cumsum(sizes), dtype=torch.int32, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(2100)
    dy = torch.randn((M, N), generator=g, device=DEV).to(torch.bfloat16)
    x = (0.5 * torch.randn((M, K), generator=g, device=DEV)).to(torch.bfloat16)
    ld = M + 128
    say("quantise into padded rows, then the weight gradient")
    qa, sa = mxw.quantize_tokens(dy, offs)
    qb, sb = mxw.quantize_tokens(x, offs)
    pa_q = torch.full((N, ld), 0x5A, dtype=torch.uint8, device=DEV)
    pa_s = torch.full((N, ld // 32), 0x5A, dtype=torch.uint8, device=DEV)
    pb_q = torch.full((K, ld), 0x5A, dtype=torch.uint8, device=DEV)
    pb_s = torch.full((K, ld // 32), 0x5A, dtype=torch.uint8, device=DEV)
    mxw.quantize_tokens(dy, offs, q=pa_q[:, :M], s=pa_s[:, :M // 32], ld=ld)
    mxw.quantize_tokens(x, offs, q=pb_q[:, :M], s=pb_s[:, :M // 32], ld=ld)
    torch.cuda.synchronize()
    assert torch.equal(pa_q[:, :M], qa) and torch.equal(pa_s[:, :M // 32], sa)
    assert torch.equal(pb_q[:, :M], qb) and torch.equal(pb_s[:, :M // 32], sb)
    assert (pa_q[:, M:] == 0x5A).all().item() and (pb_s[:, M // 32:] == 0x5A).all().item()
    contiguous = bf16_bits(mxw.wgrad(qa, sa, qb, sb, offs))
    padded = bf16_bits(mxw.wgrad(pa_q[:, :M], pa_s[:, :M // 32], pb_q[:, :M], pb_s[:, :M // 32], offs))
    np.testing.assert_array_equal(padded, contiguous)
    ref = oracle.wgrad_f64(qa.cpu().numpy(), sa.cpu().numpy(), qb.cpu().numpy(), sb.cpu().numpy(), offs.cpu().numpy())
    check_close(contiguous, ref, what="quantised operands")
