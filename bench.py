#!/usr/bin/env python3
"""Benchmark of the chunk-parallel gated delta-rule prefill on one MI355X.

One step = one whole layer of the hot path (chunk tiles + serial scan + output)
over the hybrid-model GDN layer: B=1, T=32768, 16 key heads / 48 value heads,
dk = dv = 128, bf16 q/k/v, fp32 gate and beta, chunk 64, nonzero h0 (synthetic
seeded inputs, resident in HBM before timing).  Prints one JSON line.

A step is one whole gdn_chunk_fwd call in the library's own composition for the
workload, between HIP events recorded on the library's stream.  A 1 GiB scratch
write before each step (outside its events) starts every step cache-cold; the
headline is the median step, with the minimum and a warm-cache median beside it.
The split composition's two stages are then timed one by one in a second pass
(per-kernel figures).  The oracle (fp64 token-serial, OpenMP) is timed on a
bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3

METRIC = "GDN chunk-prefill tokens/s per layer (HV=48,T=32k,d=128); MFMA % of peak"

# Context only (not a baseline of this metric): the stratat.com pull #1296 page, section
# "Measured verdict on gfx1100", times an engine's whole GDN recurrence for a 32k-token
# prefill on a Radeon 7900 XTX, over a number of layers it does not state, so no per-layer
# rate follows from these figures.
GFX1100_CONTEXT = {
    "source": "stratat.com pull #1296, 'Measured verdict on gfx1100' (Radeon 7900 XTX, nightly ROCm)",
    "workload": "engine GDN recurrence, 32k-token prefill, HV=48, state 128; layer count not stated",
    "serial_cols_pipe_ms": 1318, "wy_rocwmma_arm_ms_equivalent": 3050, "wy_fma_arm_ms": 189878,
    "comparable": False,
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(spec, chunk):
    """Algorithmic bytes and flops of the two kernels for one layer.

    prep (per chunk and key head, then per value head of the group):
      bytes: q, k chunk rows + g, beta rows + T and P fragments written (bf16)
      flops: K K^T and Q K^T lower halves 2 C^2 dk per key head; solve C^3/3 per value head
    scan (per chunk and value head, 16 state columns per wave):
      bytes: q, k rows (once per key head), v, o, g, beta, T and P fragments read; h0, hT
      flops: K.H and Ktil^T R  4 C dk dv;  Q.H  2 C dk dv;  P.R and T.X at half  2 C^2 dv / 2 each
    """
    T, hk, hv, dk, dv = spec.tokens, spec.hk, spec.hv, spec.dk, spec.dv
    n_seq = spec.n_seq
    nch = sum((l + chunk - 1) // chunk for l in spec.seq_lens)
    esz = 2
    # T and P are stored as the lower-triangle operand fragments: 6 of the 8 16x32
    # fragments of a 64 x 64 tile, both of a 32 x 32 tile
    tile = sum(mt // 2 + 1 for mt in range(chunk // 16)) * 512 * esz
    qk = 2 * T * hk * dk * 2
    # gate (per head [T][hv], or per key channel [T][hv][dk]) and beta, fp32
    gb = T * hv * (dk if spec.gate == "channel" else 1) * 4 + T * hv * 4
    prep_bytes = qk + gb + 2 * nch * hv * tile
    prep_flops = nch * hk * 2 * chunk * chunk * dk + nch * hv * chunk ** 3 / 3
    state = 2 * n_seq * hv * dk * dv * 4 if spec.h0 else n_seq * hv * dk * dv * 4
    scan_bytes = qk + gb + 2 * T * hv * dv * 2 + 2 * nch * hv * tile + state
    scan_flops = nch * hv * (6 * chunk * dk * dv + 2 * chunk * chunk * dv)
    # compulsory bytes of the whole layer: q, k, v, g, beta in; o out; h0 in, hT out
    layer_bytes = qk + gb + 2 * T * hv * dv * 2 + state
    return dict(prep_bytes=prep_bytes, prep_flops=prep_flops, scan_bytes=scan_bytes,
                scan_flops=scan_flops, chunks=nch, layer_bytes=layer_bytes)


def scope_flops(spec, chunk):
    """Algorithmic flops of one layer as the hot-path scope table counts them, per chunk of
    C tokens: 2 C^2 dk per key head (K K^T strictly lower + Q K^T lower), and per value head
    C^3 / 3 (triangular inverse) + C^2 (dk + dv) (the W and U' folds) + 4 C dk dv (state
    update) + 2 C dk dv + C^2 dv (output).  Partial chunks count as whole ones."""
    nch = sum((l + chunk - 1) // chunk for l in spec.seq_lens)
    C, dk, dv = chunk, spec.dk, spec.dv
    per_kh = 2 * C * C * dk
    per_hv = C ** 3 / 3 + C * C * (dk + dv) + 4 * C * dk * dv + 2 * C * dk * dv + C * C * dv
    return nch * spec.hk * per_kh + nch * spec.hv * per_hv


def composition_overhead_bytes(spec, chunk):
    """HBM bytes the split-type compositions move on top of the compulsory ones: every
    chunk's T and P fragments written by the prep and read back by the scan (per-channel
    gate: also the gated operands e^G K, e^{G_C - G} K, e^G Q and the chunk decay; raw
    inputs: the two row-norm rows per chunk and key head)."""
    nch = sum((l + chunk - 1) // chunk for l in spec.seq_lens)
    tile = sum(mt // 2 + 1 for mt in range(chunk // 16)) * 512 * 2
    per = 2 * tile
    if spec.gate == "channel":
        per += 3 * chunk * spec.dk * 2 + spec.dk * 4
    extra = 2 * nch * spec.hk * 2 * chunk * 4 if getattr(spec, "raw", False) else 0  # raw inputs: row norms
    return 2 * nch * spec.hv * per + extra


# the source file holding each workload's kernels and their launch code
KERNEL_SOURCE = {"decode": "gdn_decode.hip"}  # every prefill workload: gdn_kernels.hip


def source_digest(label="hybrid"):
    """Digest of a kernel source's code: comments, whitespace and the measurement build's
    stamp statements (GDN_STAMP, empty in the product library) are dropped, so an edit of
    those alone keeps the counters taken on that code valid."""
    with open(os.path.join(ROOT, "linear_attention_rnn_chunk_amd", "csrc",
                           KERNEL_SOURCE.get(label, "gdn_kernels.hip"))) as fh:
        src = fh.read()
    code = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = re.sub(r"(if \(u == 0\) )?GDN_STAMP\([^;]*\);", " ", code)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_from_profiles(label, composition, digest, kernel=None):
    """HBM bytes from the committed counter summary of workload `label`, if it was taken on
    the current kernel source (same digest) and the same composition; else None.  Without
    `kernel`: the bytes of one whole call (every launch of one step); with it, that
    kernel's bytes per launch."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.txt" % label)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"source_digest:\s*(\w+)", txt)
    c = re.search(r"composition:\s*(\w+)", txt)
    if not m or m.group(1) != digest or not c or c.group(1) != composition:
        return None
    key = r"%s\s+bytes_per_launch" % re.escape(kernel) if kernel else "bytes_per_step"
    m = re.search(r"^%s:\s*([0-9.eE+]+)" % key, txt, re.M)
    return float(m.group(1)) if m else None


def _short_kernel(name):
    m = re.search(r"(gdn_\w+)<", name) or re.search(r"(gdn_\w+)\(", name) or re.search(r"(gdn_\w+)", name)
    if m:
        return m.group(1)
    if "AUnaryFunctor" in name or "MulFunctor" in name:
        return "copy_probe"
    return None


def summarize_profiles(kt_dir, fetch_dir, write_dir, cmds, label, composition, calls, title):
    """Text summaries of rocprofv3 runs of this script (each making `calls` whole layer
    calls): kernel durations (kernel trace: per kernel, and their sum per call), and HBM
    bytes per launch and per call (FETCH_SIZE and WRITE_SIZE passes, each scaled by what
    the same counter reads for the plain copy of --copy-probe, whose true bytes are known)."""
    import csv
    import glob
    import numpy as np

    def rows(d, pat):
        out = []
        for f in glob.glob(os.path.join(d, "**", pat), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    kt = rows(kt_dir, "*kernel_stats.csv")
    lines = ["# rocprofv3 kernel trace: " + title,
             "# command: " + cmds[0],
             "composition: %s" % composition,
             "kernel  calls  avg_us  min_us  max_us  share_pct"]
    total_ns = 0.0
    for r in kt:
        k = _short_kernel(r["Name"])
        if k and k != "copy_probe":
            total_ns += float(r["TotalDurationNs"]) if "TotalDurationNs" in r else float(r["AverageNs"]) * int(r["Calls"])
            lines.append("%s  %s  %.2f  %.2f  %.2f  %s" % (k, r["Calls"], float(r["AverageNs"]) / 1e3,
                                                        float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                                                        r["Percentage"]))
    lines.append("kernel_us_per_call: %.2f  (sum of the gdn kernels' durations / %d calls)" % (total_ns / 1e3 / calls, calls))
    trace_txt = "\n".join(lines) + "\n"

    per = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        for r in rows(d, "*counter_collection.csv"):
            k = _short_kernel(r["Kernel_Name"])
            if k and r["Counter_Name"] == cname:
                per.setdefault((k, cname), []).append(float(r["Counter_Value"]))
    probe_kib = PROBE_MIB * 1024.0
    f_scale = probe_kib / np.mean(per[("copy_probe", "FETCH_SIZE")])
    w_scale = probe_kib / np.mean(per[("copy_probe", "WRITE_SIZE")])
    lines = ["# HBM traffic from rocprofv3 counters: " + title,
             "# commands: " + cmds[1], "#           " + cmds[2],
             "# copy probe: %d MiB read and written; FETCH_SIZE read %.1f KiB (scale %.4f), "
             "WRITE_SIZE %.1f KiB (scale %.4f)" % (PROBE_MIB, np.mean(per[("copy_probe", "FETCH_SIZE")]),
                                                  f_scale, np.mean(per[("copy_probe", "WRITE_SIZE")]), w_scale),
             "composition: %s" % composition,
             "source_digest: %s" % source_digest(label)]
    step = 0.0
    for k in sorted({k for k, _ in per if k != "copy_probe"}):
        fk = np.mean(per[(k, "FETCH_SIZE")]) * f_scale
        wk = np.mean(per[(k, "WRITE_SIZE")]) * w_scale
        n = len(per[(k, "FETCH_SIZE")])
        step += (np.sum(per[(k, "FETCH_SIZE")]) * f_scale + np.sum(per[(k, "WRITE_SIZE")]) * w_scale) * 1024 / calls
        lines.append("%s launches: %d (%.3g per call)" % (k, n, n / calls))
        lines.append("%s fetch_bytes: %.6g" % (k, fk * 1024))
        lines.append("%s write_bytes: %.6g" % (k, wk * 1024))
        lines.append("%s bytes_per_launch: %.6g" % (k, (fk + wk) * 1024))
    lines.append("bytes_per_step: %.6g  (every gdn launch of one call)" % step)
    return trace_txt, "\n".join(lines) + "\n"


def summarize_launches(kt_dir, cmd, title, composition):
    """The launches of one cache-cold timed step, from a per-dispatch kernel trace: each gdn
    kernel's duration and workgroups, and the span from the first launch's start to the
    last one's end."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(kt_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    # a step is a run of gdn launches between two flushes (the scratch write before each step)
    steps, cur = [], []
    for r in rows:
        if "gdn_" in r["Kernel_Name"]:
            cur.append(r)
        elif cur:
            steps.append(cur)
            cur = []
    if cur:
        steps.append(cur)
    # the timed steps: the most frequent run length (warm-up and warm-cache steps run back
    # to back and merge into longer runs; the per-kernel pass gives runs of two)
    from collections import Counter
    lens = Counter(len(st) for st in steps if len(st) >= 3) or Counter(len(st) for st in steps)
    n = lens.most_common(1)[0][0] if lens else 0
    long_steps = [st for st in steps if len(st) == n]
    step = long_steps[len(long_steps) // 2] if long_steps else []
    wg = lambda r: int(r.get("Grid_Size", r.get("Grid_Size_X", 0))) // max(1, int(r.get("Workgroup_Size", r.get("Workgroup_Size_X", 1))))
    lines = ["# launches of one cache-cold step: " + title,
             "# command: " + cmd,
             "composition: %s" % composition,
             "# timed steps of %d launches in the trace: %d (the middle one shown)" % (n, len(long_steps)),
             "kernel  workgroups  dur_us"]
    for r in step:
        m = re.search(r"(gdn_\w+)", r["Kernel_Name"])
        lines.append("%s  %d  %.1f" % (m.group(1) if m else r["Kernel_Name"][:40], wg(r),
                                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    if step:
        span = (int(step[-1]["End_Timestamp"]) - int(step[0]["Start_Timestamp"])) / 1e3
        busy = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in step) / 1e3
        lines.append("span_us: %.1f  (sum of launch durations %.1f)" % (span, busy))
    return "\n".join(lines) + "\n"


PROBE_MIB = 256

# one rocprofv3 --pmc pass (6 SQ counters, 1 GRBM counter: within one pass's limits)
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAVES",
                 "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")
N_CU = 256


def summarize_counters(pmc_dir, kt_dir, cmd, title, label, composition, calls):
    """Per-kernel MFMA and occupancy counters from one rocprofv3 --pmc pass of this script,
    with kernel durations from the kernel-trace run: executed MFMA flops (512 per bf16
    MOP) per launch and their rate, MFMA busy share (busy cycles over the per-XCD active
    cycles x CUs x 4 SIMDs), mean resident waves per CU (SQ_WAVE_CYCLES counts quad-cycles:
    x 4 over the kernel's cycles x CUs), waves and LDS bank conflicts per launch; then the
    same summed over every launch of one call."""
    import csv
    import glob
    import numpy as np

    def rows(d, pat):
        out = []
        for f in glob.glob(os.path.join(d, "**", pat), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    short = _short_kernel
    per = {}
    for r in rows(pmc_dir, "*counter_collection.csv"):
        k = short(r["Kernel_Name"])
        if k and k != "copy_probe":
            per.setdefault(k, {}).setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            per[k][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    dur = {}
    for r in rows(kt_dir, "*kernel_stats.csv"):
        k = short(r["Name"])
        if k:
            dur[k] = float(r["AverageNs"]) * 1e-9
    lines = ["# rocprofv3 MFMA and occupancy counters per launch: " + title, "# command: " + cmd,
             "# executed flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (masked triangle halves and "
             "per-slice redundancy included: not algorithmic)",
             "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x %d CUs x 4 SIMDs); "
             "GRBM_GUI_ACTIVE reads the active cycles summed over the 8 XCDs" % N_CU,
             "# waves_per_cu = SQ_WAVE_CYCLES x 4 / (GRBM_GUI_ACTIVE / 8 x %d CUs): mean resident waves "
             "per CU over the launch, idle CUs included" % N_CU,
             "composition: %s" % composition,
             "source_digest: %s" % source_digest(label)]
    tot = {}
    for k in per:
        for n, v in per[k].items():
            tot[n] = tot.get(n, 0.0) + sum(v.values())
    for k in sorted(per):
        c = {n: float(np.mean(list(v.values()))) for n, v in per[k].items()}
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        flops = mops * 512
        lines.append("%s mfma_mops_bf16: %.6g" % (k, mops))
        lines.append("%s executed_flops: %.6g" % (k, flops))
        if k in dur:
            lines.append("%s executed_tflops: %.4g (kernel %.1f us)" % (k, flops / dur[k] / 1e12, dur[k] * 1e6))
        if c.get("GRBM_GUI_ACTIVE"):
            lines.append("%s mfma_busy: %.4f" % (k, c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
                                                  / (c["GRBM_GUI_ACTIVE"] / 8 * N_CU * 4)))
        if c.get("GRBM_GUI_ACTIVE") and "SQ_WAVE_CYCLES" in c:
            lines.append("%s waves_per_cu: %.3f" % (k, c["SQ_WAVE_CYCLES"] * 4 / (c["GRBM_GUI_ACTIVE"] / 8 * N_CU)))
        lines.append("%s launches: %d (%.3g per call)" % (k, len(per[k].get("SQ_WAVES", {})),
                                                       len(per[k].get("SQ_WAVES", {})) / calls))
        for n in ("SQ_WAVES", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"):
            if n in c:
                lines.append("%s %s: %.6g" % (k, n, c[n]))
    if tot.get("GRBM_GUI_ACTIVE"):
        lines.append("per_call executed_flops: %.6g" % (tot.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / calls))
        lines.append("per_call mfma_busy: %.4f" % (tot.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
                                                   / (tot["GRBM_GUI_ACTIVE"] / 8 * N_CU * 4)))
        lines.append("per_call waves_per_cu: %.3f" % (tot.get("SQ_WAVE_CYCLES", 0.0) * 4
                                                      / (tot["GRBM_GUI_ACTIVE"] / 8 * N_CU)))
    return "\n".join(lines) + "\n"


def measured_peaks(dev):
    """HBM copy rate (1 GiB read + 1 GiB written) and a large bf16 GEMM's rate, measured
    here for context beside the spec peaks."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    out = {}
    for name, fn, work in (("hbm_copy_GBps", lambda: dst.copy_(src), 2 * n * 4 / 1e9),
                           ("bf16_gemm_8192_TFLOPs", lambda: torch.matmul(a, b), 2 * 8192 ** 3 / 1e12)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = work * 10 / (e0.elapsed_time(e1) * 1e-3)
    return out


def cpu_baseline(inp, budget_s):
    """Oracle on the first N tokens of the first sequence, every value head (N calibrated to
    ~budget_s).  Raw-input workloads run the input-side oracle in front of it, as the
    library's raw entry point does."""
    import numpy as np
    import oracle
    from oracle import prepare

    spec = inp.spec
    q64, k64, v64 = inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v")
    g64, b64, h064 = inp.as_f64("g"), inp.as_f64("beta"), inp.as_f64("h0")
    L0 = spec.seq_lens[0]

    def run(ntok):
        sl = slice(0, ntok)
        t0 = time.perf_counter()
        h = None if h064 is None else h064[:1]
        if getattr(spec, "raw", False):
            prepare.raw_fwd(q64[sl], k64[sl], v64[sl], g64[sl], b64[sl], inp.meta["q_scale"],
                            inp.meta["gate_scale"], h, seq_start=np.array([0, ntok]))
        else:
            oracle.serial_fwd(q64[sl], k64[sl], v64[sl], g64[sl], b64[sl], h, seq_start=np.array([0, ntok]))
        return time.perf_counter() - t0

    cal = min(128, L0)
    t_cal = run(cal)
    ntok = int(min(L0, max(cal, cal * budget_s / max(t_cal, 1e-6))))
    secs = run(ntok)
    cores = min(oracle.max_threads(), spec.hv)
    return dict(value=ntok / secs, unit="tokens/s", cores=cores, kind="oracle",
                sample="fp64 token-serial oracle%s, all %d value heads of the %s workload's first "
                       "sequence over its first %d tokens (%.1f s)"
                       % (" after the input-side oracle" if getattr(spec, "raw", False) else "", spec.hv,
                          spec.name, ntok, secs))


def copy_probe(mib, dev):
    """One elementwise kernel per call that reads and writes `mib` MiB of fp32, three
    times: the known-size reference for scaling HBM counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    return n * 4


def decode_bytes(B, hk, hv, dk, dv):
    """Algorithmic bytes of one step: per (sequence, value head) the fp32 state read and
    written, v in and o out (bf16), gate and beta; per (sequence, key head) q and k."""
    return B * hv * (2 * dk * dv * 4 + 2 * dv * 2 + 2 * 4) + B * hk * 2 * dk * 2


def bench_decode(args):
    """One-token steps of B sequences at the hybrid layer's shapes, states resident in
    HBM, alternating between two state buffers (each step reads one, writes the other)."""
    import numpy as np
    import torch

    from linear_attention_rnn_chunk_amd import gdn, inputs

    B = args.decode
    base = inputs.CONFIGS["hybrid"]
    spec = inputs.Spec("decode", (1,) * B, base.hk, base.hv, base.dk, base.dv, gate_law="half",
                       h0=True, packed=True, seed=2003)
    log("generating decode inputs (%d sequences)" % B)
    inp = inputs.make(spec)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def t(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v, g, beta, h0 = (t(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta", "h0"))
    prob = gdn.make_problem(B, B, 1, spec.hk, spec.hv, spec.dk, spec.dv, gdn.GATE_HEAD, 0, gdn.BF16,
                            gdn.BF16)
    o = torch.empty((B, spec.hv, spec.dv), dtype=torch.bfloat16, device=dev)
    states = [h0, torch.empty_like(h0)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        rc = gdn.decode_step_raw(prob, q, k, v, g, beta, states[i & 1], o, states[(i + 1) & 1], status,
                                 stream.cuda_stream)
        if ev is not None:
            ev[1].record(stream)
        if rc:
            raise gdn.GdnError(rc, "gdn_decode_step")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if int(status.item()):
        raise gdn.GdnStatusError(int(status.item()))
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev) if args.flush_mib else None
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        step(i, evs[i])
    torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    if args.only_timed:
        if args.copy_probe:
            copy_probe(args.copy_probe, dev)
        return
    wev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(3, args.steps // 2))]
    for i, e in enumerate(wev):
        step(i, e)
    torch.cuda.synchronize()
    warm = float(np.median([e[0].elapsed_time(e[1]) for e in wev]))
    if int(status.item()):
        raise gdn.GdnStatusError(int(status.item()))
    ms_step = float(np.median(ms))
    nbytes = decode_bytes(B, spec.hk, spec.hv, spec.dk, spec.dv)
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    log("decode B=%d: ms/step %.4f median cold (min %.4f), warm %.4f, %.0f GB/s"
        % (B, ms_step, ms.min(), warm, gbs))
    rec = {
        "metric": "GDN one-token step: sequences/s (HV=48, d=128)",
        "value": B / (ms_step * 1e-3),
        "unit": "sequences/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "one-token step of %d sequences, 16 key / 48 value heads, dk=dv=128, "
                               "bf16 q/k/v/o, fp32 state, per-head gate" % B, "sequences": B},
        "roofline": {"bound": "hbm", "kernel": "gdn_decode", "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": traffic_from_profiles("decode", "decode", source_digest("decode"), kernel="gdn_decode"),
                     "kernel_ms": ms_step, "algorithmic_bytes": nbytes},
        "timing": {"headline": "median cold-cache step (%d MiB scratch written before each step)"
                               % args.flush_mib if args.flush_mib else "median warm step",
                   "min_ms": float(ms.min()), "warm_median_ms": warm},
        "source_digest": source_digest("decode"),
    }
    if args.copy_probe:
        rec["copy_probe_bytes"] = copy_probe(args.copy_probe, dev)
    if not args.no_cpu:
        import oracle
        log("timing the oracle on a bounded sample")
        n = min(B, 64)
        sl = slice(0, n)
        a64 = [inp.as_f64(x)[sl] for x in ("q", "k", "v", "g", "beta")] + [inp.h0[sl].astype(np.float64)]
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.serial_fwd(*a64, seq_start=np.arange(n + 1))
            reps += 1
            secs = time.perf_counter() - t0
            if secs >= args.cpu_seconds:
                break
        rec["cpu_baseline"] = dict(value=reps * n / secs, unit="sequences/s",
                                   cores=min(oracle.max_threads(), n * spec.hv), kind="oracle",
                                   sample="fp64 token-serial oracle, one token of the first %d sequences "
                                          "(all 48 value heads), repeated %d times (%.1f s)"
                                          % (n, reps, secs))
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def bench_stamps(args):
    """Per-phase step timestamps of one scan workgroup, from the measurement build
    (libgdn_mi355x_stamps.so): the split composition's prep, then its scan with workgroup
    --stamp-block recording kStampSteps chunk steps from the middle of its sequence.  Writes
    the medians over steps and calls to profiles/scan_stamps_<config>.txt."""
    import ctypes
    import numpy as np
    import torch

    from linear_attention_rnn_chunk_amd import gdn, inputs
    gdn.use_library(args.stamps_library or gdn.STAMPS_LIBRARY_PATH)
    lib = gdn.load()
    lib.gdn_debug_stamps.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
    lib.gdn_debug_stamps.restype = ctypes.c_int32
    spec = inputs.CONFIGS[args.config]
    chunk = args.chunk or spec.chunk
    inp = inputs.make(spec)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def t(x):
        if x is None:
            return None
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    packed = spec.packed or len(set(spec.seq_lens)) > 1
    B, Tn = (1, spec.tokens) if packed else (spec.n_seq, spec.seq_lens[0])
    cu = torch.from_numpy(inp.cu_seqlens).to(dev) if packed else None
    shp = lambda a: a.reshape((B, Tn) + tuple(a.shape[1:]))
    q, k, v, g, beta = (shp(t(getattr(inp, n))) for n in ("q", "k", "v", "g", "beta"))
    h0 = t(inp.h0)
    p_prep = layer_problem(args, spec, gdn.COMPOSE_SPLIT, gdn.STAGE_PREP)
    p_scan = layer_problem(args, spec, gdn.COMPOSE_SPLIT, gdn.STAGE_SCAN)
    o = torch.empty((B, Tn, spec.hv, spec.dv), dtype=torch.bfloat16 if args.arm == "bf16" else torch.float32,
                    device=dev)
    hT = torch.empty((spec.n_seq, spec.hv, spec.dk, spec.dv), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, gdn.workspace_bytes(p_prep)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    per = lib.gdn_debug_stamps(None, 0, 0)
    NS, NK = 16, per // 16
    nch = min((l + chunk - 1) // chunk for l in spec.seq_lens)
    c0 = max(0, nch // 2 - NS // 2)
    buf = torch.zeros(4 * NS * NK, dtype=torch.int64, device=dev)
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev) if args.flush_mib else None
    runs, scan_ms = [], []
    for rep in range(args.steps):
        for prob, stamp in ((p_prep, False), (p_scan, True)):
            lib.gdn_debug_stamps(ctypes.c_void_p(buf.data_ptr()) if stamp else None, args.stamp_block, c0)
            if stamp:
                buf.zero_()
                if flush is not None:
                    flush.fill_(rep & 0xFF)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            rc = gdn.chunk_fwd_raw(prob, q, k, v, g, beta, h0, cu, o, hT, status, ws, stream.cuda_stream)
            if rc:
                raise gdn.GdnError(rc, "gdn_chunk_fwd")
            if stamp:
                e1.record(stream)
        torch.cuda.synchronize()
        scan_ms.append(e0.elapsed_time(e1))
        if rep >= 1:  # the first call sets the kernels' launch attributes
            runs.append(buf.cpu().numpy().reshape(4, NS, NK).astype(np.int64))
    lib.gdn_debug_stamps(None, 0, 0)
    if int(status.item()):
        raise gdn.GdnStatusError(int(status.item()))
    a = np.stack(runs)  # [reps, role, step, phase]
    med = lambda x: float(np.median(x))
    chain, out, cpy, chain1 = a[:, 0], a[:, 1], a[:, 2], a[:, 3]
    period = med(chain[:, 1:, 0] - chain[:, :-1, 0])
    step_us = float(np.median(scan_ms)) * 1e3 / nch
    rows = [("chain wave 0", [("Y = K H_in, X", chain[:, :-1, 1] - chain[:, :-1, 0]),
                              ("R = T X, R S", chain[:, :-1, 2] - chain[:, :-1, 1]),
                              ("state update, H_in of next", chain[:, :-1, 3] - chain[:, :-1, 2]),
                              ("T loads issued, wait", chain[:, :-1, 4] - chain[:, :-1, 3]),
                              ("barrier", chain[:, 1:, 0] - chain[:, :-1, 4])]),
            ("chain wave 1", [("Y = K H_in, X", chain1[:, :-1, 1] - chain1[:, :-1, 0]),
                              ("R = T X, R S", chain1[:, :-1, 2] - chain1[:, :-1, 1]),
                              ("state update, H_in of next", chain1[:, :-1, 3] - chain1[:, :-1, 2]),
                              ("T loads issued, wait", chain1[:, :-1, 4] - chain1[:, :-1, 3]),
                              ("barrier", chain1[:, 1:, 0] - chain1[:, :-1, 4])]),
            ("output wave", [("loads, P R of previous chunk, stores", out[:, :-1, 1] - out[:, :-1, 0]),
                             ("Q H_in of this chunk", out[:, :-1, 2] - out[:, :-1, 1]),
                             ("wait for loads / stores", out[:, :-1, 3] - out[:, :-1, 2]),
                             ("barrier", out[:, 1:, 0] - out[:, :-1, 3])]),
            ("loader wave", [("copies issued", cpy[:, :-1, 1] - cpy[:, :-1, 0]),
                             ("wait for the next chunk", cpy[:, :-1, 2] - cpy[:, :-1, 1]),
                             ("gate sweep, V check", cpy[:, :-1, 3] - cpy[:, :-1, 2]),
                             ("barrier", cpy[:, 1:, 0] - cpy[:, :-1, 3])])]
    cmd = ("python -m linear_attention_rnn_chunk_amd.build --stamps && python3 <repo>/bench.py --stamps --config %s "
           "--steps %d%s" % (args.config, args.steps, " --chunk %d" % args.chunk if args.chunk else ""))
    lines = ["# scan step phases (shader-clock ticks, s_memtime) of workgroup %d, chunk steps %d..%d: %s"
             % (args.stamp_block, c0, c0 + NS - 1, workload_title(args.config)),
             "# command: " + cmd,
             "# medians over %d steps x %d calls (cache-cold scan launches of the split composition);"
             " then the 10th / 90th percentiles, and the medians of even and odd chunk steps"
             " (the chain's T register sets alternate by chunk parity)" % (NS - 1, len(runs)),
             "source_digest: %s" % source_digest("hybrid"),
             "step_ticks: %.0f" % period,
             "step_us: %.3f  (scan kernel %.4f ms / %d chunk steps)" % (step_us, float(np.median(scan_ms)), nch),
             "ticks_per_us: %.0f" % (period / step_us)]
    # chunk index of each step column of a phase array (steps c0 .. c0 + NS - 2)
    even = ((c0 + np.arange(NS - 1)) % 2) == 0
    pct = lambda x, q: float(np.percentile(x, q))
    lines.append("%-42s %7s %7s %7s %7s %7s" % ("", "median", "p10", "p90", "even", "odd"))
    per = chain[:, 1:, 0] - chain[:, :-1, 0]
    lines.append("%-42s %7.0f %7.0f %7.0f %7.0f %7.0f" % ("step period (chain wave 0)", med(per), pct(per, 10),
                                                           pct(per, 90), med(per[:, even]), med(per[:, ~even])))
    for role, phases in rows:
        lines.append("%s:" % role)
        for name, d in phases:
            lines.append("  %-40s %7.0f %7.0f %7.0f %7.0f %7.0f" % (name, med(d), pct(d, 10), pct(d, 90),
                                                                   med(d[:, even]), med(d[:, ~even])))
    # histogram of the step period, 200-tick bins
    lo = int(per.min()) // 200 * 200
    hist = np.bincount(((per - lo) // 200).astype(np.int64).ravel())
    lines.append("step period histogram (200-tick bins from %d): %s" % (lo, " ".join(str(int(h)) for h in hist)))
    txt = "\n".join(lines) + "\n"
    out = args.stamps_out or os.path.join(ROOT, "profiles", "scan_stamps_%s.txt" % args.config)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        f.write(txt)
    print(txt)


def workload_title(name):
    spec = __import__("linear_attention_rnn_chunk_amd.inputs", fromlist=["CONFIGS"]).CONFIGS[name]
    seqs = ("B=%d, T=%d" % (spec.n_seq, spec.seq_lens[0]) if len(set(spec.seq_lens)) == 1 and not spec.packed
            else "%d packed sequences (%s tokens)" % (spec.n_seq, "+".join(map(str, spec.seq_lens))))
    return "%s GDN layer (%s, %d/%d heads, d=%d, %s gate, chunk %d)" % (
        name, seqs, spec.hk, spec.hv, spec.dk, "per-head" if spec.gate == "head" else "per-key-channel",
        spec.chunk)


def layer_problem(args, spec, compose, stages=0):
    """The gdn_problem bench.py times for workload `spec` (fixed-length batch, or packed)."""
    from linear_attention_rnn_chunk_amd import gdn
    packed = spec.packed or len(set(spec.seq_lens)) > 1
    chunk = args.chunk or spec.chunk
    gate = gdn.GATE_KEY_CHANNEL if spec.gate == "channel" else gdn.GATE_HEAD
    qdt = gdn.BF16 if spec.qkv_dtype == "bf16" else gdn.F32
    odt = gdn.BF16 if args.arm == "bf16" else gdn.F32
    arm = gdn.ARM_MFMA_BF16 if args.arm == "bf16" else gdn.ARM_FOLD_F32
    return gdn.make_problem(spec.n_seq, spec.tokens, 0 if packed else spec.seq_lens[0], spec.hk, spec.hv,
                            spec.dk, spec.dv, gate, chunk, qdt, odt, arm, compose, stages,
                            solve_block=getattr(args, "solve_block", 0))


COMPOSE_NAMES = ("auto", "split", "fused", "pipelined", "seqsplit")


def resolved_composition(args):
    """The composition gdn_chunk_fwd runs for this workload on the current device."""
    from linear_attention_rnn_chunk_amd import gdn, inputs
    spec = inputs.CONFIGS[args.config]
    return COMPOSE_NAMES[gdn.plan_compose(layer_problem(args, spec, COMPOSE_NAMES.index(args.compose)))]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="hybrid")
    ap.add_argument("--arm", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--solve-block", type=int, default=0, choices=[0, 8, 16, 32],
                    help="rows of the triangular solve's diagonal blocks (0: the library's)")
    ap.add_argument("--compose", default="auto", choices=list(COMPOSE_NAMES),
                    help="auto: the library's choice (gdn_plan_compose says which); split: prep "
                         "kernel then scan; fused: tile waves inside the scan workgroup, one "
                         "kernel; pipelined: scan segments with the next segment's prep beside "
                         "each; seqsplit: parts of each sequence scanned side by side")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="before each timed step, write this much scratch memory (larger than "
                         "the 256 MiB MALL and the L2s) so every step starts cache-cold; 0 = warm")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("KT_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries (kernel trace, HBM traffic) from rocprofv3 output "
                         "of this script's --only-timed form and exit")
    ap.add_argument("--summarize-launches", metavar="KT_DIR",
                    help="write profiles/ the launch sequence of one timed step from a rocprofv3 "
                         "kernel trace of this script and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DIR", "KT_DIR"),
                    help="write the MFMA / occupancy counter summary to profiles/ and exit")
    ap.add_argument("--peaks", action="store_true",
                    help="also measure an HBM copy and a large bf16 GEMM (context for the rooflines)")
    ap.add_argument("--decode", type=int, default=0, metavar="B",
                    help="time the one-token recurrent step instead: B sequences of the hybrid "
                         "layer's heads, each continuing from its own state; prints its own line")
    ap.add_argument("--only-timed", action="store_true",
                    help="run only the warm-up and the timed calls (no per-stage pass, no warm-cache "
                         "pass): the form the profiling runs take, so every launch they see belongs "
                         "to one of warmup + steps whole-layer calls")
    ap.add_argument("--stamps", action="store_true",
                    help="per-phase step timestamps of one scan workgroup from the measurement build "
                         "(python -m linear_attention_rnn_chunk_amd.build --stamps); writes "
                         "profiles/scan_stamps_<config>.txt")
    ap.add_argument("--stamp-block", type=int, default=0)
    ap.add_argument("--stamps-library", default=None, help="another measurement build to load")
    ap.add_argument("--stamps-out", default=None, help="write the summary here instead")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run a plain device copy of MIB MiB three times "
                         "(reads and writes MIB MiB each): the reference for scaling HBM counters")
    args = ap.parse_args()

    if args.summarize_counters or args.summarize_launches or args.summarize_profiles:
        # run on the box that took the profiles: the library's choice of composition there
        label = "decode" if args.decode else args.config
        composition = "decode" if args.decode else resolved_composition(args)
        calls = args.warmup + args.steps
        run = ("python3 <repo>/bench.py --config %s --steps %d --warmup %d --no-cpu --only-timed%s%s"
               % (args.config, args.steps, args.warmup,
                  " --compose %s" % args.compose if args.compose != "auto" else "",
                  " --decode %d" % args.decode if args.decode else ""))
        title = (("one-token step, %d sequences of the hybrid layer (16/48 heads, d=128)" % args.decode)
                 if args.decode else workload_title(args.config))
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        out = []
        if args.summarize_counters:
            cmd = "cd /tmp && rocprofv3 --pmc " + " ".join(MFMA_COUNTERS) + " -d <out>/prof_mfma -o m -f csv -- " + run
            txt = summarize_counters(args.summarize_counters[0], args.summarize_counters[1], cmd, title,
                                     label, composition, calls)
            out.append(("mfma_counters_%s.txt" % label, txt))
        if args.summarize_launches:
            # (the per-dispatch trace of the kernel-trace run)
            txt = summarize_launches(args.summarize_launches,
                                     "cd /tmp && rocprofv3 --kernel-trace --stats -d <out>/prof_kt -o kt -f csv -- " + run,
                                     title, composition)
            out.append(("launches_%s.txt" % label, txt))
        if args.summarize_profiles:
            cmds = ["cd /tmp && rocprofv3 --kernel-trace --stats -d <out>/prof_kt -o kt -f csv -- " + run,
                    "cd /tmp && rocprofv3 --pmc FETCH_SIZE -d <out>/prof_fetch -o f -f csv -- " + run
                    + " --copy-probe %d" % PROBE_MIB,
                    "cd /tmp && rocprofv3 --pmc WRITE_SIZE -d <out>/prof_write -o w -f csv -- " + run
                    + " --copy-probe %d" % PROBE_MIB]
            trace_txt, traffic_txt = summarize_profiles(*args.summarize_profiles, cmds, label, composition,
                                                        calls, title)
            out += [("kernel_trace_%s.txt" % label, trace_txt), ("hbm_traffic_%s.txt" % label, traffic_txt)]
        for name, txt in out:
            with open(os.path.join(ROOT, "profiles", name), "w") as f:
                f.write(txt)
            print(txt)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library runs on one GPU; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_rnn_chunk_amd import gdn, inputs

    if not os.path.exists(gdn.LIBRARY_PATH):
        import __graft_entry__
        __graft_entry__.build()

    if args.decode:
        return bench_decode(args)
    if args.stamps:
        return bench_stamps(args)

    spec = inputs.CONFIGS[args.config]
    chunk = args.chunk or spec.chunk
    log("generating %s inputs (%d tokens)" % (spec.name, spec.tokens))
    inp = inputs.make(spec)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def t(x):
        if x is None:
            return None
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    packed = spec.packed or len(set(spec.seq_lens)) > 1
    if packed:
        B, Tn = 1, spec.tokens
        cu = torch.from_numpy(inp.cu_seqlens).to(dev)
    else:
        B, Tn = spec.n_seq, spec.seq_lens[0]
        cu = None
    shp = lambda a: a.reshape((B, Tn) + tuple(a.shape[1:]))
    q, k, v, g, beta = (shp(t(getattr(inp, n))) for n in ("q", "k", "v", "g", "beta"))
    h0 = t(inp.h0)
    gate = gdn.GATE_KEY_CHANNEL if spec.gate == "channel" else gdn.GATE_HEAD
    odt_t = torch.bfloat16 if args.arm == "bf16" else torch.float32
    p_all = layer_problem(args, spec, COMPOSE_NAMES.index(args.compose))
    composition = COMPOSE_NAMES[gdn.plan_compose(p_all)]
    fused = composition == "fused"
    # the split composition's two stages, called one by one: the per-stage view
    p_prep = layer_problem(args, spec, gdn.COMPOSE_SPLIT, gdn.STAGE_PREP)
    p_scan = layer_problem(args, spec, gdn.COMPOSE_SPLIT, gdn.STAGE_SCAN)
    o = torch.empty((B, Tn, spec.hv, spec.dv), dtype=odt_t, device=dev)
    hT = torch.empty((spec.n_seq, spec.hv, spec.dk, spec.dv), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    # raw-input workloads go through gdn_chunk_fwd_raw_inputs (same tensors, the raw values)
    wsb = gdn.raw_workspace_bytes if spec.raw else gdn.workspace_bytes
    ws = torch.empty(max(1, wsb(p_all), wsb(p_prep)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call(prob):
        if spec.raw:
            rc = gdn.chunk_fwd_raw_inputs_raw(prob, inp.meta["q_scale"], inp.meta["gate_scale"], q, k, v, g, beta, h0,
                                              cu, o, hT, status, ws, stream.cuda_stream)
        else:
            rc = gdn.chunk_fwd_raw(prob, q, k, v, g, beta, h0, cu, o, hT, status, ws, stream.cuda_stream)
        if rc:
            raise gdn.GdnError(rc, "gdn_chunk_fwd")

    def step(ev=None):  # one whole gdn_chunk_fwd, events on the library's stream around it
        if ev is not None:
            ev[0].record(stream)
        call(p_all)
        if ev is not None:
            ev[1].record(stream)

    def stages(ev=None):  # the split composition's prep then scan, an event between them
        if ev is not None:
            ev[0].record(stream)
        call(p_prep)
        if ev is not None:
            ev[1].record(stream)
        call(p_scan)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(status.item()):
        raise gdn.GdnStatusError(int(status.item()))

    # Timed region: exactly `steps` layer calls between two device synchronisations.  Each
    # call is preceded (outside its events) by a scratch write that evicts the caches, so
    # the step time is cache-cold; the headline is the median step.
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev) if args.flush_mib else None
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    ms_step = float(np.median(step_ms))
    prep_ms = scan_ms = warm_ms = None
    if not args.only_timed:
        if not fused:
            # the split composition's stages, timed the same way in a second pass of as many
            # cache-cold steps (one untimed call first: launch attributes of its kernels)
            stages()
            kev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
            for i in range(args.steps):
                if flush is not None:
                    flush.fill_(i & 0xFF)
                stages(kev[i])
            torch.cuda.synchronize()
            prep_ms = float(np.median([e[0].elapsed_time(e[1]) for e in kev]))
            scan_ms = float(np.median([e[1].elapsed_time(e[2]) for e in kev]))
        # warm-cache median for context (same work, no eviction in between)
        wev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(3, args.steps // 2))]
        for e in wev:
            step(e)
        torch.cuda.synchronize()
        warm_ms = float(np.median([e[0].elapsed_time(e[1]) for e in wev]))
    if int(status.item()):
        raise gdn.GdnStatusError(int(status.item()))
    log("%s: ms/step %.4f median cold (min %.4f), wall %.3f s for %d steps; split stages: prep %s, scan %s; warm %s"
        % (composition, ms_step, step_ms.min(), wall, args.steps, prep_ms, scan_ms, warm_ms))
    if args.only_timed:
        if args.copy_probe:
            copy_probe(args.copy_probe, dev)
        return

    alg = algorithmic(spec, chunk)
    peak_mfma = MFMA_BF16_PEAK_TFLOPS if args.arm == "bf16" else MFMA_F32_PEAK_TFLOPS
    flops = scope_flops(spec, chunk)
    layer_bytes = alg["layer_bytes"]
    # The roofline's kernel is the timed call itself: every launch of one gdn_chunk_fwd (a
    # pipelined call is one prep launch and one scan launch per segment, each carrying the
    # next segment's prep), bracketed by HIP events on the library's stream.  Its
    # algorithmic bytes are the layer's compulsory bytes; what the composition moves on top
    # (the tiles' round trip through HBM) is reported beside them, not counted as work.
    achieved_gbs = layer_bytes / (ms_step * 1e-3) / 1e9
    digest = source_digest("hybrid")
    traffic = traffic_from_profiles(args.config, composition, digest)
    tokens_s = spec.tokens / (ms_step * 1e-3)
    kernels = {"split": "gdn_prep_head + gdn_scan", "pipelined": "gdn_prep_head + gdn_scan per segment",
               "fused": "gdn_scan (fused)", "seqsplit": "gdn_prep_head + 2 x gdn_scan + gdn_seq_chain"}
    if gate == gdn.GATE_KEY_CHANNEL:
        kernels["split"] = "gdn_prep_chan + gdn_scan"
    if packed:
        kernels["split"] = "gdn_chunk_table + " + kernels["split"]

    rec = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.arm == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": "%s GDN layer prefill: %s, %d key / %d value heads, "
                               "dk=dv=%d, %s gate, chunk %d%s"
                               % (spec.name, ("B=%d, T=%d" % (spec.n_seq, spec.tokens // spec.n_seq)) if not packed
                                  else "%d packed sequences (%s tokens)" % (spec.n_seq, "+".join(map(str, spec.seq_lens))),
                                  spec.hk, spec.hv, spec.dk,
                                  "per-head" if gate == gdn.GATE_HEAD else "per-key-channel",
                                  chunk, ", h0" if spec.h0 else ""),
                   "tokens": spec.tokens, "arm": args.arm, "composition": composition,
                   "solve_block": args.solve_block or 16},
        "roofline": {"bound": "hbm", "kernel": "gdn_chunk_fwd [%s: %s]" % (composition, kernels[composition]),
                     "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic, "kernel_ms": ms_step,
                     "algorithmic_bytes": layer_bytes,
                     "composition_overhead_bytes": 0 if fused else composition_overhead_bytes(spec, chunk),
                     "composition": composition},
        "mfma": {"definition": "algorithmic flops of the scope table (K K^T, Q K^T per key head; solve, "
                               "W/U' folds, state update and output per value head) / time / dense peak",
                 "peak_tflops": peak_mfma, "flops": flops,
                 "layer_frac": flops / (ms_step * 1e-3) / (peak_mfma * 1e12)},
        "timing": {"headline": "median cold-cache step (%d MiB scratch written before each step)"
                               % args.flush_mib if args.flush_mib else "median warm step",
                   "min_ms": float(step_ms.min()), "warm_median_ms": warm_ms},
        "source_digest": digest,
    }
    if prep_ms is not None:
        # the split composition's two stages, each timed with its own events in a second
        # pass of as many cache-cold steps (context: the per-stage view of the same work)
        prep_flops = alg["prep_flops"]
        rec["split_stages"] = {
            "prep_ms": prep_ms, "scan_ms": scan_ms,
            "prep_mfma_frac": prep_flops / (prep_ms * 1e-3) / (peak_mfma * 1e12),
            "scan_mfma_frac": (flops - prep_flops) / (scan_ms * 1e-3) / (peak_mfma * 1e12),
            "prep_flops": prep_flops, "scan_flops": flops - prep_flops,
        }
    if args.copy_probe:
        rec["copy_probe_bytes"] = copy_probe(args.copy_probe, dev)
    if args.peaks:
        rec["measured_peaks"] = measured_peaks(dev)
        # the same achieved rate against the copy rate measured on this machine
        rec["roofline"]["frac_of_measured_copy"] = achieved_gbs / rec["measured_peaks"]["hbm_copy_GBps"]
        rec["mfma"]["layer_frac_of_measured_gemm"] = (flops / (ms_step * 1e-3) / 1e12
                                                       / rec["measured_peaks"]["bf16_gemm_8192_TFLOPs"])
    if not args.no_cpu:
        log("timing the oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    if args.config == "hybrid":
        rec["context_gfx1100"] = GFX1100_CONTEXT
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
