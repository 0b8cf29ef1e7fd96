"""The benchmark's algorithmic byte and flop counts (the numerators of its roofline
fractions), checked on the CPU against counts made independently of its formulas; and
its summary of a per-launch kernel trace."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_rnn_chunk_amd import inputs  # noqa: E402


def test_hybrid_layer_compulsory_bytes():
    # q, k [T][16][128] bf16; v, o [T][48][128] bf16; g, beta [T][48] fp32; h0, hT
    # [1][48][128][128] fp32, at T = 32768: 1,092,616,192 bytes
    alg = bench.algorithmic(inputs.CONFIGS["hybrid"], 64)
    assert alg["layer_bytes"] == 1_092_616_192
    assert alg["chunks"] == 512


def test_scan_and_prep_bytes_add_the_tiles():
    spec = inputs.CONFIGS["hybrid"]
    alg = bench.algorithmic(spec, 64)
    # per chunk and value head, T and P each as 6 stored 16 x 32 bf16 fragments
    tiles = 2 * 512 * 48 * 6 * 512 * 2
    assert alg["scan_bytes"] == alg["layer_bytes"] + tiles
    qk = 2 * 32768 * 16 * 128 * 2
    gb = 2 * 32768 * 48 * 4
    assert alg["prep_bytes"] == qk + gb + tiles


def test_flop_counts_per_chunk():
    alg = bench.algorithmic(inputs.CONFIGS["hybrid"], 64)
    C, dk, dv, hk, hv, nch = 64, 128, 128, 16, 48, 512
    # two lower-triangular C x C products over dk per key head (counted whole), the
    # C^3 / 3 solve per value head
    assert alg["prep_flops"] == nch * hk * 2 * C * C * dk + nch * hv * C ** 3 / 3
    # K.H, Q.H and the state update (2 C dk dv each), P.R and T.X (C^2 dv each)
    assert alg["scan_flops"] == nch * hv * (6 * C * dk * dv + 2 * C * C * dv)


def test_scope_table_flops_and_bytes_of_every_workload():
    # the hot-path scope table's per-workload figures, counted per term:
    #   per (chunk, key head) 2 C^2 dk; per (chunk, value head) C^3/3 + C^2 (dk + dv)
    #   + 4 C dk dv + 2 C dk dv + C^2 dv
    f = bench.scope_flops(inputs.CONFIGS["hybrid"], 64)
    terms = [8192 * 2 * 64 * 64 * 128, 24576 * 64 ** 3 / 3, 24576 * 64 * 64 * 256,
             24576 * 4 * 64 * 128 * 128, 24576 * (2 * 64 * 128 * 128 + 64 * 64 * 128)]
    assert abs(f - sum(terms)) < 1 and abs(f / 1e9 - 204.01) < 0.01
    assert abs(bench.scope_flops(inputs.CONFIGS["kda"], 32) / 1e9 - 124.91) < 0.01
    assert abs(bench.scope_flops(inputs.CONFIGS["packed"], 64) / 1e9 - 816.04) < 0.01
    assert abs(bench.scope_flops(inputs.CONFIGS["single"], 64) / 1e9 - 9.216) < 0.001
    # compulsory bytes: the per-channel gate [T][hv][dk] fp32 is 512 MiB of the kda layer
    assert bench.algorithmic(inputs.CONFIGS["kda"], 32)["layer_bytes"] == 1_619_001_344
    assert bench.algorithmic(inputs.CONFIGS["packed"], 64)["layer_bytes"] == 4_370_464_768
    assert bench.algorithmic(inputs.CONFIGS["single"], 64)["layer_bytes"] == 68_681_728
    # the tile round trip of the split-type compositions (T and P written and read back)
    assert bench.composition_overhead_bytes(inputs.CONFIGS["hybrid"], 64) == 2 * 512 * 48 * 2 * 6 * 1024


def test_decode_bytes():
    # 256 sequences x 48 value heads: fp32 state in and out, v and o bf16, g and beta;
    # q and k per key head
    n = bench.decode_bytes(256, 16, 48, 128, 128)
    assert n == 256 * 48 * (2 * 128 * 128 * 4 + 2 * 128 * 2 + 8) + 256 * 16 * 2 * 128 * 2
    assert n == 1_619_099_648


def test_launch_summary_picks_a_timed_step(tmp_path):
    """summarize_launches reads a per-dispatch kernel trace, cuts it into steps at the
    non-library kernels (the cache flush before each timed step) and shows one of the
    most common step shape: warm-up steps (back to back, merged) and the two-launch
    per-kernel pass are not taken for it."""
    import csv
    import bench
    d = tmp_path / "kt"
    d.mkdir()
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"]
    rows, t = [], 0

    def k(name, dur, wg):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur,
                     "Workgroup_Size_X": 256, "Grid_Size_X": 256 * wg})
        t += dur + 10

    step = [("gdn_prep_head<x>", 20000, 512)] + [("gdn_scan<x>", 48000, 256)] * 3 + [("gdn_scan<x>", 43000, 192)]
    for _ in range(3):  # warm-up: back to back
        for s in step:
            k(*s)
    for _ in range(5):  # timed: a flush before each
        k("at::native::fill", 140000, 4096)
        for s in step:
            k(*s)
    for _ in range(4):  # per-kernel pass: two launches a step
        k("at::native::fill", 140000, 4096)
        k("gdn_prep_head<x>", 150000, 8192)
        k("gdn_scan<x>", 770000, 192)
    with open(d / "x_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)
    txt = bench.summarize_launches(str(d), "cmd", "hybrid", "pipelined")
    assert "timed steps of 5 launches in the trace: 5" in txt
    lines = [l for l in txt.splitlines() if l.startswith("gdn_")]
    assert lines == ["gdn_prep_head  512  20.0", "gdn_scan  256  48.0", "gdn_scan  256  48.0",
                     "gdn_scan  256  48.0", "gdn_scan  192  43.0"]
    assert "span_us: 207.0" in txt
