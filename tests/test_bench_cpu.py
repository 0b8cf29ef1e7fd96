"""The benchmark's algorithmic byte and flop counts (the numerators of its roofline
fractions), checked on the CPU against counts made independently of its formulas."""
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


def test_decode_bytes():
    # 256 sequences x 48 value heads: fp32 state in and out, v and o bf16, g and beta;
    # q and k per key head
    n = bench.decode_bytes(256, 16, 48, 128, 128)
    assert n == 256 * 48 * (2 * 128 * 128 * 4 + 2 * 128 * 2 + 8) + 256 * 16 * 2 * 128 * 2
    assert n == 1_619_099_648
