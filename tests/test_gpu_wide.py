"""The 64-column scan workgroup (two column tiles per chain wave), which the library runs
where 32-column workgroups would need more than one round of the device's compute units:
against the fp64 oracle, and bit for bit against the 32-column scan on the same problem
(every state column goes through the same products in the same order in both)."""
import os

import pytest
import torch

from linear_attention_rnn_chunk_amd import inputs
from tests.gpu_util import BOUND, oracle_ref, rel, run_gpu, to_np64

pytestmark = pytest.mark.gpu

CASES = {
    # sequences x value heads x dv/32 well above the 256 compute units: 64 columns chosen
    "grouped": inputs.Spec("wide-grouped", (150,) * 8, 16, 48, 128, 128, gate_law="full", h0=True, chunk=64,
                           seed=61),
    "packed": inputs.Spec("wide-packed", (100, 0, 1, 64, 257, 31, 190, 7), 16, 48, 128, 128, gate_law="full",
                          h0=True, chunk=64, packed=True, seed=62),
    "chunk32": inputs.Spec("wide-c32", (97,) * 8, 16, 48, 128, 128, gate_law="clip5", h0=True, chunk=32, seed=63),
    "dv64": inputs.Spec("wide-dv64", (130,) * 16, 16, 16, 128, 64, gate_law="half", h0=True, chunk=64, seed=64),
    "dk64": inputs.Spec("wide-dk64", (130,) * 16, 8, 32, 64, 128, gate_law="half", h0=True, chunk=64, seed=65),
    "channel": inputs.Spec("wide-kda", (100,) * 8, 32, 32, 128, 128, gate="channel", gate_law="uniform5",
                           chunk=32, seed=66),
}


def _run(inp, cols, compose="auto"):
    os.environ["GDN_SCAN_COLUMNS"] = cols
    try:
        return run_gpu(inp, arm="bf16", compose=compose)
    finally:
        del os.environ["GDN_SCAN_COLUMNS"]


@pytest.mark.parametrize("name", list(CASES))
def test_wide_scan_matches_oracle_and_narrow_bitwise(name):
    inp = inputs.make(CASES[name])
    o64, h64, _ = _run(inp, "64")
    o32, h32, _ = _run(inp, "32")
    o_ref, h_ref = oracle_ref(inp)
    eo, eh = rel(to_np64(o64), o_ref), rel(to_np64(h64), h_ref)
    same = torch.equal(o64, o32) and torch.equal(h64, h32)
    print("%s: 64 columns rel-L2 o %.3e hT %.3e; equal to 32 columns: %s" % (name, eo, eh, same), flush=True)
    assert eo <= BOUND["bf16"] and eh <= BOUND["bf16"]
    assert same


def test_wide_scan_pipelined_equals_split():
    # long fixed-length sequences, the pipelined composition on request: its segments carry
    # the state between 64-column scan launches
    inp = inputs.make(inputs.Spec("wide-pipe", (5000,) * 4, 16, 48, 128, 128, gate_law="half", h0=True, chunk=64,
                                  seed=67))
    op, hp, _ = _run(inp, "64", compose="pipelined")
    os_, hs, _ = _run(inp, "64", compose="split")
    assert torch.equal(op, os_) and torch.equal(hp, hs)
    o_ref, h_ref = oracle_ref(inp)
    assert rel(to_np64(op), o_ref) <= BOUND["bf16"] and rel(to_np64(hp), h_ref) <= BOUND["bf16"]
