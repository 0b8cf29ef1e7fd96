"""The oracles against small examples of the rule worked by hand, with their derivations
and sources, in tests/golden/delta_rule_by_hand.json: the token-serial fp64 oracle, and the
dense chunk form at chunk sizes that put chunk boundaries inside and between the examples'
tokens.  Each planted mistake in either oracle fails at least one example."""
import json
import pathlib

import numpy as np
import pytest

import oracle
from oracle import chunked

EX = json.loads((pathlib.Path(__file__).parent / "golden" / "delta_rule_by_hand.json").read_text())["examples"]
IDS = ["ex%d" % i for i in range(len(EX))]


def _args(e):
    a = lambda x: None if x is None else np.asarray(x, dtype=np.float64)
    return (a(e["q"]), a(e["k"]), a(e["v"]), a(e["g"]), a(e["beta"]), a(e["h0"]),
            np.asarray(e["seq_start"], dtype=np.int64))


def _close(o, hT, e):
    return (np.allclose(o, np.asarray(e["o"], np.float64), rtol=0, atol=1e-12) and
            np.allclose(hT, np.asarray(e["hT"], np.float64), rtol=0, atol=1e-12))


@pytest.mark.parametrize("i", range(len(EX)), ids=IDS)
def test_serial_oracle_by_hand(i):
    q, k, v, g, beta, h0, ss = _args(EX[i])
    o, hT = oracle.serial_fwd(q, k, v, g, beta, h0, seq_start=ss)
    assert _close(o, hT, EX[i]), (EX[i]["name"], o.ravel(), hT.ravel())


@pytest.mark.parametrize("chunk", [1, 2, 64])
@pytest.mark.parametrize("i", range(len(EX)), ids=IDS)
def test_chunked_oracle_by_hand(i, chunk):
    q, k, v, g, beta, h0, ss = _args(EX[i])
    o, hT = chunked.chunked_fwd(q, k, v, g, beta, h0, seq_start=ss, chunk=chunk)
    assert _close(o, hT, EX[i]), (EX[i]["name"], chunk, o.ravel(), hT.ravel())


@pytest.mark.parametrize("mutant", [oracle.MUT_DECAY_AFTER_WRITE, oracle.MUT_NO_BETA_ERASE, oracle.MUT_TRANSPOSED_READ,
                                    oracle.MUT_GATE_NEXT_TOKEN, oracle.MUT_OUTPUT_BEFORE_WRITE])
def test_serial_mutants_fail_by_hand(mutant):
    failed = 0
    for e in EX:
        q, k, v, g, beta, h0, ss = _args(e)
        o, hT = oracle.serial_fwd(q, k, v, g, beta, h0, seq_start=ss, mutant=mutant)
        failed += not _close(o, hT, e)
    assert failed > 0


@pytest.mark.parametrize("mutant", ["gate_off_by_one", "drop_diag", "skip_solve", "no_reset"])
def test_chunked_mutants_fail_by_hand(mutant):
    failed = 0
    for e in EX:
        q, k, v, g, beta, h0, ss = _args(e)
        o, hT = chunked.chunked_fwd(q, k, v, g, beta, h0, seq_start=ss, chunk=2, mutant=mutant)
        failed += not _close(o, hT, e)
    assert failed > 0


# ---- the input side (raw q/k rows, beta logits, raw gate values) ----

from oracle import prepare as prep_oracle  # noqa: E402

RAW = json.loads((pathlib.Path(__file__).parent / "golden" / "input_side_by_hand.json").read_text())["examples"]


def _raw(e, mutant=prep_oracle.CORRECT):
    a = lambda x: None if x is None else np.asarray(x, dtype=np.float64)
    prepared = prep_oracle.prepare(a(e["q_raw"]), a(e["k_raw"]), a(e["gate_x"]), a(e["beta_logit"]),
                                   e["q_scale"], e["gate_scale"], mutant)
    o, hT = prep_oracle.raw_fwd(a(e["q_raw"]), a(e["k_raw"]), a(e["v"]), a(e["gate_x"]), a(e["beta_logit"]),
                                e["q_scale"], e["gate_scale"], a(e["h0"]),
                                seq_start=np.asarray(e["seq_start"], np.int64), mutant=mutant)
    return prepared, o, hT


def _raw_close(e, prepared, o, hT):
    want = [np.asarray(e[n], np.float64) for n in ("q", "k", "g", "beta")]
    return (all(np.allclose(x, w, rtol=0, atol=1e-12) for x, w in zip(prepared, want)) and _close(o, hT, e))


@pytest.mark.parametrize("i", range(len(RAW)))
def test_input_side_by_hand(i):
    assert _raw_close(RAW[i], *_raw(RAW[i]))


@pytest.mark.parametrize("mutant", [prep_oracle.MUT_NORM_SQUARED, prep_oracle.MUT_GATE_SIGN, prep_oracle.MUT_SIGMOID_FLIP,
                                    prep_oracle.MUT_SCALE_BOTH])
def test_input_side_mutants_fail_by_hand(mutant):
    assert any(not _raw_close(e, *_raw(e, mutant)) for e in RAW)
