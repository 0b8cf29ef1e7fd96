"""Host-side checks of the randomized parity cases: the draw is reproducible, every case
is a problem the library accepts (gdn_validate, no device work), and the mix covers every
composition, both arms, both gate forms, raw inputs and every solve block."""
from linear_attention_rnn_chunk_amd import gdn
from tests import randomized_cases as rc


def _problem(c):
    s = c.spec
    packed = s.packed or len(set(s.seq_lens)) > 1
    comp = {"auto": gdn.COMPOSE_AUTO, "split": gdn.COMPOSE_SPLIT, "fused": gdn.COMPOSE_FUSED,
            "pipelined": gdn.COMPOSE_PIPELINED, "seqsplit": gdn.COMPOSE_SEQSPLIT}[c.compose]
    return gdn.make_problem(s.n_seq, s.tokens, 0 if packed else s.seq_lens[0], s.hk, s.hv, s.dk, s.dv,
                            gdn.GATE_KEY_CHANNEL if s.gate == "channel" else gdn.GATE_HEAD, s.chunk,
                            gdn.BF16 if s.qkv_dtype == "bf16" else gdn.F32,
                            gdn.BF16 if s.o_dtype == "bf16" else gdn.F32,
                            gdn.ARM_MFMA_BF16 if c.arm == "bf16" else gdn.ARM_FOLD_F32, comp,
                            solve_block=c.solve_block)


def test_draw_is_reproducible():
    assert [rc.draw(i) for i in range(rc.N_CASES)] == rc.CASES


def test_every_case_is_accepted():
    for c in rc.CASES:
        p = _problem(c)
        assert gdn.validate(p) == gdn.GDN_OK, c
        if c.spec.raw:
            assert gdn.raw_workspace_bytes(p) >= gdn.workspace_bytes(p)


def test_the_mix_covers_the_domain():
    got = lambda f: {f(c) for c in rc.CASES}
    assert got(lambda c: c.compose) == {"auto", "split", "fused", "pipelined", "seqsplit"}
    assert got(lambda c: c.arm) == {"bf16", "f32"}
    assert got(lambda c: c.spec.gate) == {"head", "channel"}
    assert got(lambda c: c.spec.raw) == {True, False}
    assert got(lambda c: c.solve_block) == {0, 8, 16, 32}
    assert got(lambda c: c.spec.beta_law) == {"sigmoid", "one", "zero", "eps"}
    assert got(lambda c: c.spec.packed) == {True, False}
    assert any(0 in c.spec.seq_lens for c in rc.CASES) and any(1 in c.spec.seq_lens for c in rc.CASES)


def test_step_draw_is_reproducible_and_covers_both_gates():
    assert [rc.draw_decode(i) for i in range(rc.N_DECODE)] == rc.DECODE_CASES
    assert {c.spec.gate for c in rc.DECODE_CASES} == {"head", "channel"}
    assert {c.spec.h0 for c in rc.DECODE_CASES} == {True, False}
    assert {c.o_dtype for c in rc.DECODE_CASES} == {"bf16", "f32"}
