"""The C-ABI library without a GPU: it loads, exports every symbol include/gdn.h
declares, and refuses unsupported or malformed calls on the host (nothing is
launched on these paths, so fake device addresses are safe)."""
import ctypes
import os
import re

import pytest

from linear_attention_rnn_chunk_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(gdn.LIBRARY_PATH):
        import __graft_entry__
        __graft_entry__.build()
    gdn.load()


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    declared = set(re.findall(r"^\s*(?:gdn_status|const char\*|int32_t)\s+(gdn_\w+)\s*\(", hdr, re.M))
    assert declared == set(gdn.EXPORTS)
    lib = ctypes.CDLL(gdn.LIBRARY_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_strings():
    assert gdn.abi_version() == gdn.ABI_VERSION == 2
    assert gdn.error_string(0) == "ok"
    for c in range(1, 7):
        assert gdn.error_string(c) != "unknown error code"
    assert gdn.error_string(99) == "unknown error code"
    assert gdn.status_string(0) == "ok"
    assert gdn.status_string(gdn.ST_NONFINITE_INPUT | gdn.ST_BAD_SEQLENS) == "nonfinite-input|bad-seqlens"
    assert "unknown" in gdn.status_string(0x100)


def P(**kw):
    base = dict(n_seq=1, total_tokens=256, seq_len=256, hk=2, hv=6, dk=128, dv=128)
    base.update(kw)
    return gdn.make_problem(**base)


@pytest.mark.parametrize("kw,code", [
    ({}, gdn.GDN_OK),
    (dict(dk=64, dv=32), gdn.GDN_OK),
    (dict(gate=gdn.GATE_KEY_CHANNEL, chunk=32), gdn.GDN_OK),
    (dict(gate=gdn.GATE_KEY_CHANNEL, chunk=0), gdn.GDN_OK),
    (dict(arm=gdn.ARM_FOLD_F32, qkv_dtype=gdn.F32, o_dtype=gdn.F32), gdn.GDN_OK),
    (dict(n_seq=-1), gdn.GDN_E_SHAPE),
    (dict(total_tokens=-5), gdn.GDN_E_SHAPE),
    (dict(hk=0), gdn.GDN_E_SHAPE),
    (dict(total_tokens=255), gdn.GDN_E_SHAPE),           # != n_seq * seq_len
    (dict(n_seq=0, seq_len=0), gdn.GDN_E_SHAPE),          # tokens that belong to no sequence
    (dict(n_seq=0, total_tokens=0, seq_len=0), gdn.GDN_OK),
    # packed batches: int32 offsets, rounded up to whole chunks in int32 on the device
    (dict(n_seq=3, seq_len=0, total_tokens=2**31 - 1 - 64, hk=1, hv=1, dk=32, dv=32), gdn.GDN_OK),
    (dict(n_seq=3, seq_len=0, total_tokens=2**31 - 1 - 63, hk=1, hv=1, dk=32, dv=32), gdn.GDN_E_UNSUPPORTED),
    (dict(hv=5), gdn.GDN_E_UNSUPPORTED),                 # hv % hk
    (dict(dk=96), gdn.GDN_E_UNSUPPORTED),
    (dict(dv=256), gdn.GDN_E_UNSUPPORTED),
    (dict(chunk=16), gdn.GDN_E_UNSUPPORTED),
    (dict(gate=gdn.GATE_KEY_CHANNEL, chunk=64), gdn.GDN_E_UNSUPPORTED),
    (dict(gate=7), gdn.GDN_E_UNSUPPORTED),
    (dict(qkv_dtype=3), gdn.GDN_E_UNSUPPORTED),
    (dict(arm=2), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=9), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_FUSED), gdn.GDN_OK),
    (dict(compose=gdn.COMPOSE_FUSED, chunk=32, dk=64, dv=32), gdn.GDN_OK),
    # the fused composition is built for the per-head gate, bf16 inputs, the bf16 arm
    (dict(compose=gdn.COMPOSE_FUSED, gate=gdn.GATE_KEY_CHANNEL, chunk=32), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_FUSED, qkv_dtype=gdn.F32), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_FUSED, arm=gdn.ARM_FOLD_F32), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_FUSED, stages=gdn.STAGE_PREP), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_FUSED, stages=gdn.STAGE_PREP | gdn.STAGE_SCAN), gdn.GDN_OK),
    # the pipelined composition: per-head gate, fixed-length batches, all stages, any arm
    (dict(compose=gdn.COMPOSE_PIPELINED), gdn.GDN_OK),
    (dict(compose=gdn.COMPOSE_PIPELINED, arm=gdn.ARM_FOLD_F32, qkv_dtype=gdn.F32), gdn.GDN_OK),
    (dict(compose=gdn.COMPOSE_PIPELINED, stages=gdn.STAGE_PREP | gdn.STAGE_SCAN), gdn.GDN_OK),
    (dict(compose=gdn.COMPOSE_PIPELINED, gate=gdn.GATE_KEY_CHANNEL, chunk=32), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_PIPELINED, n_seq=3, seq_len=0), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_PIPELINED, stages=gdn.STAGE_SCAN), gdn.GDN_E_UNSUPPORTED),
    # the sequence split: as pipelined, and square states (dk == dv)
    (dict(compose=gdn.COMPOSE_SEQSPLIT), gdn.GDN_OK),
    (dict(compose=gdn.COMPOSE_SEQSPLIT, dk=64, dv=64), gdn.GDN_OK),
    (dict(compose=gdn.COMPOSE_SEQSPLIT, dk=128, dv=64), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_SEQSPLIT, gate=gdn.GATE_KEY_CHANNEL, chunk=32), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_SEQSPLIT, n_seq=3, seq_len=0), gdn.GDN_E_UNSUPPORTED),
    (dict(compose=gdn.COMPOSE_SEQSPLIT, stages=gdn.STAGE_PREP), gdn.GDN_E_UNSUPPORTED),
    # the solve's diagonal block: 8, 16 or 32 rows (0: the library's); the tile stages inside
    # scan launches (fused, pipelined) are built for 16 rows only
    (dict(solve_block=8), gdn.GDN_OK),
    (dict(solve_block=16), gdn.GDN_OK),
    (dict(solve_block=32, chunk=32), gdn.GDN_OK),
    (dict(solve_block=8, gate=gdn.GATE_KEY_CHANNEL, chunk=32), gdn.GDN_OK),
    (dict(solve_block=32, compose=gdn.COMPOSE_SEQSPLIT), gdn.GDN_OK),
    (dict(solve_block=16, compose=gdn.COMPOSE_PIPELINED), gdn.GDN_OK),
    (dict(solve_block=16, compose=gdn.COMPOSE_FUSED), gdn.GDN_OK),
    (dict(solve_block=4), gdn.GDN_E_UNSUPPORTED),
    (dict(solve_block=64), gdn.GDN_E_UNSUPPORTED),
    (dict(solve_block=-16), gdn.GDN_E_UNSUPPORTED),
    (dict(solve_block=8, compose=gdn.COMPOSE_PIPELINED), gdn.GDN_E_UNSUPPORTED),
    (dict(solve_block=32, compose=gdn.COMPOSE_FUSED), gdn.GDN_E_UNSUPPORTED),
])
def test_validate_refusals(kw, code):
    assert gdn.validate(P(**kw)) == code


def test_plan_compose_host_rules():
    # explicit requests are reported as given; refused problems keep their error code;
    # AUTO resolves to split or pipelined (the latter only where the device has idle units)
    assert gdn.plan_compose(P(compose=gdn.COMPOSE_SPLIT)) == gdn.COMPOSE_SPLIT
    assert gdn.plan_compose(P(compose=gdn.COMPOSE_FUSED)) == gdn.COMPOSE_FUSED
    assert gdn.plan_compose(P(compose=gdn.COMPOSE_SEQSPLIT)) == gdn.COMPOSE_SEQSPLIT
    assert gdn.plan_compose(P(gate=gdn.GATE_KEY_CHANNEL, chunk=32)) == gdn.COMPOSE_SPLIT
    assert gdn.plan_compose(P(n_seq=3, seq_len=0)) == gdn.COMPOSE_SPLIT
    assert gdn.plan_compose(P(compose=gdn.COMPOSE_AUTO)) in (gdn.COMPOSE_SPLIT, gdn.COMPOSE_PIPELINED)
    # another diagonal block of the solve keeps the tile stage in its own kernel
    for sb in (8, 32):
        assert gdn.plan_compose(P(n_seq=8, total_tokens=8 * 32768, seq_len=32768, hk=16, hv=32,
                                  solve_block=sb)) == gdn.COMPOSE_SPLIT
    with pytest.raises(gdn.GdnError):
        gdn.plan_compose(P(dk=96))
    lib = gdn.load()
    assert lib.gdn_plan_compose(ctypes.byref(P()), None) == gdn.GDN_E_NULL


def test_validate_null_problem():
    lib = gdn.load()
    assert lib.gdn_validate(None) == gdn.GDN_E_NULL
    n = ctypes.c_size_t(0)
    assert lib.gdn_workspace_bytes(ctypes.byref(P()), None) == gdn.GDN_E_NULL


def test_workspace_bytes_scales_with_tiles():
    # per chunk slot and value head: T and P, each stored as the lower-triangle MFMA
    # fragments of a C x C tile (C = 64: 6 of the 8 fragments of 16 x 32, 3072 elements;
    # C = 32: 2 fragments, 1024), bf16 (2 B) or fp32 (4 B)
    slots, hv = 4, 6
    for C, elems in ((64, 3072), (32, 1024)):
        b16 = gdn.workspace_bytes(P(chunk=C, compose=gdn.COMPOSE_SPLIT))
        f32 = gdn.workspace_bytes(P(chunk=C, arm=gdn.ARM_FOLD_F32, compose=gdn.COMPOSE_SPLIT))
        s = slots * 64 // C
        assert 2 * s * hv * elems * 2 <= b16 < 2 * s * hv * elems * 2 + 1024
        # the fp32 arm also keeps K and Q in fp32 for the scan: [slot][hk][C][dk] each
        kq = 2 * s * 2 * C * 128 * 4
        assert 2 * s * hv * elems * 4 + kq <= f32 < 2 * s * hv * elems * 4 + kq + 1024
    # the library's choice may pipeline a fixed-length per-head-gate batch: the state
    # carried between scan segments, [n_seq][hv][dk][dv] fp32, on top of the split tiles
    # the sequence split (on request only): per-part states, transitions and chained
    # inputs, 3 x 4 parts of [n_seq][hv][dk][dv] fp32
    carry = 1 * hv * 128 * 128 * 4
    parts = 3 * 4 * carry
    assert gdn.workspace_bytes(P()) == gdn.workspace_bytes(P(compose=gdn.COMPOSE_SPLIT)) + carry
    assert gdn.workspace_bytes(P(compose=gdn.COMPOSE_PIPELINED)) == gdn.workspace_bytes(P())
    assert gdn.workspace_bytes(P(compose=gdn.COMPOSE_SEQSPLIT)) == \
        gdn.workspace_bytes(P(compose=gdn.COMPOSE_SPLIT)) + parts
    assert gdn.workspace_bytes(P(gate=gdn.GATE_KEY_CHANNEL, chunk=32)) == \
        gdn.workspace_bytes(P(gate=gdn.GATE_KEY_CHANNEL, chunk=32, compose=gdn.COMPOSE_SPLIT))
    # fused composition: no tiles in the workspace (only the chunk table of a packed batch)
    assert gdn.workspace_bytes(P(compose=gdn.COMPOSE_FUSED)) == 0
    assert 0 < gdn.workspace_bytes(P(n_seq=3, seq_len=0, compose=gdn.COMPOSE_FUSED)) <= 256
    # packed form: slots bounded by ceil(total / C) + n_seq, plus the chunk table
    pk = gdn.workspace_bytes(P(n_seq=3, seq_len=0, chunk=64))
    assert pk >= 2 * (4 + 3) * hv * 3072 * 2


def test_pipelined_request_keeps_two_segments_of_tiles():
    # sequences of 512 chunks (64 tokens each): a pipelined call keeps the tiles of the
    # segment it scans and of the next one (2 x 32 chunks per sequence), split keeps all
    r256 = lambda x: (x + 255) // 256 * 256
    kw = dict(n_seq=2, total_tokens=2 * 32768, seq_len=32768, hk=16, hv=48)
    tile = 6 * 512 * 2                                # T or P of one chunk and value head, bf16
    carry = 2 * 48 * 128 * 128 * 4                    # the state between segments
    assert gdn.workspace_bytes(P(compose=gdn.COMPOSE_PIPELINED, **kw)) == 2 * r256(2 * 64 * 48 * tile) + carry
    assert gdn.workspace_bytes(P(compose=gdn.COMPOSE_SPLIT, **kw)) == 2 * r256(2 * 512 * 48 * tile)
    # AUTO may still pick split on a device with no idle units: it sizes for every chunk
    assert gdn.workspace_bytes(P(**kw)) == 2 * r256(2 * 512 * 48 * tile) + carry
    # two segments or fewer: no ring, every chunk its own slot
    short = dict(n_seq=1, total_tokens=4096, seq_len=4096, hk=16, hv=16)
    assert gdn.workspace_bytes(P(compose=gdn.COMPOSE_PIPELINED, **short)) == \
        gdn.workspace_bytes(P(compose=gdn.COMPOSE_SPLIT, **short)) + 16 * 128 * 128 * 4


# fake, well-aligned device addresses: the host checks below return before any launch
BASE = 1 << 40


def _addrs(prob, qkv=2, osz=2):
    T, hk, hv, dk, dv = prob.total_tokens, prob.hk, prob.hv, prob.dk, prob.dv
    sizes = dict(q=T * hk * dk * qkv, k=T * hk * dk * qkv, v=T * hv * dv * qkv, g=T * hv * 4,
                 beta=T * hv * 4, h0=prob.n_seq * hv * dk * dv * 4, o=T * hv * dv * osz,
                 hT=prob.n_seq * hv * dk * dv * 4, status=4, ws=gdn.workspace_bytes(prob))
    a, out = BASE, {}
    for k_, n in sizes.items():
        out[k_] = a
        a += (n + 4095) // 4096 * 4096 + 4096
    return out, sizes


def _call(prob, a, ws_bytes=None, cu=None, **override):
    lib = gdn.load()
    args = dict(a)
    args.update(override)
    vp = ctypes.c_void_p
    return lib.gdn_chunk_fwd(ctypes.byref(prob), vp(args["q"]), vp(args["k"]), vp(args["v"]),
                             vp(args["g"]), vp(args["beta"]), vp(args["h0"]), vp(cu),
                             vp(args["o"]), vp(args["hT"]), vp(args["status"]), vp(args["ws"]),
                             ctypes.c_size_t(ws_bytes if ws_bytes is not None else
                                             gdn.workspace_bytes(prob)), vp(0))


def test_call_refusals_on_host():
    prob = P()
    a, s = _addrs(prob)
    assert _call(prob, a, status=None) == gdn.GDN_E_NULL
    assert _call(prob, a, q=None) == gdn.GDN_E_NULL
    assert _call(prob, a, ws=None) == gdn.GDN_E_NULL
    assert _call(prob, a, ws_bytes=gdn.workspace_bytes(prob) - 1) == gdn.GDN_E_WORKSPACE
    assert _call(prob, a, ws=a["ws"] + 128) == gdn.GDN_E_WORKSPACE          # not 256-aligned
    assert _call(prob, a, q=a["q"] + 8) == gdn.GDN_E_UNSUPPORTED            # not 16-aligned
    assert _call(prob, a, hT=a["h0"]) == gdn.GDN_E_ALIAS                    # hT aliases h0
    assert _call(prob, a, hT=a["h0"] + 4 * 128) == gdn.GDN_E_ALIAS          # partial overlap
    assert _call(prob, a, o=a["v"]) == gdn.GDN_E_ALIAS
    assert _call(prob, a, o=a["hT"]) == gdn.GDN_E_ALIAS
    assert _call(prob, a, ws=a["o"]) == gdn.GDN_E_ALIAS
    # fixed-length problem must not also carry cu_seqlens; packed problem needs them
    assert _call(prob, a, cu=BASE - 4096) == gdn.GDN_E_SHAPE
    pk = P(seq_len=0)
    a2, _ = _addrs(pk)
    assert _call(pk, a2) == gdn.GDN_E_NULL
    # invalid problem is refused before pointers are looked at
    assert _call(P(dk=48), a, ws_bytes=1 << 30) == gdn.GDN_E_UNSUPPORTED


def test_empty_problem_returns_ok_without_device_work():
    prob = P(n_seq=0, total_tokens=0, seq_len=0)
    lib = gdn.load()
    st = ctypes.c_void_p(BASE)
    rc = lib.gdn_chunk_fwd(ctypes.byref(prob), None, None, None, None, None, None, None, None,
                           None, st, None, ctypes.c_size_t(0), None)
    assert rc == gdn.GDN_OK


def D(**kw):
    base = dict(n_seq=4, total_tokens=4, seq_len=1, hk=2, hv=6, dk=128, dv=128)
    base.update(kw)
    return gdn.make_problem(**base)


def _daddrs(prob, qkv=2, osz=2):
    N, hk, hv, dk, dv = prob.n_seq, prob.hk, prob.hv, prob.dk, prob.dv
    gw = dk if prob.gate == gdn.GATE_KEY_CHANNEL else 1
    sizes = dict(q=N * hk * dk * qkv, k=N * hk * dk * qkv, v=N * hv * dv * qkv, g=N * hv * gw * 4,
                 beta=N * hv * 4, h_in=N * hv * dk * dv * 4, o=N * hv * dv * osz,
                 h_out=N * hv * dk * dv * 4, status=4)
    a, out = BASE, {}
    for k_, n in sizes.items():
        out[k_] = a
        a += (n + 4095) // 4096 * 4096 + 4096
    return out


def _dcall(prob, a, **override):
    args = dict(a)
    args.update(override)
    vp = ctypes.c_void_p
    return gdn.load().gdn_decode_step(
        ctypes.byref(prob), vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["g"]),
        vp(args["beta"]), vp(args["h_in"]), vp(args["o"]), vp(args["h_out"]), vp(args["status"]),
        vp(0))


def test_decode_refusals_on_host():
    a = _daddrs(D())
    lib = gdn.load()
    assert lib.gdn_decode_step(None, *([None] * 10)) == gdn.GDN_E_NULL
    assert _dcall(D(seq_len=2, total_tokens=8), a) == gdn.GDN_E_SHAPE     # not one token each
    assert _dcall(D(total_tokens=5), a) == gdn.GDN_E_SHAPE
    assert _dcall(D(n_seq=-1, total_tokens=-1), a) == gdn.GDN_E_SHAPE
    assert _dcall(D(hv=5), a) == gdn.GDN_E_UNSUPPORTED
    assert _dcall(D(dk=96), a) == gdn.GDN_E_UNSUPPORTED
    assert _dcall(D(dv=16), a) == gdn.GDN_E_UNSUPPORTED
    assert _dcall(D(gate=3), a) == gdn.GDN_E_UNSUPPORTED
    assert _dcall(D(o_dtype=5), a) == gdn.GDN_E_UNSUPPORTED
    assert _dcall(D(), a, status=None) == gdn.GDN_E_NULL
    assert _dcall(D(), a, h_out=None) == gdn.GDN_E_NULL
    assert _dcall(D(), a, v=None) == gdn.GDN_E_NULL
    assert _dcall(D(), a, h_in=a["h_in"] + 8) == gdn.GDN_E_UNSUPPORTED    # not 16-aligned
    assert _dcall(D(), a, v=a["v"] + 4) == gdn.GDN_E_UNSUPPORTED          # bf16 v: 8-aligned
    assert _dcall(D(), a, h_out=a["h_in"]) == gdn.GDN_E_ALIAS             # in-place state
    assert _dcall(D(), a, h_out=a["h_in"] + 4096) == gdn.GDN_E_ALIAS      # partial overlap
    assert _dcall(D(), a, o=a["q"]) == gdn.GDN_E_ALIAS
    assert _dcall(D(), a, status=a["o"]) == gdn.GDN_E_ALIAS
    # chunk, arm, compose and stages are not read by the step
    assert _dcall(D(n_seq=0, total_tokens=0, chunk=16, arm=7, compose=9), a) == gdn.GDN_OK


def test_decode_empty_batch_launches_nothing():
    lib = gdn.load()
    st = ctypes.c_void_p(BASE)
    rc = lib.gdn_decode_step(ctypes.byref(D(n_seq=0, total_tokens=0)), None, None, None, None,
                             None, None, None, None, st, None)
    assert rc == gdn.GDN_OK
