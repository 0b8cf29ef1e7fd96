// gdn_api.cpp -- host side of the C ABI declared in include/gdn.h: argument
// validation, supported-domain refusal, workspace sizing, status decoding.
// Nothing here touches the device except through gdn::launch().
#include <stdio.h>
#include <string.h>

#include <string>

#include "gdn_internal.h"

namespace gdn {

#ifdef GDN_SCAN_STAMPS
// measurement build: where the next calls' scan records its step timestamps
static uint64_t* g_stamps = nullptr;
static int32_t g_stamp_block = 0, g_stamp_c0 = 0;
#endif

static inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

gdn_status make_plan(const gdn_problem* p, Plan* out, bool raw) {
  if (!p || !out) return GDN_E_NULL;
  if (p->n_seq < 0 || p->total_tokens < 0 || p->seq_len < 0 || p->hk < 1 || p->hv < 1)
    return GDN_E_SHAPE;
  if (p->seq_len > 0 && (int64_t)p->n_seq * p->seq_len != p->total_tokens) return GDN_E_SHAPE;
  // tokens that belong to no sequence
  if (p->n_seq == 0 && p->total_tokens > 0) return GDN_E_SHAPE;
  if (p->hv % p->hk != 0) return GDN_E_UNSUPPORTED;
  if (!(p->dk == 32 || p->dk == 64 || p->dk == 128)) return GDN_E_UNSUPPORTED;
  if (!(p->dv == 32 || p->dv == 64 || p->dv == 128)) return GDN_E_UNSUPPORTED;
  if (p->gate != GDN_GATE_HEAD && p->gate != GDN_GATE_KEY_CHANNEL) return GDN_E_UNSUPPORTED;
  if (!(p->chunk == 0 || p->chunk == 32 || p->chunk == 64)) return GDN_E_UNSUPPORTED;
  if (p->gate == GDN_GATE_KEY_CHANNEL && p->chunk == 64) return GDN_E_UNSUPPORTED;
  if (p->qkv_dtype != GDN_BF16 && p->qkv_dtype != GDN_F32) return GDN_E_UNSUPPORTED;
  if (p->o_dtype != GDN_BF16 && p->o_dtype != GDN_F32) return GDN_E_UNSUPPORTED;
  if (p->arm != GDN_ARM_MFMA_BF16 && p->arm != GDN_ARM_FOLD_F32) return GDN_E_UNSUPPORTED;
  if (p->compose != GDN_COMPOSE_AUTO && p->compose != GDN_COMPOSE_SPLIT &&
      p->compose != GDN_COMPOSE_FUSED && p->compose != GDN_COMPOSE_PIPELINED &&
      p->compose != GDN_COMPOSE_SEQSPLIT)
    return GDN_E_UNSUPPORTED;
  if (p->stages < 0 || p->stages > (GDN_STAGE_PREP | GDN_STAGE_SCAN)) return GDN_E_UNSUPPORTED;
  if (!(p->solve_block == 0 || p->solve_block == 8 || p->solve_block == 16 || p->solve_block == 32))
    return GDN_E_UNSUPPORTED;
  // the tile stages inside the scan launches (fused, pipelined) solve with the library's
  // diagonal block only; another block size runs the split composition
  const bool any_block = p->solve_block == 0 || p->solve_block == kSolveBlock;
  if (!any_block && (p->compose == GDN_COMPOSE_FUSED || p->compose == GDN_COMPOSE_PIPELINED))
    return GDN_E_UNSUPPORTED;
  // the fused composition (tile waves inside the scan workgroup) is built for the
  // per-head gate with bf16 inputs on the bf16 arm, and has no separate stages
  if (p->compose == GDN_COMPOSE_FUSED &&
      (p->gate != GDN_GATE_HEAD || p->qkv_dtype != GDN_BF16 || p->arm != GDN_ARM_MFMA_BF16 ||
       !(p->stages == GDN_STAGE_ALL || p->stages == (GDN_STAGE_PREP | GDN_STAGE_SCAN))))
    return GDN_E_UNSUPPORTED;

  // the pipelined composition (scan segments carrying the state, the next segment's
  // prep beside each) is built for the per-head gate on fixed-length batches, all stages
  const bool fixed_all = p->gate == GDN_GATE_HEAD && p->seq_len > 0 &&
                         (p->stages == GDN_STAGE_ALL || p->stages == (GDN_STAGE_PREP | GDN_STAGE_SCAN));
  const bool pipe_ok = fixed_all && any_block;
  if (p->compose == GDN_COMPOSE_PIPELINED && !pipe_ok) return GDN_E_UNSUPPORTED;
  // the sequence split (parts scanned side by side, chained through their transitions)
  // additionally needs square states: a transition is a dk x dk state scanned like a value
  const bool seq_ok = fixed_all && p->dk == p->dv;
  if (p->compose == GDN_COMPOSE_SEQSPLIT && !seq_ok) return GDN_E_UNSUPPORTED;
  // raw inputs: the per-head gate, split or pipelined (the row norms pass through the
  // workspace from the prep to the scan; the fused composition has no such stage)
  if (raw && (p->gate != GDN_GATE_HEAD || p->compose == GDN_COMPOSE_FUSED)) return GDN_E_UNSUPPORTED;
  Plan pl;
  memset(&pl, 0, sizeof(pl));
  pl.raw = raw;
  pl.n_seq = p->n_seq;
  pl.seq_len = p->seq_len;
  pl.hk = p->hk;
  pl.hv = p->hv;
  pl.dk = p->dk;
  pl.dv = p->dv;
  pl.total = p->total_tokens;
  pl.gate_channel = p->gate == GDN_GATE_KEY_CHANNEL;
  pl.chunk = p->chunk ? p->chunk : (pl.gate_channel ? 32 : 64);
  pl.solve_block = p->solve_block ? p->solve_block : kSolveBlock;
  pl.arm_f32 = p->arm == GDN_ARM_FOLD_F32;
  pl.qkv_f32 = p->qkv_dtype == GDN_F32;
  pl.o_f32 = p->o_dtype == GDN_F32;
  pl.fused = p->compose == GDN_COMPOSE_FUSED;
  pl.pipe_ok = pipe_ok && (p->compose == GDN_COMPOSE_AUTO || p->compose == GDN_COMPOSE_PIPELINED);
  pl.pipe_req = p->compose == GDN_COMPOSE_PIPELINED ? 1 : (p->compose == GDN_COMPOSE_AUTO ? -1 : 0);
  // (only on request: measured slower than split on the shapes it is for, see seqsplit_parts)
  pl.seq_ok = seq_ok && p->compose == GDN_COMPOSE_SEQSPLIT;
  pl.seq_req = p->compose == GDN_COMPOSE_SEQSPLIT ? 1 : 0;
  pl.run_prep = p->stages == GDN_STAGE_ALL || (p->stages & GDN_STAGE_PREP);
  pl.run_scan = p->stages == GDN_STAGE_ALL || (p->stages & GDN_STAGE_SCAN);
  // The fixed-length form is chosen when seq_len > 0 or when there are no tokens at all;
  // otherwise cu_seqlens must describe the sequences (checked in gdn_chunk_fwd).
  pl.varlen = !(p->seq_len > 0 || p->total_tokens == 0);
  const int64_t C = pl.chunk;
  if (pl.varlen) {
    // int32 cu_seqlens, and the device rounds a sequence's length up to whole chunks in
    // int32 (length + C - 1)
    if (p->total_tokens > INT32_MAX - 64) return GDN_E_UNSUPPORTED;
    pl.chunks_per_seq = 0;
    pl.max_slots = (p->total_tokens + C - 1) / C + p->n_seq;
  } else {
    pl.chunks_per_seq = (int32_t)((p->seq_len + C - 1) / C);
    pl.max_slots = (int64_t)p->n_seq * pl.chunks_per_seq;
  }
  // grid sizes are flattened into blockIdx.x
  if (pl.max_slots * pl.hv > INT32_MAX) return GDN_E_UNSUPPORTED;
  if ((int64_t)pl.n_seq * pl.hv * (pl.dv / 32) > INT32_MAX) return GDN_E_UNSUPPORTED;

  // Pipelined composition on sequences longer than two segments: only the tiles of the
  // segment being scanned and of the next one are live, so the tile buffers can be a ring
  // of two segments per sequence.  An explicit PIPELINED request sizes the workspace for
  // the ring; AUTO may still pick split, so it sizes for every chunk (the ring fits in it).
  const int32_t seg = kSegTokens / pl.chunk;
  pl.tile_ring = (pl.pipe_ok && !pl.varlen && pl.chunks_per_seq > 2 * seg) ? seg : 0;
  pl.tile_slots = (pl.tile_ring && p->compose == GDN_COMPOSE_PIPELINED) ? (int64_t)pl.n_seq * 2 * seg
                                                                        : pl.max_slots;
  const size_t esz = pl.arm_f32 ? 4 : 2;
  size_t off = 0;
  pl.off_table = off;
  // packed batch: bounds and chunk prefix ([n_seq + 1] each), then the scan's dispatch order
  off = round_up(off + (pl.varlen ? sizeof(int32_t) * (3 * (size_t)pl.n_seq + 2) : 0), 256);
  // split composition: T and P of every chunk pass through the workspace
  const size_t tile = pl.fused ? 0 : (size_t)pl.tile_slots * pl.hv * gdn::tile_elems(C) * esz;
  pl.off_T = off;
  off = round_up(off + tile, 256);
  pl.off_P = off;
  off = round_up(off + tile, 256);
  // per-channel gate: gated operands and chunk decay, produced by the sequence-parallel
  // stage so the scan streams them instead of re-deriving them serially
  const size_t gated = pl.gate_channel ? (size_t)pl.max_slots * pl.hv * 3 * C * pl.dk * esz : 0;
  const size_t decb = pl.gate_channel ? (size_t)pl.max_slots * pl.hv * pl.dk * 4 : 0;
  pl.off_G = off;
  off = round_up(off + gated, 256);
  pl.off_D = off;
  off = round_up(off + decb, 256);
  // per-head gate with fp32 inputs or the fp32 arm: K and Q in the arm's element type,
  // written by the sequence-parallel stage so the scan copies them without converting
  pl.kq_ws = !pl.gate_channel && (pl.qkv_f32 || pl.arm_f32);
  const size_t kq = pl.kq_ws ? (size_t)pl.tile_slots * pl.hk * C * pl.dk * esz : 0;
  pl.off_K = off;
  off = round_up(off + kq, 256);
  pl.off_Q = off;
  off = round_up(off + kq, 256);
  // pipelined composition: the state carried from one scan segment to the next
  const size_t carry = pl.pipe_ok ? (size_t)pl.n_seq * pl.hv * pl.dk * pl.dv * 4 : 0;
  pl.off_carry = off;
  off = round_up(off + carry, 256);
  // sequence split: per-part states, transitions and chained inputs (up to kMaxParts parts)
  const size_t parts = pl.seq_ok ? 3 * (size_t)kMaxParts * pl.n_seq * pl.hv * pl.dk * pl.dv * 4 : 0;
  pl.off_parts = off;
  off = round_up(off + parts, 256);
  // raw inputs: 1 / |k| and q_scale / |q| of every row, per tile slot and key head
  const size_t norms = raw ? (size_t)pl.tile_slots * pl.hk * 2 * C * 4 : 0;
  pl.off_N = off;
  off = round_up(off + norms, 256);
  pl.bytes = off;
  *out = pl;
  return GDN_OK;
}

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace gdn

extern "C" {

gdn_status gdn_validate(const gdn_problem* p) {
  gdn::Plan pl;
  return gdn::make_plan(p, &pl);
}

gdn_status gdn_plan_compose(const gdn_problem* p, int32_t* compose) {
  if (!compose) return GDN_E_NULL;
  gdn::Plan pl;
  gdn_status s = gdn::make_plan(p, &pl);
  if (s != GDN_OK) return s;
  *compose = gdn::plan_compose(pl);
  return GDN_OK;
}
gdn_status gdn_workspace_bytes(const gdn_problem* p, size_t* bytes) {
  if (!bytes) return GDN_E_NULL;
  gdn::Plan pl;
  gdn_status s = gdn::make_plan(p, &pl);
  if (s != GDN_OK) return s;
  *bytes = pl.bytes;
  return GDN_OK;
}

}  // extern "C"

namespace gdn {

// gdn_chunk_fwd, and with `raw` gdn_chunk_fwd_raw_inputs
static gdn_status chunk_fwd(const gdn_problem* p, const gdn_raw_inputs* raw, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, const float* h0,
                            const int32_t* cu_seqlens, void* o, float* hT, uint32_t* status, void* workspace,
                            size_t workspace_bytes, void* stream) {
  gdn::Plan pl;
  gdn_status s = gdn::make_plan(p, &pl, raw != nullptr);
  if (s != GDN_OK) return s;
  if (raw && !(raw->q_scale > 0.f && raw->gate_scale > 0.f && raw->q_scale < 3.4e38f && raw->gate_scale < 3.4e38f))
    return GDN_E_UNSUPPORTED;  // positive and finite
  if (!status) return GDN_E_NULL;
  if (pl.total > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_E_NULL;
  if (p->seq_len > 0 && cu_seqlens) return GDN_E_SHAPE;  // one description of the sequences
  if (pl.varlen && !cu_seqlens) return GDN_E_NULL;
  if (pl.bytes > 0 && !workspace) return GDN_E_NULL;
  if (workspace_bytes < pl.bytes) return GDN_E_WORKSPACE;
  if (workspace && !gdn::aligned(workspace, 256)) return GDN_E_WORKSPACE;
  if (!gdn::aligned(q, 16) || !gdn::aligned(k, 16) || !gdn::aligned(v, 16) || !gdn::aligned(o, 16) ||
      !gdn::aligned(g, 4) || !gdn::aligned(beta, 4) || !gdn::aligned(h0, 4) ||
      !gdn::aligned(hT, 4) || !gdn::aligned(status, 4) || !gdn::aligned(cu_seqlens, 4))
    return GDN_E_UNSUPPORTED;

  const size_t qsz = pl.qkv_f32 ? 4 : 2, osz = pl.o_f32 ? 4 : 2;
  const size_t T = (size_t)pl.total;
  const size_t nq = T * pl.hk * pl.dk * qsz, nv = T * pl.hv * pl.dv * qsz;
  const size_t ng = T * pl.hv * (pl.gate_channel ? pl.dk : 1) * 4, nb = T * pl.hv * 4;
  const size_t nh = (size_t)pl.n_seq * pl.hv * pl.dk * pl.dv * 4;
  const size_t ncu = cu_seqlens ? (size_t)(pl.n_seq + 1) * 4 : 0;
  const size_t no = T * pl.hv * pl.dv * osz;
  struct R {
    const void* p;
    size_t n;
  };
  const R ins[] = {{q, nq}, {k, nq}, {v, nv}, {g, ng}, {beta, nb}, {h0, nh}, {cu_seqlens, ncu}};
  const R outs[] = {{o, no}, {hT, nh}, {status, 4}, {workspace, pl.bytes}};
  for (const R& a : outs) {
    for (const R& b : ins)
      if (gdn::overlap(a.p, a.n, b.p, b.n)) return GDN_E_ALIAS;
    for (const R& b : outs)
      if (&a != &b && gdn::overlap(a.p, a.n, b.p, b.n)) return GDN_E_ALIAS;
  }
  if (pl.n_seq == 0) return GDN_OK;  // nothing to compute

  gdn::Params prm;
  memset(&prm, 0, sizeof(prm));
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.g = g;
  prm.beta = beta;
  prm.h0 = h0;
  prm.cu_seqlens = cu_seqlens;
  prm.o = o;
  prm.hT = hT;
  prm.status = status;
  char* ws = (char*)workspace;
  prm.table = pl.varlen ? (int32_t*)(ws + pl.off_table) : nullptr;
  prm.Tws = ws ? ws + pl.off_T : nullptr;
  prm.Pws = ws ? ws + pl.off_P : nullptr;
  prm.Gws = (ws && pl.gate_channel) ? ws + pl.off_G : nullptr;
  prm.Dws = (ws && pl.gate_channel) ? (float*)(ws + pl.off_D) : nullptr;
  prm.Kws = (ws && pl.kq_ws) ? ws + pl.off_K : nullptr;
  prm.Qws = (ws && pl.kq_ws) ? ws + pl.off_Q : nullptr;
  prm.kq_ws = pl.kq_ws;
  prm.total = pl.total;
  prm.n_seq = pl.n_seq;
  prm.seq_len = pl.seq_len;
  prm.hk = pl.hk;
  prm.hv = pl.hv;
  prm.dv = pl.dv;
  prm.qkv_f32 = pl.qkv_f32;
  prm.o_f32 = pl.o_f32;
  prm.varlen = pl.varlen;
  prm.chunks_per_seq = pl.chunks_per_seq;
  prm.max_slots = pl.max_slots;
  prm.seg_cb = 0;
  prm.seg_ce = pl.varlen ? INT32_MAX : pl.chunks_per_seq;
  prm.prep_cb = 0;
  prm.prep_ce = prm.seg_ce;
  prm.nscan = (int32_t)((int64_t)pl.n_seq * pl.hv * (pl.dv / 32));
  prm.h0_input = 1;
  prm.solve_block = pl.solve_block;
  if (raw) {
    prm.raw = 1;
    prm.q_scale = raw->q_scale;
    prm.gate_scale = raw->gate_scale;
    prm.Nws = (float*)(ws + pl.off_N);
  }
#ifdef GDN_SCAN_STAMPS
  prm.stamps = gdn::g_stamps;
  prm.stamp_block = gdn::g_stamp_block;
  prm.stamp_c0 = gdn::g_stamp_c0;
#endif
  if (ws && pl.seq_ok) {
    const size_t one = (size_t)gdn::kMaxParts * pl.n_seq * pl.hv * pl.dk * pl.dv;
    prm.Bws = (float*)(ws + pl.off_parts);
    prm.Mws = prm.Bws + one;
    prm.Hws = prm.Mws + one;
  }
  return gdn::launch(pl, prm, ws ? ws + pl.off_carry : nullptr, stream);
}

}  // namespace gdn

extern "C" {

gdn_status gdn_chunk_fwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* h0,
                         const int32_t* cu_seqlens, void* o, float* hT, uint32_t* status,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return gdn::chunk_fwd(p, nullptr, q, k, v, g, beta, h0, cu_seqlens, o, hT, status, workspace,
                        workspace_bytes, stream);
}

gdn_status gdn_raw_workspace_bytes(const gdn_problem* p, size_t* bytes) {
  if (!bytes) return GDN_E_NULL;
  gdn::Plan pl;
  gdn_status s = gdn::make_plan(p, &pl, true);
  if (s != GDN_OK) return s;
  *bytes = pl.bytes;
  return GDN_OK;
}

gdn_status gdn_chunk_fwd_raw_inputs(const gdn_problem* p, const gdn_raw_inputs* raw, const void* q_raw,
                                    const void* k_raw, const void* v, const float* gate_x,
                                    const float* beta_logit, const float* h0, const int32_t* cu_seqlens,
                                    void* o, float* hT, uint32_t* status, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!raw) return GDN_E_NULL;
  return gdn::chunk_fwd(p, raw, q_raw, k_raw, v, gate_x, beta_logit, h0, cu_seqlens, o, hT, status, workspace,
                        workspace_bytes, stream);
}

gdn_status gdn_decode_step(const gdn_problem* p, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const float* h_in, void* o,
                           float* h_out, uint32_t* status, void* stream) {
  if (!p) return GDN_E_NULL;
  if (p->n_seq < 0 || p->hk < 1 || p->hv < 1 || p->seq_len != 1 || p->total_tokens != p->n_seq)
    return GDN_E_SHAPE;
  if (p->hv % p->hk != 0) return GDN_E_UNSUPPORTED;
  if (!(p->dk == 32 || p->dk == 64 || p->dk == 128)) return GDN_E_UNSUPPORTED;
  if (!(p->dv == 32 || p->dv == 64 || p->dv == 128)) return GDN_E_UNSUPPORTED;
  if (p->gate != GDN_GATE_HEAD && p->gate != GDN_GATE_KEY_CHANNEL) return GDN_E_UNSUPPORTED;
  if (p->qkv_dtype != GDN_BF16 && p->qkv_dtype != GDN_F32) return GDN_E_UNSUPPORTED;
  if (p->o_dtype != GDN_BF16 && p->o_dtype != GDN_F32) return GDN_E_UNSUPPORTED;
  if ((int64_t)p->n_seq * p->hv * (p->dv / 32) > INT32_MAX) return GDN_E_UNSUPPORTED;
  if (!status) return GDN_E_NULL;
  if (p->n_seq > 0 && (!q || !k || !v || !g || !beta || !o || !h_out)) return GDN_E_NULL;
  const bool qf = p->qkv_dtype == GDN_F32, of = p->o_dtype == GDN_F32;
  // vector accesses: 4 state columns (16 bytes), 4 v / o elements (8 or 16 bytes)
  if (!gdn::aligned(q, 4) || !gdn::aligned(k, 4) || !gdn::aligned(v, qf ? 16 : 8) ||
      !gdn::aligned(o, of ? 16 : 8) || !gdn::aligned(g, 4) || !gdn::aligned(beta, 4) ||
      !gdn::aligned(h_in, 16) || !gdn::aligned(h_out, 16) || !gdn::aligned(status, 4))
    return GDN_E_UNSUPPORTED;
  const size_t N = (size_t)p->n_seq, qsz = qf ? 4 : 2, osz = of ? 4 : 2;
  const size_t nq = N * p->hk * p->dk * qsz, nv = N * p->hv * p->dv * qsz;
  const size_t ng = N * p->hv * (p->gate == GDN_GATE_KEY_CHANNEL ? p->dk : 1) * 4, nb = N * p->hv * 4;
  const size_t nh = N * p->hv * p->dk * p->dv * 4, no = N * p->hv * p->dv * osz;
  struct R {
    const void* p;
    size_t n;
  };
  const R ins[] = {{q, nq}, {k, nq}, {v, nv}, {g, ng}, {beta, nb}, {h_in, nh}};
  const R outs[] = {{o, no}, {h_out, nh}, {status, 4}};
  for (const R& a : outs) {
    for (const R& b : ins)
      if (gdn::overlap(a.p, a.n, b.p, b.n)) return GDN_E_ALIAS;
    for (const R& b : outs)
      if (&a != &b && gdn::overlap(a.p, a.n, b.p, b.n)) return GDN_E_ALIAS;
  }
  if (p->n_seq == 0) return GDN_OK;
  gdn::DecodeParams prm;
  memset(&prm, 0, sizeof(prm));
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.g = g;
  prm.beta = beta;
  prm.h_in = h_in;
  prm.o = o;
  prm.h_out = h_out;
  prm.status = status;
  prm.n_seq = p->n_seq;
  prm.hk = p->hk;
  prm.hv = p->hv;
  prm.dv = p->dv;
  prm.qkv_f32 = qf;
  prm.o_f32 = of;
  return gdn::launch_decode(prm, p->dk, p->gate == GDN_GATE_KEY_CHANNEL, stream);
}

const char* gdn_error_string(int32_t code) {
  switch (code) {
    case GDN_OK: return "ok";
    case GDN_E_NULL: return "a required pointer is NULL";
    case GDN_E_SHAPE: return "sizes are negative or inconsistent";
    case GDN_E_UNSUPPORTED: return "outside the supported domain (widths, chunk, dtype, alignment)";
    case GDN_E_ALIAS: return "an output overlaps an input or another output";
    case GDN_E_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case GDN_E_LAUNCH: return "the HIP runtime refused a kernel launch";
    default: return "unknown error code";
  }
}

const char* gdn_status_string(uint32_t bits) {
  static thread_local std::string s;
  if (bits == 0) return "ok";
  s.clear();
  const struct {
    uint32_t bit;
    const char* name;
  } names[] = {{GDN_ST_NONFINITE_INPUT, "nonfinite-input"},
               {GDN_ST_GATE_DOMAIN, "gate-domain"},
               {GDN_ST_BAD_SEQLENS, "bad-seqlens"},
               {GDN_ST_NONFINITE_OUTPUT, "nonfinite-output"}};
  uint32_t rest = bits;
  for (auto& n : names) {
    if (bits & n.bit) {
      if (!s.empty()) s += "|";
      s += n.name;
      rest &= ~n.bit;
    }
  }
  if (rest) {
    char buf[32];
    snprintf(buf, sizeof(buf), "%sunknown(0x%x)", s.empty() ? "" : "|", rest);
    s += buf;
  }
  return s.c_str();
}

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

#ifdef GDN_SCAN_STAMPS
// Measurement build only (not part of the ABI in include/gdn.h): the following calls' scan
// workgroup `block` records, for kStampSteps chunk steps from chunk `c0`, a shader-clock
// timestamp at each phase boundary of its chain wave 0, output wave, loader wave and chain
// wave 1 into the device buffer `buf` ([4][kStampSteps][kStampPhases] uint64; NULL stops
// recording).
int32_t gdn_debug_stamps(void* buf, int32_t block, int32_t c0) {
  gdn::g_stamps = (uint64_t*)buf;
  gdn::g_stamp_block = block;
  gdn::g_stamp_c0 = c0;
  return gdn::kStampSteps * gdn::kStampPhases;
}
#endif

}  // extern "C"
