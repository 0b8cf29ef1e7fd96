// gdn_internal.h -- plan and kernel parameters shared by gdn_api.cpp and gdn_kernels.hip.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

// T and P of a chunk are stored as the scan's MFMA operand fragments: fragment (mt, sb)
// of a C x C lower-triangular tile covers rows 16 mt .. 16 mt + 15 and columns
// 32 sb .. 32 sb + 31, 64 lanes x 8 elements; only those with sb <= mt / 2 (touching
// the lower triangle) exist, in this order.
constexpr int tile_frag_index(int mt, int sb) {
  int f = 0;
  for (int m = 0; m < mt; ++m) f += (m >> 1) + 1;
  return f + sb;
}
constexpr int tile_frags(int C) { return tile_frag_index(C / 16, 0); }
constexpr int tile_elems(int C) { return tile_frags(C) * 512; }

// Most parts the sequence-split composition cuts a sequence into.
constexpr int kMaxParts = 4;

// Pipelined composition: the scan runs in chunk-aligned segments of this many tokens (the
// last one may be shorter); on the hybrid layer (32,768 tokens, chunk 64) 16 segments of
// 32 chunks measured 0.748 ms, against 0.844 with 8, 0.790 with 12, 0.826 with 32 and 0.922
// for the split composition.  Only two segments' tiles are live at a time (the one being
// scanned, the next one being prepared), so their workspace holds a ring of two segments.
constexpr int kSegTokens = 2048;

// Rows of the triangular solve's diagonal blocks when the problem leaves it to the library.
constexpr int kSolveBlock = 16;

// Everything a launch needs, resolved on the host from a gdn_problem.
struct Plan {
  int32_t n_seq, seq_len, hk, hv, dk, dv;
  int64_t total;
  int32_t gate_channel;  // 1: per-key-channel gate
  int32_t chunk;         // 32 or 64
  int32_t arm_f32;       // 1: fp32-fold arm
  int32_t qkv_f32, o_f32;
  int32_t fused;         // 1: fused composition
  int32_t pipe_ok;       // pipelined composition possible and not excluded by the request
                         // (per-head gate, fixed length, all stages, AUTO or PIPELINED)
  int32_t pipe_req;      // 1: pipelined requested, 0: split requested, -1: library choice
  int32_t seq_ok;        // sequence-split composition requested and possible
                         // (per-head gate, fixed length, dk == dv, all stages)
  int32_t seq_req;       // 1: sequence split requested, 0: not
  int32_t run_prep, run_scan;  // stages to launch
  int32_t varlen;        // 1: cu_seqlens given
  int32_t chunks_per_seq;  // fixed-length batches
  int64_t max_slots;     // chunk slots the prep grid covers
  int32_t tile_ring;     // chunks per ring half of the tile buffers (pipelined composition on
                         // sequences longer than two segments), else 0: every chunk its own slot
  int64_t tile_slots;    // chunk slots the tile buffers hold
  int32_t raw;           // 1: raw inputs (gdn_chunk_fwd_raw_inputs)
  int32_t solve_block;   // rows of the triangular solve's diagonal blocks: 8, 16 or 32
  // workspace carve-up (byte offsets)
  int32_t kq_ws;         // 1: K and Q copied to the workspace in the arm's type
  size_t off_table, off_T, off_P, off_G, off_D, off_K, off_Q, off_carry, off_parts, off_N, bytes;
};

// Kernel arguments (by value).
struct Params {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* h0;
  const int32_t* cu_seqlens;
  void* o;
  float* hT;
  uint32_t* status;
  int32_t* table;  // varlen: [n_seq+1] sanitised bounds, [n_seq+1] chunk prefix, then
                   // [n_seq] the scan's dispatch order (longest sequences first)
  void* Tws;       // [slot][hv][tile_elems(C)] solved T fragments (arm element type)
  void* Pws;       // [slot][hv][tile_elems(C)] masked P fragments (arm element type)
  void* Gws;       // per-channel gate: [slot][hv][3][C][dk] e^{G} K, e^{G_C-G} K, e^{G} Q
  float* Dws;      // per-channel gate: [slot][hv][dk] e^{G_C}
  void* Kws;       // kq_ws: [slot][hk][C][dk] K in the arm's element type
  void* Qws;       // kq_ws: [slot][hk][C][dk] Q in the arm's element type
  int64_t total;
  int32_t n_seq, seq_len, hk, hv, dv;
  int32_t qkv_f32, o_f32, varlen, chunks_per_seq, kq_ws;
  int64_t max_slots;
  // Tile buffers (T, P, and K / Q in the arm's type) as a ring of two segments per
  // sequence: chunk c of sequence n lives in slot n * 2 tile_ring + c mod (2 tile_ring).
  // 0: chunk slot s lives in slot s.  Set only for pipelined launches, each of whose scan
  // ranges lies inside one segment.
  int32_t tile_ring;
  // Chunk ranges of one launch (fixed-length batches; the whole sequence otherwise):
  // the scan walks chunks [seg_cb, seg_ce) of every sequence starting from h0 (checked
  // for Inf/NaN only when h0_input) and ends with hT; the prep covers chunks
  // [prep_cb, prep_ce).  Scan workgroups are blockIdx < nscan; in the pipelined
  // composition the workgroups after them run the prep of the next segment.
  int32_t seg_cb, seg_ce, prep_cb, prep_ce, nscan, h0_input;
  // Sequence-split composition (fixed-length batches, dk == dv).  pmode 0: off.  Else each
  // sequence is cut into nparts parts of part_chunks chunks, and the launch's "sequences"
  // are pvirt virtual ones per real sequence.  pmode 1: virtual v < nparts scans part v from
  // h0 (v = 0) or zero, writes its outputs and leaves its state in Bws; v >= nparts scans
  // part v - nparts + 1 from the identity with V read as zero and no outputs, leaving the
  // part's transition in Mws.  pmode 2: virtual v scans part v + 1 from Hws, writes its
  // outputs, and the last part writes hT; part 1 starts from Bws part 0, later parts from
  // Hws.  Bws, Mws, Hws: [n_seq][nparts][hv][dk][dv] fp32.
  int32_t pmode, nparts, pvirt, part_chunks;
  float* Bws;
  float* Mws;
  float* Hws;
  // Step timestamps of one scan workgroup, recorded only by a library built with
  // GDN_SCAN_STAMPS (a measurement build): [4 roles: chain wave 0, output, loader, chain wave 1]
  // [kStampSteps steps from chunk stamp_c0][kStampPhases] shader-clock counts.
  uint64_t* stamps;
  int32_t stamp_block, stamp_c0;
  // Raw inputs: q, k are raw rows (normalised per (token, head) inside, q then scaled by
  // q_scale), beta holds logits (beta = sigmoid), g raw values (g = -gate_scale softplus).
  // Nws: [tile slot][hk][2][C] fp32, 1 / |k_r| then q_scale / |q_r|, from the prep.
  int32_t raw;
  float q_scale, gate_scale;
  float* Nws;
  // Rows of the diagonal blocks of the triangular solve T = (I + A)^-1: 8, 16 or 32.
  int32_t solve_block;
};
constexpr int kStampSteps = 16, kStampPhases = 8;

// Arguments of the one-token recurrent step (by value).
struct DecodeParams {
  const void* q;      // [n_seq][hk][dk]
  const void* k;      // [n_seq][hk][dk]
  const void* v;      // [n_seq][hv][dv]
  const float* g;     // [n_seq][hv] or [n_seq][hv][dk]
  const float* beta;  // [n_seq][hv]
  const float* h_in;  // [n_seq][hv][dk][dv] or null (zeros)
  void* o;            // [n_seq][hv][dv]
  float* h_out;       // [n_seq][hv][dk][dv]
  uint32_t* status;
  int32_t n_seq, hk, hv, dv;
  int32_t qkv_f32, o_f32;
};

gdn_status make_plan(const gdn_problem* p, Plan* plan, bool raw = false);
gdn_status launch_decode(const DecodeParams& prm, int dk, bool per_channel_gate, void* stream);
gdn_status launch(const Plan& plan, const Params& prm, void* carry, void* stream);
// the composition launch() runs for this plan on the current device (GDN_COMPOSE_*)
int32_t plan_compose(const Plan& plan);

}  // namespace gdn
