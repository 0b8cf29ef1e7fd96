/*
 * gdn_oracle.h -- fp64 token-serial CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library under
 * linear_attention_rnn_chunk_amd/csrc, and the HIP library never calls it.
 *
 * What it computes (per sequence n and value head h, tokens t in order):
 *   the gated delta rule as stated on the stratat.com page "hip: chunk-parallel
 *   GDN recurrence (WY form)" (section "What this is": a serial token chain per
 *   head) and on the ROCm/rocm-libraries KDA chunkwise page (section
 *   "Correctness": the token-serial oracle walks the rule one token at a time
 *   and never chunks), in the K-first state orientation of the logismos
 *   issue #46 page (activity of Sep 6: "K-first state with precomputed
 *   beta/g and explicit grouped-head mapping"; Sep 8: natural-log decay,
 *   immutable input state, separate next state):
 *
 *     H   <- D_t H                      D_t = exp(g_t) (scalar) or diag(exp(g_t[c]))
 *     u   <- beta_t (v_t - H^T k_t)
 *     H   <- H + k_t u^T
 *     o_t <- H^T q_t
 *
 *   which is S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t
 *   with S = H^T.  No chunking, no blocking, no reordering of those steps.
 *
 * Precision: every input is read as double and all arithmetic is fp64.
 * Parity status: pinned (see tests/test_oracle_pins.py).
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Planted-mistake switch, used only by tests that show the pins catch a wrong
 * oracle.  0 is the correct rule; every other value is a deliberate bug. */
enum {
  GDN_ORACLE_CORRECT = 0,
  GDN_ORACLE_MUT_DECAY_AFTER_WRITE = 1, /* decays the new write as well */
  GDN_ORACLE_MUT_NO_BETA_ERASE = 2,     /* u = beta v - H^T k (beta missing on erase) */
  GDN_ORACLE_MUT_TRANSPOSED_READ = 3,   /* o = H q (row/column swapped; dk == dv only) */
  GDN_ORACLE_MUT_GATE_NEXT_TOKEN = 4,   /* decays token t with g_{t+1} */
  GDN_ORACLE_MUT_OUTPUT_BEFORE_WRITE = 5 /* o_t read before the write of token t */
};

/*
 * gdn_oracle_fwd
 *   n_seq        number of sequences
 *   seq_start    [n_seq+1] token offsets into the packed token axis (non-decreasing)
 *   hk, hv       key/query heads and value heads
 *   head_map     [hv] key head read by each value head, or NULL for the
 *                contiguous grouping  key head = h / (hv / hk)
 *   dk, dv       key and value widths
 *   per_channel  0: g is [tok][hv]; 1: g is [tok][hv][dk]
 *   q, k         [tok][hk][dk]
 *   v            [tok][hv][dv]
 *   g            natural-log decay, layout per per_channel
 *   beta         [tok][hv]
 *   h0           [n_seq][hv][dk][dv] or NULL (zeros); never written
 *   o            [tok][hv][dv] or NULL
 *   hT           [n_seq][hv][dk][dv] or NULL
 *   units        optional list of (seq, head) pairs to evaluate, as
 *                n_units pairs {seq, head}; NULL means every pair.  Rows of o
 *                and hT of pairs not listed are left untouched.
 *   n_threads    OpenMP threads (<= 0: library default)
 *   mutant       GDN_ORACLE_CORRECT except in planted-mistake tests
 * Returns 0 on success, a negative number on invalid arguments.
 */
int gdn_oracle_fwd(int n_seq, const int64_t* seq_start, int hk, int hv, const int32_t* head_map,
                   int dk, int dv, int per_channel, const double* q, const double* k, const double* v,
                   const double* g, const double* beta, const double* h0, double* o, double* hT,
                   const int32_t* units, int n_units, int n_threads, int mutant);

/* Threads the OpenMP runtime would use by default (for reporting). */
int gdn_oracle_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
