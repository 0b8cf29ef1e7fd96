/*
 * gdn.h -- C ABI of the MI355X (gfx950) chunk-parallel gated delta-rule prefill.
 *
 * The operation (per sequence n and value head h, tokens t in order; K-first
 * state H in R^{dk x dv}):
 *
 *     H_t = (I - beta_t k_t k_t^T) D_t H_{t-1} + beta_t k_t v_t^T,   o_t = H_t^T q_t
 *
 * with D_t = exp(g_t) I (per-head gate) or diag(exp(g_t[c])) (per-key-channel
 * gate), i.e. S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T with S = H^T.
 * It is the gated-delta-net recurrence of the stratat.com page "hip:
 * chunk-parallel GDN recurrence (WY form), two parity-gated arms" (section
 * "What this is"), evaluated chunkwise as that page and the ROCm/rocm-libraries
 * KDA chunkwise page (section "Summary") describe: per chunk one unit-lower-
 * triangular solve plus GEMM-shaped folds, then a serial state recurrence.
 * The argument contract (K-first state, precomputed beta and natural-log g,
 * explicit grouped heads, immutable h0, separate next state, sticky numerical
 * status, explicit refusal of unsupported inputs) follows the logismos issue
 * #46 page ("Verified implementation boundary", "Remaining work",
 * "Acceptance", and the Sep 6 / Sep 8 activity).
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers owned by the caller; the library
 *     allocates and frees nothing per call.  Its only state is set once per device and
 *     changes no result: which kernels have had their LDS size set, and the device
 *     address of gdn_chunk_fwd_noalloc's workspace array.
 *   - Tensors are dense, row-major, last dimension contiguous, no padding.
 *   - Host-detected errors return synchronously and launch nothing.
 *   - gdn_chunk_fwd and gdn_decode_step are asynchronous on `stream`; device-detected
 *     conditions are OR-ed into *status (sticky), which the caller reads after
 *     synchronising.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

/* Host return codes. */
typedef enum gdn_status {
  GDN_OK = 0,
  GDN_E_NULL = 1,        /* a required pointer is NULL */
  GDN_E_SHAPE = 2,       /* sizes negative or inconsistent */
  GDN_E_UNSUPPORTED = 3, /* outside the supported domain (widths, chunk, dtype, alignment) */
  GDN_E_ALIAS = 4,       /* an output overlaps an input or another output */
  GDN_E_WORKSPACE = 5,   /* workspace smaller than gdn_workspace_bytes() or misaligned */
  GDN_E_LAUNCH = 6       /* the HIP runtime refused a launch */
} gdn_status;

/* Device status bits, OR-accumulated into *status.  When any bit is set the
 * contents of o and hT are unspecified; inputs are never modified. */
#define GDN_ST_NONFINITE_INPUT 0x1u  /* NaN/Inf in q, k, v, g, beta or h0 */
#define GDN_ST_GATE_DOMAIN 0x2u      /* g > 0, or a per-channel gate below -5 */
#define GDN_ST_BAD_SEQLENS 0x4u      /* cu_seqlens not 0 = c_0 <= ... <= c_n = total_tokens */
#define GDN_ST_NONFINITE_OUTPUT 0x8u /* a NaN/Inf was produced in o or hT */

enum { GDN_GATE_HEAD = 0, GDN_GATE_KEY_CHANNEL = 1 };
enum { GDN_BF16 = 0, GDN_F32 = 1 };
/* Arithmetic arm: bf16 MFMA operands with fp32 accumulation, or fp32 MFMA
 * operands (the fp32-fold debug arm).  The state is fp32 in both. */
enum { GDN_ARM_MFMA_BF16 = 0, GDN_ARM_FOLD_F32 = 1 };
/* Kernel composition: split (a sequence-parallel prep kernel writes every chunk's T and
 * P to the workspace, then the scan reads them) or fused (two extra waves of each scan
 * workgroup form T and P a chunk ahead and hand them over in LDS; no tile round trip
 * through HBM, but the tiles are formed once per 32-column slice of the state), or
 * pipelined (split, with the scan cut into chunk-aligned segments that carry the state
 * through the workspace; the launch that scans segment s also runs the prep of segment
 * s + 1 in workgroups after the scan's own, on the compute units the scan leaves idle,
 * so only the first segment's prep is exposed).  All three give bit-identical results.
 * FUSED is built for the per-head gate with bf16 q/k/v on the bf16 arm; PIPELINED for
 * the per-head gate on fixed-length batches (GDN_E_UNSUPPORTED otherwise); neither has
 * separate stages.  AUTO picks the measured default, split or pipelined: pipelined where
 * it applies, the sequences are at least four segments (8,192 tokens) long and the scan
 * grid leaves at least a quarter of its own size idle on the device (gdn_plan_compose
 * reports the choice), else split. */
enum { GDN_COMPOSE_AUTO = 0, GDN_COMPOSE_SPLIT = 1, GDN_COMPOSE_FUSED = 2, GDN_COMPOSE_PIPELINED = 3,
       GDN_COMPOSE_SEQSPLIT = 4 };
/* GDN_COMPOSE_SEQSPLIT, for head-starved shapes (few sequences x heads): each sequence is
 * cut into 2..4 parts scanned side by side.  Every part scans from zero to its local final
 * state; each inner part also scans its transition (the product of its chunk maps, a
 * dk x dk state scanned from the identity with V read as zero); a small kernel chains the
 * parts' starting states in fp32; the parts after the first then rescan from them with
 * outputs.  About 1.7x the scan work in two rounds of a part's length instead of one
 * round of the sequence's.  Per-head gate, fixed-length batches, dk == dv, all stages.
 * Results equal the other compositions' up to rounding (not bit for bit).  Only on
 * request: AUTO never picks it (on MI355X it measured slower than split on the
 * head-starved single-sequence layer it is meant for). */
/* Stages of the split composition a call runs.  0 (or PREP|SCAN) runs both.  A
 * SCAN-only call consumes the chunk tiles a previous PREP call (same problem, same
 * inputs, same workspace) left in the workspace; the caller orders the two calls,
 * e.g. on one stream.  This lets the sequence-parallel tile stage of a layer run
 * ahead of its scan, and lets each stage be timed on its own. */
enum { GDN_STAGE_ALL = 0, GDN_STAGE_PREP = 1, GDN_STAGE_SCAN = 2 };

typedef struct gdn_problem {
  int32_t n_seq;        /* number of sequences, >= 0 */
  int64_t total_tokens; /* packed token count, >= 0; with cu_seqlens at most 2^31 - 65 */
  int32_t seq_len;      /* fixed-length batches: tokens per sequence (total = n_seq*seq_len);
                           0 when cu_seqlens describes the sequences */
  int32_t hk;           /* key/query heads, >= 1 */
  int32_t hv;           /* value heads, a multiple of hk; value head j reads key head j/(hv/hk) */
  int32_t dk;           /* key width: 32, 64 or 128 */
  int32_t dv;           /* value width: 32, 64 or 128 */
  int32_t gate;         /* GDN_GATE_HEAD: g[tok][hv];  GDN_GATE_KEY_CHANNEL: g[tok][hv][dk] */
  int32_t chunk;        /* 0 = library choice, else 32 or 64 (per-channel gate: 32 only) */
  int32_t qkv_dtype;    /* GDN_BF16 or GDN_F32 for q, k, v */
  int32_t o_dtype;      /* GDN_BF16 or GDN_F32 for o */
  int32_t arm;          /* GDN_ARM_MFMA_BF16 or GDN_ARM_FOLD_F32 */
  int32_t compose;      /* GDN_COMPOSE_* */
  int32_t stages;       /* GDN_STAGE_ALL, or PREP / SCAN alone (split composition) */
  int32_t solve_block;  /* rows of the diagonal blocks of the triangular solve T = (I + A)^-1:
                           0 = library choice (16), else 8, 16 or 32.  Each diagonal block is
                           solved by scalar forward substitution, the blocks below it by fp32
                           MFMA updates against solved blocks; the substitution's work grows
                           with the block's square, the update steps with the block count (the
                           rocm-libraries pull 11223 page, section "Levers", item 3).  Results
                           differ between block sizes by rounding only. */
} gdn_problem;

/* gdn_validate -- checks a problem description on the host (no device work): every
 * size, width, dtype, gate form, chunk and composition must lie in the supported domain,
 * and anything else is refused with a typed code rather than computed (the logismos issue
 * #46 page: unsupported inputs fail explicitly, section "Acceptance"; grouped-head
 * mapping, initial/final state, chunk boundaries, input domains and precision kept
 * explicit, section "Remaining work").
 *   p  the problem; read only
 * Returns GDN_OK, GDN_E_NULL (p is NULL), GDN_E_SHAPE (negative or inconsistent sizes,
 * tokens with no sequence) or GDN_E_UNSUPPORTED (outside the domain, including a
 * solve_block other than 0, 8, 16 or 32, and a solve_block other than 16 requested with
 * the fused or pipelined composition, whose in-scan tile stages solve with 16 rows). */
gdn_status gdn_validate(const gdn_problem* p);

/* gdn_workspace_bytes -- bytes of device workspace gdn_chunk_fwd needs for *p, written to
 * *bytes.  The workspace holds the state-independent per-chunk tiles of the chunk form (T
 * and P of every chunk: the stratat.com page, section "What this is", one unit-lower-
 * triangular solve per chunk; the ROCm/rocm-libraries KDA chunkwise page, sections
 * "Summary" and "Levers": tiles formed sequence-parallel, then a serial scan, with a tile
 * round trip through HBM), plus the composition's own buffers (the state carried between
 * pipelined segments; a pipelined request keeps only two segments of tiles).  Host-only.
 *   p      the problem; read only
 *   bytes  out: the size (0 when nothing is needed); NULL is refused
 * Same return codes as gdn_validate, plus GDN_E_NULL for a NULL `bytes`. */
gdn_status gdn_workspace_bytes(const gdn_problem* p, size_t* bytes);

/* gdn_plan_compose -- the composition gdn_chunk_fwd runs for *p on the current device,
 * written to *compose (GDN_COMPOSE_SPLIT, _FUSED, _PIPELINED or _SEQSPLIT): the requested
 * one, or for GDN_COMPOSE_AUTO the library's measured choice, which depends on the
 * device's compute-unit count (split versus fused is a measured choice on the
 * ROCm/rocm-libraries KDA chunkwise page, sections "Levers" and "The interesting result
 * is a negative one").  Host-only: a device attribute query, no device work.
 *   p        the problem; read only
 *   compose  out; NULL is refused with GDN_E_NULL
 * Same return codes as gdn_validate. */
gdn_status gdn_plan_compose(const gdn_problem* p, int32_t* compose);

/*
 * gdn_chunk_fwd -- chunkwise gated delta-rule prefill: the rule above for every sequence
 * and value head, evaluated per chunk by a unit-lower-triangular solve and GEMM-shaped
 * folds (the stratat.com page, section "What this is") and a serial scan of the state over
 * the chunks (the ROCm/rocm-libraries KDA chunkwise page, section "Summary"), under the
 * argument contract of the logismos issue #46 page (Sep 6 / Sep 8 activity: K-first
 * state, precomputed beta and natural-log g, grouped heads, immutable h0, separate final
 * state; "Verified implementation boundary": sticky numerical status).
 *   q, k        [total_tokens][hk][dk]   qkv_dtype, 16-byte aligned
 *   v           [total_tokens][hv][dv]   qkv_dtype, 16-byte aligned
 *   g           fp32 natural-log decay, [total_tokens][hv] or [total_tokens][hv][dk];
 *               a per-head gate has no lower limit: at or below -200 a token resets the
 *               state (every decay across it is below fp32's resolution and is taken as
 *               exactly zero), and the in-chunk sums are formed in fp64, so the arm's
 *               accuracy holds however large the gates
 *   beta        fp32 [total_tokens][hv]
 *   h0          fp32 [n_seq][hv][dk][dv] initial states, or NULL for zeros; never written
 *   cu_seqlens  int32 [n_seq+1] token offsets (0, ..., total_tokens), or NULL for a
 *               fixed-length batch of n_seq sequences of seq_len tokens; a sequence's
 *               state starts at its own h0 and chunks never cross a boundary
 *   o           [total_tokens][hv][dv] o_dtype, 16-byte aligned
 *   hT          fp32 [n_seq][hv][dk][dv] final states, or NULL; must not overlap h0
 *   status      one uint32 on the device, zeroed by the caller; device bits OR-ed in
 *   workspace   device scratch of at least gdn_workspace_bytes() bytes, 256-byte aligned;
 *               its contents are undefined before and after the call
 *   stream      a hipStream_t (NULL = the default stream)
 * Returns GDN_OK after enqueueing every kernel, or a host error with nothing launched.
 */
gdn_status gdn_chunk_fwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* h0,
                         const int32_t* cu_seqlens, void* o, float* hT, uint32_t* status,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_fwd_raw_inputs -- gdn_chunk_fwd from the raw per-token values next to the
 * recurrence, which the generic operation takes prepared (the logismos issue #46 page,
 * section "Remaining work": model-specific gating composed separately from the generic
 * operation contract).  Each (token, head) row of q and k is divided by its L2 norm (a zero
 * row stays zero) and q is then multiplied by q_scale; beta = sigmoid(logit); the
 * natural-log decay is g = -gate_scale softplus(x) = -gate_scale log(1 + e^x).  These are
 * the forms of the single-sequence, hybrid and packed workloads of the problem statement
 * (q, k L2-normalised with q scaled by dk^-1/2, beta = sigmoid(N(0,1)), g = -a softplus(N(0,1))
 * with a = 1/2 or 1).  Nothing is materialised: the prep kernel takes the row norms from the
 * rows it loads anyway and folds them into its K K^T and Q K^T tiles, and the scan folds
 * them into the per-row factors it already applies, so q and k are read as often as by
 * gdn_chunk_fwd.
 *   raw          q_scale > 0 and gate_scale > 0, both finite (else GDN_E_UNSUPPORTED); NULL is
 *                refused with GDN_E_NULL
 *   q_raw, k_raw [total_tokens][hk][dk] raw rows, qkv_dtype
 *   gate_x       fp32 [total_tokens][hv] raw gate values (per-head gate only)
 *   beta_logit   fp32 [total_tokens][hv]
 *   workspace    at least gdn_raw_workspace_bytes() bytes (the row norms, 8 bytes per token
 *                and key head, on top of gdn_workspace_bytes())
 *   the rest     as for gdn_chunk_fwd
 * Status bits: NONFINITE_INPUT for Inf/NaN in any raw value; GATE_DOMAIN cannot occur.
 * Returns the codes of gdn_chunk_fwd; GDN_E_UNSUPPORTED also for the per-key-channel gate or
 * the fused composition.
 */
typedef struct gdn_raw_inputs {
  float q_scale;    /* q rows are multiplied by this after normalisation (e.g. dk^-1/2) */
  float gate_scale; /* a in g = -a softplus(x) */
} gdn_raw_inputs;

/* gdn_raw_workspace_bytes -- bytes of workspace gdn_chunk_fwd_raw_inputs needs for *p
 * (written to *bytes): gdn_workspace_bytes plus the row norms.  Host-only; the codes of
 * gdn_workspace_bytes, and GDN_E_UNSUPPORTED where raw inputs are not supported. */
gdn_status gdn_raw_workspace_bytes(const gdn_problem* p, size_t* bytes);

gdn_status gdn_chunk_fwd_raw_inputs(const gdn_problem* p, const gdn_raw_inputs* raw, const void* q_raw,
                                    const void* k_raw, const void* v, const float* gate_x,
                                    const float* beta_logit, const float* h0, const int32_t* cu_seqlens,
                                    void* o, float* hT, uint32_t* status, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_fwd_noalloc -- gdn_chunk_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The same computation, kernels and launches as gdn_chunk_fwd with the composition
 * gdn_plan_compose reports, but with no workspace argument: the workspace is the
 * library's own array of GDN_NOALLOC_WORKSPACE_BYTES on each device, which the first
 * call on a device looks up (no allocation) and which that device holds until the process
 * ends.  Nothing is allocated or freed by any call.
 *   p, q ... status, stream   as for gdn_chunk_fwd
 * Every call on one device uses that device's one array: calls that overlap in time on a
 * device (different streams or host threads) race and must be ordered by the caller.  The
 * array keeps whatever the last call left; nothing in it needs clearing.
 * Returns the codes of gdn_chunk_fwd, and GDN_E_WORKSPACE (nothing launched) when the
 * problem's workspace (gdn_workspace_bytes of the resolved composition) exceeds
 * GDN_NOALLOC_WORKSPACE_BYTES: e.g. the 32,768-token, 48-value-head layer pipelined needs
 * about 39 MiB and fits; a 131,072-token packed batch does not.
 */
#define GDN_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_problem* p, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* h0,
                                 const int32_t* cu_seqlens, void* o, float* hT, uint32_t* status,
                                 void* stream);

/*
 * gdn_decode_step -- one recurrent step: one new token for each of n_seq sequences,
 * continuing from their states (the hT of a prefill, or the h_out of an earlier step).
 * It is the same rule as above for a single token, evaluated directly:
 *     H_out = D H_in + k (beta (v - (D H_in)^T k))^T,   o = H_out^T q
 * (the stratat.com page, section "What this is", at T = 1; the K-first immutable input
 * state and separate next state follow the logismos issue #46 page, "Verified
 * implementation boundary" and the Sep 8 activity).  Every step runs in fp32.
 *   p           n_seq sequences, seq_len == 1, total_tokens == n_seq; hk, hv, dk, dv,
 *               gate, qkv_dtype and o_dtype as for gdn_chunk_fwd; chunk, arm, compose
 *               and stages are not read
 *   q, k        [n_seq][hk][dk]   qkv_dtype, 4-byte aligned
 *   v           [n_seq][hv][dv]   qkv_dtype, 16-byte (fp32) / 8-byte (bf16) aligned
 *   g           fp32 natural-log decay, [n_seq][hv] or [n_seq][hv][dk]
 *   beta        fp32 [n_seq][hv]
 *   h_in        fp32 [n_seq][hv][dk][dv] states before the token, or NULL for zeros;
 *               never written; 16-byte aligned
 *   o           [n_seq][hv][dv] o_dtype, aligned as v
 *   h_out       fp32 [n_seq][hv][dk][dv] states after the token, 16-byte aligned; must
 *               not overlap h_in (or any other argument)
 *   status      one uint32 on the device, zeroed by the caller; device bits OR-ed in:
 *               NONFINITE_INPUT (q, k, v, g, beta, h_in), GATE_DOMAIN (g > 0; a
 *               single step has no lower limit on a per-channel gate), NONFINITE_OUTPUT
 *   stream      a hipStream_t (NULL = the default stream)
 * No workspace.  Returns GDN_OK after enqueueing one kernel, or a host error
 * (GDN_E_NULL, GDN_E_SHAPE, GDN_E_UNSUPPORTED, GDN_E_ALIAS, GDN_E_LAUNCH) with nothing
 * launched.
 */
gdn_status gdn_decode_step(const gdn_problem* p, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const float* h_in, void* o,
                           float* h_out, uint32_t* status, void* stream);

/* gdn_error_string -- static text naming a host return code (the explicit refusals of the
 * logismos issue #46 page, section "Acceptance"); "unknown error code" for any other
 * value.  Never NULL; the caller does not free it. */
const char* gdn_error_string(int32_t code);

/* gdn_status_string -- text naming the device status bits set in `bits` ("ok" when none,
 * "|"-separated names, "unknown(0x..)" for bits the library does not define): the sticky
 * numerical status of the logismos issue #46 page ("Verified implementation boundary",
 * nonfinite inputs and results classified before anything is published).  The returned
 * pointer refers to thread-local storage, valid until this thread's next call. */
const char* gdn_status_string(uint32_t bits);

/* gdn_abi_version -- GDN_ABI_VERSION of the loaded library (library bookkeeping, no page
 * defines it): a caller built against this header checks it before the first call. */
int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
