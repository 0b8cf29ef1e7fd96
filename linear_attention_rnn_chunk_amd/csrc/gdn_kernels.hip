// gdn_kernels.hip -- gfx950 (CDNA4) kernels of the chunk-parallel gated delta rule.
//
// Chunk (WY) form of the rule H_t = (I - b_t k_t k_t^T) D_t H_{t-1} + b_t k_t v_t^T,
// o_t = H_t^T q_t (stratat.com "hip: chunk-parallel GDN recurrence (WY form)",
// section "What this is"; ROCm/rocm-libraries KDA chunkwise pull request, section
// "Summary": state-independent per-chunk tiles plus a serial state recurrence).
// For a chunk of C rows entering with state H0 and in-chunk cumulative gate G:
//
//   A = tril_strict(beta * exp(G_r - G_s) * (k_r . k_s))     T = (I + A)^-1
//   P = tril(exp(G_r - G_s) * (q_r . k_s))
//   X = beta V - beta (K * exp(G)) H0        R = T X          (true per-token deltas)
//   O = (Q * exp(G)) H0 + P R                H = exp(G_C) H0 + Ktil^T R,
//   Ktil_s = k_s * exp(G_C - G_s)
//
// (per key channel for the per-channel gate, where the exp factors sit inside
// the contractions).  Under the per-head gate every factor comes from an fp64 in-chunk
// prefix in which a reset token (gate at most -200) counts as -2^20, so that every factor
// across one is zero (gate_prefix).  Kernels:
//   gdn_chunk_table  one block: sanitised cu_seqlens bounds + per-sequence chunk prefix
//   gdn_prep_head    per-head gate: one workgroup per (chunk, key head), one wave per
//                    value head of the group; fully sequence-parallel: gate sweep, K K^T
//                    and Q K^T on MFMA, blocked unit-lower-triangular solve (diagonal
//                    blocks of 8, 16 or 32 rows); writes T and P of each value head
//   gdn_prep_chan    per-key-channel gate: one workgroup per (chunk, value head); also
//                    writes the gated operands e^G K, e^{G_C-G} K, e^G Q and e^{G_C}
//   gdn_scan         one workgroup per (sequence, value head, 32 or 64 state columns),
//                    chain waves of 16 or 32 columns; fp32 state lives in MFMA
//                    accumulators and never leaves registers; walks the chunks
//                    serially.  Raw inputs (row norms, beta and g formed from their raw
//                    values) fold into the prep's tiles and the scan's per-row
//                    scalars; nothing extra is materialised.  It also runs
//                    any chunk range of each sequence from and to given state buffers
//                    (the pipelined composition's segments, whose launches run the next
//                    segment's prep in workgroups after the scan's own) and the parts of
//                    the sequence-split composition (own state, transition, rescan)
//   gdn_seq_chain    sequence split: one fp32 step of the chain of the parts' states
//
// MFMA fragment convention (16x16 tiles, K = 32 per fragment): lane l holds column
// (or row) l%16 and, with g = l/16, the contraction positions {4g..4g+3} and
// {16+4g..16+4g+3}.  An accumulator tile holds D[4g+i][l%16], so two stacked
// accumulator tiles ARE a B-operand fragment (and, transposed, an A-operand
// fragment) with no data movement -- the state and the deltas go from one matrix
// product to the next in registers.  The hardware pairs A and B by (lane group,
// element), so any fixed assignment of contraction positions is valid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;  // native vector (registers, not a struct)
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

extern __shared__ __align__(16) unsigned char gdn_smem[];

constexpr float kLog2e = 1.4426950408889634f;

// e^x through the hardware exp2 (v_exp_f32); e^-inf = 0, large negative x flush to 0.
__device__ __forceinline__ float nexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// The input side from raw per-token values (the gdn_chunk_fwd_raw_inputs entry point):
// beta = sigmoid(logit) and g = -a softplus(x) = -a (max(x, 0) + log(1 + e^-|x|)), through
// the hardware exp2 / log2 (v_exp_f32, v_log_f32) with no overflow for any finite input.
constexpr float kLn2 = 0.69314718055994531f;
__device__ __forceinline__ float sigmoid_f(float x) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);  // e^-|x|, in (0, 1]
  const float r = 1.f / (1.f + e);
  return x >= 0.f ? r : e * r;
}
__device__ __forceinline__ float neg_softplus(float x, float a) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  return -a * (fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * kLn2);
}

__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
// Inf/NaN tests as bit arithmetic: no short-circuit branches, so loads around them
// can still be issued back to back.
__device__ __forceinline__ uint32_t nf_f32(uint32_t u) { return (u & 0x7F800000u) == 0x7F800000u; }
__device__ __forceinline__ uint32_t nf_bf16x2(uint32_t two) {  // either half is Inf/NaN
  return (uint32_t)((two & 0x7F80u) == 0x7F80u) | (uint32_t)((two & 0x7F800000u) == 0x7F800000u);
}
__device__ __forceinline__ uint32_t f_nonfinite(float x) { return nf_f32(__float_as_uint(x)); }
// Inf/NaN accumulation for raw 16-byte input pieces: the returned word has bit 15 or 31
// (bf16) / bit 31 (fp32) set when some element's exponent field is all ones (adding one
// unit to a saturated exponent field carries into the bit above it).
template <bool QF32>
__device__ __forceinline__ uint32_t nf_bits16(u32x4 a) {
  if constexpr (QF32) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m |= (a[j] & 0x7F800000u) + 0x00800000u;  // bit 31
    return m & 0x80000000u;
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m |= (a[j] & 0x7F807F80u) + 0x00800080u;  // bits 15, 31
    return m & 0x80008000u;
  }
}
// `flag` when `c` is nonzero, else 0
__device__ __forceinline__ uint32_t flag_if(uint32_t c, uint32_t flag) { return c ? flag : 0u; }

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ f32x4 zero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }

// four fp32 values as four consecutive bf16 (round to nearest even)
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
__device__ __forceinline__ uint2 pack_bf16x4(f32x4 v) {
  bf16x4_t b;
  b[0] = (__bf16)v[0];
  b[1] = (__bf16)v[1];
  b[2] = (__bf16)v[2];
  b[3] = (__bf16)v[3];
  return __builtin_bit_cast(uint2, b);
}

// The per-head gate's in-chunk prefix, lane = token, for the factors e^{G_r - G_s} of the
// tiles and e^{G}, e^{G_C - G}, e^{G_C} of the scan.  Two things keep those exact to fp32
// however large the chunk's gates:
//  - A token whose gate is at most kResetGate is a reset: e^{-200} times any finite fp32
//    operand is below half of fp32's smallest subnormal, so every factor across such a
//    token is exactly zero.  Its gate enters the prefix as -2^20 (kResetSum), which makes
//    every such factor e^{-2^20 + ...} = 0 and keeps the sums small enough for fp64 to
//    add the other gates exactly (to about 1e-8 after 64 resets).
//  - The prefix is summed in fp64, so a chunk whose gates add up to thousands still gives
//    the small difference of two of its sums exactly (an fp32 prefix of -1e4 has a grid
//    of 1e-3).
// Inclusive prefix over the 64 lanes with DPP lane moves (no LDS round trips): shifts by
// 1, 2, 4, 8 within each row of 16 lanes, then row 0's (row 2's) last lane is added to
// row 1 (row 3), then lane 31 to rows 2 and 3.  Lanes a move has no source for add 0
// (bound_ctrl), rows outside a move's row mask keep adding 0.
constexpr float kResetGate = -200.f;
constexpr double kResetSum = -1048576.0;
__device__ __forceinline__ double gate_prefix(float x) {
  using std::integral_constant;
  auto mv = [](int v, auto CTRL, auto ROWS) __attribute__((always_inline)) {
    return __builtin_amdgcn_update_dpp(0, v, decltype(CTRL)::value, decltype(ROWS)::value, 0xf, true);
  };
  double s = x <= kResetGate ? kResetSum : (double)x;
  auto step = [&](auto CTRL, auto ROWS) __attribute__((always_inline)) {
    const int lo = mv(__double2loint(s), CTRL, ROWS), hi = mv(__double2hiint(s), CTRL, ROWS);
    s = __hiloint2double(hi, lo) + s;
  };
  step(integral_constant<int, 0x111>{}, integral_constant<int, 0xf>{});  // row_shr:1
  step(integral_constant<int, 0x112>{}, integral_constant<int, 0xf>{});  // row_shr:2
  step(integral_constant<int, 0x114>{}, integral_constant<int, 0xf>{});  // row_shr:4
  step(integral_constant<int, 0x118>{}, integral_constant<int, 0xf>{});  // row_shr:8
  step(integral_constant<int, 0x142>{}, integral_constant<int, 0xa>{});  // row_bcast:15
  step(integral_constant<int, 0x143>{}, integral_constant<int, 0xc>{});  // row_bcast:31
  return s;
}

// ---------------------------------------------------------------- arms ----
// bf16 MFMA operands (v_mfma_f32_16x16x32_bf16), fp32 accumulation.
struct ArmBF16 {
  typedef uint16_t T;
  typedef bf16x8_t F;
  static constexpr int PAD = 8;  // LDS row padding (elements): 16 bytes
  __device__ static __forceinline__ T cvt(float x) { return f2bf(x); }
  __device__ static __forceinline__ float val(T x) { return bf2f(x); }
  __device__ static __forceinline__ F pack(uint2 a, uint2 b) {
    const uint4 u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(F, u);
  }
  // A (or B^T) fragment from a row-major LDS matrix: 4 elements at p0, 4 at p1.
  __device__ static __forceinline__ F row(const T* p0, const T* p1) {
    return pack(*(const uint2*)p0, *(const uint2*)p1);
  }
  // Fragment whose contraction runs down the rows of a row-major LDS matrix:
  // lane (i = l%16, g) gets base[(k0+4g+j)*pitch + n0+i] and base[(k0+16+4g+j)*pitch + n0+i].
  // ds_read_b64_tr_b16: within 16 lanes, lane i receives element i%4 of the 8-byte rows
  // addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
  __device__ static __forceinline__ F col(const T* base, int pitch, int k0, int n0, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const T* a0 = base + (k0 + 4 * g + (i >> 2)) * pitch + n0 + 4 * (i & 3);
    const T* a1 = a0 + 16 * pitch;
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a1));
    return pack(__builtin_bit_cast(uint2, x), __builtin_bit_cast(uint2, y));
  }
  __device__ static __forceinline__ F acc(f32x4 lo, f32x4 hi) {
    F f;
    f[0] = (__bf16)lo[0];
    f[1] = (__bf16)lo[1];
    f[2] = (__bf16)lo[2];
    f[3] = (__bf16)lo[3];
    f[4] = (__bf16)hi[0];
    f[5] = (__bf16)hi[1];
    f[6] = (__bf16)hi[2];
    f[7] = (__bf16)hi[3];
    return f;
  }
  __device__ static __forceinline__ f32x4 mma(const F& a, const F& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // 8 bf16 input elements (16 bytes) as a fragment
  __device__ static __forceinline__ F from_bf16(u32x4 a) { return __builtin_bit_cast(F, a); }
  __device__ static __forceinline__ F from_f32(const float* x) {
    F f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (__bf16)x[j];
    return f;
  }
  // 8 consecutive elements (16-byte aligned) as a fragment
  __device__ static __forceinline__ F ld8(const T* p) { return *(const F*)p; }
  // 8 fp32 values (lo then hi) stored as 8 consecutive elements
  __device__ static __forceinline__ void st8(T* p, f32x4 lo, f32x4 hi) { *(F*)p = acc(lo, hi); }
  __device__ static __forceinline__ void stf(T* p, const F& f) { *(F*)p = f; }
};

// fp32 MFMA operands (v_mfma_f32_16x16x4_f32, eight per K = 32 fragment).
struct ArmF32 {
  typedef float T;
  struct F {
    float v[8];
  };
  static constexpr int PAD = 4;
  __device__ static __forceinline__ T cvt(float x) { return x; }
  __device__ static __forceinline__ float val(T x) { return x; }
  __device__ static __forceinline__ F row(const T* p0, const T* p1) {
    const float4 a = *(const float4*)p0, b = *(const float4*)p1;
    F f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
  __device__ static __forceinline__ F col(const T* base, int pitch, int k0, int n0, int lane) {
    const int i = lane & 15, g = lane >> 4;
    F f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.v[j] = base[(k0 + 4 * g + j) * pitch + n0 + i];
      f.v[4 + j] = base[(k0 + 16 + 4 * g + j) * pitch + n0 + i];
    }
    return f;
  }
  __device__ static __forceinline__ F acc(f32x4 lo, f32x4 hi) {
    F f;
    f.v[0] = lo[0]; f.v[1] = lo[1]; f.v[2] = lo[2]; f.v[3] = lo[3];
    f.v[4] = hi[0]; f.v[5] = hi[1]; f.v[6] = hi[2]; f.v[7] = hi[3];
    return f;
  }
  __device__ static __forceinline__ f32x4 mma(const F& a, const F& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
  }
  __device__ static __forceinline__ F from_bf16(u32x4 a) {
    F f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.v[2 * j] = __uint_as_float(a[j] << 16);
      f.v[2 * j + 1] = __uint_as_float(a[j] & 0xFFFF0000u);
    }
    return f;
  }
  __device__ static __forceinline__ F from_f32(const float* x) {
    F f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = x[j];
    return f;
  }
  __device__ static __forceinline__ F ld8(const T* p) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    F f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
  __device__ static __forceinline__ void st8(T* p, f32x4 lo, f32x4 hi) {
    *(float4*)p = (float4){lo[0], lo[1], lo[2], lo[3]};
    *(float4*)(p + 4) = (float4){hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static __forceinline__ void stf(T* p, const F& f) {
    *(float4*)p = (float4){f.v[0], f.v[1], f.v[2], f.v[3]};
    *(float4*)(p + 4) = (float4){f.v[4], f.v[5], f.v[6], f.v[7]};
  }
};

// ------------------------------------------------------ global I/O -------
// one input element as fp32
__device__ __forceinline__ float load1(const void* src, int64_t e, int src_f32) {
  return src_f32 ? ((const float*)src)[e] : bf2f(((const uint16_t*)src)[e]);
}

// Location of a chunk slot: sequence, first token, valid rows.  False for slots past
// the last chunk (the prep grid covers an upper bound when cu_seqlens is given).
__device__ __forceinline__ bool locate_chunk(const Params& p, int C, int64_t slot, int& n, int64_t& t0,
                                             int& L) {
  if (!p.varlen) {
    if (p.chunks_per_seq == 0) return false;
    n = (int)(slot / p.chunks_per_seq);
    const int64_t ci = slot - (int64_t)n * p.chunks_per_seq;
    if (n >= p.n_seq) return false;
    t0 = (int64_t)n * p.seq_len + ci * C;
    L = (int)min64(C, (int64_t)p.seq_len - ci * C);
    return true;
  }
  const int32_t* bnd = p.table;
  const int32_t* cpre = p.table + p.n_seq + 1;
  if (slot >= cpre[p.n_seq]) return false;
  // largest n with cpre[n] <= slot; sequences with no chunks have cpre[n] == cpre[n+1]
  int lo = 0, hi = p.n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cpre[mid] <= slot) lo = mid; else hi = mid - 1;
  }
  n = lo;
  const int64_t ci = slot - cpre[n];
  t0 = bnd[n] + ci * C;
  L = (int)min64(C, (int64_t)bnd[n + 1] - t0);
  return L > 0;
}

// The m-th chunk slot of a launch's prep range: every slot, or for a fixed-length batch
// chunks [prep_cb, prep_ce) of each sequence in turn.  False past the range.
__device__ __forceinline__ bool prep_slot(const Params& p, int64_t m, int64_t& slot) {
  if (p.varlen) {
    slot = m;
    return m < p.max_slots;
  }
  const int pw = p.prep_ce - p.prep_cb;
  if (pw <= 0) return false;
  const int64_t n = m / pw;
  if (n >= p.n_seq) return false;
  slot = n * p.chunks_per_seq + p.prep_cb + (m - n * pw);
  return true;
}

// Where the tiles of logical chunk slot `slot` (fixed-length: n * chunks_per_seq + c) are
// stored: the slot itself, or in the pipelined ring slot n * 2 R + c mod 2 R.
__device__ __forceinline__ int64_t store_slot(const Params& p, int64_t slot) {
  if (!p.tile_ring) return slot;
  const int64_t n = slot / p.chunks_per_seq, c = slot - n * p.chunks_per_seq;
  return n * (2 * p.tile_ring) + c % (2 * p.tile_ring);
}

// ---------------------------------------------------- chunk table --------
// A bucket of a sequence's chunk count, monotone in it: the count itself below 4, else
// 4 e + the two bits below the leading one (e = its bit length - 1), so a bucket spans at
// most a quarter of its lower end.  0 .. 107 for counts below 2^27.
__device__ __forceinline__ int chunk_bucket(int32_t c) {
  if (c < 4) return c;
  const int e = 31 - __clz(c);
  return min(127, 4 * e + ((c >> (e - 2)) & 3));
}

// Sanitised bounds b_0 = 0, b_i = min(total, max(0, max_{1<=j<=i} cu_j)), b_n = total,
// so every index stays inside [0, total] whatever cu_seqlens holds; any difference
// from the given offsets sets GDN_ST_BAD_SEQLENS.  Then the chunk prefix over sequences,
// and the scan's dispatch order: the sequences by descending chunk bucket (a counting
// sort over 128 buckets; ties in any order), so that the first round of a packed batch's
// scan workgroups takes its longest sequences, whatever the order of cu_seqlens.
__global__ __launch_bounds__(256) void gdn_chunk_table(Params p, int C) {
  __shared__ int32_t sbuf[256];
  __shared__ int32_t carry;
  const int tid = threadIdx.x, n = p.n_seq;
  const int32_t total = (int32_t)p.total;
  int32_t* bnd = p.table;
  int32_t* cpre = p.table + n + 1;
  bool bad = false;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base <= n; base += 256) {
    const int i = base + tid;
    int32_t c = (i <= n) ? p.cu_seqlens[i] : 0;
    int32_t x = (i >= 1 && i <= n - 1) ? max(c, 0) : 0;
    sbuf[tid] = x;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int32_t y = (tid >= off) ? sbuf[tid - off] : 0;
      __syncthreads();
      sbuf[tid] = max(sbuf[tid], y);
      __syncthreads();
    }
    const int32_t m = max(sbuf[tid], carry);
    if (i <= n) {
      const int32_t b = (i == 0) ? 0 : (i == n ? total : min(total, m));
      bnd[i] = b;
      if (c != b) bad = true;
    }
    __syncthreads();
    if (tid == 255) carry = max(carry, sbuf[255]);
    __syncthreads();
  }
  // chunk prefix: cpre[0] = 0, cpre[i+1] = cpre[i] + ceil((b_{i+1} - b_i) / C)
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 256) {
    const int i = base + tid;
    const int32_t cnt = (i < n) ? (bnd[i + 1] - bnd[i] + C - 1) / C : 0;
    sbuf[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int32_t y = (tid >= off) ? sbuf[tid - off] : 0;
      __syncthreads();
      sbuf[tid] += y;
      __syncthreads();
    }
    if (i < n) cpre[i + 1] = carry + sbuf[tid];
    __syncthreads();
    if (tid == 255) carry += sbuf[255];
    __syncthreads();
  }
  if (tid == 0) cpre[0] = 0;
  if (bad) atomicOr(p.status, GDN_ST_BAD_SEQLENS);
  __syncthreads();
  // dispatch order: bucket histogram, descending start of each bucket, then each
  // sequence takes the next place of its bucket
  __shared__ int32_t start[128];
  int32_t* order = cpre + n + 1;
  if (tid < 128) start[tid] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 256) atomicAdd(&start[127 - chunk_bucket(cpre[i + 1] - cpre[i])], 1);
  __syncthreads();
  if (tid == 0) {
    int32_t sum = 0;
    for (int b = 0; b < 128; ++b) {
      const int32_t c = start[b];
      start[b] = sum;
      sum += c;
    }
  }
  __syncthreads();
  for (int i = tid; i < n; i += 256) order[atomicAdd(&start[127 - chunk_bucket(cpre[i + 1] - cpre[i])], 1)] = i;
}

// ------------------------------------------------ 16-byte staging -------
__device__ __forceinline__ u32x4 ld16(const void* base, int64_t byte_off) {
  return *(const u32x4*)((const char*)base + byte_off);
}

template <bool QF32>
__device__ __forceinline__ uint32_t nonfinite16(u32x4 a) {
  if constexpr (QF32) return nf_f32(a.x) | nf_f32(a.y) | nf_f32(a.z) | nf_f32(a.w);
  else return nf_bf16x2(a.x) | nf_bf16x2(a.y) | nf_bf16x2(a.z) | nf_bf16x2(a.w);
}

// 16 input bytes (8 bf16 or 4 fp32) -> the same elements in the arm's LDS type
template <class Arm, bool QF32>
__device__ __forceinline__ void put16(u32x4 a, typename Arm::T* dst) {
  if constexpr (sizeof(typename Arm::T) == 2) {
    if constexpr (QF32) {
      const uint32_t w0 = (uint32_t)f2bf(__uint_as_float(a.x)) | ((uint32_t)f2bf(__uint_as_float(a.y)) << 16);
      const uint32_t w1 = (uint32_t)f2bf(__uint_as_float(a.z)) | ((uint32_t)f2bf(__uint_as_float(a.w)) << 16);
      *(uint2*)dst = (uint2){w0, w1};
    } else {
      *(u32x4*)dst = a;
    }
  } else {
    if constexpr (QF32) {
      *(u32x4*)dst = a;
    } else {
      float4* d = (float4*)dst;
      d[0] = (float4){__uint_as_float(a.x << 16), __uint_as_float(a.x & 0xFFFF0000u),
                      __uint_as_float(a.y << 16), __uint_as_float(a.y & 0xFFFF0000u)};
      d[1] = (float4){__uint_as_float(a.z << 16), __uint_as_float(a.z & 0xFFFF0000u),
                      __uint_as_float(a.w << 16), __uint_as_float(a.w & 0xFFFF0000u)};
    }
  }
}

// 16 input bytes -> fp32 in LDS
template <bool QF32>
__device__ __forceinline__ void put16f(u32x4 a, float* dst) {
  if constexpr (QF32) {
    *(u32x4*)dst = a;
  } else {
    float4* d = (float4*)dst;
    d[0] = (float4){__uint_as_float(a.x << 16), __uint_as_float(a.x & 0xFFFF0000u),
                    __uint_as_float(a.y << 16), __uint_as_float(a.y & 0xFFFF0000u)};
    d[1] = (float4){__uint_as_float(a.z << 16), __uint_as_float(a.z & 0xFFFF0000u),
                    __uint_as_float(a.w << 16), __uint_as_float(a.w & 0xFFFF0000u)};
  }
}

// ------------------------------------------------- T and P as fragments --
// The scan reads T and P only as MFMA operands whose lanes are rows: fragment (mt, sb)
// gives lane (i, g) row 16 mt + i at columns 32 sb + 4 g + e (e = 0..3) and
// 32 sb + 16 + 4 g + (e - 4) (e = 4..7).  Only fragments that touch the lower triangle
// (sb <= mt / 2) exist.  The workspace holds them exactly so -- per (chunk slot, value
// head) the fragments in tile_frag_index order, 64 lanes x 8 consecutive elements each --
// so the scan copies them verbatim and each lane reads a fragment with one 16-byte
// (bf16) LDS read, free of bank conflicts.

// Per-wave LDS of the in-wave solve: the lower 16 x 16 tiles of a C x C fp32 matrix
// (tile (rt, st) at tri(rt, st), row pitch kTP), then the chunk's G and beta rows.
constexpr int kTP = 20, kTile = 16 * kTP;
__host__ __device__ constexpr int tri(int rt, int st) { return rt * (rt + 1) / 2 + st; }
template <int C>
struct SolveLds {
  static constexpr int NT = C / 16, NTRI = NT * (NT + 1) / 2;
  // the lower tiles, then the chunk's G and beta rows, (raw inputs) 1 / |k_r| and
  // q_scale / |q_r|, and G's low-order part (gate_prefix: G = hi + lo in two floats) at
  // G_LO past G's row
  static constexpr int FLOATS = NTRI * kTile + 5 * C;
  static constexpr int G_LO = 4 * C;
};

// One wave's LDS accesses in program order, complete: data some lanes wrote is then
// read by others.  (A wave's LDS operations execute in order; this also keeps the
// compiler from moving accesses across it.)
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// element (r, q), r >= q, of a C x C lower-triangular matrix held in S as lower tiles
__device__ __forceinline__ float* tri_at(float* S, int r, int q) {
  return S + tri(r >> 4, q >> 4) * kTile + (r & 15) * kTP + (q & 15);
}

// One 16 x 16 tile product on fp32 MFMA 16x16x4, accumulated: acc += X Y with X a lower tile
// of S read with lanes as its rows (lane (i, g) supplies X[i][4 g + q] to instruction q)
// and Y given as the accumulator of an earlier product (element q of lane (i, g) is
// Y[4 g + q][i]), or as a tile of S read by columns.
__device__ __forceinline__ f32x4 tile_mma_acc(const float* X, const f32x4& Y, f32x4 acc, int i, int g) {
  const float4 x = *(const float4*)(X + i * kTP + 4 * g);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, Y[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, Y[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, Y[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, Y[3], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x4 tile_mma_tile(const float* X, const float* Y, f32x4 acc, int i, int g) {
  const float4 x = *(const float4*)(X + i * kTP + 4 * g);
  const float* y = Y + 4 * g * kTP + i;
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, y[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, y[kTP], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, y[2 * kTP], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, y[3 * kTP], acc, 0, 0, 0);
  return acc;
}

// T = (I + A)^-1 for the strictly lower fp32 A held in S (lower tiles; the diagonal
// tiles' upper parts are ignored), in place: afterwards S holds the lower tiles of T.  A
// blocked solve with diagonal blocks of B rows (B = 8, 16 or 32):
//   1. each B x B diagonal block by forward substitution, one lane per column of a block
//   2. B = 8: the lower-left 8 x 8 block of each diagonal 16 x 16 tile from its two solved
//      halves, T_10 = -T_11 A_10 T_00 (one lane per element), and its upper right cleared
//   3. the remaining blocks, block row by block row (16 x 16 tiles; for B = 32 the one
//      off-diagonal 32 x 32 block of C = 64):
//        T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj   (fp32 MFMA 16x16x4)
// Block row i only reads A's row i and T's earlier rows, so T_i* replaces A_i* once the
// row is done.  One wave, no workgroup barrier.  The substitution's serial depth is B
// rows, its work B^2 / 2 multiply-adds per lane; smaller blocks move work to the MFMA
// updates.  (LDS written by some lanes and read by others is ordered by wave_lds_sync.)
template <int C, int B = 16>
__device__ __forceinline__ void wave_solve_unit_lower(float* S, int lane) {
  static_assert(B == 8 || B == 16 || B == 32, "diagonal block of 8, 16 or 32 rows");
  static_assert(C % B == 0, "whole diagonal blocks");
  constexpr int NB = C / 16, NBB = C / B;
  const int i = lane & 15, g = lane >> 4;
  {
    const int b = (lane / B) % NBB, c = lane % B, r0 = b * B;
    float x[B];
#pragma unroll
    for (int r = 0; r < B; ++r) {
      float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int q = 0; 4 * q < r; ++q) {
        const float4 a = *(const float4*)tri_at(S, r0 + r, r0 + 4 * q);
        const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q + e < r) acc = fmaf(-av[e], x[4 * q + e], acc);
      }
      x[r] = acc;
      // (32 rows: without a point that the finished rows must reach first, the compiler
      // issues every row's reads up front and holds them all, twice the register file)
      if constexpr (B == 32)
        if (r % 4 == 3) asm volatile("" : "+v"(x[r])::"memory");
    }
    wave_lds_sync();
    if (lane < NBB * B) {
#pragma unroll
      for (int r = 0; r < B; ++r)
        if (B < 32 || r >= 16 || c < 16) *tri_at(S, r0 + r, r0 + c) = x[r];  // (stored tiles only)
    }
    wave_lds_sync();
  }
  if constexpr (B == 8) {
    const int r = lane >> 3, c = lane & 7;
#pragma unroll
    for (int d = 0; d < NB; ++d) {
      float* Dt = S + tri(d, d) * kTile;
      float z = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m)  // Z = A_10 T_00 (T_00 lower: m >= c)
        if (m >= c) z = fmaf(Dt[(8 + r) * kTP + m], Dt[m * kTP + c], z);
      wave_lds_sync();
      Dt[(8 + r) * kTP + c] = z;
      wave_lds_sync();
      float t = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m)  // T_10 = -T_11 Z (T_11 lower: m <= r)
        if (m <= r) t = fmaf(Dt[(8 + r) * kTP + 8 + m], Dt[(8 + m) * kTP + c], t);
      wave_lds_sync();
      Dt[(8 + r) * kTP + c] = -t;
      Dt[r * kTP + 8 + c] = 0.f;  // the tile's upper right stays zero for the block updates
      wave_lds_sync();
    }
  }
  if constexpr (B <= 16) {
#pragma unroll
    for (int ib = 1; ib < NB; ++ib) {
      f32x4 R[NB];
#pragma unroll
      for (int jb = 0; jb < ib; ++jb) {
        // Z = sum_m A_{ib,m} T_{m,jb}
        f32x4 Z = zero4();
#pragma unroll
        for (int m = jb; m < ib; ++m) Z = tile_mma_tile(S + tri(ib, m) * kTile, S + tri(m, jb) * kTile, Z, i, g);
        // T_{ib,jb} = -T_{ib,ib} Z
        R[jb] = tile_mma_acc(S + tri(ib, ib) * kTile, Z, zero4(), i, g);
      }
      wave_lds_sync();
#pragma unroll
      for (int jb = 0; jb < ib; ++jb)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[tri(ib, jb) * kTile + (4 * g + j) * kTP + i] = -R[jb][j];
      wave_lds_sync();
    }
  } else if constexpr (C == 64) {
    // the off-diagonal 32 x 32 block (tiles 2, 3 by 0, 1): Z = A_10 T_00 at 32-row
    // granularity (T_00 lower: its tile (0, 1) is zero), then T_10 = -T_11 Z
    f32x4 Z[2][2], R[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        Z[it][jt] = zero4();
#pragma unroll
        for (int m = jt; m < 2; ++m)
          Z[it][jt] = tile_mma_tile(S + tri(2 + it, m) * kTile, S + tri(m, jt) * kTile, Z[it][jt], i, g);
      }
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      R[0][jt] = tile_mma_acc(S + tri(2, 2) * kTile, Z[0][jt], zero4(), i, g);
      R[1][jt] = tile_mma_acc(S + tri(3, 3) * kTile, Z[1][jt],
                              tile_mma_acc(S + tri(3, 2) * kTile, Z[0][jt], zero4(), i, g), i, g);
    }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[tri(2 + it, jt) * kTile + (4 * g + j) * kTP + i] = -R[it][jt][j];
    wave_lds_sync();
  }
}

// The solve with the diagonal block size chosen at run time (8, 16 or 32 rows; anything else
// is 16).
template <int C>
__device__ __forceinline__ void wave_solve(float* S, int lane, int rows) {
  if (rows == 8) wave_solve_unit_lower<C, 8>(S, lane);
  else if (rows == 32) wave_solve_unit_lower<C, 32>(S, lane);
  else wave_solve_unit_lower<C, 16>(S, lane);
}

// From the lower tiles of the two chunk products, oriented with lanes as rows (element j
// of tile (rt, st) in lane (i, g) is row r = 16 rt + i, column s = 16 st + 4 g + j):
//   A = tril_strict(beta_r e^{G_r - G_s} KK),  P = tril(e^{G_r - G_s} QK), rows r < L
// (per-channel gate: the exponentials are already inside the products, G unused);
// then T = (I + A)^-1 in this wave's LDS S (diagonal blocks of solve_rows rows), and T, P stored
// as scan fragments.
// Raw inputs (Nk, Nq non-null: 1 / |k_r| and q_scale / |q_r| of the chunk's rows in LDS):
// the products of the raw rows become those of the normalised rows, A_rs by Nk_r Nk_s and
// P_rs by Nq_r Nk_s (without them every factor is exactly 1, so the bits are unchanged).
template <class Arm, int C, bool KDA>
__device__ __forceinline__ void wave_tiles(f32x4* accA, f32x4* accP, float* S, const float* Gs,
                                           const float* Bs, typename Arm::T* Tout,
                                           typename Arm::T* Pout, int L, int lane, int solve_rows,
                                           const float* Nk = nullptr, const float* Nq = nullptr) {
  constexpr int NT = C / 16;
  const int i = lane & 15, g = lane >> 4;
  wave_lds_sync();  // G and beta rows (and row norms) written by other lanes
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    constexpr int GL = SolveLds<C>::G_LO;
    const float Gr = KDA ? 0.f : Gs[16 * rt + i], Glr = KDA ? 0.f : Gs[GL + 16 * rt + i];
    const float nkr = Nk ? Nk[16 * rt + i] : 1.f, nqr = Nk ? Nq[16 * rt + i] : 1.f;
    const float br = Bs[16 * rt + i] * nkr;  // zero for rows past the chunk end
    const bool live = 16 * rt + i < L;
#pragma unroll
    for (int st = 0; st <= rt; ++st) {
      const int t = tri(rt, st);
      float4 G4 = {0.f, 0.f, 0.f, 0.f}, L4 = {0.f, 0.f, 0.f, 0.f}, N4 = {1.f, 1.f, 1.f, 1.f};
      if constexpr (!KDA) {
        G4 = *(const float4*)(Gs + 16 * st + 4 * g);
        L4 = *(const float4*)(Gs + GL + 16 * st + 4 * g);
      }
      if (Nk) N4 = *(const float4*)(Nk + 16 * st + 4 * g);
      const float Gsv[4] = {G4.x, G4.y, G4.z, G4.w}, Glv[4] = {L4.x, L4.y, L4.z, L4.w};
      const float Nks[4] = {N4.x, N4.y, N4.z, N4.w};
      f32x4 a, pv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool lower = st < rt || 4 * g + j < i;
        const bool ldiag = live && (st < rt || 4 * g + j <= i);
        // e^{G_r - G_s} from the two-float difference, exact for nearby rows and zero
        // across a reset (s > r entries are discarded)
        const float e = (KDA ? 1.f : nexp((Gr - Gsv[j]) + (Glr - Glv[j]))) * Nks[j];
        a[j] = lower ? br * (e * accA[t][j]) : 0.f;
        pv[j] = ldiag ? (e * accP[t][j]) * nqr : 0.f;
      }
      *(float4*)(S + t * kTile + i * kTP + 4 * g) = (float4){a[0], a[1], a[2], a[3]};
      accP[t] = pv;
    }
  }
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int sb = 0; sb <= (mt >> 1); ++sb) {
      const f32x4 hi = (2 * sb + 1 <= mt) ? accP[tri(mt, (2 * sb + 1 <= mt) ? 2 * sb + 1 : 0)] : zero4();
      Arm::st8(Pout + (tile_frag_index(mt, sb) * 64 + lane) * 8, accP[tri(mt, 2 * sb)], hi);
    }
  wave_lds_sync();
  wave_solve<C>(S, lane, solve_rows);
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int sb = 0; sb <= (mt >> 1); ++sb) {
      const float4 l4 = *(const float4*)(S + tri(mt, 2 * sb) * kTile + i * kTP + 4 * g);
      float4 h4 = {0.f, 0.f, 0.f, 0.f};
      if (2 * sb + 1 <= mt) h4 = *(const float4*)(S + tri(mt, 2 * sb + 1) * kTile + i * kTP + 4 * g);
      Arm::st8(Tout + (tile_frag_index(mt, sb) * 64 + lane) * 8, (f32x4){l4.x, l4.y, l4.z, l4.w},
               (f32x4){h4.x, h4.y, h4.z, h4.w});
    }
}

// A fragment from the raw 16-byte loads of its 8 input elements (bf16: one load, fp32: two).
template <class Arm, bool QF32>
__device__ __forceinline__ typename Arm::F frag_of(const u32x4* raw) {
  if constexpr (QF32) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __uint_as_float(raw[j >> 2][j & 3]);
    return Arm::from_f32(x);
  } else {
    return Arm::from_bf16(raw[0]);
  }
}

// ----------------------------------------------------------- prep -------
// The tile work of one (chunk, value head) under the per-head gate, in pieces shared by
// the prep kernel and the fused scan's tile waves (the same instructions on the same
// values, so both compositions produce bit-identical T and P):
//   tile_loads     K and Q operand fragments of the chunk straight from global memory
//                  (rows past a partial chunk's end re-read its last row, in bounds), and
//                  the gate and beta of row `lane`
//   tile_products  the lower 16 x 16 tiles of K K^T and Q K^T on MFMA, oriented so the
//                  accumulator lanes are the rows (A operand = rows of tile st, B operand
//                  = rows of tile rt)
//   tile_sweep     the in-chunk gate prefix G and the masked beta rows, into LDS
// then wave_tiles forms A and P, solves for T and stores both as scan fragments.
template <int DK, int C, bool QF32>
struct TileRegs {
  static constexpr int NBK = DK / 32, NT = C / 16, EPL = QF32 ? 2 : 1;  // 16-byte loads per fragment
  u32x4 rk[NBK][NT][EPL], rq[NBK][NT][EPL];
  float xl, bl;  // gate and beta of row min(lane, L - 1)
};

template <int DK, int C, bool QF32>
__device__ __forceinline__ void tile_loads(const Params& p, int64_t t0, int L, int kh, int h, int lane,
                                           TileRegs<DK, C, QF32>& R) {
  constexpr int NT = C / 16, NBK = DK / 32, ESZ = QF32 ? 4 : 2, EPL = QF32 ? 2 : 1;
  const int i = lane & 15, g = lane >> 4;
  const int rg = lane < L ? lane : L - 1;
  R.xl = p.g[(t0 + rg) * p.hv + h];
  R.bl = p.beta[(t0 + rg) * p.hv + h];
  const int64_t cbase = (t0 * p.hk + kh) * (int64_t)(DK * ESZ);  // chunk's first row
  const char* kbase = (const char*)p.k + cbase;
  const char* qbase = (const char*)p.q + cbase;
  const uint32_t rstride = (uint32_t)(p.hk * DK * ESZ);
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const int r = 16 * rt + i;
    const uint32_t o = (uint32_t)(r < L ? r : L - 1) * rstride + 8 * g * ESZ;
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
      for (int x = 0; x < EPL; ++x) {
        R.rk[kb][rt][x] = *(const u32x4*)(kbase + o + (32 * kb + 4 * x) * ESZ);
        R.rq[kb][rt][x] = *(const u32x4*)(qbase + o + (32 * kb + 4 * x) * ESZ);
      }
  }
}

// Inf/NaN anywhere in the loaded K and Q fragments
template <int DK, int C, bool QF32>
__device__ __forceinline__ uint32_t tile_kq_nonfinite(const TileRegs<DK, C, QF32>& R) {
  uint32_t nf = 0;
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
    for (int rt = 0; rt < C / 16; ++rt)
#pragma unroll
      for (int x = 0; x < (QF32 ? 2 : 1); ++x) nf |= nf_bits16<QF32>(R.rk[kb][rt][x]) | nf_bits16<QF32>(R.rq[kb][rt][x]);
  return flag_if(nf, GDN_ST_NONFINITE_INPUT);
}

template <class Arm, int DK, int C, bool QF32>
__device__ __forceinline__ void tile_products(const TileRegs<DK, C, QF32>& R, f32x4* accA, f32x4* accP) {
  using F = typename Arm::F;
  constexpr int NT = C / 16, NTRI = NT * (NT + 1) / 2;
#pragma unroll
  for (int t = 0; t < NTRI; ++t) {
    accA[t] = zero4();
    accP[t] = zero4();
  }
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb) {
    F kf[NT], qf[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      kf[rt] = frag_of<Arm, QF32>(R.rk[kb][rt]);
      qf[rt] = frag_of<Arm, QF32>(R.rq[kb][rt]);
    }
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int st = 0; st <= rt; ++st) {
        accA[tri(rt, st)] = Arm::mma(kf[st], kf[rt], accA[tri(rt, st)]);
        accP[tri(rt, st)] = Arm::mma(kf[st], qf[rt], accP[tri(rt, st)]);
      }
  }
}

// tile_loads + tile_products with fewer registers live (bf16 inputs), for the fused scan's
// tile waves: every K fragment is loaded first, the Q fragments one row tile ahead of
// their use.  Each tile still accumulates over kb = 0, 1, ... in order with the same
// operands, so its sums are bit-identical to tile_products'.  Returns the K/Q status bits.
template <class Arm, int DK, int C>
__device__ __forceinline__ uint32_t tile_products_lean(const Params& p, int64_t t0, int L, int kh, int h,
                                                       int lane, f32x4* accA, f32x4* accP, float& xl,
                                                       float& bl) {
  using F = typename Arm::F;
  constexpr int NT = C / 16, NBK = DK / 32, NTRI = NT * (NT + 1) / 2, ESZ = 2;
  const int i = lane & 15, g = lane >> 4;
  const int rg = lane < L ? lane : L - 1;
  xl = p.g[(t0 + rg) * p.hv + h];
  bl = p.beta[(t0 + rg) * p.hv + h];
  const int64_t cbase = (t0 * p.hk + kh) * (int64_t)(DK * ESZ);
  const char* kbase = (const char*)p.k + cbase;
  const char* qbase = (const char*)p.q + cbase;
  const uint32_t rstride = (uint32_t)(p.hk * DK * ESZ);
  auto roff = [&](int rt) __attribute__((always_inline)) {
    const int r = 16 * rt + i;
    return (uint32_t)(r < L ? r : L - 1) * rstride + 8 * g * ESZ;
  };
  u32x4 rk[NBK][NT], rq[2][NBK];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb) rk[kb][rt] = *(const u32x4*)(kbase + roff(rt) + 32 * kb * ESZ);
#pragma unroll
  for (int kb = 0; kb < NBK; ++kb) rq[0][kb] = *(const u32x4*)(qbase + roff(0) + 32 * kb * ESZ);
#pragma unroll
  for (int t = 0; t < NTRI; ++t) {
    accA[t] = zero4();
    accP[t] = zero4();
  }
  uint32_t nf = 0;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    if (rt + 1 < NT) {
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb) rq[(rt + 1) & 1][kb] = *(const u32x4*)(qbase + roff(rt + 1) + 32 * kb * ESZ);
    }
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb) {
      nf |= nf_bits16<false>(rk[kb][rt]) | nf_bits16<false>(rq[rt & 1][kb]);
      const F kr = frag_of<Arm, false>(&rk[kb][rt]), qr = frag_of<Arm, false>(&rq[rt & 1][kb]);
#pragma unroll
      for (int st = 0; st <= rt; ++st) {
        const F ks = frag_of<Arm, false>(&rk[kb][st]);
        accA[tri(rt, st)] = Arm::mma(ks, kr, accA[tri(rt, st)]);
        accP[tri(rt, st)] = Arm::mma(ks, qr, accP[tri(rt, st)]);
      }
    }
  }
  return flag_if(nf, GDN_ST_NONFINITE_INPUT);
}

// G (the gate's in-chunk prefix, gate_prefix) and beta of the chunk's rows into Gs, Bs
// (rows past the end contribute gate 0 and beta 0); returns the status bits of the gate and beta
// (raw inputs: xl and bl are the raw gate value and the beta logit, transformed here)
template <int C>
__device__ __forceinline__ uint32_t tile_sweep(float xl, float bl, int L, int lane, float* Gs, float* Bs,
                                               const Params& p) {
  float x = lane < L ? xl : 0.f, b = lane < L ? bl : 0.f;
  uint32_t bad = flag_if(f_nonfinite(x) | f_nonfinite(b), GDN_ST_NONFINITE_INPUT);
  if (p.raw && lane < L) {
    x = neg_softplus(x, p.gate_scale);
    b = sigmoid_f(b);
  }
  bad |= flag_if(x > 0.f, GDN_ST_GATE_DOMAIN);
  const double G = gate_prefix(x);
  if (lane < C) {
    const float hi = (float)G;
    Gs[lane] = hi;
    Gs[SolveLds<C>::G_LO + lane] = (float)(G - (double)hi);
    Bs[lane] = b;
  }
  return bad;
}

// Raw inputs: 1 / |k_r| and q_scale / |q_r| of the chunk's rows (0 for a zero row; rows past
// the chunk end repeat the last row) from the loaded K and Q fragments -- lane (i, g) holds 8
// elements of row 16 rt + i per key block, the four lanes i + 16 g together the whole row --
// into Nk, Nq (LDS) and, when `out` is set, to out[0 .. C) and out[C .. 2C) (workspace).
template <int DK, int C, bool QF32>
__device__ __forceinline__ void tile_row_norms(const TileRegs<DK, C, QF32>& R, float qs, int lane, float* Nk,
                                               float* Nq, float* out) {
  constexpr int NT = C / 16, NBK = DK / 32, EPL = QF32 ? 2 : 1;
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
      for (int x = 0; x < EPL; ++x)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t uk = R.rk[kb][rt][x][w], uq = R.rq[kb][rt][x][w];
          if constexpr (QF32) {
            const float a = __uint_as_float(uk), b = __uint_as_float(uq);
            sk = fmaf(a, a, sk);
            sq = fmaf(b, b, sq);
          } else {
            const float a0 = __uint_as_float(uk << 16), a1 = __uint_as_float(uk & 0xFFFF0000u);
            const float b0 = __uint_as_float(uq << 16), b1 = __uint_as_float(uq & 0xFFFF0000u);
            sk = fmaf(a1, a1, fmaf(a0, a0, sk));
            sq = fmaf(b1, b1, fmaf(b0, b0, sq));
          }
        }
    sk += __shfl_xor(sk, 16, 64);
    sq += __shfl_xor(sq, 16, 64);
    sk += __shfl_xor(sk, 32, 64);
    sq += __shfl_xor(sq, 32, 64);
    if (g == 0) {
      const float nk = sk > 0.f ? 1.f / __builtin_sqrtf(sk) : 0.f, nq = sq > 0.f ? qs / __builtin_sqrtf(sq) : 0.f;
      Nk[16 * rt + i] = nk;
      Nq[16 * rt + i] = nq;
      if (out) {
        out[16 * rt + i] = nk;
        out[C + 16 * rt + i] = nq;
      }
    }
  }
}

// One (chunk slot, value head) unit of the per-head-gate prep on one wave, in two
// halves: prep_fetch issues its global loads (false for a slot past the last chunk),
// prep_finish does the rest with the wave's solve scratch S -- the gate sweep, K K^T and
// Q K^T, A and P, the solve, and T and P stored as scan fragments.  Only the first value
// head of a key head's group checks K and Q and (kq_ws) writes them in the arm's type.
template <int DK, int C, bool QF32>
struct PrepUnit {
  TileRegs<DK, C, QF32> R;
  int64_t slot, t0;
  int kh, j, L;
};

template <int DK, int C, bool QF32>
__device__ __forceinline__ bool prep_fetch(const Params& p, int64_t slot, int kh, int j, int lane,
                                           PrepUnit<DK, C, QF32>& U) {
  int n;
  if (!locate_chunk(p, C, slot, n, U.t0, U.L)) return false;
  U.slot = slot;
  U.kh = kh;
  U.j = j;
  tile_loads<DK, C, QF32>(p, U.t0, U.L, kh, kh * (p.hv / p.hk) + j, lane, U.R);
  return true;
}

template <class Arm, int DK, int C, bool QF32>
__device__ __forceinline__ void prep_finish(const Params& p, const PrepUnit<DK, C, QF32>& U, int lane, float* S,
                                            int solve_rows) {
  using SL = SolveLds<C>;
  constexpr int NT = C / 16, NTRI = SL::NTRI, NBK = DK / 32;
  const int i = lane & 15, g = lane >> 4;
  const int kh = U.kh, j = U.j, L = U.L, h = kh * (p.hv / p.hk) + j;
  const int64_t slot = store_slot(p, U.slot);
  float* Gs = S + NTRI * kTile;
  float* Bs = Gs + C;
  float* Nk = p.raw ? Bs + C : nullptr;
  float* Nq = Bs + 2 * C;
  uint32_t bad = tile_sweep<C>(U.R.xl, U.R.bl, L, lane, Gs, Bs, p);
  if (p.raw)  // (the group's first value head also stores them for the scan)
    tile_row_norms<DK, C, QF32>(U.R, p.q_scale, lane, Nk, Nq,
                                j == 0 ? p.Nws + (slot * p.hk + kh) * (int64_t)(2 * C) : nullptr);
  if (j == 0) {  // once per key head (wave-uniform)
    bad |= tile_kq_nonfinite<DK, C, QF32>(U.R);
    if (p.kq_ws) {
      // K and Q in the arm's element type, [slot][key head][C][DK], for the scan (inputs
      // in fp32, or the fp32 arm); rows past the chunk end repeat its last row
      typedef typename Arm::T T;
      T* kc = (T*)p.Kws + (slot * p.hk + kh) * (int64_t)(C * DK);
      T* qc = (T*)p.Qws + (slot * p.hk + kh) * (int64_t)(C * DK);
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          const int o = (16 * rt + i) * DK + 32 * kb + 8 * g;
          Arm::stf(kc + o, frag_of<Arm, QF32>(U.R.rk[kb][rt]));
          Arm::stf(qc + o, frag_of<Arm, QF32>(U.R.rq[kb][rt]));
        }
    }
  }
  f32x4 accA[NTRI], accP[NTRI];
  tile_products<Arm, DK, C, QF32>(U.R, accA, accP);
  typedef typename Arm::T T;
  const int64_t tofs = (slot * p.hv + h) * (int64_t)tile_elems(C);
  wave_tiles<Arm, C, false>(accA, accP, S, Gs, Bs, (T*)p.Tws + tofs, (T*)p.Pws + tofs, L, lane, solve_rows, Nk, Nq);
  if (bad) atomicOr(p.status, bad);
}

// Per-head gate: one wave per (chunk slot, value head), no barrier.  A workgroup holds up
// to 4 value heads of one key head (blockDim = 64 * min(group, 4)), so the waves that read
// the same K and Q rows run side by side on one CU and fetch them from HBM once.  Every
// global load is issued first, then the math.
template <class Arm, int DK, int C, bool QF32>
__global__ __launch_bounds__(256) void gdn_prep_head(Params p) {
  using SL = SolveLds<C>;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar math
  const int group = p.hv / p.hk, wpb = blockDim.x >> 6, nblk = (group + wpb - 1) / wpb;
  // Workgroups go to the 8 XCDs round-robin: XCD x = blockIdx % 8 takes the chunk slots
  // x, x + 8, ... of the launch's range, all key heads of a slot together, so the gate
  // and beta rows of a chunk (every head's values of a token share a cache line) are
  // fetched into one L2 only.  The grid is padded to whole groups of 8 slots; workgroups
  // past the last slot exit.
  const int ipp = p.hk * nblk;  // workgroups per slot
  const int64_t pos = blockIdx.x / 8;
  const int r = (int)(pos % ipp);
  const int jb = r % nblk;
  const int kh = r / nblk;
  const int64_t m = (pos / ipp) * 8 + blockIdx.x % 8;
  const int j = jb * wpb + w;  // value head inside the key head's group
  int64_t slot;
  if (j >= group || !prep_slot(p, m, slot)) return;
  PrepUnit<DK, C, QF32> U;
  if (prep_fetch<DK, C, QF32>(p, slot, kh, j, lane, U))
    prep_finish<Arm, DK, C, QF32>(p, U, lane, (float*)gdn_smem + w * SL::FLOATS, p.solve_block);
}

// The prep of the next scan segment, run by the workgroups of a pipelined scan launch
// after the scan's own (blockIdx >= nscan; the library's choice requires nscan to be a
// multiple of 8, so these workgroups too sit on XCD blockIdx % 8 -- otherwise only the
// L2 sharing below is lost).  They stay resident and loop: wave w of prep workgroup b takes
// units (slot of the range, key head), key head fastest, among the slots m = x, x + 8,
// ... that belong to its XCD x, with a stride of all the XCD's prep waves.  A unit loads
// K and Q and forms K K^T and Q K^T once, then gates, solves and stores the tiles of each
// value head of the key head's group from a copy of the two products: the same
// instructions on the same values as the prep kernel, so the same bits.  (fp32 inputs or
// operands: units of one value head, like the prep kernel's waves.)  The solve here is
// built for the library's diagonal block only (kSolveBlock rows): the scan kernel's
// registers leave no room for the other sizes' code, so the composition runs only with it.
template <class Arm, int DK, int C, bool QF32>
__device__ __forceinline__ void prep_role(const Params& p) {
  using SL = SolveLds<C>;
  constexpr int NT = C / 16, NTRI = SL::NTRI, NBK = DK / 32, GPRE = 4;
  typedef typename Arm::T T;
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = blockDim.x >> 6;
  const int pb = (int)blockIdx.x - p.nscan, npb = (int)gridDim.x - p.nscan;
  const int x = pb % 8, group = p.hv / p.hk;
  const int64_t M = (int64_t)p.n_seq * (p.prep_ce - p.prep_cb);
  const int64_t stride = (int64_t)((npb - x + 7) / 8) * nw;
  float* S = (float*)gdn_smem + w * SL::FLOATS;
  if constexpr (QF32 || sizeof(T) == 4) {
    // fp32 inputs or operands: the load registers alone fill half the register file, so
    // one (slot, value head) unit at a time, as in the prep kernel
    const int64_t units = (M - x + 7) / 8 * p.hv;
    for (int64_t z = (int64_t)(pb / 8) * nw + w; z < units; z += stride) {
      const int64_t k = z / p.hv;
      const int h = (int)(z - k * p.hv);
      int64_t slot;
      PrepUnit<DK, C, QF32> U;
      if (prep_slot(p, 8 * k + x, slot) && prep_fetch<DK, C, QF32>(p, slot, h / group, h % group, lane, U))
        prep_finish<Arm, DK, C, QF32>(p, U, lane, S, kSolveBlock);
    }
    return;
  }
  const int64_t units = (M - x + 7) / 8 * p.hk;
  float* Gs = S + NTRI * kTile;
  float* Bs = Gs + C;
  for (int64_t z = (int64_t)(pb / 8) * nw + w; z < units; z += stride) {
    const int64_t k = z / p.hk;
    const int kh = (int)(z - k * p.hk);
    int64_t slot, t0;
    int n, L;
    if (!prep_slot(p, 8 * k + x, slot) || !locate_chunk(p, C, slot, n, t0, L)) continue;
    slot = store_slot(p, slot);  // (from here on: where the tiles go)
    const int h0 = kh * group, rg = lane < L ? lane : L - 1;
    TileRegs<DK, C, QF32> R;
    tile_loads<DK, C, QF32>(p, t0, L, kh, h0, lane, R);
    float xs[GPRE], bs[GPRE];  // gate and beta rows of the group's first value heads
    xs[0] = R.xl;
    bs[0] = R.bl;
#pragma unroll
    for (int j = 1; j < GPRE; ++j)
      if (j < group) {
        xs[j] = p.g[(t0 + rg) * p.hv + h0 + j];
        bs[j] = p.beta[(t0 + rg) * p.hv + h0 + j];
      }
    uint32_t bad = tile_kq_nonfinite<DK, C, QF32>(R);
    float* Nk = p.raw ? Bs + C : nullptr;
    float* Nq = Bs + 2 * C;
    if (p.raw)  // row norms once per key head, for every value head of the group and the scan
      tile_row_norms<DK, C, QF32>(R, p.q_scale, lane, Nk, Nq, p.Nws + (slot * p.hk + kh) * (int64_t)(2 * C));
    if (p.kq_ws) {  // K and Q in the arm's element type (as in prep_finish)
      T* kc = (T*)p.Kws + (slot * p.hk + kh) * (int64_t)(C * DK);
      T* qc = (T*)p.Qws + (slot * p.hk + kh) * (int64_t)(C * DK);
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          const int o = (16 * rt + i) * DK + 32 * kb + 8 * g;
          Arm::stf(kc + o, frag_of<Arm, QF32>(R.rk[kb][rt]));
          Arm::stf(qc + o, frag_of<Arm, QF32>(R.rq[kb][rt]));
        }
    }
    f32x4 A0[NTRI], P0[NTRI];
    tile_products<Arm, DK, C, QF32>(R, A0, P0);
    for (int j = 0; j < group; ++j) {
      float xl, bl;
      if (j < GPRE) {
        xl = xs[0];
        bl = bs[0];
#pragma unroll
        for (int jj = 1; jj < GPRE; ++jj)
          if (j == jj) {
            xl = xs[jj];
            bl = bs[jj];
          }
      } else {
        xl = p.g[(t0 + rg) * p.hv + h0 + j];
        bl = p.beta[(t0 + rg) * p.hv + h0 + j];
      }
      bad |= tile_sweep<C>(xl, bl, L, lane, Gs, Bs, p);
      f32x4 accA[NTRI], accP[NTRI];
#pragma unroll
      for (int t = 0; t < NTRI; ++t) {
        accA[t] = A0[t];
        accP[t] = P0[t];
      }
      const int64_t tofs = (slot * p.hv + h0 + j) * (int64_t)tile_elems(C);
      wave_tiles<Arm, C, false>(accA, accP, S, Gs, Bs, (T*)p.Tws + tofs, (T*)p.Pws + tofs, L, lane, kSolveBlock, Nk,
                                Nq);
    }
    if (bad) atomicOr(p.status, bad);
  }
}

// Per-channel gate (C = 32): one workgroup per (chunk slot, value head).  The gate sweep
// and the gated operands run on all 256 threads: thread (d, part) owns key channel d and
// the RP = C / (256 / DK) rows of its part, loads all its g, k and q elements at once,
// and forms the in-chunk prefix G in two levels (its own rows, then the totals of the
// earlier parts through LDS).  Factors are split around the middle row m so every stored
// factor stays below e^85 (gate >= -5, C = 32; arguments clamped, masked entries dropped
// by select):
//   Kup = K e^{G - G_m},  Kdn = K e^{G_m - G},  Qup = Q e^{G - G_m}   (LDS)
// and for the scan e^{G} K, e^{G_C - G} K, e^{G} Q and e^{G_C} (workspace).  Then wave 0
// forms Kup Kdn^T and Qup Kdn^T on MFMA and hands them to wave_tiles.
template <class Arm, int DK>
constexpr size_t prep_chan_lds_bytes() {
  return 3 * (size_t)32 * (DK + Arm::PAD) * sizeof(typename Arm::T) + SolveLds<32>::FLOATS * sizeof(float) +
         (256 / DK + 1) * DK * sizeof(float);
}

template <class Arm, int DK, bool QF32>
__global__ __launch_bounds__(256) void gdn_prep_chan(Params p) {
  using T = typename Arm::T;
  using F = typename Arm::F;
  constexpr int C = 32, NT = 2, NBK = DK / 32, KP = DK + Arm::PAD;
  constexpr int NPART = 256 / DK, RP = C / NPART;  // parts of the chunk's rows, rows per part
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int h = (int)(blockIdx.x % p.hv);
  const int64_t slot = blockIdx.x / p.hv;
  int n, L;
  int64_t t0;
  if (!locate_chunk(p, C, slot, n, t0, L)) return;  // uniform over the workgroup
  const int kh = h / (p.hv / p.hk);
  T* Kup = (T*)gdn_smem;
  T* Kdn = Kup + C * KP;
  T* Qup = Kdn + C * KP;
  float* S = (float*)(Qup + C * KP);
  float* Gs = S + SolveLds<C>::NTRI * kTile;
  float* Bs = Gs + C;
  float* Tot = S + SolveLds<C>::FLOATS;  // [NPART][DK] row totals of each part
  float* Gmid = Tot + NPART * DK;        // [DK] G at the middle row
  uint32_t bad = 0;

  const int d = tid % DK, part = tid / DK, r0 = part * RP;
  // rows r0 .. r0 + RP - 1 (past the chunk end: the last row again, masked below)
  const float* gsrc = p.g + ((t0 * p.hv + h) * (int64_t)DK + d);
  const int64_t gstride = (int64_t)p.hv * DK;
  const int64_t kqoff = (t0 * p.hk + kh) * (int64_t)DK + d, kqstride = (int64_t)p.hk * DK;
  float x[RP], kf[RP], qf[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j) {
    const int r = r0 + j, rr = r < L ? r : L - 1;
    x[j] = gsrc[rr * gstride];
  }
#pragma unroll
  for (int j = 0; j < RP; ++j) {
    const int r = r0 + j, rr = r < L ? r : L - 1;
    kf[j] = load1(p.k, kqoff + rr * kqstride, QF32);
    qf[j] = load1(p.q, kqoff + rr * kqstride, QF32);
  }
  float G[RP];
  {
    float acc = 0.f;
    uint32_t nf = 0, dom = 0;
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      const bool live = r0 + j < L;
      x[j] = live ? x[j] : 0.f;
      kf[j] = live ? kf[j] : 0.f;
      qf[j] = live ? qf[j] : 0.f;
      nf |= f_nonfinite(x[j]) | f_nonfinite(kf[j]) | f_nonfinite(qf[j]);
      dom |= (uint32_t)((x[j] > 0.f) | (x[j] < -5.f));
      acc += x[j];
      G[j] = acc;
    }
    bad |= flag_if(nf, GDN_ST_NONFINITE_INPUT) | flag_if(dom, GDN_ST_GATE_DOMAIN);
    Tot[part * DK + d] = acc;
  }
  __syncthreads();
  float off = 0.f, GC = 0.f;
#pragma unroll
  for (int q = 0; q < NPART; ++q) {
    const float t = Tot[q * DK + d];
    if (q < part) off += t;
    GC += t;
  }
#pragma unroll
  for (int j = 0; j < RP; ++j) G[j] += off;
  if (part == (C / 2) / RP) Gmid[d] = G[(C / 2) % RP];
  __syncthreads();
  const float Gm = Gmid[d];
  T* Y = (T*)p.Gws + (slot * p.hv + h) * (int64_t)(3 * C * DK) + d;
#pragma unroll
  for (int j = 0; j < RP; ++j) {
    const int r = r0 + j;
    const float up = nexp(fminf(G[j] - Gm, 85.f)), dn = nexp(fminf(Gm - G[j], 85.f));
    Kup[r * KP + d] = Arm::cvt(kf[j] * up);
    Kdn[r * KP + d] = Arm::cvt(kf[j] * dn);
    Qup[r * KP + d] = Arm::cvt(qf[j] * up);
    const float eg = nexp(G[j]);
    Y[(0 * C + r) * DK] = Arm::cvt(eg * kf[j]);
    Y[(1 * C + r) * DK] = Arm::cvt(nexp(GC - G[j]) * kf[j]);
    Y[(2 * C + r) * DK] = Arm::cvt(eg * qf[j]);
  }
  if (part == 0) p.Dws[(slot * p.hv + h) * (int64_t)DK + d] = nexp(GC);
  __syncthreads();
  if (w == 0) {
    {
      const int rr = lane < L ? lane : L - 1;
      const float bl = p.beta[(t0 + rr) * p.hv + h];
      const float b = lane < L ? bl : 0.f;
      bad |= flag_if(f_nonfinite(b), GDN_ST_NONFINITE_INPUT);
      if (lane < C) Bs[lane] = b;
    }
    f32x4 accA[3], accP[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      accA[t] = zero4();
      accP[t] = zero4();
    }
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb) {
      F up[NT], dn[NT], qu[NT];
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        const int o = (16 * rt + i) * KP + 32 * kb + 8 * g;
        up[rt] = Arm::ld8(Kup + o);
        dn[rt] = Arm::ld8(Kdn + o);
        qu[rt] = Arm::ld8(Qup + o);
      }
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int st = 0; st <= rt; ++st) {
          accA[tri(rt, st)] = Arm::mma(dn[st], up[rt], accA[tri(rt, st)]);
          accP[tri(rt, st)] = Arm::mma(dn[st], qu[rt], accP[tri(rt, st)]);
        }
    }
    const int64_t tofs = (slot * p.hv + h) * (int64_t)tile_elems(C);
    wave_tiles<Arm, C, true>(accA, accP, S, Gs, Bs, (T*)p.Tws + tofs, (T*)p.Pws + tofs, L, lane, p.solve_block);
  }
  if (bad) atomicOr(p.status, bad);
}

// ----------------------------------------------------------- scan -------
// Serial part: one workgroup per (sequence, value head, 32 state columns), 4 waves:
//   waves 0, 1  chain: each owns 16 state columns; runs only the recurrence
//               Y = K H, X = beta V - beta e^G Y, R = T X, H <- e^{G_C} H + Ktil^T R
//               with its fp32 state in MFMA accumulators; T fragments come straight
//               from global memory into registers, two chunks ahead
//   wave 2      output, one chunk behind the chain: O = e^G (Q H_in) + P R for all 32
//               columns, from H_in and R the chain waves leave in LDS and P (and Q, when
//               it fits in the ring) from the chunk buffer; otherwise it loads Q itself
//   wave 3      loader: copies K, Q, P, V and the gate / beta rows of chunk
//               ci + NBUF - 1 global -> LDS directly (no register round trip) into a ring
//               of NBUF chunk buffers, runs the in-chunk gate sweep ahead, checks V
// One workgroup barrier per chunk.  The fused composition adds two tile waves that form T
// and P in the workgroup (described with their code below).  In a pipelined launch the
// workgroups past the scan's (blockIdx >= nscan) are prep workgroups (prep_role); only the
// PIPE instance carries that code.
//
// State rows are stored permuted within each 32-key block: accumulator tile t = 2 kb + h,
// row 4 g + j holds key dim pi = 32 kb + 8 g + 4 h + j.  Two stacked accumulator tiles are
// then an MFMA operand fragment whose lane group g covers the 8 contiguous key dims
// 32 kb + 8 g .. + 7, so the K and Q row fragments are single 16-byte pieces of their rows.
__device__ __forceinline__ int state_dim(int t, int g, int j) { return 32 * (t >> 1) + 8 * g + 4 * (t & 1) + j; }

// LDS layout of a C x DK operand matrix, in 16-byte pieces.  A row of DK elements is NL
// "lines" of LP pieces (LP = 8 pieces = one 128-byte cache line when a row is that long).
// Lines are stored in blocks of RPI = 64 / LP rows: line (r, ln) at index
// ((r / RPI) * NL + ln) * RPI + r % RPI, and inside it piece p sits at p ^ SW(r).  So one
// copy instruction (64 lanes x 16 bytes) reads RPI whole cache lines, and the row fragment
// of lane (i, g) -- row 16 mt + i, key columns 32 kb + 8 g .. +7 -- is one contiguous read;
// the XOR by row spreads the 8 lanes a 16-byte LDS read serves over distinct bank groups.
template <class Arm, int DK>
struct OpLayout {
  typedef typename Arm::T T;
  static constexpr int NBK = DK / 32;
  static constexpr int EPP = 16 / (int)sizeof(T);  // elements per piece
  static constexpr int PPS = 8 / EPP;              // pieces per 8-element lane slot
  static constexpr int NP = DK / EPP;              // pieces per row
  static constexpr int LP = NP < 8 ? NP : 8;       // pieces per line
  static constexpr int NL = NP / LP;               // lines per row
  static constexpr int RPI = 64 / LP;              // rows per copy instruction
  template <int C>
  static constexpr int bytes() { return C * DK * (int)sizeof(T); }
  __device__ static __forceinline__ int sw(int r) { return ((r % RPI) * PPS) & (LP - 1); }
  // byte offset of element (r, c)
  __device__ static __forceinline__ int off(int r, int c) {
    const int pc = c / EPP, ln = pc / LP, p = pc % LP;
    return ((((r / RPI) * NL + ln) * RPI + r % RPI) * LP + (p ^ sw(r))) * 16 + (c % EPP) * (int)sizeof(T);
  }
  // (row, first column) of the elements the 16-byte piece number `pc` of the layout holds
  __device__ static __forceinline__ void piece_src(int pc, int& r, int& c) {
    const int li = pc / LP, x = pc % LP;
    const int rr = li % RPI, ln = (li / RPI) % NL, rb = li / (RPI * NL);
    r = rb * RPI + rr;
    c = (ln * LP + (x ^ sw(r))) * EPP;
  }
  // the 8-element lane slot starting at column c (a multiple of 8) of row r
  __device__ static __forceinline__ typename Arm::F ld8(const unsigned char* base, int r, int c) {
    if constexpr (PPS == 1) {
      return Arm::ld8((const T*)(base + off(r, c)));
    } else {
      const float4 a = *(const float4*)(base + off(r, c)), b = *(const float4*)(base + off(r, c + 4));
      typename Arm::F f;
      f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
      f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
      return f;
    }
  }
};

typedef __attribute__((address_space(3))) void lds_void;

// Global -> LDS without registers: one instruction moves 64 pieces (16 or 4 bytes), lane
// l's piece to dst + 16 l (dst + 4 l).
__device__ __forceinline__ void dma16(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
}

// The copy wave's workgroup barrier: its own LDS accesses complete, then s_barrier.
// __syncthreads() would also wait for every copy still in flight (the compiler counts a
// global-to-LDS copy as an LDS write under the barrier's fence), which would drain the
// chunk copied ahead at every step; the copies a step needs are waited for explicitly.
__device__ __forceinline__ void copy_wave_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt on outstanding vector memory operations only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt at their maximum, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The operand fragment of Op^T for the state update of tile t: rows = state rows of t
// (key dims state_dim), contraction over the 32 tokens of block sb, token positions
// {4g..4g+3} then {16+4g..16+4g+3} (the R accumulator layout).
template <class Arm, int DK>
__device__ __forceinline__ typename Arm::F kt_frag(const unsigned char* K, int sb, int t, int lane) {
  typedef OpLayout<Arm, DK> Lay;
  const int g = lane >> 4, l = lane & 15;
  const int kb = t >> 1, h = t & 1;
  if constexpr (sizeof(typename Arm::T) == 2) {
    // ds_read_b64_tr_b16: within 16 lanes, lane l receives element l%4 of the 8-byte rows
    // addressed by lanes l/4 + {0, 4, 8, 12}; lane l addresses token 4g + l/4 of the
    // half-block, key dims 32 kb + 8 (l%4) + 4 h .. +3.
    const int s0 = 32 * sb + 4 * g + (l >> 2);
    const int c = 32 * kb + 8 * (l & 3) + 4 * h;
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(K + Lay::off(s0, c)));
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(K + Lay::off(s0 + 16, c)));
    return Arm::pack(__builtin_bit_cast(uint2, x), __builtin_bit_cast(uint2, y));
  } else {
    const int c = state_dim(t, l >> 2, l & 3);
    typename Arm::F f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int s = 32 * sb + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
      f.v[e] = *(const float*)(K + Lay::off(s, c));
    }
    return f;
  }
}

// The scan workgroup's LDS.  NCT: column tiles (of 16 state columns) per chain wave, so the
// workgroup owns WC = 32 NCT state columns.
template <class Arm, int DK, int C, bool KDA, bool QF32, bool FUSED, int NCT = 1>
struct ScanLds {
  typedef typename Arm::T T;
  static constexpr int NBK = DK / 32, NBC = C / 32, WC = 32 * NCT;
  static constexpr int ESZV = QF32 ? 4 : 2;
  static constexpr int RND = 256, LDS_MAX = 160 * 1024;
  static constexpr int rnd(int x) { return (x + RND - 1) / RND * RND; }
  static constexpr int OPB = rnd(OpLayout<Arm, DK>::template bytes<C>());  // one C x DK operand
  // exchange, double-buffered by chunk parity: H_in and R fragments of both chain waves'
  // column tiles
  static constexpr int FRAG = 64 * 8 * (int)sizeof(T);
  static constexpr int HB = 0;
  static constexpr int RO = HB + 2 * 2 * NCT * NBK * FRAG;
  static constexpr int EXCH = RO + 2 * 2 * NCT * NBC * FRAG;
  static constexpr int TILEB = rnd(tile_elems(C) * (int)sizeof(T));  // T or P fragments of a chunk
  static constexpr int NDD = KDA ? (DK + 63) / 64 : 0;  // per-channel decay copies
  static constexpr int NSC = 4 * C + (KDA ? DK : 4);    // beta, beta e^G, e^{G_C-G}, e^G, decay
  static constexpr int SCB = rnd(NSC * 4);
  static constexpr int SSB = FUSED ? rnd(SolveLds<C>::FLOATS * 4) : 0;  // fused: solve scratch
  // A chunk buffer of the ring holds K (per-channel gate: e^G K, then e^{G_C - G} K), Q
  // (e^G Q) when it fits, 32 V columns (input type) and the raw gate / beta rows.  Two
  // layouts place the rest:
  //   split (!TL)  P and the chunk scalars inside each ring buffer; T goes straight from
  //       global memory to the chain waves' registers, two chunks ahead
  //   fused (TL)   T and P of the chunk in use and the next one in two slots each (slot =
  //       chunk parity), which the tile waves write, and the chunk scalars in CL + 1
  //       slots, all after the exchange
  // (Measured for the split scan at dk = 128, C = 64: the slot layout with the copy wave
  // moving T and P is 1.5 % slower; giving up Q in the ring for a fourth buffer, 17 %.)
  static constexpr int NRB = KDA ? 0 : 2 * C * 4;  // raw inputs: 1 / |k_r| and q_scale / |q_r| rows
  static constexpr int base_bytes(bool qr) {
    return (KDA ? 2 : 1) * OPB + (qr ? OPB : 0) + rnd(C * WC * ESZV) + (KDA ? 0 : 256) + 256 + NDD * 256 + NRB;
  }
  static constexpr int FIXA = EXCH + 4 * TILEB + SSB;
  static constexpr bool QRA = 2 * base_bytes(true) + FIXA + 2 * SCB <= LDS_MAX;
  static constexpr int BUFA = base_bytes(QRA);
  static constexpr int NBUFA = 4 * BUFA + FIXA + 3 * SCB <= LDS_MAX ? 4
                               : (3 * BUFA + FIXA + 2 * SCB <= LDS_MAX ? 3 : (2 * BUFA + FIXA + 2 * SCB <= LDS_MAX ? 2 : 0));
  // ring buffers of `buf` bytes that fit beside the exchange (at most 4; 0: not even 2)
  static constexpr int nbuf_for(int buf) {
    return 4 * buf + EXCH <= LDS_MAX ? 4 : (3 * buf + EXCH <= LDS_MAX ? 3 : (2 * buf + EXCH <= LDS_MAX ? 2 : 0));
  }
  // split: Q in the ring unless that leaves fewer buffers than Q out of it and fewer than 3
  static constexpr int NQ_IN = nbuf_for(base_bytes(true) + TILEB + SCB);
  static constexpr int NQ_OUT = nbuf_for(base_bytes(false) + TILEB + SCB);
  static constexpr bool QRB = NQ_IN >= 3 || (NQ_IN >= 2 && NQ_IN == NQ_OUT);
  static constexpr int BUFB = base_bytes(QRB) + TILEB + SCB;
  static constexpr int NBUFB = QRB ? NQ_IN : NQ_OUT;
  static constexpr bool TL = FUSED;
  static_assert(!FUSED || NBUFA >= 2, "fused scan LDS budget");
  // Q goes through the ring (copied like K, read from LDS by the output wave) when two
  // buffers still fit; otherwise the output wave loads its Q fragments itself
  static constexpr bool QR = TL ? QRA : QRB;
  static constexpr int NBUF = TL ? NBUFA : NBUFB;
  // chunks the loader keeps complete ahead of the step that reads them: two with four
  // buffers (the chain then reads the next chunk's K during the current step), else one
  static constexpr int CL = NBUF == 4 ? 2 : 1;
  static constexpr int NSCS = CL + 1;  // TL: scalar slots (chunks ci .. ci + CL)
  static constexpr int KY = 0;
  static constexpr int KH = KY + (KDA ? OPB : 0);
  static constexpr int QO = KH + OPB;
  static constexpr int PP = QO + (QR ? OPB : 0);      // !TL: P fragments
  static constexpr int VV = PP + (TL ? 0 : TILEB);
  static constexpr int GX = VV + rnd(C * WC * ESZV);  // gate rows (per-head gate)
  static constexpr int GB = GX + (KDA ? 0 : 256);     // beta rows
  static constexpr int DC = GB + 256;                 // e^{G_C} per key channel
  static constexpr int NR = DC + NDD * 256;           // raw inputs: the chunk's row norms
  static constexpr int SC = NR + NRB;                 // !TL: row scalars
  static constexpr int BUF = SC + (TL ? 0 : SCB);
  static_assert(BUF == (TL ? BUFA : BUFB), "buffer carve-up");
  // after the exchange (TL): T slots, P slots, scalar slots, then the fused solve scratch
  static constexpr int TT = EXCH;
  static constexpr int TP = TT + 2 * TILEB;
  static constexpr int SCR = TP + 2 * TILEB;
  static constexpr int SS = SCR + NSCS * SCB;
  static constexpr int FIXED = TL ? SS + SSB : EXCH;
  static constexpr int BYTES = NBUF * BUF + FIXED;
  static_assert(NBUF >= 2 && BYTES <= LDS_MAX, "scan LDS budget");
  // Loader copy instructions per chunk.  The loader's copy loops run over exactly these
  // counts, and its vmcnt waits are ND (plus NRAW for raw inputs): one definition for both.
  static constexpr int NOPS = (KDA ? 2 : 1) + (QR ? 1 : 0);  // C x DK operands (K, e^{G_C-G} K, Q)
  static constexpr int NDK = OpLayout<Arm, DK>::template bytes<C>() / 1024;  // per operand
  static constexpr int NDT = tile_elems(C) * (int)sizeof(T) / 1024;  // T or P of a chunk
  static constexpr int NDV = C * WC * ESZV / 1024;
  static constexpr int NROW = KDA ? 1 : 2;  // 4-byte rows: beta, and the gate for the per-head gate
  static constexpr int NRAW = 2;            // raw inputs: the two row-factor rows
  static constexpr int ND = NOPS * NDK + (TL ? 0 : NDT) + NDV + NROW + NDD;
  static_assert(NDK * 1024 == OpLayout<Arm, DK>::template bytes<C>(), "K copy granularity");
  static_assert(NDT * 1024 == tile_elems(C) * (int)sizeof(T), "T / P copy granularity");
  static_assert(NDV * 1024 == C * WC * ESZV, "V copy granularity");
  static_assert(!FUSED || NCT == 1, "fused composition: 32 state columns per workgroup");
};

#ifndef GDN_WIDE_SCAN
#define GDN_WIDE_SCAN 1
#endif

// Measurement build (GDN_SCAN_STAMPS): role r's shader-clock count at phase k of chunk step
// ci, from lane 0 of workgroup stamp_block, for steps stamp_c0 .. stamp_c0 + kStampSteps - 1
// (r: 0 chain wave 0, 1 output wave, 2 loader).  The scheduling barriers keep the count where
// it stands in program order; a phase that ends with a use of a matrix product's result
// therefore records when that result was ready.  The product library records nothing.
#ifdef GDN_SCAN_STAMPS
#define GDN_STAMP(r, ci, k)                                                                            \
  do {                                                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                                 \
    if (p.stamps && (int)blockIdx.x == p.stamp_block && (ci) >= p.stamp_c0 &&                          \
        (ci) < p.stamp_c0 + kStampSteps && lane == 0)                                                  \
      p.stamps[((r) * kStampSteps + (ci) - p.stamp_c0) * kStampPhases + (k)] = __builtin_amdgcn_s_memtime(); \
    __builtin_amdgcn_sched_barrier(0);                                                                 \
  } while (0)
#else
#define GDN_STAMP(r, ci, k) \
  do {                      \
  } while (0)
#endif

template <class Arm, int DK, int C, bool KDA, bool QF32, bool FUSED, int NCT = 1, bool PIPE = false>
__global__ __launch_bounds__(FUSED ? 384 : 256) void gdn_scan(Params p) {
  using T = typename Arm::T;
  using F = typename Arm::F;
  using Lay = OpLayout<Arm, DK>;
  using SL = ScanLds<Arm, DK, C, KDA, QF32, FUSED, NCT>;
  constexpr int WC = SL::WC;  // state columns of this workgroup
  static_assert(!FUSED || (!KDA && !QF32), "fused composition: per-head gate, bf16 inputs");
  // PIPE: the kernel of pipelined launches, whose workgroups past the scan's run the next
  // segment's prep.  Other launches use the instance without that code, which leaves the
  // scan's own roles more registers.
  if constexpr (PIPE) {
    static_assert(!KDA && !FUSED, "prep workgroups: per-head gate, split layout");
    if ((int)blockIdx.x >= p.nscan) {  // pipelined composition: the next segment's prep
      prep_role<Arm, DK, C, QF32>(p);
      return;
    }
  }
  constexpr int NT = C / 16, NBC = C / 32, NTK = DK / 16, NBK = DK / 32;
  constexpr int NBUF = SL::NBUF, LA = NBUF - 1;  // loader copies LA chunks ahead
  constexpr int CL = SL::CL;                      // ... and keeps CL chunks complete ahead
  constexpr bool PRE = CL >= 2;                   // chain prefetches the next chunk's K
  constexpr int ESZV = SL::ESZV;
  const int tid = threadIdx.x, lane = tid & 63, i = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // roles: 0, 1 chain; 2 output; 3 loader; 4, 5 tile waves (fused composition).  Waves go
  // to the SIMDs round-robin, so in the fused workgroup the chain waves take waves 2 and 3
  // (SIMDs of their own) and the tile waves share SIMDs with the output and loader waves.
  const int role = FUSED ? (wave < 4 ? (wave + 2) & 3 : wave) : wave;
  const int DV = p.dv, nslice = DV / WC;
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).  With
  // key heads a multiple of 8, XCD x = blockIdx % 8 takes key heads x, x + 8, ... of
  // every sequence, sequence by sequence: the workgroups reading one key head share an
  // L2, and every XCD holds an equal share of each sequence, so a long sequence of a
  // packed batch is not piled onto a few XCDs when the grid runs in several rounds.
  // Otherwise each XCD takes a contiguous range of (sequence, value head, slice) items.
  int n, h, slice;
  if (p.hk % 8 == 0) {
    const int x = (int)blockIdx.x % 8, pos = (int)blockIdx.x / 8;
    const int group = p.hv / p.hk, gs = group * nslice, per_n = (p.hk / 8) * gs;
    n = pos / per_n;
    const int r = pos % per_n, r2 = r % gs;
    h = ((r / gs) * 8 + x) * group + r2 / nslice;
    slice = r2 % nslice;
  } else {
    const int nb = p.nscan, per = nb / 8, rem = nb % 8;
    const int x = (int)blockIdx.x % 8, pos = (int)blockIdx.x / 8;
    int bid = x * per + (x < rem ? x : rem) + pos;
    slice = bid % nslice;
    bid /= nslice;
    h = bid % p.hv;
    n = bid / p.hv;
  }
  // a packed batch is dispatched longest sequences first (gdn_chunk_table)
  if (p.varlen) n = p.table[2 * (p.n_seq + 1) + n];
  const int kh = h / (p.hv / p.hk);

  // Sequence split: virtual sequence n is part `part` of real sequence nr; kind 0 scans the
  // part's own state, kind 1 its transition (identity start, V read as zero, no outputs),
  // kind 2 rescans it from its chained starting state.
  // (built only where it applies: per-head gate, split kernels)
  constexpr bool PARTS = !KDA && !FUSED;
  int nr = n, part = 0, kind = 0;
  if (PARTS && p.pmode) {
    nr = n / p.pvirt;
    const int v = n - nr * p.pvirt;
    if (p.pmode == 1) {
      part = v < p.nparts ? v : v - p.nparts + 1;
      kind = v < p.nparts ? 0 : 1;
    } else {
      part = v + 1;
      kind = 2;
    }
  }
  int64_t s0, s1, slot0;
  if (p.varlen) {
    s0 = p.table[n];
    s1 = p.table[n + 1];
    slot0 = p.table[p.n_seq + 1 + n];
  } else {  // this launch's chunks [cb, ce) of the sequence (a segment, a part or all)
    const int cb = PARTS && p.pmode ? part * p.part_chunks : p.seg_cb;
    const int ce = PARTS && p.pmode ? (part + 1) * p.part_chunks : p.seg_ce;
    const int64_t b = (int64_t)nr * p.seq_len;
    s0 = b + min64(p.seq_len, (int64_t)cb * C);
    s1 = b + min64(p.seq_len, (int64_t)ce * C);
    slot0 = store_slot(p, (int64_t)nr * p.chunks_per_seq + cb);  // a ring launch stays in one segment
  }
  // kind 1 (a transition) has no outputs; kind 0 of a part after the first scans from a
  // zero state, so its outputs are not final either (the rescan writes them)
  const bool vzero = PARTS && kind == 1, no_out = PARTS && (kind == 1 || (kind == 0 && part > 0));
  const int nch = (int)((s1 - s0 + C - 1) / C);
  uint32_t bad = 0;

  unsigned char* const ring = gdn_smem;
  unsigned char* const exch = gdn_smem + NBUF * SL::BUF;
  auto bufp = [&](int ci) __attribute__((always_inline)) { return ring + (ci % NBUF) * SL::BUF; };
  auto scal = [&](int ci) __attribute__((always_inline)) {
    if constexpr (SL::TL) return (float*)(exch + SL::SCR + (ci % SL::NSCS) * SL::SCB);
    else return (float*)(bufp(ci) + SL::SC);
  };
  auto hb_at = [&](int par, int u, int c, int kb) __attribute__((always_inline)) {
    return (T*)(exch + SL::HB + (((par * 2 + u) * NCT + c) * NBK + kb) * SL::FRAG) + lane * 8;
  };
  auto ro_at = [&](int par, int u, int c, int sb) __attribute__((always_inline)) {
    return (T*)(exch + SL::RO + (((par * 2 + u) * NCT + c) * NBC + sb) * SL::FRAG) + lane * 8;
  };
  // operand sources: row-major rows of DK arm elements, `ld` elements apart
  const int64_t hvs = (int64_t)p.hv;
  auto chunk_t0 = [&](int ci) __attribute__((always_inline)) { return s0 + (int64_t)ci * C; };
  auto chunk_L = [&](int ci) __attribute__((always_inline)) { return (int)min64(C, s1 - chunk_t0(ci)); };
  // K (and, per-channel gate, e^{G_C-G} K) and Q of chunk ci, row 0, and their row stride
  auto src_k = [&](int ci, int which) __attribute__((always_inline)) -> const T* {
    const int64_t slot = slot0 + ci;
    if constexpr (KDA) return (const T*)p.Gws + ((slot * hvs + h) * 3 + which) * (int64_t)(C * DK);
    else if (p.kq_ws) return (const T*)p.Kws + (slot * p.hk + kh) * (int64_t)(C * DK);
    else return (const T*)p.k + (chunk_t0(ci) * p.hk + kh) * (int64_t)DK;
  };
  auto src_q = [&](int ci) __attribute__((always_inline)) -> const T* {
    const int64_t slot = slot0 + ci;
    if constexpr (KDA) return (const T*)p.Gws + ((slot * hvs + h) * 3 + 2) * (int64_t)(C * DK);
    else if (p.kq_ws) return (const T*)p.Qws + (slot * p.hk + kh) * (int64_t)(C * DK);
    else return (const T*)p.q + (chunk_t0(ci) * p.hk + kh) * (int64_t)DK;
  };
  const int kq_ld = (KDA || p.kq_ws) ? DK : p.hk * DK;

  if (role == 3) {
    // ------------------------------------------------------------- loader ----
    // Only copies to LDS are issued here, one instruction per call, so the counts in
    // the waits below are exact.
    // per-lane byte offsets of this lane's pieces inside a full chunk (fixed), so that each
    // copy of a full chunk is a uniform base plus a 32-bit offset
    constexpr int VPR = WC * ESZV / 16;  // pieces per V row
    uint32_t koff[SL::NDK], voff[SL::NDV];
#pragma unroll
    for (int k = 0; k < SL::NDK; ++k) {
      int r, c;
      Lay::piece_src(k * 64 + lane, r, c);
      koff[k] = (uint32_t)((r * kq_ld + c) * (int)sizeof(T));
    }
#pragma unroll
    for (int k = 0; k < SL::NDV; ++k) {
      const int pc = k * 64 + lane;
      voff[k] = (uint32_t)((pc / VPR) * p.hv * DV * ESZV + (pc % VPR) * 16);
    }
    auto issue = [&](int ci) __attribute__((always_inline)) {  // chunk ci -> its buffer
      unsigned char* B = bufp(ci);
      const int64_t t0 = chunk_t0(ci);
      const int L = chunk_L(ci);
      const char* vsrc = (const char*)p.v + (t0 * hvs + h) * (int64_t)(DV * ESZV) + WC * slice * ESZV;
      if (L == C) {  // uniform
#pragma unroll
        for (int w = 0; w < SL::NOPS; ++w) {
          const char* src = (const char*)(w == (KDA ? 2 : 1) ? src_q(ci) : src_k(ci, w));
          const int dst = w == (KDA ? 2 : 1) ? SL::QO : (KDA && w ? SL::KH : SL::KY);
#pragma unroll
          for (int k = 0; k < SL::NDK; ++k) dma16(src + koff[k], B + dst + k * 1024);
        }
#pragma unroll
        for (int k = 0; k < SL::NDV; ++k) dma16(vsrc + voff[k], B + SL::VV + k * 1024);
      } else {  // partial last chunk: rows past the end re-read its last row (in bounds)
#pragma unroll
        for (int w = 0; w < SL::NOPS; ++w) {
          const T* src = w == (KDA ? 2 : 1) ? src_q(ci) : src_k(ci, w);
          const int dst = w == (KDA ? 2 : 1) ? SL::QO : (KDA && w ? SL::KH : SL::KY);
#pragma unroll
          for (int k = 0; k < SL::NDK; ++k) {
            int r, c;
            Lay::piece_src(k * 64 + lane, r, c);
            dma16(src + (int64_t)(r < L ? r : L - 1) * kq_ld + c, B + dst + k * 1024);
          }
        }
#pragma unroll
        for (int k = 0; k < SL::NDV; ++k) {
          const int pc = k * 64 + lane, r = pc / VPR, c = pc % VPR;
          dma16(vsrc + (int64_t)(r < L ? r : L - 1) * hvs * DV * ESZV + c * 16, B + SL::VV + k * 1024);
        }
      }
      if constexpr (!SL::TL) {
        const char* psrc = (const char*)p.Pws + ((slot0 + ci) * hvs + h) * (int64_t)(tile_elems(C) * sizeof(T));
#pragma unroll
        for (int k = 0; k < SL::NDT; ++k) dma16(psrc + (uint32_t)(k * 1024 + lane * 16), B + SL::PP + k * 1024);
      }
      // gate and beta of row min(lane, L - 1); the sweep masks rows past the end
      const int64_t e = (t0 + (lane < L ? lane : L - 1)) * hvs + h;
      static_assert(SL::NROW == (KDA ? 1 : 2), "row copies below");
      if constexpr (!KDA) dma4(p.g + e, B + SL::GX);
      dma4(p.beta + e, B + SL::GB);
      if constexpr (KDA) {
        const float* D = p.Dws + ((slot0 + ci) * hvs + h) * (int64_t)DK;
#pragma unroll
        for (int m = 0; m < SL::NDD; ++m) dma4(D + min(lane + 64 * m, DK - 1), B + SL::DC + m * 256);
      } else {
        if (p.raw) {  // the chunk's row norms, as the prep stored them (NRAW more copies)
          static_assert(SL::NRAW == 2, "row-factor copies below");
          const float* N = p.Nws + ((slot0 + ci) * p.hk + kh) * (int64_t)(2 * C) + (lane < C ? lane : C - 1);
          dma4(N, B + SL::NR);
          dma4(N + C, B + SL::NR + 4 * C);
        }
      }
    };
    auto sweep = [&](int ci) __attribute__((always_inline)) {  // scalars of chunk ci
      const unsigned char* B = bufp(ci);
      float* S = scal(ci);
      const int L = chunk_L(ci);
      const float bl = ((const float*)(B + SL::GB))[lane];
      float b = lane < L ? bl : 0.f;
      bad |= flag_if(f_nonfinite(b), GDN_ST_NONFINITE_INPUT);
      if constexpr (!KDA) {
        const float xl = ((const float*)(B + SL::GX))[lane];
        float x = lane < L ? xl : 0.f;
        bad |= flag_if(f_nonfinite(x), GDN_ST_NONFINITE_INPUT);
        // raw inputs: beta and the gate from the logit and the raw value, the row norms of
        // k (in Y = K H and the state update) and of q (with its scale) for the scalars
        float nk = 1.f, nq = 1.f;
        if (p.raw) {
          if (lane < L) {
            x = neg_softplus(x, p.gate_scale);
            b = sigmoid_f(b);
          }
          nk = ((const float*)(B + SL::NR))[lane < C ? lane : C - 1];
          nq = ((const float*)(B + SL::NR + 4 * C))[lane < C ? lane : C - 1];
        }
        bad |= flag_if(x > 0.f, GDN_ST_GATE_DOMAIN);
        // e^{G}, e^{G_C - G} and e^{G_C} of the rows from gate_prefix (zero across a reset)
        const double G = gate_prefix(x);
        const double GC = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(G), C - 1),
                                           __builtin_amdgcn_readlane(__double2loint(G), C - 1));
        if (lane < C) {
          const float eg = nexp((float)G);
          S[lane] = b;
          S[C + lane] = b * eg * nk;
          S[2 * C + lane] = nexp((float)(GC - G)) * nk;
          S[3 * C + lane] = eg * nq;
        }
        if (lane == 0) S[4 * C] = nexp((float)GC);
      } else {
        if (lane < C) S[lane] = b;
#pragma unroll
        for (int m = 0; m < SL::NDD; ++m)
          if (lane + 64 * m < DK) S[4 * C + lane + 64 * m] = ((const float*)(B + SL::DC))[lane + 64 * m];
      }
    };
    auto check_v = [&](int ci) __attribute__((always_inline)) {  // Inf/NaN in V (LDS)
      const u32x4* Vb = (const u32x4*)(bufp(ci) + SL::VV);
      uint32_t nf = 0;
#pragma unroll
      for (int k = 0; k < SL::NDV; ++k) nf |= nf_bits16<QF32>(Vb[k * 64 + lane]);
      bad |= flag_if(nf, GDN_ST_NONFINITE_INPUT);
    };
    // prologue: chunks 0 .. LA-1 copied, chunks 0 .. CL-1 complete and swept.  At most
    // one chunk's copies (LA - CL <= 1) may stay in flight past a wait, so each wait
    // allows either ND outstanding copies (when a later chunk was issued) or none.
    static_assert(LA - CL <= 1, "one chunk in flight beyond the completed window");
    // (raw inputs: NRAW more copies per chunk, the row norms)
    const bool xr = !KDA && p.raw;
#pragma unroll
    for (int j = 0; j < LA; ++j)
      if (j < nch) issue(j);
    if (LA > CL && nch > LA - 1) {
      if (xr) wait_vm<(LA > CL ? SL::ND + SL::NRAW : 0)>();
      else wait_vm<(LA > CL ? SL::ND : 0)>();
    } else {
      wait_vm<0>();
    }
#pragma unroll
    for (int j = 0; j < CL; ++j)
      if (j < nch) sweep(j);
    copy_wave_barrier();
    for (int ci = 0; ci < nch; ++ci) {
      GDN_STAMP(2, ci, 0);
      const bool more = ci + LA < nch;
      if (more) issue(ci + LA);
      GDN_STAMP(2, ci, 1);
      // chunk ci + CL complete: all copies but this step's, which stay in flight across
      // the barrier
      if (LA > CL && more) {
        if (xr) wait_vm<(LA > CL ? SL::ND + SL::NRAW : 0)>();
        else wait_vm<(LA > CL ? SL::ND : 0)>();
      } else {
        wait_vm<0>();
      }
      GDN_STAMP(2, ci, 2);
      if (ci + CL < nch) sweep(ci + CL);
      check_v(ci);
      GDN_STAMP(2, ci, 3);
      copy_wave_barrier();
    }
  } else if (role == 2) {
    // ------------------------------------------------------------- output ----
    // P fragments, loaded one chunk ahead of their use into two register sets.  Q row
    // fragments come from the chunk's LDS buffer, or, when Q does not fit in the ring,
    // are loaded here one chunk ahead as well.
    constexpr int EPL = 8 / (16 / (int)sizeof(T));  // 16-byte loads per fragment
    constexpr int NQR = SL::QR ? 1 : 2;              // register sets for Q (1 = unused)
    u32x4 pr[2][NBC][NT][EPL], qr[NQR][SL::QR ? 1 : NT][NBK][EPL];
    uint32_t qoff[NT], ooff[NT];
    const int OSZ = p.o_f32 ? 4 : 2;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      qoff[nt] = (uint32_t)(((16 * nt + i) * kq_ld + 8 * g) * (int)sizeof(T));
      ooff[nt] = (uint32_t)(((16 * nt + i) * p.hv * DV + 8 * g) * OSZ);
    }
    auto load_q = [&](int ci, int set) __attribute__((always_inline)) {
      if constexpr (!SL::QR) {
        const char* src = (const char*)src_q(ci);
        const int L = chunk_L(ci);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int r = 16 * nt + i;
          const char* row = L == C ? src + qoff[nt] : src + ((int64_t)(r < L ? r : L - 1) * kq_ld + 8 * g) * (int)sizeof(T);
#pragma unroll
          for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
            for (int x = 0; x < EPL; ++x) qr[set][nt][kb][x] = *(const u32x4*)(row + (32 * kb + x * (16 / (int)sizeof(T))) * (int)sizeof(T));
        }
      }
    };
    auto load_p = [&](int ci, int set) __attribute__((always_inline)) {  // LDS -> registers
      const T* src = SL::TL ? (const T*)(exch + SL::TP + (ci & 1) * SL::TILEB) : (const T*)(bufp(ci) + SL::PP);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int sb = 0; sb < NBC; ++sb)
          if (32 * sb <= 16 * nt + 15) {
#pragma unroll
            for (int x = 0; x < EPL; ++x)
              pr[set][sb][nt][x] = *(const u32x4*)(src + (tile_frag_index(nt, sb) * 64 + lane) * 8 + x * (16 / (int)sizeof(T)));
          }
    };
    auto frag = [&](const u32x4* raw) __attribute__((always_inline)) {
      F f;
      if constexpr (sizeof(T) == 2) f = __builtin_bit_cast(F, raw[0]);
      else f = Arm::ld8((const T*)raw);
      return f;
    };
    f32x4 OQ[2][NCT][NT];  // e^G (Q H_in) of the chunk in flight, every column tile
    auto out_q = [&](int ci, int set) __attribute__((always_inline)) {
      const int par = ci & 1;
      const float* S = scal(ci);
      const unsigned char* Qb = bufp(ci) + SL::QO;
      float e[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) e[nt] = KDA ? 1.f : S[3 * C + 16 * nt + i];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          F hb[NBK];
#pragma unroll
          for (int kb = 0; kb < NBK; ++kb) hb[kb] = Arm::ld8(hb_at(par, u, c, kb));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            f32x4 o = zero4();
#pragma unroll
            for (int kb = 0; kb < NBK; ++kb) {
              F qf;
              if constexpr (SL::QR) qf = Lay::ld8(Qb, 16 * nt + i, 32 * kb + 8 * g);
              else qf = frag(qr[set][SL::QR ? 0 : nt][kb]);
              o = Arm::mma(hb[kb], qf, o);
            }
            OQ[u][c][nt] = o * e[nt];
          }
        }
    };
    auto out_p = [&](int ci, int set) __attribute__((always_inline)) {  // finish chunk ci
      const int par = ci & 1;
      const int64_t t0 = chunk_t0(ci);
      const int L = chunk_L(ci);
      // all products first (independent accumulators), then checks and stores
      f32x4 o[2][NCT][NT];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          F ro[NBC];
#pragma unroll
          for (int sb = 0; sb < NBC; ++sb) ro[sb] = Arm::ld8(ro_at(par, u, c, sb));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            o[u][c][nt] = OQ[u][c][nt];
#pragma unroll
            for (int sb = 0; sb < NBC; ++sb)
              if (32 * sb <= 16 * nt + 15) o[u][c][nt] = Arm::mma(ro[sb], frag(pr[set][sb][nt]), o[u][c][nt]);
          }
        }
      // Inf/NaN in any row (rows past a partial chunk's end repeat finite inputs, so they
      // are nonfinite only together with a real row)
      uint32_t nf = 0;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) nf |= (__float_as_uint(o[u][c][nt][j]) & 0x7F800000u) + 0x00800000u;
      bad |= flag_if(nf & 0x80000000u, GDN_ST_NONFINITE_OUTPUT);
      // rows of this chunk: uniform base plus the lane's fixed row offsets
      char* ob = (char*)p.o + ((t0 * hvs + h) * (int64_t)DV + WC * slice) * OSZ;
      // lane (i, g) of tile (nt, c) holds row 16 nt + i, slice columns 32 c + 8 g .. + 7 (the
      // first four from chain wave 0's quad, the next four from wave 1's)
      auto st = [&](int nt) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          char* a = ob + ooff[nt] + 32 * c * OSZ;
          const f32x4 v0 = o[0][c][nt], v1 = o[1][c][nt];
          if (OSZ == 4) {
            *(float4*)a = (float4){v0[0], v0[1], v0[2], v0[3]};
            *(float4*)(a + 16) = (float4){v1[0], v1[1], v1[2], v1[3]};
          } else {
            const uint2 w0 = pack_bf16x4(v0), w1 = pack_bf16x4(v1);
            *(u32x4*)a = (u32x4){w0.x, w0.y, w1.x, w1.y};
          }
        }
      };
      if (L == C) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st(nt);
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          if (16 * nt + i < L) st(nt);
      }
    };
    if (no_out) {  // a part whose outputs are not final: only the barriers
      for (int ci = 0; ci <= nch; ++ci) __syncthreads();
      return;
    }
    if (nch > 0) load_q(0, 0);
    wait_vm<0>();
    __syncthreads();
    // step ci: finish chunk ci - 1 (P R part), start chunk ci (Q H_in part).  Register
    // sets alternate by chunk parity; the loop is unrolled by two so they are constants.
    auto ostep = [&](auto PAR, int ci) __attribute__((always_inline)) {
      constexpr int cur = decltype(PAR)::value;  // ci & 1
      GDN_STAMP(1, ci, 0);
      // prefetches first; they complete before the barrier, so no load is outstanding
      // across steps and the products below never wait on memory
      if (ci + 1 < nch) load_q(ci + 1, SL::QR ? 0 : cur ^ 1);
      load_p(ci, cur);
      if (ci > 0) out_p(ci - 1, cur ^ 1);
      GDN_STAMP(1, ci, 1);
      out_q(ci, SL::QR ? 0 : cur);
      GDN_STAMP(1, ci, 2);
      if constexpr (!SL::QR) wait_vm<0>();  // Q loads (and this step's stores)
      GDN_STAMP(1, ci, 3);
      __syncthreads();
    };
    int ci = 0;  // whole pairs, then a last odd step (as in the chain loop)
    for (; ci + 1 < nch; ci += 2) {
      ostep(std::integral_constant<int, 0>{}, ci);
      ostep(std::integral_constant<int, 1>{}, ci + 1);
    }
    if (ci < nch) ostep(std::integral_constant<int, 0>{}, ci);
    if (nch > 0) {
      if ((nch - 1) & 1) out_p(nch - 1, 1);
      else out_p(nch - 1, 0);
    }
  } else if (role < 2) {
    // -------------------------------------------------------------- chain ----
    // Each chain wave owns NCT column tiles of 16 state columns; the K fragments of a chunk
    // (rows for Y = K H, transposed for the state update) and T serve all of them.
    const int u = role;
    // this lane's state column in column tile c of the slice: the two chain waves own
    // interleaved quads of each 32 columns, so the output wave holds 8 consecutive columns
    // of a row per lane
    auto ccol = [&](int c) __attribute__((always_inline)) { return 32 * c + 8 * (i >> 2) + 4 * u + (i & 3); };
    const int col0 = WC * slice + ccol(0);  // column tile c: col0 + 32 c
    // this workgroup's starting state and where its final state goes ([dk][dv] fp32 each)
    const int64_t hsz = DK * (int64_t)DV, hbase = ((int64_t)n * p.hv + h) * hsz;
    const float* hin = p.h0 ? p.h0 + hbase : nullptr;
    float* hout = p.hT ? p.hT + hbase : nullptr;
    bool hcheck = p.h0_input;
    if (PARTS && p.pmode) {
      const int64_t real = ((int64_t)nr * p.hv + h) * hsz, pt = (((int64_t)nr * p.nparts + part) * p.hv + h) * hsz;
      // (the second part starts from the first part's own final state)
      const float* h2 = part == 1 ? p.Bws + (((int64_t)nr * p.nparts) * p.hv + h) * hsz : p.Hws + pt;
      hin = kind == 0 ? (part == 0 && p.h0 ? p.h0 + real : nullptr) : (kind == 2 ? h2 : nullptr);
      hout = kind == 0 ? p.Bws + pt : (kind == 1 ? p.Mws + pt : (part == p.nparts - 1 && p.hT ? p.hT + real : nullptr));
      hcheck = kind == 0 && part == 0;
    }
    f32x4 H[NCT][NTK];
    if (hin) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int t = 0; t < NTK; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            H[c][t][j] = hin[(int64_t)state_dim(t, g, j) * DV + col0 + 32 * c];
            bad |= flag_if(hcheck && f_nonfinite(H[c][t][j]), GDN_ST_NONFINITE_INPUT);
          }
    } else {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int t = 0; t < NTK; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            H[c][t][j] = (PARTS && kind == 1 && state_dim(t, g, j) == col0 + 32 * c) ? 1.f : 0.f;
    }
    F HB[NCT][NBK];
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb) {
        HB[c][kb] = Arm::acc(H[c][2 * kb], H[c][2 * kb + 1]);
        Arm::st8(hb_at(0, u, c, kb), H[c][2 * kb], H[c][2 * kb + 1]);
      }
    F kf[NBK][NT];  // K row fragments of the chunk being processed
    // T fragments: straight from global memory (stored in exactly this layout), two chunks
    // ahead into two register sets (set = chunk parity); the chain issues no other global
    // memory operation in its loop, so each step's wait leaves just the newest set in flight.
    // (The loads stay visible to the compiler: a load it cannot see may have its
    // destination registers moved or reused while the data is still in flight.)
    constexpr int EPL = 8 / (16 / (int)sizeof(T));
    constexpr int NTL = tile_frags(C) * EPL;  // T loads per chunk (lower fragments only)
    u32x4 trs[2][NBC][NT][EPL];
    auto load_t = [&](int ci, auto SET) __attribute__((always_inline)) {
      auto& tr_ = trs[decltype(SET)::value];
      const T* src = (const T*)p.Tws + ((slot0 + ci) * hvs + h) * (int64_t)tile_elems(C);
#pragma unroll
      for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
          if (32 * sb <= 16 * mt + 15) {
#pragma unroll
            for (int x = 0; x < EPL; ++x)
              tr_[sb][mt][x] = *(const u32x4*)(src + (tile_frag_index(mt, sb) * 64 + lane) * 8 + x * (16 / (int)sizeof(T)));
          }
    };
    auto load_kf = [&](int ci) __attribute__((always_inline)) {
      const unsigned char* B = bufp(ci) + SL::KY;
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) kf[kb][mt] = Lay::ld8(B, 16 * mt + i, 32 * kb + 8 * g);
    };
    if constexpr (!SL::TL) {
      if (nch > 0) load_t(0, std::integral_constant<int, 0>{});
      if (nch > 1) load_t(1, std::integral_constant<int, 1>{});
      wait_vm<0>();
    }
    __syncthreads();
    if (PRE && nch > 0) load_kf(0);
    auto cstep = [&](auto PAR, int ci) __attribute__((always_inline)) {
      constexpr int cur = decltype(PAR)::value;  // ci & 1: T register set of this chunk
      auto& tr_ = trs[cur];
      const unsigned char* B = bufp(ci);
      const float* S = scal(ci);
      const int par = ci & 1;
      GDN_STAMP(u == 0 ? 0 : 3, ci, 0);
      if (!PRE) load_kf(ci);
      // operands of the rest of this chunk, read (after K) while the products run
      float vv[NCT][NT][4];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 16 * mt + 4 * g + j;
            if constexpr (QF32) vv[c][mt][j] = *(const float*)(B + SL::VV + (r * WC + ccol(c)) * 4);
            else vv[c][mt][j] = bf2f(*(const uint16_t*)(B + SL::VV + (r * WC + ccol(c)) * 2));
            if (vzero) vv[c][mt][j] = 0.f;
          }
      float4 b4[NT], e4[NT];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        b4[mt] = *(const float4*)(S + 16 * mt + 4 * g);
        if constexpr (!KDA) e4[mt] = *(const float4*)(S + C + 16 * mt + 4 * g);
      }
      F tf[NBC][NT];
      const T* tsl = (const T*)(exch + SL::TT + par * SL::TILEB);  // TL: this chunk's T slot
#pragma unroll
      for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
          if (32 * sb <= 16 * mt + 15) {
            if constexpr (SL::TL) tf[sb][mt] = Arm::ld8(tsl + (tile_frag_index(mt, sb) * 64 + lane) * 8);
            else if constexpr (sizeof(T) == 2) tf[sb][mt] = __builtin_bit_cast(F, tr_[sb][mt][0]);
            else tf[sb][mt] = Arm::ld8((const T*)tr_[sb][mt]);
          }
      // Y = K H_in
      f32x4 Y[NCT][NT];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) Y[c][mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) Y[c][mt] = Arm::mma(kf[kb][mt], HB[c][kb], Y[c][mt]);
      // transposed K fragments for the state update, read while the products run
      F ktf[NBC][NTK];
#pragma unroll
      for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
        for (int t = 0; t < NTK; ++t) ktf[sb][t] = kt_frag<Arm, DK>(B + SL::KH, sb, t, lane);
      // e^{G_C} H_in (the state's old part), off the product chain
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int t = 0; t < NTK; ++t) {
          if constexpr (KDA) {
            const float4 d4 = *(const float4*)(S + 4 * C + state_dim(t, g, 0));
            H[c][t][0] *= d4.x; H[c][t][1] *= d4.y; H[c][t][2] *= d4.z; H[c][t][3] *= d4.w;
          } else {
            const float d = S[4 * C];
            H[c][t][0] *= d; H[c][t][1] *= d; H[c][t][2] *= d; H[c][t][3] *= d;
          }
        }
      __builtin_amdgcn_sched_barrier(0);
      // next chunk's K fragments (its buffer is complete one barrier early)
      if (PRE && ci + 1 < nch) load_kf(ci + 1);
      // X = beta V - beta e^G Y  (per-channel gate: K carries e^G, X = beta (V - Y))
      F XB[NCT][NBC];
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        f32x4 X[NT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
          const float bv[4] = {b4[mt].x, b4[mt].y, b4[mt].z, b4[mt].w};
          if constexpr (KDA) {
#pragma unroll
            for (int j = 0; j < 4; ++j) X[mt][j] = bv[j] * (vv[c][mt][j] - Y[c][mt][j]);
          } else {
            const float ev[4] = {e4[mt].x, e4[mt].y, e4[mt].z, e4[mt].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) X[mt][j] = bv[j] * vv[c][mt][j] - ev[j] * Y[c][mt][j];
          }
        }
#pragma unroll
        for (int sb = 0; sb < NBC; ++sb) XB[c][sb] = Arm::acc(X[2 * sb], X[2 * sb + 1]);
      }
      GDN_STAMP(u == 0 ? 0 : 3, ci, 1);  // Y = K H_in ready (X formed from it)
      // R = T X
      f32x4 R[NCT][NT];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) R[c][mt] = zero4();
#pragma unroll
      for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int mt = 0; mt < NT; ++mt)
            if (32 * sb <= 16 * mt + 15) R[c][mt] = Arm::mma(tf[sb][mt], XB[c][sb], R[c][mt]);
      __builtin_amdgcn_sched_barrier(0);
      // R for the output wave; e^{G_C - G} R for the state update (per-channel gate: the
      // factor is inside Ktil)
      F RS[NCT][NBC];
#pragma unroll
      for (int sb = 0; sb < NBC; ++sb) {
        float4 a = {0.f, 0.f, 0.f, 0.f}, cc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (!KDA) {
          a = *(const float4*)(S + 2 * C + 32 * sb + 4 * g);
          cc = *(const float4*)(S + 2 * C + 32 * sb + 16 + 4 * g);
        }
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          Arm::st8(ro_at(par, u, c, sb), R[c][2 * sb], R[c][2 * sb + 1]);
          if constexpr (KDA) {
            RS[c][sb] = Arm::acc(R[c][2 * sb], R[c][2 * sb + 1]);
          } else {
            f32x4 lo = R[c][2 * sb], hi = R[c][2 * sb + 1];
            lo[0] *= a.x; lo[1] *= a.y; lo[2] *= a.z; lo[3] *= a.w;
            hi[0] *= cc.x; hi[1] *= cc.y; hi[2] *= cc.z; hi[3] *= cc.w;
            RS[c][sb] = Arm::acc(lo, hi);
          }
        }
      }
      GDN_STAMP(u == 0 ? 0 : 3, ci, 2);  // R = T X ready (R stored, R S formed)
      // H <- e^{G_C} H_in + Ktil^T R
#pragma unroll
      for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int t = 0; t < NTK; ++t) H[c][t] = Arm::mma(ktf[sb][t], RS[c][sb], H[c][t]);
      // H_in of the next chunk, for this wave and for the output wave
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb) {
          HB[c][kb] = Arm::acc(H[c][2 * kb], H[c][2 * kb + 1]);
          Arm::stf(hb_at(par ^ 1, u, c, kb), HB[c][kb]);
        }
      GDN_STAMP(u == 0 ? 0 : 3, ci, 3);  // state update ready (H_in of the next chunk formed)
      // chunk ci + 2's T into this chunk's set; chunk ci + 1's (issued a step ago) must be
      // complete at the barrier, chunk ci + 2's may stay in flight.  (The compiler also
      // waits for the newest set before R = T X in the first step of each pair, since it
      // merges its wait-count state across the two branches below; loading unconditionally
      // removes that wait but measured 1 % slower on the hybrid layer, and loading three
      // chunks ahead, which also shortens the wait below, measured the same: the step is
      // then bounded by the other waves' share of the CU, not by the T loads.)
      if constexpr (!SL::TL) {
        if (ci + 2 < nch) {
          load_t(ci + 2, PAR);
          wait_vm<NTL>();
        } else {
          wait_vm<0>();
        }
      }
      GDN_STAMP(u == 0 ? 0 : 3, ci, 4);
      __syncthreads();
    };
    // whole pairs of steps, then a last odd step (no step skipped inside the loop body)
    int ci = 0;
    for (; ci + 1 < nch; ci += 2) {
      cstep(std::integral_constant<int, 0>{}, ci);
      cstep(std::integral_constant<int, 1>{}, ci + 1);
    }
    if (ci < nch) cstep(std::integral_constant<int, 0>{}, ci);
    if (hout) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int t = 0; t < NTK; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bad |= flag_if(f_nonfinite(H[c][t][j]), GDN_ST_NONFINITE_OUTPUT);
            hout[(int64_t)state_dim(t, g, j) * DV + col0 + 32 * c] = H[c][t][j];
          }
    }
  } else if constexpr (FUSED) {
    // ------------------------------------------------------ tiles (fused) ----
    // Chunk u's T and P are formed by tile wave u & 1 over two steps, with the prep
    // kernel's code: at step u - 2 its loads and products, at step u - 1 the gate sweep,
    // A and P, the solve, and the stores into tile slot u & 1, which the barrier ending
    // step u - 1 publishes to the chain and output waves for step u.  In any step only one
    // tile wave runs the second half, so the two share one solve scratch.  (Step -1 runs
    // before the first barrier; chunk 0's two halves both fall there.)
    constexpr int NTRI = SolveLds<C>::NTRI;
    const int tw = role - 4;
    float* Sv = (float*)(exch + SL::SS);
    float* Gs = Sv + NTRI * kTile;
    float* Bs = Gs + C;
    f32x4 accA[NTRI], accP[NTRI];
    float xl = 0.f, bl = 0.f;  // gate and beta row of this lane, carried from one half to the other
    // The lane index is passed through an empty asm in each half so the compiler derives
    // the many lane-dependent constants of the solve there, instead of keeping them live
    // (and spilled) across the whole loop.
    auto half_a = [&](int cu) __attribute__((always_inline)) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      bad |= tile_products_lean<Arm, DK, C>(p, chunk_t0(cu), chunk_L(cu), kh, h, ln, accA, accP, xl, bl);
    };
    auto half_b = [&](int cu) __attribute__((always_inline)) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int L = chunk_L(cu);
      bad |= tile_sweep<C>(xl, bl, L, ln, Gs, Bs, p);
      T* Tout = (T*)(exch + SL::TT + (cu & 1) * SL::TILEB);
      T* Pout = (T*)(exch + SL::TP + (cu & 1) * SL::TILEB);
      wave_tiles<Arm, C, false>(accA, accP, Sv, Gs, Bs, Tout, Pout, L, ln, kSolveBlock);
    };
    // every role passes nch + 1 barriers: the first one, then one per step
    int passed = 0;
    if (tw == 0) {  // chunk 0: both halves before the first barrier
      if (nch > 0) {
        half_a(0);
        half_b(0);
      }
      __syncthreads();
      ++passed;
    }
    for (int cu = tw == 0 ? 2 : 1; cu < nch; cu += 2) {
      half_a(cu);  // step cu - 2
      __syncthreads();
      half_b(cu);  // step cu - 1
      __syncthreads();
      passed += 2;
    }
    for (; passed < nch + 1; ++passed) __syncthreads();
  }
  if (bad) atomicOr(p.status, bad);
}

// Sequence split: one step of the chain of the parts' starting states, in fp32 from the
// parts' own final states B (scanned from zero) and transitions M (scanned from the
// identity with V read as zero): H_{q+1} = M_q H_q + B_q, with H_1 = B_0.  One workgroup
// per (sequence, value head, 32 state columns, 32 rows of the result); the 32 columns of
// H_q and the 32 rows of M_q are staged in LDS; fixed summation order.
__global__ __launch_bounds__(256) void gdn_seq_chain(Params p, int DK, int q) {
  __shared__ float Hs[128][33];
  __shared__ float Ms[32][129];
  const int DV = p.dv, ns = DV / 32, nr = DK / 32;
  int b = (int)blockIdx.x;
  const int rb = b % nr;
  b /= nr;
  const int slice = b % ns;
  b /= ns;
  const int h = b % p.hv, n = b / p.hv;
  const int t = threadIdx.x, c = t & 31, r0 = t >> 5;  // column; rows r0 + 8 k of the block
  const int64_t hsz = (int64_t)DK * DV;
  auto at = [&](float* base, int part) { return base + (((int64_t)n * p.nparts + part) * p.hv + h) * hsz; };
  const float* Hq = q == 1 ? at(p.Bws, 0) : at(p.Hws, q);
  const float* M = at(p.Mws, q);
  for (int i = r0; i < DK; i += 8) Hs[i][c] = Hq[(int64_t)i * DV + 32 * slice + c];
  for (int e = t; e < 32 * DK; e += 256) Ms[e / DK][e % DK] = M[(int64_t)(32 * rb + e / DK) * DK + e % DK];
  __syncthreads();
  const float* Bq = at(p.Bws, q);
  float* out = at(p.Hws, q + 1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = r0 + 8 * k, i = 32 * rb + rr;
    const int64_t e = (int64_t)i * DV + 32 * slice + c;
    float acc = Bq[e];
    for (int j = 0; j < DK; ++j) acc = fmaf(Ms[rr][j], Hs[j][c], acc);
    out[e] = acc;
  }
}

// ------------------------------------------------------------ launch -----
// Kernel attributes are set once per kernel and device (the first launch there); later
// launches reuse them.  The kernel is a template argument, so each one has its own flags
// (every kernel here has the same type, so a flag per type would be shared by all).
template <auto Fn>
bool set_lds_once(size_t lds) {
  // one flag per device (the attribute belongs to the function on the current device);
  // concurrent first calls may both set it, which is harmless
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return true;
  if (hipFuncSetAttribute((const void*)Fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return false;
  done.fetch_or(bit, std::memory_order_release);
  return true;
}

// State columns of one scan workgroup: 32, or 64 (two column tiles per chain wave, so a
// chunk's K, Q, T and P, fetched and staged once per workgroup, serve twice the columns)
// when 32-column workgroups would need more than one round of the device's compute units
// (bf16 arm, dv a multiple of 64, not fused).  Measured (scan kernel, same box): the packed
// 131,072-token batch 2.38 -> 2.18 ms with 64 columns (384 workgroups instead of 768); the
// hybrid layer 0.77 -> 1.02 ms and the per-channel layer 0.44 -> 0.50 ms, where 32 columns
// already fit in one round: a 64-column step is about 1.65x as long (the chain waves twice
// the products) and half as many units run.
// GDN_SCAN_COLUMNS=32 or 64 in the environment overrides the rule where 64 is possible (the
// tests compare the two widths on one problem).
int scan_cols(const Plan& pl) {
  if (!GDN_WIDE_SCAN || pl.arm_f32 || pl.fused || pl.dv % 64 != 0) return 32;
  if (const char* e = getenv("GDN_SCAN_COLUMNS")) {
    if (!strcmp(e, "32")) return 32;
    if (!strcmp(e, "64")) return 64;
  }
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 32;
  return (int64_t)pl.n_seq * pl.hv * (pl.dv / 32) > ncu ? 64 : 32;
}

// Pipelined composition: the scan in chunk-aligned segments of kSegTokens tokens (the
// state carried in `carry`), each launch also running the next segment's prep in
// workgroups after the scan's own.
template <class Arm, int DK, int C, bool QF32, int NCT>
gdn_status run_pipelined(const Plan& pl, const Params& prm, float* carry, int nprep, hipStream_t st) {
  constexpr int SEG = kSegTokens / C;  // chunks per segment
  const int cps = pl.chunks_per_seq;
  const int S = (cps + SEG - 1) / SEG;
  auto cut = [&](int s) { return s < S ? s * SEG : cps; };
  const int group = pl.hv / pl.hk, wpb = group < 4 ? group : 4, nblk = (group + wpb - 1) / wpb;
  if (!set_lds_once<gdn_prep_head<Arm, DK, C, QF32>>(4 * SolveLds<C>::FLOATS * sizeof(float))) return GDN_E_LAUNCH;
  using SL = ScanLds<Arm, DK, C, false, QF32, false, NCT>;
  if (!set_lds_once<gdn_scan<Arm, DK, C, false, QF32, false, NCT, true>>(SL::BYTES)) return GDN_E_LAUNCH;
  Params q = prm;
  q.tile_ring = pl.tile_ring;  // (the plan's ring half is one segment, SEG chunks)
  q.prep_cb = 0;
  q.prep_ce = cut(1);
  const int64_t m0 = (int64_t)pl.n_seq * q.prep_ce;  // 0 when the first segment is empty
  if (m0 > 0) {
    hipLaunchKernelGGL((gdn_prep_head<Arm, DK, C, QF32>), dim3((unsigned)((m0 + 7) / 8 * 8 * pl.hk * nblk)),
                       dim3(64 * wpb), wpb * SolveLds<C>::FLOATS * sizeof(float), st, q);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  for (int s = 0; s < S; ++s) {
    const bool last = s == S - 1;
    q.seg_cb = cut(s);
    q.seg_ce = cut(s + 1);
    q.prep_cb = last ? 0 : cut(s + 1);
    q.prep_ce = last ? 0 : cut(s + 2);
    q.h0 = s == 0 ? prm.h0 : carry;
    q.h0_input = s == 0;
    q.hT = last ? prm.hT : carry;
    const int grid = q.nscan + (last ? 0 : nprep);
    hipLaunchKernelGGL((gdn_scan<Arm, DK, C, false, QF32, false, NCT, true>), dim3((unsigned)grid), dim3(256), SL::BYTES,
                       st, q);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  return GDN_OK;
}

// Workgroups a pipelined launch gives the next segment's prep: the compute units the
// scan leaves idle (one scan workgroup fills a unit's LDS), in whole groups of 8 (one per
// XCD); 0 when the pipelined composition does not apply or would not pay.
int pipelined_prep_wgs(const Plan& pl, int nscan) {
  if (!pl.pipe_ok || pl.pipe_req == 0) return 0;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 0;
  int nprep = (ncu - nscan) / 8 * 8;
  if (pl.pipe_req == 1) return nprep >= 8 ? nprep : 8;  // requested: runs (correctly) even on a full device
  // library choice: at least four segments (with fewer, the first segment's prep, which
  // nothing hides, is too large a share: the single 4,096-token layer, 64 chunks, measured
  // 7 % slower pipelined), an XCD-aligned scan grid, and a prep share of at least a
  // quarter of the scan's
  if ((int64_t)pl.chunks_per_seq * pl.chunk < 4 * kSegTokens || nscan % 8 != 0 || pl.hk % 8 != 0 || nprep < 8 ||
      4 * nprep < nscan)
    return 0;
  return nprep;
}

// Parts the sequence-split composition cuts each sequence into: the most (up to kMaxParts)
// whose first launch -- every part's own scan plus the inner parts' transitions, 2 P - 2
// scan grids -- fits the device in one round; 0 when it was not requested.  The library
// never picks it itself: on the single-sequence layer (4,096 tokens, 16 heads, 64 scan
// workgroups) three parts measured 0.106 ms against 0.099 ms split, because the scan's
// step slows as the grid grows (1.5 us a step at 256 workgroups against 1.17 at 64) and
// the extra launches and the chain take the rest of the saving.
int seqsplit_parts(const Plan& pl, int nscan) {
  if (!pl.seq_ok || pl.seq_req != 1 || nscan <= 0) return 0;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 0;
  int parts = ncu / (2 * nscan) + 1;
  if (parts > kMaxParts) parts = kMaxParts;
  return parts < 2 ? 2 : parts;
}

template <class Arm, int DK, int C, bool QF32, int NCT>
gdn_status run_seqsplit(const Plan& pl, const Params& prm, int parts, hipStream_t st) {
  const int group = pl.hv / pl.hk, wpb = group < 4 ? group : 4, nblk = (group + wpb - 1) / wpb;
  if (!set_lds_once<gdn_prep_head<Arm, DK, C, QF32>>(4 * SolveLds<C>::FLOATS * sizeof(float))) return GDN_E_LAUNCH;
  using SL = ScanLds<Arm, DK, C, false, QF32, false, NCT>;
  if (!set_lds_once<gdn_scan<Arm, DK, C, false, QF32, false, NCT>>(SL::BYTES)) return GDN_E_LAUNCH;
  hipLaunchKernelGGL((gdn_prep_head<Arm, DK, C, QF32>), dim3((unsigned)((pl.max_slots + 7) / 8 * 8 * pl.hk * nblk)),
                     dim3(64 * wpb), wpb * SolveLds<C>::FLOATS * sizeof(float), st, prm);
  if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  const int per = pl.hv * (pl.dv / SL::WC);  // scan workgroups per (virtual) sequence
  Params q = prm;
  q.pmode = 1;
  q.nparts = parts;
  q.part_chunks = (pl.chunks_per_seq + parts - 1) / parts;
  q.pvirt = 2 * parts - 2;  // every part's own state, the inner parts' transitions
  q.nscan = pl.n_seq * q.pvirt * per;
  hipLaunchKernelGGL((gdn_scan<Arm, DK, C, false, QF32, false, NCT>), dim3((unsigned)q.nscan), dim3(256), SL::BYTES,
                     st, q);
  if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  // the chain kernel's own grid: 32-column slices of every state
  const int per32 = pl.hv * (pl.dv / 32);
  for (int step = 1; step + 1 < parts; ++step) {  // chain: H_{step+1} = M_step H_step + B_step
    hipLaunchKernelGGL(gdn_seq_chain, dim3((unsigned)(pl.n_seq * per32 * (DK / 32))), dim3(256), 0, st, q, DK, step);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  q.pmode = 2;
  q.pvirt = parts - 1;  // the parts after the first, from their chained states
  q.nscan = pl.n_seq * q.pvirt * per;
  hipLaunchKernelGGL((gdn_scan<Arm, DK, C, false, QF32, false, NCT>), dim3((unsigned)q.nscan), dim3(256), SL::BYTES,
                     st, q);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_E_LAUNCH;
}

template <class Arm, int DK, int C, bool KDA, bool QF32, int NCT>
gdn_status run_cols(const Plan& pl, const Params& prm0, void* carry, hipStream_t st) {
  Params prm = prm0;
  prm.nscan = (int32_t)((int64_t)pl.n_seq * pl.hv * (pl.dv / (32 * NCT)));
  if constexpr (!KDA) {  // the same decisions as plan_compose()
    const int nprep = pipelined_prep_wgs(pl, prm.nscan);
    if (nprep > 0 && pl.run_prep && pl.run_scan && pl.max_slots > 0)
      return run_pipelined<Arm, DK, C, QF32, NCT>(pl, prm, (float*)carry, nprep, st);
    const int parts = seqsplit_parts(pl, prm.nscan);
    if (parts > 0 && pl.run_prep && pl.run_scan && pl.max_slots > 0)
      return run_seqsplit<Arm, DK, C, QF32, NCT>(pl, prm, parts, st);
  }
  if (pl.run_prep && !pl.fused && pl.max_slots > 0) {
    if constexpr (KDA) {
      const size_t lds = prep_chan_lds_bytes<Arm, DK>();
      if (!set_lds_once<gdn_prep_chan<Arm, DK, QF32>>(lds)) return GDN_E_LAUNCH;
      const int64_t blocks = pl.max_slots * pl.hv;
      hipLaunchKernelGGL((gdn_prep_chan<Arm, DK, QF32>), dim3((unsigned)blocks), dim3(256), lds, st, prm);
    } else {
      const int group = pl.hv / pl.hk, wpb = group < 4 ? group : 4, nblk = (group + wpb - 1) / wpb;
      const size_t lds = wpb * SolveLds<C>::FLOATS * sizeof(float);
      if (!set_lds_once<gdn_prep_head<Arm, DK, C, QF32>>(4 * SolveLds<C>::FLOATS * sizeof(float))) return GDN_E_LAUNCH;
      const int64_t blocks = (pl.max_slots + 7) / 8 * 8 * pl.hk * nblk;  // whole groups of 8 slots
      hipLaunchKernelGGL((gdn_prep_head<Arm, DK, C, QF32>), dim3((unsigned)blocks), dim3(64 * wpb), lds, st, prm);
    }
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  if (pl.run_scan) {
    const int64_t blocks = prm.nscan;
    if constexpr (!KDA && !QF32 && NCT == 1 && std::is_same<Arm, ArmBF16>::value) {
      if (pl.fused) {
        const size_t lds = ScanLds<Arm, DK, C, KDA, QF32, true>::BYTES;
        if (!set_lds_once<gdn_scan<Arm, DK, C, KDA, QF32, true>>(lds)) return GDN_E_LAUNCH;
        hipLaunchKernelGGL((gdn_scan<Arm, DK, C, KDA, QF32, true>), dim3((unsigned)blocks), dim3(384), lds, st, prm);
        return hipGetLastError() == hipSuccess ? GDN_OK : GDN_E_LAUNCH;
      }
    }
    if (pl.fused) return GDN_E_UNSUPPORTED;  // refused on the host already
    const size_t lds = ScanLds<Arm, DK, C, KDA, QF32, false, NCT>::BYTES;
    if (!set_lds_once<gdn_scan<Arm, DK, C, KDA, QF32, false, NCT>>(lds)) return GDN_E_LAUNCH;
    hipLaunchKernelGGL((gdn_scan<Arm, DK, C, KDA, QF32, false, NCT>), dim3((unsigned)blocks), dim3(256), lds, st, prm);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  return GDN_OK;
}

template <class Arm, int DK, int C, bool KDA, bool QF32>
gdn_status run(const Plan& pl, const Params& prm, void* carry, hipStream_t st) {
  if constexpr (std::is_same<Arm, ArmBF16>::value) {
    if (scan_cols(pl) == 64) return run_cols<Arm, DK, C, KDA, QF32, 2>(pl, prm, carry, st);
  }
  return run_cols<Arm, DK, C, KDA, QF32, 1>(pl, prm, carry, st);
}

template <class Arm, int DK, bool QF32>
gdn_status run_dk(const Plan& pl, const Params& prm, void* carry, hipStream_t st) {
  if (pl.gate_channel) return run<Arm, DK, 32, true, QF32>(pl, prm, carry, st);
  if (pl.chunk == 32) return run<Arm, DK, 32, false, QF32>(pl, prm, carry, st);
  return run<Arm, DK, 64, false, QF32>(pl, prm, carry, st);
}

template <class Arm>
gdn_status run_arm(const Plan& pl, const Params& prm, void* carry, hipStream_t st) {
  if (pl.qkv_f32) {
    switch (pl.dk) {
      case 32: return run_dk<Arm, 32, true>(pl, prm, carry, st);
      case 64: return run_dk<Arm, 64, true>(pl, prm, carry, st);
      case 128: return run_dk<Arm, 128, true>(pl, prm, carry, st);
      default: return GDN_E_UNSUPPORTED;
    }
  }
  switch (pl.dk) {
    case 32: return run_dk<Arm, 32, false>(pl, prm, carry, st);
    case 64: return run_dk<Arm, 64, false>(pl, prm, carry, st);
    case 128: return run_dk<Arm, 128, false>(pl, prm, carry, st);
    default: return GDN_E_UNSUPPORTED;
  }
}

}  // namespace

int32_t plan_compose(const Plan& pl) {
  if (pl.fused) return GDN_COMPOSE_FUSED;
  const int nscan = (int)((int64_t)pl.n_seq * pl.hv * (pl.dv / scan_cols(pl)));
  if (!pl.gate_channel && pl.run_prep && pl.run_scan && pl.max_slots > 0 && pipelined_prep_wgs(pl, nscan) > 0)
    return GDN_COMPOSE_PIPELINED;
  if (!pl.gate_channel && pl.run_prep && pl.run_scan && pl.max_slots > 0 && seqsplit_parts(pl, nscan) > 0)
    return GDN_COMPOSE_SEQSPLIT;
  return GDN_COMPOSE_SPLIT;
}

gdn_status launch(const Plan& pl, const Params& prm, void* carry, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (pl.varlen && (pl.run_prep || pl.fused)) {
    hipLaunchKernelGGL(gdn_chunk_table, dim3(1), dim3(256), 0, st, prm, (int)pl.chunk);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  return pl.arm_f32 ? run_arm<ArmF32>(pl, prm, carry, st) : run_arm<ArmBF16>(pl, prm, carry, st);
}

}  // namespace gdn
