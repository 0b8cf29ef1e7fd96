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
// the contractions).  Kernels:
//   gdn_chunk_table  one block: sanitised cu_seqlens bounds + per-sequence chunk prefix
//   gdn_prep         one workgroup per (chunk, key head) [per value head for the
//                    per-channel gate]; fully sequence-parallel: gate sweep, K K^T
//                    and Q K^T on MFMA, blocked unit-lower-triangular solve; writes
//                    T and P for every value head of the group
//   gdn_scan         one workgroup per (sequence, value head, 32 state columns), one
//                    wave per 16 columns; fp32 state lives in MFMA accumulators and
//                    never leaves registers; walks the chunks serially
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

__device__ __forceinline__ float wave_prefix_sum(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
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

// ---------------------------------------------------- chunk table --------
// Sanitised bounds b_0 = 0, b_i = min(total, max(0, max_{1<=j<=i} cu_j)), b_n = total,
// so every index stays inside [0, total] whatever cu_seqlens holds; any difference
// from the given offsets sets GDN_ST_BAD_SEQLENS.  Then the chunk prefix over sequences.
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
  static constexpr int FLOATS = NTRI * kTile + 2 * C;
};

// One wave's LDS accesses in program order, complete: data some lanes wrote is then
// read by others.  (A wave's LDS operations execute in order; this also keeps the
// compiler from moving accesses across it.)
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// T = (I + A)^-1 for the strictly lower fp32 A held in S (lower tiles; the diagonal
// tiles' upper parts are ignored), in place: afterwards S holds the lower tiles of T.
//   diagonal 16 x 16 blocks: forward substitution, one lane per column of a block
//   off-diagonal blocks, block row by block row:
//     T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj   (fp32 MFMA 16x16x4)
// Block row i only reads A's row i and T's earlier rows, so T_i* replaces A_i* once
// the row is done.  One wave, no workgroup barrier.
template <int C>
__device__ __forceinline__ void wave_solve_unit_lower(float* S, int lane) {
  constexpr int NB = C / 16;
  const int i = lane & 15, g = lane >> 4;
  {
    const int b = (lane >> 4) & (NB - 1), c = lane & 15;
    float* D = S + tri(b, b) * kTile;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int q = 0; 4 * q < r; ++q) {
        const float4 a = *(const float4*)(D + r * kTP + 4 * q);
        const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q + e < r) acc = fmaf(-av[e], x[4 * q + e], acc);
      }
      x[r] = acc;
    }
    wave_lds_sync();
    if (lane < 16 * NB) {
#pragma unroll
      for (int r = 0; r < 16; ++r) D[r * kTP + c] = x[r];
    }
    wave_lds_sync();
  }
#pragma unroll
  for (int ib = 1; ib < NB; ++ib) {
    f32x4 R[NB];
#pragma unroll
    for (int jb = 0; jb < ib; ++jb) {
      // Z = sum_m A_{ib,m} T_{m,jb}: instruction q pairs k = 4 g + q of lane group g
      f32x4 Z = zero4();
#pragma unroll
      for (int m = jb; m < ib; ++m) {
        const float4 a = *(const float4*)(S + tri(ib, m) * kTile + i * kTP + 4 * g);
        const float* tm = S + tri(m, jb) * kTile + 4 * g * kTP + i;
        Z = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, tm[0], Z, 0, 0, 0);
        Z = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, tm[kTP], Z, 0, 0, 0);
        Z = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, tm[2 * kTP], Z, 0, 0, 0);
        Z = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, tm[3 * kTP], Z, 0, 0, 0);
      }
      // T_{ib,jb} = -T_{ib,ib} Z: Z's accumulator element q is its row 4 g + q
      const float4 d = *(const float4*)(S + tri(ib, ib) * kTile + i * kTP + 4 * g);
      f32x4 t = zero4();
      t = __builtin_amdgcn_mfma_f32_16x16x4f32(d.x, Z[0], t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x4f32(d.y, Z[1], t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x4f32(d.z, Z[2], t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x4f32(d.w, Z[3], t, 0, 0, 0);
      R[jb] = t;
    }
    wave_lds_sync();
#pragma unroll
    for (int jb = 0; jb < ib; ++jb)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[tri(ib, jb) * kTile + (4 * g + j) * kTP + i] = -R[jb][j];
    wave_lds_sync();
  }
}

// From the lower tiles of the two chunk products, oriented with lanes as rows (element j
// of tile (rt, st) in lane (i, g) is row r = 16 rt + i, column s = 16 st + 4 g + j):
//   A = tril_strict(beta_r e^{G_r - G_s} KK),  P = tril(e^{G_r - G_s} QK), rows r < L
// (per-channel gate: the exponentials are already inside the products, G unused);
// then T = (I + A)^-1 in this wave's LDS S, and T, P stored as scan fragments.
template <class Arm, int C, bool KDA>
__device__ __forceinline__ void wave_tiles(f32x4* accA, f32x4* accP, float* S, const float* Gs,
                                           const float* Bs, typename Arm::T* Tout,
                                           typename Arm::T* Pout, int L, int lane) {
  constexpr int NT = C / 16;
  const int i = lane & 15, g = lane >> 4;
  wave_lds_sync();  // G and beta rows written by other lanes
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const float Gr = KDA ? 0.f : Gs[16 * rt + i];
    const float br = Bs[16 * rt + i];  // zero for rows past the chunk end
    const bool live = 16 * rt + i < L;
#pragma unroll
    for (int st = 0; st <= rt; ++st) {
      const int t = tri(rt, st);
      float4 G4 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!KDA) G4 = *(const float4*)(Gs + 16 * st + 4 * g);
      const float Gsv[4] = {G4.x, G4.y, G4.z, G4.w};
      f32x4 a, pv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool lower = st < rt || 4 * g + j < i;
        const bool ldiag = live && (st < rt || 4 * g + j <= i);
        const float e = KDA ? 1.f : nexp(Gr - Gsv[j]);  // s > r entries are discarded
        a[j] = lower ? br * (e * accA[t][j]) : 0.f;
        pv[j] = ldiag ? e * accP[t][j] : 0.f;
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
  wave_solve_unit_lower<C>(S, lane);
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
// Per-head gate: one wave per (chunk slot, value head), four per workgroup, no barrier.
// The wave takes its K and Q operand fragments straight from global memory (the waves
// of one key head's value heads are neighbours and share them through the caches),
// forms KK^T and (Q K^T) lower tiles on MFMA (contraction over dk in contiguous
// 8-element pieces), runs its gate sweep, and hands the products to wave_tiles.
template <class Arm, int DK, int C, bool QF32>
__global__ __launch_bounds__(256) void gdn_prep_head(Params p) {
  using F = typename Arm::F;
  using SL = SolveLds<C>;
  constexpr int NT = C / 16, NTRI = SL::NTRI, NBK = DK / 32;
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar math
  const int64_t unit = (int64_t)blockIdx.x * 4 + w;
  const int64_t slot = unit / p.hv;
  const int h = (int)(unit - slot * p.hv);
  int n, L;
  int64_t t0;
  if (slot >= p.max_slots || !locate_chunk(p, C, slot, n, t0, L)) return;
  const int kh = h / (p.hv / p.hk);
  float* S = (float*)gdn_smem + w * SL::FLOATS;
  float* Gs = S + NTRI * kTile;
  float* Bs = Gs + C;
  uint32_t bad = 0;

  // every global load first (gate and beta, then all K and Q fragments), then the math.
  // Rows past a partial chunk's end re-read its last row (in bounds); their beta is
  // zero, so their A rows vanish, and P masks them at formation.
  const int rg = lane < L ? lane : L - 1;
  const float xl = p.g[(t0 + rg) * p.hv + h], bl = p.beta[(t0 + rg) * p.hv + h];
  constexpr int ESZ = QF32 ? 4 : 2, EPL = QF32 ? 2 : 1;  // 16-byte loads per fragment
  const int64_t cbase = (t0 * p.hk + kh) * (int64_t)(DK * ESZ);  // chunk's first row
  const char* kbase = (const char*)p.k + cbase;
  const char* qbase = (const char*)p.q + cbase;
  const uint32_t rstride = (uint32_t)(p.hk * DK * ESZ);
  u32x4 rk[NBK][NT][EPL], rq[NBK][NT][EPL];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const int r = 16 * rt + i;
    const uint32_t o = (uint32_t)(r < L ? r : L - 1) * rstride + 8 * g * ESZ;
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
      for (int x = 0; x < EPL; ++x) {
        rk[kb][rt][x] = *(const u32x4*)(kbase + o + (32 * kb + 4 * x) * ESZ);
        rq[kb][rt][x] = *(const u32x4*)(qbase + o + (32 * kb + 4 * x) * ESZ);
      }
  }
  {  // gate sweep and beta of row `lane`
    const float x = lane < L ? xl : 0.f, b = lane < L ? bl : 0.f;
    bad |= flag_if(f_nonfinite(x) | f_nonfinite(b), GDN_ST_NONFINITE_INPUT);
    bad |= flag_if(x > 0.f, GDN_ST_GATE_DOMAIN);
    const float G = wave_prefix_sum(x, lane);
    if (lane < C) {
      Gs[lane] = G;
      Bs[lane] = b;
    }
  }
  if (h % (p.hv / p.hk) == 0) {  // K and Q checked once per key head (wave-uniform)
    uint32_t nf = 0;
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int x = 0; x < EPL; ++x) nf |= nf_bits16<QF32>(rk[kb][rt][x]) | nf_bits16<QF32>(rq[kb][rt][x]);
    bad |= flag_if(nf, GDN_ST_NONFINITE_INPUT);
  }

  f32x4 accA[NTRI], accP[NTRI];
#pragma unroll
  for (int t = 0; t < NTRI; ++t) {
    accA[t] = zero4();
    accP[t] = zero4();
  }
#pragma unroll
  for (int kb = 0; kb < NBK; ++kb) {
    F kf[NT], qf[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      kf[rt] = frag_of<Arm, QF32>(rk[kb][rt]);
      qf[rt] = frag_of<Arm, QF32>(rq[kb][rt]);
    }
    // tile (rt, st): A operand = rows of tile st, B operand = rows of tile rt, so the
    // accumulator's lanes are the rows r of tile rt
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int st = 0; st <= rt; ++st) {
        accA[tri(rt, st)] = Arm::mma(kf[st], kf[rt], accA[tri(rt, st)]);
        accP[tri(rt, st)] = Arm::mma(kf[st], qf[rt], accP[tri(rt, st)]);
      }
  }
  typedef typename Arm::T T;
  const int64_t tofs = (slot * p.hv + h) * (int64_t)tile_elems(C);
  wave_tiles<Arm, C, false>(accA, accP, S, Gs, Bs, (T*)p.Tws + tofs, (T*)p.Pws + tofs, L, lane);
  if (bad) atomicOr(p.status, bad);
}

// Per-channel gate (C = 32): one workgroup per (chunk slot, value head).  One thread per
// key channel sweeps the gate down the chunk and forms the gated operands: for the
// products, factors split around the middle row m so every stored factor stays below
// e^85 (gate >= -5, C = 32; arguments clamped, masked entries dropped by select):
//   Kup = K e^{G - G_m},  Kdn = K e^{G_m - G},  Qup = Q e^{G - G_m}   (LDS)
// and for the scan e^{G} K, e^{G_C - G} K, e^{G} Q and e^{G_C} (workspace).  Then wave 0
// forms Kup Kdn^T and Qup Kdn^T on MFMA and hands them to wave_tiles.
template <class Arm, int DK>
constexpr size_t prep_chan_lds_bytes() {
  return 3 * (size_t)32 * (DK + Arm::PAD) * sizeof(typename Arm::T) + SolveLds<32>::FLOATS * sizeof(float);
}

template <class Arm, int DK, bool QF32>
__global__ __launch_bounds__(256) void gdn_prep_chan(Params p) {
  using T = typename Arm::T;
  using F = typename Arm::F;
  constexpr int C = 32, NT = 2, NBK = DK / 32, KP = DK + Arm::PAD;
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
  uint32_t bad = 0;

  if (tid < DK) {
    const int d = tid;
    float G[C];
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      const int rr = r < L ? r : L - 1;
      const float xl = p.g[((t0 + rr) * p.hv + h) * (int64_t)DK + d];
      const float x = r < L ? xl : 0.f;
      bad |= flag_if(f_nonfinite(x), GDN_ST_NONFINITE_INPUT);
      bad |= flag_if((x > 0.f) | (x < -5.f), GDN_ST_GATE_DOMAIN);
      acc += x;
      G[r] = acc;
    }
    const float Gm = G[C / 2];
    const float GC = G[C - 1];
    T* Y = (T*)p.Gws + (slot * p.hv + h) * (int64_t)(3 * C * DK) + d;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      const int rr = r < L ? r : L - 1;
      const int64_t e = ((t0 + rr) * p.hk + kh) * (int64_t)DK + d;
      const float kl = load1(p.k, e, QF32), ql = load1(p.q, e, QF32);
      const float kf = r < L ? kl : 0.f, qf = r < L ? ql : 0.f;
      bad |= flag_if(f_nonfinite(kf) | f_nonfinite(qf), GDN_ST_NONFINITE_INPUT);
      const float up = nexp(fminf(G[r] - Gm, 85.f)), dn = nexp(fminf(Gm - G[r], 85.f));
      Kup[r * KP + d] = Arm::cvt(kf * up);
      Kdn[r * KP + d] = Arm::cvt(kf * dn);
      Qup[r * KP + d] = Arm::cvt(qf * up);
      const float eg = nexp(G[r]);
      Y[(0 * C + r) * DK] = Arm::cvt(eg * kf);
      Y[(1 * C + r) * DK] = Arm::cvt(nexp(GC - G[r]) * kf);
      Y[(2 * C + r) * DK] = Arm::cvt(eg * qf);
    }
    p.Dws[(slot * p.hv + h) * (int64_t)DK + d] = nexp(GC);
  }
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
    wave_tiles<Arm, C, true>(accA, accP, S, Gs, Bs, (T*)p.Tws + tofs, (T*)p.Pws + tofs, L, lane);
  }
  if (bad) atomicOr(p.status, bad);
}

// ----------------------------------------------------------- scan -------
// Sizes of the loaders' staging in 16-byte pieces per loader thread (128 of them).
template <class Arm, int DK, int C, bool KDA, bool QF32>
struct ScanStageDims {
  using T = typename Arm::T;
  static constexpr int EPC = QF32 ? 4 : 8;                           // input elements per 16 bytes
  static constexpr int NKQ = C * DK / EPC / 128;                     // K (and Q) rows
  static constexpr int NTP = tile_elems(C) * (int)sizeof(T) / 16 / 128;  // T (and P) fragments
  static constexpr int NV = C * 32 / EPC / 128;                      // the 32 V columns
  static constexpr int NG = 3 * C * DK * (int)sizeof(T) / 16 / 128;  // gated operands
};

// LDS of one chunk buffer of the scan: operands, T, P, V (fp32), row scalars.
template <class Arm, int DK, int C>
constexpr size_t scan_buf_bytes(bool kda) {
  return (size_t)(kda ? 3 : 2) * C * (DK + Arm::PAD) * sizeof(typename Arm::T)  // K [, K~], Q
         + 2 * (size_t)tile_elems(C) * sizeof(typename Arm::T)                 // T, P fragments
         + (size_t)C * 36 * sizeof(float)                                      // V (32 columns)
         + (4 * (size_t)C + DK + 4) * sizeof(float);                           // row scalars
}
// Two chunk buffers (the next chunk is written while the current one is read) when they
// fit in the 160 KiB of LDS, else one.
template <class Arm, int DK, int C>
constexpr int scan_nbuf(bool kda) { return 2 * scan_buf_bytes<Arm, DK, C>(kda) <= 150 * 1024 ? 2 : 1; }
template <class Arm, int DK, int C>
constexpr size_t scan_lds_bytes(bool kda) {
  return scan_nbuf<Arm, DK, C>(kda) * ((scan_buf_bytes<Arm, DK, C>(kda) + 255) / 256 * 256);
}

// Scan workgroup: 4 waves for 32 state columns of one (sequence, value head).
//   waves 0, 1  compute: each owns 16 state columns; its fp32 state stays in MFMA
//               accumulators and only its matrix products run on its SIMD
//   waves 2, 3  loaders: bring chunk operands from global memory through registers into
//               the LDS chunk buffers, two chunks ahead (two register sets), and run the
//               in-chunk gate sweep
// One barrier per chunk hands a filled buffer from the loaders to the compute waves.
template <class Arm, int DK, int C, bool KDA, bool QF32>
__global__ __launch_bounds__(256) void gdn_scan(Params p) {
  using T = typename Arm::T;
  using F = typename Arm::F;
  using Stage = ScanStageDims<Arm, DK, C, KDA, QF32>;
  constexpr int NT = C / 16, NBC = C / 32, NTK = DK / 16, NBK = DK / 32;
  constexpr int KP = DK + Arm::PAD, VP = 36;
  constexpr int EPC = Stage::EPC, ESZ = QF32 ? 4 : 2;
  constexpr int EPT = 16 / (int)sizeof(T);  // arm elements per 16 bytes
  constexpr int NBUF = scan_nbuf<Arm, DK, C>(KDA);
  constexpr size_t BUF = (scan_buf_bytes<Arm, DK, C>(KDA) + 255) / 256 * 256;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, i = lane & 15, g = lane >> 4;
  const bool loader = wave >= 2;
  const int u = wave & 1;            // compute: state unit; loader: loader index
  const int ltid = tid & 127;        // loader thread index 0..127
  const int DV = p.dv, nslice = DV / 32;
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).  Give
  // each XCD a contiguous range of (sequence, value head, slice) work items, so that the
  // workgroups reading the same key head -- and the 4 slices of one value head -- share
  // an L2 and hit in it.
  int bid;
  {
    const int nb = (int)gridDim.x, per = nb / 8, rem = nb % 8;
    const int x = (int)blockIdx.x % 8, pos = (int)blockIdx.x / 8;
    bid = x * per + (x < rem ? x : rem) + pos;
  }
  const int slice = bid % nslice;
  bid /= nslice;
  const int h = bid % p.hv;
  const int n = bid / p.hv;
  const int kh = h / (p.hv / p.hk);
  const int col0 = 32 * slice + 16 * u;  // compute waves: first value column

  struct Buf {
    T *Ks, *Kl, *Qs, *Ts, *Ps;
    float *Vs, *sb_, *sbe, *seg, *sel, *sdec;
  };
  auto buf_at = [&](int b) __attribute__((always_inline)) {
    Buf B;
    B.Ks = (T*)(gdn_smem + b * BUF);      // K (per-head gate) or e^{G} K (per channel)
    B.Kl = KDA ? B.Ks + C * KP : B.Ks;    // per channel: e^{G_C - G} K
    B.Qs = B.Ks + (KDA ? 2 : 1) * C * KP; // Q or e^{G} Q
    B.Ts = B.Qs + C * KP;
    B.Ps = B.Ts + tile_elems(C);
    B.Vs = (float*)(B.Ps + tile_elems(C));
    B.sb_ = B.Vs + C * VP;  // beta
    B.sbe = B.sb_ + C;      // beta e^{G}
    B.seg = B.sbe + C;      // e^{G}
    B.sel = B.seg + C;      // e^{G_C - G}
    B.sdec = B.sel + C;     // e^{G_C} per key channel (per-channel gate) / [0] per-head gate
    return B;
  };

  int64_t s0, s1, slot0;
  if (p.varlen) {
    s0 = p.table[n];
    s1 = p.table[n + 1];
    slot0 = p.table[p.n_seq + 1 + n];
  } else {
    s0 = (int64_t)n * p.seq_len;
    s1 = s0 + p.seq_len;
    slot0 = (int64_t)n * p.chunks_per_seq;
  }
  const int64_t nch = (s1 - s0 + C - 1) / C;
  uint32_t bad = 0;

  // Loader staging: two register sets (chunks in flight).  Per-head gate: raw K and Q
  // rows, gate and beta of row `lane` (first loader wave).  Per-channel gate: the gated
  // operands from the sequence-parallel stage, beta, e^{G_C[d]}.
  constexpr int NK = KDA ? 1 : Stage::NKQ, NG = KDA ? Stage::NG : 1;
  u32x4 sk[2][NK], sq[2][NK], skg[2][NG], stt[2][Stage::NTP], spp[2][Stage::NTP], sv[2][Stage::NV];
  float sg[2] = {0.f, 0.f}, sbt[2] = {0.f, 0.f}, sdc[2] = {0.f, 0.f};

  // ---- loaders: global -> register set `rs` for chunk ci (branch-free: rows past the
  //      chunk end re-read its last row, in bounds, and are zeroed by a select)
  // Per-thread byte offsets inside a chunk (fixed), so that each load is a uniform chunk
  // base plus a 32-bit offset.  Per-head gate: K/Q rows and V columns of this slice.
  constexpr int KPR = DK / EPC;  // 16-byte pieces per K row
  constexpr int VPR = 32 / EPC;  // 16-byte pieces per row of the 32 V columns
  const int kstride = p.hk * DK * ESZ, vstride = p.hv * DV * ESZ;
  const uint32_t koff0 = (uint32_t)((ltid / KPR) * kstride + (ltid % KPR) * 16);
  const uint32_t voff0 = (uint32_t)((ltid / VPR) * vstride + (ltid % VPR) * 16);

  // ---- loaders: global -> register set `rs` for chunk ci.  A partial last chunk reads
  //      its last row again for the rows past its end (in bounds) and zeroes them.
  auto issue = [&](int rs, int64_t ci) __attribute__((always_inline)) {
    const int64_t t0 = s0 + ci * C;
    const int L = (int)min64(C, s1 - t0);
    const int64_t slot = slot0 + ci;
    const bool full = L == C;  // uniform
    if constexpr (!KDA) {
      const char* kb = (const char*)p.k + (t0 * p.hk + kh) * (int64_t)(DK * ESZ);
      const char* qb = (const char*)p.q + (t0 * p.hk + kh) * (int64_t)(DK * ESZ);
      if (full) {
#pragma unroll
        for (int j = 0; j < Stage::NKQ; ++j) {
          const uint32_t off = koff0 + (uint32_t)(j * (128 / KPR) * kstride);
          sk[rs][j] = *(const u32x4*)(kb + off);
          sq[rs][j] = *(const u32x4*)(qb + off);
        }
      } else {
#pragma unroll
        for (int j = 0; j < Stage::NKQ; ++j) {
          const int r = (ltid + 128 * j) / KPR, c = (ltid + 128 * j) % KPR;
          const uint32_t off = (uint32_t)((r < L ? r : L - 1) * kstride + c * 16);
          const u32x4 a = *(const u32x4*)(kb + off), b = *(const u32x4*)(qb + off);
          sk[rs][j] = (r < L) ? a : (u32x4)(0u);
          sq[rs][j] = (r < L) ? b : (u32x4)(0u);
        }
      }
      if (u == 0) {
        const int rr = lane < L ? lane : L - 1;
        const float x = p.g[(t0 + rr) * p.hv + h], b = p.beta[(t0 + rr) * p.hv + h];
        sg[rs] = (lane < L) ? x : 0.f;
        sbt[rs] = (lane < L) ? b : 0.f;
      }
    } else {
      if (u == 0) {
        const float b = p.beta[(t0 + (lane < L ? lane : L - 1)) * p.hv + h];
        sbt[rs] = (lane < L) ? b : 0.f;
      }
      const u32x4* Gg = (const u32x4*)((const T*)p.Gws + (slot * p.hv + h) * (int64_t)(3 * C * DK));
#pragma unroll
      for (int j = 0; j < Stage::NG; ++j) skg[rs][j] = Gg[ltid + 128 * j];
      if (ltid < DK) sdc[rs] = p.Dws[(slot * p.hv + h) * (int64_t)DK + ltid];
    }
    const u32x4* Tg = (const u32x4*)((const T*)p.Tws + (slot * p.hv + h) * (int64_t)tile_elems(C));
    const u32x4* Pg = (const u32x4*)((const T*)p.Pws + (slot * p.hv + h) * (int64_t)tile_elems(C));
#pragma unroll
    for (int j = 0; j < Stage::NTP; ++j) {
      stt[rs][j] = Tg[ltid + 128 * j];
      spp[rs][j] = Pg[ltid + 128 * j];
    }
    const char* vb = (const char*)p.v + (t0 * p.hv + h) * (int64_t)(DV * ESZ) + 32 * slice * ESZ;
    if (full) {
#pragma unroll
      for (int j = 0; j < Stage::NV; ++j)
        sv[rs][j] = *(const u32x4*)(vb + voff0 + (uint32_t)(j * (128 / VPR) * vstride));
    } else {
#pragma unroll
      for (int j = 0; j < Stage::NV; ++j) {
        const int r = (ltid + 128 * j) / VPR, c = (ltid + 128 * j) % VPR;
        const u32x4 a = *(const u32x4*)(vb + (uint32_t)((r < L ? r : L - 1) * vstride + c * 16));
        sv[rs][j] = (r < L) ? a : (u32x4)(0u);
      }
    }
  };

  // ---- loaders: register set `rs` -> LDS buffer, plus the in-chunk gate sweep
  auto commit = [&](int rs, const Buf& B) __attribute__((always_inline)) {
    if constexpr (!KDA) {
#pragma unroll
      for (int j = 0; j < Stage::NKQ; ++j) {
        const int idx = ltid + 128 * j, r = idx / (DK / EPC), c = idx % (DK / EPC);
        put16<Arm, QF32>(sk[rs][j], B.Ks + r * KP + c * EPC);
        put16<Arm, QF32>(sq[rs][j], B.Qs + r * KP + c * EPC);
      }
      if (u == 0) {
        const float G = wave_prefix_sum(sg[rs], lane);
        const float GC = __shfl(G, C - 1, 64);
        if (lane < C) {
          const float eg = nexp(G);
          B.sb_[lane] = sbt[rs];
          B.sbe[lane] = sbt[rs] * eg;
          B.seg[lane] = eg;
          B.sel[lane] = nexp(GC - G);
        }
        if (lane == 0) B.sdec[0] = nexp(GC);
      }
    } else {
      if (u == 0 && lane < C) B.sb_[lane] = sbt[rs];
      if (ltid < DK) B.sdec[ltid] = sdc[rs];
#pragma unroll
      for (int j = 0; j < Stage::NG; ++j) {
        const int e0 = (ltid + 128 * j) * EPT, m = e0 / (C * DK), r = (e0 / DK) % C, c = e0 % DK;
        *(u32x4*)(B.Ks + (m * C + r) * KP + c) = skg[rs][j];  // Ks, Kl, Qs are consecutive
      }
    }
#pragma unroll
    for (int j = 0; j < Stage::NTP; ++j) {  // fragments, verbatim
      *(u32x4*)(B.Ts + (ltid + 128 * j) * EPT) = stt[rs][j];
      *(u32x4*)(B.Ps + (ltid + 128 * j) * EPT) = spp[rs][j];
    }
#pragma unroll
    for (int j = 0; j < Stage::NV; ++j) {
      const int idx = ltid + 128 * j, r = idx / (32 / EPC), c = idx % (32 / EPC);
      bad |= flag_if(nonfinite16<QF32>(sv[rs][j]), GDN_ST_NONFINITE_INPUT);
      put16f<QF32>(sv[rs][j], B.Vs + r * VP + c * EPC);
    }
  };

  // compute waves: fp32 state of this wave's 16 columns, rows d = 16 t + 4 g + ii
  f32x4 H[NTK];
  const int64_t hbase = ((int64_t)n * p.hv + h) * DK * (int64_t)DV;

  // ---- compute waves: one chunk for this wave's 16 state columns.  Each phase's LDS
  //      fragments are read into registers before its matrix products (the scheduling
  //      barriers keep the reads batched), and the output products that do not depend
  //      on the state chain fill the chain's dependency gaps.
  auto compute = [&](const Buf& B, int64_t ci) __attribute__((always_inline)) {
    const int64_t t0 = s0 + ci * C;
    const int L = (int)min64(C, s1 - t0);
    F HB[NBK];
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb) HB[kb] = Arm::acc(H[2 * kb], H[2 * kb + 1]);

    // K and Q fragments
    F kf[NBK][NT], qf[NBK][NT];
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const T* krow = B.Ks + (16 * mt + i) * KP + 32 * kb + 4 * g;
        kf[kb][mt] = Arm::row(krow, krow + 16);
      }
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const T* qrow = B.Qs + (16 * nt + i) * KP + 32 * kb + 4 * g;
        qf[kb][nt] = Arm::row(qrow, qrow + 16);
      }
    __builtin_amdgcn_sched_barrier(0);

    // Y = K H_in (row tiles are independent accumulators, interleaved per k-block)
    f32x4 Y[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) Y[mt] = zero4();
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) Y[mt] = Arm::mma(kf[kb][mt], HB[kb], Y[mt]);

    // T fragments (lower triangle only) while O^T = H_in^T Q^T runs
    F tf[NBC][NT];
#pragma unroll
    for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
        if (32 * sb <= 16 * mt + 15) tf[sb][mt] = Arm::ld8(B.Ts + (tile_frag_index(mt, sb) * 64 + lane) * 8);
    f32x4 O[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[nt] = zero4();
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) O[nt] = Arm::mma(HB[kb], qf[kb][nt], O[nt]);
    __builtin_amdgcn_sched_barrier(0);

    // X = beta V - beta e^{G} Y   (rows r = 16 mt + 4 g + ii)
    f32x4 X[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * mt + 4 * g + ii;
        // per-channel gate: K already carries e^{G}, beta applies to the whole row
        X[mt][ii] = KDA ? B.sb_[r] * (B.Vs[r * VP + 16 * u + i] - Y[mt][ii])
                        : B.sb_[r] * B.Vs[r * VP + 16 * u + i] - B.sbe[r] * Y[mt][ii];
      }
    }
    F XB[NBC];
#pragma unroll
    for (int sb = 0; sb < NBC; ++sb) XB[sb] = Arm::acc(X[2 * sb], X[2 * sb + 1]);

    // R = T X
    f32x4 R[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) R[mt] = zero4();
#pragma unroll
    for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
        if (32 * sb <= 16 * mt + 15) R[mt] = Arm::mma(tf[sb][mt], XB[sb], R[mt]);

    // Ktil^T fragments (transposing LDS reads) and P fragments
    F ktf[NBC][NTK], pf[NBC][NT];
#pragma unroll
    for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
      for (int t = 0; t < NTK; ++t) ktf[sb][t] = Arm::col(B.Kl, KP, 32 * sb, 16 * t, lane);
#pragma unroll
    for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        if (32 * sb <= 16 * nt + 15) pf[sb][nt] = Arm::ld8(B.Ps + (tile_frag_index(nt, sb) * 64 + lane) * 8);
    __builtin_amdgcn_sched_barrier(0);

    F RO[NBC], RS[NBC];
#pragma unroll
    for (int sb = 0; sb < NBC; ++sb) {
      RO[sb] = Arm::acc(R[2 * sb], R[2 * sb + 1]);
      if constexpr (KDA) {
        RS[sb] = RO[sb];
      } else {
        f32x4 lo, hi;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          lo[ii] = B.sel[32 * sb + 4 * g + ii] * R[2 * sb][ii];
          hi[ii] = B.sel[32 * sb + 16 + 4 * g + ii] * R[2 * sb + 1][ii];
        }
        RS[sb] = Arm::acc(lo, hi);
      }
    }

    // H <- e^{G_C} H + Ktil^T R
#pragma unroll
    for (int t = 0; t < NTK; ++t) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) H[t][ii] *= KDA ? B.sdec[16 * t + 4 * g + ii] : B.sdec[0];
    }
#pragma unroll
    for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
      for (int t = 0; t < NTK; ++t) H[t] = Arm::mma(ktf[sb][t], RS[sb], H[t]);

    // O^T: gate scaling of the H_in part, then + R^T P^T
    if constexpr (!KDA) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float e = B.seg[16 * nt + i];
        O[nt][0] *= e; O[nt][1] *= e; O[nt][2] *= e; O[nt][3] *= e;
      }
    }
#pragma unroll
    for (int sb = 0; sb < NBC; ++sb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        if (32 * sb <= 16 * nt + 15) O[nt] = Arm::mma(RO[sb], pf[sb][nt], O[nt]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = 16 * nt + i;
      if (r < L) {
        const f32x4 o = O[nt];
        bad |= flag_if(f_nonfinite(o[0]) | f_nonfinite(o[1]) | f_nonfinite(o[2]) | f_nonfinite(o[3]),
                       GDN_ST_NONFINITE_OUTPUT);
        const int64_t e = ((t0 + r) * p.hv + h) * (int64_t)DV + col0 + 4 * g;
        if (p.o_f32) {
          *(float4*)((float*)p.o + e) = (float4){o[0], o[1], o[2], o[3]};
        } else {
          const uint32_t w0 = (uint32_t)f2bf(o[0]) | ((uint32_t)f2bf(o[1]) << 16);
          const uint32_t w1 = (uint32_t)f2bf(o[2]) | ((uint32_t)f2bf(o[3]) << 16);
          *(uint2*)((uint16_t*)p.o + e) = (uint2){w0, w1};
        }
      }
    }
  };

  // ---- pipeline.  Each role runs its own loop (so the loaders' staging registers and
  //      the compute waves' state never have to be live at the same time); both loops
  //      execute the same sequence of barriers.  While the compute waves work on chunk ci
  //      (LDS buffer ci&1), the loaders commit chunk ci+1 (register set (ci+1)&1, loaded
  //      two chunks earlier) into the other buffer and start loading chunk ci+3 into the
  //      set they just emptied.  Loops are unrolled by two so that buffer and register-set
  //      indices are compile-time constants.
  if (loader) {
    if (nch > 0) {
      issue(0, 0);
      if (nch > 1) issue(1, 1);
      commit(0, buf_at(0));
      if (nch > 2) issue(0, 2);
    }
    __syncthreads();
    auto lstep = [&](auto PAR, int64_t ci) __attribute__((always_inline)) {
      constexpr int par = decltype(PAR)::value;  // ci & 1
      constexpr int cur = NBUF == 2 ? par : 0;
      constexpr int rs = par ^ 1;                // register set holding chunk ci+1
      if (NBUF == 2) {
        if (ci + 1 < nch) {
          commit(rs, buf_at(cur ^ 1));
          if (ci + 3 < nch) issue(rs, ci + 3);
        }
        __syncthreads();
      } else {
        __syncthreads();
        if (ci + 1 < nch) {
          commit(rs, buf_at(0));
          if (ci + 3 < nch) issue(rs, ci + 3);
          __syncthreads();
        }
      }
    };
    for (int64_t ci = 0; ci < nch; ci += 2) {
      lstep(std::integral_constant<int, 0>{}, ci);
      if (ci + 1 < nch) lstep(std::integral_constant<int, 1>{}, ci + 1);
    }
  } else {
    // ---- compute waves: initial state
    if (p.h0) {
#pragma unroll
      for (int t = 0; t < NTK; ++t)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) H[t][ii] = p.h0[hbase + (int64_t)(16 * t + 4 * g + ii) * DV + col0 + i];
#pragma unroll
      for (int t = 0; t < NTK; ++t)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          bad |= flag_if(f_nonfinite(H[t][ii]), GDN_ST_NONFINITE_INPUT);
    } else {
#pragma unroll
      for (int t = 0; t < NTK; ++t) H[t] = zero4();
    }
    __syncthreads();
    auto cstep = [&](auto PAR, int64_t ci) __attribute__((always_inline)) {
      constexpr int par = decltype(PAR)::value;
      constexpr int cur = NBUF == 2 ? par : 0;
      compute(buf_at(cur), ci);
      __syncthreads();
      if (NBUF == 1 && ci + 1 < nch) __syncthreads();
    };
    for (int64_t ci = 0; ci < nch; ci += 2) {
      cstep(std::integral_constant<int, 0>{}, ci);
      if (ci + 1 < nch) cstep(std::integral_constant<int, 1>{}, ci + 1);
    }
    if (p.hT) {
#pragma unroll
      for (int t = 0; t < NTK; ++t) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int d = 16 * t + 4 * g + ii;
          bad |= flag_if(f_nonfinite(H[t][ii]), GDN_ST_NONFINITE_OUTPUT);
          p.hT[hbase + (int64_t)d * DV + col0 + i] = H[t][ii];
        }
      }
    }
  }
  if (bad) atomicOr(p.status, bad);
}

// ------------------------------------------------------------ launch -----
// Kernel attributes are set once per instantiation (the first launch); later launches
// reuse them.
template <class Fn>
bool set_lds_once(Fn fn, size_t lds) {
  static bool done = false;
  if (!done) {
    if (hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
        hipSuccess)
      return false;
    done = true;
  }
  return true;
}

template <class Arm, int DK, int C, bool KDA, bool QF32>
gdn_status run(const Plan& pl, const Params& prm, hipStream_t st) {
  if (pl.run_prep && pl.max_slots > 0) {
    if constexpr (KDA) {
      const size_t lds = prep_chan_lds_bytes<Arm, DK>();
      if (!set_lds_once(gdn_prep_chan<Arm, DK, QF32>, lds)) return GDN_E_LAUNCH;
      const int64_t blocks = pl.max_slots * pl.hv;
      hipLaunchKernelGGL((gdn_prep_chan<Arm, DK, QF32>), dim3((unsigned)blocks), dim3(256), lds, st, prm);
    } else {
      const size_t lds = 4 * SolveLds<C>::FLOATS * sizeof(float);
      if (!set_lds_once(gdn_prep_head<Arm, DK, C, QF32>, lds)) return GDN_E_LAUNCH;
      const int64_t blocks = (pl.max_slots * pl.hv + 3) / 4;
      hipLaunchKernelGGL((gdn_prep_head<Arm, DK, C, QF32>), dim3((unsigned)blocks), dim3(256), lds, st, prm);
    }
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  if (pl.run_scan) {
    const size_t lds = scan_lds_bytes<Arm, DK, C>(KDA);
    if (!set_lds_once(gdn_scan<Arm, DK, C, KDA, QF32>, lds)) return GDN_E_LAUNCH;
    const int64_t blocks = (int64_t)pl.n_seq * pl.hv * (pl.dv / 32);
    hipLaunchKernelGGL((gdn_scan<Arm, DK, C, KDA, QF32>), dim3((unsigned)blocks), dim3(256), lds, st, prm);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  return GDN_OK;
}

template <class Arm, int DK, bool QF32>
gdn_status run_dk(const Plan& pl, const Params& prm, hipStream_t st) {
  if (pl.gate_channel) return run<Arm, DK, 32, true, QF32>(pl, prm, st);
  if (pl.chunk == 32) return run<Arm, DK, 32, false, QF32>(pl, prm, st);
  return run<Arm, DK, 64, false, QF32>(pl, prm, st);
}

template <class Arm>
gdn_status run_arm(const Plan& pl, const Params& prm, hipStream_t st) {
  if (pl.qkv_f32) {
    switch (pl.dk) {
      case 32: return run_dk<Arm, 32, true>(pl, prm, st);
      case 64: return run_dk<Arm, 64, true>(pl, prm, st);
      case 128: return run_dk<Arm, 128, true>(pl, prm, st);
      default: return GDN_E_UNSUPPORTED;
    }
  }
  switch (pl.dk) {
    case 32: return run_dk<Arm, 32, false>(pl, prm, st);
    case 64: return run_dk<Arm, 64, false>(pl, prm, st);
    case 128: return run_dk<Arm, 128, false>(pl, prm, st);
    default: return GDN_E_UNSUPPORTED;
  }
}

}  // namespace

gdn_status launch(const Plan& pl, const Params& prm, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (pl.varlen && pl.run_prep) {
    hipLaunchKernelGGL(gdn_chunk_table, dim3(1), dim3(256), 0, st, prm, (int)pl.chunk);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  return pl.arm_f32 ? run_arm<ArmF32>(pl, prm, st) : run_arm<ArmBF16>(pl, prm, st);
}

}  // namespace gdn
