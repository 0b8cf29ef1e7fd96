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

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

extern __shared__ __align__(16) unsigned char gdn_smem[];

constexpr float kLog2e = 1.4426950408889634f;

// e^x through the hardware exp2 (v_exp_f32); e^-inf = 0, large negative x flush to 0.
__device__ __forceinline__ float nexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ bool bf_nonfinite(uint32_t two) {  // either half is Inf/NaN
  return ((two & 0x7F80u) == 0x7F80u) || ((two & 0x7F800000u) == 0x7F800000u);
}
__device__ __forceinline__ bool f_nonfinite(float x) { return !__builtin_isfinite(x); }

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
  __device__ static __forceinline__ F row_half(const T* p0) {
    const float4 a = *(const float4*)p0;
    F f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = 0.f; f.v[5] = 0.f; f.v[6] = 0.f; f.v[7] = 0.f;
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
  __device__ static __forceinline__ F col_half(const T* base, int pitch, int k0, int n0, int lane) {
    const int i = lane & 15, g = lane >> 4;
    F f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.v[j] = base[(k0 + 4 * g + j) * pitch + n0 + i];
      f.v[4 + j] = 0.f;
    }
    return f;
  }
  __device__ static __forceinline__ F acc(f32x4 lo, f32x4 hi) {
    F f;
    f.v[0] = lo[0]; f.v[1] = lo[1]; f.v[2] = lo[2]; f.v[3] = lo[3];
    f.v[4] = hi[0]; f.v[5] = hi[1]; f.v[6] = hi[2]; f.v[7] = hi[3];
    return f;
  }
  __device__ static __forceinline__ F acc_half(f32x4 lo) {
    F f;
    f.v[0] = lo[0]; f.v[1] = lo[1]; f.v[2] = lo[2]; f.v[3] = lo[3];
    f.v[4] = 0.f; f.v[5] = 0.f; f.v[6] = 0.f; f.v[7] = 0.f;
    return f;
  }
  __device__ static __forceinline__ f32x4 mma(const F& a, const F& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
  }
};

// ------------------------------------------------------ global I/O -------
// 8 consecutive input elements (bf16 or fp32 per flag) into 8 LDS elements of the arm.
// Returns true when any of them is not finite.
template <class Arm>
__device__ __forceinline__ bool load8(const void* src, int64_t e, int src_f32, typename Arm::T* dst) {
  bool bad = false;
  if (src_f32) {
    const float4* s = (const float4*)((const float*)src + e);
    const float4 a = s[0], b = s[1];
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) bad |= f_nonfinite(x[j]);
    if constexpr (sizeof(typename Arm::T) == 4) {
      float4* d = (float4*)dst;
      d[0] = a;
      d[1] = b;
    } else {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f2bf(x[2 * j]) | ((uint32_t)f2bf(x[2 * j + 1]) << 16);
      *(uint4*)dst = (uint4){w[0], w[1], w[2], w[3]};
    }
  } else {
    const uint4 a = *(const uint4*)((const uint16_t*)src + e);
    bad = bf_nonfinite(a.x) || bf_nonfinite(a.y) || bf_nonfinite(a.z) || bf_nonfinite(a.w);
    if constexpr (sizeof(typename Arm::T) == 4) {
      float4* d = (float4*)dst;
      d[0] = (float4){__uint_as_float(a.x << 16), __uint_as_float(a.x & 0xFFFF0000u),
                      __uint_as_float(a.y << 16), __uint_as_float(a.y & 0xFFFF0000u)};
      d[1] = (float4){__uint_as_float(a.z << 16), __uint_as_float(a.z & 0xFFFF0000u),
                      __uint_as_float(a.w << 16), __uint_as_float(a.w & 0xFFFF0000u)};
    } else {
      *(uint4*)dst = a;
    }
  }
  return bad;
}

template <class Arm>
__device__ __forceinline__ void zero8(typename Arm::T* dst) {
  if constexpr (sizeof(typename Arm::T) == 4) {
    ((float4*)dst)[0] = (float4){0.f, 0.f, 0.f, 0.f};
    ((float4*)dst)[1] = (float4){0.f, 0.f, 0.f, 0.f};
  } else {
    *(uint4*)dst = (uint4){0u, 0u, 0u, 0u};
  }
}

// one input element as fp32
__device__ __forceinline__ float load1(const void* src, int64_t e, int src_f32) {
  return src_f32 ? ((const float*)src)[e] : bf2f(((const uint16_t*)src)[e]);
}

// 8 input elements as fp32 (v rows)
__device__ __forceinline__ bool load8f(const void* src, int64_t e, int src_f32, float* x) {
  bool bad = false;
  if (src_f32) {
    const float4* s = (const float4*)((const float*)src + e);
    const float4 a = s[0], b = s[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
#pragma unroll
    for (int j = 0; j < 8; ++j) bad |= f_nonfinite(x[j]);
  } else {
    const uint4 a = *(const uint4*)((const uint16_t*)src + e);
    bad = bf_nonfinite(a.x) || bf_nonfinite(a.y) || bf_nonfinite(a.z) || bf_nonfinite(a.w);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  return bad;
}

// 8 arm elements from global (workspace) to LDS
template <class Arm>
__device__ __forceinline__ void copy8(const typename Arm::T* src, typename Arm::T* dst) {
  if constexpr (sizeof(typename Arm::T) == 4) {
    ((float4*)dst)[0] = ((const float4*)src)[0];
    ((float4*)dst)[1] = ((const float4*)src)[1];
  } else {
    *(uint4*)dst = *(const uint4*)src;
  }
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

// ---------------------------------------------------- blocked solve ------
// T = (I + A)^-1 for a strictly lower C x C matrix A (fp32, LDS, pitch C+4):
// 16 x 16 diagonal blocks by forward substitution (one lane per block column),
// then the off-diagonal blocks level by level, T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj,
// on fp32 MFMA (one wave per block of a level).
template <int C>
__device__ void solve_unit_lower(const float* Am, float* Tm, int tid) {
  constexpr int NB = C / 16, AP = C + 4;
  const int lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx / C, s = idx % C;
    if ((s >> 4) > (r >> 4)) Tm[r * AP + s] = 0.f;
  }
  if (w == 0 && lane < 16 * NB) {
    const int base = 16 * (lane >> 4), c = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s_ = (r == c) ? 1.f : 0.f;
      const float* arow = Am + (base + r) * AP + base;
#pragma unroll
      for (int s = 0; s < r; ++s) s_ = fmaf(-arow[s], x[s], s_);
      x[r] = s_;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tm[(base + r) * AP + base + c] = x[r];
  }
  __syncthreads();
#pragma unroll
  for (int dist = 1; dist < NB; ++dist) {
    if (w < NB - dist) {
      const int ib = w + dist, jb = w;
      f32x4 z = zero4();
      for (int m = jb; m < ib; m += 2) {
        const float* arow = Am + (16 * ib + i) * AP;
        if (m + 1 < ib) {
          ArmF32::F a = ArmF32::row(arow + 16 * m + 4 * g, arow + 16 * (m + 1) + 4 * g);
          ArmF32::F b = ArmF32::col(Tm, AP, 16 * m, 16 * jb, lane);
          z = ArmF32::mma(a, b, z);
        } else {
          ArmF32::F a = ArmF32::row_half(arow + 16 * m + 4 * g);
          ArmF32::F b = ArmF32::col_half(Tm, AP, 16 * m, 16 * jb, lane);
          z = ArmF32::mma(a, b, z);
        }
      }
      ArmF32::F a = ArmF32::row_half(Tm + (16 * ib + i) * AP + 16 * ib + 4 * g);
      f32x4 t = ArmF32::mma(a, ArmF32::acc_half(z), zero4());
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Tm[(16 * ib + 4 * g + ii) * AP + 16 * jb + i] = -t[ii];
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------- prep -------
template <class Arm, int DK, int C>
constexpr size_t prep_lds_bytes(bool kda) {
  return (size_t)(kda ? 3 : 2) * C * (DK + Arm::PAD) * sizeof(typename Arm::T)  // operands
         + 2 * (size_t)C * (C + 4) * sizeof(float)                             // A, T (fp32)
         + (size_t)C * C * sizeof(typename Arm::T)                             // P staging
         + 2 * (size_t)C * sizeof(float);                                      // G, beta
}

template <class Arm, int DK, int C, bool KDA>
__global__ __launch_bounds__(256) void gdn_prep(Params p) {
  using T = typename Arm::T;
  using F = typename Arm::F;
  constexpr int NT = C / 16, NBK = DK / 32, KP = DK + Arm::PAD, AP = C + 4;
  constexpr int NTRI = NT * (NT + 1) / 2, NTILE = 2 * NTRI, MAXT = (NTILE + 3) / 4;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int heads = KDA ? p.hv : p.hk;
  const int head = blockIdx.x % heads;
  const int64_t slot = blockIdx.x / heads;
  int n, L;
  int64_t t0;
  if (!locate_chunk(p, C, slot, n, t0, L)) return;
  const int group = p.hv / p.hk;
  const int kh = KDA ? head / group : head;

  T* X0 = (T*)gdn_smem;  // K (scalar gate) or K*e^{G-Gm} (per-channel gate)
  T* X1 = X0 + C * KP;   // Q                or K*e^{Gm-G}
  T* X2 = X1 + C * KP;   // --               or Q*e^{G-Gm}
  float* Am = (float*)(X0 + (KDA ? 3 : 2) * C * KP);
  float* Tm = Am + C * AP;
  T* Pst = (T*)(Tm + C * AP);
  float* Gs = (float*)(Pst + C * C);
  float* Bs = Gs + C;
  uint32_t bad = 0;

  if constexpr (!KDA) {
    for (int idx = tid; idx < C * DK / 8; idx += 256) {
      const int r = idx / (DK / 8), c8 = idx % (DK / 8);
      T* dk_ = X0 + r * KP + 8 * c8;
      T* dq_ = X1 + r * KP + 8 * c8;
      if (r < L) {
        const int64_t e = ((t0 + r) * p.hk + kh) * (int64_t)DK + 8 * c8;
        const bool bk = load8<Arm>(p.k, e, p.qkv_f32, dk_);
        const bool bq = load8<Arm>(p.q, e, p.qkv_f32, dq_);
        if (bk || bq) bad |= GDN_ST_NONFINITE_INPUT;
      } else {
        zero8<Arm>(dk_);
        zero8<Arm>(dq_);
      }
    }
  } else {
    // per-channel gate: one thread per key channel walks the chunk rows; factors are
    // split around the middle row m so every stored factor stays <= e^80 (gate >= -5,
    // C = 32); exponent arguments are clamped, masked entries removed by select below.
    const int hv = head;
    if (tid < DK) {
      const int d = tid;
      float G[C];
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < C; ++r) {
        float x = 0.f;
        if (r < L) {
          x = p.g[((t0 + r) * p.hv + hv) * (int64_t)DK + d];
          if (f_nonfinite(x)) bad |= GDN_ST_NONFINITE_INPUT;
          else if (x > 0.f || x < -5.f) bad |= GDN_ST_GATE_DOMAIN;
        }
        acc += x;
        G[r] = acc;
      }
      const float Gm = G[C / 2];
#pragma unroll
      for (int r = 0; r < C; ++r) {
        float kf = 0.f, qf = 0.f;
        if (r < L) {
          const int64_t e = ((t0 + r) * p.hk + kh) * (int64_t)DK + d;
          kf = load1(p.k, e, p.qkv_f32);
          qf = load1(p.q, e, p.qkv_f32);
          if (f_nonfinite(kf) || f_nonfinite(qf)) bad |= GDN_ST_NONFINITE_INPUT;
        }
        const float up = nexp(fminf(G[r] - Gm, 85.f)), dn = nexp(fminf(Gm - G[r], 85.f));
        X0[r * KP + d] = Arm::cvt(kf * up);
        X1[r * KP + d] = Arm::cvt(kf * dn);
        X2[r * KP + d] = Arm::cvt(qf * up);
      }
    }
  }
  __syncthreads();

  // Products on MFMA: tile list = lower tiles (rt >= st) of the two C x C products.
  // scalar gate: KK^T and QK^T;  per-channel gate: Kup Kdn^T and Qup Kdn^T.
  f32x4 acc[MAXT];
#pragma unroll
  for (int j = 0; j < MAXT; ++j) {
    acc[j] = zero4();
    const int tix = w + 4 * j;
    if (tix < NTILE) {
      const int which = tix / NTRI;
      int t = tix % NTRI, rt = 0;
      while (t > rt) { t -= rt + 1; ++rt; }
      const int st = t;
      const T* Am_ = which ? (KDA ? X2 : X1) : X0;
      const T* Bm_ = KDA ? X1 : X0;
      const T* arow = Am_ + (16 * rt + i) * KP;
      const T* brow = Bm_ + (16 * st + i) * KP;
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb) {
        F a = Arm::row(arow + 32 * kb + 4 * g, arow + 32 * kb + 16 + 4 * g);
        F b = Arm::row(brow + 32 * kb + 4 * g, brow + 32 * kb + 16 + 4 * g);
        acc[j] = Arm::mma(a, b, acc[j]);
      }
    }
  }

  const int nheads = KDA ? 1 : group;
  for (int jh = 0; jh < nheads; ++jh) {
    const int hv = KDA ? head : kh * group + jh;
    if (w == 0) {
      const int r = lane;
      float x = 0.f, b = 0.f;
      if (r < L) {
        const int64_t e = (t0 + r) * p.hv + hv;
        b = p.beta[e];
        if (f_nonfinite(b)) bad |= GDN_ST_NONFINITE_INPUT;
        if constexpr (!KDA) {
          x = p.g[e];
          if (f_nonfinite(x)) bad |= GDN_ST_NONFINITE_INPUT;
          else if (x > 0.f) bad |= GDN_ST_GATE_DOMAIN;
        }
      }
      const float G = wave_prefix_sum(x, lane);
      if (r < C) {
        Gs[r] = G;
        Bs[r] = b;
      }
    }
    __syncthreads();
    // A (strictly lower, beta-scaled) and P (lower with diagonal) from the accumulators
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      const int tix = w + 4 * j;
      if (tix < NTILE) {
        const int which = tix / NTRI;
        int t = tix % NTRI, rt = 0;
        while (t > rt) { t -= rt + 1; ++rt; }
        const int st = t;
        const int s = 16 * st + i;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * g + ii;
          float val;
          if constexpr (KDA) {
            val = acc[j][ii];
          } else {
            val = (s <= r) ? nexp(Gs[r] - Gs[s]) * acc[j][ii] : 0.f;
          }
          if (which == 0)
            Am[r * AP + s] = (s < r) ? Bs[r] * val : 0.f;
          else
            Pst[r * C + s] = Arm::cvt((s <= r) ? val : 0.f);
        }
      }
    }
    for (int idx = tid; idx < C * C; idx += 256) {  // tiles above the diagonal
      const int r = idx / C, s = idx % C;
      if ((s >> 4) > (r >> 4)) {
        Am[r * AP + s] = 0.f;
        Pst[r * C + s] = Arm::cvt(0.f);
      }
    }
    __syncthreads();
    T* Pg = (T*)p.Pws + (slot * p.hv + hv) * (int64_t)(C * C);
    for (int idx = tid; idx < C * C / 8; idx += 256) copy8<Arm>(Pst + 8 * idx, Pg + 8 * idx);
    solve_unit_lower<C>(Am, Tm, tid);
    T* Tg = (T*)p.Tws + (slot * p.hv + hv) * (int64_t)(C * C);
    for (int idx = tid; idx < C * C; idx += 256) {
      const int r = idx / C, s = idx % C;
      Tg[idx] = Arm::cvt(Tm[r * AP + s]);
    }
    __syncthreads();
  }
  if (bad) atomicOr(p.status, bad);
}

// ----------------------------------------------------------- scan -------
template <class Arm, int DK, int C>
constexpr size_t scan_lds_bytes(bool kda) {
  return (size_t)(kda ? 3 : 2) * C * (DK + Arm::PAD) * sizeof(typename Arm::T)  // K [, K~], Q
         + 2 * (size_t)C * (C + Arm::PAD) * sizeof(typename Arm::T)            // T, P
         + (size_t)C * 36 * sizeof(float)                                      // V (32 columns)
         + (4 * (size_t)C + DK + 4) * sizeof(float);                           // row scalars
}

template <class Arm, int DK, int C, bool KDA>
__global__ __launch_bounds__(128) void gdn_scan(Params p) {
  using T = typename Arm::T;
  using F = typename Arm::F;
  constexpr int NT = C / 16, NBC = C / 32, NTK = DK / 16, NBK = DK / 32;
  constexpr int KP = DK + Arm::PAD, CP = C + Arm::PAD, VP = 36;
  const int tid = threadIdx.x, lane = tid & 63, u = tid >> 6, i = lane & 15, g = lane >> 4;
  const int DV = p.dv, nslice = DV / 32;
  int bid = blockIdx.x;
  const int slice = bid % nslice;
  bid /= nslice;
  const int h = bid % p.hv;
  const int n = bid / p.hv;
  const int kh = h / (p.hv / p.hk);
  const int col0 = 32 * slice + 16 * u;  // first value column of this wave

  T* Ks = (T*)gdn_smem;                   // K (scalar gate) or beta e^{G} K (per channel)
  T* Kl = KDA ? Ks + C * KP : Ks;         // per channel: e^{G_C - G} K
  T* Qs = Ks + (KDA ? 2 : 1) * C * KP;    // Q or e^{G} Q
  T* Ts = Qs + C * KP;
  T* Ps = Ts + C * CP;
  float* Vs = (float*)(Ps + C * CP);
  float* sb_ = Vs + C * VP;  // beta
  float* sbe = sb_ + C;      // beta e^{G}
  float* seg = sbe + C;      // e^{G}
  float* sel = seg + C;      // e^{G_C - G}
  float* sdec = sel + C;     // e^{G_C} per key channel (per-channel gate) / [0] scalar

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
  uint32_t bad = 0;

  f32x4 H[NTK];
  const int64_t hbase = ((int64_t)n * p.hv + h) * DK * (int64_t)DV;
#pragma unroll
  for (int t = 0; t < NTK; ++t) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d = 16 * t + 4 * g + ii;
      float x = 0.f;
      if (p.h0) {
        x = p.h0[hbase + (int64_t)d * DV + col0 + i];
        if (f_nonfinite(x)) bad |= GDN_ST_NONFINITE_INPUT;
      }
      H[t][ii] = x;
    }
  }

  const int64_t nch = (s1 - s0 + C - 1) / C;
  for (int64_t ci = 0; ci < nch; ++ci) {
    const int64_t t0 = s0 + ci * C;
    const int L = (int)min64(C, s1 - t0);
    const int64_t slot = slot0 + ci;
    // ---- fill: gate scalars, operands, T, P, V
    if constexpr (!KDA) {
      if (u == 0) {
        const int r = lane;
        float x = 0.f, b = 0.f;
        if (r < L) {
          const int64_t e = (t0 + r) * p.hv + h;
          x = p.g[e];
          b = p.beta[e];
        }
        const float G = wave_prefix_sum(x, lane);
        const float GC = __shfl(G, C - 1, 64);
        if (r < C) {
          const float eg = nexp(G);
          sb_[r] = b;
          sbe[r] = b * eg;
          seg[r] = eg;
          sel[r] = nexp(GC - G);
        }
        if (r == 0) sdec[0] = nexp(GC);
      }
      for (int idx = tid; idx < C * DK / 8; idx += 128) {
        const int r = idx / (DK / 8), c8 = idx % (DK / 8);
        T* dk_ = Ks + r * KP + 8 * c8;
        T* dq_ = Qs + r * KP + 8 * c8;
        if (r < L) {
          const int64_t e = ((t0 + r) * p.hk + kh) * (int64_t)DK + 8 * c8;
          load8<Arm>(p.k, e, p.qkv_f32, dk_);
          load8<Arm>(p.q, e, p.qkv_f32, dq_);
        } else {
          zero8<Arm>(dk_);
          zero8<Arm>(dq_);
        }
      }
    } else {
      if (u == 0) {
        const int r = lane;
        if (r < C) sb_[r] = (r < L) ? p.beta[(t0 + r) * p.hv + h] : 0.f;
      }
      if (tid < DK) {
        const int d = tid;
        float G[C];
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
          acc += (r < L) ? p.g[((t0 + r) * p.hv + h) * (int64_t)DK + d] : 0.f;
          G[r] = acc;
        }
        const float GC = acc;
        sdec[d] = nexp(GC);
#pragma unroll
        for (int r = 0; r < C; ++r) {
          float kf = 0.f, qf = 0.f, b = 0.f;
          if (r < L) {
            const int64_t e = ((t0 + r) * p.hk + kh) * (int64_t)DK + d;
            kf = load1(p.k, e, p.qkv_f32);
            qf = load1(p.q, e, p.qkv_f32);
            b = p.beta[(t0 + r) * p.hv + h];
          }
          const float eg = nexp(G[r]);
          Ks[r * KP + d] = Arm::cvt(b * eg * kf);
          Kl[r * KP + d] = Arm::cvt(nexp(GC - G[r]) * kf);
          Qs[r * KP + d] = Arm::cvt(eg * qf);
        }
      }
    }
    {
      const T* Tg = (const T*)p.Tws + (slot * p.hv + h) * (int64_t)(C * C);
      const T* Pg = (const T*)p.Pws + (slot * p.hv + h) * (int64_t)(C * C);
      for (int idx = tid; idx < C * C / 8; idx += 128) {
        const int r = idx / (C / 8), c8 = idx % (C / 8);
        copy8<Arm>(Tg + 8 * idx, Ts + r * CP + 8 * c8);
        copy8<Arm>(Pg + 8 * idx, Ps + r * CP + 8 * c8);
      }
      for (int idx = tid; idx < C * 4; idx += 128) {
        const int r = idx >> 2, c8 = idx & 3;
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (r < L) {
          if (load8f(p.v, ((t0 + r) * p.hv + h) * (int64_t)DV + 32 * slice + 8 * c8, p.qkv_f32, x))
            bad |= GDN_ST_NONFINITE_INPUT;
        }
        float4* vd = (float4*)(Vs + r * VP + 8 * c8);
        vd[0] = (float4){x[0], x[1], x[2], x[3]};
        vd[1] = (float4){x[4], x[5], x[6], x[7]};
      }
    }
    __syncthreads();

    // ---- chunk step for this wave's 16 state columns
    F HB[NBK];
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb) HB[kb] = Arm::acc(H[2 * kb], H[2 * kb + 1]);

    // Y = K H ;  X = beta V - beta e^{G} Y   (rows r = 16 mt + 4 g + ii)
    f32x4 X[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      f32x4 y = zero4();
      const T* krow = Ks + (16 * mt + i) * KP;
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb)
        y = Arm::mma(Arm::row(krow + 32 * kb + 4 * g, krow + 32 * kb + 16 + 4 * g), HB[kb], y);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * mt + 4 * g + ii;
        const float ys = KDA ? y[ii] : sbe[r] * y[ii];
        X[mt][ii] = sb_[r] * Vs[r * VP + 16 * u + i] - ys;
      }
    }
    F XB[NBC];
#pragma unroll
    for (int sb = 0; sb < NBC; ++sb) XB[sb] = Arm::acc(X[2 * sb], X[2 * sb + 1]);

    // R = T X   (T lower triangular: s-blocks above the row tile are skipped)
    f32x4 R[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      R[mt] = zero4();
      const T* trow = Ts + (16 * mt + i) * CP;
#pragma unroll
      for (int sb = 0; sb < NBC; ++sb)
        if (32 * sb <= 16 * mt + 15)
          R[mt] = Arm::mma(Arm::row(trow + 32 * sb + 4 * g, trow + 32 * sb + 16 + 4 * g), XB[sb], R[mt]);
    }
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
          lo[ii] = sel[32 * sb + 4 * g + ii] * R[2 * sb][ii];
          hi[ii] = sel[32 * sb + 16 + 4 * g + ii] * R[2 * sb + 1][ii];
        }
        RS[sb] = Arm::acc(lo, hi);
      }
    }

    // O^T = H^T (Q e^{G})^T + R^T P^T: lane holds 4 consecutive value columns of one row
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 o = zero4();
      const T* qrow = Qs + (16 * nt + i) * KP;
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb)
        o = Arm::mma(HB[kb], Arm::row(qrow + 32 * kb + 4 * g, qrow + 32 * kb + 16 + 4 * g), o);
      const int r = 16 * nt + i;
      if constexpr (!KDA) {
        const float e = seg[r];
        o[0] *= e; o[1] *= e; o[2] *= e; o[3] *= e;
      }
      const T* prow = Ps + r * CP;
#pragma unroll
      for (int sb = 0; sb < NBC; ++sb)
        if (32 * sb <= 16 * nt + 15)
          o = Arm::mma(RO[sb], Arm::row(prow + 32 * sb + 4 * g, prow + 32 * sb + 16 + 4 * g), o);
      if (r < L) {
        if (f_nonfinite(o[0]) || f_nonfinite(o[1]) || f_nonfinite(o[2]) || f_nonfinite(o[3]))
          bad |= GDN_ST_NONFINITE_OUTPUT;
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

    // H <- e^{G_C} H + Ktil^T R   (Ktil^T read through the transposing LDS path)
#pragma unroll
    for (int t = 0; t < NTK; ++t) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) H[t][ii] *= KDA ? sdec[16 * t + 4 * g + ii] : sdec[0];
#pragma unroll
      for (int sb = 0; sb < NBC; ++sb) H[t] = Arm::mma(Arm::col(Kl, KP, 32 * sb, 16 * t, lane), RS[sb], H[t]);
    }
    __syncthreads();
  }

  if (p.hT) {
#pragma unroll
    for (int t = 0; t < NTK; ++t) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d = 16 * t + 4 * g + ii;
        if (f_nonfinite(H[t][ii])) bad |= GDN_ST_NONFINITE_OUTPUT;
        p.hT[hbase + (int64_t)d * DV + col0 + i] = H[t][ii];
      }
    }
  }
  if (bad) atomicOr(p.status, bad);
}

// ------------------------------------------------------------ launch -----
template <class Arm, int DK, int C, bool KDA>
gdn_status run(const Plan& pl, const Params& prm, hipStream_t st) {
  if (pl.max_slots > 0) {
    const size_t lds = prep_lds_bytes<Arm, DK, C>(KDA);
    const void* fn = (const void*)gdn_prep<Arm, DK, C, KDA>;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return GDN_E_LAUNCH;
    const int64_t blocks = pl.max_slots * (KDA ? pl.hv : pl.hk);
    hipLaunchKernelGGL((gdn_prep<Arm, DK, C, KDA>), dim3((unsigned)blocks), dim3(256), lds, st, prm);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  {
    const size_t lds = scan_lds_bytes<Arm, DK, C>(KDA);
    const void* fn = (const void*)gdn_scan<Arm, DK, C, KDA>;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return GDN_E_LAUNCH;
    const int64_t blocks = (int64_t)pl.n_seq * pl.hv * (pl.dv / 32);
    hipLaunchKernelGGL((gdn_scan<Arm, DK, C, KDA>), dim3((unsigned)blocks), dim3(128), lds, st, prm);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  return GDN_OK;
}

template <class Arm, int DK>
gdn_status run_dk(const Plan& pl, const Params& prm, hipStream_t st) {
  if (pl.gate_channel) return run<Arm, DK, 32, true>(pl, prm, st);
  if (pl.chunk == 32) return run<Arm, DK, 32, false>(pl, prm, st);
  return run<Arm, DK, 64, false>(pl, prm, st);
}

template <class Arm>
gdn_status run_arm(const Plan& pl, const Params& prm, hipStream_t st) {
  switch (pl.dk) {
    case 32: return run_dk<Arm, 32>(pl, prm, st);
    case 64: return run_dk<Arm, 64>(pl, prm, st);
    case 128: return run_dk<Arm, 128>(pl, prm, st);
    default: return GDN_E_UNSUPPORTED;
  }
}

}  // namespace

gdn_status launch(const Plan& pl, const Params& prm, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (pl.varlen) {
    hipLaunchKernelGGL(gdn_chunk_table, dim3(1), dim3(256), 0, st, prm, (int)pl.chunk);
    if (hipGetLastError() != hipSuccess) return GDN_E_LAUNCH;
  }
  return pl.arm_f32 ? run_arm<ArmF32>(pl, prm, st) : run_arm<ArmBF16>(pl, prm, st);
}

}  // namespace gdn
