// gdn_decode.hip -- gfx950 kernel of one recurrent step of the gated delta rule: one new
// token per sequence, continuing from a state a prefill (or an earlier step) produced.
//
// Per sequence n and value head h (K-first state H in R^{dk x dv}, key head kh serving h):
//   Hd = D H_in                     D = e^{g} I, or diag(e^{g[c]}) per key channel
//   w  = Hd^T k                     (one dot product over dk per state column)
//   u  = beta (v - w)               the delta the step writes
//   H_out = Hd + k u^T,   o = H_out^T q
// which is the token-serial rule of the stratat.com page "hip: chunk-parallel GDN
// recurrence (WY form), two parity-gated arms" (section "What this is") for a single
// token, with the argument contract of the logismos issue #46 page (K-first immutable
// input state and a separate next state: "Verified implementation boundary" and the
// Sep 8 activity).
//
// State columns are independent: column j needs only H_in[:, j], k, q, v[j] and the
// gate.  A workgroup owns 32 columns of one (n, h): lane (cq, r8) of wave w holds the 4
// columns 4 cq .. 4 cq + 3 of the DK / 32 rows 8 w + r8 + 32 i, so one load instruction
// of a wave reads 8 rows x 128 bytes (whole cache lines).  The two reductions over dk
// run across the 8 row lanes of a wave with lane swaps, then across the 4 waves through
// LDS, in a fixed order (results are bitwise reproducible).  The state is read once and
// written once; everything is fp32.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;

// e^x through the hardware exp2
__device__ __forceinline__ float dexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ uint32_t nonfinite(float x) {
  return (__float_as_uint(x) & 0x7F800000u) == 0x7F800000u;
}

template <bool F32>
__device__ __forceinline__ float load_elem(const void* src, int64_t e) {
  if constexpr (F32) return ((const float*)src)[e];
  return __uint_as_float((uint32_t)((const uint16_t*)src)[e] << 16);
}

// four consecutive elements (16-byte fp32 or 8-byte bf16 aligned) as fp32
template <bool F32>
__device__ __forceinline__ f32x4 load4(const void* src, int64_t e) {
  if constexpr (F32) return *(const f32x4*)((const float*)src + e);
  const uint2 b = *(const uint2*)((const uint16_t*)src + e);
  return (f32x4){__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                 __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u)};
}

__device__ __forceinline__ f32x4 swap_add(f32x4 x, int mask) {
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] += __shfl_xor(x[j], mask, 64);
  return x;
}

// sum over the 8 lanes of a wave that hold the same columns (lanes cq + 8 r8)
__device__ __forceinline__ f32x4 rows_sum(f32x4 x) {
  x = swap_add(x, 8);
  x = swap_add(x, 16);
  return swap_add(x, 32);
}

template <int DK, bool QF32, bool OF32, bool KDA>
__global__ __launch_bounds__(256) void gdn_decode(DecodeParams p) {
  constexpr int RPT = DK / 32;  // state rows per lane
  __shared__ f32x4 red[2][4][8];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cq = lane & 7, r0 = 8 * w + (lane >> 3);
  const int ns = p.dv >> 5;
  const int64_t item = blockIdx.x;
  const int slice = (int)(item % ns);
  const int64_t nh = item / ns;  // n * hv + h
  const int h = (int)(nh % p.hv);
  const int64_t n = nh / p.hv;
  const int kh = h / (p.hv / p.hk);
  const int col = 32 * slice + 4 * cq;
  const int64_t sbase = nh * DK * p.dv + col;
  const int64_t kq = (n * p.hk + kh) * DK;

  // every load first
  f32x4 s[RPT];
  if (p.h_in) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      s[i] = __builtin_nontemporal_load((const f32x4*)(p.h_in + sbase + (int64_t)(r0 + 32 * i) * p.dv));
  } else {
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  float kr[RPT], qr[RPT], gr[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    kr[i] = load_elem<QF32>(p.k, kq + r0 + 32 * i);
    qr[i] = load_elem<QF32>(p.q, kq + r0 + 32 * i);
    gr[i] = KDA ? p.g[nh * DK + r0 + 32 * i] : 0.f;
  }
  const float gh = KDA ? 0.f : p.g[nh];
  const float b = p.beta[nh];
  const f32x4 v = load4<QF32>(p.v, nh * p.dv + col);

  uint32_t bad_in = nonfinite(b) | nonfinite(v[0]) | nonfinite(v[1]) | nonfinite(v[2]) | nonfinite(v[3]);
  uint32_t bad_gate = 0;
  if constexpr (!KDA) {
    bad_in |= nonfinite(gh);
    bad_gate |= gh > 0.f;
  }
  // decay, then the partial dot products Hd^T k over this lane's rows
  const float eh = KDA ? 1.f : dexp(gh);
  f32x4 wp = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    bad_in |= nonfinite(kr[i]) | nonfinite(qr[i]);
    bad_in |= nonfinite(s[i][0]) | nonfinite(s[i][1]) | nonfinite(s[i][2]) | nonfinite(s[i][3]);
    float e = eh;
    if constexpr (KDA) {
      bad_in |= nonfinite(gr[i]);
      bad_gate |= gr[i] > 0.f;
      e = dexp(gr[i]);
    }
    s[i] *= e;
    wp += s[i] * kr[i];
  }
  wp = rows_sum(wp);
  if (lane < 8) red[0][w][cq] = wp;
  __syncthreads();
  const f32x4 wsum = ((red[0][0][cq] + red[0][1][cq]) + red[0][2][cq]) + red[0][3][cq];
  const f32x4 u = b * (v - wsum);

  // write, store the next state, partial outputs H_out^T q
  f32x4 op = (f32x4){0.f, 0.f, 0.f, 0.f};
  uint32_t bad_out = 0;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    s[i] += kr[i] * u;
    __builtin_nontemporal_store(s[i], (f32x4*)(p.h_out + sbase + (int64_t)(r0 + 32 * i) * p.dv));
    bad_out |= nonfinite(s[i][0]) | nonfinite(s[i][1]) | nonfinite(s[i][2]) | nonfinite(s[i][3]);
    op += s[i] * qr[i];
  }
  op = rows_sum(op);
  if (lane < 8) red[1][w][cq] = op;
  __syncthreads();
  if (w == 0 && lane < 8) {
    const f32x4 o = ((red[1][0][cq] + red[1][1][cq]) + red[1][2][cq]) + red[1][3][cq];
    const int64_t oe = nh * p.dv + col;
    if constexpr (OF32) {
      *(f32x4*)((float*)p.o + oe) = o;
    } else {
      uint2 pk;
      pk.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[0]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[1]) << 16);
      pk.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[2]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[3]) << 16);
      *(uint2*)((uint16_t*)p.o + oe) = pk;
    }
    bad_out |= nonfinite(o[0]) | nonfinite(o[1]) | nonfinite(o[2]) | nonfinite(o[3]);
  }
  const uint32_t bits = (bad_in ? GDN_ST_NONFINITE_INPUT : 0u) | (bad_gate ? GDN_ST_GATE_DOMAIN : 0u) |
                        (bad_out ? GDN_ST_NONFINITE_OUTPUT : 0u);
  if (bits) atomicOr(p.status, bits);
}

template <int DK, bool QF32, bool OF32>
gdn_status run_gate(const DecodeParams& prm, bool kda, int64_t blocks, hipStream_t st) {
  if (kda)
    hipLaunchKernelGGL((gdn_decode<DK, QF32, OF32, true>), dim3((unsigned)blocks), dim3(256), 0, st, prm);
  else
    hipLaunchKernelGGL((gdn_decode<DK, QF32, OF32, false>), dim3((unsigned)blocks), dim3(256), 0, st, prm);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_E_LAUNCH;
}

template <int DK>
gdn_status run_decode_dk(const DecodeParams& prm, bool kda, int64_t blocks, hipStream_t st) {
  if (prm.qkv_f32)
    return prm.o_f32 ? run_gate<DK, true, true>(prm, kda, blocks, st) : run_gate<DK, true, false>(prm, kda, blocks, st);
  return prm.o_f32 ? run_gate<DK, false, true>(prm, kda, blocks, st) : run_gate<DK, false, false>(prm, kda, blocks, st);
}

}  // namespace

gdn_status launch_decode(const DecodeParams& prm, int dk, bool kda, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int64_t blocks = (int64_t)prm.n_seq * prm.hv * (prm.dv / 32);
  if (blocks == 0) return GDN_OK;
  switch (dk) {
    case 32: return run_decode_dk<32>(prm, kda, blocks, st);
    case 64: return run_decode_dk<64>(prm, kda, blocks, st);
    case 128: return run_decode_dk<128>(prm, kda, blocks, st);
    default: return GDN_E_UNSUPPORTED;
  }
}

}  // namespace gdn
