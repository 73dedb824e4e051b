// Device-side helpers shared by the gfx950 kernels of the DiT block forward.
//
// Wave size 64.  MFMA v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) of
// A and column (l % 32) of B, each as eight bf16 at k = 8 * (l / 32) .. +7, and
// receives column (l % 32) of the 32x32 fp32 result at rows
// (r / 4) * 8 + (l / 32) * 4 + r % 4, r = 0..15.  v_mfma_f32_16x16x32_bf16:
// lane l supplies row (l % 16) of A and column (l % 16) of B, eight bf16 each at
// k = 8 * (l / 16) .. +7, and receives column (l % 16) of the 16x16 result at
// rows 4 * (l / 16) + r, r = 0..3.  On this chip the 16x16x32 form sustains a
// higher clock under the power cap (measured: 2.09 against 1.76 GHz with dense
// register operands), so the bf16 GEMMs use it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlo {
namespace {


typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// GELU(z) = z * Phi(z) = 0.5 z (1 + erf(z / sqrt 2)), with erfc(x), x = |z| / sqrt 2,
// from Abramowitz & Stegun (1964) formula 7.1.26: erfc(x) = (a1 t + ... + a5 t^5)
// exp(-x^2), t = 1 / (1 + p x), |error in erf| <= 1.5e-7 -- far below the bf16
// rounding of the stored activation, at half the VALU work of the library erff.
// The constants are folded: g = erfc(x) / 2 = (a1' t + ... + a5' t^5)
// exp2(-log2(e) z^2 / 2), ai' = ai / 2, t = 1 / (1 + (p / sqrt 2) |z|).  Then
// z Phi(z) = z - z g for z >= 0 and z g for z < 0, i.e. max(z, 0) - |z g| for
// both signs: 12 VALU instructions, two of them transcendental.
__device__ __forceinline__ float gelu_erf(float z) {
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.2316418882663604f, fabsf(z), 1.0f));
  float poly = __builtin_fmaf(0.5307027145f, t, -0.7265760135f);
  poly = __builtin_fmaf(poly, t, 0.7107068705f);
  poly = __builtin_fmaf(poly, t, -0.142248368f);
  poly = __builtin_fmaf(poly, t, 0.127414796f);
  poly *= t;
  const float g = poly * __builtin_amdgcn_exp2f(z * -0.7213475204444817f * z);
  return fmaxf(z, 0.f) - fabsf(z * g);
}

// XCD-aware tile order.  Workgroup w is dispatched to XCD w % 8; renumber so
// that the workgroups one XCD receives get consecutive logical ids and hence
// neighbouring tiles that share operands in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int NX = 8;
  int x = pid % NX, idx = pid / NX;
  int base = total / NX, rem = total % NX;
  return x * base + (x < rem ? x : rem) + idx;
}

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// The OCP E4M3 code nearest to x: ties to the even code, magnitudes of 448 and
// above saturate to 448, NaN -> 0x7F.  The encoder works on the fp32 exponent
// and a 3-bit mantissa rounded by v_rndne (every scaling by a power of two is
// exact).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  if (x != x) return 0x7Fu;
  const float a = fabsf(x);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f)  // below 2^-6: subnormal steps of 2^-9 (8 steps = the smallest normal)
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;                      // a in [2^E, 2^(E+1))
  const float f = __uint_as_float((__float_as_uint(a) & 0x7FFFFFu) | 0x3F800000u);  // a / 2^E in [1, 2)
  int m = (int)__builtin_rintf(f * 8.0f) - 8;
  if (m == 8) {
    m = 0;
    ++E;
  }
  return sign | (uint32_t)(((E + 7) << 3) | m);
}

// raw buffer descriptor: base, no stride, num_records bytes (reads past it return 0)
__device__ __forceinline__ i32x4 dl_rsrc(const void *base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 B per lane from rsrc + voff into LDS at lds_base + 16 * lane (M0 = lds_base).
// Issued as inline asm so that the compiler does not add its own (over-strict)
// counter waits before the LDS reads; the kernel waits on vmcnt explicitly.
__device__ __forceinline__ void dl_load(i32x4 rsrc, uint32_t lds_base, int voff) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :
               : "v"(voff), "s"(lds_base), "s"(rsrc)
               : "memory");
}

// as dl_load, with a wave-uniform byte offset soff added by the buffer unit
// (the per-lane offset stays loop-invariant)
__device__ __forceinline__ void dl_load_so(i32x4 rsrc, uint32_t lds_base, int voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
               :
               : "v"(voff), "s"(lds_base), "s"(rsrc), "s"(soff)
               : "memory");
}

// 4 B per lane from rsrc + voff + soff into LDS at lds_base + 4 * lane
__device__ __forceinline__ void dl_load_dw_so(i32x4 rsrc, uint32_t lds_base, int voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, %3 offen lds"
               :
               : "v"(voff), "s"(lds_base), "s"(rsrc), "s"(soff)
               : "memory");
}

// s_waitcnt vmcnt(N) then s_barrier (N an immediate)
template <int N>
__device__ __forceinline__ void vmcnt_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace
}  // namespace dlo
