// gfx950 (CDNA4) kernels of the DiT block forward and the slot digest.
//
// Block math: adaLN-Zero DiT block (adaLN 6-way modulation, LayerNorm, fused
// QKV, softmax attention, output projection, 4d GELU MLP, gated residuals) --
// the block a DiT stack streamed by the method in "Distributed Layerwise
// Offload" (vLLM-Omni blog) runs unchanged.  Operand layout: weights are
// [out, in] row-major, so every GEMM is C = A B^T with both operands contiguous
// along K.
//
//
// This file: the small kernels (SiLU, adaLN GEMV, LayerNorm + modulation) and
// the slot digest.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace dlo {
namespace {

// ---------------------------------------------------------------------------
// elementwise / small kernels
// ---------------------------------------------------------------------------

__global__ void silu_kernel(const float *__restrict__ c, float *__restrict__ out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    float v = c[i];
    out[i] = v / (1.0f + __expf(-v));
  }
}

// One wave per output row; each lane reads 16 B of the row per step.
__global__ __launch_bounds__(256) void adaln_gemv_kernel(const uint16_t *__restrict__ W,
                                                         const float *__restrict__ sc,
                                                         const float *__restrict__ b,
                                                         float *__restrict__ out, int rows,
                                                         int d) {
  const int lane = threadIdx.x % WAVE;
  const int row = blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  if (row >= rows) return;
  const uint16_t *w = W + (int64_t)row * d;
  float acc = 0.f;
  for (int c = lane * 8; c < d; c += WAVE * 8) {
    u32x4 q = *reinterpret_cast<const u32x4 *>(w + c);
    float4 s0 = *reinterpret_cast<const float4 *>(sc + c);
    float4 s1 = *reinterpret_cast<const float4 *>(sc + c + 4);
    acc += __uint_as_float(q[0] << 16) * s0.x + __uint_as_float(q[0] & 0xffff0000u) * s0.y;
    acc += __uint_as_float(q[1] << 16) * s0.z + __uint_as_float(q[1] & 0xffff0000u) * s0.w;
    acc += __uint_as_float(q[2] << 16) * s1.x + __uint_as_float(q[2] & 0xffff0000u) * s1.y;
    acc += __uint_as_float(q[3] << 16) * s1.z + __uint_as_float(q[3] & 0xffff0000u) * s1.w;
  }
  acc = wave_sum(acc);
  if (lane == 0) out[row] = acc + b[row];
}

// The same GEMV for d % 512 == 0 (NCH = d / 512 16-B chunks per lane): each
// wave keeps its lanes' share of silu(c) in registers and takes rows row,
// row + (waves in the grid), ..., issuing all NCH loads of a row before its
// sums, with a grid of as many workgroups as are resident at once.  The
// per-lane order of summation is adaln_gemv_kernel's (bit-identical results);
// the row loop saves the re-reads of silu(c) and puts NCH loads in flight per
// wave (Super shape, 315 MB: 58 -> 50 us, 6.3 TB/s).
template <int NCH>
__global__ __launch_bounds__(256) void adaln_gemv_rows_kernel(const uint16_t *__restrict__ W,
                                                              const float *__restrict__ sc,
                                                              const float *__restrict__ b,
                                                              float *__restrict__ out, int rows, int d) {
  const int lane = threadIdx.x % WAVE;
  const int nw = gridDim.x * 4;
  float4 s[2 * NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (lane + WAVE * j) * 8;
    s[2 * j] = *reinterpret_cast<const float4 *>(sc + c);
    s[2 * j + 1] = *reinterpret_cast<const float4 *>(sc + c + 4);
  }
  for (int row = blockIdx.x * 4 + threadIdx.x / WAVE; row < rows; row += nw) {
    const uint16_t *w = W + (int64_t)row * d;
    u32x4 q[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) q[j] = *reinterpret_cast<const u32x4 *>(w + (lane + WAVE * j) * 8);
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const float4 s0 = s[2 * j], s1 = s[2 * j + 1];
      acc += __uint_as_float(q[j][0] << 16) * s0.x + __uint_as_float(q[j][0] & 0xffff0000u) * s0.y;
      acc += __uint_as_float(q[j][1] << 16) * s0.z + __uint_as_float(q[j][1] & 0xffff0000u) * s0.w;
      acc += __uint_as_float(q[j][2] << 16) * s1.x + __uint_as_float(q[j][2] & 0xffff0000u) * s1.y;
      acc += __uint_as_float(q[j][3] << 16) * s1.z + __uint_as_float(q[j][3] & 0xffff0000u) * s1.w;
    }
    acc = wave_sum(acc);
    if (lane == 0) out[row] = acc + b[row];
  }
}

// The same GEMV on an FP8 block's E4M3 codes: each lane decodes 16 codes per
// step (exact in fp32), and the per-tensor scale multiplies the row's sum, so
// the weights enter as code value * scale with no bf16 rounding.
__global__ __launch_bounds__(256) void adaln_gemv_fp8_kernel(const uint8_t *__restrict__ W,
                                                             const float *__restrict__ wscale,
                                                             const float *__restrict__ sc,
                                                             const float *__restrict__ b,
                                                             float *__restrict__ out, int rows, int d) {
  const int lane = threadIdx.x % WAVE;
  const int row = blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  if (row >= rows) return;
  const uint8_t *w = W + (int64_t)row * d;
  float acc = 0.f;
  for (int c = lane * 16; c < d; c += WAVE * 16) {
    const u32x4 q = *reinterpret_cast<const u32x4 *>(w + c);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[k], false);  // codes c + 4k, c + 4k + 1
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[k], true);   // codes c + 4k + 2, + 3
      const float4 s4 = *reinterpret_cast<const float4 *>(sc + c + 4 * k);
      acc += lo[0] * s4.x + lo[1] * s4.y;
      acc += hi[0] * s4.z + hi[1] * s4.w;
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) out[row] = acc * *wscale + b[row];
}

// The LayerNorm row statistics of both LN kernels (one order of summation, so
// that the two round alike): each thread sums its float4 chunks, then the wave,
// then the four waves' partials in order; the variance in a second pass over
// the registers (chunks at or past d4 hold zeros and are skipped there).
// Two barriers; red is reused by the next row only after the second.
template <int NC>
__device__ __forceinline__ void ln_stats(const float4 (&v)[NC], int d4, float inv_d, float eps,
                                         float (&red)[2][4], float &mean, float &rstd) {
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  s = wave_sum(s);
  if (lane == 0) red[0][wv] = s;
  __syncthreads();
  mean = (red[0][0] + red[0][1] + red[0][2] + red[0][3]) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (tid + 256 * i < d4) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, e = v[i].w - mean;
      q += (a * a + b * b) + (c * c + e * e);
    }
  }
  q = wave_sum(q);
  if (lane == 0) red[1][wv] = q;
  __syncthreads();
  const float var = (red[1][0] + red[1][1] + red[1][2] + red[1][3]) * inv_d;
  rstd = 1.0f / sqrtf(var + eps);
}

// (LN(x) * gamma + beta) * (1 + scale) + shift on four columns; sc holds 1 + scale
__device__ __forceinline__ float4 ln_mod4(float4 v, float mean, float rstd, float4 g, float4 b, float4 sc,
                                          float4 sh) {
  float4 y;
  y.x = ((v.x - mean) * rstd * g.x + b.x) * sc.x + sh.x;
  y.y = ((v.y - mean) * rstd * g.y + b.y) * sc.y + sh.y;
  y.z = ((v.z - mean) * rstd * g.z + b.z) * sc.z + sh.z;
  y.w = ((v.w - mean) * rstd * g.w + b.w) * sc.w + sh.w;
  return y;
}

// the fp32 value of bf16(f), round to nearest even
__device__ __forceinline__ float bf16_round(float f) { return __uint_as_float((uint32_t)f32_to_bf16(f) << 16); }

// LayerNorm + modulate, h = bf16(LN(x[t, :d]) * (1 + scale) + shift), with
// several rows per workgroup: thread t owns the float4 column chunks t + 256 i
// (i < NC); the four per-column vectors (gamma, beta, 1 + scale, shift) are
// loaded once into registers and reused for every row the workgroup takes
// (rows blockIdx.x, + gridDim.x, ...), so the parameters cost one read per
// workgroup instead of one per row; the next row's x is loaded before the
// current row's reductions; 16-B loads, 8-B bf16x4 stores.
template <int NC>
__global__ __launch_bounds__(256) void ln_rows_kernel(const float *__restrict__ x, int64_t ldx, int T, int d,
                                                      const float *__restrict__ gamma, const float *__restrict__ beta,
                                                      const float *__restrict__ eps_p, const float *__restrict__ shift,
                                                      const float *__restrict__ scale, uint16_t *__restrict__ out) {
  __shared__ float red[2][4];
  const int tid = threadIdx.x;
  const int d4 = d / 4;
  float4 g[NC], b[NC], sc[NC], sh[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = 4 * (tid + 256 * i);
    if (c < d) {   // 4-B aligned parameters: four scalar loads
      g[i] = make_float4(gamma[c], gamma[c + 1], gamma[c + 2], gamma[c + 3]);
      b[i] = make_float4(beta[c], beta[c + 1], beta[c + 2], beta[c + 3]);
      sc[i] = make_float4(1.0f + scale[c], 1.0f + scale[c + 1], 1.0f + scale[c + 2], 1.0f + scale[c + 3]);
      sh[i] = make_float4(shift[c], shift[c + 1], shift[c + 2], shift[c + 3]);
    }
  }
  const float eps = eps_p[0];
  const float inv_d = 1.0f / (float)d;
  int row = blockIdx.x;
  float4 v[NC];
  auto load = [&](int r, float4 (&dst)[NC]) {
    const float4 *xr = reinterpret_cast<const float4 *>(x + (int64_t)r * ldx);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c4 = tid + 256 * i;
      dst[i] = (r < T && c4 < d4) ? xr[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load(row, v);
  for (; row < T; row += gridDim.x) {
    float4 vn[NC];
    load(row + gridDim.x, vn);
    float mean, rstd;
    ln_stats<NC>(v, d4, inv_d, eps, red, mean, rstd);
    uint16_t *orow = out + (int64_t)row * d;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c4 = tid + 256 * i;
      if (c4 < d4) {
        const float4 y = ln_mod4(v[i], mean, rstd, g[i], b[i], sc[i], sh[i]);
        bf16x4 o;
        o[0] = (__bf16)y.x;
        o[1] = (__bf16)y.y;
        o[2] = (__bf16)y.z;
        o[3] = (__bf16)y.w;
        *reinterpret_cast<bf16x4 *>(orow + 4 * c4) = o;
      }
      v[i] = vn[i];
    }
  }
}


// ---------------------------------------------------------------------------
// Sustained MFMA rate (measurement): every wave keeps independent accumulator
// chains busy with dense bf16 products of register operands (the values of
// `in`, random-looking bits, so the datapath toggles as in real work), no
// memory traffic in the loop.  The time per FLOP of this kernel is the chip's
// practical bf16 roofline under its power limit, for either MFMA shape.
// ---------------------------------------------------------------------------

template <int FORM>
__global__ __launch_bounds__(512, 1) void mfma_rate_kernel(const bf16x8 *__restrict__ in, float *__restrict__ out,
                                                           int iters) {
  const int t = blockIdx.x * 512 + threadIdx.x;
  const bf16x8 a = in[t % 4096], b = in[(t + 1234) % 4096];
  float sum = 0.f;
  if constexpr (FORM == 0) {   // 8 chains of v_mfma_f32_32x32x16_bf16
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[i][r];
  } else {   // 16 chains of v_mfma_f32_16x16x32_bf16: the same FLOPs per iteration
    f32x4 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum += acc[i][r];
  }
  out[t] = sum;
}


// ---------------------------------------------------------------------------
// slot digest
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void fill_u64_kernel(uint64_t *p, int n, uint64_t v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void digest_kernel(const uint8_t *__restrict__ base, int64_t off,
                                                     int64_t len, uint64_t *__restrict__ out) {
  const int64_t nw = (len + 7) / 8;
  uint64_t acc = 0;
  const uint64_t w0 = (uint64_t)(off / 8);
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nw;
       w += (int64_t)gridDim.x * blockDim.x) {
    uint64_t word;
    const int64_t bo = off + 8 * w;
    if (8 * w + 8 <= len) {
      word = *reinterpret_cast<const uint64_t *>(base + bo);
    } else {
      word = 0;
      for (int64_t b = 0; 8 * w + b < len; ++b) word |= (uint64_t)base[bo + b] << (8 * b);
    }
    acc += mix64(word + (w0 + (uint64_t)w) * 0x9E3779B97F4A7C15ull);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = (uint32_t)acc, hi = (uint32_t)(acc >> 32);
    lo = __shfl_xor(lo, o, WAVE);
    hi = __shfl_xor(hi, o, WAVE);
    acc += ((uint64_t)hi << 32) | lo;
  }
  if ((threadIdx.x % WAVE) == 0) atomicAdd((unsigned long long *)out, (unsigned long long)acc);
}


// ---------------------------------------------------------------------------
// FP8 weights: E4M3 codes -> bf16(code value * scale).  gfx950's
// v_cvt_pk_f32_fp8 decodes OCP E4M3 exactly to fp32; one fp32 multiply and a
// round-to-nearest-even to bf16 follow.  16 codes per thread: one 16-B load,
// two 16-B stores.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint32_t *__restrict__ codes,
                                                          const float *__restrict__ scale,
                                                          u32x4 *__restrict__ out, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const float sc = *scale;
  const u32x4 w = *reinterpret_cast<const u32x4 *>(codes + 4 * i);
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);  // bytes 0, 1
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);   // bytes 2, 3
    o[2 * k] = (uint32_t)f32_to_bf16(lo[0] * sc) | ((uint32_t)f32_to_bf16(lo[1] * sc) << 16);
    o[2 * k + 1] = (uint32_t)f32_to_bf16(hi[0] * sc) | ((uint32_t)f32_to_bf16(hi[1] * sc) << 16);
  }
  out[2 * i] = u32x4{o[0], o[1], o[2], o[3]};
  out[2 * i + 1] = u32x4{o[4], o[5], o[6], o[7]};
}

// INT8 weights ([Doc] "Request and loading constraints": online INT8 keeps an
// int8 weight and an fp32 scale, here one per output row): bf16(code * scale_r),
// round to nearest even.  16 codes per thread, all in one row (cols % 16 == 0).
__global__ __launch_bounds__(256) void dequant_int8_kernel(const u32x4 *__restrict__ codes,
                                                          const float *__restrict__ scales, int64_t cols16,
                                                          u32x4 *__restrict__ out, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const float sc = scales[i / cols16];
  const u32x4 w = codes[i];
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float v0 = (float)(int8_t)(w[k] & 0xFF), v1 = (float)(int8_t)((w[k] >> 8) & 0xFF);
    const float v2 = (float)(int8_t)((w[k] >> 16) & 0xFF), v3 = (float)(int8_t)(w[k] >> 24);
    o[2 * k] = (uint32_t)f32_to_bf16(v0 * sc) | ((uint32_t)f32_to_bf16(v1 * sc) << 16);
    o[2 * k + 1] = (uint32_t)f32_to_bf16(v2 * sc) | ((uint32_t)f32_to_bf16(v3 * sc) << 16);
  }
  out[2 * i] = u32x4{o[0], o[1], o[2], o[3]};
  out[2 * i + 1] = u32x4{o[4], o[5], o[6], o[7]};
}

// MXFP8 weights (same passage: an fp8 weight and an e8m0 block scale, here one
// per 32 consecutive elements of a row, stored block-major [cols / 32, rows]):
// code value * 2^(e - 127); the product is exact in fp32 and fits bf16's 8-bit
// significand, so the rounding never changes it for scales of normal range.
// E8M0 byte 255 is NaN, 0 is 2^-127.  16 codes per thread, all in one block.
__global__ __launch_bounds__(256) void dequant_mxfp8_kernel(const u32x4 *__restrict__ codes,
                                                           const uint8_t *__restrict__ scales, int64_t rows,
                                                           int64_t cols16, u32x4 *__restrict__ out,
                                                           int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const int64_t r = i / cols16, blk = (i - r * cols16) >> 1;
  const uint32_t eb = scales[blk * rows + r];
  const float sc = eb == 255u ? __uint_as_float(0x7FC00000u)
                              : eb == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(eb << 23);
  const u32x4 w = codes[i];
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);  // bytes 0, 1
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);   // bytes 2, 3
    o[2 * k] = (uint32_t)f32_to_bf16(lo[0] * sc) | ((uint32_t)f32_to_bf16(lo[1] * sc) << 16);
    o[2 * k + 1] = (uint32_t)f32_to_bf16(hi[0] * sc) | ((uint32_t)f32_to_bf16(hi[1] * sc) << 16);
  }
  out[2 * i] = u32x4{o[0], o[1], o[2], o[3]};
  out[2 * i + 1] = u32x4{o[4], o[5], o[6], o[7]};
}

// ---------------------------------------------------------------------------
// Per-row (per-token) dynamic E4M3 quantization of a bf16 activation matrix,
// the input side of an FP8 linear: scale_r = amax_r / 448 in fp32 (1 for an
// all-zero row; NaN entries ignored), code = the E4M3 value nearest to
// x / scale_r (IEEE fp32 division), ties to the even code, saturating at 448,
// NaN -> 0x7F.  One workgroup per row: an amax pass, then a quantize pass over
// the (cache-hot) row; 16-B loads of 8 bf16, 8-B stores of 8 codes; the
// encoder (e4m3_code) is shared with the GEMM's MXFP8 epilogue.
// ---------------------------------------------------------------------------

// I8: the INT8 rule instead (scale = amax / 127, code = the fp32 quotient
// rounded to nearest-even, clamped to +-127).
template <bool I8>
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                             int K, uint8_t *__restrict__ q, int64_t ldq,
                                                             float *__restrict__ scale) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int64_t row = blockIdx.x;
  const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + row * ldx);
  const int nch = K / 8;
  float amax = 0.f;
  for (int c = tid; c < nch; c += 256) {
    const u32x4 v = xr[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = fmaxf(amax, fabsf(__uint_as_float(v[e] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(v[e] & 0xffff0000u)));
    }
  }
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, WAVE));
  if (lane == 0) red[wv] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax == 0.f ? 1.0f : amax / (I8 ? 127.0f : 448.0f);
  if (tid == 0) scale[row] = s;
  uint2 *qr = reinterpret_cast<uint2 *>(q + row * ldq);
  auto code = [&](float v) -> uint32_t {
    if constexpr (I8) {
      const float t = __builtin_rintf(v / s);
      return t != t ? 0u : (uint32_t)(uint8_t)(int8_t)fmaxf(-127.f, fminf(127.f, t));
    } else {
      return e4m3_code(v / s);
    }
  };
  for (int c = tid; c < nch; c += 256) {
    const u32x4 v = xr[c];
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t c0 = code(__uint_as_float(v[2 * h] << 16));
      const uint32_t c1 = code(__uint_as_float(v[2 * h] & 0xffff0000u));
      const uint32_t c2 = code(__uint_as_float(v[2 * h + 1] << 16));
      const uint32_t c3 = code(__uint_as_float(v[2 * h + 1] & 0xffff0000u));
      w[h] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    qr[c] = make_uint2(w[0], w[1]);
  }
}

// Per-row MXFP8 quantization of a bf16 activation matrix, the input side of a
// W8A8 MXFP8 linear: each block of 32 consecutive elements of a row gets
// X = floor(log2 amax) - 8 clamped to [-127, 127] (-127 for an all-zero block),
// its E8M0 byte X + 127 written block-major (scale[b * lds + row]), and codes
// e4m3(x * 2^-X) (the scaling is exact).  One 256-thread workgroup per row, four
// lanes per block (8 elements each).  Rows M .. lds - 1 only get scale bytes
// 127 (2^0), so a block-scaled product reading whole 4-row groups sees finite
// scales there.
__global__ __launch_bounds__(256) void quant_rows_mx_kernel(const uint16_t *__restrict__ x, int64_t ldx, int M,
                                                            int K, uint8_t *__restrict__ q, int64_t ldq,
                                                            uint8_t *__restrict__ scale, int64_t lds) {
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int nblk = K / 32;
  if (row >= M) {
    for (int b = tid; b < nblk; b += 256) scale[b * lds + row] = 127;
    return;
  }
  const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + row * ldx);
  uint2 *qr = reinterpret_cast<uint2 *>(q + row * ldq);
  for (int c = tid; c < K / 8; c += 256) {   // 8 elements per thread; 4 consecutive threads = one block
    const u32x4 v = xr[c];
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(v[e] << 16);
      f[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    // floor(log2 amax) from the exponent field (bf16 values: normal, subnormal or 0)
    const int X = amax > 0.f ? max(-127, min(127, (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 8)) : -127;
    const float p2 = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X, 127 - X in [8, 254]
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[h] = e4m3_code(f[4 * h] * p2) | (e4m3_code(f[4 * h + 1] * p2) << 8) |
             (e4m3_code(f[4 * h + 2] * p2) << 16) | (e4m3_code(f[4 * h + 3] * p2) << 24);
    qr[c] = make_uint2(w[0], w[1]);
    if ((c & 3) == 0) scale[(int64_t)(c >> 2) * lds + row] = (uint8_t)(X + 127);
  }
}

// LayerNorm + modulate fused with the input quantisation of a W8A8 linear:
// the modulated row is computed with ln_rows_kernel's layout and arithmetic
// (ln_stats, ln_mod4) and rounded to bf16 as it does, then quantised from
// registers as the stand-alone quantizers do (MX = false: per-row E4M3 with an
// fp32 scale; MX = true: E8M0 per 32 columns, block-major [d / 32, lds], rows
// T .. lds - 1 set to 127), so codes and scales are bit-identical to LN followed
// by the quantizer, without the bf16 row's round trip through memory.  One row
// per workgroup; thread tid holds the float4 chunks tid + 256 i, so a 32-column
// block is eight neighbouring lanes.
template <int NC, bool MX>
__global__ __launch_bounds__(256) void ln_modulate_quant_kernel(
    const float *__restrict__ x, int64_t ldx, int T, int d, const float *__restrict__ gamma,
    const float *__restrict__ beta, const float *__restrict__ eps_p, const float *__restrict__ shift,
    const float *__restrict__ scale, uint8_t *__restrict__ q, int64_t ldq, void *__restrict__ qscale,
    int64_t lds) {
  __shared__ float red[2][4];
  __shared__ float redm[4];
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int64_t row = blockIdx.x;
  if (row >= T) {   // MX padding rows of the block-major scales
    if constexpr (MX)
      for (int b = tid; b < d / 32; b += 256) static_cast<uint8_t *>(qscale)[b * lds + row] = 127;
    return;
  }
  const int d4 = d / 4;
  const float4 *xr = reinterpret_cast<const float4 *>(x + row * ldx);
  float4 v[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c4 = tid + 256 * i;
    v[i] = c4 < d4 ? xr[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float mean, rstd;
  ln_stats<NC>(v, d4, 1.0f / (float)d, eps_p[0], red, mean, rstd);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c4 = tid + 256 * i, c = 4 * c4;
    if (c4 < d4) {
      const float4 g = make_float4(gamma[c], gamma[c + 1], gamma[c + 2], gamma[c + 3]);
      const float4 b = make_float4(beta[c], beta[c + 1], beta[c + 2], beta[c + 3]);
      const float4 sc = make_float4(1.0f + scale[c], 1.0f + scale[c + 1], 1.0f + scale[c + 2], 1.0f + scale[c + 3]);
      const float4 sh = make_float4(shift[c], shift[c + 1], shift[c + 2], shift[c + 3]);
      const float4 y = ln_mod4(v[i], mean, rstd, g, b, sc, sh);
      // the bf16 values the linear reads
      v[i] = make_float4(bf16_round(y.x), bf16_round(y.y), bf16_round(y.z), bf16_round(y.w));
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    } else {
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  uint32_t *qr = reinterpret_cast<uint32_t *>(q + row * ldq);
  if constexpr (MX) {
    uint8_t *sc = static_cast<uint8_t *>(qscale);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c4 = tid + 256 * i;
      float a = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, WAVE));
      const int X = a > 0.f ? max(-127, min(127, (int)((__float_as_uint(a) >> 23) & 0xFF) - 127 - 8)) : -127;
      const float p2 = __uint_as_float((uint32_t)(127 - X) << 23);
      if (c4 < d4) {
        qr[c4] = e4m3_code(v[i].x * p2) | (e4m3_code(v[i].y * p2) << 8) | (e4m3_code(v[i].z * p2) << 16) |
                 (e4m3_code(v[i].w * p2) << 24);
        if ((lane & 7) == 0) sc[(int64_t)(c4 / 8) * lds + row] = (uint8_t)(X + 127);
      }
    }
  } else {
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, WAVE));
    if (lane == 0) redm[wv] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(redm[0], redm[1]), fmaxf(redm[2], redm[3]));
    const float sq = amax == 0.f ? 1.0f : amax / 448.0f;
    if (tid == 0) static_cast<float *>(qscale)[row] = sq;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c4 = tid + 256 * i;
      if (c4 < d4)
        qr[c4] = e4m3_code(v[i].x / sq) | (e4m3_code(v[i].y / sq) << 8) | (e4m3_code(v[i].z / sq) << 16) |
                 (e4m3_code(v[i].w / sq) << 24);
    }
  }
}

}  // namespace

hipError_t launch_ln_modulate_quant(const float *x, int64_t ldx, int T, int d, const float *gamma,
                                    const float *beta, const float *eps, const float *shift, const float *scale,
                                    uint8_t *q, int64_t ldq, void *qscale, int64_t lds, bool mx, hipStream_t s) {
  if (T < 1 || d % 256 || d > 8192 || ldx % 4 || ldq % 4 || (mx && lds < T)) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(mx ? lds : T);
  switch ((d + 1023) / 1024) {
#define DLO_LNQ_CASE(NC)                                                                                  \
  case NC:                                                                                                \
    if (mx)                                                                                               \
      hipLaunchKernelGGL((ln_modulate_quant_kernel<NC, true>), dim3(grid), dim3(256), 0, s, x, ldx, T, d,  \
                         gamma, beta, eps, shift, scale, q, ldq, qscale, lds);                            \
    else                                                                                                  \
      hipLaunchKernelGGL((ln_modulate_quant_kernel<NC, false>), dim3(grid), dim3(256), 0, s, x, ldx, T, d, \
                         gamma, beta, eps, shift, scale, q, ldq, qscale, lds);                            \
    break;
    DLO_LNQ_CASE(1) DLO_LNQ_CASE(2) DLO_LNQ_CASE(3) DLO_LNQ_CASE(4)
    DLO_LNQ_CASE(5) DLO_LNQ_CASE(6) DLO_LNQ_CASE(7) DLO_LNQ_CASE(8)
#undef DLO_LNQ_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequant_fp8(const uint8_t *codes, int64_t n, const float *scale, uint16_t *out,
                              hipStream_t s) {
  const int64_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(dequant_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t *>(codes), scale, reinterpret_cast<u32x4 *>(out), n16);
  return hipGetLastError();
}

hipError_t launch_dequant_int8(const int8_t *codes, int64_t rows, int64_t cols, const float *scales,
                               uint16_t *out, hipStream_t s) {
  if (cols % 16) return hipErrorInvalidValue;
  const int64_t n16 = rows * cols / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_int8_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4 *>(codes), scales, cols / 16, reinterpret_cast<u32x4 *>(out),
                     n16);
  return hipGetLastError();
}

hipError_t launch_dequant_mxfp8(const uint8_t *codes, int64_t rows, int64_t cols, const uint8_t *scales,
                                uint16_t *out, hipStream_t s) {
  if (cols % 32) return hipErrorInvalidValue;
  const int64_t n16 = rows * cols / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_mxfp8_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4 *>(codes), scales, rows, cols / 16,
                     reinterpret_cast<u32x4 *>(out), n16);
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const uint16_t *x, int64_t ldx, int M, int K, uint8_t *q, int64_t ldq,
                                 float *scale, hipStream_t s) {
  if (M < 1 || K < 8 || K % 8 || ldx % 8 || ldq % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_rows_fp8_kernel<false>, dim3(M), dim3(256), 0, s, x, ldx, K, q, ldq, scale);
  return hipGetLastError();
}

hipError_t launch_quant_rows_int8(const uint16_t *x, int64_t ldx, int M, int K, int8_t *q, int64_t ldq,
                                  float *scale, hipStream_t s) {
  if (M < 1 || K < 8 || K % 8 || ldx % 8 || ldq % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_rows_fp8_kernel<true>, dim3(M), dim3(256), 0, s, x, ldx, K,
                     reinterpret_cast<uint8_t *>(q), ldq, scale);
  return hipGetLastError();
}

hipError_t launch_quant_rows_mx(const uint16_t *x, int64_t ldx, int M, int K, uint8_t *q, int64_t ldq,
                               uint8_t *scale, int64_t lds, hipStream_t s) {
  if (M < 1 || K < 32 || K % 32 || ldx % 8 || ldq % 8 || lds < M) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_rows_mx_kernel, dim3((unsigned)lds), dim3(256), 0, s, x, ldx, M, K, q, ldq, scale, lds);
  return hipGetLastError();
}

hipError_t launch_mfma_rate(int form, const uint16_t *in, float *out, int iters, hipStream_t s) {
  const bf16x8 *v = reinterpret_cast<const bf16x8 *>(in);
  if (form == 0)
    hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(MFMA_RATE_GRID), dim3(512), 0, s, v, out, iters);
  else if (form == 1)
    hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(MFMA_RATE_GRID), dim3(512), 0, s, v, out, iters);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_silu(const float *c, float *out, int n, hipStream_t s) {
  hipLaunchKernelGGL(silu_kernel, dim3((n + 255) / 256), dim3(256), 0, s, c, out, n);
  return hipGetLastError();
}

namespace {
template <int NCH>
hipError_t gemv_rows_launch(const uint16_t *W, const float *sc, const float *b, float *out, int rows, int d,
                            hipStream_t s) {
  // workgroups resident at once on the whole chip (the grid loops over rows, so
  // this sets only the speed); the same for every MI355X in the process
  static std::atomic<int> cap{0};
  int c = cap.load(std::memory_order_relaxed);
  if (c == 0) {
    int occ = 0, ncu = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, adaln_gemv_rows_kernel<NCH>, 256, 0) != hipSuccess ||
        occ < 1 || ncu < 1) {
      occ = 2;
      ncu = 256;
    }
    c = occ * ncu;
    cap.store(c, std::memory_order_relaxed);
  }
  const int need = (rows + 3) / 4;
  hipLaunchKernelGGL(adaln_gemv_rows_kernel<NCH>, dim3(need < c ? need : c), dim3(256), 0, s, W, sc, b, out,
                     rows, d);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_adaln_gemv(const uint16_t *W, const float *sc, const float *b, float *out,
                             int rows, int d, hipStream_t s) {
  // the row-looping form pays from d = 2048 on (at d = 1024 the one-row-per-wave
  // grid is 8 % faster); the two give the same bits
  if (d % 512 == 0 && d >= 2048 && d <= 8192) {
    switch (d / 512) {
#define DLO_GEMV_CASE(N) \
  case N:                \
    return gemv_rows_launch<N>(W, sc, b, out, rows, d, s);
      DLO_GEMV_CASE(4) DLO_GEMV_CASE(5) DLO_GEMV_CASE(6) DLO_GEMV_CASE(7) DLO_GEMV_CASE(8) DLO_GEMV_CASE(9)
      DLO_GEMV_CASE(10) DLO_GEMV_CASE(11) DLO_GEMV_CASE(12) DLO_GEMV_CASE(13) DLO_GEMV_CASE(14)
      DLO_GEMV_CASE(15) DLO_GEMV_CASE(16)
#undef DLO_GEMV_CASE
      default:
        break;
    }
  }
  hipLaunchKernelGGL(adaln_gemv_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, W, sc, b, out,
                     rows, d);
  return hipGetLastError();
}

// Scratch of the allocation-free adaLN entry point (dlo_op_adaln_noalloc): the
// SiLU of the conditioning vector, NOALLOC_MAX_D floats.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, looked up once per device and kept in noalloc_ptr.
static __device__ __align__(256) float scratch[NOALLOC_MAX_D];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex noalloc_mu;
float *noalloc_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(float **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(noalloc_mu);
  if (!noalloc_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    noalloc_ptr[dev] = static_cast<float *>(p);
  }
  *ptr = noalloc_ptr[dev];
  return hipSuccess;
}

hipError_t launch_adaln_noalloc(const uint16_t *W, const float *b, const float *cond, int rows, int d,
                                float *out, hipStream_t s) {
  if (d < 8 || d % 8 || d > NOALLOC_MAX_D || rows < 1) return hipErrorInvalidValue;
  float *sc = nullptr;
  hipError_t e = noalloc_scratch(&sc);
  if (e != hipSuccess) return e;
  // silu writes all d entries of the scratch before the GEMV reads them: nothing
  // carried over from an earlier call is read
  if ((e = launch_silu(cond, sc, d, s)) != hipSuccess) return e;
  return launch_adaln_gemv(W, sc, b, out, rows, d, s);
}

hipError_t launch_adaln_gemv_fp8(const uint8_t *W, const float *wscale, const float *sc, const float *b,
                                 float *out, int rows, int d, hipStream_t s) {
  if (d % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(adaln_gemv_fp8_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, W, wscale, sc, b, out,
                     rows, d);
  return hipGetLastError();
}

hipError_t launch_ln_modulate(const float *x, int64_t ldx, int T, int d, const float *gamma,
                              const float *beta, const float *eps, const float *shift,
                              const float *scale, uint16_t *out, hipStream_t s) {
  if (T < 1 || d < 4 || d % 4 || d > 8192 || ldx % 4) return hipErrorInvalidValue;
  // one workgroup per row up to the cap; past it each workgroup takes several
  // rows (the cap keeps two workgroups per CU resident at 8 chunks per thread)
  const int nc = (d + 1023) / 1024;
  const int cap = nc >= 5 ? 512 : 768;
  const dim3 grid(T < cap ? T : cap);
  switch (nc) {
#define DLO_LN_CASE(NC)                                                                                      \
  case NC:                                                                                                   \
    hipLaunchKernelGGL(ln_rows_kernel<NC>, grid, dim3(256), 0, s, x, ldx, T, d, gamma, beta, eps, shift,     \
                       scale, out);                                                                          \
    break;
    DLO_LN_CASE(1) DLO_LN_CASE(2) DLO_LN_CASE(3) DLO_LN_CASE(4)
    DLO_LN_CASE(5) DLO_LN_CASE(6) DLO_LN_CASE(7) DLO_LN_CASE(8)
#undef DLO_LN_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_digest(const void *base, const int64_t *offsets, const int64_t *lengths, int n,
                         uint64_t *out, hipStream_t s) {
  hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(64), 0, s, out, 1, (uint64_t)0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int i = 0; i < n; ++i) {
    if (lengths[i] <= 0) continue;
    const int64_t nw = (lengths[i] + 7) / 8;
    int64_t blocks = (nw + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(digest_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint8_t *>(base), offsets[i], lengths[i], out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dlo
