// gfx950 GEMM of the DiT block linears: C = A B^T with bf16, FP8 (E4M3, per-row
// and per-tensor scales) or MXFP8 (E4M3 with E8M0 block scales) operands, fp32
// accumulation and fused epilogues (bias, bias + GELU, gated residual, and bias
// with the result stored transposed).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace dlo {
namespace {

// ---------------------------------------------------------------------------
// GEMM tiles: 256 rows of A per workgroup.
// ---------------------------------------------------------------------------

constexpr int GBM = 256;

// ---------------------------------------------------------------------------
// GEMM: C[M, N] = A[M, K] B[N, K]^T, fp32 accumulate (direct-to-LDS).
// Workgroup tile 256 x 256 x (64 bytes of K: 32 bf16 or 64 E4M3 elements) with
// 8 waves of 128 x 64 (bf16: 16x16x32 MFMA tiles, one k-step per stage; 8-bit
// operands: 32x32 tiles).  Operand tiles travel HBM/L2 -> LDS
// with buffer_load ... lds (no register staging) into a ring of 4 LDS stages.
// One LDS stage = A and B tiles of 256 rows x 64 B (plus, for MXFP8, their
// scale bytes); a row holds 4 chunks of 16 B whose order is XOR-swizzled
// (dl_swz) so that the MFMA operand reads are free of bank conflicts.  A load
// instruction fills 1 KB of LDS: 64 lanes x 16 B at M0 + 16 * lane, i.e. 16
// rows.  The tile order is XCD-aware and grouped by 4 row tiles: each XCD's
// 32 concurrent tiles span 4 row tiles x 8 column tiles (groups of 2 to 6
// measure alike; 8 is 4 % slower and 16 12 % slower on the DiT shapes).
// ---------------------------------------------------------------------------

constexpr int DL_BK = 32;
constexpr int DL_TILE = GBM * DL_BK;  // bf16 elements of one operand tile (16 KB)

// chunk swizzle of row r: ((r >> 1) ^ (r >> 2)) & 3.  A 16-B read by 16
// consecutive rows (one 64-bank LDS cycle) then hits 16 distinct 16-B bank
// groups, and so do 8 consecutive rows within a 32-bank cycle.
__device__ __forceinline__ int dl_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

__device__ __forceinline__ int dl_lds_off(int row, int chunk) {  // element offset in a tile
  return row * DL_BK + ((chunk ^ dl_swz(row)) << 3);
}

// Four consecutive fp32 values from an address that is only 4-B aligned: the
// block's fp32 parameters sit back to back in a slot, so a bias or a gate
// vector may start at any multiple of 4 bytes.
__device__ __forceinline__ float4 load4(const float *p) { return make_float4(p[0], p[1], p[2], p[3]); }

// Epilogue of a 256 x BN tile held by 2 x WN waves (acc: the wave's 128 x BN/WN
// sub-tile in 32x32 MFMA tiles, transposed except for EPI_BIAS_T).  smem: at
// least 256 x (BN + 8) bf16 (bias epilogues; BN x (256 + 8) for EPI_BIAS_T) or
// 128 x (BN + 4) fp32 (gated residual), no longer in use.
template <int EPI, int BN, int WN>
__device__ __forceinline__ void gemm_epilogue(const f32x16 (&acc)[4][BN / WN / 32], uint16_t *smem,
                                              int tid, int wm, int wn, int lane, int m0, int n0,
                                              int M, const float *__restrict__ bias,
                                              const float *__restrict__ gate, void *__restrict__ Cv,
                                              int64_t ldc, uint8_t *__restrict__ out_scale = nullptr,
                                              int64_t lds_out = 0) {
  // Epilogue, staged through LDS so that global accesses are whole rows.
  // acc[i][j] holds the transposed 32x32 sub-tile (the MFMA took B as its first
  // operand): lane l has row i*32 + l%32 of the wave's rows and, for g = 0..3,
  // the four consecutive columns j*32 + 8g + 4(l/32) + 0..3 -- one 8-B (bf16)
  // or 16-B (fp32) piece of a row, written to LDS as such.  Then every thread
  // moves 16-B row segments between LDS and global memory; only the last row
  // tile checks rows against M.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // ring no longer read
  const bool full = m0 + GBM <= M;
  const int ldc32 = (int)ldc;
  constexpr int NT = 128 * WN;                // threads
  constexpr int NJ = BN / WN / 32;
  constexpr int C_LD = BN + 8, X_LD = BN + 4;
  const int frow = lane & 31, fk = lane >> 5;
  if (EPI == EPI_BIAS_T) {
    // acc[i][j] holds the 32x32 sub-tile as the MFMA lays it out with A first:
    // lane l has column j*32 + l%32 and, for g = 0..3, the four consecutive
    // rows i*32 + 8g + 4(l/32) + 0..3: one 8-B piece of a row of C^T.  Rows
    // m >= M become 0; rows of C^T are stored up to M rounded up to 64.
    const int M64 = (M + 63) & ~63;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = wn * (BN / WN) + j * 32 + frow;
      const float bv = bias[n0 + col];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = wm * 128 + i * 32 + g * 8 + fk * 4;
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = (full || m0 + row + e < M) ? (__bf16)(acc[i][j][g * 4 + e] + bv) : (__bf16)0.0f;
          *reinterpret_cast<bf16x4 *>(&smem[col * (GBM + 8) + row]) = o;
        }
    }
    __syncthreads();
    constexpr int SEG = GBM / 8;              // 16-B segments per row of C^T
    uint16_t *C = reinterpret_cast<uint16_t *>(Cv) + (int64_t)n0 * ldc + m0;
#pragma unroll
    for (int it = 0; it < BN * SEG / NT; ++it) {
      const int e = it * NT + tid, row = e / SEG, c8 = (e % SEG) * 8;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&smem[row * (GBM + 8) + c8]);
      if (full || m0 + c8 < M64) *reinterpret_cast<u32x4 *>(&C[row * ldc32 + c8]) = v;
    }
  } else if (EPI != EPI_GATED_RESIDUAL) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * (BN / WN) + j * 32 + g * 8 + fk * 4;
        const float4 bv = load4(&bias[n0 + col]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v0 = acc[i][j][g * 4 + 0] + bv.x, v1 = acc[i][j][g * 4 + 1] + bv.y;
          float v2 = acc[i][j][g * 4 + 2] + bv.z, v3 = acc[i][j][g * 4 + 3] + bv.w;
          if (EPI == EPI_BIAS_GELU || EPI == EPI_GELU_MX) {
            v0 = gelu_erf(v0);
            v1 = gelu_erf(v1);
            v2 = gelu_erf(v2);
            v3 = gelu_erf(v3);
          }
          bf16x4 o;
          o[0] = (__bf16)v0;
          o[1] = (__bf16)v1;
          o[2] = (__bf16)v2;
          o[3] = (__bf16)v3;
          *reinterpret_cast<bf16x4 *>(&smem[(wm * 128 + i * 32 + frow) * C_LD + col]) = o;
        }
      }
    __syncthreads();
    constexpr int SEG = BN / 8;               // 16-B segments per row
    if constexpr (EPI == EPI_GELU_MX) {
      // four consecutive threads hold one 32-column block of a row (SEG % 4 == 0):
      // its maximum by two shuffles, then the MX rule of quant_rows_mx_kernel
      uint8_t *Q = static_cast<uint8_t *>(Cv) + (int64_t)m0 * ldc + n0;
#pragma unroll
      for (int it = 0; it < GBM * SEG / NT; ++it) {
        const int e = it * NT + tid, row = e / SEG, c8 = (e % SEG) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(&smem[row * C_LD + c8]);
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[2 * q] = __uint_as_float(v[q] << 16);
          f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
        }
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(f[q]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        const int X = amax > 0.f ? max(-127, min(127, (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 8))
                                 : -127;
        const float p2 = __uint_as_float((uint32_t)(127 - X) << 23);
        const int64_t srow = (int64_t)((n0 + c8) >> 5) * lds_out + m0 + row;
        if (full || m0 + row < M) {
          uint32_t w[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            w[h] = e4m3_code(f[4 * h] * p2) | (e4m3_code(f[4 * h + 1] * p2) << 8) |
                   (e4m3_code(f[4 * h + 2] * p2) << 16) | (e4m3_code(f[4 * h + 3] * p2) << 24);
          *reinterpret_cast<uint2 *>(&Q[row * ldc32 + c8]) = make_uint2(w[0], w[1]);
          if ((tid & 3) == 0) out_scale[srow] = (uint8_t)(X + 127);
        } else if ((tid & 3) == 0 && m0 + row < lds_out) {
          out_scale[srow] = 127;
        }
      }
    } else {
      uint16_t *C = reinterpret_cast<uint16_t *>(Cv) + (int64_t)m0 * ldc + n0;
#pragma unroll
      for (int it = 0; it < GBM * SEG / NT; ++it) {
        const int e = it * NT + tid, row = e / SEG, c8 = (e % SEG) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(&smem[row * C_LD + c8]);
        if (full || m0 + row < M) *reinterpret_cast<u32x4 *>(&C[row * ldc32 + c8]) = v;
      }
    }
  } else {
    float *xs = reinterpret_cast<float *>(smem);
    constexpr int SEG = BN / 4;               // 16-B segments per row
    float *X = reinterpret_cast<float *>(Cv) + (int64_t)m0 * ldc + n0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = wn * (BN / WN) + j * 32 + g * 8 + fk * 4;
            const float4 bv = load4(&bias[n0 + col]);
            const float4 gv = load4(&gate[n0 + col]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float4 v;
              v.x = gv.x * (acc[i][j][g * 4 + 0] + bv.x);
              v.y = gv.y * (acc[i][j][g * 4 + 1] + bv.y);
              v.z = gv.z * (acc[i][j][g * 4 + 2] + bv.z);
              v.w = gv.w * (acc[i][j][g * 4 + 3] + bv.w);
              *reinterpret_cast<float4 *>(&xs[(i * 32 + frow) * X_LD + col]) = v;
            }
          }
      }
      __syncthreads();
      constexpr int PER = 128 * SEG / NT;     // segments per thread
      float4 xv[PER];
#pragma unroll
      for (int it = 0; it < PER; ++it) {
        const int e = it * NT + tid, row = half * 128 + e / SEG, c4 = (e % SEG) * 4;
        xv[it] = (full || m0 + row < M) ? *reinterpret_cast<const float4 *>(&X[row * ldc32 + c4])
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int it = 0; it < PER; ++it) {
        const int e = it * NT + tid, row = half * 128 + e / SEG, c4 = (e % SEG) * 4;
        const float4 u = *reinterpret_cast<const float4 *>(&xs[(e / SEG) * X_LD + c4]);
        float4 v = xv[it];
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
        if (full || m0 + row < M) *reinterpret_cast<float4 *>(&X[row * ldc32 + c4]) = v;
      }
      if (half == 0) __syncthreads();
    }
  }
}

// Epilogue of a 256 x BN tile held by 2 x WN waves in 16 x 16 MFMA tiles:
// acc[i][j] is the wave's 16 x 16 sub-tile (i < 8 row tiles, j < BN / WN / 16
// column tiles).  With B as the MFMA's first operand, lane l holds row
// i*16 + l%16 and the four consecutive columns j*16 + 4(l/16) + 0..3; for
// EPI_BIAS_T (A first) column j*16 + l%16 and the four consecutive rows
// i*16 + 4(l/16) + 0..3.  Staged through LDS like gemm_epilogue, whose
// copy-out it shares.
template <int EPI, int BN, int WN>
__device__ __forceinline__ void gemm_epilogue16(const f32x4 (&acc)[8][BN / WN / 16], uint16_t *smem, int tid,
                                                int wm, int wn, int lane, int m0, int n0, int M,
                                                const float *__restrict__ bias, const float *__restrict__ gate,
                                                void *__restrict__ Cv, int64_t ldc) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // ring no longer read
  const bool full = m0 + GBM <= M;
  const int ldc32 = (int)ldc;
  constexpr int NT = 128 * WN;
  constexpr int NJ = BN / WN / 16;
  constexpr int C_LD = BN + 8, X_LD = BN + 4;
  const int fr = lane & 15, fq = lane >> 4;
  if (EPI == EPI_BIAS_T) {
    const int M64 = (M + 63) & ~63;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = wn * (BN / WN) + j * 16 + fr;
      const float bv = bias[n0 + col];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = wm * 128 + i * 16 + fq * 4;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = (full || m0 + row + e < M) ? (__bf16)(acc[i][j][e] + bv) : (__bf16)0.0f;
        *reinterpret_cast<bf16x4 *>(&smem[col * (GBM + 8) + row]) = o;
      }
    }
    __syncthreads();
    constexpr int SEG = GBM / 8;
    uint16_t *C = reinterpret_cast<uint16_t *>(Cv) + (int64_t)n0 * ldc + m0;
#pragma unroll
    for (int it = 0; it < BN * SEG / NT; ++it) {
      const int e = it * NT + tid, row = e / SEG, c8 = (e % SEG) * 8;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&smem[row * (GBM + 8) + c8]);
      if (full || m0 + c8 < M64) *reinterpret_cast<u32x4 *>(&C[row * ldc32 + c8]) = v;
    }
  } else if (EPI != EPI_GATED_RESIDUAL) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = wn * (BN / WN) + j * 16 + fq * 4;
      const float4 bv = load4(&bias[n0 + col]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v0 = acc[i][j][0] + bv.x, v1 = acc[i][j][1] + bv.y;
        float v2 = acc[i][j][2] + bv.z, v3 = acc[i][j][3] + bv.w;
        if (EPI == EPI_BIAS_GELU) {
          v0 = gelu_erf(v0);
          v1 = gelu_erf(v1);
          v2 = gelu_erf(v2);
          v3 = gelu_erf(v3);
        }
        bf16x4 o;
        o[0] = (__bf16)v0;
        o[1] = (__bf16)v1;
        o[2] = (__bf16)v2;
        o[3] = (__bf16)v3;
        *reinterpret_cast<bf16x4 *>(&smem[(wm * 128 + i * 16 + fr) * C_LD + col]) = o;
      }
    }
    __syncthreads();
    constexpr int SEG = BN / 8;
    uint16_t *C = reinterpret_cast<uint16_t *>(Cv) + (int64_t)m0 * ldc + n0;
#pragma unroll
    for (int it = 0; it < GBM * SEG / NT; ++it) {
      const int e = it * NT + tid, row = e / SEG, c8 = (e % SEG) * 8;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&smem[row * C_LD + c8]);
      if (full || m0 + row < M) *reinterpret_cast<u32x4 *>(&C[row * ldc32 + c8]) = v;
    }
  } else {
    float *xs = reinterpret_cast<float *>(smem);
    constexpr int SEG = BN / 4;
    float *X = reinterpret_cast<float *>(Cv) + (int64_t)m0 * ldc + n0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = wn * (BN / WN) + j * 16 + fq * 4;
          const float4 bv = load4(&bias[n0 + col]);
          const float4 gv = load4(&gate[n0 + col]);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float4 v;
            v.x = gv.x * (acc[i][j][0] + bv.x);
            v.y = gv.y * (acc[i][j][1] + bv.y);
            v.z = gv.z * (acc[i][j][2] + bv.z);
            v.w = gv.w * (acc[i][j][3] + bv.w);
            *reinterpret_cast<float4 *>(&xs[(i * 16 + fr) * X_LD + col]) = v;
          }
        }
      }
      __syncthreads();
      constexpr int PER = 128 * SEG / NT;
      float4 xv[PER];
#pragma unroll
      for (int it = 0; it < PER; ++it) {
        const int e = it * NT + tid, row = half * 128 + e / SEG, c4 = (e % SEG) * 4;
        xv[it] = (full || m0 + row < M) ? *reinterpret_cast<const float4 *>(&X[row * ldc32 + c4])
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int it = 0; it < PER; ++it) {
        const int e = it * NT + tid, row = half * 128 + e / SEG, c4 = (e % SEG) * 4;
        const float4 u = *reinterpret_cast<const float4 *>(&xs[(e / SEG) * X_LD + c4]);
        float4 v = xv[it];
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
        if (full || m0 + row < M) *reinterpret_cast<float4 *>(&X[row * ldc32 + c4]) = v;
      }
      if (half == 0) __syncthreads();
    }
  }
}

// Ping-pong schedule.  Wave w owns rows 128 (w / 4) .. +127 and columns
// 64 (w % 4) .. +63 of the tile; group g = w / 4 holds one wave on every SIMD.
// Each wave alternates a memory phase (issue its share of the loads of k-tile
// s + 3, read all fragments of k-tile s from LDS) and a compute phase (the
// MFMAs on those fragments: bf16 32 of 16x16x32, the same products in the same
// k order per output element as 16 of 32x32x16, with bit-identical results,
// measured).  Group 1 runs one phase behind group 0 and a
// workgroup barrier separates phases, so on every SIMD one wave multiplies
// while the other one feeds: the MFMA pipe sees a dense run of MFMAs instead
// of MFMAs interleaved with the waits of LDS reads (5-6 % faster on the DiT
// shapes than that interleaved form, and bit-identical to it: every
// accumulator sees the same k order).  Group g loads A rows and B rows
// 128 g .. +127 of every k-tile; the 4-deep ring gives each load six phases
// to land.
//
// Q = 1 (FP8) and Q = 2 (MXFP8): A and B hold OCP E4M3 codes (1 byte per
// element) instead of bf16.  A stage row is still 64 bytes, now 64 elements:
// one v_mfma_scale_f32_32x32x64_f8f6f4 k-step per stage; each phase issues 8
// of these MFMAs, the same MFMA time as 16 bf16 ones, over twice the K.  The
// instruction's k-blocks of 32 are bytes 0-15 of both lane halves and bytes
// 16-31 of both (measured), so lane half h takes chunks h and 2 + h of the
// swizzled row: k 16h .. 16h + 15 of each 32-block.  Q = 1: the fp32 result is
// scaled by a_scale[row] * *b_scale before the epilogue.  Q = 2: a_scale and
// b_scale are E8M0 bytes, block-major ([K / 32][lds_a] and [K / 32][lds_b],
// rows from 0 and from n0 respectively); each stage's two 32-blocks of scales
// for the tile's 256 A rows and 256 B rows (1 KB) travel with the tiles, by
// DMA into LDS, and the instruction applies them (lane (row m, half h) holds
// block h's scale of its row).
// Q = 3 (INT8): A and B hold int8 codes; a stage row of 64 bytes is two
// v_mfma_i32_32x32x32_i8 k-steps of 32, each lane's 16 k-bytes read exactly as
// the bf16 fragments are; the int32 sums are exact, then converted to fp32 and
// scaled by a_scale[row] * b_scale[column] (fp32, per row of A and of B).
template <int EPI, int Q>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(
    const void *__restrict__ A, int64_t lda, const void *__restrict__ B, int64_t ldb,
    int M, int N, int K, const float *__restrict__ bias, const float *__restrict__ gate,
    void *__restrict__ Cv, int64_t ldc, const void *__restrict__ a_scale,
    const void *__restrict__ b_scale, int64_t lds_a, int64_t lds_b, uint8_t *__restrict__ out_scale,
    int64_t lds_out) {
  constexpr bool F8 = Q == 1 || Q == 2, MX = Q == 2, I8 = Q == 3;
  constexpr int ES = Q > 0 ? 1 : 2;          // bytes per element
  constexpr int KSTAGE = 64 / ES;            // elements of k per stage
  constexpr int BN = 256, WN = 4, NJ = 2, STAGES = 4;
  constexpr int B_TILE = BN * DL_BK;
  constexpr int SC_STAGE = MX ? 1024 : 0;    // MXFP8: two copies of 1 KB of scale bytes
  constexpr int STAGE = DL_TILE + B_TILE + SC_STAGE;
  constexpr int LPS = MX ? 5 : 4;            // loads per wave per stage
  constexpr int C_LD = BN + 8, X_LD = BN + 4;
  constexpr int RING = STAGES * STAGE;
  constexpr int CSTAGE = EPI == EPI_GATED_RESIDUAL ? 128 * X_LD * 2 : GBM * C_LD;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[RING > CSTAGE ? RING : CSTAGE];

  const int tid = threadIdx.x, lane = tid % WAVE;
  const int wv = __builtin_amdgcn_readfirstlane(tid / WAVE);  // wave-uniform: barriers branch on it
  const int grp = wv >> 2, wq = wv & 3;
  const int wm = grp, wn = wq;

  const int tiles_m = (M + GBM - 1) / GBM, tiles_n = N / BN;
  const int total = tiles_m * tiles_n;
  int pid = xcd_remap(blockIdx.x, total);
  constexpr int GROUP_M = 4;
  const int group = pid / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (pid % (GROUP_M * tiles_n)) % gsz;
  const int tn = (pid % (GROUP_M * tiles_n)) / gsz;
  const int m0 = tm * GBM, n0 = tn * BN;

  const int a_rows = min(M - m0, GBM);
  const i32x4 a_rsrc = dl_rsrc(static_cast<const char *>(A) + (int64_t)m0 * lda * ES,
                               (uint32_t)(a_rows * lda * ES));
  const i32x4 b_rsrc = dl_rsrc(static_cast<const char *>(B) + (int64_t)n0 * ldb * ES,
                               (uint32_t)(BN * ldb * ES));
  // MXFP8: wave wq of each group loads one 256-B scale segment per stage into
  // its group's copy: A block 2kt, A block 2kt + 1, B block 2kt, B block 2kt + 1
  // (bytes past the scale arrays read 0; A rows past lds_a read the next block
  // row's finite scales, multiplied by zero codes)
  const int sc_h = wq & 1;
  const i32x4 sc_rsrc = dl_rsrc(wq < 2 ? a_scale : b_scale,
                                (uint32_t)((int64_t)(K / 32) * (wq < 2 ? lds_a : lds_b)));
  const int sc_voff = (wq < 2 ? m0 : n0) + 4 * lane;
  const int64_t sc_ld = wq < 2 ? lds_a : lds_b;

  // 16-row load blocks 8 g + 2 wq + i (i < 2) of A and of B
  int a_voff[2], b_voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (grp * 8 + wq * 2 + i) * 16 + (lane >> 2);
    a_voff[i] = r * (int)lda * ES + ((lane & 3) ^ dl_swz(r)) * 16;
    b_voff[i] = r * (int)ldb * ES + ((lane & 3) ^ dl_swz(r)) * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)&smem[0];
  // loads of k-tile kt into stage S (a compile-time constant): per-lane
  // offsets fixed, the k offset in the buffer instruction's scalar offset
  auto issue = [&](int kt, auto st_c) {
    constexpr int S = decltype(st_c)::value;
    const uint32_t sbase = lds0 + (uint32_t)(S * STAGE * 2);
    const uint32_t koff = __builtin_amdgcn_readfirstlane(kt * 64);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dl_load_so(a_rsrc, __builtin_amdgcn_readfirstlane(sbase + (uint32_t)((grp * 8 + wq * 2 + i) * 1024)),
                 a_voff[i], koff);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dl_load_so(b_rsrc,
                 __builtin_amdgcn_readfirstlane(sbase + (uint32_t)(DL_TILE * 2 + (grp * 8 + wq * 2 + i) * 1024)),
                 b_voff[i], koff);
    if constexpr (MX)
      dl_load_dw_so(sc_rsrc,
                    __builtin_amdgcn_readfirstlane(sbase + (uint32_t)((DL_TILE + B_TILE) * 2 + grp * 1024 + wq * 256)),
                    sc_voff, __builtin_amdgcn_readfirstlane((uint32_t)((2 * kt + sc_h) * sc_ld)));
  };

  constexpr bool M16 = Q == 0;   // bf16: 16 x 16 x 32 MFMA tiles
  // 32 x 32 tiles (acc) or, M16, 16 x 16 tiles (acc16; acc unused)
  f32x16 acc[M16 ? 1 : 4][M16 ? 1 : NJ];
  f32x4 acc16[M16 ? 8 : 1][M16 ? 4 : 1];
  if constexpr (M16) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc16[i][j][r] = 0.f;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  const int nk = K / KSTAGE;
  const int frow = lane & 31, fk = lane >> 5;

  // all fragments of one stage in 32 x 32 tiles: INT8, 2 k-steps of 32 x (4 A
  // rows, 2 B columns); F8, one k-step x (4 A rows, 2 B columns) of two 16-B
  // halves each
  struct FragsB {
    bf16x8 a[2][4], b[2][NJ];
  };
  struct Frags8 {
    u32x4 a[4][2], b[NJ][2];
    int sa[4], sb[NJ];   // MXFP8: E8M0 scale bytes of the lane's rows, block fk
  };
  // M16: one k-step of 32 per stage: 8 row tiles of A, 4 column tiles of B (16 rows each)
  struct Frags16 {
    bf16x8 a[8], b[4];
  };
  using Frags = std::conditional_t<F8, Frags8, std::conditional_t<M16, Frags16, FragsB>>;
  // M16 operand of lane l: row l % 16 of a 16-row tile, k chunk l / 16 (k 8 (l / 16) ..);
  // the swizzle depends on row bits 1..3 only, so tiles 16 rows apart are immediate offsets
  const int a16_lane = dl_lds_off(wm * 128 + (lane & 15), lane >> 4) * 2;
  const int b16_lane = (DL_TILE + dl_lds_off(wn * 64 + (lane & 15), lane >> 4)) * 2;
  // fragment byte offsets inside a stage: the XOR swizzle depends on row bits
  // 1..3 only, so rows 32 apart share it and the 32-row steps are immediates
  const char *lds_bytes = reinterpret_cast<const char *>(&smem[0]);
  int a_lane[2], b_lane[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    a_lane[kk] = dl_lds_off(wm * 128 + frow, kk * 2 + fk) * 2;
    b_lane[kk] = (DL_TILE + dl_lds_off(wn * 64 + frow, kk * 2 + fk)) * 2;
  }
  // F8 operand of lane (row, fk): bytes 0-15 = chunk fk (k 16 fk ..), bytes 16-31 =
  // chunk 2 + fk (k 32 + 16 fk ..), so each instruction k-block of 32 is one
  // 32-element block of the rows
  int a8_lane[2], b8_lane[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    a8_lane[h] = dl_lds_off(wm * 128 + frow, 2 * h + fk) * 2;
    b8_lane[h] = (DL_TILE + dl_lds_off(wn * 64 + frow, 2 * h + fk)) * 2;
  }
  // MXFP8 scale bytes in a stage: this group's copy, A segment fk then B segment fk
  const int sa_lane = (DL_TILE + B_TILE) * 2 + grp * 1024 + fk * 256 + wm * 128 + frow;
  const int sb_lane = (DL_TILE + B_TILE) * 2 + grp * 1024 + 512 + fk * 256 + wn * 64 + frow;
  auto read_tile = [&](auto st_c, Frags &f) {
    constexpr int S = decltype(st_c)::value;
    const char *base = lds_bytes + S * STAGE * 2;
    if constexpr (F8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f.a[i][h] = *reinterpret_cast<const u32x4 *>(base + a8_lane[h] + i * 32 * 64);
#pragma unroll
        for (int j = 0; j < NJ; ++j) f.b[j][h] = *reinterpret_cast<const u32x4 *>(base + b8_lane[h] + j * 32 * 64);
      }
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f.sa[i] = *reinterpret_cast<const uint8_t *>(base + sa_lane + i * 32);
#pragma unroll
        for (int j = 0; j < NJ; ++j) f.sb[j] = *reinterpret_cast<const uint8_t *>(base + sb_lane + j * 32);
      }
    } else if constexpr (M16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) f.a[i] = *reinterpret_cast<const bf16x8 *>(base + a16_lane + i * 16 * DL_BK * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) f.b[j] = *reinterpret_cast<const bf16x8 *>(base + b16_lane + j * 16 * DL_BK * 2);
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          f.a[kk][i] = *reinterpret_cast<const bf16x8 *>(base + a_lane[kk] + i * 32 * DL_BK * 2);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          f.b[kk][j] = *reinterpret_cast<const bf16x8 *>(base + b_lane[kk] + j * 32 * DL_BK * 2);
      }
    }
  };
  auto drained = [&](const Frags &f) {
    if constexpr (F8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        asm volatile("" ::"v"(f.a[0][h]), "v"(f.a[1][h]), "v"(f.a[2][h]), "v"(f.a[3][h]));
        asm volatile("" ::"v"(f.b[0][h]), "v"(f.b[1][h]));
      }
      if constexpr (MX) {
        asm volatile("" ::"v"(f.sa[0]), "v"(f.sa[1]), "v"(f.sa[2]), "v"(f.sa[3]));
        asm volatile("" ::"v"(f.sb[0]), "v"(f.sb[1]));
      }
    } else if constexpr (M16) {
      asm volatile("" ::"v"(f.a[0]), "v"(f.a[1]), "v"(f.a[2]), "v"(f.a[3]));
      asm volatile("" ::"v"(f.a[4]), "v"(f.a[5]), "v"(f.a[6]), "v"(f.a[7]));
      asm volatile("" ::"v"(f.b[0]), "v"(f.b[1]), "v"(f.b[2]), "v"(f.b[3]));
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        asm volatile("" ::"v"(f.a[kk][0]), "v"(f.a[kk][1]), "v"(f.a[kk][2]), "v"(f.a[kk][3]));
        asm volatile("" ::"v"(f.b[kk][0]), "v"(f.b[kk][1]));
      }
    }
  };
  auto compute = [&](const Frags &f) {
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const u32x4 a0 = f.a[i][0], a1 = f.a[i][1], b0 = f.b[j][0], b1 = f.b[j][1];
          const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                            (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          const i32x8 bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                            (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
          // format 0 (E4M3) for both operands; MXFP8: each operand's block scale
          // (byte 0 of the scale register), else none
          if constexpr (MX)
            acc[i][j] = EPI == EPI_BIAS_T
                            ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 0, 0, 0, f.sa[i],
                                                                              0, f.sb[j])
                            : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], 0, 0, 0, f.sb[j],
                                                                              0, f.sa[i]);
          else
            acc[i][j] = EPI == EPI_BIAS_T
                            ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 0, 0, 0, 0, 0, 0)
                            : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], 0, 0, 0, 0, 0, 0);
        }
    } else if constexpr (I8) {
      // int32 sums in the fp32 accumulator registers, bit for bit
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const i32x4v av = __builtin_bit_cast(i32x4v, f.a[kk][i]), bv = __builtin_bit_cast(i32x4v, f.b[kk][j]);
            const i32x16 c = __builtin_bit_cast(i32x16, acc[i][j]);
            acc[i][j] = __builtin_bit_cast(f32x16, EPI == EPI_BIAS_T
                                                       ? __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, c, 0, 0, 0)
                                                       : __builtin_amdgcn_mfma_i32_32x32x32_i8(bv, av, c, 0, 0, 0));
          }
    } else {
      static_assert(M16, "bf16 operands run on 16x16x32 tiles");
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc16[i][j] = EPI == EPI_BIAS_T
                            ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc16[i][j], 0, 0, 0)
                            : __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[i], acc16[i][j], 0, 0, 0);
    }
  };
  // Barrier opening global phase p.  Before it, this wave's loads of the tile
  // read in phase p (tile p / 2) have landed: younger tiles of this wave's
  // group may stay in flight -- three when group 0 enters an odd phase, two
  // otherwise (four loads per tile per wave), fewer near the end.
  auto phase_barrier = [&](int p) {
    const int s = p >> 1;
    int younger = (grp == 0 && (p & 1)) ? 3 : 2;
    younger = min(younger, nk - 1 - s);
    __builtin_amdgcn_sched_barrier(0);
    if (younger >= 3)
      vmcnt_barrier<3 * LPS>();
    else if (younger == 2)
      vmcnt_barrier<2 * LPS>();
    else if (younger == 1)
      vmcnt_barrier<LPS>();
    else
      vmcnt_barrier<0>();
    __builtin_amdgcn_sched_barrier(0);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if (0 < nk) issue(0, I0{});
  if (1 < nk) issue(1, I1{});
  if (2 < nk) issue(2, I2{});
  Frags f0, f1;
  // k-tile s in stage S = s % 4 (compile-time: the loop is unrolled by the ring depth)
  auto step = [&](int s, auto st_c, Frags &f) {
    constexpr int S = decltype(st_c)::value;
    const int pm = 2 * s + grp;  // this wave's memory phase
    phase_barrier(pm);
    if (s + 3 < nk) issue(s + 3, std::integral_constant<int, (S + 3) % STAGES>{});
    read_tile(st_c, f);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    drained(f);
    phase_barrier(pm + 1);
    compute(f);
  };
  if (grp == 1) phase_barrier(0);
  for (int s = 0; s < nk; s += 4) {
    step(s, I0{}, f0);
    if (s + 1 < nk) step(s + 1, I1{}, f1);
    if (s + 2 < nk) step(s + 2, I2{}, f0);
    if (s + 3 < nk) step(s + 3, I3{}, f1);
  }
  if (grp == 0) phase_barrier(2 * nk);

  if constexpr (Q == 1) {
    // A's per-row scale times B's scale (rows past M read no scale)
    const float *a_sc = static_cast<const float *>(a_scale);
    const float sb = *static_cast<const float *>(b_scale);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (EPI == EPI_BIAS_T) {  // lane holds rows 8 (r / 4) + 4 fk + r % 4 of row block i
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + fk * 4 + (r & 3);
          const float f = (row < M ? a_sc[row] : 0.f) * sb;
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j][r] *= f;
        }
      } else {  // lane holds row frow of row block i
        const int row = m0 + wm * 128 + i * 32 + frow;
        const float f = (row < M ? a_sc[row] : 0.f) * sb;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= f;
      }
    }
  }
  if constexpr (Q == 3) {
    // the exact int32 sums to fp32 (whole-vector conversion), times A's row
    // scale and B's row (output column) scale
    const float *a_sc = static_cast<const float *>(a_scale), *b_sc = static_cast<const float *>(b_scale);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        f32x16 sc;
        if (EPI == EPI_BIAS_T) {  // lane: column j*32 + frow; rows 8 (r / 4) + 4 fk + r % 4 of row block i
          const float sbv = b_sc[n0 + wn * 64 + j * 32 + frow];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + fk * 4 + (r & 3);
            sc[r] = (row < M ? a_sc[row] : 0.f) * sbv;
          }
        } else {  // lane: row frow of row block i; columns j*32 + 8 g + 4 fk + 0..3
          const int row = m0 + wm * 128 + i * 32 + frow;
          const float fa = row < M ? a_sc[row] : 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r)  // scalar loads: a packed block's scales are only 4-B aligned
            sc[r] = fa * b_sc[n0 + wn * 64 + j * 32 + (r >> 2) * 8 + fk * 4 + (r & 3)];
        }
        acc[i][j] = __builtin_convertvector(__builtin_bit_cast(i32x16, acc[i][j]), f32x16) * sc;
      }
  }
  if constexpr (M16)
    gemm_epilogue16<EPI, BN, WN>(acc16, smem, tid, wm, wn, lane, m0, n0, M, bias, gate, Cv, ldc);
  else
    gemm_epilogue<EPI, BN, WN>(acc, smem, tid, wm, wn, lane, m0, n0, M, bias, gate, Cv, ldc, out_scale, lds_out);
}

template <int Q>
hipError_t launch_gemm_t(const void *A, int64_t lda, const void *B, int64_t ldb, int M, int N, int K,
                         const float *bias, const float *gate, void *C, int64_t ldc, int epilogue,
                         const void *a_scale, const void *b_scale, int64_t lds_a, int64_t lds_b, hipStream_t s,
                         uint8_t *out_scale = nullptr, int64_t lds_out = 0) {
  const int tiles = ((M + GBM - 1) / GBM) * (N / 256);
  switch (epilogue) {
#define DLO_GEMM_CASE(E)                                                                            \
  case E:                                                                                           \
    hipLaunchKernelGGL((gemm_pp_kernel<E, Q>), dim3(tiles), dim3(512), 0, s, A, lda, B, ldb, M, N, K, \
                       bias, gate, C, ldc, a_scale, b_scale, lds_a, lds_b, out_scale, lds_out);    \
    break;
    DLO_GEMM_CASE(EPI_BIAS)
    DLO_GEMM_CASE(EPI_BIAS_GELU)
    DLO_GEMM_CASE(EPI_GATED_RESIDUAL)
    DLO_GEMM_CASE(EPI_BIAS_T)
    case EPI_GELU_MX:
      if constexpr (Q == 2) {
        hipLaunchKernelGGL((gemm_pp_kernel<EPI_GELU_MX, 2>), dim3(tiles), dim3(512), 0, s, A, lda, B, ldb, M, N, K,
                           bias, gate, C, ldc, a_scale, b_scale, lds_a, lds_b, out_scale, lds_out);
        break;
      }
      return hipErrorInvalidValue;
#undef DLO_GEMM_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int M,
                       int N, int K, const float *bias, const float *gate, void *C, int64_t ldc,
                       int epilogue, hipStream_t s) {
  return launch_gemm_t<0>(A, lda, B, ldb, M, N, K, bias, gate, C, ldc, epilogue, nullptr, nullptr, 0, 0, s);
}

hipError_t launch_gemm_fp8(const uint8_t *A, int64_t lda, const float *a_scale, const uint8_t *B,
                           int64_t ldb, const float *b_scale, int M, int N, int K, const float *bias,
                           const float *gate, void *C, int64_t ldc, int epilogue, hipStream_t s) {
  return launch_gemm_t<1>(A, lda, B, ldb, M, N, K, bias, gate, C, ldc, epilogue, a_scale, b_scale, 0, 0, s);
}

hipError_t launch_gemm_int8(const int8_t *A, int64_t lda, const float *a_scale, const int8_t *B, int64_t ldb,
                            const float *b_scale, int M, int N, int K, const float *bias, const float *gate, void *C,
                            int64_t ldc, int epilogue, hipStream_t s) {
  if (K % 64) return hipErrorInvalidValue;
  return launch_gemm_t<3>(A, lda, B, ldb, M, N, K, bias, gate, C, ldc, epilogue, a_scale, b_scale, 0, 0, s);
}

hipError_t launch_gemm_mxfp8(const uint8_t *A, int64_t lda, const uint8_t *a_scale, int64_t lds_a,
                             const uint8_t *B, int64_t ldb, const uint8_t *b_scale, int64_t lds_b, int M, int N,
                             int K, const float *bias, const float *gate, void *C, int64_t ldc, int epilogue,
                             hipStream_t s, uint8_t *out_scale, int64_t lds_out) {
  if (lds_a < M || lds_a % 4 || lds_b % 4 || K % 64) return hipErrorInvalidValue;
  if (epilogue == EPI_GELU_MX && (!out_scale || lds_out < M || ldc % 8)) return hipErrorInvalidValue;
  return launch_gemm_t<2>(A, lda, B, ldb, M, N, K, bias, gate, C, ldc, epilogue, a_scale, b_scale, lds_a, lds_b,
                          s, out_scale, lds_out);
}

}  // namespace dlo
