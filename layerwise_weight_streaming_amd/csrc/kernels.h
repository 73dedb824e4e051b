// Internal launch interface of the gfx950 kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlo {

// out[i] = c[i] * sigmoid(c[i]), i < n
hipError_t launch_silu(const float *c, float *out, int n, hipStream_t s);

// out[r] = sum_j W[r, j] * sc[j] + b[r]   (W bf16 [rows, d], d % 8 == 0)
hipError_t launch_adaln_gemv(const uint16_t *W, const float *sc, const float *b, float *out,
                             int rows, int d, hipStream_t s);
// the adaLN GEMV with SiLU(c) staged in the library's static device scratch instead
// of a workspace: no allocation; d % 8 == 0, d <= NOALLOC_MAX_D
constexpr int NOALLOC_MAX_D = 8192;
hipError_t launch_adaln_noalloc(const uint16_t *W, const float *b, const float *cond, int rows, int d,
                                float *out, hipStream_t s);
// the adaLN GEMV on E4M3 codes W [rows, d] with per-tensor scale *wscale; d % 16 == 0
hipError_t launch_adaln_gemv_fp8(const uint8_t *W, const float *wscale, const float *sc, const float *b,
                                 float *out, int rows, int d, hipStream_t s);

// out[t, :] = bf16(LN(x[t, :d]) * (1 + scale) + shift); d % 256 == 0, d <= 8192
hipError_t launch_ln_modulate(const float *x, int64_t ldx, int T, int d, const float *gamma,
                              const float *beta, const float *eps, const float *shift,
                              const float *scale, uint16_t *out, hipStream_t s);
// the same fused with a W8A8 linear's input quantisation (no bf16 output): codes [T, ldq];
// mx = false: fp32 row scales qscale[T]; mx = true: E8M0 scales block-major [d / 32, lds],
// rows T .. lds - 1 set to 127 (lds >= T)
hipError_t launch_ln_modulate_quant(const float *x, int64_t ldx, int T, int d, const float *gamma,
                                    const float *beta, const float *eps, const float *shift, const float *scale,
                                    uint8_t *q, int64_t ldq, void *qscale, int64_t lds, bool mx, hipStream_t s);

// EPI_GELU_MX (MXFP8 GEMM only): bias + GELU, the bf16-rounded result quantised
// per 32 columns to E4M3 codes [M, ldc] and E8M0 scales block-major
// [N / 32, lds_out] (rows M .. lds_out - 1 inside the last row tile: 127)
enum GemmEpilogue { EPI_BIAS = 0, EPI_BIAS_GELU = 1, EPI_GATED_RESIDUAL = 2, EPI_BIAS_T = 3, EPI_GELU_MX = 4 };

// C = A B^T + bias (see dlo_op_gemm); N % 256 == 0, K % 64 == 0.  EPI_BIAS_T
// stores C^T [N, ldc]: rows m in [M, M rounded up to 64) as 0, nothing beyond
hipError_t launch_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int M,
                       int N, int K, const float *bias, const float *gate, void *C, int64_t ldc,
                       int epilogue, hipStream_t s);

// vt[f, t] = v[t, f] (f < d, t < T), 0 for T <= t < T rounded up to 64;
// d % 64 == 0, ldv and ldvt multiples of 8, ldvt >= T rounded up to 64
hipError_t launch_v_transpose(const uint16_t *v, int64_t ldv, int T, int d, uint16_t *vt,
                              int64_t ldvt, hipStream_t s);

// C = (A B^T) * a_scale[m] * *b_scale + bias with A, B OCP E4M3 codes ([M, K], [N, K],
// row strides in bytes), the epilogues and constraints of launch_gemm
hipError_t launch_gemm_fp8(const uint8_t *A, int64_t lda, const float *a_scale, const uint8_t *B,
                           int64_t ldb, const float *b_scale, int M, int N, int K, const float *bias,
                           const float *gate, void *C, int64_t ldc, int epilogue, hipStream_t s);
// INT8 GEMM: A [M, K] and B [N, K] int8 codes, exact int32 sums times a_scale[m] *
// b_scale[n] (fp32, b_scale 16-B aligned); the epilogues and constraints of launch_gemm
hipError_t launch_gemm_int8(const int8_t *A, int64_t lda, const float *a_scale, const int8_t *B, int64_t ldb,
                            const float *b_scale, int M, int N, int K, const float *bias, const float *gate, void *C,
                            int64_t ldc, int epilogue, hipStream_t s);
// MXFP8 GEMM: A [M, K] and B [N, K] E4M3 codes with E8M0 block scales block-major,
// a_scale [K / 32][lds_a] (row m at column m), b_scale [K / 32][lds_b] (row n at
// column n); lds_a >= M, lds_a and lds_b multiples of 4, K % 64 == 0
hipError_t launch_gemm_mxfp8(const uint8_t *A, int64_t lda, const uint8_t *a_scale, int64_t lds_a,
                             const uint8_t *B, int64_t ldb, const uint8_t *b_scale, int64_t lds_b, int M, int N,
                             int K, const float *bias, const float *gate, void *C, int64_t ldc, int epilogue,
                             hipStream_t s, uint8_t *out_scale = nullptr, int64_t lds_out = 0);

// per-head softmax(q k^T / sqrt(dh)) v: q, k from a fused qkv buffer, v from
// its feature-major copy vt (launch_v_transpose); dh in {64, 128}
hipError_t launch_attention(const uint16_t *qkv, int64_t ldqkv, const uint16_t *vt, int64_t ldvt,
                            int T, int H, int dh, uint16_t *out, int64_t ldo, hipStream_t s);

// out[i] = bf16_rne(e4m3_value(codes[i]) * *scale), i < n; n % 16 == 0, codes 16-B
// and out 32-B aligned
hipError_t launch_dequant_fp8(const uint8_t *codes, int64_t n, const float *scale, uint16_t *out,
                              hipStream_t s);
// INT8 weight [rows, cols] with one fp32 scale per row -> bf16; cols % 16 == 0
hipError_t launch_dequant_int8(const int8_t *codes, int64_t rows, int64_t cols, const float *scales,
                               uint16_t *out, hipStream_t s);
// MXFP8 weight [rows, cols] with E8M0 scales block-major [cols / 32, rows] -> bf16; cols % 32 == 0
hipError_t launch_dequant_mxfp8(const uint8_t *codes, int64_t rows, int64_t cols, const uint8_t *scales,
                                uint16_t *out, hipStream_t s);

// per-row dynamic E4M3 of bf16 x [M, K] (row stride ldx): scale[r] = amax_r / 448
// (1 for a zero row), q[r, k] = E4M3 code nearest to x / scale[r]; K, ldx, ldq
// multiples of 8, x 16-B and q 8-B aligned
hipError_t launch_quant_rows_fp8(const uint16_t *x, int64_t ldx, int M, int K, uint8_t *q, int64_t ldq,
                                 float *scale, hipStream_t s);
// per-row int8 of bf16 x [M, K]: scale[r] = amax_r / 127 (1 for a zero row), q[r, k] =
// x / scale[r] rounded to nearest-even, clamped to +-127; constraints as above
hipError_t launch_quant_rows_int8(const uint16_t *x, int64_t ldx, int M, int K, int8_t *q, int64_t ldq,
                                  float *scale, hipStream_t s);
// per-row MXFP8 of a bf16 matrix [M, K]: codes [M, ldq], E8M0 scales block-major
// [K / 32, lds] (rows M .. lds - 1: 127); K % 32 == 0, lds >= M
hipError_t launch_quant_rows_mx(const uint16_t *x, int64_t ldx, int M, int K, uint8_t *q, int64_t ldq,
                               uint8_t *scale, int64_t lds, hipStream_t s);

// sustained MFMA rate probe: MFMA_RATE_GRID workgroups of 512 threads, each wave
// iters x 262144 FLOP (form 0: 32x32x16 bf16, form 1: 16x16x32 bf16); in: 4096 x 8
// bf16 operand values; out: fp32 [MFMA_RATE_GRID * 512] checksums
constexpr int MFMA_RATE_GRID = 256;
hipError_t launch_mfma_rate(int form, const uint16_t *in, float *out, int iters, hipStream_t s);

// *out = digest of the regions (base + offsets[i], lengths[i]); offsets multiples of 8
hipError_t launch_digest(const void *base, const int64_t *offsets, const int64_t *lengths,
                         int n, uint64_t *out, hipStream_t s);

}  // namespace dlo
