// gfx950 (CDNA4) kernels of the DiT block forward and the slot digest.
//
// Block math: adaLN-Zero DiT block (adaLN 6-way modulation, LayerNorm, fused
// QKV, softmax attention, output projection, 4d GELU MLP, gated residuals) --
// the block a DiT stack streamed by the method in "Distributed Layerwise
// Offload" (vLLM-Omni blog) runs unchanged.  Operand layout: weights are
// [out, in] row-major, so every GEMM is C = A B^T with both operands contiguous
// along K.
//
// Wave size 64.  MFMA: v_mfma_f32_32x32x16_bf16.  For that instruction lane l
// supplies row (l % 32) of A and column (l % 32) of B, each as eight bf16 at
// k = 8 * (l / 32) .. +7, and receives column (l % 32) of the 32x32 fp32
// result at rows (r / 4) * 8 + (l / 32) * 4 + r % 4, r = 0..15.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dlo {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

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

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752440f));
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

template <int VPT>  // values per thread: d / 256
__global__ __launch_bounds__(256) void ln_modulate_kernel(
    const float *__restrict__ x, int64_t ldx, int d, const float *__restrict__ gamma,
    const float *__restrict__ beta, const float *__restrict__ eps_p,
    const float *__restrict__ shift, const float *__restrict__ scale, uint16_t *__restrict__ out) {
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int64_t row = blockIdx.x;
  const float *xr = x + row * ldx;
  float v[VPT];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    v[i] = xr[i * 256 + tid];
    s += v[i];
  }
  s = wave_sum(s);
  if (lane == 0) red[0][wv] = s;
  __syncthreads();
  const float mean = (red[0][0] + red[0][1] + red[0][2] + red[0][3]) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    float dv = v[i] - mean;
    q += dv * dv;
  }
  q = wave_sum(q);
  if (lane == 0) red[1][wv] = q;
  __syncthreads();
  const float var = (red[1][0] + red[1][1] + red[1][2] + red[1][3]) / (float)d;
  const float rstd = 1.0f / sqrtf(var + eps_p[0]);
  uint16_t *orow = out + row * d;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int col = i * 256 + tid;
    float y = (v[i] - mean) * rstd * gamma[col] + beta[col];
    y = y * (1.0f + scale[col]) + shift[col];
    orow[col] = f32_to_bf16(y);
  }
}

// ---------------------------------------------------------------------------
// GEMM: C[M, N] = A[M, K] B[N, K]^T, bf16 in, fp32 accumulate.
// Workgroup tile 256 x 256 x 64, 4 waves in 2 x 2, each wave 128 x 128 = 4 x 4
// MFMA 32x32 tiles.  Operand tiles are staged in LDS (two stages), rows of 64
// bf16 = 8 chunks of 16 B, chunk index XOR-swizzled with (row & 7) so that the
// 16-B MFMA operand reads of 8 consecutive rows hit distinct banks.
// ---------------------------------------------------------------------------

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int G_THREADS = 256;
constexpr int G_TILE_ELEMS = GBM * GBK;  // one operand tile, bf16 elements

__device__ __forceinline__ int g_lds_off(int row, int chunk) {  // element offset
  return row * GBK + ((chunk ^ (row & 7)) << 3);
}

template <int EPI>
__global__ __launch_bounds__(G_THREADS) void gemm_nt_kernel(
    const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
    int M, int N, int K, const float *__restrict__ bias, const float *__restrict__ gate,
    void *__restrict__ Cv, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][G_TILE_ELEMS];  // [stage][A|B]

  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int wm = wv >> 1, wn = wv & 1;

  // tile coordinates: XCD remap, then groups of 8 tile rows
  const int tiles_m = (M + GBM - 1) / GBM, tiles_n = N / GBN;
  const int total = tiles_m * tiles_n;
  int pid = xcd_remap(blockIdx.x, total);
  constexpr int GROUP_M = 8;
  const int group = pid / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (pid % (GROUP_M * tiles_n)) % gsz;
  const int tn = (pid % (GROUP_M * tiles_n)) / gsz;
  const int m0 = tm * GBM, n0 = tn * GBN;

  // global -> register staging: thread loads rows (tid / 8) + 32 j, chunk tid % 8.
  // Buffer loads: the A descriptor covers only the tile's valid rows, so rows
  // past M read as zero (and are never stored).
  const int ld_row = tid >> 3, ld_chunk = tid & 7;
  const int a_rows = min(M - m0, GBM);
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(A + (int64_t)m0 * lda), (short)0, a_rows * (int)lda * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(B + (int64_t)n0 * ldb), (short)0, GBN * (int)ldb * 2, 0x00020000);
  const int a_voff = (ld_row * (int)lda + ld_chunk * 8) * 2;
  const int b_voff = (ld_row * (int)ldb + ld_chunk * 8) * 2;
  const int a_step = 32 * (int)lda * 2, b_step = 32 * (int)ldb * 2;
  u32x4 ra_regs[8], rb_regs[8];

  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ra_regs[j] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff + j * a_step + k0 * 2, 0, 0);
      rb_regs[j] = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_voff + j * b_step + k0 * 2, 0, 0);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = ld_row + 32 * j;
      *reinterpret_cast<u32x4 *>(&smem[st][0][g_lds_off(r, ld_chunk)]) = ra_regs[j];
      *reinterpret_cast<u32x4 *>(&smem[st][1][g_lds_off(r, ld_chunk)]) = rb_regs[j];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / GBK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int frow = lane & 31, fk = lane >> 5;  // MFMA operand row / k-half of this lane
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GBK);
    const uint16_t *As = smem[st][0];
    const uint16_t *Bs = smem[st][1];
#pragma unroll
    for (int kk = 0; kk < GBK / 16; ++kk) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + frow;
        af[i] = *reinterpret_cast<const bf16x8 *>(&As[g_lds_off(r, kk * 2 + fk)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 128 + j * 32 + frow;
        bfr[j] = *reinterpret_cast<const bf16x8 *>(&Bs[g_lds_off(r, kk * 2 + fk)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 128 + j * 32 + frow;
    const float bn = bias[n];
    float gn = 0.f;
    if (EPI == EPI_GATED_RESIDUAL) gn = gate[n];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + fk * 4 + (r & 3);
        if (m < M) {
          float v = acc[i][j][r] + bn;
          if (EPI == EPI_BIAS) {
            reinterpret_cast<uint16_t *>(Cv)[(int64_t)m * ldc + n] = f32_to_bf16(v);
          } else if (EPI == EPI_BIAS_GELU) {
            reinterpret_cast<uint16_t *>(Cv)[(int64_t)m * ldc + n] = f32_to_bf16(gelu_erf(v));
          } else {
            float *xp = reinterpret_cast<float *>(Cv) + (int64_t)m * ldc + n;
            *xp = *xp + gn * v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Flash attention forward (non-causal), one head per workgroup column.
// Workgroup: 8 waves, 256 queries (32 per wave); keys in blocks of 64 staged in
// LDS (two stages).  Each wave computes S^T = K Q^T on MFMA so that a lane owns
// one query: the row statistics of the online softmax stay in the lane (plus one
// exchange with lane l ^ 32).  P^T in that layout is directly the B operand of
// O^T += V^T P^T; V is written to LDS transposed with the keys of each group of
// 16 permuted (position p holds key pi(p), pi swaps 4..7 with 8..11) so a lane's
// eight keys are one 16-B read.
// ---------------------------------------------------------------------------

constexpr int AQ = 256, AK = 64, A_WAVES = 8, A_THREADS = A_WAVES * WAVE;

__device__ __forceinline__ int perm16(int key) {  // position of key within its group of 16
  const int g = key & 15, base = key & ~15;
  const int p = (g >= 4 && g < 8) ? g + 4 : ((g >= 8 && g < 12) ? g - 4 : g);
  return base + p;
}

template <int DH>
__device__ __forceinline__ int k_lds_off(int key, int chunk) {  // K tile [AK][DH]
  return key * DH + ((chunk ^ (key & 7)) << 3);
}

__device__ __forceinline__ int vt_lds_off(int dh, int chunk) {  // V^T tile [DH][AK]
  const int sw = (dh & 7) ^ ((dh >> 3) & 7);
  return dh * AK + ((chunk ^ sw) << 3);
}

template <int DH>
__global__ __launch_bounds__(A_THREADS) void attention_kernel(const uint16_t *__restrict__ qkv,
                                                              int64_t ldq, int T, int H,
                                                              uint16_t *__restrict__ out,
                                                              int64_t ldo, float scale_log2) {
  constexpr int KCH = DH / 8;                      // 16-B chunks per K row
  constexpr int K_ITEMS = AK * KCH;                // 16-B chunks per K tile
  constexpr int K_PER_T = K_ITEMS / A_THREADS;     // 2 (DH 128) or 1 (DH 64)
  constexpr int V_ITEMS = (AK / 2) * KCH;          // (key pair, chunk) items per V tile
  constexpr int DT = DH / 32;                      // 32-row tiles of O^T
  constexpr int KK = DH / 16;                      // MFMA k-steps over dh
  static_assert(K_PER_T >= 1, "tile");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][AK * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][DH * AK];

  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int nqb = (T + AQ - 1) / AQ;
  const int lid = xcd_remap(blockIdx.x, nqb * H);
  const int head = lid / nqb, qb = lid % nqb;
  const int HD = H * DH;
  const uint16_t *Qg = qkv + head * DH;
  const uint16_t *Kg = qkv + HD + head * DH;
  const uint16_t *Vg = qkv + 2 * HD + head * DH;

  const int ql = lane & 31, hf = lane >> 5;
  const int q = qb * AQ + wv * 32 + ql;
  const int qc = q < T ? q : T - 1;

  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8 *>(Qg + (int64_t)qc * ldq + kk * 16 + hf * 8);

  // staging registers for the next key block
  u32x4 kreg[K_PER_T], vreg0, vreg1;
  const bool v_active = tid < V_ITEMS;
  const int v_kp = tid / KCH, v_dc = tid % KCH;

  auto gload = [&](int kbase) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int item = tid + i * A_THREADS;
      const int key = item / KCH, dc = item % KCH;
      int kr = kbase + key;
      kr = kr < T ? kr : T - 1;
      kreg[i] = *reinterpret_cast<const u32x4 *>(Kg + (int64_t)kr * ldq + dc * 8);
    }
    if (v_active) {
      int k0 = kbase + 2 * v_kp, k1 = k0 + 1;
      k0 = k0 < T ? k0 : T - 1;
      k1 = k1 < T ? k1 : T - 1;
      vreg0 = *reinterpret_cast<const u32x4 *>(Vg + (int64_t)k0 * ldq + v_dc * 8);
      vreg1 = *reinterpret_cast<const u32x4 *>(Vg + (int64_t)k1 * ldq + v_dc * 8);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int item = tid + i * A_THREADS;
      const int key = item / KCH, dc = item % KCH;
      *reinterpret_cast<u32x4 *>(&Ks[st][k_lds_off<DH>(key, dc)]) = kreg[i];
    }
    if (v_active) {
      const int pos = perm16(2 * v_kp);  // even position; the pair stays adjacent
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (e & 1) ? (vreg0[e >> 1] >> 16) : (vreg0[e >> 1] & 0xffffu);
        const uint32_t hi = (e & 1) ? (vreg1[e >> 1] >> 16) : (vreg1[e >> 1] & 0xffffu);
        const int dh = v_dc * 8 + e;
        *reinterpret_cast<uint32_t *>(&Vt[st][vt_lds_off(dh, pos >> 3) + (pos & 7)]) =
            lo | (hi << 16);
      }
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nkb = (T + AK - 1) / AK;
  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < nkb; ++j) {
    const int st = j & 1;
    if (j + 1 < nkb) gload((j + 1) * AK);

    // S^T = K Q^T for the block's two 32-key halves
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(
            &Ks[st][k_lds_off<DH>(kb * 32 + ql, kk * 2 + hf)]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[kb], 0, 0, 0);
      }
    }

    // online softmax (base 2), lane-local over its 32 keys + one exchange
    const int kbase = j * AK;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + kb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
        const float v = key < T ? s[kb][r] * scale_log2 : -INFINITY;
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] *= alpha;

    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kb][r] - m_new);
        l_run += p;
        pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }

    // O^T += V^T P^T over the four 16-key chunks
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(
            &Vt[st][vt_lds_off(t * 32 + ql, c * 2 + hf)]);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], o[t], 0, 0, 0);
      }

    if (j + 1 < nkb) lstore(st ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, WAVE);
  const float inv = 1.0f / l_tot;
  if (q < T) {
    uint16_t *orow = out + (int64_t)q * ldo + head * DH;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[t][g * 4 + e] * inv);
        *reinterpret_cast<bf16x4 *>(orow + t * 32 + g * 8 + hf * 4) = v;
      }
  }
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

template <int VPT>
hipError_t ln_launch(const float *x, int64_t ldx, int T, int d, const float *gamma,
                     const float *beta, const float *eps, const float *shift, const float *scale,
                     uint16_t *out, hipStream_t s) {
  hipLaunchKernelGGL(ln_modulate_kernel<VPT>, dim3(T), dim3(256), 0, s, x, ldx, d, gamma, beta,
                     eps, shift, scale, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_silu(const float *c, float *out, int n, hipStream_t s) {
  hipLaunchKernelGGL(silu_kernel, dim3((n + 255) / 256), dim3(256), 0, s, c, out, n);
  return hipGetLastError();
}

hipError_t launch_adaln_gemv(const uint16_t *W, const float *sc, const float *b, float *out,
                             int rows, int d, hipStream_t s) {
  hipLaunchKernelGGL(adaln_gemv_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, W, sc, b, out,
                     rows, d);
  return hipGetLastError();
}

hipError_t launch_ln_modulate(const float *x, int64_t ldx, int T, int d, const float *gamma,
                              const float *beta, const float *eps, const float *shift,
                              const float *scale, uint16_t *out, hipStream_t s) {
  switch (d / 256) {
#define DLO_LN_CASE(V) \
  case V:              \
    return ln_launch<V>(x, ldx, T, d, gamma, beta, eps, shift, scale, out, s);
    DLO_LN_CASE(1) DLO_LN_CASE(2) DLO_LN_CASE(3) DLO_LN_CASE(4) DLO_LN_CASE(5) DLO_LN_CASE(6)
    DLO_LN_CASE(7) DLO_LN_CASE(8) DLO_LN_CASE(9) DLO_LN_CASE(10) DLO_LN_CASE(11)
    DLO_LN_CASE(12) DLO_LN_CASE(13) DLO_LN_CASE(14) DLO_LN_CASE(15) DLO_LN_CASE(16)
    DLO_LN_CASE(17) DLO_LN_CASE(18) DLO_LN_CASE(19) DLO_LN_CASE(20) DLO_LN_CASE(21)
    DLO_LN_CASE(22) DLO_LN_CASE(23) DLO_LN_CASE(24) DLO_LN_CASE(25) DLO_LN_CASE(26)
    DLO_LN_CASE(27) DLO_LN_CASE(28) DLO_LN_CASE(29) DLO_LN_CASE(30) DLO_LN_CASE(31)
    DLO_LN_CASE(32)
#undef DLO_LN_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int M,
                       int N, int K, const float *bias, const float *gate, void *C, int64_t ldc,
                       int epilogue, hipStream_t s) {
  const int tiles = ((M + GBM - 1) / GBM) * (N / GBN);
  switch (epilogue) {
    case EPI_BIAS:
      hipLaunchKernelGGL(gemm_nt_kernel<EPI_BIAS>, dim3(tiles), dim3(G_THREADS), 0, s, A, lda, B,
                         ldb, M, N, K, bias, gate, C, ldc);
      break;
    case EPI_BIAS_GELU:
      hipLaunchKernelGGL(gemm_nt_kernel<EPI_BIAS_GELU>, dim3(tiles), dim3(G_THREADS), 0, s, A,
                         lda, B, ldb, M, N, K, bias, gate, C, ldc);
      break;
    case EPI_GATED_RESIDUAL:
      hipLaunchKernelGGL(gemm_nt_kernel<EPI_GATED_RESIDUAL>, dim3(tiles), dim3(G_THREADS), 0, s,
                         A, lda, B, ldb, M, N, K, bias, gate, C, ldc);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const uint16_t *qkv, int64_t ldqkv, int T, int H, int dh,
                            uint16_t *out, int64_t ldo, hipStream_t s) {
  const int nqb = (T + AQ - 1) / AQ;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)dh);
  if (dh == 128) {
    hipLaunchKernelGGL(attention_kernel<128>, dim3(nqb * H), dim3(A_THREADS), 0, s, qkv, ldqkv,
                       T, H, out, ldo, scale_log2);
  } else if (dh == 64) {
    hipLaunchKernelGGL(attention_kernel<64>, dim3(nqb * H), dim3(A_THREADS), 0, s, qkv, ldqkv,
                       T, H, out, ldo, scale_log2);
  } else {
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
