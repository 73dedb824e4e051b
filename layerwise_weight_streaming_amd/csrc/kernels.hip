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

#include <type_traits>

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
// GEMM tiles: 256 rows of A per workgroup.
// ---------------------------------------------------------------------------

constexpr int GBM = 256;

// ---------------------------------------------------------------------------
// GEMM: C[M, N] = A[M, K] B[N, K]^T, bf16 in, fp32 accumulate (direct-to-LDS).
// Workgroup tile 256 x 256 x 32, 2 x WN waves (128 x 256/WN each, in MFMA
// 32x32 tiles; WN = 4 on every DiT launch).  Operand tiles travel HBM/L2 -> LDS with buffer_load ... lds
// (no register staging) into a ring of 4 LDS stages, up to four tiles ahead of
// the one being multiplied.  One LDS stage = A and B tiles of 256 rows x 64 B;
// a row holds 4 chunks of 16 B whose order is XOR-swizzled (dl_swz) so that
// the MFMA operand reads are free of bank conflicts.  A load instruction fills
// 1 KB of LDS: 64 lanes x 16 B at M0 + 16 * lane, i.e. 16 rows; the waves
// share the 16 such loads per operand per tile.
// ---------------------------------------------------------------------------

constexpr int DL_BK = 32;
constexpr int DL_TILE = GBM * DL_BK;  // bf16 elements of one operand tile (16 KB)

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// chunk swizzle of row r: ((r >> 1) ^ (r >> 2)) & 3.  A 16-B read by 16
// consecutive rows (one 64-bank LDS cycle) then hits 16 distinct 16-B bank
// groups, and so do 8 consecutive rows within a 32-bank cycle.
__device__ __forceinline__ int dl_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

__device__ __forceinline__ int dl_lds_off(int row, int chunk) {  // element offset in a tile
  return row * DL_BK + ((chunk ^ dl_swz(row)) << 3);
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

// s_waitcnt vmcnt(N) then s_barrier (N an immediate)
template <int N>
__device__ __forceinline__ void vmcnt_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// BN: workgroup tile width; STAGES: depth of the LDS ring; WN: waves along N
// (the wave grid is 2 x WN, each wave owns 128 x BN / WN).
template <int EPI, int BN, int STAGES, int WN = 2>
__global__ __launch_bounds__(128 * WN, (BN == 128 && WN == 2) ? 2 : 1) void gemm_nt_dl_kernel(
    const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
    int M, int N, int K, const float *__restrict__ bias, const float *__restrict__ gate,
    void *__restrict__ Cv, int64_t ldc) {
  constexpr int NW = 2 * WN;                  // waves per workgroup
  constexpr int NJ = BN / WN / 32;            // 32-wide column tiles per wave
  constexpr int B_TILE = BN * DL_BK;          // bf16 elements of the B tile
  constexpr int STAGE = DL_TILE + B_TILE;     // bf16 elements of one stage
  constexpr int ALOADS = 16 / NW;             // A load instructions per wave per tile
  constexpr int BLOADS = BN / 16 / NW;        // B load instructions per wave per tile
  constexpr int LPT = ALOADS + BLOADS;        // load instructions per lane per tile
  constexpr int READS = 4 + NJ;               // fragment reads per half step
  __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES * STAGE];

  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int wm = wv / WN, wn = wv % WN;

  const int tiles_m = (M + GBM - 1) / GBM, tiles_n = N / BN;
  const int total = tiles_m * tiles_n;
  int pid = xcd_remap(blockIdx.x, total);
  constexpr int GROUP_M = 8;
  const int group = pid / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (pid % (GROUP_M * tiles_n)) % gsz;
  const int tn = (pid % (GROUP_M * tiles_n)) / gsz;
  const int m0 = tm * GBM, n0 = tn * BN;

  const int a_rows = min(M - m0, GBM);
  const i32x4 a_rsrc = dl_rsrc(A + (int64_t)m0 * lda, (uint32_t)(a_rows * lda * 2));
  const i32x4 b_rsrc = dl_rsrc(B + (int64_t)n0 * ldb, (uint32_t)(BN * ldb * 2));

  // this lane's source offsets: A blocks wv*ALOADS + i, B blocks wv*BLOADS + i
  // (16 rows each)
  int a_voff[ALOADS], b_voff[BLOADS];
#pragma unroll
  for (int i = 0; i < ALOADS; ++i) {
    const int r = (wv * ALOADS + i) * 16 + (lane >> 2);
    a_voff[i] = (r * (int)lda + ((lane & 3) ^ dl_swz(r)) * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < BLOADS; ++i) {
    const int r = (wv * BLOADS + i) * 16 + (lane >> 2);
    b_voff[i] = (r * (int)ldb + ((lane & 3) ^ dl_swz(r)) * 8) * 2;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)&smem[0];
  auto issue = [&](int kt) {
    const uint32_t sbase = lds0 + (uint32_t)((kt % STAGES) * STAGE * 2);
#pragma unroll
    for (int i = 0; i < ALOADS; ++i)
      dl_load(a_rsrc, __builtin_amdgcn_readfirstlane(sbase + (uint32_t)((wv * ALOADS + i) * 1024)),
              a_voff[i] + kt * DL_BK * 2);
#pragma unroll
    for (int i = 0; i < BLOADS; ++i)
      dl_load(b_rsrc,
              __builtin_amdgcn_readfirstlane(sbase + (uint32_t)(DL_TILE * 2 + (wv * BLOADS + i) * 1024)),
              b_voff[i] + kt * DL_BK * 2);
  };

  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / DL_BK;
  const int frow = lane & 31, fk = lane >> 5;

  // operand fragments of one 16-wide k step: 4 A (rows) and NJ B (columns)
  struct Frags {
    bf16x8 a[4], b[NJ];
  };
  auto read_frags = [&](int st, int kk, Frags &f) {
    const uint16_t *As = smem + st * STAGE;
    const uint16_t *Bs = As + DL_TILE;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[i] = *reinterpret_cast<const bf16x8 *>(&As[dl_lds_off(wm * 128 + i * 32 + frow, kk * 2 + fk)]);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      f.b[j] = *reinterpret_cast<const bf16x8 *>(
          &Bs[dl_lds_off(wn * (BN / WN) + j * 32 + frow, kk * 2 + fk)]);
  };
  auto mma = [&](const Frags &f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  // wait until at most `younger` tiles' loads (LPT per tile per lane) are in
  // flight, then barrier.  The wave's own LDS reads of the stage about to be
  // refilled are drained before (see `drained`), so after the barrier no wave
  // still reads it.
  auto sync_tiles = [&](int younger) {
    if (younger >= 3)
      vmcnt_barrier<3 * LPT>();
    else if (younger == 2)
      vmcnt_barrier<2 * LPT>();
    else if (younger == 1)
      vmcnt_barrier<LPT>();
    else
      vmcnt_barrier<0>();
  };
  // a use of the fragment registers: the compiler waits for their LDS reads here
  // (and knows it did, so it adds no stale waits later)
  auto drained = [&](const Frags &f) {
    asm volatile("" ::"v"(f.a[0]), "v"(f.a[1]), "v"(f.a[2]), "v"(f.a[3]));
#pragma unroll
    for (int j = 0; j < NJ; ++j) asm volatile("" ::"v"(f.b[j]));
  };
  // Within one half: the fragment reads go out one per MFMA, the remaining
  // MFMAs cover their latency.
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < READS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NJ - READS, 0);
  };

  // Pipeline: up to STAGES - 1 younger tiles are in flight while tile t is
  // multiplied.  Each tile is two half-steps: MFMAs of k-step 0 run while k-step
  // 1's fragments are read; after the tile barrier, MFMAs of k-step 1 run while
  // the next tile's k-step 0 fragments are read.
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue(s);
  sync_tiles(min(nk - 1, STAGES - 1));
  Frags f0, f1;
  read_frags(0, 0, f0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % STAGES;
    read_frags(st, 1, f1);
    mma(f0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);  // every MFMA issues before the wait below
    drained(f1);
    asm volatile("" ::: "memory");
    // tile kt+1 landed (younger tiles may still be in flight); stage st is free
    sync_tiles(min(nk - 2 - kt, STAGES - 2));
    if (kt + STAGES < nk) issue(kt + STAGES);
    // next tile's k-step 0 (on the last tile this reads a stale stage, unused);
    // unconditional so the compiler's LDS counter bookkeeping stays exact
    read_frags((kt + 1) % STAGES, 0, f0);
    mma(f1);
    interleave();
    asm volatile("" ::: "memory");
  }

  // Epilogue, one 32x32 sub-tile at a time.  Offsets are 32-bit from the tile's
  // first row; a residual sub-tile's 16 loads all issue before any of its stores;
  // only the last row tile checks rows against M.
  const bool full = m0 + GBM <= M;
  const int ldc32 = (int)ldc;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn * (BN / WN) + j * 32 + frow;
    const float bn = bias[n];
    float gn = 0.f;
    if (EPI == EPI_GATED_RESIDUAL) gn = gate[n];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mr0 = wm * 128 + i * 32 + fk * 4;  // row of r = 0, relative to m0
      if (EPI == EPI_GATED_RESIDUAL) {
        float *X = reinterpret_cast<float *>(Cv) + (int64_t)m0 * ldc;
        float xv[16];
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) xv[r] = X[(mr0 + (r >> 2) * 8 + (r & 3)) * ldc32 + n];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            X[(mr0 + (r >> 2) * 8 + (r & 3)) * ldc32 + n] = xv[r] + gn * (acc[i][j][r] + bn);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int mr = mr0 + (r >> 2) * 8 + (r & 3);
            xv[r] = m0 + mr < M ? X[mr * ldc32 + n] : 0.f;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int mr = mr0 + (r >> 2) * 8 + (r & 3);
            if (m0 + mr < M) X[mr * ldc32 + n] = xv[r] + gn * (acc[i][j][r] + bn);
          }
        }
      } else {
        uint16_t *C = reinterpret_cast<uint16_t *>(Cv) + (int64_t)m0 * ldc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mr = mr0 + (r >> 2) * 8 + (r & 3);
          float v = acc[i][j][r] + bn;
          if (EPI == EPI_BIAS_GELU) v = gelu_erf(v);
          if (full || m0 + mr < M) C[mr * ldc32 + n] = f32_to_bf16(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Flash attention forward (non-causal), one head per workgroup column.
// Workgroup: 8 waves, 256 queries (32 per wave).  Keys/values in blocks of 64
// travel HBM/L2 -> LDS by buffer_load ... lds, both key-major, into separate
// two-slot rings for K and V, K one block ahead of V.  Each wave computes
// S^T = K Q^T on MFMA, so a lane owns one query and the online-softmax
// statistics stay in the lane (one exchange with lane l ^ 32, by
// v_permlane32_swap).  P^T in that layout is the B operand of O^T += V^T P^T;
// the V^T operand comes straight from the key-major V tile via
// ds_read_b64_tr_b16 (for a group of 16 lanes, lane j receives element j % 4
// of the 4-element loads of lanes 4t + j / 4, t = 0..3).
//
// Software pipeline: block j's scores are computed one iteration ahead, so
// while the MFMAs of S_{j+1} = K_{j+1} Q^T run, the same wave takes the softmax
// of block j on the VALU (max, exp2, bf16 packing); then O^T += V_j^T P_j^T,
// with the row sums of P_j taken by v_dot2 (on the bf16 P the MFMA uses) in the
// shadow of those MFMAs.  One barrier per block; every load has a whole block
// of compute to land in.
//
// Softmax in base 2 on raw scores s: p = exp2(s * c - m * c), c = log2(e)/sqrt(dh).
// The running max m is raised only when a block's max exceeds it by more than
// 8 / c (so p <= 2^8), which leaves the rescale of O and l out of most blocks;
// the result is the same softmax, normalised by the same running sum.
// ---------------------------------------------------------------------------

constexpr int AK = 64;

typedef short v4i16 __attribute__((ext_vector_type(4)));

// 16-B chunk swizzles of the key-major K and V tiles (rows of DH bf16).
// K: MFMA A reads of 16 consecutive key rows at one chunk hit 16 distinct bank
// groups.  V: a transposed read touches 4 consecutive keys x 32 B; the swizzle
// moves each key's 32 B to its own quarter of the 256-B bank window.
template <int DH>
__device__ __forceinline__ int k_swz(int key) {
  return DH == 128 ? (key & 15) : ((key >> 1) & 7);
}
template <int DH>
__device__ __forceinline__ int v_swz(int key) {
  return (key & 3) * (DH / 32);
}

// A_WAVES waves of 32 queries per workgroup.
template <int DH, int A_WAVES>
__global__ __launch_bounds__(A_WAVES * 64, A_WAVES == 4 ? 2 : 1) void attention_kernel(
    const uint16_t *__restrict__ qkv, int64_t ldq, int T, int H, uint16_t *__restrict__ out,
    int64_t ldo, float scale_log2) {
  constexpr int AQ = 32 * A_WAVES;
  constexpr int KCH = DH / 8;
  constexpr int TILE = AK * DH;
  constexpr int ROWS_PER_LD = 1024 / (DH * 2);
  constexpr int LD_PER_WAVE = AK / ROWS_PER_LD / A_WAVES;
  constexpr int DT = DH / 32;
  constexpr int KK = DH / 16;
  // tiles: K slot 0, K slot 1, V slot 0, V slot 1
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TILE];

  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int nqb = (T + AQ - 1) / AQ;
  const int lid = xcd_remap(blockIdx.x, nqb * H);
  const int head = lid / nqb, qb = lid % nqb;
  const int HD = H * DH;

  const int ql = lane & 31, hf = lane >> 5;
  const int q = qb * AQ + wv * 32 + ql;
  const int qc = q < T ? q : T - 1;

  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8 *>(qkv + (int64_t)qc * ldq + head * DH + kk * 16 + hf * 8);

  const uint32_t rec = (uint32_t)((int64_t)T * ldq * 2);
  const i32x4 k_rsrc = dl_rsrc(qkv + HD + head * DH, rec);
  const i32x4 v_rsrc = dl_rsrc(qkv + 2 * HD + head * DH, rec);
  int k_voff[LD_PER_WAVE], v_voff[LD_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LD_PER_WAVE; ++i) {
    const int row = (wv * LD_PER_WAVE + i) * ROWS_PER_LD + lane / KCH;
    const int p = lane % KCH;
    k_voff[i] = (row * (int)ldq + (p ^ k_swz<DH>(row)) * 8) * 2;
    v_voff[i] = (row * (int)ldq + (p ^ v_swz<DH>(row)) * 8) * 2;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)&smem[0];
  auto issue_k = [&](int j, int tile) {
    const uint32_t sb = lds0 + (uint32_t)(tile * TILE * 2);
    const int off = j * AK * (int)ldq * 2;
#pragma unroll
    for (int i = 0; i < LD_PER_WAVE; ++i)
      dl_load(k_rsrc, __builtin_amdgcn_readfirstlane(sb + (uint32_t)((wv * LD_PER_WAVE + i) * 1024)),
              k_voff[i] + off);
  };
  auto issue_v = [&](int j, int tile) {
    const uint32_t sb = lds0 + (uint32_t)(tile * TILE * 2);
    const int off = j * AK * (int)ldq * 2;
#pragma unroll
    for (int i = 0; i < LD_PER_WAVE; ++i)
      dl_load(v_rsrc, __builtin_amdgcn_readfirstlane(sb + (uint32_t)((wv * LD_PER_WAVE + i) * 1024)),
              v_voff[i] + off);
  };

  const int g16 = lane >> 4, li = lane & 15;
  const int vt_key = 4 * hf + (li >> 2);
  const int vt_dh = 16 * (g16 & 1) + 4 * (li & 3);
  int k_lane[KK], v_lane[DT];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    k_lane[kk] = (ql * DH + (((kk * 2 + hf) ^ k_swz<DH>(ql)) << 3)) * 2;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const int dh = 32 * t + vt_dh;
    v_lane[t] = (vt_key * DH + (((dh >> 3) ^ v_swz<DH>(vt_key)) << 3) + (dh & 7)) * 2;
  }
  const char *lds_bytes = reinterpret_cast<const char *>(&smem[0]);

  // S^T of one block: two 32-key halves, their MFMA chains interleaved
  auto qk = [&](const char *Kb, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Kb + kb * 32 * DH * 2 + k_lane[kk]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[kb], 0, 0, 0);
      }
  };

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float tau = 8.0f / scale_log2;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  const int nkb = (T + AK - 1) / AK;
  issue_k(0, 0);
  issue_v(0, 2);
  if (nkb > 1) issue_k(1, 1);
  vmcnt_barrier<0>();
  f32x16 sa[2], sb[2];
  qk(lds_bytes, sa);

  // block j (parity P = j & 1): scores sc (computed one iteration earlier),
  // next block's scores into sn; K_{j+1} in K slot 1 - P, V_j in V slot P
  auto iter = [&](int j, auto par_c, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    constexpr int P = decltype(par_c)::value;
    // K_{j+1} and V_j landed, and every wave is done with block j - 1
    vmcnt_barrier<0>();
    if (j + 2 < nkb) issue_k(j + 2, P);         // K_j's slot
    if (j + 1 < nkb) issue_v(j + 1, 2 + 1 - P); // V_{j-1}'s slot
    const char *Kn = lds_bytes + (1 - P) * TILE * 2;
    const char *Vb = lds_bytes + (2 + P) * TILE * 2;

    const int kbase = j * AK;
    if (kbase + AK > T) {  // last, partial block: keys >= T do not exist
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + kb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3) >= T) sc[kb][r] = -INFINITY;
    }
    float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const bool need = __any(mx > m_run + tau);
    const float m_new = need ? fmaxf(m_run, mx) : m_run;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
    m_run = m_new;
    const float mc = m_new * scale_log2;
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], scale_log2, -mc));

    qk(Kn, sn);  // next block's scores (unused after the last block)
    // interleave the 16 MFMAs with the K operand reads (two ahead) and the
    // softmax VALU work
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i < 14) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // VALU
    }
    // P_j is complete here, ahead of the rescale branch (keeps the exp2 work in
    // this block, next to the MFMAs it overlaps)
    asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(pf[2]), "v"(pf[3]));

    if (need) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
    }

    // O^T += V^T P^T over the four 16-key chunks; row sums of P on the VALU
    float ls = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const char *p1 = Vb + c * 16 * DH * 2 + v_lane[t];
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16 *)(p1));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16 *)(p1 + 8 * DH * 2));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], o[t], 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[c][2 * e], pf[c][2 * e + 1]}, ones, ls, false);
    }
    l_run = l_run * alpha + ls;
  };
  int j = 0;
  for (; j + 1 < nkb; j += 2) {
    iter(j, std::integral_constant<int, 0>{}, sa, sb);
    iter(j + 1, std::integral_constant<int, 1>{}, sb, sa);
  }
  if (j < nkb) iter(j, std::integral_constant<int, 0>{}, sa, sb);

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

namespace {
template <int BN, int STAGES, int WN>
hipError_t gemm_launch(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int M, int N,
                       int K, const float *bias, const float *gate, void *C, int64_t ldc,
                       int epilogue, hipStream_t s) {
  const int tiles = ((M + GBM - 1) / GBM) * (N / BN);
  switch (epilogue) {
    case EPI_BIAS:
      hipLaunchKernelGGL((gemm_nt_dl_kernel<EPI_BIAS, BN, STAGES, WN>), dim3(tiles), dim3(128 * WN), 0,
                         s, A, lda, B, ldb, M, N, K, bias, gate, C, ldc);
      break;
    case EPI_BIAS_GELU:
      hipLaunchKernelGGL((gemm_nt_dl_kernel<EPI_BIAS_GELU, BN, STAGES, WN>), dim3(tiles),
                         dim3(128 * WN), 0, s, A, lda, B, ldb, M, N, K, bias, gate, C, ldc);
      break;
    case EPI_GATED_RESIDUAL:
      hipLaunchKernelGGL((gemm_nt_dl_kernel<EPI_GATED_RESIDUAL, BN, STAGES, WN>), dim3(tiles),
                         dim3(128 * WN), 0, s, A, lda, B, ldb, M, N, K, bias, gate, C, ldc);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int M,
                       int N, int K, const float *bias, const float *gate, void *C, int64_t ldc,
                       int epilogue, hipStream_t s) {
  // 256 x 256 tiles, a 4-deep ring and eight waves (2 x 4, 128 x 64 each):
  // faster than four 128 x 128 waves (5-12 % on the DiT shapes: two waves per
  // SIMD hide the LDS latency of each other's fragment reads) and than
  // 256 x 128 tiles at two workgroups per CU
  return gemm_launch<256, 4, 4>(A, lda, B, ldb, M, N, K, bias, gate, C, ldc, epilogue, s);
}

hipError_t launch_attention(const uint16_t *qkv, int64_t ldqkv, int T, int H, int dh,
                            uint16_t *out, int64_t ldo, hipStream_t s) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)dh);
  // 8 waves (256 queries) per workgroup, one workgroup per CU: faster than
  // 4 waves at two workgroups per CU (each K/V tile then serves twice the
  // queries; 3.6 % on the Super attention shape)
  const int nqb = (T + 255) / 256;
  if (dh == 128) {
    hipLaunchKernelGGL((attention_kernel<128, 8>), dim3(nqb * H), dim3(512), 0, s, qkv, ldqkv, T,
                       H, out, ldo, scale_log2);
  } else if (dh == 64) {
    hipLaunchKernelGGL((attention_kernel<64, 8>), dim3(nqb * H), dim3(512), 0, s, qkv, ldqkv, T, H,
                       out, ldo, scale_log2);
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
