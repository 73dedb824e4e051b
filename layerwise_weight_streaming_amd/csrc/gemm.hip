// gfx950 GEMM of the DiT block linears: C = A B^T with bf16 operands, fp32
// accumulation and fused epilogues (bias, bias + GELU, gated residual).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace dlo {
namespace {

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

// chunk swizzle of row r: ((r >> 1) ^ (r >> 2)) & 3.  A 16-B read by 16
// consecutive rows (one 64-bank LDS cycle) then hits 16 distinct 16-B bank
// groups, and so do 8 consecutive rows within a 32-bank cycle.
__device__ __forceinline__ int dl_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

__device__ __forceinline__ int dl_lds_off(int row, int chunk) {  // element offset in a tile
  return row * DL_BK + ((chunk ^ dl_swz(row)) << 3);
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
  // the epilogue reuses the ring as a staging tile: 256 rows of bf16 (row
  // stride C_LD) or 128 rows of fp32 (row stride X_LD)
  constexpr int C_LD = BN + 8;                // bf16 elements
  constexpr int X_LD = BN + 4;                // fp32 elements
  constexpr int RING = STAGES * STAGE;
  constexpr int CSTAGE = EPI == EPI_GATED_RESIDUAL ? 128 * X_LD * 2 : GBM * C_LD;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[RING > CSTAGE ? RING : CSTAGE];

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
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
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
  if (EPI != EPI_GATED_RESIDUAL) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * (BN / WN) + j * 32 + g * 8 + fk * 4;
        const float4 bv = *reinterpret_cast<const float4 *>(&bias[n0 + col]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v0 = acc[i][j][g * 4 + 0] + bv.x, v1 = acc[i][j][g * 4 + 1] + bv.y;
          float v2 = acc[i][j][g * 4 + 2] + bv.z, v3 = acc[i][j][g * 4 + 3] + bv.w;
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
          *reinterpret_cast<bf16x4 *>(&smem[(wm * 128 + i * 32 + frow) * C_LD + col]) = o;
        }
      }
    __syncthreads();
    constexpr int SEG = BN / 8;               // 16-B segments per row
    uint16_t *C = reinterpret_cast<uint16_t *>(Cv) + (int64_t)m0 * ldc + n0;
#pragma unroll
    for (int it = 0; it < GBM * SEG / NT; ++it) {
      const int e = it * NT + tid, row = e / SEG, c8 = (e % SEG) * 8;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&smem[row * C_LD + c8]);
      if (full || m0 + row < M) *reinterpret_cast<u32x4 *>(&C[row * ldc32 + c8]) = v;
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
            const float4 bv = *reinterpret_cast<const float4 *>(&bias[n0 + col]);
            const float4 gv = *reinterpret_cast<const float4 *>(&gate[n0 + col]);
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

}  // namespace

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

}  // namespace dlo
