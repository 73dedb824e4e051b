// gfx950 flash attention forward of the DiT block (non-causal softmax
// attention over all tokens, per head).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace dlo {
namespace {

// ---------------------------------------------------------------------------
// Flash attention forward (non-causal), one head per workgroup column.
// Workgroup: 8 waves, 256 queries (32 per wave).  Keys in blocks of 64 travel
// HBM/L2 -> LDS by buffer_load ... lds into a two-slot ring, key-major; values
// come from a feature-major copy V^T (rows of the head's dh features, T keys
// each) into a second two-slot ring, K one block ahead of V.  Each wave
// computes S^T = K Q^T on MFMA, so a lane owns one query and the
// online-softmax statistics stay in the lane (one exchange with lane l ^ 32, by
// v_permlane32_swap).  P^T in that layout is the B operand of O^T += V^T P^T,
// whose A operand (32 features x 16 keys) is one 16-B LDS read per lane in the
// feature-major tile.  Every operand read is one ds_read_b128 (the key-major
// V tile needed two 8-B transposing reads per operand: twice the LDS
// instructions and waits, 1.5 % slower on the Super shape).
//
// Software pipeline: block j's scores are computed one iteration ahead, so
// while the MFMAs of S_{j+1} = K_{j+1} Q^T run, the same wave turns the first
// 32 keys of block j into P on the VALU (exp2, bf16 packing, row sums by
// v_dot2 on the bf16 P the MFMA uses); then O^T += V_j^T P_j^T, with the
// second half's P in the shadow of the first half's MFMAs.  One barrier per
// block; every load has a whole block of compute to land in.
//
// Softmax in base 2: q is scaled by c = log2(e)/sqrt(dh) once (rounded to
// bf16, a relative change of at most 2^-9 per element), so the MFMA yields
// scores in log2 units, and each block's accumulators start at -m, the running
// max: the registers hold score - m and p = exp2 of them directly.  m starts at
// block 0's max and is not recomputed per block.  Each 32-key half is checked
// instead: while every lane's sum of p over the half stays below 2^64, every p
// does too, and fp32 O and l cannot overflow over any T; when it does not (a
// score more than 64 above m), the wave raises m to the half's max, rescales O
// and l, shifts every score register still to be used by the same amount and
// redoes the half's P -- the online-softmax update with each half as a step.
// The result is the same softmax, normalised by the same running sum, without
// a max reduction or a scale-and-subtract per score on the common path.
// ---------------------------------------------------------------------------

constexpr int AK = 64;
constexpr float P_LIMIT = 18446744073709551616.0f;  // 2^64

// 16-B chunk swizzles.  K (key-major, rows of DH bf16): MFMA A reads of 16
// consecutive key rows at one chunk hit 16 distinct bank groups.  V^T
// (feature-major, rows of 64 keys = 128 B): 16 consecutive feature rows at one
// chunk cover both 128-B halves of the 256-B bank window and, within a half,
// 8 distinct chunks.
template <int DH>
__device__ __forceinline__ int k_swz(int key) {
  return DH == 128 ? (key & 15) : ((key >> 1) & 7);
}
__device__ __forceinline__ int vt_swz(int feature) { return (feature >> 1) & 7; }

// A_WAVES waves of 32 queries per workgroup.
template <int DH, int A_WAVES>
__global__ __launch_bounds__(A_WAVES * 64, A_WAVES == 4 ? 2 : 1) void attention_kernel(
    const uint16_t *__restrict__ qkv, int64_t ldq, const uint16_t *__restrict__ vt, int64_t ldvt,
    int T, int H, uint16_t *__restrict__ out, int64_t ldo, float scale_log2) {
  constexpr int AQ = 32 * A_WAVES;
  constexpr int KCH = DH / 8;
  constexpr int TILE = AK * DH;
  constexpr int ROWS_PER_LD = 1024 / (DH * 2);
  constexpr int LD_PER_WAVE = AK / ROWS_PER_LD / A_WAVES;
  constexpr int VLD_PER_WAVE = DH / 8 / A_WAVES;  // 1 KB = 8 feature rows of 64 keys
  constexpr int DT = DH / 32;
  constexpr int KK = DH / 16;
  // tiles: K slot 0, K slot 1, V^T slot 0, V^T slot 1
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TILE];

  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int nqb = (T + AQ - 1) / AQ;
  const int lid = xcd_remap(blockIdx.x, nqb * H);
  const int head = lid / nqb, qb = lid % nqb;
  const int HD = H * DH;

  const int ql = lane & 31, hf = lane >> 5;
  const int q = qb * AQ + wv * 32 + ql;
  const int qc = q < T ? q : T - 1;

  // q * c in bf16: scores come out of the MFMA in log2 units
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 raw = *reinterpret_cast<const bf16x8 *>(qkv + (int64_t)qc * ldq + head * DH + kk * 16 + hf * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)((float)raw[e] * scale_log2);
  }

  const uint32_t rec = (uint32_t)((int64_t)T * ldq * 2);
  const i32x4 k_rsrc = dl_rsrc(qkv + HD + head * DH, rec);
  const i32x4 v_rsrc = dl_rsrc(vt + (int64_t)head * DH * ldvt, (uint32_t)(DH * ldvt * 2));
  int k_voff[LD_PER_WAVE], v_voff[VLD_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LD_PER_WAVE; ++i) {
    const int row = (wv * LD_PER_WAVE + i) * ROWS_PER_LD + lane / KCH;
    const int p = lane % KCH;
    k_voff[i] = (row * (int)ldq + (p ^ k_swz<DH>(row)) * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < VLD_PER_WAVE; ++i) {
    const int f = (wv * VLD_PER_WAVE + i) * 8 + lane / 8;
    v_voff[i] = (f * (int)ldvt + ((lane % 8) ^ vt_swz(f)) * 8) * 2;
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
    const int off = j * AK * 2;
#pragma unroll
    for (int i = 0; i < VLD_PER_WAVE; ++i)
      dl_load(v_rsrc, __builtin_amdgcn_readfirstlane(sb + (uint32_t)((wv * VLD_PER_WAVE + i) * 1024)),
              v_voff[i] + off);
  };

  // Key order: MFMA row i of a 32-key half reads key row i with bits 2 and 3
  // swapped.  Accumulator r of lane (ql, hf) then holds key 16 (r / 8) + 8 hf +
  // r % 8, so the eight bf16 P values a lane packs per 16-key chunk are eight
  // consecutive keys: the layout of one 16-B read of a V^T row.
  const int kr = (ql & ~12) | ((ql & 4) << 1) | ((ql & 8) >> 1);
  int k_lane[KK], v_lane[4];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    k_lane[kk] = (kr * DH + (((kk * 2 + hf) ^ k_swz<DH>(kr)) << 3)) * 2;
  // V^T operand of key chunk c (16 keys): feature row ql (+ 32 t), keys
  // 16 c + 8 hf .. + 7; the 32 t rows add 4096 B
#pragma unroll
  for (int c = 0; c < 4; ++c) v_lane[c] = ql * AK * 2 + (((2 * c + hf) ^ vt_swz(ql)) << 4);
  const char *lds_bytes = reinterpret_cast<const char *>(&smem[0]);

  // S^T - s0 of one block: two 32-key halves, their MFMA chains interleaved
  auto qk = [&](const char *Kb, f32x16 (&s)[2], float s0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = s0;
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
  float m_run = 0.f, l_run = 0.f;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // p = exp2(score - m) of the 16 scores of one 32-key half held by this lane
  // (the registers hold score - m), as bf16
  auto half_p = [&](const f32x16 &sv, bf16x8 &p0, bf16x8 &p1) {
#pragma unroll
    for (int r = 0; r < 8; ++r) p0[r] = (__bf16)__builtin_amdgcn_exp2f(sv[r]);
#pragma unroll
    for (int r = 0; r < 8; ++r) p1[r] = (__bf16)__builtin_amdgcn_exp2f(sv[8 + r]);
  };
  // their sum, from the bf16 values the MFMA multiplies
  auto half_sum = [&](const bf16x8 &p0, const bf16x8 &p1) {
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[2 * e], p0[2 * e + 1]}, ones, ls, false);
#pragma unroll
    for (int e = 0; e < 4; ++e) ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[2 * e], p1[2 * e + 1]}, ones, ls, false);
    return ls;
  };
  // max over both lane halves of one half's 16 values per lane
  auto half_max = [&](const f32x16 &sv) {
    float mx = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sv[r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };
  // Taken when some lane's p sum of the half is not below 2^64 (a score more
  // than 64 above m, in log2 units): raise m to the half's max, rescale O and
  // l, shift every score register still to be used (this half, then `more`)
  // by the same amount, redo the half's P.
  auto raise = [&](f32x16 &sv, bf16x8 &p0, bf16x8 &p1, float &ls, auto &&more) {
    const float delta = fmaxf(half_max(sv), 0.f);
    m_run += delta;
    const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
    l_run *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] -= delta;
    more(delta);
    half_p(sv, p0, p1);
    ls = half_sum(p0, p1);
  };

  const int nkb = (T + AK - 1) / AK;
  issue_k(0, 0);
  issue_v(0, 2);
  if (nkb > 1) issue_k(1, 1);
  vmcnt_barrier<0>();
  f32x16 sa[2], sb[2];
  qk(lds_bytes, sa, 0.f);
  // m starts at block 0's max (over existing keys), the scores relative to it
  if (T < AK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + (r >> 3) * 16 + hf * 8 + (r & 7) >= T) sa[kb][r] = -INFINITY;
  }
  m_run = fmaxf(half_max(sa[0]), half_max(sa[1]));
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[kb][r] -= m_run;

  // Scheduling of the 2 DT PV MFMAs of two 16-key chunks: their V^T operand
  // reads three ahead, NV VALU instructions after each MFMA.
  auto pv_schedule = [&](auto nv_c) {
    constexpr int NV = decltype(nv_c)::value;
    constexpr int RV = 3;
    __builtin_amdgcn_sched_group_barrier(0x100, RV, 0);  // LDS read
#pragma unroll
    for (int i = 0; i < 2 * DT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i < 2 * DT - RV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if constexpr (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
    }
  };

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
          if (kbase + kb * 32 + (r >> 3) * 16 + hf * 8 + (r & 7) >= T) sc[kb][r] = -INFINITY;
    }
    // P of the first 32-key half against the running max, and its row sums
    bf16x8 pf[4];
    half_p(sc[0], pf[0], pf[1]);
    float ls0 = half_sum(pf[0], pf[1]);

    qk(Kn, sn, -m_run);  // next block's scores - m (unused after the last block)
    // interleave the 16 MFMAs with the K operand reads (two ahead) and the
    // softmax VALU work
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i < 14) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    }
    asm volatile("" ::"v"(pf[0]), "v"(pf[1]));
    if (__any(!(ls0 < P_LIMIT)))
      raise(sc[0], pf[0], pf[1], ls0, [&](float delta) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[1][r] -= delta;
          sn[0][r] -= delta;
          sn[1][r] -= delta;
        }
      });
    l_run += ls0;

    // O^T += V^T P^T over the four 16-key chunks; the second half's P and row
    // sums on the VALU under the first two chunks' MFMAs
    half_p(sc[1], pf[2], pf[3]);
    float ls1 = half_sum(pf[2], pf[3]);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(Vb + t * 32 * AK * 2 + v_lane[c]);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], o[t], 0, 0, 0);
      }
    // V^T reads three MFMAs ahead, four VALU instructions of the second half's
    // P under each MFMA (left to itself the compiler issues each read just
    // before its MFMA and waits on it: 1.5-1.9 % slower on the Super shape)
    pv_schedule(std::integral_constant<int, 4>{});
    if (__any(!(ls1 < P_LIMIT)))
      raise(sc[1], pf[2], pf[3], ls1, [&](float delta) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sn[0][r] -= delta;
          sn[1][r] -= delta;
        }
      });
    l_run += ls1;
#pragma unroll
    for (int c = 2; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(Vb + t * 32 * AK * 2 + v_lane[c]);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], o[t], 0, 0, 0);
      }
    pv_schedule(std::integral_constant<int, 0>{});
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

// V^T for the attention: vt[f, t] = v[t, f] for t < T, 0 for T <= t < T64
// (T64 = T rounded up to 64, so every 64-key block of V^T holds finite values).
// One workgroup per 64 tokens x 64 features: 16-B row loads into an LDS tile
// whose 132-B rows put the eight 2-B reads of a 16-B output segment on eight
// distinct banks, then 16-B stores along the feature rows.
__global__ __launch_bounds__(256) void v_transpose_kernel(const uint16_t *__restrict__ v, int64_t ldv,
                                                          int T, uint16_t *__restrict__ vt,
                                                          int64_t ldvt) {
  constexpr int LDT = 66;  // u16 per LDS row (132 B)
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * LDT];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64, f0 = blockIdx.y * 64;
#pragma unroll
  for (int L = 0; L < 2; ++L) {
    const int idx = L * 256 + tid, r = idx >> 3, c = idx & 7;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (t0 + r < T) val = *reinterpret_cast<const u32x4 *>(v + (int64_t)(t0 + r) * ldv + f0 + c * 8);
    uint32_t *dst = reinterpret_cast<uint32_t *>(tile + r * LDT + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = val[e];
  }
  __syncthreads();
#pragma unroll
  for (int L = 0; L < 2; ++L) {
    const int idx = L * 256 + tid, f = idx >> 3, c = idx & 7;
    u32x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      val[e] = (uint32_t)tile[(c * 8 + 2 * e) * LDT + f] | ((uint32_t)tile[(c * 8 + 2 * e + 1) * LDT + f] << 16);
    *reinterpret_cast<u32x4 *>(vt + (int64_t)(f0 + f) * ldvt + t0 + c * 8) = val;
  }
}

}  // namespace

hipError_t launch_v_transpose(const uint16_t *v, int64_t ldv, int T, int d, uint16_t *vt,
                              int64_t ldvt, hipStream_t s) {
  if (T < 1 || d % 64 || ldv % 8 || ldvt % 8 || ldvt < (int64_t)(T + 63) / 64 * 64)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(v_transpose_kernel, dim3((T + 63) / 64, d / 64), dim3(256), 0, s, v, ldv, T, vt,
                     ldvt);
  return hipGetLastError();
}

hipError_t launch_attention(const uint16_t *qkv, int64_t ldqkv, const uint16_t *vt, int64_t ldvt,
                            int T, int H, int dh, uint16_t *out, int64_t ldo, hipStream_t s) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)dh);
  // 8 waves (256 queries) per workgroup, one workgroup per CU: faster than
  // 4 waves at two workgroups per CU (each K/V tile then serves twice the
  // queries; 3.6 % on the Super attention shape)
  const int nqb = (T + 255) / 256;
  if (dh == 128) {
    hipLaunchKernelGGL((attention_kernel<128, 8>), dim3(nqb * H), dim3(512), 0, s, qkv, ldqkv, vt,
                       ldvt, T, H, out, ldo, scale_log2);
  } else if (dh == 64) {
    hipLaunchKernelGGL((attention_kernel<64, 8>), dim3(nqb * H), dim3(512), 0, s, qkv, ldqkv, vt,
                       ldvt, T, H, out, ldo, scale_log2);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dlo
