// libdlo host side: plan, host store, two-slot schedule, executor, C ABI.
//
// Pages cited (by title):
//   [Jul] "Distributed Layerwise Offload", vLLM-Omni project blog, 2026-07-30.
//   [Aug] "Distributed Layerwise Offload: Scaling Toward 200B+ DiT Models
//         Efficiently in vLLM-Omni", vLLM blog, 2026-08-17.
//   [Doc] "Distributed Layerwise Offload", vLLM-Omni design documentation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/dlo.h"
#include "kernels.h"

static_assert(DLO_NOALLOC_MAX_D == dlo::NOALLOC_MAX_D, "the header's scratch limit is the kernel's");
static_assert(DLO_MFMA_RATE_THREADS == dlo::MFMA_RATE_GRID * 512, "the header's probe size is the kernel's");

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return DLO_OK;
}

int64_t elt_bytes(int dtype) { return dtype == DLO_BF16 ? 2 : dtype == DLO_F32 ? 4 : 1; }
bool known_dtype(int dtype) {
  return dtype == DLO_BF16 || dtype == DLO_F32 || dtype == DLO_FP8_E4M3 || dtype == DLO_I8 || dtype == DLO_E8M0;
}
int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

float widen_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// rows [0, rows) split over up to 16 threads (each row's result is independent)
template <typename Fn>
void for_rows(int64_t rows, int64_t cols, Fn &&fn) {
  const int nt = (int)std::min<int64_t>(16, std::max<int64_t>(1, (rows * cols) >> 20));
  const int64_t chunk = (rows + nt - 1) / nt;
  std::vector<std::thread> th;
  for (int t = 1; t < nt; ++t)
    th.emplace_back([&, t] {
      for (int64_t r = t * chunk; r < std::min(rows, (t + 1) * chunk); ++r) fn(r);
    });
  for (int64_t r = 0; r < std::min(rows, chunk); ++r) fn(r);
  for (auto &x : th) x.join();
}

// OCP FP8 E4M3 code nearest to x: ties to the even code, magnitudes of 448 and
// above saturate to 448, NaN -> 0x7F.  Arithmetic on the exponent and the
// 3-bit mantissa: every scaling by a power of two is exact, and nearbyintf
// rounds ties to even in the default rounding mode.
uint8_t e4m3_encode(float x) {
  uint32_t bits;
  std::memcpy(&bits, &x, 4);
  const uint8_t sign = (uint8_t)((bits >> 24) & 0x80);
  if (std::isnan(x)) return 0x7F;
  const float a = std::fabs(x);
  if (a >= 448.0f) return sign | 0x7E;
  if (a < 0.015625f)  // below 2^-6: subnormal steps of 2^-9; 8 steps is the smallest normal
    return sign | (uint8_t)std::nearbyintf(a * 512.0f);
  int e2;
  (void)std::frexp(a, &e2);  // a = f * 2^e2, f in [0.5, 1)
  int E = e2 - 1;            // a in [2^E, 2^(E+1)), E in [-6, 8]
  int m = (int)std::nearbyintf(std::ldexp(a, -E) * 8.0f) - 8;
  if (m == 8) {
    m = 0;
    ++E;
  }
  return sign | (uint8_t)(((E + 7) << 3) | m);
}

// ---------------------------------------------------------------------------
// DiT block schema (registration order)
// ---------------------------------------------------------------------------

struct SchemaEntry {
  const char *name;
  int dtype;
  int64_t rows_per_d;  // numel = rows_per_d * d * cols_per_d * d / div, or fixed
  int64_t cols_per_d;
  int64_t fixed;       // > 0: numel is this constant
  int64_t div = 1;     // MX block scales: one per 32 elements
};

// numel(d) = fixed if fixed > 0, else rows_per_d * d * (cols_per_d ? cols_per_d * d : 1) / div
const SchemaEntry kDit[DLO_DIT_N_PARAMS] = {
    {"adaln.weight", DLO_BF16, 6, 1, 0},    {"adaln.bias", DLO_F32, 6, 0, 0},
    {"norm1.weight", DLO_F32, 1, 0, 0},     {"norm1.bias", DLO_F32, 1, 0, 0},
    {"norm1.eps", DLO_F32, 0, 0, 1},        {"attn.qkv.weight", DLO_BF16, 3, 1, 0},
    {"attn.qkv.bias", DLO_F32, 3, 0, 0},    {"attn.out.weight", DLO_BF16, 1, 1, 0},
    {"attn.out.bias", DLO_F32, 1, 0, 0},    {"norm2.weight", DLO_F32, 1, 0, 0},
    {"norm2.bias", DLO_F32, 1, 0, 0},       {"norm2.eps", DLO_F32, 0, 0, 1},
    {"mlp.fc1.weight", DLO_BF16, 4, 1, 0},  {"mlp.fc1.bias", DLO_F32, 4, 0, 0},
    {"mlp.fc2.weight", DLO_BF16, 1, 4, 0},  {"mlp.fc2.bias", DLO_F32, 1, 0, 0},
};
// FP8 form ([Doc] "Request and loading constraints": per-tensor online FP8
// linears keep a 1-byte weight and an fp32 scale): each bf16 matrix becomes an
// E4M3 matrix followed by its one-element scale.
const SchemaEntry kDitFp8[DLO_DIT_FP8_N_PARAMS] = {
    {"adaln.weight", DLO_FP8_E4M3, 6, 1, 0},    {"adaln.weight_scale", DLO_F32, 0, 0, 1},
    {"adaln.bias", DLO_F32, 6, 0, 0},           {"norm1.weight", DLO_F32, 1, 0, 0},
    {"norm1.bias", DLO_F32, 1, 0, 0},           {"norm1.eps", DLO_F32, 0, 0, 1},
    {"attn.qkv.weight", DLO_FP8_E4M3, 3, 1, 0}, {"attn.qkv.weight_scale", DLO_F32, 0, 0, 1},
    {"attn.qkv.bias", DLO_F32, 3, 0, 0},        {"attn.out.weight", DLO_FP8_E4M3, 1, 1, 0},
    {"attn.out.weight_scale", DLO_F32, 0, 0, 1}, {"attn.out.bias", DLO_F32, 1, 0, 0},
    {"norm2.weight", DLO_F32, 1, 0, 0},         {"norm2.bias", DLO_F32, 1, 0, 0},
    {"norm2.eps", DLO_F32, 0, 0, 1},            {"mlp.fc1.weight", DLO_FP8_E4M3, 4, 1, 0},
    {"mlp.fc1.weight_scale", DLO_F32, 0, 0, 1}, {"mlp.fc1.bias", DLO_F32, 4, 0, 0},
    {"mlp.fc2.weight", DLO_FP8_E4M3, 1, 4, 0},  {"mlp.fc2.weight_scale", DLO_F32, 0, 0, 1},
    {"mlp.fc2.bias", DLO_F32, 1, 0, 0},
};
// INT8 form ([Doc] "Request and loading constraints": online INT8 keeps an int8
// weight and an fp32 scale): each bf16 matrix becomes int8 codes followed by
// one fp32 scale per output row.
const SchemaEntry kDitInt8[DLO_DIT_FP8_N_PARAMS] = {
    {"adaln.weight", DLO_I8, 6, 1, 0},          {"adaln.weight_scale", DLO_F32, 6, 0, 0},
    {"adaln.bias", DLO_F32, 6, 0, 0},           {"norm1.weight", DLO_F32, 1, 0, 0},
    {"norm1.bias", DLO_F32, 1, 0, 0},           {"norm1.eps", DLO_F32, 0, 0, 1},
    {"attn.qkv.weight", DLO_I8, 3, 1, 0},       {"attn.qkv.weight_scale", DLO_F32, 3, 0, 0},
    {"attn.qkv.bias", DLO_F32, 3, 0, 0},        {"attn.out.weight", DLO_I8, 1, 1, 0},
    {"attn.out.weight_scale", DLO_F32, 1, 0, 0}, {"attn.out.bias", DLO_F32, 1, 0, 0},
    {"norm2.weight", DLO_F32, 1, 0, 0},         {"norm2.bias", DLO_F32, 1, 0, 0},
    {"norm2.eps", DLO_F32, 0, 0, 1},            {"mlp.fc1.weight", DLO_I8, 4, 1, 0},
    {"mlp.fc1.weight_scale", DLO_F32, 4, 0, 0}, {"mlp.fc1.bias", DLO_F32, 4, 0, 0},
    {"mlp.fc2.weight", DLO_I8, 1, 4, 0},        {"mlp.fc2.weight_scale", DLO_F32, 1, 0, 0},
    {"mlp.fc2.bias", DLO_F32, 1, 0, 0},
};
// MXFP8 form (same passage: an fp8 weight and an e8m0 block scale): each bf16
// matrix becomes E4M3 codes followed by one E8M0 scale per 32 elements of a row.
const SchemaEntry kDitMx[DLO_DIT_FP8_N_PARAMS] = {
    {"adaln.weight", DLO_FP8_E4M3, 6, 1, 0},          {"adaln.weight_scale", DLO_E8M0, 6, 1, 0, 32},
    {"adaln.bias", DLO_F32, 6, 0, 0},                 {"norm1.weight", DLO_F32, 1, 0, 0},
    {"norm1.bias", DLO_F32, 1, 0, 0},                 {"norm1.eps", DLO_F32, 0, 0, 1},
    {"attn.qkv.weight", DLO_FP8_E4M3, 3, 1, 0},       {"attn.qkv.weight_scale", DLO_E8M0, 3, 1, 0, 32},
    {"attn.qkv.bias", DLO_F32, 3, 0, 0},              {"attn.out.weight", DLO_FP8_E4M3, 1, 1, 0},
    {"attn.out.weight_scale", DLO_E8M0, 1, 1, 0, 32}, {"attn.out.bias", DLO_F32, 1, 0, 0},
    {"norm2.weight", DLO_F32, 1, 0, 0},               {"norm2.bias", DLO_F32, 1, 0, 0},
    {"norm2.eps", DLO_F32, 0, 0, 1},                  {"mlp.fc1.weight", DLO_FP8_E4M3, 4, 1, 0},
    {"mlp.fc1.weight_scale", DLO_E8M0, 4, 1, 0, 32},  {"mlp.fc1.bias", DLO_F32, 4, 0, 0},
    {"mlp.fc2.weight", DLO_FP8_E4M3, 1, 4, 0},        {"mlp.fc2.weight_scale", DLO_E8M0, 1, 4, 0, 32},
    {"mlp.fc2.bias", DLO_F32, 1, 0, 0},
};
// logical parameters of the block forward (indices into kDit)
enum {
  P_ADA_W, P_ADA_B, P_N1_W, P_N1_B, P_N1_EPS, P_QKV_W, P_QKV_B, P_OUT_W, P_OUT_B, P_N2_W, P_N2_B,
  P_N2_EPS, P_FC1_W, P_FC1_B, P_FC2_W, P_FC2_B
};
// where each logical parameter sits in the FP8, INT8 and MXFP8 schemas
const int kFp8Index[DLO_DIT_N_PARAMS] = {0, 2, 3, 4, 5, 6, 8, 9, 11, 12, 13, 14, 15, 17, 18, 20};
// the five weights (ada, qkv, out, fc1, fc2): logical index, scale index in the
// quantised schemas, and rows / d, columns / d
const int kWeightP[5] = {P_ADA_W, P_QKV_W, P_OUT_W, P_FC1_W, P_FC2_W};
const int kFp8Scale[5] = {1, 7, 10, 16, 19};
const int64_t kWeightRows[5] = {6, 3, 1, 4, 1};
const int64_t kWeightCols[5] = {1, 1, 1, 1, 4};
const int64_t kWeightD2[5] = {6, 3, 1, 4, 4};
enum { KIND_NONE = 0, KIND_DIT = 1, KIND_DIT_FP8 = 2, KIND_DIT_INT8 = 3, KIND_DIT_MX = 4 };

int64_t schema_numel(const SchemaEntry &e, int64_t d) {
  if (e.fixed > 0) return e.fixed;
  return e.rows_per_d * d * (e.cols_per_d ? e.cols_per_d * d : 1) / e.div;
}

const char *kKernelNames[DLO_KERNELS_PER_BLOCK] = {
    "dequant_weights", "adaln_gemv", "ln1_modulate", "quant_h", "gemm_qk", "gemm_v_t", "attention",
    "quant_attn", "gemm_out_residual", "ln2_modulate", "quant_h2", "gemm_fc1_gelu", "quant_u",
    "gemm_fc2_residual"};

}  // namespace

// ---------------------------------------------------------------------------
// objects
// ---------------------------------------------------------------------------

struct BlockPlan {
  int32_t d = 0, heads = 0;
  std::vector<std::string> names;
  std::vector<int32_t> dtypes;
  std::vector<int64_t> numels;
  std::vector<int32_t> pgroup;   // param -> group
  std::vector<int64_t> poff;     // param -> element offset in its group
  int32_t n_groups = 0;
  int32_t gdtype[DLO_MAX_GROUPS] = {0, 0};
  int64_t gnumel[DLO_MAX_GROUPS] = {0, 0};
  int64_t gshard[DLO_MAX_GROUPS] = {0, 0};
  int64_t gregion[DLO_MAX_GROUPS] = {0, 0};
  int64_t extent = 0, copy_bytes = 0;
  int kind = KIND_NONE;            // KIND_DIT: bf16 weights; else a quantised form

  int64_t param_byte(int p) const {
    const int g = pgroup[p];
    return gregion[g] + poff[p] * elt_bytes(gdtype[g]);
  }
  // slot byte offset of a logical parameter (P_*) of either schema
  int64_t logical_byte(int lp) const { return param_byte(kind >= KIND_DIT_FP8 ? kFp8Index[lp] : lp); }
};

struct dlo_run;

struct dlo_plan {
  int32_t k = 1;
  std::vector<BlockPlan> blocks;
  int64_t slot_bytes = 0;
  int32_t max_d = 0;
  int32_t max_fp8_d = 0;   // widest per-tensor FP8 block (0: none)
  int32_t max_q_d = 0;     // widest INT8 or MXFP8 block (0: none)
  int32_t max_mx_d = 0;    // widest MXFP8 block (0: none)
  int32_t max_i8_d = 0;    // widest INT8 block (0: none)
  uint64_t id = 0;
  mutable std::mutex mu;
  mutable std::vector<dlo_run *> detached;   // runs started without a handle
  mutable hipEvent_t last_done = nullptr;    // end of the previous run (any stream)
  mutable dlo_run *enqueuing = nullptr;      // DLO_ASYNC_ENQUEUE run still being enqueued
};

struct dlo_host_store {
  const dlo_plan *plan = nullptr;
  uint64_t plan_id = 0;
  std::vector<char *> mem;                     // per block
  std::vector<uint8_t> pinned;                 // per block: shards in pinned memory
  std::vector<std::vector<int64_t>> shard_at;  // per block: byte offset of (g * k + r)
  std::vector<uint8_t> packed;                 // per block flag
  // two bounded pinned staging buffers (one slot each) for pageable blocks
  char *staging[2] = {nullptr, nullptr};
  std::mutex mu;                        // guards enqueuing
  dlo_run *enqueuing = nullptr;         // DLO_ASYNC_ENQUEUE run still being enqueued
  hipEvent_t last_copy = nullptr;       // recorded after every placement from the store
  hipEvent_t staging_free[2] = {nullptr, nullptr};    // DMA out of buffer j done
  int64_t staging_bytes = 0;
  int64_t staged_uses = 0;
  const void *shard(int b, int g, int r) const {
    return mem[b] + shard_at[b][g * plan->k + r];
  }
};

struct dlo_run {
  int device = 0;
  hipEvent_t ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  hipEvent_t final_ev = nullptr;
  bool timing = false, digest = false;
  std::vector<dlo_slot_event> recs;
  // timing events, per step: copy begin, copy end, compute begin, kernel ends
  // [DLO_KERNELS_PER_BLOCK], compute end; kmask[t] bit j: kernel slot j of step
  // t launched work and recorded its end event (an empty slot records none)
  std::vector<hipEvent_t> tev;
  std::vector<uint32_t> kmask;
  uint64_t *d_digest = nullptr;
  bool finished = false;
  std::vector<float> kernel_ms;
  // DLO_ASYNC_ENQUEUE: the thread enqueuing the program, its status and message,
  // and its own copy of the caller's arguments
  const dlo_plan *plan = nullptr;
  dlo_host_store *store = nullptr;
  std::thread worker;
  int enqueue_rc = 0;
  std::string enqueue_msg;
  dlo_forward_args args{};
  std::vector<const void *> res_blocks;
};

// Joins a DLO_ASYNC_ENQUEUE run's enqueue thread (no-op otherwise) and lets the
// plan start runs again.
void finish_enqueue(dlo_run *r) {
  if (!r) return;
  if (r->worker.joinable()) r->worker.join();
  if (r->plan) {
    std::lock_guard<std::mutex> lk(r->plan->mu);
    if (r->plan->enqueuing == r) r->plan->enqueuing = nullptr;
    r->plan = nullptr;
  }
  if (r->store) {
    std::lock_guard<std::mutex> lk(r->store->mu);
    if (r->store->enqueuing == r) r->store->enqueuing = nullptr;
    r->store = nullptr;
  }
}

namespace {

std::atomic<uint64_t> g_plan_ids{1};

int check_hip(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(DLO_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return DLO_OK;
}

void run_free(dlo_run *r) {
  if (!r) return;
  finish_enqueue(r);
  if (r->final_ev) (void)hipEventSynchronize(r->final_ev);
  for (auto &e : r->ev)
    if (e) (void)hipEventDestroy(e);
  if (r->final_ev) (void)hipEventDestroy(r->final_ev);
  for (auto e : r->tev)
    if (e) (void)hipEventDestroy(e);
  if (r->d_digest) (void)hipFree(r->d_digest);
  delete r;
}

void reap_detached(const dlo_plan *p, bool wait) {
  std::vector<dlo_run *> keep;
  for (dlo_run *r : p->detached) {
    if (wait || hipEventQuery(r->final_ev) == hipSuccess)
      run_free(r);
    else
      keep.push_back(r);
  }
  p->detached.swap(keep);
}

// ---------------------------------------------------------------------------
// the schedule: hook rule -> program of stream operations
// ---------------------------------------------------------------------------

struct Step {
  int64_t t;
  int32_t pass, block, slot, next_block, next_slot;  // slot -1: a resident block
  int64_t next_step;                                  // step that reads the prefetch, -1 if none
};

// [Jul] "Slot Tracking: i%2 + Dynamic Correction": the hooks form a ring; a step
// reads the slot its ring predecessor last prefetched into, or its own parity
// h % 2 while the predecessor has prefetched nothing, and prefetches the next
// block of the ring into the other slot.  With n_res resident blocks ([Doc]
// "Validation coverage": resident-layer requests), blocks 0 .. n_res-1 read no
// slot and the ring holds only the streamed blocks.
std::vector<Step> hook_steps(int n, int passes, int n_res) {
  const int m = n - n_res;
  std::vector<int> pref((size_t)std::max(m, 1), -1);   // hook -> slot of its latest prefetch
  const int64_t total = (int64_t)n * passes, streamed_total = (int64_t)m * passes;
  std::vector<Step> out;
  out.reserve((size_t)total);
  int64_t u = 0;
  for (int64_t t = 0; t < total; ++t) {
    const int i = (int)(t % n), p = (int)(t / n);
    Step s{t, p, i, -1, -1, -1, -1};
    if (i >= n_res) {
      const int h = i - n_res, prev = (h + m - 1) % m;
      s.slot = pref[prev] >= 0 ? pref[prev] : h % 2;
      if (u + 1 < streamed_total) {
        s.next_block = n_res + (h + 1) % m;
        s.next_slot = 1 - s.slot;
        pref[h] = s.next_slot;
      }
      ++u;
    }
    out.push_back(s);
  }
  // the step that reads each prefetch: the next streamed step
  int64_t next_streamed = -1;
  for (int64_t t = total - 1; t >= 0; --t) {
    Step &s = out[(size_t)t];
    if (s.next_block >= 0) s.next_step = next_streamed;
    if (s.slot >= 0) next_streamed = t;
  }
  return out;
}

std::vector<dlo_sched_op> build_program(const std::vector<Step> &steps, bool all_resident) {
  std::vector<dlo_sched_op> prog;
  auto op = [&](int kind, int stream, int block, int slot, int event, int64_t step) {
    dlo_sched_op o;
    o.kind = kind; o.stream = stream; o.block = block; o.slot = slot; o.event = event;
    o.pad = 0; o.step = step;
    prog.push_back(o);
  };
  const Step *first = nullptr;
  for (const Step &s : steps)
    if (s.slot >= 0) {
      first = &s;
      break;
    }
  if (all_resident || !first) {
    for (const Step &s : steps) op(DLO_OP_COMPUTE, DLO_STREAM_COMPUTE, s.block, -1, -1, s.t);
    return prog;
  }
  op(DLO_OP_RECORD, DLO_STREAM_COMPUTE, -1, -1, DLO_EV_START, -1);
  op(DLO_OP_WAIT, DLO_STREAM_COPY, -1, -1, DLO_EV_START, -1);
  // initial prefetch: the first streamed block into slot 0 ([Doc] "Pre-service
  // transaction boundary")
  op(DLO_OP_COPY, DLO_STREAM_COPY, first->block, first->slot, -1, first->t);
  op(DLO_OP_RECORD, DLO_STREAM_COPY, -1, -1, DLO_EV_COPIED0 + first->slot, -1);
  bool first_streamed = true;
  for (const Step &s : steps) {
    if (s.slot < 0) {  // resident block: reads no slot, nothing to wait for
      op(DLO_OP_COMPUTE, DLO_STREAM_COMPUTE, s.block, -1, -1, s.t);
      continue;
    }
    // step t's block, from its slot, once the copy that placed it is done
    op(DLO_OP_WAIT, DLO_STREAM_COMPUTE, -1, -1, DLO_EV_COPIED0 + s.slot, -1);
    op(DLO_OP_COMPUTE, DLO_STREAM_COMPUTE, s.block, s.slot, -1, s.t);
    op(DLO_OP_RECORD, DLO_STREAM_COMPUTE, -1, -1, DLO_EV_COMPUTED0 + s.slot, -1);
    // prefetch the next streamed block into the other slot, whose last reader
    // was the previous streamed step.  Enqueued after this step's compute so
    // that a host-staged copy never delays it.
    if (s.next_block >= 0) {
      if (!first_streamed) op(DLO_OP_WAIT, DLO_STREAM_COPY, -1, -1, DLO_EV_COMPUTED0 + s.next_slot, -1);
      op(DLO_OP_COPY, DLO_STREAM_COPY, s.next_block, s.next_slot, -1, s.next_step);
      op(DLO_OP_RECORD, DLO_STREAM_COPY, -1, -1, DLO_EV_COPIED0 + s.next_slot, -1);
    }
    first_streamed = false;
  }
  return prog;
}

// ---------------------------------------------------------------------------
// host copies for packing: split into chunks over a few threads
// ---------------------------------------------------------------------------

struct CopyTask {
  char *dst;
  const char *src;   // nullptr: zero-fill
  int64_t bytes;
};

void run_copies(std::vector<CopyTask> &tasks) {
  constexpr int64_t CHUNK = 16 << 20;
  std::vector<CopyTask> pieces;
  int64_t total = 0;
  for (const CopyTask &t : tasks) {
    for (int64_t o = 0; o < t.bytes; o += CHUNK) {
      const int64_t n = std::min(CHUNK, t.bytes - o);
      pieces.push_back({t.dst + o, t.src ? t.src + o : nullptr, n});
    }
    total += t.bytes;
  }
  unsigned hw = std::thread::hardware_concurrency();
  int nth = (int)std::min<int64_t>(std::max(1u, std::min(hw, 16u)), (int64_t)pieces.size());
  if (total < (64 << 20)) nth = 1;
  std::atomic<size_t> next{0};
  auto worker = [&]() {
    for (size_t i = next++; i < pieces.size(); i = next++) {
      const CopyTask &p = pieces[i];
      if (p.src)
        std::memcpy(p.dst, p.src, (size_t)p.bytes);
      else
        std::memset(p.dst, 0, (size_t)p.bytes);
    }
  };
  if (nth <= 1) {
    worker();
    return;
  }
  std::vector<std::thread> th;
  for (int i = 0; i < nth; ++i) th.emplace_back(worker);
  for (auto &t : th) t.join();
}

int64_t round_up64(int64_t T) { return (T + 63) / 64 * 64; }

// bytes of the dequantised-weight region: a per-tensor FP8 block's four linear
// weights (12 f^2 bf16), an INT8 or MXFP8 block's five (18 q^2 bf16)
int64_t dequant_bytes(int64_t f, int64_t q) { return std::max(24 * f * f, 36 * q * q); }

// bytes of a W8A8 linear input's scales: fp32 per row (FP8 and INT8, widest
// such block f), or E8M0 per 32 elements block-major [4 mx / 32, T64] (MXFP8)
int64_t act_scale_bytes(int64_t T, int64_t f, int64_t mx) {
  return std::max(f > 0 ? 4 * T : 0, mx * round_up64(T) / 8);
}

int64_t workspace_bytes_for(int32_t max_d, int64_t T, int32_t fp8_d, int32_t q_d, int32_t mx_d, int32_t i8_d) {
  const int64_t d = max_d, f = std::max(fp8_d, i8_d), mx = mx_d;
  // quantised blocks: their dequantised weights; all of them also the 1-byte
  // codes [T, 4d] and the scales of a linear's input in the W8A8 form
  const int64_t dq = align_up(dequant_bytes(fp8_d, q_d), DLO_ALIGN);
  const int64_t w8a8 = (f > 0 || mx > 0) ? align_up(4 * T * std::max(f, mx), DLO_ALIGN) +
                                             align_up(act_scale_bytes(T, f, mx), DLO_ALIGN)
                                       : 0;
  return align_up(4 * d, DLO_ALIGN) + align_up(24 * d, DLO_ALIGN) + align_up(2 * T * d, DLO_ALIGN) +
         align_up(8 * round_up64(T) * d, DLO_ALIGN) + dq + w8a8;
}

int validate_block_against(const BlockPlan &bp, const dlo_block &blk, int b, bool need_src) {
  if (blk.n_params != (int32_t)bp.names.size())
    return fail(DLO_E_PLAN_MISMATCH, "block %d: %d parameters, plan has %zu", b, blk.n_params,
                bp.names.size());
  if (blk.n_params > 0 && !blk.params) return fail(DLO_E_ARG, "block %d: params is NULL", b);
  for (int p = 0; p < blk.n_params; ++p) {
    const dlo_param &pr = blk.params[p];
    if (!pr.name || bp.names[p] != pr.name || pr.dtype != bp.dtypes[p] || pr.numel != bp.numels[p])
      return fail(DLO_E_PLAN_MISMATCH, "block %d parameter %d (%s) does not match the plan", b, p,
                  pr.name ? pr.name : "(null)");
    if (need_src && pr.numel > 0 && !pr.src)
      return fail(DLO_E_ARG, "block %d parameter %d (%s) has no source", b, p, pr.name);
  }
  return DLO_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================

extern "C" {

const char *dlo_last_error(void) { return g_err.c_str(); }

int dlo_block_schema(int32_t d, int32_t i, const char **name, int32_t *dtype, int64_t *numel) {
  if (i < 0 || i >= DLO_DIT_N_PARAMS || d < 1) return fail(DLO_E_ARG, "schema index out of range");
  if (name) *name = kDit[i].name;
  if (dtype) *dtype = kDit[i].dtype;
  if (numel) *numel = schema_numel(kDit[i], d);
  return ok();
}

int dlo_block_schema_fp8(int32_t d, int32_t i, const char **name, int32_t *dtype, int64_t *numel) {
  if (i < 0 || i >= DLO_DIT_FP8_N_PARAMS || d < 1) return fail(DLO_E_ARG, "schema index out of range");
  if (name) *name = kDitFp8[i].name;
  if (dtype) *dtype = kDitFp8[i].dtype;
  if (numel) *numel = schema_numel(kDitFp8[i], d);
  return ok();
}

int dlo_block_schema_int8(int32_t d, int32_t i, const char **name, int32_t *dtype, int64_t *numel) {
  if (i < 0 || i >= DLO_DIT_FP8_N_PARAMS || d < 1) return fail(DLO_E_ARG, "schema index out of range");
  if (name) *name = kDitInt8[i].name;
  if (dtype) *dtype = kDitInt8[i].dtype;
  if (numel) *numel = schema_numel(kDitInt8[i], d);
  return ok();
}

int dlo_block_schema_mxfp8(int32_t d, int32_t i, const char **name, int32_t *dtype, int64_t *numel) {
  if (i < 0 || i >= DLO_DIT_FP8_N_PARAMS || d < 1) return fail(DLO_E_ARG, "schema index out of range");
  if (d % 32) return fail(DLO_E_ARG, "MXFP8 blocks need d %% 32 == 0 (32-element scale blocks)");
  if (name) *name = kDitMx[i].name;
  if (dtype) *dtype = kDitMx[i].dtype;
  if (numel) *numel = schema_numel(kDitMx[i], d);
  return ok();
}

int dlo_quantize_int8(const uint16_t *w, int64_t rows, int64_t cols, int8_t *codes, float *scales) {
  if (rows < 0 || cols < 0 || (rows > 0 && (!w || !codes || !scales)))
    return fail(DLO_E_ARG, "bad arguments");
  for_rows(rows, cols, [&](int64_t r) {
    const uint16_t *wr = w + r * cols;
    float amax = 0.f;
    for (int64_t j = 0; j < cols; ++j) {
      const float a = std::fabs(widen_bf16(wr[j]));
      if (a > amax) amax = a;  // NaN never compares greater
    }
    const float sc = amax > 0.f ? amax / 127.0f : 1.0f;
    scales[r] = sc;
    for (int64_t j = 0; j < cols; ++j) {
      const float q = std::nearbyintf(widen_bf16(wr[j]) / sc);  // default rounding: to nearest even
      codes[r * cols + j] = q != q ? 0 : (int8_t)std::max(-127.0f, std::min(127.0f, q));
    }
  });
  return ok();
}

int dlo_quantize_mxfp8(const uint16_t *w, int64_t rows, int64_t cols, uint8_t *codes, uint8_t *scales) {
  if (rows < 0 || cols < 0 || cols % 32 || (rows > 0 && (!w || !codes || !scales)))
    return fail(DLO_E_ARG, "bad arguments (cols must be a multiple of 32)");
  const int64_t nb = cols / 32;
  for_rows(rows, cols, [&](int64_t r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint16_t *wb = w + r * cols + b * 32;
      float amax = 0.f;
      for (int j = 0; j < 32; ++j) {
        const float a = std::fabs(widen_bf16(wb[j]));
        if (a > amax) amax = a;
      }
      // shared exponent floor(log2 amax) - 8: the exponent field of amax (bf16
      // values are normal or zero), clamped to the E8M0 range
      int X = -127;
      if (amax > 0.f) {
        uint32_t u;
        std::memcpy(&u, &amax, 4);
        X = std::max(-127, std::min(127, (int)((u >> 23) & 0xFF) - 127 - 8));
      }
      scales[b * rows + r] = (uint8_t)(X + 127);   // block-major [cols / 32, rows]
      for (int j = 0; j < 32; ++j) codes[r * cols + b * 32 + j] = e4m3_encode(std::ldexp(widen_bf16(wb[j]), -X));
    }
  });
  return ok();
}

int dlo_quantize_fp8(const uint16_t *w, int64_t n, uint8_t *codes, float *scale) {
  if (!scale || n < 0 || (n > 0 && (!w || !codes))) return fail(DLO_E_ARG, "bad arguments");
  auto widen = [](uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  };
  // large tensors on up to 16 threads (a max and an elementwise map: the result
  // does not depend on the split)
  const int nt = (int)std::min<int64_t>(16, std::max<int64_t>(1, n >> 20));
  const int64_t chunk = (n + nt - 1) / nt;
  std::vector<float> part((size_t)nt, 0.f);
  auto run = [&](auto &&fn) {
    std::vector<std::thread> th;
    for (int t = 1; t < nt; ++t) th.emplace_back(fn, t);
    fn(0);
    for (auto &x : th) x.join();
  };
  run([&](int t) {
    float m = 0.f;
    for (int64_t i = t * chunk; i < std::min(n, (t + 1) * chunk); ++i) {
      const float a = std::fabs(widen(w[i]));
      if (a > m) m = a;  // NaN never compares greater
    }
    part[(size_t)t] = m;
  });
  float amax = 0.f;
  for (float m : part) amax = std::max(amax, m);
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  *scale = sc;
  run([&](int t) {
    for (int64_t i = t * chunk; i < std::min(n, (t + 1) * chunk); ++i) codes[i] = e4m3_encode(widen(w[i]) / sc);
  });
  return ok();
}

const char *dlo_kernel_name(int32_t j) {
  return (j >= 0 && j < DLO_KERNELS_PER_BLOCK) ? kKernelNames[j] : nullptr;
}

// --------------------------------------------------------------------------- plan

int dlo_plan_blocks(const dlo_block *blocks, int32_t n_blocks, int32_t k, dlo_plan **out) {
  if (!out) return fail(DLO_E_ARG, "out is NULL");
  *out = nullptr;
  if (!blocks) return fail(DLO_E_ARG, "blocks is NULL");
  if (n_blocks < 1) return fail(DLO_E_ARG, "n_blocks must be >= 1 (got %d)", n_blocks);
  if (k < 1) return fail(DLO_E_ARG, "k must be >= 1 (got %d)", k);
  dlo_plan *pl = new (std::nothrow) dlo_plan;
  if (!pl) return fail(DLO_E_HOSTMEM, "out of host memory");
  pl->k = k;
  pl->blocks.resize(n_blocks);
  for (int b = 0; b < n_blocks; ++b) {
    const dlo_block &blk = blocks[b];
    BlockPlan &bp = pl->blocks[b];
    if (blk.n_params < 0 || (blk.n_params > 0 && !blk.params)) {
      delete pl;
      return fail(DLO_E_ARG, "block %d: bad parameter list", b);
    }
    bp.d = blk.d_model;
    bp.heads = blk.n_heads;
    // dtype groups in order of first appearance ([Aug] s.2: flattened by dtype)
    for (int p = 0; p < blk.n_params; ++p) {
      const dlo_param &pr = blk.params[p];
      if (!pr.name) {
        delete pl;
        return fail(DLO_E_ARG, "block %d parameter %d has no name", b, p);
      }
      if (!known_dtype(pr.dtype)) {
        delete pl;
        return fail(DLO_E_ARG, "block %d parameter %s: unknown dtype %d", b, pr.name, pr.dtype);
      }
      if (pr.numel < 0) {
        delete pl;
        return fail(DLO_E_ARG, "block %d parameter %s: negative numel", b, pr.name);
      }
      int g = -1;
      for (int q = 0; q < bp.n_groups; ++q)
        if (bp.gdtype[q] == pr.dtype) g = q;
      if (g < 0) {
        g = bp.n_groups++;
        bp.gdtype[g] = pr.dtype;
      }
      bp.names.emplace_back(pr.name);
      bp.dtypes.push_back(pr.dtype);
      bp.numels.push_back(pr.numel);
      bp.pgroup.push_back(g);
      bp.poff.push_back(bp.gnumel[g]);
      bp.gnumel[g] += pr.numel;
    }
    // ceil-div equal shards; regions at the all-gather offsets, 256-B aligned
    int64_t cursor = 0;
    for (int g = 0; g < bp.n_groups; ++g) {
      bp.gshard[g] = ceil_div(bp.gnumel[g], k);
      bp.gregion[g] = cursor;
      const int64_t bytes = (int64_t)k * bp.gshard[g] * elt_bytes(bp.gdtype[g]);
      bp.copy_bytes += bytes;
      cursor = align_up(cursor + bytes, DLO_ALIGN);
    }
    bp.extent = cursor;
    pl->slot_bytes = std::max(pl->slot_bytes, bp.extent);
    // DiT schema, bf16 or FP8 form?
    auto matches = [&](const SchemaEntry *sch, int np) {
      bool ok_ = blk.n_params == np && bp.d > 0;
      for (int p = 0; ok_ && p < np; ++p)
        ok_ = bp.names[p] == sch[p].name && bp.dtypes[p] == sch[p].dtype &&
              bp.numels[p] == schema_numel(sch[p], bp.d);
      return ok_;
    };
    bp.kind = matches(kDit, DLO_DIT_N_PARAMS)                              ? KIND_DIT
              : matches(kDitFp8, DLO_DIT_FP8_N_PARAMS)                     ? KIND_DIT_FP8
              : matches(kDitInt8, DLO_DIT_FP8_N_PARAMS)                    ? KIND_DIT_INT8
              : bp.d % 32 == 0 && matches(kDitMx, DLO_DIT_FP8_N_PARAMS) ? KIND_DIT_MX
                                                                           : KIND_NONE;
    pl->max_d = std::max(pl->max_d, bp.d);
    if (bp.kind == KIND_DIT_FP8) pl->max_fp8_d = std::max(pl->max_fp8_d, bp.d);
    if (bp.kind == KIND_DIT_INT8 || bp.kind == KIND_DIT_MX) pl->max_q_d = std::max(pl->max_q_d, bp.d);
    if (bp.kind == KIND_DIT_MX) pl->max_mx_d = std::max(pl->max_mx_d, bp.d);
    if (bp.kind == KIND_DIT_INT8) pl->max_i8_d = std::max(pl->max_i8_d, bp.d);
  }
  pl->id = g_plan_ids++;
  *out = pl;
  return ok();
}

void dlo_plan_destroy(dlo_plan *plan) {
  if (!plan) return;
  {
    std::lock_guard<std::mutex> lk(plan->mu);
    if (plan->enqueuing) {   // a run still being enqueued: let it finish enqueuing
      if (plan->enqueuing->worker.joinable()) plan->enqueuing->worker.join();
      plan->enqueuing->plan = nullptr;
      plan->enqueuing = nullptr;
    }
    reap_detached(plan, true);
    if (plan->last_done) (void)hipEventDestroy(plan->last_done);
  }
  delete plan;
}

int32_t dlo_plan_n_blocks(const dlo_plan *plan) { return plan ? (int32_t)plan->blocks.size() : -1; }
int32_t dlo_plan_k(const dlo_plan *plan) { return plan ? plan->k : -1; }
int64_t dlo_plan_slot_bytes(const dlo_plan *plan) { return plan ? plan->slot_bytes : -1; }

int dlo_plan_block_info(const dlo_plan *plan, int32_t b, dlo_block_info *out) {
  if (!plan || !out) return fail(DLO_E_ARG, "NULL argument");
  if (b < 0 || b >= (int32_t)plan->blocks.size()) return fail(DLO_E_ARG, "block %d out of range", b);
  const BlockPlan &bp = plan->blocks[b];
  std::memset(out, 0, sizeof *out);
  out->d_model = bp.d;
  out->n_heads = bp.heads;
  out->n_params = (int32_t)bp.names.size();
  out->n_groups = bp.n_groups;
  for (int g = 0; g < bp.n_groups; ++g) {
    out->dtype[g] = bp.gdtype[g];
    out->numel[g] = bp.gnumel[g];
    out->shard[g] = bp.gshard[g];
    out->region[g] = bp.gregion[g];
  }
  out->extent = bp.extent;
  out->copy_bytes = bp.copy_bytes;
  out->is_dit = bp.kind;
  return ok();
}

int dlo_plan_param_offset(const dlo_plan *plan, int32_t b, int32_t p, int64_t *byte_offset) {
  if (!plan || !byte_offset) return fail(DLO_E_ARG, "NULL argument");
  if (b < 0 || b >= (int32_t)plan->blocks.size()) return fail(DLO_E_ARG, "block %d out of range", b);
  const BlockPlan &bp = plan->blocks[b];
  if (p < 0 || p >= (int32_t)bp.names.size()) return fail(DLO_E_ARG, "param %d out of range", p);
  *byte_offset = bp.param_byte(p);
  return ok();
}

int64_t dlo_plan_workspace_bytes(const dlo_plan *plan, int32_t tokens) {
  if (!plan || tokens < 1) {
    fail(DLO_E_ARG, "bad plan or tokens");
    return -1;
  }
  g_err.clear();
  return workspace_bytes_for(plan->max_d, tokens, plan->max_fp8_d, plan->max_q_d, plan->max_mx_d, plan->max_i8_d);
}

int dlo_plan_schedule(const dlo_plan *plan, int32_t passes, dlo_sched_op *ops, int64_t cap,
                      int64_t *n_ops) {
  return dlo_plan_schedule_ex(plan, passes, 0, ops, cap, n_ops);
}

int dlo_plan_schedule_ex(const dlo_plan *plan, int32_t passes, int32_t n_resident,
                         dlo_sched_op *ops, int64_t cap, int64_t *n_ops) {
  if (!plan || !n_ops) return fail(DLO_E_ARG, "NULL argument");
  if (passes < 1) return fail(DLO_E_ARG, "passes must be >= 1");
  const int n = (int)plan->blocks.size();
  if (n_resident < 0 || n_resident > n) return fail(DLO_E_ARG, "n_resident %d not in [0, %d]", n_resident, n);
  const std::vector<Step> steps = hook_steps(n, passes, n_resident);
  const std::vector<dlo_sched_op> prog = build_program(steps, false);
  *n_ops = (int64_t)prog.size();
  if (!ops) return ok();
  if (cap < (int64_t)prog.size()) return fail(DLO_E_ARG, "cap %lld < %zu ops", (long long)cap, prog.size());
  std::memcpy(ops, prog.data(), prog.size() * sizeof(dlo_sched_op));
  return ok();
}

// --------------------------------------------------------------------------- store

void dlo_host_store_destroy(dlo_host_store *store) {
  if (!store) return;
  {   // a run still being enqueued reads the store: let it finish enqueuing
    std::lock_guard<std::mutex> lk(store->mu);
    if (store->enqueuing) {
      if (store->enqueuing->worker.joinable()) store->enqueuing->worker.join();
      store->enqueuing->store = nullptr;
      store->enqueuing = nullptr;
    }
  }
  if (store->last_copy) {   // the copies that read the store have completed
    (void)hipEventSynchronize(store->last_copy);
    (void)hipEventDestroy(store->last_copy);
  }
  for (int j = 0; j < 2; ++j) {
    if (store->staging_free[j]) {
      (void)hipEventSynchronize(store->staging_free[j]);
      (void)hipEventDestroy(store->staging_free[j]);
    }
    if (store->staging[j]) (void)hipHostFree(store->staging[j]);
  }
  for (size_t b = 0; b < store->mem.size(); ++b) {
    char *m = store->mem[b];
    if (!m) continue;
    if (store->pinned[b])
      (void)hipHostFree(m);
    else
      std::free(m);
  }
  delete store;
}

namespace {
int ensure_staging(dlo_host_store *st) {
  if (st->staging[0]) return DLO_OK;
  const int64_t bytes = std::max<int64_t>(st->plan->slot_bytes, 4096);
  for (int j = 0; j < 2; ++j) {
    void *m = nullptr;
    hipError_t e = hipHostMalloc(&m, (size_t)bytes, hipHostMallocDefault);
    if (e != hipSuccess)
      return fail(DLO_E_PIN, "pinned staging buffer of %lld bytes: %s", (long long)bytes,
                  hipGetErrorString(e));
    st->staging[j] = static_cast<char *>(m);
    e = hipEventCreateWithFlags(&st->staging_free[j], hipEventDisableTiming);
    if (e != hipSuccess) return fail(DLO_E_HIP, "hipEventCreate: %s", hipGetErrorString(e));
  }
  st->staging_bytes = bytes;
  return DLO_OK;
}
}  // namespace

int dlo_host_store_create_ex(const dlo_plan *plan, uint32_t flags, int64_t pinned_limit_bytes,
                             dlo_host_store **out) {
  if (!out) return fail(DLO_E_ARG, "out is NULL");
  *out = nullptr;
  if (!plan) return fail(DLO_E_ARG, "plan is NULL");
  if (flags > DLO_STORE_AUTO) return fail(DLO_E_ARG, "unknown store flags 0x%x", flags);
  if (pinned_limit_bytes < 0) return fail(DLO_E_ARG, "negative pinned limit");
  dlo_host_store *st = new (std::nothrow) dlo_host_store;
  if (!st) return fail(DLO_E_HOSTMEM, "out of host memory");
  st->plan = plan;
  st->plan_id = plan->id;
  const int nb = (int)plan->blocks.size(), k = plan->k;
  st->mem.assign(nb, nullptr);
  st->pinned.assign(nb, 0);
  st->shard_at.resize(nb);
  st->packed.assign(nb, 0);
  if (flags == DLO_STORE_AUTO) {
    // reserve the staging buffers first: pageable blocks cannot move without them
    int rc = ensure_staging(st);
    if (rc) {
      dlo_host_store_destroy(st);
      return rc;
    }
  }
  bool may_pin = flags != DLO_STORE_PAGEABLE;
  int64_t pinned_total = 0;
  for (int b = 0; b < nb; ++b) {
    const BlockPlan &bp = plan->blocks[b];
    int64_t cursor = 0;
    st->shard_at[b].resize((size_t)bp.n_groups * k);
    for (int g = 0; g < bp.n_groups; ++g)
      for (int r = 0; r < k; ++r) {
        st->shard_at[b][g * k + r] = cursor;
        cursor = align_up(cursor + bp.gshard[g] * elt_bytes(bp.gdtype[g]), 4096);
      }
    const size_t bytes = (size_t)std::max<int64_t>(cursor, 4096);
    void *m = nullptr;
    if (may_pin && flags == DLO_STORE_AUTO && pinned_limit_bytes > 0 &&
        pinned_total + (int64_t)bytes > pinned_limit_bytes)
      may_pin = false;
    if (may_pin) {
      // [Aug] s.2: the shard is a pinned DMA buffer for fast H2D
      hipError_t e = hipHostMalloc(&m, bytes, hipHostMallocDefault);
      if (e != hipSuccess) {
        m = nullptr;
        (void)hipGetLastError();
        if (flags == DLO_STORE_PINNED) {
          dlo_host_store_destroy(st);
          return fail(DLO_E_PIN, "hipHostMalloc(%zu) for block %d failed: %s", bytes, b,
                      hipGetErrorString(e));
        }
        may_pin = false;   // AUTO: this and every later block is staged
      } else {
        st->pinned[b] = 1;
        pinned_total += (int64_t)bytes;
      }
    }
    if (!m) {
      m = std::aligned_alloc(4096, align_up((int64_t)bytes, 4096));
      if (!m) {
        dlo_host_store_destroy(st);
        return fail(DLO_E_HOSTMEM, "host allocation of %zu bytes for block %d failed", bytes, b);
      }
    }
    st->mem[b] = static_cast<char *>(m);
  }
  *out = st;
  return ok();
}

int dlo_host_store_create(const dlo_plan *plan, uint32_t flags, dlo_host_store **out) {
  return dlo_host_store_create_ex(plan, flags, 0, out);
}

int dlo_host_store_info(const dlo_host_store *store, int32_t *pinned_blocks,
                        int64_t *pinned_bytes, int32_t *staged_blocks) {
  if (!store) return fail(DLO_E_ARG, "store is NULL");
  int32_t pb = 0, sb = 0;
  int64_t bytes = 0;
  for (size_t b = 0; b < store->mem.size(); ++b) {
    if (store->pinned[b]) {
      ++pb;
      const BlockPlan &bp = store->plan->blocks[b];
      int64_t c = 0;
      for (int g = 0; g < bp.n_groups; ++g) c += store->plan->k * align_up(bp.gshard[g] * elt_bytes(bp.gdtype[g]), 4096);
      bytes += std::max<int64_t>(c, 4096);
    } else {
      ++sb;
    }
  }
  if (pinned_blocks) *pinned_blocks = pb;
  if (pinned_bytes) *pinned_bytes = bytes;
  if (staged_blocks) *staged_blocks = sb;
  return ok();
}

int dlo_pack_host_shards(dlo_host_store *store, int32_t b_begin, int32_t b_end,
                         const dlo_block *blocks) {
  if (!store || !blocks) return fail(DLO_E_ARG, "NULL argument");
  const dlo_plan *plan = store->plan;
  const int nb = (int)plan->blocks.size(), k = plan->k;
  if (b_begin < 0 || b_end > nb || b_begin >= b_end)
    return fail(DLO_E_ARG, "block range [%d, %d) invalid for %d blocks", b_begin, b_end, nb);
  for (int b = b_begin; b < b_end; ++b) {
    int rc = validate_block_against(plan->blocks[b], blocks[b - b_begin], b, true);
    if (rc) return rc;
  }
  std::vector<CopyTask> tasks;
  for (int b = b_begin; b < b_end; ++b) {
    const BlockPlan &bp = plan->blocks[b];
    const dlo_block &blk = blocks[b - b_begin];
    for (int g = 0; g < bp.n_groups; ++g) {
      const int64_t S = bp.gshard[g], elt = elt_bytes(bp.gdtype[g]);
      if (S == 0) continue;
      auto shard_ptr = [&](int r) { return const_cast<char *>(static_cast<const char *>(store->shard(b, g, r))); };
      // [Aug] s.2: shard r holds flat[r*S, (r+1)*S) of the group's flat buffer
      for (int p = 0; p < (int)bp.names.size(); ++p) {
        if (bp.pgroup[p] != g || bp.numels[p] == 0) continue;
        const char *src = static_cast<const char *>(blk.params[p].src);
        int64_t e = bp.poff[p];
        const int64_t end = e + bp.numels[p];
        while (e < end) {
          const int64_t r = e / S, pos = e % S, len = std::min(S - pos, end - e);
          tasks.push_back({shard_ptr((int)r) + pos * elt, src + (e - bp.poff[p]) * elt, len * elt});
          e += len;
        }
      }
      // zero padding beyond N_g, so that every shard has S_g elements
      int64_t e = bp.gnumel[g];
      const int64_t end = (int64_t)k * S;
      while (e < end) {
        const int64_t r = e / S, pos = e % S, len = std::min(S - pos, end - e);
        tasks.push_back({shard_ptr((int)r) + pos * elt, nullptr, len * elt});
        e += len;
      }
    }
  }
  run_copies(tasks);
  for (int b = b_begin; b < b_end; ++b) store->packed[b] = 1;
  return ok();
}

int dlo_host_store_shard(const dlo_host_store *store, int32_t b, int32_t g, int32_t r,
                         const void **ptr, int64_t *bytes) {
  if (!store || !ptr || !bytes) return fail(DLO_E_ARG, "NULL argument");
  const dlo_plan *plan = store->plan;
  if (b < 0 || b >= (int32_t)plan->blocks.size()) return fail(DLO_E_ARG, "block out of range");
  const BlockPlan &bp = plan->blocks[b];
  if (g < 0 || g >= bp.n_groups || r < 0 || r >= plan->k) return fail(DLO_E_ARG, "shard out of range");
  *ptr = store->shard(b, g, r);
  *bytes = bp.gshard[g] * elt_bytes(bp.gdtype[g]);
  return ok();
}

int32_t dlo_host_store_complete(const dlo_host_store *store) {
  if (!store) return 0;
  for (uint8_t f : store->packed)
    if (!f) return 0;
  return 1;
}

// --------------------------------------------------------------------------- placement

namespace {
// the k shards of every group at region_g + r * S_g * elt_g ([Jul] "Weight
// Sharding + AllGather": the all-gather output is the rank-ordered concatenation)
hipError_t place_from(const dlo_plan *plan, int b, const void *(*src)(const dlo_host_store *, const char *, int, int, int, int64_t),
                      const dlo_host_store *st, const char *staging, char *dst, hipStream_t s) {
  const BlockPlan &bp = plan->blocks[b];
  for (int g = 0; g < bp.n_groups; ++g) {
    const int64_t sb = bp.gshard[g] * elt_bytes(bp.gdtype[g]);
    if (sb == 0) continue;
    // shard r goes to region_g + r * sb; consecutive shards whose host bytes are
    // also consecutive move in one DMA (the same bytes to the same offsets)
    for (int r = 0; r < plan->k;) {
      const int64_t off = bp.gregion[g] + r * sb;
      const char *from = static_cast<const char *>(src(st, staging, b, g, r, off));
      int r2 = r + 1;
      while (r2 < plan->k &&
             static_cast<const char *>(src(st, staging, b, g, r2, bp.gregion[g] + r2 * sb)) == from + (r2 - r) * sb)
        ++r2;
      hipError_t e = hipMemcpyAsync(dst + off, from, (size_t)((r2 - r) * sb), hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return e;
      r = r2;
    }
  }
  return hipSuccess;
}

const void *from_store(const dlo_host_store *st, const char *, int b, int g, int r, int64_t) {
  return st->shard(b, g, r);
}

const void *from_staging(const dlo_host_store *, const char *staging, int, int, int, int64_t off) {
  return staging + off;
}

// One block into `dst` on stream s.  A pinned block is copied directly.  A
// pageable block goes through staging buffer j = (use count) mod 2 ([Doc]
// "Rank-local path without DLO AllGather": two bounded pinned staging slots):
// the calling thread waits until the buffer's previous DMA has drained, copies
// the block's shards into it (several threads) laid out as the slot image, and
// enqueues the DMA into dst; the fill of one buffer overlaps the DMA out of the
// other.  (A fill run as a host function on a stream of its own, so that the
// call would not wait, made the runtime serialise the copy and compute streams
// of the whole run: measured overlap 0 on the Super stack.)  `begin`
// (optional) is recorded on s just before the DMAs.  Returns a dlo status.
int place_copies(const dlo_plan *plan, dlo_host_store *st, int b, char *dst, hipStream_t s, hipEvent_t begin);

int place(const dlo_plan *plan, dlo_host_store *st, int b, char *dst, hipStream_t s,
          hipEvent_t begin = nullptr) {
  int rc = DLO_OK;
  if (!st->last_copy)
    rc = check_hip(hipEventCreateWithFlags(&st->last_copy, hipEventDisableTiming), "hipEventCreate");
  if (!rc) rc = place_copies(plan, st, b, dst, s, begin);
  if (!rc) rc = check_hip(hipEventRecord(st->last_copy, s), "hipEventRecord");
  return rc;
}

int place_copies(const dlo_plan *plan, dlo_host_store *st, int b, char *dst, hipStream_t s, hipEvent_t begin) {
  if (st->pinned[b]) {
    if (begin) {
      int rc = check_hip(hipEventRecord(begin, s), "hipEventRecord");
      if (rc) return rc;
    }
    return check_hip(place_from(plan, b, from_store, st, nullptr, dst, s), "hipMemcpyAsync");
  }
  int rc = ensure_staging(st);
  if (rc) return rc;
  const int j = (int)(st->staged_uses++ & 1);
  rc = check_hip(hipEventSynchronize(st->staging_free[j]), "hipEventSynchronize(staging)");
  if (rc) return rc;
  const BlockPlan &bp = plan->blocks[b];
  std::vector<CopyTask> tasks;
  for (int g = 0; g < bp.n_groups; ++g) {
    const int64_t sb = bp.gshard[g] * elt_bytes(bp.gdtype[g]);
    for (int r = 0; r < plan->k && sb > 0; ++r)
      tasks.push_back({st->staging[j] + bp.gregion[g] + r * sb,
                       static_cast<const char *>(st->shard(b, g, r)), sb});
  }
  run_copies(tasks);
  if (begin) {
    rc = check_hip(hipEventRecord(begin, s), "hipEventRecord");
    if (rc) return rc;
  }
  rc = check_hip(place_from(plan, b, from_staging, st, st->staging[j], dst, s), "hipMemcpyAsync");
  if (rc) return rc;
  return check_hip(hipEventRecord(st->staging_free[j], s), "hipEventRecord(staging)");
}
}  // namespace

int dlo_place_block(const dlo_plan *plan, const dlo_host_store *store, int32_t b, void *dst,
                    int64_t dst_bytes, void *stream) {
  if (!plan || !store || !dst) return fail(DLO_E_ARG, "NULL argument");
  if (store->plan_id != plan->id) return fail(DLO_E_PLAN_MISMATCH, "store was made by another plan");
  if (b < 0 || b >= (int32_t)plan->blocks.size()) return fail(DLO_E_ARG, "block out of range");
  if (!store->packed[b]) return fail(DLO_E_STATE, "block %d has not been packed", b);
  if (dst_bytes < plan->blocks[b].extent)
    return fail(DLO_E_SLOT_SMALL, "destination %lld < extent %lld", (long long)dst_bytes,
                (long long)plan->blocks[b].extent);
  int rc = place(plan, const_cast<dlo_host_store *>(store), b, static_cast<char *>(dst),
                 (hipStream_t)stream);
  return rc ? rc : ok();
}

// --------------------------------------------------------------------------- forward

namespace {

struct Workspace {
  float *silu_c, *mod, *act_scale;
  uint16_t *h, *big, *dq;
  uint8_t *act_codes;
};

Workspace carve(void *ws, int32_t max_d, int64_t T, int32_t fp8_d, int32_t q_d, int32_t mx_d, int32_t i8_d) {
  char *p = static_cast<char *>(ws);
  Workspace w;
  w.silu_c = reinterpret_cast<float *>(p);
  p += align_up(4 * (int64_t)max_d, DLO_ALIGN);
  w.mod = reinterpret_cast<float *>(p);
  p += align_up(24 * (int64_t)max_d, DLO_ALIGN);
  w.h = reinterpret_cast<uint16_t *>(p);    // h [T,d]
  p += align_up(2 * T * max_d, DLO_ALIGN);
  w.big = reinterpret_cast<uint16_t *>(p);  // qk [T,2d], V^T [d,T64], a [T,d]; later u [T,4d]
  p += align_up(8 * round_up64(T) * max_d, DLO_ALIGN);
  w.dq = reinterpret_cast<uint16_t *>(p);   // a quantised block's weights, dequantised to bf16
  p += align_up(dequant_bytes(fp8_d, q_d), DLO_ALIGN);
  w.act_codes = reinterpret_cast<uint8_t *>(p);  // W8A8: a linear input's 1-byte codes [T, <= 4d]
  const int32_t wq = std::max(std::max(fp8_d, i8_d), mx_d);
  p += wq > 0 ? align_up(4 * T * wq, DLO_ALIGN) : 0;
  w.act_scale = reinterpret_cast<float *>(p);    // ... and its scales (fp32 per row, or E8M0 block-major)
  return w;
}

// One block forward on the compute stream, parameters re-pointed into `base`
// (a slot or a resident image) with no copy ([Jul] "How It Works", step 3).
// An FP8 block's adaLN GEMV reads the E4M3 codes and scale in place; its four
// linears either run on bf16 copies of their weights (dequantised into the
// workspace) or, with fp8 compute, as W8A8 products: each input quantised per
// row to E4M3, times the weight's codes and per-tensor scale ([Doc] "Request
// and loading constraints", online FP8 linears).
hipError_t block_forward(const BlockPlan &bp, const char *base, const dlo_forward_args *a,
                         const Workspace &w, hipStream_t s, hipEvent_t *kernel_end, uint32_t *kmask,
                         float *x, bool prep) {
  const int d = bp.d, H = bp.heads, dh = d / H, T = a->tokens;
  auto P = [&](int lp) { return base + bp.logical_byte(lp); };
  auto F = [&](int lp) { return reinterpret_cast<const float *>(P(lp)); };
  const bool fp8 = bp.kind == KIND_DIT_FP8, mx = bp.kind == KIND_DIT_MX, i8 = bp.kind == KIND_DIT_INT8;
  const bool w8a8 = (fp8 || mx || i8) && (a->flags & DLO_FP8_COMPUTE);
  hipError_t e;
  // bf16 weights: in the slot, or (quantised block, W8A16) dequantised into the
  // workspace; codes and scales of a quantised block: in the slot
  const uint16_t *Wt[5] = {};
  const uint8_t *W8[5] = {};
  const float *S8[5] = {};
  const uint8_t *SM[5] = {};   // MXFP8: E8M0 scales, block-major [in / 32, out]
  if (fp8) {
    uint16_t *dst = w.dq;
    for (int i = 0; i < 5; ++i) {
      W8[i] = reinterpret_cast<const uint8_t *>(P(kWeightP[i]));
      S8[i] = reinterpret_cast<const float *>(base + bp.param_byte(kFp8Scale[i]));
      if (i == 0 || w8a8) continue;
      const int64_t n = kWeightD2[i] * d * d;
      if (prep && (e = dlo::launch_dequant_fp8(W8[i], n, S8[i], dst, s)) != hipSuccess) return e;
      Wt[i] = dst;
      dst += n;
    }
  } else if (bp.kind == KIND_DIT_INT8 || bp.kind == KIND_DIT_MX) {
    // INT8 / MXFP8: all five weights dequantised (MXFP8 exactly: an E4M3 value
    // times a power of two fits bf16)
    uint16_t *dst = w.dq;
    for (int i = 0; i < 5; ++i) {
      const int64_t rows = kWeightRows[i] * d, cols = kWeightCols[i] * d;
      const char *sc = base + bp.param_byte(kFp8Scale[i]);
      W8[i] = reinterpret_cast<const uint8_t *>(P(kWeightP[i]));
      SM[i] = reinterpret_cast<const uint8_t *>(sc);
      if (w8a8 && i > 0) continue;   // W8A8: only the adaLN weight runs in bf16
      e = !prep ? hipSuccess
          : bp.kind == KIND_DIT_INT8
              ? dlo::launch_dequant_int8(reinterpret_cast<const int8_t *>(P(kWeightP[i])), rows, cols,
                                         reinterpret_cast<const float *>(sc), dst, s)
              : dlo::launch_dequant_mxfp8(reinterpret_cast<const uint8_t *>(P(kWeightP[i])), rows, cols,
                                          reinterpret_cast<const uint8_t *>(sc), dst, s);
      if (e != hipSuccess) return e;
      Wt[i] = dst;
      dst += rows * cols;
    }
  } else {
    for (int i = 0; i < 5; ++i) Wt[i] = reinterpret_cast<const uint16_t *>(P(kWeightP[i]));
  }
  // kernel slot j's end event is recorded only when the slot launched work: an
  // event record between kernels costs the stream a few microseconds, and an
  // empty slot's duration is 0
  auto mark = [&](bool launched, int j) {
    if (!kernel_end || !launched) return hipSuccess;
    *kmask |= 1u << j;
    return hipEventRecord(kernel_end[j], s);
  };
  const bool dequant = prep && ((fp8 && !w8a8) || i8 || mx);
  if ((e = mark(dequant, 0)) != hipSuccess) return e;
  const int64_t ldx = a->x_row_stride;
  const float *mod = w.mod;
  // q and k from one GEMM; v from a second one that stores V^T, the layout the
  // attention reads its values in
  const int64_t ldvt = round_up64(T);
  uint16_t *qk = w.big;
  uint16_t *vt = w.big + (int64_t)T * 2 * d;
  uint16_t *attn = vt + (int64_t)d * ldvt;
  uint16_t *u = w.big;
  uint8_t *q8 = w.act_codes;
  float *qs = w.act_scale;
  uint8_t *mxs = reinterpret_cast<uint8_t *>(w.act_scale);   // MXFP8: [K / 32, T64] block-major
  const int64_t T64 = round_up64(T);
  // a linear: A [T, K] bf16 (row stride K) times weight i's rows n0 .. n0 + N - 1
  auto linear = [&](const uint16_t *A, int K, int i, int64_t n0, int N, const float *bias,
                    const float *gate, void *C, int64_t ldc, int epi) {
    if (w8a8 && mx)
      return dlo::launch_gemm_mxfp8(q8, K, mxs, T64, W8[i] + n0 * K, K, SM[i] + n0, kWeightRows[i] * d, T, N,
                                    K, bias, gate, C, ldc, epi, s);
    if (w8a8 && i8)
      return dlo::launch_gemm_int8(reinterpret_cast<const int8_t *>(q8), K, qs,
                                   reinterpret_cast<const int8_t *>(W8[i]) + n0 * K, K,
                                   reinterpret_cast<const float *>(SM[i]) + n0, T, N, K, bias, gate, C, ldc, epi, s);
    if (w8a8)
      return dlo::launch_gemm_fp8(q8, K, qs, W8[i] + n0 * K, K, S8[i], T, N, K, bias, gate, C, ldc, epi, s);
    return dlo::launch_gemm(A, K, Wt[i] + n0 * K, K, T, N, K, bias, gate, C, ldc, epi, s);
  };
  // W8A8: a linear input's codes (per-row E4M3 or int8, or MXFP8 per 32 columns); otherwise nothing
  auto quant = [&](const uint16_t *A, int K) {
    if (!w8a8) return hipSuccess;
    if (i8) return dlo::launch_quant_rows_int8(A, K, T, K, reinterpret_cast<int8_t *>(q8), K, qs, s);
    return mx ? dlo::launch_quant_rows_mx(A, K, T, K, q8, K, mxs, T64, s)
              : dlo::launch_quant_rows_fp8(A, K, T, K, q8, K, qs, s);
  };
#define DLO_STEP_IF(launched, call, j)                                      \
  if ((e = (call)) != hipSuccess) return e;                                 \
  if ((e = mark((launched), j)) != hipSuccess) return e;
#define DLO_STEP(call, j) DLO_STEP_IF(true, call, j)
  DLO_STEP(fp8 ? dlo::launch_adaln_gemv_fp8(W8[0], S8[0], w.silu_c, F(P_ADA_B), w.mod, 6 * d, d, s)
               : dlo::launch_adaln_gemv(Wt[0], w.silu_c, F(P_ADA_B), w.mod, 6 * d, d, s), 1)
  // W8A8 FP8 / MXFP8: LayerNorm + modulate writes the next linear's codes
  // directly (quant_h and quant_h2 then record nothing); INT8 quantises h in
  // its own pass
  auto ln = [&](int pw, int pb, int pe, const float *shift_, const float *scale_) {
    if (w8a8 && !i8)
      return dlo::launch_ln_modulate_quant(x, ldx, T, d, F(pw), F(pb), F(pe), shift_, scale_, q8, d,
                                           mx ? static_cast<void *>(mxs) : static_cast<void *>(qs), T64, mx, s);
    return dlo::launch_ln_modulate(x, ldx, T, d, F(pw), F(pb), F(pe), shift_, scale_, w.h, s);
  };
  DLO_STEP(ln(P_N1_W, P_N1_B, P_N1_EPS, mod + 0 * d, mod + 1 * d), 2)
  DLO_STEP_IF(i8 && w8a8, i8 ? quant(w.h, d) : hipSuccess, 3)
  DLO_STEP(linear(w.h, d, 1, 0, 2 * d, F(P_QKV_B), nullptr, qk, 2 * d, dlo::EPI_BIAS), 4)
  DLO_STEP(linear(w.h, d, 1, 2 * d, d, F(P_QKV_B) + 2 * d, nullptr, vt, ldvt, dlo::EPI_BIAS_T), 5)
  DLO_STEP(dlo::launch_attention(qk, 2 * d, vt, ldvt, T, H, dh, attn, d, s), 6)
  DLO_STEP_IF(w8a8, quant(attn, d), 7)
  DLO_STEP(linear(attn, d, 2, 0, d, F(P_OUT_B), mod + 2 * d, x, ldx, dlo::EPI_GATED_RESIDUAL), 8)
  DLO_STEP(ln(P_N2_W, P_N2_B, P_N2_EPS, mod + 3 * d, mod + 4 * d), 9)
  DLO_STEP_IF(i8 && w8a8, i8 ? quant(w.h, d) : hipSuccess, 10)
  if (w8a8 && mx) {
    // MXFP8: the fc1 epilogue quantises u itself (32-column blocks never leave
    // its column tile); u's codes and scales take the place of the bf16 u
    uint8_t *uq = reinterpret_cast<uint8_t *>(w.big);
    uint8_t *us = uq + align_up((int64_t)T * 4 * d, DLO_ALIGN);
    DLO_STEP(dlo::launch_gemm_mxfp8(q8, d, mxs, T64, W8[3], d, SM[3], kWeightRows[3] * d, T, 4 * d, d,
                                    F(P_FC1_B), nullptr, uq, 4 * d, dlo::EPI_GELU_MX, s, us, T64), 11)
    DLO_STEP_IF(false, hipSuccess, 12)
    DLO_STEP(dlo::launch_gemm_mxfp8(uq, 4 * d, us, T64, W8[4], 4 * d, SM[4], kWeightRows[4] * d, T, d, 4 * d,
                                    F(P_FC2_B), mod + 5 * d, x, ldx, dlo::EPI_GATED_RESIDUAL, s), 13)
  } else {
    DLO_STEP(linear(w.h, d, 3, 0, 4 * d, F(P_FC1_B), nullptr, u, 4 * d, dlo::EPI_BIAS_GELU), 11)
    DLO_STEP_IF(w8a8, quant(u, 4 * d), 12)
    DLO_STEP(linear(u, 4 * d, 4, 0, d, F(P_FC2_B), mod + 5 * d, x, ldx, dlo::EPI_GATED_RESIDUAL), 13)
  }
#undef DLO_STEP
#undef DLO_STEP_IF
  return hipSuccess;
}


int validate_forward(const dlo_plan *plan, const dlo_host_store *store, const dlo_forward_args *a) {
  if (!plan || !a) return fail(DLO_E_ARG, "NULL plan or args");
  if (a->flags & ~(DLO_TRACE_DIGEST | DLO_TRACE_TIMING | DLO_RESIDENT | DLO_FP8_COMPUTE | DLO_ASYNC_ENQUEUE))
    return fail(DLO_E_ARG, "unknown flags 0x%x", a->flags);
  if (a->batch < 0) return fail(DLO_E_ARG, "batch %d < 0", a->batch);
  if (a->cond_stride < 0 || (a->cond_stride > 0 && a->cond_stride < plan->max_d))
    return fail(DLO_E_ARG, "cond_stride %lld below the widest block %d", (long long)a->cond_stride, plan->max_d);
  const int n = (int)plan->blocks.size();
  if (!(a->flags & DLO_RESIDENT) && (a->n_resident < 0 || a->n_resident > n))
    return fail(DLO_E_ARG, "n_resident %d not in [0, %d]", a->n_resident, n);
  const int n_res = (a->flags & DLO_RESIDENT) ? n : a->n_resident;
  const bool resident = n_res == n;  // nothing streams
  if (!resident) {
    if (!store) return fail(DLO_E_ARG, "store is NULL");
    if (store->plan_id != plan->id)
      return fail(DLO_E_PLAN_MISMATCH, "the host store was built for another plan");
    if (!dlo_host_store_complete(store)) return fail(DLO_E_STATE, "the host store is not fully packed");
  }
  if (a->tokens < 1) return fail(DLO_E_ARG, "tokens must be >= 1");
  if (a->passes < 1) return fail(DLO_E_ARG, "passes must be >= 1");
  if (!a->x || !a->cond || !a->workspace) return fail(DLO_E_ARG, "x, cond and workspace are required");
  if (!a->compute_stream) return fail(DLO_E_ARG, "compute_stream is NULL");
  if (!resident && (!a->copy_stream || a->copy_stream == a->compute_stream))
    return fail(DLO_E_ARG, "copy_stream must be non-NULL and distinct from compute_stream");
  for (size_t b = 0; b < plan->blocks.size(); ++b) {
    const BlockPlan &bp = plan->blocks[b];
    if (bp.kind == KIND_NONE)
      return fail(DLO_E_UNSUPPORTED, "block %zu does not carry the DiT block schema (bf16 or FP8)", b);
    if (bp.d % 256 || bp.d > 8192)
      return fail(DLO_E_UNSUPPORTED, "block %zu: d = %d (need a multiple of 256, at most 8192)", b, bp.d);
    if (bp.heads < 1 || bp.d % bp.heads)
      return fail(DLO_E_UNSUPPORTED, "block %zu: %d heads do not divide d = %d", b, bp.heads, bp.d);
    const int dh = bp.d / bp.heads;
    if (dh != 64 && dh != 128) return fail(DLO_E_UNSUPPORTED, "block %zu: head dim %d (need 64 or 128)", b, dh);
  }
  if (a->x_row_stride < plan->max_d)
    return fail(DLO_E_ARG, "x_row_stride %lld < widest block %d", (long long)a->x_row_stride, plan->max_d);
  if (a->x_row_stride % 4 || (uintptr_t)a->x % 16)
    return fail(DLO_E_ARG, "x must be 16-B aligned with x_row_stride %% 4 == 0");
  if ((int64_t)256 * a->x_row_stride * 4 >= ((int64_t)1 << 31))
    return fail(DLO_E_UNSUPPORTED, "x_row_stride too large for 32-bit tile offsets");
  if (((int64_t)a->tokens + 64) * 3 * plan->max_d * 2 >= ((int64_t)1 << 31))
    return fail(DLO_E_UNSUPPORTED, "tokens x 3 d too large for 32-bit buffer offsets");
  const int64_t need = workspace_bytes_for(plan->max_d, a->tokens, plan->max_fp8_d, plan->max_q_d, plan->max_mx_d, plan->max_i8_d);
  if (a->workspace_bytes < need)
    return fail(DLO_E_WORKSPACE, "workspace %lld < %lld bytes", (long long)a->workspace_bytes, (long long)need);
  if (!resident) {
    if (!a->slot[0] || !a->slot[1]) return fail(DLO_E_ARG, "both slots are required");
    if (a->slot_bytes < plan->slot_bytes)
      return fail(DLO_E_SLOT_SMALL, "slot %lld < plan slot %lld bytes", (long long)a->slot_bytes,
                  (long long)plan->slot_bytes);
    const char *s0 = static_cast<const char *>(a->slot[0]), *s1 = static_cast<const char *>(a->slot[1]);
    const int64_t gap = s0 < s1 ? s1 - s0 : s0 - s1;
    if (gap < plan->slot_bytes) return fail(DLO_E_ARG, "the two slots overlap");
  }
  if (n_res > 0) {
    if (!a->resident_blocks) return fail(DLO_E_ARG, "resident blocks need resident_blocks");
    for (int b = 0; b < n_res; ++b)
      if (!a->resident_blocks[b]) return fail(DLO_E_ARG, "resident block %d is NULL", b);
  }
  return DLO_OK;
}

}  // namespace

namespace {
// A streamed run starts enqueueing once the plan's previous run has completed:
// copies enqueued behind a run still executing ran 6-29 % slower on the
// link-bound stacks (the irregular and Nano stacks, five to eight runs back to
// back against the same runs each enqueued after the previous one finished),
// while a compute-bound stack measured the same either way; within a run the
// copy/compute pipeline is enqueued whole as before.
int wait_previous_run(const dlo_plan *plan) {
  if (!plan->last_done) return DLO_OK;
  return check_hip(hipEventSynchronize(plan->last_done), "hipEventSynchronize (previous run)");
}

// Enqueues a validated run's program on its two streams; the calling thread
// fills the staging buffers of pageable blocks.  Returns a dlo status.
int enqueue_program(const dlo_plan *plan, dlo_host_store *store, const dlo_forward_args *a, dlo_run *run,
                    const std::vector<dlo_sched_op> &prog, bool resident) {
  constexpr int TEV = 4 + DLO_KERNELS_PER_BLOCK;  // copy begin, copy end, compute begin, kernels, compute end
  hipStream_t cs = (hipStream_t)a->compute_stream, ps = (hipStream_t)a->copy_stream;
  const int batch = a->batch < 1 ? 1 : a->batch;
  const int64_t cond_stride = a->cond_stride > 0 ? a->cond_stride : plan->max_d;
  const Workspace w = carve(a->workspace, plan->max_d, a->tokens, plan->max_fp8_d, plan->max_q_d, plan->max_mx_d, plan->max_i8_d);
  hipEvent_t t0 = run->timing ? run->tev.back() : nullptr;
  auto tev = [&](int64_t t, int j) { return run->tev[(size_t)(t * TEV + j)]; };
  hipError_t e = hipSuccess;
  int place_rc = DLO_OK;
  auto HIP = [&](hipError_t x) {
    if (e == hipSuccess && x != hipSuccess) e = x;
    return e == hipSuccess;
  };

  // order after the previous run (even one on other streams) and after the caller's
  // work on the compute stream
  HIP(hipStreamWaitEvent(cs, plan->last_done, 0));
  if (!resident) HIP(hipStreamWaitEvent(ps, plan->last_done, 0));
  if (t0) HIP(hipEventRecord(t0, cs));
  HIP(dlo::launch_silu(a->cond, w.silu_c, plan->max_d, cs));

  for (const dlo_sched_op &op : prog) {
    if (e != hipSuccess) break;
    hipStream_t s = op.stream == DLO_STREAM_COMPUTE ? cs : ps;
    switch (op.kind) {
      case DLO_OP_RECORD:
        HIP(hipEventRecord(run->ev[op.event], s));
        break;
      case DLO_OP_WAIT:
        HIP(hipStreamWaitEvent(s, run->ev[op.event], 0));
        break;
      case DLO_OP_COPY: {
        if (e == hipSuccess) {
          int prc = place(plan, store, op.block,
                          static_cast<char *>(a->slot[op.slot]), ps,
                          run->timing ? tev(op.step, 0) : nullptr);
          if (prc) {
            place_rc = prc;
            e = hipErrorUnknown;
          }
        }
        if (run->timing) HIP(hipEventRecord(tev(op.step, 1), ps));
        break;
      }
      case DLO_OP_COMPUTE: {
        const BlockPlan &bp = plan->blocks[op.block];
        const char *base = op.slot < 0 ? static_cast<const char *>(a->resident_blocks[op.block])
                                       : static_cast<const char *>(a->slot[op.slot]);
        int64_t offs[DLO_MAX_GROUPS], lens[DLO_MAX_GROUPS];
        for (int g = 0; g < bp.n_groups; ++g) {
          offs[g] = bp.gregion[g];
          lens[g] = (int64_t)plan->k * bp.gshard[g] * elt_bytes(bp.gdtype[g]);
        }
        if (run->digest)
          HIP(dlo::launch_digest(base, offs, lens, bp.n_groups, run->d_digest + 2 * op.step, cs));
        if (run->timing) HIP(hipEventRecord(tev(op.step, 2), cs));
        // the batch's samples one after another on the slot's weights (a quantised
        // block's dequantised weights made once); each sample's SiLU(c) first
        for (int b = 0; b < batch && e == hipSuccess; ++b) {
          if (batch > 1) HIP(dlo::launch_silu(a->cond + b * cond_stride, w.silu_c, plan->max_d, cs));
          if (e == hipSuccess)
            HIP(block_forward(bp, base, a, w, cs,
                              run->timing && b == 0 ? &run->tev[(size_t)(op.step * TEV + 3)] : nullptr,
                              run->timing ? &run->kmask[(size_t)op.step] : nullptr,
                              a->x + b * (int64_t)a->tokens * a->x_row_stride, b == 0));
        }
        if (run->timing) HIP(hipEventRecord(tev(op.step, 3 + DLO_KERNELS_PER_BLOCK), cs));
        if (run->digest)
          HIP(dlo::launch_digest(base, offs, lens, bp.n_groups, run->d_digest + 2 * op.step + 1, cs));
        break;
      }
    }
  }
  HIP(hipEventRecord(run->final_ev, cs));
  HIP(hipEventRecord(plan->last_done, cs));
  if (e != hipSuccess) {
    if (place_rc) return place_rc;
    return fail(DLO_E_HIP, "enqueue failed: %s (synchronise both streams; x is undefined)",
                hipGetErrorString(e));
  }
  return DLO_OK;
}
}  // namespace

int dlo_forward_stack(const dlo_plan *plan, const dlo_host_store *store,
                      const dlo_forward_args *a, dlo_run **run_out) {
  if (run_out) *run_out = nullptr;
  int rc = validate_forward(plan, store, a);
  if (rc) return rc;
  if ((a->flags & DLO_ASYNC_ENQUEUE) && !run_out)
    return fail(DLO_E_ARG, "DLO_ASYNC_ENQUEUE needs run_out (the run must be joined by dlo_run_enqueued)");
  std::lock_guard<std::mutex> lk(plan->mu);
  if (plan->enqueuing)
    return fail(DLO_E_STATE, "a DLO_ASYNC_ENQUEUE run of this plan is still being enqueued (dlo_run_enqueued first)");
  reap_detached(plan, false);

  const int n = (int)plan->blocks.size();
  const int n_res = (a->flags & DLO_RESIDENT) ? n : a->n_resident;
  const bool resident = n_res == n;  // nothing streams
  const std::vector<Step> steps = hook_steps(n, a->passes, n_res);
  const std::vector<dlo_sched_op> prog = build_program(steps, resident);

  dlo_run *run = new (std::nothrow) dlo_run;
  if (!run) return fail(DLO_E_HOSTMEM, "out of host memory");
  run->timing = a->flags & DLO_TRACE_TIMING;
  run->digest = a->flags & DLO_TRACE_DIGEST;
  const int64_t total = (int64_t)steps.size();
  constexpr int TEV = 4 + DLO_KERNELS_PER_BLOCK;  // copy begin, copy end, compute begin, kernels, compute end

  // --- resources (events, digest buffer): failures here have enqueued nothing
  (void)hipGetDevice(&run->device);
  rc = DLO_OK;
  for (auto &e : run->ev)
    if (!rc) rc = check_hip(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreate");
  if (!rc) rc = check_hip(hipEventCreateWithFlags(&run->final_ev, hipEventDisableTiming), "hipEventCreate");
  if (!rc && !plan->last_done)
    rc = check_hip(hipEventCreateWithFlags(&plan->last_done, hipEventDisableTiming), "hipEventCreate");
  if (!rc && run->timing) {
    run->kmask.assign((size_t)total, 0u);
    run->tev.assign((size_t)(total * TEV + 1), nullptr);
    for (auto &e : run->tev)
      if (!rc) rc = check_hip(hipEventCreate(&e), "hipEventCreate");
  }
  if (!rc && run->digest)
    rc = check_hip(hipMalloc(&run->d_digest, (size_t)(2 * total) * sizeof(uint64_t)), "hipMalloc");
  if (rc) {
    run_free(run);
    return rc;
  }

  run->recs.resize((size_t)total);
  for (const Step &s : steps) {
    dlo_slot_event &r = run->recs[(size_t)s.t];
    std::memset(&r, 0, sizeof r);
    r.step = s.t;
    r.pass = s.pass;
    r.block = s.block;
    r.read_slot = s.slot;
    r.prefetch_block = s.next_block;
    r.prefetch_slot = s.next_slot;
    r.prefetch_bytes = s.next_block < 0 ? 0 : plan->blocks[s.next_block].copy_bytes;
    r.t_copy_begin = r.t_copy_end = r.t_compute_begin = r.t_compute_end = -1.f;
  }

  if (a->flags & DLO_ASYNC_ENQUEUE) {
    // the caller's arguments outlive the call in the run; the thread takes the
    // calling thread's device and releases the plan when it has enqueued all
    run->args = *a;
    if (n_res > 0 && a->resident_blocks) {
      run->res_blocks.assign(a->resident_blocks, a->resident_blocks + n_res);
      run->args.resident_blocks = run->res_blocks.data();
    }
    dlo_host_store *st = const_cast<dlo_host_store *>(store);
    try {
      run->worker = std::thread([plan, st, run, prog, resident]() {
        int rc = check_hip(hipSetDevice(run->device), "hipSetDevice");
        if (!rc && !resident) rc = wait_previous_run(plan);
        if (!rc) rc = enqueue_program(plan, st, &run->args, run, prog, resident);
        if (rc) run->enqueue_msg = dlo_last_error();
        run->enqueue_rc = rc;
      });
    } catch (...) {
      run_free(run);   // nothing enqueued
      return fail(DLO_E_HOSTMEM, "could not start the enqueue thread");
    }
    run->plan = plan;
    plan->enqueuing = run;
    if (st && !resident) {
      std::lock_guard<std::mutex> slk(st->mu);
      run->store = st;
      st->enqueuing = run;
    }
    *run_out = run;
    return ok();
  }
  rc = resident ? DLO_OK : wait_previous_run(plan);
  if (rc) {
    run_free(run);   // nothing enqueued
    return rc;
  }
  rc = enqueue_program(plan, const_cast<dlo_host_store *>(store), a, run, prog, resident);
  if (rc) {
    // work may already be enqueued: keep the run until it drains
    plan->detached.push_back(run);
    return rc;
  }
  if (run_out)
    *run_out = run;
  else
    plan->detached.push_back(run);
  return ok();
}

int dlo_run_enqueued(dlo_run *run) {
  if (!run) return fail(DLO_E_ARG, "NULL run");
  finish_enqueue(run);
  if (run->enqueue_rc) return fail(run->enqueue_rc, "%s", run->enqueue_msg.c_str());
  return ok();
}

int dlo_slot_trace(dlo_run *run, dlo_slot_event *out, int64_t cap, int64_t *n_out) {
  if (!run || !n_out) return fail(DLO_E_ARG, "NULL argument");
  finish_enqueue(run);
  if (run->enqueue_rc) return fail(run->enqueue_rc, "%s", run->enqueue_msg.c_str());
  const int64_t total = (int64_t)run->recs.size();
  *n_out = total;
  if (!run->finished) {
    int rc = check_hip(hipEventSynchronize(run->final_ev), "hipEventSynchronize");
    if (rc) return rc;
    if (run->digest) {
      std::vector<uint64_t> dg((size_t)(2 * total));
      rc = check_hip(hipMemcpy(dg.data(), run->d_digest, dg.size() * sizeof(uint64_t),
                               hipMemcpyDeviceToHost), "hipMemcpy");
      if (rc) return rc;
      for (int64_t t = 0; t < total; ++t) {
        run->recs[(size_t)t].digest_pre = dg[(size_t)(2 * t)];
        run->recs[(size_t)t].digest_post = dg[(size_t)(2 * t + 1)];
      }
    }
    if (run->timing) {
      constexpr int TEV = 4 + DLO_KERNELS_PER_BLOCK;
      hipEvent_t t0 = run->tev.back();
      auto since = [&](hipEvent_t ev) {
        float ms = -1.f;
        if (hipEventElapsedTime(&ms, t0, ev) != hipSuccess) ms = -1.f;
        return ms;
      };
      run->kernel_ms.assign((size_t)(total * DLO_KERNELS_PER_BLOCK), -1.f);
      for (int64_t t = 0; t < total; ++t) {
        dlo_slot_event &r = run->recs[(size_t)t];
        auto ev = [&](int j) { return run->tev[(size_t)(t * TEV + j)]; };
        if (r.read_slot >= 0) {  // a streamed step: the copy that fed it
          r.t_copy_begin = since(ev(0));
          r.t_copy_end = since(ev(1));
        }
        r.t_compute_begin = since(ev(2));
        r.t_compute_end = since(ev(3 + DLO_KERNELS_PER_BLOCK));
        float prev = r.t_compute_begin;
        for (int j = 0; j < DLO_KERNELS_PER_BLOCK; ++j) {
          float dt = 0.f;   // an empty slot recorded no event
          if (run->kmask[(size_t)t] >> j & 1u) {
            const float tj = since(ev(3 + j));
            dt = tj - prev;
            prev = tj;
          }
          run->kernel_ms[(size_t)(t * DLO_KERNELS_PER_BLOCK + j)] = dt;
        }
      }
    }
    run->finished = true;
  }
  if (out) std::memcpy(out, run->recs.data(), (size_t)std::min(cap, total) * sizeof(dlo_slot_event));
  return ok();
}

int dlo_run_kernel_times(dlo_run *run, float *ms, int64_t cap, int64_t *n_out) {
  if (!run || !n_out) return fail(DLO_E_ARG, "NULL argument");
  if (!run->timing) return fail(DLO_E_STATE, "the run was not started with DLO_TRACE_TIMING");
  int64_t n_steps = 0;
  int rc = dlo_slot_trace(run, nullptr, 0, &n_steps);
  if (rc) return rc;
  *n_out = (int64_t)run->kernel_ms.size();
  if (ms) std::memcpy(ms, run->kernel_ms.data(), (size_t)std::min(cap, *n_out) * sizeof(float));
  return ok();
}

void dlo_run_destroy(dlo_run *run) { run_free(run); }

// --------------------------------------------------------------------------- single ops

int dlo_op_adaln(const uint16_t *W, const float *b, const float *cond, int32_t rows, int32_t d,
                 float *out, void *workspace, int64_t workspace_bytes, void *stream) {
  if (!W || !b || !cond || !out || !workspace) return fail(DLO_E_ARG, "NULL argument");
  if (rows < 1 || d < 8 || d % 8) return fail(DLO_E_UNSUPPORTED, "adaln: rows >= 1, d % 8 == 0 required");
  if (workspace_bytes < 4 * (int64_t)d) return fail(DLO_E_WORKSPACE, "adaln: workspace < 4 d bytes");
  hipStream_t s = (hipStream_t)stream;
  float *sc = static_cast<float *>(workspace);
  int rc = check_hip(dlo::launch_silu(cond, sc, d, s), "silu");
  if (!rc) rc = check_hip(dlo::launch_adaln_gemv(W, sc, b, out, rows, d, s), "adaln_gemv");
  return rc ? rc : ok();
}

int dlo_op_adaln_noalloc(const uint16_t *W, const float *b, const float *cond, int32_t rows, int32_t d,
                         float *out, void *stream) {
  if (!W || !b || !cond || !out) return fail(DLO_E_ARG, "NULL argument");
  if (rows < 1 || d < 8 || d % 8) return fail(DLO_E_UNSUPPORTED, "adaln_noalloc: rows >= 1, d %% 8 == 0 required");
  if (d > DLO_NOALLOC_MAX_D)
    return fail(DLO_E_UNSUPPORTED, "adaln_noalloc: d = %d exceeds the static scratch (%d floats)", d,
                DLO_NOALLOC_MAX_D);
  int rc = check_hip(dlo::launch_adaln_noalloc(W, b, cond, rows, d, out, (hipStream_t)stream), "adaln_noalloc");
  return rc ? rc : ok();
}

int dlo_op_adaln_fp8(const uint8_t *W, const float *w_scale, const float *b, const float *cond, int32_t rows,
                     int32_t d, float *out, void *workspace, int64_t workspace_bytes, void *stream) {
  if (!W || !w_scale || !b || !cond || !out || !workspace) return fail(DLO_E_ARG, "NULL argument");
  if (rows < 1 || d < 16 || d % 16) return fail(DLO_E_UNSUPPORTED, "adaln_fp8: rows >= 1, d %% 16 == 0 required");
  if ((uintptr_t)W % 16 || (uintptr_t)cond % 16)
    return fail(DLO_E_UNSUPPORTED, "adaln_fp8: W and cond must be 16-B aligned");
  if (workspace_bytes < 4 * (int64_t)d) return fail(DLO_E_WORKSPACE, "adaln_fp8: workspace < 4 d bytes");
  hipStream_t s = (hipStream_t)stream;
  float *sc = static_cast<float *>(workspace);
  int rc = check_hip(dlo::launch_silu(cond, sc, d, s), "silu");
  if (!rc) rc = check_hip(dlo::launch_adaln_gemv_fp8(W, w_scale, sc, b, out, rows, d, s), "adaln_gemv_fp8");
  return rc ? rc : ok();
}

int dlo_op_ln_modulate(const float *x, int64_t ldx, int32_t T, int32_t d, const float *gamma,
                       const float *beta, const float *eps, const float *shift,
                       const float *scale, uint16_t *out, void *stream) {
  if (!x || !gamma || !beta || !eps || !shift || !scale || !out) return fail(DLO_E_ARG, "NULL argument");
  if (T < 1 || d < 256 || d % 256 || d > 8192 || ldx < d)
    return fail(DLO_E_UNSUPPORTED, "ln_modulate: d %% 256 == 0, d <= 8192, ldx >= d required");
  if ((uintptr_t)x % 16 || ldx % 4 || (uintptr_t)out % 8)
    return fail(DLO_E_UNSUPPORTED, "ln_modulate: x 16-B aligned with ldx %% 4 == 0, out 8-B aligned required");
  int rc = check_hip(dlo::launch_ln_modulate(x, ldx, T, d, gamma, beta, eps, shift, scale, out,
                                             (hipStream_t)stream), "ln_modulate");
  return rc ? rc : ok();
}

int dlo_op_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int32_t M,
                int32_t N, int32_t K, const float *bias, const float *gate, void *C, int64_t ldc,
                int32_t epilogue, void *stream) {
  if (!A || !B || !bias || !C) return fail(DLO_E_ARG, "NULL argument");
  if (epilogue < 0 || epilogue > 3) return fail(DLO_E_ARG, "unknown epilogue %d", epilogue);
  if (epilogue == DLO_EPI_GATED_RESIDUAL && !gate) return fail(DLO_E_ARG, "gate is required");
  const bool trans = epilogue == DLO_EPI_BIAS_T;
  if (M < 1 || N < 256 || N % 256 || K < 64 || K % 64 || lda < K || ldb < K ||
      ldc < (trans ? round_up64(M) : N) || lda % 8 || ldb % 8 || (trans && ldc % 8))
    return fail(DLO_E_UNSUPPORTED, "gemm: N %% 256 == 0, K %% 64 == 0, ld >= extent, ld %% 8 == 0");
  if ((int64_t)256 * lda * 2 >= (int64_t)1 << 31 || (int64_t)256 * ldb * 2 >= (int64_t)1 << 31 ||
      (int64_t)256 * ldc * 4 >= (int64_t)1 << 31)
    return fail(DLO_E_UNSUPPORTED, "gemm: leading dimension too large for 32-bit tile offsets");
  if (ldc % 4 || (uintptr_t)C % 16 || (uintptr_t)bias % 4 || (gate && (uintptr_t)gate % 4))
    return fail(DLO_E_UNSUPPORTED, "gemm: C 16-B, bias and gate 4-B aligned, ldc %% 4 == 0");
  int rc = check_hip(dlo::launch_gemm(A, lda, B, ldb, M, N, K, bias, gate, C, ldc, epilogue,
                                      (hipStream_t)stream), "gemm");
  return rc ? rc : ok();
}

int dlo_op_quantize_rows_fp8(const uint16_t *x, int64_t ldx, int32_t M, int32_t K, uint8_t *codes,
                             int64_t ldq, float *scales, void *stream) {
  if (!x || !codes || !scales) return fail(DLO_E_ARG, "NULL argument");
  if (M < 1 || K < 8 || K % 8 || ldx < K || ldq < K || ldx % 8 || ldq % 8)
    return fail(DLO_E_UNSUPPORTED, "quantize_rows_fp8: K %% 8 == 0, ldx and ldq >= K and multiples of 8");
  if ((uintptr_t)x % 16 || (uintptr_t)codes % 8 || (uintptr_t)scales % 4)
    return fail(DLO_E_UNSUPPORTED, "quantize_rows_fp8: x 16-B, codes 8-B and scales 4-B aligned");
  int rc = check_hip(dlo::launch_quant_rows_fp8(x, ldx, M, K, codes, ldq, scales, (hipStream_t)stream),
                     "quantize_rows_fp8");
  return rc ? rc : ok();
}

int dlo_op_gemm_fp8(const uint8_t *A, int64_t lda, const float *a_scale, const uint8_t *B, int64_t ldb,
                    const float *b_scale, int32_t M, int32_t N, int32_t K, const float *bias,
                    const float *gate, void *C, int64_t ldc, int32_t epilogue, void *stream) {
  if (!A || !a_scale || !B || !b_scale || !bias || !C) return fail(DLO_E_ARG, "NULL argument");
  if (epilogue < 0 || epilogue > 3) return fail(DLO_E_ARG, "unknown epilogue %d", epilogue);
  if (epilogue == DLO_EPI_GATED_RESIDUAL && !gate) return fail(DLO_E_ARG, "gate is required");
  const bool trans = epilogue == DLO_EPI_BIAS_T;
  if (M < 1 || N < 256 || N % 256 || K < 64 || K % 64 || lda < K || ldb < K ||
      ldc < (trans ? round_up64(M) : N) || lda % 16 || ldb % 16 || (trans && ldc % 8))
    return fail(DLO_E_UNSUPPORTED,
                "gemm_fp8: N %% 256 == 0, K %% 64 == 0, ld >= extent, lda and ldb multiples of 16");
  if ((int64_t)256 * lda >= (int64_t)1 << 31 || (int64_t)256 * ldb >= (int64_t)1 << 31 ||
      (int64_t)256 * ldc * 4 >= (int64_t)1 << 31)
    return fail(DLO_E_UNSUPPORTED, "gemm_fp8: leading dimension too large for 32-bit tile offsets");
  if (ldc % 4 || (uintptr_t)C % 16 || (uintptr_t)bias % 4 || (gate && (uintptr_t)gate % 4) ||
      (uintptr_t)A % 16 || (uintptr_t)B % 16)
    return fail(DLO_E_UNSUPPORTED, "gemm_fp8: A, B and C 16-B, bias and gate 4-B aligned, ldc %% 4 == 0");
  int rc = check_hip(dlo::launch_gemm_fp8(A, lda, a_scale, B, ldb, b_scale, M, N, K, bias, gate, C, ldc,
                                          epilogue, (hipStream_t)stream), "gemm_fp8");
  return rc ? rc : ok();
}

int dlo_op_quantize_rows_int8(const uint16_t *x, int64_t ldx, int32_t M, int32_t K, int8_t *codes,
                              int64_t ldq, float *scales, void *stream) {
  if (!x || !codes || !scales) return fail(DLO_E_ARG, "NULL argument");
  if (M < 1 || K < 8 || K % 8 || ldx < K || ldq < K || ldx % 8 || ldq % 8)
    return fail(DLO_E_UNSUPPORTED, "quantize_rows_int8: K %% 8 == 0, ldx and ldq >= K and multiples of 8");
  if ((uintptr_t)x % 16 || (uintptr_t)codes % 8 || (uintptr_t)scales % 4)
    return fail(DLO_E_UNSUPPORTED, "quantize_rows_int8: x 16-B, codes 8-B and scales 4-B aligned");
  int rc = check_hip(dlo::launch_quant_rows_int8(x, ldx, M, K, codes, ldq, scales, (hipStream_t)stream),
                     "quantize_rows_int8");
  return rc ? rc : ok();
}

int dlo_op_gemm_int8(const int8_t *A, int64_t lda, const float *a_scale, const int8_t *B, int64_t ldb,
                     const float *b_scale, int32_t M, int32_t N, int32_t K, const float *bias,
                     const float *gate, void *C, int64_t ldc, int32_t epilogue, void *stream) {
  if (!A || !a_scale || !B || !b_scale || !bias || !C) return fail(DLO_E_ARG, "NULL argument");
  if (epilogue < 0 || epilogue > 3) return fail(DLO_E_ARG, "unknown epilogue %d", epilogue);
  if (epilogue == DLO_EPI_GATED_RESIDUAL && !gate) return fail(DLO_E_ARG, "gate is required");
  const bool trans = epilogue == DLO_EPI_BIAS_T;
  if (M < 1 || N < 256 || N % 256 || K < 64 || K % 64 || lda < K || ldb < K ||
      ldc < (trans ? round_up64(M) : N) || lda % 16 || ldb % 16 || (trans && ldc % 8))
    return fail(DLO_E_UNSUPPORTED,
                "gemm_int8: N %% 256 == 0, K %% 64 == 0, ld >= extent, lda and ldb multiples of 16");
  if ((int64_t)256 * lda >= (int64_t)1 << 31 || (int64_t)256 * ldb >= (int64_t)1 << 31 ||
      (int64_t)256 * ldc * 4 >= (int64_t)1 << 31)
    return fail(DLO_E_UNSUPPORTED, "gemm_int8: leading dimension too large for 32-bit tile offsets");
  if (ldc % 4 || (uintptr_t)C % 16 || (uintptr_t)bias % 4 || (gate && (uintptr_t)gate % 4) ||
      (uintptr_t)A % 16 || (uintptr_t)B % 16 || (uintptr_t)a_scale % 4 || (uintptr_t)b_scale % 4)
    return fail(DLO_E_UNSUPPORTED, "gemm_int8: A, B and C 16-B, bias, gate and scales 4-B aligned, ldc %% 4 == 0");
  int rc = check_hip(dlo::launch_gemm_int8(A, lda, a_scale, B, ldb, b_scale, M, N, K, bias, gate, C, ldc,
                                           epilogue, (hipStream_t)stream), "gemm_int8");
  return rc ? rc : ok();
}

int dlo_op_v_transpose(const uint16_t *qkv, int64_t ldqkv, int32_t T, int32_t d, uint16_t *vt,
                       int64_t ldvt, void *stream) {
  if (!qkv || !vt) return fail(DLO_E_ARG, "NULL argument");
  if (T < 1 || d < 64 || d % 64 || ldqkv < 3LL * d || ldqkv % 8 || ldvt % 8 || ldvt < round_up64(T))
    return fail(DLO_E_UNSUPPORTED,
                "v_transpose: d %% 64 == 0, ldqkv >= 3 d and ldvt >= T rounded up to 64 (multiples of 8)");
  if ((uintptr_t)qkv % 16 || (uintptr_t)vt % 16)
    return fail(DLO_E_UNSUPPORTED, "v_transpose: qkv and vt must be 16-B aligned");
  int rc = check_hip(dlo::launch_v_transpose(qkv + 2 * (int64_t)d, ldqkv, T, d, vt, ldvt,
                                             (hipStream_t)stream), "v_transpose");
  return rc ? rc : ok();
}

int dlo_op_attention(const uint16_t *qkv, int64_t ldqkv, const uint16_t *vt, int64_t ldvt, int32_t T,
                     int32_t H, int32_t dh, uint16_t *out, int64_t ldo, void *stream) {
  if (!qkv || !vt || !out) return fail(DLO_E_ARG, "NULL argument");
  if (T < 1 || H < 1 || (dh != 64 && dh != 128) || ldqkv < 2LL * H * dh || ldo < (int64_t)H * dh ||
      ldqkv % 8 || ldo % 4 || ldvt % 8 || ldvt < round_up64(T))
    return fail(DLO_E_UNSUPPORTED,
                "attention: dh in {64,128}, ldqkv >= 2 H dh, ldvt >= T rounded up to 64 (multiples of 8)");
  if (((int64_t)T + 64) * ldqkv * 2 >= ((int64_t)1 << 31) || (int64_t)dh * ldvt * 2 >= ((int64_t)1 << 31))
    return fail(DLO_E_UNSUPPORTED, "attention: T * ldqkv too large for 32-bit buffer offsets");
  if ((uintptr_t)qkv % 16 || (uintptr_t)vt % 16)
    return fail(DLO_E_UNSUPPORTED, "attention: qkv and vt must be 16-B aligned");
  int rc = check_hip(dlo::launch_attention(qkv, ldqkv, vt, ldvt, T, H, dh, out, ldo,
                                           (hipStream_t)stream), "attention");
  return rc ? rc : ok();
}

int dlo_op_dequant_fp8(const uint8_t *codes, int64_t n, const float *scale, uint16_t *out,
                       void *stream) {
  if (!codes || !scale || !out) return fail(DLO_E_ARG, "NULL argument");
  if (n < 0 || n % 16 || (uintptr_t)codes % 16 || (uintptr_t)out % 32)
    return fail(DLO_E_UNSUPPORTED, "dequant: n %% 16 == 0, codes 16-B and out 32-B aligned required");
  int rc = check_hip(dlo::launch_dequant_fp8(codes, n, scale, out, (hipStream_t)stream), "dequant_fp8");
  return rc ? rc : ok();
}

int dlo_op_quantize_rows_mxfp8(const uint16_t *x, int64_t ldx, int32_t M, int32_t K, uint8_t *codes,
                               int64_t ldq, uint8_t *scales, int64_t lds, void *stream) {
  if (!x || !codes || !scales) return fail(DLO_E_ARG, "NULL argument");
  if (M < 1 || K < 32 || K % 32 || ldx < K || ldq < K || ldx % 8 || ldq % 8 || lds < M)
    return fail(DLO_E_UNSUPPORTED, "quantize_rows_mxfp8: K %% 32 == 0, ldx and ldq >= K and multiples of 8, lds >= M");
  if ((uintptr_t)x % 16 || (uintptr_t)codes % 8)
    return fail(DLO_E_UNSUPPORTED, "quantize_rows_mxfp8: x 16-B and codes 8-B aligned");
  int rc = check_hip(dlo::launch_quant_rows_mx(x, ldx, M, K, codes, ldq, scales, lds, (hipStream_t)stream),
                     "quantize_rows_mxfp8");
  return rc ? rc : ok();
}

int dlo_op_gemm_mxfp8(const uint8_t *A, int64_t lda, const uint8_t *a_scales, int64_t lds_a, const uint8_t *B,
                      int64_t ldb, const uint8_t *b_scales, int64_t lds_b, int32_t M, int32_t N, int32_t K,
                      const float *bias, const float *gate, void *C, int64_t ldc, int32_t epilogue, void *stream) {
  if (!A || !a_scales || !B || !b_scales || !bias || !C) return fail(DLO_E_ARG, "NULL argument");
  if (epilogue < 0 || epilogue > 3) return fail(DLO_E_ARG, "unknown epilogue %d", epilogue);
  if (epilogue == DLO_EPI_GATED_RESIDUAL && !gate) return fail(DLO_E_ARG, "gate is required");
  const bool trans = epilogue == DLO_EPI_BIAS_T;
  if (M < 1 || N < 256 || N % 256 || K < 64 || K % 64 || lda < K || ldb < K ||
      ldc < (trans ? round_up64(M) : N) || lda % 16 || ldb % 16 || (trans && ldc % 8) || lds_a < M ||
      lds_a % 4 || lds_b < N || lds_b % 4)
    return fail(DLO_E_UNSUPPORTED, "gemm_mxfp8: N %% 256 == 0, K %% 64 == 0, ld >= extent, lda and ldb "
                                   "multiples of 16, lds_a >= M and lds_b >= N multiples of 4");
  if ((int64_t)256 * lda >= (int64_t)1 << 31 || (int64_t)256 * ldb >= (int64_t)1 << 31 ||
      (int64_t)256 * ldc * 4 >= (int64_t)1 << 31 || (int64_t)(K / 32) * std::max(lds_a, lds_b) >= (int64_t)1 << 31)
    return fail(DLO_E_UNSUPPORTED, "gemm_mxfp8: leading dimension too large for 32-bit offsets");
  if (ldc % 4 || (uintptr_t)C % 16 || (uintptr_t)bias % 4 || (gate && (uintptr_t)gate % 4) ||
      (uintptr_t)A % 16 || (uintptr_t)B % 16 || (uintptr_t)a_scales % 4 || (uintptr_t)b_scales % 4)
    return fail(DLO_E_UNSUPPORTED, "gemm_mxfp8: A, B and C 16-B, bias, gate and scales 4-B aligned, ldc %% 4 == 0");
  int rc = check_hip(dlo::launch_gemm_mxfp8(A, lda, a_scales, lds_a, B, ldb, b_scales, lds_b, M, N, K, bias, gate,
                                            C, ldc, epilogue, (hipStream_t)stream), "gemm_mxfp8");
  return rc ? rc : ok();
}

int dlo_op_dequant_int8(const int8_t *codes, int64_t rows, int64_t cols, const float *scales, uint16_t *out,
                        void *stream) {
  if (!codes || !scales || !out) return fail(DLO_E_ARG, "NULL argument");
  if (rows < 0 || cols < 16 || cols % 16 || (uintptr_t)codes % 16 || (uintptr_t)out % 32)
    return fail(DLO_E_UNSUPPORTED, "dequant_int8: cols %% 16 == 0, codes 16-B and out 32-B aligned required");
  int rc = check_hip(dlo::launch_dequant_int8(codes, rows, cols, scales, out, (hipStream_t)stream), "dequant_int8");
  return rc ? rc : ok();
}

int dlo_op_dequant_mxfp8(const uint8_t *codes, int64_t rows, int64_t cols, const uint8_t *scales, uint16_t *out,
                         void *stream) {
  if (!codes || !scales || !out) return fail(DLO_E_ARG, "NULL argument");
  if (rows < 0 || cols < 32 || cols % 32 || (uintptr_t)codes % 16 || (uintptr_t)out % 32)
    return fail(DLO_E_UNSUPPORTED, "dequant_mxfp8: cols %% 32 == 0, codes 16-B and out 32-B aligned required");
  int rc = check_hip(dlo::launch_dequant_mxfp8(codes, rows, cols, scales, out, (hipStream_t)stream),
                     "dequant_mxfp8");
  return rc ? rc : ok();
}

int dlo_op_mfma_rate(int32_t form, const uint16_t *in, float *out, int32_t iters, double *flops, void *stream) {
  if (!in || !out) return fail(DLO_E_ARG, "NULL argument");
  if ((form != 0 && form != 1) || iters < 1) return fail(DLO_E_ARG, "mfma_rate: form 0 or 1, iters >= 1");
  if ((uintptr_t)in % 16 || (uintptr_t)out % 4) return fail(DLO_E_UNSUPPORTED, "mfma_rate: in 16-B, out 4-B aligned");
  if (flops) *flops = (double)dlo::MFMA_RATE_GRID * 8 * iters * 262144.0;
  int rc = check_hip(dlo::launch_mfma_rate(form, in, out, iters, (hipStream_t)stream), "mfma_rate");
  return rc ? rc : ok();
}

int dlo_op_digest(const void *base, const int64_t *offsets, const int64_t *lengths,
                  int32_t n_regions, uint64_t *out, void *stream) {
  if (!base || !offsets || !lengths || !out) return fail(DLO_E_ARG, "NULL argument");
  if (n_regions < 0 || n_regions > DLO_MAX_GROUPS) return fail(DLO_E_ARG, "n_regions out of range");
  for (int i = 0; i < n_regions; ++i)
    if (offsets[i] < 0 || offsets[i] % 8 || lengths[i] < 0) return fail(DLO_E_ARG, "bad region");
  int rc = check_hip(dlo::launch_digest(base, offsets, lengths, n_regions, out, (hipStream_t)stream),
                     "digest");
  return rc ? rc : ok();
}

}  // extern "C"
