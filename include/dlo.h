/*
 * dlo.h -- C ABI of libdlo: double-buffered, layerwise weight streaming of a
 * DiT block stack on one AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title):
 *   [Jul] "Distributed Layerwise Offload", vLLM-Omni project blog, 2026-07-30.
 *   [Aug] "Distributed Layerwise Offload: Scaling Toward 200B+ DiT Models
 *         Efficiently in vLLM-Omni", vLLM blog, 2026-08-17.
 *   [Doc] "Distributed Layerwise Offload", vLLM-Omni design documentation.
 *
 * What the library does, end to end:
 *   1. dlo_plan_blocks      -- per block, flatten parameters by dtype, split each
 *                              flat buffer into k equal zero-padded shards, and lay
 *                              the block out in a slot at the offsets an all-gather
 *                              of those shards would produce ([Aug] s.2).
 *   2. dlo_pack_host_shards -- copy parameters into the shards, held in pinned host
 *                              memory ([Jul] "Weight Sharding + AllGather").
 *   3. dlo_forward_stack    -- stream the blocks through exactly two device slots:
 *                              a copy stream places block N+1's k shards into the
 *                              free slot while the compute stream runs block N from
 *                              the other, parameters re-pointed into the slot with
 *                              no copy, compute waiting on the copy event
 *                              ([Jul] "How It Works", [Aug] s.3, [Doc] "AllGather
 *                              path").  One GPU: the shards are assembled locally,
 *                              no collective is issued.
 *   4. dlo_slot_trace       -- the per-step slot record of a run (which block read
 *                              which slot, what was prefetched where), with
 *                              optional slot digests and timestamps ([Jul] "Slot
 *                              Tracking: i%2 + Dynamic Correction").
 *
 * Conventions for every entry point:
 *   - Status codes: DLO_OK (0) or a negative dlo_status.  On any error nothing is
 *     enqueued on any stream, output handles are set to NULL, and
 *     dlo_last_error() returns a message (fail closed, [Jul] "Fail-Closed
 *     Design").  The one exception is DLO_E_HIP during dlo_forward_stack: a HIP
 *     call failed after work was enqueued; the caller must synchronise both
 *     streams and treat x as undefined.
 *   - "device pointer" = memory from hipMalloc (e.g. a PyTorch tensor on the GPU);
 *     "host pointer" = ordinary or pinned CPU memory.  Streams are hipStream_t
 *     values passed as void*.
 *   - Caller-owned memory (slots, x, cond, workspace, streams, parameter sources)
 *     is never freed or retained by the library beyond the documented lifetime.
 *   - A plan and its stores may be used from one host thread at a time.
 */
#ifndef DLO_H
#define DLO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DLO_OK = 0,
  DLO_E_ARG = -1,           /* invalid argument (null pointer, bad size, bad index) */
  DLO_E_HOSTMEM = -2,       /* ordinary host allocation failed */
  DLO_E_PIN = -3,           /* pinned host allocation failed */
  DLO_E_SLOT_SMALL = -4,    /* a slot buffer is smaller than the plan's slot size */
  DLO_E_PLAN_MISMATCH = -5, /* store / parameter list does not belong to this plan */
  DLO_E_HIP = -6,           /* a HIP runtime call failed */
  DLO_E_STATE = -7,         /* object in the wrong state (e.g. store not packed) */
  DLO_E_UNSUPPORTED = -8,   /* valid but unsupported (block schema, head dim, width) */
  DLO_E_WORKSPACE = -9      /* workspace smaller than dlo_plan_workspace_bytes */
} dlo_status;

/* element types of parameter groups */
enum {
  DLO_BF16 = 0,
  DLO_F32 = 1,
  DLO_FP8_E4M3 = 2, /* OCP FP8 E4M3, 1 byte */
  DLO_I8 = 3,       /* int8, 1 byte */
  DLO_E8M0 = 4      /* OCP MX E8M0 block scale 2^(b - 127), 1 byte (255: NaN) */
};

#define DLO_MAX_GROUPS 3   /* one group per element type */
#define DLO_ALIGN 256      /* byte alignment of regions and extents inside a slot */

/* One parameter, in the block's registration order.  `src` is a host pointer to
 * numel elements of `dtype` (read by dlo_pack_host_shards only; may be NULL for
 * dlo_plan_blocks).  `name` is copied by the plan. */
typedef struct {
  const char *name;
  int32_t dtype;
  int64_t numel;
  const void *src;
} dlo_param;

/* One block: its width d_model (the residual columns it reads and updates), its
 * attention heads, and its parameters in registration order. */
typedef struct {
  int32_t d_model;
  int32_t n_heads;
  int32_t n_params;
  const dlo_param *params;
} dlo_block;

typedef struct dlo_plan dlo_plan;
typedef struct dlo_host_store dlo_host_store;
typedef struct dlo_run dlo_run;

/* ---------------------------------------------------------------------------
 * Plan ([Aug] s.2 "Weight Sharding with AllGather Reconstruction"; [Jul]
 * "Double-Buffer Memory Bound")
 *
 * For block b and dtype group g (groups in order of first appearance):
 *   N_g = total elements, S_g = ceil(N_g / k) (equal shards, zero padded),
 *   region_g = byte offset of the group in a slot: region_0 = 0,
 *   region_{g+1} = align256(region_g + k * S_g * elt_g);
 *   extent = align256(end of the last region);
 *   parameter p lives at region_{g(p)} + (elements before p in its group) * elt.
 * slot_bytes = max extent over the blocks: the two device slots are each this
 * large whatever the block count.
 * ------------------------------------------------------------------------- */

/* Plans n_blocks blocks for k shards.  k >= 1, n_blocks >= 1, every dtype known
 * (DLO_BF16: groups of 2 bytes per element, DLO_F32: 4, DLO_FP8_E4M3, DLO_I8 and
 * DLO_E8M0: 1),
 * numel >= 0.  The plan copies names and sizes and never keeps `src`.  *out is
 * set to a new plan (free with dlo_plan_destroy) or NULL on error. */
int dlo_plan_blocks(const dlo_block *blocks, int32_t n_blocks, int32_t k, dlo_plan **out);
void dlo_plan_destroy(dlo_plan *plan);   /* waits for runs started without a handle */

int32_t dlo_plan_n_blocks(const dlo_plan *plan);
int32_t dlo_plan_k(const dlo_plan *plan);
int64_t dlo_plan_slot_bytes(const dlo_plan *plan);   /* -1 if plan is NULL */

typedef struct {
  int32_t d_model, n_heads, n_params, n_groups;
  int32_t dtype[DLO_MAX_GROUPS];
  int64_t numel[DLO_MAX_GROUPS];   /* N_g */
  int64_t shard[DLO_MAX_GROUPS];   /* S_g, elements per shard */
  int64_t region[DLO_MAX_GROUPS];  /* byte offset of the group in the slot */
  int64_t extent;                  /* bytes of the slot the block occupies */
  int64_t copy_bytes;              /* sum_g k * S_g * elt_g: bytes moved per placement */
  int32_t is_dit;                  /* 1: the DiT block schema (bf16 weights); 2, 3, 4: its
                                      FP8, INT8 and MXFP8 forms (dlo_block_schema_fp8,
                                      _int8, _mxfp8); 0: none of these */
} dlo_block_info;

int dlo_plan_block_info(const dlo_plan *plan, int32_t b, dlo_block_info *out);

/* Byte offset of parameter p of block b inside a slot (the zero-copy re-point). */
int dlo_plan_param_offset(const dlo_plan *plan, int32_t b, int32_t p, int64_t *byte_offset);

/* Device workspace needed by dlo_forward_stack for `tokens` rows (batch 1):
 * activations of one block at the widest d, plus, when the plan holds quantised
 * blocks, the bf16 weights their forward dequantises into (an FP8 block's four
 * linears, 12 d^2 elements; an INT8 or MXFP8 block's five, 18 d^2) and the
 * 1-byte codes (tokens x 4 d) and scales of a W8A8 linear's input
 * (DLO_FP8_COMPUTE: fp32 per row for FP8 and INT8, E8M0 [4 d / 32, tokens
 * rounded up to 64] for MXFP8); -1 on error. */
int64_t dlo_plan_workspace_bytes(const dlo_plan *plan, int32_t tokens);

/* ---------------------------------------------------------------------------
 * Host store ([Aug] s.2: each shard is a pinned DMA buffer)
 * ------------------------------------------------------------------------- */

#define DLO_STORE_PINNED 0u     /* every shard in hipHostMalloc'd memory (the default) */
#define DLO_STORE_PAGEABLE 1u   /* every shard in ordinary host memory (no GPU needed) */
#define DLO_STORE_AUTO 2u       /* pin blocks while the pinned ceiling allows, rest pageable */

/* Allocates every shard of every block of the plan.  Shards start on 4096-byte
 * boundaries; their bytes are undefined until packed.  Fails with DLO_E_PIN /
 * DLO_E_HOSTMEM after freeing whatever it had allocated.
 *
 * Blocks held in ordinary (pageable) memory reach the GPU through two bounded
 * pinned staging buffers of one slot each ([Doc] "Rank-local path without DLO
 * AllGather": complete blocks from host views through two bounded pinned host
 * staging slots): the host copies the block's shards into a staging buffer at
 * their slot offsets, then the DMA engine copies them into the slot.  The
 * staging buffers are allocated on the first forward that needs them (GPU
 * required then). */
int dlo_host_store_create(const dlo_plan *plan, uint32_t flags, dlo_host_store **out);

/* As dlo_host_store_create; with DLO_STORE_AUTO, `pinned_limit_bytes` (> 0) caps
 * the pinned bytes of block shards (the two staging buffers are reserved first and
 * not counted) -- the analogue of a per-worker registration ceiling ([Doc]
 * "Registered mmap transport").  Blocks are pinned in order until the next one
 * would cross the ceiling or the pinned allocation fails; the rest are pageable.
 * pinned_limit_bytes = 0 means no ceiling. */
int dlo_host_store_create_ex(const dlo_plan *plan, uint32_t flags, int64_t pinned_limit_bytes,
                             dlo_host_store **out);

/* Number of blocks whose shards are pinned, their bytes, and the number staged. */
int dlo_host_store_info(const dlo_host_store *store, int32_t *pinned_blocks,
                        int64_t *pinned_bytes, int32_t *staged_blocks);

/* Destroys the store once nothing reads it: a DLO_ASYNC_ENQUEUE run still
 * being enqueued from it is joined first, then the call waits for the last copy
 * placed from it (every placement records an event on its copy stream; runs of
 * one plan are ordered, so that copy is the last of all). */
void dlo_host_store_destroy(dlo_host_store *store);

/* Packs blocks [b_begin, b_end): blocks[i] describes block b_begin + i and must
 * list the same parameters (name, dtype, numel, order) as the plan
 * (DLO_E_PLAN_MISMATCH otherwise), with non-NULL host `src` pointers.  Shard r of
 * group g receives flat_g[r*S_g, (r+1)*S_g), zero beyond N_g ([Aug] s.2).
 * Host-only; the sources may be freed afterwards. */
int dlo_pack_host_shards(dlo_host_store *store, int32_t b_begin, int32_t b_end,
                         const dlo_block *blocks);

/* Host pointer to shard r of group g of block b, and its size in bytes
 * (S_g * elt_g).  The memory belongs to the store. */
int dlo_host_store_shard(const dlo_host_store *store, int32_t b, int32_t g, int32_t r,
                         const void **ptr, int64_t *bytes);

/* 1 if every block has been packed, else 0. */
int32_t dlo_host_store_complete(const dlo_host_store *store);

/* ---------------------------------------------------------------------------
 * Schedule (host-only view of what dlo_forward_stack enqueues)
 *
 * Hook rule ([Jul] "Slot Tracking"): hook i starts at slot i % 2; when the
 * previous hook (block i-1 mod n) has a prefetched slot, hook i uses it; hook i
 * prefetches block (i+1) mod n into the other slot.  Block 0 is placed in slot 0
 * before step 0; the last step prefetches nothing.
 *
 * Program per run: RECORD(compute, START), WAIT(copy, START),
 * COPY(block 0 -> slot 0), RECORD(copy, COPIED[0]); then for step t (pass p,
 * block i, read slot s):
 *   WAIT(compute, COPIED[s]), COMPUTE(block i, slot s), RECORD(compute, COMPUTED[s])
 *   if t is not the last step:  [t >= 1: WAIT(copy, COMPUTED[s'])]
 *                               COPY(next block -> s'), RECORD(copy, COPIED[s'])
 * where s' = 1 - s: the copy into s' waits for step t-1, the last reader of s'.
 * COPY places the k shards of every dtype group at slot + region_g + r * S_g * elt_g
 * with hipMemcpyAsync, one call per run of shards whose host bytes are adjacent
 * (at most k calls per group).
 * ------------------------------------------------------------------------- */

enum { DLO_OP_COPY = 0, DLO_OP_COMPUTE = 1, DLO_OP_RECORD = 2, DLO_OP_WAIT = 3 };
enum { DLO_STREAM_COMPUTE = 0, DLO_STREAM_COPY = 1 };
enum { DLO_EV_COPIED0 = 0, DLO_EV_COPIED1 = 1, DLO_EV_COMPUTED0 = 2, DLO_EV_COMPUTED1 = 3,
       DLO_EV_START = 4 };

typedef struct {
  int32_t kind;     /* DLO_OP_* */
  int32_t stream;   /* DLO_STREAM_* */
  int32_t block;    /* COPY / COMPUTE: block index; else -1 */
  int32_t slot;     /* COPY / COMPUTE: slot; else -1 */
  int32_t event;    /* RECORD / WAIT: DLO_EV_*; else -1 */
  int32_t pad;
  int64_t step;     /* COMPUTE: step t; COPY: the step that will read it; else -1 */
} dlo_sched_op;

/* Writes the program for `passes` passes (passes >= 1).  If ops is NULL or cap is
 * too small, only *n_ops is set (and DLO_OK is returned when ops is NULL). */
int dlo_plan_schedule(const dlo_plan *plan, int32_t passes, dlo_sched_op *ops, int64_t cap,
                      int64_t *n_ops);

/* As dlo_plan_schedule with the first n_resident blocks resident (0 <= n_resident
 * <= n, else DLO_E_ARG): their steps are a lone COMPUTE(block, slot -1) each, with
 * no waits or copies.  The other blocks follow the hook rule among themselves:
 * the first streamed block is copied to slot 0 before the run, the u-th
 * streamed step reads slot u % 2 and prefetches the next streamed block
 * (circularly) into the other slot, and a COPY's step is the streamed step that
 * reads it.  n_resident = n gives n COMPUTE ops and nothing else. */
int dlo_plan_schedule_ex(const dlo_plan *plan, int32_t passes, int32_t n_resident,
                         dlo_sched_op *ops, int64_t cap, int64_t *n_ops);

/* ---------------------------------------------------------------------------
 * Forward ([Jul] "How It Works"; [Aug] s.3 "Double-Buffered Prefetch")
 *
 * Block forward (every block must carry the DiT schema of dlo_block_schema or its
 * FP8 form, dlo_block_schema_fp8 -- whose weights are first dequantised to bf16;
 * width d % 256 == 0, d <= 8192, head dim d / n_heads in {64, 128}):
 *   mod = SiLU(cond[:d]) W_ada^T + b_ada -> shift1, scale1, gate1, shift2, scale2, gate2
 *   h   = LN1(x[:, :d]) * (1 + scale1) + shift1                      (bf16)
 *   qkv = h W_qkv^T + b_qkv                                           (bf16)
 *   a   = per head softmax(q k^T / sqrt(dh)) v                        (bf16)
 *   x[:, :d] += gate1 * (a W_out^T + b_out)                           (fp32)
 *   h2  = LN2(x[:, :d]) * (1 + scale2) + shift2                       (bf16)
 *   u   = GELU_erf(h2 W_1^T + b_1)                                    (bf16)
 *   x[:, :d] += gate2 * (u W_2^T + b_2)                               (fp32)
 * bf16 MFMA products accumulate in fp32; LayerNorm statistics and softmax in fp32.
 * ------------------------------------------------------------------------- */

#define DLO_TRACE_DIGEST 1u  /* digest the slot's regions before and after each block */
#define DLO_TRACE_TIMING 2u  /* timestamp copies, block computes and every kernel */
#define DLO_RESIDENT 4u      /* no streaming: block b is read from resident_blocks[b] (same as
                                n_resident = number of blocks) */
#define DLO_FP8_COMPUTE 8u   /* FP8, MXFP8 and INT8 blocks run their qkv, out, fc1 and
                                fc2 linears as W8A8 products ([Doc] "Request and loading
                                constraints", online FP8, INT8 and MXFP8 linears), the
                                weight's codes and scales read in place from the slot:
                                per-tensor FP8 quantises each input per row to E4M3
                                (dlo_op_quantize_rows_fp8, dlo_op_gemm_fp8); MXFP8 per row
                                in blocks of 32 (dlo_op_quantize_rows_mxfp8,
                                dlo_op_gemm_mxfp8); INT8 per row to int8
                                (dlo_op_quantize_rows_int8, dlo_op_gemm_int8).  Without it
                                their linears run on dequantised bf16 weights (W8A16).  An
                                FP8 block's adaLN GEMV reads its codes (dlo_op_adaln_fp8);
                                MXFP8 and INT8 blocks' run on the dequantised weight.  bf16
                                blocks are unaffected. */
#define DLO_ASYNC_ENQUEUE 16u /* the call returns once the run is validated and its
                                 resources exist; a library thread enqueues the program on
                                 the two streams (filling the staging buffers of pageable
                                 blocks, [Doc] "Rank-local path without DLO AllGather": the
                                 staging slots as a pipeline stage of their own) while the
                                 caller goes on.  Needs run_out.  Until dlo_run_enqueued
                                 returns, the caller enqueues nothing on either stream (their
                                 order is enqueue order), starts no other run on the plan
                                 (DLO_E_STATE) and keeps the plan, the store and the args'
                                 device buffers alive; the args struct itself is copied. */

typedef struct {
  void *slot[2];            /* device, slot_bytes each, distinct (unused if nothing streams) */
  int64_t slot_bytes;       /* capacity of each slot */
  float *x;                 /* device fp32 [batch x tokens, x_row_stride], updated in place;
                               16-B aligned, x_row_stride % 4 == 0 (else DLO_E_ARG) */
  int64_t x_row_stride;     /* elements; >= the widest block's d */
  const float *cond;        /* device fp32 [batch, cond_stride]: a conditioning vector per
                               sample (>= widest d floats each) */
  void *workspace;          /* device, >= dlo_plan_workspace_bytes(plan, tokens) */
  int64_t workspace_bytes;
  void *compute_stream;     /* hipStream_t */
  void *copy_stream;        /* hipStream_t, distinct from compute_stream (unused if nothing
                               streams) */
  int32_t tokens;           /* rows of x (batch 1), >= 1; (tokens + 64) * 3 * widest d * 2
                               < 2^31, else DLO_E_UNSUPPORTED */
  int32_t passes;           /* chained passes over the stack, >= 1 */
  uint32_t flags;           /* DLO_TRACE_* | DLO_RESIDENT | DLO_FP8_COMPUTE | DLO_ASYNC_ENQUEUE */
  int32_t n_resident;       /* resident layers R in [0, n] ([Doc] "Validation coverage":
                               resident-layer requests): blocks 0 .. R-1 are read from
                               resident_blocks[b] and never copied; blocks R .. n-1 stream
                               through the two slots by the hook rule, their hooks linked
                               circularly among themselves (see dlo_plan_schedule_ex).
                               Ignored with DLO_RESIDENT.  Outside [0, n]: DLO_E_ARG. */
  const void *const *resident_blocks; /* device pointer per resident block (entries 0 .. R-1,
                                         or all with DLO_RESIDENT), holding the block's slot
                                         image (see dlo_place_block); NULL entry: DLO_E_ARG */
  int32_t batch;            /* samples, 0 read as 1 (< 0: DLO_E_ARG).  Sample b is rows
                               b*tokens .. (b+1)*tokens - 1 of x and row b of cond; every block
                               runs the samples one after another on its slot (a quantised
                               block's weights dequantised once), so one copy of a block serves
                               the whole batch.  The workspace is per sample
                               (dlo_plan_workspace_bytes of tokens).  With DLO_TRACE_TIMING the
                               kernel times are the first sample's; t_compute_* span the batch. */
  int32_t reserved0;        /* 0 */
  int64_t cond_stride;      /* floats between the samples' conditioning vectors; 0: the widest
                               block's d; between 1 and the widest d - 1: DLO_E_ARG */
} dlo_forward_args;

/* Enqueues `passes` passes of the stack.  x is updated on the compute stream;
 * everything the caller enqueued on the compute stream before the call happens
 * before the run, and the copy stream waits for it too.  Each call starts afresh
 * at block 0 in slot 0.  Caller memory must stay valid until the compute stream
 * has drained.  A run that streams blocks first waits on the host until the
 * plan's previous run has completed (copies enqueued behind a run still
 * executing measured 6-29 % slower on link-bound stacks), then enqueues its whole
 * copy/compute program; a run with every block resident does not wait.  With a
 * fully pinned store the call then returns without waiting; when blocks are
 * staged, the calling thread fills each staging buffer in step order (waiting
 * for the buffer's previous DMA first), so the call returns once the last
 * staged block has been handed to the copy stream -- unless DLO_ASYNC_ENQUEUE
 * hands all of that, the wait for the previous run included, to a library
 * thread.
 * If run_out is non-NULL it receives a handle for dlo_slot_trace (free with
 * dlo_run_destroy); otherwise the library releases the run's resources once it
 * has completed. */
int dlo_forward_stack(const dlo_plan *plan, const dlo_host_store *store,
                      const dlo_forward_args *args, dlo_run **run_out);

/* Places block b (its k shards per group, at the all-gather offsets) into the
 * device buffer dst (>= the block's extent) on `stream`: the same copies a
 * prefetch performs.  Used to build resident images. */
int dlo_place_block(const dlo_plan *plan, const dlo_host_store *store, int32_t b, void *dst,
                    int64_t dst_bytes, void *stream);

typedef struct {
  int64_t step;
  int32_t pass, block;
  int32_t read_slot;        /* -1 for a resident block */
  int32_t prefetch_block;   /* -1 on the last streamed step and for a resident block */
  int32_t prefetch_slot;    /* -1 likewise */
  int32_t pad;
  int64_t prefetch_bytes;   /* bytes copied by this step's prefetch (0 if none) */
  uint64_t digest_pre;      /* DLO_TRACE_DIGEST: slot regions before the block ran */
  uint64_t digest_post;     /* ... and after (0 without the flag) */
  /* DLO_TRACE_TIMING, milliseconds since the run's start event, else -1: */
  float t_copy_begin, t_copy_end;       /* the copy placing this step's block */
  float t_compute_begin, t_compute_end; /* this step's block forward */
} dlo_slot_event;

/* Waits for the run to complete, then copies up to cap records (one per step, in
 * step order) to out and sets *n_out to the number of steps.  The digest of a
 * slot is the wrap-around sum, over its regions' 8-byte little-endian words w at
 * slot byte offset o (a region's last partial word zero-extended), of
 * splitmix64_finalizer(w + (o / 8) * 0x9E3779B97F4A7C15). */
int dlo_slot_trace(dlo_run *run, dlo_slot_event *out, int64_t cap, int64_t *n_out);

/* DLO_TRACE_TIMING: per step, the duration in ms of each of the block's kernels in
 * launch order (DLO_KERNELS_PER_BLOCK per step), after the run completed: the
 * weight dequantisation of a quantised block (dequant_weights; 0 for a bf16
 * block and for W8A8), adaln_gemv, ln1_modulate, quant_h,
 * gemm_qk, gemm_v_t, attention, quant_attn, gemm_out_residual, ln2_modulate,
 * quant_h2, gemm_fc1_gelu, quant_u, gemm_fc2_residual (dlo_kernel_name).  The
 * quant_* entries are the W8A8 input quantisations, 0 unless a quantised block
 * runs with DLO_FP8_COMPUTE; for FP8 and MXFP8 LayerNorm + modulate writes the
 * quantised h and h2 itself (counted in ln1_modulate / ln2_modulate), so
 * quant_h and quant_h2 stay 0, and for MXFP8 the fc1 GEMM's epilogue writes the
 * quantised u (quant_u stays 0); INT8 quantises all four inputs in their own
 * passes.  A slot that launches nothing records no event (each timed event
 * between two kernels costs the stream a few microseconds) and reads exactly 0. */
#define DLO_KERNELS_PER_BLOCK 14
int dlo_run_kernel_times(dlo_run *run, float *ms, int64_t cap, int64_t *n_out);
/* name of kernel j (0 <= j < DLO_KERNELS_PER_BLOCK) of a block forward */
const char *dlo_kernel_name(int32_t j);

void dlo_run_destroy(dlo_run *run);   /* waits for the run first */

/* DLO_ASYNC_ENQUEUE: waits until the run's program is fully enqueued and returns
 * the status of that enqueue (the error a synchronous call would have returned;
 * DLO_OK at once for a run started without the flag).  After it the streams and
 * the plan are the caller's again.  dlo_slot_trace, dlo_run_kernel_times and
 * dlo_run_destroy call it first. */
int dlo_run_enqueued(dlo_run *run);

/* Message for the last failure on this thread (valid until the next call). */
const char *dlo_last_error(void);

/* ---------------------------------------------------------------------------
 * The DiT block schema and its single kernels
 * ------------------------------------------------------------------------- */

/* Parameter i (0 <= i < 16) of the DiT block schema for width d: name, dtype and
 * numel, in registration order (adaln.weight [6d,d] bf16, adaln.bias, norm1.weight,
 * norm1.bias, norm1.eps [1], attn.qkv.weight [3d,d] bf16, attn.qkv.bias,
 * attn.out.weight [d,d] bf16, attn.out.bias, norm2.weight, norm2.bias, norm2.eps,
 * mlp.fc1.weight [4d,d] bf16, mlp.fc1.bias, mlp.fc2.weight [d,4d] bf16,
 * mlp.fc2.bias; all others fp32).  Returns DLO_E_ARG for i out of range. */
#define DLO_DIT_N_PARAMS 16
int dlo_block_schema(int32_t d, int32_t i, const char **name, int32_t *dtype, int64_t *numel);

/* Parameter i (0 <= i < 21) of the FP8 form of the DiT block ([Doc] "Request and
 * loading constraints": per-tensor online FP8 linears keep a 1-byte weight plus
 * an fp32 scale and are sharded like any other dtype group): every bf16 matrix
 * X.weight of dlo_block_schema becomes X.weight (DLO_FP8_E4M3, same shape)
 * followed by X.weight_scale (fp32, 1 element); the other parameters are
 * unchanged, so each linear registers weight, weight_scale, bias.  The block's
 * dtype groups are then FP8 (18 d^2 elements) and fp32 (19 d + 7).  Its forward
 * dequantises each weight to bf16(code_value * scale) into the workspace on the
 * compute stream, then runs the bf16 block forward.  DLO_E_ARG for i out of
 * range. */
#define DLO_DIT_FP8_N_PARAMS 21
int dlo_block_schema_fp8(int32_t d, int32_t i, const char **name, int32_t *dtype, int64_t *numel);

/* The loader's finalisation of one weight for the FP8 block (host memory, not
 * on the streamed path): scale = amax|w| / 448 in fp32 (1 for an all-zero or
 * empty tensor); codes[i] = the OCP E4M3 code nearest to float(w[i]) / scale,
 * ties to the even code, saturating at +-448 (never NaN for finite input; NaN
 * input gives 0x7F).  w: n bf16 values; codes: n bytes; n >= 0.  DLO_E_ARG for
 * NULL pointers or n < 0. */
int dlo_quantize_fp8(const uint16_t *w, int64_t n, uint8_t *codes, float *scale);

/* Parameter i (0 <= i < 21) of the INT8 form of the DiT block ([Doc] "Request and
 * loading constraints": online INT8 linears keep an int8 weight plus an fp32
 * scale, sharded like any other dtype group): every bf16 matrix X.weight
 * [out, in] becomes X.weight (DLO_I8, same shape) followed by X.weight_scale
 * (fp32, one per output row: out elements); the other parameters are
 * unchanged.  Groups: int8 (18 d^2 elements) and fp32.  Its forward dequantises
 * each weight to bf16(code * scale_row) into the workspace, then runs the bf16
 * block forward.  DLO_E_ARG for i out of range. */
int dlo_block_schema_int8(int32_t d, int32_t i, const char **name, int32_t *dtype, int64_t *numel);

/* Parameter i (0 <= i < 21) of the MXFP8 form (same passage: online MXFP8 keeps
 * an fp8 weight plus an e8m0 block scale, possibly as a transposed view): X.weight
 * [out, in] becomes X.weight (DLO_FP8_E4M3, same shape) followed by
 * X.weight_scale (DLO_E8M0, one per 32 consecutive elements of a row, stored
 * block-major [in / 32, out]: out * in / 32 elements).  Groups: E4M3
 * (18 d^2), E8M0 (18 d^2 / 32) and fp32.  Its forward dequantises each weight
 * to bf16(code_value * 2^(e - 127)) (exact), then runs the bf16 block forward.
 * DLO_E_ARG for i out of range or d % 32 != 0. */
int dlo_block_schema_mxfp8(int32_t d, int32_t i, const char **name, int32_t *dtype, int64_t *numel);

/* The loader's finalisation of one weight [rows, cols] (bf16, row-major, host
 * memory) for the INT8 block: scales[r] = amax_r|w| / 127 in fp32 (1 for an
 * all-zero row); codes[r, j] = float(w[r, j]) / scales[r] rounded to the
 * nearest integer, ties to even, clamped to [-127, 127] (NaN -> 0).  DLO_E_ARG
 * for NULL pointers or negative sizes. */
int dlo_quantize_int8(const uint16_t *w, int64_t rows, int64_t cols, int8_t *codes, float *scales);

/* The same for the MXFP8 block (OCP MX, E4M3 elements): for each 32-element
 * block b of row r, X = floor(log2 amax) - 8 clamped to [-127, 127] (-127 for
 * an all-zero block), scales[b * rows + r] = X + 127 (block-major: the
 * transposed view of [rows, cols / 32]), codes = the E4M3 code nearest to
 * float(w) / 2^X, ties to the even code, saturating at +-448.  cols % 32 == 0,
 * else DLO_E_ARG. */
int dlo_quantize_mxfp8(const uint16_t *w, int64_t rows, int64_t cols, uint8_t *codes, uint8_t *scales);

/* The kernels the block forward is made of, callable one at a time (device
 * pointers, row-major, enqueued on `stream`, asynchronous).  Each validates its
 * shapes and returns DLO_E_UNSUPPORTED for shapes its kernel does not take. */

/* out[r] = sum_j W[r, j] * silu(c[j]) + b[r], r < rows; W bf16 [rows, d]. */
int dlo_op_adaln(const uint16_t *W, const float *b, const float *cond, int32_t rows, int32_t d,
                 float *out, void *workspace, int64_t workspace_bytes, void *stream);

/* dlo_op_adaln without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): SiLU(cond[:d]) is staged in a static device array of
 * DLO_NOALLOC_MAX_D floats inside the library instead of a caller workspace.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the array's device address is looked up once per device, on the
 * first call with that device current.  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (different streams, or other threads)
 * race and give undefined results; calls ordered on one stream are safe (each
 * call writes all d entries it reads).  Same arguments and results as
 * dlo_op_adaln, bit for bit; d > DLO_NOALLOC_MAX_D is DLO_E_UNSUPPORTED. */
#define DLO_NOALLOC_MAX_D 8192
int dlo_op_adaln_noalloc(const uint16_t *W, const float *b, const float *cond, int32_t rows, int32_t d,
                         float *out, void *stream);

/* The same on an FP8 block's adaLN weight ([Doc] "Request and loading
 * constraints": a 1-byte weight plus an fp32 scale): out[r] = w_scale[0] *
 * sum_j value(W[r, j]) * silu(c[j]) + b[r], W OCP E4M3 codes [rows, d] (16-B
 * aligned, d % 16 == 0, else DLO_E_UNSUPPORTED), w_scale one fp32 value; code
 * values are exact in fp32, so the weights carry no bf16 rounding.  workspace
 * >= 4 d bytes (silu(c)), else DLO_E_WORKSPACE. */
int dlo_op_adaln_fp8(const uint8_t *W, const float *w_scale, const float *b, const float *cond, int32_t rows,
                     int32_t d, float *out, void *workspace, int64_t workspace_bytes, void *stream);

/* out[t, :] = bf16( LN(x[t, :d]; gamma, beta, *eps) * (1 + scale) + shift ), t < T;
 * x fp32 with row stride ldx (x 16-B aligned, ldx % 4 == 0); out bf16 [T, d]
 * (8-B aligned); d % 256 == 0, d <= 8192.  Else DLO_E_UNSUPPORTED. */
int dlo_op_ln_modulate(const float *x, int64_t ldx, int32_t T, int32_t d, const float *gamma,
                       const float *beta, const float *eps, const float *shift,
                       const float *scale, uint16_t *out, void *stream);

/* C = A B^T + bias with A bf16 [M, K] (row stride lda), B bf16 [N, K] (ldb):
 *   epilogue 0: C bf16 [M, N] (ldc)
 *   epilogue 1: C bf16 = GELU_erf(A B^T + bias)
 *   epilogue 2: X fp32 (ldc) += gate[n] * (A B^T + bias)  (C points at X)
 *   epilogue 3: C bf16 [N, ldc] = (A B^T + bias)^T, i.e. C[n, m]; columns m in
 *               [M, M64) (M rounded up to 64) are 0, columns from M64 on are
 *               not written; ldc >= M64 and ldc % 8 == 0.  The block computes
 *               its v part this way, in the layout dlo_op_attention reads.
 * N % 256 == 0, K % 64 == 0, M >= 1; lda, ldb multiples of 8; C 16-B aligned,
 * bias and gate 4-B aligned (as the fp32 parameters packed back to back in a slot
 * are) and ldc % 4 == 0 (else DLO_E_UNSUPPORTED). */
enum { DLO_EPI_BIAS = 0, DLO_EPI_BIAS_GELU = 1, DLO_EPI_GATED_RESIDUAL = 2, DLO_EPI_BIAS_T = 3 };
int dlo_op_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int32_t M,
                int32_t N, int32_t K, const float *bias, const float *gate, void *C, int64_t ldc,
                int32_t epilogue, void *stream);

/* Per-row (per-token) dynamic E4M3 quantization of an activation matrix, the
 * input side of an FP8 block's online FP8 linears in the W8A8 form (the pages
 * only fix the weight side: [Doc] "Request and loading constraints"; the
 * activation scaling is this library's reading): for each row r of x bf16
 * [M, K] (row stride ldx), scales[r] = amax_r / 448 in fp32 (1 for an all-zero
 * row; NaN entries ignored), codes[r, k] = the OCP E4M3 code nearest to
 * x[r, k] / scales[r] (IEEE fp32 division), ties to the even code, saturating
 * at 448, NaN -> 0x7F.  codes uint8 [M, ldq], scales fp32 [M]; all device,
 * caller-owned.  K % 8 == 0, ldx and ldq multiples of 8 and >= K, x 16-B and
 * codes 8-B aligned, else DLO_E_UNSUPPORTED. */
int dlo_op_quantize_rows_fp8(const uint16_t *x, int64_t ldx, int32_t M, int32_t K, uint8_t *codes,
                             int64_t ldq, float *scales, void *stream);

/* The FP8 form of dlo_op_gemm: C = (A B^T) * a_scale[m] * b_scale[0] + bias, then
 * the epilogue (0..3 as for dlo_op_gemm), with A [M, K] and B [N, K] OCP E4M3
 * codes (row strides lda, ldb in bytes), a_scale fp32 [M] (per row, as
 * dlo_op_quantize_rows_fp8 writes it) and b_scale one fp32 value (the weight's
 * per-tensor scale, [Doc] "Request and loading constraints"); every product is
 * exact and accumulates in fp32 on v_mfma_f32_32x32x64_f8f6f4.  All device,
 * caller-owned.  N % 256 == 0, K % 64 == 0, lda and ldb multiples of 16, A, B,
 * C 16-B aligned, bias and gate 4-B aligned, ldc as for dlo_op_gemm, else
 * DLO_E_UNSUPPORTED. */
int dlo_op_gemm_fp8(const uint8_t *A, int64_t lda, const float *a_scale, const uint8_t *B, int64_t ldb,
                    const float *b_scale, int32_t M, int32_t N, int32_t K, const float *bias,
                    const float *gate, void *C, int64_t ldc, int32_t epilogue, void *stream);

/* Per-row INT8 quantization of an activation matrix, the input side of a W8A8
 * INT8 linear ([Doc] "Request and loading constraints", online INT8 linears;
 * the symmetric rule of dlo_quantize_int8 applied to each row of x bf16 [M, K],
 * row stride ldx): scales fp32 [M] = amax / 127 (1 for a row of zeros), codes
 * int8 [M, ldq] = x / scale (fp32 division) rounded to nearest-even, clamped to
 * +-127.  All device, caller-owned.  K % 8 == 0, ldx and ldq multiples of 8 and
 * >= K, x 16-B and codes 8-B aligned, else DLO_E_UNSUPPORTED. */
int dlo_op_quantize_rows_int8(const uint16_t *x, int64_t ldx, int32_t M, int32_t K, int8_t *codes,
                              int64_t ldq, float *scales, void *stream);

/* The INT8 form of dlo_op_gemm (W8A8 INT8, same passage): C = float(A B^T) *
 * a_scale[m] * b_scale[n] + bias, then the epilogue (0..3 as for dlo_op_gemm),
 * with A [M, K] and B [N, K] int8 codes (row strides lda, ldb in bytes), a_scale
 * fp32 [M] (as dlo_op_quantize_rows_int8 writes it) and b_scale fp32 [N] (the
 * weight's per-output-row scales, as dlo_quantize_int8 writes them, 4-B
 * aligned); the sums are exact int32 on v_mfma_i32_32x32x32_i8 (|sum| <= K *
 * 127^2 < 2^31 for K < 133 000), converted to fp32 once.  All device,
 * caller-owned.  N % 256 == 0, K % 64 == 0, lda and ldb multiples of 16, A, B,
 * C 16-B aligned, bias and gate 4-B aligned, ldc as for dlo_op_gemm, else
 * DLO_E_UNSUPPORTED. */
int dlo_op_gemm_int8(const int8_t *A, int64_t lda, const float *a_scale, const int8_t *B, int64_t ldb,
                     const float *b_scale, int32_t M, int32_t N, int32_t K, const float *bias,
                     const float *gate, void *C, int64_t ldc, int32_t epilogue, void *stream);

/* Per-row MXFP8 quantization of an activation matrix, the input side of a W8A8
 * MXFP8 linear (the MX rule of dlo_quantize_mxfp8 applied to each row of x bf16
 * [M, K], row stride ldx): codes uint8 [M, ldq] (OCP E4M3), scales E8M0
 * block-major [K / 32, lds] (row r of block b at b * lds + r); rows M .. lds - 1
 * of scales are set to 127 (2^0).  All device, caller-owned.  K % 32 == 0, ldx
 * and ldq multiples of 8 and >= K, lds >= M, x 16-B and codes 8-B aligned, else
 * DLO_E_UNSUPPORTED. */
int dlo_op_quantize_rows_mxfp8(const uint16_t *x, int64_t ldx, int32_t M, int32_t K, uint8_t *codes,
                               int64_t ldq, uint8_t *scales, int64_t lds, void *stream);

/* The MXFP8 form of dlo_op_gemm: C = sum over 32-blocks b of (A_b B_b^T) *
 * 2^(sa[b, m] - 127) * 2^(sb[b, n] - 127) + bias, then the epilogue (0..3 as for
 * dlo_op_gemm), with A [M, K] and B [N, K] OCP E4M3 codes (row strides lda, ldb
 * in bytes), a_scales E8M0 block-major [K / 32, lds_a] and b_scales [K / 32,
 * lds_b] (as dlo_op_quantize_rows_mxfp8 and the MXFP8 block form store them);
 * the block scales are applied by v_mfma_scale_f32_32x32x64_f8f6f4 itself.  All
 * device, caller-owned.  N % 256 == 0, K % 64 == 0, lds_a >= M and lds_b >= N
 * multiples of 4, scales 4-B aligned, the rest as for dlo_op_gemm_fp8, else
 * DLO_E_UNSUPPORTED. */
int dlo_op_gemm_mxfp8(const uint8_t *A, int64_t lda, const uint8_t *a_scales, int64_t lds_a, const uint8_t *B,
                      int64_t ldb, const uint8_t *b_scales, int64_t lds_b, int32_t M, int32_t N, int32_t K,
                      const float *bias, const float *gate, void *C, int64_t ldc, int32_t epilogue, void *stream);

/* Feature-major copy of the v part of a fused qkv buffer, the layout the
 * block's attention reads its values in:
 * vt[f, t] = qkv[t, 2 d + f] for f < d, t < T, and vt[f, t] = 0 for
 * T <= t < T64 (T rounded up to 64); columns from T64 to ldvt are not written.
 * qkv bf16 [T, >= 3 d] (row stride ldqkv), vt bf16 [d, ldvt], both device,
 * caller-owned, 16-B aligned.  d % 64 == 0, ldqkv >= 3 d, ldvt >= T64, ldqkv
 * and ldvt multiples of 8, else DLO_E_UNSUPPORTED.  (The block forward gets the
 * same layout straight from its v GEMM, dlo_op_gemm epilogue 3.) */
int dlo_op_v_transpose(const uint16_t *qkv, int64_t ldqkv, int32_t T, int32_t d, uint16_t *vt,
                       int64_t ldvt, void *stream);

/* Per head j < H: out[:, j*dh:(j+1)*dh] = softmax(q_j k_j^T / sqrt(dh)) v_j (the
 * block's non-causal self-attention), with q, k read from qkv bf16
 * [T, >= 2*H*dh] (row stride ldqkv) at column offsets 0 and H*dh, and v from a
 * feature-major copy vt bf16 [H*dh, ldvt] as dlo_op_v_transpose writes it
 * (columns T .. T64-1 must hold finite values; that op writes zeros there);
 * out bf16 [T, H*dh] (row stride ldo).  All device, caller-owned; qkv and vt
 * 16-B aligned.  dh in {64, 128}; ldqkv and ldvt multiples of 8, ldvt >= T64.
 * DLO_E_UNSUPPORTED when (T + 64) * ldqkv * 2 >= 2^31 (32-bit buffer offsets). */
int dlo_op_attention(const uint16_t *qkv, int64_t ldqkv, const uint16_t *vt, int64_t ldvt,
                     int32_t T, int32_t H, int32_t dh, uint16_t *out, int64_t ldo, void *stream);

/* out[i] = bf16_rne(e4m3_value(codes[i]) * *scale), i < n (device pointers; scale
 * is read on the device).  n % 16 == 0, codes 16-B and out 32-B aligned, else
 * DLO_E_UNSUPPORTED.  The FP8 block's forward runs this on each weight. */
int dlo_op_dequant_fp8(const uint8_t *codes, int64_t n, const float *scale, uint16_t *out,
                       void *stream);

/* Slot digest (see dlo_slot_trace) of up to DLO_MAX_GROUPS regions of `base`,
 * written to *out (device uint64). */
/* INT8 weight dequantisation (the INT8 block's forward runs this on each
 * weight): out[r, j] = bf16(code[r, j] * scales[r]) rounded to nearest even;
 * codes int8 [rows, cols] (16-B aligned), scales fp32 [rows], out bf16 (32-B
 * aligned).  cols % 16 == 0, else DLO_E_UNSUPPORTED. */
int dlo_op_dequant_int8(const int8_t *codes, int64_t rows, int64_t cols, const float *scales, uint16_t *out,
                        void *stream);

/* MXFP8 weight dequantisation: out[r, j] = bf16(value(codes[r, j]) *
 * 2^(scales[(j / 32) * rows + r] - 127)) (scales block-major, as the MXFP8 block
 * form stores them), exact for scales whose products stay in bf16's normal
 * range; E8M0 byte 255 gives NaN.  cols % 32 == 0, codes 16-B and out 32-B
 * aligned, else DLO_E_UNSUPPORTED. */
int dlo_op_dequant_mxfp8(const uint8_t *codes, int64_t rows, int64_t cols, const uint8_t *scales, uint16_t *out,
                         void *stream);

int dlo_op_digest(const void *base, const int64_t *offsets, const int64_t *lengths,
                  int32_t n_regions, uint64_t *out, void *stream);

/* Measurement: the sustained dense bf16 MFMA rate of the GPU with operands in
 * registers and no memory traffic in the loop -- the practical roofline of the
 * block's MFMA kernels under the chip's power limit, which the published dense
 * peak (256 CUs at 2.4 GHz) assumes away.  form 0: v_mfma_f32_32x32x16_bf16,
 * form 1: v_mfma_f32_16x16x32_bf16 (the same FLOPs per iteration).  Launches
 * one pass of `iters` iterations on `stream`; *flops (host, optional) receives
 * the FLOPs it performs.  in: device, 4096 x 8 bf16 operand values (16-B
 * aligned); out: device fp32 [DLO_MFMA_RATE_THREADS] checksums (caller-owned).
 * DLO_E_ARG for a NULL pointer, another form or iters < 1. */
#define DLO_MFMA_RATE_THREADS (256 * 512)
int dlo_op_mfma_rate(int32_t form, const uint16_t *in, float *out, int32_t iters, double *flops, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DLO_H */
