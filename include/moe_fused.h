/*
 * moe_fused.h -- C ABI of the MI355X (gfx950) fused Mixture-of-Experts forward layer.
 *
 * The layer is the fused MoE of the tilelang.dataflow README, section 3.5
 * ("Fused MoE: map -> reshared -> map"): routed tokens are grouped by expert
 * (group sizes, offsets, padded offsets, expert of each group block), GEMM-1
 * applies each expert's gate and up weights and forms the gated intermediate,
 * GEMM-2 applies the down projection, scales each row by its routing weight and
 * the per-token rows are summed.  The activation is SwiGLU, silu(gate) * up,
 * taken on the unrounded fp32 accumulator (PipeLink, section 5.5 "Fused GEMM
 * and Activation").  FP8 is OCP E4M3FN with fp32 block scales.  MXFP8, which
 * the pages name as a variant of the Mixture-of-Kittens MoE kernels (PipeLink,
 * section 5.3) without defining it, is taken as the OCP Microscaling format:
 * E4M3FN values with one E8M0 scale per 32 consecutive values along K.
 * The clamped activation (moe_dims.activation) is the GPT-OSS variant of
 * SwiGLU, which the same page names as an independent activation owner; its
 * published definition is taken.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP global memory) of the current
 *    device, dense row-major, 16-byte aligned.  Sizes are element counts.
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *    stream).  Work is only enqueued: no call synchronises the host, none
 *    reads routing back to the host, and none allocates device memory.
 *  - The caller owns every buffer and keeps it alive until the stream work has
 *    completed.  Outputs must not alias inputs.  Calls that share a workspace
 *    must be ordered on one stream.
 *  - Return value: MOE_OK (0) or an error code.  Argument checks run on the host
 *    before anything is enqueued; on error nothing is enqueued.  MOE_ERR_HIP
 *    reports a failed launch (the HIP error is then cleared).
 *  - The caller lends all device memory, the workspace included (PipeLink,
 *    section 5.3: each owner of the MoE megakernel builds its descriptors from
 *    caller-lent buffers).  So the library holds no device allocation: there
 *    is no call to install or release a library-owned workspace, no
 *    out-of-memory error, and nothing to shut down.  Faults of enqueued device
 *    work surface through the stream (hipStreamSynchronize and the like), as
 *    for any kernel; no kernel here waits on the device, so there is no
 *    watchdog word to poll.
 *  - Shapes travel in moe_dims (plain integers); each pointer is a dense
 *    row-major array whose dtype the mode fixes.
 */
#ifndef MOE_FUSED_H
#define MOE_FUSED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported symbols of the shared library (everything else is hidden). */
#define MOE_API __attribute__((visibility("default")))

/* Error codes. */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1 /* null pointer, bad shape, misaligned pointer */
#define MOE_ERR_UNSUPPORTED 2 /* shape outside the supported envelope (see moe_dims) */
#define MOE_ERR_WORKSPACE 3   /* workspace missing or smaller than moe_workspace_bytes() */
#define MOE_ERR_HIP 4         /* a HIP launch or device query failed */
#define MOE_ERR_SCRATCH 5     /* moe_fused_forward_noalloc: the dims need more than MOE_NOALLOC_SCRATCH_BYTES */

/* Data modes (dtypes of x / weights / out):
 *  MOE_MODE_F32ACT  x fp32 [T,d_h]; W1, W2 bf16; out fp32.  The GEMMs run on
 *                   bf16 MFMA, so x is rounded to bf16 (nearest-even) on load.
 *  MOE_MODE_BF16    x, W1, W2, out bf16.
 *  MOE_MODE_FP8     x, W1, W2 e4m3 codes with fp32 128x128 block scales; out
 *                   bf16.  The intermediate is requantised per row per 128
 *                   columns (scale amax/448).
 *  MOE_MODE_MXFP8   x, W1, W2 e4m3 codes with E8M0 scales per 32 values along
 *                   K; out bf16.  The intermediate is requantised per row per
 *                   32 columns (shared exponent floor(log2 amax) - 8, elements
 *                   saturated to +-448).
 *  MOE_MODE_INT8    x int8 codes with one fp32 scale per token (tokens
 *                   quantised to int8 and dequantised by GEMM-1: the CUCo
 *                   page, section 4, DeepSeek-V3 MoE Dispatch and Combine,
 *                   steps (1) and (3)); W1, W2 bf16; out bf16.  The codes are
 *                   widened to bf16 exactly, the bf16 GEMMs run on them and
 *                   each row's fp32 accumulators take its token's scale before
 *                   the activation; the intermediate is bf16 as in BF16 mode. */
#define MOE_MODE_F32ACT 0
#define MOE_MODE_BF16 1
#define MOE_MODE_FP8 2
#define MOE_MODE_MXFP8 3
#define MOE_MODE_INT8 4

/* Storage order of W1 and W2 (moe_dims.weight_layout):
 *  MOE_WEIGHTS_ROW_MAJOR  w1 [E, 2*d_e, d_h], w2 [E, d_h, d_e] as described for
 *                         moe_fused_forward.
 *  MOE_WEIGHTS_PACKED     the tile order moe_pack_weights writes: the same
 *                         bytes, permuted so that every weight tile a GEMM
 *                         task streams is one contiguous block. */
#define MOE_WEIGHTS_ROW_MAJOR 0
#define MOE_WEIGHTS_PACKED 1

/* Activation of GEMM-1's gate and up values g, u (moe_dims.activation), taken
 * on the fp32 accumulators:
 *  MOE_ACT_SWIGLU          h = silu(g) * u
 *  MOE_ACT_SWIGLU_CLAMPED  g' = min(g, 7), u' = clamp(u, -7, 7),
 *                          h = g' * sigmoid(1.702 * g') * (u' + 1) */
#define MOE_ACT_SWIGLU 0
#define MOE_ACT_SWIGLU_CLAMPED 1

/* Launch form of moe_fused_forward (moe_dims.launch):
 *  MOE_LAUNCH_MULTI   routing, GEMM-1, GEMM-2 and the combine as four kernels
 *                     (plus the conversion of x in the F32ACT and INT8 modes).
 *  MOE_LAUNCH_SINGLE  the whole layer in one persistent kernel: GEMM-1 and
 *                     GEMM-2 under one launch, their dependency resolved without
 *                     a kernel barrier (tilelang.dataflow README, section 3.5,
 *                     "Fused MoE: map -> reshared -> map").  Every workgroup
 *                     derives the routing plan from the ids; tasks are claimed in
 *                     order from one queue; a GEMM-2 task waits (bounded) on a
 *                     completion counter of its M-tile's GEMM-1 tasks; the last
 *                     GEMM-2 task to store a (token, 128-column block) sums that
 *                     token's slots in ascending order.  The weighted rows stay in
 *                     fp32 (no bf16 rounding before the sum), so the output may
 *                     differ from MOE_LAUNCH_MULTI's in the last bf16 bit; it is
 *                     bitwise identical across calls.  Envelope: MOE_MODE_BF16,
 *                     MOE_MODE_FP8 or MOE_MODE_MXFP8, num_tokens*top_k <= 2048,
 *                     num_tokens*(d_hidden/128) <= 65536; MOE_ERR_UNSUPPORTED
 *                     otherwise.  The workspace's synchronisation block (its
 *                     first MOE_SYNC_BYTES) must hold zeros before the first
 *                     single-launch call on that workspace (moe_workspace_init, or
 *                     any zero fill); every single-launch call leaves it zero, and
 *                     MOE_LAUNCH_MULTI calls do not touch it. */
#define MOE_LAUNCH_MULTI 0
#define MOE_LAUNCH_SINGLE 1
#define MOE_SYNC_BYTES 265216u

/* Layer shape.  Supported envelope: 0 <= num_tokens, 1 <= num_experts <= 256,
 * 1 <= top_k <= 8, num_tokens*top_k < 2^31, d_hidden and d_expert positive
 * multiples of 128.  Zero-initialising weight_layout, activation and launch
 * selects row-major weights, SwiGLU and the four-kernel launch. */
typedef struct {
    int32_t mode;          /* MOE_MODE_* */
    int32_t num_tokens;    /* T */
    int32_t num_experts;   /* E */
    int32_t top_k;         /* k */
    int32_t d_hidden;      /* d_h */
    int32_t d_expert;      /* d_e */
    int32_t weight_layout; /* MOE_WEIGHTS_* */
    int32_t activation;    /* MOE_ACT_* */
    int32_t launch;        /* MOE_LAUNCH_* */
} moe_dims;

/* Scales of the quantised modes (dequantised value = code * scale).  Required
 * in MOE_MODE_FP8 and MOE_MODE_MXFP8 (all three) and MOE_MODE_INT8 (x_scale
 * only), ignored otherwise.
 * MOE_MODE_FP8, fp32:
 *  x_scale   [T, d_h/128]                 one scale per token per 128 columns
 *  w1_scale  [E, 2*d_e/128, d_h/128]      one scale per 128x128 block of W1
 *  w2_scale  [E, d_h/128, d_e/128]        one scale per 128x128 block of W2
 * MOE_MODE_MXFP8, uint8 E8M0 (byte s means 2^(s-127); s = 255 is NaN and
 * makes the rows it scales NaN):
 *  x_scale   [T, d_h/32]                  one byte per token per 32 columns
 *  w1_scale  [E, 2*d_e, d_h/32]           one byte per W1 row per 32 columns
 *  w2_scale  [E, d_h, d_e/32]             one byte per W2 row per 32 columns
 * MOE_MODE_INT8, fp32:
 *  x_scale   [T]                          one scale per token (w1_scale, w2_scale unused) */
typedef struct {
    const void* x_scale;
    const void* w1_scale;
    const void* w2_scale;
} moe_scales;

/* Bytes of device workspace moe_fused_forward needs for these dims (routing
 * metadata, task lists, the intermediate and the per-assignment rows): the
 * caller-lent buffer of PipeLink section 5.3 (the MoE megakernel's owners
 * take their buffers from the caller), sized on the host with no device call.
 * Returns 0 if the dims are invalid. */
MOE_API size_t moe_workspace_bytes(const moe_dims* dims);

/*
 * Fused MoE forward (tilelang.dataflow README, section 3.5 "Fused MoE: map ->
 * reshared -> map", steps 1 to 5: grouping metadata, GEMM-1 with the gated
 * activation, GEMM-2, routing weights, output rows).  The whole call is
 * enqueued without host computation and can be captured in a HIP graph, the
 * property PipeLink section 4 ("Contract-Guided Linking") states for an open
 * session behind its C interface.
 *   out[t] = sum_{j<k} topk_w[t,j] * W2[e] . ( silu(W1[e][0:d_e] . x[t]) * (W1[e][d_e:2d_e] . x[t]) ),
 *   e = topk_ids[t,j]  (or the clamped activation in place of silu(g) * u).
 *
 *  x         [T, d_h]            fp32 / bf16 / e4m3 / int8 per mode
 *  topk_ids  [T, k] int32        expert of each assignment p = t*k + j; ids
 *                                outside [0,E) are dropped (contribute 0)
 *  topk_w    [T, k] fp32         routing weights, used as given
 *  w1        [E, 2*d_e, d_h]     rows [0,d_e) gate, [d_e,2*d_e) up; K (d_h) contiguous
 *  w2        [E, d_h, d_e]       K (d_e) contiguous
 *                                (with MOE_WEIGHTS_PACKED: the outputs of moe_pack_weights)
 *  scales    FP8, MXFP8 and INT8 modes only (may be NULL otherwise)
 *  out       [T, d_h]            fp32 (F32ACT) or bf16; every row is written
 *  workspace device buffer of at least moe_workspace_bytes(dims) bytes, 256-byte aligned
 *
 * Steps enqueued on `stream`: routing (histogram, prefix scan, stable scatter,
 * block map and per-XCD task lists), grouped GEMM-1 with the SwiGLU epilogue,
 * grouped GEMM-2 with the routing-weight epilogue, and the top-k combine in
 * ascending slot order; as four kernels, or as one with MOE_LAUNCH_SINGLE
 * (see there).  The result is bitwise identical across calls.
 * Ownership: every buffer is the caller's; the call keeps no pointer past
 * the stream work it enqueues.  num_tokens == 0 returns MOE_OK and enqueues
 * nothing.  Errors: MOE_ERR_INVALID_ARG (null dims, a field of dims out of
 * range, a null or misaligned tensor pointer, missing scales in a quantised
 * mode); MOE_ERR_UNSUPPORTED (dims within range but outside the envelope
 * above, e.g. d_hidden not a multiple of 128); MOE_ERR_WORKSPACE (workspace
 * null, too small or not 256-byte aligned); MOE_ERR_HIP (a launch failed).
 */
MOE_API int moe_fused_forward(const moe_dims* dims, const void* x, const int32_t* topk_ids, const float* topk_w,
                      const void* w1, const void* w2, const moe_scales* scales, void* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * moe_fused_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) of device memory inside the library: each
 * GPU the library runs on holds its own copy until the process ends.  Its
 * device address is looked up once per device, on the first call with that
 * device current (make one call before capturing the call in a graph).  The
 * call allocates nothing and frees nothing; same kernels and result, bit for
 * bit, as moe_fused_forward with a workspace of its own.
 * The scratch keeps the last call's contents; every call writes what it reads
 * before reading it.  Calls on one GPU share that GPU's scratch: calls that
 * overlap in time on one GPU (two streams, or two host threads) race and give
 * wrong results; order them on one stream.
 * Errors: those of moe_fused_forward, with MOE_ERR_SCRATCH (checked on the
 * host before anything else, nothing enqueued) when moe_workspace_bytes(dims)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES (e.g. 8192 tokens of the 7168/2048 top-2
 * layer, whose per-assignment rows alone take 235 MB), and MOE_ERR_HIP if the
 * scratch's address cannot be obtained.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
MOE_API int moe_fused_forward_noalloc(const moe_dims* dims, const void* x, const int32_t* topk_ids,
                                      const float* topk_w, const void* w1, const void* w2,
                                      const moe_scales* scales, void* out, void* stream);

/* moe_fused_forward with kernel timing (kernel durations are what the
 * tilelang.dataflow README's "Fused MoE vs MegaMoE" comparison times for the
 * competitor, from its profiler): events[0..7] (hipEvent_t, created by
 * the caller with timing enabled) receive the start and end of the routing,
 * GEMM-1, GEMM-2 and combine kernels as their dispatches record them
 * (events[2i] start, events[2i+1] end of kernel i), so hipEventElapsedTime on
 * a pair gives that kernel's duration.  With MOE_LAUNCH_SINGLE, events[0] and
 * events[1] bracket the one kernel and events[2..7] are recorded right after
 * it.  Same result and errors as moe_fused_forward; MOE_ERR_INVALID_ARG if
 * events or any of its 8 entries is NULL. */
MOE_API int moe_fused_forward_profiled(const moe_dims* dims, const void* x, const int32_t* topk_ids,
                                       const float* topk_w, const void* w1, const void* w2,
                                       const moe_scales* scales, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream, void* const* events);

/* Zero the synchronisation block of a workspace (its first MOE_SYNC_BYTES), as
 * a single-launch call needs it before its first use of that workspace (see
 * MOE_LAUNCH_SINGLE); enqueues one small kernel on `stream` (no memset, so the
 * call can be captured in a graph).  MOE_ERR_WORKSPACE if workspace is null,
 * not 256-byte aligned or smaller than MOE_SYNC_BYTES; MOE_ERR_HIP if the
 * launch fails. */
MOE_API int moe_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Rewrite row-major W1 and W2 (bf16 or e4m3 as dims->mode says) into the
 * packed tile order, once, when the weights are loaded (a storage choice for
 * the weight shard each GEMM task loads, tilelang.dataflow README section 3.5
 * step 2; no page defines this order); the forward call then
 * streams each task's weight tile as one contiguous block instead of one
 * 128-byte piece per weight row (dims->weight_layout is ignored here).  The
 * permutation moves 16-byte chunks; block scales keep their layout.
 *
 * With eb bytes per element (2 for bf16, 1 for e4m3) and the column-block
 * widths of moe_ws_layout (block_n1: 64 in the bf16 modes, 128 in the FP8 and
 * MXFP8 modes;
 * block_n2: 128), let R1 = d_h*eb/128 and R2 = d_e*eb/128 (128-byte K blocks
 * per weight row), n1 = d_e/block_n1, n2 = d_h/128.  Then, for 0 <= s < 8:
 *  w1_packed chunk (((e*n1 + c)*R1 + b)*2*block_n1 + r)*8 + s holds bytes
 *    [128*b + 16*(s ^ (r & 7)), +16) of W1[e] row c*block_n1 + r (gate rows,
 *    r < block_n1) or d_e + c*block_n1 + r - block_n1 (up rows);
 *  w2_packed chunk (((e*n2 + c)*R2 + b)*128 + r)*8 + s holds bytes
 *    [128*b + 16*(s ^ (r & 7)), +16) of W2[e] row c*128 + r.
 * The packed buffers have the byte sizes of w1 and w2, are caller-owned,
 * 16-byte aligned and must not overlap the inputs.  MOE_ERR_INVALID_ARG for
 * invalid dims, a null or misaligned pointer, or overlapping buffers.
 */
MOE_API int moe_pack_weights(const moe_dims* dims, const void* w1, const void* w2, void* w1_packed,
                             void* w2_packed, void* stream);

/*
 * Backward pass with recompute (the MoE megakernel of PipeLink section 5.3
 * serves forward, backward and recompute passes; the gradients are the chain
 * rule of the forward above).  BF16 mode, row-major weights and SwiGLU only
 * (MOE_ERR_UNSUPPORTED otherwise).  Nothing of the forward is kept: the gate
 * and up accumulators and h are recomputed from x and W1.
 *
 *  x, topk_ids, topk_w, w1, w2  as for moe_fused_forward (bf16 x, W1, W2)
 *  dout      [T, d_h] bf16       gradient of the layer output
 *  dx        [T, d_h] fp32       out: gradient of x
 *  dw1       [E, 2*d_e, d_h] fp32  out: gradient of W1 (every expert written; 0 for experts without rows)
 *  dw2       [E, d_h, d_e] fp32  out: gradient of W2
 *  dtopk_w   [T, k] fp32         out: gradient of the routing weights (0 for dropped ids)
 *  workspace at least moe_backward_workspace_bytes(dims) bytes, 256-byte aligned
 *
 * Per routed row p (token t, expert e, weight w), with h = bf16(silu(g) u):
 *   q = dout[t] . W2[e],  dtopk_w[p] = <q, h>,  dh = w q,
 *   dg = bf16(dh u silu'(g)),  du = bf16(dh silu(g)),
 *   dx[t] = sum over the token's slots (ascending) of [dg du] . W1[e],
 *   dW1[e] = sum_p [dg du]^T x[t],  dW2[e] = sum_p bf16(w dout[t])^T h.
 * The bf16 roundings of dg, du and w dout are where the backward's bf16 GEMMs
 * take their operands.  Errors as for moe_fused_forward; every pointer 16-byte
 * aligned.  The caller owns all buffers; nothing is allocated.
 */
MOE_API size_t moe_backward_workspace_bytes(const moe_dims* dims);
MOE_API int moe_fused_backward(const moe_dims* dims, const void* x, const int32_t* topk_ids, const float* topk_w,
                               const void* w1, const void* w2, const void* dout, float* dx, float* dw1, float* dw2,
                               float* dtopk_w, void* workspace, size_t workspace_bytes, void* stream);

/* Rows per group block: each expert's group of routed rows is padded to a
 * multiple of this (tilelang.dataflow README section 3.5, "padded offsets"). */
MOE_API int32_t moe_block_m(void);

/* Capacities of the padded row space and of the block map (tilelang.dataflow
 * README section 3.5 step 1: padded offsets, expert of each group block) for
 * N = T*k assignments over E experts: n_pad_cap = N + min(E,N)*(block_m-1),
 * tile_cap = n_pad_cap / block_m. */
MOE_API int moe_route_caps(int32_t num_tokens, int32_t top_k, int32_t num_experts, int64_t* n_pad_cap,
                   int64_t* tile_cap);

/* Device output buffers of moe_route (all int32, caller-owned):
 *  counts[E]          rows routed to each expert
 *  offsets[E+1]       exclusive prefix sum of counts
 *  padded_offsets[E+1] exclusive prefix sum of block_m*ceil(counts/block_m)
 *  pos[N]             offsets[e] + rank of p among expert e's assignments (ascending p), -1 if dropped
 *  sorted_p[N]        sorted_p[pos[p]] = p; -1 beyond offsets[E]
 *  ppos[N]            padded_offsets[e] + rank, -1 if dropped
 *  row_src[n_pad_cap] p for each padded row, -1 on padding rows and beyond padded_offsets[E]
 *  tile_expert[tile_cap], tile_row0[tile_cap]  expert and first padded row of each
 *                     block in ascending expert order, -1 beyond the last block
 *  stats[4]           {dropped, number of blocks, padded rows, 0} */
typedef struct {
    int32_t* counts;
    int32_t* offsets;
    int32_t* padded_offsets;
    int32_t* pos;
    int32_t* sorted_p;
    int32_t* ppos;
    int32_t* row_src;
    int32_t* tile_expert;
    int32_t* tile_row0;
    int32_t* stats;
} moe_route_out;

/* Routing metadata alone (the first step of moe_fused_forward, same kernel),
 * for N = T*k flat assignment ids: the group sizes, offsets, padded offsets
 * and expert of each group block that tilelang.dataflow README section 3.5
 * step 1 takes as the fused MoE's input, plus the stable permutation.
 * MOE_ERR_INVALID_ARG for a null output pointer (or null ids with N > 0) or
 * top_k / num_experts outside [1,8] / [1,256]; MOE_ERR_UNSUPPORTED for
 * N >= 2^31. */
MOE_API int moe_route(int32_t num_tokens, int32_t top_k, int32_t num_experts, const int32_t* topk_ids,
              const moe_route_out* out, void* stream);

/* Byte offsets of the workspace sections moe_fused_forward uses, for tests and
 * inspection after a call.  The task lists are the device-built form of the
 * per-queue plans of tilelang.dataflow README section 3.5 (a hot expert
 * yields more group-block tasks; queues may take unequal amounts of work).  Of the routing arrays described for moe_route the
 * layer writes counts, offsets, padded_offsets and row_src (the padded
 * permutation its GEMMs consume, with the task lists below); pos, ppos,
 * sorted_p and the block map (tile_expert, tile_row0) are sized here but
 * written by moe_route only.  row_w (fp32 [n_pad_cap]) holds the routing weight of each padded
 * row below padded_offsets[E] (0 on padding rows).  `stats` is a control block of int32 words: [0..4] = {dropped,
 * blocks, padded rows, GEMM-1 tasks, GEMM-2 tasks}; words [272..280] and
 * [288..296] hold the start of each of the 8 per-XCD segments (and the end of
 * the last) of the GEMM-1 and GEMM-2 task lists.  Tasks are int32 quadruples
 * {expert, first padded row, row blocks, column block}; within a segment they
 * are ordered by descending expert row count, and all M-tiles of one
 * (expert, column block) sit in the same segment, next to each other.
 * `sync` (always 0) is the synchronisation block of MOE_LAUNCH_SINGLE: its
 * int32 word 64 counts the bounded waits of single-launch calls that ran out
 * (each such call's output is not valid; 0 unless the grid could not make
 * progress), and no call resets it.  y holds fp32 rows with MOE_LAUNCH_SINGLE.
 * block_n1 / block_n2: output columns of a GEMM-1 / GEMM-2 task (GEMM-2 takes
 * 256 from 1024 assignments on in FP8 mode, and in MXFP8 mode with d_e of at
 * least 1024, with four launches and d_h a multiple of 256; else 128);
 * max_row_blocks: the largest task of either list, in 16-row group blocks (16
 * where an 8-wave GEMM runs: GEMM-1 from 2048 assignments in FP8 mode, 4096 in
 * MXFP8 mode, or the 256-column GEMM-2; else 8).
 * Returns MOE_ERR_INVALID_ARG for invalid dims. */
typedef struct {
    size_t counts, offsets, padded_offsets, pos, sorted_p, ppos, row_src, row_w, tile_expert, tile_row0, stats;
    size_t tasks1, tasks2, h, h_scale, y, zero, x_bf16, sync, total;
    int64_t n_pad_cap, tile_cap, task1_cap, task2_cap;
    int32_t block_n1, block_n2, max_row_blocks;
} moe_ws_layout;

MOE_API int moe_workspace_layout(const moe_dims* dims, moe_ws_layout* layout);

/* Human-readable name of an error code (static string). */
MOE_API const char* moe_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FUSED_H */
