/*
 * mok.h — C ABI of the MI355X (gfx950) Mixture-of-Kittens-style MoE layer library.
 *
 * One MoE layer on one GPU's share of an expert-parallel layer: a schedule (per-expert
 * counts, offsets and a dispatch table), dispatch of routed rows into a fixed ring of
 * minibatch slots, the SwiGLU expert FFN as grouped MFMA GEMMs, and the gate-weighted
 * combine back to token order — forward in one persistent kernel whose workgroups are
 * split between data movement (dispatch/combine) and MFMA compute, handing work to
 * each other through device-memory counters.
 *
 * Sources (web pages on Cursor's open-sourced Mixture-of-Kittens, MoK):
 *   [L] Leiphone, "MoK：把 token 调度、跨 GPU 通信和专家计算塞进同一个 GPU 内核",
 *       sections 01, 02, 03;
 *   [M] news brief "Cursor开源MoK：GB300 NVL72机架上的确定性MoE训练大内核",
 *       section "三个重要的设计决策".
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the caller.  The
 *     library never allocates or frees device memory and keeps no global state; calls
 *     on different workspaces are independent.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; no entry point synchronises except mok_read_device_status.
 *   - Host-side argument checks (null pointers, shapes, workspace size, unsupported
 *     modes) return an error code synchronously and enqueue nothing.  These checks run
 *     before any HIP runtime call, so they work on a machine without a GPU.  One check
 *     needs the device: the fused forward's comm_cus must be below the number of
 *     workgroups its persistent kernel runs (one per compute unit), so mok_moe_fwd first
 *     queries the current device (device, attribute and occupancy queries only) and
 *     returns MOK_E_SHAPE, with nothing enqueued, when comm_cus is too large.
 *   - Data-dependent faults are recorded in a sticky device status word inside the
 *     workspace (MOK_DEV_* bits), read back with mok_read_device_status.
 *   - Same inputs and descriptor give bitwise-identical outputs (fixed-order sums, no
 *     floating-point atomics).
 *
 * Layouts (row-major, "nn.Linear" convention: the K dimension of every GEMM operand
 * is contiguous):
 *   x, y, dy, dx      [T, D]           bf16
 *   topk_ids          [T, k]           int32  (global expert id, -1 = masked slot)
 *   topk_w, d_topk_w  [T, k]           fp32   (gate weights and their gradient)
 *   w_gate, w_up      [E_loc, I, D]    bf16   (index 0 = expert e0)
 *   w_down            [E_loc, D, I]    bf16
 *   dw_gate, dw_up    [E_loc, I, D]    fp32;   dw_down [E_loc, D, I] fp32
 *   MXFP8 weights: e4m3 codes with the same shapes (uint8) plus e8m0 scales, one byte
 *   per 32 consecutive elements along the contiguous K axis ([E_loc, I, D/32] and
 *   [E_loc, D, I/32]).
 */
#ifndef MOK_H
#define MOK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOK_OK = 0,
  MOK_E_NULL = 1,        /* a required pointer is NULL                               */
  MOK_E_SHAPE = 2,       /* a size is out of range or inconsistent                   */
  MOK_E_UNSUPPORTED = 3, /* valid request the library does not implement            */
  MOK_E_WORKSPACE = 4,   /* workspace smaller than mok_workspace_size                */
  MOK_E_LAUNCH = 5,      /* the HIP runtime refused a launch                         */
  MOK_E_DEVICE = 6       /* no usable gfx950 device / runtime error                  */
} mok_status_t;

/* precision */
#define MOK_PREC_BF16 0
#define MOK_PREC_MXFP8 1

/* flags */
#define MOK_FLAG_SAVE_FOR_BWD 0x1u  /* forward keeps X and the gate/up pre-activations of
                                       the resident minibatches for mok_moe_bwd (MXFP8:
                                       the pre-activations of every routed row, for
                                       mok_moe_bwd_mx)                                   */
#define MOK_FLAG_UNFUSED 0x2u       /* run the same steps as separate kernels over
                                       full-size buffers (comparison / phase timing)     */
#define MOK_FLAG_SHORT_WAITS 0x4u   /* bounded waits of the fused forward and of the
                                       backward's persistent launch expire after 1 us instead
                                       of 2 s: the run sets MOK_DEV_TIMEOUT and exits
                                       early with its outputs undefined (tests the
                                       timeout path; never for production use)           */
#define MOK_FLAG_PERTURB 0x8u       /* debug: before each cross-workgroup signal (a gathered
                                       minibatch, a finished tile) and before each drain or
                                       row-sum chunk, the workgroup sleeps for a pseudo-random
                                       0-28 us.  Changes the interleaving of the persistent
                                       kernels only: outputs must stay bitwise the same
                                       (tests the handoffs for ordering races)           */
#define MOK_FLAG_OVERLAP_NEXT 0x20u /* macrobatch interleave ([L] section 02: the combine of
                                       one macrobatch runs while the next is dispatched):
                                       the fused forward's compute workgroups leave as soon
                                       as no tile is left instead of helping with the final
                                       combine, which the comm_cus data movers finish; a
                                       forward of the next macrobatch, launched on another
                                       stream with its own workspace, starts on the freed
                                       compute units and dispatches while this one still
                                       combines.  Outputs are bitwise the same as without
                                       the flag                                          */
#define MOK_FLAG_TRACE 0x10u        /* the fused forward and the backward's persistent
                                       launch write timestamps of every ticket and
                                       workgroup into a trace region of the workspace
                                       (mok_trace_layout)                                */

/* sticky device status bits (mok_read_device_status) */
#define MOK_DEV_BAD_ID 0x1u   /* an id was < -1 or >= E; that pair was skipped          */
#define MOK_DEV_TIMEOUT 0x2u  /* a bounded wait inside a persistent kernel expired      */

/* Layer descriptor.  Symbols follow the pages' vocabulary: a minibatch is the number of
 * routed rows handed to expert compute at once ([L] section 02); the ring of
 * minibatch slots is the fixed-size token buffer ([L] section 02, [M] design
 * decisions); comm_cus is the explicit split of compute units between data movement
 * and expert FFN ([L] section 02). */
typedef struct {
  int32_t num_tokens;        /* T: tokens in the pool                                   */
  int32_t hidden;            /* D: hidden size (multiple of 64)                         */
  int32_t intermediate;      /* I: expert intermediate size (multiple of 64)            */
  int32_t num_experts;       /* E: experts over all GPUs                                */
  int32_t top_k;             /* k: slots per token (1..64)                              */
  int32_t expert_begin;      /* e0: first local expert                                  */
  int32_t num_local_experts; /* E_loc: local experts [e0, e0+E_loc), 1..1024            */
  int32_t minibatch_rows;    /* M: routed rows per minibatch / ring slot                */
  int32_t ring_slots;        /* S: slots in the ring (>= 1)                             */
  int32_t comm_cus;          /* workgroups doing dispatch/combine in the fused kernel:
                                1 .. (device CUs - 1), checked by mok_moe_fwd            */
  int32_t precision;         /* MOK_PREC_BF16 or MOK_PREC_MXFP8                         */
  uint32_t flags;            /* MOK_FLAG_*                                              */
} mok_desc_t;

/* Bytes of workspace the layer needs for `desc` (host only, no HIP call).
 * The workspace holds the schedule, the ring of S minibatch slots, the per-slot
 * result buffer and the device counters.  Errors: MOK_E_NULL, MOK_E_SHAPE,
 * MOK_E_UNSUPPORTED. */
mok_status_t mok_workspace_size(const mok_desc_t* desc, size_t* bytes);

/* Schedule ([L] section 01: count every expert's rows, choose their positions, keep
 * one expert's rows contiguous for the grouped GEMM; [M] design decisions: one table
 * serves the four transfers).  Reads topk_ids [T, k] and writes into the workspace:
 * per-local-expert counts and offsets, perm[r] = t*k + j for every routed row r (rows
 * of one expert contiguous, in ascending (token, slot) order), pos[t*k+j] = row or -1,
 * and the minibatch tile table.  Ids outside [e0, e0+E_loc) are not local; -1 is
 * masked; ids < -1 or >= E set MOK_DEV_BAD_ID and are skipped.  Also clears the
 * device status word.  Must precede mok_moe_fwd with the same ids and workspace. */
mok_status_t mok_schedule(const mok_desc_t* desc, const int32_t* topk_ids, void* ws,
                          size_t ws_bytes, void* stream);

/* Copy the schedule tables out of the workspace (device to device, async on stream):
 * counts [E_loc], offsets [E_loc+1], perm [T*k] (entries >= R are unspecified),
 * pos [T*k], and hdr[4] = {R, number of minibatches, number of m-tiles, status}.
 * Any output pointer may be NULL to skip it. */
mok_status_t mok_schedule_tables(const mok_desc_t* desc, const void* ws, size_t ws_bytes,
                                 int32_t* counts, int32_t* offsets, int32_t* perm,
                                 int32_t* pos, int32_t* hdr, void* stream);

/* Quantise bf16 rows to MXFP8 ([L] section 03 names the MXFP8 mode; the block format is
 * OCP MX: e4m3 elements, one e8m0 scale per 32 elements).  src [rows, cols] bf16 (cols
 * a multiple of 32) -> codes [rows, cols] uint8, scales [rows, cols/32] uint8.  The
 * shared exponent is the smallest n with amax * 2^-n <= 448 (clamped to [-127, 127];
 * an all-zero block gets n = -127), code = e4m3 round-to-nearest-even of v * 2^-n,
 * saturating at 448.  The forward's dispatch quantises X rows with the same routine.
 * Used for the weights before a MXFP8 forward.  src and codes must be 16-byte aligned
 * (MOK_E_SHAPE otherwise).  Asynchronous on stream; the caller owns every buffer. */
mok_status_t mok_quantize_mx(const void* src_bf16, int64_t rows, int32_t cols, uint8_t* codes,
                             uint8_t* scales, void* stream);

/* Forward ([L] sections 02-03: dispatch, expert FFN, combine and the final weighted sum
 * in one persistent kernel; [M] design decisions).  y [T, D] bf16:
 *   y[t] = sum over slots j in ascending order with a local expert e = ids[t,j]-e0 of
 *          topk_w[t,j] * ( silu(x[t] W_gate[e]^T) * (x[t] W_up[e]^T) ) W_down[e]^T
 * accumulated in fp32, rounded once to bf16; tokens with no local slot get 0.
 * x [T, D] bf16; topk_ids [T, k] int32; topk_w [T, k] fp32; w_gate, w_up [E_loc, I, D];
 * w_down [E_loc, D, I]; all row-major.
 * bf16 mode: weights are bf16 (s_* must be NULL, MOK_E_SHAPE otherwise).
 * MXFP8 mode ([L] section 03): w_* point to e4m3 codes of the same shapes and s_* to
 * their e8m0 scales, s_gate and s_up [E_loc, I, D/32], s_down [E_loc, D, I/32] (from
 * mok_quantize_mx); X rows are quantised during dispatch and H inside the SwiGLU
 * epilogue (blocks of 32 along I); the products run on scaled MFMA with fp32
 * accumulation.  x, y and the weights must be 16-byte aligned and the scales 4-byte
 * aligned (MOK_E_SHAPE otherwise).  Requires a preceding mok_schedule on `ws`.
 * Asynchronous on stream. */
mok_status_t mok_moe_fwd(const mok_desc_t* desc, const void* x, const int32_t* topk_ids,
                         const float* topk_w, const void* w_gate, const void* w_up,
                         const void* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                         const uint8_t* s_down, void* y, void* ws, size_t ws_bytes,
                         void* stream);

/* Backward (bf16; MXFP8: mok_moe_bwd_mx) ([L] section 02: reverse-combine pulls dY,
 * reverse-dispatch pushes dX;
 * [M] design decisions: the ring is walked in reverse to limit replay of forward
 * activations, and the router-weight gradient is formed inside the SwiGLU backward).
 * Needs the workspace of a preceding mok_moe_fwd run with MOK_FLAG_SAVE_FOR_BWD and the
 * same inputs.  Outputs: dx [T, D] bf16, d_topk_w [T, k] fp32 (0 for non-local slots),
 * dw_gate, dw_up [E_loc, I, D] fp32 and dw_down [E_loc, D, I] fp32 (overwritten, not
 * accumulated; experts with no rows get 0).  dW sums over rows run in a fixed order.
 * Asynchronous on stream; every launch goes to `stream`.  dH, dX, dW and the sums back
 * to token order run as one persistent launch whose waits are bounded: should one
 * expire, the device status gets MOK_DEV_TIMEOUT (mok_read_device_status) and the
 * outputs are undefined; the next mok_schedule clears the status. */
mok_status_t mok_moe_bwd(const mok_desc_t* desc, const void* dy, const void* x,
                         const int32_t* topk_ids, const float* topk_w, const void* w_gate,
                         const void* w_up, const void* w_down, void* dx, float* d_topk_w,
                         float* dw_gate, float* dw_up, float* dw_down, void* ws,
                         size_t ws_bytes, void* stream);

/* Transposing MXFP8 quantiser for the backward's weight operands, whose contraction runs
 * over the stored rows ([L] section 03: the MXFP8 mode).  src [batch, rows, cols] bf16
 * (rows a multiple of 32) -> codes[b][c][r] = e4m3 code of src[b][r][c] at
 * codes + (b * cols + c) * ld_codes + r, and one e8m0 scale per 32 consecutive r at
 * scales + (b * cols + c) * ld_scales + r / 32; the same rule as mok_quantize_mx, so the
 * result equals mok_quantize_mx of each transposed matrix.  ld_codes >= rows and a
 * multiple of 16, ld_scales >= rows / 32; codes 16-byte aligned (MOK_E_SHAPE otherwise).
 * The MXFP8 backward takes
 *   wd_t  = W_down^T: mok_quantize_mx_t(w_down, E_loc, D, I, codes, D, scales, D / 32)
 *           -> codes [E_loc, I, D], scales [E_loc, I, D / 32];
 *   wgu_t = [W_gate; W_up]^T, row d = W_gate[:, d] then W_up[:, d]: two calls,
 *           (w_gate, E_loc, I, D, codes, 2I, scales, 2I / 32) and
 *           (w_up, E_loc, I, D, codes + I, 2I, scales + I / 32, 2I / 32)
 *           -> codes [E_loc, D, 2I], scales [E_loc, D, 2I / 32].
 * Asynchronous on stream; the caller owns every buffer. */
mok_status_t mok_quantize_mx_t(const void* src_bf16, int64_t batch, int32_t rows, int32_t cols,
                               uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                               int64_t ld_scales, void* stream);

/* MXFP8 backward ([L] section 03: MXFP8 forward and backward; [L] section 02 and [M]
 * design decisions as for mok_moe_bwd).  Needs the workspace of a preceding MXFP8
 * mok_moe_fwd run with MOK_FLAG_SAVE_FOR_BWD (which keeps a, b of every routed row) and
 * the same inputs; outputs and their layouts as for mok_moe_bwd.  The two data-gradient
 * GEMMs run on scaled e4m3 MFMA with fp32 accumulation, each operand quantised along
 * that GEMM's K in blocks of 32: u = dY W_down with dY rows quantised along D (inside the
 * call) and W_down^T codes wd_t / wd_t_scales; dx = [da | db] [W_gate; W_up] with
 * [da | db] rows quantised along I (inside the call) and wgu_t / wgu_t_scales (layouts
 * above, from mok_quantize_mx_t).  dG, da, db are formed from u as in mok_moe_bwd; the
 * weight gradients dW_gate = da^T x, dW_up = db^T x, dW_down = (g dY)^T h run in bf16
 * on the unquantised rows (x, dY bf16; da, db, g h rounded to bf16), fp32 accumulation.
 * dy, x, dx and the codes 16-byte aligned, the scales 4-byte aligned.  Errors as for
 * mok_moe_bwd; MOK_E_UNSUPPORTED unless desc is MXFP8 with MOK_FLAG_SAVE_FOR_BWD.
 * Asynchronous on stream. */
mok_status_t mok_moe_bwd_mx(const mok_desc_t* desc, const void* dy, const void* x,
                            const int32_t* topk_ids, const float* topk_w, const uint8_t* wd_t,
                            const uint8_t* wd_t_scales, const uint8_t* wgu_t,
                            const uint8_t* wgu_t_scales, void* dx, float* d_topk_w,
                            float* dw_gate, float* dw_up, float* dw_down, void* ws,
                            size_t ws_bytes, void* stream);

/* Where the trace of a forward run with MOK_FLAG_TRACE lies in the workspace (host
 * only): *offset_bytes from the workspace start, *words uint32 words.  Timestamps are
 * the low 32 bits of the GPU's 100 MHz constant clock (10 ns units).  The region holds
 *   tile records, 8 words per tile ticket t (t < the number of forward tiles):
 *     [workgroup, (minibatch << 1) | (1 for GEMM2, 0 for GEMM1), ticket taken,
 *      inputs ready (its wait ended), K loop done, signal done (the tile's stores
 *      complete and published), epilogue stores issued, 0];
 *   then workgroup records, 8 words per workgroup w (w < MOK_TRACE_MAX_WORKGROUPS):
 *     [start, minibatch 0 gathered (fill done), role done, drain done,
 *      role (1 comm, 0 compute), drain chunks taken, 0, 0].
 * The backward's records (which replace the forward's) use the same layout: per ticket
 *   [workgroup, kind (0 dH, 1 dX, 2 dW tile, 3 row-sum chunk, 4 MXFP8 quantisation of an
 *    m-tile's [da | db] rows), ticket taken, inputs
 *    ready, K loop (or sum) done, end, 0, 0], per workgroup [start, start, end, end, 0,
 *   tickets taken, 0, 0].  The region holds as many ticket records as the larger of the
 *   two launches has tickets.
 * With MOK_FLAG_UNFUSED the forward writes instead: words 0-3 = the number of
 * workgroups g0..g3 of its gather, GEMM1, GEMM2 and combine launches, words 4-7 = 0;
 * then, launch after launch, one record per workgroup of two 64-bit values of the same
 * clock (not truncated): its start and its end (taken once its memory operations have
 * completed).  A launch's time is its latest end minus its earliest start.
 * The caller reads the region after the forward has completed.  Errors: MOK_E_NULL,
 * the descriptor's errors, MOK_E_UNSUPPORTED when the flag is not set. */
#define MOK_TRACE_MAX_WORKGROUPS 1024
mok_status_t mok_trace_layout(const mok_desc_t* desc, size_t* offset_bytes, size_t* words);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): mok_schedule followed by mok_moe_fwd
 * in one call, same kernels and results, with the workspace taken from a static device
 * area of MOK_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on, from
 * the first call there until the process ends.  The call allocates nothing.
 * Arguments as for mok_moe_fwd (bf16 or MXFP8, same alignment rules), plus dev_status:
 * NULL, or a 4-byte-aligned device word that receives the call's MOK_DEV_* status bits.
 * Errors (returned before anything is enqueued): those of mok_moe_fwd; MOK_E_WORKSPACE
 * when mok_workspace_size(desc) exceeds MOK_NOALLOC_SCRATCH_BYTES; MOK_E_UNSUPPORTED with
 * MOK_FLAG_SAVE_FOR_BWD or MOK_FLAG_TRACE (their results would stay in the area).
 * Every call on a GPU uses that GPU's one area, which keeps the last call's contents:
 * calls that overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  Asynchronous on stream. */
#define MOK_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
mok_status_t mok_moe_fwd_noalloc(const mok_desc_t* desc, const void* x, const int32_t* topk_ids,
                                 const float* topk_w, const void* w_gate, const void* w_up,
                                 const void* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                                 const uint8_t* s_down, void* y, uint32_t* dev_status,
                                 void* stream);

/* Synchronise `stream`, then read the sticky device status word (MOK_DEV_* bits). */
mok_status_t mok_read_device_status(const void* ws, void* stream, uint32_t* out);

/* Static text for a status code. */
const char* mok_status_string(mok_status_t s);

/* Number of compute units of the current device (0 on error); a helper for choosing
 * comm_cus. */
int32_t mok_device_cus(void);

#ifdef __cplusplus
}
#endif
#endif /* MOK_H */
