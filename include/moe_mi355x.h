/*
 * moe_mi355x.h -- C ABI of the MI355X (gfx950) MoE dispatch / combine library.
 *
 * One GPU's share of expert-parallel token dispatch and combine in the
 * "expanded layout": one row per (token, local expert) slot, rows grouped by
 * local expert, each row carrying that slot's routing weight; the combine sums
 * rows back to token order.  Sources:
 *   - "Add the deepep expert-parallel implementation" (huggingface/transformers
 *     pull request 49638), section "What this adds": bullets "Expanded layout",
 *     "Eager vs captured", "Custom ops", "Training", "Buffers", and the
 *     requirements paragraph (hidden size a multiple of 256);
 *   - "feat: add hybridep" (NVIDIA-NeMo/Automodel pull request 1333): Changelog
 *     (top-k indices converted to multihot routing metadata) and the reviewed
 *     HybridEP dispatch call (routing_map, fp32 probs, num_local_experts,
 *     pad_multiple in; dispatched rows, dispatched probs, tokens_per_expert and
 *     a handle out).
 *
 * Conventions for every entry point
 *   - All tensors are caller-allocated; the library never allocates device
 *     memory.  "device" pointers are HIP device (or managed) memory on the
 *     current device; "host" pointers are host memory.
 *   - State kept between calls: per host thread, the message of
 *     moe_last_error() and a pending moe_time_next_call() request (consumed
 *     by the next call); per GPU, the fixed route scratch array of
 *     moe_route_build_noalloc (with its device address, resolved on the
 *     first such call).  Nothing else outlives a call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every launch goes on that stream.
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, and every
 *     row pointer must be 16-byte aligned.
 *   - Return value is a moe_status; on failure moe_last_error() names the
 *     violated requirement.  Argument errors are detected on the host before
 *     anything is launched.  Nothing throws.  A problem too large for one
 *     launch (a kernel grid past 2^32 work-items, which the dispatch packet
 *     cannot hold: row arrays past about 64 GiB) is one such error,
 *     MOE_ERR_ARG.
 *   - Only the eager route calls (moe_route_build, moe_route_build_noalloc
 *     and moe_route_dispatch in MOE_EAGER mode) wait for the device, once
 *     each, to read the row count back ("Eager vs captured").  Every other
 *     call, and every call in MOE_SYNC_FREE mode, is asynchronous,
 *     allocation-free and safe to record into a HIP graph ("Custom ops",
 *     "Buffers").
 *   - Calls that share output buffers must not overlap; calls on different
 *     buffers may run concurrently.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_ARG = 1,       /* bad sizes, null or misaligned pointers, bad flags */
    MOE_ERR_HIDDEN = 2,    /* H <= 0 or H % 256 != 0 (requirements paragraph) */
    MOE_ERR_CAPACITY = 3,  /* sync-free capacity below the worst case */
    MOE_ERR_WORKSPACE = 4, /* workspace null or smaller than moe_route_workspace_size */
    MOE_ERR_INDEX = 5,     /* eager: an expert id outside [-1, E) was seen (and dropped) */
    MOE_ERR_HIP = 6,       /* a HIP runtime call failed */
    MOE_ERR_DEVICE = 7     /* no usable gfx950 device */
} moe_status;

typedef enum moe_mode {
    /* Row count read back to the host; the caller sizes rows to exactly
     * `total` ("Eager vs captured", eager half). */
    MOE_EAGER = 0,
    /* No host sync: rows sized for the worst case (`capacity`); rows past the
     * device-side total are zero and belong to the sentinel expert
     * `num_local` ("Eager vs captured", captured half). */
    MOE_SYNC_FREE = 1
} moe_mode;

/* Bits of handle.status[1]. */
enum {
    MOE_FLAG_BAD_ID = 1,      /* an id outside [-1, E); the slot was treated as -1 */
    MOE_FLAG_DUPLICATE = 2,   /* a token named the same expert twice; the slots were merged */
    MOE_FLAG_ROWS_MISMATCH = 4 /* eager: R passed to dispatch/combine != device total */
};

/* Problem description, shared by every call of one layer. */
typedef struct moe_desc {
    int64_t T;            /* tokens (>= 0) */
    int32_t k;            /* slots per token, 1..64 (top-k) */
    int32_t E;            /* global experts (>= 1) */
    int32_t local_begin;  /* first local expert lb */
    int32_t num_local;    /* local experts EL, 1..1024, lb + EL <= E */
    int32_t pad_multiple; /* P >= 1: each expert's row group is padded to a multiple of P */
    int32_t mode;         /* moe_mode */
    int32_t idx_is_i64;   /* 0: topk_idx is int32 [T,k]; 1: int64 [T,k] */
    int32_t reserved;     /* must be 0 */
    int64_t capacity;     /* MOE_SYNC_FREE: rows C >= T*min(k,EL) + EL*(P-1); else ignored */
} moe_desc;

/* The dispatch handle: plain device buffers, so it can travel through an op
 * boundary as tensors and be rebuilt ("Custom ops").  Caller-owned; written by
 * moe_route_build and read by the calls after it, so it must stay alive and
 * unchanged until the last of them has run on the stream. */
typedef struct moe_handle {
    uint8_t *routing_map;       /* [T,E] u8 multihot map, or NULL to skip writing it */
    int32_t *tokens_per_expert; /* [EL] exact (unpadded) routes per local expert */
    int32_t *padded_offsets;    /* [EL+1] first row of each expert's group; [EL] = total */
    int32_t *row_of_slot;       /* [T,k] row of each slot, -1 if invalid or not local;
                                   repeated ids point at the first slot's row */
    int32_t *status;            /* [4] {total, flags (MOE_FLAG_*), data rows, 0} */
    void *workspace;            /* >= moe_route_workspace_size(desc) bytes of device
                                   memory: the route's scratch (per-block counts)
                                   and, for dense routing, its row list (below);
                                   the calls after the route accept NULL */
    size_t workspace_bytes;
} moe_handle;

/* Smallest legal sync-free capacity: T*min(k,EL) + EL*(P-1) (worst case: every
 * token routes all of its slots locally and every group needs P-1 pad rows). */
int64_t moe_capacity_min(const moe_desc *desc);

/* Device bytes of handle.workspace for this description (0 if the description
 * is invalid): the route's scratch, about ceil(T/floor(B/k)) * (EL + 1) * 4
 * bytes (route blocks of B = 512 slots up to 512 local experts, else 256; a
 * route of T <= floor(1024/k) tokens with EL <= 256, or T <= floor(2048/k)
 * with EL <= 64, is one block), plus the row list when the route writes one.
 *
 * The row list: for dense routing the route also writes, into the workspace,
 * every row's (row, token) pair, grouped by tiles of about 512 tokens and
 * dealt over the GPU's 8 XCDs, rows of a tile in address order.
 * moe_dispatch and moe_combine_bwd then walk that list instead of the tokens
 * when the handle they get brings this workspace: each XCD's L2 holds its
 * tiles' token rows while the expert rows stream past.  Results are the
 * same either way.  The route writes the list when it takes more than one
 * route block, (route blocks) * EL <= 65536, and k * EL >= 2 * E
 * (under uniform routing a token then has two or more local slots); it
 * takes about 8 * T * min(k, EL) bytes, rounded up to whole tiles on every
 * XCD.  The list belongs to the handle: a route written through another
 * handle that shares this workspace replaces it.  moe_route_build_noalloc
 * writes no list (its handles have no workspace). */
size_t moe_route_workspace_size(const moe_desc *desc);

/*
 * Routing preprocessing: top-k ids -> multihot map, tokens_per_expert, padded
 * offsets and the row of every slot ("feat: add hybridep", Changelog: top-k
 * indices to multihot routing metadata; dispatch hunk: tokens_per_expert,
 * pad_multiple).
 *   topk_idx        device [T,k] int32 or int64 (desc->idx_is_i64); -1 = empty
 *                   slot; any other id outside [-1, E) is dropped and flagged.
 *   topk_w          device [T,k] fp32 or NULL; needed only for multihot_probs.
 *   multihot_probs  device [T,E] fp32 or NULL: the routed weight at each routed
 *                   expert (repeated ids summed in slot order), 0 elsewhere.
 *   handle          outputs (see moe_handle); status is fully rewritten; its
 *                   workspace must hold moe_route_workspace_size bytes.
 *   host_status     host int32[4]: MOE_EAGER receives {total, flags, data rows, 0}
 *                   before the call returns.  Pinned (device-visible) memory is
 *                   written by the route kernel directly and the call waits
 *                   only for that write; the handle's device tensors are then
 *                   complete in stream order (work queued next on the same
 *                   stream sees them).  Pageable memory gets a copy and one
 *                   stream sync.  MOE_SYNC_FREE: unused, may be NULL.
 * Rows inside an expert's group are in ascending token order.  Returns
 * MOE_ERR_INDEX in eager mode when MOE_FLAG_BAD_ID is set (outputs valid).
 */
int moe_route_build(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                    float *multihot_probs, const moe_handle *handle, int32_t *host_status,
                    void *stream);

/* Bytes of the fixed route scratch array that moe_route_build_noalloc uses
 * on each GPU (4 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES 4194304u

/*
 * moe_route_build for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  Its
 * outputs, errors and waits are exactly moe_route_build's; the difference is
 * where the route's scratch (per-block expert counts and flags) lives:
 *   - in a fixed array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one
 *     per GPU, held by every GPU the library runs on until the process ends;
 *   - handle.workspace must be NULL and handle.workspace_bytes 0 (else
 *     MOE_ERR_ARG: the buffer would be ignored);
 *   - a route whose scratch, moe_route_workspace_size(desc), would exceed the
 *     array returns MOE_ERR_WORKSPACE before anything is launched (with
 *     512-thread route blocks that is about T*k*EL/128 bytes: 4 Mi slots of
 *     top-k at 128 local experts, 256 Ki slots at 1024);
 *   - the call allocates nothing, host or device.  The first call on a device
 *     resolves the array's device address on the current device (a symbol
 *     lookup, no allocation); make that first call outside graph capture.
 * Every call on one GPU shares that GPU's array and finds there whatever the
 * last call left (no word of it needs to start at zero: each route writes its
 * scratch before reading it).  Calls whose kernels may overlap on one GPU
 * (different streams or host threads without ordering between them) race on
 * the array and give wrong results: order them, e.g. on one stream.
 */
int moe_route_build_noalloc(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                            float *multihot_probs, const moe_handle *handle,
                            int32_t *host_status, void *stream);

/*
 * Dispatch into the expanded layout ("Expanded layout"; "Eager vs captured").
 *   x           device [T,H] bf16 token rows.
 *   H           hidden size, a positive multiple of 256.
 *   topk_w      device [T,k] fp32 routing weights, or NULL (then row_w must be NULL).
 *   R           rows: MOE_EAGER = host total from moe_route_build;
 *               MOE_SYNC_FREE = desc->capacity.
 *   rows        device [R,H] bf16 out: row r = x[row_token[r]] bit for bit; pad
 *               rows and rows >= total are zero.
 *   row_w       device [R] fp32 out (the dispatched probs) or NULL: the slot's
 *               weight (repeated ids summed), 0 on pad and sentinel rows.
 *   row_token   device [R] int32 out or NULL: source token, -1 on pad/sentinel.
 *   row_expert  device [R] int32 out or NULL: local expert of the row; pad rows
 *               carry their group's expert, rows >= total the sentinel num_local.
 * Writes never go past R.  In eager mode a device total != R sets
 * MOE_FLAG_ROWS_MISMATCH (and rows in [total, R) are written as sentinel rows).
 */
int moe_dispatch(const moe_desc *desc, const moe_handle *handle, const uint16_t *x, int32_t H,
                 const float *topk_w, int64_t R, uint16_t *rows, float *row_w,
                 int32_t *row_token, int32_t *row_expert, void *stream);

/*
 * Route and dispatch in one call ("Eager vs captured").  Every argument of
 * both halves is checked before anything is launched; the handle's
 * workspace rules are moe_route_build's.
 *   topk_idx, multihot_probs, handle: as for moe_route_build.
 *   topk_w         device [T,k] fp32 or NULL: read for multihot_probs and for
 *                  row_w, and needed by either.
 *   x, H           as for moe_dispatch.
 *   rows           device [R_cap,H] bf16 out; row_w, row_token, row_expert:
 *                  device [R_cap] out or NULL.
 * MOE_EAGER (the eager mode's one readback, taken off the device's critical
 * path), for callers whose row buffers hold the worst case, such as a loop
 * over persistent buffers:
 *   R_cap          rows the buffers hold, >= moe_capacity_min(desc), else
 *                  MOE_ERR_CAPACITY.
 *   host_status    as for moe_route_build.
 * The dispatch is queued right behind the route, before the row count is
 * read back.  So the device goes from the route to the dispatch without
 * waiting for the host, while the host waits for the count as
 * moe_route_build does.  On return host_status holds {total, flags, data
 * rows} as after moe_route_build, and rows [0, total) of every output are
 * exactly what moe_dispatch with R = total writes.  Rows at or past total
 * are not written.  An out-of-range id returns MOE_ERR_INDEX after the
 * readback, as moe_route_build does; the dispatch has then still run, with
 * such slots treated as empty.
 * MOE_SYNC_FREE (nothing waits; safe to record into a HIP graph):
 *   R_cap          must equal desc->capacity (else MOE_ERR_ARG).
 *   host_status    unused, may be NULL.
 * The handle and every row are exactly what moe_route_build followed by
 * moe_dispatch with R = capacity write.  A route of at most 16 slots
 * (T*k <= 16: decode sizes) whose row array is small (at most 32 MiB) and
 * whose multihot map has at most 65536 entries runs in the dispatch's own
 * launch: each workgroup computes that small route itself, so the pair
 * costs one kernel launch instead of two.
 */
int moe_route_dispatch(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                       float *multihot_probs, const moe_handle *handle, int32_t *host_status,
                       const uint16_t *x, int32_t H, int64_t R_cap, uint16_t *rows, float *row_w,
                       int32_t *row_token, int32_t *row_expert, void *stream);

/*
 * FP8 dispatch ("What this adds": FP8 dispatch, named there as a follow-up
 * that halves the dispatched bytes; the page fixes no format, this library
 * takes the following one).  As moe_dispatch, except that each row holds the
 * token's row quantized to 8-bit floats:
 *   rows_q      device [R,H] uint8 out: OCP E4M3 codes ("e4m3fn": bias 7, no
 *               infinities, largest finite 448).
 *   row_scale   device [R,H/128] fp32 out: one scale per 128 consecutive
 *               elements, so that x ~= value(rows_q) * row_scale.
 * Per token and block of 128 elements:
 *   a = max(max|x|, 1e-4); scale = a / 448; q = e4m3(clamp(x * (448 / a),
 *   -448, 448)), each fp32 operation rounded to nearest-even and e4m3()
 *   the nearest code, ties to even (so a block's largest magnitude maps to
 *   +-448).  Pad rows and rows >= total are zero bytes with scale 0.
 * The token is quantized once and its codes written to each of its rows.
 * x must be finite (for NaN or infinite elements the codes are unspecified).
 * rows_q and row_scale must be 16-byte aligned; row_w, row_token, row_expert,
 * errors and flags are those of moe_dispatch.
 */
int moe_dispatch_fp8(const moe_desc *desc, const moe_handle *handle, const uint16_t *x, int32_t H,
                     const float *topk_w, int64_t R, uint8_t *rows_q, float *row_scale,
                     float *row_w, int32_t *row_token, int32_t *row_expert, void *stream);

/*
 * Combine: out[t] = sum of Y[row] over t's distinct local slots, in ascending
 * slot order, in fp32 (the accumulator starts from the first term).  No
 * weight is applied here: in the expanded layout the experts weight their
 * own rows and the combine is a plain sum ("Expanded layout").  A token with
 * no local slot gets +0.
 *   Y           device [R,H] bf16 expert outputs.
 *   out         device [T,H]: bf16 rounded to nearest-even (NaN -> 0x7FC0) when
 *               out_is_f32 == 0, fp32 when out_is_f32 == 1.
 */
int moe_combine(const moe_desc *desc, const moe_handle *handle, const uint16_t *Y, int32_t H,
                int64_t R, void *out, int32_t out_is_f32, void *stream);

/*
 * Combine backward = a cached dispatch of grad_out along the forward's rows
 * ("Custom ops": the combine's backward is a cached dispatch), plus the
 * routing-weight gradients ("Training").
 *   grad_out    device [T,H] bf16.
 *   expert_out  device [R,H] bf16 expert outputs before the routing weight is
 *               applied, or NULL (then dw must be NULL).
 *   grad_rows   device [R,H] bf16 out: grad_out[row_token[r]]; pad and
 *               sentinel rows zero.
 *   dw          device [T,k] fp32 out or NULL: dot(grad_out[t], expert_out[row
 *               of slot (t,j)]) with exact products and an fp64 sum, rounded
 *               once to fp32; repeated ids share the value; 0 for slots that
 *               are empty or not local.
 */
int moe_combine_bwd(const moe_desc *desc, const moe_handle *handle, const uint16_t *grad_out,
                    const uint16_t *expert_out, int32_t H, int64_t R, uint16_t *grad_rows,
                    float *dw, void *stream);

/*
 * Dispatch backward ("Training": gradients reach the tokens and the routing
 * weights, the weight gradients going back through a combine).  The adjoint of
 * moe_dispatch along the same handle:
 *   grad_rows    device [R,H] bf16 gradients of the dispatched rows.
 *   grad_row_w   device [R] fp32 gradients of the dispatched probs (row_w), or
 *                NULL (then grad_topk_w must be NULL, unless R == 0).
 *   grad_x       device [T,H] out: the sum of grad_rows over t's distinct local
 *                slots in ascending slot order, fp32 adds, bf16 RNE
 *                (grad_x_is_f32 == 0) or fp32; +0 for a token without a local
 *                slot -- exactly moe_combine of grad_rows.
 *   grad_topk_w  device [T,k] fp32 out or NULL: grad_row_w of the slot's row for
 *                every local slot (repeated ids each get their row's value), 0
 *                for empty or non-local slots.
 */
int moe_dispatch_bwd(const moe_desc *desc, const moe_handle *handle, const uint16_t *grad_rows,
                     int32_t H, int64_t R, const float *grad_row_w, void *grad_x,
                     int32_t grad_x_is_f32, float *grad_topk_w, void *stream);

/* Message of the last failing call on this thread ("" if none). */
const char *moe_last_error(void);

/* MOE_OK if `device` is a gfx950 GPU the library can run on; otherwise
 * MOE_ERR_DEVICE (or MOE_ERR_HIP) with the reason in moe_last_error().
 * Does not launch anything. */
int moe_device_check(int device);

/* Kernel timing, for callers that measure the library (a benchmark, a
 * profiler hook).  The next moe_route_build, moe_route_build_noalloc,
 * moe_route_dispatch, moe_dispatch, moe_dispatch_fp8, moe_combine,
 * moe_combine_bwd or moe_dispatch_bwd call made on this host thread times
 * its own kernels into two HIP events:
 *   start_event  hipEvent_t (created by the caller, timing enabled) or NULL:
 *                takes the start time of the call's first kernel.
 *   stop_event   hipEvent_t or NULL: takes the end time of the call's last
 *                kernel.
 * hipEventElapsedTime(start, stop) then gives the device time of that call's
 * kernels.  The events are attached to the kernels' own dispatch packets, so
 * unlike hipEventRecord around the call they add no packet, and no gap, to
 * the stream.  Events created with hipEventDisableSystemFence suit this use
 * best: without it, each event's completion writes back the caches at system
 * scope, which delays the next kernel by a few microseconds.
 * The request is dropped when that call returns, whether or not
 * it launched anything (a call that fails or has nothing to launch leaves the
 * events as they were).  Events stay owned by the caller.  Returns MOE_OK. */
int moe_time_next_call(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
