// api.hip -- the C ABI of libmoe_mi355x (declared in include/moe_mi355x.h).
//
// Host side only: argument checks (all before any launch), launch geometry,
// and the one host readback of eager routing.  Requirements it enforces come
// from "Add the deepep expert-parallel implementation": hidden size a
// multiple of 256 (requirements paragraph), worst-case sync-free capacity
// ("Eager vs captured"), nothing allocated and no sync on the sync-free path
// ("Buffers", "Custom ops"); and from the review on "feat: add hybridep" that
// accepted flags must not be silently ignored (every optional argument either
// takes effect or is rejected).
#include "moe_mi355x.h"
#include "moe_internal.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <chrono>
#include <mutex>
#include <thread>

// The host's wait for the eager row count spins on a word of pinned memory;
// the spin hint is the x86 pause where there is one, a yield elsewhere.
static inline void spin_hint()
{
#if defined(__x86_64__) || defined(__i386__)
    __builtin_ia32_pause();
#else
    std::this_thread::yield();
#endif
}

namespace {

thread_local char g_err[512] = "";

// Drops the calling thread's timing request when an entry point returns, so
// that a request applies to one call only.
struct TimingScope {
    ~TimingScope() { moe::launch_timing() = moe::LaunchTiming{}; }
};

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = '\0';
    return MOE_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t cap_min(const moe_desc *d)
{
    const int64_t kk = d->k < d->num_local ? d->k : d->num_local;
    return d->T * kk + static_cast<int64_t>(d->num_local) * (d->pad_multiple - 1);
}

constexpr int64_t kI32Max = 2147483647;

int check_desc(const moe_desc *d)
{
    if (!d)
        return fail(MOE_ERR_ARG, "desc is NULL");
    if (d->T < 0)
        return fail(MOE_ERR_ARG, "T must be >= 0 (got %lld)", (long long)d->T);
    if (d->k < 1 || d->k > moe::kMaxK)
        return fail(MOE_ERR_ARG, "k must be in [1, %d] (got %d)", moe::kMaxK, d->k);
    if (d->E < 1)
        return fail(MOE_ERR_ARG, "E must be >= 1 (got %d)", d->E);
    if (d->pad_multiple < 1)
        return fail(MOE_ERR_ARG, "pad_multiple must be >= 1 (got %d)", d->pad_multiple);
    if (d->local_begin < 0 || d->num_local < 1 ||
        static_cast<int64_t>(d->local_begin) + d->num_local > d->E)
        return fail(MOE_ERR_ARG, "local experts [%d, %d+%d) must lie inside [0, E=%d) and be non-empty",
                    d->local_begin, d->local_begin, d->num_local, d->E);
    if (d->num_local > moe::kMaxLocal)
        return fail(MOE_ERR_ARG, "num_local must be <= %d (got %d)", moe::kMaxLocal, d->num_local);
    if (d->mode != MOE_EAGER && d->mode != MOE_SYNC_FREE)
        return fail(MOE_ERR_ARG, "mode must be MOE_EAGER (0) or MOE_SYNC_FREE (1) (got %d)", d->mode);
    if (d->idx_is_i64 != 0 && d->idx_is_i64 != 1)
        return fail(MOE_ERR_ARG, "idx_is_i64 must be 0 or 1 (got %d)", d->idx_is_i64);
    if (d->reserved != 0)
        return fail(MOE_ERR_ARG, "reserved must be 0");
    if (d->T > kI32Max || d->T * d->k > kI32Max || cap_min(d) > kI32Max)
        return fail(MOE_ERR_ARG, "T*k and the worst-case row count must fit in int32");
    if (d->mode == MOE_SYNC_FREE) {
        if (d->capacity < cap_min(d))
            return fail(MOE_ERR_CAPACITY,
                        "sync-free capacity %lld is below the worst case T*min(k,EL) + EL*(P-1) = %lld",
                        (long long)d->capacity, (long long)cap_min(d));
        if (d->capacity > kI32Max)
            return fail(MOE_ERR_ARG, "capacity must fit in int32");
    }
    return MOE_OK;
}

struct WsLayout {
    size_t counts_off, flags_off, pairs_off, bytes;
    bool pairs;          // the route writes its row list at pairs_off
    moe::PairGeom pg;
};

// The handle's workspace: route scratch (per-block expert counts and flags)
// and, for dense routing, the route's row list, which the dispatch and the
// combine backward read.  with_pairs = false: the scratch alone (the fixed
// array of moe_route_build_noalloc).
WsLayout ws_layout(const moe_desc *d, bool with_pairs = true)
{
    const moe::RouteGeom g = moe::route_geom(d->T, d->k, d->num_local);
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    WsLayout w;
    w.counts_off = 0;
    w.flags_off = up(static_cast<size_t>(g.nblk) * d->num_local * sizeof(int32_t));
    w.pairs_off = w.flags_off + up(static_cast<size_t>(g.nblk) * sizeof(int32_t));
    w.bytes = w.pairs_off;
    w.pairs = with_pairs && moe::pairs_form(d->T, d->k, d->E, d->num_local, g.tokens_per_block,
                                            g.nblk);
    if (w.pairs) {
        w.pg = moe::pair_geom(d->T, d->k, d->num_local, g.tokens_per_block, g.nblk);
        w.bytes += up(static_cast<size_t>(w.pg.entries) * sizeof(int2));
    }
    if (w.bytes == 0)
        w.bytes = 256;
    return w;
}

// The route's row list in a handle, for the row kernels: present when the
// description's route writes one and the handle brings a workspace large
// enough to hold it (handles without a workspace walk tokens).
const int2 *handle_pairs(const moe_desc *d, const moe_handle *h, moe::PairGeom &pg)
{
    const WsLayout wl = ws_layout(d);
    if (!wl.pairs || !h->workspace || h->workspace_bytes < wl.bytes)
        return nullptr;
    pg = wl.pg;
    return reinterpret_cast<const int2 *>(static_cast<const char *>(h->workspace) + wl.pairs_off);
}

// The route needs the workspace (need_ws; with room for its row list unless
// pairs is false); the calls after it read the row list when it is there and
// walk tokens otherwise, so only the route checks the workspace.
int check_handle(const moe_desc *d, const moe_handle *h, bool need_ws = false, bool pairs = true)
{
    if (!h)
        return fail(MOE_ERR_ARG, "handle is NULL");
    if (need_ws) {
        const WsLayout wl = ws_layout(d, pairs);
        if (!h->workspace || h->workspace_bytes < wl.bytes)
            return fail(MOE_ERR_WORKSPACE, "handle.workspace needs %zu bytes (got %zu%s)", wl.bytes,
                        h->workspace_bytes, h->workspace ? "" : ", NULL");
    }
    if (!h->tokens_per_expert || !h->padded_offsets || !h->status)
        return fail(MOE_ERR_ARG, "handle tensors tokens_per_expert, padded_offsets and status must be "
                                 "non-NULL");
    if (d->T > 0 && !h->row_of_slot)
        return fail(MOE_ERR_ARG, "handle.row_of_slot must be non-NULL when T > 0");
    return MOE_OK;
}

int check_hidden(int32_t H)
{
    if (H <= 0 || H % 256 != 0)
        return fail(MOE_ERR_HIDDEN, "hidden size H must be a positive multiple of 256 (got %d)", H);
    return MOE_OK;
}

int check_rows(const moe_desc *d, int64_t R)
{
    if (d->mode == MOE_SYNC_FREE) {
        if (R != d->capacity)
            return fail(MOE_ERR_ARG, "sync-free mode: R must equal desc->capacity (%lld), got %lld",
                        (long long)d->capacity, (long long)R);
    } else if (R < 0 || R > kI32Max) {
        return fail(MOE_ERR_ARG, "R must be in [0, 2^31) (got %lld)", (long long)R);
    }
    return MOE_OK;
}

int hip_fail(hipError_t e, const char *what)
{
    // the launchers' own refusal of a grid past 2^32 work-items (no HIP call made)
    if (e == hipErrorInvalidConfiguration)
        return fail(MOE_ERR_ARG, "%s: the problem is too large for one launch (its grid would pass "
                                 "2^32 work-items)", what);
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}



// Argument rules shared by the bf16 and the FP8 dispatch.
int check_dispatch(const moe_desc *desc, const moe_handle *handle, const uint16_t *x, int32_t H,
                   const float *topk_w, int64_t R, const float *row_w)
{
    int rc;
    if ((rc = check_desc(desc)) != MOE_OK)
        return rc;
    if ((rc = check_handle(desc, handle)) != MOE_OK)
        return rc;
    if ((rc = check_hidden(H)) != MOE_OK)
        return rc;
    if ((rc = check_rows(desc, R)) != MOE_OK)
        return rc;
    if (desc->T > 0 && (!x || !aligned16(x)))
        return fail(MOE_ERR_ARG, "x must be a non-NULL, 16-byte aligned [T,H] bf16 tensor");
    if (row_w && !topk_w && desc->T > 0)
        return fail(MOE_ERR_ARG, "row_w requested without topk_w");
    if (topk_w && !row_w)
        return fail(MOE_ERR_ARG, "topk_w given but row_w is NULL (the weights would be ignored)");
    return MOE_OK;
}

// One launch of the dispatch: bf16 rows, or (rows_q set) E4M3 rows and scales.
// The arguments and launch shape of one dispatch: bf16 rows, or (rows_q set)
// E4M3 rows and scales.
moe::RowArgs dispatch_args(const moe_desc *desc, const moe_handle *handle, const uint16_t *x,
                           int32_t H, const float *topk_w, int64_t R, uint16_t *rows,
                           uint8_t *rows_q, float *row_scale, float *row_w, int32_t *row_token,
                           int32_t *row_expert, bool keep_tail)
{
    moe::RowArgs a;
    a.keep_tail = keep_tail;
    a.src = x;
    a.topk_w = topk_w;
    a.F = nullptr;
    a.rows = rows;
    a.rows_q = rows_q;
    a.row_scale = row_scale;
    a.row_w = row_w;
    a.row_token = row_token;
    a.row_expert = row_expert;
    a.dw = nullptr;
    a.row_of_slot = handle->row_of_slot;
    a.tpe = handle->tokens_per_expert;
    a.off = handle->padded_offsets;
    a.status = handle->status;
    a.T = desc->T;
    a.R = R;
    a.k = desc->k;
    a.EL = desc->num_local;
    a.E_total = desc->E;
    a.P = desc->pad_multiple;
    a.H = H;
    a.eager = desc->mode == MOE_EAGER;
    a.pairs = rows_q ? nullptr : handle_pairs(desc, handle, a.pg);
    moe::row_shape(a);
    return a;
}

// One launch of the dispatch.
int launch_dispatch(const moe_desc *desc, const moe_handle *handle, const uint16_t *x, int32_t H,
                    const float *topk_w, int64_t R, uint16_t *rows, uint8_t *rows_q,
                    float *row_scale, float *row_w, int32_t *row_token, int32_t *row_expert,
                    void *stream)
{
    const moe::RowArgs a = dispatch_args(desc, handle, x, H, topk_w, R, rows, rows_q, row_scale,
                                         row_w, row_token, row_expert, false);
    hipError_t e = moe::launch_move_rows(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, rows_q ? "fp8 dispatch launch" : "dispatch launch");
    return ok();
}

}  // namespace

extern "C" {

int64_t moe_capacity_min(const moe_desc *desc)
{
    if (!desc)
        return -1;
    return cap_min(desc);
}

size_t moe_route_workspace_size(const moe_desc *desc)
{
    if (check_desc(desc) != MOE_OK)
        return 0;
    return ws_layout(desc).bytes;
}

}  // extern "C"

namespace {

// The route's argument rules; need_ws: the handle brings the workspace.
int route_check(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                const float *multihot_probs, const moe_handle *handle,
                const int32_t *host_status, bool need_ws, bool pairs = true)
{
    int rc;
    if ((rc = check_desc(desc)) != MOE_OK)
        return rc;
    if ((rc = check_handle(desc, handle, need_ws, pairs)) != MOE_OK)
        return rc;
    if (desc->T > 0 && !topk_idx)
        return fail(MOE_ERR_ARG, "topk_idx is NULL");
    if (multihot_probs && !topk_w)
        return fail(MOE_ERR_ARG, "multihot_probs requested without topk_w");
    if (topk_w && !multihot_probs)
        return fail(MOE_ERR_ARG, "topk_w given but multihot_probs is NULL: route_build only reads "
                                 "weights to write multihot_probs (pass weights to moe_dispatch)");
    if (desc->mode == MOE_EAGER && !host_status)
        return fail(MOE_ERR_ARG, "eager mode needs host_status (int32[4]) to return the row count");
    return MOE_OK;
}

// The route's kernel arguments (device side only; the eager host status is
// set up by route_launch).  pairs: write the row list (when the description
// has one) into the workspace.
moe::RouteGeom route_args(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                          float *multihot_probs, const moe_handle *handle, moe::RouteArgs &a,
                          bool pairs = true)
{
    const WsLayout wl = ws_layout(desc, pairs);
    char *workspace = static_cast<char *>(handle->workspace);
    const moe::RouteGeom g = moe::route_geom(desc->T, desc->k, desc->num_local);
    a.idx = topk_idx;
    a.w = topk_w;
    a.probs = multihot_probs;
    a.map = handle->routing_map;
    a.row_of_slot = handle->row_of_slot;
    a.counts = reinterpret_cast<int32_t *>(workspace + wl.counts_off);
    a.blockflags = reinterpret_cast<int32_t *>(workspace + wl.flags_off);
    a.tpe = handle->tokens_per_expert;
    a.off = handle->padded_offsets;
    a.status = handle->status;
    a.T = desc->T;
    a.k = desc->k;
    a.E = desc->E;
    a.lb = desc->local_begin;
    a.EL = desc->num_local;
    a.P = desc->pad_multiple;
    a.tokens_per_block = g.tokens_per_block;
    a.slots = g.slots;
    a.nblk = g.nblk;
    a.idx_i64 = desc->idx_is_i64;
    a.host_status = nullptr;
    a.pairs = nullptr;
    if (wl.pairs) {
        a.pairs = reinterpret_cast<int2 *>(workspace + wl.pairs_off);
        a.pg = wl.pg;
    }
    return g;
}

// The route's checks and launches.  `a` keeps what route_wait needs.
int route_launch(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                 float *multihot_probs, const moe_handle *handle, int32_t *host_status,
                 void *stream, moe::RouteArgs &a, bool pairs = true)
{
    int rc;
    if ((rc = route_check(desc, topk_idx, topk_w, multihot_probs, handle, host_status, true,
                          pairs)) != MOE_OK)
        return rc;
    const moe::RouteGeom g = route_args(desc, topk_idx, topk_w, multihot_probs, handle, a, pairs);
    if (desc->mode == MOE_EAGER) {
        // Pinned (device-visible) host memory: the kernel writes the status
        // there directly; pageable memory takes a copy after the kernels.
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, host_status) == hipSuccess &&
            attr.type == hipMemoryTypeHost && attr.devicePointer)
            a.host_status = static_cast<int32_t *>(attr.devicePointer);
        else
            (void)hipGetLastError(); // an unregistered pointer is not an error here
    }
    if (a.host_status)
        static_cast<volatile int32_t *>(host_status)[3] = -1; // the kernel turns it to 0 last
    hipError_t e = moe::launch_route(a, g.threads, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "route launch");
    return MOE_OK;
}

// Eager mode: "Eager vs captured" -- the counts come back to the host once.
// With a device-visible status the host waits only for that word (a bounded
// spin, then a stream sync); the rest of the route, and whatever was queued
// after it, runs on.  Pageable memory takes a copy and a stream sync.
int route_wait(const moe_handle *handle, int32_t *host_status, void *stream,
               const moe::RouteArgs &a)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    volatile int32_t *hs = host_status;
    hipError_t e;
    bool ready = false;
    if (a.host_status) {
        const auto t0 = std::chrono::steady_clock::now();
        while (!(ready = (hs[3] == 0))) {
            spin_hint();
            if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(5))
                break;
        }
    } else if ((e = hipMemcpyAsync(host_status, handle->status, 4 * sizeof(int32_t),
                                   hipMemcpyDeviceToHost, s)) != hipSuccess) {
        return hip_fail(e, "status readback");
    }
    if (!ready && (e = hipStreamSynchronize(s)) != hipSuccess)
        return hip_fail(e, "stream sync");
    return MOE_OK;
}

// Eager mode's report of out-of-range ids, from the status read back.
int bad_id_check(const moe_desc *desc, const int32_t *host_status)
{
    if (host_status[1] & MOE_FLAG_BAD_ID)
        return fail(MOE_ERR_INDEX, "an expert id outside [-1, E=%d) was seen; such slots were "
                                   "treated as empty", desc->E);
    return MOE_OK;
}

// moe_route_build's work (checks, launches, eager readback) for a handle
// whose workspace is set; pairs: the workspace takes the row list too.
int route_build(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                float *multihot_probs, const moe_handle *handle, int32_t *host_status,
                void *stream, bool pairs = true)
{
    moe::RouteArgs a;
    int rc = route_launch(desc, topk_idx, topk_w, multihot_probs, handle, host_status, stream, a,
                          pairs);
    if (rc == MOE_OK && desc->mode == MOE_EAGER) {
        if ((rc = route_wait(handle, host_status, stream, a)) == MOE_OK)
            rc = bad_id_check(desc, host_status);
    }
    return rc == MOE_OK ? ok() : rc;
}

// ---------------------------------------------------------------------------
// Fixed route scratch of moe_route_build_noalloc, for callers that cannot
// allocate.  One copy of the array per GPU, loaded with the library's code
// object and held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is resolved once
// per device (that device current) and only that address is handed to
// kernels.  Nothing in it has to start at zero: every route writes each count
// and flag word before reading it.
// ---------------------------------------------------------------------------
constexpr size_t kNoallocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchAddr {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchAddr g_scratch_addr[kMaxDevices];

int noalloc_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_DEVICE, "device %d: moe_route_build_noalloc serves devices 0..%d", dev,
                    kMaxDevices - 1);
    ScratchAddr &s = g_scratch_addr[dev];
    std::call_once(s.once, [&s] {
        s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch));
        if (s.err == hipSuccess && !s.ptr)
            s.err = hipErrorInvalidSymbol;
    });
    if (s.err != hipSuccess)
        return hip_fail(s.err, "hipGetSymbolAddress of the route scratch");
    *out = s.ptr;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_route_build(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                    float *multihot_probs, const moe_handle *handle, int32_t *host_status,
                    void *stream)
{
    TimingScope timing_scope;
    return route_build(desc, topk_idx, topk_w, multihot_probs, handle, host_status, stream);
}

int moe_route_build_noalloc(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                            float *multihot_probs, const moe_handle *handle,
                            int32_t *host_status, void *stream)
{
    TimingScope timing_scope;
    int rc;
    // every rule checked before the first HIP call
    if ((rc = route_check(desc, topk_idx, topk_w, multihot_probs, handle, host_status, false)) !=
        MOE_OK)
        return rc;
    if (handle->workspace || handle->workspace_bytes)
        return fail(MOE_ERR_ARG, "moe_route_build_noalloc takes its scratch from the library's "
                                 "fixed array: handle.workspace must be NULL and "
                                 "workspace_bytes 0 (it would be ignored)");
    const size_t need = ws_layout(desc, false).bytes;
    if (need > kNoallocScratchBytes)
        return fail(MOE_ERR_WORKSPACE, "this route needs %zu bytes of scratch, more than the "
                                       "library's fixed %zu-byte array: use moe_route_build "
                                       "with a workspace of moe_route_workspace_size bytes",
                    need, kNoallocScratchBytes);
    void *ws = nullptr;
    if ((rc = noalloc_scratch(&ws)) != MOE_OK)
        return rc;
    moe_handle h = *handle;
    h.workspace = ws;
    h.workspace_bytes = kNoallocScratchBytes;
    // the caller's handle has no workspace, so the calls after it walk tokens:
    // the route writes no row list into the shared array
    return route_build(desc, topk_idx, topk_w, multihot_probs, &h, host_status, stream, false);
}

int moe_route_dispatch(const moe_desc *desc, const void *topk_idx, const float *topk_w,
                       float *multihot_probs, const moe_handle *handle, int32_t *host_status,
                       const uint16_t *x, int32_t H, int64_t R_cap, uint16_t *rows, float *row_w,
                       int32_t *row_token, int32_t *row_expert, void *stream)
{
    TimingScope timing_scope;
    int rc;
    // every argument of both halves is checked before anything is launched
    if ((rc = check_desc(desc)) != MOE_OK)
        return rc;
    const bool eager = desc->mode == MOE_EAGER;
    if ((rc = check_handle(desc, handle, true)) != MOE_OK)
        return rc;
    if ((rc = check_hidden(H)) != MOE_OK)
        return rc;
    if (!eager && R_cap != desc->capacity)
        return fail(MOE_ERR_ARG, "sync-free mode: R_cap must equal desc->capacity (%lld), got %lld",
                    (long long)desc->capacity, (long long)R_cap);
    if (eager && (R_cap < cap_min(desc) || R_cap > kI32Max))
        return fail(MOE_ERR_CAPACITY, "R_cap %lld must hold the worst case T*min(k,EL) + EL*(P-1) = "
                                      "%lld rows (and fit in int32)",
                    (long long)R_cap, (long long)cap_min(desc));
    if (desc->T > 0 && (!x || !aligned16(x)))
        return fail(MOE_ERR_ARG, "x must be a non-NULL, 16-byte aligned [T,H] bf16 tensor");
    if (R_cap > 0 && (!rows || !aligned16(rows)))
        return fail(MOE_ERR_ARG, "rows must be a non-NULL, 16-byte aligned [R_cap,H] bf16 tensor");
    if ((multihot_probs || row_w) && !topk_w && desc->T > 0)
        return fail(MOE_ERR_ARG, "multihot_probs or row_w requested without topk_w");
    if (topk_w && !multihot_probs && !row_w)
        return fail(MOE_ERR_ARG, "topk_w given but neither multihot_probs nor row_w is requested");
    if (eager && !host_status)
        return fail(MOE_ERR_ARG, "eager mode needs host_status (int32[4]) to return the row count");
    if (desc->T > 0 && !topk_idx)
        return fail(MOE_ERR_ARG, "topk_idx is NULL");
    // eager: the dispatch, bounded by the buffers' capacity, writes the rows
    // [0, total) and leaves the rest; sync-free: every row, as moe_dispatch
    const moe::RowArgs ra = dispatch_args(desc, handle, x, H, row_w ? topk_w : nullptr, R_cap, rows,
                                          nullptr, nullptr, row_w, row_token, row_expert, eager);
    if (!moe::move_rows_fits(ra))
        return hip_fail(hipErrorInvalidConfiguration, "dispatch");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;

    moe::RouteArgs a;
    if (!eager) {
        // nothing waits; a route of at most kTinySlots slots goes into the
        // dispatch's own launch
        route_args(desc, topk_idx, multihot_probs ? topk_w : nullptr, multihot_probs, handle, a);
        if (moe::route_move_tiny_fits(ra, a)) {
            if ((e = moe::launch_route_move_tiny(ra, a, s)) != hipSuccess)
                return hip_fail(e, "route and dispatch launch");
            return ok();
        }
        if ((rc = route_launch(desc, topk_idx, multihot_probs ? topk_w : nullptr, multihot_probs,
                               handle, host_status, stream, a)) != MOE_OK)
            return rc;
        if ((e = moe::launch_move_rows(ra, s)) != hipSuccess)
            return hip_fail(e, "dispatch launch");
        return ok();
    }
    if ((rc = route_launch(desc, topk_idx, multihot_probs ? topk_w : nullptr, multihot_probs, handle,
                           host_status, stream, a)) != MOE_OK)
        return rc;
    // pageable status: its copy (and sync) go ahead of the dispatch
    if (!a.host_status && (rc = route_wait(handle, host_status, stream, a)) != MOE_OK)
        return rc;
    // the dispatch, queued before the row count is known
    if ((e = moe::launch_move_rows(ra, s)) != hipSuccess)
        return hip_fail(e, "dispatch launch");
    if (a.host_status && (rc = route_wait(handle, host_status, stream, a)) != MOE_OK)
        return rc;
    rc = bad_id_check(desc, host_status);
    return rc == MOE_OK ? ok() : rc;
}

int moe_dispatch(const moe_desc *desc, const moe_handle *handle, const uint16_t *x, int32_t H,
                 const float *topk_w, int64_t R, uint16_t *rows, float *row_w, int32_t *row_token,
                 int32_t *row_expert, void *stream)
{
    TimingScope timing_scope;
    int rc;
    if ((rc = check_dispatch(desc, handle, x, H, topk_w, R, row_w)) != MOE_OK)
        return rc;
    if (R > 0 && (!rows || !aligned16(rows)))
        return fail(MOE_ERR_ARG, "rows must be a non-NULL, 16-byte aligned [R,H] bf16 tensor");
    return launch_dispatch(desc, handle, x, H, topk_w, R, rows, nullptr, nullptr, row_w, row_token,
                           row_expert, stream);
}

int moe_dispatch_fp8(const moe_desc *desc, const moe_handle *handle, const uint16_t *x, int32_t H,
                     const float *topk_w, int64_t R, uint8_t *rows_q, float *row_scale,
                     float *row_w, int32_t *row_token, int32_t *row_expert, void *stream)
{
    TimingScope timing_scope;
    int rc;
    if ((rc = check_dispatch(desc, handle, x, H, topk_w, R, row_w)) != MOE_OK)
        return rc;
    if (R > 0 && (!rows_q || !aligned16(rows_q)))
        return fail(MOE_ERR_ARG, "rows_q must be a non-NULL, 16-byte aligned [R,H] byte tensor");
    if (R > 0 && (!row_scale || !aligned16(row_scale)))
        return fail(MOE_ERR_ARG, "row_scale must be a non-NULL, 16-byte aligned [R,H/128] fp32 "
                                 "tensor");
    return launch_dispatch(desc, handle, x, H, topk_w, R, nullptr, rows_q, row_scale, row_w,
                           row_token, row_expert, stream);
}

int moe_combine(const moe_desc *desc, const moe_handle *handle, const uint16_t *Y, int32_t H,
                int64_t R, void *out, int32_t out_is_f32, void *stream)
{
    TimingScope timing_scope;
    int rc;
    if ((rc = check_desc(desc)) != MOE_OK)
        return rc;
    if ((rc = check_handle(desc, handle)) != MOE_OK)
        return rc;
    if ((rc = check_hidden(H)) != MOE_OK)
        return rc;
    if ((rc = check_rows(desc, R)) != MOE_OK)
        return rc;
    if (out_is_f32 != 0 && out_is_f32 != 1)
        return fail(MOE_ERR_ARG, "out_is_f32 must be 0 or 1 (got %d)", out_is_f32);
    if (R > 0 && (!Y || !aligned16(Y)))
        return fail(MOE_ERR_ARG, "Y must be a non-NULL, 16-byte aligned [R,H] bf16 tensor");
    if (desc->T > 0 && (!out || !aligned16(out)))
        return fail(MOE_ERR_ARG, "out must be a non-NULL, 16-byte aligned [T,H] tensor");

    moe::CombineArgs a;
    a.Y = Y;
    a.out = out;
    a.row_of_slot = handle->row_of_slot;
    a.grad_row_w = nullptr;
    a.grad_w = nullptr;
    a.status = handle->status;
    a.T = desc->T;
    a.R = R;
    a.k = desc->k;
    a.H = H;
    a.out_f32 = out_is_f32;
    a.eager = desc->mode == MOE_EAGER;
    hipError_t e = moe::launch_combine(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "combine launch");
    return ok();
}

int moe_combine_bwd(const moe_desc *desc, const moe_handle *handle, const uint16_t *grad_out,
                    const uint16_t *expert_out, int32_t H, int64_t R, uint16_t *grad_rows,
                    float *dw, void *stream)
{
    TimingScope timing_scope;
    int rc;
    if ((rc = check_desc(desc)) != MOE_OK)
        return rc;
    if ((rc = check_handle(desc, handle)) != MOE_OK)
        return rc;
    if ((rc = check_hidden(H)) != MOE_OK)
        return rc;
    if ((rc = check_rows(desc, R)) != MOE_OK)
        return rc;
    if (desc->T > 0 && (!grad_out || !aligned16(grad_out)))
        return fail(MOE_ERR_ARG, "grad_out must be a non-NULL, 16-byte aligned [T,H] bf16 tensor");
    if (R > 0 && (!grad_rows || !aligned16(grad_rows)))
        return fail(MOE_ERR_ARG, "grad_rows must be a non-NULL, 16-byte aligned [R,H] bf16 tensor");
    if (expert_out && !dw)
        return fail(MOE_ERR_ARG, "expert_out given but dw is NULL (expert_out is only read for dw)");
    if (dw && !expert_out && R > 0)
        return fail(MOE_ERR_ARG, "dw requested without expert_out");
    if (expert_out && R > 0 && !aligned16(expert_out))
        return fail(MOE_ERR_ARG, "expert_out must be 16-byte aligned");

    moe::RowArgs a;
    a.src = grad_out;
    a.topk_w = nullptr;
    a.F = expert_out;
    a.rows = grad_rows;
    a.rows_q = nullptr;
    a.row_scale = nullptr;
    a.row_w = nullptr;
    a.row_token = nullptr;
    a.row_expert = nullptr;
    a.dw = dw;
    a.row_of_slot = handle->row_of_slot;
    a.tpe = handle->tokens_per_expert;
    a.off = handle->padded_offsets;
    a.status = handle->status;
    a.T = desc->T;
    a.R = R;
    a.k = desc->k;
    a.EL = desc->num_local;
    a.E_total = desc->E;
    a.P = desc->pad_multiple;
    a.H = H;
    a.eager = desc->mode == MOE_EAGER;
    a.pairs = handle_pairs(desc, handle, a.pg);
    moe::row_shape(a);
    hipError_t e = moe::launch_move_rows(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "combine_bwd launch");
    return ok();
}

int moe_dispatch_bwd(const moe_desc *desc, const moe_handle *handle, const uint16_t *grad_rows,
                     int32_t H, int64_t R, const float *grad_row_w, void *grad_x,
                     int32_t grad_x_is_f32, float *grad_topk_w, void *stream)
{
    TimingScope timing_scope;
    int rc;
    if ((rc = check_desc(desc)) != MOE_OK)
        return rc;
    if ((rc = check_handle(desc, handle)) != MOE_OK)
        return rc;
    if ((rc = check_hidden(H)) != MOE_OK)
        return rc;
    if ((rc = check_rows(desc, R)) != MOE_OK)
        return rc;
    if (grad_x_is_f32 != 0 && grad_x_is_f32 != 1)
        return fail(MOE_ERR_ARG, "grad_x_is_f32 must be 0 or 1 (got %d)", grad_x_is_f32);
    if (R > 0 && (!grad_rows || !aligned16(grad_rows)))
        return fail(MOE_ERR_ARG, "grad_rows must be a non-NULL, 16-byte aligned [R,H] bf16 tensor");
    if (desc->T > 0 && (!grad_x || !aligned16(grad_x)))
        return fail(MOE_ERR_ARG, "grad_x must be a non-NULL, 16-byte aligned [T,H] tensor");
    if (grad_row_w && !grad_topk_w)
        return fail(MOE_ERR_ARG, "grad_row_w given but grad_topk_w is NULL (it would be ignored)");
    if (grad_topk_w && !grad_row_w && R > 0)
        return fail(MOE_ERR_ARG, "grad_topk_w requested without grad_row_w");

    moe::CombineArgs a;
    a.Y = grad_rows;
    a.out = grad_x;
    a.row_of_slot = handle->row_of_slot;
    a.grad_row_w = grad_row_w;
    a.grad_w = grad_topk_w;
    a.status = handle->status;
    a.T = desc->T;
    a.R = R;
    a.k = desc->k;
    a.H = H;
    a.out_f32 = grad_x_is_f32;
    a.eager = desc->mode == MOE_EAGER;
    hipError_t e = moe::launch_combine(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "dispatch_bwd launch");
    return ok();
}

const char *moe_last_error(void) { return g_err; }

int moe_time_next_call(void *start_event, void *stop_event)
{
    moe::LaunchTiming &t = moe::launch_timing();
    t.start = static_cast<hipEvent_t>(start_event);
    t.stop = static_cast<hipEvent_t>(stop_event);
    return ok();
}

int moe_device_check(int device)
{
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDeviceCount");
    if (device < 0 || device >= n)
        return fail(MOE_ERR_DEVICE, "device %d not present (%d HIP devices)", device, n);
    hipDeviceProp_t p;
    if ((e = hipGetDeviceProperties(&p, device)) != hipSuccess)
        return hip_fail(e, "hipGetDeviceProperties");
    if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
        return fail(MOE_ERR_DEVICE, "device %d is %s; this library is built for gfx950 (MI355X) only",
                    device, p.gcnArchName);
    return ok();
}

}  // extern "C"

namespace moe {
LaunchTiming &launch_timing()
{
    thread_local LaunchTiming t;
    return t;
}
}  // namespace moe
