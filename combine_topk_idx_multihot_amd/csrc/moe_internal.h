// moe_internal.h -- private declarations shared by the HIP sources of libmoe_mi355x.
// Not installed; the public interface is include/moe_mi355x.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxK = 64;         // slots per token handled lane-parallel by one wave
constexpr int kMaxLocal = 1024;   // local experts (LDS bitmap bound)
constexpr int kRowWaves = 4;      // waves per workgroup in the row kernels
constexpr int kRowThreads = kRowWaves * kWave;

// A kernel dispatch packet carries the grid size in work-items as a 32-bit
// number, so a row launch takes at most this many workgroups; the launchers
// return hipErrorInvalidConfiguration, before any launch, for a problem that
// would need more (a row array past 64 GiB, for instance).
constexpr int64_t kMaxRowBlocks = 0xFFFFFFFFll / kRowThreads;

// A route whose count table has at most this many entries (blocks x local
// experts) is finished by one pass of one workgroup per block.
constexpr int64_t kFusedFinishMax = 65536;
constexpr int kXcds = 8;  // MI355X: workgroup j runs on XCD j mod 8

// The route's row list.  For layers whose local experts take most routes
// (k * EL >= 2 E), the finishing pass also writes, into the handle's
// workspace, the (row, token) of every data row in an order made for the
// row kernels: tokens are cut into tiles of about 512 (whole route blocks),
// tile tau belongs to XCD tau mod 8, and a tile's rows are listed in
// address order (expert by expert, ascending token).  Entry i is consumed by
// wave i % 4 of workgroup i / 4, which runs on XCD (i / 4) mod 8, so the
// rows of a tile are written by one XCD one after another, in address order,
// while the tile's token rows (about 512 x 2H bytes) stay in that XCD's L2
// for their up to k reads.  Each tile has a fixed range of cap positions in
// its XCD's sequence; positions past the tile's rows hold row -1.
struct PairGeom {
    int64_t bpt = 0;           // route blocks per tile
    int64_t tile_tokens = 0;   // tokens per tile (the last tile may have fewer)
    int64_t ntiles = 0;
    int64_t tiles_per_xcd = 0;
    int64_t kk = 0;            // min(k, EL): rows a token can have
    int64_t cap = 0;           // positions per tile, tile_tokens * kk
    int64_t entries = 0;       // kXcds * (tiles_per_xcd * cap rounded up to a multiple of 4)
};
// Whether the route of this description writes the row list: several route
// blocks, the fused finishing pass, and dense routing.
bool pairs_form(int64_t T, int k, int E, int EL, int tokens_per_block, int64_t nblk);
PairGeom pair_geom(int64_t T, int k, int EL, int tokens_per_block, int64_t nblk);

// Launch geometry of the routing-count kernel: one workgroup covers
// tokens_per_block whole tokens (k slots each, `slots` slots per thread).
struct RouteGeom {
    int threads;          // 1024, 512 or 256 (the LDS bitmaps hold EL x threads x slots bits)
    int slots;            // slots per thread: 1, or 2 for a one-workgroup route of up to 2048 slots
    int tokens_per_block; // threads * slots / k
    int64_t nblk;         // ceil(T / tokens_per_block)
};
RouteGeom route_geom(int64_t T, int k, int EL);

struct RouteArgs {
    const void *idx;       // [T,k] int32 or int64
    const float *w;        // [T,k] or null
    float *probs;          // [T,E] or null
    uint8_t *map;          // [T,E] or null
    int32_t *row_of_slot;  // [T,k]
    int32_t *counts;       // workspace [nblk][EL]
    int32_t *blockflags;   // workspace [nblk]
    int32_t *tpe;          // [EL]
    int32_t *off;          // [EL+1]
    int32_t *status;       // [4]
    int32_t *host_status;  // [4] device-visible alias of the caller's host copy, or null
    int64_t T;
    int32_t k, E, lb, EL, P;
    int32_t tokens_per_block;
    int32_t slots = 1;     // slots per thread of the counting kernel (RouteGeom)
    int64_t nblk;
    int32_t idx_i64;
    int2 *pairs = nullptr;   // the row list (workspace), or null: not written
    PairGeom pg;
};

// K1 counts + multihot map + in-block ranks; K2 offsets and final rows.
hipError_t launch_route(const RouteArgs &a, int threads, hipStream_t s);

struct RowArgs {
    const uint16_t *src;       // [T,H] token rows (x or grad_out)
    const float *topk_w;       // [T,k] or null
    const uint16_t *F;         // [R,H] expert outputs for dw, or null
    uint16_t *rows;            // [R,H] bf16, or null with rows_q set
    uint8_t *rows_q;           // [R,H] E4M3 codes (FP8 dispatch) or null
    float *row_scale;          // [R,H/128] scales of rows_q (FP8 dispatch)
    float *row_w;              // [R] or null
    int32_t *row_token;        // [R] or null
    int32_t *row_expert;       // [R] or null
    float *dw;                 // [T,k] or null
    const int32_t *row_of_slot;
    const int32_t *tpe;
    const int32_t *off;
    int32_t *status;
    int64_t T, R;
    int32_t k, EL, H;
    int32_t E_total;           // all experts (E), for launch heuristics
    int32_t eager;
    int32_t seg;               // 16-byte chunks per lane per segment
    int32_t waves_per_token;   // 1, 2 or 4: a token's segments are dealt over these waves
    int32_t dot_seg;           // combine backward: chunks per lane per dot segment
    int32_t dot_wpt;           // combine backward: waves sharing one token's dots (1, 2 or 4)
    int32_t P = 1;             // pad_multiple
    int32_t exp_slices = 1;    // workgroups per expert group (pad rows and row_expert)
    int64_t ntok_blocks, nexp_blocks, nsent_blocks;
    int64_t ndot_blocks;       // combine backward with dw: periods of 4 tokens, 0 otherwise
    int32_t keep_tail = 0;     // eager, R = the buffers' capacity: rows past the total are
                               // left as they are (no sentinel fill)
    const int2 *pairs = nullptr; // the route's row list: rows are walked from it, not by token
    PairGeom pg;
    int64_t npair_blocks = 0;  // workgroups walking the row list (4 entries each)
    int64_t nzero_blocks = 0;  // combine backward from the list: dw of slots without a row
};

// Row movement: dispatch (x -> rows, or with rows_q set x -> E4M3 rows and
// block scales) and the combine backward (grad_out -> grad rows, optional
// dw), token-major; plus pad / sentinel fill.
// row_shape fills in the launch shape (segment size, waves per token, block
// counts) from the other fields.
void row_shape(RowArgs &a);
bool move_rows_fits(const RowArgs &a); // launch_move_rows' grids within kMaxRowBlocks
hipError_t launch_move_rows(const RowArgs &a, hipStream_t s);

// Decode-sized sync-free route and dispatch in one launch: every workgroup
// computes the route of at most kTinySlots slots (T*k <= 16) in its own LDS,
// workgroup 0 publishes the handle.  Only for sync-free bf16 dispatches whose
// zero tail is filled by the rows' launch and whose multihot map has at most
// kTinyMapEntries entries; route_move_tiny_fits says whether `a` and `r`
// qualify, and the launcher refuses (hipErrorInvalidConfiguration) otherwise.
constexpr int64_t kTinyMapEntries = 65536;
#ifndef MOE_TINY_SLOTS
#define MOE_TINY_SLOTS 16
#endif
constexpr int kTinySlots = MOE_TINY_SLOTS;  // at most 64 (one wave)
static_assert(kTinySlots >= 0 && kTinySlots <= kWave, "tiny routes fit one wave");
bool route_move_tiny_fits(const RowArgs &a, const RouteArgs &r);
hipError_t launch_route_move_tiny(const RowArgs &a, const RouteArgs &r, hipStream_t s);

struct CombineArgs {
    const uint16_t *Y;          // [R,H]
    void *out;                  // [T,H] bf16 or f32
    const int32_t *row_of_slot; // [T,k]
    const float *grad_row_w;    // [R] or null (dispatch backward: per-row weight gradients)
    float *grad_w;              // [T,k] or null (dispatch backward: per-slot weight gradients)
    int32_t *status;
    int64_t T, R;
    int32_t k, H;
    int32_t out_f32;
    int32_t eager;
};

// Combine; with grad_w set it is also the dispatch backward (the weight
// gradients of the slots are gathered from their rows).
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);

// Kernel timing request of the calling host thread (moe_time_next_call).
// The events ride on the kernels' own dispatch packets: the first kernel of
// the next entry point records `start`, and every kernel of it re-records
// `stop`, so the pair spans that call's kernels with no packet between them.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchTiming &launch_timing();

// Every kernel of the library is launched through this.
template <typename A>
inline void launch(void (*kernel)(A), dim3 grid, dim3 block, size_t lds, hipStream_t s, const A &arg)
{
    LaunchTiming &t = launch_timing();
    if (t.start || t.stop) {
        hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), s, t.start, t.stop,
                              0u, arg);
        t.start = nullptr;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, s, arg);
    }
}

}  // namespace moe
