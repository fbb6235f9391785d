// rows.hip -- the row-moving kernels of the expanded layout on gfx950.
//
// "Add the deepep expert-parallel implementation", "What this adds":
//   "Expanded layout"  one row per (token, local expert) slot grouped by local
//                      expert, each with its routing weight; combine is a plain
//                      sum of rows back to token order;
//   "Eager vs captured" sync-free rows are sized for the worst case; rows past
//                      the received total are zero and belong to a sentinel
//                      expert;
//   "Custom ops"       the combine's backward is a cached dispatch;
//   "Training"         gradients reach the routing weights.
//
// All of it is HBM-bound data movement (no contraction, so no MFMA).  Design:
//   * token-major: the token's row is read from HBM once and written to each
//     of its local rows (dispatch), or its local rows are gathered and added
//     (combine).  The token's k slots sit one per lane: row lookup,
//     repeated-id detection and weight merging are a few lane reads and
//     ballots, no LDS.
//   * a row is walked in segments of SEG 16-byte chunks per lane (SEG KiB
//     per wave), and a token's segments are dealt over 1, 2 or 4 waves of the
//     workgroup, so that even a few thousand tokens keep enough waves (and
//     bytes) in flight on 256 CUs.  Within a segment a wave issues the loads
//     of a batch of rows (4 for combine and for the dots) before consuming
//     any of them.
//   * the combine backward is the dispatch of grad_out plus, in workgroups of
//     their own interleaved with the copying ones, the dots of grad_out with
//     the expert-output rows of the token's slots.  A token's row is dealt
//     over 1 to 4 dot waves; each keeps its exact bf16 x bf16 products summed
//     in fp64 registers, wave sums (for a batch of four rows with 1 KiB
//     segments, lane-half swaps and DPP moves without LDS; a butterfly per
//     row otherwise) end each wave's part, and the token's first wave adds
//     the parts in wave order through LDS before the single rounding to fp32,
//     so dw is the same on every run.
//   * pad rows are zeroed by extra workgroups of the rows' launch (1 to 16
//     per expert, about 64 KiB of pad rows each).  The sync-free tail
//     [total, R) -- most of the bytes when the worst case is far from the
//     routed total -- is a launch of its own just before, of one-shot waves
//     that each zero one 1 KiB piece in address order: the writes in flight
//     then form one window sliding through the tail, which MI355X's HBM
//     takes markedly faster than the same writes spread over the range.  In
//     eager mode the tail is normally empty; a few workgroups of the rows'
//     launch cover it in 64 KiB wave tasks.  A sync-free worst case of at
//     most 32 MiB of rows (decode sizes) is zeroed the same way, by
//     workgroups of the rows' launch, saving a launch.
//   * combine adds the token's rows in fp32 in ascending slot order (the
//     accumulator starts from the first row) and writes bf16 (nearest-even)
//     or fp32; one wave per (token, segment).
//   * rows that are written once and not read again by this step (dispatched
//     rows, grad rows, zeros) use non-temporal stores, and rows read once
//     (the combine's gather, the backward's expert outputs) non-temporal
//     loads: measured on MI355X, this keeps the write-back of one kernel from
//     landing in the next one and shortens the whole step.
#include "moe_internal.h"

// Compile-time launch parameters.  The defaults are the fastest settings
// measured on MI355X; the others exist for measurement and give the same
// bits, except dw, whose fp64 summation order follows the dot segmentation
// (within the dw tolerance of the parity tests):
//   MOE_*_SEG         KiB of a row one wave moves per segment (1, 2 or 4);
//                     MOE_COPY_SEG_DENSE is the bf16 dispatch's when most
//                     tokens have local rows;
//   MOE_MAX_WPT       most waves sharing one token's row in the row kernels;
//   MOE_DOT_MAX_WPT   the same for the combine backward's dots;
//   MOE_*_BATCH       rows whose loads or stores one wave keeps in flight;
//   MOE_NT_*          non-temporal stores (zeros, copied rows) and loads
//                     (expert-output rows of the dots);
//   MOE_FP8_HW        E4M3 conversion by instruction (1) or bit arithmetic (0);
//   MOE_TAIL_PIECE_KIB  KiB per wave of the sync-free tail fill.

#ifndef MOE_COMBINE_SEG
#define MOE_COMBINE_SEG 2
#endif
#ifndef MOE_COPY_SEG
#define MOE_COPY_SEG 2
#endif
#ifndef MOE_COPY_SEG_DENSE
#define MOE_COPY_SEG_DENSE 1
#endif
#ifndef MOE_MAX_WPT
#define MOE_MAX_WPT 4
#endif
#ifndef MOE_NT_ZERO
#define MOE_NT_ZERO 1
#endif
#ifndef MOE_NT_DOT_F
#define MOE_NT_DOT_F 1
#endif
#ifndef MOE_NT_COPY_ROWS
#define MOE_NT_COPY_ROWS 1
#endif
#ifndef MOE_FP8_HW
#define MOE_FP8_HW 1
#endif
#ifndef MOE_DOT_MAX_WPT
#define MOE_DOT_MAX_WPT 4
#endif
#ifndef MOE_DOT_SEG
#define MOE_DOT_SEG 1
#endif
#ifndef MOE_DOT_SEG_SPARSE
#define MOE_DOT_SEG_SPARSE 2
#endif
#ifndef MOE_TAIL_PIECE_KIB
#define MOE_TAIL_PIECE_KIB 1
#endif
#ifndef MOE_COPY_BATCH
#define MOE_COPY_BATCH 8
#endif
#ifndef MOE_DOT_BATCH
#define MOE_DOT_BATCH 4
#endif
#ifndef MOE_COMBINE_BATCH
#define MOE_COMBINE_BATCH 4
#endif


namespace moe {

#define MOE_SEG_OK(x) ((x) == 1 || (x) == 2 || (x) == 4)
static_assert(MOE_SEG_OK(MOE_COMBINE_SEG) && MOE_SEG_OK(MOE_COPY_SEG) &&
                  MOE_SEG_OK(MOE_COPY_SEG_DENSE) && MOE_SEG_OK(MOE_DOT_SEG) &&
                  MOE_SEG_OK(MOE_DOT_SEG_SPARSE),
              "segment sizes are 1, 2 or 4 KiB");
#undef MOE_SEG_OK
static_assert(MOE_COPY_BATCH >= 1 && MOE_DOT_BATCH >= 1 && MOE_COMBINE_BATCH >= 1 &&
                  MOE_DOT_BATCH <= kMaxK && MOE_COPY_BATCH <= kMaxK && MOE_COMBINE_BATCH <= kMaxK,
              "batch sizes are 1..64 rows");
static_assert(MOE_TAIL_PIECE_KIB >= 1, "tail pieces are at least 1 KiB");

// rows whose loads (or stores) a wave keeps in flight together: dispatch and
// FP8 dispatch (stores), the combine backward (loads of expert rows), combine
constexpr int kCopyBatch = MOE_COPY_BATCH;
constexpr int kDotBatch = MOE_DOT_BATCH;
constexpr int kCombBatch = MOE_COMBINE_BATCH;
constexpr int64_t kZeroTask = 4096;  // 16-byte chunks (64 KiB) per zero-fill wave task

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest, ties to even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool NT>
__device__ __forceinline__ void put16(u32x4 *p, const u32x4 &v)
{
    if (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// The token's slots, one per lane: its row (or -1), whether the row is valid
// (inside [0, R)), and the lane of the first slot naming that row.
struct Slots {
    int row;
    bool valid;
    int first;
    uint64_t prim_mask; // lanes that are the first slot of their row
    uint64_t dup_mask;  // valid lanes that repeat an earlier slot's row
};

__device__ __forceinline__ Slots load_slots(const int32_t *__restrict__ row_of_slot, int64_t t,
                                            int k, int64_t R, int lane, bool active)
{
    Slots s;
    s.row = (active && lane < k) ? row_of_slot[t * k + lane] : -1;
    s.valid = active && lane < k && s.row >= 0 && s.row < R;
    s.first = lane;
    for (int q = 0; q < k; ++q) {
        const int rq = __builtin_amdgcn_readlane(s.row, q);
        if (q < lane && s.valid && rq == s.row && s.first == lane)
            s.first = q;
    }
    const bool prim = s.valid && s.first == lane;
    s.prim_mask = __ballot(prim);
    s.dup_mask = __ballot(s.valid && !prim);
    return s;
}

// Up to NB slots taken (ascending) off a lane mask: their lanes and rows
// (wave-uniform values).
template <int NB>
struct Batch {
    int n;
    int lane[NB];
    int64_t row[NB];
};

template <int NB>
__device__ __forceinline__ Batch<NB> take_batch(uint64_t &m, int row)
{
    Batch<NB> bt;
    bt.n = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        bt.lane[b] = 0;
        bt.row[b] = 0;
        if (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            bt.lane[b] = j;
            bt.row[b] = __builtin_amdgcn_readlane(row, j);
            bt.n = b + 1;
        }
    }
    return bt;
}

// NT: non-temporal loads, for rows read once (the combine's gather).
template <int SEG, bool NT = false>
__device__ __forceinline__ void load_seg(u32x4 (&v)[SEG], const uint16_t *base, int64_t r, int H,
                                         int c0, int nch, int lane)
{
    const u32x4 *__restrict__ p = reinterpret_cast<const u32x4 *>(base + r * H);
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
        const int c = c0 + i * kWave + lane;
        if (c < nch) {
            if (NT)
                v[i] = __builtin_nontemporal_load(p + c);
            else
                v[i] = p[c];
        }
    }
}

// Zero the 16-byte chunks [q0, q1) of `dst` in wave tasks of kZeroTask
// contiguous chunks; wave `w` of `nw` takes tasks w, w + nw, ...
__device__ __forceinline__ void zero_chunks(u32x4 *__restrict__ dst, int64_t q0, int64_t q1, int64_t w,
                                            int64_t nw, int lane)
{
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int64_t ntask = (q1 - q0 + kZeroTask - 1) / kZeroTask;
    for (int64_t task = w; task < ntask; task += nw) {
        const int64_t b = q0 + task * kZeroTask;
        const int64_t e = min(q1, b + kZeroTask);
        int64_t i = b + lane;
        for (; i + 3 * kWave < e; i += 4 * kWave) {
            put16<MOE_NT_ZERO != 0>(dst + i, z);
            put16<MOE_NT_ZERO != 0>(dst + i + kWave, z);
            put16<MOE_NT_ZERO != 0>(dst + i + 2 * kWave, z);
            put16<MOE_NT_ZERO != 0>(dst + i + 3 * kWave, z);
        }
        for (; i < e; i += kWave)
            put16<MOE_NT_ZERO != 0>(dst + i, z);
    }
}

// Zero the 4-byte words [w0, w1) of `base` (16-byte aligned): whole 16-byte
// chunks as wave tasks, the unaligned head and tail (under 4 words each) by
// wave 0.
__device__ __forceinline__ void zero_words(uint32_t *__restrict__ base, int64_t w0, int64_t w1,
                                           int64_t w, int64_t nw, int lane)
{
    if (w1 <= w0)
        return;
    const int64_t a0 = (w0 + 3) & ~static_cast<int64_t>(3);
    const int64_t a1 = w1 & ~static_cast<int64_t>(3);
    if (a0 >= a1) { // no whole chunk: fewer than 8 words
        if (w == 0 && lane < w1 - w0)
            base[w0 + lane] = 0u;
        return;
    }
    if (w == 0) {
        if (lane < a0 - w0)
            base[w0 + lane] = 0u;
        if (lane < w1 - a1)
            base[a1 + lane] = 0u;
    }
    zero_chunks(reinterpret_cast<u32x4 *>(base), a0 >> 2, a1 >> 2, w, nw, lane);
}

// Zero rows [r0, r1) of the dispatch output: bf16 rows, or E4M3 rows and
// their scales; `w` of `nw` waves.
__device__ __forceinline__ void zero_rows(const RowArgs &a, int64_t r0, int64_t r1, int64_t w,
                                          int64_t nw, int lane)
{
    if (a.rows_q) {
        zero_chunks(reinterpret_cast<u32x4 *>(a.rows_q), r0 * (a.H >> 4), r1 * (a.H >> 4), w, nw,
                    lane);
        zero_words(reinterpret_cast<uint32_t *>(a.row_scale), r0 * (a.H >> 7), r1 * (a.H >> 7), w,
                   nw, lane);
    } else {
        zero_chunks(reinterpret_cast<u32x4 *>(a.rows), r0 * (a.H >> 3), r1 * (a.H >> 3), w, nw,
                    lane);
    }
}

// Token and weight of each of the token's rows (dispatch): the row of a
// repeated id carries the first slot's weight plus the later ones', in slot
// order.
__device__ __forceinline__ void write_row_meta(const RowArgs &a, const Slots &sl, int64_t t,
                                               int lane, bool active)
{
    if (!a.row_w && !a.row_token)
        return;
    const int k = a.k;
    const bool prim = sl.valid && sl.first == lane;
    float W = 0.f;
    if (a.topk_w && active) {
        const float myw = lane < k ? a.topk_w[t * k + lane] : 0.f;
        W = myw;
        if (sl.dup_mask) {
            for (int q = 0; q < k; ++q) {
                const int rq = __builtin_amdgcn_readlane(sl.row, q);
                const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myw), q));
                if (prim && q > lane && rq == sl.row)
                    W = W + wq;
            }
        }
    }
    if (prim) {
        if (a.row_token)
            a.row_token[sl.row] = static_cast<int32_t>(t);
        if (a.row_w)
            a.row_w[sl.row] = W;
    }
}

// ---------------------------------------------------------------------------
// dispatch (x -> rows) and the grad rows of the combine backward (grad_out ->
// rows): a token's row read once, written to each of its local rows
// ---------------------------------------------------------------------------
template <int SEG>
__device__ __forceinline__ void move_token(const RowArgs &a, int64_t bid)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nwt = a.waves_per_token;
    const int tl = wave / nwt;        // token of this wave inside the workgroup
    const int wt = wave - tl * nwt;   // this wave's share of the token's segments
    const int64_t t = bid * (kRowWaves / nwt) + tl;
    if (t >= a.T)
        return;
    const Slots sl = load_slots(a.row_of_slot, t, a.k, a.R, lane, true);

    // metadata of the token's rows (dispatch only), by the token's first wave
    if (wt == 0)
        write_row_meta(a, sl, t, lane, true);

    const int nch = a.H >> 3; // 16-byte chunks per row
    constexpr int SPAN = SEG * kWave;
    const int nseg = (nch + SPAN - 1) / SPAN;
    if (!sl.prim_mask)
        return;
    for (int sg = wt; sg < nseg; sg += nwt) {
        const int c0 = sg * SPAN;
        u32x4 v[SEG];
        load_seg<SEG>(v, a.src, t, a.H, c0, nch, lane);
        uint64_t mrest = sl.prim_mask;
        while (mrest) {
            const Batch<kCopyBatch> bt = take_batch<kCopyBatch>(mrest, sl.row);
#pragma unroll
            for (int b = 0; b < kCopyBatch; ++b) {
                if (b < bt.n) {
                    u32x4 *__restrict__ dst = reinterpret_cast<u32x4 *>(a.rows + bt.row[b] * a.H);
#pragma unroll
                    for (int i = 0; i < SEG; ++i) {
                        const int c = c0 + i * kWave + lane;
                        if (c < nch)
                            put16<MOE_NT_COPY_ROWS != 0>(dst + c, v[i]);
                    }
                }
            }
        }
    }
}

// Pad rows of an expert's group: zero data, token -1, weight 0; every row of
// the group gets row_expert = e.  Expert workgroup j takes slice j % S of
// expert j / S (S = exp_slices): that contiguous share of the group's rows
// and of its pad rows.
__device__ __forceinline__ void fill_expert(const RowArgs &a, int j)
{
    const int S = a.exp_slices;
    const int e = j / S;
    const int sl = j - e * S;
    // clamped into [0, R] so that no handle content can move a write out of bounds
    const int64_t lo = max<int64_t>(0, min<int64_t>(a.off[e], a.R));
    const int64_t hi = max<int64_t>(lo, min<int64_t>(a.off[e + 1], a.R));
    const int64_t pad0 = max<int64_t>(lo, min<int64_t>(lo + a.tpe[e], hi));
    const int64_t gs = (hi - lo + S - 1) / S;
    const int64_t g0 = min(hi, lo + sl * gs), g1 = min(hi, g0 + gs);
    const int64_t ps = (hi - pad0 + S - 1) / S;
    const int64_t p0 = min(hi, pad0 + sl * ps), p1 = min(hi, p0 + ps);
    const int tid = threadIdx.x;
    if (a.row_expert)
        for (int64_t r = g0 + tid; r < g1; r += kRowThreads)
            a.row_expert[r] = e;
    for (int64_t r = p0 + tid; r < p1; r += kRowThreads) {
        if (a.row_token)
            a.row_token[r] = -1;
        if (a.row_w)
            a.row_w[r] = 0.f;
    }
    zero_rows(a, p0, p1, threadIdx.x / kWave, kRowWaves, tid & (kWave - 1));
}

// One-shot form of the sync-free tail fill: wave gw of the sentinel grid owns
// piece gw, MOE_TAIL_PIECE_KIB KiB of the row array (bf16 rows, or E4M3 rows
// followed by their scale array), zeroes the part of it at or past row
// `total` and exits.  Workgroups start in index order, so the pieces being
// written at any moment lie in one window that slides through the tail.  The
// sentinel metadata of a row is written by the wave whose piece holds the
// row's first chunk.
// Sentinel metadata of the tail's rows (token -1, expert EL, weight 0), one
// wave per kMetaRows consecutive rows, 4 per lane: every cache line of the
// three arrays is written whole by one wave at once.  (Written one row at a
// time by the waves that zero the rows, the lines were filled piecemeal by
// waves far apart, and the later kernels of a step paid for it: on the
// 16-of-128-expert share at 16384 tokens the combine backward that followed
// took 243-248 instead of 231 us, 4 runs each.)
constexpr int64_t kMetaRows = 4 * kWave;

template <typename V>
__device__ __forceinline__ void put_meta4(V *__restrict__ p, int64_t r, int64_t r0, int64_t R, V v)
{
    if (r >= r0 && r + 4 <= R && (reinterpret_cast<uintptr_t>(p + r) & 15u) == 0) {
        typedef V v4 __attribute__((ext_vector_type(4)));
        const v4 q = {v, v, v, v};
        *reinterpret_cast<v4 *>(p + r) = q;
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (r + i >= r0 && r + i < R)
            p[r + i] = v;
}

__device__ __forceinline__ void sentinel_meta(const RowArgs &a, int64_t g, int64_t r0, int lane)
{
    const int64_t r = g * kMetaRows + 4 * lane;
    if (r >= a.R || r + 4 <= r0)
        return;
    if (a.row_token)
        put_meta4<int32_t>(a.row_token, r, r0, a.R, -1);
    if (a.row_expert)
        put_meta4<int32_t>(a.row_expert, r, r0, a.R, a.EL);
    if (a.row_w)
        put_meta4<float>(a.row_w, r, r0, a.R, 0.f);
}

__device__ __forceinline__ void fill_sentinel_oneshot(const RowArgs &a, int64_t sb)
{
    constexpr int64_t PC = static_cast<int64_t>(MOE_TAIL_PIECE_KIB) * kWave; // 16-byte chunks per piece
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = sb * kRowWaves + (threadIdx.x / kWave);
    const int64_t total = a.status[0];
    const int64_t r0 = max<int64_t>(0, min<int64_t>(total, a.R));
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int64_t nch = a.rows_q ? (a.H >> 4) : (a.H >> 3); // chunks per row
    const int64_t nrow_pieces = (a.R * nch + PC - 1) / PC;
    if (gw < nrow_pieces) {
        const int64_t p0 = gw * PC;
        const int64_t lo = max(p0, r0 * nch);
        const int64_t hi = min(p0 + PC, a.R * nch);
        if (lo >= hi)
            return;
        u32x4 *__restrict__ dst = a.rows_q ? reinterpret_cast<u32x4 *>(a.rows_q)
                                           : reinterpret_cast<u32x4 *>(a.rows);
#pragma unroll
        for (int j = 0; j < MOE_TAIL_PIECE_KIB; ++j) {
            const int64_t i = p0 + j * kWave + lane;
            if (i >= lo && i < hi)
                put16<MOE_NT_ZERO != 0>(dst + i, z);
        }
        return;
    }
    int64_t g2 = gw - nrow_pieces;
    const int64_t nb = a.H >> 7;
    const int64_t nsc_pieces = a.rows_q ? (a.R * nb + PC * 4 - 1) / (PC * 4) : 0;
    if (g2 >= nsc_pieces) {
        sentinel_meta(a, g2 - nsc_pieces, r0, lane);
        return;
    }
    // E4M3 scales: words [r0 * nb, R * nb), pieces of PC * 4 words; a chunk
    // that straddles the start of the tail is written word by word
    const int64_t w0 = g2 * PC * 4;
    const int64_t lo = max(w0, r0 * nb);
    const int64_t hi = min(w0 + PC * 4, a.R * nb);
    if (lo >= hi)
        return;
    uint32_t *__restrict__ base = reinterpret_cast<uint32_t *>(a.row_scale);
#pragma unroll
    for (int j = 0; j < MOE_TAIL_PIECE_KIB; ++j) {
        const int64_t w = w0 + (j * kWave + lane) * 4;
        if (w >= lo && w + 4 <= hi) {
            put16<MOE_NT_ZERO != 0>(reinterpret_cast<u32x4 *>(base + w), z);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (w + q >= lo && w + q < hi)
                    base[w + q] = 0u;
        }
    }
}

// Rows [total, R) by workgroups of the rows' launch: in eager mode (normally
// none: R is the total read back; a different R sets flag bit 2), and in
// sync-free mode when the worst-case row array is small
// (tail_in_rows_launch): zero data, token -1, expert EL (the sentinel),
// weight 0.
__device__ __forceinline__ void fill_sentinel(const RowArgs &a, int64_t sb)
{
    const int64_t total = a.status[0];
    const int64_t r0 = max<int64_t>(0, min<int64_t>(total, a.R));
    const int64_t r1 = a.R;
    const int64_t gtid = sb * kRowThreads + threadIdx.x;
    const int64_t gstride = a.nsent_blocks * kRowThreads;
    if (sb == 0 && threadIdx.x == 0 && a.eager && total != a.R)
        atomicOr(&a.status[1], 4);
    for (int64_t r = r0 + gtid; r < r1; r += gstride) {
        if (a.row_token)
            a.row_token[r] = -1;
        if (a.row_expert)
            a.row_expert[r] = a.EL;
        if (a.row_w)
            a.row_w[r] = 0.f;
    }
    const int64_t wave = sb * kRowWaves + (threadIdx.x / kWave);
    zero_rows(a, r0, r1, wave, a.nsent_blocks * kRowWaves, threadIdx.x & (kWave - 1));
}

// Grid: [sentinel blocks][token blocks][expert blocks].  Sentinel blocks are
// eager mode's few workgroups for the (normally empty) [total, R), or the
// workgroups that zero a small sync-free tail; a large sync-free tail has a
// launch of its own and there are none here.
template <int SEG>
__global__ void __launch_bounds__(kRowThreads) k_move_rows(RowArgs a)
{
    int64_t bid = blockIdx.x;
    if (bid < a.nsent_blocks) {
        fill_sentinel(a, bid);
        return;
    }
    bid -= a.nsent_blocks;
    if (bid < a.ntok_blocks)
        move_token<SEG>(a, bid);
    else
        fill_expert(a, static_cast<int>(bid - a.ntok_blocks));
}

// ---------------------------------------------------------------------------
// Rows walked from the route's row list (dense routing, a handle with its
// workspace): one wave per data row, the list entries laid out so that the
// rows of a token tile are written one after another, in address order, by
// the XCD whose L2 holds the tile's token rows (their up to k reads hit it).
// Measured on MI355X against the token-major walk, which writes each token's
// row to its k scattered rows: the combine backward at T = 4096, H = 2048
// 55-56 -> 47.5 us, at T = 16384, H = 4096 448 -> 403 us.
// ---------------------------------------------------------------------------
// The list entry of wave `wave` of list workgroup pb: (row, token), or row -1
// for an empty position, a position past the last tile, or a row outside
// [0, R).  Uniform over the wave.
__device__ __forceinline__ int2 list_entry(const RowArgs &a, int64_t pb, int wave)
{
    // positions and tiles fit 32 bits (the list has at most T * k < 2^31 entries)
    const int2 none = make_int2(-1, -1);
    const int x = static_cast<int>(pb % kXcds);
    const int p = static_cast<int>(pb / kXcds) * 4 + wave;
    const int cap = static_cast<int>(a.pg.cap);
    const int i = p / cap;
    const int tau = x + kXcds * i;
    if (tau >= a.pg.ntiles)
        return none;
    const int q = p - i * cap;
    const int64_t t0 = static_cast<int64_t>(tau) * a.pg.tile_tokens;
    const int64_t tt = min(a.pg.tile_tokens, a.T - t0);
    if (q >= tt * a.pg.kk)
        return none;
    const int2 pr = a.pairs[pb * 4 + wave];
    // a row past R, or a token outside the entry's tile, is no row: the
    // accesses stay inside the buffers whatever the workspace holds
    if (pr.x < 0 || pr.x >= a.R || pr.y < t0 || pr.y >= t0 + tt)
        return none;
    return make_int2(__builtin_amdgcn_readfirstlane(pr.x), __builtin_amdgcn_readfirstlane(pr.y));
}

// 16-byte chunks per lane that a wave of the list kernels loads before it
// stores: the dispatch takes rows of up to 8 chunks per lane (8 KiB,
// H = 4096) in one batch, the backward, which loads two rows (grad_out and
// the expert output), up to 4 pairs.  A wave's loads also wait for its
// earlier stores (one counter), so one batch per row keeps the row's loads
// together; how many rows are in flight is set by the residency
// (list_waves).  The backward measured 2 % slower with batches of 8 pairs.
constexpr int kListCopyMax = 8;
constexpr int kListBwdMax = 4;

// N chunks per lane, c0 + i * 64 + lane for i < N, all present: no per-chunk
// test, so the loads issue back to back.
template <int N>
__device__ __forceinline__ void list_copy_n(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int c0,
                                            int lane)
{
    u32x4 v[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = src[c0 + i * kWave + lane];
#pragma unroll
    for (int i = 0; i < N; ++i)
        put16<MOE_NT_COPY_ROWS != 0>(dst + c0 + i * kWave + lane, v[i]);
}

// list_copy_n<n> for a wave-uniform n in [1, N].
template <int N>
__device__ __forceinline__ void list_copy_upto(int n, const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                               int c0, int lane)
{
    if (n == N)
        list_copy_n<N>(src, dst, c0, lane);
    else if constexpr (N > 1)
        list_copy_upto<N - 1>(n, src, dst, c0, lane);
}

// A row of nch chunks (nch a multiple of 32): batches of kListCopyMax chunks
// per lane, the rest in one batch of its own size, then the half-wave chunk
// of an H that is an odd multiple of 256.
__device__ __forceinline__ void list_copy_row(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int nch,
                                              int lane)
{
    int n = nch / kWave;
    int c0 = 0;
    for (; n > kListCopyMax; n -= kListCopyMax, c0 += kListCopyMax * kWave)
        list_copy_n<kListCopyMax>(src, dst, c0, lane);
    if (n > 0)
        list_copy_upto<kListCopyMax>(n, src, dst, c0, lane);
    c0 += n * kWave;
    if (c0 + lane < nch)
        put16<MOE_NT_COPY_ROWS != 0>(dst + c0 + lane, src[c0 + lane]);
}

// Dispatch of one row from the list: the token's row copied whole, its token
// and merged weight recorded (the first slot's weight plus its repeats', in
// slot order).
__device__ __forceinline__ void list_dispatch(const RowArgs &a, int64_t pb)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int2 rt = list_entry(a, pb, wave);
    const int r = rt.x, t = rt.y;
    if (r < 0)
        return;
    // the token's slots and weights (for row_w), loaded now so that their
    // latency overlaps the row's
    const int k = a.k;
    const int64_t s = static_cast<int64_t>(t) * k + lane;
    const int rj = (a.row_w && lane < k) ? a.row_of_slot[s] : -1;
    const float wj = (a.row_w && lane < k && a.topk_w) ? a.topk_w[s] : 0.f;
    const int nch = a.H >> 3;
    const u32x4 *__restrict__ src = reinterpret_cast<const u32x4 *>(a.src + static_cast<int64_t>(t) * a.H);
    u32x4 *__restrict__ dst = reinterpret_cast<u32x4 *>(a.rows + static_cast<int64_t>(r) * a.H);
    list_copy_row(src, dst, nch, lane);
    if (a.row_token && lane == 0)
        a.row_token[r] = t;
    if (a.row_w) {
        uint64_t m = __ballot(rj == r);
        float W = 0.f;
        bool first = true;
        while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j));
            W = first ? v : W + v;
            first = false;
        }
        if (lane == 0)
            a.row_w[r] = W;
    }
}

// The combine backward's step on one 16-byte chunk: grad_out's chunk stored
// to the grad row and multiplied with the expert output's into the fp64 sum.
__device__ __forceinline__ void list_bwd_chunk(u32x4 *__restrict__ dst, const u32x4 &g, const u32x4 &f,
                                               double &acc)
{
    put16<MOE_NT_COPY_ROWS != 0>(dst, g);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc = fma(static_cast<double>(bf16_lo(g[q])), static_cast<double>(bf16_lo(f[q])), acc);
        acc = fma(static_cast<double>(bf16_hi(g[q])), static_cast<double>(bf16_hi(f[q])), acc);
    }
}

// N chunk pairs per lane, all present, loads first (as list_copy_n).
template <int N>
__device__ __forceinline__ void list_bwd_n(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                           const u32x4 *__restrict__ frow, int c0, int lane, double &acc)
{
    u32x4 g[N], f[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        g[i] = src[c0 + i * kWave + lane];
        f[i] = __builtin_nontemporal_load(frow + c0 + i * kWave + lane);
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
        list_bwd_chunk(dst + c0 + i * kWave + lane, g[i], f[i], acc);
}

template <int N>
__device__ __forceinline__ void list_bwd_upto(int n, const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                              const u32x4 *__restrict__ frow, int c0, int lane, double &acc)
{
    if (n == N)
        list_bwd_n<N>(src, dst, frow, c0, lane, acc);
    else if constexpr (N > 1)
        list_bwd_upto<N - 1>(n, src, dst, frow, c0, lane, acc);
}

// Combine backward of one row from the list (launched with dw; expert_out is
// given whenever a row exists): grad_out's token row copied to the grad row,
// and its dot with the expert-output row (exact products, fp64 sums: each
// lane's elements in order, then a fixed butterfly) given to every slot of
// the token that names the row.
__device__ __forceinline__ void list_bwd(const RowArgs &a, int64_t pb)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int2 rt = list_entry(a, pb, wave);
    const int r = rt.x, t = rt.y;
    if (r < 0)
        return;
    // the token's slots (for dw), loaded now so that their latency overlaps
    // the rows'
    const int k = a.k;
    const int64_t s = static_cast<int64_t>(t) * k + lane;
    const int rj = lane < k ? a.row_of_slot[s] : -1;
    const int nch = a.H >> 3;
    const u32x4 *__restrict__ src = reinterpret_cast<const u32x4 *>(a.src + static_cast<int64_t>(t) * a.H);
    u32x4 *__restrict__ dst = reinterpret_cast<u32x4 *>(a.rows + static_cast<int64_t>(r) * a.H);
    const u32x4 *__restrict__ frow = reinterpret_cast<const u32x4 *>(a.F + static_cast<int64_t>(r) * a.H);
    // each lane's chunks in ascending order: batches of kListBwdMax pairs,
    // the rest in one batch, then the half-wave chunk (as list_copy_row)
    double acc = 0.0;
    int n = nch / kWave;
    int c0 = 0;
    for (; n > kListBwdMax; n -= kListBwdMax, c0 += kListBwdMax * kWave)
        list_bwd_n<kListBwdMax>(src, dst, frow, c0, lane, acc);
    if (n > 0)
        list_bwd_upto<kListBwdMax>(n, src, dst, frow, c0, lane, acc);
    c0 += n * kWave;
    if (c0 + lane < nch)
        list_bwd_chunk(dst + c0 + lane, src[c0 + lane], __builtin_nontemporal_load(frow + c0 + lane), acc);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1)
        acc += __shfl_xor(acc, o);
    if (rj == r)
        a.dw[s] = static_cast<float>(acc);
}

// dw of the slots that have no row (empty, not local, or outside [0, R)):
// one thread per slot.
__device__ __forceinline__ void zero_dw_no_row(const RowArgs &a, int64_t zb)
{
    const int64_t s = zb * kRowThreads + threadIdx.x;
    if (s >= a.T * a.k)
        return;
    const int r = a.row_of_slot[s];
    if (r < 0 || r >= a.R)
        a.dw[s] = 0.f;
}

// Grid: [sentinel blocks][list blocks][expert blocks].
__global__ void __launch_bounds__(kRowThreads) k_rows_list(RowArgs a)
{
    int64_t bid = blockIdx.x;
    if (bid < a.nsent_blocks) {
        fill_sentinel(a, bid);
        return;
    }
    bid -= a.nsent_blocks;
    if (bid < a.npair_blocks) {
        list_dispatch(a, bid);
        return;
    }
    fill_expert(a, static_cast<int>(bid - a.npair_blocks));
}

// Grid: [sentinel blocks][list blocks][dw-zero blocks][expert blocks].
__global__ void __launch_bounds__(kRowThreads) k_bwd_list(RowArgs a)
{
    int64_t bid = blockIdx.x;
    if (bid < a.nsent_blocks) {
        fill_sentinel(a, bid);
        return;
    }
    bid -= a.nsent_blocks;
    if (bid < a.npair_blocks) {
        list_bwd(a, bid);
        return;
    }
    bid -= a.npair_blocks;
    if (bid < a.nzero_blocks) {
        zero_dw_no_row(a, bid);
        return;
    }
    fill_expert(a, static_cast<int>(bid - a.nzero_blocks));
}

// ---------------------------------------------------------------------------
// Decode-sized route and dispatch in one launch.  A sync-free route of at
// most kTinySlots slots (T*k <= 16) is cheap enough for every workgroup of
// the dispatch to compute it from the ids into its own LDS, so no workgroup
// waits for another.  Measured on MI355X (16 decode layers per HIP graph, H =
// 2048): 9.07 -> 7.48 us per layer at 8 slots, 9.91 -> 9.09 at 16, but 10.1
// -> 11.6 at 32 slots, where the route's lane loops cost more than the
// launch they save.  The dispatch's own code then moves the rows, reading
// that LDS copy of the handle, and workgroup 0 publishes the handle (multihot
// map and probs, tokens_per_expert, offsets, row of every slot, status).  The
// route is the same as route.hip's: repeated ids keep their first slot's row,
// rows inside an expert's group follow ascending slots (hence tokens), and
// offsets are padded to P.
// ---------------------------------------------------------------------------
struct TinyRoute {
    int32_t ros[kWave];         // row of each slot, -1 if empty or not local
    int32_t tpe[kMaxLocal];     // routes per local expert
    int32_t off[kMaxLocal + 1]; // padded offsets, off[EL] = total
    int32_t status[4];          // {total, flags, data rows, 0}
    int32_t id[kWave];          // id of each first slot of a valid id, else -1
    float w[kWave];             // that slot's merged weight (multihot probs)
    int32_t wsum[kRowWaves];    // per-wave sums of the offsets scan
};

// Every thread of the workgroup calls this; wave 0 holds one slot per lane,
// and its lanes compare slots by lane reads over the n = T*k slots.
__device__ void tiny_route(const RouteArgs &r, TinyRoute &tr)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int EL = r.EL;
    const int k = r.k;
    const int n = static_cast<int>(r.T * k);
    for (int x = tid; x < EL; x += kRowThreads)
        tr.tpe[x] = 0;
    __syncthreads();
    int id = -1, rank = 0, first = lane;
    if (wave == 0) {
        bool bad = false;
        float myw = 0.f;
        if (lane < n) {
            const int64_t v = r.idx_i64 ? static_cast<const int64_t *>(r.idx)[lane]
                                        : static_cast<const int32_t *>(r.idx)[lane];
            if (v >= -1 && v < r.E)
                id = static_cast<int>(v);
            else
                bad = true;
            if (r.w)
                myw = r.w[lane];
        }
        // a repeated id points back at the token's first slot of that id
        const int t0 = (lane / k) * k;
        for (int q = 0; q < n; ++q) {
            const int iq = __builtin_amdgcn_readlane(id, q);
            if (q >= t0 && q < first && iq == id && id >= 0)
                first = q;
        }
        const bool dup = id >= 0 && first != lane;
        // first slots of local ids: rank among the earlier ones of the same
        // expert (ascending slot = ascending token), and the expert's count
        const int e = (id >= r.lb && id < r.lb + EL && !dup) ? id - r.lb : -1;
        int cnt = 0;
        for (int q = 0; q < n; ++q) {
            const int eq = __builtin_amdgcn_readlane(e, q);
            if (e >= 0 && eq == e) {
                ++cnt;
                rank += q < lane ? 1 : 0;
            }
        }
        if (e >= 0 && rank == 0)
            tr.tpe[e] = cnt;
        // a first slot's merged weight: its own plus its repeats', in slot order
        float wt = myw;
        if (r.w) {
            const int t1 = t0 + k;
            for (int q = 0; q < n; ++q) {
                const int iq = __builtin_amdgcn_readlane(id, q);
                const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myw), q));
                if (q > lane && q < t1 && iq == id && id >= 0 && !dup)
                    wt = wt + wq;
            }
        }
        tr.id[lane] = (id >= 0 && !dup) ? id : -1;
        tr.w[lane] = wt;
        const uint64_t mbad = __ballot(bad), mdup = __ballot(dup), mdata = __ballot(e >= 0);
        if (lane == 0) {
            tr.status[1] = (mbad ? 1 : 0) | (mdup ? 2 : 0);
            tr.status[2] = __popcll(mdata);
            tr.status[3] = 0;
        }
    }
    __syncthreads();
    // offsets: each thread sums the padded counts of a run of experts, then a
    // workgroup exclusive scan over the runs
    const int P = r.P;
    const int per = (EL + kRowThreads - 1) / kRowThreads;
    const int e0 = min(EL, tid * per), e1 = min(EL, e0 + per);
    int sp = 0;
    for (int x = e0; x < e1; ++x)
        sp += (tr.tpe[x] + P - 1) / P * P;
    int incl = sp;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o)
            incl += v;
    }
    if (lane == kWave - 1)
        tr.wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w2 = 0; w2 < wave; ++w2)
        before += tr.wsum[w2];
    int run = before + incl - sp;
    for (int x = e0; x < e1; ++x) {
        tr.off[x] = run;
        run += (tr.tpe[x] + P - 1) / P * P;
    }
    if (tid == kRowThreads - 1) {
        tr.off[EL] = before + incl;
        tr.status[0] = before + incl;
    }
    __syncthreads();
    if (wave == 0) {
        // a slot's row: its first slot's, at the expert's offset plus rank
        const int rf = __shfl(rank, first);
        const int el = id - r.lb;
        const bool local = id >= 0 && el >= 0 && el < EL;
        tr.ros[lane] = local ? tr.off[el] + rf : -1;
    }
    __syncthreads();
}

// Workgroup 0 writes the handle of the tiny route to global memory.
__device__ void publish_tiny(const RouteArgs &r, const TinyRoute &tr)
{
    const int tid = threadIdx.x;
    const int EL = r.EL;
    const int k = r.k;
    for (int e = tid; e < EL; e += kRowThreads) {
        r.tpe[e] = tr.tpe[e];
        r.off[e] = tr.off[e];
    }
    if (tid == 0) {
        r.off[EL] = tr.off[EL];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.status[i] = tr.status[i];
    }
    if (tid < r.T * k)
        r.row_of_slot[tid] = tr.ros[tid];
    if (!r.map && !r.probs)
        return;
    const int64_t ne = r.T * r.E;
    for (int64_t i = tid; i < ne; i += kRowThreads) {
        const int t = static_cast<int>(i / r.E);
        const int ex = static_cast<int>(i - static_cast<int64_t>(t) * r.E);
        uint8_t m = 0;
        float p = 0.f;
        for (int j = 0; j < k; ++j) {
            if (tr.id[t * k + j] == ex) {
                m = 1;
                p = tr.w[t * k + j];
            }
        }
        if (r.map)
            r.map[i] = m;
        if (r.probs)
            r.probs[i] = p;
    }
}

struct TinyArgs {
    RowArgs rows;
    RouteArgs route;
};

// Grid as k_move_rows, the sync-free tail zeroed by its sentinel blocks.
template <int SEG>
__global__ void __launch_bounds__(kRowThreads) k_route_move_tiny(TinyArgs f)
{
    __shared__ TinyRoute tr;
    tiny_route(f.route, tr);
    if (blockIdx.x == 0)
        publish_tiny(f.route, tr);
    RowArgs a = f.rows;
    a.row_of_slot = tr.ros;
    a.tpe = tr.tpe;
    a.off = tr.off;
    a.status = tr.status;
    int64_t bid = blockIdx.x;
    if (bid < a.nsent_blocks) {
        fill_sentinel(a, bid);
        return;
    }
    bid -= a.nsent_blocks;
    if (bid < a.ntok_blocks)
        move_token<SEG>(a, bid);
    else
        fill_expert(a, static_cast<int>(bid - a.ntok_blocks));
}

// ---------------------------------------------------------------------------
// combine backward, split form: the grad rows are a plain dispatch of
// grad_out (move_token), and dw comes from dot workgroups of their own.  In a
// dot workgroup a token's row is dealt over dot_wpt waves (1, 2 or 4), each
// walking its segments of SEG chunks per lane with the fp64 partial dots of
// up to kDotBatch rows in registers; the wave sums (wave_sums4 for 1 KiB
// segments and batches of four, a butterfly per row otherwise), then the
// token's first wave adding its waves' sums in wave order through LDS, end
// each batch.  So dw is the same on every run.  The dot workgroups hold only
// dot waves, all running the same number of batch rounds, so their barriers
// never wait on copying work.  Copy and dot workgroups are interleaved by
// token: every four tokens get waves_per_token copy workgroups, then dot_wpt
// dot workgroups.
// ---------------------------------------------------------------------------
// Exchange of two fp64 values across lane halves with gfx950's lane-half
// swaps: v_permlane32_swap (O = 32) trades the upper 32 lanes of its first
// operand with the lower 32 lanes of its second, v_permlane16_swap (O = 16)
// the odd 16-lane rows of the first with the even rows of the second.  After
// swapping (a, b), a lane whose bit O is clear holds (its a, its partner's a)
// and the other lane (its partner's b, its b), so one add leaves each lane
// the two-lane sum of the value it keeps: a in the lower lanes, b in the
// upper ones.
template <int O>
__device__ __forceinline__ double swap_halves_add(double a, double b)
{
    static_assert(O == 16 || O == 32, "lane-half swaps exist for 16 and 32");
    const uint64_t ua = static_cast<uint64_t>(__double_as_longlong(a));
    const uint64_t ub = static_cast<uint64_t>(__double_as_longlong(b));
    const uint32_t alo = static_cast<uint32_t>(ua), ahi = static_cast<uint32_t>(ua >> 32);
    const uint32_t blo = static_cast<uint32_t>(ub), bhi = static_cast<uint32_t>(ub >> 32);
    uint32_t na_lo, na_hi, nb_lo, nb_hi;
    if constexpr (O == 32) {
        const auto lo = __builtin_amdgcn_permlane32_swap(alo, blo, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(ahi, bhi, false, false);
        na_lo = lo[0], nb_lo = lo[1], na_hi = hi[0], nb_hi = hi[1];
    } else {
        const auto lo = __builtin_amdgcn_permlane16_swap(alo, blo, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(ahi, bhi, false, false);
        na_lo = lo[0], nb_lo = lo[1], na_hi = hi[0], nb_hi = hi[1];
    }
    const double na = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(na_hi) << 32) | na_lo));
    const double nb = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(nb_hi) << 32) | nb_lo));
    return na + nb;
}

// An fp64 value moved across lanes by a DPP lane pattern (within each 16-lane
// row; every source lane exists for the patterns used here).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, 0xF, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, 0xF, 0xF, false));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i in each 8-lane half-row
constexpr int kDppMirror = 0x140;    // lane i <-> 15 - i in each 16-lane row

// Wave sums of the 4 fp64 values each lane holds (one per row of a dot
// batch), in a fixed order and without LDS.  Two lane-half exchanges halve
// the values a lane carries (4 -> 2 -> 1; lane l keeps row 2*bit5 + bit4 of
// l, i.e. l >> 4); then each 16-lane row is summed by DPP: xor 1 and xor 2,
// then the half-row and row mirrors, which pair the already equal quads and
// half-rows as xor 4 and xor 8 would.  Every lane of row group b ends with
// the wave's sum of value b.
__device__ __forceinline__ double wave_sums4(double (&v)[4])
{
    v[0] = swap_halves_add<32>(v[0], v[2]);
    v[1] = swap_halves_add<32>(v[1], v[3]);
    double s = swap_halves_add<16>(v[0], v[1]);
    s = s + dpp_f64<kDppXor1>(s);
    s = s + dpp_f64<kDppXor2>(s);
    s = s + dpp_f64<kDppHalfMirror>(s);
    s = s + dpp_f64<kDppMirror>(s);
    return s;
}

template <int SEG>
__device__ __forceinline__ void dot_tokens(const RowArgs &a, int64_t db)
{
    __shared__ double red[kRowWaves][kDotBatch];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wpt = a.dot_wpt;
    const int tl = wave / wpt;
    const int wt = wave - tl * wpt;
    const int64_t t = db * (kRowWaves / wpt) + tl;
    const bool active = t < a.T;
    const int k = a.k;
    const Slots sl = load_slots(a.row_of_slot, t, k, a.R, lane, active);
    float mydw = 0.f;
    const int nch = a.H >> 3;
    constexpr int SPAN = SEG * kWave;
    const int nseg = (nch + SPAN - 1) / SPAN;
    // the same number of rounds in every wave of the workgroup (barriers)
    const int rounds = (k + kDotBatch - 1) / kDotBatch;
    uint64_t mrest = sl.prim_mask;
    for (int rd = 0; rd < rounds; ++rd) {
        const Batch<kDotBatch> bt = take_batch<kDotBatch>(mrest, sl.row);
        double part[kDotBatch];
#pragma unroll
        for (int b = 0; b < kDotBatch; ++b)
            part[b] = 0.0;
        if (bt.n > 0) {
            for (int sg = wt; sg < nseg; sg += wpt) {
                const int c0 = sg * SPAN;
                u32x4 v[SEG];
                load_seg<SEG>(v, a.src, t, a.H, c0, nch, lane);
                u32x4 f[kDotBatch][SEG];
#pragma unroll
                for (int b = 0; b < kDotBatch; ++b)
                    if (b < bt.n)
                        load_seg<SEG, MOE_NT_DOT_F != 0>(f[b], a.F, bt.row[b], a.H, c0, nch, lane);
                // 1 KiB segments: grad_out's 8 elements widened once for every
                // row of the batch.  Larger segments widen them per use, which
                // keeps 16 VGPRs per KiB free for occupancy.
                constexpr bool kWiden = SEG == 1;
                double gd[kWiden ? 8 : 1];
                if constexpr (kWiden) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        gd[2 * q] = static_cast<double>(bf16_lo(v[0][q]));
                        gd[2 * q + 1] = static_cast<double>(bf16_hi(v[0][q]));
                    }
                }
#pragma unroll
                for (int b = 0; b < kDotBatch; ++b) {
                    if (b < bt.n) {
#pragma unroll
                        for (int i = 0; i < SEG; ++i) {
                            if (c0 + i * kWave + lane < nch) {
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const uint32_t gw = v[i][q], fw = f[b][i][q];
                                    const double g0 = kWiden ? gd[2 * q] : static_cast<double>(bf16_lo(gw));
                                    const double g1 =
                                        kWiden ? gd[2 * q + 1] : static_cast<double>(bf16_hi(gw));
                                    part[b] = fma(g0, static_cast<double>(bf16_lo(fw)), part[b]);
                                    part[b] = fma(g1, static_cast<double>(bf16_hi(fw)), part[b]);
                                }
                            }
                        }
                    }
                }
            }
        }
        if constexpr (SEG == 1 && kDotBatch == 4) {
            // the batch's four rows summed over the wave at once; row b ends
            // in lanes 16 b .. 16 b + 15
            const double sum = wave_sums4(part);
            const int b = lane >> 4;
            if ((lane & 15) == 0 && b < bt.n)
                red[wave][b] = sum;
        } else {
            // one butterfly per row: fewer registers live at once.  Every
            // lane ends with the row's wave sum, so a wave that is its
            // token's only dot wave takes its dots from there, with no LDS.
#pragma unroll
            for (int b = 0; b < kDotBatch; ++b) {
                if (b < bt.n) {
                    double sum = part[b];
#pragma unroll
                    for (int o = kWave / 2; o >= 1; o >>= 1)
                        sum += __shfl_xor(sum, o);
                    if (wpt == 1) {
                        if (sl.valid && sl.first == bt.lane[b])
                            mydw = static_cast<float>(sum);
                    } else if (lane == 0) {
                        red[wave][b] = sum;
                    }
                }
            }
            // one dot wave per token (the same for the whole workgroup): no
            // exchange between waves, so no barrier
            if (wpt == 1)
                continue;
        }
        __syncthreads();
        if (wt == 0) {
#pragma unroll
            for (int b = 0; b < kDotBatch; ++b) {
                if (b < bt.n) {
                    double sum = red[wave][b];
                    for (int w = 1; w < wpt; ++w)
                        sum += red[wave + w][b];
                    if (sl.valid && sl.first == bt.lane[b])
                        mydw = static_cast<float>(sum);
                }
            }
        }
        __syncthreads();
    }
    if (active && wt == 0 && lane < k)
        a.dw[t * k + lane] = sl.valid ? mydw : 0.f;
}

// Workgroups per period (four tokens) of the combine backward's middle part.
__host__ __device__ __forceinline__ int64_t bwd_period_blocks(const RowArgs &a)
{
    return a.waves_per_token + a.dot_wpt;
}

// Workgroups of the middle part of the combine backward's grid: the periods,
// padded to a multiple of 8 for the XCD-aware order.
__host__ __device__ __forceinline__ int64_t bwd_mid_blocks(const RowArgs &a)
{
    const int64_t np = (a.ndot_blocks + 7) / 8 * 8;
    return np * bwd_period_blocks(a);
}

// Grid: [sentinel blocks][periods of (waves_per_token copy blocks, dot_wpt
// dot blocks), 4 tokens each][expert blocks].
template <int SEG, int DSEG>
__global__ void __launch_bounds__(kRowThreads) k_bwd_split(RowArgs a)
{
    int64_t bid = blockIdx.x;
    if (bid < a.nsent_blocks) {
        fill_sentinel(a, bid);
        return;
    }
    bid -= a.nsent_blocks;
    const int64_t per = bwd_period_blocks(a);
    const int64_t nmid = bwd_mid_blocks(a);
    if (bid < nmid) {
        // Workgroup j is dispatched to XCD j % 8 (nsent_blocks is a multiple
        // of 8): all workgroups of a period go to XCD period % 8, one after
        // another, so the dot waves find grad_out in that XCD's L2 where the
        // copy waves just read it.
        const int64_t slot = bid >> 3;
        const int64_t period = (slot / per) * 8 + (bid & 7);
        const int64_t pos = slot % per;
        if (period >= a.ndot_blocks)
            return;
        if (pos < a.waves_per_token)
            move_token<SEG>(a, period * a.waves_per_token + pos);
        else
            dot_tokens<DSEG>(a, period * a.dot_wpt + (pos - a.waves_per_token));
        return;
    }
    fill_expert(a, static_cast<int>(bid - nmid));
}

// ---------------------------------------------------------------------------
// FP8 dispatch: each token row is quantized once, in 128-element blocks with
// one fp32 scale each, and the E4M3 codes are written to every one of the
// token's rows.  A lane holds 8 consecutive elements (one 16-byte chunk of
// the bf16 row), so a block is 16 consecutive lanes: its amax is a 4-step
// butterfly inside the 16-lane group, and the lane at the group's start
// writes the block's scale.  Quantization (one fp32 scale per 128 elements):
//   a = max(amax, 1e-4), scale = a / 448, q = e4m3(clamp(x * (448 / a))).
// ---------------------------------------------------------------------------
constexpr float kE4M3Max = 448.0f;
constexpr float kAmaxFloor = 1e-4f;

// E4M3 code of y (|y| <= 448, not NaN), nearest with ties to even: normal
// magnitudes keep 3 of the 23 fp32 mantissa bits (round half to even on the
// 20 dropped bits, a carry moving into the exponent), and the exponent bias
// moves from 127 to 7; below 2^-6 the code is the count of 2^-9 steps.
__device__ __forceinline__ uint32_t e4m3_sw(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t m = u & 0x7FFFFFFFu;
    uint32_t code;
    if (m >= 0x3C800000u) // 2^-6
        code = ((m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
    else
        code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(m) * 512.0f));
    return sign | code;
}

// Eight values -> eight E4M3 codes, element i in byte i.
__device__ __forceinline__ u32x2 e4m3_pack8(const float (&y)[8])
{
    u32x2 r;
#if MOE_FP8_HW
    // gfx950 converts to the OCP E4M3 format, rounding to nearest even
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
    r[0] = static_cast<uint32_t>(w0);
    r[1] = static_cast<uint32_t>(w1);
#else
    r[0] = e4m3_sw(y[0]) | (e4m3_sw(y[1]) << 8) | (e4m3_sw(y[2]) << 16) | (e4m3_sw(y[3]) << 24);
    r[1] = e4m3_sw(y[4]) | (e4m3_sw(y[5]) << 8) | (e4m3_sw(y[6]) << 16) | (e4m3_sw(y[7]) << 24);
#endif
    return r;
}

template <int SEG>
__device__ __forceinline__ void quant_token(const RowArgs &a, int64_t bid)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nwt = a.waves_per_token;
    const int tl = wave / nwt;
    const int wt = wave - tl * nwt;
    const int64_t t = bid * (kRowWaves / nwt) + tl;
    if (t >= a.T)
        return;
    const Slots sl = load_slots(a.row_of_slot, t, a.k, a.R, lane, true);
    if (wt == 0)
        write_row_meta(a, sl, t, lane, true);
    if (!sl.prim_mask)
        return;
    const int nch = a.H >> 3; // bf16 chunks of 8 elements per token row
    const int nb = a.H >> 7;  // scale blocks per row
    constexpr int SPAN = SEG * kWave;
    const int nseg = (nch + SPAN - 1) / SPAN;
    for (int sg = wt; sg < nseg; sg += nwt) {
        const int c0 = sg * SPAN;
        u32x4 v[SEG];
        load_seg<SEG>(v, a.src, t, a.H, c0, nch, lane);
        u32x2 q[SEG];
        float sc[SEG];
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            const bool in = c0 + i * kWave + lane < nch;
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = in ? bf16_lo(v[i][j]) : 0.f;
                x[2 * j + 1] = in ? bf16_hi(v[i][j]) : 0.f;
            }
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                m = fmaxf(m, fabsf(x[j]));
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1)
                m = fmaxf(m, __shfl_xor(m, o, 16));
            const float am = fmaxf(m, kAmaxFloor);
            sc[i] = __fdiv_rn(am, kE4M3Max);
            const float inv = __fdiv_rn(kE4M3Max, am);
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                y[j] = fminf(fmaxf(x[j] * inv, -kE4M3Max), kE4M3Max);
            q[i] = e4m3_pack8(y);
        }
        uint64_t mrest = sl.prim_mask;
        while (mrest) {
            const Batch<kCopyBatch> bt = take_batch<kCopyBatch>(mrest, sl.row);
#pragma unroll
            for (int b = 0; b < kCopyBatch; ++b) {
                if (b < bt.n) {
                    u32x2 *__restrict__ dst = reinterpret_cast<u32x2 *>(a.rows_q + bt.row[b] * a.H);
                    float *__restrict__ ds = a.row_scale + bt.row[b] * nb;
#pragma unroll
                    for (int i = 0; i < SEG; ++i) {
                        const int c = c0 + i * kWave + lane;
                        if (c < nch) {
                            if (MOE_NT_COPY_ROWS)
                                __builtin_nontemporal_store(q[i], dst + c);
                            else
                                dst[c] = q[i];
                            if ((lane & 15) == 0)
                                ds[c >> 4] = sc[i];
                        }
                    }
                }
            }
        }
    }
}

// Grid as k_move_rows: [sentinel blocks][token blocks][expert blocks].
template <int SEG>
__global__ void __launch_bounds__(kRowThreads) k_dispatch_fp8(RowArgs a)
{
    int64_t bid = blockIdx.x;
    if (bid < a.nsent_blocks) {
        fill_sentinel(a, bid);
        return;
    }
    bid -= a.nsent_blocks;
    if (bid < a.ntok_blocks)
        quant_token<SEG>(a, bid);
    else
        fill_expert(a, static_cast<int>(bid - a.ntok_blocks));
}

// ---------------------------------------------------------------------------
// combine (and the dispatch backward, which is the same sum plus a gather of
// the weight gradients): one wave per (token, segment); the waves of a
// workgroup read all segments of a token's rows at about the same time
// ---------------------------------------------------------------------------
// GW: the dispatch backward (also gathers the weight gradients of the slots).
template <int SEG, bool OUT_F32, bool GW>
__global__ void __launch_bounds__(kRowThreads) k_combine(CombineArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nch = a.H >> 3;
    constexpr int SPAN = SEG * kWave;
    const int nseg = (nch + SPAN - 1) / SPAN;
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * kRowWaves + wave;
    const int64_t t = gw / nseg;
    const int c0 = static_cast<int>(gw - t * nseg) * SPAN;
    if (gw == 0 && lane == 0 && a.eager && a.status[0] != a.R)
        atomicOr(&a.status[1], 4);
    if (t >= a.T)
        return;
    const Slots sl = load_slots(a.row_of_slot, t, a.k, a.R, lane, true);
    float acc[SEG][8];
#pragma unroll
    for (int i = 0; i < SEG; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[i][q] = 0.f;
    bool first = true;
    uint64_t mrest = sl.prim_mask;
    while (mrest) {
        const Batch<kCombBatch> bt = take_batch<kCombBatch>(mrest, sl.row);
        u32x4 f[kCombBatch][SEG];
#pragma unroll
        for (int b = 0; b < kCombBatch; ++b)
            if (b < bt.n)
                load_seg<SEG, true>(f[b], a.Y, bt.row[b], a.H, c0, nch, lane);
#pragma unroll
        for (int b = 0; b < kCombBatch; ++b) {
            if (b < bt.n) {
#pragma unroll
                for (int i = 0; i < SEG; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float lo = bf16_lo(f[b][i][q]);
                        const float hi = bf16_hi(f[b][i][q]);
                        acc[i][2 * q] = first ? lo : acc[i][2 * q] + lo;
                        acc[i][2 * q + 1] = first ? hi : acc[i][2 * q + 1] + hi;
                    }
                }
                first = false;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
        const int c = c0 + i * kWave + lane;
        if (c >= nch)
            continue;
        if (OUT_F32) {
            f32x4 *o = reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + t * a.H) + 2 * c;
            const f32x4 v0 = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
            const f32x4 v1 = {acc[i][4], acc[i][5], acc[i][6], acc[i][7]};
            o[0] = v0;
            o[1] = v1;
        } else {
            u32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[q] = bf16_rne(acc[i][2 * q]) | (bf16_rne(acc[i][2 * q + 1]) << 16);
            reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.out) + t * a.H)[c] = v;
        }
    }
    // dispatch backward: a slot's weight gradient is its row's (repeated ids
    // share the row, whose weight is the plain sum of theirs); 0 without a
    // row.  Last, so that its load does not hold up the rows' loads.
    if (GW && c0 == 0 && lane < a.k)
        a.grad_w[t * a.k + lane] = (sl.valid && a.grad_row_w) ? a.grad_row_w[sl.row] : 0.f;
}

// ---------------------------------------------------------------------------
// launch shapes
// ---------------------------------------------------------------------------
// 16-byte chunks per lane that cover one row (power of two, at most 16).
static int chunks_per_lane(int H)
{
    const int nch = H >> 3;
    const int need = (nch + kWave - 1) / kWave;
    int n = 1;
    while (n < need && n < 16)
        n <<= 1;
    return n;
}

// A sync-free worst-case row array of at most this many bytes has its tail
// zeroed by workgroups of the rows' launch, in 64 KiB wave tasks as in eager
// mode, instead of by a launch of its own: at decode sizes a second launch
// costs more than the writes.  Larger arrays keep the one-shot tail launch,
// whose address-ordered writes are the faster way to zero hundreds of MB.
constexpr int64_t kInlineTailBytes = int64_t(32) << 20;

static int64_t row_array_bytes(const RowArgs &a)
{
    return a.rows_q ? a.R * (a.H + (a.H >> 7) * 4) : a.R * 2 * a.H;
}

static bool tail_in_rows_launch(const RowArgs &a)
{
    return !a.eager && !a.keep_tail && row_array_bytes(a) <= kInlineTailBytes;
}

// Sentinel-fill workgroups: in sync-free mode, those of the tail's own
// launch, one piece per wave over the whole worst-case row array, or for a
// small array enough of the rows' launch for one 64 KiB task per wave; eager
// mode keeps a handful in the rows' launch for the (normally empty)
// [total, R).
static int64_t sentinel_blocks(const RowArgs &a)
{
    // always a multiple of 8, so that the workgroups after them keep their
    // index modulo the XCD count
    if (a.keep_tail)
        return 0;
    if (a.eager)
        return 8;
    if (tail_in_rows_launch(a)) {
        const int64_t task_bytes = kZeroTask * 16;
        const int64_t tasks = (row_array_bytes(a) + task_bytes - 1) / task_bytes;
        return ((tasks + kRowWaves - 1) / kRowWaves + 7) / 8 * 8;
    }
    // sync-free: the tail's own launch, one piece per wave over the whole row
    // array (the host does not know where the tail starts), and over the
    // scale array of E4M3 rows
    const int64_t pc = static_cast<int64_t>(MOE_TAIL_PIECE_KIB) * kWave;
    const int64_t nch = a.rows_q ? (a.H >> 4) : (a.H >> 3);
    int64_t pieces = (a.R * nch + pc - 1) / pc;
    if (a.rows_q)
        pieces += (a.R * (a.H >> 7) + pc * 4 - 1) / (pc * 4);
    if (a.row_token || a.row_expert || a.row_w)
        pieces += (a.R + kMetaRows - 1) / kMetaRows; // the metadata waves
    return ((pieces + kRowWaves - 1) / kRowWaves + 7) / 8 * 8;
}

static int nch_of(const RowArgs &a) { return a.H >> 3; }

#ifndef MOE_PAD_SLICE_BYTES
#define MOE_PAD_SLICE_BYTES 65536
#endif

void row_shape(RowArgs &a)
{
    const int whole = chunks_per_lane(a.H);
    // Dots: a token with about k local rows gets its row dealt over up to
    // four waves in 1 KiB segments (more loads in flight at small T).  When
    // the local experts are a small share of all experts (fewer than two
    // local rows per token on uniform routing), one wave per token in 2 KiB
    // segments does better: most dot workgroups then have little to do, and
    // their barriers would cost more than the rows they share.
    const bool sparse = static_cast<int64_t>(a.k) * a.EL < 2 * static_cast<int64_t>(a.E_total);
    const int dseg = sparse ? MOE_DOT_SEG_SPARSE : MOE_DOT_SEG;
    a.dot_seg = whole < dseg ? whole : dseg;
    const int dnseg = (nch_of(a) + a.dot_seg * kWave - 1) / (a.dot_seg * kWave);
    a.dot_wpt = sparse ? 1 : (dnseg >= 4 && MOE_DOT_MAX_WPT >= 4 ? 4 : (dnseg >= 2 && MOE_DOT_MAX_WPT >= 2 ? 2 : 1));
    // combine backward with dw: periods of four tokens
    a.ndot_blocks = a.dw ? (a.T + kRowWaves - 1) / kRowWaves : 0;
    // Copy segments: the bf16 dispatch of a layer whose local experts take
    // most routes moves 1 KiB per wave and segment (measured on MI355X: T =
    // 4096 dispatch 31.1 -> 29.9 us, T = 16384 255 -> 252 us); the FP8
    // dispatch, the sparse share and the combine backward's copy keep 2 KiB
    // (1 KiB measured slower or no faster there).
    const int cap = (!a.rows_q && !a.dw && !sparse) ? MOE_COPY_SEG_DENSE : MOE_COPY_SEG;
    a.seg = whole < cap ? whole : cap;
    const int nch = a.H >> 3;
    const int nseg = (nch + a.seg * kWave - 1) / (a.seg * kWave);
    a.waves_per_token = nseg >= 4 && MOE_MAX_WPT >= 4 ? 4 : (nseg >= 2 && MOE_MAX_WPT >= 2 ? 2 : 1);
    const int64_t tpb = kRowWaves / a.waves_per_token;
    a.ntok_blocks = (a.T + tpb - 1) / tpb;
    // Pad rows: each expert's group has at most P - 1; its workgroups share
    // them so that none zeroes more than about 64 KiB (1 to 16 per expert).
    // One workgroup zeroing 127 rows of 4 KiB (P = 128) ran alone at the end
    // of the grid.
    const int64_t row_bytes = a.rows_q ? a.H + (a.H >> 7) * 4 : static_cast<int64_t>(a.H) * 2;
    const int64_t pad_bytes = static_cast<int64_t>(a.P > 1 ? a.P - 1 : 0) * row_bytes;
    const int64_t sl = (pad_bytes + MOE_PAD_SLICE_BYTES - 1) / MOE_PAD_SLICE_BYTES;
    a.exp_slices = static_cast<int32_t>(sl < 1 ? 1 : (sl > 16 ? 16 : sl));
    a.nexp_blocks = a.R > 0 ? static_cast<int64_t>(a.EL) * a.exp_slices : 0;
    a.nsent_blocks = sentinel_blocks(a);
    // rows walked from the route's row list: the bf16 dispatch and the
    // combine backward of a handle that carries one
    if (a.rows_q)
        a.pairs = nullptr;
    a.npair_blocks = a.pairs ? a.pg.entries / 4 : 0;
    a.nzero_blocks = (a.pairs && a.dw) ? (a.T * a.k + kRowThreads - 1) / kRowThreads : 0;
}

// The sync-free tail fill, a launch of its own.
__global__ void __launch_bounds__(kRowThreads) k_sentinel_oneshot(RowArgs a)
{
    fill_sentinel_oneshot(a, blockIdx.x);
}

#ifndef MOE_LIST_FLIGHT_COPY
#define MOE_LIST_FLIGHT_COPY 16384
#endif
#ifndef MOE_LIST_FLIGHT_BWD
#define MOE_LIST_FLIGHT_BWD 24576
#endif

// Dynamic LDS that lets at most `waves` workgroups of kRowThreads threads
// (one wave per SIMD each) reside on a CU at once (160 KiB of LDS per CU;
// 512 bytes left for a kernel's own LDS); 0 = no cap.
static size_t lds_cap(int waves)
{
    constexpr size_t kLdsPerCu = 160 * 1024;
    if (waves <= 0 || waves >= 8)
        return 0;
    return ((kLdsPerCu / waves) & ~static_cast<size_t>(511)) - 512;
}

// Waves per SIMD for a list kernel: about `flight` bytes of rows per SIMD in
// flight, 2 to 8 waves.  Measured on MI355X (16384 and 4096 tokens, top-8,
// all experts local): the list dispatch of 8 KiB rows (H = 4096) runs in
// 245 us with 8 waves per SIMD, 219 us with 2 (16 KiB per SIMD) and 304 us
// with 1; with 4 KiB rows 4 waves are as fast as 8 or slightly faster.  The
// list backward (two rows loaded per wave) 417 -> 405 us with 3 waves of
// 8 KiB rows (421 with 2), best with 6 for 4 KiB rows (24 KiB).  The
// token-major kernels and the tail fill lose at any cap (up to 2x at 2
// waves), so they have none.
static int list_waves(int32_t H, int64_t flight)
{
    const int64_t w = flight / (static_cast<int64_t>(H) * 2);
    return static_cast<int>(w < 2 ? 2 : (w > 8 ? 8 : w));
}

bool move_rows_fits(const RowArgs &a)
{
    // the sync-free tail's launch and the rows' launch, each within the limit
    return a.nsent_blocks <= kMaxRowBlocks &&
           a.nsent_blocks + a.ntok_blocks + a.nexp_blocks + bwd_mid_blocks(a) <= kMaxRowBlocks &&
           a.nsent_blocks + a.npair_blocks + a.nzero_blocks + a.nexp_blocks <= kMaxRowBlocks;
}

hipError_t launch_move_rows(const RowArgs &a0, hipStream_t s)
{
    RowArgs a = a0;
    if (!move_rows_fits(a0))
        return hipErrorInvalidConfiguration;
    if (!a0.eager && a0.nsent_blocks > 0 && !tail_in_rows_launch(a0)) {
        // sync-free: the tail first, on its own, then the rows
        launch(k_sentinel_oneshot, dim3(static_cast<unsigned>(a0.nsent_blocks)), dim3(kRowThreads), 0, s, a0);
        a.nsent_blocks = 0;
    }
    if (a.pairs) {
        const int64_t nbl = a.nsent_blocks + a.npair_blocks + a.nzero_blocks + a.nexp_blocks;
        if (nbl == 0)
            return hipSuccess;
        const dim3 gl(static_cast<unsigned>(nbl));
        if (a.dw)
            launch(k_bwd_list, gl, dim3(kRowThreads), lds_cap(list_waves(a.H, MOE_LIST_FLIGHT_BWD)), s, a);
        else
            launch(k_rows_list, gl, dim3(kRowThreads), lds_cap(list_waves(a.H, MOE_LIST_FLIGHT_COPY)), s,
                   a);
        return hipGetLastError();
    }
    const int64_t nmid = a.dw ? bwd_mid_blocks(a) : a.ntok_blocks;
    const int64_t nb = a.nsent_blocks + nmid + a.nexp_blocks;
    if (nb == 0)
        return hipSuccess;
    const dim3 g(static_cast<unsigned>(nb));
    const dim3 blk(kRowThreads);
    if (a.rows_q) {
        switch (a.seg) {
        case 1: launch(k_dispatch_fp8<1>, g, blk, 0, s, a); break;
        case 2: launch(k_dispatch_fp8<2>, g, blk, 0, s, a); break;
        default: launch(k_dispatch_fp8<4>, g, blk, 0, s, a); break;
        }
    } else if (a.dw) {
        switch (a.seg * 8 + a.dot_seg) {
        case 1 * 8 + 1: launch(k_bwd_split<1, 1>, g, blk, 0, s, a); break;
        case 1 * 8 + 2: launch(k_bwd_split<1, 2>, g, blk, 0, s, a); break;
        case 1 * 8 + 4: launch(k_bwd_split<1, 4>, g, blk, 0, s, a); break;
        case 2 * 8 + 1: launch(k_bwd_split<2, 1>, g, blk, 0, s, a); break;
        case 2 * 8 + 2: launch(k_bwd_split<2, 2>, g, blk, 0, s, a); break;
        case 2 * 8 + 4: launch(k_bwd_split<2, 4>, g, blk, 0, s, a); break;
        case 4 * 8 + 1: launch(k_bwd_split<4, 1>, g, blk, 0, s, a); break;
        case 4 * 8 + 2: launch(k_bwd_split<4, 2>, g, blk, 0, s, a); break;
        default: launch(k_bwd_split<4, 4>, g, blk, 0, s, a); break;
        }
    } else {
        switch (a.seg) {
        case 1: launch(k_move_rows<1>, g, blk, 0, s, a); break;
        case 2: launch(k_move_rows<2>, g, blk, 0, s, a); break;
        default: launch(k_move_rows<4>, g, blk, 0, s, a); break;
        }
    }
    return hipGetLastError();
}

bool route_move_tiny_fits(const RowArgs &a, const RouteArgs &r)
{
    return !a.eager && !a.rows_q && !a.dw && a.T >= 1 && a.T * a.k <= kTinySlots &&
           a.T * static_cast<int64_t>(r.E) <= kTinyMapEntries && tail_in_rows_launch(a) &&
           move_rows_fits(a);
}

hipError_t launch_route_move_tiny(const RowArgs &a, const RouteArgs &r, hipStream_t s)
{
    if (!route_move_tiny_fits(a, r))
        return hipErrorInvalidConfiguration;
    TinyArgs f;
    f.rows = a;
    f.route = r;
    const int64_t nb = a.nsent_blocks + a.ntok_blocks + a.nexp_blocks;
    const dim3 g(static_cast<unsigned>(nb));
    switch (a.seg) {
    case 1: launch(k_route_move_tiny<1>, g, dim3(kRowThreads), 0, s, f); break;
    case 2: launch(k_route_move_tiny<2>, g, dim3(kRowThreads), 0, s, f); break;
    default: launch(k_route_move_tiny<4>, g, dim3(kRowThreads), 0, s, f); break;
    }
    return hipGetLastError();
}

template <bool F32, bool GW>
static void launch_comb(int seg, dim3 g, const CombineArgs &a, hipStream_t s)
{
    switch (seg) {
    case 1: launch(k_combine<1, F32, GW>, g, dim3(kRowThreads), 0, s, a); break;
    case 2: launch(k_combine<2, F32, GW>, g, dim3(kRowThreads), 0, s, a); break;
    default: launch(k_combine<4, F32, GW>, g, dim3(kRowThreads), 0, s, a); break;
    }
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t s)
{
    const int whole = chunks_per_lane(a.H);
    const int seg = whole < MOE_COMBINE_SEG ? whole : MOE_COMBINE_SEG;
    const int64_t span = static_cast<int64_t>(seg) * kWave;
    const int64_t nseg = ((a.H >> 3) + span - 1) / span;
    const int64_t nb = (a.T * nseg + kRowWaves - 1) / kRowWaves;
    if (nb == 0)
        return hipSuccess;
    if (nb > kMaxRowBlocks)
        return hipErrorInvalidConfiguration;
    const dim3 g(static_cast<unsigned>(nb));
    const bool gw = a.grad_w != nullptr;
    if (a.out_f32)
        gw ? launch_comb<true, true>(seg, g, a, s) : launch_comb<true, false>(seg, g, a, s);
    else
        gw ? launch_comb<false, true>(seg, g, a, s) : launch_comb<false, false>(seg, g, a, s);
    return hipGetLastError();
}

}  // namespace moe
