// route.hip -- routing preprocessing on gfx950: top-k ids -> multihot map,
// tokens_per_expert, padded offsets and the row of every slot.
//
// "feat: add hybridep", Changelog: the HybridEP path converts top-k indices to
// multihot routing metadata; its dispatch returns tokens_per_expert and pads
// each expert's rows to pad_multiple.  "Add the deepep expert-parallel
// implementation", "What this adds" / "Expanded layout": one row per (token,
// local expert) slot, grouped by local expert (here in ascending token order).
//
// The layout is identical on every run: the only atomics are bit-ORs into
// LDS bitmaps, whose result does not depend on their order.
//   K1 route_count   one thread per slot, one workgroup per block of whole
//                    tokens.  The block's ids (and weights) are staged in LDS
//                    with one coalesced load each.  It zero-fills its rows of
//                    the multihot map (and probs) and scatters the routed
//                    entries, detects bad and repeated ids, and sets the bit of
//                    each primary local slot in its expert's slot bitmap.  A
//                    slot's in-block rank is then the popcount of its expert's
//                    bits below it (slots are in token order, so the rank is
//                    the ascending-token rank).  Per-block expert counts go to
//                    the workspace; each slot keeps (expert << 11 | in-block
//                    rank) until the final pass.
//   K2 route_finish  one workgroup per K1 block: every block reads the whole
//                    (small) count table, forms its own per-expert base and the
//                    global totals, scans the padded totals into offsets in LDS
//                    and rewrites its slots to final rows; block 0 publishes
//                    tokens_per_expert, offsets and the status word.
//   A route that fits one K1 workgroup (decode sizes) ends in K1: its block
//   counts are the totals, so it publishes offsets and status and writes the
//   final rows itself, and K2 is not launched.
//   Large T (count table > 64 Ki entries) takes a three-launch form instead:
//   K2s route_scan (one workgroup) then K3 route_rows (one thread per slot).
#include "moe_internal.h"

#ifndef MOE_ROUTE_MAX_THREADS
#define MOE_ROUTE_MAX_THREADS 512
#endif
// 0: no row list (the row kernels walk tokens), for measurement
#ifndef MOE_ROW_LIST
#define MOE_ROW_LIST 1
#endif
#ifndef MOE_LIST_TILE_TOKENS
#define MOE_LIST_TILE_TOKENS 512
#endif

namespace moe {

// Between the passes a slot holds (expert << 11) | in-block rank: the rank is
// < 2048 (workgroups are <= 1024 threads) and the local expert < 1024.
constexpr int kRankBits = 11;
constexpr int kExpertBits = 10;

__device__ __forceinline__ int packed_expert(int v) { return (v >> kRankBits) & ((1 << kExpertBits) - 1); }
__device__ __forceinline__ int packed_rank(int v) { return v & ((1 << kRankBits) - 1); }

bool pairs_form(int64_t T, int k, int E, int EL, int tokens_per_block, int64_t nblk)
{
    (void)T;
    (void)tokens_per_block;
    return MOE_ROW_LIST && nblk > 1 && nblk * EL <= kFusedFinishMax &&
           static_cast<int64_t>(k) * EL >= 2 * static_cast<int64_t>(E);
}

PairGeom pair_geom(int64_t T, int k, int EL, int tokens_per_block, int64_t nblk)
{
    PairGeom g;
    // tiles of whole route blocks, at most about 512 tokens (4 MB of token
    // rows at H = 4096: one XCD's L2; smaller tiles read the tokens fewer
    // times but write shorter runs per expert and measure slower), tile t on
    // XCD t mod 8.  The size is the largest whose busiest XCD walks at most
    // 5 % more blocks than the best size's: 47 route blocks make 8 tiles of
    // 6 (6 blocks on the busiest XCD) rather than 6 tiles of 8 (8), 94 make
    // 16 of 6 (12) rather than 12 of 8 (16 on four XCDs, 8 on the others),
    // and 625 make tiles of 8 (80) rather than of 1 (79).
    int64_t most = MOE_LIST_TILE_TOKENS / tokens_per_block;
    if (most < 1)
        most = 1;
    auto load = [&](int64_t b) { return b * (((nblk + b - 1) / b + kXcds - 1) / kXcds); };
    int64_t least = load(1);
    for (int64_t b = 2; b <= most; ++b)
        least = load(b) < least ? load(b) : least;
    int64_t bpt = 1;
    for (int64_t b = most; b >= 1; --b)
        if (load(b) * 20 <= least * 21) {
            bpt = b;
            break;
        }
    g.bpt = bpt;
    g.tile_tokens = bpt * tokens_per_block;
    g.ntiles = T > 0 ? (T + g.tile_tokens - 1) / g.tile_tokens : 0;
    g.tiles_per_xcd = (g.ntiles + kXcds - 1) / kXcds;
    g.kk = k < EL ? k : EL;
    g.cap = g.tile_tokens * g.kk;
    // each XCD's sequence rounded up to whole workgroups (4 entries)
    g.entries = kXcds * ((g.tiles_per_xcd * g.cap + 3) / 4 * 4);
    return g;
}

constexpr int kOneBlockThreads = 1024;

RouteGeom route_geom(int64_t T, int k, int EL)
{
    RouteGeom g;
    // LDS bitmaps hold EL x threads bits: keep EL * threads <= 256 Ki
    // Workgroups of at most 512 threads: at T = 4096 that is 64 blocks for
    // 256 CUs, and their latency chains (stage, bitmap, scan, rank) are
    // shorter than at 1024 threads; measured 2 us faster per route on MI355X.
    g.threads = EL <= 256 ? 1024 : (EL <= 512 ? 512 : 256);
    if (g.threads > MOE_ROUTE_MAX_THREADS)
        g.threads = MOE_ROUTE_MAX_THREADS;
    g.tokens_per_block = g.threads / k;
    g.nblk = T > 0 ? (T + g.tokens_per_block - 1) / g.tokens_per_block : 0;
    g.slots = 1;
    // A small route in one workgroup of 1024 threads, which publishes the
    // route itself (no finishing pass): up to 1024 slots with at most 256
    // local experts, or 2048 slots at 2 per thread with at most 64.  Measured
    // on MI355X (top-8, 128 local experts, map and probs): 96 and 128 tokens
    // 10.2 and 10.5 us (two passes) -> 8.0 and 8.5 us; but 256 tokens at 2
    // slots per thread 10.8 -> 13.7 us, the scans over 64 bitmap words per
    // expert costing more than the second pass; with 32 local experts the
    // captured decode layer of 256 tokens gained 0.4-1.3 us.
    if (g.nblk > 1) {
        const int sp = (T <= kOneBlockThreads / k && EL <= 256) ? 1
                     : (T <= 2 * kOneBlockThreads / k && EL <= 64) ? 2 : 0;
        if (sp) {
            g.threads = kOneBlockThreads;
            g.slots = sp;
            g.tokens_per_block = kOneBlockThreads * sp / k;
            g.nblk = 1;
        }
    }
    return g;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// K1
// ---------------------------------------------------------------------------
// LDS of K1 for a block of `slots` slots: slot bitmaps [EL][W] u32 and their
// popcount prefixes [EL][W] u16 (W = slots/32 words per expert), staged ids
// and weights, one flag word.
static size_t count_lds_bytes(int slots, int EL)
{
    const size_t words = static_cast<size_t>(EL) * (slots / 32);
    return words * 4 + ((words + 1) & ~static_cast<size_t>(1)) * 2 +
           static_cast<size_t>(slots) * 8 + 4 +
           (2 * static_cast<size_t>(EL) + 1) * 4; // totals and offsets (one-block routes)
}

__device__ void publish(const RouteArgs &a, const int32_t *tot, int32_t *offl, int flags);

// S slots per thread: slot j*blockDim + tid of the block for j < S (S > 1
// only for a route in one workgroup of up to 2048 slots).
template <typename IT, int S>
__global__ void __launch_bounds__(1024) k_route_count(RouteArgs a)
{
    extern __shared__ int32_t lds[];
    const int nthreads = blockDim.x;
    const int nsl = nthreads * S;  // slots of a full block
    const int W = nsl / 32;        // bitmap words per expert (a divisor of 64)
    const int EL = a.EL;
    uint32_t *bm = reinterpret_cast<uint32_t *>(lds);          // [EL][W] slots of each expert
    uint16_t *pref = reinterpret_cast<uint16_t *>(bm + EL * W); // [EL][W] exclusive popcounts
    int32_t *sid = reinterpret_cast<int32_t *>(pref + ((EL * W + 1) & ~1)); // staged ids
    float *sw = reinterpret_cast<float *>(sid + nsl);                        // staged weights
    int32_t *bflag = reinterpret_cast<int32_t *>(sw + nsl);
    int32_t *tot = bflag + 1;  // [EL] the block's counts (one-block routes)
    int32_t *offl = tot + EL;  // [EL+1] offsets (one-block routes)

    const IT *__restrict__ idx = static_cast<const IT *>(a.idx);
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int64_t b = blockIdx.x;
    const int k = a.k;
    const int64_t t0 = b * a.tokens_per_block;
    const int64_t t1 = min(a.T, t0 + a.tokens_per_block);
    const int nslots = static_cast<int>((t1 - t0) * k);
    const int64_t s0 = t0 * k; // the block's first slot

    for (int i = tid; i < EL * W; i += nthreads)
        bm[i] = 0;
    int myid[S]; // -2 marks an id outside [-1, E)
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const int ls = j * nthreads + tid;
        myid[j] = -1;
        if (ls < nslots) {
            const int64_t e = static_cast<int64_t>(idx[s0 + ls]);
            myid[j] = (e >= -1 && e < a.E) ? static_cast<int>(e) : -2;
        }
        sid[ls] = myid[j];
        if (a.probs)
            sw[ls] = ls < nslots ? a.w[s0 + ls] : 0.f;
    }
    if (tid == 0)
        *bflag = 0;
    // Zero this block's rows of the map and the probs (coalesced); the routed
    // entries are written after the barrier below.
    if (a.map) {
        uint8_t *base = a.map + t0 * a.E;
        const int64_t nb = (t1 - t0) * a.E;
        if ((nb & 15) == 0 && (reinterpret_cast<uintptr_t>(base) & 15) == 0) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            for (int64_t q = tid; q < (nb >> 4); q += nthreads)
                reinterpret_cast<u32x4 *>(base)[q] = z;
        } else {
            for (int64_t q = tid; q < nb; q += nthreads)
                base[q] = 0;
        }
    }
    if (a.probs) {
        float *base = a.probs + t0 * a.E;
        const int64_t nf = (t1 - t0) * a.E;
        if ((nf & 3) == 0 && (reinterpret_cast<uintptr_t>(base) & 15) == 0) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            for (int64_t q = tid; q < (nf >> 2); q += nthreads)
                reinterpret_cast<f32x4 *>(base)[q] = z;
        } else {
            for (int64_t q = tid; q < nf; q += nthreads)
                base[q] = 0.f;
        }
    }
    __syncthreads();

    // One thread per slot: a repeated id points back at its first slot; the
    // first slot of a local expert sets its bit in that expert's bitmap.
    bool dup[S];
    int prim_back[S], tl[S], jt[S], ep[S];
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const int ls = j * nthreads + tid;
        const int id = myid[j];
        const bool bad = id == -2;
        dup[j] = false;
        prim_back[j] = 0;
        tl[j] = 0;
        jt[j] = 0;
        if (id >= 0) {
            tl[j] = ls / k;
            jt[j] = ls - tl[j] * k;
            for (int q = 0; q < jt[j]; ++q) {
                if (sid[tl[j] * k + q] == id) {
                    dup[j] = true;
                    prim_back[j] = jt[j] - q;
                    break;
                }
            }
        }
        ep[j] = (id >= a.lb && id < a.lb + EL) ? id - a.lb : -1;
        if (id >= 0 && !dup[j]) {
            if (ep[j] >= 0)
                atomicOr(&bm[ep[j] * W + (ls >> 5)], 1u << (ls & 31));
            if (a.map)
                a.map[(t0 + tl[j]) * a.E + id] = 1;
        }
        const uint64_t mbad = __ballot(bad);
        const uint64_t mdup = __ballot(dup[j]);
        if (lane == 0 && (mbad | mdup))
            atomicOr(bflag, (mbad ? 1 : 0) | (mdup ? 2 : 0));
    }
    __syncthreads();

    const int bf = *bflag;
    if (a.probs) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            if (myid[j] < 0 || dup[j])
                continue;
            // the first slot's weight plus later repeats of the id, in slot order
            const int ls = j * nthreads + tid;
            float wt = sw[ls];
            if (bf & 2)
                for (int q = jt[j] + 1; q < k; ++q)
                    if (sid[tl[j] * k + q] == myid[j])
                        wt = wt + sw[tl[j] * k + q];
            a.probs[(t0 + tl[j]) * a.E + myid[j]] = wt;
        }
    }
    // Exclusive popcount prefix of each expert's bitmap; the total is the
    // block's count for that expert.  W consecutive lanes take one expert's W
    // words and scan their popcounts together (W divides the wave).
    for (int i = tid; i < EL * W; i += nthreads) {
        const int c = __popc(bm[i]);
        int incl = c;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            if (o < W) {
                const int n = __shfl_up(incl, o, W);
                if ((lane & (W - 1)) >= o)
                    incl += n;
            }
        }
        pref[i] = static_cast<uint16_t>(incl - c);
        if ((i & (W - 1)) == W - 1) {
            a.counts[b * EL + i / W] = incl;
            tot[i / W] = incl;
        }
    }
    if (tid == 0)
        a.blockflags[b] = bf;
    __syncthreads();

    // In-block rank = earlier slots of the same expert = prefix + popcount of
    // the bits below the owning slot (the first slot, for a repeated id).
    // The whole route in this workgroup: its counts are the totals, so it
    // publishes the offsets and the status itself and writes final rows; no
    // finishing pass is launched.
    const bool one = a.nblk == 1;
    if (one)
        publish(a, tot, offl, bf);
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const int ls = j * nthreads + tid;
        if (ls >= nslots)
            continue;
        int v = -1;
        if (ep[j] >= 0) {
            const int p = ls - prim_back[j];
            const int w = p >> 5;
            const int r = pref[ep[j] * W + w] + __popc(bm[ep[j] * W + w] & ((1u << (p & 31)) - 1u));
            v = one ? offl[ep[j]] + r : (ep[j] << kRankBits) | r;
        }
        a.row_of_slot[s0 + ls] = v;
    }
}

// ---------------------------------------------------------------------------
// wave scan helper
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_up(v, o);
        if (lane >= o)
            v += n;
    }
    return v;
}

// Publish tokens_per_expert, offsets and the status word from LDS totals.
// Called by every thread of one workgroup.  Wave 0 scans the padded totals
// (lane l takes a run of consecutive experts, then a wave scan over the runs'
// sums), and one barrier makes the offsets in LDS visible to the workgroup.
// With a host alias of the status (eager mode, pinned host memory), the status
// is also written there with system-scope stores, so the host needs no copy
// after the sync.
__device__ void publish(const RouteArgs &a, const int32_t *tot, int32_t *offl, int flags)
{
    __shared__ int32_t st[4];
    const int tid = threadIdx.x;
    const int EL = a.EL;
    const int P = a.P;
    if (tid < kWave) {
        const int per = (EL + kWave - 1) / kWave;
        const int e0 = min(EL, tid * per);
        const int e1 = min(EL, e0 + per);
        int sp = 0, sd = 0;
        for (int e = e0; e < e1; ++e) {
            const int c = tot[e];
            sp += (c + P - 1) / P * P;
            sd += c;
        }
        const int incl = wave_incl_scan(sp, tid);
        const int data_incl = wave_incl_scan(sd, tid);
        int run = incl - sp;
        for (int e = e0; e < e1; ++e) {
            const int c = tot[e];
            offl[e] = run;
            if (a.status) {
                a.tpe[e] = c;
                a.off[e] = run;
            }
            run += (c + P - 1) / P * P;
        }
        if (tid == kWave - 1) {
            offl[EL] = incl;
            if (a.status) {
                a.off[EL] = incl;
                a.status[0] = incl;
                a.status[1] = flags;
                a.status[2] = data_incl;
                a.status[3] = 0;
                st[0] = incl;
                st[1] = flags;
                st[2] = data_incl;
                st[3] = 0;
            }
        }
    }
    __syncthreads();
    if (a.status && a.host_status && tid == 0) {
        // words 0..2 first, then word 3 (the host waits for it to turn 0),
        // whose release store orders the three before it at system scope
        // (system-scope fences around the stores measured 0.3 us slower per
        // route on MI355X and are not needed for that order)
#pragma unroll
        for (int i = 0; i < 3; ++i)
            __hip_atomic_store(a.host_status + i, st[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(a.host_status + 3, st[3], __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// ---------------------------------------------------------------------------
// K2 (fused finish)
// ---------------------------------------------------------------------------
// Entry of position p of XCD x's sequence in the row list: workgroup
// (p / 4) * 8 + x (which runs on XCD x), wave p % 4.
__device__ __forceinline__ int64_t pair_index(int64_t p, int64_t x)
{
    return ((p >> 2) * kXcds + x) * 4 + (p & 3);
}

// LISTS: the route also writes the row list (a.pairs); the instance without
// it keeps the shorter count loop (measured 1 us faster per route).
template <bool LISTS>
__global__ void __launch_bounds__(1024) k_route_finish(RouteArgs a)
{
    __shared__ int32_t pall[1024];  // [G][EL] partial totals
    __shared__ int32_t pbef[1024];  // [G][EL] partial sums over blocks before this one
    __shared__ int32_t tot[1024];   // per-expert totals
    __shared__ int32_t base[1024];  // this block's per-expert base
    __shared__ int32_t offl[1025];  // offsets
    // row list: [G][EL] partial sums of the tile's blocks before this one and
    // of the whole tile, then per expert; the tile rows of the experts
    // before, [EL] = tile rows
    __shared__ int32_t ptb[LISTS ? 1024 : 1], ptc[LISTS ? 1024 : 1];
    __shared__ int32_t tpref[LISTS ? 1025 : 1];
    const int tid = threadIdx.x;
    const int EL = a.EL;
    const int64_t nblk = a.nblk;
    const int64_t b = blockIdx.x;
    constexpr bool lists = LISTS;
    const int64_t bt0 = lists ? (b / a.pg.bpt) * a.pg.bpt : 0; // the tile's first block
    const int64_t bt1 = lists ? min(nblk, bt0 + a.pg.bpt) : 0;

    // this block's slots, fetched now so their latency overlaps the count reads
    const int64_t t0 = b * a.tokens_per_block;
    const int64_t t1 = min(a.T, t0 + a.tokens_per_block);
    const int nslots = static_cast<int>((t1 - t0) * a.k);
    const int64_t s = t0 * a.k + tid;
    const int packed = tid < nslots ? a.row_of_slot[s] : -1;
    // block 0's first wave: the OR of every block's flags, in all its lanes
    // (only that wave of that block publishes the status)
    int flags = 0;
    if (b == 0 && tid < kWave) {
        for (int64_t bb = tid; bb < nblk; bb += kWave)
            flags |= a.blockflags[bb];
#pragma unroll
        for (int o = kWave / 2; o >= 1; o >>= 1)
            flags |= __shfl_xor(flags, o);
    }
    const int G = 1024 / EL;
    const int g = tid / EL;
    const int e = tid - g * EL;
    if (g < G) {
        const int64_t per = (nblk + G - 1) / G;
        const int64_t b0 = static_cast<int64_t>(g) * per;
        const int64_t b1 = min(nblk, b0 + per);
        int all = 0, before = 0, tb = 0, tc = 0;
#pragma unroll 8
        for (int64_t bb = b0; bb < b1; ++bb) {
            const int c = a.counts[bb * EL + e];
            all += c;
            before += bb < b ? c : 0;
            if (lists) {
                tb += (bb >= bt0 && bb < b) ? c : 0;
                tc += (bb >= bt0 && bb < bt1) ? c : 0;
            }
        }
        pall[g * EL + e] = all;
        pbef[g * EL + e] = before;
        if (lists) {
            ptb[g * EL + e] = tb;
            ptc[g * EL + e] = tc;
        }
    }
    __syncthreads();
    if (tid < EL) {
        int tot_e = 0, base_e = 0, tb_e = 0, tc_e = 0;
        for (int gg = 0; gg < G; ++gg) {
            tot_e += pall[gg * EL + tid];
            base_e += pbef[gg * EL + tid];
            if (lists) {
                tb_e += ptb[gg * EL + tid];
                tc_e += ptc[gg * EL + tid];
            }
        }
        tot[tid] = tot_e;
        base[tid] = base_e;
        if (lists) {
            // read back by this thread only, then the tile's scan below
            ptb[tid] = tb_e; // per expert: this block's base within its tile
            ptc[tid] = tc_e; // per expert: the tile's count
        }
    }
    __syncthreads();
    // the tile's rows in address order: exclusive scan of its per-expert
    // counts (wave 1; publish's scan runs on wave 0, and its barrier covers both)
    if (lists && tid >= kWave && tid < 2 * kWave) {
        const int lane = tid - kWave;
        const int per = (EL + kWave - 1) / kWave;
        const int e0 = min(EL, lane * per);
        const int e1 = min(EL, e0 + per);
        int sc = 0;
        for (int x = e0; x < e1; ++x)
            sc += ptc[x];
        const int incl = wave_incl_scan(sc, lane);
        int run = incl - sc;
        for (int x = e0; x < e1; ++x) {
            tpref[x] = run;
            run += ptc[x];
        }
        if (lane == kWave - 1)
            tpref[EL] = incl;
    }
    RouteArgs pa = a;
    if (b != 0)
        pa.status = nullptr; // only block 0 publishes
    publish(pa, tot, offl, flags);

    const int64_t tau = lists ? b / a.pg.bpt : 0;                // this block's tile
    const int64_t tile_pos = lists ? (tau / kXcds) * a.pg.cap : 0; // its first position
    if (tid < nslots && packed >= 0) {
        const int ex = packed_expert(packed);
        const int row = offl[ex] + base[ex] + packed_rank(packed);
        a.row_of_slot[s] = row;
        if (lists) {
            // repeated ids write their first slot's entry again (same value)
            const int64_t q = tpref[ex] + ptb[ex] + packed_rank(packed);
            a.pairs[pair_index(tile_pos + q, tau % kXcds)] =
                make_int2(row, static_cast<int>(t0 + tid / a.k));
        }
    }
    if (lists && b == bt0) {
        // the tile's positions past its rows are empty
        const int64_t tt = min(a.pg.tile_tokens, a.T - tau * a.pg.tile_tokens);
        for (int64_t q = tpref[EL] + tid; q < tt * a.pg.kk; q += 1024)
            a.pairs[pair_index(tile_pos + q, tau % kXcds)] = make_int2(-1, -1);
    }
}

// ---------------------------------------------------------------------------
// large-T form: K2s scan (one workgroup), K3 rows (one thread per slot)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_route_scan(RouteArgs a)
{
    __shared__ int32_t part[1024]; // [G][EL] group sums, then group bases
    __shared__ int32_t tot[1024];
    __shared__ int32_t offl[1025];
    __shared__ int32_t flag_s;
    const int tid = threadIdx.x;
    const int EL = a.EL;
    const int64_t nblk = a.nblk;

    if (tid == 0)
        flag_s = 0;
    __syncthreads();
    int f = 0;
    for (int64_t b = tid; b < nblk; b += 1024)
        f |= a.blockflags[b];
    if (f)
        atomicOr(&flag_s, f);

    const int G = 1024 / EL;
    const int g = tid / EL;
    const int e = tid - g * EL;
    const int64_t per = (nblk + G - 1) / G;
    const int64_t b0 = static_cast<int64_t>(g) * per;
    const int64_t b1 = min(nblk, b0 + per);
    if (g < G) {
        int sum = 0;
#pragma unroll 8
        for (int64_t b = b0; b < b1; ++b)
            sum += a.counts[b * EL + e];
        part[g * EL + e] = sum;
    }
    __syncthreads();
    if (tid < EL) {
        int run = 0;
        for (int gg = 0; gg < G; ++gg) {
            const int c = part[gg * EL + tid];
            part[gg * EL + tid] = run;
            run += c;
        }
        tot[tid] = run;
    }
    __syncthreads();
    publish(a, tot, offl, flag_s);
    if (g < G) {
        int run = part[g * EL + e];
        for (int64_t b = b0; b < b1; ++b) {
            const int c = a.counts[b * EL + e];
            a.counts[b * EL + e] = run;
            run += c;
        }
    }
}

__global__ void __launch_bounds__(256) k_route_rows(RouteArgs a)
{
    const int64_t s = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (s >= a.T * a.k)
        return;
    const int v = a.row_of_slot[s];
    if (v < 0)
        return;
    const int64_t b = (s / a.k) / a.tokens_per_block;
    const int ex = packed_expert(v);
    a.row_of_slot[s] = a.off[ex] + a.counts[b * a.EL + ex] + packed_rank(v);
}

hipError_t launch_route(const RouteArgs &a, int threads, hipStream_t s)
{
    hipError_t err;
    if (a.nblk > 0) {
        const size_t lds = count_lds_bytes(threads * a.slots, a.EL);
        const dim3 g(static_cast<unsigned>(a.nblk)), blk(threads);
        if (a.slots == 2) {
            if (a.idx_i64)
                launch(k_route_count<int64_t, 2>, g, blk, lds, s, a);
            else
                launch(k_route_count<int32_t, 2>, g, blk, lds, s, a);
        } else {
            if (a.idx_i64)
                launch(k_route_count<int64_t, 1>, g, blk, lds, s, a);
            else
                launch(k_route_count<int32_t, 1>, g, blk, lds, s, a);
        }
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    }
    if (a.nblk == 1)
        return hipSuccess; // the counting pass finished the route (one workgroup)
    if (a.nblk > 0 && a.nblk * a.EL <= kFusedFinishMax) {
        if (a.pairs)
            launch(k_route_finish<true>, dim3(static_cast<unsigned>(a.nblk)), dim3(1024), 0, s, a);
        else
            launch(k_route_finish<false>, dim3(static_cast<unsigned>(a.nblk)), dim3(1024), 0, s, a);
        return hipGetLastError();
    }
    launch(k_route_scan, dim3(1), dim3(1024), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    const int64_t nslots = a.T * a.k;
    if (nslots > 0) {
        launch(k_route_rows, dim3(static_cast<unsigned>((nslots + 255) / 256)), dim3(256), 0, s, a);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    }
    return hipSuccess;
}

}  // namespace moe
