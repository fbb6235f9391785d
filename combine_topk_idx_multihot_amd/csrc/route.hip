// route.hip -- routing preprocessing on gfx950: top-k ids -> multihot map,
// tokens_per_expert, padded offsets and the row of every slot.
//
// "feat: add hybridep", Changelog: the HybridEP path converts top-k indices to
// multihot routing metadata; its dispatch returns tokens_per_expert and pads
// each expert's rows to pad_multiple.  "Add the deepep expert-parallel
// implementation", "What this adds" / "Expanded layout": one row per (token,
// local expert) slot, grouped by local expert (here in ascending token order).
//
// Three launches, no atomics on the ordering path, so the layout is the same
// on every run:
//   K1 route_count  one thread per slot, one workgroup per block of whole
//                   tokens.  Writes the multihot map (and probs), detects bad
//                   and repeated ids, and ranks each primary local slot among
//                   the block's slots of the same expert with wave ballots
//                   (lanes are in token order, so a ballot prefix popcount is
//                   a stable rank).  Per-block expert counts go to workspace.
//   K2 route_scan   one workgroup: per-expert exclusive scan over blocks,
//                   tokens_per_expert, padded sizes and their exclusive scan
//                   over experts (= padded offsets), device total, flags.
//   K3 route_rows   one thread per slot: row = offset[e] + block base[e] +
//                   in-block rank.
#include "moe_internal.h"

namespace moe {

RouteGeom route_geom(int64_t T, int k, int EL)
{
    RouteGeom g;
    g.threads = EL > 512 ? 512 : 1024;
    g.tokens_per_block = g.threads / k;
    g.nblk = T > 0 ? (T + g.tokens_per_block - 1) / g.tokens_per_block : 0;
    return g;
}

template <typename IT>
__device__ __forceinline__ int64_t id_at(const IT *__restrict__ p, int64_t i)
{
    return static_cast<int64_t>(p[i]);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// K1
// ---------------------------------------------------------------------------
template <typename IT>
__global__ void __launch_bounds__(1024) k_route_count(RouteArgs a)
{
    extern __shared__ int32_t lds[];
    const int nthreads = blockDim.x;
    const int nwaves = nthreads / kWave;
    const int EL = a.EL;
    int32_t *cnt = lds;                    // [nwaves][EL] per-wave counts, then wave bases
    int32_t *lrank = cnt + nwaves * EL;    // [nthreads] in-block rank of each slot
    int32_t *bflag = lrank + nthreads;     // block flag word

    const IT *__restrict__ idx = static_cast<const IT *>(a.idx);
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t b = blockIdx.x;
    const int k = a.k;
    const int64_t t0 = b * a.tokens_per_block;
    const int64_t t1 = min(a.T, t0 + a.tokens_per_block);

    for (int i = tid; i < nwaves * EL; i += nthreads)
        cnt[i] = 0;
    if (tid == 0)
        *bflag = 0;

    // Phase A: this block's rows of the multihot map and of the probs.
    if (a.map) {
        uint8_t *base = a.map + t0 * a.E;
        if ((a.E & 15) == 0 && (reinterpret_cast<uintptr_t>(a.map) & 15) == 0) {
            const int cpt = a.E >> 4; // 16-byte chunks per token row
            const int64_t nch = (t1 - t0) * cpt;
            for (int64_t q = tid; q < nch; q += nthreads) {
                const int64_t t = t0 + q / cpt;
                const int eb = static_cast<int>(q % cpt) * 16;
                uint64_t lo = 0, hi = 0;
                for (int j = 0; j < k; ++j) {
                    const int64_t d = id_at(idx, t * k + j) - eb;
                    if (d >= 0 && d < 16) {
                        const uint64_t bit = 1ull << ((d & 7) * 8);
                        if (d < 8)
                            lo |= bit;
                        else
                            hi |= bit;
                    }
                }
                u32x4 v = {static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                           static_cast<uint32_t>(hi), static_cast<uint32_t>(hi >> 32)};
                *reinterpret_cast<u32x4 *>(base + q * 16) = v;
            }
        } else {
            const int64_t nb = (t1 - t0) * a.E;
            for (int64_t q = tid; q < nb; q += nthreads) {
                const int64_t t = t0 + q / a.E;
                const int64_t e = q % a.E;
                uint8_t v = 0;
                for (int j = 0; j < k; ++j)
                    v |= (id_at(idx, t * k + j) == e) ? 1 : 0;
                base[q] = v;
            }
        }
    }
    if (a.probs) {
        // routed weight at each routed expert; a repeated id adds its weight
        // to the first one, in slot order
        float *base = a.probs + t0 * a.E;
        const int width =
            ((a.E & 3) == 0 && (reinterpret_cast<uintptr_t>(a.probs) & 15) == 0) ? 4 : 1;
        const int cpt = a.E / width;
        const int64_t nch = (t1 - t0) * cpt;
        for (int64_t q = tid; q < nch; q += nthreads) {
            const int64_t t = t0 + q / cpt;
            const int eb = static_cast<int>(q % cpt) * width;
            float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
            unsigned seen = 0;
            for (int j = 0; j < k; ++j) {
                const int64_t d = id_at(idx, t * k + j) - eb;
                if (d >= 0 && d < width) {
                    const float wj = a.w[t * k + j];
                    const bool again = (seen >> d) & 1u;
                    if (d == 0) v0 = again ? v0 + wj : wj;
                    if (d == 1) v1 = again ? v1 + wj : wj;
                    if (d == 2) v2 = again ? v2 + wj : wj;
                    if (d == 3) v3 = again ? v3 + wj : wj;
                    seen |= 1u << d;
                }
            }
            if (width == 4) {
                f32x4 v = {v0, v1, v2, v3};
                *reinterpret_cast<f32x4 *>(base + q * 4) = v;
            } else {
                base[q] = v0;
            }
        }
    }
    __syncthreads();

    // Phase B: one thread per slot of the block's tokens.
    const int64_t nslots = (t1 - t0) * k;
    const int64_t s = t0 * k + tid;
    int ep = -1;          // local expert of a primary local slot
    int prim_back = 0;    // repeated id: distance back to its first slot
    bool bad = false, dup = false, dup_local = false;
    if (tid < nslots) {
        const int64_t t = s / k;
        const int j = static_cast<int>(s - t * k);
        const int64_t e = id_at(idx, s);
        bad = (e < -1) || (e >= a.E);
        if (e >= 0 && e < a.E) {
            for (int q = 0; q < j; ++q) {
                if (id_at(idx, t * k + q) == e) {
                    dup = true;
                    prim_back = j - q;
                    break;
                }
            }
            if (e >= a.lb && e < static_cast<int64_t>(a.lb) + EL) {
                if (dup)
                    dup_local = true;
                else
                    ep = static_cast<int>(e - a.lb);
            }
        }
    }
    const uint64_t mbad = __ballot(bad);
    const uint64_t mdup = __ballot(dup);
    if (lane == 0 && (mbad | mdup))
        atomicOr(bflag, (mbad ? 1 : 0) | (mdup ? 2 : 0));

    // Rank of each slot among the wave's slots of the same expert.  Lanes are
    // in token order and a token holds at most one primary slot per expert,
    // so the ballot prefix count is the ascending-token rank.
    int my_rank = 0;
    uint64_t rem = __ballot(ep >= 0);
    while (rem) {
        const int lead = __builtin_ctzll(rem);
        const int e0 = __builtin_amdgcn_readlane(ep, lead);
        const uint64_t m = __ballot(ep == e0);
        if (ep == e0)
            my_rank = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0)
            cnt[wave * EL + e0] = __popcll(m);
        rem &= ~m;
    }
    __syncthreads();

    // Exclusive prefix over waves per expert; block totals to the workspace.
    for (int e = tid; e < EL; e += nthreads) {
        int run = 0;
        for (int w = 0; w < nwaves; ++w) {
            const int c = cnt[w * EL + e];
            cnt[w * EL + e] = run;
            run += c;
        }
        a.counts[b * EL + e] = run;
    }
    if (tid == 0)
        a.blockflags[b] = *bflag;
    __syncthreads();
    if (ep >= 0)
        lrank[tid] = cnt[wave * EL + ep] + my_rank;
    __syncthreads();
    if (tid < nslots) {
        int v = -1;
        if (ep >= 0)
            v = lrank[tid];
        else if (dup_local)
            v = lrank[tid - prim_back]; // a repeated id shares its first slot's row
        a.row_of_slot[s] = v;
    }
}

// ---------------------------------------------------------------------------
// K2
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

// Inclusive scan over a 1024-thread workgroup.  tmp: 16 ints of LDS.
__device__ int block_incl_scan(int v, int *tmp)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    v = wave_incl_scan(v, lane);
    if (lane == kWave - 1)
        tmp[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int w = lane < 16 ? tmp[lane] : 0;
        w = wave_incl_scan(w, lane);
        if (lane < 16)
            tmp[lane] = w;
    }
    __syncthreads();
    if (wave > 0)
        v += tmp[wave - 1];
    __syncthreads();
    return v;
}

__global__ void __launch_bounds__(1024) k_route_scan(RouteArgs a)
{
    __shared__ int32_t part[1024]; // [G][EL] group sums, then group bases
    __shared__ int32_t tot[1024];  // per-expert totals
    __shared__ int32_t tmp[16];
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

    // Blocks are split into G contiguous ranges; thread (g, e) sums range g.
    const int G = EL >= 1024 ? 1 : 1024 / EL;
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
        a.tpe[tid] = run;
    }
    __syncthreads();
    if (g < G) {
        int run = part[g * EL + e];
        for (int64_t b = b0; b < b1; ++b) {
            const int c = a.counts[b * EL + e];
            a.counts[b * EL + e] = run;
            run += c;
        }
    }
    const int cnt = tid < EL ? tot[tid] : 0;
    const int padded = tid < EL ? ((cnt + a.P - 1) / a.P) * a.P : 0;
    const int incl = block_incl_scan(padded, tmp);
    const int data_incl = block_incl_scan(cnt, tmp);
    if (tid < EL)
        a.off[tid] = incl - padded;
    if (tid == EL - 1) {
        a.off[EL] = incl;
        a.status[0] = incl;
        a.status[2] = data_incl;
        a.status[3] = 0;
    }
    if (tid == 0)
        a.status[1] = flag_s;
}

// ---------------------------------------------------------------------------
// K3
// ---------------------------------------------------------------------------
template <typename IT>
__global__ void __launch_bounds__(256) k_route_rows(RouteArgs a)
{
    const int64_t s = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (s >= a.T * a.k)
        return;
    const int lr = a.row_of_slot[s];
    if (lr < 0)
        return;
    const IT *__restrict__ idx = static_cast<const IT *>(a.idx);
    const int64_t t = s / a.k;
    const int64_t b = t / a.tokens_per_block;
    const int e = static_cast<int>(id_at(idx, s) - a.lb);
    a.row_of_slot[s] = a.off[e] + a.counts[b * a.EL + e] + lr;
}

hipError_t launch_route(const RouteArgs &a, int threads, hipStream_t s)
{
    hipError_t err;
    if (a.nblk > 0) {
        const size_t lds = (static_cast<size_t>(threads / kWave) * a.EL + threads + 1) * sizeof(int32_t);
        if (a.idx_i64)
            k_route_count<int64_t><<<dim3(static_cast<unsigned>(a.nblk)), dim3(threads), lds, s>>>(a);
        else
            k_route_count<int32_t><<<dim3(static_cast<unsigned>(a.nblk)), dim3(threads), lds, s>>>(a);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    }
    k_route_scan<<<dim3(1), dim3(1024), 0, s>>>(a);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    const int64_t nslots = a.T * a.k;
    if (nslots > 0) {
        const unsigned grid = static_cast<unsigned>((nslots + 255) / 256);
        if (a.idx_i64)
            k_route_rows<int64_t><<<dim3(grid), dim3(256), 0, s>>>(a);
        else
            k_route_rows<int32_t><<<dim3(grid), dim3(256), 0, s>>>(a);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    }
    return hipSuccess;
}

}  // namespace moe
