// rows.hip -- the row-moving kernels of the expanded layout on gfx950.
//
// "Add the deepep expert-parallel implementation", "What this adds":
//   "Expanded layout"  one row per (token, local expert) slot grouped by local
//                      expert, each with its routing weight; the combine only
//                      sums rows back to token order;
//   "Eager vs captured" sync-free rows are sized for the worst case and rows
//                      past the received total are zero and belong to a
//                      sentinel expert;
//   "Custom ops"       the combine's backward is a cached dispatch;
//   "Training"         gradients reach the routing weights.
//
// All of it is HBM-bound data movement (no contraction, so no MFMA).  Design:
//   * token-major: one wave per token; the wave reads the token's row once
//     into VGPRs with 16-byte loads (64 lanes x 16 B = 1 KiB per instruction)
//     and writes it to each of its local rows, so x is read from HBM once no
//     matter how many local experts the token picked;
//   * the token's k slots are handled lane-parallel (lane j = slot j): row
//     lookup, repeated-id detection and weight merging are a few ballots and
//     lane reads, no LDS;
//   * pad rows (one workgroup per expert) and the sentinel tail [total, R)
//     (a grid-stride flat fill, since those rows are contiguous) are zeroed by
//     extra workgroups of the same launch, so the fill overlaps the gather;
//   * combine is token-major too: the wave gathers its token's rows (the next
//     row's loads are issued before the current one is added) and adds them in
//     fp32 in ascending slot order, then writes bf16 (nearest-even) or fp32.
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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

// The token's slots, one per lane: its row (or -1), whether the row is valid
// (inside [0, R)), whether the lane is the first slot naming that row, and the
// lane of that first slot.
struct Slots {
    int row;
    bool valid;
    bool prim;
    int first;
    uint64_t prim_mask;
    uint64_t dup_mask;
};

__device__ __forceinline__ Slots load_slots(const int32_t *__restrict__ row_of_slot, int64_t t,
                                            int k, int64_t R, int lane)
{
    Slots s;
    s.row = lane < k ? row_of_slot[t * k + lane] : -1;
    s.valid = lane < k && s.row >= 0 && s.row < R;
    s.first = lane;
    for (int q = 0; q < k; ++q) {
        const int rq = __builtin_amdgcn_readlane(s.row, q);
        if (q < lane && s.valid && rq == s.row && s.first == lane)
            s.first = q;
    }
    s.prim = s.valid && s.first == lane;
    s.prim_mask = __ballot(s.prim);
    s.dup_mask = __ballot(s.valid && !s.prim);
    return s;
}

// ---------------------------------------------------------------------------
// dispatch / combine backward
// ---------------------------------------------------------------------------
template <int NCH, bool DOT>
__device__ __forceinline__ void move_token(const RowArgs &a, int64_t bid)
{
    __shared__ double dotacc[kRowWaves][kMaxK];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = bid * kRowWaves + wave;
    if (t >= a.T)
        return;
    const int k = a.k;
    const Slots sl = load_slots(a.row_of_slot, t, k, a.R, lane);

    // metadata of the token's rows (dispatch only)
    if (a.row_w || a.row_token) {
        float W = 0.f;
        if (a.topk_w) {
            const float myw = lane < k ? a.topk_w[t * k + lane] : 0.f;
            W = myw;
            if (sl.dup_mask) {
                // repeated ids: the first slot's weight plus the later ones, in slot order
                for (int q = 0; q < k; ++q) {
                    const int rq = __builtin_amdgcn_readlane(sl.row, q);
                    const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myw), q));
                    if (sl.prim && q > lane && rq == sl.row)
                        W = W + wq;
                }
            }
        }
        if (sl.prim) {
            if (a.row_token)
                a.row_token[sl.row] = static_cast<int32_t>(t);
            if (a.row_w)
                a.row_w[sl.row] = W;
        }
    }

    if (DOT) {
        if (lane < k)
            dotacc[wave][lane] = 0.0;
    }
    if (sl.prim_mask) {
        const int nch = a.H >> 3; // 16-byte chunks per row
        const u32x4 *__restrict__ src = reinterpret_cast<const u32x4 *>(a.src + t * a.H);
        for (int c0 = 0; c0 < nch; c0 += NCH * kWave) {
            u32x4 v[NCH];
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = c0 + i * kWave + lane;
                if (c < nch)
                    v[i] = src[c];
            }
            uint64_t m = sl.prim_mask;
            while (m) {
                const int j = __builtin_ctzll(m);
                m &= m - 1;
                const int64_t r = __builtin_amdgcn_readlane(sl.row, j);
                u32x4 *__restrict__ dst = reinterpret_cast<u32x4 *>(a.rows + r * a.H);
                if (DOT) {
                    const u32x4 *__restrict__ fr = reinterpret_cast<const u32x4 *>(a.F + r * a.H);
                    u32x4 fv[NCH];
#pragma unroll
                    for (int i = 0; i < NCH; ++i) {
                        const int c = c0 + i * kWave + lane;
                        if (c < nch)
                            fv[i] = fr[c];
                    }
#pragma unroll
                    for (int i = 0; i < NCH; ++i) {
                        const int c = c0 + i * kWave + lane;
                        if (c < nch)
                            dst[c] = v[i];
                    }
                    double acc = 0.0;
#pragma unroll
                    for (int i = 0; i < NCH; ++i) {
                        const int c = c0 + i * kWave + lane;
                        if (c < nch) {
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                acc = fma(static_cast<double>(bf16_lo(v[i][q])),
                                          static_cast<double>(bf16_lo(fv[i][q])), acc);
                                acc = fma(static_cast<double>(bf16_hi(v[i][q])),
                                          static_cast<double>(bf16_hi(fv[i][q])), acc);
                            }
                        }
                    }
#pragma unroll
                    for (int o = kWave / 2; o >= 1; o >>= 1)
                        acc += __shfl_xor(acc, o);
                    if (lane == 0)
                        dotacc[wave][j] += acc;
                } else {
#pragma unroll
                    for (int i = 0; i < NCH; ++i) {
                        const int c = c0 + i * kWave + lane;
                        if (c < nch)
                            dst[c] = v[i];
                    }
                }
            }
        }
    }
    if (DOT && a.dw) {
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        if (lane < k)
            a.dw[t * k + lane] = sl.valid ? static_cast<float>(dotacc[wave][sl.first]) : 0.f;
    }
}

// Pad rows of one expert's group: zero data, token -1, weight 0; every row of
// the group gets row_expert = e.
__device__ __forceinline__ void fill_expert(const RowArgs &a, int e)
{
    // clamped into [0, R] so that no handle content can move a write out of bounds
    const int64_t lo = max<int64_t>(0, min<int64_t>(a.off[e], a.R));
    const int64_t hi = max<int64_t>(lo, min<int64_t>(a.off[e + 1], a.R));
    const int64_t pad0 = max<int64_t>(lo, min<int64_t>(lo + a.tpe[e], hi));
    const int tid = threadIdx.x;
    if (a.row_expert)
        for (int64_t r = lo + tid; r < hi; r += kRowThreads)
            a.row_expert[r] = e;
    for (int64_t r = pad0 + tid; r < hi; r += kRowThreads) {
        if (a.row_token)
            a.row_token[r] = -1;
        if (a.row_w)
            a.row_w[r] = 0.f;
    }
    const int64_t nch = a.H >> 3;
    u32x4 *__restrict__ dst = reinterpret_cast<u32x4 *>(a.rows);
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t q = pad0 * nch + tid; q < hi * nch; q += kRowThreads)
        dst[q] = z;
}

// Rows [total, R): zero data, token -1, expert EL (the sentinel), weight 0.
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
    const int64_t nch = a.H >> 3;
    u32x4 *__restrict__ dst = reinterpret_cast<u32x4 *>(a.rows);
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int64_t q1 = r1 * nch;
    for (int64_t q = r0 * nch + gtid; q < q1; q += gstride)
        dst[q] = z;
}

template <int NCH, bool DOT>
__global__ void __launch_bounds__(kRowThreads) k_move_rows(RowArgs a)
{
    const int64_t bid = blockIdx.x;
    if (bid < a.ntok_blocks)
        move_token<NCH, DOT>(a, bid);
    else if (bid < a.ntok_blocks + a.nexp_blocks)
        fill_expert(a, static_cast<int>(bid - a.ntok_blocks));
    else
        fill_sentinel(a, bid - a.ntok_blocks - a.nexp_blocks);
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------
template <int NCH>
__device__ __forceinline__ void load_row(u32x4 (&v)[NCH], const uint16_t *base, int64_t r, int H,
                                         int c0, int nch, int lane)
{
    const u32x4 *__restrict__ p = reinterpret_cast<const u32x4 *>(base + r * H);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = c0 + i * kWave + lane;
        if (c < nch)
            v[i] = p[c];
    }
}

template <int NCH, bool OUT_F32>
__global__ void __launch_bounds__(kRowThreads) k_combine(CombineArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kRowWaves + wave;
    if (t == 0 && lane == 0 && a.eager && a.status[0] != a.R)
        atomicOr(&a.status[1], 4);
    if (t >= a.T)
        return;
    const Slots sl = load_slots(a.row_of_slot, t, a.k, a.R, lane);
    const int nch = a.H >> 3;
    for (int c0 = 0; c0 < nch; c0 += NCH * kWave) {
        float acc[NCH][8];
        uint64_t m = sl.prim_mask;
        if (!m) {
#pragma unroll
            for (int i = 0; i < NCH; ++i)
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[i][q] = 0.f;
        } else {
            u32x4 cur[NCH];
            int j = __builtin_ctzll(m);
            m &= m - 1;
            load_row<NCH>(cur, a.Y, __builtin_amdgcn_readlane(sl.row, j), a.H, c0, nch, lane);
            bool first = true;
            while (true) {
                const bool more = m != 0;
                u32x4 nxt[NCH];
                if (more) {
                    j = __builtin_ctzll(m);
                    m &= m - 1;
                    load_row<NCH>(nxt, a.Y, __builtin_amdgcn_readlane(sl.row, j), a.H, c0, nch, lane);
                }
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float lo = bf16_lo(cur[i][q]);
                        const float hi = bf16_hi(cur[i][q]);
                        acc[i][2 * q] = first ? lo : acc[i][2 * q] + lo;
                        acc[i][2 * q + 1] = first ? hi : acc[i][2 * q + 1] + hi;
                    }
                }
                first = false;
                if (!more)
                    break;
#pragma unroll
                for (int i = 0; i < NCH; ++i)
                    cur[i] = nxt[i];
            }
        }
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
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
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int chunks_per_lane(int H)
{
    const int nch = H >> 3;
    const int need = (nch + kWave - 1) / kWave;
    int n = 1;
    while (n < need && n < 16)
        n <<= 1;
    return n;
}

template <bool DOT>
static void launch_move(int nch, dim3 g, const RowArgs &a, hipStream_t s)
{
    switch (nch) {
    case 1: k_move_rows<1, DOT><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    case 2: k_move_rows<2, DOT><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    case 4: k_move_rows<4, DOT><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    case 8: k_move_rows<8, DOT><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    default: k_move_rows<16, DOT><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    }
}

hipError_t launch_move_rows(const RowArgs &a, hipStream_t s)
{
    const int64_t nb = a.ntok_blocks + a.nexp_blocks + a.nsent_blocks;
    if (nb == 0)
        return hipSuccess;
    const dim3 g(static_cast<unsigned>(nb));
    const int nch = chunks_per_lane(a.H);
    if (a.dw)
        launch_move<true>(nch, g, a, s);
    else
        launch_move<false>(nch, g, a, s);
    return hipGetLastError();
}

template <bool F32>
static void launch_comb(int nch, dim3 g, const CombineArgs &a, hipStream_t s)
{
    switch (nch) {
    case 1: k_combine<1, F32><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    case 2: k_combine<2, F32><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    case 4: k_combine<4, F32><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    case 8: k_combine<8, F32><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    default: k_combine<16, F32><<<g, dim3(kRowThreads), 0, s>>>(a); break;
    }
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t s)
{
    const int64_t nb = (a.T + kRowWaves - 1) / kRowWaves;
    if (nb == 0)
        return hipSuccess;
    const dim3 g(static_cast<unsigned>(nb));
    const int nch = chunks_per_lane(a.H);
    if (a.out_f32)
        launch_comb<true>(nch, g, a, s);
    else
        launch_comb<false>(nch, g, a, s);
    return hipGetLastError();
}

}  // namespace moe
