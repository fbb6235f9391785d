// ceiling.hip -- reference kernels that bound what MI355X's memory gives for
// the access patterns of libmoe_mi355x's row kernels (declared in
// include/moe_ceiling.h).  They are not the method's path (the gather's sum
// truncates to bf16); a benchmark times them beside the library's kernels on
// the same buffers.
//
//   fill     one-shot zero fill in address order: wave g writes piece g
//            (piece_kib KiB) with non-temporal 16-byte stores and exits, so
//            the writes in flight form one window sliding through the buffer
//            (the pattern of the sync-free tail fill).
//   copy     the same walk reading piece g of src and writing it to dst
//            (as many bytes in as out, both in address order).
//   scatter  write-only token-major scatter into the expanded layout: one
//            workgroup of four waves per token, each wave writing zero
//            segments of seg_kib KiB to every row the token's slots name,
//            exactly the destinations (and the order of destinations in
//            flight) of the dispatch's row stores, with no source reads.
//   gather   the combine's reads: one wave per (token, segment), the
//            segments of the token's named rows loaded (non-temporal) in
//            batches of four before any is added, summed in fp32; with an output
//            the summed segment is stored (truncated to bf16), without one
//            nothing is (a read-only gather).
//   xcd_map  the accelerator complex die (XCD) each workgroup of a grid ran
//            on, read from the wave's XCC_ID hardware register: the row
//            kernels number their workgroups on the assumption that
//            workgroup j runs on XCD j mod 8.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int64_t kMaxBlocks = 0xFFFFFFFFll / (kWave * kWaves);

template <int PK>
__global__ void __launch_bounds__(kWave *kWaves) k_fill(u32x4 *__restrict__ dst, int64_t nch)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x / kWave);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < PK; ++i) {
        const int64_t c = (g * PK + i) * kWave + lane;
        if (c < nch)
            __builtin_nontemporal_store(z, dst + c);
    }
}

template <int PK>
__global__ void __launch_bounds__(kWave *kWaves) k_copy(const u32x4 *__restrict__ src,
                                                        u32x4 *__restrict__ dst, int64_t nch)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x / kWave);
    u32x4 v[PK];
#pragma unroll
    for (int i = 0; i < PK; ++i) {
        const int64_t c = (g * PK + i) * kWave + lane;
        if (c < nch)
            v[i] = src[c];
    }
#pragma unroll
    for (int i = 0; i < PK; ++i) {
        const int64_t c = (g * PK + i) * kWave + lane;
        if (c < nch)
            __builtin_nontemporal_store(v[i], dst + c);
    }
}

// One workgroup per token; the row's segments are dealt over the four waves.
template <int SEG>
__global__ void __launch_bounds__(kWave *kWaves) k_scatter(const int32_t *__restrict__ row_of_slot,
                                                           int64_t T, int k, int64_t R, int nch,
                                                           u32x4 *__restrict__ rows)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t t = blockIdx.x;
    if (t >= T)
        return;
    const int myrow = lane < k ? row_of_slot[t * k + lane] : -1;
    const u32x4 z = {0u, 0u, 0u, 0u};
    constexpr int SPAN = SEG * kWave;
    const int nseg = (nch + SPAN - 1) / SPAN;
    for (int sg = wave; sg < nseg; sg += kWaves) {
        for (int j = 0; j < k; ++j) {
            const int r = __builtin_amdgcn_readlane(myrow, j);
            if (r < 0 || r >= R)
                continue;
            u32x4 *dst = rows + static_cast<int64_t>(r) * nch;
#pragma unroll
            for (int i = 0; i < SEG; ++i) {
                const int c = sg * SPAN + i * kWave + lane;
                if (c < nch)
                    __builtin_nontemporal_store(z, dst + c);
            }
        }
    }
}

// One wave per (token, segment of SEG chunks per lane).  FULL: every chunk
// of the segment exists (no per-chunk test).  out NULL: read only; the sink
// word is written only when a sum has the all-ones NaN pattern, which finite
// rows never give (it keeps the loads).
template <int SEG, bool FULL>
__global__ void __launch_bounds__(kWave *kWaves) k_gather(const int32_t *__restrict__ row_of_slot,
                                                          int64_t T, int k, int64_t R, int nch,
                                                          const u32x4 *__restrict__ Y,
                                                          u32x4 *__restrict__ out,
                                                          uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int SPAN = SEG * kWave;
    const int nseg = (nch + SPAN - 1) / SPAN;
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x / kWave);
    const int64_t t = gw / nseg;
    if (t >= T)
        return;
    const int c0 = static_cast<int>(gw - t * nseg) * SPAN;
    const int myrow = lane < k ? row_of_slot[t * k + lane] : -1;
    float acc[SEG][8];
#pragma unroll
    for (int i = 0; i < SEG; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[i][q] = 0.f;
    // the named rows only, in slot order, four at a time
    uint64_t m = __ballot(myrow >= 0 && myrow < R);
    while (m) {
        int r[4];
        int n = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            r[u] = -1;
            if (m) {
                r[u] = __builtin_amdgcn_readlane(myrow, __builtin_ctzll(m));
                m &= m - 1;
                n = u + 1;
            }
        }
        u32x4 f[4][SEG];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 *src = Y + static_cast<int64_t>(u < n ? r[u] : 0) * nch;
#pragma unroll
            for (int i = 0; i < SEG; ++i) {
                const int c = c0 + i * kWave + lane;
                f[u][i] = (u < n && (FULL || c < nch)) ? __builtin_nontemporal_load(src + c)
                                                       : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < SEG; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[i][2 * q] += __uint_as_float(f[u][i][q] << 16);
                    acc[i][2 * q + 1] += __uint_as_float(f[u][i][q] & 0xFFFF0000u);
                }
    }
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
        const int c = c0 + i * kWave + lane;
        if (!FULL && c >= nch)
            continue;
        if (out) {
            u32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[q] = (__float_as_uint(acc[i][2 * q]) >> 16) |
                       (__float_as_uint(acc[i][2 * q + 1]) & 0xFFFF0000u);
            out[t * nch + c] = v;
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (__float_as_uint(acc[i][q]) == 0xFFFFFFFFu)
                    *sink = 1u;
        }
    }
}

template <int SEG>
void launch_gather(bool full, dim3 g, hipStream_t s, const int32_t *ros, int64_t T, int k, int64_t R,
                   int nch, const u32x4 *y, u32x4 *o, uint32_t *sink)
{
    if (full)
        hipLaunchKernelGGL((k_gather<SEG, true>), g, dim3(kWave * kWaves), 0, s, ros, T, k, R, nch, y, o, sink);
    else
        hipLaunchKernelGGL((k_gather<SEG, false>), g, dim3(kWave * kWaves), 0, s, ros, T, k, R, nch, y, o, sink);
}

// XCC_ID hardware register (id 20), bits [3:0]: s_getreg's immediate is
// (size - 1) << 11 | offset << 6 | id.
constexpr int kXccIdReg = (3 << 11) | (0 << 6) | 20;

__global__ void __launch_bounds__(kWave *kWaves) k_xcd_map(int32_t *__restrict__ out)
{
    if (threadIdx.x == 0)
        out[blockIdx.x] = __builtin_amdgcn_s_getreg(kXccIdReg);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int pieces_blocks(size_t bytes, int pk, int64_t *nch, unsigned *blocks)
{
    *nch = static_cast<int64_t>(bytes / 16);
    const int64_t waves = (*nch + pk * kWave - 1) / (pk * kWave);
    const int64_t nb = (waves + kWaves - 1) / kWaves;
    if (nb > kMaxBlocks)
        return MOE_CEILING_ERR_ARG;
    *blocks = static_cast<unsigned>(nb);
    return MOE_CEILING_OK;
}

int launched()
{
    return hipGetLastError() == hipSuccess ? MOE_CEILING_OK : MOE_CEILING_ERR_HIP;
}

}  // namespace

extern "C" {

int moe_ceiling_fill(void *dst, size_t bytes, int piece_kib, void *stream)
{
    if (!dst || !aligned16(dst) || bytes % 16 != 0 ||
        (piece_kib != 1 && piece_kib != 2 && piece_kib != 4))
        return MOE_CEILING_ERR_ARG;
    int64_t nch;
    unsigned nb;
    if (pieces_blocks(bytes, piece_kib, &nch, &nb) != MOE_CEILING_OK)
        return MOE_CEILING_ERR_ARG;
    if (nb == 0)
        return MOE_CEILING_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    u32x4 *d = static_cast<u32x4 *>(dst);
    switch (piece_kib) {
    case 1: hipLaunchKernelGGL(k_fill<1>, dim3(nb), dim3(kWave * kWaves), 0, s, d, nch); break;
    case 2: hipLaunchKernelGGL(k_fill<2>, dim3(nb), dim3(kWave * kWaves), 0, s, d, nch); break;
    default: hipLaunchKernelGGL(k_fill<4>, dim3(nb), dim3(kWave * kWaves), 0, s, d, nch); break;
    }
    return launched();
}

int moe_ceiling_copy(const void *src, void *dst, size_t bytes, int piece_kib, void *stream)
{
    if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes % 16 != 0 ||
        (piece_kib != 1 && piece_kib != 2 && piece_kib != 4))
        return MOE_CEILING_ERR_ARG;
    int64_t nch;
    unsigned nb;
    if (pieces_blocks(bytes, piece_kib, &nch, &nb) != MOE_CEILING_OK)
        return MOE_CEILING_ERR_ARG;
    if (nb == 0)
        return MOE_CEILING_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *a = static_cast<const u32x4 *>(src);
    u32x4 *d = static_cast<u32x4 *>(dst);
    switch (piece_kib) {
    case 1: hipLaunchKernelGGL(k_copy<1>, dim3(nb), dim3(kWave * kWaves), 0, s, a, d, nch); break;
    case 2: hipLaunchKernelGGL(k_copy<2>, dim3(nb), dim3(kWave * kWaves), 0, s, a, d, nch); break;
    default: hipLaunchKernelGGL(k_copy<4>, dim3(nb), dim3(kWave * kWaves), 0, s, a, d, nch); break;
    }
    return launched();
}

int moe_ceiling_scatter(const int32_t *row_of_slot, int64_t T, int32_t k, int64_t R, int32_t H,
                        void *rows, int seg_kib, void *stream)
{
    if (T < 0 || k < 1 || k > kWave || R < 0 || H <= 0 || H % 256 != 0 || T > kMaxBlocks ||
        (seg_kib != 1 && seg_kib != 2 && seg_kib != 4))
        return MOE_CEILING_ERR_ARG;
    if (T == 0)
        return MOE_CEILING_OK;
    if (!row_of_slot || !rows || !aligned16(rows))
        return MOE_CEILING_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int nch = H / 8;
    u32x4 *d = static_cast<u32x4 *>(rows);
    const dim3 g(static_cast<unsigned>(T)), b(kWave * kWaves);
    switch (seg_kib) {
    case 1: hipLaunchKernelGGL(k_scatter<1>, g, b, 0, s, row_of_slot, T, k, R, nch, d); break;
    case 2: hipLaunchKernelGGL(k_scatter<2>, g, b, 0, s, row_of_slot, T, k, R, nch, d); break;
    default: hipLaunchKernelGGL(k_scatter<4>, g, b, 0, s, row_of_slot, T, k, R, nch, d); break;
    }
    return launched();
}

int moe_ceiling_gather(const int32_t *row_of_slot, int64_t T, int32_t k, int64_t R, int32_t H,
                       const void *Y, void *out, uint32_t *sink, int seg_kib, void *stream)
{
    if (T < 0 || k < 1 || k > kWave || R < 0 || H <= 0 || H % 256 != 0 ||
        (seg_kib != 1 && seg_kib != 2 && seg_kib != 4))
        return MOE_CEILING_ERR_ARG;
    if (T == 0)
        return MOE_CEILING_OK;
    if (!row_of_slot || (R > 0 && (!Y || !aligned16(Y))) || (out && !aligned16(out)) ||
        (!out && !sink))
        return MOE_CEILING_ERR_ARG;
    const int nch = H / 8;
    const int span = seg_kib * kWave;
    const int64_t waves = T * ((nch + span - 1) / span);
    const int64_t nb = (waves + kWaves - 1) / kWaves;
    if (nb > kMaxBlocks)
        return MOE_CEILING_ERR_ARG;
    const bool full = nch % span == 0;
    const dim3 g(static_cast<unsigned>(nb));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *y = static_cast<const u32x4 *>(Y);
    u32x4 *o = static_cast<u32x4 *>(out);
    switch (seg_kib) {
    case 1: launch_gather<1>(full, g, s, row_of_slot, T, k, R, nch, y, o, sink); break;
    case 2: launch_gather<2>(full, g, s, row_of_slot, T, k, R, nch, y, o, sink); break;
    default: launch_gather<4>(full, g, s, row_of_slot, T, k, R, nch, y, o, sink); break;
    }
    return launched();
}

int moe_ceiling_xcd_map(int32_t *out, int32_t nblocks, void *stream)
{
    if (nblocks < 0 || (nblocks > 0 && !out))
        return MOE_CEILING_ERR_ARG;
    if (nblocks == 0)
        return MOE_CEILING_OK;
    hipLaunchKernelGGL(k_xcd_map, dim3(static_cast<unsigned>(nblocks)), dim3(kWave * kWaves), 0,
                       static_cast<hipStream_t>(stream), out);
    return launched();
}

}  // extern "C"
