/*
 * abi_check.c -- the library called from plain C, with no Python and no torch:
 * HIP runtime allocations, the header include/moe_mi355x.h, and the shared
 * library.  Built by the package build with gcc; run by tests/test_gpu_c_abi.py.
 *
 * One top-1 layer (T tokens, E experts, every expert local, pad_multiple 4) in
 * eager mode and one in sync-free mode.  With one slot per token, dispatch
 * then combine is the identity on every token with a valid id, and zero on the
 * others; the checks below are that identity, the counts against a host
 * histogram, the padded offsets, the row of every slot, the sync-free tail,
 * the dispatch backward, the error path for a bad hidden size, the
 * dispatch's device time from moe_time_next_call, and (eager) the same route
 * and dispatch as one moe_route_dispatch call into worst-case buffers.
 * Prints "abi ok" and exits 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_mi355x.h"

#define CHECK(c)                                                                      \
    do {                                                                              \
        if (!(c)) {                                                                   \
            fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #c,        \
                    moe_last_error());                                                \
            exit(1);                                                                  \
        }                                                                             \
    } while (0)
#define HIPCHECK(x) CHECK((x) == hipSuccess)

enum { T = 1000, E = 24, H = 512, P = 4 };

static uint32_t lcg(uint32_t *s)
{
    *s = *s * 1664525u + 1013904223u;
    return *s >> 8;
}

static void *dev(size_t bytes)
{
    void *p = NULL;
    HIPCHECK(hipMalloc(&p, bytes ? bytes : 16));
    return p;
}

static int run(int sync_free)
{
    uint32_t seed = 12345u + (uint32_t)sync_free;
    int32_t *idx = malloc(sizeof(int32_t) * T);
    float *w = malloc(sizeof(float) * T);
    uint16_t *x = malloc(sizeof(uint16_t) * T * H);
    int32_t hist[E] = {0};
    for (int t = 0; t < T; ++t) {
        uint32_t r = lcg(&seed);
        idx[t] = (r % 10 == 0) ? -1 : (int32_t)(r % E); /* ~10 % empty slots */
        w[t] = (float)(lcg(&seed) % 1000) / 1000.0f;
        if (idx[t] >= 0)
            hist[idx[t]]++;
        for (int h = 0; h < H; ++h)
            x[(size_t)t * H + h] = (uint16_t)(lcg(&seed) & 0x7F7F); /* finite bf16 patterns */
    }

    moe_desc d;
    memset(&d, 0, sizeof d);
    d.T = T;
    d.k = 1;
    d.E = E;
    d.local_begin = 0;
    d.num_local = E;
    d.pad_multiple = P;
    d.mode = sync_free ? MOE_SYNC_FREE : MOE_EAGER;
    d.idx_is_i64 = 0;
    d.capacity = sync_free ? moe_capacity_min(&d) + 7 : 0;
    CHECK(d.capacity >= 0);

    moe_handle hd;
    memset(&hd, 0, sizeof hd);
    hd.routing_map = dev((size_t)T * E);
    hd.tokens_per_expert = dev(sizeof(int32_t) * E);
    hd.padded_offsets = dev(sizeof(int32_t) * (E + 1));
    hd.row_of_slot = dev(sizeof(int32_t) * T);
    hd.status = dev(sizeof(int32_t) * 4);
    hd.workspace_bytes = moe_route_workspace_size(&d);
    CHECK(hd.workspace_bytes > 0);
    hd.workspace = dev(hd.workspace_bytes);

    int32_t *host_status = NULL;
    HIPCHECK(hipHostMalloc((void **)&host_status, sizeof(int32_t) * 4, hipHostMallocDefault));
    int32_t *d_idx = dev(sizeof(int32_t) * T);
    float *d_w = dev(sizeof(float) * T);
    uint16_t *d_x = dev(sizeof(uint16_t) * T * H);
    HIPCHECK(hipMemcpy(d_idx, idx, sizeof(int32_t) * T, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_w, w, sizeof(float) * T, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_x, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));

    CHECK(moe_route_build(&d, d_idx, NULL, NULL, &hd, host_status, NULL) == MOE_OK);
    HIPCHECK(hipDeviceSynchronize());
    int32_t st[4];
    HIPCHECK(hipMemcpy(st, hd.status, sizeof st, hipMemcpyDeviceToHost));
    int64_t R = sync_free ? d.capacity : host_status[0];
    if (!sync_free)
        CHECK(host_status[0] == st[0]);

    /* counts, offsets */
    int32_t tpe[E], off[E + 1];
    HIPCHECK(hipMemcpy(tpe, hd.tokens_per_expert, sizeof tpe, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(off, hd.padded_offsets, sizeof off, hipMemcpyDeviceToHost));
    CHECK(off[0] == 0);
    for (int e = 0; e < E; ++e) {
        CHECK(tpe[e] == hist[e]);
        CHECK(off[e + 1] - off[e] == (hist[e] + P - 1) / P * P);
    }
    CHECK(st[0] == off[E]);

    uint16_t *d_rows = dev(sizeof(uint16_t) * R * H);
    float *d_row_w = dev(sizeof(float) * R);
    int32_t *d_rt = dev(sizeof(int32_t) * R);
    int32_t *d_re = dev(sizeof(int32_t) * R);
    float *d_out = dev(sizeof(float) * T * H);
    /* the dispatch timed through its own launches */
    hipEvent_t ev0, ev1;
    HIPCHECK(hipEventCreateWithFlags(&ev0, hipEventDisableSystemFence));
    HIPCHECK(hipEventCreateWithFlags(&ev1, hipEventDisableSystemFence));
    CHECK(moe_time_next_call(ev0, ev1) == MOE_OK);
    CHECK(moe_dispatch(&d, &hd, d_x, H, d_w, R, d_rows, d_row_w, d_rt, d_re, NULL) == MOE_OK);
    CHECK(moe_combine(&d, &hd, d_rows, H, R, d_out, 1, NULL) == MOE_OK);
    /* dispatch backward of (grad rows = the rows, grad row weights = row weights) */
    float *d_gx = dev(sizeof(float) * T * H);
    float *d_gtw = dev(sizeof(float) * T);
    CHECK(moe_dispatch_bwd(&d, &hd, d_rows, H, R, d_row_w, d_gx, 1, d_gtw, NULL) == MOE_OK);
    /* a bad hidden size is rejected before any launch */
    CHECK(moe_combine(&d, &hd, d_rows, 100, R, d_out, 1, NULL) == MOE_ERR_HIDDEN);
    HIPCHECK(hipDeviceSynchronize());
    float disp_ms = 0.0f;
    HIPCHECK(hipEventElapsedTime(&disp_ms, ev0, ev1));
    CHECK(disp_ms > 0.0f && disp_ms < 1000.0f);
    HIPCHECK(hipEventDestroy(ev0));
    HIPCHECK(hipEventDestroy(ev1));

    int32_t *ros = malloc(sizeof(int32_t) * T);
    int32_t *rt = malloc(sizeof(int32_t) * R);
    int32_t *re = malloc(sizeof(int32_t) * R);
    float *rw = malloc(sizeof(float) * R);
    uint16_t *rows = malloc(sizeof(uint16_t) * R * H);
    float *out = malloc(sizeof(float) * T * H);
    float *gx = malloc(sizeof(float) * T * H);
    float *gtw = malloc(sizeof(float) * T);
    HIPCHECK(hipMemcpy(ros, hd.row_of_slot, sizeof(int32_t) * T, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(rt, d_rt, sizeof(int32_t) * R, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(re, d_re, sizeof(int32_t) * R, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(rw, d_row_w, sizeof(float) * R, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(rows, d_rows, sizeof(uint16_t) * R * H, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(out, d_out, sizeof(float) * T * H, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(gx, d_gx, sizeof(float) * T * H, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(gtw, d_gtw, sizeof(float) * T, hipMemcpyDeviceToHost));

    int32_t next[E];
    memcpy(next, off, sizeof next);
    for (int t = 0; t < T; ++t) {
        const int e = idx[t];
        if (e < 0) {
            CHECK(ros[t] == -1);
            CHECK(gtw[t] == 0.0f);
        } else {
            /* rows of an expert in ascending token order */
            CHECK(ros[t] == next[e]);
            next[e]++;
            CHECK(rt[ros[t]] == t && re[ros[t]] == e && rw[ros[t]] == w[t]);
            CHECK(memcmp(rows + (size_t)ros[t] * H, x + (size_t)t * H, sizeof(uint16_t) * H) == 0);
            CHECK(gtw[t] == w[t]);
        }
        for (int h = 0; h < H; ++h) {
            uint32_t u = (uint32_t)x[(size_t)t * H + h] << 16;
            float xv;
            memcpy(&xv, &u, sizeof xv);
            const float want = e < 0 ? 0.0f : xv; /* top-1: combine(dispatch(x)) = x */
            CHECK(out[(size_t)t * H + h] == want);
            CHECK(gx[(size_t)t * H + h] == want);
        }
    }
    /* pad rows and the sync-free tail: token -1, weight 0, zero data */
    for (int e = 0; e < E; ++e)
        for (int r = off[e] + tpe[e]; r < off[e + 1]; ++r)
            CHECK(rt[r] == -1 && re[r] == e && rw[r] == 0.0f);
    for (int64_t r = off[E]; r < R; ++r)
        CHECK(rt[r] == -1 && re[r] == E && rw[r] == 0.0f);
    for (int64_t r = 0; r < R; ++r)
        if (rt[r] < 0)
            for (int h = 0; h < H; ++h)
                CHECK(rows[(size_t)r * H + h] == 0);

    /* eager: the same route and dispatch as one call into worst-case buffers
       gives the same rows [0, total) and leaves the rest as it was */
    if (!sync_free) {
        const int64_t cap = moe_capacity_min(&d);
        CHECK(cap >= R);
        uint16_t *d_rows2 = dev(sizeof(uint16_t) * cap * H);
        float *d_rw2 = dev(sizeof(float) * cap);
        HIPCHECK(hipMemset(d_rows2, 0xAB, sizeof(uint16_t) * cap * H));
        CHECK(moe_route_dispatch(&d, d_idx, d_w, NULL, &hd, host_status, d_x, H, cap, d_rows2,
                                 d_rw2, NULL, NULL, NULL) == MOE_OK);
        CHECK(host_status[0] == R);
        uint16_t *rows2 = malloc(sizeof(uint16_t) * cap * H);
        float *rw2 = malloc(sizeof(float) * cap);
        HIPCHECK(hipMemcpy(rows2, d_rows2, sizeof(uint16_t) * cap * H, hipMemcpyDeviceToHost));
        HIPCHECK(hipMemcpy(rw2, d_rw2, sizeof(float) * cap, hipMemcpyDeviceToHost));
        CHECK(memcmp(rows2, rows, sizeof(uint16_t) * R * H) == 0);
        CHECK(memcmp(rw2, rw, sizeof(float) * R) == 0);
        for (int64_t i = R * H; i < cap * H; ++i)
            CHECK(rows2[i] == 0xABAB);
        free(rows2); free(rw2);
        hipFree(d_rows2); hipFree(d_rw2);
    }

    printf("%s: T=%d E=%d H=%d rows=%lld total=%d dispatch %.1f us\n",
           sync_free ? "sync-free" : "eager", T, E, H, (long long)R, st[0], disp_ms * 1e3f);
    free(idx); free(w); free(x); free(ros); free(rt); free(re); free(rw); free(rows); free(out);
    free(gx); free(gtw);
    hipFree(hd.routing_map); hipFree(hd.tokens_per_expert); hipFree(hd.padded_offsets);
    hipFree(hd.row_of_slot); hipFree(hd.status); hipFree(hd.workspace); hipHostFree(host_status);
    hipFree(d_idx); hipFree(d_w); hipFree(d_x); hipFree(d_rows); hipFree(d_row_w); hipFree(d_rt);
    hipFree(d_re); hipFree(d_out); hipFree(d_gx); hipFree(d_gtw);
    return 0;
}

int main(void)
{
    CHECK(moe_device_check(0) == MOE_OK);
    run(0);
    run(1);
    printf("abi ok\n");
    return 0;
}
