/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU statement of what the MoE routing /
 * dispatch / combine / combine-backward path computes.  It exists so that the
 * GPU library can be checked against something written independently of it:
 * it shares no code, header, table or constant with the HIP sources, and it is
 * only ever loaded by the tests, by the smoke check and by the benchmark's
 * CPU-baseline leg.  Nothing in the product path may call it.
 *
 * Sources (the pages this statement follows):
 *   [HEP]  "feat: add hybridep" (NVIDIA-NeMo/Automodel pull request 1333):
 *          Changelog (top-k indices -> multihot routing metadata), the review
 *          of the HybridEP dispatch hunk (routing_map + fp32 probs in,
 *          tokens_per_expert out, rows padded to pad_multiple), and the review
 *          note on _indices_to_multihot edge cases (all -1, duplicates, topk=1).
 *   [DEP]  "Add the deepep expert-parallel implementation" (huggingface/
 *          transformers pull request 49638), section "What this adds":
 *          bullets "Expanded layout", "Eager vs captured", "Custom ops",
 *          "Training", and the requirements paragraph (H multiple of 256).
 *
 * Where the pages leave a step open, this file takes one plain reading and
 * says so at the step (readings R1..R13 below are also listed in the design
 * notes of the repository):
 *   R1  rows inside one expert's group are in ascending token order;
 *   R2  repeated expert ids inside one token collapse into one row whose
 *       weight is the fp32 sum of the repeated slots' weights, ascending slot;
 *   R3  ids outside [-1, E) are treated as -1 and raise flag bit 0;
 *   R4  tokens_per_expert is the exact (unpadded) count; the padded total is
 *       padded_offsets[EL];
 *   R5  pad rows: zero data, weight +0, token -1, expert = owning expert;
 *   R6  the sentinel expert id is EL (one past the last local expert);
 *   R7  sync-free capacity must be >= T*min(k,EL) + EL*(P-1);
 *   R8  combine output is bf16 rounded to nearest-even from the fp32 sum
 *       (fp32 selectable); NaN results become the quiet NaN 0x7FC0;
 *   R9  combine adds the primary local slots in ascending slot order, the
 *       accumulator starting from the first term;
 *   R10 combine applies no weight;
 *   R11 dw uses the expert output before the routing weight is applied and is
 *       returned in [T,k] slot layout (repeated slots share the value);
 *   R12 dw is the exact dot product (exact bf16 x bf16 products, fp64 sum in
 *       ascending h), rounded once to fp32;
 *   R13 a token with no primary local slot combines to +0.
 * The FP8 dispatch (readings R14..R17) is stated at the end of the file.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Return codes: the oracle's own statement of the error contract. */
enum { ORC_OK = 0, ORC_ERR_ARG = 1, ORC_ERR_HIDDEN = 2, ORC_ERR_CAPACITY = 3, ORC_ERR_INDEX = 5 };
/* Flag bits. */
enum { ORC_FLAG_BAD_ID = 1, ORC_FLAG_DUP = 2 };

/* ------------------------------------------------------------------------- */
/* bfloat16 <-> binary32, from the format definitions.                       */
/* ------------------------------------------------------------------------- */

/* A bfloat16 is the upper half of a binary32 with the same sign, exponent and
 * leading significand bits, so widening is exact. */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a binary32 to the nearest bfloat16, ties to the even significand
 * (IEEE 754 roundTiesToEven).  Written as "pick the nearer of the two
 * bracketing bfloat16 values" with exact double arithmetic, not as a bit
 * trick.  Overflow: the value past the largest finite bfloat16 is treated as
 * 2^128 (the unbounded-exponent successor), so anything at or beyond the
 * midpoint rounds to infinity, as the standard requires. */
uint16_t oracle_bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return 0x7FC0; /* R8: canonical quiet NaN */
    uint16_t lo = (uint16_t)(u >> 16); /* same sign, magnitude truncated toward zero */
    if ((u & 0xFFFFu) == 0)
        return lo; /* exactly representable (includes +-0 and +-inf) */
    uint16_t hi = (uint16_t)(lo + 1); /* next bfloat16 away from zero */
    double v = fabs((double)f);
    double a = fabs(bf16_value(lo));
    double b = ((hi & 0x7F80u) == 0x7F80u) ? ldexp(1.0, 128) : fabs(bf16_value(hi));
    double da = v - a, db = b - v; /* both exact: operands share a binade */
    if (da < db)
        return lo;
    if (db < da)
        return hi;
    return (lo & 1u) ? hi : lo;
}

/* Array form of the rounding above, for tests that sweep many values. */
void oracle_bf16_round_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_round(in[i]);
}

/* ------------------------------------------------------------------------- */
/* Argument rules ([DEP] requirements: H a multiple of 256; [DEP] "Eager vs   */
/* captured": worst-case capacity must not overflow).                         */
/* ------------------------------------------------------------------------- */

int64_t oracle_capacity_min(int64_t T, int32_t k, int32_t EL, int32_t P)
{
    int64_t kk = k < EL ? k : EL;
    return T * kk + (int64_t)EL * (P - 1); /* R7 */
}

int oracle_check_args(int64_t T, int32_t k, int32_t E, int32_t lb, int32_t EL, int32_t P,
                      int32_t sync_free, int64_t C)
{
    if (T < 0 || k < 1 || E < 1 || P < 1 || lb < 0 || EL < 1 || (int64_t)lb + EL > E)
        return ORC_ERR_ARG;
    if (sync_free && C < oracle_capacity_min(T, k, EL, P))
        return ORC_ERR_CAPACITY;
    return ORC_OK;
}

int oracle_check_hidden(int64_t H)
{
    return (H <= 0 || H % 256 != 0) ? ORC_ERR_HIDDEN : ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Routing: multihot map, counts, padded offsets, row assignment.            */
/* ------------------------------------------------------------------------- */

/*
 * Inputs
 *   idx [T,k]  expert id per slot, -1 = no expert ([HEP] multihot conversion)
 *   w   [T,k]  fp32 routing weight per slot, or NULL ([HEP]: probs are fp32)
 *   x   [T,H]  bf16 hidden rows, or NULL for metadata only
 * Outputs (caller-allocated; R_cap rows of row storage)
 *   map [T,E] u8, probs [T,E] f32 (NULL allowed; needs w), tpe [EL],
 *   off [EL+1], row_of_slot [T,k], row_token/row_expert [R_cap],
 *   row_w [R_cap] (NULL allowed; needs w), rows [R_cap,H] (needs x),
 *   total_out (padded total), flags_out.
 * Returns ORC_OK / ORC_ERR_*; for R_cap smaller than the rows needed,
 * ORC_ERR_CAPACITY.
 */
int oracle_route(int64_t T, int32_t k, int32_t E, int32_t lb, int32_t EL, int32_t P,
                 int32_t sync_free, int64_t C,
                 const int64_t *idx, const float *w, const uint16_t *x, int64_t H,
                 uint8_t *map, float *probs, int32_t *tpe, int32_t *off, int32_t *row_of_slot,
                 int64_t R_cap, int32_t *row_token, int32_t *row_expert, float *row_w,
                 uint16_t *rows, int64_t *total_out, int32_t *flags_out)
{
    int rc = oracle_check_args(T, k, E, lb, EL, P, sync_free, C);
    if (rc != ORC_OK)
        return rc;
    if (x && oracle_check_hidden(H) != ORC_OK)
        return ORC_ERR_HIDDEN;

    int32_t flags = 0;
    /* merged weight per (token, expert); local scratch of the oracle */
    float *W = (float *)calloc((size_t)(T > 0 ? T : 1) * (size_t)E, sizeof(float));
    if (!W)
        return ORC_ERR_ARG;
    memset(map, 0, (size_t)T * (size_t)E);

    /* Step 1-2: multihot map.  Walk slots in order; the first slot naming an
     * expert sets the map entry and its weight, a later slot naming the same
     * expert adds its weight (R2).  Out-of-range ids count as -1 (R3). */
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int64_t e = idx[t * k + j];
            if (e == -1)
                continue;
            if (e < -1 || e >= E) {
                flags |= ORC_FLAG_BAD_ID;
                continue;
            }
            if (map[t * E + e]) {
                flags |= ORC_FLAG_DUP;
                if (w)
                    W[t * E + e] = W[t * E + e] + w[t * k + j];
            } else {
                map[t * E + e] = 1;
                if (w)
                    W[t * E + e] = w[t * k + j];
            }
        }
    }
    if (probs) {
        for (int64_t i = 0; i < T * (int64_t)E; ++i)
            probs[i] = map[i] ? W[i] : 0.0f;
    }

    /* Step 3: tokens_per_expert = number of tokens routed to each local
     * expert (R4: exact, not padded). */
    for (int32_t e = 0; e < EL; ++e) {
        int32_t c = 0;
        for (int64_t t = 0; t < T; ++t)
            c += map[t * E + lb + e];
        tpe[e] = c;
    }

    /* Step 4: each expert's group padded up to a multiple of P. */
    off[0] = 0;
    for (int32_t e = 0; e < EL; ++e) {
        int32_t padded = ((tpe[e] + P - 1) / P) * P;
        off[e + 1] = off[e] + padded;
    }
    int64_t total = off[EL];
    int64_t R = sync_free ? C : total;
    if (R > R_cap) {
        free(W);
        return ORC_ERR_CAPACITY;
    }

    /* Step 5: rows, expert by expert, tokens ascending inside (R1). */
    for (int64_t i = 0; i < T * (int64_t)k; ++i)
        row_of_slot[i] = -1;
    for (int32_t e = 0; e < EL; ++e) {
        int64_t r = off[e];
        for (int64_t t = 0; t < T; ++t) {
            if (!map[t * E + lb + e])
                continue;
            row_token[r] = (int32_t)t;
            row_expert[r] = e;
            if (row_w)
                row_w[r] = W[t * E + lb + e];
            if (rows)
                memcpy(rows + r * H, x + t * H, (size_t)H * sizeof(uint16_t));
            for (int32_t j = 0; j < k; ++j)
                if (idx[t * k + j] == (int64_t)lb + e)
                    row_of_slot[t * k + j] = (int32_t)r;
            ++r;
        }
        for (; r < off[e + 1]; ++r) { /* R5: pad rows */
            row_token[r] = -1;
            row_expert[r] = e;
            if (row_w)
                row_w[r] = 0.0f;
            if (rows)
                memset(rows + r * H, 0, (size_t)H * sizeof(uint16_t));
        }
    }
    /* Step 6: sync-free tail rows [total, C) belong to the sentinel expert
     * EL and are zero ([DEP] "Eager vs captured"; R6). */
    for (int64_t r = total; r < R; ++r) {
        row_token[r] = -1;
        row_expert[r] = EL;
        if (row_w)
            row_w[r] = 0.0f;
        if (rows)
            memset(rows + r * H, 0, (size_t)H * sizeof(uint16_t));
    }

    free(W);
    *total_out = total;
    *flags_out = flags;
    return (flags & ORC_FLAG_BAD_ID) ? ORC_ERR_INDEX : ORC_OK;
}

/* Is slot (t, j) a primary local slot: a valid id inside the local range,
 * not repeated by an earlier slot of the same token? */
static int primary_local(const int64_t *idx, int64_t t, int32_t j, int32_t k, int32_t E,
                         int32_t lb, int32_t EL)
{
    int64_t e = idx[t * k + j];
    if (e < 0 || e >= E || e < lb || e >= (int64_t)lb + EL)
        return 0;
    for (int32_t q = 0; q < j; ++q)
        if (idx[t * k + q] == e)
            return 0;
    return 1;
}

/* ------------------------------------------------------------------------- */
/* Combine ([DEP] "Expanded layout": a plain sum, weights belong to experts) */
/* ------------------------------------------------------------------------- */

/* out[t] = sum over the primary local slots of t, ascending slot order, of
 * Y[row_of_slot[t][j]]; fp32 adds (R9), no weights (R10), +0 for a token
 * without such a slot (R13).  Output bf16 (out_bf16) and/or fp32 (out_f32). */
int oracle_combine(int64_t T, int32_t k, int32_t E, int32_t lb, int32_t EL,
                   const int64_t *idx, const int32_t *row_of_slot, int64_t R, int64_t H,
                   const uint16_t *Y, uint16_t *out_bf16, float *out_f32)
{
    if (oracle_check_hidden(H) != ORC_OK)
        return ORC_ERR_HIDDEN;
    float *acc = (float *)malloc((size_t)H * sizeof(float));
    if (!acc)
        return ORC_ERR_ARG;
    for (int64_t t = 0; t < T; ++t) {
        int have = 0;
        for (int32_t j = 0; j < k; ++j) {
            if (!primary_local(idx, t, j, k, E, lb, EL))
                continue;
            int64_t r = row_of_slot[t * k + j];
            if (r < 0 || r >= R)
                continue;
            for (int64_t h = 0; h < H; ++h) {
                float v = (float)bf16_value(Y[r * H + h]);
                acc[h] = have ? acc[h] + v : v;
            }
            have = 1;
        }
        for (int64_t h = 0; h < H; ++h) {
            float s = have ? acc[h] : 0.0f;
            if (out_bf16)
                out_bf16[t * H + h] = oracle_bf16_round(s);
            if (out_f32)
                out_f32[t * H + h] = s;
        }
    }
    free(acc);
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Combine backward ([DEP] "Custom ops": the combine's backward is a cached   */
/* dispatch; "Training": gradients reach the routing weights).               */
/* ------------------------------------------------------------------------- */

/* grad_rows: the dispatch of grad_out along the forward's rows (same walk as
 * oracle_route with x = grad_out; pad and sentinel rows zero).
 * dw[t][j] (F != NULL): exact dot of grad_out[t] with F[row of slot (t,j)],
 * fp64 sum in ascending h, one rounding to fp32 (R11, R12); 0 for a slot with
 * no local row. */
int oracle_combine_bwd(int64_t T, int32_t k, int32_t E, int32_t lb, int32_t EL,
                       const int64_t *idx, const int32_t *row_of_slot, const int32_t *row_token,
                       int64_t R, int64_t H, const uint16_t *grad_out, const uint16_t *F,
                       uint16_t *grad_rows, float *dw)
{
    if (oracle_check_hidden(H) != ORC_OK)
        return ORC_ERR_HIDDEN;
    for (int64_t r = 0; r < R; ++r) {
        int64_t t = row_token[r];
        if (t >= 0)
            memcpy(grad_rows + r * H, grad_out + t * H, (size_t)H * sizeof(uint16_t));
        else
            memset(grad_rows + r * H, 0, (size_t)H * sizeof(uint16_t));
    }
    if (dw) {
        for (int64_t t = 0; t < T; ++t) {
            for (int32_t j = 0; j < k; ++j) {
                int64_t e = idx[t * k + j];
                int64_t r = row_of_slot[t * k + j];
                if (e < lb || e >= (int64_t)lb + EL || e >= E || r < 0 || r >= R || !F) {
                    dw[t * k + j] = 0.0f;
                    continue;
                }
                double s = 0.0;
                for (int64_t h = 0; h < H; ++h)
                    s += bf16_value(grad_out[t * H + h]) * bf16_value(F[r * H + h]);
                dw[t * k + j] = (float)s;
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Dispatch backward ([DEP] "Training": gradients reach the tokens and the    */
/* routing weights; the weight gradients go back through a combine).          */
/* ------------------------------------------------------------------------- */

/* Dispatch copies x[t] to the row of each of t's local slots and the slot's
 * weight to that row's weight (repeated ids: the sum of their weights), so its
 * adjoint is:
 *   grad_x[t]         = sum over t's primary local slots, ascending slot, of
 *                       grad_rows[row]   -- the combine of the grad rows (R9)
 *   grad_topk_w[t][j] = grad_row_w[row of slot (t,j)] for every local valid
 *                       slot (a repeated id gets its row's gradient too, since
 *                       the row's weight is the plain sum of the slots'), and 0
 *                       for a slot with no local row.
 * grad_row_w and grad_topk_w may both be NULL. */
int oracle_dispatch_bwd(int64_t T, int32_t k, int32_t E, int32_t lb, int32_t EL,
                        const int64_t *idx, const int32_t *row_of_slot, int64_t R, int64_t H,
                        const uint16_t *grad_rows, const float *grad_row_w,
                        uint16_t *grad_x_bf16, float *grad_x_f32, float *grad_topk_w)
{
    int rc = oracle_combine(T, k, E, lb, EL, idx, row_of_slot, R, H, grad_rows, grad_x_bf16,
                            grad_x_f32);
    if (rc != ORC_OK || !grad_topk_w)
        return rc;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int64_t e = idx[t * k + j];
            int64_t r = row_of_slot[t * k + j];
            int local = e >= lb && e < (int64_t)lb + EL && e < E;
            grad_topk_w[t * k + j] = (local && r >= 0 && r < R && grad_row_w) ? grad_row_w[r] : 0.0f;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* FP8 dispatch ([DEP] "What this adds": FP8 dispatch is named as a follow-up */
/* to halve the dispatched bytes; the page fixes no format).                  */
/* ------------------------------------------------------------------------- */
/*
 * Readings (R14..R17):
 *   R14 element format: the OCP 8-bit floating point E4M3 encoding
 *       ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 *       infinities; S.1111.111 is NaN; largest finite magnitude 448;
 *       exponent field 0 holds the subnormals m * 2^-9.
 *   R15 one fp32 scale per token and per 128 consecutive hidden elements:
 *         a     = max(max_i |x_i|, 1e-4f)
 *         scale = a / 448            (fp32, nearest-even)
 *         inv   = 448 / a            (fp32, nearest-even)
 *         q_i   = e4m3(clamp(x_i * inv, -448, 448))   (fp32 product)
 *       so that x_i ~= value(q_i) * scale.
 *   R16 e4m3(v) is the representable value nearest to v, ties to the even
 *       code (IEEE roundTiesToEven); the sign of v is kept (so -0 -> 0x80).
 *   R17 pad and sentinel rows are all-zero bytes with scale +0; row weights,
 *       tokens and experts are those of the bf16 dispatch.
 * x is expected finite; for NaN or infinite x the result is unspecified.
 */

/* Value of an E4M3 code, from the field definitions (R14). */
double oracle_e4m3_value(uint8_t c)
{
    int e = (c >> 3) & 15, m = c & 7;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    if (e == 15 && m == 7)
        mag = NAN;
    return (c & 0x80) ? -mag : mag;
}

/* Nearest E4M3 code (R16) by a scan of the 127 finite non-negative codes:
 * a later code replaces the best so far if it is strictly nearer, or equally
 * near and even while the best is odd.  Magnitudes past 448 go to 448. */
uint8_t oracle_e4m3_round(float f)
{
    double v = fabs((double)f);
    int best = 0;
    for (int c = 1; c <= 0x7E; ++c) {
        double dc = fabs(oracle_e4m3_value((uint8_t)c) - v);
        double db = fabs(oracle_e4m3_value((uint8_t)best) - v);
        if (dc < db || (dc == db && (c & 1) == 0 && (best & 1) != 0))
            best = c;
    }
    return (uint8_t)((signbit(f) ? 0x80 : 0) | best);
}

void oracle_e4m3_round_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_round(in[i]);
}

/* One token's row x[H] (bf16) -> q[H] (E4M3 codes) and scale[H/128] (R15). */
void oracle_fp8_quantize_row(int64_t H, const uint16_t *x, uint8_t *q, float *scale)
{
    for (int64_t b = 0; b < H / 128; ++b) {
        const uint16_t *xb = x + b * 128;
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            float m = fabsf((float)bf16_value(xb[i]));
            if (m > amax)
                amax = m;
        }
        float a = amax > 1e-4f ? amax : 1e-4f;
        float s = a / 448.0f;
        float inv = 448.0f / a;
        scale[b] = s;
        for (int i = 0; i < 128; ++i) {
            float y = (float)bf16_value(xb[i]) * inv;
            if (y > 448.0f)
                y = 448.0f;
            if (y < -448.0f)
                y = -448.0f;
            q[b * 128 + i] = oracle_e4m3_round(y);
        }
    }
}

/* The FP8 dispatch of rows [0, R): a data row (row_token[r] >= 0) holds the
 * quantized row of its token, every other row zero bytes and zero scales
 * (R17).  row_token is the routing's (oracle_route). */
int oracle_dispatch_fp8(int64_t T, int64_t H, const uint16_t *x, int64_t R,
                        const int32_t *row_token, uint8_t *rows_q, float *row_scale)
{
    if (oracle_check_hidden(H) != ORC_OK)
        return ORC_ERR_HIDDEN;
    const int64_t nb = H / 128;
    for (int64_t r = 0; r < R; ++r) {
        int64_t t = row_token[r];
        if (t >= 0 && t < T) {
            oracle_fp8_quantize_row(H, x + t * H, rows_q + r * H, row_scale + r * nb);
        } else {
            memset(rows_q + r * H, 0, (size_t)H);
            for (int64_t b = 0; b < nb; ++b)
                row_scale[r * nb + b] = 0.0f;
        }
    }
    return ORC_OK;
}
