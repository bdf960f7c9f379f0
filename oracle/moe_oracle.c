/*
 * moe_oracle.c - plain CPU oracle of one MoE FFN layer (test infrastructure).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
 * this file. It shares no code with the GPU library. Build with
 * -O2 -ffp-contract=off so that every multiply and add rounds on its own.
 * The definitions it follows are listed in moe_oracle.h; each function below
 * names the passage it restates.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the upper half of an fp32 bit pattern: widening is exact. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static double elem(const void* base, int dtype, int64_t i)
{
    if (dtype == MOE_ORACLE_BF16)
        return (double)bf16_to_f32(((const uint16_t*)base)[i]);
    return (double)((const float*)base)[i];
}

static int layer_ok(const moe_oracle_layer_t* L)
{
    if (!L || L->d <= 0 || L->f <= 0 || L->E <= 0 || L->k <= 0 || L->k > L->E)
        return 0;
    if (L->dtype != MOE_ORACLE_F32 && L->dtype != MOE_ORACLE_BF16)
        return 0;
    return L->w_router && L->w_gate && L->w_up && L->w_down;
}

int moe_oracle_widen(const void* src, int dtype, int64_t n, float* dst)
{
    if (!src || !dst || n < 0)
        return -1;
    if (dtype != MOE_ORACLE_F32 && dtype != MOE_ORACLE_BF16)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = (float)elem(src, dtype, i);
    return 0;
}

/* Router projection, «Colibri 是什么» (xxqk.cn) §3.2: a linear map of the
 * token plus a router bias, one logit per expert. The router matrix is
 * (hidden_dim, n_experts) as «Colibri不是一只蜂鸟» (discosf.com) §4.3 stores it.
 * The double sum is rounded once to fp32. */
static float router_logit(const moe_oracle_layer_t* L, const void* x, int64_t t, int e)
{
    const int64_t d = L->d, E = L->E;
    double acc = 0.0;
    for (int64_t i = 0; i < d; ++i)
        acc += elem(x, L->dtype, t * d + i) * elem(L->w_router, L->dtype, i * E + e);
    if (L->b_router)
        acc += (double)L->b_router[e];
    return (float)acc;
}

int moe_oracle_router(const moe_oracle_layer_t* L, const void* x, int32_t T, float* logits)
{
    if (!layer_ok(L) || !x || !logits || T < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < L->E; ++e)
            logits[(int64_t)t * L->E + e] = router_logit(L, x, t, e);
    return 0;
}

/* "a precedes b" in the selection order: larger logit first, equal logits
 * broken to the lower expert index. */
static int precedes(const float* l, int a, int b)
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

/* The k winners of one token, slot 0 first, in the selection order. */
static void select_topk(const float* l, int E, int k, int32_t* ids)
{
    unsigned char taken[1024];
    int big = E > 1024;
    unsigned char* tk = big ? (unsigned char*)calloc((size_t)E, 1) : taken;
    if (!big)
        memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (tk[e])
                continue;
            if (best < 0 || precedes(l, e, best))
                best = e;
        }
        tk[best] = 1;
        ids[j] = best;
    }
    if (big)
        free(tk);
}

/* Routing weights of the given k experts: the softmax restricted to their
 * logits, renormalised, with the exponent shifted by the slot-0 logit, in
 * double. */
static void route_weights(const float* l, int k, const int32_t* ids, double* wd)
{
    double l0 = (double)l[ids[0]];
    double s = 0.0;
    for (int j = 0; j < k; ++j) {
        wd[j] = exp((double)l[ids[j]] - l0);
        s += wd[j];
    }
    for (int j = 0; j < k; ++j)
        wd[j] = wd[j] / s;
}

/* Top-k selection and routing weights for one token. Selection on the raw
 * logits («Colibri 是什么» (xxqk.cn) §3.2 selects on logits; softmax is
 * monotone so the set equals the top-k of the softmax that
 * «Colibri：面向MoE模型的高性能C语言推理引擎» (zskr.cn) §2.2 fuses in); the
 * weights are the softmax restricted to the k winners. */
static void topk_one(const float* l, int E, int k, int32_t* ids, double* wd)
{
    select_topk(l, E, k, ids);
    route_weights(l, k, ids, wd);
}

int moe_oracle_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                    int32_t* ids, float* w, double* w_f64)
{
    if (!logits || !ids || !w || T < 0 || E <= 0 || k <= 0 || k > E)
        return -1;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
        double wd[256];
        double* wp = k <= 256 ? wd : (double*)malloc(sizeof(double) * (size_t)k);
        topk_one(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, wp);
        for (int j = 0; j < k; ++j) {
            w[(int64_t)t * k + j] = (float)wp[j];
            if (w_f64)
                w_f64[(int64_t)t * k + j] = wp[j];
        }
        if (wp != wd)
            free(wp);
    }
    return 0;
}

int moe_oracle_route_weights(const float* logits, int32_t T, int32_t E, int32_t k,
                             const int32_t* ids, float* w, double* w_f64)
{
    if (!logits || !ids || !w || T < 0 || E <= 0 || k <= 0 || k > E)
        return -1;
    for (int64_t a = 0; a < (int64_t)T * k; ++a)
        if (ids[a] < 0 || ids[a] >= E)
            return -2;
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
        double wd[256];
        double* wp = k <= 256 ? wd : (double*)malloc(sizeof(double) * (size_t)k);
        route_weights(logits + (int64_t)t * E, k, ids + (int64_t)t * k, wp);
        for (int j = 0; j < k; ++j) {
            w[(int64_t)t * k + j] = (float)wp[j];
            if (w_f64)
                w_f64[(int64_t)t * k + j] = wp[j];
        }
        if (wp != wd)
            free(wp);
    }
    return 0;
}

/* Dispatch, «Colibri 是什么» (xxqk.cn) §2.1 and §2.3: each token is scattered
 * into the input buffers of its k experts. Restated as a stable counting sort:
 * a histogram of expert ids, an exclusive prefix sum, then a scatter that
 * visits assignments in (token, slot) order so that each expert's segment
 * lists its tokens in ascending token order. */
int moe_oracle_dispatch(const int32_t* ids, int32_t T, int32_t k, int32_t E,
                        int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* perm_slot, int32_t* inv)
{
    if (!ids || !counts || !offsets || T < 0 || k <= 0 || E <= 0)
        return -1;
    const int64_t A = (int64_t)T * k;
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t a = 0; a < A; ++a) {
        if (ids[a] < 0 || ids[a] >= E)
            return -2;
        counts[ids[a]] += 1;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!fill)
        return -3;
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = ids[(int64_t)t * k + j];
            int32_t p = offsets[e] + fill[e];
            fill[e] += 1;
            if (perm)
                perm[p] = t;
            if (perm_slot)
                perm_slot[p] = j;
            if (inv)
                inv[(int64_t)t * k + j] = p;
        }
    }
    free(fill);
    return 0;
}

/* One expert's SwiGLU FFN on one row, in double.
 * Three GEMMs per expert as «Colibri 是什么» (nxbn.cn) §4.3 lists them
 * (w1*x, w3*x, then w2 applied to the SwiGLU output), with the Mixtral shapes
 * of «Colibri：面向MoE模型的高性能C语言推理引擎» (zskr.cn) §4.2: gate and up are
 * (d_ff, d), down is (d, d_ff), each (out, in) row-major.
 *   g_i = sum_c v_c W_g[e][i][c];  u_i = sum_c v_c W_u[e][i][c]
 *   h_i = SiLU(g_i) * u_i = g_i / (1 + exp(-g_i)) * u_i
 *   out_o = sum_i h_i W_d[e][o][i] */
static void quantize_row_values(double* v, int64_t n);

/* With act_fp8 (8-bit activations, reading in moe_oracle.h) the input row
 * enters the gate and up products as its 8-bit row-quantized value; h stays
 * in double. xv is scratch of d doubles. */
static void expert_ffn(const moe_oracle_layer_t* L, int32_t e, const void* xbase, int64_t xoff,
                       double* h, double* out, int act_fp8, double* xv)
{
    const int64_t d = L->d, f = L->f;
    const int dt = L->dtype;
    const int64_t wg0 = (int64_t)e * f * d;
    const int64_t wd0 = (int64_t)e * d * f;
    for (int64_t c = 0; c < d; ++c)
        xv[c] = elem(xbase, dt, xoff + c);
    if (act_fp8)
        quantize_row_values(xv, d);
    for (int64_t i = 0; i < f; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t c = 0; c < d; ++c) {
            g += xv[c] * elem(L->w_gate, dt, wg0 + i * d + c);
            u += xv[c] * elem(L->w_up, dt, wg0 + i * d + c);
        }
        h[i] = g / (1.0 + exp(-g)) * u;
    }
    for (int64_t o = 0; o < d; ++o) {
        double acc = 0.0;
        for (int64_t i = 0; i < f; ++i)
            acc += h[i] * elem(L->w_down, dt, wd0 + o * f + i);
        out[o] = acc;
    }
}

int moe_oracle_expert_ffn_ex(const moe_oracle_layer_t* L, int32_t e, const void* v,
                             double* out, double* h_out, int32_t flags)
{
    if (!layer_ok(L) || !v || !out || e < 0 || e >= L->E || (flags & ~MOE_ORACLE_ACT_FP8))
        return -1;
    double* h = h_out ? h_out : (double*)malloc(sizeof(double) * (size_t)L->f);
    double* xv = (double*)malloc(sizeof(double) * (size_t)L->d);
    if (!h || !xv) {
        if (!h_out)
            free(h);
        free(xv);
        return -3;
    }
    expert_ffn(L, e, v, 0, h, out, flags & MOE_ORACLE_ACT_FP8, xv);
    if (!h_out)
        free(h);
    free(xv);
    return 0;
}

int moe_oracle_expert_ffn(const moe_oracle_layer_t* L, int32_t e, const void* v,
                          double* out, double* h_out)
{
    return moe_oracle_expert_ffn_ex(L, e, v, out, h_out, 0);
}

/* Whole layer per token: route, select, run the k experts, weighted sum.
 * The combine follows «Colibri 是什么» (xxqk.cn) §2.3 (outputs weighted by
 * the gating score and summed) and «Colibri：面向MoE模型的高性能C语言推理引擎»
 * (zskr.cn) §3.3 (the main thread sums the expert outputs with the gate
 * weights). Summation over slots is in slot order, in double. */
int moe_oracle_forward(const moe_oracle_layer_t* L, const void* x, int32_t T,
                       const int32_t* forced_ids, const int32_t* token_list, int32_t n,
                       double* y, double* Y_slots)
{
    return moe_oracle_forward_ex(L, x, T, forced_ids, token_list, n, y, Y_slots, 0);
}

int moe_oracle_forward_ex(const moe_oracle_layer_t* L, const void* x, int32_t T,
                          const int32_t* forced_ids, const int32_t* token_list, int32_t n,
                          double* y, double* Y_slots, int32_t flags)
{
    if (!layer_ok(L) || !x || !y || T < 0 || n < 0 || (flags & ~MOE_ORACLE_ACT_FP8))
        return -1;
    const int act_fp8 = (flags & MOE_ORACLE_ACT_FP8) != 0;
    if (!token_list && n != T)
        return -1;
    const int32_t E = L->E, k = L->k;
    const int64_t d = L->d, f = L->f;
    int err = 0;
    for (int32_t r = 0; r < n; ++r) {
        int32_t t = token_list ? token_list[r] : r;
        if (t < 0 || t >= T)
            return -1;
        if (forced_ids)
            for (int32_t j = 0; j < k; ++j)
                if (forced_ids[(int64_t)t * k + j] < 0 || forced_ids[(int64_t)t * k + j] >= E)
                    return -2;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < n; ++r) {
        int32_t t = token_list ? token_list[r] : r;
        float* lg = (float*)malloc(sizeof(float) * (size_t)E);
        int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
        double* wd = (double*)malloc(sizeof(double) * (size_t)k);
        double* h = (double*)malloc(sizeof(double) * (size_t)f);
        double* ye = (double*)malloc(sizeof(double) * (size_t)d);
        double* xv = (double*)malloc(sizeof(double) * (size_t)d);
        if (!lg || !ids || !wd || !h || !ye || !xv) {
#pragma omp atomic write
            err = -3;
        } else {
            for (int32_t e = 0; e < E; ++e)
                lg[e] = router_logit(L, x, t, e);
            if (forced_ids) {
                for (int32_t j = 0; j < k; ++j)
                    ids[j] = forced_ids[(int64_t)t * k + j];
                route_weights(lg, k, ids, wd);
            } else {
                topk_one(lg, E, k, ids, wd);
            }
            double* yr = y + (int64_t)r * d;
            for (int64_t o = 0; o < d; ++o)
                yr[o] = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                expert_ffn(L, ids[j], x, (int64_t)t * d, h, ye, act_fp8, xv);
                if (Y_slots)
                    memcpy(Y_slots + ((int64_t)r * k + j) * d, ye, sizeof(double) * (size_t)d);
                for (int64_t o = 0; o < d; ++o)
                    yr[o] += wd[j] * ye[o];
            }
        }
        free(lg);
        free(ids);
        free(wd);
        free(h);
        free(ye);
        free(xv);
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* 8-bit expert weights: OCP FP8 E4M3 codes with one power-of-two scale per
 * weight row (the reading stated in moe_oracle.h). Written from the format's
 * definition: value = (-1)^s * 2^(E-7) * (1 + m/8) for E > 0, and
 * (-1)^s * 2^-6 * (m/8) for E = 0. */

double moe_oracle_fp8_value(uint8_t code)
{
    const int s = code >> 7, E = (code >> 3) & 15, m = code & 7;
    if (E == 15 && m == 7)
        return NAN;
    const double v = (E == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, E - 10);
    return s ? -v : v;
}

/* Nearest integer to x >= 0, ties to even. */
static double round_half_even(double x)
{
    const double f = floor(x);
    const double r = x - f;
    if (r > 0.5)
        return f + 1.0;
    if (r < 0.5)
        return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* E4M3 code of v, |v| <= 448, ties to even. */
static uint8_t fp8_encode(double v)
{
    const int neg = signbit(v) ? 1 : 0;
    const double a = fabs(v);
    int E, m;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: steps of 2^-9; a count of 8 is the smallest normal */
        const int q = (int)round_half_even(ldexp(a, 9));
        E = q >> 3;
        m = q & 7;
    } else {
        int x;
        (void)frexp(a, &x); /* a = f * 2^x, f in [0.5, 1): exponent of a is x-1 */
        E = x - 1 + 7;
        const double frac = ldexp(a, -(x - 1)) - 1.0; /* in [0, 1) */
        m = (int)round_half_even(frac * 8.0);
        if (m == 8) {
            m = 0;
            E += 1;
        }
    }
    return (uint8_t)((neg << 7) | (E << 3) | m);
}

/* Exponent e of a row's power-of-two scale from its largest magnitude (the
 * rule of the reading: smallest e with amax <= 448 * 2^e, 0 for a zero row,
 * at least -126). */
static int row_scale_exp(double amax)
{
    if (!(amax > 0.0))
        return 0;
    int x;
    const double f = frexp(amax, &x); /* amax = f * 2^x, f in [0.5, 1) */
    /* 448 = 0.875 * 2^9: amax <= 448 * 2^e  <=>  f * 2^(x-9-e) <= 0.875 */
    const int e = (f <= 0.875) ? x - 9 : x - 8;
    return e < -126 ? -126 : e;
}

/* v[0..n) replaced by its 8-bit row quantization, dequantized: code * 2^e. */
static void quantize_row_values(double* v, int64_t n)
{
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    const int e = row_scale_exp(amax);
    for (int64_t i = 0; i < n; ++i)
        v[i] = ldexp(moe_oracle_fp8_value(fp8_encode(ldexp(v[i], -e))), e);
}

int moe_oracle_quantize_fp8(const void* w, int dtype, int64_t rows, int64_t cols,
                            uint8_t* codes, float* scales)
{
    if (!w || !codes || !scales || rows <= 0 || cols <= 0)
        return -1;
    if (dtype != MOE_ORACLE_F32 && dtype != MOE_ORACLE_BF16)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double amax = 0.0;
        for (int64_t i = 0; i < cols; ++i) {
            const double a = fabs(elem(w, dtype, r * cols + i));
            if (a > amax)
                amax = a;
        }
        const int e = row_scale_exp(amax);
        scales[r] = (float)ldexp(1.0, e);
        for (int64_t i = 0; i < cols; ++i)
            codes[r * cols + i] = fp8_encode(ldexp(elem(w, dtype, r * cols + i), -e));
    }
    return 0;
}

int moe_oracle_dequantize_fp8(const uint8_t* codes, const float* scales, int64_t rows,
                              int64_t cols, uint16_t* bf16_out)
{
    if (!codes || !scales || !bf16_out || rows <= 0 || cols <= 0)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < cols; ++i) {
            const double v = moe_oracle_fp8_value(codes[r * cols + i]) * (double)scales[r];
            const float f = (float)v;
            uint32_t u;
            memcpy(&u, &f, 4);
            if ((double)f != v || (u & 0xFFFFu) != 0)
                return -2;
            bf16_out[r * cols + i] = (uint16_t)(u >> 16);
        }
    }
    return 0;
}
