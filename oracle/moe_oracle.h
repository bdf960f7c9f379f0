/*
 * moe_oracle.h - plain, slow CPU oracle of one Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code with the GPU library.
 *
 * What it computes (sources: the Colibri pages --
 *   «Colibri 是什么» (xxqk.cn) §2.1 MoE flow, §2.3 dispatch/expert/combine
 *     kernels, §3.2 router projection and top-k;
 *   «Colibri：面向MoE模型的高性能C语言推理引擎» (zskr.cn) §1 gate -> top-k
 *     -> experts -> weighted sum, §2.2 fused gate matmul + softmax + top-k,
 *     §3.3 per-expert forward then weighted sum, §4.2 Mixtral w1/w2/w3 shapes;
 *   «Colibri 是什么» (nxbn.cn) §4.3 expert GEMMs w1*x, w3*x, w2*swiglu_out;
 *   «Colibri不是一只蜂鸟» (discosf.com) §4.3 (out_dim, in_dim) row-major
 *     expert matrices and a (hidden_dim, n_experts) router matrix):
 *
 *   logits[t][e] = sum_i x[t][i] * W_r[i][e] + b_r[e]            (fp32 result)
 *   TopK(t)      = first k experts in the order (logit desc, index asc)
 *   w[t][j]      = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0)    (over the k winners)
 *   FFN_e(v)     = W_d[e] (SiLU(W_g[e] v) .* (W_u[e] v)),  SiLU(z) = z / (1 + e^-z)
 *   y[t]         = sum_j w[t][j] * FFN_{e_tj}(x[t])
 *
 * and the dispatch as a stable counting sort of the (token, slot) assignments
 * by expert, in token order.
 *
 * Precision: inputs are widened exactly to fp32 (bf16 bits << 16); every dot
 * product accumulates in double in index order; logits are rounded once to
 * fp32 (selection uses those fp32 values); routing weights are computed in
 * double and also reported as fp32; the FFN and the combine stay in double
 * (h is not rounded), so y is the exact function of the given inputs up to
 * double rounding.
 *
 * Errors: functions return 0 on success and a negative value for an invalid
 * argument (null pointer, non-positive size, k > E, unknown dtype). Buffers are
 * caller-owned host memory; nothing is allocated that outlives a call.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_ORACLE_F32 = 0, MOE_ORACLE_BF16 = 1 };

/* Flags of the _ex entry points. MOE_ORACLE_ACT_FP8: 8-bit activations in the
 * expert FFN (reading below, after the 8-bit weights). */
enum { MOE_ORACLE_ACT_FP8 = 1 };

/* Host description of one layer. Matrices are row-major:
 *   w_router [d][E], b_router [E] fp32 (NULL = zeros),
 *   w_gate, w_up [E][f][d], w_down [E][d][f].
 * dtype says how w_* and x are stored (fp32 values or bf16 bit patterns). */
typedef struct {
    int32_t d, f, E, k, dtype;
    const void* w_router;
    const float* b_router;
    const void* w_gate;
    const void* w_up;
    const void* w_down;
} moe_oracle_layer_t;

/* Exact widening of n elements of a tensor of the given dtype to fp32. */
int moe_oracle_widen(const void* src, int dtype, int64_t n, float* dst);

/* Router projection: logits [T][E] fp32 (the double sum rounded once). */
int moe_oracle_router(const moe_oracle_layer_t* L, const void* x, int32_t T, float* logits);

/* Top-k by (logit desc, index asc) and the renormalised softmax over the k
 * winners. ids [T][k] int32; w [T][k] fp32; w_f64 [T][k] (nullable). */
int moe_oracle_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                    int32_t* ids, float* w, double* w_f64);

/* Routing weights of given experts: for each token the softmax over the
 * logits of ids[t][0..k) renormalised, exponents shifted by the slot-0 logit
 * (the weights the top-k would give if these were its winners, in this slot
 * order). ids must lie in [0, E) (else -2). w [T][k] fp32; w_f64 nullable. */
int moe_oracle_route_weights(const float* logits, int32_t T, int32_t E, int32_t k,
                             const int32_t* ids, float* w, double* w_f64);

/* Stable counting sort of assignments (t, j) by expert ids[t*k+j].
 * counts [E], offsets [E+1], perm [T*k] token ids, perm_slot [T*k] slots,
 * inv [T*k]: inv[t*k+j] = position p of that assignment. Any output but
 * counts and offsets may be NULL. Fails if an id is outside [0, E). */
int moe_oracle_dispatch(const int32_t* ids, int32_t T, int32_t k, int32_t E,
                        int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* perm_slot, int32_t* inv);

/* FFN of expert e on one input row v [d] (dtype of the layer), in double:
 * out [d]. If h_out is not NULL it receives the f values of h. */
int moe_oracle_expert_ffn(const moe_oracle_layer_t* L, int32_t e, const void* v,
                          double* out, double* h_out);
int moe_oracle_expert_ffn_ex(const moe_oracle_layer_t* L, int32_t e, const void* v,
                             double* out, double* h_out, int32_t flags);

/* Whole layer for the tokens in token_list (NULL = all T tokens, in order).
 * Routing uses the oracle's own logits unless forced_ids [T][k] is given, in
 * which case those experts are used and their weights come from the oracle's
 * logits of those experts, taken in the forced slot order (slot 0 is the
 * reference of the exponent shift).
 *   y        [n][d] double, row r belongs to token token_list[r] (required)
 *   Y_slots  [n][k][d] double per-slot expert outputs (nullable)
 * Returns 0 or a negative error. Parallel over tokens with OpenMP; every
 * element's arithmetic is independent of the thread count. */
int moe_oracle_forward(const moe_oracle_layer_t* L, const void* x, int32_t T,
                       const int32_t* forced_ids, const int32_t* token_list, int32_t n,
                       double* y, double* Y_slots);
int moe_oracle_forward_ex(const moe_oracle_layer_t* L, const void* x, int32_t T,
                          const int32_t* forced_ids, const int32_t* token_list, int32_t n,
                          double* y, double* Y_slots, int32_t flags);

/* 8-bit expert weights («Colibri 是什么» (xxqk.cn) §4.2: the model converter can
 * quantize only the expert FFN weights, with 8 bits, keeping the router in full
 * precision). The pages fix neither the 8-bit format nor the scaling; the
 * reading implemented here:
 *   - format: OCP FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa
 *     bits; largest finite 448; 0x7f/0xff are NaN and never produced);
 *   - one scale per weight row (per output unit), a power of two 2^e with the
 *     smallest integer e such that max_i |w[r][i]| <= 448 * 2^e (e = 0 for an
 *     all-zero row; never below -126), so w * 2^-e is exact;
 *   - code = w * 2^-e rounded to the nearest E4M3 value, ties to the even
 *     mantissa; values below half the smallest subnormal (2^-10) give a
 *     signed zero (the sign bit follows the sign of w, -0 included).
 * The quantized layer is the same layer with every expert weight replaced by
 * its dequantized value code * 2^e, which a bf16 tensor holds exactly.
 * quantize: w [rows][cols] (dtype) -> codes [rows][cols], scales [rows] (2^e).
 * dequantize: codes, scales -> bf16 bit patterns; fails (returns -2) if a value
 * is not exactly representable in bf16. */
int moe_oracle_quantize_fp8(const void* w, int dtype, int64_t rows, int64_t cols,
                            uint8_t* codes, float* scales);
int moe_oracle_dequantize_fp8(const uint8_t* codes, const float* scales, int64_t rows,
                              int64_t cols, uint16_t* bf16_out);
/* Value of one E4M3 code (NaN for 0x7f/0xff). */
double moe_oracle_fp8_value(uint8_t code);

/* 8-bit activations (MOE_ORACLE_ACT_FP8): the pages store the expert weights
 * in 8 bits and say nothing of the activations; this optional mode reads the
 * roadmap's FP8 as an FP8 matrix product for the first expert GEMM, which
 * needs 8-bit inputs on both sides. Reading: the token row x[t] (as given,
 * per token; the router still sees the full-precision x) is quantized by the
 * rule above (E4M3, one power-of-two scale per row) before the gate and up
 * products; h and the down product keep the layer's precision (the weights'
 * dequantized values, h in double here). The products and sums are those of
 * the dequantized values, in double as always. */

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */
