/*
 * colibri_moe.h - C ABI of one Mixture-of-Experts FFN layer on an MI355X (gfx950).
 *
 * The layer (the computation the Colibri engine pages describe: «Colibri 是什么»
 * (xxqk.cn) §2.1 and §2.3; «Colibri：面向MoE模型的高性能C语言推理引擎»
 * (zskr.cn) §1 and §3.3):
 *
 *   logits[t][e] = sum_i x[t][i] * W_r[i][e] + b_r[e]                 (fp32)
 *   TopK(t)      = the k largest logits, equal logits -> lower expert index,
 *                  slot 0 = largest
 *   w[t][j]      = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0)       (softmax over the winners)
 *   y[t]         = sum_j w[t][j] * W_down[e] (SiLU(W_gate[e] x[t]) .* (W_up[e] x[t])),  e = ids[t][j]
 *
 * computed on the GPU as: fused router (projection + top-k + softmax), dispatch
 * (histogram, prefix sum, stable permutation by expert), grouped gate/up GEMM
 * with a SiLU*up epilogue, grouped down GEMM, weighted combine. Experts that
 * receive no token get no GEMM tiles and their weights are not read.
 *
 * Shape of the API: init / forward / free with a status code and a status
 * string, as the pages' host interface has it (init, infer, free in
 * «Colibri 是什么» (xxqk.cn) §2.3; the status enum, status string, fixed
 * expert count and top-k at init, and device-resident caller buffers in
 * «Colibri不是一只蜂鸟» (discosf.com) §4.4 and §6.1). All library memory is
 * allocated once by init («Colibri不是一只蜂鸟» (discosf.com) §3.1); forward
 * allocates nothing.
 *
 * Conventions
 *  - Every tensor pointer is a DEVICE pointer on the device that was current at
 *    init. Matrices are row-major, dense, no padding.
 *  - dtype BF16: x, y and all weights are bf16 (raw 16-bit patterns); the router
 *    bias is fp32; logits, routing weights and all accumulation are fp32.
 *    dtype F32: everything fp32.
 *  - The caller owns x, y, the weights it passes to init and every routing_out
 *    buffer. Init copies (and repacks) the weights into library memory, so the
 *    caller may free its weight buffers after init returns.
 *  - Forward runs on the stream given at init (NULL = the default stream). It
 *    is synchronous (returns when the GPU is done) unless COLIBRI_MOE_FLAG_ASYNC
 *    is set, in which case it returns after enqueueing. A handle serves one
 *    stream; calls on one handle must not overlap.
 *  - On a non-OK return, outputs are undefined.
 *
 * 8-bit expert weights (COLIBRI_MOE_FLAG_FP8_WEIGHTS, bf16 layers only): the
 * pages' converter may store the expert FFN weights alone in 8 bits while the
 * router keeps full precision («Colibri 是什么» (xxqk.cn) §4.2). The pages fix
 * no format; this library uses OCP FP8 E4M3 codes with one power-of-two scale
 * per weight row (per output unit of the gate, up and down projections):
 * scale = 2^e with the smallest integer e (>= -126) such that the row's
 * largest magnitude is at most 448 * 2^e (e = 0 for an all-zero row), code =
 * w / scale rounded to the nearest E4M3 value, ties to even mantissa, zero
 * keeping the sign. Init quantizes the bf16 weights it is given; forward then
 * computes the layer of the dequantized weights (code value * scale, exact in
 * bf16) with bf16 activations and fp32 accumulation, reading half the weight
 * bytes of the bf16 layer.
 *
 * 8-bit activations (COLIBRI_MOE_FLAG_FP8_ACTIVATIONS, on top of FP8_WEIGHTS):
 * the roadmap's FP8 read as an FP8 matrix product for the first expert GEMM.
 * Each token row x[t] is quantized by the same rule (E4M3, one power-of-two
 * scale per row; the router still sees the full x), and the gate/up GEMM
 * multiplies E4M3 by E4M3 on gfx950's fp8 MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4, the scales applied as E8M0 exponents),
 * exact products summed in fp32. h stays bf16 and the down GEMM is the 8-bit
 * weight one. With stage timing, stage 1 includes the x quantization.
 */
#ifndef COLIBRI_MOE_H
#define COLIBRI_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    COLIBRI_MOE_OK = 0,
    COLIBRI_MOE_ERR_INVALID_ARG = 1,  /* null where required, T < 0 or > max_tokens, k < 1 or > E, bad dtype */
    COLIBRI_MOE_ERR_UNSUPPORTED = 2,  /* d_model not a multiple of 128, d_ff not a multiple of 128
                                         (bf16) or 64 (f32), E > 256, k > 8, max_tokens > 2^24,
                                         max_tokens*k*d_ff, max_tokens*d_model or
                                         2*d_ff*d_model reaching 2^31, FP8_WEIGHTS with
                                         dtype F32, FP8_ACTIVATIONS without FP8_WEIGHTS
                                         or with d_model or d_ff below 256 */
    COLIBRI_MOE_ERR_ALIGNMENT = 3,    /* x, y, a weight or topk_ids not 16-byte aligned, another
                                         routing buffer or b_router not 4-byte aligned */
    COLIBRI_MOE_ERR_OUT_OF_MEMORY = 4,/* init could not allocate its memory */
    COLIBRI_MOE_ERR_HIP = 5,          /* a HIP launch, copy or sync failed */
    COLIBRI_MOE_ERR_TOO_LARGE = 6     /* colibri_moe_forward_static: the call's working memory
                                         exceeds COLIBRI_MOE_STATIC_SCRATCH_BYTES */
} colibri_moe_status_t;

/* Size of the static working-memory array of colibri_moe_forward_static, one
 * per GPU the library runs on (64 MiB). */
#define COLIBRI_MOE_STATIC_SCRATCH_BYTES (64 << 20)

typedef enum { COLIBRI_MOE_F32 = 0, COLIBRI_MOE_BF16 = 1 } colibri_moe_dtype_t;

enum {
    COLIBRI_MOE_FLAG_ASYNC = 1u << 0,       /* forward returns after enqueueing */
    COLIBRI_MOE_FLAG_STAGE_TIMING = 1u << 1, /* record per-stage GPU times (hipEvents) */
    COLIBRI_MOE_FLAG_FP8_WEIGHTS = 1u << 2,  /* bf16 only: keep expert weights as 8-bit codes
                                                (format above) */
    COLIBRI_MOE_FLAG_FP8_ACTIVATIONS = 1u << 3 /* with FP8_WEIGHTS, d_model and d_ff >= 256:
                                                  8-bit token rows, fp8 MFMA gate/up GEMM (above) */
};

typedef struct {
    int32_t d_model;     /* d: token width */
    int32_t d_ff;        /* f: expert hidden width */
    int32_t n_experts;   /* E, 1..256 */
    int32_t top_k;       /* k, 1..min(8, E) */
    int32_t max_tokens;  /* largest T forward will accept; sizes the workspace */
    colibri_moe_dtype_t dtype;
    uint32_t flags;      /* COLIBRI_MOE_FLAG_* */
} colibri_moe_config_t;

/* Device pointers, read only during init (copied and repacked). */
typedef struct {
    const void* w_router;  /* [d_model][E], dtype */
    const float* b_router; /* [E] fp32, or NULL for zeros */
    const void* w_gate;    /* [E][d_ff][d_model], dtype */
    const void* w_up;      /* [E][d_ff][d_model], dtype */
    const void* w_down;    /* [E][d_model][d_ff], dtype */
} colibri_moe_weights_t;

/* Optional routing outputs of forward, caller-owned device buffers; any field
 * may be NULL (then that output is not written). A = T * k assignments,
 * assignment a = t * k + j is slot j of token t. */
typedef struct {
    float* logits;          /* [T][E] fp32 router logits (bias included) */
    int32_t* topk_ids;      /* [T][k] selected experts, slot 0 = largest logit; 16-byte aligned
                               (the other fields: 4-byte aligned), else ERR_ALIGNMENT */
    float* topk_w;          /* [T][k] routing weights, sum to 1 per token */
    int32_t* expert_counts; /* [E] assignments per expert */
    int32_t* expert_offsets;/* [E+1] exclusive prefix sum of counts */
    int32_t* perm;          /* [A] token of sorted position p (segments by expert, tokens ascending) */
    int32_t* perm_slot;     /* [A] slot j of sorted position p */
    int32_t* inv;           /* [A] inv[t*k+j] = sorted position of assignment (t, j) */
} colibri_moe_routing_t;

typedef struct colibri_moe colibri_moe_t; /* opaque handle */

/* Validate cfg, allocate all device memory for max_tokens, copy and repack the
 * weights, synchronize. hip_stream is a hipStream_t (NULL = default stream)
 * used by every later forward. On success *out receives the handle. */
colibri_moe_status_t colibri_moe_init(colibri_moe_t** out, const colibri_moe_config_t* cfg,
                                      const colibri_moe_weights_t* w, void* hip_stream);

/* y [T][d_model] = MoE layer of x [T][d_model]. T = 0 returns OK and does
 * nothing. routing_out may be NULL. Allocates nothing. */
colibri_moe_status_t colibri_moe_forward(colibri_moe_t* h, const void* x, int32_t T, void* y,
                                         const colibri_moe_routing_t* routing_out);

/* colibri_moe_forward for callers that cannot allocate device memory at all
 * (work under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, checks and results (y and every routing
 * output bit-identical to colibri_moe_forward's), but the call's working
 * memory (routing buffers the caller does not supply, H, the fp32 partial
 * sums) lives in one static device array of COLIBRI_MOE_STATIC_SCRATCH_BYTES
 * in the library, one per GPU, held until the process ends, instead of the
 * handle's workspace. It allocates nothing and needs no clearing: every kernel
 * writes what the next one reads. A call whose working memory does not fit
 * returns COLIBRI_MOE_ERR_TOO_LARGE before enqueueing anything (bf16 layers:
 * about (k * (2*d_ff + 8*d_model + 16)) bytes per token plus the small-batch
 * K-slice partials; the Mixtral-shaped layer fits 500 tokens). Every call on
 * one GPU uses that GPU's array, whichever handle makes it: calls that
 * overlap on one GPU (several streams, threads or handles) race, and the
 * caller must order them. The combine always runs as its own kernel here.
 * ERR_HIP if the array's device address could not be found at init. */
colibri_moe_status_t colibri_moe_forward_static(colibri_moe_t* h, const void* x, int32_t T, void* y,
                                                const colibri_moe_routing_t* routing_out);

/* Release everything init allocated (waits for the handle's stream first).
 * NULL is a no-op. The library keeps a registry of live handles: forward and
 * free reject a pointer that is not a live handle (never created, or already
 * freed) with INVALID_ARG instead of touching it. */
colibri_moe_status_t colibri_moe_free(colibri_moe_t* h);

/* The 8-bit codes init stores for bf16 weight rows under
 * COLIBRI_MOE_FLAG_FP8_WEIGHTS (format in the header comment; «Colibri 是什么»
 * (xxqk.cn) §4.2), row-major: for w [rows][cols] bf16, codes [rows][cols]
 * E4M3 bytes and scales [rows] fp32 (powers of two), so that w[r][c] is
 * approximated by value(codes[r][c]) * scales[r]. All three are caller-owned
 * DEVICE buffers; w must be 16-byte and codes 8-byte aligned. rows >= 1,
 * cols >= 8 and a multiple of 8, rows * cols < 2^40; otherwise INVALID_ARG.
 * Runs on hip_stream (NULL = default stream) and returns when it is done.
 * Needs no handle. */
colibri_moe_status_t colibri_moe_quantize_fp8(const void* w, int64_t rows, int64_t cols, uint8_t* codes,
                                              float* scales, void* hip_stream);

/* Measurement helper, not a step of the layer: copies `bytes` bytes from src
 * to dst (caller-owned DEVICE buffers, 16-byte aligned, not overlapping;
 * bytes a multiple of 16, at least 16) with the library's streaming copy
 * kernel on hip_stream (NULL = default stream), and returns without waiting
 * (time it with events on that stream). It states the HBM rate the chip
 * reaches on plain streaming traffic beside the nominal peak, and a copy of
 * known size scales the rocprofv3 byte counters. INVALID_ARG or ALIGNMENT
 * otherwise; HIP if the launch fails. Needs no handle. */
colibri_moe_status_t colibri_moe_stream_copy(const void* src, void* dst, int64_t bytes, void* hip_stream);

/* Static text for a status value. */
const char* colibri_moe_status_string(colibri_moe_status_t s);

/* Stage names and GPU times (ms) of the last forward when the handle was
 * created with COLIBRI_MOE_FLAG_STAGE_TIMING (waits for that forward to
 * finish). Stages: 0 router, 1 dispatch, 2 gate/up GEMM, 3 gate/up reduce
 * (the K-slice sum and SiLU of the small-batch path; empty otherwise),
 * 4 down GEMM, 5 combine. Writes min(n, 6) values; returns the number of
 * stages. */
int32_t colibri_moe_stage_times(colibri_moe_t* h, float* ms, int32_t n);
const char* colibri_moe_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif

#endif /* COLIBRI_MOE_H */
