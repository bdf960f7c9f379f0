// router.hip - fused router: projection, top-k and softmax over the winners.
//
// One launch computes, for a block of 16 tokens,
//   logits[t][e] = sum_i x[t][i] * W_r[i][e] + b_r[e]      (fp32 accumulation)
// then selects the k largest logits per token (equal logits -> lower expert
// index, slot 0 = largest) and the renormalised softmax over those k:
//   w[t][j] = exp(l_j - l_0) / sum_j' exp(l_j' - l_0).
// This is the router of «Colibri 是什么» (xxqk.cn) §3.2 (a linear projection plus
// router bias, then a top-k selection on the logits) fused the way
// «Colibri：面向MoE模型的高性能C语言推理引擎» (zskr.cn) §2.2 and
// «Colibri不是一只蜂鸟» (discosf.com) §5.1 describe (projection, softmax and
// top-k in one pass with the intermediates kept on chip). Selection only needs
// the order of the logits, so exponentials are taken for the k winners only.
//
// bf16 path: the projection runs on v_mfma_f32_16x16x32_bf16 (16 tokens x 16
// experts per MFMA; init stores the router weights as 1 KiB operand blocks,
// one per 16 experts and 32-wide K step, so that each B fragment is one
// contiguous load); the 16 waves of a block (8 for more than 128 experts)
// split the reduction dimension in interleaved 32-wide steps and add their
// partial sums through LDS in a fixed order, so results are bit-reproducible
// and do not depend on the number of tokens in the call.
// fp32 path: plain FMA dot products (gfx950 has no faster fp32 matrix rate).
#include "common.hpp"

namespace cmoe {

namespace {

constexpr int kTok = 16;     // tokens per block
constexpr int kThreads = 256;  // fp32 path

// Monotone map of a float to an unsigned key (larger float -> larger key).
// -0 is first turned into +0 so that the two zeros tie, as they compare equal.
__device__ __forceinline__ uint32_t order_key(float f)
{
    if (f == 0.0f)
        f = 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key (a -0 logit comes back as +0, which compares equal).
__device__ __forceinline__ float key_value(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// One step of the wave maximum: v and the value of the lane that the DPP
// control CTRL names (lanes outside ROW_MASK, or without a source lane, take
// 0, the smallest key).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false));
}

// Largest v over the wave, in a scalar register: within each row of 16 lanes
// by swaps of neighbours, of quads and of half rows, then across the rows by
// the row broadcasts of lane 15 and lane 31, so that lane 63 holds the
// maximum. (DPP moves data between lanes without an LDS round trip.)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = dpp_max<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_max<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_max<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_max<0x140, 0xF>(v);  // row_mirror: every lane holds its row's maximum
    v = dpp_max<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_max<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k + softmax for the block's bt tokens, reading logits (bias included)
// from LDS `lg` laid out [bt][ldl]. Wave w of W handles tokens w, w+W, ...;
// lane l holds the keys of experts l + 64q (q < NQ, NQ = ceil(E / 64) at
// most) and, once they are chosen, slot l's expert and logit (l < k), so
// that the k softmax weights are computed and stored by k lanes at once.
template <int NQ>
__device__ void topk_softmax_epilogue(const float* lg, int ldl, int bt, int t0, int T, int E, int k,
                                      int32_t* ids, float* wout)
{
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    for (int r = wv; r < bt; r += (int)blockDim.x / kWave) {
        const int t = t0 + r;
        if (t >= T)
            break;
        // Order keys of the token's logits (expert e = lane + 64q); an expert
        // not present, or already taken, has key 0, below every logit's key.
        // The largest key wins; among equal keys the lowest expert index.
        uint32_t key[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = lane + q * kWave;
            key[q] = e < E ? order_key(lg[r * ldl + e]) : 0u;
        }
        int my_id = 0;
        float my_l = 0.0f;
        for (int j = 0; j < k; ++j) {
            uint32_t best = key[0];
#pragma unroll
            for (int q = 1; q < NQ; ++q)
                best = max(best, key[q]);
            best = wave_max_u32(best);
            int e = E - 1;
#pragma unroll
            for (int q = NQ - 1; q >= 0; --q) {
                const uint64_t m = __ballot(key[q] == best && lane + q * kWave < E);
                if (m != 0)
                    e = q * kWave + __builtin_ctzll(m);
            }
            if (lane == j) {
                my_id = e;
                my_l = key_value(best);
            }
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (lane + q * kWave == e)
                    key[q] = 0u;
        }
        // w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), the sum taken in slot
        // order (the same value in every lane).
        const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
        const float ex = __expf(my_l - l0);
        float sum = 0.0f;
        for (int j = 0; j < k; ++j)
            sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
        const float inv = 1.0f / sum;
        if (lane < k) {
            ids[(int64_t)t * k + lane] = my_id;
            wout[(int64_t)t * k + lane] = ex * inv;
        }
    }
}

__device__ void store_logits(const float* lg, int ldl, int bt, int t0, int T, int E, float* logits)
{
    if (!logits)
        return;
    for (int i = threadIdx.x; i < bt * E; i += (int)blockDim.x) {
        const int r = i / E, e = i % E;
        if (t0 + r < T)
            logits[(int64_t)(t0 + r) * E + e] = lg[r * ldl + e];
    }
}

// NG = number of 16-expert column groups (E <= 16 * NG); TG = number of
// 16-token groups per block; W = waves per block, which split the reduction
// dimension. Each wave's loads form a chain of dependent batches (one memory
// round trip each, and the router's inputs are usually cold: the expert GEMMs
// stream gigabytes through the caches between two calls), so W is as large as
// the register budget allows: 16 waves (8 for 256 experts). A token's logits
// do not depend on T or TG: every token is reduced by the same interleaving
// of K over the W waves and the same LDS summation order.
template <int NG, int TG, int W>
__global__ __launch_bounds__(W * kWave) void router_bf16_kernel(RouterArgs a)
{
    constexpr int EP = 16 * NG;      // padded expert count
    constexpr int LDL = EP + 1;      // LDS row stride (floats)
    constexpr int BT = kTok * TG;    // tokens per block
    __shared__ float part[BT][LDL];

    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int t0 = blockIdx.x * BT;
    const int d = a.d;

    // A fragment rows: token rows, clamped (padded rows read valid memory and
    // their results are dropped); B fragments: whole blocks of the blocked
    // router weights (experts past E are zero rows there).
    const int kq = (lane >> 4) * 8;
    const uint16_t* xr[TG];
#pragma unroll
    for (int g = 0; g < TG; ++g)
        xr[g] = (const uint16_t*)a.x + (int64_t)min(t0 + g * kTok + (lane & 15), a.T - 1) * d + kq;
    // Router weights in MFMA operand blocks: the fragment of expert group n at
    // K step s is the 1 KiB block n * steps + s, lane l's 16 bytes at l*16.
    const int steps = d / 32;
    const Vec16* wb = (const Vec16*)a.w_rt + lane;

    floatx4 acc[TG][NG];
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
        for (int n = 0; n < NG; ++n)
            acc[g][n] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Wave w takes steps w, w+W, w+2W, ... in order; the loads of U of its
    // steps are issued before their MFMAs. The summation order does not
    // depend on U. Past the last step a batch reloads the last step with a
    // zero token fragment (adding exact zeros), so that every MFMA and every
    // load is unconditional: a step under a branch lets the compiler move its
    // loads into the branch and wait for each of them there.
    constexpr int U = NG * TG >= 8 ? 1 : 8 / (NG * TG);
    for (int s0 = wv; s0 < steps; s0 += W * U) {
        Vec16 av[U][TG], bv[U][NG];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int st = min(s0 + W * u, steps - 1);
#pragma unroll
            for (int g = 0; g < TG; ++g)
                av[u][g] = *(const Vec16*)(xr[g] + st * 32);
#pragma unroll
            for (int n = 0; n < NG; ++n)
                bv[u][n] = wb[(int64_t)(n * steps + st) * kWave];
        }
        __builtin_amdgcn_sched_barrier(0);  // all loads of the batch first
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool past = s0 + W * u >= steps;  // wave-uniform
#pragma unroll
            for (int g = 0; g < TG; ++g) {
                const Vec16 z = {0u, 0u, 0u, 0u};
                const Vec16 a_ = past ? z : av[u][g];
#pragma unroll
                for (int n = 0; n < NG; ++n)
                    acc[g][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a_), as_bf16x8(bv[u][n]), acc[g][n],
                                                                        0, 0, 0);
            }
        }
    }

    // D layout of a 16x16 MFMA: lane holds rows 4*(lane/16)+i, column lane%16.
    // The W partial sums are added in wave order (((w0 + w1) + w2) + ...):
    // groups of up to 8 waves store their partials to LDS side by side, then
    // every thread adds the group's partials of its elements in wave order.
    constexpr int WG = W < 8 ? W : 8;
    constexpr int NE = BT * EP;                       // logits of the block (padded)
    constexpr int NS = (NE + W * kWave - 1) / (W * kWave);  // elements per thread
    __shared__ float red[WG][NE];
    float sum[NS];
    for (int wg = 0; wg < W; wg += WG) {
        if (wv >= wg && wv < wg + WG) {
            float* dst = red[wv - wg];
#pragma unroll
            for (int g = 0; g < TG; ++g)
#pragma unroll
                for (int n = 0; n < NG; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[(g * kTok + (lane >> 4) * 4 + i) * EP + n * 16 + (lane & 15)] = acc[g][n][i];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int idx = threadIdx.x + j * W * kWave;
            if (idx < NE) {
#pragma unroll
                for (int w = 0; w < WG; ++w)
                    sum[j] = (wg + w == 0) ? red[w][idx] : sum[j] + red[w][idx];
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int idx = threadIdx.x + j * W * kWave;
        const int e = idx % EP;
        if (idx < NE)
            part[idx / EP][e] = e < a.E ? sum[j] + a.b[e] : sum[j];  // then the bias
    }
    __syncthreads();
    store_logits(&part[0][0], LDL, BT, t0, a.T, a.E, a.logits);
    topk_softmax_epilogue<(EP + kWave - 1) / kWave>(&part[0][0], LDL, BT, t0, a.T, a.E, a.k, a.ids, a.w);
}

__global__ __launch_bounds__(kThreads) void router_f32_kernel(RouterArgs a)
{
    __shared__ float lg[kTok][kMaxExperts + 1];
    const int t0 = blockIdx.x * kTok;
    const float* x = (const float*)a.x;
    const float* wt = (const float*)a.w_rt;
    for (int i = threadIdx.x; i < kTok * a.E; i += kThreads) {
        const int r = i / a.E, e = i % a.E;
        const int t = min(t0 + r, a.T - 1);
        const float* xr = x + (int64_t)t * a.d;
        const float* wr = wt + (int64_t)e * a.d;
        float s = 0.0f;
        for (int c = 0; c < a.d; ++c)
            s = fmaf(xr[c], wr[c], s);
        lg[r][e] = s + a.b[e];
    }
    __syncthreads();
    store_logits(&lg[0][0], kMaxExperts + 1, kTok, t0, a.T, a.E, a.logits);
    topk_softmax_epilogue<kMaxExperts / kWave>(&lg[0][0], kMaxExperts + 1, kTok, t0, a.T, a.E, a.k, a.ids, a.w);
}

__global__ void transpose_router_kernel(const uint8_t* src, uint8_t* dst, int d, int E, int esize)
{
    // dst[e][i] = src[i][e]
    const int64_t n = (int64_t)d * E;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = idx / d, i = idx % d;
        const uint8_t* s = src + (i * E + e) * esize;
        uint8_t* o = dst + idx * esize;
        for (int b = 0; b < esize; ++b)
            o[b] = s[b];
    }
}

// Groups of 16 experts the bf16 router kernel multiplies (its NG).
int router_groups(int E)
{
    return E <= 16 ? 1 : E <= 32 ? 2 : E <= 64 ? 4 : E <= 128 ? 8 : 16;
}

// bf16 router weights [d][E] -> MFMA operand blocks for router_groups(E)
// groups of 16 experts (the layout router_weight_bytes sizes).
__global__ void block_router_kernel(const uint16_t* src, uint16_t* dst, int d, int E, int groups)
{
    const int steps = d / 32;
    const int64_t n = (int64_t)groups * steps * 512;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int j = (int)(idx & 7), lane = (int)((idx >> 3) & 63);
        const int64_t blk = idx >> 9;
        const int st = (int)(blk % steps), g = (int)(blk / steps);
        const int e = g * 16 + (lane & 15), i = st * 32 + (lane >> 4) * 8 + j;
        dst[idx] = e < E ? src[(int64_t)i * E + e] : (uint16_t)0;
    }
}

template <int NG, int TG>
hipError_t launch_router_tg(const RouterArgs& a, hipStream_t s)
{
    constexpr int W = NG >= 16 ? 8 : 16;  // 16 waves need <= 128 registers
    const int bt = kTok * TG;
    hipLaunchKernelGGL((router_bf16_kernel<NG, TG, W>), dim3((a.T + bt - 1) / bt), dim3(W * kWave), 0, s, a);
    return hipGetLastError();
}

// Token groups per block: with many experts and many tokens, blocks of 32
// (128 experts) or 64 tokens (64 experts) read the router weights fewer
// times (measured on MI355X: 16384 tokens x 64 experts 99 -> 68 us, 8192 x 128
// 58 -> 46 us); with few tokens or experts, 16-token blocks keep more blocks
// in flight.
template <int NG>
hipError_t launch_router_ng(const RouterArgs& a, hipStream_t s)
{
    if constexpr (NG == 4 || NG == 8) {
        if (a.T >= 4096)
            return launch_router_tg<NG, NG == 4 ? 4 : 2>(a, s);
    }
    return launch_router_tg<NG, 1>(a, s);
}

}  // namespace

hipError_t launch_router_bf16(const RouterArgs& a, hipStream_t s)
{
    // NG = router_groups(E): the weight blocks hold exactly that many groups
    switch (router_groups(a.E)) {
    case 1:
        return launch_router_ng<1>(a, s);
    case 2:
        return launch_router_ng<2>(a, s);
    case 4:
        return launch_router_ng<4>(a, s);
    case 8:
        return launch_router_ng<8>(a, s);
    default:
        return launch_router_ng<16>(a, s);
    }
}

hipError_t launch_router_f32(const RouterArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(router_f32_kernel, dim3((a.T + kTok - 1) / kTok), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

size_t router_weight_bytes(int d, int E, int esize)
{
    return esize == 2 ? (size_t)router_groups(E) * 16 * d * 2 : (size_t)E * d * esize;
}

hipError_t launch_transpose_router(const void* w_r, void* w_rt, int d, int E, int esize, hipStream_t s)
{
    if (esize == 2)
        hipLaunchKernelGGL(block_router_kernel, dim3(256), dim3(256), 0, s, (const uint16_t*)w_r, (uint16_t*)w_rt,
                           d, E, router_groups(E));
    else
        hipLaunchKernelGGL(transpose_router_kernel, dim3(256), dim3(256), 0, s, (const uint8_t*)w_r,
                           (uint8_t*)w_rt, d, E, esize);
    return hipGetLastError();
}

}  // namespace cmoe
