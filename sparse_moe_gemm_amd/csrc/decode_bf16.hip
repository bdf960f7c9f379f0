// decode_bf16.hip - expert GEMMs of bf16 layers for small token counts.
//
// The same two expert GEMMs as gemm_bf16.hip (the per-expert SwiGLU FFN of
// «Colibri 是什么» (xxqk.cn) §2.3, batched over the active experts as in
// «Colibri不是一只蜂鸟» (discosf.com) §3.2), for steps where every active expert
// holds only a few tokens, as when generating one token per sequence. There the
// work is reading each active expert's weights once: the MFMA work is tiny, and
// a 256-row output tile would spend most of its matrix time on rows that do not
// exist. So this path has no LDS and no barriers at all:
//   - a work item is (expert e, two 32-row weight blocks nb and nb+1, K
//     slice s); every wave takes items w, w + W, ... (W = waves in the grid)
//     on its own;
//   - for the expert's tokens, 32-row groups taken two at a time, it
//     multiplies the tokens' K slice (A fragments, through perm for gate/up;
//     each one feeds both blocks) with the two weight blocks (B fragments,
//     fetched straight into registers from the blocked MFMA layout, each one
//     feeding both token groups) with v_mfma_f32_32x32x16_bf16, P k-steps of
//     loads in flight ahead of the MFMAs (plain loads, so the compiler's wait
//     counts are exact); an expert with up to 64 rows streams its weights
//     once;
//   - it writes the fp32 partial sums of its slice: P[s][p][nb*32 + j].
// K slices split every expert's weights into many equal, independent items,
// which keeps all compute units streaming. Weights are read with
// non-temporal loads: each is used once per call, and not keeping them in
// the caches streams them ~5-7% faster. A gate/up GEMM without K slices
// applies SiLU(g)*u to its items' own sums and writes H directly; with slices
// a second kernel sums them and applies SiLU(g)*u into H. For down the slices
// are the Ys partials that combine already sums.
// With 8-bit expert weights (E4M3 codes in the fp8 blocked layout, one scale
// per weight row) the same items step through K 32 at a time: per step and
// weight block one 1 KiB block of codes (one 16-byte load per lane: its B
// fragments of the step's two 16-wide MFMA k steps), turned into exact bf16
// (code times the row scale) in registers; the bytes read per weight are
// halved, the arithmetic is the bf16 path's.
#include "common.hpp"

namespace cmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kP = 4;  // k-steps of loads in flight per wave and register set (two sets)

// Results of one item for its token group r0 .. r0+31 (32x32 MFMA D layout:
// lane holds column lane%32 and rows 8*(q/4) + 4*(lane/32) + q%4): the fp32
// slice partials of its two weight blocks at out (row stride N), or, for a
// gate/up item that covers the whole K (g.h set, no slices), H itself: blocks
// nb and nb+1 are the gate and up rows of H columns 16*nb .. +32, and
// H = bf16(SiLU(g)*u), the same values the slice-sum pass computes from one
// slice.
template <bool GATE_UP>
__device__ __forceinline__ void store_item(const DecodeArgs& g, float* out, int N, int seg0, int r0, int cnt, int nb,
                                           int lane, const floatx16& acc0, const floatx16& acc1)
{
    if (GATE_UP && g.h != nullptr) {
        uint16_t* hcol = g.h + nb * 16 + (lane & 31);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = r0 + 8 * (q / 4) + 4 * (lane >> 5) + (q % 4);
            if (row < cnt)
                hcol[(int64_t)(seg0 + row) * g.f] = f32_to_bf16_bits(silu(acc0[q]) * acc1[q]);
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int row = r0 + 8 * (q / 4) + 4 * (lane >> 5) + (q % 4);
        if (row < cnt) {
            out[(int64_t)(seg0 + row) * N] = acc0[q];
            out[(int64_t)(seg0 + row) * N + 32] = acc1[q];
        }
    }
}

// One pass of an item's K slice over G consecutive 32-token groups of the
// expert, from row r0 on: every weight fragment fetched feeds the MFMAs of
// all G groups, so an expert with up to 32*G rows streams its weight blocks
// once. Each group's accumulators see the same MFMA sequence as in a pass of
// its own (the results do not depend on G).
template <bool GATE_UP, int G>
__device__ __forceinline__ void decode_pass(const DecodeArgs& g, const Vec16* bp, int64_t bst, float* out, int N, int K,
                                            int seg0, int r0, int cnt, int nb, int kb0, int kb1, int lane)
{
    static_assert(G == 1 || G == 2, "one or two token groups per pass");
    const Vec16* ap[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        const int r = min(r0 + 32 * gi + (lane & 31), cnt - 1);
        const int src = GATE_UP ? g.perm[seg0 + r] : seg0 + r;
        ap[gi] = (const Vec16*)((const uint16_t*)g.a + (int64_t)src * K) + (lane >> 5);
    }
    // accumulators as named values (group, weight block): the conditional
    // MFMAs below then update them in place, with no copies between blocks
    floatx16 acc00, acc01, acc10, acc11;
#pragma unroll
    for (int q = 0; q < 16; ++q)
        acc00[q] = acc01[q] = acc10[q] = acc11[q] = 0.f;
    Vec16 a0[G][kP], b0[kP], c0[kP], a1[G][kP], b1[kP], c1[kP];
    auto mfma4 = [&](const Vec16 (&a)[G][kP], const Vec16& b, const Vec16& c, int i) {
        acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[0][i]), as_bf16x8(b), acc00, 0, 0, 0);
        acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[0][i]), as_bf16x8(c), acc01, 0, 0, 0);
        if constexpr (G == 2) {
            acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[G - 1][i]), as_bf16x8(b), acc10, 0, 0, 0);
            acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[G - 1][i]), as_bf16x8(c), acc11, 0, 0, 0);
        }
    };
#pragma unroll
    for (int i = 0; i < kP; ++i) {
        const int kb = min(kb0 + i, kb1 - 1);
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
            a0[gi][i] = ap[gi][kb * 2];
        b0[i] = __builtin_nontemporal_load(&bp[(int64_t)kb * kWave]);
        c0[i] = __builtin_nontemporal_load(&bp[bst + (int64_t)kb * kWave]);
    }
    for (int kb = kb0; kb < kb1; kb += 2 * kP) {
#pragma unroll
        for (int i = 0; i < kP; ++i) {
            const int kk = min(kb + kP + i, kb1 - 1);
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
                a1[gi][i] = ap[gi][kk * 2];
            b1[i] = __builtin_nontemporal_load(&bp[(int64_t)kk * kWave]);
            c1[i] = __builtin_nontemporal_load(&bp[bst + (int64_t)kk * kWave]);
        }
#pragma unroll
        for (int i = 0; i < kP; ++i)
            if (kb + i < kb1)
                mfma4(a0, b0[i], c0[i], i);
#pragma unroll
        for (int i = 0; i < kP; ++i) {
            const int kk = min(kb + 2 * kP + i, kb1 - 1);
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
                a0[gi][i] = ap[gi][kk * 2];
            b0[i] = __builtin_nontemporal_load(&bp[(int64_t)kk * kWave]);
            c0[i] = __builtin_nontemporal_load(&bp[bst + (int64_t)kk * kWave]);
        }
#pragma unroll
        for (int i = 0; i < kP; ++i)
            if (kb + kP + i < kb1)
                mfma4(a1, b1[i], c1[i], i);
    }
    store_item<GATE_UP>(g, out, N, seg0, r0, cnt, nb, lane, acc00, acc01);
    if constexpr (G == 2)
        store_item<GATE_UP>(g, out, N, seg0, r0 + 32, cnt, nb, lane, acc10, acc11);
}

// GMAX: token groups per weight pass, at most (1 for calls whose experts
// hold at most 32 rows each, where the pair code would only cost)
template <bool GATE_UP, int GMAX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_gemm_kernel(DecodeArgs g)
{
    constexpr bool gate_up = GATE_UP;
    if (g.gate_rows > 0 && max_expert_rows(g.offsets, g.E) > g.gate_rows)
        return;  // the tiled kernels take this call
    const int lane = threadIdx.x % kWave;
    const int W = gridDim.x * (kThreads / kWave);
    const int w0 = blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int N = gate_up ? 2 * g.f : g.d;
    const int K = gate_up ? g.d : g.f;
    const int NB = N / 32, KB = K / 16, S = g.split;
    const int NB2 = NB / 2;  // items cover two weight blocks
    const int items = g.E * NB2 * S;
    const Vec16* B = (const Vec16*)g.b;

    for (int it = w0; it < items; it += W) {
        const int s = it % S;
        const int rest = it / S;
        const int nb = (rest % NB2) * 2;
        const int e = rest / NB2;
        const int seg0 = g.offsets[e];
        const int cnt = g.offsets[e + 1] - seg0;
        if (cnt <= 0)
            continue;
        const int kb0 = (int)((int64_t)s * KB / S), kb1 = (int)((int64_t)(s + 1) * KB / S);
        const Vec16* bp = B + ((int64_t)e * NB + nb) * KB * kWave + lane;
        const int64_t bst = (int64_t)KB * kWave;  // next weight block
        float* out = g.part + (int64_t)s * g.A * N + nb * 32 + (lane & 31);

        // token groups in pairs (one weight pass per 64 rows), a last single
        // group where at most 32 rows remain
        for (int r0 = 0; r0 < cnt; r0 += 32 * GMAX) {
            if constexpr (GMAX == 2) {
                if (cnt - r0 > 32) {
                    decode_pass<gate_up, 2>(g, bp, bst, out, N, K, seg0, r0, cnt, nb, kb0, kb1, lane);
                    continue;
                }
            }
            decode_pass<gate_up, 1>(g, bp, bst, out, N, K, seg0, r0, cnt, nb, kb0, kb1, lane);
        }
    }
}

template <bool GATE_UP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_gemm_f8_kernel(DecodeArgs g)
{
    constexpr bool gate_up = GATE_UP;
    constexpr int kQ = 4;  // 32-wide k steps of loads in flight per wave (two sets)
    if (g.gate_rows > 0 && max_expert_rows(g.offsets, g.E) > g.gate_rows)
        return;  // the tiled kernels take this call
    const int lane = threadIdx.x % kWave;
    const int W = gridDim.x * (kThreads / kWave);
    const int w0 = blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int N = gate_up ? 2 * g.f : g.d;
    const int K = gate_up ? g.d : g.f;
    const int NB = N / 32, KB = K / 32, S = g.split;
    const int NB2 = NB / 2;
    const int items = g.E * NB2 * S;
    const Vec16* B = (const Vec16*)g.b;
    const uint16_t* Abase = (const uint16_t*)g.a;

    for (int it = w0; it < items; it += W) {
        const int s = it % S;
        const int rest = it / S;
        const int nb = (rest % NB2) * 2;
        const int e = rest / NB2;
        const int seg0 = g.offsets[e];
        const int cnt = g.offsets[e + 1] - seg0;
        if (cnt <= 0)
            continue;
        const int kb0 = (int)((int64_t)s * KB / S), kb1 = (int)((int64_t)(s + 1) * KB / S);
        // lane's 16 bytes of k step kb of row block nb: both halves' codes
        const Vec16* bp = B + ((int64_t)e * NB + nb) * KB * kWave + lane;
        const int64_t bst = (int64_t)KB * kWave;  // next weight block
        const float s0 = g.scales[(int64_t)e * N + nb * 32 + (lane & 31)];
        const float s1 = g.scales[(int64_t)e * N + nb * 32 + 32 + (lane & 31)];
        float* out = g.part + (int64_t)s * g.A * N + nb * 32 + (lane & 31);

        for (int r0 = 0; r0 < cnt; r0 += 32) {
            const int r = min(r0 + (lane & 31), cnt - 1);
            const int src = gate_up ? g.perm[seg0 + r] : seg0 + r;
            // k order of the 8-bit weight layout: in 32-wide step kb, lane half
            // lane/32 holds k kb*32 + 16*(lane/32) .. +16, 8 per 16-wide k step
            // h; the activations are read in the same order (Vec16 kb*4 + h
            // from the lane half's base)
            const Vec16* ap = (const Vec16*)(Abase + (int64_t)src * K) + 2 * (lane >> 5);
            floatx16 acc0, acc1;
#pragma unroll
            for (int q = 0; q < 16; ++q)
                acc0[q] = acc1[q] = 0.f;
            Vec16 a0[kQ][2], a1[kQ][2];
            Vec16 b0[kQ], c0[kQ], b1[kQ], c1[kQ];
#pragma unroll
            for (int i = 0; i < kQ; ++i) {
                const int kb = min(kb0 + i, kb1 - 1);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    a0[i][h] = ap[kb * 4 + h];
                b0[i] = __builtin_nontemporal_load(&bp[(int64_t)kb * kWave]);
                c0[i] = __builtin_nontemporal_load(&bp[bst + (int64_t)kb * kWave]);
            }
            for (int kb = kb0; kb < kb1; kb += 2 * kQ) {
#pragma unroll
                for (int i = 0; i < kQ; ++i) {
                    const int kk = min(kb + kQ + i, kb1 - 1);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        a1[i][h] = ap[kk * 4 + h];
                    b1[i] = __builtin_nontemporal_load(&bp[(int64_t)kk * kWave]);
                    c1[i] = __builtin_nontemporal_load(&bp[bst + (int64_t)kk * kWave]);
                }
#pragma unroll
                for (int i = 0; i < kQ; ++i)
                    if (kb + i < kb1) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const bf16x8 fa = as_bf16x8(a0[i][h]);
                            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fp8x8_to_bf16(b0[i][2 * h], b0[i][2 * h + 1], s0),
                                                                           acc0, 0, 0, 0);
                            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fp8x8_to_bf16(c0[i][2 * h], c0[i][2 * h + 1], s1),
                                                                           acc1, 0, 0, 0);
                        }
                    }
#pragma unroll
                for (int i = 0; i < kQ; ++i) {
                    const int kk = min(kb + 2 * kQ + i, kb1 - 1);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        a0[i][h] = ap[kk * 4 + h];
                    b0[i] = __builtin_nontemporal_load(&bp[(int64_t)kk * kWave]);
                    c0[i] = __builtin_nontemporal_load(&bp[bst + (int64_t)kk * kWave]);
                }
#pragma unroll
                for (int i = 0; i < kQ; ++i)
                    if (kb + kQ + i < kb1) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const bf16x8 fa = as_bf16x8(a1[i][h]);
                            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fp8x8_to_bf16(b1[i][2 * h], b1[i][2 * h + 1], s0),
                                                                           acc0, 0, 0, 0);
                            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fp8x8_to_bf16(c1[i][2 * h], c1[i][2 * h + 1], s1),
                                                                           acc1, 0, 0, 0);
                        }
                    }
            }
            store_item<gate_up>(g, out, N, seg0, r0, cnt, nb, lane, acc0, acc1);
        }
    }
}

// 8-bit weights and activations (W8A8): the same items in 64-wide k steps on
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, per-lane E8M0 scales). A lane
// takes, of each step, k 16*(l/32) .. +16 of both 32-k halves: activation
// chunks l/32 and 2 + l/32 of the row's 64 codes, and its 16 bytes of the two
// 1 KiB weight blocks of the step.
__device__ __forceinline__ int e8m0_byte(float s)
{
    return (int)((__float_as_uint(s) >> 23) & 0xFFu);
}

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i cat16(const Vec16& lo, const Vec16& hi)
{
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <bool GATE_UP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_gemm_q8_kernel(DecodeArgs g)
{
    constexpr bool gate_up = GATE_UP;
    constexpr int kQ = 3;  // 64-wide k steps of loads in flight per wave (two sets)
    if (g.gate_rows > 0 && max_expert_rows(g.offsets, g.E) > g.gate_rows)
        return;  // the tiled kernels take this call
    const int lane = threadIdx.x % kWave;
    const int W = gridDim.x * (kThreads / kWave);
    const int w0 = blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int N = gate_up ? 2 * g.f : g.d;
    const int K = gate_up ? g.d : g.f;
    const int NB = N / 32, KB = K / 64, KB32 = K / 32, S = g.split;
    const int NB2 = NB / 2;
    const int items = g.E * NB2 * S;
    const Vec16* B = (const Vec16*)g.b;
    const uint8_t* Abase = (const uint8_t*)g.a;

    for (int it = w0; it < items; it += W) {
        const int s = it % S;
        const int rest = it / S;
        const int nb = (rest % NB2) * 2;
        const int e = rest / NB2;
        const int seg0 = g.offsets[e];
        const int cnt = g.offsets[e + 1] - seg0;
        if (cnt <= 0)
            continue;
        const int kb0 = (int)((int64_t)s * KB / S), kb1 = (int)((int64_t)(s + 1) * KB / S);
        // lane's 16 bytes of 1 KiB block q of row block nb: bp[q * 64]
        const Vec16* bp = B + ((int64_t)e * NB + nb) * KB32 * kWave + lane;
        const int64_t bst = (int64_t)KB32 * kWave;  // next weight block
        const int sb0 = e8m0_byte(g.scales[(int64_t)e * N + nb * 32 + (lane & 31)]);
        const int sb1 = e8m0_byte(g.scales[(int64_t)e * N + nb * 32 + 32 + (lane & 31)]);
        float* out = g.part + (int64_t)s * g.A * N + nb * 32 + (lane & 31);

        for (int r0 = 0; r0 < cnt; r0 += 32) {
            const int r = min(r0 + (lane & 31), cnt - 1);
            const int src = gate_up ? g.perm[seg0 + r] : seg0 + r;
            const int sa = e8m0_byte(g.a_scales[seg0 + r]);
            // 16-byte chunk c of step kb of the row: ap[kb * 4 + c]
            const Vec16* ap = (const Vec16*)(Abase + (int64_t)src * K) + (lane >> 5);
            floatx16 acc0, acc1;
#pragma unroll
            for (int q = 0; q < 16; ++q)
                acc0[q] = acc1[q] = 0.f;
            Vec16 a0[kQ][2], b0[kQ][2], c0[kQ][2], a1[kQ][2], b1[kQ][2], c1[kQ][2];
#pragma unroll
            for (int i = 0; i < kQ; ++i) {
                const int kb = min(kb0 + i, kb1 - 1);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    a0[i][h] = ap[kb * 4 + 2 * h];
                    b0[i][h] = __builtin_nontemporal_load(&bp[(int64_t)(2 * kb + h) * kWave]);
                    c0[i][h] = __builtin_nontemporal_load(&bp[bst + (int64_t)(2 * kb + h) * kWave]);
                }
            }
            for (int kb = kb0; kb < kb1; kb += 2 * kQ) {
#pragma unroll
                for (int i = 0; i < kQ; ++i) {
                    const int kk = min(kb + kQ + i, kb1 - 1);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        a1[i][h] = ap[kk * 4 + 2 * h];
                        b1[i][h] = __builtin_nontemporal_load(&bp[(int64_t)(2 * kk + h) * kWave]);
                        c1[i][h] = __builtin_nontemporal_load(&bp[bst + (int64_t)(2 * kk + h) * kWave]);
                    }
                }
#pragma unroll
                for (int i = 0; i < kQ; ++i)
                    if (kb + i < kb1) {
                        const v8i fa = cat16(a0[i][0], a0[i][1]);
                        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, cat16(b0[i][0], b0[i][1]), acc0, 0, 0,
                                                                               0, sa, 0, sb0);
                        acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, cat16(c0[i][0], c0[i][1]), acc1, 0, 0,
                                                                               0, sa, 0, sb1);
                    }
#pragma unroll
                for (int i = 0; i < kQ; ++i) {
                    const int kk = min(kb + 2 * kQ + i, kb1 - 1);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        a0[i][h] = ap[kk * 4 + 2 * h];
                        b0[i][h] = __builtin_nontemporal_load(&bp[(int64_t)(2 * kk + h) * kWave]);
                        c0[i][h] = __builtin_nontemporal_load(&bp[bst + (int64_t)(2 * kk + h) * kWave]);
                    }
                }
#pragma unroll
                for (int i = 0; i < kQ; ++i)
                    if (kb + kQ + i < kb1) {
                        const v8i fa = cat16(a1[i][0], a1[i][1]);
                        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, cat16(b1[i][0], b1[i][1]), acc0, 0, 0,
                                                                               0, sa, 0, sb0);
                        acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, cat16(c1[i][0], c1[i][1]), acc1, 0, 0,
                                                                               0, sa, 0, sb1);
                    }
            }
            store_item<gate_up>(g, out, N, seg0, r0, cnt, nb, lane, acc0, acc1);
        }
    }
}

// H[p][c] = bf16(SiLU(sum_s P[s][p][gate row of c]) * sum_s P[s][p][up row of c]),
// with gate/up interleaved by 32 rows: h column c is gate row (c/32)*64 + c%32
// and up row (c/32)*64 + 32 + c%32 of the combined [2f] weight rows. Four
// consecutive columns per thread, slices summed in order.
__global__ __launch_bounds__(256) void decode_silu_kernel(const float* part, uint16_t* H, int A, int f, int S,
                                                          const int32_t* offsets, int E, int gate_rows)
{
    if (gate_rows > 0 && max_expert_rows(offsets, E) > gate_rows)
        return;  // the tiled gate/up GEMM wrote H
    const int64_t groups = (int64_t)A * (f / 4);
    const int64_t sstride = (int64_t)A * 2 * f;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < groups;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = idx / (f / 4);
        const int c = (int)(idx % (f / 4)) * 4;
        const int n = (c / 32) * 64 + (c % 32);
        const float* gp = part + p * 2 * f + n;
        float4 gs = *(const float4*)gp;
        float4 us = *(const float4*)(gp + 32);
        for (int s = 1; s < S; ++s) {
            const float4 a = *(const float4*)(gp + s * sstride);
            const float4 b = *(const float4*)(gp + s * sstride + 32);
            gs.x += a.x;
            gs.y += a.y;
            gs.z += a.z;
            gs.w += a.w;
            us.x += b.x;
            us.y += b.y;
            us.z += b.z;
            us.w += b.w;
        }
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_bits(silu(gs.x) * us.x) | ((uint32_t)f32_to_bf16_bits(silu(gs.y) * us.y) << 16);
        packed.y = (uint32_t)f32_to_bf16_bits(silu(gs.z) * us.z) | ((uint32_t)f32_to_bf16_bits(silu(gs.w) * us.w) << 16);
        *(uint2*)(H + p * f + c) = packed;
    }
}

}  // namespace

int decode_waves(int cus)
{
    return cus * 2 * (kThreads / kWave);
}

int decode_split(int E, int N, int K, int kstep, int waves, int max_split)
{
    // Enough K slices for about one item (of two 32-row blocks) per two
    // waves, at least four k-steps each. Long items stream best: on the
    // 8-expert decode layer (4096 x 14336) the gate/up GEMM without slices
    // (1.75 items per wave) reads at 6.45 TB/s where two slices gave 6.0,
    // and the down GEMM takes 146 us with 2 slices (half the waves busy),
    // 147 with 4, 150 with 8 and 190 with 1.
    const int64_t blocks = (int64_t)E * (N / 64);
    int64_t s = ((int64_t)waves + 2 * blocks - 1) / (2 * blocks);
    const int64_t cap = std::min<int64_t>(max_split, std::max(1, K / kstep / 4));
    s = std::max<int64_t>(1, std::min(s, cap));
    return (int)s;
}

hipError_t launch_decode_gemm(const DecodeArgs& a, int gate_up, int cus, hipStream_t s)
{
    if (a.a_scales) {  // 8-bit A rows feed the gate/up GEMM only
        if (!gate_up)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(decode_gemm_q8_kernel<true>, dim3(cus * 2), dim3(kThreads), 0, s, a);
    } else if (a.scales) {
        if (gate_up)
            hipLaunchKernelGGL(decode_gemm_f8_kernel<true>, dim3(cus * 2), dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL(decode_gemm_f8_kernel<false>, dim3(cus * 2), dim3(kThreads), 0, s, a);
    } else {
        const bool single = a.max_rows >= 1 && a.max_rows <= 32;
        auto k = gate_up ? (single ? decode_gemm_kernel<true, 1> : decode_gemm_kernel<true, 2>)
                         : (single ? decode_gemm_kernel<false, 1> : decode_gemm_kernel<false, 2>);
        hipLaunchKernelGGL(k, dim3(cus * 2), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_decode_silu(const float* part, void* H, int A, int f, int S, const int32_t* offsets, int E,
                              int gate_rows, hipStream_t s)
{
    const int64_t groups = (int64_t)A * (f / 4);
    int64_t blocks = (groups + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (blocks < 1)
        return hipSuccess;
    hipLaunchKernelGGL(decode_silu_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part, (uint16_t*)H, A, f, S,
                       offsets, E, gate_rows);
    return hipGetLastError();
}

}  // namespace cmoe
