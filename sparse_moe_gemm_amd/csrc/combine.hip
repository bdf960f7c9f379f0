// combine.hip - weighted sum of each token's k expert outputs.
//
// The combine kernel of «Colibri 是什么» (xxqk.cn) §2.3 (the k expert outputs
// weighted by the gating scores and summed) and the final step of
// «Colibri：面向MoE模型的高性能C语言推理引擎» (zskr.cn) §3.3:
//   y[t][o] = sum_{j<k} w[t][j] * Ys[inv[t*k + j]][o]
// accumulated in fp32 in slot order (fused multiply-add), then rounded to
// the output dtype (round to nearest even for bf16). The down GEMM wrote each
// expert output at its sorted position p; inv maps assignment t*k+j to it.
// When the down GEMM split K, Ys holds `split` partial sums per row (at
// strides of T*k rows), added in split order before the weighting; without a
// split (tiled path) the rows are bf16, widened exactly here. Each
// thread handles 4 consecutive outputs with 16-byte loads; the kernel is
// bound by HBM.
#include "common.hpp"

namespace cmoe {

namespace {

__device__ __forceinline__ void store_out(const CombineArgs& g, int64_t t, int o, float4 acc)
{
    if (g.bf16_out) {
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_bits(acc.x) | ((uint32_t)f32_to_bf16_bits(acc.y) << 16);
        packed.y = (uint32_t)f32_to_bf16_bits(acc.z) | ((uint32_t)f32_to_bf16_bits(acc.w) << 16);
        *(uint2*)((uint16_t*)g.y + t * g.d + o) = packed;
    } else {
        *(float4*)((float*)g.y + t * g.d + o) = acc;
    }
}

// K slots and S partials known at compile time: the token's positions and
// weights are loaded first, then all K*S row loads are in flight together.
template <int K, int S>
__global__ __launch_bounds__(256) void combine_ks_kernel(CombineArgs g)
{
    const int64_t groups = (int64_t)g.T * (g.d / 4);
    const int64_t stride = (int64_t)g.T * K * g.d;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < groups;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = idx / (g.d / 4);
        const int o = (int)(idx % (g.d / 4)) * 4;
        int pos[K];
        float wgt[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            pos[j] = g.inv[t * K + j];
            wgt[j] = g.w[t * K + j];
        }
        float4 v[K][S];
#pragma unroll
        for (int j = 0; j < K; ++j)
#pragma unroll
            for (int s = 0; s < S; ++s)
                v[j][s] = *(const float4*)(g.ys + (int64_t)pos[j] * g.d + o + s * stride);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            float4 u = v[j][0];
#pragma unroll
            for (int s = 1; s < S; ++s) {
                u.x += v[j][s].x;
                u.y += v[j][s].y;
                u.z += v[j][s].z;
                u.w += v[j][s].w;
            }
            acc.x = fmaf(wgt[j], u.x, acc.x);
            acc.y = fmaf(wgt[j], u.y, acc.y);
            acc.z = fmaf(wgt[j], u.z, acc.z);
            acc.w = fmaf(wgt[j], u.w, acc.w);
        }
        store_out(g, t, o, acc);
    }
}

// Expert outputs stored as bf16 (no K split), K slots known at compile
// time: eight consecutive outputs per thread, one 16-byte load per slot, all
// K in flight together, widened exactly and summed in fp32 in slot order.
template <int K>
__global__ __launch_bounds__(256) void combine_b16_kernel(CombineArgs g)
{
    const int64_t groups = (int64_t)g.T * (g.d / 8);
    const uint16_t* yb = (const uint16_t*)g.ys;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < groups;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = idx / (g.d / 8);
        const int o = (int)(idx % (g.d / 8)) * 8;
        int pos[K];
        float wgt[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            pos[j] = g.inv[t * K + j];
            wgt[j] = g.w[t * K + j];
        }
        uint4 v[K];
#pragma unroll
        for (int j = 0; j < K; ++j)
            v[j] = *(const uint4*)(yb + (int64_t)pos[j] * g.d + o);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(wgt[j], __uint_as_float(w4[q] << 16), acc[2 * q]);
                acc[2 * q + 1] = fmaf(wgt[j], __uint_as_float(w4[q] & 0xFFFF0000u), acc[2 * q + 1]);
            }
        }
        store_out(g, t, o, make_float4(acc[0], acc[1], acc[2], acc[3]));
        store_out(g, t, o + 4, make_float4(acc[4], acc[5], acc[6], acc[7]));
    }
}

// Any k and number of partials (the small-batch path's K slices), and calls
// that enqueued both GEMM paths: the Ys format of the path the device chose
// (bf16 rows widened exactly, or fp32 partials added in order). The same
// arithmetic as the kernels above, so the same results bit for bit.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs g)
{
    const int64_t groups = (int64_t)g.T * (g.d / 4);
    const int64_t stride = (int64_t)g.T * g.k * g.d;
    int split = g.split;
    bool ysb = g.ys_bf16 != 0;
    if (g.gate_rows > 0 && max_expert_rows(g.offsets, g.E) <= g.gate_rows) {
        split = g.small_split;
        ysb = false;
    }
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < groups;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = idx / (g.d / 4);
        const int o = (int)(idx % (g.d / 4)) * 4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < g.k; ++j) {
            const float wj = g.w[t * g.k + j];
            const int64_t pos = (int64_t)g.inv[t * g.k + j] * g.d + o;
            float4 v;
            if (ysb) {
                const uint2 b = *(const uint2*)((const uint16_t*)g.ys + pos);
                v = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                                __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u));
            } else {
                const float* row = g.ys + pos;
                v = *(const float4*)row;
                for (int s = 1; s < split; ++s) {
                    const float4 u = *(const float4*)(row + s * stride);
                    v.x += u.x;
                    v.y += u.y;
                    v.z += u.z;
                    v.w += u.w;
                }
            }
            acc.x = fmaf(wj, v.x, acc.x);
            acc.y = fmaf(wj, v.y, acc.y);
            acc.z = fmaf(wj, v.z, acc.z);
            acc.w = fmaf(wj, v.w, acc.w);
        }
        store_out(g, t, o, acc);
    }
}

template <int K>
bool launch_ks(const CombineArgs& a, dim3 grid, hipStream_t s)
{
    if (a.k != K || a.split > 2)
        return false;
    if (a.ys_bf16) {
        const int64_t groups = (int64_t)a.T * (a.d / 8);
        const unsigned blocks = (unsigned)std::min<int64_t>((groups + 255) / 256, 8192);
        hipLaunchKernelGGL((combine_b16_kernel<K>), dim3(blocks), dim3(256), 0, s, a);
        return true;
    }
    if (a.split == 1)
        hipLaunchKernelGGL((combine_ks_kernel<K, 1>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((combine_ks_kernel<K, 2>), grid, dim3(256), 0, s, a);
    return true;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s)
{
    const int64_t groups = (int64_t)a.T * (a.d / 4);
    int64_t blocks = (groups + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    const dim3 grid((unsigned)blocks);
    if (a.gate_rows > 0) {  // format known on the device only
        hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    if (launch_ks<1>(a, grid, s) || launch_ks<2>(a, grid, s) || launch_ks<3>(a, grid, s) ||
        launch_ks<4>(a, grid, s) || launch_ks<5>(a, grid, s) || launch_ks<6>(a, grid, s) ||
        launch_ks<7>(a, grid, s) || launch_ks<8>(a, grid, s))
        return hipGetLastError();
    if (a.ys_bf16)  // bf16 expert outputs come with k <= 8 and no K split
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace cmoe
