// gemm_f32.hip - grouped expert GEMMs for fp32 layers (FMA on the vector ALUs).
//
// Same two GEMMs as gemm_bf16.hip (gate/up with the SiLU(g)*u epilogue, then
// down), for layers stored in fp32. gfx950's fp32 matrix rate equals its fp32
// vector rate, so these use plain FMA with LDS tiles: 64x64 output tiles, 256
// threads, 4x4 outputs per thread, K staged 16 at a time. Each block finds its
// tile with the bf16 kernels' walker (tiles.hpp: derived on the device from
// offsets[], empty experts get none); the gate/up weights use the same 32-row
// gate/up interleave.
#include "common.hpp"
#include "tiles.hpp"

namespace cmoe {

namespace {

constexpr int kT = 64, kBK = 16, kThreads = 256;

template <bool GATE_UP>
__global__ __launch_bounds__(kThreads) void grouped_gemm_f32_kernel(GemmArgs g)
{
    __shared__ float sA[kBK][kT + 1];
    __shared__ float sG[kBK][kT + 1];
    __shared__ float sU[kBK][kT + 1];

    const int NOUT = GATE_UP ? g.f : g.d;  // output columns per expert
    const int K = GATE_UP ? g.d : g.f;
    const int NT = NOUT / kT;
    // Every wave derives the block's tile from offsets[] (the same walker as
    // the bf16 GEMMs: one m-tile count per expert, a wave prefix sum, a ballot).
    TileTable tt;
    const int total = make_table<kT>(g.offsets, g.E, threadIdx.x % kWave, NT, tt);
    if ((int)blockIdx.x >= total)
        return;
    const Tile tl = decode<kT>(tt, blockIdx.x, NT, 1, NT, 1);
    const int e = tl.e;
    const int row0 = tl.row0;
    const int rows = tl.rows;
    const int col0 = tl.n * kT;

    const float* A = (const float*)g.a;
    const float* B = (const float*)g.b;
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;

    float ag[4][4] = {}, au[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kBK) {
        // Each thread loads 4 elements of each tile: (row lr, k lk).
        for (int i = threadIdx.x; i < kT * kBK; i += kThreads) {
            const int lr = i / kBK, lk = i % kBK;
            const int p = row0 + min(lr, rows - 1);
            const int src = GATE_UP ? g.perm[p] : p;
            sA[lk][lr] = A[(int64_t)src * K + k0 + lk];
            const int c = col0 + lr;  // output column
            if (GATE_UP) {
                const int64_t grow = (int64_t)e * 2 * g.f + (c / 32) * 64 + (c % 32);
                sG[lk][lr] = B[grow * K + k0 + lk];
                sU[lk][lr] = B[(grow + 32) * K + k0 + lk];
            } else {
                sG[lk][lr] = B[((int64_t)e * g.d + c) * K + k0 + lk];
            }
        }
        __syncthreads();
        for (int kk = 0; kk < kBK; ++kk) {
            float a[4], b[4], u[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = sA[kk][ty * 4 + i];
                b[i] = sG[kk][tx * 4 + i];
                u[i] = GATE_UP ? sU[kk][tx * 4 + i] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ag[i][j] = fmaf(a[i], b[j], ag[i][j]);
                    if (GATE_UP)
                        au[i][j] = fmaf(a[i], u[j], au[i][j]);
                }
        }
        __syncthreads();
    }
    float* out = (float*)g.out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = ty * 4 + i;
        if (r >= rows)
            continue;
        const int p = row0 + r;
        if (GATE_UP) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                out[(int64_t)p * g.f + col0 + tx * 4 + j] = silu(ag[i][j]) * au[i][j];
        } else {
            float* yrow = out + (int64_t)p * g.d;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                yrow[col0 + tx * 4 + j] = ag[i][j];
        }
    }
}

}  // namespace

hipError_t launch_gate_up_f32(const GemmArgs& a, hipStream_t s)
{
    const int grid = (a.A_max / kT + a.E) * (a.f / kT);
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down_f32(const GemmArgs& a, hipStream_t s)
{
    const int grid = (a.A_max / kT + a.E) * (a.d / kT);
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace cmoe
