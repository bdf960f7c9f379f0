// gemm_f32.hip - grouped expert GEMMs for fp32 layers (FMA on the vector ALUs).
//
// Same two GEMMs as gemm_bf16.hip (gate/up with the SiLU(g)*u epilogue, then
// down), for layers stored in fp32. gfx950's fp32 matrix rate equals its fp32
// vector rate, so these use plain FMA with LDS tiles: 64x64 output tiles, 256
// threads, 4x4 outputs per thread, K staged 16 at a time. Tiles are mapped as
// in the bf16 kernels (derived on the device from offsets[], empty experts get
// none); the gate/up weights use the same 32-row gate/up interleave.
#include "common.hpp"

namespace cmoe {

namespace {

constexpr int kT = 64, kBK = 16, kThreads = 256;

struct TileF {
    int e, m, n, valid;
};

__device__ void find_tile_f32(const int32_t* offsets, int E, int NT, TileF* out)
{
    // Serial walk by one thread: these layers are small.
    int L = blockIdx.x;
    for (int e = 0; e < E; ++e) {
        const int c = offsets[e + 1] - offsets[e];
        const int tiles = ((c + kT - 1) / kT) * NT;
        if (L < tiles) {
            *out = TileF{e, L / NT, L % NT, 1};
            return;
        }
        L -= tiles;
    }
    out->valid = 0;
}

template <bool GATE_UP>
__global__ __launch_bounds__(kThreads) void grouped_gemm_f32_kernel(GemmArgs g)
{
    __shared__ float sA[kBK][kT + 1];
    __shared__ float sG[kBK][kT + 1];
    __shared__ float sU[kBK][kT + 1];
    __shared__ TileF s_tile;

    const int NOUT = GATE_UP ? g.f : g.d;  // output columns per expert
    const int K = GATE_UP ? g.d : g.f;
    const int NT = NOUT / kT;
    if (threadIdx.x == 0)
        find_tile_f32(g.offsets, g.E, NT, &s_tile);
    __syncthreads();
    if (!s_tile.valid)
        return;
    const int e = s_tile.e;
    const int row0 = g.offsets[e] + s_tile.m * kT;
    const int rows = min(kT, g.offsets[e + 1] - row0);
    const int col0 = s_tile.n * kT;

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
