// dispatch.hip - route assignments to per-expert contiguous segments.
//
// The dispatch step of «Colibri 是什么» (xxqk.cn) §2.1 and §2.3 scatters every
// token into the input buffers of its k experts. Here it is a stable counting
// sort of the A = T*k assignments (t, j) by expert id, keeping token order
// inside each expert's segment:
//   counts[e]   = #{a : ids[a] == e}
//   offsets[e]  = #{a : ids[a] <  e}            (exclusive prefix sum)
//   perm[p]     = t, perm_slot[p] = j, inv[t*k+j] = p
// No token activations move: the gate/up GEMM gathers rows through perm.
//
// One workgroup per expert e. It needs only two numbers besides its own
// assignments: how many ids are below e and how many equal e, so each thread
// counts in registers over a strided share of the id array (no atomics, no
// histogram contention on hot experts). Ranks inside the segment come from a
// block-wide exclusive scan over threads that own consecutive runs of 16
// assignments, so the order is the (t, j) order and the result is exact and
// reproducible.
#include "common.hpp"

namespace cmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kRun = 16;                   // consecutive assignments per thread
constexpr int kChunk = kThreads * kRun;    // assignments per block iteration

__device__ __forceinline__ void load_run(const int32_t* ids, int a0, int A, int (&v)[kRun])
{
    if (a0 + kRun <= A) {
        const int4* p = (const int4*)(ids + a0);
#pragma unroll
        for (int q = 0; q < kRun / 4; ++q) {
            int4 x = p[q];
            v[4 * q + 0] = x.x;
            v[4 * q + 1] = x.y;
            v[4 * q + 2] = x.z;
            v[4 * q + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kRun; ++q)
            v[q] = (a0 + q < A) ? ids[a0 + q] : 0x7FFFFFFF;
    }
}

// Block-wide exclusive scan of one int per thread; also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int& total)
{
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(incl, off, kWave);
        if (lane >= off)
            incl += o;
    }
    if (lane == kWave - 1)
        s_wave[wv] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
        const int t = s_wave[w];
        before += (w < wv) ? t : 0;
        total += t;
    }
    __syncthreads();
    return before + incl - v;
}

__global__ __launch_bounds__(kThreads) void dispatch_kernel(DispatchArgs g)
{
    __shared__ int s_wave[kThreads / kWave];
    const int e = blockIdx.x;
    const int A = g.T * g.k;

    // Pass 1: count ids below e and equal to e.
    int below = 0, equal = 0;
    for (int c = 0; c < A; c += kChunk) {
        int v[kRun];
        load_run(g.ids, c + threadIdx.x * kRun, A, v);
#pragma unroll
        for (int q = 0; q < kRun; ++q) {
            below += v[q] < e;
            equal += v[q] == e;
        }
    }
    int tot_below, tot_equal;
    (void)block_exclusive_scan(below, s_wave, tot_below);
    (void)block_exclusive_scan(equal, s_wave, tot_equal);
    if (threadIdx.x == 0) {
        g.counts[e] = tot_equal;
        g.offsets[e] = tot_below;
        if (e == g.E - 1)
            g.offsets[g.E] = tot_below + tot_equal;
    }
    if (tot_equal == 0)
        return;

    // Pass 2: stable compaction of this expert's assignments.
    int base = tot_below;
    for (int c = 0; c < A; c += kChunk) {
        const int a0 = c + threadIdx.x * kRun;
        int v[kRun];
        load_run(g.ids, a0, A, v);
        int mine = 0;
#pragma unroll
        for (int q = 0; q < kRun; ++q)
            mine += v[q] == e;
        int chunk_total;
        int p = base + block_exclusive_scan(mine, s_wave, chunk_total);
#pragma unroll
        for (int q = 0; q < kRun; ++q) {
            if (v[q] == e) {
                const int a = a0 + q;
                g.perm[p] = a / g.k;
                g.perm_slot[p] = a % g.k;
                g.inv[a] = p;
                ++p;
            }
        }
        base += chunk_total;
    }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(dispatch_kernel, dim3(a.E), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace cmoe
