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
// 1 to 8 workgroups per expert e, each writing e's assignments in one range
// of the id array. A workgroup needs only three numbers besides those: how
// many ids are below e, how many equal e, and how many equal e before its
// range, so each thread counts in registers over its share of the id array
// (no atomics, no histogram contention on hot experts). Ranks inside the
// segment come from a block-wide exclusive scan over threads that own
// consecutive runs of assignments, so the order is the (t, j) order and the
// result is exact and reproducible. A block covers 4096 assignments per
// iteration up to 8192 assignments (256 threads, runs of 16), else 32768
// (1024 threads, runs of 32), so most calls need one or two loads and scans
// per pass: the loop over chunks is a chain of dependent loads and block
// barriers.
#include "common.hpp"

namespace cmoe {

namespace {


template <int kRun>
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

// Block-wide exclusive scan of one int per thread (NT threads); also returns
// the total.
template <int NT>
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
    for (int w = 0; w < NT / kWave; ++w) {
        const int t = s_wave[w];
        before += (w < wv) ? t : 0;
        total += t;
    }
    __syncthreads();
    return before + incl - v;
}

// NT threads, kRun consecutive assignments per thread.
template <int NT, int kRun>
__global__ __launch_bounds__(NT) void dispatch_kernel(DispatchArgs g, int parts)
{
    constexpr int kChunk = NT * kRun;  // assignments per block iteration
    __shared__ int s_wave[NT / kWave];
    const int e = blockIdx.x / parts;
    const int part = blockIdx.x % parts;
    const int A = g.T * g.k;
    // This block writes the assignments of expert e in [r0, r1), the part-th
    // of `parts` ranges of whole runs (a hot expert's compaction is spread
    // over several blocks).
    const int runs = (A + kRun - 1) / kRun;
    const int rpp = (runs + parts - 1) / parts;
    const int r0 = min(part * rpp, runs) * kRun;
    const int r1 = min((part + 1) * rpp, runs) * kRun;

    // Pass 1: count ids below e, equal to e, and equal to e before r0.
    int below = 0, equal = 0, before = 0;
    for (int c = 0; c < A; c += kChunk) {
        const int a0 = c + threadIdx.x * kRun;
        int v[kRun];
        load_run(g.ids, a0, A, v);
        int eq = 0;
#pragma unroll
        for (int q = 0; q < kRun; ++q) {
            below += v[q] < e;
            eq += v[q] == e;
        }
        equal += eq;
        before += a0 < r0 ? eq : 0;  // r0 is a run boundary
    }
    int tot_below, tot_equal, tot_before = 0;
    (void)block_exclusive_scan<NT>(below, s_wave, tot_below);
    (void)block_exclusive_scan<NT>(equal, s_wave, tot_equal);
    if (parts > 1)
        (void)block_exclusive_scan<NT>(before, s_wave, tot_before);
    if (part == 0 && threadIdx.x == 0) {
        g.counts[e] = tot_equal;
        g.offsets[e] = tot_below;
        if (e == g.E - 1)
            g.offsets[g.E] = tot_below + tot_equal;
    }
    if (tot_equal == tot_before)  // none of this expert's assignments in [r0, r1)
        return;

    // Pass 2: stable compaction of this expert's assignments in [r0, r1).
    int base = tot_below + tot_before;
    for (int c = r0; c < r1; c += kChunk) {
        const int a0 = c + threadIdx.x * kRun;
        int v[kRun];
        load_run(g.ids, a0, A, v);
        int mine = 0;
        if (a0 < r1) {
#pragma unroll
            for (int q = 0; q < kRun; ++q)
                mine += v[q] == e;
        }
        int chunk_total;
        int p = base + block_exclusive_scan<NT>(mine, s_wave, chunk_total);
        if (a0 < r1) {
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
        }
        base += chunk_total;
    }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s)
{
    // Blocks per expert: enough for about 256 blocks (few experts), at most 8
    // and at most one per run of assignments; one below 4096 assignments,
    // where the compaction is short anyway.
    const int64_t A = (int64_t)a.T * a.k;
    const int run = A <= 8192 ? 16 : 32;
    const int runs = (int)((A + run - 1) / run);
    const int parts = A < 4096 ? 1 : std::max(1, std::min({8, 256 / std::max(a.E, 1), runs}));
    if (A <= 8192)
        hipLaunchKernelGGL((dispatch_kernel<256, 16>), dim3(a.E * parts), dim3(256), 0, s, a, parts);
    else
        hipLaunchKernelGGL((dispatch_kernel<1024, 32>), dim3(a.E * parts), dim3(1024), 0, s, a, parts);
    return hipGetLastError();
}

}  // namespace cmoe
