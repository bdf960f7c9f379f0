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
// result is exact and reproducible. The three counts need only block totals
// (one shuffle reduction per wave and one LDS exchange), and when the ids fit
// one block iteration each thread keeps its run in registers for the second
// pass. A block covers 4096 assignments per
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

// Block-wide sums of NV ints per thread (NT threads): each wave adds its
// lanes' values with butterfly shuffles, then every thread adds the waves'
// sums from LDS (one barrier pair for all NV values).
template <int NT, int NV>
__device__ __forceinline__ void block_sums(int (&v)[NV], int (*s_red)[NV])
{
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1)
            v[i] += __shfl_xor(v[i], off, kWave);
    if (lane == 0)
#pragma unroll
        for (int i = 0; i < NV; ++i)
            s_red[wv][i] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int t = 0;
#pragma unroll
        for (int w = 0; w < NT / kWave; ++w)
            t += s_red[w][i];
        v[i] = t;
    }
    __syncthreads();
}

// NT threads, kRun consecutive assignments per thread.
template <int NT, int kRun>
__global__ __launch_bounds__(NT) void dispatch_kernel(DispatchArgs g, int parts)
{
    constexpr int kChunk = NT * kRun;  // assignments per block iteration
    __shared__ int s_wave[NT / kWave];
    __shared__ int s_red[NT / kWave][3];
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

    // Pass 1: count ids below e, equal to e, and equal to e before r0. When
    // the ids fit one chunk, this thread's run stays in v for pass 2.
    int below = 0, equal = 0, before = 0;
    int v[kRun];
    for (int c = 0; c < A; c += kChunk) {
        const int a0 = c + threadIdx.x * kRun;
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
    int tot[3] = {below, equal, before};
    block_sums<NT, 3>(tot, s_red);
    const int tot_below = tot[0], tot_equal = tot[1], tot_before = tot[2];
    if (part == 0 && threadIdx.x == 0) {
        g.counts[e] = tot_equal;
        g.offsets[e] = tot_below;
        if (e == g.E - 1)
            g.offsets[g.E] = tot_below + tot_equal;
    }
    if (tot_equal == tot_before)  // none of this expert's assignments in [r0, r1)
        return;

    // Pass 2: stable compaction of this expert's assignments in [r0, r1),
    // over the chunks of pass 1 that meet that range (runs outside it count
    // none of this block's assignments).
    int base = tot_below + tot_before;
    const bool one = A <= kChunk;  // v still holds this thread's run
    for (int c = (r0 / kChunk) * kChunk; c < r1; c += kChunk) {
        const int a0 = c + threadIdx.x * kRun;
        if (!one)
            load_run(g.ids, a0, A, v);
        const bool in = a0 >= r0 && a0 < r1;  // runs are whole: r0, r1 are run boundaries
        int mine = 0;
        if (in) {
#pragma unroll
            for (int q = 0; q < kRun; ++q)
                mine += v[q] == e;
        }
        int chunk_total;
        int p = base + block_exclusive_scan<NT>(mine, s_wave, chunk_total);
        if (in) {
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
