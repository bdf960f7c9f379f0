// gemm_bf16.hip - grouped expert GEMMs on bf16 MFMA (gfx950).
//
// The expert GEMMs of «Colibri 是什么» (xxqk.cn) §2.3 (one GEMM kernel over the
// experts' row-major weights) in the batched form of «Colibri不是一只蜂鸟»
// (discosf.com) §1 and §3.2 (one fused launch over all active experts, the
// SiLU epilogue inlined into the first GEMM), with weight tiles staged in
// shared memory (LDS) as §5.1 of that page describes.
//
//   gate/up:  H[p][c]  = SiLU(sum_i X[perm[p]][i] Wg[e][c][i]) * (sum_i X[perm[p]][i] Wu[e][c][i])
//   down:     Ys[q][o] = sum_c H[p][c] Wd[e][o][c],     q = perm[p]*k + perm_slot[p]
// for every sorted position p of expert e's segment [offsets[e], offsets[e+1]).
//
// Operands: v_mfma_f32_32x32x16_bf16 (it keeps the matrix pipe full from a
// single wave per SIMD; the 16x16x32 form does not) takes, from lane l, 8
// consecutive k of row l%32 of A and of B. Token rows (A) are K-contiguous and
// are gathered through perm straight into LDS with gfx950's direct
// global->LDS loads; each wave reads its A fragments from there. Weights (B)
// do not pass through LDS at all: init stores them pre-blocked in MFMA operand
// order (32 rows x 16 k per 1 KiB block, lane-major), so each wave fetches its
// B fragments with fully coalesced 16-byte loads straight into VGPRs, one
// stage ahead. This halves LDS traffic, which otherwise caps the MFMA rate.
// Gate and up weights are interleaved in blocks of 32 rows (32 gate rows,
// then the 32 up rows of the same hidden units), so each wave holds the gate
// and up accumulators of the same outputs and applies SiLU(g)*u in registers.
//
// Work decomposition: a tile is (expert, m-tile of BM sorted rows, n-tile of
// BN weight rows). Experts with no rows have no tiles, so their weights are
// never read. The host only knows an upper bound of the tile count (the counts
// live on the device); each workgroup derives its tile from offsets[] and
// exits if it has none. Workgroup ids are spread over the 8 XCDs round-robin,
// so consecutive tile indices are handed to the same XCD, and tiles are
// ordered expert -> group of GN n-tiles -> m-tile -> n-tile: the workgroups
// one XCD runs together share weight panels and token panels in its L2.
#include "common.hpp"

namespace cmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;            // k per LDS stage
constexpr int kCH = kBK / 8;       // 16-byte chunks per row per stage
constexpr int kXCD = 8;

// XOR swizzle of the 16-byte chunk index inside an LDS row, so that the 16
// lanes reading one column of chunks of 16 consecutive rows hit distinct banks.
__device__ __forceinline__ int swz(int row, int chunk)
{
    return chunk ^ ((row >> 1) & 7);
}

struct Tile {
    int e, m, n, valid;
};

// Map this workgroup to a tile. Executed by wave 0; result in *out.
template <int BM>
__device__ void find_tile(const int32_t* offsets, int E, int NT, int GN, int remap, Tile* out)
{
    const int lane = threadIdx.x;
    int tl[4];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane * 4 + q;
        const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
        tl[q] = ((c + BM - 1) / BM) * NT;
        sum += tl[q];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (lane >= off)
            incl += o;
    }
    const int total = __shfl(incl, kWave - 1, kWave);
    const int wg = blockIdx.x;
    if (wg >= total) {
        if (lane == 0)
            out->valid = 0;
        return;
    }
    // XCD-aware renumbering: workgroup wg runs on XCD wg % 8; give each XCD a
    // contiguous range of tile indices.
    const int xcd = wg % kXCD, local = wg / kXCD;
    const int base = total / kXCD, rem = total % kXCD;
    const int L = remap ? xcd * base + min(xcd, rem) + local : wg;
    int start = incl - sum;
    if (L >= start && L < incl) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (L >= start && L < start + tl[q]) {
                const int e = lane * 4 + q;
                const int Me = tl[q] / NT;
                const int l = L - start;
                const int g = l / (Me * GN);
                const int gn = min(GN, NT - g * GN);
                const int idx = l - g * Me * GN;
                out->e = e;
                out->m = idx / gn;
                out->n = g * GN + idx % gn;
                out->valid = 1;
            }
            start += tl[q];
        }
    }
}

typedef __attribute__((address_space(3))) void lds_void_t;

// One K-stage of A lives in LDS as rows of 8 16-byte chunks (64 bf16 of K),
// chunk index XOR-swizzled per row. Stages are filled with direct global->LDS
// loads (global_load_lds_dwordx4): one instruction moves 64 lanes x 16 B into
// 1 KiB of LDS, i.e. 8 rows; lane s lands in slot s, so the lane fetches the
// chunk that the swizzle maps to that slot. No VGPR staging.
template <int INS>
__device__ __forceinline__ void issue_a_stage(const uint16_t* base, const uint32_t (&off)[INS], int k0,
                                              Vec16* stage, int n_ins)
{
#pragma unroll
    for (int i = 0; i < INS; ++i) {
        if (i >= n_ins)
            continue;
        Vec16* dst = stage + i * 8 * kCH;
        __builtin_amdgcn_global_load_lds((const void*)(base + off[i] + k0), (lds_void_t*)dst, 16, 0, 0);
    }
}

// B fragments of one stage: NI 32-row blocks x KS k-steps, 16 B per lane each,
// from the blocked weight layout (bw points at this lane's slot of the wave's
// first block row; kb0 = first k-block of the stage; KB = k-blocks per row).
template <int NI, int KS>
__device__ __forceinline__ void load_b_stage(const Vec16* bw, int kb0, int KB, Vec16 (&bq)[KS][NI])
{
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            bq[ks][j] = bw[((int64_t)j * KB + kb0 + ks) * 64];
}

// Scheduling pins: R LDS reads spread evenly between M MFMAs (mask 0x008 =
// MFMA, 0x100 = LDS read, as the sched_group_barrier builtin defines them).
template <int R, int M, int r>
__device__ __forceinline__ void sched_spread()
{
    if constexpr (r < R) {
        constexpr int n = (M * (r + 1)) / R - (M * r) / R;
        if constexpr (n > 0)
            __builtin_amdgcn_sched_group_barrier(0x008, n, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        sched_spread<R, M, r + 1>();
    }
}

// One k step: its M MFMAs, with the R reads of the next step spread over the
// first half of them (so they land before the next step starts).
template <int N, int R, int M>
__device__ __forceinline__ void sched_repeat()
{
    if constexpr (N > 0) {
        sched_spread<R, M / 2, 0>();
        __builtin_amdgcn_sched_group_barrier(0x008, M - M / 2, 0);
        sched_repeat<N - 1, R, M>();
    }
}

// MFMA work on one stage (four 16-wide k steps of 32x32x16 MFMAs): A fragments
// from LDS, B fragments from registers. PARTIAL tiles (the last m-tile of an
// expert) skip the A reads and MFMAs of 32-row groups that hold no valid row.
// For full tiles the instruction order is pinned: the NLOAD global loads of
// the next stage issued just before (when in the same block), the A reads of
// the first k step, then each k step's MFMAs with the next step's reads spread
// between them, so memory and LDS latency hide behind matrix work.
template <int WM, int WN, bool PARTIAL, int NLOAD>
__device__ __forceinline__ void mfma_stage(const Vec16* As, const Vec16 (&bq)[kBK / 16][WN / 32], int wm,
                                           int lane, int mi_lim, floatx16 (&acc)[WM / 32][WN / 32])
{
    constexpr int MI = WM / 32, NI = WN / 32, KS = kBK / 16;
    const int lr = lane & 31;
    bf16x8 afr[KS][MI];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 2 + (lane >> 5);
        const int col = c ^ ((lr >> 1) & 7);  // swz() of a row whose low 5 bits are lr
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if (PARTIAL && i >= mi_lim)
                continue;
            afr[ks][i] = as_bf16x8(As[(wm * WM + i * 32 + lr) * kCH + col]);
        }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if (PARTIAL && i >= mi_lim)
                continue;
#pragma unroll
            for (int j = 0; j < NI; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[ks][i], as_bf16x8(bq[ks][j]), acc[i][j],
                                                                   0, 0, 0);
        }
    }
    if constexpr (!PARTIAL) {
        constexpr int R = MI;       // A reads per k step
        constexpr int M = MI * NI;  // MFMAs per k step
        // the next stage's loads (if issued in this block) go first
        if constexpr (NLOAD > 0)
            __builtin_amdgcn_sched_group_barrier(0x010, NLOAD, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
        sched_repeat<KS - 1, R, M>();
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    }
}

// Wait until this wave's loads of the current stage have landed, then
// barrier. The scheduling barrier keeps the scheduler from moving the MFMAs
// of the previous stage across the wait.
__device__ __forceinline__ void wait_stage_loads()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// The K loop of one tile: stage kt+1 (A into the other LDS buffer, B into the
// other register set) is loaded while stage kt is multiplied; one barrier per
// stage. Unrolled by two so both register sets have fixed names.
template <int WM, int WN, int A_INS, bool PARTIAL>
__device__ __forceinline__ void tile_k_loop(const uint16_t* A, const uint32_t (&aoff)[A_INS], const Vec16* bw,
                                            int KB, Vec16* sA0, Vec16* sA1, Vec16* sA0w, Vec16* sA1w, int KT,
                                            int wm, int lane, int a_ins, int mi_lim,
                                            floatx16 (&acc)[WM / 32][WN / 32])
{
    constexpr int NI = WN / 32, KS = kBK / 16;
    Vec16 bq0[KS][NI], bq1[KS][NI];
    issue_a_stage<A_INS>(A, aoff, 0, sA0w, a_ins);
    load_b_stage<NI, KS>(bw, 0, KB, bq0);
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        wait_stage_loads();  // stage kt landed (LDS buffer 0, registers bq0)
        issue_a_stage<A_INS>(A, aoff, (kt + 1) * kBK, sA1w, a_ins);
        load_b_stage<NI, KS>(bw, (kt + 1) * KS, KB, bq1);
        mfma_stage<WM, WN, PARTIAL, A_INS + NI * KS>(sA0, bq0, wm, lane, mi_lim, acc);
        wait_stage_loads();  // stage kt+1 landed (LDS buffer 1, registers bq1)
        if (kt + 2 < KT) {
            issue_a_stage<A_INS>(A, aoff, (kt + 2) * kBK, sA0w, a_ins);
            load_b_stage<NI, KS>(bw, (kt + 2) * KS, KB, bq0);
        }
        mfma_stage<WM, WN, PARTIAL, 0>(sA1, bq1, wm, lane, mi_lim, acc);
    }
    if (kt < KT) {  // odd number of stages: the last one is in buffer 0
        wait_stage_loads();
        mfma_stage<WM, WN, PARTIAL, 0>(sA0, bq0, wm, lane, mi_lim, acc);
    }
}

template <int BM, int BN, int WM, int WN, bool GATE_UP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_kernel(GemmArgs g)
{
    constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int A_INS = BM / 4 / 8;  // direct-load instructions per wave per stage
    static_assert(WAVES_M * WAVES_N == kThreads / kWave, "4 waves");
    static_assert(A_INS >= 1, "tile too small");
    static_assert(!GATE_UP || (NI % 2 == 0 && WN % 64 == 0), "gate/up pairs per wave");

    // Two A stages, separate arrays so the compiler sees the buffers as distinct.
    __shared__ Vec16 sA0[BM * kCH], sA1[BM * kCH];
    __shared__ Tile s_tile;

    const int N = GATE_UP ? 2 * g.f : g.d;  // weight rows per expert
    const int K = GATE_UP ? g.d : g.f;
    const int NT = N / BN;
    const int KB = K / 16;                 // 16-wide k blocks per weight row block

    if (threadIdx.x < kWave)
        find_tile<BM>(g.offsets, g.E, NT, g.group_n, g.xcd_remap, &s_tile);
    __syncthreads();
    if (!s_tile.valid)
        return;
    const int e = s_tile.e, mt = s_tile.m, nt = s_tile.n;
    const int seg0 = g.offsets[e];
    const int row0 = seg0 + mt * BM;
    const int rows = min(BM, g.offsets[e + 1] - row0);

    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wv / WAVES_N, wn = wv % WAVES_N;

    // A: per-lane source offsets (elements) of the 8-row groups this wave
    // loads into LDS. Rows are gathered through perm for gate/up; rows past the
    // segment end are clamped to its last row (loaded only when they share an
    // instruction with valid rows; their results are never stored).
    const uint16_t* A = (const uint16_t*)g.a;
    const int rsub = lane / 8, pch = lane % 8;
    uint32_t aoff[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int r = wv * (BM / 4) + i * 8 + rsub;
        const int p = row0 + min(r, rows - 1);
        const int src = GATE_UP ? g.perm[p] : p;
        aoff[i] = (uint32_t)src * (uint32_t)K + (uint32_t)((pch ^ swz(r, 0)) * 8);
    }
    const int a_ins = min(A_INS, max(0, (rows - wv * (BM / 4) + 7) / 8));
    Vec16* sA0w = sA0 + wv * (BM / 4) * kCH;  // this wave's slice of each stage
    Vec16* sA1w = sA1 + wv * (BM / 4) * kCH;

    // B: this lane's slot in the first 32-row block of the wave's columns.
    const int nb0 = (nt * BN + wn * WN) / 32;
    const Vec16* bw = (const Vec16*)g.b + ((int64_t)e * (N / 32) + nb0) * KB * 64 + lane;

    floatx16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                acc[i][j][q] = 0.f;

    const int KT = K / kBK;
    if (rows == BM)
        tile_k_loop<WM, WN, A_INS, false>(A, aoff, bw, KB, sA0, sA1, sA0w, sA1w, KT, wm, lane, A_INS, MI, acc);
    else
        tile_k_loop<WM, WN, A_INS, true>(A, aoff, bw, KB, sA0, sA1, sA0w, sA1w, KT, wm, lane, a_ins,
                                         min(MI, max(0, (rows - wm * WM + 31) / 32)), acc);

    // Epilogue. 32x32 accumulator layout: lane holds column lane%32 and, for
    // q = 0..15, row 8*(q/4) + 4*(lane/32) + q%4.
    if constexpr (GATE_UP) {
        uint16_t* H = (uint16_t*)g.out;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int r = wm * WM + i * 32 + 8 * (q / 4) + 4 * (lane >> 5) + (q % 4);
                if (r >= rows)
                    continue;
                uint16_t* hrow = H + (int64_t)(row0 + r) * g.f;
#pragma unroll
                for (int j = 0; j < NI; j += 2) {
                    const int wrow = nt * BN + wn * WN + j * 32;  // first gate row of the pair
                    const int col = wrow / 2 + (lane & 31);
                    const float gv = acc[i][j][q], uv = acc[i][j + 1][q];
                    hrow[col] = f32_to_bf16_bits(silu(gv) * uv);
                }
            }
        }
    } else {
        float* Ys = (float*)g.out;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int r = wm * WM + i * 32 + 8 * (q / 4) + 4 * (lane >> 5) + (q % 4);
                if (r >= rows)
                    continue;
                const int p = row0 + r;
                float* yrow = Ys + ((int64_t)g.perm[p] * g.k + g.perm_slot[p]) * g.d;
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    yrow[nt * BN + wn * WN + j * 32 + (lane & 31)] = acc[i][j][q];
            }
        }
    }
}

template <int BM>
int m_tile_bound(int A_max, int E)
{
    // sum_e ceil(c_e / BM) <= floor(A / BM) + E  for sum_e c_e = A
    return A_max / BM + E;
}

// Init-time weight repack into the blocked MFMA operand layout: for expert e,
// row block nb (32 weight rows) and k block kb (16 k), one 1 KiB block in lane
// order, lane l holding row nb*32 + l%32, k = kb*16 + 8*(l/32) .. +8. With
// gate/up interleaving, weight row n of the combined [2f][d] matrix is gate
// row (n/64)*32 + n%32 when n%64 < 32, else up row (n/64)*32 + n%32 - 32.
__global__ void pack_blocked_kernel(const uint16_t* w0, const uint16_t* w1, Vec16* out, int E, int N, int K,
                                    int gate_up)
{
    const int NB = N / 32, KB = K / 16;
    const int64_t total = (int64_t)E * NB * KB * 64;
    const int Nsrc = gate_up ? N / 2 : N;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(idx % 64);
        const int64_t blk = idx / 64;
        const int kb = (int)(blk % KB);
        const int64_t rb = blk / KB;
        const int nb = (int)(rb % NB);
        const int e = (int)(rb / NB);
        const int n = nb * 32 + (l % 32);
        const int k = kb * 16 + 8 * (l / 32);
        const uint16_t* src;
        int srow;
        if (gate_up) {
            const int w = n % 64;
            srow = (n / 64) * 32 + (w % 32);
            src = w < 32 ? w0 : w1;
        } else {
            srow = n;
            src = w0;
        }
        out[idx] = *(const Vec16*)(src + ((int64_t)e * Nsrc + srow) * K + k);
    }
}

__global__ void interleave_gate_up_kernel(const uint8_t* wg, const uint8_t* wu, uint8_t* wgu, int E,
                                          int f, int64_t row_bytes)
{
    // wgu[e][r] = (r % 64 < 32 ? wg : wu)[e][(r / 64) * 32 + r % 32], whole rows.
    const int64_t rows = (int64_t)E * 2 * f;
    const int64_t words = row_bytes / 16;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < rows * words;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t R = idx / words, w = idx % words;
        const int64_t e = R / (2 * f), r = R % (2 * f);
        const int64_t src_row = e * f + (r / 64) * 32 + (r % 32);
        const uint8_t* src = ((r % 64) < 32 ? wg : wu) + src_row * row_bytes;
        ((Vec16*)(wgu + R * row_bytes))[w] = ((const Vec16*)src)[w];
    }
}

}  // namespace

// Tile shapes: 256x256 output tiles, 4 waves of 128x128 (256 fp32 accumulators
// per lane, held in AGPRs), 2 x 32 KiB LDS stages of A. When the weight-row
// count is not a multiple of 256, 256x128 tiles (waves of 128x64) are used.
constexpr int kBM = 256;

template <bool GATE_UP>
hipError_t launch_grouped(const GemmArgs& a, hipStream_t s)
{
    const int N = GATE_UP ? 2 * a.f : a.d;
    const int mt = m_tile_bound<kBM>(a.A_max, a.E);
    if (N % 256 == 0)
        hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 256, 128, 128, GATE_UP>), dim3(mt * (N / 256)),
                           dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 128, 128, 64, GATE_UP>), dim3(mt * (N / 128)),
                           dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gate_up_bf16(const GemmArgs& a, hipStream_t s)
{
    return launch_grouped<true>(a, s);
}

hipError_t launch_down_bf16(const GemmArgs& a, hipStream_t s)
{
    return launch_grouped<false>(a, s);
}

hipError_t launch_pack_blocked(const void* w0, const void* w1, void* out, int E, int N, int K, int gate_up,
                               hipStream_t s)
{
    hipLaunchKernelGGL(pack_blocked_kernel, dim3(2048), dim3(256), 0, s, (const uint16_t*)w0, (const uint16_t*)w1,
                       (Vec16*)out, E, N, K, gate_up);
    return hipGetLastError();
}

hipError_t launch_interleave_gate_up(const void* wg, const void* wu, void* wgu, int E, int f, int d,
                                     int esize, hipStream_t s)
{
    hipLaunchKernelGGL(interleave_gate_up_kernel, dim3(1024), dim3(256), 0, s, (const uint8_t*)wg,
                       (const uint8_t*)wu, (uint8_t*)wgu, E, f, (int64_t)d * esize);
    return hipGetLastError();
}

}  // namespace cmoe
