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
// Both operands are K-contiguous (token rows, and (out, in) weight rows), which
// is the operand order v_mfma_f32_16x16x32_bf16 wants: lane l supplies 8
// consecutive k of row l%16 for both A and B. Gate and up weights are
// interleaved at init in blocks of 16 rows (16 gate rows, then the 16 up rows
// of the same hidden units), so each wave holds the gate and up accumulators
// of the same outputs in registers and applies SiLU(g)*u before the store.
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
template <int BM, int GN>
__device__ void find_tile(const int32_t* offsets, int E, int NT, Tile* out)
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
    const int L = xcd * base + min(xcd, rem) + local;
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

// One K-stage of a tile lives in LDS as rows of 8 16-byte chunks (64 bf16 of
// K), chunk index XOR-swizzled per row. Stages are filled with gfx950's direct
// global->LDS loads (global_load_lds_dwordx4): one instruction moves 64 lanes x
// 16 B into 1 KiB of LDS, i.e. 8 rows; lane s lands in slot s, so the lane
// fetches the chunk that the swizzle maps to that slot. No VGPR staging.
template <int ROWS, int INS>
__device__ __forceinline__ void issue_stage(const uint16_t* base, const uint32_t (&off)[INS], int k0,
                                            Vec16* stage, int wave, int first_ins, int n_ins)
{
#pragma unroll
    for (int i = 0; i < INS; ++i) {
        if (i < first_ins || i >= n_ins)
            continue;
        Vec16* dst = stage + (wave * (ROWS / 4) + i * 8) * kCH;
        __builtin_amdgcn_global_load_lds((const void*)(base + off[i] + k0), (lds_void_t*)dst, 16, 0, 0);
    }
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

// MFMA work on one LDS stage (two 32-wide k steps). PARTIAL tiles (the last
// m-tile of an expert) skip the A-fragment reads and MFMAs of 16-row groups
// that hold no valid row. For full tiles the instruction order is pinned:
// the 16 fragment reads of the first k step, then the 64 MFMAs of that step
// with the 16 reads of the second step spread between them, then the second
// step's 64 MFMAs, so LDS latency hides behind matrix work.
template <int BM, int BN, int WM, int WN, bool PARTIAL>
__device__ __forceinline__ void mfma_stage(const Vec16* As, const Vec16* Bs, int wm, int wn, int lane, int mi_lim,
                                           floatx4 (&acc)[WM / 16][WN / 16])
{
    constexpr int MI = WM / 16, NI = WN / 16, KS = kBK / 32;
    const int lr = lane & 15;
    bf16x8 bfr[KS][NI], afr[KS][MI];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 4 + (lane >> 4);
        const int col = c ^ ((lr >> 1) & 7);  // swz() of a row whose low 4 bits are lr
#pragma unroll
        for (int j = 0; j < NI; ++j)
            bfr[ks][j] = as_bf16x8(Bs[(wn * WN + j * 16 + lr) * kCH + col]);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if (PARTIAL && i >= mi_lim)
                continue;
            afr[ks][i] = as_bf16x8(As[(wm * WM + i * 16 + lr) * kCH + col]);
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
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
        }
    }
    if constexpr (!PARTIAL && KS == 2) {
        constexpr int R = MI + NI;  // fragment reads per k step
        constexpr int M = MI * NI;  // MFMAs per k step
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
        sched_spread<R, M, 0>();
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    }
}

__device__ __forceinline__ void wait_stage_loads()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// The K loop of one tile: stage kt+1 is loaded straight into the other LDS
// buffer while stage kt is multiplied; one barrier per stage.
template <int BM, int BN, int WM, int WN, int A_INS, int B_INS, bool PARTIAL>
__device__ __forceinline__ void tile_k_loop(const uint16_t* A, const uint32_t (&aoff)[A_INS], const uint16_t* B,
                                            const uint32_t (&boff)[B_INS], Vec16* sA0, Vec16* sA1, Vec16* sB0,
                                            Vec16* sB1, int KT, int wv, int wm, int wn, int lane, int a_ins,
                                            int mi_lim, floatx4 (&acc)[WM / 16][WN / 16])
{
    issue_stage<BM, A_INS>(A, aoff, 0, sA0, wv, 0, a_ins);
    issue_stage<BN, B_INS>(B, boff, 0, sB0, wv, 0, B_INS);
    for (int kt = 0; kt < KT; ++kt) {
        const bool odd = kt & 1;
        wait_stage_loads();  // stage kt has landed; the other buffer is free
        if (kt + 1 < KT) {
            issue_stage<BM, A_INS>(A, aoff, (kt + 1) * kBK, odd ? sA0 : sA1, wv, 0, a_ins);
            issue_stage<BN, B_INS>(B, boff, (kt + 1) * kBK, odd ? sB0 : sB1, wv, 0, B_INS);
        }
        mfma_stage<BM, BN, WM, WN, PARTIAL>(odd ? sA1 : sA0, odd ? sB1 : sB0, wm, wn, lane, mi_lim, acc);
    }
}

template <int BM, int BN, int WM, int WN, int GN, bool GATE_UP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_kernel(GemmArgs g)
{
    constexpr int WAVES_N = BN / WN;
    constexpr int MI = WM / 16, NI = WN / 16;
    constexpr int A_INS = BM / 4 / 8;  // direct-load instructions per wave per stage
    constexpr int B_INS = BN / 4 / 8;
    static_assert((BM / WM) * (BN / WN) == kThreads / kWave, "4 waves");
    static_assert(A_INS >= 1 && B_INS >= 1, "tile too small");
    static_assert(!GATE_UP || (NI % 2 == 0 && WN % 32 == 0), "gate/up pairs per wave");

    // Two stages, separate arrays so the compiler sees the buffers as distinct.
    __shared__ Vec16 sA0[BM * kCH], sA1[BM * kCH];
    __shared__ Vec16 sB0[BN * kCH], sB1[BN * kCH];
    __shared__ Tile s_tile;

    const int N = GATE_UP ? 2 * g.f : g.d;  // weight rows per expert
    const int K = GATE_UP ? g.d : g.f;
    const int NT = N / BN;

    if (threadIdx.x < kWave)
        find_tile<BM, GN>(g.offsets, g.E, NT, &s_tile);
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

    // Per-lane source offsets (elements) of the rows this wave loads. A rows are
    // gathered through perm for gate/up; rows past the segment end are clamped
    // to its last row (loaded only when they share an instruction with valid
    // rows; their results are never stored).
    const uint16_t* A = (const uint16_t*)g.a;
    const uint16_t* B = (const uint16_t*)g.b + ((int64_t)e * N + (int64_t)nt * BN) * K;
    const int rsub = lane / 8, pch = lane % 8;
    uint32_t aoff[A_INS], boff[B_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int r = wv * (BM / 4) + i * 8 + rsub;
        const int p = row0 + min(r, rows - 1);
        const int src = GATE_UP ? g.perm[p] : p;
        aoff[i] = (uint32_t)src * (uint32_t)K + (uint32_t)((pch ^ swz(r, 0)) * 8);
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int r = wv * (BN / 4) + i * 8 + rsub;
        boff[i] = (uint32_t)r * (uint32_t)K + (uint32_t)((pch ^ swz(r, 0)) * 8);
    }
    // A instructions of this wave that hold at least one valid row.
    const int a_ins = min(A_INS, max(0, (rows - wv * (BM / 4) + 7) / 8));

    floatx4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int KT = K / kBK;
    if (rows == BM)
        tile_k_loop<BM, BN, WM, WN, A_INS, B_INS, false>(A, aoff, B, boff, sA0, sA1, sB0, sB1, KT, wv, wm, wn,
                                                         lane, A_INS, MI, acc);
    else
        tile_k_loop<BM, BN, WM, WN, A_INS, B_INS, true>(A, aoff, B, boff, sA0, sA1, sB0, sB1, KT, wv, wm, wn,
                                                        lane, a_ins, min(MI, max(0, (rows - wm * WM + 15) / 16)),
                                                        acc);

    // Epilogue. Accumulator layout: lane holds rows 4*(lane/16)+q, column lane%16.
    if constexpr (GATE_UP) {
        uint16_t* H = (uint16_t*)g.out;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = wm * WM + i * 16 + (lane >> 4) * 4 + q;
                if (r >= rows)
                    continue;
                uint16_t* hrow = H + (int64_t)(row0 + r) * g.f;
#pragma unroll
                for (int j = 0; j < NI; j += 2) {
                    const int wrow = nt * BN + wn * WN + j * 16;  // first gate row of the pair
                    const int col = wrow / 2 + (lane & 15);
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
            for (int q = 0; q < 4; ++q) {
                const int r = wm * WM + i * 16 + (lane >> 4) * 4 + q;
                if (r >= rows)
                    continue;
                const int p = row0 + r;
                float* yrow = Ys + ((int64_t)g.perm[p] * g.k + g.perm_slot[p]) * g.d;
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    yrow[nt * BN + wn * WN + j * 16 + (lane & 15)] = acc[i][j][q];
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

__global__ void interleave_gate_up_kernel(const uint8_t* wg, const uint8_t* wu, uint8_t* wgu, int E,
                                          int f, int64_t row_bytes)
{
    // wgu[e][r] = (r % 32 < 16 ? wg : wu)[e][(r / 32) * 16 + r % 16], whole rows.
    const int64_t rows = (int64_t)E * 2 * f;
    const int64_t words = row_bytes / 16;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < rows * words;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t R = idx / words, w = idx % words;
        const int64_t e = R / (2 * f), r = R % (2 * f);
        const int64_t src_row = e * f + (r / 32) * 16 + (r % 16);
        const uint8_t* src = ((r % 32) < 16 ? wg : wu) + src_row * row_bytes;
        ((Vec16*)(wgu + R * row_bytes))[w] = ((const Vec16*)src)[w];
    }
}

}  // namespace

// Tile shapes: 256x256 output tiles, 4 waves of 128x128 (256 fp32 accumulators
// per lane, held in AGPRs), 2 x 64 KiB LDS stages: one workgroup per CU. When
// the weight-row count is not a multiple of 256, 256x128 tiles (waves of
// 128x64) are used instead.
constexpr int kBM = 256, kGN = 8;

template <bool GATE_UP>
hipError_t launch_grouped(const GemmArgs& a, hipStream_t s)
{
    const int N = GATE_UP ? 2 * a.f : a.d;
    const int mt = m_tile_bound<kBM>(a.A_max, a.E);
    if (N % 256 == 0)
        hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 256, 128, 128, kGN, GATE_UP>), dim3(mt * (N / 256)),
                           dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 128, 128, 64, kGN, GATE_UP>), dim3(mt * (N / 128)),
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

hipError_t launch_interleave_gate_up(const void* wg, const void* wu, void* wgu, int E, int f, int d,
                                     int esize, hipStream_t s)
{
    hipLaunchKernelGGL(interleave_gate_up_kernel, dim3(1024), dim3(256), 0, s, (const uint8_t*)wg,
                       (const uint8_t*)wu, (uint8_t*)wgu, E, f, (int64_t)d * esize);
    return hipGetLastError();
}

}  // namespace cmoe
