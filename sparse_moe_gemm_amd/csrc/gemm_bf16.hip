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
constexpr int kBK = 32;            // k per LDS stage
constexpr int kCH = kBK / 8;       // 16-byte chunks per A row per stage
constexpr int kNBUF = 4;           // LDS ring of stages
constexpr int kDIST = 3;           // stages in flight ahead of the one being multiplied
constexpr int kXCD = 8;

// XOR swizzle of the 16-byte chunk index inside an A row of the LDS stage:
// the 16 lanes that read one chunk column of 16 consecutive rows (rows are 64 B
// apart) land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk)
{
    return chunk ^ ((row >> 2) & 3);
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

// LDS stage layout (one 32-wide K stage of a 256 x 256 tile):
//   A: BM rows x 4 chunks of 16 B (8 bf16), chunk index swizzled per row;
//   B: BN/32 x 2 blocks of 1 KiB, each a 32-row x 16-k weight block in MFMA
//      operand order (lane l's 8 values at l*16 B), copied whole from the
//      blocked weight layout.
// Both are filled with direct global->LDS loads (global_load_lds_dwordx4: 64
// lanes x 16 B into 1 KiB of LDS, lane s into slot s); no VGPR staging.
template <int BM, int BN>
struct Stage {
    Vec16 a[BM * kCH];
    Vec16 b[(BN / 32) * 2 * 64];
};

// One direct global->LDS load: 64 lanes x 16 B from per-lane addresses into
// the 1 KiB of LDS at the wave-uniform address lds (through M0). Written as
// inline assembly on purpose: the ordering of these LDS writes against the
// LDS reads of other stages is handled explicitly (vmcnt wait + barrier at
// each stage), and an opaque instruction keeps the compiler from inserting
// its own conservative full waits before every LDS read, which would drain the
// stages in flight. Nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds)
{
    const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_void_t*)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(a)
                 : "memory");
}

// This wave's share of one stage's loads: A_INS instructions of 16 A rows each
// and B_INS whole weight blocks.
template <int BM, int BN, int A_INS, int B_INS>
__device__ __forceinline__ void issue_stage(const uint16_t* A, const uint32_t (&aoff)[A_INS], const Vec16* bsrc,
                                            int KB, int kt, Stage<BM, BN>* st, int wv)
{
#pragma unroll
    for (int i = 0; i < A_INS; ++i)
        dma16(A + aoff[i] + kt * kBK, st->a + (wv * A_INS + i) * 64);
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int blk = wv * B_INS + i;  // = row block * 2 + k block within the stage
        dma16(bsrc + ((int64_t)(blk >> 1) * KB + kt * 2 + (blk & 1)) * 64, st->b + blk * 64);
    }
}

// Scheduling pins: R LDS reads spread evenly between M MFMAs (mask 0x008 =
// MFMA, 0x100 = LDS read, 0x010 = global load, as the sched_group_barrier
// builtin defines them).
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

// MFMA work on one stage (two 16-wide k steps of 32x32x16 MFMAs). PARTIAL
// tiles (the last m-tile of an expert) skip the A reads and MFMAs of 32-row
// groups that hold no valid row. For full tiles the order is pinned: the
// NLOAD global loads issued just before, the first k step's fragment reads,
// its MFMAs with the second step's reads spread over their first half, then
// the second step's MFMAs.
template <int BM, int BN, int WM, int WN, bool PARTIAL, int NLOAD>
__device__ __forceinline__ void mfma_stage(const Stage<BM, BN>* st, int wm, int wn, int lane, int mi_lim,
                                           floatx16 (&acc)[WM / 32][WN / 32])
{
    constexpr int MI = WM / 32, NI = WN / 32, KS = kBK / 16;
    const int lr = lane & 31;
    bf16x8 afr[KS][MI], bfr[KS][NI];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 2 + (lane >> 5);
        const int col = c ^ ((lr >> 2) & 3);  // swz() of a row whose low 5 bits are lr
#pragma unroll
        for (int j = 0; j < NI; ++j)
            bfr[ks][j] = as_bf16x8(st->b[((wn * NI + j) * 2 + ks) * 64 + lane]);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if (PARTIAL && i >= mi_lim)
                continue;
            afr[ks][i] = as_bf16x8(st->a[(wm * WM + i * 32 + lr) * kCH + col]);
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
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
        }
    }
    if constexpr (!PARTIAL) {
        constexpr int R = MI + NI;  // fragment reads per k step
        constexpr int M = MI * NI;  // MFMAs per k step
        if constexpr (NLOAD > 0)
            __builtin_amdgcn_sched_group_barrier(0x010, NLOAD, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
        sched_spread<R, M / 2, 0>();
        __builtin_amdgcn_sched_group_barrier(0x008, M - M / 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    }
}

// Wait until at most N of this wave's loads are still in flight (the N most
// recently issued), then barrier: the stage about to be multiplied has landed
// for every wave, and every wave is done with the stage multiplied before.
// The scheduling barrier keeps MFMAs of the previous stage from moving across.
template <int N>
__device__ __forceinline__ void wait_loads_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    __syncthreads();
}

// The K loop of one tile: a ring of kNBUF LDS stages with kDIST stages in
// flight ahead of the one being multiplied, one barrier per stage. (A single
// copy of the MFMA code in the loop keeps the accumulators in place.)
template <int BM, int BN, int WM, int WN, int A_INS, int B_INS, bool PARTIAL>
__device__ __forceinline__ void tile_k_loop(const uint16_t* A, const uint32_t (&aoff)[A_INS], const Vec16* bsrc,
                                            int KB, int KT, Stage<BM, BN>* ring, int wv, int wm, int wn, int lane,
                                            int mi_lim, floatx16 (&acc)[WM / 32][WN / 32])
{
    constexpr int PER = A_INS + B_INS;  // loads per wave per stage
    static_assert(kDIST == 3 && kNBUF >= kDIST + 1, "ring layout");
#pragma unroll
    for (int s = 0; s < kDIST; ++s)
        if (s < KT)
            issue_stage<BM, BN, A_INS, B_INS>(A, aoff, bsrc, KB, s, &ring[s], wv);
    for (int kt = 0; kt < KT; ++kt) {
        const int ahead = KT - 1 - kt;  // stages after this one, already issued up to kDIST - 1
        if (ahead >= 2)
            wait_loads_barrier<2 * PER>();
        else if (ahead == 1)
            wait_loads_barrier<PER>();
        else
            wait_loads_barrier<0>();
        if (kt + kDIST < KT)
            issue_stage<BM, BN, A_INS, B_INS>(A, aoff, bsrc, KB, kt + kDIST, &ring[(kt + kDIST) % kNBUF], wv);
        mfma_stage<BM, BN, WM, WN, PARTIAL, 0>(&ring[kt % kNBUF], wm, wn, lane, mi_lim, acc);
    }
}

template <int BM, int BN, int WM, int WN, bool GATE_UP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_kernel(GemmArgs g)
{
    constexpr int WAVES_N = BN / WN;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int A_INS = BM * kCH / 64 / 4;      // A direct-load instructions per wave per stage
    constexpr int B_INS = (BN / 32) * 2 / 4;      // weight blocks per wave per stage
    static_assert((BM / WM) * WAVES_N == kThreads / kWave, "4 waves");
    static_assert(A_INS * 4 * 16 == BM && B_INS * 4 == (BN / 32) * 2, "stage split over 4 waves");
    static_assert(!GATE_UP || (NI % 2 == 0 && WN % 64 == 0), "gate/up pairs per wave");

    __shared__ Stage<BM, BN> ring[kNBUF];
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

    // A: per-lane source offsets (elements) of this wave's 16-row groups. Rows
    // are gathered through perm for gate/up; rows past the segment end are
    // clamped to its last row (their results are never stored).
    const uint16_t* A = (const uint16_t*)g.a;
    uint32_t aoff[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int r = (wv * A_INS + i) * 16 + lane / 4;  // slot lane of this instruction
        const int p = row0 + min(r, rows - 1);
        const int src = GATE_UP ? g.perm[p] : p;
        aoff[i] = (uint32_t)src * (uint32_t)K + (uint32_t)(swz(r, lane % 4) * 8);
    }
    // B: this lane's slot in the tile's first weight block.
    const Vec16* bsrc = (const Vec16*)g.b + ((int64_t)e * (N / 32) + (int64_t)nt * (BN / 32)) * KB * 64 + lane;

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
        tile_k_loop<BM, BN, WM, WN, A_INS, B_INS, false>(A, aoff, bsrc, KB, KT, ring, wv, wm, wn, lane, MI, acc);
    else
        tile_k_loop<BM, BN, WM, WN, A_INS, B_INS, true>(A, aoff, bsrc, KB, KT, ring, wv, wm, wn, lane,
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
