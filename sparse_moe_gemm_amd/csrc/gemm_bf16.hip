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
// inline assembly on purpose: the ordering of these LDS writes against the LDS
// reads of other stages is handled explicitly (a vmcnt wait and a barrier per
// stage), and an opaque instruction keeps the compiler from adding its own
// full waits before LDS reads, which would drain the stages in flight.
// Nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds)
{
    const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_void_t*)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(a)
                 : "memory");
}

// This wave's share of one stage's loads: A_INS instructions of 16 A rows each,
// then B_INS whole weight blocks; instruction q is issued by issue(q, ...).
template <int BM, int BN, int A_INS, int B_INS>
struct StageLoader {
    const uint16_t* A;
    const uint32_t* aoff;
    const Vec16* bsrc;
    int KB, wv;

    __device__ __forceinline__ void issue(int q, int kt, Stage<BM, BN>* st) const
    {
        if (q < A_INS) {
            dma16(A + aoff[q] + kt * kBK, st->a + (wv * A_INS + q) * 64);
        } else {
            const int blk = wv * B_INS + (q - A_INS);  // = row block * 2 + k block within the stage
            dma16(bsrc + ((int64_t)(blk >> 1) * KB + kt * 2 + (blk & 1)) * 64, st->b + blk * 64);
        }
    }
    __device__ __forceinline__ void issue_all(int kt, Stage<BM, BN>* st) const
    {
#pragma unroll
        for (int q = 0; q < A_INS + B_INS; ++q)
            issue(q, kt, st);
    }
};

// One stage: wait for its loads and barrier, then its MFMAs (two 16-wide k
// steps of 32x32x16) while this wave's loads of a later stage are issued.
// Full tiles use a fixed, hand-placed instruction order (sched_barrier
// between the pieces keeps the compiler's scheduler from regrouping them):
// the first k step's fragment reads; then its MFMAs with the second step's
// reads after every other MFMA and a global load after every fourth; then
// the second step's MFMAs with the remaining loads. No wave ever issues a
// burst of memory instructions while its matrix pipe sits idle.
// PARTIAL tiles (the last m-tile of an expert) skip the A reads and MFMAs of
// 32-row groups that hold no valid row, and issue their loads up front.
template <int BM, int BN, int WM, int WN, int A_INS, int B_INS, bool PARTIAL>
__device__ __forceinline__ void stage_step(const StageLoader<BM, BN, A_INS, B_INS>& ld, int kt_load,
                                           Stage<BM, BN>* ld_st, const Stage<BM, BN>* st, int wm, int wn,
                                           int lane, int mi_lim, floatx16 (&acc)[WM / 32][WN / 32])
{
    constexpr int MI = WM / 32, NI = WN / 32, KS = kBK / 16;
    constexpr int NLD = A_INS + B_INS;
    static_assert(KS == 2, "two k steps per stage");
    // Stage kt landed for this wave once at most two later stages (2 * NLD
    // loads) are in flight; the barrier makes that true for every wave and
    // frees the buffer the later stage is loaded into. (A bare s_barrier: a
    // __syncthreads() fence would wait for all loads in flight.)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NLD) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    const int lr = lane & 31;
    auto read_a = [&](int ks, int i) {
        const int c = ks * 2 + (lane >> 5);
        return as_bf16x8(st->a[(wm * WM + i * 32 + lr) * kCH + (c ^ ((lr >> 2) & 3))]);
    };
    auto read_b = [&](int ks, int j) { return as_bf16x8(st->b[((wn * NI + j) * 2 + ks) * 64 + lane]); };

    if constexpr (PARTIAL) {
        ld.issue_all(kt_load, ld_st);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 bfr[NI];
#pragma unroll
            for (int j = 0; j < NI; ++j)
                bfr[j] = read_b(ks, j);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (i >= mi_lim)
                    continue;
                const bf16x8 a = read_a(ks, i);
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfr[j], acc[i][j], 0, 0, 0);
            }
        }
    } else {
        constexpr int M = MI * NI;  // MFMAs per k step
        constexpr int R = MI + NI;  // fragment reads per k step
        constexpr int L0 = NLD / 2; // loads placed in the first k step, the rest in the second
        bf16x8 f0a[MI], f0b[NI], f1a[MI], f1b[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j)
            f0b[j] = read_b(0, j);
#pragma unroll
        for (int i = 0; i < MI; ++i)
            f0a[i] = read_a(0, i);
        __builtin_amdgcn_sched_barrier(0);
        int nread = 0, nld = 0;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int i = m / NI, j = m % NI;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0a[i], f0b[j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            // spread: after MFMA m, reads up to ceil((m+1) R / M), loads up to (m+1) L0 / M
#pragma unroll
            for (; nread < ((m + 1) * R + M - 1) / M; ++nread) {
                if (nread < NI)
                    f1b[nread] = read_b(1, nread);
                else
                    f1a[nread - NI] = read_a(1, nread - NI);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (; nld < ((m + 1) * L0) / M; ++nld) {
                ld.issue(nld, kt_load, ld_st);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int i = m / NI, j = m % NI;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1a[i], f1b[j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (; nld < L0 + ((m + 1) * (NLD - L0)) / M; ++nld) {
                ld.issue(nld, kt_load, ld_st);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (; nld < NLD; ++nld)
            ld.issue(nld, kt_load, ld_st);
    }
}

// The K loop of one tile: a ring of four LDS stages (separate arrays, so the
// compiler can tell them apart) with three stages in flight ahead of the one
// being multiplied, one barrier per stage. Requires KT % 4 == 0. Stages past
// the end are replaced by reloads of the last stage, which keeps the number of
// loads per stage, and so every wait count, the same.
template <int BM, int BN, int WM, int WN, int A_INS, int B_INS, bool PARTIAL>
__device__ __forceinline__ void tile_k_loop(const StageLoader<BM, BN, A_INS, B_INS>& ld, int KT,
                                            Stage<BM, BN>* s0, Stage<BM, BN>* s1, Stage<BM, BN>* s2,
                                            Stage<BM, BN>* s3, int wm, int wn, int lane, int mi_lim,
                                            floatx16 (&acc)[WM / 32][WN / 32])
{
    ld.issue_all(0, s0);
    ld.issue_all(1, s1);
    ld.issue_all(2, s2);
    const int last = KT - 1;
    for (int kt = 0; kt < KT; kt += 4) {
        stage_step<BM, BN, WM, WN, A_INS, B_INS, PARTIAL>(ld, min(kt + 3, last), s3, s0, wm, wn, lane, mi_lim, acc);
        stage_step<BM, BN, WM, WN, A_INS, B_INS, PARTIAL>(ld, min(kt + 4, last), s0, s1, wm, wn, lane, mi_lim, acc);
        stage_step<BM, BN, WM, WN, A_INS, B_INS, PARTIAL>(ld, min(kt + 5, last), s1, s2, wm, wn, lane, mi_lim, acc);
        stage_step<BM, BN, WM, WN, A_INS, B_INS, PARTIAL>(ld, min(kt + 6, last), s2, s3, wm, wn, lane, mi_lim, acc);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the trailing reloads
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

    __shared__ Stage<BM, BN> st0, st1, st2, st3;
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

    const int KT = K / kBK;  // a multiple of 4 (K % 128 == 0)
    const StageLoader<BM, BN, A_INS, B_INS> ld{A, aoff, bsrc, KB, wv};
    if (rows == BM)
        tile_k_loop<BM, BN, WM, WN, A_INS, B_INS, false>(ld, KT, &st0, &st1, &st2, &st3, wm, wn, lane, MI, acc);
    else
        tile_k_loop<BM, BN, WM, WN, A_INS, B_INS, true>(ld, KT, &st0, &st1, &st2, &st3, wm, wn, lane,
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
