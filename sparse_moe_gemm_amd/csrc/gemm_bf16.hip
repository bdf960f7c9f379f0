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

template <int BM, int BN, int WM, int WN, int GN, bool GATE_UP>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs g)
{
    constexpr int WAVES_N = BN / WN;
    constexpr int MI = WM / 16, NI = WN / 16;
    constexpr int A_LD = BM * kCH / kThreads;  // 16-byte chunks per thread per stage
    constexpr int B_LD = BN * kCH / kThreads;
    static_assert((BM / WM) * (BN / WN) == kThreads / kWave, "4 waves");
    static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for one load per thread");
    static_assert(!GATE_UP || (NI % 2 == 0 && WN % 32 == 0), "gate/up pairs per wave");

    __shared__ Vec16 sA[2][BM * kCH];
    __shared__ Vec16 sB[2][BN * kCH];
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

    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int wm = wv / WAVES_N, wn = wv % WAVES_N;

    // Global sources of this thread's chunks (A rows gathered through perm for
    // gate/up; rows past the segment end are clamped to its last row and their
    // results are never stored).
    const uint16_t* ga[A_LD];
    int la[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int id = tid + i * kThreads, r = id / kCH, c = id % kCH;
        const int p = row0 + min(r, rows - 1);
        const int src = GATE_UP ? g.perm[p] : p;
        ga[i] = (const uint16_t*)g.a + (int64_t)src * K + c * 8;
        la[i] = r * kCH + swz(r, c);
    }
    const uint16_t* gb[B_LD];
    int lb[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int id = tid + i * kThreads, r = id / kCH, c = id % kCH;
        gb[i] = (const uint16_t*)g.b + ((int64_t)e * N + (int64_t)nt * BN + r) * K + c * 8;
        lb[i] = r * kCH + swz(r, c);
    }

    floatx4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    Vec16 ra[A_LD], rb[B_LD];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            ra[i] = *(const Vec16*)(ga[i] + k0);
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            rb[i] = *(const Vec16*)(gb[i] + k0);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            sA[buf][la[i]] = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            sB[buf][lb[i]] = rb[i];
    };

    const int KT = K / kBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT)
            gload((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            bf16x8 af[MI], bfg[NI];
            const int c = ks * 4 + (lane >> 4);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int r = wm * WM + i * 16 + (lane & 15);
                af[i] = as_bf16x8(sA[buf][r * kCH + swz(r, c)]);
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int r = wn * WN + j * 16 + (lane & 15);
                bfg[j] = as_bf16x8(sB[buf][r * kCH + swz(r, c)]);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfg[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT)
            lstore(buf ^ 1);
        __syncthreads();
    }

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

// Tile shapes of the first kernel generation: 128x128 tiles, 4 waves of 64x64.
constexpr int kBM = 128, kBN = 128, kWM = 64, kWN = 64, kGN = 4;

hipError_t launch_gate_up_bf16(const GemmArgs& a, hipStream_t s)
{
    const int NT = 2 * a.f / kBN;
    const int grid = m_tile_bound<kBM>(a.A_max, a.E) * NT;
    hipLaunchKernelGGL((grouped_gemm_kernel<kBM, kBN, kWM, kWN, kGN, true>), dim3(grid), dim3(kThreads), 0,
                       s, a);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const GemmArgs& a, hipStream_t s)
{
    const int NT = a.d / kBN;
    const int grid = m_tile_bound<kBM>(a.A_max, a.E) * NT;
    hipLaunchKernelGGL((grouped_gemm_kernel<kBM, kBN, kWM, kWN, kGN, false>), dim3(grid), dim3(kThreads), 0,
                       s, a);
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
