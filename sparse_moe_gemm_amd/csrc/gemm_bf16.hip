// gemm_bf16.hip - grouped expert GEMMs on bf16 MFMA (gfx950).
//
// The expert GEMMs of «Colibri 是什么» (xxqk.cn) §2.3 (one GEMM kernel over the
// experts' row-major weights) in the batched form of «Colibri不是一只蜂鸟»
// (discosf.com) §1 and §3.2 (one fused launch over all active experts, the
// SiLU epilogue inlined into the first GEMM), with weight tiles staged in
// shared memory (LDS) as §5.1 of that page describes.
//
//   gate/up:  H[p][c]    = SiLU(sum_i X[perm[p]][i] Wg[e][c][i]) * (sum_i X[perm[p]][i] Wu[e][c][i])
//   down:     Ys_s[p][o] = sum_{c in K split s} H[p][c] Wd[e][o][c]
// for every sorted position p of expert e's segment [offsets[e], offsets[e+1]).
//
// Operands: v_mfma_f32_32x32x16_bf16 (it keeps the matrix pipe full from a
// single wave per SIMD) takes, from lane l, 8 consecutive k of row l%32 of A
// and of B. Init stores the weights pre-blocked in MFMA operand order (32 rows
// x 16 k per 1 KiB block, lane-major). For every 32-wide K stage of a tile the
// token rows (A; gathered through perm for gate/up) and whole weight blocks
// (B) are copied into LDS by gfx950's buffer->LDS loads, which use no VGPRs
// and whose addressing is scalar apart from one per-lane offset; the waves
// read their fragments from LDS with 16-byte reads. Gate and up weights are
// interleaved in blocks of 32 rows, so each wave holds the gate and up
// accumulators of the same outputs and applies SiLU(g)*u in registers.
//
// Work decomposition: a tile is (expert, m-tile of BM sorted rows, n-tile of
// BN weight rows, K split). Experts with no rows have no tiles, so their
// weights are never read. The kernel is persistent: one workgroup per compute
// unit takes tiles blockIdx.x, + gridDim.x, ... and runs all their K stages as
// one stream through a ring of five LDS stages, so the first stages of the
// next tile load while the current one finishes and writes its outputs. The
// tile count depends on the routing and lives on the device: every wave
// derives it, and the tile behind an index, from offsets[] held in registers.
// Tiles are ordered expert -> split -> group of GN n-tiles -> m-tile ->
// n-tile; workgroups are spread over the 8 XCDs round robin, so the tiles one
// XCD runs together share a few token and weight panels in its L2.
#include "common.hpp"
#include "tiles.hpp"

namespace cmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;                 // k per LDS stage
constexpr int kCH = kBK / 8;            // 16-byte chunks per A row per stage
constexpr int kRing = 5;                // LDS stages in the ring
constexpr int kAhead = kRing - 1;       // stages in flight ahead of the one multiplied

// XOR swizzle of the 16-byte chunk index inside an A row of the LDS stage:
// the 16 lanes that read one chunk column of 16 consecutive rows (rows are 64 B
// apart) land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk)
{
    return chunk ^ ((row >> 2) & 3);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// SiLU with the hardware reciprocal (about 1 ulp) instead of an IEEE divide;
// the result is rounded to bf16 right after.
__device__ __forceinline__ float silu_rcp(float z)
{
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(size_t)(lds_void_t*)p;
}

// LDS stage layout (one 32-wide K stage of a BM x BN tile):
//   A: BM rows x 4 chunks of 16 B (8 bf16), chunk index swizzled per row;
//   B: bf16 weights: BN/32 x 2 blocks of 1 KiB, each a 32-row x 16-k weight
//      block in MFMA operand order (lane l's 8 values at l*16 B); fp8 weights
//      (F8): BN/32 blocks of 1 KiB, each 32 rows x 32 k (lane l's 16 codes
//      at l*16 B: k 16*(l/32) .. +16, 8 for each 16-wide k step); either way
//      copied whole from the blocked weight layout.
template <int BM, int BN, bool F8>
struct Stage {
    Vec16 a[BM * kCH];
    Vec16 b[(BN / 32) * (F8 ? 1 : 2) * 64];
};
// The ring of stages; with fp8 weights the epilogues that stage bf16 rows
// (gate/up, and the down GEMM's bf16 outputs) have a buffer of their own (a
// 24 KiB slot is too small for them).
template <int BM, int BN, bool F8, bool EPBUF>
struct Ring {
    Stage<BM, BN, F8> st[kRing];
};
template <int BM, int BN, bool F8>
struct Ring<BM, BN, F8, true> {
    Stage<BM, BN, F8> st[kRing];
    float ep[4 * 2048];
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// B fragment as read from LDS (bf16x8 values, or 8 fp8 codes) and as the MFMA
// takes it: fp8 codes become bf16 times the row's scale 2^e, which is exact.
template <bool F8>
struct BFrag {
    typedef bf16x8 raw;
};
template <>
struct BFrag<true> {
    typedef u32x2 raw;
};
__device__ __forceinline__ bf16x8 to_bf16(bf16x8 r, float)
{
    return r;
}
__device__ __forceinline__ bf16x8 to_bf16(u32x2 r, float sc)
{
    return fp8x8_to_bf16(r[0], r[1], sc);
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource of a raw byte buffer: base address, size in bytes (loads
// past it return zeros instead of touching memory), stride 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int32_t)((a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
    r[3] = 0x00020000;  // raw buffer, 32-bit data format (CDNA)
    return r;
}

// One direct buffer->LDS load: 64 lanes x 16 B from rsrc + voff (per lane) +
// soff (wave-uniform) into the 1 KiB of LDS at byte address lds (through M0),
// lane s into slot s. Written as inline assembly on purpose: the ordering of
// these LDS writes against the LDS reads of other stages is handled
// explicitly (vmcnt waits and barriers), and an opaque instruction keeps the
// compiler from adding its own full waits before LDS reads, which would drain
// the stages in flight. M0 is declared clobbered, so the compiler keeps none of
// its own values there across the load.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(soff), "s"(lds)
                 : "memory", "m0");
}

// Where the loads of one stage come from: the tile's weight panel, the
// per-lane byte offsets of its A rows (chunk included) and the k stage.
template <int A_INS>
struct LoadSrc {
    i32x4 rb;
    uint32_t aoff[A_INS];
    int kt;
};

// Load q of this wave's share of one stage into the stage at LDS byte address
// lds: A_INS instructions of 16 A rows each, then B_INS whole weight blocks.
// KB is the number of 1 KiB blocks per 32 weight rows along K (K/16 for bf16
// weights, K/32 for fp8).
template <int BM, int BN, bool F8, int A_INS, int B_INS>
__device__ __forceinline__ void issue_load(int q, const i32x4& ra, const LoadSrc<A_INS>& ls, int KB, int wv,
                                           uint32_t lane16, uint32_t lds)
{
    using St = Stage<BM, BN, F8>;
    constexpr uint32_t kOffA = (uint32_t)offsetof(St, a);
    constexpr uint32_t kOffB = (uint32_t)offsetof(St, b);
    if (q < A_INS) {
        dma16(ra, ls.aoff[q], (uint32_t)ls.kt * (kBK * 2), lds + kOffA + (uint32_t)(wv * A_INS + q) * 1024u);
    } else {
        const int blk = wv * B_INS + (q - A_INS);
        uint32_t soff;
        if constexpr (F8)  // blk = row block
            soff = ((uint32_t)blk * (uint32_t)KB + (uint32_t)ls.kt) * 1024u;
        else  // blk = row block * 2 + k block within the stage
            soff = ((uint32_t)(blk >> 1) * (uint32_t)KB + (uint32_t)ls.kt * 2u + (uint32_t)(blk & 1)) * 1024u;
        dma16(ls.rb, lane16, soff, lds + kOffB + (uint32_t)blk * 1024u);
    }
}

// Fragment readers of one LDS stage for wave (wm, wn): A fragment i (rows
// wm*WM + i*32 ..) and B fragment j (weight rows wn*WN + j*32 ..) of k step ks.
template <int BM, int BN, int WM, int WN, bool F8>
struct FragReader {
    const Stage<BM, BN, F8>* st;
    int wm, wn, lane;
    __device__ __forceinline__ bf16x8 a(int ks, int i) const
    {
        const int lr = lane & 31;
        // k order inside a 32-wide stage: bf16 weights step-major (k step ks,
        // lane half lane/32 holds 8 k); 8-bit weights lane-half-major (lane
        // half lane/32 holds 16 consecutive k, 8 per k step), the order of the
        // 8-bit weight layout. Any order works if A and B agree.
        const int c = F8 ? (lane >> 5) * 2 + ks : ks * 2 + (lane >> 5);
        return as_bf16x8(st->a[(wm * WM + i * 32 + lr) * kCH + (c ^ ((lr >> 2) & 3))]);
    }
    __device__ __forceinline__ typename BFrag<F8>::raw b(int ks, int j) const
    {
        if constexpr (F8)
            return ((const u32x2*)st->b)[((wn * (WN / 32) + j) * 64 + lane) * 2 + ks];
        else
            return as_bf16x8(st->b[((wn * (WN / 32) + j) * 2 + ks) * 64 + lane]);
    }
};

// One K stage, software-pipelined so that the matrix pipe never waits on a
// barrier or on a fragment read:
//   first half:  MFMAs of k step 0 (fragments fa/fb, read during the previous
//                stage); the reads of k step 1's fragments spread over its
//                first half; half of this wave's loads of the stage kAhead
//                later spread over all of it.
//   middle:      wait for those reads and until the next stage has landed for
//                this wave, then barrier. After it every wave has landed the
//                next stage and has finished every read of this stage and of
//                all earlier ones.
//   second half: MFMAs of k step 1; the reads of the NEXT stage's k step 0
//                fragments into fa/fb; the other half of the loads.
// The loads issued in stage s fill the ring slot of stage s-1, whose last
// reads completed before the middle barrier of stage s-1. The wait count is
// exact: loads complete in issue order, and when the middle of stage s is
// reached, the loads issued after those of stage s+1 are the ones of stages
// s+2 and s+3 and the first half of stage s+4's. The instruction order is
// fixed by hand (sched_barrier between the pieces keeps the compiler's
// scheduler from regrouping them).
// The last m-tile of an expert: its rows past the segment end repeat the
// last valid row (their results are stored to that row again, same values);
// 32-row groups made only of such rows are skipped (below).
// With fp8 weights (F8) the B fragments are read as 8 codes each and turned
// into bf16 (row scale sc[j]) in the shadow of the MFMA before their first use.
// Only the wave's first RG 32-row groups hold rows of the tile (RG < WM/32 in
// an expert's last, partial m-tile): the MFMAs of the other groups, and the
// reads of their k step 1 fragments, are left out. Loads, waits, barriers and
// the next stage's fragment reads are the same in every variant.
template <int BM, int BN, int WM, int WN, bool F8, int A_INS, int B_INS, int RG>
__device__ __forceinline__ void stage(const i32x4& ra, const LoadSrc<A_INS>& ls, uint32_t ld_lds, int KB, int wv,
                                      uint32_t lane16, const Stage<BM, BN, F8>* st,
                                      const Stage<BM, BN, F8>* st_next, int wm, int wn, int lane,
                                      bf16x8 (&fa)[WM / 32], typename BFrag<F8>::raw (&fb)[WN / 32],
                                      const float (&sc)[WN / 32], floatx16 (&acc)[WM / 32][WN / 32])
{
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int NLD = A_INS + B_INS;
    constexpr int M = MI * NI;   // MFMAs per k step
    constexpr int R = MI + NI;   // fragment reads per k step
    constexpr int RS = M / 2;    // reads are spread over the first RS MFMAs
    constexpr int L0 = NLD / 2;  // loads in the first half
    static_assert(kBK == 32, "two k steps per stage");
    const FragReader<BM, BN, WM, WN, F8> rd{st, wm, wn, lane}, rn{st_next, wm, wn, lane};
    bf16x8 ga[MI];
    typename BFrag<F8>::raw gb[NI];
    bf16x8 cb[NI];

    int nread = 0, nld = 0;
    if constexpr (RG > 0)
        cb[0] = to_bf16(fb[0], sc[0]);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int i = m / NI, j = m % NI;
        if (i < RG)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], cb[j], acc[i][j], 0, 0, 0);
        if (RG > 0 && i == 0 && j + 1 < NI)
            cb[j + 1] = to_bf16(fb[j + 1], sc[j + 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (; nread < R && nread < ((m + 1) * R + RS - 1) / RS; ++nread) {
            if (nread < NI)
                gb[nread] = rd.b(1, nread);
            else if (nread - NI < RG)
                ga[nread - NI] = rd.a(1, nread - NI);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (; nld < ((m + 1) * L0) / M; ++nld) {
            issue_load<BM, BN, F8, A_INS, B_INS>(nld, ra, ls, KB, wv, lane16, ld_lds);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(%0)" ::"n"(2 * NLD + L0) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    nread = 0;
    if constexpr (RG > 0)
        cb[0] = to_bf16(gb[0], sc[0]);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int i = m / NI, j = m % NI;
        if (i < RG)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[i], cb[j], acc[i][j], 0, 0, 0);
        if (RG > 0 && i == 0 && j + 1 < NI)
            cb[j + 1] = to_bf16(gb[j + 1], sc[j + 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (; nread < R && nread < ((m + 1) * R + RS - 1) / RS; ++nread) {
            if (nread < NI)
                fb[nread] = rn.b(0, nread);
            else
                fa[nread - NI] = rn.a(0, nread - NI);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (; nld < L0 + ((m + 1) * (NLD - L0)) / M; ++nld) {
            issue_load<BM, BN, F8, A_INS, B_INS>(nld, ra, ls, KB, wv, lane16, ld_lds);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 weights on v_mfma_f32_16x16x32_bf16 (M16 path): one MFMA k step per
// 32-wide K stage. A wave's 128 x 128 block is 8 x 8 MFMA blocks of 16 x 16;
// Acc4 holds the four 16x16 blocks of one 32x32 region, q[2*ri + cj] for
// rows 16*ri .. and columns 16*cj ... Fragment lanes: a token-row fragment's
// lane l holds row l%16 and k 8*(l/16) .. +8 (chunk l/16 of the stage's A
// row), a weight fragment's lane l the same k of weight row l%16. With the
// token fragment as the MFMA's first operand (SW false) lane l of a result
// block holds output column l%16 of token rows 4*(l/16) + q; with the weight
// fragment first (SW true) the block is transposed: token row l%16, output
// columns 4*(l/16) + q. The products and their order are the same either
// way, and so are the results, bit for bit. Per
// element of work this shape moves half the accumulator registers of the
// 32x32x16 shape, which saves power in a power-bound loop.
struct Acc4 {
    floatx4 q[4];
};

// Epilogues of the M16 path on transposed blocks (SW): lane l holds token row
// l%16 and the four consecutive output columns 4*(l/16) .. +3 of each 16x16
// block, so it can store its own row segment without a trip through LDS.
// bf16_pair: two fp32 values as two bf16 in one register, first in the low half.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b)
{
    return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

// Row segment of 8 bf16 from the two 16x16 blocks of a 32-column block (c0:
// columns 0..15, c1: 16..31; lo/hi: the lane's columns 0,1 and 2,3 of its
// four). One v_permlane16_swap per register pair trades the odd 16-lane rows
// of c0 for the even rows of c1: afterwards lanes of an even row group g hold
// columns 4g .. 4g+7 (their own four of c0, then those of lane l+16), lanes of
// an odd group columns 16 + 4(g-1) .. +7 (lane l-16's four of c1, then their
// own), i.e. 8 consecutive columns starting at row8_col(lane).
__device__ __forceinline__ Vec16 row8(uint32_t c0lo, uint32_t c0hi, uint32_t c1lo, uint32_t c1hi)
{
    const auto lo = __builtin_amdgcn_permlane16_swap(c0lo, c1lo, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(c0hi, c1hi, false, false);
    return Vec16{lo[0], hi[0], lo[1], hi[1]};
}

// An accumulator block read out of its AGPRs where the epilogue uses it (the
// vector ALU cannot take AGPR operands; left to itself the compiler copies
// every accumulator to VGPRs at the start of the epilogue, which spills).
__device__ __forceinline__ floatx4 acc_read(const floatx4& a)
{
    floatx4 r;
    asm volatile("v_accvgpr_read_b32 %0, %4\n\tv_accvgpr_read_b32 %1, %5\n\t"
                 "v_accvgpr_read_b32 %2, %6\n\tv_accvgpr_read_b32 %3, %7"
                 : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3])
                 : "a"(a[0]), "a"(a[1]), "a"(a[2]), "a"(a[3]));
    return r;
}

__device__ __forceinline__ int row8_col(int lane)
{
    const int g = lane >> 4;
    return 8 * (g >> 1) + 16 * (g & 1);
}

template <int BM, int BN, int WM, int WN>
struct FragReader16 {
    const Stage<BM, BN, false>* st;
    int wm, wn, lane;
    // A fragment of the wave's 16-row group i.
    __device__ __forceinline__ bf16x8 a(int i) const
    {
        const int r = wm * WM + i * 16 + (lane & 15);
        return as_bf16x8(st->a[r * kCH + swz(r, lane >> 4)]);
    }
    // B fragment of the wave's 16-row weight group j: weight row n of the
    // tile and k chunk c = lane/16 are lane slot n%32 + 32*(c%2) of the 1 KiB
    // block (n/32, 16-k step c/2).
    __device__ __forceinline__ bf16x8 b(int j) const
    {
        const int n = wn * WN + j * 16 + (lane & 15);
        const int c = lane >> 4;
        return as_bf16x8(st->b[((n >> 5) * 2 + (c >> 1)) * 64 + (n & 31) + 32 * (c & 1)]);
    }
};

// One K stage of the M16 path, software-pipelined like stage():
//   first half:  MFMAs of the upper row groups (0 .. MH-1), column-major,
//                with fragments read during the previous stage; the reads of
//                this stage's lower-row A fragments; half of the loads.
//   middle:      the same wait and barrier as stage().
//   second half: MFMAs of the lower row groups, column-major; right after a
//                column's last MFMA its B fragment is read again from the
//                NEXT stage, and the next stage's upper-row A fragments are
//                read first thing; the other half of the loads.
// Row groups (32 rows) past RG hold only padding: their MFMAs and their
// this-stage reads are left out; loads, waits and barriers are the same in
// every variant. Inside a partial tile (RG below all) the next stage has the
// same row groups, so its A fragments of padding groups are not read, nor,
// with RG = 0, its B fragments; only the tile's last stage (`last`, whose
// next stage starts the next tile) reads them all. An expert's ragged last
// m-tile then costs far fewer LDS reads than a full one.
template <int BM, int BN, int WM, int WN, int A_INS, int B_INS, int RG, bool SW>
__device__ __forceinline__ void stage16(const i32x4& ra, const LoadSrc<A_INS>& ls, uint32_t ld_lds, int KB, int wv,
                                        uint32_t lane16, const Stage<BM, BN, false>* st,
                                        const Stage<BM, BN, false>* st_next, int wm, int wn, int lane,
                                        bf16x8 (&fa)[WM / 16], bf16x8 (&fb)[WN / 16], Acc4 (&acc)[WM / 32][WN / 32],
                                        bool last)
{
    constexpr int MI = WM / 16, NI = WN / 16;  // 16-row and 16-column groups
    constexpr bool FULL = RG == WM / 32;       // every row group holds rows
    constexpr int MH = MI / 2;                 // row groups per half
    constexpr int NLD = A_INS + B_INS;
    constexpr int L0 = NLD / 2;                // loads in the first half
    constexpr int M = MH * NI;                 // MFMAs per half
    constexpr int RS = M / 2;                  // first-half reads spread over the first RS MFMAs
    const FragReader16<BM, BN, WM, WN> rd{st, wm, wn, lane}, rn{st_next, wm, wn, lane};

    int nread = 0, nld = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int j = m / MH, i = m % MH;
        if ((i >> 1) < RG) {
            floatx4& c = acc[i >> 1][j >> 1].q[(i & 1) * 2 + (j & 1)];
            c = SW ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], c, 0, 0, 0)
                   : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], c, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (; nread < MH && nread < ((m + 1) * MH + RS - 1) / RS; ++nread) {
            if (((MH + nread) >> 1) < RG)
                fa[MH + nread] = rd.a(MH + nread);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (; nld < ((m + 1) * L0) / M; ++nld) {
            issue_load<BM, BN, false, A_INS, B_INS>(nld, ra, ls, KB, wv, lane16, ld_lds);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(%0)" ::"n"(2 * NLD + L0) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int j = m / MH, i = MH + m % MH;
        if ((i >> 1) < RG) {
            floatx4& c = acc[i >> 1][j >> 1].q[(i & 1) * 2 + (j & 1)];
            c = SW ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], c, 0, 0, 0)
                   : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], c, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (m < MH && (FULL || (m >> 1) < RG || last)) {  // the upper-row A fragments are free after the first half
            fa[m] = rn.a(m);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (m % MH == MH - 1 && (RG > 0 || last)) {  // column j done
            fb[j] = rn.b(j);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (; nld < L0 + ((m + 1) * (NLD - L0)) / M; ++nld) {
            issue_load<BM, BN, false, A_INS, B_INS>(nld, ra, ls, KB, wv, lane16, ld_lds);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// ---------------------------------------------------------------------------
// 8-bit activations and weights (Q8): v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x
// E4M3, one 64-wide k step per stage. A stage has the bf16 stage's shape in
// bytes: A rows of 64 codes (four 16-byte chunks, swizzled as for bf16), and
// per 32 weight rows two 1 KiB blocks (k 0..31 and 32..63 of the stage in the
// 8-bit weight layout). The MFMA's lane l takes row l%32 and, in its 32
// bytes, k 16*(l/32) .. +16 of the first 32-k half and the same of the second:
// A chunks l/32 and 2 + l/32, and the lane's 16 bytes of both weight blocks.
// Each lane's operands are scaled by 2^(byte - 127) per operand (the rows'
// power-of-two scales, E8M0); products and sums are exact fp8 products summed
// in fp32.
typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i cat16(const Vec16& lo, const Vec16& hi)
{
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// E8M0 byte of a power-of-two fp32 scale (its biased exponent).
__device__ __forceinline__ int e8m0(float s)
{
    return (int)((__float_as_uint(s) >> 23) & 0xFFu);
}

template <int BM, int BN, int WM, int WN>
struct FragReaderQ8 {
    const Stage<BM, BN, false>* st;
    int wm, wn, lane;
    __device__ __forceinline__ v8i a(int i) const
    {
        const int lr = lane & 31, h = lane >> 5, sw = (lr >> 2) & 3;
        const Vec16* row = st->a + (wm * WM + i * 32 + lr) * kCH;
        return cat16(row[h ^ sw], row[(2 + h) ^ sw]);
    }
    __device__ __forceinline__ v8i b(int j) const
    {
        const int rb = wn * (WN / 32) + j;
        return cat16(st->b[(rb * 2) * 64 + lane], st->b[(rb * 2 + 1) * 64 + lane]);
    }
};

// One Q8 stage, pipelined like the bf16 one: first half = the MFMAs of the
// wave's first two 32-row groups (fragments read during the previous stage)
// while the other two groups' A fragments of this stage are read; middle =
// the same wait and barrier; second half = the last two row groups' MFMAs,
// ordered by weight block, each block's fragment re-read for the next stage
// as soon as its last MFMA is issued, then the next stage's first A
// fragments. Half of the loads in each half.
template <int BM, int BN, int WM, int WN, int A_INS, int B_INS, int RG>
__device__ __forceinline__ void stage_q8(const i32x4& ra, const LoadSrc<A_INS>& ls, uint32_t ld_lds, int KB, int wv,
                                         uint32_t lane16, const Stage<BM, BN, false>* st,
                                         const Stage<BM, BN, false>* st_next, int wm, int wn, int lane,
                                         v8i (&fa)[2], v8i (&fb)[WN / 32], const int (&sa)[WM / 32],
                                         const int (&sb)[WN / 32], floatx16 (&acc)[WM / 32][WN / 32])
{
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int NLD = A_INS + B_INS;
    constexpr int M = 2 * NI;    // MFMAs per half
    constexpr int L0 = NLD / 2;  // loads in the first half
    static_assert(MI == 4, "two row groups per half");
    const FragReaderQ8<BM, BN, WM, WN> rd{st, wm, wn, lane}, rn{st_next, wm, wn, lane};
    v8i ga[2];

    int nld = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int i = m / NI, j = m % NI;
        if (i < RG)
            acc[i][j] =
                __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
        __builtin_amdgcn_sched_barrier(0);
        if ((m == 0 && RG > 2) || (m == NI / 2 && RG > 3)) {
            ga[m == 0 ? 0 : 1] = rd.a(m == 0 ? 2 : 3);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (; nld < ((m + 1) * L0) / M; ++nld) {
            issue_load<BM, BN, false, A_INS, B_INS>(nld, ra, ls, KB, wv, lane16, ld_lds);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(%0)" ::"n"(2 * NLD + L0) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int j = m / 2, ii = m % 2;
        if (2 + ii < RG)
            acc[2 + ii][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga[ii], fb[j], acc[2 + ii][j], 0, 0, 0,
                                                                             sa[2 + ii], 0, sb[j]);
        __builtin_amdgcn_sched_barrier(0);
        if (ii == 1) {
            fb[j] = rn.b(j);
            __builtin_amdgcn_sched_barrier(0);
            if (j >= NI - 2) {
                fa[j - (NI - 2)] = rn.a(j - (NI - 2));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (; nld < L0 + ((m + 1) * (NLD - L0)) / M; ++nld) {
            issue_load<BM, BN, false, A_INS, B_INS>(nld, ra, ls, KB, wv, lane16, ld_lds);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The combine, fused into the down GEMM's epilogue: after a tile has stored
// its partial rows (rows row0 .. row0+rows of split s, columns n*BN .. +BN),
// each of them counts one arrival for its token and n-tile. The arrival that
// completes a count (k assignments times the K splits) finds every partial
// row of that token and n-tile stored, and its wave computes the token's
// columns of y exactly as the combine kernel does: partials added in split
// order (bf16 weights without a K split: each row rounded to bf16 first, as
// the unfused path stores it), weighted sum over the k slots in slot order
// (fused multiply-add in fp32), rounded to bf16. Which workgroup does it changes nothing in the
// result. Ordering: every wave's stores are released at device scope before
// the barrier after which the counts are incremented; a wave that completed
// counts acquires at device scope before it reads the other rows. Lane l of
// wave w counts tile row w*64 + l (BM = 256 rows, 4 waves).
template <int BN>
__device__ __forceinline__ void fused_combine(const GemmArgs& g, int row0, int rows, int n, int wv, int lane)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __builtin_amdgcn_s_barrier();
    const int NTd = g.d / BN;
    const int r = wv * kWave + lane;
    int t = 0;
    bool last = false;
    if (r < rows) {
        t = g.perm[row0 + r];
        const int old = __hip_atomic_fetch_add(g.cnt + (int64_t)t * NTd + n, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        last = old == g.k * g.split - 1;
    }
    uint64_t m = __ballot(last);
    if (m == 0)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // Lane b of a completed count fetches its token's k sorted positions and
    // weights (k <= kMaxTopK) at once; the wave then sums the tokens one by one with
    // all k*split row loads of a token in flight together.
    int pos[kMaxTopK];
    float wgt[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        const bool on = last && j < g.k;
        pos[j] = on ? g.inv[(int64_t)t * g.k + j] : 0;
        wgt[j] = on ? g.topw[(int64_t)t * g.k + j] : 0.f;
    }
    const float* Ys = (const float*)g.out;
    const int64_t stride = (int64_t)g.A_max * g.d;  // between K-split partials
    const int c = n * BN + min(lane * 4, BN - 4);   // this lane's 4 columns (BN / 4 lanes)
    while (m != 0) {
        const int b = __builtin_ctzll(m);
        m &= m - 1;
        const int tt = __builtin_amdgcn_readlane(t, b);
        float4 v[kMaxTopK][kMaxSplit];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            const int p = __builtin_amdgcn_readlane(pos[j], b);
            const float* row = Ys + (int64_t)p * g.d + c;
            v[j][0] = *(const float4*)row;
            v[j][1] = g.split > 1 ? *(const float4*)(row + stride) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j < g.k) {
                const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wgt[j]), b));
                float4 u = v[j][0];
                if (g.split == 1) {  // the values the unfused path stores as bf16 (no K split)
                    u.x = bf16_to_f32(f32_to_bf16_bits(u.x));
                    u.y = bf16_to_f32(f32_to_bf16_bits(u.y));
                    u.z = bf16_to_f32(f32_to_bf16_bits(u.z));
                    u.w = bf16_to_f32(f32_to_bf16_bits(u.w));
                }
                if (g.split > 1) {
                    u.x += v[j][1].x;
                    u.y += v[j][1].y;
                    u.z += v[j][1].z;
                    u.w += v[j][1].w;
                }
                acc.x = fmaf(wj, u.x, acc.x);
                acc.y = fmaf(wj, u.y, acc.y);
                acc.z = fmaf(wj, u.z, acc.z);
                acc.w = fmaf(wj, u.w, acc.w);
            }
        }
        if (lane * 4 < BN) {
            uint2 packed;
            packed.x = (uint32_t)f32_to_bf16_bits(acc.x) | ((uint32_t)f32_to_bf16_bits(acc.y) << 16);
            packed.y = (uint32_t)f32_to_bf16_bits(acc.z) | ((uint32_t)f32_to_bf16_bits(acc.w) << 16);
            *(uint2*)((uint16_t*)g.y + (int64_t)tt * g.d + c) = packed;
        }
        if (lane == 0)
            __hip_atomic_store(g.cnt + (int64_t)tt * NTd + n, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Buffer resource of a tile's weight panel (blocked layout), bounded by the
// end of its expert's weights.
template <int BN>
__device__ __forceinline__ i32x4 panel_rsrc(const void* b, const Tile& t, int N, int KB)
{
    const uint8_t* p = (const uint8_t*)b + (((int64_t)t.e * (N / 32) + (int64_t)t.n * (BN / 32)) * KB) * 1024;
    return make_rsrc(p, (uint32_t)((N / 32 - t.n * (BN / 32)) * KB) * 1024u);
}

// The K stages of one tile, continuing the stream: stage j multiplies ring
// slot b and loads stream stage j + kAhead, which is stage j + kAhead of this
// tile, or of the next tile (its A rows are `held`), or, past the last
// tile, a reload of this tile's last stage that nobody reads (it keeps the
// loads per stage, and so every wait count, the same).
template <int BM, int BN, int WM, int WN, bool F8, bool EPBUF, int A_INS, int B_INS, int RG>
__device__ __forceinline__ void tile_stages(const i32x4& ra, const LoadSrc<A_INS>& cs, int nkt, bool has_nxt,
                                            const i32x4& nrb, int nkt0, const uint32_t (&cpart)[A_INS],
                                            uint32_t Kbytes, int KB, int wv, uint32_t lane16,
                                            Ring<BM, BN, F8, EPBUF>& ring, uint32_t ring0, int& b, int wm, int wn,
                                            int lane, bf16x8 (&fa)[WM / 32], typename BFrag<F8>::raw (&fb)[WN / 32],
                                            const float (&sc)[WN / 32], const uint32_t (&held)[A_INS],
                                            floatx16 (&acc)[WM / 32][WN / 32])
{
    constexpr uint32_t kStageBytes = sizeof(Stage<BM, BN, F8>);
    int j = 0;
    do {  // a tile has at least kAhead stages
        const int ja = j + kAhead;
        LoadSrc<A_INS> ls = cs;
        if (ja < nkt) {
            ls.kt = cs.kt + ja;
        } else if (has_nxt) {
            ls.rb = nrb;
#pragma unroll
            for (int i = 0; i < A_INS; ++i)
                ls.aoff[i] = held[i] * Kbytes + cpart[i];
            ls.kt = nkt0 + (ja - nkt);
        } else {
            ls.kt = cs.kt + nkt - 1;
        }
        if constexpr (F8)  // uniform, but the compiler may keep it in a VGPR
            ls.kt = __builtin_amdgcn_readfirstlane(ls.kt);
        const int bl = b + kAhead >= kRing ? b + kAhead - kRing : b + kAhead;
        const int bn = b + 1 >= kRing ? 0 : b + 1;
        stage<BM, BN, WM, WN, F8, A_INS, B_INS, RG>(ra, ls, ring0 + (uint32_t)bl * kStageBytes, KB, wv, lane16,
                                                   &ring.st[b], &ring.st[bn], wm, wn, lane, fa, fb, sc, acc);
        b = bn;
    } while (++j < nkt);
}

// tile_stages for the M16 path (stage16 per stage).
template <int BM, int BN, int WM, int WN, int A_INS, int B_INS, int RG, bool SW>
__device__ __forceinline__ void tile_stages16(const i32x4& ra, const LoadSrc<A_INS>& cs, int nkt, bool has_nxt,
                                              const i32x4& nrb, int nkt0, const uint32_t (&cpart)[A_INS],
                                              uint32_t Kbytes, int KB, int wv, uint32_t lane16,
                                              Ring<BM, BN, false, false>& ring, uint32_t ring0, int& b, int wm,
                                              int wn, int lane, bf16x8 (&fa)[WM / 16], bf16x8 (&fb)[WN / 16],
                                              const uint32_t (&held)[A_INS], Acc4 (&acc)[WM / 32][WN / 32])
{
    constexpr uint32_t kStageBytes = sizeof(Stage<BM, BN, false>);
    int j = 0;
    do {  // a tile has at least kAhead stages
        const int ja = j + kAhead;
        LoadSrc<A_INS> ls = cs;
        if (ja < nkt) {
            ls.kt = cs.kt + ja;
        } else if (has_nxt) {
            ls.rb = nrb;
#pragma unroll
            for (int i = 0; i < A_INS; ++i)
                ls.aoff[i] = held[i] * Kbytes + cpart[i];
            ls.kt = nkt0 + (ja - nkt);
        } else {
            ls.kt = cs.kt + nkt - 1;
        }
        const int bl = b + kAhead >= kRing ? b + kAhead - kRing : b + kAhead;
        const int bn = b + 1 >= kRing ? 0 : b + 1;
        stage16<BM, BN, WM, WN, A_INS, B_INS, RG, SW>(ra, ls, ring0 + (uint32_t)bl * kStageBytes, KB, wv, lane16,
                                                 &ring.st[b], &ring.st[bn], wm, wn, lane, fa, fb, acc, j == nkt - 1);
        b = bn;
    } while (++j < nkt);
}

// tile_stages for Q8 (same stream, stage_q8 per stage).
template <int BM, int BN, int WM, int WN, int A_INS, int B_INS, int RG>
__device__ __forceinline__ void tile_stages_q8(const i32x4& ra, const LoadSrc<A_INS>& cs, int nkt, bool has_nxt,
                                               const i32x4& nrb, int nkt0, const uint32_t (&cpart)[A_INS],
                                               uint32_t Kbytes, int KB, int wv, uint32_t lane16,
                                               Ring<BM, BN, false, false>& ring, uint32_t ring0, int& b, int wm,
                                               int wn, int lane, v8i (&fa)[2], v8i (&fb)[WN / 32],
                                               const int (&sa)[WM / 32], const int (&sb)[WN / 32],
                                               const uint32_t (&held)[A_INS], floatx16 (&acc)[WM / 32][WN / 32])
{
    constexpr uint32_t kStageBytes = sizeof(Stage<BM, BN, false>);
    int j = 0;
    do {
        const int ja = j + kAhead;
        LoadSrc<A_INS> ls = cs;
        if (ja < nkt) {
            ls.kt = cs.kt + ja;
        } else if (has_nxt) {
            ls.rb = nrb;
#pragma unroll
            for (int i = 0; i < A_INS; ++i)
                ls.aoff[i] = held[i] * Kbytes + cpart[i];
            ls.kt = nkt0 + (ja - nkt);
        } else {
            ls.kt = cs.kt + nkt - 1;
        }
        ls.kt = __builtin_amdgcn_readfirstlane(ls.kt);
        const int bl = b + kAhead >= kRing ? b + kAhead - kRing : b + kAhead;
        const int bn = b + 1 >= kRing ? 0 : b + 1;
        stage_q8<BM, BN, WM, WN, A_INS, B_INS, RG>(ra, ls, ring0 + (uint32_t)bl * kStageBytes, KB, wv, lane16,
                                                  &ring.st[b], &ring.st[bn], wm, wn, lane, fa, fb, sa, sb, acc);
        b = bn;
    } while (++j < nkt);
}

// Per-lane scales of a Q8 tile: A rows wm*WM + i*32 + lane%32 (clamped to the
// tile's valid rows, as the rows themselves) from a_scales by sorted
// position, weight rows as load_scales. Raw fp32 values: they become E8M0
// bytes (e8m0) only after the loads are pinned, so that no use waits for
// them early.
template <int BN, int WM, int WN>
__device__ __forceinline__ void load_scales_q8(const float* a_scales, const float* b_scales, const Tile& t, int N,
                                               int wm, int wn, int lane, float (&sa)[WM / 32], float (&sb)[WN / 32])
{
#pragma unroll
    for (int i = 0; i < WM / 32; ++i)
        sa[i] = a_scales[t.row0 + min(wm * WM + i * 32 + (lane & 31), t.rows - 1)];
    const float* p = b_scales + (int64_t)t.e * N + t.n * BN + wn * WN + (lane & 31);
#pragma unroll
    for (int j = 0; j < WN / 32; ++j)
        sb[j] = p[j * 32];
}

// Source row of slot r of a tile's A rows: token perm[p] (gate/up) or the
// sorted position p itself (down); rows past the segment end are clamped to
// its last row (their results are never stored).
template <bool GATE_UP>
__device__ __forceinline__ int row_src(const int32_t* perm, const Tile& t, int r)
{
    const int p = t.row0 + min(r, t.rows - 1);
    return GATE_UP ? perm[p] : p;
}

// Per-lane row scales of fp8 weights: the wave's column j*32 + lane%32 of
// tile t (weight row n*BN + wn*WN + j*32 + lane%32 of expert e).
template <int BN, int WN>
__device__ __forceinline__ void load_scales(const float* scales, const Tile& t, int N, int wn, int lane,
                                            float (&sc)[WN / 32])
{
    const float* p = scales + (int64_t)t.e * N + t.n * BN + wn * WN + (lane & 31);
#pragma unroll
    for (int j = 0; j < WN / 32; ++j)
        sc[j] = p[j * 32];
}

// F8: 8-bit weights multiplied as bf16 (W8A16); Q8: 8-bit weights and
// activations on the fp8 MFMA (W8A8; F8 is false then: the stage has the
// bf16 layout's shape).
// FC: the down GEMM with the combine fused into its epilogue (a separate
// instantiation: its epilogue code would cost the plain kernel registers).
// YB: the down GEMM without a K split stores each expert output row rounded
// to bf16 (the activation type, like H) instead of fp32: half the bytes to
// write here and to read in the combine.
// Tile order (tiles.hpp): the down GEMM spreads the tiles of experts with at
// most 64 rows over the other experts' tiles (SM = 64): each reads a whole
// weight panel for little matrix work, and run together at the end they
// queue on HBM (skewed routing: 7-11% less time for the down GEMM; no change
// for the gate/up GEMM, whose tiles are longer, so it keeps the plain order).
template <int BM, int BN, int WM, int WN, bool GATE_UP, bool F8, bool Q8, bool FC = false, bool YB = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_kernel(GemmArgs g)
{
    static_assert(!YB || (!GATE_UP && !FC), "bf16 expert outputs: plain down GEMM");
    constexpr int SM = GATE_UP ? 0 : 64;
    static_assert(!(F8 && Q8), "one weight mode");
    constexpr int WAVES_N = BN / WN;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int A_INS = BM * kCH / 64 / 4;             // A loads per wave per stage
    constexpr int B_INS = (BN / 32) * (F8 ? 1 : 2) / 4;  // weight blocks per wave per stage
    constexpr int NLD = A_INS + B_INS;
    constexpr bool EPBUF = (GATE_UP || YB) && F8;        // bf16 epilogue outside the ring
    // M16 path: transposed accumulator blocks (weight fragment as the MFMA's
    // first operand) for the epilogues that store bf16 rows straight from the
    // accumulators; the fp32 partial sums keep the plain layout (their 4-byte
    // stores measured faster than 16-byte ones of the transposed blocks).
    constexpr bool SW = GATE_UP || YB;
    static_assert((BM / WM) * WAVES_N == kThreads / kWave, "4 waves");
    static_assert(A_INS * 4 * 16 == BM && B_INS * 4 == (BN / 32) * (F8 ? 1 : 2), "stage split over 4 waves");
    static_assert(!GATE_UP || (NI % 2 == 0 && WN % 64 == 0), "gate/up pairs per wave");
    static_assert(sizeof(Ring<BM, BN, F8, EPBUF>) <= 160 * 1024, "LDS");
    static_assert(!GATE_UP || EPBUF || sizeof(Stage<BM, BN, F8>) >= 4 * 2048 * sizeof(float), "epilogue in a slot");

    __shared__ Ring<BM, BN, F8, EPBUF> ring;

    const int N = GATE_UP ? 2 * g.f : g.d;  // weight rows per expert
    const int K = GATE_UP ? g.d : g.f;
    const int NT = N / BN;
    const int KB = K / (F8 || Q8 ? 32 : 16);  // 1 KiB weight blocks per weight row block
    const int KT = K / (Q8 ? 64 : kBK);       // K stages (at least kAhead)
    const int S = GATE_UP ? 1 : g.split;
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wv / WAVES_N, wn = wv % WAVES_N;

    TileTable tt;
    const int total = make_table<BM, SM>(g.offsets, g.E, lane, NT * S, tt);
    if (g.skip_rows > 0 && table_max_rows(tt) <= g.skip_rows)
        return;  // the small-batch kernels take this call
    int L = blockIdx.x;
    const int GRID = gridDim.x;
    const bool xm = g.xcd_map != 0;
    const int t0 = tile_index(L, total, xm);
    if (t0 < 0)
        return;

    // Per-lane slot rows and swizzled chunk byte offsets of this wave's A loads.
    const uint32_t Kbytes = (uint32_t)K * (Q8 ? 1u : 2u);
    int slot[A_INS];
    uint32_t cpart[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        slot[i] = (wv * A_INS + i) * 16 + lane / 4;
        cpart[i] = (uint32_t)swz(slot[i], lane % 4) * 16u;
    }
    const uint32_t a_rows = GATE_UP ? (uint32_t)(g.A_max / g.k) : (uint32_t)g.A_max;
    const i32x4 ra = make_rsrc(g.a, a_rows * Kbytes);
    const uint32_t lane16 = (uint32_t)lane * 16u;

    Tile cur = decode<BM, SM>(tt, t0, NT, S, g.group_n, KT);
    LoadSrc<A_INS> cs;
    cs.rb = panel_rsrc<BN>(g.b, cur, N, KB);
    cs.kt = cur.kt0;
#pragma unroll
    for (int i = 0; i < A_INS; ++i)
        cs.aoff[i] = (uint32_t)row_src<GATE_UP>(g.perm, cur, slot[i]) * Kbytes + cpart[i];
    const int t1 = tile_index(L + GRID, total, xm);
    bool has_nxt = t1 >= 0;
    Tile nxt = cur;
    i32x4 nrb = cs.rb;
    uint32_t held[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i)
        held[i] = 0;
    if (has_nxt) {
        nxt = decode<BM, SM>(tt, t1, NT, S, g.group_n, KT);
        nrb = panel_rsrc<BN>(g.b, nxt, N, KB);
#pragma unroll
        for (int i = 0; i < A_INS; ++i)
            held[i] = (uint32_t)row_src<GATE_UP>(g.perm, nxt, slot[i]);
    }
    // Waited for here, before the stream starts (see the scales below).
#pragma unroll
    for (int i = 0; i < A_INS; ++i)
        asm volatile("" : "+v"(held[i]) : : "memory");

    float sc[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j)
        sc[j] = 1.0f;
    if constexpr (F8) {
        // Wait for them here, before any stream load is in flight: a load
        // still pending when the tile loop is entered would make the
        // compiler wait for it (and so for every stage load) in each stage.
        load_scales<BN, WN>(g.scales, cur, N, wn, lane, sc);
#pragma unroll
        for (int j = 0; j < NI; ++j)
            asm volatile("" : "+v"(sc[j]) : : "memory");
    }
    int sa[MI], sb[NI];  // Q8: E8M0 row scales of the current tile
#pragma unroll
    for (int i = 0; i < MI; ++i)
        sa[i] = 127;
#pragma unroll
    for (int j = 0; j < NI; ++j)
        sb[j] = 127;
    if constexpr (Q8) {
        float fa_s[MI], fb_s[NI];
        load_scales_q8<BN, WM, WN>(g.a_scales, g.scales, cur, N, wm, wn, lane, fa_s, fb_s);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            asm volatile("" : "+v"(fa_s[i]) : : "memory");
            sa[i] = e8m0(fa_s[i]);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            asm volatile("" : "+v"(fb_s[j]) : : "memory");
            sb[j] = e8m0(fb_s[j]);
        }
    }

    // bf16 weights run the M16 path (16x16x32 MFMAs); fp8 weights the
    // 32x32 shapes.
    constexpr bool M16 = !F8 && !Q8;
    using AccT = typename std::conditional<M16, Acc4, floatx16>::type;
    AccT acc[MI][NI];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if constexpr (M16) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[i][j].q[c] = floatx4{0.f, 0.f, 0.f, 0.f};
                } else {
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        acc[i][j][q] = 0.f;
                }
            }
    };
    zero_acc();

    // Prologue: the first kAhead stages of the stream (all of the first tile,
    // which has at least kAhead stages), then the k step 0 fragments of the
    // first one.
    const uint32_t ring0 = lds_addr(&ring);
    constexpr uint32_t kStageBytes = sizeof(Stage<BM, BN, F8>);
#pragma unroll
    for (int p = 0; p < kAhead; ++p) {
        LoadSrc<A_INS> ls = cs;
        ls.kt = cs.kt + p;
#pragma unroll
        for (int q = 0; q < NLD; ++q)
            issue_load<BM, BN, F8, A_INS, B_INS>(q, ra, ls, KB, wv, lane16, ring0 + (uint32_t)p * kStageBytes);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAhead - 1) * NLD) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    bf16x8 fa[MI];
    typename BFrag<F8>::raw fb[NI];
    v8i qa[2], qb[NI];                   // Q8 fragments
    bf16x8 fa16[2 * MI], fb16[2 * NI];  // M16 fragments
    if constexpr (M16) {
        const FragReader16<BM, BN, WM, WN> r0{&ring.st[0], wm, wn, lane};
#pragma unroll
        for (int j = 0; j < 2 * NI; ++j)
            fb16[j] = r0.b(j);
#pragma unroll
        for (int i = 0; i < MI; ++i)  // the upper row groups (first half)
            fa16[i] = r0.a(i);
    } else if constexpr (Q8) {
        const FragReaderQ8<BM, BN, WM, WN> r0{&ring.st[0], wm, wn, lane};
#pragma unroll
        for (int j = 0; j < NI; ++j)
            qb[j] = r0.b(j);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            qa[i] = r0.a(i);
    } else {
        const FragReader<BM, BN, WM, WN, F8> r0{&ring.st[0], wm, wn, lane};
#pragma unroll
        for (int j = 0; j < NI; ++j)
            fb[j] = r0.b(0, j);
#pragma unroll
        for (int i = 0; i < MI; ++i)
            fa[i] = r0.a(0, i);
    }
    int b = 0;

    for (;;) {
        // 32-row groups of this wave that hold rows of the tile (the rest of
        // an expert's last m-tile is padding): 0, 1, 2 or all.
        const int wrows = cur.rows - wm * WM;
        const int RG = wrows <= 0 ? 0 : wrows <= 32 ? 1 : wrows <= 64 ? 2 : MI;
        auto run = [&](auto g_const) {
            constexpr int GG = decltype(g_const)::value;
            if constexpr (Q8)
                tile_stages_q8<BM, BN, WM, WN, A_INS, B_INS, GG>(ra, cs, cur.nkt, has_nxt, nrb, nxt.kt0, cpart,
                                                                 Kbytes, KB, wv, lane16, ring, ring0, b, wm, wn,
                                                                 lane, qa, qb, sa, sb, held, acc);
            else if constexpr (M16)
                tile_stages16<BM, BN, WM, WN, A_INS, B_INS, GG, SW>(ra, cs, cur.nkt, has_nxt, nrb, nxt.kt0, cpart, Kbytes,
                                                                KB, wv, lane16, ring, ring0, b, wm, wn, lane, fa16,
                                                                fb16, held, acc);
            else
                tile_stages<BM, BN, WM, WN, F8, EPBUF, A_INS, B_INS, GG>(ra, cs, cur.nkt, has_nxt, nrb, nxt.kt0,
                                                                         cpart, Kbytes, KB, wv, lane16, ring, ring0,
                                                                         b, wm, wn, lane, fa, fb, sc, held, acc);
        };
        static_assert(MI == 4 || MI == 2, "row-group variants");
        if (RG == MI)
            run(std::integral_constant<int, MI>{});
        else if (RG == 2)
            run(std::integral_constant<int, 2>{});
        else if (RG == 1)
            run(std::integral_constant<int, 1>{});
        else
            run(std::integral_constant<int, 0>{});

        // The tile after next: decode it and fetch its token rows now, so the
        // fetch overlaps the epilogue. Its first use is pinned after the
        // epilogue (below); loads complete in issue order, so the wait the
        // compiler puts there also covers the loads of the next tile's first
        // stages, which have had the whole epilogue to land.
        const int t2 = has_nxt ? tile_index(L + 2 * GRID, total, xm) : -1;
        const bool has_nn = t2 >= 0;
        Tile nn = nxt;
        i32x4 nnrb = nrb;
        uint32_t nheld[A_INS];
#pragma unroll
        for (int i = 0; i < A_INS; ++i)
            nheld[i] = held[i];
        if (has_nn) {
            nn = decode<BM, SM>(tt, t2, NT, S, g.group_n, KT);
            nnrb = panel_rsrc<BN>(g.b, nn, N, KB);
#pragma unroll
            for (int i = 0; i < A_INS; ++i)
                nheld[i] = (uint32_t)row_src<GATE_UP>(g.perm, nn, slot[i]);
        }
        // The next tile's row scales, fetched the same way (first use pinned
        // after the epilogue).
        float nsc[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j)
            nsc[j] = sc[j];
        if constexpr (F8)
            if (has_nxt)
                load_scales<BN, WN>(g.scales, nxt, N, wn, lane, nsc);
        float nsa[MI], nsb[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
            nsa[i] = 1.0f;
#pragma unroll
        for (int j = 0; j < NI; ++j)
            nsb[j] = 1.0f;
        if constexpr (Q8)
            if (has_nxt)
                load_scales_q8<BN, WM, WN>(g.a_scales, g.scales, nxt, N, wm, wn, lane, nsa, nsb);

        // Epilogue of the tile. 32x32 accumulator layout: lane holds column
        // lane%32 and, for q = 0..15, row 8*(q/4) + 4*(lane/32) + q%4. Rows
        // past the segment end were computed from the clamped last row, so
        // their results equal that row's: they are stored to it again (same
        // values), which keeps the epilogue free of branches. The lane's row
        // base goes through an opaque move so that the row and address
        // arithmetic is not hoisted out of the tile loop.
        // The epilogue and the pins of the prefetched values, in one copy for
        // full tiles and one for partial ones: the stores a copy issues are
        // then known, and so is the wait the compiler puts at the pins (with
        // the skipped stores of a partial tile it has to wait for all).
        auto epilogue = [&](auto partial) {
            constexpr bool PARTIAL = decltype(partial)::value;
            (void)nheld, (void)nsc, (void)nsa, (void)nsb;  // captured (used only in asm operands)
            // Row of the lane's q = 0 accumulator inside a 32-row group (M16:
            // of its 16-row block).
            const int lq = M16 ? (lane >> 4) : (lane >> 5);
            int rbase = wm * WM + 4 * lq;
            asm volatile("" : "+v"(rbase));
            if constexpr (GATE_UP && M16) {
                // Straight from the accumulators (transposed blocks): per
                // 32-row group, gate/up block pair and 16-row half, each lane
                // applies SiLU(g)*u to its four columns of both 16x16 blocks,
                // rounds them to bf16, and after one register swap between
                // neighbouring 16-lane groups stores 8 consecutive values of
                // its row with one 16-byte store.
                static_assert(BN == 256 && WN == 128 && NI == 4, "gate/up epilogue layout");
                uint16_t* H = (uint16_t*)g.out;
                int rl = wm * WM + (lane & 15);
                asm volatile("" : "+v"(rl));
                const int c8 = row8_col(lane);
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    if (PARTIAL && i >= RG)  // padding rows only: nothing to store
                        continue;
#pragma unroll
                    for (int jp = 0; jp < NI; jp += 2) {
#pragma unroll
                        for (int ri = 0; ri < 2; ++ri) {
                            uint32_t d[2][2];
#pragma unroll
                            for (int cj = 0; cj < 2; ++cj) {
                                const floatx4 gv = acc_read(acc[i][jp].q[2 * ri + cj]);
                                const floatx4 uv = acc_read(acc[i][jp + 1].q[2 * ri + cj]);
                                d[cj][0] = bf16_pair(silu_rcp(gv[0]) * uv[0], silu_rcp(gv[1]) * uv[1]);
                                d[cj][1] = bf16_pair(silu_rcp(gv[2]) * uv[2], silu_rcp(gv[3]) * uv[3]);
                            }
                            const Vec16 v = row8(d[0][0], d[0][1], d[1][0], d[1][1]);
                            const int row = min(rl + i * 32 + ri * 16, cur.rows - 1);
                            const int col = (cur.n * BN + wn * WN + jp * 32) / 2 + c8;
                            *(Vec16*)(H + (int64_t)(cur.row0 + row) * g.f + col) = v;
                            __builtin_amdgcn_sched_barrier(0);  // one segment at a time
                        }
                    }
                }
            } else if constexpr (GATE_UP) {
                // Through LDS, one (32-row group, gate/up block pair) at a time:
                // the accumulators go from AGPRs straight into this wave's 8 KiB
                // of the ring slot the tile's last stage used (free until the
                // next stage refills it, after the barrier below; with fp8
                // weights a slot is too small and the ring has an epilogue buffer
                // of its own), as fp32 rows of 32 with the 16-byte chunk index
                // XORed with row%8 (conflict-free writes and reads); each lane
                // then reads back 16 consecutive gate and up values of one row,
                // applies SiLU(g)*u and stores 16 bf16 of H with two 16-byte
                // stores.
                static_assert(BN == 256 && WN == 128 && NI == 4, "gate/up epilogue layout");
                float* ep;
                if constexpr (EPBUF) {
                    ep = ring.ep + wv * 2048;
                } else {
                    const int bfree = b == 0 ? kRing - 1 : b - 1;
                    ep = (float*)&ring.st[bfree] + wv * 2048;
                }
                const int wr = 8 * 0 + 4 * (lane >> 5);  // row of q = 0 inside the 32-row group
                const int wc = lane & 31;
                const int rr = lane >> 1;                  // row read back by this lane
                const int rc = (lane & 1) * 4;             // first 16-byte chunk read back
                uint16_t* H = (uint16_t*)g.out;
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    if (PARTIAL && i >= RG)  // padding rows only: nothing to store
                        continue;
#pragma unroll
                    for (int jp = 0; jp < NI; jp += 2) {
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const int r = wr + 8 * (q / 4) + (q % 4);
                            const int o = r * 32 + (((wc >> 2) ^ (r & 7)) << 2) + (wc & 3);
                            ep[o] = acc[i][jp][q];
                            ep[1024 + o] = acc[i][jp + 1][q];
                        }
                        uint32_t hv[8];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const int o = rr * 32 + (((rc + t) ^ (rr & 7)) << 2);
                            const floatx4 gv = *(const floatx4*)(ep + o);
                            const floatx4 uv = *(const floatx4*)(ep + 1024 + o);
                            hv[2 * t] = (uint32_t)f32_to_bf16_bits(silu_rcp(gv[0]) * uv[0]) |
                                        ((uint32_t)f32_to_bf16_bits(silu_rcp(gv[1]) * uv[1]) << 16);
                            hv[2 * t + 1] = (uint32_t)f32_to_bf16_bits(silu_rcp(gv[2]) * uv[2]) |
                                            ((uint32_t)f32_to_bf16_bits(silu_rcp(gv[3]) * uv[3]) << 16);
                        }
                        const int row = min(rbase - 4 * lq + i * 32 + rr, cur.rows - 1);
                        const int col = (cur.n * BN + wn * WN + jp * 32) / 2 + rc * 4;
                        Vec16* dst = (Vec16*)(H + (int64_t)(cur.row0 + row) * g.f + col);
                        dst[0] = Vec16{hv[0], hv[1], hv[2], hv[3]};
                        dst[1] = Vec16{hv[4], hv[5], hv[6], hv[7]};
                    }
                }
                // Every wave is done with the slot before the next stage loads it
                // (a wave's own epilogue buffer needs no barrier).
                if constexpr (!EPBUF) {
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                }
            } else {
                float* Ys = (float*)g.out + (int64_t)cur.s * g.A_max * g.d;
                if constexpr (YB && M16) {
                    // bf16 rows straight from the accumulators, as the M16
                    // gate/up epilogue: per 32-row group, 32-column block and
                    // 16-row half one register swap and one 16-byte store of 8
                    // consecutive values of the lane's row.
                    static_assert(NI % 2 == 0, "bf16 outputs: column block pairs");
                    uint16_t* Yb = (uint16_t*)g.out;
                    int rl = wm * WM + (lane & 15);
                    asm volatile("" : "+v"(rl));
                    const int c8 = row8_col(lane);
#pragma unroll
                    for (int i = 0; i < MI; ++i) {
                        if (PARTIAL && i >= RG)  // padding rows only: nothing to store
                            continue;
#pragma unroll
                        for (int j = 0; j < NI; ++j)
#pragma unroll
                            for (int ri = 0; ri < 2; ++ri) {
                                const floatx4 v0 = acc_read(acc[i][j].q[2 * ri]);
                                const floatx4 v1 = acc_read(acc[i][j].q[2 * ri + 1]);
                                const Vec16 v = row8(bf16_pair(v0[0], v0[1]), bf16_pair(v0[2], v0[3]),
                                                     bf16_pair(v1[0], v1[1]), bf16_pair(v1[2], v1[3]));
                                const int row = min(rl + i * 32 + ri * 16, cur.rows - 1);
                                const int col = cur.n * BN + wn * WN + j * 32 + c8;
                                *(Vec16*)(Yb + (int64_t)(cur.row0 + row) * g.d + col) = v;
                                __builtin_amdgcn_sched_barrier(0);  // one segment at a time
                            }
                    }
                } else if constexpr (YB) {
                    // bf16 rows through LDS, as the gate/up epilogue: two
                    // 32x32 accumulator blocks at a time go into this wave's
                    // 8 KiB of the free ring slot (8-bit weights: of the
                    // epilogue buffer; rows of 32 fp32, chunk index XORed with
                    // row%8), then each lane reads back 16 consecutive values
                    // of each block from one row, rounds them to bf16 and
                    // writes them with 16-byte stores.
                    static_assert(NI % 2 == 0, "bf16 outputs: column block pairs");
                    float* ep;
                    if constexpr (EPBUF) {
                        ep = ring.ep + wv * 2048;
                    } else {
                        const int bfree = b == 0 ? kRing - 1 : b - 1;
                        ep = (float*)&ring.st[bfree] + wv * 2048;
                    }
                    const int wr = 4 * (lane >> 5);  // 32x32 layout: row of q = 0 inside the group
                    const int wc = lane & 31;
                    const int rr = lane >> 1;       // row read back by this lane
                    const int rc = (lane & 1) * 4;  // first 16-byte chunk read back
                    uint16_t* Yb = (uint16_t*)g.out;
#pragma unroll
                    for (int i = 0; i < MI; ++i) {
                        if (PARTIAL && i >= RG)  // padding rows only: nothing to store
                            continue;
#pragma unroll
                        for (int jp = 0; jp < NI; jp += 2) {
#pragma unroll
                            for (int q = 0; q < 16; ++q) {
                                const int r = wr + 8 * (q / 4) + (q % 4);
                                const int o = r * 32 + (((wc >> 2) ^ (r & 7)) << 2) + (wc & 3);
                                ep[o] = acc[i][jp][q];
                                ep[1024 + o] = acc[i][jp + 1][q];
                            }
                            const int row = min(rbase - 4 * lq + i * 32 + rr, cur.rows - 1);
#pragma unroll
                            for (int h = 0; h < 2; ++h) {  // the two column blocks
                                uint32_t hv[8];
#pragma unroll
                                for (int t = 0; t < 4; ++t) {
                                    const int o = h * 1024 + rr * 32 + (((rc + t) ^ (rr & 7)) << 2);
                                    const floatx4 v = *(const floatx4*)(ep + o);
                                    hv[2 * t] = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
                                    hv[2 * t + 1] =
                                        (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
                                }
                                const int col = cur.n * BN + wn * WN + (jp + h) * 32 + rc * 4;
                                Vec16* dst = (Vec16*)(Yb + (int64_t)(cur.row0 + row) * g.d + col);
                                dst[0] = Vec16{hv[0], hv[1], hv[2], hv[3]};
                                dst[1] = Vec16{hv[4], hv[5], hv[6], hv[7]};
                            }
                        }
                    }
                    // Every wave is done with the slot before the next stage
                    // loads it (a wave's own epilogue buffer needs no barrier).
                    if constexpr (!EPBUF) {
                        __builtin_amdgcn_s_barrier();
                        asm volatile("" ::: "memory");
                    }
                } else {
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    if (PARTIAL && i >= RG)  // padding rows only: nothing to store
                        continue;
                    if constexpr (M16) {  // plain (not transposed) blocks: lane l holds column l%16
#pragma unroll
                        for (int ri = 0; ri < 2; ++ri)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int r = min(rbase + i * 32 + 16 * ri + q, cur.rows - 1);
                                float* yrow = Ys + (int64_t)(cur.row0 + r) * g.d + cur.n * BN + wn * WN + (lane & 15);
#pragma unroll
                                for (int j = 0; j < NI; ++j)
#pragma unroll
                                    for (int cj = 0; cj < 2; ++cj)
                                        yrow[j * 32 + 16 * cj] = acc[i][j].q[ri * 2 + cj][q];
                            }
                    } else {
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const int r = min(rbase + i * 32 + 8 * (q / 4) + (q % 4), cur.rows - 1);
                            float* yrow = Ys + (int64_t)(cur.row0 + r) * g.d + cur.n * BN + wn * WN + (lane & 31);
#pragma unroll
                            for (int j = 0; j < NI; ++j)
                                yrow[j * 32] = acc[i][j][q];
                        }
                    }
                }
                }
                if constexpr (FC)
                    fused_combine<BN>(g, cur.row0, cur.rows, cur.n, wv, lane);
            }
            zero_acc();
            if constexpr (GATE_UP)
                asm volatile("" : "+v"(nheld[0]), "+v"(nheld[1]), "+v"(nheld[2]), "+v"(nheld[3]) : : "memory");
            if constexpr (F8) {
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    asm volatile("" : "+v"(nsc[j]) : : "memory");
            }
            if constexpr (Q8) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    asm volatile("" : "+v"(nsa[i]) : : "memory");
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    asm volatile("" : "+v"(nsb[j]) : : "memory");
            }
        };
        if (RG == MI)
            epilogue(std::false_type{});
        else
            epilogue(std::true_type{});
        if (!has_nxt)
            break;

        // Switch to the next tile; its loads are already in flight.
        cur = nxt;
        cs.rb = nrb;
        cs.kt = cur.kt0;
#pragma unroll
        for (int i = 0; i < A_INS; ++i)
            cs.aoff[i] = held[i] * Kbytes + cpart[i];
        L += GRID;
        has_nxt = has_nn;
        nxt = nn;
        nrb = nnrb;
#pragma unroll
        for (int i = 0; i < A_INS; ++i)
            held[i] = nheld[i];
#pragma unroll
        for (int j = 0; j < NI; ++j)
            sc[j] = nsc[j];
        if constexpr (Q8) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
                sa[i] = e8m0(nsa[i]);
#pragma unroll
            for (int j = 0; j < NI; ++j)
                sb[j] = e8m0(nsb[j]);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the trailing reloads
}

// ---------------------------------------------------------------------------
// 64-wide K stages (bf16 weights, 16x16x32 MFMAs; selected with GemmArgs::k64).
// The same persistent tile walk and 256x256 tiles on 4 waves of 128x128 as
// grouped_gemm_kernel's M16 path, but each LDS stage holds 64 k: A rows of
// 128 bytes (whole cache lines; one buffer->LDS load covers 8 rows) and four
// 16-k weight blocks per 32 weight rows. Two 64 KiB stages form the ring;
// the accumulator blocks are transposed (SW) and the epilogues store straight
// from them, without LDS. Per stage and wave: 16 loads, 32 fragment reads, 128 MFMAs, one
// barrier. Schedule of stage s (slot s%2):
//   first half:  k-step 0 MFMAs (fragments read in stage s-1), reads of this
//                stage's k-step 1 fragments;
//   middle:      wait for every read and every load issued so far (stage
//                s+1's, issued in stage s-1's second half), barrier;
//   second half: k-step 1 MFMAs, reads of stage s+1's k-step 0 fragments, and
//                the loads of stage s+2 into slot s%2, which no wave reads
//                after the barrier.
// A chunk c (16 bytes) of tile row r sits at position c ^ ((r >> 1) & 7) of
// the row: the 16 rows one fragment read covers land in 16 distinct 16-byte
// bank groups.
struct Stage64 {
    Vec16 a[256 * 8];
    Vec16 b[8 * 4 * 64];
};
struct Ring64 {
    Stage64 st[2];
};
static_assert(sizeof(Ring64) == 128 * 1024, "LDS");

__device__ __forceinline__ int swz64(int r, int c)
{
    return c ^ ((r >> 1) & 7);
}

struct Src64 {
    i32x4 rb;          // weight panel
    uint32_t aoff[8];  // per A load: row byte offset + this lane's chunk
    int kt;            // 64-wide stage index along K
};

// Load q (0..15) of this wave's share of a stage at LDS byte address lds:
// q < 8: tile rows (wv*8 + q)*8 .. +8, 128 bytes each; q >= 8: weight block
// wv*8 + q - 8 (32-row block /4, 16-k block %4).
__device__ __forceinline__ void issue64(int q, const i32x4& ra, const Src64& ls, int KB, int wv, uint32_t lane16,
                                        uint32_t lds)
{
    if (q < 8) {
        dma16(ra, ls.aoff[q], (uint32_t)ls.kt * 128u, lds + (uint32_t)(wv * 8 + q) * 1024u);
    } else {
        const int blk = wv * 8 + (q - 8);
        const uint32_t soff = ((uint32_t)(blk >> 2) * (uint32_t)KB + (uint32_t)ls.kt * 4u + (uint32_t)(blk & 3)) * 1024u;
        dma16(ls.rb, lane16, soff, lds + (uint32_t)offsetof(Stage64, b) + (uint32_t)blk * 1024u);
    }
}

struct Frag64 {
    const Stage64* st;
    int wm, wn, lane;
    // A fragment of the wave's 16-row group i at k-step ks (32 k)
    __device__ __forceinline__ bf16x8 a(int ks, int i) const
    {
        const int r = wm * 128 + i * 16 + (lane & 15);
        return as_bf16x8(st->a[r * 8 + swz64(r, ks * 4 + (lane >> 4))]);
    }
    // B fragment of the wave's 16-row weight group j at k-step ks
    __device__ __forceinline__ bf16x8 b(int ks, int j) const
    {
        const int n = wn * 128 + j * 16 + (lane & 15);
        const int c = lane >> 4;
        return as_bf16x8(st->b[((n >> 5) * 4 + ks * 2 + (c >> 1)) * 64 + (n & 31) + 32 * (c & 1)]);
    }
};

template <int RG, bool SW>
__device__ __forceinline__ void stage64(const i32x4& ra, const Src64& ls, uint32_t ld_lds, int KB, int wv,
                                        uint32_t lane16, const Stage64* st, const Stage64* st_next, int wm, int wn,
                                        int lane, bf16x8 (&fa)[8], bf16x8 (&fb)[8], Acc4 (&acc)[4][4])
{
    const Frag64 rd{st, wm, wn, lane}, rn{st_next, wm, wn, lane};
    bf16x8 ga[8], gb[8];
    int nread = 0;
#pragma unroll
    for (int m = 0; m < 64; ++m) {
        const int j = m / 8, i = m % 8;
        if ((i >> 1) < RG) {
            floatx4& c = acc[i >> 1][j >> 1].q[(i & 1) * 2 + (j & 1)];
            c = SW ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], c, 0, 0, 0)
                   : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], c, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (; nread < 16 && nread < ((m + 1) * 16 + 47) / 48; ++nread) {
            if (nread < 8)
                gb[nread] = rd.b(1, nread);
            else if (((nread - 8) >> 1) < RG)
                ga[nread - 8] = rd.a(1, nread - 8);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    nread = 0;
    int nld = 0;
#pragma unroll
    for (int m = 0; m < 64; ++m) {
        const int j = m / 8, i = m % 8;
        if ((i >> 1) < RG) {
            floatx4& c = acc[i >> 1][j >> 1].q[(i & 1) * 2 + (j & 1)];
            c = SW ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(gb[j], ga[i], c, 0, 0, 0)
                   : __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[i], gb[j], c, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (; nread < 16 && nread < ((m + 1) * 16 + 47) / 48; ++nread) {
            if (nread < 8)
                fb[nread] = rn.b(0, nread);
            else
                fa[nread - 8] = rn.a(0, nread - 8);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (; nld < ((m + 1) * 16) / 64; ++nld) {
            issue64(nld, ra, ls, KB, wv, lane16, ld_lds);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The K stages of one tile, continuing the stream: stage j multiplies slot b
// and loads stream stage j + 2 (this tile's, the next tile's first two, or,
// past the last tile, a reload of this tile's last stage that nobody reads).
template <int RG, bool SW>
__device__ __forceinline__ void tile_stages64(const i32x4& ra, const Src64& cs, int nkt, bool has_nxt,
                                              const i32x4& nrb, int nkt0, const uint32_t (&cpart)[2],
                                              uint32_t Kbytes, int KB, int wv, uint32_t lane16, Ring64& ring,
                                              uint32_t ring0, int& b, int wm, int wn, int lane, bf16x8 (&fa)[8],
                                              bf16x8 (&fb)[8], const uint32_t (&held)[8], Acc4 (&acc)[4][4])
{
    int j = 0;
    do {
        const int ja = j + 2;
        Src64 ls = cs;
        if (ja < nkt) {
            ls.kt = cs.kt + ja;
        } else if (has_nxt) {
            ls.rb = nrb;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ls.aoff[i] = held[i] * Kbytes + cpart[i & 1];
            ls.kt = nkt0 + (ja - nkt);
        } else {
            ls.kt = cs.kt + nkt - 1;
        }
        stage64<RG, SW>(ra, ls, ring0 + (uint32_t)b * (uint32_t)sizeof(Stage64), KB, wv, lane16, &ring.st[b],
                    &ring.st[b ^ 1], wm, wn, lane, fa, fb, acc);
        b ^= 1;
    } while (++j < nkt);
}

template <bool GATE_UP, bool YB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm64_kernel(GemmArgs g)
{
    constexpr int BM = 256, BN = 256, WM = 128, WN = 128, MI = 4, NI = 4;
    constexpr bool SW = true;  // transposed accumulator blocks (the epilogue below)
    constexpr int SM = GATE_UP ? 0 : 64;
    __shared__ Ring64 ring;

    const int N = GATE_UP ? 2 * g.f : g.d;
    const int K = GATE_UP ? g.d : g.f;
    const int NT = N / BN;
    const int KB = K / 16;
    const int KT = K / 64;
    const int S = GATE_UP ? 1 : g.split;
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wv / 2, wn = wv % 2;

    TileTable tt;
    const int total = make_table<BM, SM>(g.offsets, g.E, lane, NT * S, tt);
    if (g.skip_rows > 0 && table_max_rows(tt) <= g.skip_rows)
        return;  // the small-batch kernels take this call
    int L = blockIdx.x;
    const int GRID = gridDim.x;
    const bool xm = g.xcd_map != 0;
    const int t0 = tile_index(L, total, xm);
    if (t0 < 0)
        return;

    // A loads: load q covers tile rows (wv*8 + q)*8 + lane/8; this lane's
    // chunk position is lane%8, holding global chunk (lane%8) ^ ((row >> 1) & 7),
    // which depends on q only through its parity.
    const uint32_t Kbytes = (uint32_t)K * 2u;
    int slot[8];
    uint32_t cpart[2];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        slot[q] = (wv * 8 + q) * 8 + (lane >> 3);
#pragma unroll
    for (int p = 0; p < 2; ++p)
        cpart[p] = (uint32_t)swz64(slot[p], lane & 7) * 16u;
    const uint32_t a_rows = GATE_UP ? (uint32_t)(g.A_max / g.k) : (uint32_t)g.A_max;
    const i32x4 ra = make_rsrc(g.a, a_rows * Kbytes);
    const uint32_t lane16 = (uint32_t)lane * 16u;

    Tile cur = decode<BM, SM>(tt, t0, NT, S, g.group_n, KT);
    Src64 cs;
    cs.rb = panel_rsrc<BN>(g.b, cur, N, KB);
    cs.kt = cur.kt0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        cs.aoff[q] = (uint32_t)row_src<GATE_UP>(g.perm, cur, slot[q]) * Kbytes + cpart[q & 1];
    const int t1 = tile_index(L + GRID, total, xm);
    bool has_nxt = t1 >= 0;
    Tile nxt = cur;
    i32x4 nrb = cs.rb;
    uint32_t held[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        held[q] = 0;
    if (has_nxt) {
        nxt = decode<BM, SM>(tt, t1, NT, S, g.group_n, KT);
        nrb = panel_rsrc<BN>(g.b, nxt, N, KB);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            held[q] = (uint32_t)row_src<GATE_UP>(g.perm, nxt, slot[q]);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
        asm volatile("" : "+v"(held[q]) : : "memory");

    Acc4 acc[MI][NI];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc[i][j].q[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    };
    zero_acc();

    // Prologue: stream stages 0 and 1 (the first tile has at least 2), then
    // stage 0's k-step 0 fragments.
    const uint32_t ring0 = lds_addr(&ring);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        Src64 ls = cs;
        ls.kt = cs.kt + p;
#pragma unroll
        for (int q = 0; q < 16; ++q)
            issue64(q, ra, ls, KB, wv, lane16, ring0 + (uint32_t)p * (uint32_t)sizeof(Stage64));
    }
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    bf16x8 fa[8], fb[8];
    {
        const Frag64 r0{&ring.st[0], wm, wn, lane};
#pragma unroll
        for (int j = 0; j < 8; ++j)
            fb[j] = r0.b(0, j);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            fa[i] = r0.a(0, i);
    }
    int b = 0;

    for (;;) {
        const int wrows = cur.rows - wm * WM;
        const int RG = wrows <= 0 ? 0 : wrows <= 32 ? 1 : wrows <= 64 ? 2 : MI;
        auto run = [&](auto g_const) {
            constexpr int GG = decltype(g_const)::value;
            tile_stages64<GG, SW>(ra, cs, cur.nkt, has_nxt, nrb, nxt.kt0, cpart, Kbytes, KB, wv, lane16, ring, ring0, b,
                              wm, wn, lane, fa, fb, held, acc);
        };
        if (RG == MI)
            run(std::integral_constant<int, MI>{});
        else if (RG == 2)
            run(std::integral_constant<int, 2>{});
        else if (RG == 1)
            run(std::integral_constant<int, 1>{});
        else
            run(std::integral_constant<int, 0>{});

        // The tile after next: its token rows, fetched during the epilogue.
        const int t2 = has_nxt ? tile_index(L + 2 * GRID, total, xm) : -1;
        const bool has_nn = t2 >= 0;
        Tile nn = nxt;
        i32x4 nnrb = nrb;
        uint32_t nheld[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            nheld[q] = held[q];
        if (has_nn) {
            nn = decode<BM, SM>(tt, t2, NT, S, g.group_n, KT);
            nnrb = panel_rsrc<BN>(g.b, nn, N, KB);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                nheld[q] = (uint32_t)row_src<GATE_UP>(g.perm, nn, slot[q]);
        }

        // Epilogue straight from the accumulators (transposed 16x16 blocks:
        // lane l holds token row l%16 and four consecutive output columns),
        // as grouped_gemm_kernel's M16 epilogues: SiLU(g)*u or bf16 rows as
        // 8 consecutive values per lane and 16-byte store after one register
        // swap, fp32 partial sums as the lane's four columns per store.
        {
            int rl = wm * WM + (lane & 15);
            asm volatile("" : "+v"(rl));
            const int c8 = row8_col(lane);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (i >= RG)
                    continue;
#pragma unroll
                for (int ri = 0; ri < 2; ++ri) {
                    const int row = min(rl + i * 32 + ri * 16, cur.rows - 1);
                    if constexpr (GATE_UP) {
#pragma unroll
                        for (int jp = 0; jp < NI; jp += 2) {
                            uint32_t d[2][2];
#pragma unroll
                            for (int cj = 0; cj < 2; ++cj) {
                                const floatx4 gv = acc_read(acc[i][jp].q[2 * ri + cj]);
                                const floatx4 uv = acc_read(acc[i][jp + 1].q[2 * ri + cj]);
                                d[cj][0] = bf16_pair(silu_rcp(gv[0]) * uv[0], silu_rcp(gv[1]) * uv[1]);
                                d[cj][1] = bf16_pair(silu_rcp(gv[2]) * uv[2], silu_rcp(gv[3]) * uv[3]);
                            }
                            const int col = (cur.n * BN + wn * WN + jp * 32) / 2 + c8;
                            *(Vec16*)((uint16_t*)g.out + (int64_t)(cur.row0 + row) * g.f + col) =
                                row8(d[0][0], d[0][1], d[1][0], d[1][1]);
                            __builtin_amdgcn_sched_barrier(0);  // one segment at a time
                        }
                    } else if constexpr (YB) {
#pragma unroll
                        for (int j = 0; j < NI; ++j) {
                            const floatx4 v0 = acc_read(acc[i][j].q[2 * ri]);
                            const floatx4 v1 = acc_read(acc[i][j].q[2 * ri + 1]);
                            const int col = cur.n * BN + wn * WN + j * 32 + c8;
                            *(Vec16*)((uint16_t*)g.out + (int64_t)(cur.row0 + row) * g.d + col) =
                                row8(bf16_pair(v0[0], v0[1]), bf16_pair(v0[2], v0[3]), bf16_pair(v1[0], v1[1]),
                                     bf16_pair(v1[2], v1[3]));
                            __builtin_amdgcn_sched_barrier(0);  // one segment at a time
                        }
                    } else {
                        float* yrow = (float*)g.out + (int64_t)cur.s * g.A_max * g.d +
                                      (int64_t)(cur.row0 + row) * g.d + cur.n * BN + wn * WN + 4 * (lane >> 4);
#pragma unroll
                        for (int j = 0; j < NI; ++j)
#pragma unroll
                            for (int cj = 0; cj < 2; ++cj)
                                *(floatx4*)(yrow + j * 32 + 16 * cj) = acc[i][j].q[2 * ri + cj];
                    }
                }
            }
            zero_acc();
#pragma unroll
            for (int q = 0; q < 8; ++q)
                asm volatile("" : "+v"(nheld[q]) : : "memory");
        }
        if (!has_nxt)
            break;
        cur = nxt;
        cs.rb = nrb;
        cs.kt = cur.kt0;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            cs.aoff[q] = held[q] * Kbytes + cpart[q & 1];
        L += GRID;
        has_nxt = has_nn;
        nxt = nn;
        nrb = nnrb;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            held[q] = nheld[q];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
// per lane, held in AGPRs), a ring of 5 x 32 KiB LDS stages. When the
// weight-row count is not a multiple of 256 (down GEMM with d_model % 256 ==
// 128), 256x128 tiles (waves of 128x64, 5 x 24 KiB stages).
constexpr int kBM = 256;

int down_split_bf16(int A, int E, int d, int f, int cus, int q8)
{
    // Split K in two when the down GEMM has fewer than three tiles per compute
    // unit: whole-tile rounds then waste much of the last round, and halves
    // fill it better at the price of one more fp32 partial for combine to read.
    const int BN = d % 256 == 0 ? 256 : 128;
    const int64_t tiles = ((int64_t)A / kBM + E) * (d / BN);
    const int KT = f / (q8 ? 64 : kBK);
    return (KT >= 16 && tiles < 3 * (int64_t)cus) ? 2 : 1;
}

template <bool GATE_UP, bool F8, bool Q8>
hipError_t launch_grouped(const GemmArgs& a, hipStream_t s)
{
    const int N = GATE_UP ? 2 * a.f : a.d;
    const int S = GATE_UP ? 1 : a.split;
    const int BN = N % 256 == 0 ? 256 : 128;
    int64_t bound = ((int64_t)a.A_max / kBM + a.E) * (N / BN) * S;  // tiles, upper bound
    // XCD-contiguous placement needs every workgroup's indices on one XCD:
    // a grid that is a multiple of 8.
    const bool xm = a.xcd_map != 0 && a.grid % 8 == 0;
    if (xm)
        bound = (bound + 7) / 8 * 8;
    const int grid = (int)(bound < a.grid ? bound : a.grid);
    if (grid <= 0)
        return hipSuccess;
    GemmArgs ga = a;
    ga.xcd_map = xm ? 1 : 0;
    if constexpr (!F8 && !Q8) {
        if (a.k64 && a.cnt == nullptr && N % 256 == 0) {
            if constexpr (GATE_UP)
                hipLaunchKernelGGL((grouped_gemm64_kernel<true, false>), dim3(grid), dim3(kThreads), 0, s, ga);
            else if (a.ys_bf16)
                hipLaunchKernelGGL((grouped_gemm64_kernel<false, true>), dim3(grid), dim3(kThreads), 0, s, ga);
            else
                hipLaunchKernelGGL((grouped_gemm64_kernel<false, false>), dim3(grid), dim3(kThreads), 0, s, ga);
            return hipGetLastError();
        }
    }
    if constexpr (GATE_UP) {
        // 2 * d_ff is a multiple of 256 (d_ff % 128 == 0 is checked at init)
        hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 256, 128, 128, true, F8, Q8>), dim3(grid), dim3(kThreads), 0,
                           s, ga);
    } else if (a.cnt != nullptr) {
        if (BN == 256)
            hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 256, 128, 128, false, F8, Q8, true>), dim3(grid),
                               dim3(kThreads), 0, s, ga);
        else
            hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 128, 128, 64, false, F8, Q8, true>), dim3(grid),
                               dim3(kThreads), 0, s, ga);
    } else if (a.ys_bf16) {
        if constexpr (Q8) {  // 8-bit A rows feed the gate/up GEMM only
            return hipErrorInvalidValue;
        } else {
            if (BN == 256)
                hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 256, 128, 128, false, F8, Q8, false, true>), dim3(grid),
                                   dim3(kThreads), 0, s, ga);
            else
                hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 128, 128, 64, false, F8, Q8, false, true>), dim3(grid),
                                   dim3(kThreads), 0, s, ga);
        }
    } else {
        if (BN == 256)
            hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 256, 128, 128, false, F8, Q8>), dim3(grid), dim3(kThreads),
                               0, s, ga);
        else
            hipLaunchKernelGGL((grouped_gemm_kernel<kBM, 128, 128, 64, false, F8, Q8>), dim3(grid), dim3(kThreads),
                               0, s, ga);
    }
    return hipGetLastError();
}

hipError_t launch_gate_up_bf16(const GemmArgs& a, hipStream_t s)
{
    if (a.a_scales)
        return launch_grouped<true, false, true>(a, s);
    return a.scales ? launch_grouped<true, true, false>(a, s) : launch_grouped<true, false, false>(a, s);
}

hipError_t launch_down_bf16(const GemmArgs& a, hipStream_t s)
{
    if (a.a_scales)  // 8-bit A rows feed the gate/up GEMM only
        return hipErrorInvalidValue;
    return a.scales ? launch_grouped<false, true, false>(a, s) : launch_grouped<false, false, false>(a, s);
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
