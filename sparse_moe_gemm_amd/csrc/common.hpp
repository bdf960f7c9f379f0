// common.hpp - types and small device helpers shared by the gfx950 kernels of
// the MoE layer, plus the host-side launch declarations used by api.cpp.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <stdint.h>

namespace cmoe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;

// Raw 16-byte vector moved between global memory, LDS and MFMA operands (a
// native vector type, so it always lives in registers).
typedef uint32_t Vec16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(const Vec16& v)
{
    return __builtin_bit_cast(bf16x8, v);
}

// Eight OCP E4M3 codes (little-endian in two words) to bf16, each multiplied
// by sc (a power of two here, so exact): v_cvt_scalef32_pk_bf16_fp8, two codes
// per instruction.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi, float sc)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

// Round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<bf16>(f));
}

__device__ __forceinline__ float silu(float z)
{
    return z / (1.0f + __expf(-z));
}

// Most rows any expert holds in this call (offsets [E+1]), the same value in
// every lane of the wave. Calls that enqueue both GEMM paths let each kernel
// decide from it, on the device, whether the call is its own.
__device__ __forceinline__ int max_expert_rows(const int32_t* offsets, int E)
{
    const int lane = threadIdx.x % kWave;
    int m = 0;
    for (int e = lane; e < E; e += kWave)
        m = max(m, offsets[e + 1] - offsets[e]);
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1)
        m = max(m, __shfl_xor(m, d, kWave));
    return __builtin_amdgcn_readfirstlane(m);
}

// ---------------------------------------------------------------------------
// Host-side launchers (each defined in the .hip file of its kernel).
// All enqueue on `s` and return the launch status.
// ---------------------------------------------------------------------------

struct RouterArgs {
    const void* x;      // [T][d] dtype
    const void* w_rt;   // router weights: bf16 blocked (router_weight_bytes), fp32 [E][d]
    const float* b;     // [E] fp32 (never NULL: zeros when the caller gave none)
    int T, d, E, k;
    float* logits;      // [T][E] (may be NULL)
    int32_t* ids;       // [T][k]
    float* w;           // [T][k]
};
hipError_t launch_router_bf16(const RouterArgs& a, hipStream_t s);
hipError_t launch_router_f32(const RouterArgs& a, hipStream_t s);

struct DispatchArgs {
    const int32_t* ids; // [A]
    int T, k, E;
    int32_t* counts;    // [E]
    int32_t* offsets;   // [E+1]
    int32_t* perm;      // [A]
    int32_t* perm_slot; // [A]
    int32_t* inv;       // [A]
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);

struct GemmArgs {
    // gate/up: A rows are x[perm[p]] ([T][d]); B = interleaved gate/up weights
    //   [E][2f][d]; out = H [A][f] (row p = sorted position p).
    // down:    A rows are H[p] ([A][f]);        B = down weights [E][d][f];
    //   out = Ys: split partial sums over K, partial s at Ys + s*A*d, each
    //   [A][d] fp32 with row p = sorted position p (combine gathers them
    //   through inv).
    // bf16 weights are in the blocked MFMA layout, fp32 weights row-major;
    // 8-bit weights (scales != null) are E4M3 codes in the fp8 blocked layout
    // with one fp32 scale per weight row, scales[e*N + n]. With a_scales the
    // A rows are 8-bit too (E4M3 codes, one power-of-two scale per A row,
    // indexed by sorted position p) and the fp8 MFMA runs (W8A8).
    const void* a;
    const void* b;
    const float* scales;
    const float* a_scales;
    void* out;
    const int32_t* offsets;   // [E+1]
    const int32_t* perm;      // [A]
    int A_max;                // A = T*k of this call (bounds the tile grid)
    int E, k, d, f;
    int group_n;              // tile order (tiles.hpp): > 0 n-tiles per group; -G: groups of G m-tiles
    int split;                // K splits of the down GEMM (1 or 2; gate/up: 1)
    int grid;                 // workgroups of a persistent launch (compute units)
    // Combine fused into the down GEMM (bf16 tiled path, optional; cnt ==
    // nullptr: the combine kernel runs instead). cnt [T][d/128] counts, per token and
    // n-tile, the k*split partial rows stored so far; the workgroup whose
    // increment completes a count sums that token's columns of the tile
    // (inv, topw: as for combine) into y (bf16 [T][d]) and resets the count
    // to zero, so the counts are zero between calls.
    int32_t* cnt;
    const int32_t* inv;
    const float* topw;
    void* y;
    // down GEMM with split == 1, without the fused combine: out is [A][d] bf16
    // (each expert output row rounded to nearest even) instead of fp32
    int ys_bf16;
    // tile placement (tiles.hpp tile_index): 0 = consecutive tiles to the 8
    // XCDs in turn; 1 = each XCD runs one contiguous eighth of the tile order
    // (the launch's grid must then be a multiple of 8)
    int xcd_map;
    // bf16 weights, 256-row weight tiles, no fused combine: 1 runs the
    // 64-wide K stage kernel (grouped_gemm64_kernel)
    int k64;
    // > 0: the call also went to the small-batch kernels, which take it when
    // no expert holds more than skip_rows rows; the tiled kernel then does
    // nothing (0: always run)
    int skip_rows;
};
hipError_t launch_gate_up_bf16(const GemmArgs& a, hipStream_t s);
hipError_t launch_down_bf16(const GemmArgs& a, hipStream_t s);
// K splits the bf16 down GEMM uses for a call with A = T*k assignments on
// `cus` compute units (1 or 2; the Ys workspace holds kMaxSplit partials).
constexpr int kMaxSplit = 2;
// (the fused combine's loads in gemm_bf16.hip cover at most two partials)
static_assert(kMaxSplit == 2, "fused combine: one or two K-split partials");
int down_split_bf16(int A, int E, int d, int f, int cus, int q8);
hipError_t launch_gate_up_f32(const GemmArgs& a, hipStream_t s);
hipError_t launch_down_f32(const GemmArgs& a, hipStream_t s);

// Small-batch (decode) path of the bf16 expert GEMMs (decode_bf16.hip).
struct DecodeArgs {
    const void* a;            // gate/up: x [T][d] (rows through perm); down: H [A][f]
    const void* b;            // blocked bf16 or fp8 weights (as in the grouped GEMMs)
    const float* scales;      // fp8 row scales [E][N], or null for bf16 weights
    const float* a_scales;    // W8A8: A is E4M3 codes, row scales by sorted position; else null
    float* part;              // fp32 slice partials [split][A][N], N = 2f (gate/up) or d (down)
    const int32_t* offsets;   // [E+1]
    const int32_t* perm;      // [A]
    int A;                    // T*k of this call
    int E, d, f;
    int split;                // K slices
    // gate/up with split == 1: H [A][f] bf16 written directly as
    // SiLU(g)*u (no partials, no separate slice-sum pass); else null
    uint16_t* h;
    // most rows one expert can hold in this call (T: a token picks an
    // expert at most once); 1..32 lets the bf16 kernel skip its code for
    // token-group pairs, 0 means not known
    int max_rows;
    // > 0: the call also went to the tiled kernels, which take it when some
    // expert holds more than gate_rows rows; this kernel then does nothing
    // (0: always run)
    int gate_rows;
};
// Waves a decode launch runs on `cus` compute units.
int decode_waves(int cus);
// K slices for an (E experts, N weight rows, K) decode GEMM on `waves` waves
// that steps through K in kstep-wide steps (16 for bf16 weights, 32 for fp8).
int decode_split(int E, int N, int K, int kstep, int waves, int max_split);
hipError_t launch_decode_gemm(const DecodeArgs& a, int gate_up, int cus, hipStream_t s);
// H = SiLU(sum of gate slices) * (sum of up slices), bf16; gate_rows as in
// DecodeArgs (offsets [E+1]).
hipError_t launch_decode_silu(const float* part, void* H, int A, int f, int S, const int32_t* offsets, int E,
                              int gate_rows, hipStream_t s);

// 8-bit expert weights (quant_fp8.hip). Row scales of bf16 weight rows: rows
// of [rows][cols], or with w1 != null the interleaved gate/up rows of
// [E][rows_per_e] (rows_per_e = 2f) built from w0 (gate) and w1 (up).
hipError_t launch_fp8_row_scales(const void* w0, const void* w1, float* scales, int64_t rows, int rows_per_e,
                                 int cols, hipStream_t s);
// E4M3 codes in the fp8 blocked GEMM layout ([E][N][K] weights, gate/up
// interleaved when w1 != null), scaled by the row scales.
hipError_t launch_fp8_pack_blocked(const void* w0, const void* w1, const float* scales, void* out, int E, int N,
                                   int K, hipStream_t s);
// 8-bit activation rows: codes [rows][cols] of a bf16 [rows][cols] matrix and
// the rows' power-of-two scales, at scales[row], or with inv at
// scales[inv[row*k + j]] for j < k.
hipError_t launch_act_quant(const void* x, int64_t rows, int cols, int k, const int32_t* inv, uint8_t* codes,
                            float* scales, hipStream_t s);
// Row-major E4M3 codes of [rows][cols] bf16 with the given row scales.
hipError_t launch_fp8_encode_rows(const void* w, const float* scales, uint8_t* codes, int64_t rows, int cols,
                                  hipStream_t s);

struct CombineArgs {
    const float* ys;    // split partials, each [A][d] fp32 by sorted position (ys_bf16: one [A][d] bf16)
    const int32_t* inv; // [A]: sorted position of assignment t*k+j
    const float* w;     // [T][k]
    void* y;            // [T][d] dtype
    int T, k, d;
    int split;          // number of partials, at ys + s*T*k*d
    int bf16_out;
    int ys_bf16;        // the expert outputs are bf16 (split == 1)
    // Calls that enqueue both GEMM paths (gate_rows > 0): when no expert
    // holds more than gate_rows rows (offsets [E+1]) the small-batch kernels
    // wrote Ys, as small_split fp32 partials; otherwise the tiled ones, as
    // split and ys_bf16 say.
    const int32_t* offsets;
    int E;
    int gate_rows;
    int small_split;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// Init-time weight repacks.
// Router weights as the router kernels read them, from the caller's [d][E]
// matrix: fp32 layers [E][d] (transposed); bf16 layers in MFMA operand blocks,
// for each group of 16 experts and 32-wide K step one 1 KiB block in which
// lane l's 8 values (expert 16g + l%16, k = 32s + 8(l/16) .. +8) sit at
// l*16 bytes; experts past E are zero rows.
size_t router_weight_bytes(int d, int E, int esize);
// Measurement only (stream_copy.hip): dst = src, bytes a multiple of 16.
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, int cus, hipStream_t s);
hipError_t launch_transpose_router(const void* w_r, void* w_rt, int d, int E, int esize, hipStream_t s);
hipError_t launch_interleave_gate_up(const void* wg, const void* wu, void* wgu, int E, int f, int d,
                                     int esize, hipStream_t s);
// bf16 weights in the blocked MFMA operand layout (see gemm_bf16.hip); with
// gate_up, w0/w1 are the gate/up matrices [E][N/2][K] and rows are interleaved.
hipError_t launch_pack_blocked(const void* w0, const void* w1, void* out, int E, int N, int K, int gate_up,
                               hipStream_t s);

}  // namespace cmoe
