// quant_fp8.hip - 8-bit expert weights: quantization at init.
//
// «Colibri 是什么» (xxqk.cn) §4.2: the model converter can quantize the expert
// FFN weights alone to 8 bits, keeping the router in full precision. The
// pages fix neither the 8-bit format nor the scaling; this library uses
//   - OCP FP8 E4M3 codes (gfx950's native 8-bit float: bias 7, 3 mantissa
//     bits, largest finite 448, no infinities);
//   - one scale per weight row (output unit), the power of two 2^e with the
//     smallest integer e such that max_i |w[r][i]| <= 448 * 2^e (e = 0 for an
//     all-zero row, e >= -126), so w * 2^-e is exact;
//   - code = w * 2^-e rounded to the nearest E4M3 value, ties to the even
//     mantissa, values below 2^-10 to a zero that keeps the sign of w.
// Dequantization, code * 2^e, is exact in bf16, so the GEMMs convert codes to
// bf16 in registers (v_cvt_scalef32_pk_bf16_fp8, scale = 2^e) and multiply
// on the bf16 MFMA path; only the bytes read from memory change.
//
// Layout written for the GEMMs (blocked, like the bf16 one but one 1 KiB block
// per 32 rows x 32 k): block (e, nb, kb) holds rows nb*32 .. +32 and
// k = kb*32 .. +32; lane l's 16 bytes at l*16 are the codes of row
// nb*32 + l%32, k = kb*32 + 16*(l/32) .. +16. This k order serves both ways
// the codes are multiplied: as bf16 on the 16-wide bf16 MFMA (the lane's
// 8-byte halves are its B fragments of two k steps, the activations are read
// in the same order), and on the 64-wide fp8 MFMA, whose lane l takes k
// 16*(l/32) .. +16 of each 32-k half of its 64 (two consecutive blocks). The
// small-batch GEMMs fetch a lane's 16 bytes with one load; the tiled GEMMs
// read them from LDS.
#include "common.hpp"

namespace cmoe {

namespace {

// Exponent e of the row scale from the row's largest magnitude.
__device__ __forceinline__ int fp8_scale_exp(float amax)
{
    if (!(amax > 0.f))
        return 0;
    int x;
    const float f = frexpf(amax, &x);  // amax = f * 2^x, f in [0.5, 1)
    // 448 = 0.875 * 2^9: amax <= 448 * 2^e  <=>  f * 2^(x - 9 - e) <= 0.875
    const int e = (f <= 0.875f) ? x - 9 : x - 8;
    return e < -126 ? -126 : e;
}

// Per-row scales. One wave per row of `cols` bf16 values (cols % 8 == 0);
// with `two_src`, combined row n of a [E][2f] matrix comes from w0 (gate) when
// n % 64 < 32, else from w1 (up), source row (n/64)*32 + n%32 of expert e.
__global__ __launch_bounds__(256) void fp8_row_scale_kernel(const uint16_t* w0, const uint16_t* w1, float* scales,
                                                            int64_t rows, int rows_per_e, int cols, int two_src)
{
    const int lane = threadIdx.x % kWave;
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x / kWave);
    for (int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; r < rows; r += nw) {
        const uint16_t* src;
        if (two_src) {
            const int64_t e = r / rows_per_e;
            const int n = (int)(r % rows_per_e);
            const int w = n % 64;
            src = (w < 32 ? w0 : w1) + (e * (rows_per_e / 2) + (n / 64) * 32 + (w % 32)) * (int64_t)cols;
        } else {
            src = w0 + r * (int64_t)cols;
        }
        float amax = 0.f;
        for (int c = lane * 8; c < cols; c += kWave * 8) {
            const Vec16 v = *(const Vec16*)(src + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                amax = fmaxf(amax, fabsf(__uint_as_float(v[i] << 16)));
                amax = fmaxf(amax, fabsf(__uint_as_float(v[i] & 0xFFFF0000u)));
            }
        }
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1)
            amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
        if (lane == 0)
            scales[r] = ldexpf(1.0f, fp8_scale_exp(amax));
    }
}

// 1 / s for a power of two s = 2^e (-126 <= e <= 127): exact, from the exponent.
__device__ __forceinline__ float inv_pow2(float s)
{
    int x;
    (void)frexpf(s, &x);  // s = 0.5 * 2^x
    return ldexpf(1.0f, 1 - x);
}

// Codes of 8 consecutive bf16 values (16 bytes) scaled by 1/scale, packed
// little-endian into two words.
// E4M3 codes of 8 bf16 values times 2^-e (exact, |v| <= 448), value i in
// byte i. v_cvt_pk_fp8_f32 rounds to the nearest E4M3 value, ties to the even
// mantissa, and gives a small value that rounds to zero the sign of its input:
// the rule above (it agrees with an integer model of the rule on every f32
// input of magnitude at most 448). It packs its two inputs into bytes 0, 1 of
// the result, or into bytes 2, 3 over the old value.
__device__ __forceinline__ uint2 encode8(const Vec16 v, float inv_scale)
{
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t a = v[2 * h], b = v[2 * h + 1];
        int r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(a << 16) * inv_scale,
                                                __uint_as_float(a & 0xFFFF0000u) * inv_scale, 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(b << 16) * inv_scale,
                                            __uint_as_float(b & 0xFFFF0000u) * inv_scale, r, true);
        w[h] = (uint32_t)r;
    }
    return make_uint2(w[0], w[1]);
}

// Blocked fp8 layout (see the file comment), one 16-byte lane chunk per thread.
__global__ __launch_bounds__(256) void fp8_pack_blocked_kernel(const uint16_t* w0, const uint16_t* w1,
                                                               const float* scales, Vec16* out, int E, int N, int K,
                                                               int two_src)
{
    const int NB = N / 32, KB = K / 32;
    const int64_t total = (int64_t)E * NB * KB * kWave;
    const int Nsrc = two_src ? N / 2 : N;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(idx % kWave);
        const int64_t blk = idx / kWave;
        const int kb = (int)(blk % KB);
        const int64_t rb = blk / KB;
        const int nb = (int)(rb % NB);
        const int e = (int)(rb / NB);
        const int n = nb * 32 + (l % 32);
        const int k = kb * 32 + 16 * (l / 32);
        const uint16_t* src;
        int srow;
        if (two_src) {
            const int w = n % 64;
            srow = (n / 64) * 32 + (w % 32);
            src = w < 32 ? w0 : w1;
        } else {
            srow = n;
            src = w0;
        }
        const uint16_t* rowp = src + ((int64_t)e * Nsrc + srow) * K;
        // multiplying by the exact 2^-e is the exact w * 2^-e
        const float inv = inv_pow2(scales[(int64_t)e * N + n]);
        const uint2 lo = encode8(*(const Vec16*)(rowp + k), inv);
        const uint2 hi = encode8(*(const Vec16*)(rowp + k + 8), inv);
        out[idx] = Vec16{lo.x, lo.y, hi.x, hi.y};
    }
}

// Row-major codes: codes[r][c] for c < cols (cols % 8 == 0).
__global__ __launch_bounds__(256) void fp8_encode_rows_kernel(const uint16_t* w, const float* scales, uint8_t* codes,
                                                              int64_t rows, int cols)
{
    const int64_t chunks = rows * (cols / 8);
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < chunks;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / (cols / 8);
        const int c = (int)(idx % (cols / 8)) * 8;
        *(uint2*)(codes + r * cols + c) = encode8(*(const Vec16*)(w + r * cols + c), inv_pow2(scales[r]));
    }
}

// 8-bit activation rows (the layer's optional W8A8 mode): row t of a [rows][cols]
// bf16 matrix becomes codes [rows][cols] with its power-of-two scale (the
// weights' rule), one wave per row. The scale goes to scales[t], or, with
// inv, to scales[inv[t*k + j]] for each of token t's k assignments (the
// sorted positions the GEMMs index their A rows by).
// One 256-thread block per row: a row of up to kActChunks * 2048 values is
// read once into registers (every load in flight together), its largest
// magnitude reduced across the block, then encoded from the registers;
// longer rows are read twice.
constexpr int kActChunks = 8;

__device__ __forceinline__ float amax8(const Vec16& v, float amax)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        amax = fmaxf(amax, fabsf(__uint_as_float(v[i] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(v[i] & 0xFFFF0000u)));
    }
    return amax;
}

__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* x, int64_t rows, int cols, int k,
                                                        const int32_t* inv, uint8_t* codes, float* scales)
{
    __shared__ float red[256 / kWave];
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int step = 256 * 8;  // values per block-wide chunk
    for (int64_t t = blockIdx.x; t < rows; t += gridDim.x) {
        const uint16_t* src = x + t * (int64_t)cols;
        uint8_t* dst = codes + t * (int64_t)cols;
        const bool regs = cols <= kActChunks * step;
        Vec16 v[kActChunks];
        float amax = 0.f;
        if (regs) {
            // Every chunk load is unconditional (a chunk past the row end
            // re-reads the row's last 8 values and is not used): loads under
            // a branch each get a wait for all earlier ones, which would
            // serialise the row's loads.
#pragma unroll
            for (int i = 0; i < kActChunks; ++i)
                v[i] = *(const Vec16*)(src + min(tid * 8 + i * step, cols - 8));
#pragma unroll
            for (int i = 0; i < kActChunks; ++i)
                if (tid * 8 + i * step < cols)
                    amax = amax8(v[i], amax);
        } else {
            for (int c = tid * 8; c < cols; c += step)
                amax = amax8(*(const Vec16*)(src + c), amax);
        }
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1)
            amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
        if (lane == 0)
            red[wv] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();  // red is reused by the next row
        const int e = fp8_scale_exp(amax);
        const float inv_s = ldexpf(1.0f, -e);  // exact: multiplying by it is exact
        if (regs) {
#pragma unroll
            for (int i = 0; i < kActChunks; ++i)
                if (tid * 8 + i * step < cols)
                    *(uint2*)(dst + tid * 8 + i * step) = encode8(v[i], inv_s);
        } else {
            for (int c = tid * 8; c < cols; c += step)
                *(uint2*)(dst + c) = encode8(*(const Vec16*)(src + c), inv_s);
        }
        if (inv) {
            if (tid < k)
                scales[inv[t * k + tid]] = ldexpf(1.0f, e);
        } else if (tid == 0) {
            scales[t] = ldexpf(1.0f, e);
        }
    }
}

// The same for rows of at most 4096 values, one wave per row (4 rows per
// block): lane l holds values l*8 + i*512, i < kCh, with cols <= kCh*512
// (chunk loads unconditional, as above), the row maximum is a wave
// reduction, and no barrier is needed.
template <int kCh>
__global__ __launch_bounds__(256) void act_quant_rows_kernel(const uint16_t* x, int64_t rows, int cols, int k,
                                                             const int32_t* inv, uint8_t* codes, float* scales)
{
    constexpr int kStep = kWave * 8;
    const int lane = threadIdx.x % kWave;
    const int64_t w0 = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + threadIdx.x / kWave));
    const int64_t nw = (int64_t)gridDim.x * 4;
    for (int64_t t = w0; t < rows; t += nw) {
        const uint16_t* src = x + t * (int64_t)cols;
        uint8_t* dst = codes + t * (int64_t)cols;
        Vec16 v[kCh];
#pragma unroll
        for (int i = 0; i < kCh; ++i)
            v[i] = *(const Vec16*)(src + min(lane * 8 + i * kStep, cols - 8));
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < kCh; ++i)
            if (lane * 8 + i * kStep < cols)
                amax = amax8(v[i], amax);
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1)
            amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
        const int e = fp8_scale_exp(amax);
        const float inv_s = ldexpf(1.0f, -e);
#pragma unroll
        for (int i = 0; i < kCh; ++i)
            if (lane * 8 + i * kStep < cols)
                *(uint2*)(dst + lane * 8 + i * kStep) = encode8(v[i], inv_s);
        if (inv) {
            if (lane < k)
                scales[inv[t * k + lane]] = ldexpf(1.0f, e);
        } else if (lane == 0) {
            scales[t] = ldexpf(1.0f, e);
        }
    }
}

}  // namespace

hipError_t launch_act_quant(const void* x, int64_t rows, int cols, int k, const int32_t* inv, uint8_t* codes,
                            float* scales, hipStream_t s)
{
    if (rows < 1)
        return hipSuccess;
    if (cols <= 4096) {
        const int64_t blocks = std::min<int64_t>((rows + 3) / 4, 16384);
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t*)x, rows, cols, k, inv,
                               codes, scales);
        };
        if (cols <= 512)
            go(act_quant_rows_kernel<1>);
        else if (cols <= 1024)
            go(act_quant_rows_kernel<2>);
        else if (cols <= 2048)
            go(act_quant_rows_kernel<4>);
        else
            go(act_quant_rows_kernel<8>);
    } else {
        const int64_t blocks = std::min<int64_t>(rows, 16384);
        hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t*)x, rows, cols,
                           k, inv, codes, scales);
    }
    return hipGetLastError();
}

hipError_t launch_fp8_row_scales(const void* w0, const void* w1, float* scales, int64_t rows, int rows_per_e, int cols,
                                 hipStream_t s)
{
    const int64_t blocks = std::min<int64_t>((rows + 3) / 4, 8192);
    hipLaunchKernelGGL(fp8_row_scale_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t*)w0,
                       (const uint16_t*)w1, scales, rows, rows_per_e, cols, w1 ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_fp8_pack_blocked(const void* w0, const void* w1, const float* scales, void* out, int E, int N, int K,
                                   hipStream_t s)
{
    hipLaunchKernelGGL(fp8_pack_blocked_kernel, dim3(2048), dim3(256), 0, s, (const uint16_t*)w0, (const uint16_t*)w1,
                       scales, (Vec16*)out, E, N, K, w1 ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_fp8_encode_rows(const void* w, const float* scales, uint8_t* codes, int64_t rows, int cols,
                                  hipStream_t s)
{
    const int64_t chunks = rows * (cols / 8);
    const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 8192);
    if (blocks < 1)
        return hipSuccess;
    hipLaunchKernelGGL(fp8_encode_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t*)w, scales,
                       codes, rows, cols);
    return hipGetLastError();
}

}  // namespace cmoe
