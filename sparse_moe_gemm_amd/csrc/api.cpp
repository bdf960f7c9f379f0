// api.cpp - the C ABI (include/colibri_moe.h): validation, one-shot device
// memory, init-time weight repacking, and the five launches of a forward.
//
// Shape of the interface: the pages' init / infer / free with status codes
// («Colibri 是什么» (xxqk.cn) §2.3, «Colibri不是一只蜂鸟» (discosf.com) §4.4).
// All device memory is allocated by init in one allocation and carved into
// weights and workspace («Colibri不是一只蜂鸟» (discosf.com) §3.1 and §5.4:
// allocate once, no runtime allocation, no fragmentation); forward only
// enqueues kernels.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <algorithm>
#include <mutex>
#include <new>
#include <unordered_set>

#include "colibri_moe.h"
#include "common.hpp"

using namespace cmoe;

namespace {

constexpr uint32_t kMagic = 0xC011B41Eu;
constexpr int kStages = 6;
constexpr int32_t kMaxTokensLimit = 1 << 24;

const char* const kStageNames[kStages] = {"router",         "dispatch",  "gate_up_gemm",
                                          "gate_up_reduce", "down_gemm", "combine"};

}  // namespace

// Per-call working memory of a forward, for A = T*k assignments: routing
// buffers the caller did not supply, H, the fp32 partial sums, and the 8-bit
// token rows of the W8A8 mode.
struct Workspace {
    uint8_t* xq;  // q8: token rows as E4M3 codes [T][d]
    float* xsc;   // q8: their scales by sorted position [A]
    float* topw;
    int32_t* ids;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* perm_slot;
    int32_t* inv;
    void* H;      // [A][f] dtype
    float* Ys;    // down GEMM output: kMaxSplit (bf16) or 1 (f32) partials of [A][d] fp32; on the
                  // small-batch path first the gate/up slice partials
};

struct colibri_moe {
    uint32_t magic;
    colibri_moe_config_t cfg;
    int device;
    hipStream_t stream;
    int esize;
    void* arena;
    size_t arena_bytes;
    // weights (library copies, repacked)
    void* w_rt;   // router weights in the router kernels' layout
    float* b_r;   // [E]
    void* w_gu;   // [E][2f][d], gate/up interleaved by 32 rows (bf16: blocked MFMA layout;
                  // fp8: E4M3 codes in the fp8 blocked layout)
    void* w_d;    // [E][d][f] (bf16: blocked MFMA layout; fp8: as w_gu)
    float* s_gu;  // fp8 row scales [E][2f] (interleaved rows), else null
    float* s_d;   // fp8 row scales [E][d], else null
    bool fp8;
    bool q8;      // 8-bit token rows for the gate/up GEMM too (fp8 MFMA)
    Workspace ws; // in the arena, sized for max_tokens
    int32_t* ccnt;  // fused combine: arrivals per token and 128-column tile [max_tokens][d/128], zero between calls
    bool timing;
    hipEvent_t ev[kStages + 1];
    int group_n_gu, group_n_dn;  // tile order of the grouped GEMMs (n-tiles per group)
    int order_m_rows;            // m-tile groups when the mean rows per expert are at most this
    int xcd_map;                 // bit 0: gate/up, bit 1: down GEMM with XCD-contiguous tile placement
    int k64;                     // bit 0: gate/up, bit 1: down GEMM on 64-wide K stages
    bool dec_fuse_silu;          // small-batch gate/up writes H itself (no K slices)
    bool fuse_combine;  // bf16 tiled path: combine in the down GEMM's epilogue
    int cus;        // compute units of the device (persistent GEMM grid)
    int dec_max_a;      // bf16 calls with T*k <= dec_max_a may take the small-batch path,
    int dec_gate_rows;  // those whose experts hold at most this many rows (0: all of them)
    int dec_split_gu, dec_split_dn;  // its K slices (gate/up, down)
};

namespace {

std::mutex g_mu;
std::unordered_set<colibri_moe*> g_live;

bool is_live(colibri_moe* h)
{
    std::lock_guard<std::mutex> lk(g_mu);
    return g_live.count(h) != 0;
}

int env_int(const char* name, int dflt, int lo, int hi)
{
    const char* v = std::getenv(name);
    if (!v || !*v)
        return dflt;
    const long x = std::strtol(v, nullptr, 10);
    return (x < lo || x > hi) ? dflt : (int)x;
}

bool aligned16(const void* p)
{
    return ((uintptr_t)p & 15u) == 0;
}

size_t round_up(size_t v, size_t a)
{
    return (v + a - 1) / a * a;
}

// Carves sub-buffers out of one allocation, 256-byte aligned.
struct Carver {
    size_t off = 0;
    size_t take(size_t bytes)
    {
        const size_t at = off;
        off = round_up(off + bytes, 256);
        return at;
    }
};

// Working memory of colibri_moe_forward_static: one fixed array per GPU in
// the library's code object, so that call allocates nothing. In host code
// `scratch` names a host-side stand-in, not device memory: kernels and copies
// get the device address that hipGetSymbolAddress returns for it, looked up
// once per device (with that device current) and kept here.
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[COLIBRI_MOE_STATIC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
bool g_scratch_done[kMaxDevices];

// Looks up this device's copy of `scratch` (the device must be current).
// Failure leaves the pointer null: only colibri_moe_forward_static needs it.
void setup_static_scratch(int device)
{
    if (device < 0 || device >= kMaxDevices)
        return;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_done[device])
        return;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr) {
        g_scratch_ptr[device] = p;
        g_scratch_done[device] = true;
    } else {
        (void)hipGetLastError();
    }
}

void* static_scratch(int device)
{
    if (device < 0 || device >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    return g_scratch_ptr[device];
}

colibri_moe_status_t validate_config(const colibri_moe_config_t* c)
{
    if (c->dtype != COLIBRI_MOE_F32 && c->dtype != COLIBRI_MOE_BF16)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    if (c->d_model <= 0 || c->d_ff <= 0 || c->n_experts <= 0 || c->max_tokens <= 0)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    if (c->top_k < 1 || c->top_k > c->n_experts)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    if (c->n_experts > kMaxExperts || c->top_k > kMaxTopK)
        return COLIBRI_MOE_ERR_UNSUPPORTED;
    // bf16 GEMMs stage K in 32-wide steps, four per loop trip (K % 128); the
    // fp32 GEMMs use 64-wide tiles.
    if (c->d_model % 128 != 0 || c->d_ff % (c->dtype == COLIBRI_MOE_BF16 ? 128 : 64) != 0)
        return COLIBRI_MOE_ERR_UNSUPPORTED;
    if (c->max_tokens > kMaxTokensLimit)
        return COLIBRI_MOE_ERR_UNSUPPORTED;
    if ((c->flags & COLIBRI_MOE_FLAG_FP8_WEIGHTS) && c->dtype != COLIBRI_MOE_BF16)
        return COLIBRI_MOE_ERR_UNSUPPORTED;
    // 8-bit activations: on top of 8-bit weights; the tiled fp8 GEMMs stream
    // K in 64-wide stages, at least four.
    if ((c->flags & COLIBRI_MOE_FLAG_FP8_ACTIVATIONS) &&
        (!(c->flags & COLIBRI_MOE_FLAG_FP8_WEIGHTS) || c->d_model < 256 || c->d_ff < 256))
        return COLIBRI_MOE_ERR_UNSUPPORTED;
    // GEMM source offsets are 32-bit element offsets.
    const int64_t lim = (int64_t)1 << 31;
    if ((int64_t)c->max_tokens * c->d_model >= lim || (int64_t)c->max_tokens * c->top_k * c->d_ff >= lim ||
        (int64_t)2 * c->d_ff * c->d_model >= lim)
        return COLIBRI_MOE_ERR_UNSUPPORTED;
    return COLIBRI_MOE_OK;
}

#define CMOE_HIP(call)                      \
    do {                                    \
        if ((call) != hipSuccess)           \
            return COLIBRI_MOE_ERR_HIP;     \
    } while (0)

void release(colibri_moe* h)
{
    if (h->arena)
        (void)hipFree(h->arena);
    for (int i = 0; i <= kStages; ++i)
        if (h->ev[i])
            (void)hipEventDestroy(h->ev[i]);
    h->magic = 0;
    delete h;
}

// Layout of the working memory of a call with T tokens (up_to: of every call
// with at most T tokens), carved from `base` (nullptr: sizes only). Returns the
// bytes it spans.
size_t layout_workspace(const colibri_moe* h, int64_t T, bool up_to, uint8_t* base, Workspace* ws)
{
    const colibri_moe_config_t& c = h->cfg;
    const size_t es = (size_t)h->esize;
    const size_t d = c.d_model, f = c.d_ff, E = c.n_experts, k = c.top_k;
    const size_t A = (size_t)T * k;
    Carver cv;
    const size_t o_xq = h->q8 ? cv.take((size_t)T * d) : 0;
    const size_t o_xsc = h->q8 ? cv.take(A * sizeof(float)) : 0;
    const size_t o_topw = cv.take(A * sizeof(float));
    const size_t o_ids = cv.take(A * sizeof(int32_t));
    const size_t o_cnt = cv.take(E * sizeof(int32_t));
    const size_t o_off = cv.take((E + 1) * sizeof(int32_t));
    const size_t o_perm = cv.take(A * sizeof(int32_t));
    const size_t o_ps = cv.take(A * sizeof(int32_t));
    const size_t o_inv = cv.take(A * sizeof(int32_t));
    const size_t o_h = cv.take(A * f * es);
    // Ys: the down GEMM's partial sums (kMaxSplit for bf16), and on the
    // small-batch path also the gate/up slice partials before SiLU.
    size_t ys_floats = (c.dtype == COLIBRI_MOE_BF16 ? (size_t)cmoe::kMaxSplit : 1) * A * d;
    // (calls with A <= dec_max_a may take the small-batch path)
    if (c.dtype == COLIBRI_MOE_BF16 && h->dec_max_a > 0 && (up_to || A <= (size_t)h->dec_max_a)) {
        const size_t ad = std::min(A, (size_t)h->dec_max_a);
        if (!h->dec_fuse_silu)  // else the gate/up kernel writes H itself
            ys_floats = std::max(ys_floats, (size_t)h->dec_split_gu * ad * 2 * f);
        ys_floats = std::max(ys_floats, (size_t)h->dec_split_dn * ad * d);
    }
    const size_t o_ys = cv.take(ys_floats * sizeof(float));
    if (base && ws) {
        ws->xq = h->q8 ? base + o_xq : nullptr;
        ws->xsc = h->q8 ? (float*)(base + o_xsc) : nullptr;
        ws->topw = (float*)(base + o_topw);
        ws->ids = (int32_t*)(base + o_ids);
        ws->counts = (int32_t*)(base + o_cnt);
        ws->offsets = (int32_t*)(base + o_off);
        ws->perm = (int32_t*)(base + o_perm);
        ws->perm_slot = (int32_t*)(base + o_ps);
        ws->inv = (int32_t*)(base + o_inv);
        ws->H = base + o_h;
        ws->Ys = (float*)(base + o_ys);
    }
    return cv.off;
}

colibri_moe_status_t init_impl(colibri_moe* h, const colibri_moe_weights_t* w)
{
    const colibri_moe_config_t& c = h->cfg;
    const size_t es = (size_t)h->esize;
    const size_t d = c.d_model, f = c.d_ff, E = c.n_experts;

    Carver cv;
    const size_t o_wrt = cv.take(router_weight_bytes((int)d, (int)E, (int)es));
    const size_t o_br = cv.take(E * sizeof(float));
    const size_t wes = h->fp8 ? 1 : es;  // bytes per stored expert weight
    const size_t o_wgu = cv.take(E * 2 * f * d * wes);
    const size_t o_wd = cv.take(E * d * f * wes);
    const size_t o_sgu = h->fp8 ? cv.take(E * 2 * f * sizeof(float)) : 0;
    const size_t o_sd = h->fp8 ? cv.take(E * d * sizeof(float)) : 0;
    const size_t o_ccnt = h->fuse_combine ? cv.take((size_t)c.max_tokens * (d / 128) * sizeof(int32_t)) : 0;
    const size_t o_ws = cv.take(layout_workspace(h, c.max_tokens, true, nullptr, nullptr));
    h->arena_bytes = cv.off;

    if (hipMalloc(&h->arena, h->arena_bytes) != hipSuccess) {
        h->arena = nullptr;
        (void)hipGetLastError();
        return COLIBRI_MOE_ERR_OUT_OF_MEMORY;
    }
    uint8_t* base = (uint8_t*)h->arena;
    h->w_rt = base + o_wrt;
    h->b_r = (float*)(base + o_br);
    h->w_gu = base + o_wgu;
    h->w_d = base + o_wd;
    h->s_gu = h->fp8 ? (float*)(base + o_sgu) : nullptr;
    h->s_d = h->fp8 ? (float*)(base + o_sd) : nullptr;
    h->ccnt = h->fuse_combine ? (int32_t*)(base + o_ccnt) : nullptr;
    layout_workspace(h, c.max_tokens, true, base + o_ws, &h->ws);

    hipStream_t s = h->stream;
    if (h->ccnt)
        CMOE_HIP(hipMemsetAsync(h->ccnt, 0, (size_t)c.max_tokens * (d / 128) * sizeof(int32_t), s));
    CMOE_HIP(launch_transpose_router(w->w_router, h->w_rt, (int)d, (int)E, (int)es, s));
    if (w->b_router)
        CMOE_HIP(hipMemcpyAsync(h->b_r, w->b_router, E * sizeof(float), hipMemcpyDeviceToDevice, s));
    else
        CMOE_HIP(hipMemsetAsync(h->b_r, 0, E * sizeof(float), s));
    if (h->fp8) {
        // row scales, then E4M3 codes in the fp8 blocked layout (gate/up
        // interleaved by 32 rows, scales in the interleaved row order)
        CMOE_HIP(launch_fp8_row_scales(w->w_gate, w->w_up, h->s_gu, (int64_t)E * 2 * f, (int)(2 * f), (int)d, s));
        CMOE_HIP(launch_fp8_row_scales(w->w_down, nullptr, h->s_d, (int64_t)E * d, (int)d, (int)f, s));
        CMOE_HIP(launch_fp8_pack_blocked(w->w_gate, w->w_up, h->s_gu, h->w_gu, (int)E, (int)(2 * f), (int)d, s));
        CMOE_HIP(launch_fp8_pack_blocked(w->w_down, nullptr, h->s_d, h->w_d, (int)E, (int)d, (int)f, s));
    } else if (c.dtype == COLIBRI_MOE_BF16) {
        // blocked MFMA operand layout (gate/up interleaved by 32 rows)
        CMOE_HIP(launch_pack_blocked(w->w_gate, w->w_up, h->w_gu, (int)E, (int)(2 * f), (int)d, 1, s));
        CMOE_HIP(launch_pack_blocked(w->w_down, nullptr, h->w_d, (int)E, (int)d, (int)f, 0, s));
    } else {
        CMOE_HIP(launch_interleave_gate_up(w->w_gate, w->w_up, h->w_gu, (int)E, (int)f, (int)d, (int)es, s));
        CMOE_HIP(hipMemcpyAsync(h->w_d, w->w_down, E * d * f * es, hipMemcpyDeviceToDevice, s));
    }
    if (h->timing)
        for (int i = 0; i <= kStages; ++i)
            CMOE_HIP(hipEventCreate(&h->ev[i]));
    CMOE_HIP(hipStreamSynchronize(s));
    return COLIBRI_MOE_OK;
}

}  // namespace

extern "C" {

colibri_moe_status_t colibri_moe_init(colibri_moe_t** out, const colibri_moe_config_t* cfg,
                                      const colibri_moe_weights_t* w, void* hip_stream)
{
    if (!out || !cfg || !w)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    *out = nullptr;
    colibri_moe_status_t st = validate_config(cfg);
    if (st != COLIBRI_MOE_OK)
        return st;
    if (!w->w_router || !w->w_gate || !w->w_up || !w->w_down)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    if (!aligned16(w->w_router) || !aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down) ||
        ((uintptr_t)w->b_router & 3u))
        return COLIBRI_MOE_ERR_ALIGNMENT;

    colibri_moe* h = new (std::nothrow) colibri_moe();
    if (!h)
        return COLIBRI_MOE_ERR_OUT_OF_MEMORY;
    h->magic = kMagic;
    h->cfg = *cfg;
    h->stream = (hipStream_t)hip_stream;
    h->esize = cfg->dtype == COLIBRI_MOE_BF16 ? 2 : 4;
    h->timing = (cfg->flags & COLIBRI_MOE_FLAG_STAGE_TIMING) != 0;
    h->fp8 = (cfg->flags & COLIBRI_MOE_FLAG_FP8_WEIGHTS) != 0;
    h->q8 = (cfg->flags & COLIBRI_MOE_FLAG_FP8_ACTIVATIONS) != 0;
    // Tile order of the grouped GEMMs (tuning only; results do not depend
    // on it): n-tiles per group, CMOE_GROUP_N for both GEMMs.
    // Consecutive tiles go to the 8 XCDs in turn. With groups of 16 n-tiles
    // each XCD takes two n-tiles of a group for all of its m-tiles, so a
    // weight panel is read into one XCD's L2 and reused there, and each
    // m-tile's token rows serve two tiles running side by side on that XCD.
    // Measured with the gate/up GEMM's 64-wide K stages: one expert of 8192
    // rows x 28672 x 4096 1.73 -> 1.47 ms against groups of 8, 4096 rows
    // 798 -> 785 us, mixtral 1.70 -> 1.69 ms, the skewed shape unchanged.
    // The down GEMM keeps groups of 64 (1-3% better there than 8 or 16).
    const int gn = env_int("CMOE_GROUP_N", 0, 0, 1 << 20);
    h->group_n_gu = gn > 0 ? gn : 16;
    h->group_n_dn = gn > 0 ? gn : 64;
    // Many experts of one or two m-tiles each (fine-grained layers): token
    // rows are the data read again and again (once per n-tile), weight
    // panels once or twice; there the tile order keeps an m-tile's n-tiles on
    // one XCD (groups of 8 m-tiles) instead. Chosen per call from the mean
    // rows per expert (threshold CMOE_M_ORDER_ROWS, 0 = never).
    h->order_m_rows = env_int("CMOE_M_ORDER_ROWS", 384, 0, 1 << 30);
    h->xcd_map = env_int("CMOE_XCD_MAP", 0, 0, 3);
    // 64-wide K stages (grouped_gemm64_kernel) for the bf16 gate/up GEMM
    // (with tile groups of 16 n-tiles): mixtral gate/up 1.76 -> 1.68 ms, one
    // expert of 8192 rows 1.66 -> 1.44 ms; the down GEMM keeps 32-wide stages
    // (with 64: mixtral 915 -> 920 us, fine-grained 164 -> 167, skewed
    // 428 -> 449, with the current epilogues). Same sums in the same order, so outputs are
    // bit-identical either way. CMOE_K64: bit 0 gate/up, bit 1 down, bit 2
    // gate/up whatever the rows per expert.
    h->k64 = env_int("CMOE_K64", 1, 0, 7);
    // Combine fused into the down GEMM's epilogue (bf16 layers, tiled path)
    // with CMOE_FUSE_COMBINE=1; the default runs the combine kernel, which is
    // faster here: the fused form needs device-scope release/acquire fences
    // in every tile's epilogue (L2 write-back and invalidation across the
    // XCDs' separate L2s) and reads the other rows of a token with little
    // memory parallelism on the GEMM's critical path. Results are identical
    // either way.
    h->fuse_combine = cfg->dtype == COLIBRI_MOE_BF16 && env_int("CMOE_FUSE_COMBINE", 0, 0, 1) != 0;
    if (hipGetDevice(&h->device) != hipSuccess ||
        hipDeviceGetAttribute(&h->cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess ||
        h->cus <= 0) {
        (void)hipGetLastError();
        release(h);
        return COLIBRI_MOE_ERR_HIP;
    }
    setup_static_scratch(h->device);
    // Small-batch path (bf16): calls with at most CMOE_DECODE_MAX_A
    // assignments (default 2048; 0 turns the path off) and, for calls of
    // more than CMOE_DECODE_MAX_ROWS tokens (default 48, 32 with 8-bit
    // weights, whose kernels take 32 rows per weight pass; 0: no such test),
    // only when no expert holds more rows than that (decided on the device).
    // Results do not depend on the path beyond fp32 summation order.
    h->dec_max_a = 0;
    h->dec_gate_rows = 0;
    h->dec_split_gu = h->dec_split_dn = 1;
    if (cfg->dtype == COLIBRI_MOE_BF16) {
        const int64_t amax = (int64_t)cfg->max_tokens * cfg->top_k;
        h->dec_max_a = (int)std::min<int64_t>(amax, env_int("CMOE_DECODE_MAX_A", 2048, 0, 1 << 16));
        h->dec_gate_rows = env_int("CMOE_DECODE_MAX_ROWS", h->fp8 ? 32 : 48, 0, 1 << 16);
        const int waves = cmoe::decode_waves(h->cus);
        // k step of the small-batch kernels: 16 (bf16 weights), 32 (8-bit
        // weights), 64 (8-bit token rows, gate/up only)
        const int kstep_dn = h->fp8 ? 32 : 16;
        const int kstep_gu = h->q8 ? 64 : kstep_dn;
        h->dec_split_gu = cmoe::decode_split(cfg->n_experts, 2 * cfg->d_ff, cfg->d_model, kstep_gu, waves, 64);
        // No K slices: the gate/up items write H themselves (SiLU(g)*u in
        // their epilogue) instead of partials for a separate sum pass
        // (CMOE_DECODE_FUSE_SILU=0 keeps the pass)
        h->dec_fuse_silu = h->dec_split_gu == 1 && env_int("CMOE_DECODE_FUSE_SILU", 1, 0, 1) != 0;
        h->dec_split_dn = cmoe::decode_split(cfg->n_experts, cfg->d_model, cfg->d_ff, kstep_dn, waves, 64);
    }
    st = init_impl(h, w);
    if (st != COLIBRI_MOE_OK) {
        release(h);
        return st;
    }
    {
        std::lock_guard<std::mutex> lk(g_mu);
        g_live.insert(h);
    }
    *out = h;
    return COLIBRI_MOE_OK;
}

}  // extern "C"

namespace {

// The enqueued work of one forward (T >= 1, arguments checked by
// check_call) with its working memory in ws; fused: the combine runs in the
// down GEMM's epilogue (handle arena only: its counters must be zero).
colibri_moe_status_t forward_impl(colibri_moe* h, const void* x, int32_t T, void* y,
                                  const colibri_moe_routing_t& ro, const Workspace& ws, bool fused_ok)
{
    const colibri_moe_config_t& c = h->cfg;
    // Caller-provided routing buffers double as the working buffers (no copy).
    float* topw = ro.topk_w ? ro.topk_w : ws.topw;
    int32_t* ids = ro.topk_ids ? ro.topk_ids : ws.ids;
    int32_t* counts = ro.expert_counts ? ro.expert_counts : ws.counts;
    int32_t* offsets = ro.expert_offsets ? ro.expert_offsets : ws.offsets;
    int32_t* perm = ro.perm ? ro.perm : ws.perm;
    int32_t* perm_slot = ro.perm_slot ? ro.perm_slot : ws.perm_slot;
    int32_t* inv = ro.inv ? ro.inv : ws.inv;
    const bool bf = c.dtype == COLIBRI_MOE_BF16;
    hipStream_t s = h->stream;
    const bool tm = h->timing;
    if (tm)
        CMOE_HIP(hipEventRecord(h->ev[0], s));

    RouterArgs ra{x, h->w_rt, h->b_r, T, c.d_model, c.n_experts, c.top_k, ro.logits, ids, topw};
    CMOE_HIP(bf ? launch_router_bf16(ra, s) : launch_router_f32(ra, s));
    if (tm)
        CMOE_HIP(hipEventRecord(h->ev[1], s));

    DispatchArgs da{ids, T, c.top_k, c.n_experts, counts, offsets, perm, perm_slot, inv};
    CMOE_HIP(launch_dispatch(da, s));
    const bool q8 = h->q8;
    if (q8)  // token rows to 8 bits, scales by sorted position
        CMOE_HIP(launch_act_quant(x, T, c.d_model, c.top_k, inv, ws.xq, ws.xsc, s));
    if (tm)
        CMOE_HIP(hipEventRecord(h->ev[2], s));

    const int A = T * c.top_k;
    // Path choice. Calls with A <= dec_max_a go to the small-batch kernels
    // (weight streaming: K slices, then the slice sum and SiLU(g)*u), the
    // others to the tiled grouped GEMMs. The small-batch kernels win while
    // every expert holds few rows, which the host cannot see (skewed routing
    // puts most tokens on a few experts): a call that may hold an expert with
    // more than dec_gate_rows rows (T > dec_gate_rows) enqueues both paths,
    // and each kernel takes or leaves the call from offsets on the device.
    const bool small = bf && A <= h->dec_max_a;
    const int gate = small && h->dec_gate_rows > 0 && T > h->dec_gate_rows ? h->dec_gate_rows : 0;
    const bool tiled = !small || gate > 0;
    const bool order_m = (int64_t)A <= (int64_t)h->order_m_rows * c.n_experts;
    if (small) {
        DecodeArgs gu{q8 ? (const void*)ws.xq : x, h->w_gu, h->s_gu, q8 ? ws.xsc : nullptr, ws.Ys, offsets, perm,
                      A, c.n_experts, c.d_model, c.d_ff, h->dec_split_gu};
        gu.h = h->dec_fuse_silu ? (uint16_t*)ws.H : nullptr;
        gu.max_rows = T;
        gu.gate_rows = gate;
        CMOE_HIP(launch_decode_gemm(gu, 1, h->cus, s));
    }
    if (tiled) {
        GemmArgs gu{q8 ? (const void*)ws.xq : x, h->w_gu, h->s_gu, q8 ? ws.xsc : nullptr, ws.H, offsets, perm, A,
                    c.n_experts, c.top_k, c.d_model, c.d_ff, order_m ? -8 : h->group_n_gu, 1, h->cus};
        gu.xcd_map = h->xcd_map & 1;
        // 64-wide K stages for layers of at least three m-tiles per expert on
        // average (mixtral, one big expert) and for layers in m-tile order
        // (many experts of one or two m-tiles: fine-grained, 1.8% less layer
        // time); in between (skewed, 512 rows on average but two experts of
        // ~15 k rows and 62 of at most 56) they measured 2% slower than
        // 32-wide stages (CMOE_K64 bit 2 drops this condition)
        gu.k64 = (h->k64 & 1) && ((h->k64 & 4) || order_m || (int64_t)A >= (int64_t)768 * c.n_experts);
        gu.skip_rows = gate;
        CMOE_HIP(bf ? launch_gate_up_bf16(gu, s) : launch_gate_up_f32(gu, s));
    }
    if (tm)
        CMOE_HIP(hipEventRecord(h->ev[3], s));
    if (small && !h->dec_fuse_silu)
        CMOE_HIP(launch_decode_silu(ws.Ys, ws.H, A, c.d_ff, h->dec_split_gu, offsets, c.n_experts, gate, s));
    if (tm)
        CMOE_HIP(hipEventRecord(h->ev[4], s));

    int split = 1;
    bool fused = false;    // combine done by the down GEMM
    int ys_bf16 = 0;       // expert outputs stored as bf16
    if (small) {
        DecodeArgs dn{ws.H, h->w_d, h->s_d, nullptr, ws.Ys, offsets, perm,
                      A, c.n_experts, c.d_model, c.d_ff, h->dec_split_dn};
        dn.max_rows = T;
        dn.gate_rows = gate;
        CMOE_HIP(launch_decode_gemm(dn, 0, h->cus, s));
        split = h->dec_split_dn;
    }
    if (tiled) {
        split = bf ? down_split_bf16(A, c.n_experts, c.d_model, c.d_ff, h->cus, 0) : 1;
        GemmArgs dn{ws.H, h->w_d, h->s_d, nullptr, ws.Ys, offsets, perm, A,
                    c.n_experts, c.top_k, c.d_model, c.d_ff, order_m ? -8 : h->group_n_dn, split, h->cus};
        if (bf && h->ccnt && fused_ok && gate == 0) {
            dn.cnt = h->ccnt;
            dn.inv = inv;
            dn.topw = topw;
            dn.y = y;
            fused = true;
        }
        // Without a K split the expert outputs go to Ys as bf16 rows (any
        // weight precision of a bf16 layer).
        dn.ys_bf16 = bf && split == 1 && !fused;
        dn.xcd_map = (h->xcd_map >> 1) & 1;
        dn.k64 = (h->k64 >> 1) & 1;
        dn.skip_rows = gate;
        ys_bf16 = dn.ys_bf16;
        CMOE_HIP(bf ? launch_down_bf16(dn, s) : launch_down_f32(dn, s));
    }
    if (tm)
        CMOE_HIP(hipEventRecord(h->ev[5], s));

    if (!fused) {
        CombineArgs ca{ws.Ys, inv, topw, y, T, c.top_k, c.d_model, split, bf ? 1 : 0, ys_bf16};
        if (gate > 0) {
            ca.offsets = offsets;
            ca.E = c.n_experts;
            ca.gate_rows = gate;
            ca.small_split = h->dec_split_dn;
        }
        CMOE_HIP(launch_combine(ca, s));
    }
    if (tm)
        CMOE_HIP(hipEventRecord(h->ev[6], s));

    if (!(c.flags & COLIBRI_MOE_FLAG_ASYNC))
        CMOE_HIP(hipStreamSynchronize(s));
    return COLIBRI_MOE_OK;
}

// Argument checks shared by both forward entry points. Returns OK with
// *skip set for T = 0 (nothing to do).
colibri_moe_status_t check_call(colibri_moe* h, const void* x, int32_t T, void* y,
                                const colibri_moe_routing_t* r, colibri_moe_routing_t* ro, bool* skip)
{
    *skip = false;
    if (!h || !is_live(h) || h->magic != kMagic)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    if (T < 0 || T > h->cfg.max_tokens)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    if (T == 0) {
        *skip = true;
        return COLIBRI_MOE_OK;
    }
    if (!x || !y)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(y))
        return COLIBRI_MOE_ERR_ALIGNMENT;
    *ro = colibri_moe_routing_t{};
    if (r)
        *ro = *r;
    // topk_ids is read as whole 16-byte rows by the dispatch kernel; the
    // other routing buffers hold 4-byte elements.
    if (((uintptr_t)ro->topk_ids & 15u) || ((uintptr_t)ro->topk_w & 3u) || ((uintptr_t)ro->expert_counts & 3u) ||
        ((uintptr_t)ro->expert_offsets & 3u) || ((uintptr_t)ro->perm & 3u) || ((uintptr_t)ro->perm_slot & 3u) ||
        ((uintptr_t)ro->inv & 3u) || ((uintptr_t)ro->logits & 3u))
        return COLIBRI_MOE_ERR_ALIGNMENT;
    return COLIBRI_MOE_OK;
}

}  // namespace

extern "C" {

colibri_moe_status_t colibri_moe_forward(colibri_moe_t* h, const void* x, int32_t T, void* y,
                                         const colibri_moe_routing_t* r)
{
    colibri_moe_routing_t ro;
    bool skip;
    const colibri_moe_status_t st = check_call(h, x, T, y, r, &ro, &skip);
    if (st != COLIBRI_MOE_OK || skip)
        return st;
    return forward_impl(h, x, T, y, ro, h->ws, true);
}

colibri_moe_status_t colibri_moe_forward_static(colibri_moe_t* h, const void* x, int32_t T, void* y,
                                                const colibri_moe_routing_t* r)
{
    colibri_moe_routing_t ro;
    bool skip;
    const colibri_moe_status_t st = check_call(h, x, T, y, r, &ro, &skip);
    if (st != COLIBRI_MOE_OK || skip)
        return st;
    if (layout_workspace(h, T, false, nullptr, nullptr) > (size_t)COLIBRI_MOE_STATIC_SCRATCH_BYTES)
        return COLIBRI_MOE_ERR_TOO_LARGE;
    uint8_t* base = (uint8_t*)static_scratch(h->device);
    if (!base)
        return COLIBRI_MOE_ERR_HIP;
    Workspace ws;
    layout_workspace(h, T, false, base, &ws);
    return forward_impl(h, x, T, y, ro, ws, false);
}


colibri_moe_status_t colibri_moe_free(colibri_moe_t* h)
{
    if (!h)
        return COLIBRI_MOE_OK;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!g_live.erase(h))
            return COLIBRI_MOE_ERR_INVALID_ARG;
    }
    const bool ok = hipStreamSynchronize(h->stream) == hipSuccess;
    release(h);
    return ok ? COLIBRI_MOE_OK : COLIBRI_MOE_ERR_HIP;
}

colibri_moe_status_t colibri_moe_quantize_fp8(const void* w, int64_t rows, int64_t cols, uint8_t* codes,
                                              float* scales, void* hip_stream)
{
    if (!w || !codes || !scales || rows < 1 || cols < 8 || cols % 8 != 0 || cols > INT32_MAX ||
        rows > ((int64_t)1 << 40) / cols)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    if (!aligned16(w) || ((uintptr_t)codes & 7u) || ((uintptr_t)scales & 3u))
        return COLIBRI_MOE_ERR_ALIGNMENT;
    hipStream_t s = (hipStream_t)hip_stream;
    CMOE_HIP(launch_fp8_row_scales(w, nullptr, scales, rows, 0, (int)cols, s));
    CMOE_HIP(launch_fp8_encode_rows(w, scales, codes, rows, (int)cols, s));
    CMOE_HIP(hipStreamSynchronize(s));
    return COLIBRI_MOE_OK;
}

colibri_moe_status_t colibri_moe_stream_copy(const void* src, void* dst, int64_t bytes, void* hip_stream)
{
    if (!src || !dst || bytes < 16 || bytes % 16 != 0)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(dst))
        return COLIBRI_MOE_ERR_ALIGNMENT;
    const uint8_t *s0 = (const uint8_t*)src, *d0 = (const uint8_t*)dst;
    if (s0 < d0 + bytes && d0 < s0 + bytes)
        return COLIBRI_MOE_ERR_INVALID_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return COLIBRI_MOE_ERR_HIP;
    }
    CMOE_HIP(launch_stream_copy(src, dst, bytes, cus, (hipStream_t)hip_stream));
    return COLIBRI_MOE_OK;
}

const char* colibri_moe_status_string(colibri_moe_status_t s)
{
    switch (s) {
    case COLIBRI_MOE_OK:
        return "ok";
    case COLIBRI_MOE_ERR_INVALID_ARG:
        return "invalid argument";
    case COLIBRI_MOE_ERR_UNSUPPORTED:
        return "unsupported configuration";
    case COLIBRI_MOE_ERR_ALIGNMENT:
        return "pointer not aligned (16 bytes for x, y, weights and topk_ids; 4 for the other routing buffers)";
    case COLIBRI_MOE_ERR_OUT_OF_MEMORY:
        return "out of device memory";
    case COLIBRI_MOE_ERR_HIP:
        return "HIP runtime error";
    case COLIBRI_MOE_ERR_TOO_LARGE:
        return "batch needs more working memory than the static scratch array holds";
    }
    return "unknown status";
}

int32_t colibri_moe_stage_times(colibri_moe_t* h, float* ms, int32_t n)
{
    if (!h || !is_live(h) || !h->timing)
        return -1;
    if (hipEventSynchronize(h->ev[kStages]) != hipSuccess)
        return -1;
    for (int i = 0; i < kStages && i < n; ++i) {
        float v = 0.f;
        if (hipEventElapsedTime(&v, h->ev[i], h->ev[i + 1]) != hipSuccess)
            return -1;
        if (ms)
            ms[i] = v;
    }
    return kStages;
}

const char* colibri_moe_stage_name(int32_t stage)
{
    return (stage >= 0 && stage < kStages) ? kStageNames[stage] : nullptr;
}

}  // extern "C"
