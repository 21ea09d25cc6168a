// C ABI of libmoe.so: argument validation, workspace carving and kernel
// launches on the caller's stream.  No allocation, no host synchronisation,
// no reads of device memory on the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_map>

#include "launch.h"
#include "moe.h"

static_assert((int)moe::K_COUNT == (int)MOE_K_COUNT, "kernel ids out of sync");
static_assert((int)moe::K_GATEUP_LIGHT == (int)MOE_K_GATEUP_LIGHT, "kernel ids out of sync");
static_assert((int)moe::K_COMBINE == (int)MOE_K_COMBINE, "kernel ids out of sync");
static_assert((int)moe::K_PERM_SMALL == (int)MOE_K_PERM_SMALL, "kernel ids out of sync");

namespace moe {
ProfileHook g_profile;
}

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

}  // namespace

namespace moe {
int report_error(int code, const char* msg) { return fail(code, msg); }
}  // namespace moe

namespace {

constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    // max_tiles: heavy-grid bound when every token's ids are distinct (the
    // router's output); plan_tiles: tile capacity of the plan region, which
    // also holds the tiles of ids that repeat within a token (moe_permute
    // accepts them, so an expert can then get more than T rows).
    int splits = 1, nchunks = 1, light_max = 0, max_tiles = 0, max_light = 0, plan_tiles = 0;
    size_t part = 0, ids = 0, w = 0, chunk = 0, counts = 0, offsets = 0, sorted = 0, inv = 0,
           plan = 0, sync = 0, h = 0, y = 0, hs = 0, total = 0;
};

#ifndef MOE_ROUTER_MIN_BLOCKS
#define MOE_ROUTER_MIN_BLOCKS 512
#endif

// Split-K factor of the router GEMM: doubled while the grid has fewer than
// MOE_ROUTER_MIN_BLOCKS blocks and each split keeps >= 64 of H.
int router_splits(int T, int H, int E) {
    const long long base = (long long)((E + moe::kRouterBE - 1) / moe::kRouterBE) *
                           ((T + moe::kRouterBT - 1) / moe::kRouterBT);
    int s = 1;
    while (base * s < MOE_ROUTER_MIN_BLOCKS && H % (2 * s * moe::kRouterBK) == 0 && H / (2 * s) >= 64)
        s *= 2;
    return s;
}

// Storage of the routed outputs y: 0 fp32, 1 bf16, 2 fp16.
int y_format(const moe_shape* s) { return s->y_fp16 ? 2 : (s->y_bf16 ? 1 : 0); }

int check_shape(const moe_shape* s) {
    if (!s) return fail(MOE_ERR_NULL, "shape is NULL");
    if (s->T < 0 || s->H <= 0 || s->E <= 0 || s->k <= 0 || s->I <= 0 || s->I_shared < 0)
        return fail(MOE_ERR_SHAPE, "sizes must be T >= 0 and H, E, k, I > 0, I_shared >= 0");
    if (s->k > s->E) return fail(MOE_ERR_SHAPE, "k > E");
    if ((long long)s->T * s->k >= (1LL << 31)) return fail(MOE_ERR_SHAPE, "T*k >= 2^31");
    if ((long long)s->T * s->H >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*H must be < 2^31");
    if ((long long)s->I * s->H >= (1LL << 30) || (long long)s->I_shared * s->H >= (1LL << 30))
        return fail(MOE_ERR_UNSUPPORTED, "I*H and I_shared*H must be < 2^30");
    if (s->H % 64) return fail(MOE_ERR_UNSUPPORTED, "H must be a multiple of 64");
    if (s->I % 32) return fail(MOE_ERR_UNSUPPORTED, "I must be a multiple of 32");
    if (s->I_shared % 32) return fail(MOE_ERR_UNSUPPORTED, "I_shared must be a multiple of 32");
    if (s->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E must be <= 1024");
    if (s->k > 32) return fail(MOE_ERR_UNSUPPORTED, "k must be <= 32");
    if (s->renorm != 0 && s->renorm != 1) return fail(MOE_ERR_UNSUPPORTED, "renorm must be 0 or 1");
    if (s->light_max_rows < -1 || s->light_max_rows > moe::kLightRowsMax)
        return fail(MOE_ERR_UNSUPPORTED, "light_max_rows must be -1 or in [0, 64]");
    if (s->heavy_tile_rows != 0 && !moe::valid_tile_height(s->heavy_tile_rows))
        return fail(MOE_ERR_UNSUPPORTED, "heavy_tile_rows must be 0, 128, 160, 192, 224 or 256");
    if (s->y_bf16 != 0 && s->y_bf16 != 1) return fail(MOE_ERR_UNSUPPORTED, "y_bf16 must be 0 or 1");
    if (s->y_fp16 != 0 && s->y_fp16 != 1) return fail(MOE_ERR_UNSUPPORTED, "y_fp16 must be 0 or 1");
    if (s->y_bf16 && s->y_fp16) return fail(MOE_ERR_UNSUPPORTED, "y_bf16 and y_fp16 are exclusive");
    if (s->w_mxfp8 != 0 && s->w_mxfp8 != 1)
        return fail(MOE_ERR_UNSUPPORTED, "w_mxfp8 must be 0 or 1");
    if (s->w_mxfp8 && s->heavy_tile_rows > -moe::kTileMaxMx)
        return fail(MOE_ERR_UNSUPPORTED, "MXFP8 heavy tiles are at most 192 rows");
    return MOE_OK;
}

Layout layout(const moe_shape* s) {
    Layout L;
    const long long T = s->T, H = s->H, E = s->E, k = s->k, I = s->I, A = T * k;
    L.splits = router_splits(s->T, s->H, s->E);
    L.nchunks = (int)std::max<long long>(1, (A + moe::kPermChunk - 1) / moe::kPermChunk);
    // Each token picks k distinct experts, so no expert gets more than T rows:
    // with T <= light_max every expert is light and no heavy tile can exist.
    // The default is the per-call choice on the device (kLightAdaptive) from
    // 65 tokens on, with grids sized for either outcome; up to 64 tokens
    // every expert is light and no heavy kernel is launched.
    if (s->light_max_rows < 0 && T <= moe::kLightRowsMax) {
        L.light_max = moe::kLightRowsMax;
        L.max_tiles = 0;
        L.max_light = (int)std::min<long long>(E, A);
    } else if (s->light_max_rows < 0 && moe::adaptive_light_max(A, E) < moe::kLightRowsMax) {
        // No more than E experts are touched, so beyond MOE_LIGHT_MEAN_ROWS * E
        // routed rows the rule always picks the tail threshold: fix it.
        L.light_max = moe::adaptive_light_max(A, E);
        L.max_tiles = moe::max_heavy_tiles(A, s->E, L.light_max);
        L.max_light = L.light_max > 0 ? (int)std::min<long long>(E, A) : 0;
    } else if (s->light_max_rows < 0) {
        L.light_max = moe::kLightAdaptive;
        L.max_tiles = moe::max_heavy_tiles(A, s->E, 0);
        L.max_light = (int)std::min<long long>(E, A);
    } else {
        L.light_max = s->light_max_rows;
        L.max_tiles = (T <= L.light_max) ? 0 : moe::max_heavy_tiles(A, s->E, L.light_max);
        L.max_light = L.light_max > 0 ? (int)std::min<long long>(E, A) : 0;
    }
    L.plan_tiles = moe::max_heavy_tiles(A, s->E, L.light_max > 0 ? L.light_max : 0);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += up(bytes);
        return at;
    };
    L.part = take((size_t)L.splits * T * E * 4);
    L.ids = take((size_t)A * 4);
    L.w = take((size_t)A * 4);
    L.chunk = take((size_t)L.nchunks * E * 4);
    L.counts = take((size_t)E * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.sorted = take((size_t)A * 4);
    L.inv = take((size_t)A * 4);
    L.plan = take((size_t)(moe::kPlanHeader + E + 2LL * L.plan_tiles) * 4);
    L.sync = take((size_t)moe::sync_ints(s->E) * 4);
    L.h = take((size_t)A * I * 2);
    L.y = take((size_t)A * H * (y_format(s) ? 2 : 4));
    L.hs = take((size_t)T * 2 * s->I_shared * 2);  // [hi | lo] rows
    L.total = off;
    return L;
}

bool aligned(const void* p, size_t a = 16) { return ((uintptr_t)p % a) == 0; }

// Tile height rule handed to the plan kernels (see tile_split).
int plan_force_tm(const moe_shape* s) {
    if (s->w_mxfp8 && s->heavy_tile_rows == 0) return moe::kTileMaxMx;
    return s->heavy_tile_rows;
}

int check_ws(const moe_shape* s, const void* ws, size_t ws_bytes) {
    if (!ws) return fail(MOE_ERR_NULL, "workspace is NULL");
    if (!aligned(ws, kAlign)) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
    const size_t need = layout(s).total;
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                           " bytes, got " + std::to_string(ws_bytes));
    return MOE_OK;
}

#define REQUIRE_PTR(p)                                                     \
    do {                                                                   \
        if (!(p)) return fail(MOE_ERR_NULL, #p " is NULL");                \
        if (!aligned(p)) return fail(MOE_ERR_ALIGN, #p " is not 16-byte aligned"); \
    } while (0)
#define OPTIONAL_PTR(p)                                                    \
    do {                                                                   \
        if ((p) && !aligned(p)) return fail(MOE_ERR_ALIGN, #p " is not 16-byte aligned"); \
    } while (0)
#define HIP_TRY(expr, what)                                                \
    do {                                                                   \
        hipError_t e_ = (expr);                                            \
        if (e_ != hipSuccess)                                              \
            return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e_)); \
    } while (0)

int device_cu_count(int* out) {
    static std::mutex mu;
    static std::unordered_map<int, int> cache;
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it == cache.end()) {
        int n = 0;
        HIP_TRY(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev),
                "hipDeviceGetAttribute");
        it = cache.emplace(dev, std::max(n, 1)).first;
    }
    *out = it->second;
    return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int run_router(const moe_shape* s, const Layout& L, const uint16_t* x, const float* wr,
               const float* bias, int32_t* ids, float* w, float* probs, void* ws,
               hipStream_t st) {
    float* part = at<float>(ws, L.part);
    HIP_TRY(moe::launch_router_gemm(x, wr, part, s->T, s->H, s->E, L.splits, st), "router gemm");
    HIP_TRY(moe::launch_router_select(part, L.splits, bias, s->T, s->E, s->k, s->renorm, ids, w,
                                      probs, st),
            "router select");
    return MOE_OK;
}

// Tiles per round of the heavy GEMMs' XCD slices on this device (see
// moe::xcd_bounds).
int plan_round_tiles(const moe_shape* s, int* out) {
    int ncu = 0;
    if (int rc = device_cu_count(&ncu)) return rc;
    const int nblk_gu = (2 * s->I + moe::kTileN - 1) / moe::kTileN;
    const int nblk_dn = (s->H + moe::kTileN - 1) / moe::kTileN;
    *out = moe::slice_round_tiles(ncu, nblk_gu, nblk_dn);
    return MOE_OK;
}

// The shared expert depends on x alone, so moe_forward runs it on a second
// stream of the device beside the routing and the routed FFN (which read x,
// the router and expert weights and write only the workspace): the side
// stream waits for an event recorded on the caller's stream before the
// router, and the caller's stream waits for the side stream's last launch
// before the combine, which adds the routed outputs to the shared expert's.
// One side stream and one fork/join event pair per device, created at the
// first call that needs them (default priority, non-blocking); g_side_mu is
// held from the fork until the join is enqueued, so calls from several host
// threads pair their own records and waits (and their shared experts queue
// on the one side stream).  Built with MOE_SHARED_OVERLAP=0, everything is
// enqueued on the caller's stream.
#ifndef MOE_SHARED_OVERLAP
#define MOE_SHARED_OVERLAP 1
#endif
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxSideDevices];

// Call with g_side_mu held.
int side_stream(SideStream** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxSideDevices)
        return fail(MOE_ERR_UNSUPPORTED, "device index beyond the side-stream table");
    SideStream& ss = g_side[dev];
    if (!ss.s) {
        HIP_TRY(hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming), "side fork event");
        HIP_TRY(hipEventCreateWithFlags(&ss.join, hipEventDisableTiming), "side join event");
        HIP_TRY(hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking), "side stream");
    }
    *out = &ss;
    return MOE_OK;
}

// Returns through *plan_ready whether the permute also wrote the FFN plan
// (single-block path); then run_ffn skips its plan kernel.
int run_permute(const moe_shape* s, const Layout& L, const int32_t* ids, int32_t* counts,
                int32_t* offsets, int32_t* sorted, int32_t* inv, void* ws, hipStream_t st,
                bool* plan_ready = nullptr) {
    const bool small = (long long)s->T * s->k <= moe::kPermChunk;
    int32_t* plan = (plan_ready && small) ? at<int32_t>(ws, L.plan) : nullptr;
    int round_tiles = 1;
    if (plan)
        if (int rc = plan_round_tiles(s, &round_tiles)) return rc;
    HIP_TRY(moe::launch_permute(ids, s->T, s->k, s->E, at<int32_t>(ws, L.chunk), L.nchunks,
                                counts, offsets, sorted, inv, plan, L.light_max,
                                plan_force_tm(s), round_tiles, at<int32_t>(ws, L.sync), st),
            "permute");
    if (plan_ready) *plan_ready = plan != nullptr;
    return MOE_OK;
}

// distinct_ids: the rows come from the router (each token's k ids distinct,
// so no expert has more than T rows); otherwise (moe_grouped_ffn on any
// moe_permute output) the heavy grid covers every tile the plan can hold.
int run_ffn(const moe_shape* s, const Layout& L, const uint16_t* x, const int32_t* sorted,
            const int32_t* offsets, const uint16_t* wgu, const uint16_t* wdn,
            const void* packed, uint16_t* h, void* y, void* ws, hipStream_t st,
            bool plan_ready, bool distinct_ids) {
    int ncu = 0;
    if (int rc = device_cu_count(&ncu)) return rc;
    int32_t* plan = at<int32_t>(ws, L.plan);
    if (!plan_ready) {
        int round_tiles = 1;
        if (int rc = plan_round_tiles(s, &round_tiles)) return rc;
        HIP_TRY(moe::launch_ffn_plan(offsets, s->E, L.light_max, plan_force_tm(s), round_tiles,
                                     plan, at<int32_t>(ws, L.sync), st),
                "ffn plan");
    }
    moe::FfnArgs a{};
    a.x = x;
    a.sorted_ids = sorted;
    a.offsets = offsets;
    a.w_gu = wgu;
    a.w_dn = wdn;
    a.h = h ? h : at<uint16_t>(ws, L.h);
    a.y = y;
    a.plan = plan;
    a.sync = at<int32_t>(ws, L.sync);
    a.T = s->T;
    a.H = s->H;
    a.I = s->I;
    a.E = s->E;
    a.dense_rows = 0;
    a.dense_tm = 0;
    a.split_h = 0;
    a.max_tiles = distinct_ids ? L.max_tiles : L.plan_tiles;
    a.max_light = L.max_light;
    a.num_cu = ncu;
    a.y_fmt = y_format(s);
    a.w_mxfp8 = s->w_mxfp8;
    if (packed && s->w_mxfp8) {
        const uint8_t* p = static_cast<const uint8_t*>(packed);
        a.q_gu = p;
        a.q_dn = a.q_gu + moe::mx_codes_gu_bytes(s->E, s->H, s->I);
        a.qs_gu = a.q_dn + moe::mx_codes_dn_bytes(s->E, s->H, s->I);
        a.qs_dn = a.qs_gu + moe::mx_scales_gu_bytes(s->E, s->H, s->I);
        a.hq_gu = a.qs_dn + moe::mx_scales_dn_bytes(s->E, s->H, s->I);
        a.hq_dn = a.hq_gu + moe::mx_heavy_gu_bytes(s->E, s->H, s->I);
    } else if (packed) {
        const char* p = static_cast<const char*>(packed);
        a.hr_gu = reinterpret_cast<const uint16_t*>(p);
        a.hr_dn = reinterpret_cast<const uint16_t*>(p + moe::rec16_gu_bytes(s->E, s->H, s->I));
    }
    HIP_TRY(moe::launch_ffn_gateup(a, st), "ffn gate|up");
    HIP_TRY(moe::launch_ffn_down(a, st), "ffn down");
    return MOE_OK;
}

int run_shared(const moe_shape* s, const Layout& L, const uint16_t* x, const uint16_t* wgu,
               const uint16_t* wdn, float* out, void* ws, hipStream_t st) {
    int ncu = 0;
    if (int rc = device_cu_count(&ncu)) return rc;
    moe::FfnArgs a{};
    a.x = x;
    a.sorted_ids = nullptr;
    a.offsets = nullptr;
    a.w_gu = wgu;
    a.w_dn = wdn;
    a.h = at<uint16_t>(ws, L.hs);
    a.y = out;
    a.plan = nullptr;
    a.T = s->T;
    a.H = s->H;
    a.I = s->I_shared;
    a.E = 1;
    a.dense_rows = s->T;
    a.dense_tm = s->heavy_tile_rows ? s->heavy_tile_rows : moe::dense_tile_height(s->T);
    // The shared expert's output enters the sum with weight 1, so its h
    // carries a bf16 hi/lo pair: h = hi + lo to ~16 bits.
    a.split_h = 1;
    a.max_tiles = 0;
    a.max_light = 0;
    a.num_cu = ncu;
    a.y_fmt = 0;  // written straight into the fp32 output
    HIP_TRY(moe::launch_ffn_gateup(a, st), "shared gate|up");
    HIP_TRY(moe::launch_ffn_down(a, st), "shared down");
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_shape* shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return layout(shape).total;
}

size_t moe_packed_weight_bytes(const moe_shape* shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    const int E = shape->E, H = shape->H, I = shape->I;
    if (shape->w_mxfp8)
        return moe::mx_codes_gu_bytes(E, H, I) + moe::mx_codes_dn_bytes(E, H, I) +
               moe::mx_scales_gu_bytes(E, H, I) + moe::mx_scales_dn_bytes(E, H, I) +
               moe::mx_heavy_gu_bytes(E, H, I) + moe::mx_heavy_dn_bytes(E, H, I);
    return moe::rec16_gu_bytes(E, H, I) + moe::rec16_dn_bytes(E, H, I);
}

int moe_quantize_mxfp8(const uint16_t* w, int64_t rows, int32_t K, uint8_t* codes,
                       uint8_t* scales, void* stream) {
    g_last_error.clear();
    if (rows < 0 || K <= 0) return fail(MOE_ERR_SHAPE, "rows must be >= 0 and K > 0");
    if (K % 32) return fail(MOE_ERR_UNSUPPORTED, "K must be a multiple of 32");
    if (rows == 0) return MOE_OK;
    REQUIRE_PTR(w);
    REQUIRE_PTR(codes);
    if (!scales) return fail(MOE_ERR_NULL, "scales is NULL");
    HIP_TRY(moe::launch_mxfp8_quantize(w, rows, K, codes, scales, (hipStream_t)stream),
            "quantize mxfp8");
    return MOE_OK;
}

int moe_pack_weights_mxfp8(const moe_shape* shape, const uint8_t* codes_gate_up,
                           const uint8_t* scales_gate_up, const uint8_t* codes_down,
                           const uint8_t* scales_down, void* packed, void* stream) {
    g_last_error.clear();
    if (int rc = check_shape(shape)) return rc;
    if (!shape->w_mxfp8) return fail(MOE_ERR_SHAPE, "moe_pack_weights_mxfp8 needs w_mxfp8 = 1");
    REQUIRE_PTR(codes_gate_up);
    REQUIRE_PTR(codes_down);
    if (!scales_gate_up || !scales_down) return fail(MOE_ERR_NULL, "a scales array is NULL");
    if (!packed) return fail(MOE_ERR_NULL, "packed is NULL");
    if (!aligned(packed, kAlign)) return fail(MOE_ERR_ALIGN, "packed must be 256-byte aligned");
    HIP_TRY(moe::launch_pack_mxfp8(codes_gate_up, scales_gate_up, codes_down, scales_down,
                                   shape->E, shape->H, shape->I, static_cast<char*>(packed),
                                   (hipStream_t)stream),
            "pack mxfp8 weights");
    return MOE_OK;
}

int moe_pack_weights(const moe_shape* shape, const uint16_t* w_gate_up, const uint16_t* w_down,
                     void* packed, void* stream) {
    g_last_error.clear();
    if (int rc = check_shape(shape)) return rc;
    REQUIRE_PTR(w_gate_up);
    REQUIRE_PTR(w_down);
    if (!packed) return fail(MOE_ERR_NULL, "packed is NULL");
    if (!aligned(packed, kAlign)) return fail(MOE_ERR_ALIGN, "packed must be 256-byte aligned");
    HIP_TRY(moe::launch_pack_weights(w_gate_up, w_down, shape->E, shape->H, shape->I,
                                     static_cast<char*>(packed), (hipStream_t)stream),
            "pack weights");
    return MOE_OK;
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "invalid shape";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape";
        case MOE_ERR_ALIGN: return "misaligned pointer";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_profile_kernel_launch(int kernel, int launch, void* start, void* stop) {
    g_last_error.clear();
    if (kernel == -1) {
        moe::g_profile = moe::ProfileHook{};
        return MOE_OK;
    }
    if (kernel < 0 || kernel >= MOE_K_COUNT) return fail(MOE_ERR_SHAPE, "unknown kernel id");
    if (launch < -1) return fail(MOE_ERR_SHAPE, "launch must be -1 or >= 0");
    if (!start || !stop) return fail(MOE_ERR_NULL, "profile events are NULL");
    moe::g_profile.kernel = kernel;
    moe::g_profile.which = launch;
    moe::g_profile.start = (hipEvent_t)start;
    moe::g_profile.stop = (hipEvent_t)stop;
    moe::g_profile.launches = 0;
    return MOE_OK;
}

int moe_profile_kernel(int kernel, void* start, void* stop) {
    return moe_profile_kernel_launch(kernel, -1, start, stop);
}

long long moe_profile_launches(void) { return moe::g_profile.launches; }

int moe_router(const moe_shape* shape, const uint16_t* x, const float* w_router,
               const float* bias, int32_t* topk_ids, float* topk_w, float* probs,
               void* workspace, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (int rc = check_shape(shape)) return rc;
    if (shape->T == 0) return MOE_OK;
    REQUIRE_PTR(x);
    REQUIRE_PTR(w_router);
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(topk_w);
    OPTIONAL_PTR(bias);
    OPTIONAL_PTR(probs);
    if (int rc = check_ws(shape, workspace, ws_bytes)) return rc;
    return run_router(shape, layout(shape), x, w_router, bias, topk_ids, topk_w, probs, workspace,
                      (hipStream_t)stream);
}

int moe_permute(const moe_shape* shape, const int32_t* topk_ids, int32_t* counts,
                int32_t* offsets, int32_t* sorted_token_ids, int32_t* inv_pos, void* workspace,
                size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (int rc = check_shape(shape)) return rc;
    REQUIRE_PTR(counts);
    REQUIRE_PTR(offsets);
    if (shape->T > 0) {
        REQUIRE_PTR(topk_ids);
        REQUIRE_PTR(sorted_token_ids);
        REQUIRE_PTR(inv_pos);
    }
    if (int rc = check_ws(shape, workspace, ws_bytes)) return rc;
    return run_permute(shape, layout(shape), topk_ids, counts, offsets, sorted_token_ids, inv_pos,
                       workspace, (hipStream_t)stream);
}

int moe_grouped_ffn(const moe_shape* shape, const uint16_t* x, const int32_t* sorted_token_ids,
                    const int32_t* offsets, const uint16_t* w_gate_up, const uint16_t* w_down,
                    const void* packed_weights, uint16_t* h, void* y, void* workspace,
                    size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (int rc = check_shape(shape)) return rc;
    if (shape->T == 0) return MOE_OK;
    REQUIRE_PTR(x);
    REQUIRE_PTR(sorted_token_ids);
    REQUIRE_PTR(offsets);
    if (shape->w_mxfp8 && !packed_weights)
        return fail(MOE_ERR_NULL, "w_mxfp8 = 1 needs packed_weights");
    if (!packed_weights) {
        REQUIRE_PTR(w_gate_up);
        REQUIRE_PTR(w_down);
    } else {
        OPTIONAL_PTR(w_gate_up);
        OPTIONAL_PTR(w_down);
    }
    REQUIRE_PTR(y);
    OPTIONAL_PTR(h);
    if (packed_weights && !aligned(packed_weights, kAlign))
        return fail(MOE_ERR_ALIGN, "packed_weights must be 256-byte aligned");
    if (int rc = check_ws(shape, workspace, ws_bytes)) return rc;
    return run_ffn(shape, layout(shape), x, sorted_token_ids, offsets, w_gate_up, w_down,
                   packed_weights, h, y, workspace, (hipStream_t)stream, false, false);
}

int moe_shared_ffn(const moe_shape* shape, const uint16_t* x, const uint16_t* ws_gate_up,
                   const uint16_t* ws_down, float* out, void* workspace, size_t ws_bytes,
                   void* stream) {
    g_last_error.clear();
    if (int rc = check_shape(shape)) return rc;
    if (shape->I_shared <= 0) return fail(MOE_ERR_SHAPE, "moe_shared_ffn needs I_shared > 0");
    if (shape->T == 0) return MOE_OK;
    REQUIRE_PTR(x);
    REQUIRE_PTR(ws_gate_up);
    REQUIRE_PTR(ws_down);
    REQUIRE_PTR(out);
    if (int rc = check_ws(shape, workspace, ws_bytes)) return rc;
    return run_shared(shape, layout(shape), x, ws_gate_up, ws_down, out, workspace,
                      (hipStream_t)stream);
}

int moe_combine(const moe_shape* shape, const void* y, const int32_t* inv_pos,
                const float* topk_w, int32_t accumulate, float* out, void* stream) {
    g_last_error.clear();
    if (int rc = check_shape(shape)) return rc;
    if (shape->T == 0) return MOE_OK;
    REQUIRE_PTR(y);
    REQUIRE_PTR(inv_pos);
    REQUIRE_PTR(topk_w);
    REQUIRE_PTR(out);
    HIP_TRY(moe::launch_combine(y, y_format(shape), inv_pos, topk_w, shape->T, shape->H, shape->k,
                                accumulate ? 1 : 0, out, (hipStream_t)stream),
            "combine");
    return MOE_OK;
}

}  // extern "C"

namespace moe {

// moe_forward; overlap_shared: the shared expert on the device's side stream
// (else on `stream` after the routed FFN).
int forward(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias,
            const uint16_t* w_gate_up, const uint16_t* w_down, const void* packed_weights,
            const uint16_t* ws_gate_up, const uint16_t* ws_down, float* out,
            int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, void* workspace,
            size_t ws_bytes, void* stream, bool overlap_shared) {
    g_last_error.clear();
    if (int rc = check_shape(shape)) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (shape->T == 0) {
        // Nothing routed: only the optional counts are written (all zero).
        OPTIONAL_PTR(counts_out);
        if (!counts_out) return MOE_OK;
        if (int rc = check_ws(shape, workspace, ws_bytes)) return rc;
        const Layout L0 = layout(shape);
        return run_permute(shape, L0, nullptr, counts_out, at<int32_t>(workspace, L0.offsets),
                           nullptr, nullptr, workspace, st);
    }
    REQUIRE_PTR(x);
    REQUIRE_PTR(w_router);
    if (shape->w_mxfp8 && !packed_weights)
        return fail(MOE_ERR_NULL, "w_mxfp8 = 1 needs packed_weights");
    if (!packed_weights) {
        REQUIRE_PTR(w_gate_up);
        REQUIRE_PTR(w_down);
    } else {
        OPTIONAL_PTR(w_gate_up);
        OPTIONAL_PTR(w_down);
    }
    REQUIRE_PTR(out);
    OPTIONAL_PTR(bias);
    OPTIONAL_PTR(topk_ids_out);
    OPTIONAL_PTR(topk_w_out);
    OPTIONAL_PTR(counts_out);
    if (shape->I_shared > 0) {
        REQUIRE_PTR(ws_gate_up);
        REQUIRE_PTR(ws_down);
    }
    if (packed_weights && !aligned(packed_weights, kAlign))
        return fail(MOE_ERR_ALIGN, "packed_weights must be 256-byte aligned");
    if (int rc = check_ws(shape, workspace, ws_bytes)) return rc;
    const Layout L = layout(shape);
    int32_t* counts = counts_out ? counts_out : at<int32_t>(workspace, L.counts);
    int32_t* offsets = at<int32_t>(workspace, L.offsets);
    int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(workspace, L.ids);
    float* w = topk_w_out ? topk_w_out : at<float>(workspace, L.w);
    int32_t* sorted = at<int32_t>(workspace, L.sorted);
    int32_t* inv = at<int32_t>(workspace, L.inv);
    void* y = at<char>(workspace, L.y);
    std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
    SideStream* side = nullptr;
    if (shape->I_shared > 0 && overlap_shared) {
        // fork point: the side stream starts from here once its work is
        // enqueued (after the routed launches, which keeps their order)
        side_lock.lock();
        if (int rc = side_stream(&side)) return rc;
        HIP_TRY(hipEventRecord(side->fork, st), "fork");
    }
    if (int rc = run_router(shape, L, x, w_router, bias, ids, w, nullptr, workspace, st)) return rc;
    bool plan_ready = false;
    if (int rc = run_permute(shape, L, ids, counts, offsets, sorted, inv, workspace, st, &plan_ready))
        return rc;
    if (int rc = run_ffn(shape, L, x, sorted, offsets, w_gate_up, w_down, packed_weights, nullptr,
                         y, workspace, st, plan_ready, true))
        return rc;
    if (side) {
        HIP_TRY(hipStreamWaitEvent(side->s, side->fork, 0), "fork wait");
        if (int rc = run_shared(shape, L, x, ws_gate_up, ws_down, out, workspace, side->s))
            return rc;
        HIP_TRY(hipEventRecord(side->join, side->s), "join");
        HIP_TRY(hipStreamWaitEvent(st, side->join, 0), "join wait");
        side_lock.unlock();
    } else if (shape->I_shared > 0) {
        if (int rc = run_shared(shape, L, x, ws_gate_up, ws_down, out, workspace, st)) return rc;
    }
    HIP_TRY(moe::launch_combine(y, y_format(shape), inv, w, shape->T, shape->H, shape->k,
                                shape->I_shared > 0 ? 1 : 0, out, st),
            "combine");
    return MOE_OK;
}

}  // namespace moe

extern "C" {

int moe_forward(const moe_shape* shape, const uint16_t* x, const float* w_router,
                const float* bias, const uint16_t* w_gate_up, const uint16_t* w_down,
                const void* packed_weights, const uint16_t* ws_gate_up, const uint16_t* ws_down,
                float* out,
                int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, void* workspace,
                size_t ws_bytes, void* stream) {
    return moe::forward(shape, x, w_router, bias, w_gate_up, w_down, packed_weights, ws_gate_up,
                        ws_down, out, topk_ids_out, topk_w_out, counts_out, workspace, ws_bytes,
                        stream, MOE_SHARED_OVERLAP != 0);
}

}  // extern "C"
