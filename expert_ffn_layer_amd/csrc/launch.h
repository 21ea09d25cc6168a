// Host-side launchers of the MoE kernels (internal to libmoe.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- measurement hook (moe_profile_kernel) --------------------------------
struct ProfileHook {
    int kernel = -1;
    hipEvent_t start = nullptr, stop = nullptr;
    long long launches = 0;
};
extern ProfileHook g_profile;

inline void prof_begin(int kernel, hipStream_t st) {
    if (g_profile.kernel == kernel) {
        (void)hipEventRecord(g_profile.start, st);
        ++g_profile.launches;
    }
}
inline void prof_end(int kernel, hipStream_t st) {
    if (g_profile.kernel == kernel) (void)hipEventRecord(g_profile.stop, st);
}

// Kernel ids (same values as enum moe_kernel in moe.h).
enum KernelId {
    K_ROUTER_GEMM = 0, K_ROUTER_SELECT, K_PERM_COUNT, K_PERM_SCAN, K_PERM_SCATTER, K_FFN_PLAN,
    K_GATEUP_LIGHT, K_GATEUP_HEAVY, K_DOWN_LIGHT, K_DOWN_HEAVY, K_COMBINE, K_PERM_SMALL, K_COUNT
};

// ---- router -------------------------------------------------------------
constexpr int kRouterBT = 128;  // tokens per router GEMM tile
constexpr int kRouterBE = 128;  // experts per router GEMM tile
constexpr int kRouterBK = 32;   // K (hidden) per LDS stage

// part[s][t][e] = sum over split s's hidden slice of x[t,h] * wg[h,e]
hipError_t launch_router_gemm(const uint16_t* x, const float* wg, float* part, int T, int H,
                              int E, int splits, hipStream_t st);
// logits = sum_s part[s] (+ bias); softmax; top-k; weights.
hipError_t launch_router_select(const float* part, int splits, const float* bias, int T, int E,
                                int k, int renorm, int32_t* ids, float* w, float* probs,
                                hipStream_t st);

// ---- permute ------------------------------------------------------------
constexpr int kPermChunk = 4096;  // assignments per permute block

// A <= kPermChunk runs as one fused block; then `plan` (may be nullptr)
// also receives the grouped-FFN plan for `light_max`.
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* chunk_counts,
                          int nchunks, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                          int32_t* inv_pos, int32_t* plan, int light_max, hipStream_t st);

// ---- grouped FFN --------------------------------------------------------
constexpr int kLightRowsMax = 64;  // up to four 16-row MFMA sub-tiles
constexpr int kHeavyBM = 256;      // rows per heavy tile
// Plan layout (int32): [0] n_light, [1] n_tiles, [16 ..16+E) light expert
// ids, [16+E ..) heavy tiles as (expert, first row) pairs.
constexpr int kPlanHeader = 16;

int max_heavy_tiles(long long A, int E, int light_max);

hipError_t launch_ffn_plan(const int32_t* offsets, int E, int light_max, int32_t* plan,
                           hipStream_t st);

struct FfnArgs {
    const uint16_t* x;           // [T,H]
    const int32_t* sorted_ids;   // [A] or nullptr = identity rows (dense group)
    const int32_t* offsets;      // [E+1] or nullptr for a dense group
    const uint16_t* w_gu;        // [E,2I,H]
    const uint16_t* w_dn;        // [E,H,I]
    uint16_t* h;                 // [rows,I] bf16 ([rows,2I] when split_h)
    float* y;                    // [rows,H] fp32
    const int32_t* plan;         // device plan, or nullptr for a dense group
    int T, H, I, E;
    int dense_rows;              // rows of a dense group (plan == nullptr)
    int split_h;                 // 1: h rows hold [hi | lo] bf16 halves (2I wide) and the
                                 //    down GEMM runs over both against the same weights
    int max_tiles;               // grid bound for heavy tiles
    int max_light;               // grid bound for light experts
    int num_cu;
};

hipError_t launch_ffn_gateup(const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t st);

// ---- combine ------------------------------------------------------------
hipError_t launch_combine(const float* y, const int32_t* inv_pos, const float* w, int T,
                          int H, int k, int accumulate, float* out, hipStream_t st);

}  // namespace moe
