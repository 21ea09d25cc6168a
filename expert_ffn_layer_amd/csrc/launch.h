// Host-side launchers of the MoE kernels (internal to libmoe.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- measurement hook (moe_profile_kernel) --------------------------------
struct ProfileHook {
    int kernel = -1;
    int which = -1;  // bracket only this launch (counted from the hook's setting), -1 = each
    hipEvent_t start = nullptr, stop = nullptr;
    long long launches = 0;
};
extern ProfileHook g_profile;

inline void prof_begin(int kernel, hipStream_t st) {
    if (g_profile.kernel == kernel) {
        if (g_profile.which < 0 || g_profile.launches == g_profile.which)
            (void)hipEventRecord(g_profile.start, st);
        ++g_profile.launches;
    }
}
inline void prof_end(int kernel, hipStream_t st) {
    if (g_profile.kernel == kernel &&
        (g_profile.which < 0 || g_profile.launches - 1 == g_profile.which))
        (void)hipEventRecord(g_profile.stop, st);
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
                          int32_t* inv_pos, int32_t* plan, int light_max, int force_tm,
                          int round_tiles, int32_t* sync, hipStream_t st);

// ---- grouped FFN --------------------------------------------------------
constexpr int kLightRowsMax = 64;  // up to four 16-row MFMA sub-tiles
// light_max given to the plan kernels: >= 0 a fixed threshold (experts with
// 1..light_max rows take the light loop); kLightAdaptive decides per call on
// the device: when the routed rows average at most MOE_LIGHT_MEAN_ROWS per
// touched expert, experts with up to kLightRowsMax rows take the light loop,
// otherwise only experts with up to MOE_LIGHT_TAIL_ROWS rows do (the cold
// tail of a skewed routing) and the rest take the heavy tiles.  (Measured on
// MI355X: the heavy tiles stream a small expert's weights about as fast as
// the light loop, light experts of 17..64 rows cost up to 40% at 10..80 rows
// per expert, and the tail rule takes 2% off the hot-expert skew layer while
// leaving uniform routings at 512..8192 tokens within 0.5%.)
constexpr int kLightAdaptive = -1;
#ifndef MOE_LIGHT_MEAN_ROWS
#define MOE_LIGHT_MEAN_ROWS 8
#endif
#ifndef MOE_LIGHT_TAIL_ROWS
#define MOE_LIGHT_TAIL_ROWS 8
#endif
inline __host__ __device__ int adaptive_light_max(long long rows, long long touched) {
    return rows <= (long long)MOE_LIGHT_MEAN_ROWS * touched ? kLightRowsMax : MOE_LIGHT_TAIL_ROWS;
}
// Heavy tiles are 256 columns wide and 128..256 rows high in steps of 32.
// An expert's rows are cut into equal tiles of the height with the least
// estimated time, ntiles * tm * cost(tm), cost = relative time per tile row
// (x1000; smaller tiles re-read more weights per row).  Equal heights keep
// the row tiles that share an expert's weights in step, so the weights are
// fetched once (a short last tile would run ahead of the others and drift
// out of the L2 window).
#ifndef MOE_TILE_COST_224
#define MOE_TILE_COST_224 1020
#endif
#ifndef MOE_TILE_COST_192
#define MOE_TILE_COST_192 1060
#endif
#ifndef MOE_TILE_COST_160
#define MOE_TILE_COST_160 1130
#endif
#ifndef MOE_TILE_COST_128
#define MOE_TILE_COST_128 1250
#endif
constexpr int kTileTMMax = 256, kTileTMStep = 32, kTileTMMin = 128;
constexpr int kTileN = 256;  // heavy tile width (output columns; gate|up: 128 gate + 128 up rows)
constexpr int kNumTileHeights = (kTileTMMax - kTileTMMin) / kTileTMStep + 1;  // 5
constexpr int kHeavyBMMin = kTileTMMin;  // sizes the plan's tile list
// Height index i: height 256 - 32 i.
inline __host__ __device__ int tile_height(int idx) { return kTileTMMax - kTileTMStep * idx; }
inline __host__ __device__ int tile_tm_index(int tm) { return (kTileTMMax - tm) / kTileTMStep; }
inline __host__ __device__ bool valid_tile_height(int tm) {
    return tm >= kTileTMMin && tm <= kTileTMMax && tm % kTileTMStep == 0;
}
inline __host__ __device__ int tile_cost(int idx) {
    return idx == 0 ? 1000
                    : (idx == 1 ? MOE_TILE_COST_224
                                : (idx == 2 ? MOE_TILE_COST_192
                                            : (idx == 3 ? MOE_TILE_COST_160 : MOE_TILE_COST_128)));
}
// Plan layout (int32): [0] n_light, [1] n_tiles, [2] forced tile height or 0,
// [16 ..16+E) light expert ids, [16+E ..) heavy tiles as (expert, first row
// | height index << kTileTmShift) pairs (height 256 - 32 * index).
constexpr int kPlanHeader = 16;
// MI355X: 8 XCDs, workgroups dispatched round-robin.  The heavy work list is
// cut into kXcds contiguous slices of about equal cost; plan[kPlanXcdBounds
// + x] is the first tile of slice x (x = 0..kXcds, the last = n_tiles).
#ifndef MOE_HEAVY_XCD_SLICES
#define MOE_HEAVY_XCD_SLICES 8
#endif
constexpr int kXcds = MOE_HEAVY_XCD_SLICES;
constexpr int kPlanXcdBounds = 3;
static_assert(kPlanXcdBounds + kXcds + 1 <= kPlanHeader, "plan header");
constexpr int kTileTmShift = 29;
constexpr int kTileRowMask = (1 << kTileTmShift) - 1;
// Relative time of one tile of height index tmi (about tm * cost(tm) / 16000).
inline __host__ __device__ int tile_cost_units(int tmi) {
    return (tile_height(tmi) * tile_cost(tmi) + 8000) / 16000;
}
inline __host__ __device__ int tiles_cost_units(int nt, int main_tmi, int last_tmi) {
    return nt > 0 ? (nt - 1) * tile_cost_units(main_tmi) + tile_cost_units(last_tmi) : 0;
}
// The XCD slice bounds that fall in one expert's tiles [t0, t0 + nt), whose
// cost before them is cb out of a total C: slice x - 1 ends after the first
// tile at which the cumulative cost reaches ceil(x C / kXcds), rounded to the
// nearest multiple of round_tiles (and at most the tile count ttot).  The
// blocks of a slice take its work items round-robin, so a slice whose items
// are a whole number of rounds of its blocks leaves none of them a short
// extra round: round_tiles is the tiles per round of the GEMM with the fewest
// N blocks (measured on the prefill layer: slices of 504..520 items gave
// some blocks 17 rounds of 16; rounded, every block runs 16).
inline __host__ __device__ void xcd_bounds(int32_t* plan, int t0, int nt, int main_tmi,
                                           int last_tmi, long long cb, long long C,
                                           int round_tiles, int ttot) {
    const long long ce = cb + tiles_cost_units(nt, main_tmi, last_tmi);
    for (int x = 1; x < kXcds; ++x) {
        const long long target = (C * x + kXcds - 1) / kXcds;
        if (target <= cb || target > ce) continue;
        long long cum = cb;
        int i = 0;
        for (; i < nt; ++i) {
            cum += tile_cost_units(i + 1 < nt ? main_tmi : last_tmi);
            if (cum >= target) break;
        }
        int b = t0 + i + 1;
        if (round_tiles > 1) b = (b + round_tiles / 2) / round_tiles * round_tiles;
        plan[kPlanXcdBounds + x] = b < ttot ? b : ttot;
    }
}
// Tiles of an expert with n heavy rows: ntiles tiles of one height (index
// main_tmi; last_tmi, the last tile's, is the same), first rows 0, tm, 2 tm,
// ...; the height with the least ntiles * tm * cost(tm).  force_tm (128 ..
// 256) puts every tile at that height; a negative force_tm = -m chooses as
// with 0 among the heights up to m (kTileMaxMx for MXFP8 weights, whose
// larger tile bodies do not fit the register file).
constexpr int kTileMaxMx = -192;
inline __host__ __device__ void tile_split(int n, int force_tm, int& ntiles, int& main_tmi,
                                           int& last_tmi) {
    if (force_tm > 0) {
        main_tmi = last_tmi = tile_tm_index(force_tm);
        ntiles = (n + force_tm - 1) / force_tm;
        return;
    }
    const int i0 = force_tm < 0 ? tile_tm_index(-force_tm) : 0;
    long long best = -1;
    ntiles = 0;
    main_tmi = last_tmi = i0;
    for (int i = i0; i < kNumTileHeights; ++i) {
        const int tm = tile_height(i);
        const int k = (n + tm - 1) / tm;
        const long long c = (long long)k * tm * tile_cost(i);
        if (best < 0 || c < best) {
            best = c;
            ntiles = k;
            main_tmi = last_tmi = i;
        }
    }
}

int max_heavy_tiles(long long A, int E, int light_max);
int dense_tile_height(int rows);  // tile height for a dense group of `rows` rows

// force_tm: 0 = pick the heavy tile height from the counts, else that height.
// round_tiles: multiple of tiles the XCD slice bounds are rounded to (xcd_bounds).
hipError_t launch_ffn_plan(const int32_t* offsets, int E, int light_max, int force_tm,
                           int round_tiles, int32_t* plan, int32_t* sync, hipStream_t st);
// Counters of the fused light loop (FfnArgs::sync), zeroed by whichever
// kernel writes the plan (when given): [kSyncTicket] the next work item,
// [kSyncTimeouts] readiness waits that gave up (0 unless something is
// broken), [kSyncReady + slot] gate|up items finished for light slot `slot`.
constexpr int kSyncTicket = 0, kSyncTimeouts = 1, kSyncReady = 2;
inline __host__ __device__ int sync_ints(int E) { return kSyncReady + E; }
// Tiles per round of a heavy GEMM's XCD slice for `num_cu` CUs (one block per
// CU, kXcds slices) with N blocks of nblk_gu (gate|up) and nblk_dn (down): the
// rounding of the slice bounds; 1 when it does not divide evenly.
inline int slice_round_tiles(int num_cu, int nblk_gu, int nblk_dn) {
    const int per_slice = num_cu / kXcds;
    const int nb = nblk_gu < nblk_dn ? nblk_gu : nblk_dn;
    if (nb <= 0 || per_slice <= 0 || per_slice % nb) return 1;
    return per_slice / nb;
}

struct FfnArgs {
    const uint16_t* x;           // [T,H]
    const int32_t* sorted_ids;   // [A] or nullptr = identity rows (dense group)
    const int32_t* offsets;      // [E+1] or nullptr for a dense group
    const uint16_t* w_gu;        // [E,2I,H]
    const uint16_t* w_dn;        // [E,H,I]
    uint16_t* h;                 // [rows,I] bf16 ([rows,2I] when split_h)
    void* y;                     // [rows,H]: fp32, bf16 or fp16 (y_fmt)
    const int32_t* plan;         // device plan, or nullptr for a dense group
    int T, H, I, E;
    int dense_rows;              // rows of a dense group (plan == nullptr)
    int dense_tm;                // tile height of a dense group (plan == nullptr)
    int split_h;                 // 1: h rows hold [hi | lo] bf16 halves (2I wide) and the
                                 //    down GEMM runs over both against the same weights
    int max_tiles;               // grid bound for heavy tiles
    int max_light;               // grid bound for light experts
    int num_cu;
    int y_fmt;                   // y storage: 0 fp32, 1 bf16, 2 fp16 (round to nearest even)
    // MXFP8 routed weights (w_mxfp8 = 1): the light loop and the heavy tiles
    // read these instead of hr_gu / hr_dn and w_gu / w_dn.
    int w_mxfp8;
    const uint8_t* q_gu;         // packed E4M3 codes of W_gate|up
    const uint8_t* q_dn;         // packed E4M3 codes of W_down
    const uint8_t* qs_gu;        // per-chunk E8M0 scales of W_gate|up
    const uint8_t* qs_dn;        // per-chunk E8M0 scales of W_down
    const uint8_t* hq_gu;        // heavy-tile records of W_gate|up (codes + scales)
    const uint8_t* hq_dn;        // heavy-tile records of W_down
    const uint16_t* hr_gu;       // packed bf16 records of W_gate|up (both loops), or nullptr
    const uint16_t* hr_dn;       // packed bf16 records of W_down
    int32_t* sync;               // fused light loop's counters (zeroed with the plan), or
                                 // nullptr: the light loop runs as two launches
};

// Row groups of the MXFP8 light loop's packed chunks (mxfp8.hip): 8 h
// columns (8 gate + the 8 matching up rows) or 16 W_down rows per group.
inline __host__ __device__ int packed_gu_groups(int I) { return I / 8; }
inline __host__ __device__ int packed_dn_groups(int H) { return H / 16; }
// Packed bf16 expert weights: one kRec16Bytes record per (expert, 256-row
// weight tile, 64-wide K stage), ordered (expert, tile, stage); W_gate|up's
// records first, then W_down's.  The tile's rows (gate|up: 16-row blocks
// alternate between the gate rows and the up rows of 16 h columns, block 2p
// gate and 2p+1 up of columns tile*128 + 16p..; down: W_down rows in order)
// are 16 blocks of 16 rows; block j holds two 1 KB chunks, K values 0..31
// and 32..63 of the stage, each one bf16 MFMA B operand in lane order (lane
// l: row 16j + l % 16, K values 8(l / 16)..+7 of the chunk).  Zero past the
// weights (rows to a multiple of 256, K to 64).  A light wave's operand for
// one K step is one chunk; a heavy tile's stage is the whole record, each
// DMA load of 8 rows reading 8 whole 128-byte lines.
constexpr int kRec16Bytes = 256 * 64 * 2;
constexpr int kRecElems = kRec16Bytes / 2;  // bf16 values of a record
constexpr int kRecChunkElems = 16 * 32;     // one chunk: 16 rows x 32 K
constexpr int kRecBlockElems = 16 * 64;     // one 16-row block: two chunks
// 256-row weight tiles of `rows` rows (the last one padded with zero rows).
inline __host__ __device__ int rec_tiles(int rows) { return (rows + 255) / 256; }
size_t rec16_gu_bytes(int E, int H, int I);
size_t rec16_dn_bytes(int E, int H, int I);
// Where the heavy tiles read B from.
constexpr int kBRowMajor = 0;  // w_gu / w_dn
constexpr int kBRec16 = 1;     // bf16 records of the packed copy
constexpr int kBRecMx = 2;     // MXFP8 records
hipError_t launch_pack_weights(const uint16_t* w_gu, const uint16_t* w_dn, int E, int H, int I,
                               char* packed, hipStream_t st);

// Packed MXFP8 expert weights (OCP MX: E4M3 codes, one E8M0 scale per 32
// values along K).  Codes: 1 KB chunks of 16 weight rows x 64 K in lane order
// -- lane l holds row l % 16, its 16 bytes the codes of K 8(l/16)..+7 of the
// chunk's first 32-wide K step, then those of its second; rows grouped as in
// the bf16 packing (gate|up: gate rows 8g..8g+7 then up rows I+8g..; down:
// W_down rows 16g..16g+15); chunks ordered (e, g, c) with c over ceil(K/64)
// (down pads K past I with code 0).  Scales: 32 bytes per chunk, byte
// 2*row + s the scale of the chunk's K step s for that row (127 = 2^0 for
// padded steps), in the same (e, g, c) order.  Sections: gate|up codes, down
// codes, gate|up scales, down scales, then the heavy tiles' copies of gate|up
// and down.
inline __host__ __device__ int mx_chunks(int K) { return (K + 63) / 64; }
// Heavy tiles read a second copy (sections 5 and 6 of the packed buffer): one
// record per (expert, 256-row B tile, 64-wide K chunk) = the 256 rows' codes
// (64 bytes each) then their 512 scale bytes; see pack_mxfp8_heavy_kernel.
constexpr int kMxCodeBytes = 256 * 64;
constexpr int kMxStageBytes = kMxCodeBytes + 512;
size_t mx_heavy_gu_bytes(int E, int H, int I);
size_t mx_heavy_dn_bytes(int E, int H, int I);
size_t mx_codes_gu_bytes(int E, int H, int I);
size_t mx_codes_dn_bytes(int E, int H, int I);
size_t mx_scales_gu_bytes(int E, int H, int I);
size_t mx_scales_dn_bytes(int E, int H, int I);
// Row-major MXFP8 of bf16 rows: codes [rows,K], scales [rows,K/32].
hipError_t launch_mxfp8_quantize(const uint16_t* w, long long rows, int K, uint8_t* codes,
                                 uint8_t* scales, hipStream_t st);
// Row-major codes/scales of both expert weights -> the packed layout above.
hipError_t launch_pack_mxfp8(const uint8_t* c_gu, const uint8_t* s_gu, const uint8_t* c_dn,
                             const uint8_t* s_dn, int E, int H, int I, char* packed,
                             hipStream_t st);

hipError_t launch_ffn_gateup(const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t st);

// ---- combine ------------------------------------------------------------
// y: [A,H] fp32 (y_fmt 0), bf16 (1) or fp16 (2).
hipError_t launch_combine(const void* y, int y_fmt, const int32_t* inv_pos, const float* w,
                          int T, int H, int k, int accumulate, float* out, hipStream_t st);

}  // namespace moe
