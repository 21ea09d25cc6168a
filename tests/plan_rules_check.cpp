// Host-only check of the plan rules in launch.h (tile split per expert,
// cost-balanced XCD slices, the default light rule).  Built and run by
// tests/test_plan_rules.py; prints one line per expert row count:
//   n ntiles main_tm last_tm cost
// and then "xcd" followed by the slice bounds of a synthetic expert list.
#include <cstdio>
#include <vector>

#include "launch.h"

int main() {
    for (int n = 1; n <= 3000; ++n) {
        int nt = 0, mt = 0, lt = 0;
        moe::tile_split(n, 0, nt, mt, lt);
        std::printf("%d %d %d %d %d\n", n, nt, moe::tile_height(mt), moe::tile_height(lt),
                    moe::tiles_cost_units(nt, mt, lt));
    }
    // XCD bounds over experts with row counts 1..700 step 7 (every one heavy)
    std::vector<int> counts;
    for (int n = 1; n <= 700; n += 7) counts.push_back(n);
    long long C = 0;
    int T = 0;
    for (int n : counts) {
        int nt, mt, lt;
        moe::tile_split(n, 0, nt, mt, lt);
        C += moe::tiles_cost_units(nt, mt, lt);
        T += nt;
    }
    std::vector<int> tile_cost;
    for (int n : counts) {
        int nt, mt, lt;
        moe::tile_split(n, 0, nt, mt, lt);
        for (int i = 0; i < nt; ++i) tile_cost.push_back(moe::tile_cost_units(i + 1 < nt ? mt : lt));
    }
    // slice bounds without rounding ("xcd"/"slices") and rounded to 4 tiles
    // ("xcdr"/"slicesr")
    for (int round_tiles : {1, 4}) {
        int32_t plan[moe::kPlanHeader] = {0};
        long long cb = 0;
        int t0 = 0;
        for (int n : counts) {
            int nt, mt, lt;
            moe::tile_split(n, 0, nt, mt, lt);
            moe::xcd_bounds(plan, t0, nt, mt, lt, cb, C, round_tiles, T);
            cb += moe::tiles_cost_units(nt, mt, lt);
            t0 += nt;
        }
        plan[moe::kPlanXcdBounds] = 0;
        plan[moe::kPlanXcdBounds + moe::kXcds] = T;
        const char* tag = round_tiles > 1 ? "r" : "";
        std::printf("xcd%s %lld %d", tag, C, T);
        for (int x = 0; x <= moe::kXcds; ++x) std::printf(" %d", plan[moe::kPlanXcdBounds + x]);
        std::printf("\nslices%s", tag);
        for (int x = 0; x < moe::kXcds; ++x) {
            long long c = 0;
            for (int t = plan[moe::kPlanXcdBounds + x]; t < plan[moe::kPlanXcdBounds + x + 1]; ++t)
                c += tile_cost[t];
            std::printf(" %lld", c);
        }
        std::printf("\n");
    }
    std::printf("round %d %d %d %d\n", moe::slice_round_tiles(256, 8, 16),
                moe::slice_round_tiles(256, 16, 32), moe::slice_round_tiles(256, 3, 16),
                moe::slice_round_tiles(304, 8, 16));
    // heights limited to 192 (MXFP8 weights): prefix "mx"
    for (int n = 1; n <= 1500; ++n) {
        int nt = 0, mt = 0, lt = 0;
        moe::tile_split(n, moe::kTileMaxMx, nt, mt, lt);
        std::printf("mx %d %d %d %d\n", n, nt, moe::tile_height(mt), moe::tile_height(lt));
    }
    std::printf("light %d %d %d %d\n", moe::adaptive_light_max(4000, 500),
                moe::adaptive_light_max(4001, 500), moe::kLightRowsMax, MOE_LIGHT_TAIL_ROWS);
    return 0;
}
