// Grouped expert FFN on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
//   gate|up:  h[r, i] = bf16( silu(x[tok_r] . Wg[e,i]) * (x[tok_r] . Wu[e,i]) )
//   down:     y[r, c] = h[r] . Wd[e,c]            (fp32 sum; stored fp32 or bf16)
//
// for the expert-major rows r of expert e (pwwt.cn article on Qwen 3.5-397B
// MoE on Ironwood, section 4.2: grouped GEMM with SwiGLU fused into the
// matmul, each expert's slice bounded by its own token count).  Token rows
// are gathered by index inside the A-operand load; no permuted copy of x is
// built.
//
// Two loops, after the yuxiaoba.github.io summary of "Optimizing Muse Spark
// Open on TPU v7 with SGLang-TorchTPU" (section on changing dependencies):
// experts with few rows do not share a loop body with heavy experts, so the
// light loop carries no heavy accumulators.
//  * light: an expert with 1..64 rows; each wave streams 16 weight rows
//    straight from HBM into registers (from the packed lane-order chunks when
//    given, one contiguous run per wave) and keeps one accumulator per
//    16-row sub-tile.  This is the decode path: it is bound by weight bytes.
//    Which experts take it is the plan's choice (light_max; by default a
//    per-call rule that sends every expert one way, see launch.h).
//    Its gate|up tiles hold 8 gate rows and the 8 matching up rows, so lanes
//    n and n+8 carry g and u of one h column (one lane shuffle).
//  * heavy: TM x 256 output tiles (TM = 256, 192 or 128, chosen from the row
//    counts), A and B staged through LDS rings by direct-to-LDS loads, tiles
//    of one expert scheduled together on one XCD.  Gate and up rows alternate
//    by 16-row blocks, so g and u of an h column meet in one lane.  B comes
//    from the row-major weights, or from the packed copy's per-stage records.
// Both paths give every output element the same chain of MFMAs over K in
// ascending 32-wide steps with the same K-slot assignment, and the same
// epilogue, so a row's h and y are bitwise identical whichever loop ran it.
// MXFP8 weights (OCP MX: E4M3 codes, an E8M0 scale per 32 values) run the
// same loops: each 8 codes become the bf16 operand times the block scale by
// the hardware's scaled conversion (exact), so the results are those of the
// bf16 loops on the dequantised weights, bit for bit.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {

int max_heavy_tiles(long long A, int E, int light_max) {
    // sum over heavy experts of ceil(n_e / BM) <= A / BM + (#heavy experts),
    // at the smallest tile height
    const long long heavy = std::min<long long>(E, A / (light_max + 1));
    return (int)std::min<long long>(A / kHeavyBMMin + heavy + 1, A + 1);
}

int dense_tile_height(int rows) {
    int nt, main_tmi, last_tmi;
    tile_split(rows, 0, nt, main_tmi, last_tmi);
    return tile_height(main_tmi);
}

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- plan
// One block, one thread per expert: pick the heavy tile height from the
// experts' row counts, then compact the light experts (ascending id) and the
// heavy experts' row tiles (ascending id, then first row).
__global__ __launch_bounds__(1024) void ffn_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int E, int light_max, int force_tm,
                                                        int round_tiles,
                                                        int32_t* __restrict__ plan,
                                                        int32_t* __restrict__ sync) {
    __shared__ int wl[16], wt[16], wcs[16], wtouch[16];
    const int e = threadIdx.x;
    if (sync)  // the fused light loop's counters start at zero
        for (int i = threadIdx.x; i < sync_ints(E); i += blockDim.x) sync[i] = 0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
    const int n = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    int lm = light_max;
    if (lm == kLightAdaptive) {  // uniform: every thread takes this branch or none
        int tch = n > 0 ? 1 : 0;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) tch += __shfl_xor(tch, o, 64);
        if (lane == 0) wtouch[wave] = tch;
        __syncthreads();
        int touched = 0;
        for (int w = 0; w < nwave; ++w) touched += wtouch[w];
        lm = adaptive_light_max(offsets[E] - offsets[0], touched);
    }
    const bool heavy = n > lm;
    int nt = 0, main_tmi = 0, last_tmi = 0;
    if (heavy) tile_split(n, force_tm, nt, main_tmi, last_tmi);
    const int is_light = (n >= 1 && n <= lm) ? 1 : 0;
    const int cost = tiles_cost_units(nt, main_tmi, last_tmi);
    int il = is_light, it = nt, ic = cost;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int vl = __shfl_up(il, o, 64);
        const int vt = __shfl_up(it, o, 64);
        const int vc = __shfl_up(ic, o, 64);
        if (lane >= o) {
            il += vl;
            it += vt;
            ic += vc;
        }
    }
    if (lane == 63) {
        wl[wave] = il;
        wt[wave] = it;
        wcs[wave] = ic;
    }
    __syncthreads();
    int bl = 0, bt = 0, bc = 0, ctot = 0, ttot = 0;
    for (int w = 0; w < nwave; ++w) {
        if (w < wave) {
            bl += wl[w];
            bt += wt[w];
            bc += wcs[w];
        }
        ctot += wcs[w];
        ttot += wt[w];
    }
    const int el = bl + il - is_light, et = bt + it - nt;
    xcd_bounds(plan, et, nt, main_tmi, last_tmi, bc + ic - cost, ctot, round_tiles, ttot);
    if (is_light) plan[kPlanHeader + el] = e;
    int32_t* tiles = plan + kPlanHeader + E;
    const int tm = tile_height(main_tmi);
    for (int i = 0; i < nt; ++i) {
        tiles[2 * (et + i)] = e;
        tiles[2 * (et + i) + 1] = (i * tm) | ((i + 1 < nt ? main_tmi : last_tmi) << kTileTmShift);
    }
    if (threadIdx.x == blockDim.x - 1) {
        plan[0] = el + is_light;
        plan[1] = et + nt;
        plan[2] = force_tm;
        plan[kPlanXcdBounds] = 0;
        plan[kPlanXcdBounds + kXcds] = et + nt;
        if (ctot == 0)
            for (int x = 1; x < kXcds; ++x) plan[kPlanXcdBounds + x] = 0;
    }
}

// Tunables of the light loops (compile-time; the defaults are the measured best).
#ifndef MOE_LIGHT_GU_U
#define MOE_LIGHT_GU_U 4        // K steps of 32 in flight per wave (gate|up: 2 loads each)
#endif
// Blocks per CU in the light grids.  bf16: 32, so that up to 8192 items a
// block takes one item and the dispatcher hands the items out as blocks
// finish; MXFP8: 2 (gate|up) and 4 (down), about the resident blocks, each
// taking a fixed share (its items stream half the bytes, and block turnover
// costs more than the uneven finish).  Measured on MI355X at decode T=64:
// bf16 1.438 -> 1.427 ms against 8 per CU, MXFP8 0.832 -> 0.812 ms.
#ifndef MOE_LIGHT_GU_BPC
#define MOE_LIGHT_GU_BPC 32
#endif
#ifndef MOE_LIGHT_DN_U
#define MOE_LIGHT_DN_U 4
#endif
#ifndef MOE_LIGHT_DN_TILES
#define MOE_LIGHT_DN_TILES 2
#endif
#ifndef MOE_LIGHT_DN_BPC
#define MOE_LIGHT_DN_BPC 32
#endif
#ifndef MOE_LIGHT_NT_LOADS
#define MOE_LIGHT_NT_LOADS 1    // 0: weights read with the default cache policy
#endif

// Expert weights are read once per step: with the non-temporal hint they are
// not retained in the caches (measured on MI355X: a plain stream of 16-byte
// loads over 4 GiB reads at 6.2 TB/s with the default policy and 7.0 TB/s
// with the hint; decode step -8%, gate|up light loop at 6.8 TB/s).
template <bool kNonTemporal>
__device__ __forceinline__ bf16x8_t load_weights(const uint16_t* p) {
    if constexpr (kNonTemporal)
        return __builtin_bit_cast(bf16x8_t,
                                  __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
    else
        return load_bf16x8(p);
}

// Offset of 32-wide K step kb from a light lane's first weight: along the
// weight row, or, in the packed records, chunk kb % 2 of the operand's
// 16-row block in record kb / 2.
template <bool kRecords>
__device__ __forceinline__ size_t light_koff(int kb) {
    if constexpr (kRecords)
        return (size_t)(kb >> 1) * kRecElems + (size_t)(kb & 1) * kRecChunkElems;
    else
        return (size_t)kb * 32;
}

// Row sub-tiles of the light loop: experts with up to 16 rows run one 16-row
// MFMA tile with deep weight prefetch; experts with 17..64 rows run four
// sub-tiles (those past the row count skipped) with shallower prefetch, so
// both branches fit the same register budget.
constexpr int kLightSubTiles = kLightRowsMax / 16;  // 4
constexpr int kLightWideU = 2;                      // K steps in flight, wide branch

// ------------------------------------------------------- y in 16 bits
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Storage of y (FfnArgs::y_fmt): fp32, bf16 or fp16.
constexpr int kYF32 = 0, kYBF16 = 1, kYF16 = 2;

// Two fp32 values as one word of two bf16 (round to nearest even), a in the
// low half.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2_t{a, b}, bf16x2_t));
}
// The same as two fp16 (round to nearest even; past 65504 rounds to inf).
__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2_t{a, b}, f16x2_t));
}
template <int YF>
__device__ __forceinline__ uint32_t pack_y16(float a, float b) {
    static_assert(YF == kYBF16 || YF == kYF16, "16-bit y");
    return YF == kYBF16 ? pack_bf16_rne(a, b) : pack_f16_rne(a, b);
}

// A lane of a 16x16 MFMA result holds rows 4g..4g+3 of column c = l16.  For
// 32-bit stores of 16-bit y the lanes of columns c and c^1 swap halves: the
// even column's lane then holds rows 4g, 4g+1 and the odd column's lane rows
// 4g+2, 4g+3, each as the word (column c & ~1, column c | 1).  Every lane of
// the wave must call this (a lane exchange).
template <int YF>
__device__ __forceinline__ void y16_pairs(const floatx4_t v, int l16, uint32_t& w0, uint32_t& w1) {
    const bool odd = l16 & 1;
    const float s0 = __shfl_xor(odd ? v[0] : v[2], 1, 64);
    const float s1 = __shfl_xor(odd ? v[1] : v[3], 1, 64);
    w0 = odd ? pack_y16<YF>(s0, v[2]) : pack_y16<YF>(v[0], s0);
    w1 = odd ? pack_y16<YF>(s1, v[3]) : pack_y16<YF>(v[1], s1);
}

// The light loops' 16-bit y epilogue: rows r0.. of the wave's MT x NT tiles
// at columns c0 + 16t ...
template <int YF, int MT, int NT>
__device__ __forceinline__ void light_store_y16(const FfnArgs& a, const floatx4_t (&acc)[MT][NT],
                                                int r0, int n, int c0, int l16, int g) {
    const int odd = l16 & 1;
    uint32_t* y = static_cast<uint32_t*>(a.y);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            uint32_t w[2];
            y16_pairs<YF>(acc[m][t], l16, w[0], w[1]);
            const int c = c0 + t * 16 + l16 - odd;  // even
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int row = m * 16 + 4 * g + 2 * odd + r;
                if (row < n) y[((size_t)(r0 + row) * a.H + c) / 2] = w[r];
            }
        }
    }
}

// ------------------------------------------------------- light: gate|up
// One wave: MT row sub-tiles x 16 h columns i0..i0+15 of one expert, K = H:
// one MFMA tile over the 16 gate rows and one over the matching 16 up rows,
// so a lane ends with g and u of the same h column.
template <int MT, int U, bool NTL, bool PK>
__device__ __forceinline__ void gateup_light_rows(const FfnArgs& a, int e, int r0, int n, int i0,
                                                  int l16, int g) {
    const int nk = a.H / 32;
    const uint16_t* Bg;  // gate operand; the up operand is `uoff` further
    size_t uoff;
    if constexpr (PK) {
        // record chunks: the gate rows of h columns i0.. are 16-row block
        // 2 (i0 % 128) / 16 of tile i0 / 128, their up rows the next block
        const int lane = g * 16 + l16;
        const size_t rec = ((size_t)e * rec_tiles(2 * a.I) + (i0 >> 7)) * mx_chunks(a.H);
        Bg = a.hr_gu + rec * kRecElems + (size_t)(((i0 & 127) >> 4) * 2) * kRecBlockElems + lane * 8;
        uoff = kRecBlockElems;
    } else {
        Bg = a.w_gu + ((size_t)e * 2 * a.I + i0 + l16) * a.H + 8 * g;
        uoff = (size_t)a.I * a.H;
    }
    const uint16_t* Ap[MT];
    bool has_a[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int row = m * 16 + l16;
        has_a[m] = row < n;
        const int tok = has_a[m] ? (a.sorted_ids ? a.sorted_ids[r0 + row] : r0 + row) : 0;
        Ap[m] = a.x + (size_t)tok * a.H + 8 * g;
    }
    const int mt_live = (n + 15) / 16;  // wave-uniform

    floatx4_t acc[MT][2];  // [m][0] gate, [m][1] up
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m][0] = acc[m][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t ca[U][MT], cb[U][2];
    auto load_step = [&](int kb, bf16x8_t (&aa)[MT], bf16x8_t (&bb)[2]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) aa[m] = zero_bf16x8();
        bb[0] = bb[1] = zero_bf16x8();
        if (kb < nk) {
            const size_t ko = light_koff<PK>(kb);
            bb[0] = load_weights<NTL>(Bg + ko);
            bb[1] = load_weights<NTL>(Bg + uoff + ko);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (has_a[m]) aa[m] = load_bf16x8(Ap[m] + kb * 32);
        }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) load_step(u, ca[u], cb[u]);
    for (int k0 = 0; k0 < nk; k0 += U) {
        bf16x8_t na[U][MT], nb_[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) load_step(k0 + U + u, na[u], nb_[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (k0 + u < nk) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < mt_live) {
                        acc[m][0] = mfma_16x16x32(ca[u][m], cb[u][0], acc[m][0]);
                        acc[m][1] = mfma_16x16x32(ca[u][m], cb[u][1], acc[m][1]);
                    }
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < MT; ++m) ca[u][m] = na[u][m];
            cb[u][0] = nb_[u][0];
            cb[u][1] = nb_[u][1];
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m * 16 + 4 * g + r;
            if (row < n)
                a.h[(size_t)(r0 + row) * a.I + i0 + l16] =
                    (uint16_t)f32_to_bf16_bits(swiglu(acc[m][0][r], acc[m][1][r]));
        }
    }
}

// Work item = (light expert, 4 waves x 16 h-columns).
template <int U, bool NTL, bool PK>
__global__ __launch_bounds__(kThreads) void gateup_light_kernel(FfnArgs a) {
    constexpr int kCols = 4 * 16;
    const int nlight = a.plan[0];
    const int nblk = (a.I + kCols - 1) / kCols;
    const long long nwork = (long long)nlight * nblk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    for (long long wi = blockIdx.x; wi < nwork; wi += gridDim.x) {
        const int slot = (int)(wi / nblk), nb = (int)(wi % nblk);
        const int i0 = nb * kCols + wave * 16;
        if (i0 >= a.I) continue;  // I % 32 == 0: a wave is all in or all out
        const int e = a.plan[kPlanHeader + slot];
        const int r0 = a.offsets[e];
        const int n = a.offsets[e + 1] - r0;
        if (n <= 16)
            gateup_light_rows<1, U, NTL, PK>(a, e, r0, n, i0, l16, g);
        else
            gateup_light_rows<kLightSubTiles, kLightWideU, NTL, PK>(a, e, r0, n, i0, l16, g);
    }
}

// --------------------------------------------------------- light: down
// One wave: MT row sub-tiles x NT column tiles (16 output columns each), K = I.
template <int MT, int U, int NT, bool NTL, bool PK>
__device__ __forceinline__ void down_light_rows(const FfnArgs& a, int e, int r0, int n, int c0,
                                                int l16, int g) {
    const int nk = a.I / 32;
    // Lane l16 holds W_down row c0 + 16t + l16, K values 8g.. of each step.
    const uint16_t* Bt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int c = c0 + 16 * t + l16;
        if constexpr (PK) {
            // record chunks: 16-row block (c % 256) / 16 of tile c / 256
            const int lane = g * 16 + l16;
            const size_t rec = ((size_t)e * rec_tiles(a.H) + (c >> 8)) * mx_chunks(a.I);
            Bt[t] = a.hr_dn + rec * kRecElems + (size_t)((c & 255) >> 4) * kRecBlockElems + lane * 8;
        } else {
            Bt[t] = a.w_dn + ((size_t)e * a.H + c) * a.I + 8 * g;
        }
    }
    const uint16_t* Ap[MT];
    bool has_a[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int row = m * 16 + l16;
        has_a[m] = row < n;
        Ap[m] = a.h + (size_t)(r0 + (has_a[m] ? row : 0)) * a.I + 8 * g;
    }
    const int mt_live = (n + 15) / 16;

    floatx4_t acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t ca[U][MT], cb[U][NT];
    auto load_step = [&](int kb, bf16x8_t (&aa)[MT], bf16x8_t (&bb)[NT]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) aa[m] = zero_bf16x8();
#pragma unroll
        for (int t = 0; t < NT; ++t) bb[t] = zero_bf16x8();
        if (kb < nk) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (has_a[m]) aa[m] = load_bf16x8(Ap[m] + kb * 32);
#pragma unroll
            for (int t = 0; t < NT; ++t) bb[t] = load_weights<NTL>(Bt[t] + light_koff<PK>(kb));
        }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) load_step(u, ca[u], cb[u]);
    for (int k0 = 0; k0 < nk; k0 += U) {
        bf16x8_t na[U][MT], nb_[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) load_step(k0 + U + u, na[u], nb_[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (k0 + u < nk) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < mt_live) {
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            acc[m][t] = mfma_16x16x32(ca[u][m], cb[u][t], acc[m][t]);
                    }
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < MT; ++m) ca[u][m] = na[u][m];
#pragma unroll
            for (int t = 0; t < NT; ++t) cb[u][t] = nb_[u][t];
        }
    }
    if (a.y_fmt == kYBF16) {
        light_store_y16<kYBF16>(a, acc, r0, n, c0, l16, g);
        return;
    }
    if (a.y_fmt == kYF16) {
        light_store_y16<kYF16>(a, acc, r0, n, c0, l16, g);
        return;
    }
    float* y = static_cast<float*>(a.y);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int c = c0 + t * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m * 16 + 4 * g + r;
                if (row < n) y[(size_t)(r0 + row) * a.H + c] = acc[m][t][r];
            }
        }
    }
}

// Work item = (light expert, 4 waves x NT x 16 output columns).
template <int NT, int U, bool NTL, bool PK>
__global__ __launch_bounds__(kThreads) void down_light_kernel(FfnArgs a) {
    static_assert(64 % (NT * 16) == 0, "a wave's columns must divide H's multiple of 64");
    constexpr int kCols = 4 * NT * 16;
    const int nlight = a.plan[0];
    const int nblk = (a.H + kCols - 1) / kCols;
    const long long nwork = (long long)nlight * nblk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    for (long long wi = blockIdx.x; wi < nwork; wi += gridDim.x) {
        const int slot = (int)(wi / nblk), nb = (int)(wi % nblk);
        const int c0 = nb * kCols + wave * NT * 16;
        if (c0 >= a.H) continue;  // H % 64 == 0 and NT*16 divides 64: all in or all out
        const int e = a.plan[kPlanHeader + slot];
        const int r0 = a.offsets[e];
        const int n = a.offsets[e + 1] - r0;
        if (n <= 16)
            down_light_rows<1, U, NT, NTL, PK>(a, e, r0, n, c0, l16, g);
        else
            down_light_rows<kLightSubTiles, kLightWideU, NT, NTL, PK>(a, e, r0, n, c0, l16, g);
    }
}

// ----------------------------------------------- light: fused gate|up -> down
// Both light GEMMs in one persistent launch (after the lumevalley.com
// article on serving Ling-2.6-1T, section on hiding data movement inside
// the compute: Fused MoE V2 runs scatter, FFN and gather as one kernel).
// Blocks take work items from a ticket counter: first every gate|up item
// (as gateup_light_kernel's), then every down item (as down_light_kernel's).
// A down item of light slot s needs all of h for s, so it waits until the
// slot's counter of finished gate|up items reaches their number; each
// gate|up item counts itself after its h stores are released at device
// scope.  Tickets are taken in order, so when a block holds a down ticket
// every gate|up ticket is held by a running block whose item waits for
// nothing: each wait ends.  (A wait is still bounded: past
// MOE_FUSED_SPIN_LIMIT polls it gives up, counts itself in
// sync[kSyncTimeouts] and writes NaN into its y rows instead of a result.)  The items run the separate kernels' code, so h
// and y are bitwise those of the two launches.
// Off by default (MOE_FUSED_LIGHT=1 builds it in): measured on MI355X at
// decode (T=64, H=4096, E=512, k=10, I=1024) it takes 2.67 ms against
// 0.92 + 0.46 ms for the two launches.  h crosses XCDs, each with its own
// L2, so every gate|up item writes back its XCD's L2 and every down item
// invalidates it; the weight stream around them pays for that.
#ifndef MOE_FUSED_LIGHT
#define MOE_FUSED_LIGHT 0
#endif
#ifndef MOE_FUSED_BPC
#define MOE_FUSED_BPC 8  // blocks per CU of the fused light launch
#endif
#ifndef MOE_FUSED_SPIN_LIMIT
#define MOE_FUSED_SPIN_LIMIT (1 << 18)
#endif
// NaN into y rows r0..r0+n-1, columns c0..c0+ncols-1 (all y formats: every
// bit set is a NaN in fp32, bf16 and fp16).
__device__ __forceinline__ void light_poison_y(const FfnArgs& a, int r0, int n, int c0, int ncols,
                                               int lane) {
    const int esz = a.y_fmt == kYF32 ? 4 : 2;
    char* y = static_cast<char*>(a.y);
    for (int i = lane; i < n * ncols; i += 64) {
        const size_t off = ((size_t)(r0 + i / ncols) * a.H + c0 + i % ncols) * esz;
        if (esz == 4)
            *reinterpret_cast<uint32_t*>(y + off) = 0xffffffffu;
        else
            *reinterpret_cast<uint16_t*>(y + off) = 0xffffu;
    }
}

template <int UGU, int NTDN, int UDN, bool NTL, bool PK>
__global__ __launch_bounds__(kThreads) void light_fused_kernel(FfnArgs a) {
    constexpr int kColsGu = 4 * 16, kColsDn = 4 * NTDN * 16;
    __shared__ int s_ticket, s_gave_up;  // s_gave_up is rewritten only after the next
                                         // item's ticket barriers
    const int nlight = a.plan[0];
    const int nbg = (a.I + kColsGu - 1) / kColsGu, nbd = (a.H + kColsDn - 1) / kColsDn;
    const int ngu = nlight * nbg, nwork = ngu + nlight * nbd;  // < 2^31 (host check)
    int32_t* ticket = a.sync + kSyncTicket;
    int32_t* ready = a.sync + kSyncReady;
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;
    // Every branch around the barriers below is wave-uniform (scalar): the
    // counters are updated by all 64 lanes of wave 0 adding 1 from lane 0
    // only, and shared values are read back with readfirstlane.  A branch
    // the compiler takes for per-lane (thread 0 alone, or a plain LDS read
    // deciding the loop's exit) is laid out with lane masks, and then the
    // other lanes of wave 0 can pass the barriers and re-read s_ticket while
    // thread 0, masked off, never takes the next ticket.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int one = lane == 0 ? 1 : 0;
    for (;;) {
        if (wave == 0) {
            const int t = __hip_atomic_fetch_add(ticket, one, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            s_ticket = __builtin_amdgcn_readfirstlane(t);  // lane 0's: the ticket taken
        }
        __syncthreads();
        const int wi = __builtin_amdgcn_readfirstlane(s_ticket);
        __syncthreads();  // every lane has read s_ticket before it is rewritten
        if (wi >= nwork) break;
        if (wi < ngu) {
            const int slot = wi / nbg, nb = wi % nbg;
            const int i0 = nb * kColsGu + wave * 16;
            if (i0 < a.I) {  // I % 32 == 0: a wave is all in or all out
                const int e = a.plan[kPlanHeader + slot];
                const int r0 = a.offsets[e];
                const int n = a.offsets[e + 1] - r0;
                if (n <= 16)
                    gateup_light_rows<1, UGU, NTL, PK>(a, e, r0, n, i0, l16, g);
                else
                    gateup_light_rows<kLightSubTiles, kLightWideU, NTL, PK>(a, e, r0, n, i0, l16, g);
            }
            // Each wave's h stores complete and released at device scope (the
            // barrier alone does not wait for other waves' stores), then counted.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (wave == 0)
                __hip_atomic_fetch_add(ready + slot, one, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const int slot = (wi - ngu) / nbd, nb = (wi - ngu) % nbd;
            if (wave == 0) {
                // relaxed polls (no cache invalidation each), one acquire after
                int spins = 0, gave_up = 0;
                while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                           ready + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < nbg) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++spins > MOE_FUSED_SPIN_LIMIT) {
                        __hip_atomic_fetch_add(a.sync + kSyncTimeouts, one, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        gave_up = 1;
                        break;
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                s_gave_up = gave_up;
            }
            // the other waves read h after wave 0's acquire (the CU's vector
            // cache and the L2 invalidated once for the item)
            __syncthreads();
            const bool gave_up = __builtin_amdgcn_readfirstlane(s_gave_up) != 0;
            const int c0 = nb * kColsDn + wave * NTDN * 16;
            if (c0 < a.H) {  // H % 64 == 0: all in or all out
                const int e = a.plan[kPlanHeader + slot];
                const int r0 = a.offsets[e];
                const int n = a.offsets[e + 1] - r0;
                if (gave_up)  // h may be incomplete: the item's y rows become NaN
                    light_poison_y(a, r0, n, c0, NTDN * 16, lane);
                else if (n <= 16)
                    down_light_rows<1, UDN, NTDN, NTL, PK>(a, e, r0, n, c0, l16, g);
                else
                    down_light_rows<kLightSubTiles, kLightWideU, NTDN, NTL, PK>(a, e, r0, n, c0, l16, g);
            }
        }
    }
}

// ------------------------------------------------ light: MXFP8 weights
// The same loops over packed MXFP8 weights: a lane's 16-byte load carries
// the codes of two 32-wide K steps (see the packed layout in launch.h) and
// each is turned into the bf16 operand of the bf16 loop by the hardware's
// scaled conversion, code * 2^(scale - 127): exact, since an E4M3 value has
// 4 significant bits.  Each accumulator then takes the same chain of MFMAs
// over the same operands as the bf16 loop given the dequantised weights, so
// the two give bitwise identical results.  (The plan gives the light loop at
// most 64 rows per expert; the kernels still step through larger counts in
// passes of 64 rows, so no count can leave rows unwritten.)
#ifndef MOE_LIGHT_MX_GU_U
#define MOE_LIGHT_MX_GU_U 2     // 64-wide K chunks in flight per wave (gate|up)
#endif
#ifndef MOE_LIGHT_MX_DN_U
#define MOE_LIGHT_MX_DN_U 2
#endif
#ifndef MOE_LIGHT_MX_GU_TILES
#define MOE_LIGHT_MX_GU_TILES 2
#endif
#ifndef MOE_LIGHT_MX_DN_TILES
#define MOE_LIGHT_MX_DN_TILES 2
#endif
#ifndef MOE_LIGHT_MX_GU_BPC
#define MOE_LIGHT_MX_GU_BPC 2   // blocks per CU in the grid (see MOE_LIGHT_GU_BPC)
#endif
#ifndef MOE_LIGHT_MX_DN_BPC
#define MOE_LIGHT_MX_DN_BPC 4
#endif
// 16 weight codes, streamed like the bf16 weights (load_weights).
__device__ __forceinline__ u32x4_t load_codes(const uint8_t* p) {
    if constexpr (MOE_LIGHT_NT_LOADS != 0)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    else
        return *reinterpret_cast<const u32x4_t*>(p);
}
constexpr int kLightMxWideU = 1;  // chunks in flight, 17..64-row branch

// Eight E4M3 codes (words w0, w1 in K order) times 2^(sb - 127) as an MFMA
// operand.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1, uint32_t sb) {
    const float sc = __uint_as_float(sb << 23);
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Position swizzle of MXFP8 heavy B rows in LDS (64-byte rows of four
// 16-byte units): unit u of row r sits at u ^ mx_swz(r), so that the 16
// rows of one fragment read fall on distinct banks in groups of 8 or 16
// lanes.
__device__ __forceinline__ int mx_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

__device__ __forceinline__ uint32_t load_u16(const uint8_t* p) {
    return *reinterpret_cast<const uint16_t*>(p);
}

// gate|up over MXFP8 weights: one wave, MT row sub-tiles x NTILE column
// tiles (h columns 8*grp0 ..), K = H in 64-wide chunks.
template <int MT, int U, int NTILE>
__device__ __forceinline__ void gateup_light_rows_mx(const FfnArgs& a, int e, int r0, int n,
                                                     int grp0, int l16, int g) {
    const int nc = a.H / 64;
    const int nk = a.H / 32;
    const int lane = g * 16 + l16;
    const size_t grp = (size_t)e * packed_gu_groups(a.I) + grp0;
    const uint8_t* Bp = a.q_gu + grp * nc * 1024 + lane * 16;
    const uint8_t* Sp = a.qs_gu + grp * nc * 32 + l16 * 2;
    const size_t bstride = (size_t)nc * 1024, sstride = (size_t)nc * 32;
    const uint16_t* Ap[MT];
    bool has_a[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int row = m * 16 + l16;
        has_a[m] = row < n;
        const int tok = has_a[m] ? (a.sorted_ids ? a.sorted_ids[r0 + row] : r0 + row) : 0;
        Ap[m] = a.x + (size_t)tok * a.H + 8 * g;
    }
    const int mt_live = (n + 15) / 16;

    floatx4_t acc[MT][NTILE];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NTILE; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t ca[U][MT][2];
    u32x4_t cb[U][NTILE];
    uint32_t cs[U][NTILE];
    auto load_chunk = [&](int c, bf16x8_t (&aa)[MT][2], u32x4_t (&bb)[NTILE],
                          uint32_t (&ss)[NTILE]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) aa[m][0] = aa[m][1] = zero_bf16x8();
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
            bb[t] = u32x4_t{0u, 0u, 0u, 0u};
            ss[t] = 0u;
        }
        if (c < nc) {
#pragma unroll
            for (int t = 0; t < NTILE; ++t) {
                bb[t] = load_codes(Bp + t * bstride + (size_t)c * 1024);
                ss[t] = load_u16(Sp + t * sstride + (size_t)c * 32);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (has_a[m]) {
                    aa[m][0] = load_bf16x8(Ap[m] + c * 64);
                    aa[m][1] = load_bf16x8(Ap[m] + c * 64 + 32);
                }
        }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) load_chunk(u, ca[u], cb[u], cs[u]);
    for (int c0 = 0; c0 < nc; c0 += U) {
        bf16x8_t na[U][MT][2];
        u32x4_t nb_[U][NTILE];
        uint32_t ns[U][NTILE];
#pragma unroll
        for (int u = 0; u < U; ++u) load_chunk(c0 + U + u, na[u], nb_[u], ns[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c0 + u < nc) {
#pragma unroll
                for (int t = 0; t < NTILE; ++t) {
                    const bf16x8_t b0 = e4m3x8_to_bf16(cb[u][t][0], cb[u][t][1], cs[u][t] & 0xffu);
                    const bf16x8_t b1 = e4m3x8_to_bf16(cb[u][t][2], cb[u][t][3], cs[u][t] >> 8);
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        if (m < mt_live) {
                            acc[m][t] = mfma_16x16x32(ca[u][m][0], b0, acc[m][t]);
                            if (2 * (c0 + u) + 1 < nk)
                                acc[m][t] = mfma_16x16x32(ca[u][m][1], b1, acc[m][t]);
                        }
                }
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                ca[u][m][0] = na[u][m][0];
                ca[u][m][1] = na[u][m][1];
            }
#pragma unroll
            for (int t = 0; t < NTILE; ++t) {
                cb[u][t] = nb_[u][t];
                cs[u][t] = ns[u][t];
            }
        }
    }
    const int i0 = grp0 * 8;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float up = __shfl_down(acc[m][t][r], 8, 64);
                const int row = m * 16 + 4 * g + r;
                if (l16 < 8 && row < n)
                    a.h[(size_t)(r0 + row) * a.I + i0 + 8 * t + l16] =
                        (uint16_t)f32_to_bf16_bits(swiglu(acc[m][t][r], up));
            }
        }
    }
}

template <int U, int NTILE>
__global__ __launch_bounds__(kThreads) void gateup_light_mx_kernel(FfnArgs a) {
    static_assert(32 % (NTILE * 8) == 0, "a wave's columns must divide I's multiple of 32");
    constexpr int kCols = 4 * NTILE * 8;
    const int nlight = a.plan[0];
    const int nblk = (a.I + kCols - 1) / kCols;
    const long long nwork = (long long)nlight * nblk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    for (long long wi = blockIdx.x; wi < nwork; wi += gridDim.x) {
        const int slot = (int)(wi / nblk), nb = (int)(wi % nblk);
        const int i0 = nb * kCols + wave * NTILE * 8;
        if (i0 >= a.I) continue;  // I % 32 == 0: a wave is all in or all out
        const int e = a.plan[kPlanHeader + slot];
        const int r0 = a.offsets[e];
        const int n = a.offsets[e + 1] - r0;
        for (int p = 0; p < n; p += kLightRowsMax) {
            const int np = min(kLightRowsMax, n - p);
            if (np <= 16)
                gateup_light_rows_mx<1, U, NTILE>(a, e, r0 + p, np, i0 / 8, l16, g);
            else
                gateup_light_rows_mx<kLightSubTiles, kLightMxWideU, NTILE>(a, e, r0 + p, np,
                                                                           i0 / 8, l16, g);
        }
    }
}

// down over MXFP8 weights: MT row sub-tiles x NT column tiles (16 output
// columns each, c0 ..), K = I in 64-wide chunks; a chunk's second K step
// past I (I % 64 == 32) is padding and is skipped.
template <int MT, int U, int NT>
__device__ __forceinline__ void down_light_rows_mx(const FfnArgs& a, int e, int r0, int n, int c0,
                                                   int l16, int g) {
    const int nc = mx_chunks(a.I);
    const int nk = a.I / 32;
    const int lane = g * 16 + l16;
    const size_t grp = (size_t)e * packed_dn_groups(a.H) + c0 / 16;
    const uint8_t* Bp = a.q_dn + grp * nc * 1024 + lane * 16;
    const uint8_t* Sp = a.qs_dn + grp * nc * 32 + l16 * 2;
    const size_t bstride = (size_t)nc * 1024, sstride = (size_t)nc * 32;
    const uint16_t* Ap[MT];
    bool has_a[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int row = m * 16 + l16;
        has_a[m] = row < n;
        Ap[m] = a.h + (size_t)(r0 + (has_a[m] ? row : 0)) * a.I + 8 * g;
    }
    const int mt_live = (n + 15) / 16;

    floatx4_t acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t ca[U][MT][2];
    u32x4_t cb[U][NT];
    uint32_t cs[U][NT];
    auto load_chunk = [&](int c, bf16x8_t (&aa)[MT][2], u32x4_t (&bb)[NT], uint32_t (&ss)[NT]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) aa[m][0] = aa[m][1] = zero_bf16x8();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            bb[t] = u32x4_t{0u, 0u, 0u, 0u};
            ss[t] = 0u;
        }
        if (c < nc) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                bb[t] = load_codes(Bp + t * bstride + (size_t)c * 1024);
                ss[t] = load_u16(Sp + t * sstride + (size_t)c * 32);
            }
            const bool second = 2 * c + 1 < nk;
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (has_a[m]) {
                    aa[m][0] = load_bf16x8(Ap[m] + c * 64);
                    if (second) aa[m][1] = load_bf16x8(Ap[m] + c * 64 + 32);
                }
        }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) load_chunk(u, ca[u], cb[u], cs[u]);
    for (int k0 = 0; k0 < nc; k0 += U) {
        bf16x8_t na[U][MT][2];
        u32x4_t nb_[U][NT];
        uint32_t ns[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) load_chunk(k0 + U + u, na[u], nb_[u], ns[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (k0 + u < nc) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const bf16x8_t b0 = e4m3x8_to_bf16(cb[u][t][0], cb[u][t][1], cs[u][t] & 0xffu);
                    const bf16x8_t b1 = e4m3x8_to_bf16(cb[u][t][2], cb[u][t][3], cs[u][t] >> 8);
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        if (m < mt_live) {
                            acc[m][t] = mfma_16x16x32(ca[u][m][0], b0, acc[m][t]);
                            if (2 * (k0 + u) + 1 < nk)
                                acc[m][t] = mfma_16x16x32(ca[u][m][1], b1, acc[m][t]);
                        }
                }
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                ca[u][m][0] = na[u][m][0];
                ca[u][m][1] = na[u][m][1];
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                cb[u][t] = nb_[u][t];
                cs[u][t] = ns[u][t];
            }
        }
    }
    if (a.y_fmt == kYBF16) {
        light_store_y16<kYBF16>(a, acc, r0, n, c0, l16, g);
        return;
    }
    if (a.y_fmt == kYF16) {
        light_store_y16<kYF16>(a, acc, r0, n, c0, l16, g);
        return;
    }
    float* y = static_cast<float*>(a.y);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int c = c0 + t * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m * 16 + 4 * g + r;
                if (row < n) y[(size_t)(r0 + row) * a.H + c] = acc[m][t][r];
            }
        }
    }
}

template <int NT, int U>
__global__ __launch_bounds__(kThreads) void down_light_mx_kernel(FfnArgs a) {
    static_assert(64 % (NT * 16) == 0, "a wave's columns must divide H's multiple of 64");
    constexpr int kCols = 4 * NT * 16;
    const int nlight = a.plan[0];
    const int nblk = (a.H + kCols - 1) / kCols;
    const long long nwork = (long long)nlight * nblk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    for (long long wi = blockIdx.x; wi < nwork; wi += gridDim.x) {
        const int slot = (int)(wi / nblk), nb = (int)(wi % nblk);
        const int c0 = nb * kCols + wave * NT * 16;
        if (c0 >= a.H) continue;
        const int e = a.plan[kPlanHeader + slot];
        const int r0 = a.offsets[e];
        const int n = a.offsets[e + 1] - r0;
        for (int p = 0; p < n; p += kLightRowsMax) {
            const int np = min(kLightRowsMax, n - p);
            if (np <= 16)
                down_light_rows_mx<1, U, NT>(a, e, r0 + p, np, c0, l16, g);
            else
                down_light_rows_mx<kLightSubTiles, kLightMxWideU, NT>(a, e, r0 + p, np, c0, l16,
                                                                      g);
        }
    }
}

// ---------------------------------------------------------------- heavy
// 256x256 output tiles computed by 8 waves (2 per SIMD) in a 2 (rows) x 4
// (columns) grid; each wave owns a 128x64 block of 16x16 MFMA tiles (32
// accumulators per lane).  Operands are staged with direct-to-LDS 16-byte
// loads (buffer_load_dwordx4 ... lds) into LDS rings, one 64-wide K step
// per buffer, so that every load instruction reads 8 whole rows of 128
// contiguous bytes (full cache lines).
//
// LDS layout of a stage: A then B, each a run of 1 KB blocks, block b holding
// tile rows 8b..8b+7 x the stage's 64 K values.  Inside a block, 16-byte slot
// p holds row p/8, K chunk (p%8) ^ (p/8) (chunk c = K values 8c..8c+7).  The
// load that fills a block therefore reads one 128-byte line per 8 lanes, and
// the MFMA fragment read (lane l: row l%16, chunk l/16 + 4*half) puts the 8
// lanes of each row group on 8 different 16-byte bank groups.  (Measured on
// MI355X: this read runs at the speed of a contiguous 1 KB read; also
// xor-ing the block parity into the chunk costs a third of it.)
enum class Mode { GateUp, Down };

constexpr int kHeavyThreads = 512;
constexpr int kHeavyWaves = kHeavyThreads / 64;
constexpr int kTN = 256;       // B rows per tile (output columns, or 128 gate + 128 up rows)
constexpr int kWTN = kTN / 4;  // 64 columns per wave
// LDS rings, one per operand: A (rows of x or h, TM x 64 K per stage) and B
// (the expert weights, 256 x 64 per stage; MXFP8: 16 KB of codes + 512 B of
// scales), each as deep as the 160 KB allow for the tile height.  The loads
// are split by role: waves 0..3 fill the A ring, waves 4..7 the B ring, so
// every wave keeps one ring's loads in flight and waits for its own stage
// with one vmcnt count, whatever the tile height.  A stage is issued `depth
// - 1` stages before it is read: a deeper ring covers a longer load latency
// (the weights come from HBM; on MI355X the latency under load is about the
// MFMA time of one 64-wide stage of a 256-row tile).
constexpr int kKS = 64;            // K values per stage
constexpr int kHeavyLds = 160 * 1024;  // LDS of the heavy kernels: the largest ring pair below
constexpr int kBlk = 1024;         // bytes of one 8-row x 64-K block
constexpr int kBlocksB = kTN / 8;  // 32
constexpr int kRoleWaves = 4;      // waves per DMA role (A: 0..3, B: 4..7)
constexpr int kBInst16 = kBlocksB / kRoleWaves;  // 8 bf16 B blocks per B wave and stage
static_assert(kBInst16 % 2 == 0, "a B wave's blocks start a record row block");
constexpr int kB8Blk = 4;          // MXFP8 code blocks (16 rows x 64 codes) per B wave and stage
constexpr int kBInst8 = kB8Blk + 1;  // ... plus one load of 128 scale bytes

// Ring depths (A, B) per tile height (compile-time tunables).
#ifndef MOE_RING_256
#define MOE_RING_256 2, 3
#endif
#ifndef MOE_RING_256_DOWN
#define MOE_RING_256_DOWN 3, 2
#endif
#ifndef MOE_RING_224
#define MOE_RING_224 2, 3
#endif
#ifndef MOE_RING_192
#define MOE_RING_192 2, 3
#endif
#ifndef MOE_RING_160
#define MOE_RING_160 3, 3
#endif
#ifndef MOE_RING_128
#define MOE_RING_128 3, 3
#endif
#ifndef MOE_RING_MX
#define MOE_RING_MX 3, 3
#endif
struct RingDepth {
    int a, b;
};
template <Mode M, int TM, bool W8>
constexpr RingDepth ring_depth() {
    if (W8) return RingDepth{MOE_RING_MX};
    if (TM == 256) return M == Mode::Down ? RingDepth{MOE_RING_256_DOWN} : RingDepth{MOE_RING_256};
    if (TM == 224) return RingDepth{MOE_RING_224};
    if (TM == 192) return RingDepth{MOE_RING_192};
    if (TM == 160) return RingDepth{MOE_RING_160};
    return RingDepth{MOE_RING_128};
}

// Per tile height TM (a multiple of 32 in [128, 256]): each wave row group
// holds TM/2 rows = TM/32 MFMA row tiles; a stage holds TM/8 A blocks, TM/32
// per A wave, and 32 B blocks, 8 per B wave.
template <Mode M, int TM, bool W8>
struct HeavyGeom {
    static_assert(TM % 32 == 0 && TM >= 128 && TM <= 256, "tile height");
    static constexpr int kRF = TM / 32;                   // row tiles per wave
    static constexpr int kBlocksA = TM / 8;
    static constexpr int kAInst = kBlocksA / kRoleWaves;  // A loads per A wave and stage
    static constexpr int kABytes = kBlocksA * kBlk;       // A bytes per stage
    static constexpr int kBBytes = W8 ? kMxStageBytes : kBlocksB * kBlk;
    static constexpr int kBInst = W8 ? kBInst8 : kBInst16;
    static constexpr int kAStages = ring_depth<M, TM, W8>().a;
    static constexpr int kBStages = ring_depth<M, TM, W8>().b;
    static_assert(kAStages >= 2 && kBStages >= 2 && kAStages <= 4 && kBStages <= 4, "ring depth");
    static_assert(kAStages * kABytes + kBStages * kBBytes <= kHeavyLds, "LDS rings");
    static_assert(kAInst * 3 < 64 && kBInst * 3 < 64, "vmcnt range");
};

// Epilogue staging of the down GEMM's y.  A finished tile is written to LDS
// (the ring is idle by then) in row-major order, rows padded by 16 bytes,
// then read back in 16-byte chunks of whole rows and stored with 16-byte
// lane stores: each store instruction writes 1 KB of whole cache lines.
// Stored straight from the MFMA layout a lane holds 4 rows of one column, so
// every store instruction wrote 2- or 4-byte pieces of 4 or 8 rows (measured
// on MI355X: down -10% at prefill, -3% at the Ling-like layer with staging).
// gate|up keeps the direct stores: its h tile is half as wide, and staging
// it cost more than it saved (+4%).  fp32 y is staged in two passes of half
// the rows (one wave row each) to fit the 160 KB.
#ifndef MOE_HEAVY_STAGED_EPI
#define MOE_HEAVY_STAGED_EPI 1
#endif
constexpr int kStgPad = 16;
template <Mode M, int TM, int YF>
struct Staging {
    static constexpr int kCols = M == Mode::GateUp ? kTN / 2 : kTN;  // output columns of a tile
    static constexpr int kElt = (M == Mode::Down && YF == kYF32) ? 4 : 2;
    static constexpr int kRowBytes = kCols * kElt;  // 256 (h), 512 (16-bit y), 1024 (fp32 y)
    static constexpr int kPitch = kRowBytes + kStgPad;
    static constexpr int kPasses = (M == Mode::Down && YF == kYF32) ? 2 : 1;
    static constexpr int kPassRows = TM / kPasses;
    static constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per row
    static constexpr int kIters = kPassRows * kChunks / kHeavyThreads;  // chunks per lane and pass
    static_assert(kPassRows * kChunks % kHeavyThreads == 0, "staging split");
    // gate|up with split h stages two planes (hi, lo)
    static_assert(2 * kPassRows * kPitch <= kHeavyLds || M == Mode::Down, "staging size");
    static_assert(kPassRows * kPitch <= kHeavyLds, "staging size");
};

typedef __attribute__((address_space(3))) void* lptr_t;

// Raw buffer resource over [base, base + bytes): loads past the end read 0
// instead of touching memory.  Word 3 = 0x00020000: 32-bit data format, no
// swizzle (the CDNA raw-buffer setting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from rsrc + voff + soff into LDS at dst + 16*lane
// (buffer_load_dwordx4 ... lds).
// NT: non-temporal hint (the cache policy's nt bit), for data no other tile
// will read.
template <bool NT = false>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              char* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)dst, 16, (int)voff, (int)soff, 0,
                                             NT ? 2 : 0);
}

// Wait until at most n of this wave's vector-memory instructions are
// outstanding (vmcnt; expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier without the memory fences __syncthreads() adds: those
// wait for every outstanding load (vmcnt(0)) and would drain the LDS ring.
// Each wave first waits for its own part of the stage (wait_vmcnt); the empty
// asm statements keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Read of a plan or offsets entry at a wave-uniform index through the
// constant address space: a scalar load, so it does not count against the
// vector-memory counter that the LDS ring's waits are written for.  The
// heavy kernels never write these arrays.
__device__ __forceinline__ int32_t sload(const int32_t* p, int i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Height index (height 256 - 32 * index) of row tile `tile`: from the
// plan's tile list, or the dense group's one height.
__device__ __forceinline__ int tile_tmi(const FfnArgs& a, int tile) {
    if (a.plan)
        return (int)((uint32_t)sload(a.plan, kPlanHeader + a.E + 2 * tile + 1) >> kTileTmShift);
    return tile_tm_index(a.dense_tm);
}

// Order of the work items of one expert (its row tiles x N blocks, a
// contiguous range of the work list), per GEMM: 0 = the N block runs
// fastest, 1 = the row tile runs fastest (the row tiles that read one N
// block's weights are then neighbours in the list, and so run at the same
// time).  Measured at long prefill (three 224-row tiles per expert, 8 N
// blocks of gate|up and 16 of down per row tile): gate|up with 1 fetches
// 15.5 GB instead of 23.4 GB and runs 1-2% faster; down with 1 fetches
// 5.8 GB instead of 10.5 GB but runs 3-4% slower (its 48 items per expert
// then straddle two rounds of an XCD's blocks, and h rows are read again).
// Results do not depend on it.
#ifndef MOE_HEAVY_ORDER_GU
#define MOE_HEAVY_ORDER_GU 1
#endif
#ifndef MOE_HEAVY_ORDER_DN
#define MOE_HEAVY_ORDER_DN 0
#endif

// Row tile and N block of work item w of GEMM M.  The expert-major order
// (MOE_HEAVY_ORDER_* = 1) applies to experts whose items fit one round of an
// XCD slice's blocks (num_cu / kXcds): their row tiles then run together and
// share each N block's weights.  An expert with more tiles keeps the N block
// fastest, so that each row tile's N blocks (which share its A rows) run
// together instead of over several rounds.
template <Mode M>
__device__ __forceinline__ int item_tile(const FfnArgs& a, long long w, int nblk, int& nb) {
    const int tg = (int)(w / nblk);
    if ((M == Mode::GateUp ? MOE_HEAVY_ORDER_GU : MOE_HEAVY_ORDER_DN) == 0 || !a.plan) {
        nb = (int)(w % nblk);
        return tg;
    }
    // The expert of tile tg, its tile count and tg's index among its tiles:
    // an expert's tiles all have one height (tile_split), so first rows are
    // multiples of it and the count is the rows over it, rounded up.
    const int base = kPlanHeader + a.E + 2 * tg;
    const int e = sload(a.plan, base);
    const uint32_t ent = (uint32_t)sload(a.plan, base + 1);
    const int tm = tile_height((int)(ent >> kTileTmShift));
    const int n = sload(a.offsets, e + 1) - sload(a.offsets, e);
    const int nt = (n + tm - 1) / tm;
    if (nt * nblk > a.num_cu / kXcds) {
        nb = (int)(w % nblk);
        return tg;
    }
    const int t0 = tg - (int)(ent & (uint32_t)kTileRowMask) / tm;
    const int q = (int)(w - (long long)t0 * nblk);
    nb = q / nt;
    return t0 + q % nt;
}

// Runs this block's work items wi, wi + nb_x, ... (below wend) while their
// row tiles are TM rows high, and returns the first item of another height
// (or one at or past wend).
// YF (down only): y storage, fp32, bf16 or fp16 (a.y_fmt).
// BS: where B (the weights) comes from -- kBRowMajor: w_gu / w_dn; kBRec16:
// the bf16 heavy-tile records of the packed copy (a.hr_gu / a.hr_dn: one
// 32 KB run per (expert, 256-row tile, K stage), so a stage is one
// contiguous read instead of 256 row pieces 2H bytes apart); kBRecMx (W8):
// the MXFP8 heavy-tile records (a.hq_gu / a.hq_dn):
// a stage is 256 rows x 64 codes plus their scales, staged by the same LDS
// DMA; each fragment read takes both 32-wide halves of a row's chunk (16
// bytes) and its two scales, and the hardware's scaled conversion turns
// them into the bf16 operands of the bf16 path -- the same MFMA chains on the
// dequantised weights, so the results equal the bf16 path's bit for bit.
// Wait until at most `stages` whole stages of this wave's ring (kInst loads
// each) are outstanding; `stages` is 0..3 (wave-uniform).
template <int kInst>
__device__ __forceinline__ void wait_stages(int stages) {
    if (stages <= 0)
        wait_vmcnt<0>();
    else if (stages == 1)
        wait_vmcnt<kInst>();
    else if (stages == 2)
        wait_vmcnt<2 * kInst>();
    else
        wait_vmcnt<3 * kInst>();
}

template <Mode M, int TM, int YF, int BS>
__device__ __forceinline__ long long ffn_heavy_run(const FfnArgs& a, char* lds, long long wi,
                                                 long long wend, int nb_x, int nblk) {
    constexpr bool W8 = BS == kBRecMx;
    using G = HeavyGeom<M, TM, W8>;
    constexpr int kRF = G::kRF, kAInst = G::kAInst, kBInst = G::kBInst;
    constexpr int kABytes = G::kABytes, kBBytes = G::kBBytes;
    constexpr int ast = G::kAStages, bst = G::kBStages;
    constexpr int kTmi = (kTileTMMax - TM) / kTileTMStep;
    // One LDS object for both rings (A stages, then B stages): with two
    // objects the compiler waits for every LDS DMA before any LDS read.
    auto a_slot = [&](int slot) -> char* { return lds + slot * kABytes; };
    auto b_slot = [&](int slot) -> char* { return lds + ast * kABytes + slot * kBBytes; };

    // split_h: the down GEMM's K runs over [hi | lo] (2I) against W_down twice.
    const int K = (M == Mode::GateUp) ? a.H : (a.split_h ? 2 * a.I : a.I);
    const int hstride = a.split_h ? 2 * a.I : a.I;  // row pitch of h
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: LDS offsets in SGPRs
    const int wm = wave >> 2, wn = wave & 3;
    // DMA role (wave-uniform): waves 0..3 load A, waves 4..7 load B; rw is
    // the wave's index within its role.
    const bool a_role = wave < kRoleWaves;
    const int rw = wave & (kRoleWaves - 1);
    const int depth = a_role ? ast : bst;
    const int l16 = lane & 15, g = lane >> 4;
    const int nh = K / 32;         // 32-wide MFMA K steps (K % 32 == 0)
    const int nst = (nh + 1) / 2;  // 64-wide stages; the last one is half full if nh is odd
    // DMA side: lane L fills slot L of a block: row L/8, chunk (L%8)^(L/8).
    const int drow = lane >> 3;
    const int dchunk = (lane & 7) ^ drow;
    // Lanes whose chunk is in the upper half of the stage (K values 32..63).
    const bool upper = (dchunk & 4) != 0;
    // Fragment side: lane l reads row l%16 (block 2f + (l%16)/8), chunk g + 4*half.
    const int fblk = (lane >> 3) & 1;
    const int frow = lane & 7;
    const int foff0 = fblk * kBlk + frow * 128 + ((g ^ frow) << 4);
    const int foff1 = fblk * kBlk + frow * 128 + (((g + 4) ^ frow) << 4);

    // Per-tile state: output block nb of row tile (e, m0); rows of the tile
    // that exist; buffer resources and per-lane byte offsets of the loads.
    struct Tile {
        int nb, e, r0, m0, rows;
        bool once;  // the expert's only row tile: no other tile reads its weights
    };
    // Where work item w sits (scalar reads only).
    auto locate = [&](long long w) -> Tile {
        Tile t;
        const int tile = item_tile<M>(a, w, nblk, t.nb);
        if (a.plan) {
            const int base = kPlanHeader + a.E + 2 * tile;
            t.e = sload(a.plan, base);
            t.m0 = sload(a.plan, base + 1) & kTileRowMask;
            t.r0 = sload(a.offsets, t.e);
            const int total = sload(a.offsets, t.e + 1) - t.r0;
            t.rows = min(TM, total - t.m0);
            t.once = t.m0 == 0 && total <= TM;
        } else {
            t.e = 0;
            t.r0 = 0;
            t.m0 = tile * TM;
            t.rows = min(TM, a.dense_rows - t.m0);
            t.once = a.dense_rows <= TM;
        }
        return t;
    };
    int nb = 0, r0 = 0, m0 = 0, rows = 0;
    // Weights of a tile that is its expert's only one are streamed past the
    // caches' retention (nt): they are read once, and keeping them would
    // push out the A rows the tile's N blocks share.  Weights that several
    // row tiles read stay cached.  (Measured: Ling-like step -6%, prefill
    // -2.5%; long prefill, three row tiles per expert, +8% if all were nt.)
    bool b_once = false;
    __amdgpu_buffer_rsrc_t src;  // this wave's ring source
    // Per-lane byte offsets of this wave's loads within `src` (A waves: row
    // and K chunk of each A block; B waves: of each B block, or for the
    // records the first block's, the others following 1 KB apart).
    constexpr int kDOff = kAInst > kBInst16 ? kAInst : kBInst16;
    uint32_t doff[kDOff];
    // Load sources of tile t for this wave's role.
    auto use_tile = [&](const Tile& t) {
        nb = t.nb;
        r0 = t.r0;
        m0 = t.m0;
        rows = t.rows;
        b_once = t.once;
        if (a_role) {
            if (M == Mode::GateUp)
                src = make_rsrc(a.x, (uint32_t)((size_t)a.T * a.H * 2));
            else
                src = make_rsrc(a.h + (size_t)(r0 + m0) * hstride, (uint32_t)((size_t)TM * hstride * 2));
#pragma unroll
            for (int i = 0; i < kAInst; ++i) {
                const int b = kAInst * rw + i;
                const int r = b * 8 + drow;         // row within the tile
                const int rr = r < rows ? r : 0;    // rows past the count: any valid row
                const uint32_t cb = (uint32_t)dchunk * 16u;
                if (M == Mode::GateUp) {
                    const int tok = a.sorted_ids ? a.sorted_ids[r0 + m0 + rr] : r0 + m0 + rr;
                    doff[i] = (uint32_t)tok * (uint32_t)a.H * 2u + cb;
                } else {
                    doff[i] = (uint32_t)rr * (uint32_t)hstride * 2u + cb;
                }
            }
            return;
        }
        if constexpr (W8) {
            // the tile's records: one per K chunk, kMxStageBytes each.  Code
            // block b = 4*rw + i holds tile rows 16b..16b+15; lane L fills
            // LDS slot L: row L/4, 16-byte unit L%4, which takes unit
            // (L%4) ^ mx_swz(row) of the record's row (the swizzle spreads
            // the fragment reads of 16 rows over all banks).
            const uint8_t* base = M == Mode::GateUp ? a.hq_gu : a.hq_dn;
            const size_t rec = (size_t)nst * kMxStageBytes;
            src = make_rsrc(base + ((size_t)t.e * nblk + nb) * rec, (uint32_t)rec);
#pragma unroll
            for (int i = 0; i < kB8Blk; ++i) {
                const int r = (kB8Blk * rw + i) * 16 + (lane >> 2);
                doff[i] = (uint32_t)r * 64u + 16u * (uint32_t)((lane & 3) ^ mx_swz(r));
            }
            // scales: this wave's 128 bytes, lanes 0..7
            doff[kB8Blk] = (uint32_t)kMxCodeBytes + 128u * (uint32_t)rw + 16u * (uint32_t)(lane & 7);
            return;
        }
        if constexpr (BS == kBRec16) {
            // the record's 1 KB chunks are copied as they are: LDS block
            // 2jb + h holds chunk h of the tile's row block jb, lane L's
            // operand at 16 L; this wave's 8 chunks are 8 KB contiguous
            const uint16_t* base = M == Mode::GateUp ? a.hr_gu : a.hr_dn;
            const size_t rec = (size_t)nst * kRec16Bytes;
            src = make_rsrc(reinterpret_cast<const char*>(base) + ((size_t)t.e * nblk + nb) * rec,
                            (uint32_t)rec);
            doff[0] = (uint32_t)(kBInst16 * rw) * (uint32_t)kBlk + (uint32_t)lane * 16u;
            return;
        }
        if (M == Mode::GateUp)
            src = make_rsrc(a.w_gu + (size_t)t.e * 2 * a.I * a.H, (uint32_t)((size_t)2 * a.I * a.H * 2));
        else
            src = make_rsrc(a.w_dn + (size_t)t.e * a.H * a.I, (uint32_t)((size_t)a.H * a.I * 2));
#pragma unroll
        for (int i = 0; i < kBInst16; ++i) {
            const int b = kBInst16 * rw + i;
            const int r = b * 8 + drow;  // B row within the tile
            const uint32_t cb = (uint32_t)dchunk * 16u;
            if (M == Mode::GateUp) {
                // 16-row blocks alternate: block 2p = gate rows, 2p+1 = the
                // matching up rows, so g and u of an element share a lane.
                const int hc = nb * (kTN / 2) + (r >> 5) * 16 + (r & 15);
                const int wr = (hc < a.I) ? (((r & 16) == 0) ? hc : a.I + hc) : 0;
                doff[i] = (uint32_t)wr * (uint32_t)a.H * 2u + cb;
            } else {
                const int c = nb * kTN + r;
                doff[i] = (uint32_t)(c < a.H ? c : 0) * (uint32_t)a.I * 2u + cb;
            }
        }
    };
    auto setup = [&](long long w) { use_tile(locate(w)); };
    auto adjust = [&](int kk, uint32_t& adj_a, uint32_t& adj_b) {
        // Upper-half lanes in two rare stages: in the half-full last stage
        // they reload an in-row chunk that is never used; in the stage that
        // straddles I (split_h with I % 64 == 32) their B columns wrap back
        // onto W_down.  The adjustment is made opaque so that no adjusted copy
        // of the offsets is hoisted out of the loop.
        const bool tail = kk + kKS > K;
        const bool straddle = M == Mode::Down && kk < a.I && kk + kKS > a.I && K > a.I;
        adj_a = (tail && upper) ? 64u : 0u;
        adj_b = (tail && upper) ? 64u : ((straddle && upper) ? (uint32_t)a.I * 2u : 0u);
        asm volatile("" : "+v"(adj_a), "+v"(adj_b));
    };
    // This wave's loads of stage st (of the current source) into ring slot
    // `slot`: A blocks kAInst*rw.. or B blocks of the wave's share.  The
    // whole offset goes in the lane's VGPR; the 32-bit sum is exact because
    // the true offset is never negative.
    auto issue = [&](int st, int slot) {
        if (a_role) {
            char* buf = a_slot(slot) + kAInst * rw * kBlk;
            const int kk = st * kKS;
            uint32_t adj_a, adj_b;
            adjust(kk, adj_a, adj_b);
            const uint32_t sa = (uint32_t)kk * 2u - adj_a;
#pragma unroll
            for (int i = 0; i < kAInst; ++i) lds_dma16(src, doff[i] + sa, 0u, buf + i * kBlk);
            return;
        }
        char* buf = b_slot(slot);
        if constexpr (W8) {
            const uint32_t sb = (uint32_t)st * (uint32_t)kMxStageBytes;
            char* cbuf = buf + kB8Blk * rw * kBlk;
            char* sbuf = buf + kMxCodeBytes + 128 * rw;
            if (b_once) {
#pragma unroll
                for (int i = 0; i < kB8Blk; ++i) lds_dma16<true>(src, doff[i] + sb, 0u, cbuf + i * kBlk);
                if (lane < 8) lds_dma16<true>(src, doff[kB8Blk] + sb, 0u, sbuf);
            } else {
#pragma unroll
                for (int i = 0; i < kB8Blk; ++i) lds_dma16(src, doff[i] + sb, 0u, cbuf + i * kBlk);
                if (lane < 8) lds_dma16(src, doff[kB8Blk] + sb, 0u, sbuf);
            }
            return;
        }
        buf += kBInst16 * rw * kBlk;
        if constexpr (BS == kBRec16) {
            // padded records: no tail adjustment; the wave's 8 blocks are
            // 8 KB contiguous in the record
            const uint32_t sb = (uint32_t)st * (uint32_t)kRec16Bytes + doff[0];
            if (b_once) {
#pragma unroll
                for (int i = 0; i < kBInst16; ++i)
                    lds_dma16<true>(src, sb + (uint32_t)(i * kBlk), 0u, buf + i * kBlk);
            } else {
#pragma unroll
                for (int i = 0; i < kBInst16; ++i)
                    lds_dma16(src, sb + (uint32_t)(i * kBlk), 0u, buf + i * kBlk);
            }
            return;
        }
        const int kk = st * kKS;
        // down with split_h: K columns past I wrap back onto W_down
        const int kb = (M == Mode::Down && kk >= a.I) ? kk - a.I : kk;
        uint32_t adj_a, adj_b;
        adjust(kk, adj_a, adj_b);
        const uint32_t sb = (uint32_t)kb * 2u - adj_b;
        if (b_once) {
#pragma unroll
            for (int i = 0; i < kBInst16; ++i) lds_dma16<true>(src, doff[i] + sb, 0u, buf + i * kBlk);
        } else {
#pragma unroll
            for (int i = 0; i < kBInst16; ++i) lds_dma16(src, doff[i] + sb, 0u, buf + i * kBlk);
        }
    };
    // A tile's first loads: this wave's ring, stages 0 .. depth-1 (those
    // that exist) into slots 0 .. depth-1.
    auto issue_first = [&]() {
        for (int st = 0; st < depth && st < nst; ++st) issue(st, st);
    };
    // Wait until this wave's loads leave at most `stages` stages outstanding.
    auto wait_own = [&](int stages) {
        if (a_role)
            wait_stages<kAInst>(stages);
        else
            wait_stages<kBInst>(stages);
    };
    // Fragment reads of one 32-wide K half of a stage.  A fragment i of this
    // wave is tile rows wm*TM/2 + 16i.., B fragment j is B rows (wn*4 + j)*16..
    auto rd_a = [&](int slot, int half, int blk) -> bf16x8_t {
        const char* p = a_slot(slot) + blk * kBlk + (half ? foff1 : foff0);
        return *reinterpret_cast<const bf16x8_t*>(p);
    };
    // (From the packed records the stage is in chunk order: fragment j's
    // half is chunk 2 (wn*4 + j) + half, lane l's operand at 16 l.)
    auto read_b = [&](int slot, int half, bf16x8_t (&bf)[4]) {
        const char* base = b_slot(slot);
        if constexpr (BS == kBRec16)
            base += half * kBlk + lane * 16;
        else
            base += half ? foff1 : foff0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[j] = *reinterpret_cast<const bf16x8_t*>(base + (wn * 4 + j) * 2 * kBlk);
    };
    // W8: raw codes of both halves of B fragment j (row (wn*4 + j)*16 + l16,
    // unit g: K 8g.. then 32+8g..) and the lane's 8 scale bytes (2j: first
    // half of fragment j, 2j+1: second half).
    const int b8off = l16 * 64 + 16 * (g ^ mx_swz(l16));
    auto read_b8 = [&](int slot, u32x4_t (&raw)[4], u32x2_t& sc) {
        const char* base = b_slot(slot);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            raw[j] = *reinterpret_cast<const u32x4_t*>(base + (wn * 4 + j) * 16 * 64 + b8off);
        sc = *reinterpret_cast<const u32x2_t*>(base + kMxCodeBytes + (wn * 16 + l16) * 8);
    };
    // One 32-wide half of the B fragments from the raw codes: half 0 is
    // converted after the barrier (its MFMAs come first), half 1 behind the
    // stage's first MFMA group, so that the two waves of a SIMD (which read
    // the same fragments) do not stall their MFMAs on all of it at once.
    auto cvt_b8 = [&](const u32x4_t (&raw)[4], const u32x2_t& sc, int half, bf16x8_t (&b)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t sw = sc[j >> 1] >> (16 * (j & 1));
            b[j] = half ? e4m3x8_to_bf16(raw[j][2], raw[j][3], (sw >> 8) & 0xffu)
                        : e4m3x8_to_bf16(raw[j][0], raw[j][1], sw & 0xffu);
        }
    };
    // A fragments in two groups: rows [0, kG0) and [kG0, kRF).
    constexpr int kG0 = kRF / 2;
    auto read_a = [&](int slot, int half, int grp, bf16x8_t (&af)[kRF]) {
        const int i0 = grp ? kG0 : 0, i1 = grp ? kRF : kG0;
#pragma unroll
        for (int i = i0; i < i1; ++i) af[i] = rd_a(slot, half, (wm * kRF + i) * 2);
    };

    // Cross-tile prefetch (down only): while a tile runs its last stages, the
    // ring slots it frees take the next tile's first stages, as if the two
    // tiles' K loops were one stream, so the next tile starts with its first
    // stage in LDS and its first fragments in registers.  Each wave switches
    // its source to the next tile just before its ring's first load of it.
    // Down only: its setup needs scalar reads alone, while gate|up gathers
    // row ids with vector loads, which the ring's vmcnt waits do not count.
    // Needs whole stages (nh even) and at least as many stages as a ring is
    // deep; not for 256-row tiles (the extra state spills).
    constexpr int kDeepest = ast > bst ? ast : bst;
    // (The down GEMM's staged epilogue reuses the ring, so it leaves no room
    // for a prefetch.)
    const bool pf_ok = !MOE_HEAVY_STAGED_EPI && M == Mode::Down && TM != 256 && (nh & 1) == 0 &&
                       nst >= kDeepest;

    setup(wi);
    issue_first();
    int rs = 0;             // this wave's ring slot of the current stage
    int as = 0, bs = 0;     // A and B slots of the current stage (fragment reads)
    bool primed = false;    // stage 0 already in, its first fragments in af / bf0
    bf16x8_t af[kRF], bf0[4], bf1[4];
    u32x4_t raw[4];  // W8: next stage's B codes, converted behind the MFMAs
    u32x2_t sc;
    while (true) {
        floatx4_t acc[kRF][4];
#pragma unroll
        for (int i = 0; i < kRF; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        auto mfma_rows = [&](int grp, const bf16x8_t (&af)[kRF], const bf16x8_t (&bf)[4]) {
            const int i0 = grp ? kG0 : 0, i1 = grp ? kRF : kG0;
#pragma unroll
            for (int i = i0; i < i1; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(af[i], bf[j], acc[i][j]);
        };

        const int t_nb = nb, t_base = r0 + m0, t_rows = rows;
        const long long wnext = wi + nb_x;
        int nb_next;
        const bool more = wnext < wend && tile_tmi(a, item_tile<M>(a, wnext, nblk, nb_next)) == kTmi;
        const bool pf = pf_ok && more;
        Tile nx{};
        if (pf) nx = locate(wnext);

        if (!primed) {
            // The first loads were requested after the previous tile's
            // epilogue stores (or above, for the first tile); vector-memory
            // operations retire in order, so stage 0 is in once at most the
            // wave's later stages are pending.
            wait_own(min(depth, nst) - 1);
            ring_barrier();
            if constexpr (W8) {
                read_b8(0, raw, sc);
                cvt_b8(raw, sc, 0, bf0);
            } else {
                read_b(0, 0, bf0);
            }
            read_a(0, 0, 0, af);
            read_a(0, 0, 1, af);
        }
        // Each 32-wide half step runs its MFMAs in two groups of rows; the
        // fragments of the next half step are read behind them: B and the
        // first half of the A rows after the first group (those rows are done
        // with), the second half of the A rows after the second group.  At a
        // stage boundary the first group also covers the wait for the next
        // stage and the barrier that frees this stage's buffers for the loads
        // `depth` stages ahead.  One loop with a branch-free body (no peeled
        // copies): peeling made the register allocator stop keeping each
        // accumulator in place and spill.
        const int nfull = nh / 2;  // stages with both halves
        for (int st = 0; st < nfull; ++st) {
            const int bn = (bs + 1 == bst) ? 0 : bs + 1;  // B slot of stage st+1
            const int an = (as + 1 == ast) ? 0 : as + 1;  // A slot of stage st+1
            mfma_rows(0, af, bf0);
            if constexpr (W8)
                cvt_b8(raw, sc, 1, bf1);  // raw: both halves came with stage st
            else
                read_b(bs, 1, bf1);
            read_a(as, 1, 0, af);
            mfma_rows(1, af, bf0);
            read_a(as, 1, 1, af);
            mfma_rows(0, af, bf1);
            // After the last stage without a prefetch this wait, barrier and
            // the reads of the (absent) next stage are harmless: no load is
            // outstanding and the ring addresses are valid.  With one, the
            // next stage is the next tile's stage 0.
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of st done
            // Stage st+1 in: this wave has issued stages up to st+depth-1 (of
            // this tile, then the next one's with a prefetch), so at most
            // depth-2 later stages may be pending.  After the previous tile's
            // epilogue the stores are pending too, behind those loads;
            // counting them out only waits for them as well.
            wait_own(pf ? depth - 2 : min(depth - 2, nst - st - 2));
            ring_barrier();
            // Refill the slot stage st used with stage st + depth; stages
            // past this tile's last are the next tile's.
            auto refill = [&]() {
                if (st + depth < nst) {
                    issue(st + depth, rs);
                } else if (pf) {
                    if (st + depth == nst) use_tile(nx);
                    issue(st + depth - nst, rs);
                }
                rs = (rs + 1 == depth) ? 0 : rs + 1;
            };
            // The weight (B) waves, and the A waves of tiles with a 3-deep A
            // ring (MXFP8 tiles, bf16 160- and 128-row tiles), issue the
            // refill after the MFMA group below: the group then starts at
            // once after the barrier instead of behind the DMA issue.  A
            // waves with a 2-deep ring (bf16 192- to 256-row tiles) refill
            // first: a late issue shortens their one stage of lead.
            // (Measured on MI355X, two interleaved runs each: bf16 long
            // prefill gate|up -4% with the B waves late, against +2% with
            // every wave late; prefill -1.7% more with the 3-deep A waves
            // late; MXFP8 gate|up -4.5% at prefill, -7% skew, -3.5% long
            // prefill.)
            const bool late = !a_role || ast >= 3;  // wave-uniform
            if (!late) refill();
            if constexpr (W8)
                read_b8(bn, raw, sc);
            else
                read_b(bn, 0, bf0);
            read_a(an, 0, 0, af);
            mfma_rows(1, af, bf1);
            if (late) refill();
            read_a(an, 0, 1, af);
            if constexpr (W8) cvt_b8(raw, sc, 0, bf0);
            bs = bn;
            as = an;
        }
        if (nh & 1) {  // half-full last stage (down with I % 64 == 32)
            mfma_rows(0, af, bf0);
            mfma_rows(1, af, bf0);
        }
        if (!pf) {
            // Every wave's reads of the ring are complete before the next
            // tile's loads are requested into it (after the epilogue below).
            __builtin_amdgcn_s_waitcnt(0xc07f);
            ring_barrier();
        }

        // Epilogue.  Lane (l16, g) of wave (wm, wn) holds rows
        // wm*TM/2 + 16i + 4g + r of its MFMA tiles; the row offsets 16i + r are
        // compile-time constants times a uniform pitch.  Without a prefetch
        // the next tile's setup (gate|up's row ids are loads) runs first, so
        // that waiting for those loads does not also wait for this tile's
        // stores to drain.
        const int row0 = wm * (TM / 2) + 4 * g;
        if (more && !pf) setup(wnext);
        if constexpr (MOE_HEAVY_STAGED_EPI != 0 && M == Mode::Down) {
            using S = Staging<M, TM, YF>;
            const int tid = threadIdx.x;
            for (int pass = 0; pass < S::kPasses; ++pass) {
                // 1. this wave's results into the staging rows
                if constexpr (M == Mode::GateUp) {
#pragma unroll
                    for (int i = 0; i < kRF; ++i)
#pragma unroll
                        for (int jp = 0; jp < 2; ++jp)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float hv = swiglu(acc[i][2 * jp][r], acc[i][2 * jp + 1][r]);
                                const uint32_t hi = f32_to_bf16_bits(hv);
                                char* q = lds + (row0 + i * 16 + r) * S::kPitch +
                                          (wn * 32 + jp * 16 + l16) * 2;
                                *reinterpret_cast<uint16_t*>(q) = (uint16_t)hi;
                                if (a.split_h)
                                    *reinterpret_cast<uint16_t*>(q + TM * S::kPitch) =
                                        (uint16_t)f32_to_bf16_bits(hv - bf16_bits_to_f32(hi));
                            }
                } else if constexpr (YF != kYF32) {
                    const int odd = l16 & 1;
#pragma unroll
                    for (int i = 0; i < kRF; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            uint32_t w[2];
                            y16_pairs<YF>(acc[i][j], l16, w[0], w[1]);
#pragma unroll
                            for (int r = 0; r < 2; ++r)
                                *reinterpret_cast<uint32_t*>(
                                    lds + (row0 + 2 * odd + i * 16 + r) * S::kPitch +
                                    (wn * kWTN + j * 16 + l16 - odd) * 2) = w[r];
                        }
                } else {
                    if (wm == pass) {
#pragma unroll
                        for (int i = 0; i < kRF; ++i)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    *reinterpret_cast<float*>(
                                        lds + (4 * g + i * 16 + r) * S::kPitch +
                                        (wn * kWTN + j * 16 + l16) * 4) = acc[i][j][r];
                    }
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);
                ring_barrier();
                // 2. whole-row 16-byte chunks read back and stored with
                // 16-byte lane stores (1 KB of whole lines per instruction)
                const int planes = (M == Mode::GateUp && a.split_h) ? 2 : 1;
                const int prow0 = pass * S::kPassRows;
                for (int pl = 0; pl < planes; ++pl) {
#pragma unroll 4
                    for (int q = 0; q < S::kIters; ++q) {
                        const int c = q * kHeavyThreads + tid;
                        const int row = c / S::kChunks, ch = c % S::kChunks;
                        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
                            lds + pl * TM * S::kPitch + row * S::kPitch + ch * 16);
                        if (prow0 + row >= t_rows) continue;
                        if constexpr (M == Mode::GateUp) {
                            const int col = t_nb * (kTN / 2) + ch * 8;
                            if (col < a.I)
                                *reinterpret_cast<u32x4_t*>(
                                    a.h + (size_t)(t_base + row) * hstride + pl * a.I + col) = v;
                        } else {
                            const int col = t_nb * kTN + ch * (16 / S::kElt);
                            if (col < a.H) {
                                char* yb = static_cast<char*>(a.y) +
                                           ((size_t)(t_base + prow0 + row) * a.H + col) * S::kElt;
                                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(yb));
                            }
                        }
                    }
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);
                ring_barrier();  // staging read: the LDS is free for the next pass / tile
            }
        } else if constexpr (M == Mode::GateUp) {
            const int hc0 = t_nb * (kTN / 2) + wn * 32 + l16;
            uint16_t* hp = a.h + (size_t)(t_base + row0) * hstride + hc0;
            const bool full = t_rows == TM && t_nb * (kTN / 2) + kTN / 2 <= a.I;
            // SwiGLU of every element first, with no branch around it (gate
            // tile 2jp and up tile 2jp+1 hold the same (row, i) in the same
            // lane; h overwrites the gate value), then the stores, each under
            // its row and column predicate.  (Computed under the store's
            // predicate, the per-element branches cost more than the work.)
#pragma unroll
            for (int i = 0; i < kRF; ++i)
#pragma unroll
                for (int jp = 0; jp < 2; ++jp)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[i][2 * jp][r] = swiglu(acc[i][2 * jp][r], acc[i][2 * jp + 1][r]);
#pragma unroll
            for (int i = 0; i < kRF; ++i) {
#pragma unroll
                for (int jp = 0; jp < 2; ++jp) {
                    const bool col_ok = hc0 + jp * 16 < a.I;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int dr = i * 16 + r;
                        if (full || (row0 + dr < t_rows && col_ok)) {
                            const float hv = acc[i][2 * jp][r];
                            const uint32_t hi = f32_to_bf16_bits(hv);
                            uint16_t* q = hp + (size_t)dr * hstride + jp * 16;
                            q[0] = (uint16_t)hi;
                            if (a.split_h)
                                q[a.I] = (uint16_t)f32_to_bf16_bits(hv - bf16_bits_to_f32(hi));
                        }
                    }
                }
            }
        } else if constexpr (YF != kYF32) {
            // 16-bit y: lanes of adjacent columns pair up (y16_pairs), so
            // each lane writes 2 rows x 2 columns as two 32-bit words.
            const int odd = l16 & 1;
            const int c0 = t_nb * kTN + wn * kWTN + l16 - odd;  // even
            uint32_t* yp = static_cast<uint32_t*>(a.y) +
                           ((size_t)(t_base + row0 + 2 * odd) * a.H + c0) / 2;
            const bool full = t_rows == TM && t_nb * kTN + kTN <= a.H;
#pragma unroll
            for (int i = 0; i < kRF; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t w[2];
                    y16_pairs<YF>(acc[i][j], l16, w[0], w[1]);
                    const bool col_ok = c0 + j * 16 < a.H;
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int dr = i * 16 + r;
                        if (full || (row0 + 2 * odd + dr < t_rows && col_ok))
                            yp[((size_t)dr * a.H + j * 16) / 2] = w[r];
                    }
                }
            }
        } else {
            const int c0 = t_nb * kTN + wn * kWTN + l16;
            float* yp = static_cast<float*>(a.y) + (size_t)(t_base + row0) * a.H + c0;
            const bool full = t_rows == TM && t_nb * kTN + kTN <= a.H;
#pragma unroll
            for (int i = 0; i < kRF; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool col_ok = c0 + j * 16 < a.H;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int dr = i * 16 + r;
                        if (full || (row0 + dr < t_rows && col_ok))
                            yp[(size_t)dr * a.H + j * 16] = acc[i][j][r];
                    }
                }
            }
        }

        wi = wnext;
        if (!more) break;
        primed = pf;
        if (!pf) {
            as = bs = rs = 0;
            issue_first();
        }
    }
    return wi;
}

// One launch per GEMM: every row tile runs with the body of its own height
// (the plan mixes heights within an expert); the bodies share one LDS
// allocation, the largest ring.
template <Mode M, int YF, int BS>
__global__ __launch_bounds__(kHeavyThreads) void ffn_heavy_kernel(FfnArgs a) {
    __shared__ __attribute__((aligned(1024))) char lds[kHeavyLds];
    const int N = (M == Mode::GateUp) ? 2 * a.I : a.H;
    const int nblk = (N + kTN - 1) / kTN;
    const int ntiles = a.plan ? a.plan[1] : (a.dense_rows + a.dense_tm - 1) / a.dense_tm;
    const long long nwork = (long long)ntiles * nblk;

    // XCD-aware static schedule.  The work list is tile-major (tiles of one
    // expert are adjacent) with the N block fastest; it is cut into nslice
    // contiguous slices and slice x is served, round-robin, by the blocks that
    // share XCD x (blockIdx % nslice), so the M and N tiles of one expert run
    // at the same time on one XCD and share weights and rows through its L2.
    const int nslice = min(kXcds, (int)gridDim.x);
    const int xs = blockIdx.x % nslice;
    const int nb_x = ((int)gridDim.x - xs + nslice - 1) / nslice;
    const int jx = blockIdx.x / nslice;
    long long wbeg, wend;
    if (a.plan && nslice == kXcds) {
        // slices of about equal cost from the plan (tile heights differ)
        wbeg = (long long)a.plan[kPlanXcdBounds + xs] * nblk;
        wend = (long long)a.plan[kPlanXcdBounds + xs + 1] * nblk;
    } else {
        const long long per = (nwork + nslice - 1) / nslice;
        wbeg = xs * per;
        wend = min(nwork, wbeg + per);
    }

    long long wi = wbeg + jx;
    while (wi < wend) {
        int nb_i;
        const int tmi = tile_tmi(a, item_tile<M>(a, wi, nblk, nb_i));
        if constexpr (BS == kBRecMx) {
            // MXFP8 plans hold tiles of at most 192 rows (the larger bodies
            // spill); the host rejects a forced 224 or 256 with MXFP8 weights.
            if (tmi == 2)
                wi = ffn_heavy_run<M, 192, YF, BS>(a, lds, wi, wend, nb_x, nblk);
            else if (tmi == 3)
                wi = ffn_heavy_run<M, 160, YF, BS>(a, lds, wi, wend, nb_x, nblk);
            else if (tmi == 4)
                wi = ffn_heavy_run<M, 128, YF, BS>(a, lds, wi, wend, nb_x, nblk);
            else
                wi = wend;
        } else {
            if (tmi == 0)
                wi = ffn_heavy_run<M, 256, YF, BS>(a, lds, wi, wend, nb_x, nblk);
            else if (tmi == 1)
                wi = ffn_heavy_run<M, 224, YF, BS>(a, lds, wi, wend, nb_x, nblk);
            else if (tmi == 2)
                wi = ffn_heavy_run<M, 192, YF, BS>(a, lds, wi, wend, nb_x, nblk);
            else if (tmi == 3)
                wi = ffn_heavy_run<M, 160, YF, BS>(a, lds, wi, wend, nb_x, nblk);
            else
                wi = ffn_heavy_run<M, 128, YF, BS>(a, lds, wi, wend, nb_x, nblk);
        }
    }
}

int grid_for(long long work, int per_cu, int num_cu) {
    return (int)std::max<long long>(1, std::min<long long>(work, (long long)per_cu * num_cu));
}

// Packed bf16 records (layout in launch.h): one thread per 16-byte unit u
// of the output, unit u % 2048 of record u / 2048 = lane L of chunk h of
// row block j (u % 2048 = 128 j + 64 h + L): tile row rr = 16 j + L % 16,
// K values 64 c + 32 h + 8 (L / 16) .. +7 of the weight row it stands for
// (gate|up: h column nb*128 + 16*(rr/32) + rr%16, gate row where rr % 32 <
// 16, else the up row; down: W_down row nb*256 + rr), zero past the weights.
template <bool kGateUp>
__global__ __launch_bounds__(256) void pack_rec_kernel(const uint16_t* __restrict__ w, int E,
                                                       int rows_per, int K, int I, int nblk,
                                                       int nchunks, uint16_t* __restrict__ out) {
    const long long nunits = (long long)E * nblk * nchunks * 2048;
    for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < nunits;
         u += (long long)gridDim.x * blockDim.x) {
        const int q = (int)(u & 2047);
        const int L = q & 63, half = (q >> 6) & 1, j = q >> 7;
        const int rr = 16 * j + (L & 15);
        const long long rec = u >> 11;
        const int c = (int)(rec % nchunks);
        const long long enb = rec / nchunks;
        const int nb = (int)(enb % nblk), e = (int)(enb / nblk);
        int row;
        bool valid;
        if (kGateUp) {
            const int hc = nb * 128 + (rr >> 5) * 16 + (rr & 15);
            valid = hc < I;
            row = ((rr & 16) == 0) ? hc : I + hc;
        } else {
            row = nb * 256 + rr;
            valid = row < rows_per;
        }
        u32x4_t v = {0u, 0u, 0u, 0u};
        const int k0 = 64 * c + 32 * half + 8 * (L >> 4);
        if (valid && k0 < K)  // K % 32 == 0: a unit is all in or all out
            v = *reinterpret_cast<const u32x4_t*>(w + ((long long)e * rows_per + row) * K + k0);
        *reinterpret_cast<u32x4_t*>(out + u * 8) = v;
    }
}

// Upper bound on the heavy kernels' grid (0: none).  A small cap makes every
// block run many work items in a row, which is how the cross-tile paths
// (same-height chaining, the down GEMM's prefetch of the next tile) are put
// under test on small shapes; the default build leaves it off.
#ifndef MOE_HEAVY_MAX_GRID
#define MOE_HEAVY_MAX_GRID 0
#endif
int heavy_grid(long long work, int num_cu) {
    const int g = grid_for(work, 1, num_cu);
    return MOE_HEAVY_MAX_GRID > 0 ? std::min(g, MOE_HEAVY_MAX_GRID) : g;
}

// Heavy tiles of one GEMM: one launch, one block per CU (the tile heights are
// the plan's, read on the device); a dense group has one height.
template <Mode M, int YF>
hipError_t launch_heavy(const FfnArgs& a, int ncols, hipStream_t st) {
    const long long nblk = (ncols + kTN - 1) / kTN;
    if (a.plan) {
        if (a.max_tiles <= 0) return hipSuccess;
        const int grid = heavy_grid((long long)a.max_tiles * nblk, a.num_cu);
        if (a.w_mxfp8)
            ffn_heavy_kernel<M, YF, kBRecMx><<<grid, kHeavyThreads, 0, st>>>(a);
        else if (a.hr_gu)
            ffn_heavy_kernel<M, YF, kBRec16><<<grid, kHeavyThreads, 0, st>>>(a);
        else
            ffn_heavy_kernel<M, YF, kBRowMajor><<<grid, kHeavyThreads, 0, st>>>(a);
        return hipGetLastError();
    }
    if (a.dense_rows <= 0) return hipSuccess;
    const long long tiles = (a.dense_rows + a.dense_tm - 1) / a.dense_tm;
    const int grid = heavy_grid(tiles * nblk, a.num_cu);
    if (!valid_tile_height(a.dense_tm)) return hipErrorInvalidValue;
    ffn_heavy_kernel<M, YF, kBRowMajor><<<grid, kHeavyThreads, 0, st>>>(a);  // dense groups
    return hipGetLastError();
}

}  // namespace

size_t rec16_gu_bytes(int E, int H, int I) {
    return (size_t)E * rec_tiles(2 * I) * mx_chunks(H) * kRec16Bytes;
}

size_t rec16_dn_bytes(int E, int H, int I) {
    return (size_t)E * rec_tiles(H) * mx_chunks(I) * kRec16Bytes;
}

hipError_t launch_pack_weights(const uint16_t* w_gu, const uint16_t* w_dn, int E, int H, int I,
                               char* packed, hipStream_t st) {
    const int nbg = rec_tiles(2 * I), nbd = rec_tiles(H);
    const long long ug = (long long)E * nbg * mx_chunks(H) * 2048;
    const long long ud = (long long)E * nbd * mx_chunks(I) * 2048;
    pack_rec_kernel<true><<<(int)std::min<long long>((ug + 255) / 256, 65536), 256, 0, st>>>(
        w_gu, E, 2 * I, H, I, nbg, mx_chunks(H), reinterpret_cast<uint16_t*>(packed));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    pack_rec_kernel<false><<<(int)std::min<long long>((ud + 255) / 256, 65536), 256, 0, st>>>(
        w_dn, E, H, I, I, nbd, mx_chunks(I),
        reinterpret_cast<uint16_t*>(packed + rec16_gu_bytes(E, H, I)));
    return hipGetLastError();
}

hipError_t launch_ffn_plan(const int32_t* offsets, int E, int light_max, int force_tm,
                           int round_tiles, int32_t* plan, int32_t* sync, hipStream_t st) {
    prof_begin(K_FFN_PLAN, st);
    ffn_plan_kernel<<<1, 1024, 0, st>>>(offsets, E, light_max, force_tm, round_tiles, plan, sync);
    prof_end(K_FFN_PLAN, st);
    return hipGetLastError();
}

// The fused light loop replaces the two light launches for bf16 weights
// when the counters are given and the ticket range fits 32 bits.
static bool use_fused_light(const FfnArgs& a) {
    if (!MOE_FUSED_LIGHT || !a.sync || !a.plan || a.max_light <= 0 || a.w_mxfp8) return false;
    const long long items = (long long)a.max_light *
                            ((a.I + 63) / 64 + (a.H + 4 * MOE_LIGHT_DN_TILES * 16 - 1) /
                                                   (4 * MOE_LIGHT_DN_TILES * 16));
    return items + (long long)MOE_FUSED_BPC * a.num_cu < (1LL << 31);
}

hipError_t launch_ffn_gateup(const FfnArgs& a, hipStream_t st) {
    if (use_fused_light(a)) {
        const long long work = (long long)a.max_light *
                               ((a.I + 63) / 64 + (a.H + 4 * MOE_LIGHT_DN_TILES * 16 - 1) /
                                                      (4 * MOE_LIGHT_DN_TILES * 16));
        const int grid = grid_for(work, MOE_FUSED_BPC, a.num_cu);
        prof_begin(K_GATEUP_LIGHT, st);
        if (a.hr_gu)
            light_fused_kernel<MOE_LIGHT_GU_U, MOE_LIGHT_DN_TILES, MOE_LIGHT_DN_U,
                               MOE_LIGHT_NT_LOADS != 0, true><<<grid, kThreads, 0, st>>>(a);
        else
            light_fused_kernel<MOE_LIGHT_GU_U, MOE_LIGHT_DN_TILES, MOE_LIGHT_DN_U,
                               MOE_LIGHT_NT_LOADS != 0, false><<<grid, kThreads, 0, st>>>(a);
        prof_end(K_GATEUP_LIGHT, st);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    } else if (a.plan && a.max_light > 0) {
        const int kCols = a.w_mxfp8 ? 4 * MOE_LIGHT_MX_GU_TILES * 8 : 4 * 16;
        const long long work = (long long)a.max_light * ((a.I + kCols - 1) / kCols);
        prof_begin(K_GATEUP_LIGHT, st);
        const int grid =
            grid_for(work, a.w_mxfp8 ? MOE_LIGHT_MX_GU_BPC : MOE_LIGHT_GU_BPC, a.num_cu);
        if (a.w_mxfp8)
            gateup_light_mx_kernel<MOE_LIGHT_MX_GU_U, MOE_LIGHT_MX_GU_TILES>
                <<<grid, kThreads, 0, st>>>(a);
        else if (a.hr_gu)
            gateup_light_kernel<MOE_LIGHT_GU_U, MOE_LIGHT_NT_LOADS != 0, true>
                <<<grid, kThreads, 0, st>>>(a);
        else
            gateup_light_kernel<MOE_LIGHT_GU_U, MOE_LIGHT_NT_LOADS != 0, false>
                <<<grid, kThreads, 0, st>>>(a);
        prof_end(K_GATEUP_LIGHT, st);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if ((a.plan && a.max_tiles > 0) || (!a.plan && a.dense_rows > 0)) {
        prof_begin(K_GATEUP_HEAVY, st);
        hipError_t err = launch_heavy<Mode::GateUp, kYF32>(a, 2 * a.I, st);
        prof_end(K_GATEUP_HEAVY, st);
        return err;
    }
    return hipSuccess;
}

hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t st) {
    if (a.plan && a.max_light > 0 && !use_fused_light(a)) {
        const int kCols = 4 * (a.w_mxfp8 ? MOE_LIGHT_MX_DN_TILES : MOE_LIGHT_DN_TILES) * 16;
        const long long work = (long long)a.max_light * ((a.H + kCols - 1) / kCols);
        prof_begin(K_DOWN_LIGHT, st);
        const int grid =
            grid_for(work, a.w_mxfp8 ? MOE_LIGHT_MX_DN_BPC : MOE_LIGHT_DN_BPC, a.num_cu);
        if (a.w_mxfp8)
            down_light_mx_kernel<MOE_LIGHT_MX_DN_TILES, MOE_LIGHT_MX_DN_U>
                <<<grid, kThreads, 0, st>>>(a);
        else if (a.hr_dn)
            down_light_kernel<MOE_LIGHT_DN_TILES, MOE_LIGHT_DN_U, MOE_LIGHT_NT_LOADS != 0, true>
                <<<grid, kThreads, 0, st>>>(a);
        else
            down_light_kernel<MOE_LIGHT_DN_TILES, MOE_LIGHT_DN_U, MOE_LIGHT_NT_LOADS != 0, false>
                <<<grid, kThreads, 0, st>>>(a);
        prof_end(K_DOWN_LIGHT, st);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if ((a.plan && a.max_tiles > 0) || (!a.plan && a.dense_rows > 0)) {
        prof_begin(K_DOWN_HEAVY, st);
        hipError_t err = a.y_fmt == kYBF16  ? launch_heavy<Mode::Down, kYBF16>(a, a.H, st)
                         : a.y_fmt == kYF16 ? launch_heavy<Mode::Down, kYF16>(a, a.H, st)
                                            : launch_heavy<Mode::Down, kYF32>(a, a.H, st);
        prof_end(K_DOWN_HEAVY, st);
        return err;
    }
    return hipSuccess;
}

}  // namespace moe
