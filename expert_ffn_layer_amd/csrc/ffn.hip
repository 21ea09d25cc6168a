// Grouped expert FFN on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
//   gate|up:  h[r, i] = bf16( silu(x[tok_r] . Wg[e,i]) * (x[tok_r] . Wu[e,i]) )
//   down:     y[r, c] = h[r] . Wd[e,c]            (fp32)
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
//    straight from HBM into registers and keeps one accumulator per 16-row
//    sub-tile.  This is the decode path: it is bound by weight bytes.
//  * heavy: 128x128 output tiles, A and B staged through double-buffered LDS,
//    row sub-tiles past the expert's count skipped.
// Both paths give every output element the same chain of MFMAs over K in
// ascending 32-wide steps with the same K-slot assignment, and the same
// epilogue, so a row's h and y are bitwise identical whichever loop ran it.
//
// gate|up column pairing: every 16-column MFMA tile holds 8 gate rows and the
// 8 matching up rows of W_gate_up, so lane n (n < 8) and lane n+8 carry g_i
// and u_i of the same i and the SwiGLU epilogue is one lane shuffle.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {

int max_heavy_tiles(long long A, int E, int light_max) {
    // sum over heavy experts of ceil(n_e / BM) <= A / BM + (#heavy experts)
    const long long heavy = std::min<long long>(E, A / (light_max + 1));
    return (int)std::min<long long>(A / kHeavyBM + heavy + 1, A + 1);
}

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- plan
// One block, one thread per expert: compact the light experts (ascending id)
// and the heavy experts' row tiles (ascending id, then first row).
__global__ __launch_bounds__(1024) void ffn_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int E, int light_max,
                                                        int32_t* __restrict__ plan) {
    __shared__ int wl[16], wt[16];
    const int e = threadIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    const int is_light = (n >= 1 && n <= light_max) ? 1 : 0;
    const int nt = (n > light_max) ? (n + kHeavyBM - 1) / kHeavyBM : 0;
    int il = is_light, it = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int vl = __shfl_up(il, o, 64);
        const int vt = __shfl_up(it, o, 64);
        if (lane >= o) {
            il += vl;
            it += vt;
        }
    }
    if (lane == 63) {
        wl[wave] = il;
        wt[wave] = it;
    }
    __syncthreads();
    int bl = 0, bt = 0;
    for (int w = 0; w < wave; ++w) {
        bl += wl[w];
        bt += wt[w];
    }
    const int el = bl + il - is_light, et = bt + it - nt;
    if (is_light) plan[kPlanHeader + el] = e;
    int32_t* tiles = plan + kPlanHeader + E;
    for (int i = 0; i < nt; ++i) {
        tiles[2 * (et + i)] = e;
        tiles[2 * (et + i) + 1] = i * kHeavyBM;
    }
    if (threadIdx.x == blockDim.x - 1) {
        plan[0] = el + is_light;
        plan[1] = et + nt;
    }
}

// Tunables of the light loops (compile-time; the defaults are the measured best).
#ifndef MOE_LIGHT_GU_U
#define MOE_LIGHT_GU_U 8        // K steps of 32 in flight per wave (gate|up)
#endif
#ifndef MOE_LIGHT_GU_TILES
#define MOE_LIGHT_GU_TILES 1    // 16-column MFMA tiles per wave (8 h-columns each)
#endif
#ifndef MOE_LIGHT_GU_BPC
#define MOE_LIGHT_GU_BPC 8      // blocks per CU in the grid
#endif
#ifndef MOE_LIGHT_DN_U
#define MOE_LIGHT_DN_U 4
#endif
#ifndef MOE_LIGHT_DN_TILES
#define MOE_LIGHT_DN_TILES 2
#endif
#ifndef MOE_LIGHT_DN_BPC
#define MOE_LIGHT_DN_BPC 8
#endif
#ifndef MOE_LIGHT_NT_LOADS
#define MOE_LIGHT_NT_LOADS 0    // 1: weights streamed with non-temporal loads
#endif

// Expert weights are read once per step: optionally bypass cache retention.
template <bool kNonTemporal>
__device__ __forceinline__ bf16x8_t load_weights(const uint16_t* p) {
    if constexpr (kNonTemporal)
        return __builtin_bit_cast(bf16x8_t,
                                  __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
    else
        return load_bf16x8(p);
}

// Row sub-tiles of the light loop: experts with up to 16 rows run one 16-row
// MFMA tile with deep weight prefetch; experts with 17..64 rows run four
// sub-tiles (those past the row count skipped) with shallower prefetch, so
// both branches fit the same register budget.
constexpr int kLightSubTiles = kLightRowsMax / 16;  // 4
constexpr int kLightWideU = 2;                      // K steps in flight, wide branch

// ------------------------------------------------------- light: gate|up
// One wave: MT row sub-tiles x NTILE column tiles of one expert, K = H.
// Tile t pairs gate rows i0+8t.. and the matching up rows, so lanes
// l16 < 8 end with g and lanes l16 >= 8 with u of the same h column.
template <int MT, int U, int NTILE, bool NTL>
__device__ __forceinline__ void gateup_light_rows(const FfnArgs& a, int e, int r0, int n, int i0,
                                                  int l16, int g) {
    const int nk = a.H / 32;
    const int wrow = (l16 < 8) ? (i0 + l16) : (a.I + i0 + l16 - 8);
    const uint16_t* Bp = a.w_gu + ((size_t)e * 2 * a.I + wrow) * a.H + 8 * g;
    const size_t bstride = (size_t)8 * a.H;  // next column tile: 8 rows further
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

    floatx4_t acc[MT][NTILE];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NTILE; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t ca[U][MT], cb[U][NTILE];
    auto load_step = [&](int kb, bf16x8_t (&aa)[MT], bf16x8_t (&bb)[NTILE]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) aa[m] = zero_bf16x8();
#pragma unroll
        for (int t = 0; t < NTILE; ++t) bb[t] = zero_bf16x8();
        if (kb < nk) {
#pragma unroll
            for (int t = 0; t < NTILE; ++t) bb[t] = load_weights<NTL>(Bp + t * bstride + kb * 32);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (has_a[m]) aa[m] = load_bf16x8(Ap[m] + kb * 32);
        }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) load_step(u, ca[u], cb[u]);
    for (int k0 = 0; k0 < nk; k0 += U) {
        bf16x8_t na[U][MT], nb_[U][NTILE];
#pragma unroll
        for (int u = 0; u < U; ++u) load_step(k0 + U + u, na[u], nb_[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (k0 + u < nk) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < mt_live) {
#pragma unroll
                        for (int t = 0; t < NTILE; ++t)
                            acc[m][t] = mfma_16x16x32(ca[u][m], cb[u][t], acc[m][t]);
                    }
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < MT; ++m) ca[u][m] = na[u][m];
#pragma unroll
            for (int t = 0; t < NTILE; ++t) cb[u][t] = nb_[u][t];
        }
    }
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

// Work item = (light expert, 4 waves x NTILE x 8 h-columns).
template <int U, int NTILE, bool NTL>
__global__ __launch_bounds__(kThreads) void gateup_light_kernel(FfnArgs a) {
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
        if (n <= 16)
            gateup_light_rows<1, U, NTILE, NTL>(a, e, r0, n, i0, l16, g);
        else
            gateup_light_rows<kLightSubTiles, kLightWideU, NTILE, NTL>(a, e, r0, n, i0, l16, g);
    }
}

// --------------------------------------------------------- light: down
// One wave: MT row sub-tiles x NT column tiles (16 output columns each), K = I.
template <int MT, int U, int NT, bool NTL>
__device__ __forceinline__ void down_light_rows(const FfnArgs& a, int e, int r0, int n, int c0,
                                                int l16, int g) {
    const int nk = a.I / 32;
    const uint16_t* Bp = a.w_dn + ((size_t)e * a.H + c0 + l16) * a.I + 8 * g;
    const size_t bstride = (size_t)16 * a.I;
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
            for (int t = 0; t < NT; ++t) bb[t] = load_weights<NTL>(Bp + t * bstride + kb * 32);
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
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int c = c0 + t * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m * 16 + 4 * g + r;
                if (row < n) a.y[(size_t)(r0 + row) * a.H + c] = acc[m][t][r];
            }
        }
    }
}

// Work item = (light expert, 4 waves x NT x 16 output columns).
template <int NT, int U, bool NTL>
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
            down_light_rows<1, U, NT, NTL>(a, e, r0, n, c0, l16, g);
        else
            down_light_rows<kLightSubTiles, kLightWideU, NT, NTL>(a, e, r0, n, c0, l16, g);
    }
}

// ---------------------------------------------------------------- heavy
enum class Mode { GateUp, Down };

constexpr int HBM_ = kHeavyBM;  // 128 rows
constexpr int HBN = 128;        // B rows (output columns, or gate+up rows)
constexpr int HBK = 64;         // K per LDS stage
constexpr int HLDK = HBK + 8;   // padded LDS row (bf16)

template <Mode M>
__global__ __launch_bounds__(kThreads) void ffn_heavy_kernel(FfnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][HBM_][HLDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][HBN][HLDK];

    const int N = (M == Mode::GateUp) ? 2 * a.I : a.H;
    // split_h: the down GEMM's K runs over [hi | lo] (2I) against W_down twice.
    const int K = (M == Mode::GateUp) ? a.H : (a.split_h ? 2 * a.I : a.I);
    const int hstride = a.split_h ? 2 * a.I : a.I;  // row pitch of h
    const int nblk = (N + HBN - 1) / HBN;
    const int ntiles = a.plan ? a.plan[1] : (a.dense_rows + HBM_ - 1) / HBM_;
    const long long nwork = (long long)ntiles * nblk;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l16 = lane & 15, g = lane >> 4;
    const int nst = (K + HBK - 1) / HBK;
    // global->LDS copy: thread covers rows (tid/8) + 32q, 16 bytes at (tid%8)*8
    const int ld_row = tid >> 3, ld_k = (tid & 7) * 8;

    for (long long wi = blockIdx.x; wi < nwork; wi += gridDim.x) {
        const int tile = (int)(wi / nblk), nb = (int)(wi % nblk);
        int e, r0, m0, rows;
        if (a.plan) {
            const int32_t* tl = a.plan + kPlanHeader + a.E;
            e = tl[2 * tile];
            m0 = tl[2 * tile + 1];
            r0 = a.offsets[e];
            rows = min(HBM_, a.offsets[e + 1] - r0 - m0);
        } else {
            e = 0;
            r0 = 0;
            m0 = tile * HBM_;
            rows = min(HBM_, a.dense_rows - m0);
        }

        const uint16_t* arow[4];
        const uint16_t* brow[4];
        bool aok[4], bok[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ld_row + 32 * q;
            aok[q] = r < rows;
            const int rr = aok[q] ? r : 0;
            if (M == Mode::GateUp) {
                const int tok = a.sorted_ids ? a.sorted_ids[r0 + m0 + rr] : r0 + m0 + rr;
                arow[q] = a.x + (size_t)tok * a.H + ld_k;
                const int hc = nb * (HBN / 2) + (r >> 4) * 8 + (r & 7);
                bok[q] = hc < a.I;
                const int wr = ((r & 15) < 8) ? hc : a.I + hc;
                brow[q] = a.w_gu + ((size_t)e * 2 * a.I + (bok[q] ? wr : 0)) * a.H + ld_k;
            } else {
                arow[q] = a.h + (size_t)(r0 + m0 + rr) * hstride + ld_k;
                const int c = nb * HBN + r;
                bok[q] = c < a.H;
                brow[q] = a.w_dn + ((size_t)e * a.H + (bok[q] ? c : 0)) * a.I + ld_k;
            }
        }

        u32x4_t ra[4], rb[4];
        auto gload = [&](int st) {
            const int kk = st * HBK;
            const bool kin = kk + ld_k < K;
            // down with split_h: K columns past I wrap back onto W_down
            const int kb = (M == Mode::Down && kk + ld_k >= a.I) ? kk - a.I : kk;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                ra[q] = (aok[q] && kin) ? *reinterpret_cast<const u32x4_t*>(arow[q] + kk)
                                        : u32x4_t{0u, 0u, 0u, 0u};
                rb[q] = (bok[q] && kin) ? *reinterpret_cast<const u32x4_t*>(brow[q] + kb)
                                        : u32x4_t{0u, 0u, 0u, 0u};
            }
        };
        auto sstore = [&](int buf) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                *reinterpret_cast<u32x4_t*>(&As[buf][ld_row + 32 * q][ld_k]) = ra[q];
                *reinterpret_cast<u32x4_t*>(&Bs[buf][ld_row + 32 * q][ld_k]) = rb[q];
            }
        };

        floatx4_t acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        // row sub-tiles of this wave that hold any of the tile's rows
        const int mt_live = max(0, min(4, (rows - wm * 64 + 15) / 16));

        gload(0);
        sstore(0);
        __syncthreads();
        for (int st = 0; st < nst; ++st) {
            const int buf = st & 1;
            if (st + 1 < nst) gload(st + 1);
#pragma unroll
            for (int kk = 0; kk < HBK / 32; ++kk) {
                if (st * HBK + kk * 32 < K) {
                    bf16x8_t af[4], bfr[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        bfr[j] = __builtin_bit_cast(
                            bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                          &Bs[buf][wn * 64 + j * 16 + l16][kk * 32 + 8 * g]));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (i < mt_live) {
                            af[i] = __builtin_bit_cast(
                                bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                              &As[buf][wm * 64 + i * 16 + l16][kk * 32 + 8 * g]));
#pragma unroll
                            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
                        }
                    }
                }
            }
            if (st + 1 < nst) sstore(buf ^ 1);
            __syncthreads();
        }

        // epilogue
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm * 64 + i * 16 + 4 * g + r;
                    const float v = acc[i][j][r];
                    if (M == Mode::GateUp) {
                        const float up = __shfl_down(v, 8, 64);
                        const int hc = nb * (HBN / 2) + (wn * 4 + j) * 8 + l16;
                        if (l16 < 8 && row < rows && hc < a.I) {
                            const float hv = swiglu(v, up);
                            const uint32_t hi = f32_to_bf16_bits(hv);
                            uint16_t* hr = a.h + (size_t)(r0 + m0 + row) * hstride;
                            hr[hc] = (uint16_t)hi;
                            if (a.split_h)
                                hr[a.I + hc] = (uint16_t)f32_to_bf16_bits(hv - bf16_bits_to_f32(hi));
                        }
                    } else {
                        const int c = nb * HBN + wn * 64 + j * 16 + l16;
                        if (row < rows && c < a.H) a.y[(size_t)(r0 + m0 + row) * a.H + c] = v;
                    }
                }
            }
        }
    }
}

int grid_for(long long work, int per_cu, int num_cu) {
    return (int)std::max<long long>(1, std::min<long long>(work, (long long)per_cu * num_cu));
}

}  // namespace

hipError_t launch_ffn_plan(const int32_t* offsets, int E, int light_max, int32_t* plan,
                           hipStream_t st) {
    prof_begin(K_FFN_PLAN, st);
    ffn_plan_kernel<<<1, 1024, 0, st>>>(offsets, E, light_max, plan);
    prof_end(K_FFN_PLAN, st);
    return hipGetLastError();
}

hipError_t launch_ffn_gateup(const FfnArgs& a, hipStream_t st) {
    if (a.plan && a.max_light > 0) {
        constexpr int kCols = 4 * MOE_LIGHT_GU_TILES * 8;
        const long long work = (long long)a.max_light * ((a.I + kCols - 1) / kCols);
        prof_begin(K_GATEUP_LIGHT, st);
        gateup_light_kernel<MOE_LIGHT_GU_U, MOE_LIGHT_GU_TILES, MOE_LIGHT_NT_LOADS != 0>
            <<<grid_for(work, MOE_LIGHT_GU_BPC, a.num_cu), kThreads, 0, st>>>(a);
        prof_end(K_GATEUP_LIGHT, st);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const long long tiles = a.plan ? a.max_tiles : (a.dense_rows + HBM_ - 1) / HBM_;
    const long long work = tiles * ((2 * a.I + HBN - 1) / HBN);
    if (work > 0) {
        prof_begin(K_GATEUP_HEAVY, st);
        ffn_heavy_kernel<Mode::GateUp><<<grid_for(work, 2, a.num_cu), kThreads, 0, st>>>(a);
        prof_end(K_GATEUP_HEAVY, st);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t st) {
    if (a.plan && a.max_light > 0) {
        constexpr int kCols = 4 * MOE_LIGHT_DN_TILES * 16;
        const long long work = (long long)a.max_light * ((a.H + kCols - 1) / kCols);
        prof_begin(K_DOWN_LIGHT, st);
        down_light_kernel<MOE_LIGHT_DN_TILES, MOE_LIGHT_DN_U, MOE_LIGHT_NT_LOADS != 0>
            <<<grid_for(work, MOE_LIGHT_DN_BPC, a.num_cu), kThreads, 0, st>>>(a);
        prof_end(K_DOWN_LIGHT, st);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const long long tiles = a.plan ? a.max_tiles : (a.dense_rows + HBM_ - 1) / HBM_;
    const long long work = tiles * ((a.H + HBN - 1) / HBN);
    if (work > 0) {
        prof_begin(K_DOWN_HEAVY, st);
        ffn_heavy_kernel<Mode::Down><<<grid_for(work, 2, a.num_cu), kThreads, 0, st>>>(a);
        prof_end(K_DOWN_HEAVY, st);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace moe
