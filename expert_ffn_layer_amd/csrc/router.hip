// Router: fp32 gate GEMM on MFMA, then a wave-per-token softmax and
// register top-k.
//
// The pages compute the router logits on the matrix unit and hand them to
// the vector unit for top_k, and name the hand-off as a serialisation point
// they plan to remove by fusing the two (pwwt.cn article on Qwen 3.5-397B
// MoE on Ironwood, section 8.2).  Here the GEMM writes per-split partial
// logits and one short kernel reduces them in a fixed order and selects;
// the logits never round-trip through a separate softmax or sort pass.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int BT = kRouterBT;
constexpr int BE = kRouterBE;
constexpr int BK = kRouterBK;
constexpr int PAD = 16;  // floats; spreads consecutive K rows over the LDS banks

// part[s][t][e] for one 128x128 (token x expert) tile and one hidden slice.
// 256 threads = 4 waves in a 2x2 grid, each a 64x64 block of 16x16 MFMA
// tiles (v_mfma_f32_16x16x4_f32: lane l gives A[l%16][l/16], B[l/16][l%16]).
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wg,
                                                          float* __restrict__ part, int T,
                                                          int H, int E, int k_per_split) {
    __shared__ __attribute__((aligned(16))) float xs[BK][BT + PAD];
    __shared__ __attribute__((aligned(16))) float ws[BK][BE + PAD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l16 = lane & 15, g = lane >> 4;
    const int e0 = blockIdx.x * BE;
    const int t0 = blockIdx.y * BT;
    const int s = blockIdx.z;
    const int kbeg = s * k_per_split;
    const int kend = kbeg + k_per_split;
    const bool e_vec = (E % 4) == 0;

    // Register staging of one K stage: 2 x-chunks (8 bf16) and 4 wg float4.
    u32x4_t xr[2];
    float4 wr[4];

    auto load_stage = [&](int k0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + 256 * q;
            const int t = c >> 2, kc = (c & 3) * 8;
            if (t0 + t < T)
                xr[q] = *reinterpret_cast<const u32x4_t*>(x + (size_t)(t0 + t) * H + k0 + kc);
            else
                xr[q] = u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = tid + 256 * q;
            const int kk = c >> 5, e4 = (c & 31) * 4;
            const float* src = wg + (size_t)(k0 + kk) * E + e0 + e4;
            if (e_vec && e0 + e4 + 3 < E) {
                wr[q] = *reinterpret_cast<const float4*>(src);
            } else {
                wr[q].x = (e0 + e4 + 0 < E) ? src[0] : 0.f;
                wr[q].y = (e0 + e4 + 1 < E) ? src[1] : 0.f;
                wr[q].z = (e0 + e4 + 2 < E) ? src[2] : 0.f;
                wr[q].w = (e0 + e4 + 3 < E) ? src[3] : 0.f;
            }
        }
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + 256 * q;
            const int t = c >> 2, kc = (c & 3) * 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xs[kc + 2 * j][t] = bf16_bits_to_f32(xr[q][j] & 0xffffu);
                xs[kc + 2 * j + 1][t] = bf16_bits_to_f32(xr[q][j] >> 16);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = tid + 256 * q;
            const int kk = c >> 5, e4 = (c & 31) * 4;
            *reinterpret_cast<float4*>(&ws[kk][e4]) = wr[q];
        }
    };

    floatx4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    load_stage(kbeg);
    store_stage();
    __syncthreads();
    for (int k0 = kbeg; k0 < kend; k0 += BK) {
        const bool more = k0 + BK < kend;
        if (more) load_stage(k0 + BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 4) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk + g][wm * 64 + i * 16 + l16];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[kk + g][wn * 64 + j * 16 + l16];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
        if (more) {
            store_stage();
            __syncthreads();
        }
    }

    float* out = part + (size_t)s * T * E;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + wn * 64 + j * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + wm * 64 + i * 16 + 4 * g + r;
                if (t < T && e < E) out[(size_t)t * E + e] = acc[i][j][r];
            }
        }
    }
}

constexpr int kMaxPerLane = 16;  // E <= 1024 = 16 * 64

// One 256-thread block per token.  All threads reduce the split partials
// (ascending split order) and add the bias into LDS; wave 0 then runs the
// softmax over E and k rounds of a wave-wide argmax over (probability,
// -expert id) keys held in registers.  Any k <= 32 works without padding k
// to a power of 2.
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ part, int splits, const float* __restrict__ bias, int T, int E,
    int k, int renorm, int32_t* __restrict__ ids, float* __restrict__ w_out,
    float* __restrict__ probs) {
    __shared__ float lg[64 * kMaxPerLane];
    const int t = blockIdx.x;
    const size_t plane = (size_t)T * E;
    // Each thread owns experts tid + 256q (q < 4, E <= 1024); 8 splits of
    // each are loaded together, then added in ascending split order.
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += 8) {
        float v[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = threadIdx.x + 256 * q;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[q][u] = (e < E && s0 + u < splits)
                              ? part[(size_t)(s0 + u) * plane + (size_t)t * E + e]
                              : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < splits) acc[q] += v[q][u];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = threadIdx.x + 256 * q;
        if (e < E) {
            float l = acc[q];
            if (bias) l += bias[e];
            lg[e] = __builtin_isnan(l) ? -INFINITY : l;
        }
    }
    __syncthreads();
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    const int nv = (E + 63) >> 6;

    float p[kMaxPerLane];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        const float l = (i < nv && e < E) ? lg[e] : -INFINITY;
        p[i] = l;
        mx = fmaxf(mx, l);
    }
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        float z = 0.f;
        if (i < nv && e < E) {
            if (mx == INFINITY)
                z = (p[i] == INFINITY) ? 1.f : 0.f;
            else if (mx == -INFINITY)
                z = 1.f;
            else
                z = expf(p[i] - mx);
        }
        p[i] = z;
        sum += z;
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        if (i < nv && e < E) {
            p[i] = p[i] / sum;
            if (probs) probs[(size_t)t * E + e] = p[i];
        } else {
            p[i] = -1.f;  // never selected: every real probability is >= 0
        }
    }

    // k rounds of wave argmax.  Lane j keeps the j-th winner.
    float my_p = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bp = -2.f;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            const int e = lane + 64 * i;
            if (p[i] > bp) {  // ascending e within a lane: the first max wins ties
                bp = p[i];
                be = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float op = __shfl_xor(bp, o, 64);
            const int oe = __shfl_xor(be, o, 64);
            if (op > bp || (op == bp && oe < be)) {
                bp = op;
                be = oe;
            }
        }
        if (lane == j) {
            my_p = bp;
            my_e = be;
        }
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            if (lane + 64 * i == be) p[i] = -2.f;
    }
    // Renormalise over the selected, summing in ascending j.
    float ssum = 0.f;
    for (int j = 0; j < k; ++j) ssum += __shfl(my_p, j, 64);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w_out[(size_t)t * k + lane] = renorm ? my_p / ssum : my_p;
    }
}

}  // namespace

hipError_t launch_router_gemm(const uint16_t* x, const float* wg, float* part, int T, int H,
                              int E, int splits, hipStream_t st) {
    dim3 grid((E + BE - 1) / BE, (T + BT - 1) / BT, splits);
    prof_begin(K_ROUTER_GEMM, st);
    router_gemm_kernel<<<grid, 256, 0, st>>>(x, wg, part, T, H, E, H / splits);
    prof_end(K_ROUTER_GEMM, st);
    return hipGetLastError();
}

hipError_t launch_router_select(const float* part, int splits, const float* bias, int T, int E,
                                int k, int renorm, int32_t* ids, float* w, float* probs,
                                hipStream_t st) {
    prof_begin(K_ROUTER_SELECT, st);
    router_select_kernel<<<T, 256, 0, st>>>(part, splits, bias, T, E, k, renorm, ids, w, probs);
    prof_end(K_ROUTER_SELECT, st);
    return hipGetLastError();
}

}  // namespace moe
