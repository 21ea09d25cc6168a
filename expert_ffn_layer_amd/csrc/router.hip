// Router: fp32 gate GEMM (on bf16 MFMA with exact three-term weights), then
// a block-per-token softmax and register top-k.
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
constexpr int LDK = BK + 8;  // bf16 row pitch in LDS (80 bytes): spreads rows over the banks

// Two fp32 values -> three packed bf16 pairs with hi + mid + lo == v exactly
// for normal v (each term is the round-to-nearest-even bf16 of the exact fp32
// remainder of the previous ones; 8 + 8 + 8 significand bits cover fp32's 24).
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& hi, uint32_t& mid,
                                            uint32_t& lo) {
    const floatx2_t v = {a, b};
    const bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    const floatx2_t r1 = v - __builtin_convertvector(h, floatx2_t);
    const bf16x2_t m = __builtin_convertvector(r1, bf16x2_t);
    const floatx2_t r2 = r1 - __builtin_convertvector(m, floatx2_t);
    const bf16x2_t l = __builtin_convertvector(r2, bf16x2_t);
    hi = __builtin_bit_cast(uint32_t, h);
    mid = __builtin_bit_cast(uint32_t, m);
    lo = __builtin_bit_cast(uint32_t, l);
}

// part[s][t][e] for one 128x128 (token x expert) tile and one hidden slice.
// The fp32 router product runs on bf16 MFMA: x is bf16 already, and every
// router weight enters as three bf16 terms (split3_pair), so each product
// x*w_term is exact and the MFMA accumulates in fp32.  256 threads = 4 waves
// in a 2x2 grid, each a 64x64 block of 16x16 tiles
// (v_mfma_f32_16x16x32_bf16, 3 MFMAs per tile and K step).
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wg,
                                                          float* __restrict__ part, int T,
                                                          int H, int E, int k_per_split) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BT][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][3][BE][LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l16 = lane & 15, g = lane >> 4;
    // Blocks go round-robin to the 8 XCDs; each XCD takes a contiguous run of
    // tiles, expert tile fastest, so the tiles sharing an x slice share an L2.
    const int nb = gridDim.x, b = blockIdx.x;
    const int tile = (nb & 7) ? b : (b & 7) * (nb >> 3) + (b >> 3);
    const int ne = (E + BE - 1) / BE, nt = (T + BT - 1) / BT;
    const int e0 = (tile % ne) * BE;
    const int t0 = ((tile / ne) % nt) * BT;
    const int s = tile / (ne * nt);
    const int kbeg = s * k_per_split;
    const int kend = kbeg + k_per_split;
    // router-weight staging: this thread owns expert e0+el, 16 consecutive k
    const int el = tid & (BE - 1), kh = tid >> 7;
    const bool e_ok = e0 + el < E;

    u32x4_t xr[2];
    float wr[16];
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + 256 * q;
            const int t = c >> 2, kc = (c & 3) * 8;
            xr[q] = (t0 + t < T) ? *reinterpret_cast<const u32x4_t*>(x + (size_t)(t0 + t) * H + k0 + kc)
                                 : u32x4_t{0u, 0u, 0u, 0u};
        }
        const float* src = wg + (size_t)(k0 + 16 * kh) * E + e0 + el;
#pragma unroll
        for (int j = 0; j < 16; ++j) wr[j] = e_ok ? src[(size_t)j * E] : 0.f;
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + 256 * q;
            const int t = c >> 2, kc = (c & 3) * 8;
            *reinterpret_cast<u32x4_t*>(&xs[buf][t][kc]) = xr[q];
        }
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            uint32_t p[3][4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                split3_pair(wr[8 * h8 + 2 * j], wr[8 * h8 + 2 * j + 1], p[0][j], p[1][j], p[2][j]);
#pragma unroll
            for (int pl = 0; pl < 3; ++pl)
                *reinterpret_cast<u32x4_t*>(&ws[buf][pl][el][16 * kh + 8 * h8]) =
                    u32x4_t{p[pl][0], p[pl][1], p[pl][2], p[pl][3]};
        }
    };

    floatx4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    load_stage(kbeg);
    store_stage(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = kbeg; k0 < kend; k0 += BK) {
        const bool more = k0 + BK < kend;
        if (more) load_stage(k0 + BK);
        bf16x8_t af[4], bf[3][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const bf16x8_t*>(&xs[buf][wm * 64 + i * 16 + l16][8 * g]);
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[pl][j] =
                    *reinterpret_cast<const bf16x8_t*>(&ws[buf][pl][wn * 64 + j * 16 + l16][8 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) acc[i][j] = mfma_16x16x32(af[i], bf[pl][j], acc[i][j]);
        if (more) store_stage(buf ^ 1);
        __syncthreads();
        buf ^= 1;
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

// Softmax over the E logits held by one wave (lane holds experts lane + 64i,
// i < NV; -inf marks a masked logit) and k rounds of a wave-wide argmax over
// (probability, -expert id) keys held in registers.  Any k <= 32 works
// without padding k to a power of 2.  Each lane sums its own slots in
// ascending i and the lane sums are combined by a butterfly, so the result
// does not depend on NV (slots past E hold 0).
template <int NV>
__device__ __forceinline__ void softmax_topk(float (&p)[NV], int lane, int t, int E, int k,
                                             int renorm, int32_t* __restrict__ ids,
                                             float* __restrict__ w_out,
                                             float* __restrict__ probs) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) mx = fmaxf(mx, p[i]);
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        float z = 0.f;
        if (e < E) {
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
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
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
        for (int i = 0; i < NV; ++i) {
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
        for (int i = 0; i < NV; ++i)
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

// One block of 256*NG threads per token.  The threads reduce the split
// partials and add the bias into LDS: group g of 256 threads sums splits
// [g*S/NG, (g+1)*S/NG) in ascending order and the NG group sums are added in
// ascending g (NG = 4 when there are few tokens, so each thread has fewer
// dependent loads).  Wave 0 then selects (softmax_topk).
template <int NG, int QN, int UB>
__global__ __launch_bounds__(256 * NG) void router_select_kernel(
    const float* __restrict__ part, int splits, const float* __restrict__ bias, int T, int E,
    int k, int renorm, int32_t* __restrict__ ids, float* __restrict__ w_out,
    float* __restrict__ probs) {
    __shared__ float lg[64 * kMaxPerLane];
    __shared__ float gsum[NG > 1 ? NG - 1 : 1][64 * kMaxPerLane];
    const int t = blockIdx.x;
    const size_t plane = (size_t)T * E;
    const int col = threadIdx.x & 255, grp = threadIdx.x >> 8;
    const int per = (splits + NG - 1) / NG;
    const int sb = min(splits, grp * per), se = min(splits, sb + per);
    // Each thread owns experts col + 256q (q < QN, E <= 256 QN); UB splits
    // of each are loaded together, then added in ascending split order.
    float acc[QN];
#pragma unroll
    for (int q = 0; q < QN; ++q) acc[q] = 0.f;
    for (int s0 = sb; s0 < se; s0 += UB) {
        float v[QN][UB];
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const int e = col + 256 * q;
#pragma unroll
            for (int u = 0; u < UB; ++u)
                v[q][u] = (e < E && s0 + u < se)
                              ? part[(size_t)(s0 + u) * plane + (size_t)t * E + e]
                              : 0.f;
        }
#pragma unroll
        for (int q = 0; q < QN; ++q)
#pragma unroll
            for (int u = 0; u < UB; ++u)
                if (s0 + u < se) acc[q] += v[q][u];
    }
    if (NG > 1) {
        if (grp > 0) {
#pragma unroll
            for (int q = 0; q < QN; ++q) {
                const int e = col + 256 * q;
                if (e < E) gsum[grp - 1][e] = acc[q];
            }
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int q = 0; q < QN; ++q) {
                const int e = col + 256 * q;
                if (e < E)
                    for (int gg = 0; gg < NG - 1; ++gg) acc[q] += gsum[gg][e];
            }
        }
    }
    if (grp == 0) {
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const int e = col + 256 * q;
            if (e < E) {
                float l = acc[q];
                if (bias) l += bias[e];
                lg[e] = __builtin_isnan(l) ? -INFINITY : l;
            }
        }
    }
    __syncthreads();  // every thread of the block reaches both barriers
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    constexpr int NV = 4 * QN;  // expert slots per lane
    float p[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        p[i] = e < E ? lg[e] : -INFINITY;
    }
    softmax_topk<NV>(p, lane, t, E, k, renorm, ids, w_out, probs);
}

// One wave per token, four tokens per block: lane l sums the split partials
// of experts l + 64i (i < NV) in ascending split order, adds the bias and
// selects.  The logits equal router_select_kernel<1>'s bit for bit.
template <int NV>
__global__ __launch_bounds__(256) void router_select_wave_kernel(
    const float* __restrict__ part, int splits, const float* __restrict__ bias, int T, int E,
    int k, int renorm, int32_t* __restrict__ ids, float* __restrict__ w_out,
    float* __restrict__ probs) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // no block barrier below
    const size_t plane = (size_t)T * E;
    const float* src = part + (size_t)t * E + lane;
    float p[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) p[i] = 0.f;
    for (int s = 0; s < splits; ++s) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + 64 * i < E) p[i] += src[(size_t)s * plane + 64 * i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            float l = p[i];
            if (bias) l += bias[e];
            p[i] = __builtin_isnan(l) ? -INFINITY : l;
        } else {
            p[i] = -INFINITY;
        }
    }
    softmax_topk<NV>(p, lane, t, E, k, renorm, ids, w_out, probs);
}

}  // namespace

hipError_t launch_router_gemm(const uint16_t* x, const float* wg, float* part, int T, int H,
                              int E, int splits, hipStream_t st) {
    const long long nblk = (long long)((E + BE - 1) / BE) * ((T + BT - 1) / BT) * splits;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nblk);
    prof_begin(K_ROUTER_GEMM, st);
    router_gemm_kernel<<<grid, 256, 0, st>>>(x, wg, part, T, H, E, H / splits);
    prof_end(K_ROUTER_GEMM, st);
    return hipGetLastError();
}

hipError_t launch_router_select(const float* part, int splits, const float* bias, int T, int E,
                                int k, int renorm, int32_t* ids, float* w, float* probs,
                                hipStream_t st) {
    prof_begin(K_ROUTER_SELECT, st);
    // Few tokens: four thread groups per token shorten each thread's chain
    // of dependent partial loads.
    if (T < 1024 && splits >= 16) {
        if (E <= 512)
            router_select_kernel<4, 2, 16><<<T, 1024, 0, st>>>(part, splits, bias, T, E, k, renorm,
                                                           ids, w, probs);
        else
            router_select_kernel<4, 4, 8><<<T, 1024, 0, st>>>(part, splits, bias, T, E, k, renorm, ids,
                                                           w, probs);
    }
    else if (E <= 512)
        router_select_wave_kernel<8><<<(T + 3) / 4, 256, 0, st>>>(part, splits, bias, T, E, k,
                                                                  renorm, ids, w, probs);
    else
        router_select_wave_kernel<16><<<(T + 3) / 4, 256, 0, st>>>(part, splits, bias, T, E, k,
                                                                   renorm, ids, w, probs);
    prof_end(K_ROUTER_SELECT, st);
    return hipGetLastError();
}

}  // namespace moe
