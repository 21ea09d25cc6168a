// Weighted gather-combine back to token order (pwwt.cn article on Qwen
// 3.5-397B MoE on Ironwood, section 7.2: local un-permute and gather-reduce
// of the expert-major rows).  One writer per output element, fp32, the k
// routed rows summed in ascending j: deterministic, no atomics.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMaxK = 32;
#ifndef MOE_COMBINE_SMALL_T
#define MOE_COMBINE_SMALL_T 512
#endif


// Storage of y: fp32, bf16 or fp16 (launch_combine's y_fmt).
constexpr int kYF32 = 0, kYBF16 = 1, kYF16 = 2;

// The 16-bit half of word u holding value c (c even: low half), widened to
// fp32 exactly.
template <int F>
__device__ __forceinline__ float y16_elem(uint32_t u, int c) {
    const uint32_t h = (c & 1) ? (u >> 16) : (u & 0xffffu);
    if constexpr (F == kYBF16) return __uint_as_float(h << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// C consecutive y values (C = 4: any storage; C = 8: 16-bit) as one raw
// vector load, read non-temporally (each y row is read once); elem() widens
// value c to fp32 exactly.
template <int C, int F>
struct YLoad;
template <>
struct YLoad<4, kYF32> {
    typedef floatx4_t raw_t;
    static __device__ __forceinline__ float elem(const raw_t& r, int c) { return r[c]; }
};
template <int F>
struct YLoad<4, F> {
    typedef u32x2_t raw_t;
    static __device__ __forceinline__ float elem(const raw_t& r, int c) {
        return y16_elem<F>(r[c >> 1], c);
    }
};
template <int F>
struct YLoad<8, F> {
    static_assert(F != kYF32, "8 values per load: 16-bit y");
    typedef u32x4_t raw_t;
    static __device__ __forceinline__ float elem(const raw_t& r, int c) {
        return y16_elem<F>(r[c >> 1], c);
    }
};

template <int C, int F>
__device__ __forceinline__ typename YLoad<C, F>::raw_t load_y(const void* y, size_t idx) {
    typedef typename YLoad<C, F>::raw_t R;
    const char* p = static_cast<const char*>(y) + idx * (F == kYF32 ? 4 : 2);
    return __builtin_nontemporal_load(reinterpret_cast<const R*>(p));
}

// grid (T, ceil(H / (256 C kV))); each thread owns kV groups of C
// consecutive columns, 256 C columns apart.  The token's k (row, weight)
// pairs are uniform across the block.  y is read once and out written once,
// so both go through non-temporal accesses (measured 9-14% faster at
// T = 4096..8192).  Every element sums its k rows in ascending j.
template <int kV, int C, int F>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                     const int32_t* __restrict__ inv_pos,
                                                     const float* __restrict__ w, int H, int k,
                                                     int accumulate, float* __restrict__ out) {
    typedef YLoad<C, F> L;
    constexpr int kSpan = 256 * C;
    const int t = blockIdx.x;
    const int cb = blockIdx.y * kSpan * kV + threadIdx.x * C;
    const int32_t* ip = inv_pos + (size_t)t * k;
    const float* wt = w + (size_t)t * k;
    bool all_valid = true;
    for (int j = 0; j < k; ++j) all_valid &= ip[j] >= 0;
#pragma unroll
    for (int q = 0; q < kV; ++q) {
        const int c0 = cb + q * kSpan;
        if (c0 >= H) break;
        float acc[C];
#pragma unroll
        for (int c = 0; c < C; ++c) acc[c] = 0.f;
        if (all_valid) {
            // every row present: issue the k row loads back to back
            typename L::raw_t v[kMaxK];
#pragma unroll
            for (int j = 0; j < kMaxK; ++j)
                if (j < k) v[j] = load_y<C, F>(y, (size_t)ip[j] * H + c0);
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k) {
                    const float wj = wt[j];
#pragma unroll
                    for (int c = 0; c < C; ++c) acc[c] += wj * L::elem(v[j], c);
                }
            }
        } else {
            for (int j = 0; j < k; ++j) {
                const int p = ip[j];
                if (p < 0) continue;
                const float wj = wt[j];
                const typename L::raw_t v = load_y<C, F>(y, (size_t)p * H + c0);
#pragma unroll
                for (int c = 0; c < C; ++c) acc[c] += wj * L::elem(v, c);
            }
        }
        floatx4_t* o = reinterpret_cast<floatx4_t*>(out + (size_t)t * H + c0);
#pragma unroll
        for (int c4 = 0; c4 < C / 4; ++c4) {
            floatx4_t r = {acc[4 * c4], acc[4 * c4 + 1], acc[4 * c4 + 2], acc[4 * c4 + 3]};
            if (accumulate) {
                const floatx4_t prev = o[c4];
                r = floatx4_t{prev[0] + r[0], prev[1] + r[1], prev[2] + r[2], prev[3] + r[3]};
            }
            __builtin_nontemporal_store(r, o + c4);
        }
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_fmt, const int32_t* inv_pos, const float* w,
                          int T, int H, int k, int accumulate, float* out, hipStream_t st) {
    prof_begin(K_COMBINE, st);
    // Few tokens: one column group per thread, so that T * H / 1024 blocks
    // spread the gather over the whole chip (decode: 256 blocks, not 64).
    // From 512 tokens: 16-byte row loads (4 fp32 or 8 16-bit columns), 4096
    // columns per block.
    const dim3 g1(T, (H + 1023) / 1024), g4(T, (H + 4095) / 4096);
    if (T < MOE_COMBINE_SMALL_T) {
        if (y_fmt == kYBF16)
            combine_kernel<1, 4, kYBF16><<<g1, 256, 0, st>>>(y, inv_pos, w, H, k, accumulate, out);
        else if (y_fmt == kYF16)
            combine_kernel<1, 4, kYF16><<<g1, 256, 0, st>>>(y, inv_pos, w, H, k, accumulate, out);
        else
            combine_kernel<1, 4, kYF32><<<g1, 256, 0, st>>>(y, inv_pos, w, H, k, accumulate, out);
    } else {
        if (y_fmt == kYBF16)
            combine_kernel<2, 8, kYBF16><<<g4, 256, 0, st>>>(y, inv_pos, w, H, k, accumulate, out);
        else if (y_fmt == kYF16)
            combine_kernel<2, 8, kYF16><<<g4, 256, 0, st>>>(y, inv_pos, w, H, k, accumulate, out);
        else
            combine_kernel<4, 4, kYF32><<<g4, 256, 0, st>>>(y, inv_pos, w, H, k, accumulate, out);
    }
    prof_end(K_COMBINE, st);
    return hipGetLastError();
}

}  // namespace moe
