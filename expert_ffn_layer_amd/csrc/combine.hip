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

// grid (T, ceil(H / (1024 kV))); each thread owns kV groups of 4 consecutive
// columns, 1024 columns apart.  The token's k (row, weight) pairs are uniform
// across the block.  y is read once and out written once, so both go through
// non-temporal accesses (measured 9-14% faster at T = 4096..8192).
template <int kV>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                     const int32_t* __restrict__ inv_pos,
                                                     const float* __restrict__ w, int H, int k,
                                                     int accumulate, float* __restrict__ out) {
    const int t = blockIdx.x;
    const int cb = blockIdx.y * 1024 * kV + threadIdx.x * 4;
    const int32_t* ip = inv_pos + (size_t)t * k;
    const float* wt = w + (size_t)t * k;
    bool all_valid = true;
    for (int j = 0; j < k; ++j) all_valid &= ip[j] >= 0;
#pragma unroll
    for (int q = 0; q < kV; ++q) {
        const int c0 = cb + q * 1024;
        if (c0 >= H) break;
        float4 acc = {0.f, 0.f, 0.f, 0.f};
        if (all_valid) {
            // every row present: issue the k row loads back to back
            float4 v[kMaxK];
#pragma unroll
            for (int j = 0; j < kMaxK; ++j)
                if (j < k) {
                    const floatx4_t u = __builtin_nontemporal_load(
                        reinterpret_cast<const floatx4_t*>(y + (size_t)ip[j] * H + c0));
                    v[j] = float4{u[0], u[1], u[2], u[3]};
                }
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k) {
                    const float wj = wt[j];
                    acc.x += wj * v[j].x;
                    acc.y += wj * v[j].y;
                    acc.z += wj * v[j].z;
                    acc.w += wj * v[j].w;
                }
            }
        } else {
            for (int j = 0; j < k; ++j) {
                const int p = ip[j];
                if (p < 0) continue;
                const float wj = wt[j];
                const float4 v = *reinterpret_cast<const float4*>(y + (size_t)p * H + c0);
                acc.x += wj * v.x;
                acc.y += wj * v.y;
                acc.z += wj * v.z;
                acc.w += wj * v.w;
            }
        }
        float4* o = reinterpret_cast<float4*>(out + (size_t)t * H + c0);
        if (accumulate) {
            const float4 prev = *o;
            acc = {prev.x + acc.x, prev.y + acc.y, prev.z + acc.z, prev.w + acc.w};
        }
        __builtin_nontemporal_store(floatx4_t{acc.x, acc.y, acc.z, acc.w},
                                    reinterpret_cast<floatx4_t*>(o));
    }
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* inv_pos, const float* w, int T,
                          int H, int k, int accumulate, float* out, hipStream_t st) {
    prof_begin(K_COMBINE, st);
    // Few tokens: one column group per thread, so that T * H / 1024 blocks
    // spread the gather over the whole chip (decode: 256 blocks, not 64).
    if (T < MOE_COMBINE_SMALL_T)
        combine_kernel<1><<<dim3(T, (H + 1023) / 1024), 256, 0, st>>>(y, inv_pos, w, H, k,
                                                                     accumulate, out);
    else
        combine_kernel<4><<<dim3(T, (H + 4095) / 4096), 256, 0, st>>>(y, inv_pos, w, H, k,
                                                                     accumulate, out);
    prof_end(K_COMBINE, st);
    return hipGetLastError();
}

}  // namespace moe
