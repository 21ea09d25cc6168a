// Weighted gather-combine back to token order (pwwt.cn article on Qwen
// 3.5-397B MoE on Ironwood, section 7.2: local un-permute and gather-reduce
// of the expert-major rows).  One writer per output element, fp32, the k
// routed rows summed in ascending j: deterministic, no atomics.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// grid (T, ceil(H / 2048)); each thread owns 8 consecutive columns.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                     const int32_t* __restrict__ inv_pos,
                                                     const float* __restrict__ w, int H, int k,
                                                     int accumulate, float* __restrict__ out) {
    const int t = blockIdx.x;
    const int c0 = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (c0 >= H) return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
        const int p = inv_pos[(size_t)t * k + j];
        if (p < 0) continue;
        const float wj = w[(size_t)t * k + j];
        const float4* src = reinterpret_cast<const float4*>(y + (size_t)p * H + c0);
        const float4 v0 = src[0], v1 = src[1];
        acc[0] += wj * v0.x;
        acc[1] += wj * v0.y;
        acc[2] += wj * v0.z;
        acc[3] += wj * v0.w;
        acc[4] += wj * v1.x;
        acc[5] += wj * v1.y;
        acc[6] += wj * v1.z;
        acc[7] += wj * v1.w;
    }
    float4* o = reinterpret_cast<float4*>(out + (size_t)t * H + c0);
    float4 lo = {acc[0], acc[1], acc[2], acc[3]};
    float4 hi = {acc[4], acc[5], acc[6], acc[7]};
    if (accumulate) {
        const float4 plo = o[0], phi = o[1];
        lo = {plo.x + lo.x, plo.y + lo.y, plo.z + lo.z, plo.w + lo.w};
        hi = {phi.x + hi.x, phi.y + hi.y, phi.z + hi.z, phi.w + hi.w};
    }
    o[0] = lo;
    o[1] = hi;
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* inv_pos, const float* w, int T,
                          int H, int k, int accumulate, float* out, hipStream_t st) {
    dim3 grid(T, (H + 2047) / 2048);
    prof_begin(K_COMBINE, st);
    combine_kernel<<<grid, 256, 0, st>>>(y, inv_pos, w, H, k, accumulate, out);
    prof_end(K_COMBINE, st);
    return hipGetLastError();
}

}  // namespace moe
