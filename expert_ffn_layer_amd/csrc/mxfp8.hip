// MXFP8 expert weights: quantisation of bf16 weight rows and the packed
// layout the light loop streams.
//
// Format (OCP Microscaling Formats (MX) specification v1.0, MXFP8 with E4M3
// elements): 32 consecutive values of a row share one E8M0 scale 2^(s8-127);
// each value is an E4M3 code (bias 7, 3 mantissa bits, subnormals below
// 2^-6, largest finite 448, no infinities).  A block is quantised with the
// specification's conversion: shared exponent floor(log2 max|v|) - 8,
// clamped to [-127, 127] (an all-zero block takes -127); each value divided
// by 2^shared and rounded to the nearest E4M3 value, ties to the even
// mantissa, saturating at +-448, the sign bit kept (also for zeros).
// The pages name FP8 scaling blocks (pwwt.cn article, section 6) and MX
// formats (first page, section 3) without fixing a weight format.
//
// Everything here is integer arithmetic on the bf16 bit patterns: the
// division by a power of two only moves the exponent, so the rounding is
// decided on the exact value.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// floor(log2 |v|) of a nonzero bf16 magnitude (bits & 0x7fff).
__device__ __forceinline__ int bf16_ilog2(uint32_t mag) {
    const uint32_t eb = mag >> 7, mb = mag & 0x7f;
    if (eb != 0) return (int)eb - 127;
    return (31 - __clz(mb)) - 133;  // subnormal: mb * 2^-133
}

// E4M3 code of (bf16 value b) / 2^s, rounded to nearest even, saturating.
__device__ __forceinline__ uint32_t e4m3_code(uint32_t b, int s) {
    const uint32_t sign = (b >> 8) & 0x80u;
    const uint32_t mag = b & 0x7fffu;
    if (mag == 0) return sign;
    // 8-bit significand with its leading one at bit 7; ev = exponent of that
    // bit after the division: the value is sig * 2^(ev - 7).
    const uint32_t eb = mag >> 7, mb = mag & 0x7f;
    uint32_t sig;
    int ev;
    if (eb != 0) {
        sig = 0x80u | mb;
        ev = (int)eb - 127;
    } else {
        const int p = 31 - __clz(mb);
        sig = mb << (7 - p);
        ev = p - 133;
    }
    ev -= s;
    // Keep the bits down to the spacing 2^(max(ev, -6) - 3): drop `shift`
    // low bits of sig, round half to even.
    const int shift = 4 + (ev < -6 ? -6 - ev : 0);
    uint32_t q = 0;
    if (shift <= 8) {
        const uint32_t rem = sig & ((1u << shift) - 1u), half = 1u << (shift - 1);
        q = sig >> shift;
        if (rem > half || (rem == half && (q & 1u))) ++q;
    }
    if (ev >= -6) {  // normal range: q in [8, 16]
        if (q == 16) {
            q = 8;
            ++ev;
        }
        if (ev > 8 || (ev == 8 && q > 14)) return sign | 0x7eu;  // saturate at 448
        return sign | ((uint32_t)(ev + 7) << 3) | (q - 8u);
    }
    return sign | q;  // subnormal m = q; q == 8 is the smallest normal, same bits
}

// One thread per 32-value block: 4 x 16-byte loads, 2 x 16-byte stores.
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint16_t* __restrict__ w,
                                                             long long nblocks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
    for (long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks;
         b += (long long)gridDim.x * blockDim.x) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w + b * 32);
        uint32_t v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4_t q = src[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * i + j] = q[j];
        }
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            amax = max(amax, v[i] & 0x7fffu);
            amax = max(amax, (v[i] >> 16) & 0x7fffu);
        }
        int s = amax ? bf16_ilog2(amax) - 8 : -127;
        s = s < -127 ? -127 : (s > 127 ? 127 : s);
        u32x4_t out[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t p = v[2 * i + j];
                word |= e4m3_code(p & 0xffffu, s) << (16 * j);
                word |= e4m3_code(p >> 16, s) << (16 * j + 8);
            }
            out[i / 4][i % 4] = word;
        }
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + b * 32);
        dst[0] = out[0];
        dst[1] = out[1];
        scales[b] = (uint8_t)(s + 127);
    }
}

// One thread per 16-byte lane slot of a code chunk (and, for lanes 0..15,
// the row's two scale bytes).  rows_per = weight rows per expert; a lane's
// weight row follows the bf16 packing: gate|up lanes l16 < 8 take gate row
// 8g + l16, the others up row I + 8g + l16 - 8; down lanes W_down row
// 16g + l16.
template <bool kGateUp>
__global__ __launch_bounds__(256) void pack_mxfp8_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         int E, int rows_per, int K, int I,
                                                         int groups, int nchunks,
                                                         uint8_t* __restrict__ pk,
                                                         uint8_t* __restrict__ pks) {
    const long long nslots = (long long)E * groups * nchunks * 64;
    const int nks = K / 32;
    for (long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x; q < nslots;
         q += (long long)gridDim.x * blockDim.x) {
        const int lane = (int)(q % 64);
        const long long chunk = q / 64;
        const int c = (int)(chunk % nchunks);
        const long long eg = chunk / nchunks;
        const int g = (int)(eg % groups), e = (int)(eg / groups);
        const int l16 = lane & 15, kg = lane >> 4;
        const int row = kGateUp ? (l16 < 8 ? 8 * g + l16 : I + 8 * g + l16 - 8) : 16 * g + l16;
        const uint8_t* src = codes + ((long long)e * rows_per + row) * K;
        uint32_t word[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int k0 = 64 * c + 32 * half + 8 * kg;
#pragma unroll
            for (int wv = 0; wv < 2; ++wv) {
                uint32_t x = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kk = k0 + 4 * wv + i;
                    if (kk < K) x |= (uint32_t)src[kk] << (8 * i);
                }
                word[2 * half + wv] = x;
            }
        }
        *reinterpret_cast<u32x4_t*>(pk + q * 16) = u32x4_t{word[0], word[1], word[2], word[3]};
        if (kg == 0) {
            const uint8_t* ss = scales + ((long long)e * rows_per + row) * nks;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int ks = 2 * c + st;
                pks[chunk * 32 + 2 * l16 + st] = ks < nks ? ss[ks] : (uint8_t)127;
            }
        }
    }
}

// Heavy-tile layout: one record of kMxStageBytes per (expert, 256-row B tile
// nb, 64-wide K chunk c) -- the tile rows' codes (64 bytes each, the 16-byte
// unit q holding K 8q..8q+7 then 32+8q..32+8q+7 of the chunk), then their
// scales (two bytes per row: the chunk's two K steps) in the order the MFMA
// fragment reads take them: row rr at byte 2 * (4 * (16 * (rr / 64) + rr % 16)
// + (rr / 16) % 4).  Tile rows follow the heavy kernel's B tile: gate|up rows
// alternate in 16-row blocks of gate and up rows of the same h columns
// (column nb*128 + 16*(rr/32) + rr%16); down rows are W_down rows nb*256 + rr.
// Rows past the weights and K past the end hold code 0 (scale 127).
// One thread per 16-byte code unit; units 0..3 of a row also write its scales.
template <bool kGateUp>
__global__ __launch_bounds__(256) void pack_mxfp8_heavy_kernel(const uint8_t* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales,
                                                               int E, int rows_per, int K, int I,
                                                               int nblk, int nchunks,
                                                               uint8_t* __restrict__ out) {
    const long long nunits = (long long)E * nblk * nchunks * 256 * 4;
    const int nks = K / 32;
    for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < nunits;
         u += (long long)gridDim.x * blockDim.x) {
        const int q = (int)(u & 3);
        const int rr = (int)((u >> 2) & 255);
        const long long rec = u >> 10;
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
        uint32_t word[4] = {0u, 0u, 0u, 0u};
        if (valid) {
            const uint8_t* src = codes + ((long long)e * rows_per + row) * K;
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int kk = 64 * c + 32 * half + 8 * q + i;
                    if (kk < K) word[2 * half + i / 4] |= (uint32_t)src[kk] << (8 * (i % 4));
                }
        }
        uint8_t* dst = out + rec * kMxStageBytes;
        *reinterpret_cast<u32x4_t*>(dst + rr * 64 + 16 * q) =
            u32x4_t{word[0], word[1], word[2], word[3]};
        if (q < 2) {
            const int ks = 2 * c + q;
            uint8_t sv = 127;
            if (valid && ks < nks) sv = scales[((long long)e * rows_per + row) * nks + ks];
            const int slot = 4 * (16 * (rr >> 6) + (rr & 15)) + ((rr >> 4) & 3);
            dst[kMxCodeBytes + 2 * slot + q] = sv;
        }
    }
}

int grid_of(long long items) {
    return (int)std::min<long long>((items + 255) / 256, 65536);
}

}  // namespace

size_t mx_codes_gu_bytes(int E, int H, int I) {
    return (size_t)E * packed_gu_groups(I) * mx_chunks(H) * 1024;
}
size_t mx_codes_dn_bytes(int E, int H, int I) {
    return (size_t)E * packed_dn_groups(H) * mx_chunks(I) * 1024;
}
size_t mx_scales_gu_bytes(int E, int H, int I) {
    return (size_t)E * packed_gu_groups(I) * mx_chunks(H) * 32;
}
size_t mx_scales_dn_bytes(int E, int H, int I) {
    return (size_t)E * packed_dn_groups(H) * mx_chunks(I) * 32;
}
size_t mx_heavy_gu_bytes(int E, int H, int I) {
    return (size_t)E * ((2 * I + 255) / 256) * mx_chunks(H) * kMxStageBytes;
}
size_t mx_heavy_dn_bytes(int E, int H, int I) {
    return (size_t)E * ((H + 255) / 256) * mx_chunks(I) * kMxStageBytes;
}

hipError_t launch_mxfp8_quantize(const uint16_t* w, long long rows, int K, uint8_t* codes,
                                 uint8_t* scales, hipStream_t st) {
    const long long nblocks = rows * (K / 32);
    if (nblocks <= 0) return hipSuccess;
    mxfp8_quantize_kernel<<<grid_of(nblocks), 256, 0, st>>>(w, nblocks, codes, scales);
    return hipGetLastError();
}

hipError_t launch_pack_mxfp8(const uint8_t* c_gu, const uint8_t* s_gu, const uint8_t* c_dn,
                             const uint8_t* s_dn, int E, int H, int I, char* packed,
                             hipStream_t st) {
    uint8_t* base = reinterpret_cast<uint8_t*>(packed);
    uint8_t* q_gu = base;
    uint8_t* q_dn = q_gu + mx_codes_gu_bytes(E, H, I);
    uint8_t* qs_gu = q_dn + mx_codes_dn_bytes(E, H, I);
    uint8_t* qs_dn = qs_gu + mx_scales_gu_bytes(E, H, I);
    const int gg = packed_gu_groups(I), cg = mx_chunks(H);
    const int gd = packed_dn_groups(H), cd = mx_chunks(I);
    pack_mxfp8_kernel<true><<<grid_of((long long)E * gg * cg * 64), 256, 0, st>>>(
        c_gu, s_gu, E, 2 * I, H, I, gg, cg, q_gu, qs_gu);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    pack_mxfp8_kernel<false><<<grid_of((long long)E * gd * cd * 64), 256, 0, st>>>(
        c_dn, s_dn, E, H, I, I, gd, cd, q_dn, qs_dn);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    uint8_t* hq_gu = qs_dn + mx_scales_dn_bytes(E, H, I);
    uint8_t* hq_dn = hq_gu + mx_heavy_gu_bytes(E, H, I);
    const int nbg = (2 * I + 255) / 256, nbd = (H + 255) / 256;
    pack_mxfp8_heavy_kernel<true><<<grid_of((long long)E * nbg * cg * 1024), 256, 0, st>>>(
        c_gu, s_gu, E, 2 * I, H, I, nbg, cg, hq_gu);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    pack_mxfp8_heavy_kernel<false><<<grid_of((long long)E * nbd * cd * 1024), 256, 0, st>>>(
        c_dn, s_dn, E, H, I, I, nbd, cd, hq_dn);
    return hipGetLastError();
}

}  // namespace moe
