// Permute: histogram -> exclusive scan -> stable scatter of the routed rows.
//
// Only int32 row indices move; activation rows are gathered later inside
// the expert GEMM, so no padded [E x capacity] buffer ever exists (the pages
// gather routed token rows into a contiguous buffer without materialising a
// padded intermediate because top_k = 10 is not a power of 2: pwwt.cn
// article on Qwen 3.5-397B MoE on Ironwood, section 4.2).
//
// Assignments a = t*k + j are split into chunks of kPermChunk.  Block c
// counts its chunk (LDS integer atomics: the count does not depend on
// order); one block turns the [chunk][expert] counts into the global
// offsets and each chunk's first slot per expert; block c then ranks its
// chunk's assignments in assignment order (wave ballots match equal expert
// ids) and writes each to its slot.  Integer arithmetic throughout, so the
// result is exact and deterministic.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kPermChunk / kThreads;  // 16
constexpr int kWavesPerBlock = kThreads / 64;

__device__ __forceinline__ bool valid_id(int e, int E) { return e >= 0 && e < E; }

// 64 consecutive assignments, one per lane: the lane's rank among this
// wave's assignments to the same expert so far (earlier steps and lower
// lanes).  Lanes holding equal ids are matched with one ballot per id bit;
// the group's last lane advances my[e].  A wave's own LDS accesses complete
// in program order, so the next step sees the update.
__device__ __forceinline__ int wave_stable_rank(int e, bool ok, int nbits, uint64_t lt,
                                                int32_t* my) {
    uint64_t match = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(bit);
        match &= bit ? bal : ~bal;
    }
    const int rank = __popcll(match & lt);
    const int n = __popcll(match);
    int loc = 0;
    if (ok) {
        loc = my[e] + rank;
        if (rank == n - 1) my[e] = loc + 1;
    }
    return loc;
}

// Exclusive scan over a 256-thread block of one int per thread; returns the
// thread's exclusive prefix and writes the block total to *total.
__device__ __forceinline__ int block256_exclusive_scan(int v, int32_t* wsum, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    return before + incl - v;
}

__global__ __launch_bounds__(kThreads) void perm_count_kernel(const int32_t* __restrict__ ids,
                                                             long long A, int E,
                                                             int32_t* __restrict__ chunk_counts) {
    extern __shared__ int32_t cnt[];
    for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
    __syncthreads();
    const long long base = (long long)blockIdx.x * kPermChunk;
#pragma unroll 4
    for (int q = 0; q < kPerThread; ++q) {
        const long long a = base + q * kThreads + threadIdx.x;
        if (a < A) {
            const int e = ids[a];
            if (valid_id(e, E)) atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    int32_t* out = chunk_counts + (size_t)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += kThreads) out[e] = cnt[e];
}

// Single block, one thread per expert (E <= 1024).
// In: chunk_counts[c][e].  Out: counts[e], offsets[0..E], and
// chunk_counts[c][e] replaced by the first slot of chunk c's rows of e.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ chunk_counts,
                                                         int nchunks, int E,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
    __shared__ int32_t wsum[16];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        int c = 0;
        for (; c + 8 <= nchunks; c += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = chunk_counts[(size_t)(c + u) * E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                chunk_counts[(size_t)(c + u) * E + e] = run;
                run += v[u];
            }
        }
        for (; c < nchunks; ++c) {
            const int v = chunk_counts[(size_t)c * E + e];
            chunk_counts[(size_t)c * E + e] = run;
            run += v;
        }
        counts[e] = run;
    }
    // Block-wide exclusive scan of run over e.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int excl = before + incl - run;
    if (e < E) {
        offsets[e] = excl;
        if (e == E - 1) offsets[E] = excl + run;
#pragma unroll 8
        for (int c = 0; c < nchunks; ++c) chunk_counts[(size_t)c * E + e] += excl;
    }
}

__global__ __launch_bounds__(kThreads) void perm_scatter_kernel(
    const int32_t* __restrict__ ids, long long A, int k, int E, int nbits,
    const int32_t* __restrict__ chunk_base, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ inv_pos) {
    extern __shared__ int32_t wcnt[];  // [kWavesPerBlock][E]
    for (int i = threadIdx.x; i < kWavesPerBlock * E; i += kThreads) wcnt[i] = 0;
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long base = (long long)blockIdx.x * kPermChunk + (long long)wave * (kPermChunk / kWavesPerBlock);
    const uint64_t lt = lanemask_lt(lane);
    int32_t* my = wcnt + wave * E;

    int local[kPerThread];
    int eid[kPerThread];
    // Each wave walks its quarter of the chunk in assignment order, 64 at a
    // time; lanes holding the same expert id are matched with ballots.  The
    // group's last lane advances my[e] for the next 64; a wave's own LDS
    // accesses complete in program order.
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const long long a = base + (long long)q * 64 + lane;
        const int e = (a < A) ? ids[a] : -1;
        const bool ok = valid_id(e, E);
        local[q] = wave_stable_rank(e, ok, nbits, lt, my);
        eid[q] = ok ? e : -1;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const long long a = base + (long long)q * 64 + lane;
        if (a >= A) continue;
        const int e = eid[q];
        if (e < 0) {
            inv_pos[a] = -1;
            continue;
        }
        int pos = chunk_base[(size_t)blockIdx.x * E + e] + local[q];
        for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
        sorted_ids[pos] = (int32_t)a / k;
        inv_pos[a] = pos;
    }
}

// The whole permute in one block when all assignments fit one chunk
// (A <= kPermChunk): per-wave stable ranks give the counts, a block scan
// gives the offsets, then every assignment is written to its slot.  With a
// plan pointer it also emits the grouped-FFN plan (same layout as
// ffn_plan_kernel: light experts with 1..light_max rows, heavy row tiles).
__global__ __launch_bounds__(kThreads) void perm_small_kernel(
    const int32_t* __restrict__ ids, int A, int k, int E, int nbits,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ inv_pos, int32_t* __restrict__ plan, int light_max, int force_tm,
    int round_tiles, int32_t* __restrict__ sync) {
    extern __shared__ int32_t sm[];  // wcnt[4][E], off[E]
    __shared__ int32_t wsum[4];
    int32_t* wcnt = sm;
    int32_t* off = sm + kWavesPerBlock * E;
    for (int i = threadIdx.x; i < (kWavesPerBlock + 1) * E; i += kThreads) sm[i] = 0;
    if (plan && sync)  // the fused light loop's counters start at zero
        for (int i = threadIdx.x; i < sync_ints(E); i += kThreads) sync[i] = 0;
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // Each wave ranks a contiguous quarter of the assignments (rounded up to
    // whole 64-lane steps), so the four waves share the serial rank chain.
    const int per_wave = (A + kWavesPerBlock * 64 - 1) / (kWavesPerBlock * 64) * 64;
    const int steps = per_wave / 64;  // <= kPerThread since A <= kPermChunk
    const int base = wave * per_wave;
    const uint64_t lt = lanemask_lt(lane);
    int local[kPerThread];
    int eid[kPerThread];
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        local[q] = 0;
        eid[q] = -1;
        if (q < steps) {
            const int a = base + q * 64 + lane;
            const int e = (a < A) ? ids[a] : -1;
            const bool ok = valid_id(e, E);
            local[q] = wave_stable_rank(e, ok, nbits, lt, wcnt + wave * E);
            eid[q] = ok ? e : -1;
        }
    }
    __syncthreads();

    // counts and exclusive offsets; each thread owns experts 4t..4t+3
    int c[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * threadIdx.x + j;
        c[j] = 0;
        if (e < E) c[j] = wcnt[e] + wcnt[E + e] + wcnt[2 * E + e] + wcnt[3 * E + e];
        sum += c[j];
    }
    int total = 0;
    int run = block256_exclusive_scan(sum, wsum, &total);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * threadIdx.x + j;
        if (e < E) {
            off[e] = run;
            counts[e] = c[j];
            offsets[e] = run;
        }
        run += c[j];
    }
    if (threadIdx.x == 0) offsets[E] = total;
    __syncthreads();

#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int a = base + q * 64 + lane;
        if (q >= steps || a >= A) continue;
        const int e = eid[q];
        if (e < 0) {
            inv_pos[a] = -1;
            continue;
        }
        int pos = off[e] + local[q];
        for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
        sorted_ids[pos] = a / k;
        inv_pos[a] = pos;
    }

    if (!plan) return;
    int lm = light_max;
    if (lm == kLightAdaptive) {  // uniform: every thread takes this branch or none
        int touched = 0;
        (void)block256_exclusive_scan((c[0] > 0) + (c[1] > 0) + (c[2] > 0) + (c[3] > 0), wsum,
                                      &touched);
        lm = adaptive_light_max(total, touched);
    }
    // Heavy tiles per expert (tile_split, the rule of ffn_plan_kernel).
    int lj[4], tj[4], tmain[4], tlast[4], lsum = 0, tsum = 0, csum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        lj[j] = (c[j] >= 1 && c[j] <= lm) ? 1 : 0;
        tj[j] = 0;
        tmain[j] = tlast[j] = 0;
        if (c[j] > lm) tile_split(c[j], force_tm, tj[j], tmain[j], tlast[j]);
        lsum += lj[j];
        tsum += tj[j];
        csum += tiles_cost_units(tj[j], tmain[j], tlast[j]);
    }
    int ltot = 0, ttot = 0, ctot = 0;
    int lrun = block256_exclusive_scan(lsum, wsum, &ltot);
    int trun = block256_exclusive_scan(tsum, wsum, &ttot);
    int crun = block256_exclusive_scan(csum, wsum, &ctot);
    int32_t* tiles = plan + kPlanHeader + E;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * threadIdx.x + j;
        if (lj[j]) plan[kPlanHeader + lrun++] = e;
        xcd_bounds(plan, trun, tj[j], tmain[j], tlast[j], crun, ctot, round_tiles, ttot);
        crun += tiles_cost_units(tj[j], tmain[j], tlast[j]);
        const int tm = tile_height(tmain[j]);
        for (int i = 0; i < tj[j]; ++i, ++trun) {
            tiles[2 * trun] = e;
            tiles[2 * trun + 1] = (i * tm) | ((i + 1 < tj[j] ? tmain[j] : tlast[j]) << kTileTmShift);
        }
    }
    if (threadIdx.x == 0) {
        plan[0] = ltot;
        plan[1] = ttot;
        plan[2] = force_tm;
        plan[kPlanXcdBounds] = 0;
        plan[kPlanXcdBounds + kXcds] = ttot;
        if (ctot == 0)
            for (int x = 1; x < kXcds; ++x) plan[kPlanXcdBounds + x] = 0;
    }
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* chunk_counts,
                          int nchunks, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                          int32_t* inv_pos, int32_t* plan, int light_max, int force_tm,
                          int round_tiles, int32_t* sync, hipStream_t st) {
    const long long A = (long long)T * k;
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    if (A <= kPermChunk) {
        prof_begin(K_PERM_SMALL, st);
        perm_small_kernel<<<1, kThreads, (kWavesPerBlock + 1) * E * sizeof(int32_t), st>>>(
            ids, (int)A, k, E, nbits, counts, offsets, sorted_ids, inv_pos, plan, light_max,
            force_tm, round_tiles, sync);
        prof_end(K_PERM_SMALL, st);
        return hipGetLastError();
    }
    prof_begin(K_PERM_COUNT, st);
    perm_count_kernel<<<nchunks, kThreads, E * sizeof(int32_t), st>>>(ids, A, E, chunk_counts);
    prof_end(K_PERM_COUNT, st);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    prof_begin(K_PERM_SCAN, st);
    perm_scan_kernel<<<1, 1024, 0, st>>>(chunk_counts, nchunks, E, counts, offsets);
    prof_end(K_PERM_SCAN, st);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    prof_begin(K_PERM_SCATTER, st);
    perm_scatter_kernel<<<nchunks, kThreads, kWavesPerBlock * E * sizeof(int32_t), st>>>(
        ids, A, k, E, nbits, chunk_counts, sorted_ids, inv_pos);
    prof_end(K_PERM_SCATTER, st);
    return hipGetLastError();
}

}  // namespace moe
