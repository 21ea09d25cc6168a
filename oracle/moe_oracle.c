/*
 * moe_oracle.c -- plain, slow CPU reference of the sparse mixture-of-experts
 * layer.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the GPU library never does, and the
 * two share no code, headers or tables.
 *
 * What it computes (the plain definition of the layer):
 *
 *   out_t = sum_{j<k} w_{t,j} * FFN_{e_{t,j}}(x_t)   [ + FFN_shared(x_t) ]
 *   FFN_e(x) = W_down[e] (silu(W_gate[e] x) * (W_up[e] x)),  silu(z) = z/(1+e^-z)
 *
 * Sources (state of the method, restated, not quoted):
 *  - route -> top-k -> permute tokens to experts -> grouped SwiGLU expert FFN:
 *    pwwt.cn article on Qwen 3.5-397B MoE on Ironwood (TPU v7x), section 4.2
 *    ("MoE track"): top_k = 10 routing, token gather per expert, grouped GEMM
 *    with SwiGLU fused into the matmul.
 *  - un-permute and weighted gather-reduce back to token order: same article,
 *    section 7.2 (chunked pipeline over the [81920, 4096] permuted rows).
 *  - router logits, then top-k on the selected logits: same article, section
 *    8.2 (router gate and top-k fusion).
 *  - shared expert added to the routed sum: lumevalley.com article on
 *    SGLang-JAX serving Ling-2.6-1T, opening paragraph (256 routed experts,
 *    top-8 plus a shared expert).
 * The pages give no formulas for scoring, tie-breaking or renormalisation.
 * Readings used here: softmax over all E experts in fp32; order by
 * descending probability, the lower expert index winning ties; the selected
 * probabilities renormalised to sum to 1 when renorm != 0; expert linears
 * have no bias; the shared expert has weight 1 and is outside the top-k.
 *
 * Arithmetic: fp32 scalars, every sum accumulated one term at a time in
 * ascending index order; build with -O2 -ffp-contract=off (no fused
 * multiply-add, no reassociation).  OpenMP splits only independent rows, so
 * results do not depend on the thread count.
 *
 * Non-finite logits (a reading; the pages are silent): NaN is treated as
 * -inf; if the largest logit is +inf, the +inf entries share the mass
 * equally and the rest get 0; if every logit is -inf the distribution is
 * uniform.  Ties (including exact zeros) still go to the lower index, so the
 * k ids are always distinct and in [0, E).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OREF_EXPORT __attribute__((visibility("default")))

OREF_EXPORT void oref_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

OREF_EXPORT int oref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Router projection: logits[t,e] = (sum_h x[t,h] * wg[h,e]) + bias[e].
 * x [T,H], wg [H,E], bias [E] or NULL, logits [T,E]. */
OREF_EXPORT void oref_logits(int T, int H, int E, const float* x, const float* wg,
                             const float* bias, float* logits) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float* l = logits + (size_t)t * E;
        for (int e = 0; e < E; ++e) l[e] = 0.0f;
        for (int h = 0; h < H; ++h) {
            const float xv = x[(size_t)t * H + h];
            const float* w = wg + (size_t)h * E;
            for (int e = 0; e < E; ++e) l[e] = l[e] + xv * w[e];
        }
        if (bias)
            for (int e = 0; e < E; ++e) l[e] = l[e] + bias[e];
    }
}

typedef struct {
    float p;
    int e;
} oref_pe;

/* Total order: larger probability first; equal probabilities -> lower id. */
static int oref_cmp_pe(const void* a, const void* b) {
    const oref_pe* A = (const oref_pe*)a;
    const oref_pe* B = (const oref_pe*)b;
    if (A->p > B->p) return -1;
    if (A->p < B->p) return 1;
    return (A->e < B->e) ? -1 : (A->e > B->e ? 1 : 0);
}

/* Softmax over E, top-k, renormalisation.
 *  logits [T,E] -> ids [T,k] (descending probability), w [T,k],
 *  probs [T,E] (optional), gap_k [T] (optional; p_(k) - p_(k+1), +inf when
 *  k == E), gap_in [T] (optional; smallest adjacent gap among the first
 *  min(k+1, E) ranks, +inf when that is a single rank).
 *  Returns 0, or -1 on bad sizes. */
OREF_EXPORT int oref_route(int T, int E, int k, int renorm, const float* logits, int32_t* ids,
                           float* w, float* probs, float* gap_k, float* gap_in) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
    int bad = 0;
#pragma omp parallel
    {
        float* z = (float*)malloc(sizeof(float) * (size_t)E);
        float* lc = (float*)malloc(sizeof(float) * (size_t)E);
        oref_pe* order = (oref_pe*)malloc(sizeof(oref_pe) * (size_t)E);
        if (!z || !lc || !order) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            if (!z || !lc || !order) continue;
            const float* l = logits + (size_t)t * E;
            for (int e = 0; e < E; ++e) lc[e] = isnan(l[e]) ? -INFINITY : l[e];
            float m = -INFINITY;
            for (int e = 0; e < E; ++e)
                if (lc[e] > m) m = lc[e];
            for (int e = 0; e < E; ++e) {
                if (m == INFINITY)
                    z[e] = (lc[e] == INFINITY) ? 1.0f : 0.0f;
                else if (m == -INFINITY)
                    z[e] = 1.0f;
                else
                    z[e] = expf(lc[e] - m);
            }
            float S = 0.0f;
            for (int e = 0; e < E; ++e) S = S + z[e];
            for (int e = 0; e < E; ++e) {
                order[e].p = z[e] / S;
                order[e].e = e;
                if (probs) probs[(size_t)t * E + e] = order[e].p;
            }
            qsort(order, (size_t)E, sizeof(oref_pe), oref_cmp_pe);
            float s = 0.0f;
            for (int j = 0; j < k; ++j) s = s + order[j].p;
            for (int j = 0; j < k; ++j) {
                ids[(size_t)t * k + j] = order[j].e;
                w[(size_t)t * k + j] = renorm ? order[j].p / s : order[j].p;
            }
            if (gap_k) gap_k[t] = (k < E) ? order[k - 1].p - order[k].p : INFINITY;
            if (gap_in) {
                const int last = (k < E) ? k + 1 : k;
                float g = INFINITY;
                for (int r = 0; r + 1 < last; ++r) {
                    const float d = order[r].p - order[r + 1].p;
                    if (d < g) g = d;
                }
                gap_in[t] = g;
            }
        }
        free(z);
        free(lc);
        free(order);
    }
    return bad ? -2 : 0;
}

/* Routing weights of given ids (used when another router's choice differs
 * from this one's only inside a near-tie): the same softmax as oref_route,
 * then w_j = p[ids_j] / sum_{j'<k} p[ids_j'] (or p[ids_j] when renorm == 0).
 * Returns 0, or -1 on bad sizes or ids. */
OREF_EXPORT int oref_weights_for_ids(int T, int E, int k, int renorm, const float* logits,
                                     const int32_t* ids, float* w) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
    int bad = 0;
#pragma omp parallel
    {
        float* z = (float*)malloc(sizeof(float) * (size_t)E);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            if (!z) { bad = 1; continue; }
            const float* l = logits + (size_t)t * E;
            float m = -INFINITY;
            for (int e = 0; e < E; ++e) {
                const float v = isnan(l[e]) ? -INFINITY : l[e];
                if (v > m) m = v;
            }
            float S = 0.0f;
            for (int e = 0; e < E; ++e) {
                const float v = isnan(l[e]) ? -INFINITY : l[e];
                if (m == INFINITY)
                    z[e] = (v == INFINITY) ? 1.0f : 0.0f;
                else if (m == -INFINITY)
                    z[e] = 1.0f;
                else
                    z[e] = expf(v - m);
                S = S + z[e];
            }
            float s = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int e = ids[(size_t)t * k + j];
                if (e < 0 || e >= E) { bad = 1; break; }
                s = s + z[e] / S;
            }
            for (int j = 0; j < k; ++j) {
                const int e = ids[(size_t)t * k + j];
                if (e < 0 || e >= E) break;
                const float p = z[e] / S;
                w[(size_t)t * k + j] = renorm ? p / s : p;
            }
        }
        free(z);
    }
    return bad ? -1 : 0;
}

/* Permutation of the T*k routed assignments into expert-major order.
 *  counts[e]  = number of assignments to expert e
 *  offsets    = exclusive prefix sum of counts, offsets[E] = T*k
 *  Assignments a = t*k + j are visited in ascending a; each takes the next
 *  free slot of its expert:  sorted_token_ids[pos] = t,  inv_pos[a] = pos.
 *  Returns 0, or -1 if an id is outside [0, E). */
OREF_EXPORT int oref_permute(int T, int k, int E, const int32_t* ids, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_token_ids, int32_t* inv_pos) {
    const long A = (long)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long a = 0; a < A; ++a) {
        if (ids[a] < 0 || ids[a] >= E) return -1;
        counts[ids[a]] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    if (!cursor) return -2;
    for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            const long a = (long)t * k + j;
            const int e = ids[a];
            const int32_t pos = cursor[e];
            cursor[e] = pos + 1;
            sorted_token_ids[pos] = t;
            inv_pos[a] = pos;
        }
    }
    free(cursor);
    return 0;
}

static float oref_silu(float z) { return z / (1.0f + expf(-z)); }

/* One expert's SwiGLU FFN on n rows.
 *  xr [n,H]; w_gu [2I,H] (rows 0..I-1 W_gate^T, rows I..2I-1 W_up^T);
 *  w_dn [H,I] (W_down^T); y [n,H]:
 *    g_i = sum_h x_h W_gate[h,i],  u_i = sum_h x_h W_up[h,i]
 *    a_i = silu(g_i) * u_i,        y_c = sum_i a_i W_down[i,c]  */
OREF_EXPORT void oref_expert_ffn(int n, int H, int I, const float* xr, const float* w_gu,
                                 const float* w_dn, float* y) {
#pragma omp parallel
    {
        float* a = (float*)malloc(sizeof(float) * (size_t)I);
#pragma omp for schedule(static)
        for (int r = 0; r < n; ++r) {
            if (!a) continue;
            const float* x = xr + (size_t)r * H;
            for (int i = 0; i < I; ++i) {
                const float* wgate = w_gu + (size_t)i * H;
                const float* wup = w_gu + (size_t)(I + i) * H;
                float g = 0.0f, u = 0.0f;
                for (int h = 0; h < H; ++h) {
                    g = g + x[h] * wgate[h];
                    u = u + x[h] * wup[h];
                }
                a[i] = oref_silu(g) * u;
            }
            float* yr = y + (size_t)r * H;
            for (int c = 0; c < H; ++c) {
                const float* wd = w_dn + (size_t)c * I;
                float acc = 0.0f;
                for (int i = 0; i < I; ++i) acc = acc + a[i] * wd[i];
                yr[c] = acc;
            }
        }
        free(a);
    }
}

/* Weighted gather-combine back to token order.
 *  w [T,k]; y [T*k,H] with row t*k+j = FFN_{e_{t,j}}(x_t);
 *  shared [T,H] or NULL;  out[t,c] = shared[t,c] + sum_{j<k} w[t,j] y[t*k+j,c]
 *  (the routed sum is formed first, in ascending j, then added to shared). */
OREF_EXPORT void oref_combine(int T, int H, int k, const float* w, const float* y,
                              const float* shared, float* out) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < H; ++c) {
            float s = 0.0f;
            for (int j = 0; j < k; ++j)
                s = s + w[(size_t)t * k + j] * y[((size_t)t * k + j) * H + c];
            out[(size_t)t * H + c] = shared ? shared[(size_t)t * H + c] + s : s;
        }
    }
}

/* ---------------------------------------------------------------------------
 * MXFP8 expert weights (a variant of the layer with 8-bit routed expert
 * weights).  The pages mention FP8 scaling blocks (pwwt.cn article, section 6:
 * the gating kernels' accumulation is audited across FP8 scaling blocks) and
 * MX formats (first page, section 3: MXFP6 units), but fix no format for
 * expert weights.  Reading: the OCP Microscaling Formats (MX) specification
 * v1.0, format MXFP8 with E4M3 elements:
 *  - a block is 32 consecutive values of one weight row (along the reduction
 *    dimension: H for W_gate|up, I for W_down) and shares one E8M0 scale,
 *    code s8 meaning X = 2^(s8 - 127);
 *  - an element is an FP8 E4M3 number: sign, 4 exponent bits (bias 7),
 *    3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the
 *    largest finite magnitude is 1.75 * 2^8 = 448; S.1111.111 is NaN; there
 *    are no infinities.
 * Quantising a block (the specification's conversion rule, restated):
 *  - shared exponent s = floor(log2(max_i |v_i|)) - 8 (8 = exponent of the
 *    largest normal E4M3 value), clamped to [-127, 127]; an all-zero block
 *    takes -127;
 *  - element i = v_i / 2^s rounded to the nearest E4M3 value, ties to the
 *    even mantissa; magnitudes past 448 become 448 (saturation); the sign bit
 *    is the sign of v_i, so -0 and negative values rounding to 0 give 0x80.
 * Dequantised weight: value(code) * 2^s (exact in fp32).
 * Plain double arithmetic: frexp/ldexp are exact, nearbyint rounds half to
 * even in the default rounding mode.
 */
static double oref_e4m3_value(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);          /* m/8 * 2^-6 */
    else
        mag = ldexp(8.0 + m, e - 7 - 3);     /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

static uint8_t oref_e4m3_encode(double v) {
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double a = fabs(v);
    int ex = 0;
    /* exponent of the binade holding a; below 2^-6 the spacing stays that of
     * the subnormals, 2^-9 */
    int E = -6;
    if (a > 0.0) {
        frexp(a, &ex);                       /* a = f * 2^ex, f in [0.5, 1) */
        E = ex - 1;
        if (E < -6) E = -6;
    }
    /* round to a multiple of the spacing 2^(E-3) (3 mantissa bits) */
    double r = ldexp(nearbyint(ldexp(a, 3 - E)), E - 3);
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    frexp(r, &ex);
    const int Er = ex - 1;
    if (Er < -6) return (uint8_t)(sign | (uint8_t)ldexp(r, 9)); /* subnormal: m = r / 2^-9 */
    return (uint8_t)(sign | ((Er + 7) << 3) | (int)(ldexp(r, 3 - Er) - 8.0));
}

/* w [rows,K] fp32 (finite) -> codes [rows,K], scales [rows,K/32].
 * Returns 0, or 1 if K % 32 != 0, 2 on a non-finite input. */
OREF_EXPORT int oref_mxfp8_quantize(long rows, int K, const float* w, uint8_t* codes,
                                    uint8_t* scales) {
    if (K % 32 != 0) return 1;
    const int nb = K / 32;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (long r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const float* v = w + r * K + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                if (!isfinite(v[i])) bad = 1;
                if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
            }
            int s = -127;
            if (amax > 0.0) {
                int ex = 0;
                frexp(amax, &ex);
                s = ex - 1 - 8;
            }
            if (s < -127) s = -127;
            if (s > 127) s = 127;
            scales[r * nb + b] = (uint8_t)(s + 127);
            for (int i = 0; i < 32; ++i)
                codes[r * K + b * 32 + i] = oref_e4m3_encode(ldexp((double)v[i], -s));
        }
    }
    return bad ? 2 : 0;
}

/* codes [rows,K], scales [rows,K/32] -> out [rows,K] fp32. */
OREF_EXPORT void oref_mxfp8_dequantize(long rows, int K, const uint8_t* codes,
                                       const uint8_t* scales, float* out) {
    const int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r)
        for (int i = 0; i < K; ++i)
            out[r * K + i] =
                (float)ldexp(oref_e4m3_value(codes[r * K + i]), (int)scales[r * nb + i / 32] - 127);
}
