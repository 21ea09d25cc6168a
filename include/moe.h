/*
 * moe.h -- C ABI of libmoe.so, the MI355X (gfx950) sparse mixture-of-experts
 * layer: router GEMM -> softmax -> top-k -> permute -> grouped SwiGLU expert
 * FFN (gate|up, then down) -> weighted gather-combine.
 *
 * The calls follow the statement of the problem on the source pages:
 *  - pwwt.cn article on optimising Qwen 3.5-397B MoE on Ironwood (TPU v7x):
 *      section 8.2  router logits are computed, then top-k selects experts;
 *      section 4.2  top_k = 10 is not a power of 2, so permuting the routed
 *                   rows must not pad; token rows are gathered by routing
 *                   index into one contiguous buffer without a padded
 *                   intermediate; the grouped expert GEMM fuses SwiGLU into
 *                   its matmul and bounds each expert's slice by its own
 *                   token count;
 *      section 7.2  the routed rows are un-permuted and gather-reduced back
 *                   into token order.
 *  - lumevalley.com article on SGLang-JAX serving Ling-2.6-1T, opening
 *    paragraph: top-8 routing plus an always-on shared expert.
 *  - yuxiaoba.github.io summary of "Optimizing Muse Spark Open on TPU v7
 *    with SGLang-TorchTPU", section on changing dependencies: experts with
 *    few rows run a loop of their own, separate from the heavy-row loop, and
 *    the output stays bitwise identical.
 *
 * Conventions shared by every call
 *  - Shapes: T tokens, H hidden, E routed experts, k experts per token,
 *    I expert intermediate size, A = T*k routed rows.  All arrays are dense
 *    row-major.  "bf16" arrays hold raw bfloat16 bit patterns (uint16_t).
 *  - Pointers are DEVICE pointers (HIP device memory, 16-byte aligned) unless
 *    stated otherwise; `shape` is a HOST pointer.  The caller owns every
 *    buffer; the library allocates nothing and keeps no state between calls
 *    except a per-device cache of the compute-unit count.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; no call synchronises the stream or
 *    reads device memory on the host.  A fault inside a kernel surfaces at
 *    the caller's next synchronisation, as usual for HIP.
 *  - Scratch memory comes from `workspace` (device, 256-byte aligned) of at
 *    least moe_workspace_bytes(shape) bytes.  Calls on one stream may reuse
 *    one workspace; calls that may overlap need separate workspaces.
 *  - Return value: MOE_OK, or an error code below; on error nothing has
 *    been enqueued (argument errors) or the failing launch is reported
 *    (MOE_ERR_HIP).  moe_last_error() gives a text for the calling thread.
 *  - Results are bitwise deterministic for identical inputs, shape, device
 *    and build: no floating-point atomics are used anywhere.
 *  - Supported sizes: T >= 0 (T == 0 is a no-op), H % 64 == 0,
 *    I % 32 == 0, 1 <= k <= min(E, 32), E <= 1024, T*k < 2^31,
 *    T*H < 2^31, I*H < 2^30 and I_shared*H < 2^30 (byte offsets into x and
 *    into one expert's weights fit 32 bits), I_shared % 32 == 0 (or 0).  With T == 0 the activation and output
 *    pointers may be NULL; only moe_permute (and moe_forward's counts_out)
 *    write anything: all-zero counts and offsets.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,       /* a size is negative/zero where it must not be, k > E, T*k overflow */
    MOE_ERR_UNSUPPORTED = 3, /* valid but outside the supported sizes listed above */
    MOE_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned (workspace: 256) */
    MOE_ERR_WORKSPACE = 5,   /* ws_bytes < moe_workspace_bytes(shape) */
    MOE_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed */
};

typedef struct moe_shape {
    int32_t T;              /* tokens */
    int32_t H;              /* hidden size */
    int32_t E;              /* routed experts */
    int32_t k;              /* experts per token */
    int32_t I;              /* routed expert intermediate size */
    int32_t I_shared;       /* shared expert intermediate size; 0 = no shared expert */
    int32_t renorm;         /* 1: selected weights renormalised to sum to 1; 0: raw probabilities */
    int32_t light_max_rows; /* experts with 1..light_max_rows rows take the light-row loop,
                               the others the heavy tiles; 0 = every expert takes the heavy
                               tiles; at most 64.  When each token's ids are distinct
                               (always so in moe_forward) an expert gets at most T
                               rows, so with T <= light_max_rows no heavy kernel runs.
                               -1 = library default: with T <= 64 every expert takes the
                               light loop (no heavy kernel runs); with more tokens the
                               device decides per call from the routing: experts with up
                               to 64 rows take the light loop when the routed rows
                               average at most 8 per touched expert, otherwise only
                               experts with up to 8 rows do and the others take the
                               heavy tiles (faster on MI355X from about 10 rows per
                               expert on); with T*k > 8*E always the latter.  Results
                               do not depend on it. */
    int32_t heavy_tile_rows; /* rows per heavy tile: 0 = chosen per expert from its row
                               count (equal tiles of the one height among 256, 224, 192,
                               160 and 128 with the least estimated time); 128, 160, 192,
                               224 or 256 = every tile that height.  Results do not
                               depend on it. */
    int32_t y_bf16;         /* storage of the routed expert outputs y: 0 = fp32, 1 = bf16
                               (round to nearest even).  bf16 halves the y round trip
                               between the down GEMM and the combine (2*T*k*H bytes less
                               written and read); it rounds each y to 8 significant bits
                               before the fp32 weighted sum, so it suits layers whose
                               |y| are small against the output tolerance.  The shared
                               expert's output is always fp32. */
    int32_t w_mxfp8;        /* routed expert weights: 0 = bf16 (w_gate_up / w_down, optionally
                               packed); 1 = MXFP8, given only as the packed buffer of
                               moe_pack_weights_mxfp8 (see there).  With 1 the light/heavy
                               choice is as for bf16 but heavy tiles are at most 192 rows
                               (heavy_tile_rows = 256 is MOE_ERR_UNSUPPORTED), and the results
                               are those of the bf16 path on the dequantised weights, bit for
                               bit.  The shared expert stays bf16. */
    int32_t y_fp16;         /* 1: the routed expert outputs y are stored as fp16 (round to
                               nearest even) instead: the same bytes as bf16 with 11
                               significant bits, for layers whose |y| stay well below
                               65504 (larger values round to infinity).  Exclusive with
                               y_bf16 (both 1: MOE_ERR_UNSUPPORTED). */
} moe_shape;

/* Bytes of workspace every call below needs for `shape` (host-only, pure;
 * returns 0 for an invalid shape). */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Bytes of the packed expert-weight buffer for `shape` (host-only, pure;
 * 0 for an invalid shape).  bf16 (w_mxfp8 = 0): one copy of W_gate|up and
 * W_down, 2 bytes per weight with weight rows padded to a multiple of 256
 * and K to a multiple of 64 (E * 3 * I * H * 2 when 2I and H are multiples
 * of 256 and I of 64).  MXFP8 (w_mxfp8 = 1): two copies (light loop, heavy
 * tiles) of one byte per weight (K padded to a multiple of 64, the heavy
 * copy's weight rows to a multiple of 256) plus one scale byte per 32
 * weights. */
size_t moe_packed_weight_bytes(const moe_shape* shape);

/* Static text for a status code. */
const char* moe_status_string(int status);

/* Text describing the calling thread's most recent failed call ("" if none). */
const char* moe_last_error(void);

/* Router: logits = x . w_router (+ bias) in fp32; softmax over the E experts;
 * top-k by descending probability, the lower expert index winning ties;
 * weights renormalised over the k selected (shape->renorm).
 * (pwwt.cn article, sections 4.2 and 8.2.)
 *   x        bf16 [T,H]
 *   w_router fp32 [H,E]
 *   bias     fp32 [E] added to the logits, or NULL
 *   topk_ids int32 [T,k] out: expert ids in descending-probability order,
 *            distinct, in [0,E) for every input (NaN logits count as -inf)
 *   topk_w   fp32 [T,k] out: routing weights
 *   probs    fp32 [T,E] out: softmax probabilities, or NULL
 */
int moe_router(const moe_shape* shape, const uint16_t* x, const float* w_router,
               const float* bias, int32_t* topk_ids, float* topk_w, float* probs,
               void* workspace, size_t ws_bytes, void* stream);

/* Permute: per-expert histogram, exclusive scan, stable scatter of the
 * routed rows into expert-major order (no padding; pwwt.cn section 4.2).
 *   topk_ids         int32 [T,k] in: ids in [0,E) (others are skipped:
 *                    not counted, inv_pos = -1)
 *   counts           int32 [E]   out: rows per expert
 *   offsets          int32 [E+1] out: exclusive prefix of counts
 *   sorted_token_ids int32 [T*k] out: token of each expert-major row; within
 *                    an expert, rows keep ascending assignment order t*k+j
 *   inv_pos          int32 [T*k] out: expert-major row of assignment t*k+j
 */
int moe_permute(const moe_shape* shape, const int32_t* topk_ids, int32_t* counts,
                int32_t* offsets, int32_t* sorted_token_ids, int32_t* inv_pos,
                void* workspace, size_t ws_bytes, void* stream);

/* Optional one-time re-layout of the routed expert weights (the expert
 * weights are constant across calls, as a serving engine loads them once),
 * read by both the light loop and the heavy tiles.  One 32 KB record per
 * (expert e, 256-row weight tile nb, 64-wide K stage c), ordered (e, nb, c),
 * W_gate|up's records first, then W_down's.  A record's 256 tile rows --
 * gate|up: 16-row blocks alternating between the gate rows and the up rows
 * of h columns nb*128 + 16p .. +15 (block 2p gate, 2p+1 up); down: W_down
 * rows nb*256 + r -- form 16 row blocks j, each two 1 KB chunks (K values
 * 64c..64c+31, then 64c+32..64c+63), each chunk one bf16 MFMA operand in
 * lane order (lane l: row 16j + l%16, K values 8(l/16)..+7 of the chunk).
 * Zeros past the weights (rows padded to 256, K to 64).  A heavy stage is
 * then one contiguous 32 KB read and a light wave's operand one contiguous
 * 1 KB read, where the row-major layout's 16-row operands read 64 bytes
 * from each of 16 rows a whole weight row apart.
 *   w_gate_up, w_down  bf16, layouts as for moe_grouped_ffn (read)
 *   packed             device buffer of moe_packed_weight_bytes(shape)
 *                      bytes, 256-byte aligned (written; caller-owned)
 * Enqueued on `stream`; the packed buffer may be passed to moe_grouped_ffn
 * and moe_forward once that work has completed (the plain weights are then
 * optional there and may be freed).  Results are bitwise identical with and
 * without it. */
int moe_pack_weights(const moe_shape* shape, const uint16_t* w_gate_up, const uint16_t* w_down,
                     void* packed, void* stream);

/* MXFP8 quantisation of bf16 weight rows (a variant with 8-bit routed expert
 * weights; the pages name FP8 scaling blocks -- pwwt.cn article, section 6 --
 * and MX formats -- first page, section 3 -- but fix no weight format).
 * Format: OCP Microscaling Formats (MX) specification v1.0, MXFP8 with E4M3
 * elements: each 32 consecutive values of a row share an E8M0 scale code s8
 * (X = 2^(s8 - 127)); each value is an E4M3 code (bias 7, 3 mantissa bits,
 * largest finite 448).  Per block, as the specification converts:
 * shared exponent floor(log2 max|v|) - 8 clamped to [-127, 127] (an all-zero
 * block: -127); value / X rounded to the nearest E4M3 value, ties to the
 * even mantissa, saturated at +-448, sign kept (also for zero).
 *   w       bf16 [rows,K], finite (codes of non-finite values are unspecified)
 *   codes   uint8 [rows,K] out (16-byte aligned)
 *   scales  uint8 [rows,K/32] out (any alignment)
 * K % 32 == 0 (else MOE_ERR_UNSUPPORTED); rows == 0 is a no-op.  For expert
 * weights pass W_gate|up as rows = E*2I, K = H and W_down as rows = E*H,
 * K = I (blocks run along the reduction dimension). */
int moe_quantize_mxfp8(const uint16_t* w, int64_t rows, int32_t K, uint8_t* codes,
                       uint8_t* scales, void* stream);

/* Packs MXFP8 expert weights (codes and scales as moe_quantize_mxfp8 writes
 * them for W_gate|up [E,2I,H] and W_down [E,H,I]) for the light loop, into
 * `packed` (moe_packed_weight_bytes(shape) bytes, 256-byte aligned) with
 * shape->w_mxfp8 = 1.  Two copies: for the light loop, codes in 1 KB chunks
 * of 16 weight rows x 64 K in lane order (lane l: row l%16, the codes of K
 * 8(l/16)..+7 of the chunk's first 32-wide K step, then of its second), rows
 * grouped as for moe_pack_weights, each chunk's scales 32 bytes (row r's two
 * steps at 2r, 2r+1); for the heavy tiles, one record per (expert, 256-row
 * weight tile, 64-wide K chunk): the tile rows' 64 codes each, then their
 * 512 scale bytes.  The result is passed to moe_grouped_ffn / moe_forward as
 * packed_weights. */
int moe_pack_weights_mxfp8(const moe_shape* shape, const uint8_t* codes_gate_up,
                           const uint8_t* scales_gate_up, const uint8_t* codes_down,
                           const uint8_t* scales_down, void* packed, void* stream);

/* Grouped expert FFN over the expert-major rows (pwwt.cn section 4.2):
 *   h[r,:] = bf16( silu(x[tok_r] . W_gate[e]) * (x[tok_r] . W_up[e]) )
 *   y[r,:] = h[r,:] . W_down[e]   (fp32 sum)      for rows r of expert e,
 * bf16 MFMA with fp32 accumulation; token rows are gathered inside the GEMM.
 * Experts with 1..light_max_rows rows run the light-row loop, the others
 * the heavy tiles; both give bitwise identical rows.  Any moe_permute output
 * is accepted, including ids repeated within a token (an expert may then
 * hold more than T rows).
 *   x                bf16 [T,H]
 *   sorted_token_ids int32 [T*k], offsets int32 [E+1]  (from moe_permute)
 *   w_gate_up        bf16 [E,2I,H]: rows 0..I-1 = W_gate^T, I..2I-1 = W_up^T
 *   w_down           bf16 [E,H,I]:  W_down^T
 *   packed_weights   the same weights from moe_pack_weights, or NULL; when
 *                    given, the light loop and the heavy tiles read it
 *                    instead of w_gate_up / w_down, which are then not read
 *                    and may be NULL (a caller may keep only the packed
 *                    copy resident).  With shape->w_mxfp8 = 1 it is
 *                    required (from moe_pack_weights_mxfp8)
 *   h                bf16 [T*k,I] out, or NULL (then kept in the workspace)
 *   y                [T*k,H] out: fp32 (shape->y_bf16 == y_fp16 == 0; large |y|
 *                    entering the weighted sum keep 24 significant bits), bf16
 *                    (shape->y_bf16 == 1) or fp16 (shape->y_fp16 == 1), rounded
 *                    to nearest even
 */
int moe_grouped_ffn(const moe_shape* shape, const uint16_t* x,
                    const int32_t* sorted_token_ids, const int32_t* offsets,
                    const uint16_t* w_gate_up, const uint16_t* w_down,
                    const void* packed_weights, uint16_t* h, void* y, void* workspace,
                    size_t ws_bytes, void* stream);

/* Shared expert (lumevalley.com Ling-2.6-1T article): one dense SwiGLU FFN
 * over all T tokens through the same heavy GEMM kernels, written in fp32:
 *   h = silu(x W_gate_s) * (x W_up_s),  out[t,:] = h W_down_s
 * Because this output enters the layer with weight 1, h is kept as a pair
 * of bf16 values (hi + lo, ~16 significant bits) and the down GEMM runs
 * over both halves against the same weights.
 *   ws_gate_up bf16 [2*I_shared,H], ws_down bf16 [H,I_shared], out fp32 [T,H]
 * Requires shape->I_shared > 0. */
int moe_shared_ffn(const moe_shape* shape, const uint16_t* x, const uint16_t* ws_gate_up,
                   const uint16_t* ws_down, float* out, void* workspace, size_t ws_bytes,
                   void* stream);

/* Weighted gather-combine back to token order (pwwt.cn section 7.2):
 *   s[t,c]   = sum_{j<k} topk_w[t,j] * y[inv_pos[t*k+j], c]   (ascending j,
 *              fp32; rows with inv_pos < 0 are skipped)
 *   out[t,c] = accumulate ? out[t,c] + s[t,c] : s[t,c]
 *   y [T*k,H] fp32, bf16 or fp16 as shape->y_bf16 / y_fp16 say, inv_pos int32 [T*k],
 *   topk_w fp32 [T,k], out fp32 [T,H].  No workspace. */
int moe_combine(const moe_shape* shape, const void* y, const int32_t* inv_pos,
                const float* topk_w, int32_t accumulate, float* out, void* stream);

/* The whole layer: router, permute, grouped FFN, shared expert (when
 * shape->I_shared > 0), combine.  out fp32 [T,H]:
 *   out[t] = sum_j w[t,j] FFN_{ids[t,j]}(x[t])  (+ FFN_shared(x[t]))
 * (pwwt.cn article on Qwen 3.5-397B MoE on Ironwood: section 8.2 routing,
 * section 4.2 permute and grouped SwiGLU FFN, section 7.2 un-permute and
 * gather-reduce; lumevalley.com Ling-2.6-1T article, opening paragraph: the
 * shared expert added to the routed sum.)
 * ws_gate_up / ws_down are required iff I_shared > 0; packed_weights is
 * optional, as for moe_grouped_ffn (required with shape->w_mxfp8 = 1); when
 * it is given, w_gate_up / w_down are not read and may be NULL.  topk_ids_out [T,k],
 * topk_w_out [T,k] and counts_out [E] are optional copies of the routing
 * (NULL = not written).
 * Streams: with a shared expert, its two GEMMs run on a side stream the
 * library keeps per device (default priority, non-blocking, created at the
 * first such call), which waits for an event recorded on `stream` before
 * the router and which `stream` waits for before the combine: the shared
 * expert, which needs only x, runs beside the routing and the routed FFN
 * (after the yuxiaoba.github.io summary of "Optimizing Muse Spark Open on
 * TPU v7 with SGLang-TorchTPU", section on chaining one verify pass's 62
 * layers into a continuous data flow: weight traffic does not wait for
 * work it does not depend on).
 * All work is ordered after what `stream` held at the call and before what
 * it is given next, also under HIP graph capture; calls from several host
 * threads on one device are serialised between fork and join. */
int moe_forward(const moe_shape* shape, const uint16_t* x, const float* w_router,
                const float* bias, const uint16_t* w_gate_up, const uint16_t* w_down,
                const void* packed_weights, const uint16_t* ws_gate_up, const uint16_t* ws_down,
                float* out,
                int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                void* workspace, size_t ws_bytes, void* stream);

/* Size of the fixed scratch array behind moe_forward_noalloc (per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_forward for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * layer, arguments and results as moe_forward, with no workspace argument:
 * the scratch memory is a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on holds
 * until the process ends.  Its device address is looked up once per device
 * (hipGetSymbolAddress, on the first call made with that device current);
 * no call allocates or frees memory.  Shapes whose moe_workspace_bytes
 * exceeds the array are rejected with MOE_ERR_WORKSPACE before anything is
 * enqueued (64 MiB covers, e.g., a decode step of 64 tokens at H = 4096,
 * E = 512, k = 10, I = 1024 with fp32 y).  Every call on one GPU uses that
 * GPU's one array and leaves its contents behind (no step relies on them
 * being zero): calls that may overlap on one GPU -- on different streams,
 * or from different host threads -- race on it and must be serialised by
 * the caller.  All its work, the shared expert's too, goes on `stream`: no
 * stream or event is created. */
int moe_forward_noalloc(const moe_shape* shape, const uint16_t* x, const float* w_router,
                        const float* bias, const uint16_t* w_gate_up, const uint16_t* w_down,
                        const void* packed_weights, const uint16_t* ws_gate_up,
                        const uint16_t* ws_down, float* out, int32_t* topk_ids_out,
                        float* topk_w_out, int32_t* counts_out, void* stream);

/* Kernels of the layer, for moe_profile_kernel. */
enum moe_kernel {
    MOE_K_ROUTER_GEMM = 0,
    MOE_K_ROUTER_SELECT = 1,
    MOE_K_PERM_COUNT = 2,
    MOE_K_PERM_SCAN = 3,
    MOE_K_PERM_SCATTER = 4,
    MOE_K_FFN_PLAN = 5,
    MOE_K_GATEUP_LIGHT = 6,
    MOE_K_GATEUP_HEAVY = 7,
    MOE_K_DOWN_LIGHT = 8,
    MOE_K_DOWN_HEAVY = 9,
    MOE_K_COMBINE = 10,
    MOE_K_PERM_SMALL = 11, /* whole permute in one block when T*k <= 4096 */
    MOE_K_COUNT = 12
};

/* Measurement hook (process-wide, not thread-safe): from now on every launch
 * of kernel `kernel` (an enum moe_kernel value) is bracketed by
 * hipEventRecord(start) and hipEventRecord(stop) on the stream it is launched
 * on.  `start` and `stop` are caller-created hipEvent_t handles passed as
 * void*.  kernel = -1 turns the hook off.  If a call launches the kernel more
 * than once (the shared expert reuses the heavy kernels), the events bracket
 * the last launch.  Returns MOE_OK, or MOE_ERR_SHAPE for an unknown kernel,
 * MOE_ERR_NULL for a NULL event while turning the hook on. */
int moe_profile_kernel(int kernel, void* start, void* stop);

/* As moe_profile_kernel, but only the launch-th launch (0-based, counted from
 * this call) of the kernel is bracketed; launch = -1 brackets every launch.
 * moe_forward launches the heavy GEMM kernels twice when the layer has a
 * shared expert: launch 0 runs the routed experts, launch 1 the shared one.
 * MOE_ERR_SHAPE for launch < -1, otherwise as moe_profile_kernel. */
int moe_profile_kernel_launch(int kernel, int launch, void* start, void* stop);

/* Launches of the hooked kernel since the last moe_profile_kernel call. */
long long moe_profile_launches(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
