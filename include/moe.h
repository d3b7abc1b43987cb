/*
 * moe.h — C ABI of libmoe: the routed mixture-of-experts FFN layer over
 * group-quantized expert weights, for AMD Instinct MI355X (gfx950).
 *
 * The layer: top-k routing of each token over E experts, grouping the T*k
 * routed slots by expert, a grouped gate/up projection with weights used as
 * stored (int4 codes dequantized in registers, or int8 x int8), SwiGLU, a
 * grouped down projection, and a weighted combine of each token's k expert
 * outputs. Sources of each step are cited at its entry point:
 *   [PV-fast]   page "Performance and verification", section "Why it is fast"
 *               (each active expert's weights are streamed once per call for
 *               all of the rows routed to it; one grouped launch covers all
 *               experts; the quantized weights enter the dot products as
 *               stored; prompt-sized batches of routed experts run as grouped
 *               int8 tensor-core GEMMs; a decode step is one graph with no
 *               host synchronization inside).
 *   [PV-verify] same page, section "How it is verified" (router ids and other
 *               integer outputs exact; floats within rounding bands).
 *   [MR]        page "Measured results" (header: W4A16 g128 weights; "Speed":
 *               W4A16 / W4A8 paths; "Memory": one weight layout, not two).
 *   [MS]        forum post "DeepSeek V4.1 Flash TP2 Spark running w/ spec
 *               decoding", section "MOE Streaming" (a per-layer host check
 *               drains the GPU pipeline; here nothing syncs inside a layer).
 *
 * Conventions (all entry points):
 *   - Every call returns a moe_status; MOE_OK means the work was enqueued.
 *   - Tensor pointers are DEVICE pointers to row-major contiguous arrays,
 *     16-byte aligned. bf16 and fp16 travel as uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Every call validates its arguments on the host first; a non-OK return
 *     means nothing was enqueued. On MOE_OK the work is enqueued on `stream`
 *     and the call returns without synchronizing. Device faults, if any,
 *     surface at the caller's next synchronization.
 *   - Ownership: the caller owns every buffer, including workspaces sized by
 *     the *_workspace queries; the library keeps no pointer past the call and
 *     allocates nothing. Buffers must stay alive until the stream work ends.
 *     Outputs must not alias inputs; inputs are never written.
 *   - Calls on distinct streams with distinct workspaces may run concurrently.
 *   - Numerics are deterministic: integer atomics only (counts, maxima), no
 *     float atomics; two runs on the same inputs give identical bits.
 *   - T = 0 is a valid empty batch. T*k*max(H, I) and 2*H*I must stay below
 *     2^31 (32-bit element offsets); H and I are at most MOE_MAX_DIM (a grouped
 *     GEMM block holds the scales of its 256 weight rows in LDS).
 *   - Out-of-range expert ids or non-finite logits are outside the contract.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32
#define MOE_GROUP 128
#define MOE_MAX_DIM 16384   /* largest H and I of the FFN and layer calls */

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* null pointer or invalid scalar argument            */
  MOE_ESHAPE = 2,       /* shape outside the supported set                    */
  MOE_EALIGN = 3,       /* pointer not 16-byte aligned                        */
  MOE_EWORKSPACE = 4,   /* workspace smaller than the *_workspace query       */
  MOE_EUNSUPPORTED = 5, /* current device is not gfx950 (no other path)       */
  MOE_EDEVICE = 6       /* HIP runtime error; text in moe_last_error()        */
} moe_status;

/* Static string for a status code. */
MOE_API const char* moe_status_str(moe_status status);
/* Detail of the last non-OK status returned on this thread ("" if none). */
MOE_API const char* moe_last_error(void);
MOE_API int moe_abi_version(void);

/*
 * moe_router_logits — router projection ahead of the top-k. [PV-verify]
 * (router ids exact: they are decided on these logits)
 * logits[t, e] = sum_h x[t, h] * w_router[e, h]: bf16 x bf16 products, exact
 * in float32, accumulated in float32 in a fixed order (deterministic; the
 * order differs between T <= 8 and larger T).
 *   x        bf16    [T, H]  (input)
 *   w_router bf16    [E, H]  (input; row e is expert e's router row)
 *   logits   float32 [T, E]  (output; feeds moe_route_topk or moe_layer_w4a16)
 * Requires H % 64 == 0, 1 <= E <= MOE_MAX_EXPERTS, T >= 0.
 */
MOE_API moe_status moe_router_logits(const uint16_t* x, const uint16_t* w_router, int32_t T,
                      int32_t H, int32_t E, float* logits, void* stream);

/*
 * moe_route_topk — top-k routing. [PV-verify] (router ids exact)
 * For each token t: topk_ids[t, 0..k) = the k largest logits[t, :] in
 * descending order, ties broken by the lower expert index (+0.0 and -0.0 are
 * equal); topk_w[t, j] = softmax over the k selected logits, float32.
 *   logits   float32 [T, E]  (input)
 *   topk_ids int32   [T, k]  (output)
 *   topk_w   float32 [T, k]  (output)
 * Requires 1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E, MOE_MAX_TOPK), T >= 0.
 */
MOE_API moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                   int32_t* topk_ids, float* topk_w, void* stream);

/*
 * moe_permute — group the R = T*k routed slots by expert. [PV-fast] (each
 * routed expert read once per batch; grouped dispatch)
 * Flat slot f = t*k + j carries expert topk_ids[t, j]. Outputs:
 *   expert_offsets int32 [E+1]: exclusive prefix sum of per-expert counts;
 *                               expert_offsets[E] = R.
 *   sorted_slot    int32 [R]:   flat slot at each position of the grouped
 *                               order; stable (within an expert, f ascends).
 *   slot_pos       int32 [R]:   inverse map, slot_pos[sorted_slot[p]] = p.
 *   active         int32 [min(E,R)]: experts with a nonzero count, ascending;
 *                               entries past n_active are left unwritten.
 *   n_active       int32 [1]
 * All outputs are bit-exact (integer counting sort). `ws` must hold
 * moe_permute_workspace(T, E, k) bytes (may be NULL when that is 0).
 * Ids must lie in [0, E).
 */
MOE_API size_t moe_permute_workspace(int32_t T, int32_t E, int32_t k);
MOE_API moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k,
                int32_t* expert_offsets, int32_t* sorted_slot, int32_t* slot_pos,
                int32_t* active, int32_t* n_active,
                void* ws, size_t ws_bytes, void* stream);

typedef struct {
  int32_t T; /* tokens                  */
  int32_t H; /* hidden size             */
  int32_t I; /* expert intermediate size */
  int32_t E; /* experts                 */
  int32_t k; /* experts per token       */
} moe_shape;

/*
 * moe_grouped_w4a16_ffn — grouped SwiGLU expert FFN, W4A16 g128. [MR] (format,
 * one weight layout for decode and prefill) [PV-fast] (weights as stored,
 * each routed expert read once per call)
 * For every grouped position p in [0, R), with e the expert whose block holds
 * p and t = sorted_slot[p] / k:
 *   gate = x[t] . W13[e][n]^T,  up = x[t] . W13[e][I + n]^T   (n < I)
 *   h[p, n] = silu(gate) * up
 *   y[p, :] = h[p] . W2[e]^T                    (stored float32, grouped order)
 * Weight format: codes packed two per byte along K (low nibble = even k),
 * implicit zero point 8, one fp16 scale per (output row, 128-wide K group):
 *   W[n, k] = (q[n, k] - 8) * scale[n, k / 128].
 *   x   bf16  [T, H]
 *   w13 uint8 [E, 2I, H/2]     s13 fp16 [E, 2I, H/128]   (rows [0,I) gate, [I,2I) up)
 *   w2  uint8 [E, H, I/2]      s2  fp16 [E, H, I/128]
 *   expert_offsets, sorted_slot, active, n_active: as written by moe_permute.
 *   y   float32 [T*k, H]       (output, grouped order)
 * Accumulation is float32; h is rounded to bf16 between the two projections
 * (it is the bf16 MFMA operand of the down projection); y stays float32.
 * Requires H % 128 == 0, I % 128 == 0. `ws` must hold
 * moe_w4a16_workspace(shape) bytes. Small T runs a register-dequant grouped
 * GEMV; larger T a bf16 MFMA grouped GEMM; both meet the same tolerance.
 */
MOE_API size_t moe_w4a16_workspace(const moe_shape* shape);
MOE_API moe_status moe_grouped_w4a16_ffn(const moe_shape* shape, const uint16_t* x,
                          const uint8_t* w13, const uint16_t* s13,
                          const uint8_t* w2, const uint16_t* s2,
                          const int32_t* expert_offsets, const int32_t* sorted_slot,
                          const int32_t* active, const int32_t* n_active,
                          float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_w4a16 — the whole W4A16 layer in one call, with the outputs of
 * moe_route_topk (topk_ids, topk_w), moe_permute (expert_offsets,
 * sorted_slot, slot_pos, active, n_active), moe_grouped_w4a16_ffn (y) and
 * moe_combine (out), computed by the same definitions. [PV-fast] (one graph
 * per decode step, no host synchronization inside) [MS] (no per-layer host
 * probe)
 * For T <= 4 (decode) it runs two kernels instead of the five launches of the
 * separate calls. In the first, every block routes all T tokens itself, finds
 * which rows of the grouped order its expert owns, and runs its gate/up units,
 * writing h; one extra block, the last of the grid, does no GEMV work and
 * writes the routing outputs, the permutation and a per-expert record for the
 * second kernel. In the second, each block owns a tile of output rows of H for
 * every active expert: it stages all routed h rows in LDS, keeps every expert
 * output of its tile there, and takes the combine for its rows inside the
 * block, summing the k picks in increasing j (the order of moe_combine). No
 * counters, atomics or fences cross blocks.
 * For larger T it enqueues the four steps. `logits` float32 [T, E]; other
 * arguments as in the individual calls. Requires H % 128 == 0, I % 128 == 0.
 * `ws` must hold moe_layer_w4a16_workspace(shape) bytes.
 */
MOE_API size_t moe_layer_w4a16_workspace(const moe_shape* shape);
MOE_API moe_status moe_layer_w4a16(const moe_shape* shape, const float* logits, const uint16_t* x,
                            const uint8_t* w13, const uint16_t* s13,
                            const uint8_t* w2, const uint16_t* s2,
                            int32_t* topk_ids, float* topk_w,
                            int32_t* expert_offsets, int32_t* sorted_slot,
                            int32_t* slot_pos, int32_t* active, int32_t* n_active,
                            float* y, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_w4a16_noalloc — moe_layer_w4a16 for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments minus the workspace, same kernels and outputs
 * (bit for bit); the layer's workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends. The call allocates nothing. A shape whose
 * moe_layer_w4a16_workspace() exceeds MOE_NOALLOC_SCRATCH_BYTES is refused
 * with MOE_EWORKSPACE before anything is enqueued. Every call on one GPU
 * shares that GPU's array, which keeps the last call's contents: calls that
 * overlap in time on one GPU (other streams, other host threads) race, so the
 * caller must order them. Nothing in the array needs to start at zero (each
 * call writes what it reads). The first call on a device looks up the array's
 * address there (MOE_EDEVICE if that fails).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
MOE_API moe_status moe_layer_w4a16_noalloc(const moe_shape* shape, const float* logits,
                                           const uint16_t* x, const uint8_t* w13,
                                           const uint16_t* s13, const uint8_t* w2,
                                           const uint16_t* s2, int32_t* topk_ids, float* topk_w,
                                           int32_t* expert_offsets, int32_t* sorted_slot,
                                           int32_t* slot_pos, int32_t* active, int32_t* n_active,
                                           float* y, float* out, void* stream);

/* Optional W8A8 intermediate outputs (device pointers; any may be NULL). */
typedef struct {
  int8_t* xq;     /* [T, H]   per-token int8 activations                 */
  float* xs;      /* [T]      their scales                               */
  int32_t* acc13; /* [R, 2I]  gate/up int32 accumulators, grouped order   */
  int8_t* hq;     /* [R, I]   per-row int8 SwiGLU output                 */
  float* hs;      /* [R]      its scales                                 */
  int32_t* acc2;  /* [R, H]   down int32 accumulators, grouped order      */
} moe_w8a8_debug;

/*
 * moe_grouped_w8a8_ffn — grouped SwiGLU expert FFN, int8 x int8 on int8 MFMA.
 * [PV-fast] (routed experts of a prompt as grouped int8 tensor-core GEMMs)
 * Each token row of x is quantized per row: s = absmax / 127 (float32, IEEE
 * division), q = round-half-even(x / s) clamped to [-127, 127] (s = 0 and
 * q = 0 for an all-zero row). Then, per grouped position p (expert e, token t):
 *   acc13[p, n] = sum_k xq[t, k] * w13[e, n, k]              (exact int32)
 *   gate = acc13[p, n] * xs[t] * s13[e, n], up likewise with row I + n
 *   h[p, n] = silu(gate) * up       (float32), quantized per row by the same
 *                                   rule -> hq[p, :], hs[p]
 *   acc2[p, m] = sum_n hq[p, n] * w2[e, m, n]                (exact int32)
 *   y[p, m] = acc2[p, m] * hs[p] * s2[e, m]                  (float32)
 *   x   bf16 [T, H]; w13 int8 [E, 2I, H], s13 float32 [E, 2I];
 *   w2  int8 [E, H, I], s2 float32 [E, H]; y float32 [T*k, H] (grouped order).
 * Requires H % 16 == 0, I % 16 == 0 (K tails shorter than the GEMM's 64-wide
 * stage are zero-filled). `dbg` may be NULL; non-NULL members receive the
 * intermediates. `ws` must hold moe_w8a8_workspace(shape) bytes.
 */
MOE_API size_t moe_w8a8_workspace(const moe_shape* shape);
MOE_API moe_status moe_grouped_w8a8_ffn(const moe_shape* shape, const uint16_t* x,
                         const int8_t* w13, const float* s13,
                         const int8_t* w2, const float* s2,
                         const int32_t* expert_offsets, const int32_t* sorted_slot,
                         const int32_t* active, const int32_t* n_active,
                         float* y, const moe_w8a8_debug* dbg,
                         void* ws, size_t ws_bytes, void* stream);

typedef struct {
  int8_t* xq;     /* [T, H]   per-token int8 activations                 */
  float* xs;      /* [T]      their scales                               */
  int8_t* hq;     /* [R, I]   per-row int8 h, grouped order (R = T*k)     */
  float* hs;      /* [R]      its scales                                 */
} moe_w4a8_debug;

/*
 * moe_grouped_w4a8_ffn — grouped SwiGLU expert FFN, int4 g128 weights x int8
 * activations on int8 MFMA. [MR] (W4A8 beside W4A16; one weight layout)
 * Weights are the W4A16 storage (codes q, W = (q - 8) * s per 128-wide K
 * group). Token rows are quantized as for W8A8 (absmax / 127, half-even,
 * [-127, 127]). Per grouped position p (expert e, token t), output n:
 *   gate = xs[t] * sum_g s13[e, n, g] * sum_{k in g} xq[t, k] * (q13[e, n, k] - 8)
 *   (each group's sum an exact integer; the sum over groups in float32),
 *   up likewise with row I + n; h = silu(gate) * up (float32), quantized per
 *   row -> hq[p, :], hs[p]; y[p, m] = hs[p] * sum_g s2[e, m, g] * (exact
 *   group sums of hq[p, k] * (q2[e, m, k] - 8)), float32.
 *   x bf16 [T, H]; w13/s13/w2/s2 as moe_grouped_w4a16_ffn; y float32
 *   [T*k, H] (grouped order).
 * Requires H % 128 == 0, I % 128 == 0. `dbg` may be NULL. `ws` must hold
 * moe_w4a8_workspace(shape) bytes.
 */
MOE_API size_t moe_w4a8_workspace(const moe_shape* shape);
MOE_API moe_status moe_grouped_w4a8_ffn(const moe_shape* shape, const uint16_t* x,
                         const uint8_t* w13, const uint16_t* s13,
                         const uint8_t* w2, const uint16_t* s2,
                         const int32_t* expert_offsets, const int32_t* sorted_slot,
                         const int32_t* active, const int32_t* n_active,
                         float* y, const moe_w4a8_debug* dbg,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine — weighted sum of each token's k expert outputs. [PV-verify]
 * (floats within rounding bands of an f64 reference; results reproducible)
 * The pages print no formula for this step; this call takes its plainest
 * reading: a token's output is the sum of its k expert outputs weighted by
 * its router weights, in pick order j (the order moe_route_topk writes),
 * accumulated in float32 with no atomics, so two runs give the same bits:
 * out[t, :] = sum_{j = 0..k-1} topk_w[t, j] * y[slot_pos[t*k + j], :].
 *   y float32 [T*k, H] (grouped order), slot_pos int32 [T*k],
 *   topk_w float32 [T, k], out float32 [T, H].
 * Requires H % 8 == 0.
 */
MOE_API moe_status moe_combine(const float* y, const int32_t* slot_pos, const float* topk_w,
                int32_t T, int32_t H, int32_t k, float* out, void* stream);

/*
 * moe_expert_counts_accumulate — expert-load telemetry. [PV-fast] (the
 * engines count their own routing as they run and move the experts used most)
 * For each layer l < L: counts[l, e] += expert_offsets_l[e+1] - expert_offsets_l[e]
 * (the routed rows expert e received in that call; moe_permute and
 * moe_layer_w4a16 write expert_offsets), where expert_offsets_l =
 * expert_offsets + l * offsets_stride. Exact integer counts.
 *   expert_offsets int32  [L][offsets_stride] (input; first E+1 of each row used)
 *   counts         uint64 [L, E] (input/output, owned by the caller; zero it
 *                                 to start a window)
 * Requires L >= 0, 1 <= E <= MOE_MAX_EXPERTS, offsets_stride >= E + 1.
 * Calls that update the same counts must be ordered (one stream).
 */
MOE_API moe_status moe_expert_counts_accumulate(const int32_t* expert_offsets, int64_t offsets_stride,
                                 int32_t L, int32_t E, uint64_t* counts, void* stream);

/*
 * moe_expert_hot_rank — each layer's experts ranked by load. [PV-fast]
 * hot_ids[l, 0..n) = the n experts with the largest counts[l, :], in
 * descending order of count, ties broken by the lower expert index (exact).
 *   counts  uint64 [L, E] (input)
 *   hot_ids int32  [L, n] (output)
 * Requires L >= 0, 1 <= E <= MOE_MAX_EXPERTS, 0 <= n <= E.
 */
MOE_API moe_status moe_expert_hot_rank(const uint64_t* counts, int32_t L, int32_t E, int32_t n,
                        int32_t* hot_ids, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
