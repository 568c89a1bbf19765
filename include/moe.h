/*
 * moe.h - C ABI of libmoe.so, one GPU's share of a mixture-of-experts (MoE)
 * layer of LLM inference on AMD Instinct MI355X (gfx950).
 *
 * The layer (router top-k -> dispatch into expert-contiguous groups ->
 * grouped expert GEMM with SwiGLU -> weighted combine) as the source pages
 * state it:
 *   - router: "Lower latency and higher throughput with multi-node DeepSeek
 *     deployment", section MoE Router (sort with index tracking, top-k indices
 *     and scores per token);
 *   - dispatch / combine: "CuTeDSL at Perplexity", section MoE Dispatch/Combine,
 *     local (single-GPU) kernel: per-expert counts, a unique index per token in
 *     its expert's list, a copy into per-expert buffers, then a weighted
 *     accumulation in registers using the dispatch offsets;
 *   - expert FFN: Qwen3.5-397B on Ironwood TPU v7x (xxmr.cn), section 4.2.2,
 *     grouped matmul with SwiGLU fused into the loop (gate and up streams);
 *   - FP8: DeepSeek-deployment page, section Quantization: weights with one
 *     scale per 128x128 block, activations quantised on the fly per
 *     128-element vector;
 *   - group sizes read on the device, never synchronised back to the host:
 *     DeepSeek-deployment page, Quantization (routing-aware persistent
 *     kernels) and CUDA Graph sections;
 *   - expert-parallel share (moe_shape.e_local > 0): "CuTeDSL at Perplexity",
 *     MoE Dispatch/Combine, tensor-parallel deployment (input replicated; the
 *     local dispatch keeps the tokens routed to this rank's experts, the local
 *     combine sums them, an all-reduce across ranks, not part of this library,
 *     adds the shares up) and "Hosting Qwen on Blackwell" (expert-parallel
 *     prefill kernel).
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise; the
 *     caller owns every buffer.  The library never allocates, frees or
 *     synchronises; each call only enqueues kernels on `stream` (a
 *     hipStream_t; NULL = the default stream) and returns.
 *   - Row-major layouts; "[A, B]" means B is the contiguous dimension.
 *   - bf16 = IEEE bfloat16 bit patterns (uint16); fp8 = OCP e4m3fn codes
 *     (uint8, bias 7, max 448).  Device pointers must be 16-byte aligned.
 *   - Return value: MOE_OK or a negative moe_status.  Argument errors are
 *     detected on the host before anything is launched (nothing is written).
 *     A launch failure returns MOE_ERR_HIP.  moe_last_error() then returns a
 *     thread-local message.  No exception crosses the ABI.
 *   - Supported shapes: 0 <= T, T*(k+n_shared) < 2^31, 1 <= k <= min(E, 16),
 *     1 <= E <= 1024, n_shared in {0, 1}, H and I positive multiples of 128,
 *     H, I <= 131072 and H*I < 2^31; e_local = 0 and e_first = 0, or
 *     1 <= e_local and 0 <= e_first <= E - e_local.
 *     T == 0 is a valid no-op.  Other shapes return MOE_ERR_UNSUPPORTED.
 *   - The library keeps no state between calls; calls on different streams
 *     with disjoint buffers may run concurrently.  Its only persistent
 *     objects are host-side: moe_grouped_ffn and moe_forward fork the tiled
 *     kernels of large groups onto a second stream of their own (one per
 *     host thread and device, default priority, created on first use and
 *     kept for the life of the process) and join it back into `stream`
 *     with events before returning, so the work stays ordered on `stream`
 *     and can be captured into a HIP graph.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* NULL pointer, bad enum, misaligned pointer */
  MOE_ERR_UNSUPPORTED = -2, /* shape outside the supported set */
  MOE_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than required */
  MOE_ERR_HIP = -4          /* a HIP launch failed; see moe_last_error() */
} moe_status;

typedef enum {
  MOE_BF16 = 0,              /* bf16 activations and expert weights */
  MOE_FP8_E4M3_BLOCK128 = 1, /* e4m3fn expert weights + fp32 scale per 128x128
                                block; x and h quantised per row per 128 channels
                                ("Lower latency and higher throughput with
                                multi-node DeepSeek deployment", Quantization) */
  MOE_MXFP8 = 2              /* MXFP8: e4m3fn codes with one E8M0 (power-of-two)
                                scale per 32 values along K, for the expert
                                weights and for x and h per row ("Hosting Qwen
                                on Blackwell", Quantization; "CuTeDSL at
                                Perplexity": absolute max over 32 elements).
                                E8M0 byte = floor(log2(amax)) - 8 + 127, 0 for
                                an all-zero block; codes = round-to-nearest-even
                                of v / 2^(byte - 127), saturated at +-448 */
} moe_wdtype;

/* Shape of one layer call.  L = (e_local ? e_local : E) routed experts held
   here; G = L + n_shared expert groups; R = T*(k + n_shared) rows bound the
   permuted (expert-contiguous) matrices.

   Expert-parallel share (e_local > 0): this GPU holds routed experts
   [e_first, e_first + e_local) of the E and sees all T tokens.  Routing is
   over all E experts; group g < L holds the pairs routed to expert
   e_first + g, pairs routed to other experts get dest = -1 and no row, the
   shared expert's group (if n_shared) follows the local groups, and the
   output is this share's partial sum: summing the outputs of shares that
   partition the experts (with the shared expert in one of them) gives the
   whole layer, up to the bf16 rounding of each share.  Expert weight and
   scale arrays hold the G local groups.  e_local = 0 (with e_first = 0) is
   the whole layer. */
typedef struct {
  int32_t T;        /* tokens */
  int32_t H;        /* hidden size */
  int32_t E;        /* routed experts */
  int32_t k;        /* experts chosen per token */
  int32_t I;        /* SwiGLU intermediate size */
  int32_t n_shared; /* always-on shared experts, 0 or 1 (group E) */
  int32_t wdtype;   /* moe_wdtype */
  int32_t e_first;  /* first routed expert held here (expert-parallel share) */
  int32_t e_local;  /* routed experts held here; 0 = all E (the whole layer) */
} moe_shape;

/* Thread-local description of the last non-OK return on this thread. */
const char* moe_last_error(void);

/* Library ABI version (increments on any signature change). */
int moe_abi_version(void);

/* Bytes of device workspace moe_forward needs for `shape` (256-byte aligned
   sub-buffers).  Returns 0 for an unsupported shape. */
size_t moe_forward_workspace_bytes(const moe_shape* shape);

/* The same value as moe_forward_workspace_bytes, under the name of the
   layer-level workspace query (the whole layer in one call needs this much). */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Bytes of device workspace moe_grouped_ffn needs (h, its fp8 scales and the
   on-device tile schedule).  Returns 0 for an unsupported shape. */
size_t moe_ffn_workspace_bytes(const moe_shape* shape);

/* Bytes of device workspace moe_route needs for `shape` (0 when the router
   GEMM runs unsplit; then workspace may be NULL).  Only T, H and E are read;
   returns 0 for an unsupported shape as well. */
size_t moe_route_workspace_bytes(const moe_shape* shape);

/*
 * Router: logits = x W_r^T (+ router_bias), then top-k and renormalised
 * softmax weights (DeepSeek-deployment page, MoE Router).
 *   x           [T, H] bf16
 *   w_router    [E, H] fp32 (torch Linear layout)
 *   router_bias [E] fp32 or NULL (added to every token's logits)
 *   logits      [T, E] fp32, written
 *   topk_idx    [T, k] int32, written: slot j holds the j-th largest logit;
 *               equal logits (+0 == -0) go to the lower expert index
 *   topk_w      [T, k] fp32, written: exp(l_j - l_0) / sum_j' exp(l_j' - l_0)
 *   workspace   >= moe_route_workspace_bytes(shape) bytes of device memory,
 *               16-byte aligned (partial sums over slices of H); caller-owned
 * Logits are fp32 sums of exact products, over slices of H added in a fixed
 * order: the same inputs give the same bits on every call.  Logits must be
 * finite (a NaN logit gives unspecified routing).  H <= 131072.
 */
int moe_route(const moe_shape* shape, const void* x, const float* w_router,
              const float* router_bias, float* logits, int32_t* topk_idx,
              float* topk_w, void* workspace, size_t ws_bytes, void* stream);

/* Top-k + weights alone, from caller-given fp32 logits [T, E] (same rules as
   moe_route).  Only T, E and k of `shape` are read. */
int moe_route_from_logits(const moe_shape* shape, const float* logits,
                          int32_t* topk_idx, float* topk_w, void* stream);

/* Bytes of device workspace moe_permute needs (ceil(T/256) * L int32).  Only
   T, E and the share are read; returns 0 for an unsupported shape as well. */
size_t moe_permute_workspace_bytes(const moe_shape* shape);

/*
 * Dispatch ("CuTeDSL at Perplexity", MoE Dispatch/Combine, local kernel):
 * counting sort of the (token, slot) pairs by expert into unpadded,
 * expert-contiguous groups, token-ascending within a group, and the row copy.
 *   topk_idx     [T, k] int32 in [0, E) (distinct per token)
 *   x            [T, H] bf16
 *   counts       [G] int32, written: rows per group (group L = shared, = T)
 *   offsets      [G + 1] int32, written: exclusive prefix sum of counts
 *   dest         [T, k] int32, written: row of (t, j) in the permuted matrix,
 *                -1 when the pair's expert is not held here (share only)
 *   src_row      [R] int32, written: token of each permuted row
 *                (shared group: rows offsets[L] + t hold token t;
 *                offsets[L] = T*k for the whole layer)
 *   x_perm       [R, H], written: bf16 copy of x[src_row[r]], or for
 *                MOE_FP8_E4M3_BLOCK128 the e4m3fn codes of that row quantised
 *                per 128 channels (scale = amax / 448, 1 for an all-zero group,
 *                codes rounded to nearest even after clamping to +-448), or for
 *                MOE_MXFP8 its MXFP8 codes (blocks of 32)
 *   x_perm_scale written for fp8: [H/128, R] fp32, K-block-major (the scale
 *                of row r, channels 128 b .. 128 b + 127, at b * R + r, so
 *                one block's scales of consecutive rows are adjacent); for
 *                mxfp8: [R, H/32] uint8 E8M0; NULL for bf16
 *   workspace    >= moe_permute_workspace_bytes(shape) bytes of device memory,
 *                16-byte aligned (per-tile expert counts); caller-owned
 * Ranks come from counts and bit masks, not atomic counters: the same routing
 * gives the same dest / src_row on every call.  Routing entries outside
 * [0, E) make the results unspecified.
 */
int moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x,
                int32_t* counts, int32_t* offsets, int32_t* dest,
                int32_t* src_row, void* x_perm, void* x_perm_scale,
                void* workspace, size_t ws_bytes, void* stream);

/*
 * Grouped expert FFN over the permuted rows (Qwen3.5-397B on Ironwood, section
 * 4.2.2): for every group g with rows [offsets[g], offsets[g+1]):
 *   h = silu(X W_gate[g]^T) * (X W_up[g]^T)   (fp32 accumulation)
 *   y_perm rows = h W_down[g]^T                (fp32 accumulation, bf16 out)
 * bf16 layers keep h in bf16.  fp8 layers quantise h per row per 128
 * channels like x_perm before the down projection; mxfp8 layers quantise h
 * per row in MX blocks of 32, and the products are the block-scaled ones
 * (each 32-value block's E8M0 scales applied to its partial sum).
 *   offsets      [G + 1] int32 (device; read only on the device)
 *   x_perm       [R, H] bf16 or e4m3fn codes; x_perm_scale [H/128, R] fp32
 *                (fp8, K-block-major as moe_permute writes it, R = T*(k +
 *                n_shared) slots per block) or [R, H/32] uint8 E8M0 (mxfp8),
 *                NULL for bf16
 *   w_gate, w_up [G, I, H] bf16 or e4m3fn codes
 *   w_down       [G, H, I] bf16 or e4m3fn codes
 *   s_gate, s_up fp8: [G, I/128, H/128] fp32 block scales; mxfp8: [G, I, H/32]
 *                uint8 E8M0; NULL for bf16
 *   s_down       fp8: [G, H/128, I/128] fp32; mxfp8: [G, H, I/32] uint8 E8M0
 *   y_perm       [R, H] bf16, written (rows of empty groups untouched)
 *   workspace    >= moe_ffn_workspace_bytes(shape) bytes of device memory
 * Groups whose offsets are not non-decreasing within [0, R] give unspecified
 * results.
 */
int moe_grouped_ffn(const moe_shape* shape, const int32_t* offsets,
                    const void* x_perm, const void* x_perm_scale,
                    const void* w_gate, const void* w_up, const void* w_down,
                    const void* s_gate, const void* s_up, const void* s_down,
                    void* y_perm, void* workspace, size_t ws_bytes,
                    void* stream);

/*
 * Combine ("CuTeDSL at Perplexity", local combine; shared expert added as in
 * the DeepSeek-deployment page, Expert parallelism section):
 *   out[t] = bf16( sum_{j = 0..k-1, dest[t, j] >= 0} topk_w[t, j] * y_perm[dest[t, j]]
 *                  + y_perm[offsets[L] + t] if n_shared )
 * summed in fp32 in that fixed order, one rounded product and one rounded add
 * per term (no fused multiply-add), one round-to-nearest-even at the end.
 * Pairs with dest < 0 (experts held by another share) add nothing.
 * Deterministic, no atomics.
 *   y_perm [R, H] bf16; dest [T, k] int32; topk_w [T, k] fp32; out [T, H] bf16
 *   offsets [G + 1] int32 from moe_permute: read (on the device) only when
 *           n_shared = 1, for the start of the shared rows; may be NULL otherwise
 */
int moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* dest,
                const float* topk_w, const int32_t* offsets, void* out, void* stream);

/*
 * The whole layer in one call: moe_route -> moe_permute -> moe_grouped_ffn ->
 * moe_combine on `stream`, intermediates in `workspace`
 * (>= moe_forward_workspace_bytes(shape)).  The permuted activation matrix is
 * never materialised here: the grouped GEMMs gather each row through src_row
 * from x (bf16) or from x quantised once per token (fp8, mxfp8), which gives
 * the same operands as moe_permute's x_perm.  Requires T*H*2 < 2^32.  Arguments as above;
 * topk_idx_out / topk_w_out may be NULL (then the routing lives in the
 * workspace only).  out [T, H] bf16: the layer's output, or for an
 * expert-parallel share (e_local > 0) this share's partial sum.
 */
int moe_forward(const moe_shape* shape, const void* x, const float* w_router,
                const float* router_bias, const void* w_gate, const void* w_up,
                const void* w_down, const void* s_gate, const void* s_up,
                const void* s_down, void* out, int32_t* topk_idx_out,
                float* topk_w_out, void* workspace, size_t ws_bytes,
                void* stream);

/*
 * moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The intermediates live in a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held from
 * the library's load on that GPU until the process ends; the call itself
 * allocates and frees nothing, and runs every kernel on `stream` (the
 * grouped FFN's two kernel chains one after the other, no side stream).
 * Arguments, layouts and results are those of moe_forward.
 *   - A shape whose moe_forward_workspace_bytes exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE (nothing launched);
 *     decode-sized batches fit (e.g. T = 64 tokens, H = 4096, E = 128, k = 8,
 *     I = 1536 needs about 8 MB).
 *   - Every call on one GPU uses that GPU's one array, and its contents are
 *     whatever the last call left: calls that overlap on one GPU (two streams,
 *     two host threads) race and give undefined results.  Serialise them.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_router,
                        const float* router_bias, const void* w_gate, const void* w_up,
                        const void* w_down, const void* s_gate, const void* s_up,
                        const void* s_down, void* out, int32_t* topk_idx_out,
                        float* topk_w_out, void* stream);

/*
 * Measurement hook (not a step of the layer).  After moe_profile_start, the
 * entry-point calls made on this thread record a pair of HIP events on their
 * stream around kernel launches:
 *   mode 1: around every launch, in launch order, up to `capacity` pairs;
 *           the grouped FFN's two kernel chains (tiled groups and
 *           weight-streaming groups) then run one after the other on the
 *           caller's stream, so each launch is timed alone;
 *   mode 2: around launch number `which` (0-based, counted from the start of
 *           each entry-point call) only, up to `capacity` pairs.
 * The events are created here (host objects; no device memory).
 * moe_profile_count: pairs recorded so far.  moe_profile_read: waits for pair
 * i, returns its elapsed milliseconds and the launched kernel's name (a static
 * string).  moe_profile_stop: stop recording and destroy the events.
 * Returns MOE_OK, MOE_ERR_INVALID_ARG (bad mode/index) or MOE_ERR_HIP.
 */
int moe_profile_start(int mode, int which, int capacity);
int moe_profile_count(void);
int moe_profile_read(int i, float* ms, const char** name);
int moe_profile_stop(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
