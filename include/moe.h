/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer with
 * 2-, 3- or 4-bit block-quantised experts.
 *
 * The layer (sources: "How Strata runs a 125-billion-parameter model on a
 * single 12 GB to 24 GB graphics card", intro and Step 2; "Strata Open-Source
 * Runtime: Running a 125B-Parameter Qwen3 Model on a 12GB GPU", section "The
 * Model Itself: The Compute-Storage Gap in Sparse MoE"): for every token a
 * router scores E experts and keeps the top k; the k selected experts and one
 * always-on shared expert run; the finished expert vectors are summed on the
 * GPU with the router weights.  The pages fix the counts (E = 512, k = 10,
 * one shared expert, 48 layers) and that experts are read from 2-bit storage;
 * the expert function (SwiGLU), the renormalised softmax and the block format
 * below are the workload's own definition.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership  : every pointer argument is caller-owned memory.  Tensor
 *              arguments are DEVICE pointers (hipMalloc'd or from a device
 *              allocator); structs passed by pointer (moe_shape, moe_layer,
 *              moe_options) are HOST memory read during the call only.  The
 *              library never allocates device memory; scratch comes from the
 *              caller's workspace.
 * Streams    : `stream` is a hipStream_t passed as void* (NULL = the default
 *              stream).  Every call is asynchronous on that stream and never
 *              synchronises the host, except moe_read_error.
 * Errors     : arguments are validated on the host before any HIP call; a
 *              failed check returns a negative moe_status and launches
 *              nothing.  A launch failure returns MOE_ERR_DEVICE.  C++
 *              exceptions never cross this boundary.  moe_status_string()
 *              names a status; moe_last_error_detail() gives a one-line
 *              explanation of the last failure on the calling thread.
 * T == 0     : is valid and launches nothing.
 *
 * Quantised block format (the pages give none; this is the workload's format
 * with the bit layout chosen here).  For a matrix W of shape [rows][K] whose
 * reduction axis is K (K a multiple of 32):
 *   - blocks of 32 consecutive weights along K share one fp16 scale s;
 *   - code c in [-2^(b-1), 2^(b-1)-1], weight = c * s, stored offset-binary
 *     q = c + 2^(b-1);
 *   - canonical layout (what moe_quantize writes and moe_dequant and
 *     moe_repack read), row-major planes:
 *       low plane   [rows][K/4] bytes: bits 0..1 of q for weight k of a row
 *                   at bits 2*(k%4) of byte k/4 (the 2-bit codes themselves);
 *       3 bits:     then a high plane [rows][K/8]: bit 2 of q at bit k%8 of
 *                   byte k/8;
 *       4 bits:     then a second plane [rows][K/4] in the low plane's
 *                   layout holding bits 2..3 of q (the pages' quantisation
 *                   ladder tops out at a 4-bit file: "Strata serves a 125B
 *                   MoE at 94 tokens/s ...", section "Quality is a sizing
 *                   decision");
 *       scales      [rows][K/32] fp16 bit patterns;
 *     so a matrix takes rows*K*b/8 code bytes and rows*K/32 scales;
 *   - kernel layout (what moe_qweights must hold): the same bytes rearranged
 *     by moe_repack, once, when weights are uploaded.  Buffer sizes, plane
 *     offsets and per-expert strides are the canonical ones; the placement
 *     inside a matrix belongs to the kernels (it groups rows so that one
 *     weight load reads one contiguous piece) and is not part of this ABI.
 * Expert matrices: gate [I][H], up [I][H] (K = H) and down [H][I] (K = I).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer */
  MOE_ERR_UNSUPPORTED = -2, /* a valid request the library does not handle */
  MOE_ERR_WORKSPACE = -3,   /* workspace too small; see moe_last_required_workspace */
  MOE_ERR_DEVICE = -4,      /* a HIP call or kernel launch failed */
  MOE_ERR_INDEX = -5        /* an expert id outside [0, E) reached moe_permute */
} moe_status;

/* Element types.  Activations x: MOE_F32, MOE_BF16 or MOE_F16 (every kernel
 * converts them to fp16 MFMA operands, exactly for fp16; the router then
 * runs its fp32 path unless x and the router weights are both bf16).
 * Router weights: MOE_F32 or MOE_BF16 (MOE_F16 there is MOE_ERR_INVALID_ARG). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_F16 = 2 } moe_dtype;

/* Expert-FFN algorithm.  GEMV: fused dequant-GEMV for few tokens per expert
 * (decode).  GROUPED: dequantise tiles into LDS and run a grouped MFMA GEMM
 * (prefill).  AUTO picks GEMV when T <= 16, else GROUPED.  Both compute the
 * same function. */
typedef enum { MOE_ALGO_AUTO = 0, MOE_ALGO_GEMV = 1, MOE_ALGO_GROUPED = 2 } moe_algo;

typedef struct {
  int32_t hidden;       /* H: model width, multiple of 32 */
  int32_t inter;        /* I: routed expert intermediate size, multiple of 32 */
  int32_t n_experts;    /* E: routed experts, 1..4096 */
  int32_t top_k;        /* k: experts per token, 1..min(E, 32) */
  int32_t shared_inter; /* shared expert intermediate size (multiple of 32), 0 = none */
  int32_t qbits;        /* 2, 3 or 4 */
} moe_shape;

/* Quantised weights of a set of experts, in the kernel layout (moe_repack).
 * Matrix m (0 = gate, 1 = up, 2 = down) of expert e starts at codes[m] +
 * e * code_stride bytes, and its scales at scales[m] + e * scale_stride fp16
 * elements.  codes[m] and
 * code_stride must be multiples of 16 bytes; scales[m] must be 4-byte aligned
 * and scale_stride even. */
typedef struct {
  const uint8_t* codes[3];
  const uint16_t* scales[3];
  int64_t code_stride;
  int64_t scale_stride;
} moe_qweights;

typedef struct {
  const void* w_router;     /* [E][H] router weights, row-major, dtype router_dtype */
  moe_dtype router_dtype;   /* MOE_F32 or MOE_BF16 */
  const float* router_bias; /* [E] fp32, or NULL for no bias */
  moe_qweights experts;     /* E routed experts, inter = shape.inter */
  moe_qweights shared;      /* one expert (index 0), inter = shape.shared_inter;
                               ignored when shared_inter == 0 */
} moe_layer;

/* Phase control of moe_expert_ffn (flags of moe_options; moe_layer_forward
 * takes none).  For running one projection kernel alone, e.g. to time it:
 * REUSE_PLAN skips building the slot table from offsets and the grouped
 * GEMM's fp16 copy of x (reusing what the previous moe_expert_ffn call on
 * this workspace built, for the same x, offsets and T); SKIP_GATEUP skips the gate/up projection (reusing the activations
 * left in the workspace by the previous call); SKIP_DOWN skips the down
 * projection (y_sorted and shared_out are then not written). */
enum {
  MOE_FFN_REUSE_PLAN = 1,
  MOE_FFN_SKIP_GATEUP = 2,
  MOE_FFN_SKIP_DOWN = 4
};

/* Option of moe_layer_forward (and moe_layer_forward_noalloc): the route
 * tail skip of a verify window ("How Strata runs a 125-billion-parameter
 * model ...", Step 2, "Verify-window route tail skip (STRATA_ROUTE_TAIL_SKIP=7)").
 * With T <= 4 tokens (one window) on the GEMV path, an expert that no token
 * of the window ranks 0..6 of its top-k (every token that chose it ranks it
 * 7 or later, the smallest router weights) is neither read nor computed, and
 * its pairs add nothing to the sum; the other weights are not renormalised.
 * An approximation: the output differs from the exact layer (the pages keep
 * it for experts missing from VRAM and report a small distribution shift).
 * topk_idx / topk_w still return the full selection.  No effect when T > 4
 * or top_k <= 7; MOE_ERR_UNSUPPORTED with MOE_ALGO_GROUPED at T <= 4. */
enum { MOE_LAYER_ROUTE_TAIL_SKIP = 8 };

typedef struct {
  moe_algo ffn_algo;
  int32_t flags; /* MOE_FFN_* bits for moe_expert_ffn; MOE_LAYER_ROUTE_TAIL_SKIP for
                    moe_layer_forward; 0 for every other call */
} moe_options;

/* Bytes of workspace moe_layer_forward needs for T tokens (also enough for
 * moe_route, moe_permute and moe_expert_ffn at the same T).  Returns 0 for an
 * invalid shape. */
size_t moe_workspace_bytes(const moe_shape* shape, int64_t T, const moe_options* opts);

/* Router (page 1, Step 2, "Mapped host doorbell and a single captured CUDA
 * graph": the router picks the experts of each layer on the GPU).
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h] + bias[e]   (fp32 accumulate)
 *   topk_idx[t][j] = the k largest logits of token t, descending; ties go to
 *                    the lower expert index
 *   topk_w[t][j]   = softmax over the selected logits (= softmax over all E
 *                    renormalised over the selection); weights sum to 1.
 * x [T][H] (dtype x_dtype), logits [T][E] fp32 or NULL (then the workspace
 * holds them), topk_idx [T][k] int32, topk_w [T][k] fp32. */
int moe_route(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer,
              const moe_shape* shape, float* logits, int32_t* topk_idx, float* topk_w,
              void* workspace, size_t workspace_bytes, void* stream);

/* Token-to-expert permutation (the analogue of the partition of a layer's
 * selected experts, page 1, Step 2, "Mapped host doorbell ...").  Pair
 * p = t*k + j.  Outputs: counts [E], offsets [E+1] (exclusive scan of counts),
 * sorted_pair [T*k] (pairs grouped by expert, ascending p inside a group) and
 * pair_pos [T*k] (inverse: sorted_pair[pair_pos[p]] == p).  Expert ids outside
 * [0, E) are skipped (never written out of bounds) and recorded in the
 * workspace; moe_read_error then returns MOE_ERR_INDEX. */
int moe_permute(const int32_t* topk_idx, int64_t T, const moe_shape* shape, int32_t* counts,
                int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* workspace,
                size_t workspace_bytes, void* stream);

/* Routed and shared expert FFN read directly from the quantised weights
 * (page 1 intro and Step 1: the experts are computed from their 2-bit
 * storage).  For every sorted position s with pair p = sorted_pair[s] in
 * expert e's segment [offsets[e], offsets[e+1]):
 *   y_sorted[s] = W_down_e (silu(W_gate_e x_t) * (W_up_e x_t)),  t = p / k
 * and, when shared_inter > 0 and shared_out != NULL, for every token t:
 *   shared_out[t] = the same function with the shared expert's weights.
 * x [T][H]; y_sorted [T*k][H] fp32; shared_out [T][H] fp32 or NULL. */
int moe_expert_ffn(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer,
                   const moe_shape* shape, const int32_t* offsets, const int32_t* sorted_pair,
                   float* y_sorted, float* shared_out, const moe_options* opts, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Weighted combine (page 1, Step 2, "Dynamic PCIe and CPU co-execution": the
 * GPU sums the finished expert vectors):
 *   out[t] = shared_out[t] + sum_j topk_w[t][j] * y_sorted[pair_pos[t*k+j]]
 * (j ascending; shared_out may be NULL).  Optional stack glue for stacked
 * layers: if residual != NULL then residual[t] += out[t]; if also
 * next_in_bf16 != NULL then next_in_bf16[t] = bf16_RNE(r / sqrt(mean(r^2) +
 * 1e-6)) with r the updated residual row.  out [T][H] fp32 (may be NULL when
 * residual is given). */
int moe_combine(const float* y_sorted, const int32_t* pair_pos, const float* topk_w,
                const float* shared_out, int64_t T, const moe_shape* shape, float* out,
                float* residual, uint16_t* next_in_bf16, void* stream);

/* The whole layer: route, permute, expert FFN, shared expert and combine in
 * one call, with the optional stack glue of moe_combine.  topk_idx / topk_w
 * may be NULL (then the workspace holds them).  With the grouped-GEMM
 * algorithm the routed and shared expert outputs pass from the down
 * projection to the combine as fp16 (the weights and the sum stay fp32), so
 * its bits differ from moe_expert_ffn + moe_combine, which keep y_sorted and
 * shared_out in fp32;
 * both are within the output tolerance of the fp64 layer.  The selection
 * (topk_idx, topk_w) equals moe_route's bit for bit on every path. */
int moe_layer_forward(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer,
                      const moe_shape* shape, float* out, float* residual,
                      uint16_t* next_in_bf16, int32_t* topk_idx, float* topk_w,
                      const moe_options* opts, void* workspace, size_t workspace_bytes,
                      void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the whole
 * layer exactly as moe_layer_forward computes it (same kernels, same bits),
 * with its workspace taken from a scratch array the library holds on each
 * GPU instead of from the caller.  The array has MOE_NOALLOC_SCRATCH_BYTES
 * (16 MiB: every shape whose moe_workspace_bytes fits, e.g. the full-shape
 * layer of 512 experts, top-10, hidden 2048, inter 704 up to 149 tokens); it
 * comes with the library's device code on each GPU the library runs on and
 * is held until the process ends.  A larger shape
 * returns MOE_ERR_UNSUPPORTED before any device work.  The call allocates
 * nothing.  Every call on one GPU uses that GPU's one array, which keeps the
 * previous call's contents (the layer needs nothing in it zeroed): calls that
 * overlap on one GPU (other streams, other threads) race, so serialise them
 * on one stream.  The first call on a device looks the array up on that
 * device (hipGetSymbolAddress). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int moe_layer_forward_noalloc(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer,
                              const moe_shape* shape, float* out, float* residual,
                              uint16_t* next_in_bf16, int32_t* topk_idx, float* topk_w,
                              const moe_options* opts, void* stream);

/* a[t] = bf16_RNE(r[t] / sqrt(mean(r[t]^2) + 1e-6)) for r [T][H] fp32 (the
 * input of the first layer of a stack). */
int moe_rmsnorm_bf16(const float* r, int64_t T, int32_t H, uint16_t* a, void* stream);

/* out[r][k] = (q - 2^(b-1)) * scale[r][k/32] in fp32 (exact) for one matrix
 * [rows][cols] in the canonical layout.  codes 8-byte, scales 2-byte and out
 * 16-byte aligned. */
int moe_dequant(const uint8_t* codes, const uint16_t* scales, int64_t rows, int32_t cols,
                int32_t qbits, float* out, void* stream);

/* Quantise fp32 w [rows][cols] to the canonical layout (used to build
 * synthetic expert arenas).  Per block: m = signed element of largest
 * magnitude (first on ties), d = fp16_RNE(m / c_min), c = clamp(
 * rint_half_even(w / d), c_min, c_max), c = 0 for the whole block when d == 0
 * (then d is stored as +0); all in fp32.  codes 8-byte, scales 2-byte and w
 * 16-byte aligned. */
int moe_quantize(const float* w, int64_t rows, int32_t cols, int32_t qbits, uint8_t* codes,
                 uint16_t* scales, void* stream);

/* Rearrange one matrix [rows][cols] from the canonical layout (codes,
 * scales) into the kernel layout (packed_codes, packed_scales: the same byte
 * counts, rows*cols*qbits/8 and rows*cols/32 * 2), the form moe_qweights
 * holds.  Out of place: the output buffers must not overlap the inputs
 * (MOE_ERR_INVALID_ARG).  Allocates nothing; asynchronous on `stream`.
 * codes and packed_codes 8-byte aligned, scales and packed_scales 2-byte
 * aligned.  A matrix of an arena is repacked on its own (its rows start a
 * new row group), at the arena's per-expert offset. */
int moe_repack(const uint8_t* codes, const uint16_t* scales, int64_t rows, int32_t cols, int32_t qbits,
               uint8_t* packed_codes, uint16_t* packed_scales, void* stream);

/* Synchronises `stream`, then returns MOE_ERR_INDEX if the most recent
 * moe_permute (or moe_layer_forward) on this workspace met an expert id
 * outside [0, E), else MOE_OK; clears the record.  The only call that waits
 * for the device. */
int moe_read_error(void* workspace, size_t workspace_bytes, void* stream);

const char* moe_status_string(int status);
const char* moe_last_error_detail(void);
/* Set when a call returns MOE_ERR_WORKSPACE: the bytes that call needed. */
size_t moe_last_required_workspace(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
