/*
 * routed_fp4.h -- C ABI of the MI355X (gfx950) routed-expert FFN library
 * (libroutedfp4.so).
 *
 * The library evaluates one mixture-of-experts FFN layer at decode time: a
 * router mat-vec, top-k selection, and for every selected expert the SwiGLU FFN
 * with 4-bit block-scaled weights dequantised in registers, followed by the
 * weighted sum of the expert outputs.  This is the indexed expert product the
 * page "Kimi-K3 on 2x A40 -- measured findings" benchmarks as MUL_MAT_ID
 * (section "Why the placement experiments all looked the same"), inside the
 * layer structure of page "SparkInfer-K3", section "How the TP module works"
 * (router over replicated weights -> top-16 -> selected experts -> sum), with the
 * routing and the final add beside the expert work and the partial sums added
 * in a fixed order as on page "Kimi-K3 on the same pod, two engines", sections
 * "Same hardware, same weights" and "Reason 1".  Routing stays on the device
 * between the steps (no host read-back), like the device-side router and
 * expert dispatch the "SparkInfer-K3" page lists in its layout table.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Its only global state is per
 *    device and written once: the CU count, whether the single-launch decode
 *    kernel fits (atomics, so concurrent first calls are safe), and the
 *    device array of moe_layer_fwd_noalloc.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    device work is enqueued on it; results are ready when the stream is.
 *  - Arguments are validated on the host before anything is enqueued; on error
 *    nothing is launched and a negative moe_status is returned.  A launch that
 *    the runtime rejects returns MOE_ERR_DEVICE.
 *  - Device-resident data is a precondition, not an error path: expert indices
 *    passed to moe_expert_fwd must lie in [0, num_experts), and inputs should
 *    be finite.  An out-of-range expert index is skipped (it contributes zero)
 *    so that a bad index never reads outside the bank.
 *  - Calls that run concurrently need separate workspaces.
 *  - The single-launch decode kernel (one token, built shapes) hands values
 *    between its workgroups through the workspace; every such wait is bounded.
 *    Should one expire (other work holding CUs indefinitely), the kernel sets
 *    the uint32 at byte offset 16 of the workspace to 1, exits, and that
 *    call's outputs are undefined.  The word stays set until the caller
 *    clears it (moe_workspace_init); a host can read it after the stream
 *    has finished.
 *  - All fp32 tensors are row-major and densely packed.
 */
#ifndef ROUTED_FP4_H
#define ROUTED_FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* NULL pointer, bad size, misaligned layout     */
  MOE_ERR_UNSUPPORTED = -2,   /* shape or token count outside what is built    */
  MOE_ERR_WORKSPACE = -3,     /* workspace NULL or smaller than required       */
  MOE_ERR_DEVICE = -4         /* the HIP runtime rejected a launch             */
} moe_status;

/* Weight formats named for the routed experts on the pages: MXFP4 for the
 * 3584->3072 expert shapes of the MUL_MAT_ID microbenchmark ("Kimi-K3 on 2x A40"
 * page), NVFP4 for the K3 checkpoint ("Kimi-K3 on the same pod" page, section
 * "Same hardware, same weights").  Element encodings are the OCP ones.
 *   MXFP4: e2m1 codes, one e8m0 scale byte per 32 consecutive elements of a
 *          row; w = e2m1(code) * 2^(byte-127).
 *   NVFP4: e2m1 codes, one fp8-e4m3 scale byte per 16 consecutive elements of
 *          a row, and one fp32 scale g per tensor; w = e2m1(code) * e4m3 * g. */
typedef enum { MOE_FMT_MXFP4 = 1, MOE_FMT_NVFP4 = 2 } moe_format;

/* Tensors of one expert record. */
enum {
  MOE_T_GATE_CODES = 0,  /* [I][H/2] bytes                                    */
  MOE_T_UP_CODES = 1,    /* [I][H/2] bytes                                    */
  MOE_T_DOWN_CODES = 2,  /* [H][I/2] bytes                                    */
  MOE_T_GATE_SCALES = 3, /* [I][H/B] bytes (B = 32 MXFP4, 16 NVFP4)           */
  MOE_T_UP_SCALES = 4,   /* [I][H/B] bytes                                    */
  MOE_T_DOWN_SCALES = 5, /* [H][I/B] bytes                                    */
  MOE_T_GLOBALS = 6,     /* NVFP4: 3 fp32 (gate, up, down g); unused by MXFP4 */
  MOE_NUM_TENSORS = 7
};

/* An expert bank in device memory.  Expert e's tensor t starts at
 *   (const uint8_t*)base + e * expert_stride + offset[t].
 * Codes are row-major with K contiguous (K = H for gate/up, I for down), two
 * elements per byte: element 2j in bits 3..0, element 2j+1 in bits 7..4.
 * Scales are row-major [N][K/B], one byte per block of B elements.
 * Requirements (checked): H and I multiples of 32; base, expert_stride and
 * every code offset multiples of 16; the globals offset a multiple of 4. */
typedef struct {
  int32_t format;        /* moe_format                                       */
  int32_t num_experts;   /* E, 1 .. 1024                                     */
  int32_t hidden;        /* H: input/output width of an expert               */
  int32_t inter;         /* I: intermediate width of an expert               */
  const void *base;      /* device pointer to expert 0's record              */
  int64_t expert_stride; /* bytes between consecutive expert records         */
  int64_t offset[MOE_NUM_TENSORS];
} moe_bank;

/* The record layout this library streams best: the seven tensors in id order,
 * each section 256-byte aligned, the record padded to 4 KiB.  Fills offset[]
 * and *expert_stride.  (Any layout meeting the moe_bank requirements works.) */
moe_status moe_bank_layout(int32_t format, int32_t hidden, int32_t inter,
                           int64_t offset[MOE_NUM_TENSORS], int64_t *expert_stride);

/* Limits.  Up to MOE_MAX_DECODE_TOKENS tokens per call the router is a
 * split-K mat-vec and the experts run as row dot products (each distinct
 * expert streamed once for all its tokens); more tokens (up to
 * MOE_MAX_TOKENS, e.g. a prefill chunk) take the batched path, whose router
 * and expert products run on the matrix cores.  Both batched expert paths
 * need H and I to be multiples of 512. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32
#define MOE_MAX_DECODE_TOKENS 16
#define MOE_MAX_TOKENS 4096

/* Bytes of device workspace the calls below need for C tokens.  The workspace
 * holds router partial sums and logits, the selection, the expert dispatch
 * tables, the intermediate activations, one output row per (token, slot) and a
 * few counters: about C*k*(4H + 6I) + 6*C*H bytes plus small terms (1.2 GB for
 * C = 2048, k = 16, H = 7168, I = 1536).  Returns 0 for arguments outside the
 * supported range (1 <= C <= MOE_MAX_TOKENS). */
size_t moe_workspace_size(int32_t num_experts, int32_t hidden, int32_t inter,
                          int32_t top_k, int32_t C);

/* Zero-fills a workspace (a fill kernel on `stream`, no memset node).  Must
 * run once before a workspace's first use; every call leaves the counters it
 * uses at zero again, so later calls need no re-initialisation. */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Router and top-k (the router of page "SparkInfer-K3", section "How the TP
 * module works"; selection rule and weights as the plainest reading: sigmoid
 * scores renormalised over the selected k).
 *  x        [C][H] fp32 activations, or NULL for "logits-in" mode.
 *  w_router [E][H] fp32 router matrix (ignored in logits-in mode).
 *  logits   [C][E] fp32: written when x != NULL (may then be NULL to skip),
 *           read when x == NULL.
 *  topk_idx [C][k] int32 out: the k experts with the largest logits, ordered by
 *           logit descending, equal logits by ascending index (-0 == +0; NaN
 *           ranks below every number).
 *  topk_w   [C][k] fp32 out: sigmoid(logit) / sum over the k of sigmoid(logit).
 * 1 <= C <= MOE_MAX_TOKENS, 1 <= k <= min(E, MOE_MAX_TOPK), H % 32 == 0.
 * For C > MOE_MAX_DECODE_TOKENS the logits come from fp32 matrix-core
 * products (same fp32 arithmetic, another summation order). */
moe_status moe_route(const float *x, const float *w_router, float *logits, int32_t C,
                     int32_t H, int32_t E, int32_t k, int32_t *topk_idx, float *topk_w,
                     void *ws, size_t ws_bytes, void *stream);

/* Selected experts and their weighted sum, for a given selection:
 *   out[t] = sum_{s<k} topk_w[t][s] * W_down,e (silu(W_gate,e x_t) * (W_up,e x_t)),
 *   e = topk_idx[t][s], summed in slot order s = 0..k-1.
 * Each distinct expert's weights are read once per call (once per tile of up
 * to 64 of its tokens when C > 64) for all the tokens that selected it
 * ("MUL_MAT_ID" of the "Kimi-K3 on 2x A40" page).  One token on a shape the
 * single-launch decode kernel is built for runs there; otherwise, for H and I
 * multiples of 512, C <= MOE_MAX_DECODE_TOKENS runs the decode-batch row
 * streams and larger C the matrix-core grouped GEMMs; for
 * C <= MOE_MAX_DECODE_TOKENS and other shapes the per-expert mat-vec kernels
 * run.
 *  x   [C][H] fp32 in; out [C][H] fp32 out (may not alias x).
 * Expert indices should be in [0, E); an index outside it is skipped (its
 * slot contributes zero), and an expert named by several slots of a token
 * counts once per slot. */
moe_status moe_expert_fwd(const moe_bank *bank, const float *x, int32_t C, int32_t k,
                          const int32_t *topk_idx, const float *topk_w, float *out,
                          void *ws, size_t ws_bytes, void *stream);

/* The whole layer: moe_route followed by moe_expert_fwd on device-resident
 * routing.  topk_idx_out / topk_w_out ([C][k]) may be NULL; when given they
 * receive the selection. */
moe_status moe_layer_fwd(const moe_bank *bank, const float *w_router, const float *x,
                         int32_t C, int32_t k, float *out, int32_t *topk_idx_out,
                         float *topk_w_out, void *ws, size_t ws_bytes, void *stream);

/* A latent MoE layer: the steps either side of the routed experts (page
 * "SparkInfer-K3", section "How the TP module works": router -> routed_down ->
 * routed experts, then routed_norm -> routed_up -> shared experts; section
 * "Why the reduce is at 3584 and not 7168": the RMS norm comes after the sum
 * of the routed experts; section "The model": 896 routed experts, top-16, 2
 * shared experts, latent width 3584, expert FFN 3072).
 *   idx, w  = top-k of x W_r^T, as moe_route            (router on the hidden x)
 *   x_lat   = W_down x                                   ([L][H] bf16)
 *   y_lat   = sum_s w_s FFN_e(s)(x_lat)                  (routed bank, hidden = L)
 *   out     = W_up (gamma * y_lat / sqrt(mean(y_lat^2) + eps))
 *             + sum_j FFN_shared_j(x)                    ([H][L] bf16; shared bank,
 *                                                         hidden = H, weight 1 each)
 * Dense products are bf16 x fp32 with fp32 sums; the experts run in the
 * library's expert paths.  All pointers are device pointers owned by the
 * caller; w_down, w_up and norm_gamma 16-byte aligned. */
typedef struct {
  int32_t hidden;               /* H                                          */
  const float *w_router;        /* [E][H] fp32, E = routed.num_experts        */
  const uint16_t *w_down;       /* [L][H] bf16 (routed_down), L = routed.hidden */
  const float *norm_gamma;      /* [L] fp32 (routed_norm weight)              */
  float norm_eps;               /* routed_norm epsilon, >= 0                  */
  const uint16_t *w_up;         /* [H][L] bf16 (routed_up)                    */
  moe_bank routed;              /* routed experts in the latent space          */
  moe_bank shared;              /* shared experts (hidden = H), 1 .. 32 of them */
} moe_latent_layer;

/* Workspace bytes for moe_latent_layer_fwd (0 outside the supported range:
 * 1 <= C <= MOE_MAX_DECODE_TOKENS, 1 <= k <= min(E, MOE_MAX_TOPK)). */
size_t moe_latent_workspace_size(const moe_latent_layer *layer, int32_t top_k, int32_t C);

/* The whole latent layer for C <= MOE_MAX_DECODE_TOKENS tokens.
 *  x [C][H] fp32 in (16-byte aligned); out [C][H] fp32 out (may not alias x).
 *  topk_idx_out / topk_w_out ([C][k]) may be NULL; when given they receive
 *  the routed selection.  The workspace must have been initialised with
 *  moe_workspace_init; its uint32 at byte offset 16 is the error word of the
 *  single-launch expert kernel, as for moe_expert_fwd.  Returns
 *  MOE_ERR_UNSUPPORTED for shapes outside: H and L multiples of 32, shared
 *  bank hidden = H, 1 .. 32 shared experts. */
moe_status moe_latent_layer_fwd(const moe_latent_layer *layer, const float *x, int32_t C,
                                int32_t k, float *out, int32_t *topk_idx_out, float *topk_w_out,
                                void *ws, size_t ws_bytes, void *stream);

/* MXFP4 experts on the block-scaled FP4 matrix cores (page "SparkInfer-K3",
 * Roadmap, "Later · B200 / B300 -- the Blackwell delta": without FP4 tensor
 * cores every low-bit expert product dequantises to bf16 first; CDNA4's
 * v_mfma_scale_f32_16x16x128_f8f6f4 takes the MXFP4 codes and their e8m0
 * block scales as they are stored).
 * The same computation as moe_expert_fwd for an MXFP4 bank: the fp32
 * activations (x, and h after SwiGLU) enter as `terms` e4m3 terms with an
 * e8m0 scale per 32 values; terms = 1 is a lossy single-term mode, and each
 * further term takes about 4 more bits.  The instruction truncates inside
 * each group of 8 products below 2^(largest exponent sum - 13) (measured);
 * the terms are built so that no product of a group falls below that
 * quantum, so from terms = 4 on the result is within the library's bar
 * (rel-L2 2e-5, max-abs 1e-4 of the largest output): a near-exact mode, not
 * bit-for-bit the fp32 path.
 *  bank: MXFP4, hidden and inter multiples of 256.  1 <= C <= MOE_MAX_TOKENS,
 *  1 <= k <= min(E, MOE_MAX_TOPK), 1 <= terms <= 6.  x [C][H] and out [C][H]
 *  fp32, 16-byte aligned, not aliased; topk_idx / topk_w [C][k] (an
 *  out-of-range expert index contributes zero).  The workspace (256-byte
 *  aligned) needs no initialisation.  Returns MOE_ERR_UNSUPPORTED outside
 *  these limits (including NVFP4 banks). */
size_t moe_mx_mma_workspace_size(const moe_bank *bank, int32_t top_k, int32_t C, int32_t terms);
moe_status moe_expert_fwd_mx_mma(const moe_bank *bank, const float *x, int32_t C, int32_t k,
                                 const int32_t *topk_idx, const float *topk_w, float *out,
                                 int32_t terms, void *ws, size_t ws_bytes, void *stream);

/* moe_layer_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops that must not call the allocator): the
 * same arguments without a workspace, which is instead a device array of the
 * library's own, one per GPU, 40 MiB, held until the process ends.  Its
 * limit covers every call of up to MOE_MAX_DECODE_TOKENS tokens at every
 * supported shape (the largest, E 1024, H 8192, I 4096, k 32, C 16, needs
 * 37.4 MiB) and the K3 shape up to 64 tokens; calls whose moe_workspace_size
 * exceeds it return MOE_ERR_WORKSPACE with nothing enqueued.
 *  - The first call on a device zero-fills the array (a fill kernel on
 *    `stream`); every call on that GPU shares it and leaves it ready for the
 *    next, so calls that overlap on one GPU (other streams, other threads)
 *    race and must be serialised by the caller.  Make that first call
 *    outside any stream capture: a captured zero-fill would be replayed and
 *    reset the call counter the decode kernel's hand-offs are tagged with.
 *  - error_out: NULL, or a device int32 that receives the decode kernel's
 *    error word (1 if one of its bounded waits expired during this or an
 *    earlier call, whose outputs are then undefined; see above), which is
 *    then cleared; one extra one-thread launch.
 * Otherwise as moe_layer_fwd (arguments, errors, outputs). */
moe_status moe_layer_fwd_noalloc(const moe_bank *bank, const float *w_router, const float *x,
                                 int32_t C, int32_t k, float *out, int32_t *topk_idx_out,
                                 float *topk_w_out, int32_t *error_out, void *stream);

/* Test export: dequantise one matrix of one expert to fp32.
 *  matrix 0 = gate [I][H], 1 = up [I][H], 2 = down [H][I].
 *  MXFP4: w = e2m1 * 2^(b-127), exact (IEEE denormals kept).
 *  NVFP4: w = round_fp32(e2m1 * e4m3 * g), the exact product rounded once. */
moe_status moe_dequant(const moe_bank *bank, int32_t expert, int32_t matrix, float *out,
                       void *stream);

const char *moe_status_string(moe_status s);
int32_t moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ROUTED_FP4_H */
