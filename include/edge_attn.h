/*
 * edge_attn.h — C ABI of the MI355X (gfx950) edge-aware attention layer.
 *
 * The layer is the edge-aware attention layer of "Efficient Edge-aware
 * Attention Network for Graph Generation" (ai-frontier-tracker digest,
 * full-text summary; the kongchang.com explainer, "Design Strategy of the
 * Edge-aware Attention Layer"). On a dense padded batch of B graphs with n
 * node slots it computes, per graph b, query row i, key j and head h:
 *
 *   Q, K, V      = X W_{q,k,v}^T + b_{q,k,v}, split into H heads of dh (c = h*dh + t)
 *   s            = q_i . k_j / sqrt(dh)                     (scaled dot product)
 *   gamma_e      = 1 + E_ij W_emul^T + b_emul,  beta_e = E_ij W_eadd^T + b_eadd
 *   gamma_y      = 1 + y W_ymul^T + b_ymul,     beta_y = y W_yadd^T + b_yadd
 *   u            = (s * gamma_e + beta_e) * gamma_y + beta_y  (head-wise FiLM)
 *   u            = -inf unless mask_i and mask_j              (graph mask)
 *   A            = softmax_j(u)   (a row with no real key gives A = 0)
 *   O_i          = sum_j A_ij V_j, heads merged to [d]        (A [V | I] gives O and A)
 *   E'_ij        = E_ij + W_e A_ij + b_e on real pairs, +0.0 elsewhere
 *                                                             (residual edge update)
 *
 * Graphs whose edge tensor is too large for one pass use the two-pass scheme
 * the same page names: pass 1 computes softmax statistics and O, pass 2
 * recomputes the scores and applies the edge update.
 *
 * Conventions for every entry point:
 *  - All tensors are contiguous, row-major, in device memory of the current
 *    HIP device, of element type desc.dtype (float32, or bfloat16 stored as
 *    uint16) unless stated otherwise. Weights use the nn.Linear [out, in]
 *    layout. X, E, O, A, E_out, every weight matrix and the workspace must be
 *    16-byte aligned (the workspace 256-byte aligned).
 *  - The caller owns every buffer and the stream; the library allocates no
 *    device memory and keeps no device state between calls. Calls are
 *    asynchronous on `stream` (a hipStream_t; NULL is the default stream).
 *  - Every argument is validated before anything is enqueued. On error the
 *    call returns a status, enqueues nothing, and ea_last_error() describes
 *    the problem. A kernel launch failure returns EA_E_HIP. Faults inside a
 *    kernel surface at the caller's next synchronization.
 *  - Padded entries (mask 0) of X and E may hold any bits, NaN/Inf included;
 *    no output depends on them. Masked outputs are written as +0.0.
 *  - bfloat16 mode rounds Q, K, V to bfloat16 after their projection and
 *    rounds A to bfloat16 before it is stored, multiplied with V and used in
 *    the edge update; all other arithmetic accumulates in float32.
 */
#ifndef EDGE_ATTN_H
#define EDGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EA_OK = 0,
  EA_E_NULLPTR = 1,     /* a required pointer is NULL                         */
  EA_E_SHAPE = 2,       /* inconsistent or out-of-range sizes                 */
  EA_E_UNSUPPORTED = 3, /* valid but not built: (H, dh, de) combination, dtype */
  EA_E_ALIGN = 4,       /* a pointer breaks the alignment rule                */
  EA_E_WORKSPACE = 5,   /* workspace missing or smaller than required         */
  EA_E_STATE = 6,       /* call order violated (two-pass update before forward) */
  EA_E_HIP = 7          /* a HIP runtime call or kernel launch failed         */
} ea_status;

typedef enum { EA_FP32 = 0, EA_BF16 = 1 } ea_dtype;

/* desc.flags */
#define EA_FORCE_TWO_PASS 0x1u /* use the two-pass scheme even when one pass fits */
/*
 * Ablation variants of the layer (desc.flags). "Efficient Edge-aware Attention
 * Network for Graph Generation", full-text summary: the ablations drop the
 * per-edge modulation ("Light Edge"), drop the score modulation, or feed the
 * edge update unnormalized instead of normalized attention coefficients.
 *   EA_VARIANT_LIGHT_EDGE: no per-edge FiLM (gamma_e = 1, beta_e = 0), so
 *     u = s * gamma_y + beta_y; w_emul, w_eadd, b_emul, b_eadd are not read
 *     and may be NULL.
 *   EA_VARIANT_NO_SCORE_MOD: no FiLM at all, u = s (masked scaled dot-product
 *     attention); every FiLM weight and bias and y are not read and may be
 *     NULL.
 *   EA_VARIANT_UNNORMALIZED: the edge update takes the masked logits u (0 at
 *     masked pairs) instead of A: E' = E + W_e u + b_e. O and A are the
 *     normalized ones. The edge update then recomputes u from E and the
 *     forward's workspace (edge_update needs p, y, ws and a preceding
 *     edge_attn_forward on the context, as in two-pass mode; A is ignored),
 *     and edge_attn_layer runs the forward and that update as two kernels.
 * The variants combine (LIGHT_EDGE with NO_SCORE_MOD is NO_SCORE_MOD).
 */
#define EA_VARIANT_LIGHT_EDGE 0x2u
#define EA_VARIANT_NO_SCORE_MOD 0x4u
#define EA_VARIANT_UNNORMALIZED 0x8u

/* Largest n handled in one pass (full rows on chip); larger n is two-pass. */
#define EA_SINGLE_PASS_MAX_N 256

typedef struct {
  int32_t B;     /* graphs in the batch, >= 1                        */
  int32_t n;     /* node slots per graph (padded), >= 1              */
  int32_t d;     /* node feature width, d = H * dh                   */
  int32_t de;    /* edge feature width                               */
  int32_t dy;    /* global feature width, >= 1                       */
  int32_t H;     /* heads                                            */
  int32_t dh;    /* head width                                       */
  int32_t dtype; /* ea_dtype                                         */
  uint32_t flags;
} ea_desc;

/*
 * Supported shapes: dh in {16, 32, 64}, de a positive multiple of 16,
 * 1 <= H <= 16 (2H <= 32), d = H dh; any B, n, dy (B <= 65535, n <= 2^20,
 * B n^2 de < 2^46); otherwise EA_E_UNSUPPORTED or EA_E_SHAPE.
 * (H, dh, de) = (4, 16, 16) and (8, 32, 64) run tuned kernels (MFMA, E held
 * on chip from the scores to the edge update); every other shape runs the
 * generic path (one block per query row, runtime sizes, VALU arithmetic,
 * E read twice per row), with the same results up to float32 rounding.
 * The backward is built for the two tuned shapes only; the block for
 * (d, de, dy) = (64, 16, 16) and, in bfloat16, (256, 64, 64).
 */

typedef struct {
  const void *w_q, *w_k, *w_v;            /* [d, d]                       */
  const void *b_q, *b_k, *b_v;            /* [d] or NULL (= 0)            */
  const void *w_emul, *w_eadd;            /* [H, de]  edge FiLM gamma/beta */
  const void *b_emul, *b_eadd;            /* [H] or NULL                  */
  const void *w_ymul, *w_yadd;            /* [H, dy]  global FiLM         */
  const void *b_ymul, *b_yadd;            /* [H] or NULL                  */
} ea_attn_params;

typedef struct {
  const void *w_e; /* [de, H] residual edge-update map      */
  const void *b_e; /* [de] or NULL                          */
} ea_update_params;

typedef struct ea_ctx ea_ctx; /* opaque, host memory only */

/* Validate desc and create a host-side context (mode, workspace plan). */
ea_status ea_ctx_create(const ea_desc* desc, ea_ctx** out);
void ea_ctx_destroy(ea_ctx* ctx);

/* Workspace bytes the context needs (Q, K, V^T per head, softmax statistics,
 * global FiLM coefficients, the attention kernel's work order). */
size_t ea_workspace_bytes(const ea_ctx* ctx);

/* 1 when the context runs the two-pass scheme, else 0 (-1 for NULL). */
int ea_is_two_pass(const ea_ctx* ctx);

/*
 * Attention forward: node output O [B, n, d] and, in single-pass mode, the
 * attention map A [B, H, n, n] (j contiguous). In two-pass mode A must be
 * NULL; the softmax statistics stay in the workspace for edge_update.
 * X [B, n, d], E [B, n, n, de], y [B, dy], node_mask [B, n] uint8 (nonzero =
 * real node; any pattern is allowed).
 */
ea_status edge_attn_forward(ea_ctx* ctx, const ea_attn_params* p,
                            const void* X, const void* E, const void* y,
                            const uint8_t* node_mask, void* O, void* A,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Residual edge update E_out = E + W_e A + b_e on real pairs (+0.0 elsewhere),
 * E_out [B, n, n, de] (may alias E). Single-pass: A is the map written by
 * edge_attn_forward (required; p may be NULL). Two-pass: A is ignored and
 * recomputed from E, p and the statistics a previous edge_attn_forward on
 * this context left in ws (same ws, same stream, inputs unchanged);
 * otherwise EA_E_STATE.
 */
ea_status edge_update(ea_ctx* ctx, const ea_attn_params* p, const ea_update_params* u,
                      const void* E, const void* y, const uint8_t* node_mask,
                      const void* A, void* E_out,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * The whole layer in one call: the same outputs as edge_attn_forward followed
 * by edge_update. Single-pass mode runs attention and the edge update in one
 * fused kernel; two-pass mode runs both passes. A as in edge_attn_forward,
 * except that in two-pass mode A may also be given (no variant flag, a tuned
 * shape, else EA_E_UNSUPPORTED): the second pass then writes the attention
 * map too, +0.0 at masked pairs (the values its edge update used), and
 * edge_attn_backward may read it instead of recomputing it. E_out may alias E.
 */
ea_status edge_attn_layer(ea_ctx* ctx, const ea_attn_params* p, const ea_update_params* u,
                          const void* X, const void* E, const void* y,
                          const uint8_t* node_mask, void* O, void* A, void* E_out,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * The same call as edge_attn_layer for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): it takes no workspace and allocates nothing; the
 * workspace is a device array inside the library, one copy per GPU, held
 * until the process ends. The caller still passes inputs and outputs, with
 * the same rules as edge_attn_layer. A context whose workspace
 * (ea_workspace_bytes) exceeds ea_noalloc_max_workspace_bytes() (16 MiB)
 * gets EA_E_WORKSPACE and nothing is enqueued. Every call on one GPU uses
 * the same array: calls that overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller. Nothing may rely on what
 * a call leaves in that array: the backward and a two-pass edge_update
 * cannot follow this call (they get EA_E_STATE).
 */
size_t ea_noalloc_max_workspace_bytes(void);
ea_status edge_attn_layer_noalloc(ea_ctx* ctx, const ea_attn_params* p, const ea_update_params* u,
                                  const void* X, const void* E, const void* y,
                                  const uint8_t* node_mask, void* O, void* A, void* E_out, void* stream);

/*
 * Backward of the layer (forward plus residual edge update): the gradients
 * of a loss L with respect to the inputs and every weight, given dL/dO and
 * dL/dE'. The derivative of the definition ("Efficient Edge-aware Attention
 * Network for Graph Generation", full-text summary: FiLM-modulated scaled
 * dot-product scores, mask, normalized softmax, A [V | I], E' = E + W_e A +
 * b_e), with the forward's stored A (bfloat16 mode: its rounding points pass
 * gradients through unchanged). Supported: B n_p^2 < 2^31 (n_p = n rounded
 * up to 16), no variant flag, bfloat16 for both built shapes and float32 for
 * (4, 16, 16) (else EA_E_UNSUPPORTED). Two-pass contexts: when A is the
 * buffer the preceding edge_attn_layer call on this context wrote, the
 * backward reads it; otherwise (NULL, or any other buffer) it recomputes A,
 * exp(u - lse) from the forward's row statistics, in its own workspace.
 *
 * Needs a preceding edge_attn_layer or edge_attn_forward on this context with
 * the same inputs, parameters, ws and stream (its Q, K, V, global FiLM and,
 * two-pass, row statistics stay in ws), and, single-pass, that call's A
 * (else EA_E_STATE). dO [B, n, d] and dE_out
 * [B, n, n, de] are in the context's dtype, and so are the outputs dX
 * [B, n, d], dE [B, n, n, de] and dy [B, dy]. Weight gradients are float32,
 * in the parameters' layouts, overwritten (not accumulated). bws is the
 * backward's own workspace (ea_backward_workspace_bytes, 256-byte aligned).
 * Masked pairs get dE = +0.0; padded rows of dX are +0.0.
 * Repeatability: every output is a sum in a fixed order (no atomics: blocks
 * write partial sums to slots of their own, which a later kernel adds in
 * order), so identical calls give the same bits.
 */
typedef struct {
  float *w_q, *w_k, *w_v;       /* [d, d] */
  float *b_q, *b_k, *b_v;       /* [d]    */
  float *w_emul, *w_eadd;       /* [H, de] */
  float *b_emul, *b_eadd;       /* [H]    */
  float *w_ymul, *w_yadd;       /* [H, dy] */
  float *b_ymul, *b_yadd;       /* [H]    */
  float *w_e, *b_e;             /* [de, H], [de] */
} ea_grads;

size_t ea_backward_workspace_bytes(const ea_ctx* ctx);
ea_status edge_attn_backward(ea_ctx* ctx, const ea_attn_params* p, const ea_update_params* u,
                             const void* X, const void* E, const void* y, const uint8_t* node_mask,
                             const void* A, const void* dO, const void* dE_out,
                             void* dX, void* dE, void* dy, const ea_grads* grads,
                             void* ws, size_t ws_bytes, void* bws, size_t bws_bytes, void* stream);

const char* ea_status_str(ea_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char* ea_last_error(void);

/*
 * Stage export for parity tests: the masked logits u [B, H, n, n] (float32,
 * -inf at masked pairs), computed by the same score stage as the layer
 * (tuned shapes: n <= 256, else EA_E_UNSUPPORTED; generic shapes: any n).
 */
ea_status ea_debug_logits(ea_ctx* ctx, const ea_attn_params* p,
                          const void* X, const void* E, const void* y,
                          const uint8_t* node_mask, float* U,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Stage export for parity tests: the softmax stage alone. U [B, H, n, n]
 * float32 logits (-inf at masked pairs), A [B, H, n, n] in the context's
 * dtype: A = softmax over the last axis, a row without a finite logit gives
 * 0, masked entries +0.0, rounded to the storage type (bfloat16: nearest
 * even). The same row softmax as the generic path's. No workspace.
 */
ea_status ea_debug_softmax(ea_ctx* ctx, const float* U, void* A, void* stream);

/*
 * Graph-transformer block around the layer. The method's page ("Efficient
 * Edge-aware Attention Network for Graph Generation", full-text summary)
 * swaps the attention inside a graph transformer and keeps the block around
 * it, which it does not write out; the block computed here is the usual one
 * of the denoising graph transformers it builds on:
 *   (O, A, E') = edge_attn_layer(X, E, y, mask)
 *   X1 = LN(X + O W_o^T + b_o),   X2 = LN(X1 + W_x2 relu(W_x1 X1 + b_x1) + b_x2)
 *   E1 = LN(E'),                  E2 = LN(E1 + W_e2 relu(W_e1 E1 + b_e1) + b_e2)
 *   y1 = LN(y + W_yy y + W_yx xbar + W_ye ebar + b_yo)
 *   y2 = LN(y1 + W_y2 relu(W_y1 y1 + b_y1) + b_y2)
 * xbar and ebar are the means of X2 over real nodes and of E2 over real
 * pairs (0 for a graph without real nodes); LN normalizes over the feature
 * axis (population variance, eps 1e-5) with a gain and a shift. Widths:
 * W_o, W_x1, W_x2 [d, d]; W_e1 [2 de, de], W_e2 [de, 2 de]; W_yy, W_y1,
 * W_y2 [dy, dy]; W_yx [dy, d]; W_ye [dy, de]; every parameter in the
 * context's dtype, nn.Linear [out, in] layout, 16-byte aligned, none NULL.
 * Rows of masked nodes of X2 and masked pairs of E2 are +0.0.
 *
 * Built for (d, de, dy) = (64, 16, 16) (float32 and bfloat16) and
 * (256, 64, 64) (bfloat16), no variant flag (else EA_E_UNSUPPORTED);
 * single-pass and two-pass contexts. X_out may alias X, E_out may alias E
 * and y_out may alias y. ws holds ea_block_workspace_bytes (the layer's
 * workspace, then O, A and per-block partial sums). bfloat16 mode stores O
 * and E' in bfloat16 and rounds X1, E1 and the hidden layers to bfloat16
 * where they enter a matrix product (float32 accumulation).
 */
typedef struct {
  const void *w_o, *b_o, *ln_x1_g, *ln_x1_b, *w_x1, *b_x1, *w_x2, *b_x2, *ln_x2_g, *ln_x2_b;
  const void *ln_e1_g, *ln_e1_b, *w_e1, *b_e1, *w_e2, *b_e2, *ln_e2_g, *ln_e2_b;
  const void *w_yy, *w_yx, *w_ye, *b_yo, *ln_y1_g, *ln_y1_b, *w_y1, *b_y1, *w_y2, *b_y2, *ln_y2_g, *ln_y2_b;
} ea_block_params;

size_t ea_block_workspace_bytes(const ea_ctx* ctx);
ea_status edge_attn_block(ea_ctx* ctx, const ea_attn_params* p, const ea_update_params* u,
                          const ea_block_params* bp, const void* X, const void* E, const void* y,
                          const uint8_t* node_mask, void* X_out, void* E_out, void* y_out,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Kernel timing with HIP events recorded on the launch stream around every
 * kernel the context launches while enabled. ea_profile_begin starts a
 * window (at most 4096 launches are recorded); ea_profile_end waits for the
 * last event and returns, per kernel id, the summed milliseconds and the
 * launch count (arrays of EA_NUM_KERNELS entries).
 */
enum { EA_K_QKV = 0, EA_K_ATTN = 1, EA_K_UPDATE = 2, EA_K_FUSED = 3, EA_K_BACKWARD = 4, EA_K_BLOCK = 5,
       EA_NUM_KERNELS = 6 };
ea_status ea_profile_begin(ea_ctx* ctx);
ea_status ea_profile_end(ea_ctx* ctx, double* total_ms, int64_t* launches);
const char* ea_kernel_name(int kernel_id);

/*
 * Bandwidth probes (measurement context, not part of the layer): the HBM rate
 * this GPU reaches on a plain stream, for a benchmark to report next to the
 * layer's kernels (the pages give the layer's cost as memory traffic, not
 * arithmetic: "Efficient Edge-aware Attention Network for Graph Generation",
 * digest, full-text summary).
 *
 * ea_probe_copy copies `bytes` from src to dst (device memory, 16-byte
 *   aligned, bytes a multiple of 16, the ranges must not overlap); bytes = 0
 *   does nothing.
 * ea_probe_read reads `bytes` at src and XORs every 32-bit word into
 *   *xor_out (device memory, 4-byte aligned; the caller zeroes it first if
 *   it wants the XOR itself); bytes = 0 only checks the pointers.
 * Both are asynchronous on `stream`; errors as for every other entry point.
 */
ea_status ea_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
ea_status ea_probe_read(const void* src, size_t bytes, uint32_t* xor_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EDGE_ATTN_H */
