/*
 * olmoe_moe.h - C ABI of the OLMoE mixture-of-experts feed-forward layer on
 * MI355X (gfx950).
 *
 * The layer (sources: "OLMoE Guide: 64-Expert Fine-Grained Open MoE
 * Architecture", Router Mechanics & Loss Formulations items 1-3;
 * "Mixture-of-experts LLMs from scratch with OLMoE", sections 2 and 3;
 * "OLMoE: Open Mixture-of-Experts Language Models", Pretraining architecture):
 *
 *   logits  l[t,e] = sum_k x[t,k] * W_router[e,k]             (2048 -> 64)
 *   p[t,e]  = softmax over all 64 experts (fp32)
 *   S_t     = the 8 largest logits; equal logits go to the lower expert id
 *   out[t]  = sum_{e in S_t} p[t,e] * W_down[e] (SiLU(W_gate[e] x_t) * (W_up[e] x_t))
 *
 * The routing weights are the 64-way probabilities themselves: they are not
 * renormalised over the chosen 8 and sum to less than one.  Routing is
 * dropless token choice: every (token, expert) pair is computed.
 *
 * Conventions for every entry point:
 *   - tensor pointers are DEVICE pointers (HBM), row-major, 16-byte aligned;
 *   - bf16 tensors are passed as void* holding IEEE bfloat16 bit patterns;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *     all device work is enqueued on it and returns before it completes, so
 *     every buffer must stay alive until the stream has passed this call;
 *   - the caller allocates and owns every buffer, workspace included; the
 *     library allocates no device memory and keeps no pointer after return;
 *   - arguments are checked on the host before anything is enqueued; on any
 *     status other than OLMOE_OK nothing was enqueued (except OLMOE_EHIP,
 *     where a launch itself failed) and olmoe_last_error() holds a message
 *     (thread-local, valid until the next call on the same thread);
 *   - results are bitwise reproducible for identical inputs on one device
 *     and build (no floating-point atomics anywhere).
 */
#ifndef OLMOE_MOE_H
#define OLMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define OLMOE_API __attribute__((visibility("default")))
#else
#define OLMOE_API
#endif

#define OLMOE_ABI_VERSION 10

#define OLMOE_D 2048 /* hidden size */
#define OLMOE_F 1024 /* expert width (SwiGLU intermediate size) */
#define OLMOE_E 64   /* experts per layer */
#define OLMOE_K 8    /* experts per token */
#define OLMOE_MAX_TOKENS ((int64_t)1 << 24) /* T limit: 8*T row indices fit in int32 */

typedef enum {
  OLMOE_OK = 0,
  OLMOE_EINVAL = 1,     /* bad argument: null, negative/too large T, misaligned, aliasing */
  OLMOE_EWORKSPACE = 2, /* workspace missing or smaller than olmoe_moe_workspace_bytes(T) */
  OLMOE_EHIP = 3,       /* a HIP call or kernel launch failed */
  OLMOE_ENODEVICE = 4   /* no usable gfx950 device is current */
} olmoe_status_t;

/* ABI version of the loaded library (OLMOE_ABI_VERSION it was built with). */
OLMOE_API int olmoe_abi_version(void);

/* Text of the last non-OK status on this thread ("" if none). */
OLMOE_API const char* olmoe_last_error(void);

/* Byte offset, in every workspace and `saved` buffer, of the int32 count of
 * fp16 intermediates stored clipped by the last call that used it (see
 * olmoe_moe_forward). */
#define OLMOE_WORKSPACE_CLIP_COUNT_OFFSET 0

/* Bytes of device workspace olmoe_moe_forward needs for T tokens (pure host
 * function, no device access).  Returns 0 for T < 0 or T > OLMOE_MAX_TOKENS.
 * Grows as about 8*T*(1024+2048)*2 bytes (the SwiGLU activations and the
 * per-slot expert outputs) plus routing tables. */
OLMOE_API size_t olmoe_moe_workspace_bytes(int64_t T);

/* Where the dispatch tables live inside the workspace, as byte offsets from
 * its start (pure host function; for inspection and tests):
 *   perm    int32 [8T]   token of each row in expert-contiguous order; rows of
 *                        expert e occupy [offsets[e], offsets[e+1]), tokens
 *                        ascending inside each expert (a stable sort of the
 *                        (token, slot) pairs by expert id)
 *   inv     int32 [T,8]  row holding (t, route_ids[t,j])
 *   offsets int32 [65]   exclusive prefix sum of the per-expert counts
 * Any out-pointer may be NULL. */
OLMOE_API olmoe_status_t olmoe_moe_workspace_layout(int64_t T, size_t* perm_off, size_t* inv_off,
                                          size_t* offsets_off);

/* One OLMoE MoE layer forward for T tokens.
 *
 *   x             bf16 [T,2048]         input rows
 *   W_router      fp32 [64,2048]        router weights (no bias)
 *   W_gate        bf16 [64,1024,2048]   per expert [out,in], in contiguous
 *   W_up          bf16 [64,1024,2048]
 *   W_down        bf16 [64,2048,1024]
 *   T             tokens, 0 <= T <= OLMOE_MAX_TOKENS
 *   out           bf16 [T,2048]         must not overlap any input
 *   route_ids     int32 [T,8] or NULL   chosen experts by descending logit,
 *                                       equal logits -> lower id first
 *   route_probs   fp32 [T,8] or NULL    their 64-way softmax probabilities
 *                                       (not renormalised)
 *   expert_counts int32 [64] or NULL    tokens routed to each expert (sum 8T)
 *   aux_loss      fp32 [1] or NULL      Switch load-balancing loss
 *                                       0.01 * 64 * sum_e f_e P_e with
 *                                       f_e = counts_e / (8T), P_e = mean_t p[t,e]
 *                                       ("OLMoE Guide", item 2)
 *   z_loss        fp32 [1] or NULL      router z-loss 0.001 * mean_t lse_t^2,
 *                                       lse_t = log sum_e exp(l[t,e]) (item 3)
 *   workspace     device buffer of at least olmoe_moe_workspace_bytes(T) bytes,
 *                 256-byte aligned; contents on entry are ignored
 *
 * Arithmetic: router logits, softmax and losses in fp32 (the router is
 * evaluated exactly as an fp32 dot product of the bf16 inputs and fp32
 * weights); expert GEMMs on MFMA with fp32 accumulation (gate/up on bf16 MFMA;
 * down on f16 MFMA, with W_down converted to fp16 after an exact scaling by
 * 16 that the fp32 result undoes exactly: exact for 2^-18 <= |w| < 4096,
 * rounded toward zero with an absolute error below 2^-28 under that, saturated
 * above); the SwiGLU activation is formed in fp32 and stored as fp16, expert
 * outputs are stored as fp16 (both rounded to nearest even), and the weighted
 * sum is accumulated in fp32 over the 8 slots in route order and rounded once
 * to bf16.  An activation or expert output outside fp16's range (|v| > 65504)
 * or NaN is stored clipped to +-65504 and counted: the int32 at byte
 * OLMOE_WORKSPACE_CLIP_COUNT_OFFSET of the workspace holds, once the call has
 * completed on its stream, the number of such values (0 in normal use; the
 * backward, expert-choice and training entry points keep the same count in
 * their workspace or `saved` buffer).
 *
 * T == 0 is valid: expert_counts is zeroed and the losses are set to 0.
 * Errors: OLMOE_EINVAL for a NULL required pointer, T out of range,
 * a pointer not 16-byte aligned, `out` overlapping x, a weight or the
 * workspace, or an optional output (route_ids T*8*4 bytes, route_probs
 * T*8*4, expert_counts 256, aux_loss 4, z_loss 4) overlapping an input, the
 * workspace, `out` or another optional output;
 * OLMOE_EWORKSPACE for a NULL or short workspace; OLMOE_ENODEVICE when the
 * current device is not gfx950; OLMOE_EHIP when a launch fails. */
OLMOE_API olmoe_status_t olmoe_moe_forward(const void* x, const float* W_router, const void* W_gate,
                                 const void* W_up, const void* W_down, int64_t T, void* out,
                                 int32_t* route_ids, float* route_probs,
                                 int32_t* expert_counts, float* aux_loss, float* z_loss,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Router variants ("Mixture-of-experts LLMs from scratch with OLMoE"):
 *   OLMOE_ROUTE_RENORMALIZE in route_flags: route_probs (and so the weights of
 *     the sum) are the chosen probabilities divided by their sum over the 8
 *     slots, the renormalised router of that page's section 2 (equal to a
 *     softmax over the 8 chosen logits, the formula of "OLMoE Guide", item 1);
 *   keep_mask: bit e clear prunes expert e, whose score becomes -inf before the
 *     softmax (section 5 of that page), so it is never chosen, its probability
 *     and count are 0, and lse (hence the z-loss) runs over the kept experts.
 *     OLMOE_KEEP_ALL keeps every expert.
 * The losses always use the (masked) 64-way softmax, not the renormalised
 * weights.  Everything else is as olmoe_moe_forward, which equals
 * olmoe_moe_forward_ex with route_flags 0 and OLMOE_KEEP_ALL.
 * Errors: as olmoe_moe_forward, plus OLMOE_EINVAL for unknown route_flags bits
 * or a keep_mask with fewer than 8 bits set. */
#define OLMOE_ROUTE_RENORMALIZE 1u
#define OLMOE_KEEP_ALL (~(uint64_t)0)
OLMOE_API olmoe_status_t olmoe_moe_forward_ex(const void* x, const float* W_router, const void* W_gate,
                                    const void* W_up, const void* W_down, int64_t T, void* out,
                                    int32_t* route_ids, float* route_probs,
                                    int32_t* expert_counts, float* aux_loss, float* z_loss,
                                    uint32_t route_flags, uint64_t keep_mask,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* One layer of the residual stack with the residual update and the next
 * layer's RMSNorm fused into the layer's last kernel ("Mixture-of-experts LLMs
 * from scratch with OLMoE", section 3: the block adds the MoE output of
 * RMSNorm(h) to the fp32 residual h):
 *   h[t]      += sum_j w[t,j] * Y[t,j]   in fp32 (the layer output is not
 *                rounded to bf16 on the way; h fp32 [T,2048], updated in place)
 *   x_next[t]  = bf16(h[t] / sqrt(mean_k h[t,k]^2 + eps))   if x_next != NULL
 * x is the layer's bf16 input (normally the previous call's x_next); x_next may
 * be the same buffer as x.  Routing outputs, losses, route_flags, keep_mask and
 * the workspace are as olmoe_moe_forward_ex.
 * Errors: as olmoe_moe_forward_ex, plus OLMOE_EINVAL when h is NULL (T > 0),
 * misaligned or overlapping an input or the workspace, when x_next overlaps h,
 * the workspace or an input other than x, or when eps is not > 0 with x_next. */
OLMOE_API olmoe_status_t olmoe_moe_forward_residual(const void* x, const float* W_router,
                                          const void* W_gate, const void* W_up, const void* W_down,
                                          int64_t T, float* h, void* x_next, float eps,
                                          int32_t* route_ids, float* route_probs,
                                          int32_t* expert_counts, float* aux_loss, float* z_loss,
                                          uint32_t route_flags, uint64_t keep_mask,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* Training pair for the default router (token choice): a forward that keeps its
 * state, and a backward that starts from it instead of recomputing the forward.
 *
 * olmoe_moe_forward_train: the layer exactly as olmoe_moe_forward (same outputs,
 * bit for bit), which also leaves in `saved` the routing, the probabilities and
 * lse, the fp32 pre-activations G = x W_gate^T and U = x W_up^T of every routed row,
 * and the expert outputs.  saved: device buffer of at least
 * olmoe_moe_saved_bytes(T) bytes (the backward workspace size), 256-byte aligned,
 * not overlapping any argument.
 *
 * olmoe_moe_backward_saved: the gradients of olmoe_moe_backward (same results, bit
 * for bit) from `saved` as the last olmoe_moe_forward_train left it for the same x,
 * weights and T; the caller keeps that pairing (the library cannot detect a
 * mismatch, and results are then meaningless).  saved is used as the backward's
 * workspace, so its forward state is consumed: run olmoe_moe_forward_train again
 * before another olmoe_moe_backward_saved.  Internal streams as olmoe_moe_backward.
 * Errors: as olmoe_moe_forward / olmoe_moe_backward (EWORKSPACE for a NULL or
 * short `saved`). */
OLMOE_API size_t olmoe_moe_saved_bytes(int64_t T);   /* 0 for T out of range; host only */
OLMOE_API olmoe_status_t olmoe_moe_forward_train(const void* x, const float* W_router, const void* W_gate,
                                       const void* W_up, const void* W_down, int64_t T, void* out,
                                       int32_t* route_ids, float* route_probs,
                                       int32_t* expert_counts, float* aux_loss, float* z_loss,
                                       void* saved, size_t saved_bytes, void* stream);
OLMOE_API olmoe_status_t olmoe_moe_backward_saved(const void* x, const float* W_router, const void* W_gate,
                                        const void* W_up, const void* W_down, int64_t T,
                                        const void* dout, float g_aux, float g_z, float* dx,
                                        float* dW_router, float* dW_gate, float* dW_up,
                                        float* dW_down, void* saved, size_t saved_bytes,
                                        void* stream);

/* Expert-choice routing: the experts choose their tokens ("OLMoE: Open
 * Mixture-of-Experts Language Models", section 4.1.4, where it is compared with
 * token choice; the page gives no formulas, and this is the plainest reading
 * built from the token-choice layer's steps, "OLMoE Guide", items 1-3):
 *   p[t,e]  the same 64-way softmax of the router logits (fp32)
 *   C       = ceil(8T / 64) tokens per expert (the 8T pairs of token choice
 *             shared equally)
 *   S_e     the C tokens with the largest p[t,e]; equal probabilities go to
 *           the lower token id (selection on the fp32 probabilities)
 *   out[t]  = sum over the experts e with t in S_e of p[t,e] * Expert_e(x_t),
 *             accumulated in fp32 in ascending e; a token no expert took gets 0
 *
 *   x, W_*, out   as olmoe_moe_forward;  0 <= T <= OLMOE_EC_MAX_TOKENS
 *   choice_tokens int32 [64,C] or NULL  row e: the tokens of S_e, ascending
 *   choice_probs  fp32 [64,C] or NULL   p[t,e] of those tokens
 *   token_counts  int32 [T] or NULL     experts that took each token (0..64,
 *                                       sum 64C)
 *   aux_loss      fp32 [1] or NULL      0.01 * 64 * sum_e f_e P_e with
 *                                       f_e = C / (8T), P_e = mean_t p[t,e]
 *   z_loss        fp32 [1] or NULL      0.001 * mean_t lse_t^2
 *   workspace     at least olmoe_moe_ec_workspace_bytes(T) bytes, 256-byte
 *                 aligned; contents on entry are ignored
 * The expert GEMMs and their precisions are those of olmoe_moe_forward.
 * T == 0 is valid (the losses are set to 0).
 * Errors: as olmoe_moe_forward (EINVAL for T > OLMOE_EC_MAX_TOKENS, and for any
 * output overlapping an input, another output or the workspace). */
#define OLMOE_EC_MAX_TOKENS ((int64_t)1 << 16) /* the selection holds a column per workgroup in registers */
OLMOE_API size_t olmoe_moe_ec_workspace_bytes(int64_t T);   /* 0 for T out of range; host only */
OLMOE_API olmoe_status_t olmoe_moe_forward_expert_choice(const void* x, const float* W_router,
                                               const void* W_gate, const void* W_up,
                                               const void* W_down, int64_t T, void* out,
                                               int32_t* choice_tokens, float* choice_probs,
                                               int32_t* token_counts, float* aux_loss, float* z_loss,
                                               void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass of the expert-choice layer (olmoe_moe_forward_expert_choice):
 * the gradients of  L = sum_t <dout[t], out[t]> + g_aux * aux_loss + g_z * z_loss
 * with respect to x and every weight, by the chain rule through the layer's
 * steps ("OLMoE Guide", items 1-3; the routing weights are the 64-way
 * probabilities of the pairs the experts took).  Which tokens each expert takes
 * and the shares f_e = C / (8T) are piecewise constant and carry no gradient.
 * The forward is recomputed inside.  Arguments, outputs (fp32, overwritten),
 * precisions, internal streams and errors as olmoe_moe_backward, with 0 <= T <=
 * OLMOE_EC_MAX_TOKENS and a workspace of olmoe_moe_ec_backward_workspace_bytes(T). */
OLMOE_API size_t olmoe_moe_ec_backward_workspace_bytes(int64_t T);   /* 0 for T out of range; host only */
OLMOE_API olmoe_status_t olmoe_moe_backward_expert_choice(const void* x, const float* W_router,
                                                const void* W_gate, const void* W_up,
                                                const void* W_down, int64_t T, const void* dout,
                                                float g_aux, float g_z, float* dx, float* dW_router,
                                                float* dW_gate, float* dW_up, float* dW_down,
                                                void* workspace, size_t workspace_bytes, void* stream);

/* Training pair of the expert-choice layer, as olmoe_moe_forward_train /
 * olmoe_moe_backward_saved for token choice: the forward gives
 * olmoe_moe_forward_expert_choice's outputs bit for bit and keeps its state in
 * `saved` (at least olmoe_moe_ec_saved_bytes(T) bytes, 256-byte aligned); the
 * backward gives olmoe_moe_backward_expert_choice's gradients bit for bit from that
 * state (same x, weights and T; consumed by the call). */
OLMOE_API size_t olmoe_moe_ec_saved_bytes(int64_t T);   /* 0 for T out of range; host only */
OLMOE_API olmoe_status_t olmoe_moe_forward_expert_choice_train(const void* x, const float* W_router,
                                                     const void* W_gate, const void* W_up,
                                                     const void* W_down, int64_t T, void* out,
                                                     int32_t* choice_tokens, float* choice_probs,
                                                     int32_t* token_counts, float* aux_loss,
                                                     float* z_loss, void* saved, size_t saved_bytes,
                                                     void* stream);
OLMOE_API olmoe_status_t olmoe_moe_backward_expert_choice_saved(const void* x, const float* W_router,
                                                      const void* W_gate, const void* W_up,
                                                      const void* W_down, int64_t T, const void* dout,
                                                      float g_aux, float g_z, float* dx,
                                                      float* dW_router, float* dW_gate, float* dW_up,
                                                      float* dW_down, void* saved, size_t saved_bytes,
                                                      void* stream);

/* RMSNorm of the residual stream with unit weight, rounded to the layer's
 * input type: x_out[t] = bf16(h[t] / sqrt(mean_k h[t,k]^2 + eps)), computed in
 * fp32 ("Mixture-of-experts LLMs from scratch with OLMoE", section 3, RMSNorm;
 * the residual stream is kept in fp32 there).
 *   h      fp32 [T,2048]
 *   x_out  bf16 [T,2048], must not overlap h
 * Errors: OLMOE_EINVAL for NULL pointers, T out of range, eps not > 0 or
 * misalignment; OLMOE_ENODEVICE / OLMOE_EHIP as above. */
OLMOE_API olmoe_status_t olmoe_rmsnorm_bf16(const float* h, float eps, int64_t T, void* x_out,
                                  void* stream);

/* Residual update h[t,k] += float(y[t,k]) in fp32 (same section: the block
 * adds the MoE output to the fp32 residual stream).
 *   h  fp32 [T,2048] (updated in place);  y  bf16 [T,2048], must not overlap h. */
OLMOE_API olmoe_status_t olmoe_residual_add(float* h, const void* y, int64_t T, void* stream);

/* Backward pass of one layer with the default router (64-way softmax, top-8,
 * not renormalised, every expert kept): the gradients of
 *     L = sum_t <dout[t], out[t]> + g_aux * aux_loss + g_z * z_loss
 * with respect to x and every weight, by the chain rule through the steps of
 * olmoe_moe_forward ("OLMoE Guide", items 1-3; "Mixture-of-experts LLMs from
 * scratch with OLMoE", section 2).  The routing choice and the routed shares
 * f_e are piecewise constant and carry no gradient.  The forward is recomputed
 * inside (no state is kept between calls): routing, and G = x W_gate^T and
 * U = x W_up^T of every routed row.  The routing weights' gradient
 * <dout[t], Y[t,j]> is taken as <dout[t] W_down[e_j], H[t,j]> from the
 * gradient GEMM through W_down, so the expert outputs are not recomputed.
 *
 *   dout       bf16 [T,2048]          upstream gradient of out
 *   g_aux, g_z                        upstream gradients of the two losses (finite)
 *   dx         fp32 [T,2048]          written
 *   dW_router  fp32 [64,2048]         written (not accumulated)
 *   dW_gate    fp32 [64,1024,2048]    written; zero for experts no token chose
 *   dW_up      fp32 [64,1024,2048]
 *   dW_down    fp32 [64,2048,1024]
 *   workspace  device buffer of olmoe_moe_backward_workspace_bytes(T) bytes,
 *              256-byte aligned (about 230 KiB per token)
 *
 * Arithmetic: the gradient GEMMs run on bf16 MFMA with fp32 accumulation; their
 * bf16 operands are the upstream gradient, the weights, the gathered inputs,
 * dG / dU and w*H (rounded to nearest even); G and U are kept in fp32; the
 * router gradient and the sums into dx run in fp32 in a fixed order.
 * Streams: the two weight-gradient GEMMs run on two internal streams of the
 * calling thread (one pair per device, default priority, created on the first
 * backward call and kept until the process ends), ordered after the earlier
 * work of this call on `stream` and joined back into `stream` with events, so
 * `stream` still passes the call only when all of it is done (also under
 * graph capture, where the fork and join become graph edges; the thread's first
 * backward call on a device creates the pair, so make it outside a capture).
 * Backward calls from one thread share that pair.
 * Errors: OLMOE_EINVAL for NULL / misaligned pointers, T out of range,
 * non-finite g_aux / g_z, outputs overlapping an input, each other or the
 * workspace; OLMOE_EWORKSPACE for a NULL or short workspace; OLMOE_ENODEVICE /
 * OLMOE_EHIP as olmoe_moe_forward (also when the internal streams cannot be
 * created). */
OLMOE_API size_t olmoe_moe_backward_workspace_bytes(int64_t T);
OLMOE_API olmoe_status_t olmoe_moe_backward(const void* x, const float* W_router, const void* W_gate,
                                  const void* W_up, const void* W_down, int64_t T, const void* dout,
                                  float g_aux, float g_z, float* dx, float* dW_router, float* dW_gate,
                                  float* dW_up, float* dW_down, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* One entry point for every backward variant, with one more choice: the
 * expert weight gradients in the weights' own type.  The model was trained in
 * bf16 ("OLMoE: Open Mixture-of-Experts Language Models", Additional
 * Experiments, Figure 27; "OLMoE Guide", item 3 speaks of the backward in
 * FP16/BF16), so a caller may want bf16 weight gradients: OLMOE_BWD_GRAD_BF16
 * returns the fp32 gradients rounded to bf16, in half the bytes.
 *
 * flags (any other bit set is OLMOE_EINVAL):
 *   OLMOE_BWD_SAVED          workspace is the `saved` buffer of the matching
 *                            training forward (olmoe_moe_forward_train, or
 *                            olmoe_moe_forward_expert_choice_train with the next
 *                            flag) for the same x, weights and T; its state is
 *                            consumed; else the forward is recomputed inside
 *   OLMOE_BWD_EXPERT_CHOICE  the expert-choice layer (0 <= T <=
 *                            OLMOE_EC_MAX_TOKENS; workspace of
 *                            olmoe_moe_ec_backward_workspace_bytes(T)), else
 *                            token choice (olmoe_moe_backward_workspace_bytes(T))
 *   OLMOE_BWD_GRAD_BF16      dW_gate, dW_up and dW_down are bf16 (same shapes):
 *                            each value is the fp32 gradient the call computes
 *                            without this flag, rounded to nearest even (the
 *                            same bits as rounding that call's outputs); dx and
 *                            dW_router stay fp32
 * With flags 0, OLMOE_BWD_SAVED, OLMOE_BWD_EXPERT_CHOICE and both, the call is
 * olmoe_moe_backward, olmoe_moe_backward_saved,
 * olmoe_moe_backward_expert_choice and
 * olmoe_moe_backward_expert_choice_saved (bit for bit).  Arguments, internal
 * streams and errors as those, with the output sizes of the chosen gradient
 * type in the overlap checks. */
#define OLMOE_BWD_SAVED ((uint32_t)1 << 0)
#define OLMOE_BWD_EXPERT_CHOICE ((uint32_t)1 << 1)
#define OLMOE_BWD_GRAD_BF16 ((uint32_t)1 << 2)
OLMOE_API olmoe_status_t olmoe_moe_backward_ex(const void* x, const float* W_router, const void* W_gate,
                                     const void* W_up, const void* W_down, int64_t T, const void* dout,
                                     float g_aux, float g_z, float* dx, float* dW_router, void* dW_gate,
                                     void* dW_up, void* dW_down, void* workspace,
                                     size_t workspace_bytes, uint32_t flags, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer
 * exactly as olmoe_moe_forward (same kernels, same results bit for bit), with
 * the workspace in a device array of OLMOE_NOALLOC_SCRATCH_BYTES that the
 * library owns, one per GPU, held until the process ends.  Enough for up to
 * OLMOE_NOALLOC_MAX_TOKENS tokens; a larger T gives OLMOE_EINVAL.  The call
 * allocates and frees nothing (its first call on a GPU looks the array's device
 * address up once).  Every call on a GPU uses that GPU's one array, so calls
 * that overlap on one GPU (two streams, two threads) race and give undefined
 * results: serialise them.  Nothing in the array needs to start at zero.
 * Arguments and errors otherwise as olmoe_moe_forward. */
#define OLMOE_NOALLOC_MAX_TOKENS 1024
#define OLMOE_NOALLOC_SCRATCH_BYTES ((size_t)60 << 20)
OLMOE_API olmoe_status_t olmoe_moe_forward_noalloc(const void* x, const float* W_router, const void* W_gate,
                                         const void* W_up, const void* W_down, int64_t T, void* out,
                                         int32_t* route_ids, float* route_probs,
                                         int32_t* expert_counts, float* aux_loss, float* z_loss,
                                         void* stream);

/* Per-stage timing of olmoe_moe_forward with HIP events recorded on the
 * caller's stream at the boundaries of its stages: 0 router (logits,
 * softmax, top-8), 1 dispatch (scan and permutation), 2 gateup, 3 down,
 * 4 combine.  olmoe_timing_enable(stage_mask) starts recording for later
 * calls on this thread (bit i of the mask brackets stage i; 0 stops
 * recording; OLMOE_TIMING_ALL brackets every stage) and clears the sums; a
 * mask with bits beyond the stages gives OLMOE_EINVAL.  olmoe_timing_read()
 * waits for the recorded events, fills up to `max_stages` per-stage sums in
 * milliseconds (0 for stages outside the mask), writes the number of timed
 * calls to *calls, and returns the number of stages (or -1 on error).  Names
 * of the stages: olmoe_timing_stage_name(i).  Each recorded boundary costs
 * the stream a little time, so bracket only the stages of interest, and
 * olmoe_timing_every(n) (n >= 1, else OLMOE_EINVAL) brackets only every n-th
 * call on this thread from then on (the first call after it is bracketed;
 * olmoe_timing_enable resets n to 1), so a long run can be timed on a sample
 * of its calls. */
#define OLMOE_TIMING_ALL 0x1F
OLMOE_API olmoe_status_t olmoe_timing_enable(int stage_mask);
OLMOE_API int olmoe_timing_read(double* stage_ms, int max_stages, int* calls);
OLMOE_API olmoe_status_t olmoe_timing_every(int n);
OLMOE_API const char* olmoe_timing_stage_name(int stage);

#ifdef __cplusplus
}
#endif
#endif /* OLMOE_MOE_H */
