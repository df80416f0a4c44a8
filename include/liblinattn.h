/*
 * liblinattn -- kernelized linear attention on AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI.  Every tensor argument is a DEVICE pointer owned by the caller;
 * the library allocates nothing, keeps no per-call state and never blocks the
 * host.  Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 * the default stream).  Argument errors are reported synchronously, before any
 * work is enqueued, and leave every output untouched; la_last_error_message()
 * then holds a one-line explanation (thread-local).
 *
 * Notation follows the pages: B batch, T tokens in this call, H heads, Dk
 * query/key head size, Dv value head size, phi the feature map, eps the
 * normalization epsilon.  All layouts are row-major with the innermost index
 * last:
 *   q, k       : (B, T, H, Dk)        v, out : (B, T, H, Dv)
 *   mask       : (B, T) uint8, nonzero = valid token; NULL = all valid
 *   state kv   : (B, H, Dk, Dv) float32  ("key_value_state")
 *   state k    : (B, H, Dk)     float32  ("key_state"), only with the normalizer
 * q, k, v and out share one floating dtype (la_dtype); state is always float32
 * ("[Feature] LinearAttention layer for Keras", sections "Mathematical
 * definition", "Streaming State", "Numerical Stability").
 *
 * Supported head sizes: Dk and Dv each one of 32, 64, 128 (la_forward,
 * la_forward_noalloc, la_step); the gated and delta calls and la_backward need
 * Dk == Dv.  Other sizes return LA_ERR_UNSUPPORTED (no slower path covers
 * them).  With Dk != Dv the kernels run at the larger size with the smaller
 * side zero-padded in registers and LDS (memory is read and written at the
 * caller's sizes).
 */
#ifndef LIBLINATTN_H
#define LIBLINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
  LA_ERR_DTYPE = 2,        /* dtype code is not a supported floating type */
  LA_ERR_SHAPE = 3,        /* negative / zero sizes, Hq not a multiple of Hkv, ... */
  LA_ERR_STATE = 4,        /* state pointers inconsistent with mode / normalizer */
  LA_ERR_BAD_ARG = 5,      /* bad enum, eps < 0, partial overlap of buffers, ... */
  LA_ERR_UNSUPPORTED = 6,  /* valid request this library does not implement */
  LA_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than la_*_workspace_size */
  LA_ERR_DEVICE = 8        /* the HIP runtime reported an error at launch */
} la_status;

/* Element type of q, k, v, decay and out.  Arithmetic is the same for both
 * 16-bit types: they are widened to float32 for the feature map and rounded to
 * bf16 for the matrix products, which accumulate in float32 (fp16 products
 * would overflow on the running sums of long sequences); fp16 results are
 * rounded to fp16 on the way out.  F32 computes in float32 throughout. */
typedef enum { LA_DT_F32 = 0, LA_DT_BF16 = 1, LA_DT_F16 = 2 } la_dtype;

/* phi: elu(x)+1 (x+1 for x>0, exp(x) otherwise), or relu(x)+eps with the same
 * eps as the denominator ("[Feature] LinearAttention layer for Keras", section
 * "Feature maps"). */
typedef enum { LA_FM_ELU_PLUS_ONE = 0, LA_FM_RELU_EPS = 1 } la_feature_map;

/* Zero-fill a streaming state: kv (B,H,Dk,Dv) and, if k != NULL, k (B,H,Dk).
 * The initial state of a causal stream is all zeros ("[Feature] LinearAttention
 * layer for Keras", section "Streaming State", get_initial_state). */
la_status la_initial_state(float* kv, float* k, int64_t B, int64_t H, int64_t Dk, int64_t Dv,
                           void* stream);

/* Bytes of device workspace la_forward needs for this shape (0 = none).  The
 * value depends only on the arguments, never on the device. */
la_status la_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                            int32_t dtype, int32_t causal, size_t* bytes);

/* Full-sequence (or chunk-of-a-stream) attention.
 *
 * causal != 0 ("Mathematical definition / Causal", "Masking / Causal"): per
 * (b,h), token by token, S += phi(k_t) v_t^T and Z += phi(k_t) for valid t, then
 * out_t = phi(q_t)^T S / (phi(q_t)^T Z + eps) (or phi(q_t)^T S when
 * use_normalizer == 0); the current token is in its own context; invalid tokens
 * leave S, Z unchanged and get out_t = 0.  state_in_* (NULL = zeros) is the
 * state before the first token, state_out_* (NULL = not returned) receives the
 * state after the last one, so consecutive calls chain exactly like one call
 * over the concatenated tokens ("Streaming State").  state_out may be the same
 * buffers as state_in (in-place streaming); any other overlap is LA_ERR_BAD_ARG.
 * With use_normalizer == 0 the k parts must be NULL (only kv is carried); with
 * use_normalizer != 0, state_in_k / state_out_k are required whenever the
 * matching kv pointer is given.
 *
 * causal == 0 ("Mathematical definition / Non-causal", "Masking / Non-causal"):
 * S, Z are sums over all valid tokens, out_i = phi(q_i)^T S / (phi(q_i)^T Z + eps)
 * at valid i and 0 at invalid i.  Non-causal attention exposes no state: all
 * four state pointers must be NULL (else LA_ERR_STATE).
 *
 * T == 0 is allowed: nothing is read, state_out receives state_in (or zeros).
 * workspace must hold la_workspace_size() bytes (may be NULL when that is 0);
 * its contents on entry do not matter. */
la_status la_forward(const void* q, const void* k, const void* v, const uint8_t* mask,
                     const float* state_in_kv, const float* state_in_k,
                     float* state_out_kv, float* state_out_k,
                     int32_t causal, int32_t feature_map, int32_t use_normalizer, float eps,
                     void* out, int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                     int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* la_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments and results without the workspace, which is replaced by a
 * scratch array of LA_NOALLOC_SCRATCH_BYTES that the library keeps on each GPU
 * it runs on until the process ends.  No call allocates, frees or runs an
 * allocating library routine.  Where la_forward would split a sequence (few
 * (batch, head) units), the split is bounded by the scratch size: a causal
 * call then uses fewer, longer segments (at worst one, which needs no
 * scratch), so every causal call is accepted; a non-causal call needs at least
 * B*H*(Dk*Dv + Dk)*4 bytes and returns LA_ERR_WORKSPACE beyond the scratch
 * size (B*H > 1016 at Dk = Dv = 128, for example).  The stream must belong to
 * the current device (else LA_ERR_DEVICE).  Every call on one GPU shares that
 * GPU's scratch: calls that overlap in time on one GPU (two streams, two host
 * threads) race and give wrong results; calls ordered on one stream are safe.
 * The scratch needs no clearing: each call writes every byte it reads. */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
la_status la_forward_noalloc(const void* q, const void* k, const void* v, const uint8_t* mask,
                             const float* state_in_kv, const float* state_in_k,
                             float* state_out_kv, float* state_out_k,
                             int32_t causal, int32_t feature_map, int32_t use_normalizer, float eps,
                             void* out, int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                             int32_t dtype, void* stream);

/* One causal decode step (T == 1): q, k, v are (B, H, Dk/Dv), mask is (B) or
 * NULL, out is (B, H, Dv).  Same semantics as la_forward with T == 1
 * ("Streaming State": token-by-token execution; "Execution Modes": a single
 * token runs the recurrence).  state_in_kv is required (a stream always has a
 * state; start one with la_initial_state); state_out may alias state_in
 * exactly. */
la_status la_step(const void* q, const void* k, const void* v, const uint8_t* mask,
                  const float* state_in_kv, const float* state_in_k,
                  float* state_out_kv, float* state_out_k,
                  int32_t feature_map, int32_t use_normalizer, float eps,
                  void* out, int64_t B, int64_t H, int64_t Dk, int64_t Dv, int32_t dtype,
                  void* stream);

/* Bytes of device workspace la_gated_forward needs (0 = none); shape-only.
 * per_dim_decay as in la_gated_forward.  With few (batch, kv head) units and a
 * long sequence the sequence is split, and the workspace holds one fp32 state
 * per segment; a per-dim decay adds one int flag per (unit, segment), so it
 * needs a workspace whenever T > 1 (except fp32 at Dk = 128, see below). */
la_status la_gated_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk,
                                  int64_t Dv, int32_t dtype, int32_t per_dim_decay, size_t* bytes);

/* Gated linear recurrence with grouped-query heads (the LinearAttention
 * operator page, ai.onnx since version 27: "gated" rule, or the "linear" rule
 * when decay == NULL):
 *   S_t = diag(exp(g_t)) S_{t-1} + k_t v_t^T   (per kv head)
 *   o_t = scale * q_t^T S_t                    (per query head, S after the update)
 * g_t is one log-space value per kv head (per_dim_decay == 0: decay (B,T,Hkv),
 * scaling all of S) or one per key dimension (per_dim_decay != 0: decay
 * (B,T,Hkv*Dk), scaling row dk of S; the page's "gated" rule with a decay of
 * shape (B, T, kv_num_heads * d_k)).  Query head h reads kv head h / (Hq/Hkv).
 * No feature map, no normalizer, no mask.  Packed layouts (byte-identical to
 * the 4-D ones):
 *   q (B,T,Hq*Dk), k (B,T,Hkv*Dk), v (B,T,Hkv*Dv), out (B,T,Hq*Dv) and decay
 *   in `dtype`, the decay log-space (NULL = all zero);
 *   past_state (B,Hkv,Dk,Dv) float32 (NULL = zeros); present_state (same shape,
 *   float32) is always written and may alias past_state exactly.
 * scale == 0 means 1/sqrt(Dk).  Hq must be a positive multiple of Hkv
 * (else LA_ERR_SHAPE); any multiple is supported, multi-query (Hkv = 1)
 * included.  Decays of any strength are supported.  A per-dim decay is
 * evaluated chunk-parallel with keys rescaled relative to a reference token;
 * where some dimension's cumulative decay inside a 64-token chunk exceeds 60
 * in magnitude, the segment concerned is flagged in the workspace and a
 * second launch re-evaluates its tokens one at a time (exact, and slower by a
 * large factor for that segment).  fp32 inputs at Dk = 128 with a per-dim
 * decay and T > 1 (whose chunk tiles exceed the LDS) run a token-by-token
 * recurrence over the whole sequence instead, the state held on chip: no
 * workspace (la_gated_workspace_size reports 0).
 * workspace: la_gated_workspace_size bytes, 16-byte aligned, overlapping no
 * other argument (NULL when that is 0); a smaller one is LA_ERR_WORKSPACE.
 * Its contents need no initialisation and are scratch after the call. */
la_status la_gated_forward(const void* q, const void* k, const void* v, const void* decay,
                           int32_t per_dim_decay, const float* past_state, float* present_state,
                           void* out, int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk,
                           int64_t Dv, int32_t dtype, float scale, void* workspace,
                           size_t workspace_bytes, void* stream);

/* One token of the gated / linear recurrence with grouped-query heads: the
 * T == 1 case of la_gated_forward, as a decode step that streams the fp32 state
 * once (the LinearAttention operator page, "Description": the recurrence is
 * token-by-token; its decode example is a single token with a past state):
 *   S' = diag(exp(g)) S + k v^T   (per kv head),   o = scale q^T S'   (per query head).
 * q (B, Hq*Dk), k (B, Hkv*Dk), v (B, Hkv*Dv), out (B, Hq*Dv) in `dtype`;
 * decay in `dtype`, log-space: (B, Hkv), or (B, Hkv*Dk) with per_dim_decay
 * (NULL = all zero);
 * past_state (B,Hkv,Dk,Dv) float32 (NULL = zeros); present_state (same shape,
 * float32) is always written and may alias past_state exactly (in-place step).
 * The states must be 16-byte aligned.  scale == 0 means 1/sqrt(Dk).  Sizes,
 * dtypes and errors as la_gated_forward; no workspace. */
la_status la_gated_step(const void* q, const void* k, const void* v, const void* decay,
                        int32_t per_dim_decay, const float* past_state, float* present_state,
                        void* out, int64_t B, int64_t Hq, int64_t Hkv, int64_t Dk, int64_t Dv,
                        int32_t dtype, float scale, void* stream);

/* Delta-rule recurrences with grouped-query heads (the LinearAttention operator
 * page, ai.onnx since version 27, update rules "delta" and "gated_delta"):
 *   delta:        S_t = S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T
 *   gated_delta:  S_t = E_t S_{t-1} + beta_t k_t (v_t - (E_t S_{t-1})^T k_t)^T,
 *                 E_t = exp(g_t) (per kv head) or diag(exp(g_t)) (per key dim)
 *   o_t = scale * q_t^T S_t   (per query head, S after the update)
 * decay == NULL selects "delta"; otherwise decay is (B,T,Hkv) or, with
 * per_dim_decay, (B,T,Hkv*Dk), log-space.  beta (required) is (B,T,Hkv) with
 * beta_per_head, else (B,T,1) shared by all kv heads.  Other layouts, dtypes,
 * scale, past/present state and GQA as la_gated_forward; keys are expected
 * L2-normalised (operator page, "Inputs").  Evaluated chunk-parallel (64-token
 * chunks, a 64 x 64 triangular solve per chunk) by one workgroup per (batch,
 * kv head, query-head group) over the whole sequence.  With few of those (at
 * most 64) and a workspace of la_delta_workspace_size bytes, the sequence is
 * split into segments of whole chunks instead: every segment's state map
 * S_end = M S_start + N (M = the product of its (I - beta k k^T) E_t factors)
 * is formed by the same kernels, run from S = I with zero values (M) and from
 * S = 0 (N), the start states follow by composing the maps in order (fp32
 * D x D products), and every segment then runs with outputs from its start
 * state.  workspace NULL, or fewer bytes than reported, runs without the split
 * (same results up to rounding, one workgroup per unit).  Decays of any strength are
 * supported: per-dim decays, and per-head decays with fp16 inputs, rescale the
 * keys relative to a reference token, and a workgroup whose cumulative decay
 * inside a 64-token chunk exceeds 60 in magnitude re-evaluates its whole
 * sequence one token at a time (exact, and slower by a large factor for that
 * workgroup).  fp32 inputs at Dk = 128 with a per-dim decay and T > 1 run the
 * step below once per token (slower: one state read and write per token).
 * T == 1 runs a streaming step instead: one read and one write of the state
 * per (batch, kv head), in place allowed (present_state == past_state), every
 * dtype and head size. */
la_status la_delta_forward(const void* q, const void* k, const void* v, const void* decay,
                           int32_t per_dim_decay, const void* beta, int32_t beta_per_head,
                           const float* past_state, float* present_state, void* out, int64_t B,
                           int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk, int64_t Dv, int32_t dtype,
                           float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace (16-byte aligned, not overlapping any argument)
 * with which la_delta_forward splits these sizes over T; 0 = it never splits
 * them (enough workgroups already, T == 1, or the token-by-token path).  Sizes
 * and errors as la_delta_forward; per_dim_decay as passed there. */
la_status la_delta_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk, int64_t Dv,
                                  int32_t dtype, int32_t per_dim_decay, size_t* bytes);

/* Bytes of device workspace la_backward needs for these sizes (0 = none). */
la_status la_backward_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                     int32_t dtype, int32_t use_normalizer, size_t* bytes);

/* Gradients of causal la_forward (the Keras proposal asks for recurrent/parallel
 * gradient parity and finite gradients, "Stability" and "Acceptance"), for the
 * loss sum(dout * out) + sum(dstate_out_kv * S_T) + sum(dstate_out_k * Z_T):
 *   q, k, v, mask, state_in_kv/k, feature_map, use_normalizer, eps: as passed to
 *     the causal forward (its output is not needed);
 *   dout (B,T,H,Dv) in `dtype`; dstate_out_kv (B,H,Dk,Dv) and, with the
 *     normalizer, dstate_out_k (B,H,Dk), float32, or NULL (zero);
 *   dq, dk (B,T,H,Dk), dv (B,T,H,Dv) in `dtype`: written; 0 at invalid tokens;
 *   dstate_in_kv (B,H,Dk,Dv), dstate_in_k (B,H,Dk, normalizer only), float32:
 *     the gradient of the initial state, always written.
 * Outputs may not overlap the inputs or each other; every buffer is 16-byte
 * aligned (else LA_ERR_BAD_ARG).  Evaluated as three
 * chunk-parallel linear-rule recurrences (two in reversed time) plus prefix
 * sums, in float32; needs la_backward_workspace_size bytes of workspace. */
la_status la_backward(const void* q, const void* k, const void* v, const uint8_t* mask,
                      const float* state_in_kv, const float* state_in_k, const void* dout,
                      const float* dstate_out_kv, const float* dstate_out_k, int32_t feature_map,
                      int32_t use_normalizer, float eps, void* dq, void* dk, void* dv,
                      float* dstate_in_kv, float* dstate_in_k, int64_t B, int64_t T, int64_t H,
                      int64_t Dk, int64_t Dv, int32_t dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Static string naming a status code. */
const char* la_status_string(la_status s);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* la_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBLINATTN_H */
