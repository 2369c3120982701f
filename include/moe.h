/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts
 * feed-forward layer, forward pass.
 *
 * The layer (page "MoE: how sparse activation saves compute", sections 3.1,
 * 3.2, 3.5, 3.6):
 *   z_t   = W_route u_t                      router scores, [T, N]
 *   p_t   = softmax(z_t)                     fp32
 *   S_t   = the k experts of largest p       descending p, ties -> lower index
 *   a_t,i = p_t,i / sum_{j in S_t} p_t,j     (MOE_GATE_RENORM)
 *         = p_t,i                            (MOE_GATE_PROB, Switch top-1 style)
 *   dispatch: (token, slot) pairs grouped by expert in token order; with a
 *   capacity C only the first C tokens reaching an expert are kept, the
 *   others contribute 0 (their token skips the layer through the residual)
 *   F_i(x) = W_down,i act(W_gate,i x, W_up,i x)
 *   y_t   = sum over kept slots of a_t,i F_i(u_t)
 * with act = SwiGLU, SiLU(g) * v, or SiTU-GLU, SiLU(bg tanh(g/bg)) * bu tanh(v/bu)
 * (page "Stable LatentMoE interactive demo", SiTU-GLU passage).
 *
 * Latent variant (same page, width-separation and RMSNorm passages):
 *   x_l = W_ldown u (d -> l); routing still reads u; experts map l -> h -> l;
 *   r   = sum a E_i(x_l);  y = W_lup (r / sqrt(mean(r^2) + eps))
 *         + sum_j SwiGLU_j(u) over n_shared shared experts of hidden h_shared.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never frees or keeps them.  Layouts are row-major and densely packed.
 *   - bf16 tensors hold raw bfloat16 bit patterns (uint16).
 *   - Calls are asynchronous on the given HIP stream (0 = the null stream),
 *     allocate nothing and never synchronise the host with the device.
 *   - Arguments are validated synchronously before any launch.  On error no
 *     kernel is launched and a status other than MOE_OK is returned:
 *       MOE_ERR_ARG          a null required pointer, an unset or out-of-range
 *                            descriptor field (see moe_desc_init)
 *       MOE_ERR_UNSUPPORTED  a valid layer these kernels do not implement
 *                            (there is no fallback path)
 *       MOE_ERR_WORKSPACE    ws is null or smaller than moe_workspace_bytes()
 *       MOE_ERR_HIP          a launch failed (hipGetLastError after launch)
 *   - No exceptions cross the ABI; apart from the per-GPU scratch array of
 *     moe_forward_noalloc the library holds no mutable global state, so
 *     calls on different streams with different workspaces may overlap.
 *     Results are bitwise deterministic (no floating-point atomics).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status_t;

/* MOE_FP8_E4M3: OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
   mantissa bits; no infinities, S.1111.111 is NaN; largest finite 448, the
   bound page "Stable LatentMoE interactive demo" quotes in its SiTU-GLU
   passage), with one fp32 scale per weight row.
   MOE_MXFP4: OCP MX FP4 (the 4-bit experts of page "Kestrel-MCU notes #13",
   section 二, in the OCP microscaling form): E2M1 codes (1 sign, 2 exponent
   bits with bias 1, 1 mantissa bit: +-0, 0.5, 1, 1.5, 2, 3, 4, 6) packed two
   per byte, element 2i of a row in the low nibble of byte i, and one E8M0
   scale byte (2^(s - 127), 0xFF NaN) per 32 consecutive elements of a row.
   Both only for the routed experts' weights (w_dtype) under bf16
   activations.  MXFP4 on the decode path (T <= 64) needs each contraction
   width (the expert input width and h) below 2048 or a multiple of 512
   (MOE_ERR_UNSUPPORTED otherwise). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP4 = 3 } moe_dtype_t;

/* Combine weight of a selected expert (page "MoE: how sparse activation
   saves compute", section 3.2: Mixtral renormalises over S_t; Switch top-1
   keeps the selected probability). */
typedef enum { MOE_GATE_RENORM = 0, MOE_GATE_PROB = 1 } moe_gate_t;

typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_SITU_GLU = 1 } moe_act_t;

/* Layer descriptor.  Every field must be set explicitly: moe_desc_init()
   fills all of them with an "unset" sentinel and validation rejects any
   field still holding it (a silently inherited default is a bug source). */
typedef struct moe_desc {
  int64_t T;          /* tokens, >= 1 */
  int32_t d;          /* model width */
  int32_t h;          /* routed-expert hidden width (H of the latent layer) */
  int32_t N;          /* routed experts, 1..1024 */
  int32_t k;          /* experts per token, 1..min(N, 32) */
  int32_t capacity;   /* slots per expert C >= 0, or -1 for unlimited */
  int32_t act_dtype;  /* moe_dtype_t of u, y and intermediate activations */
  int32_t w_dtype;    /* moe_dtype_t of the routed experts' weights; the latent
                         projections and shared experts use act_dtype */
  int32_t router_dtype; /* moe_dtype_t of W_route */
  int32_t gate;       /* moe_gate_t */
  int32_t act;        /* moe_act_t of the routed experts */
  float beta_g;       /* SiTU-GLU caps (> 0, finite); ignored by SwiGLU */
  float beta_u;
  int32_t l;          /* 0: plain layer; > 0: latent width */
  int32_t n_shared;   /* latent: shared SwiGLU experts (>= 0); plain: 0 */
  int32_t h_shared;   /* latent: shared-expert hidden width; plain: 0 */
  float rms_eps;      /* latent: RMSNorm epsilon (>= 0); plain: any finite */
  float aux_alpha;    /* alpha of the auxiliary balance term (finite) */
} moe_desc_t;

/* Device pointers of the layer's weights.
   Plain layer: W_route [N, d]; W_gate, W_up [N, h, d]; W_down [N, d, h].
   Latent layer: W_route [N, d]; W_gate, W_up [N, h, l]; W_down [N, l, h];
   W_ldown [l, d]; W_lup [d, l]; Ws_gate, Ws_up [n_shared, h_shared, d];
   Ws_down [n_shared, d, h_shared].  Unused pointers may be null.
   Each expert's matrices are contiguous and experts follow one another, so
   only the selected experts' bytes are ever read.
   selection_bias [N] fp32, nullable: the router picks the top-k of z + b
   (Quantile Balancing bias, see moe_qb_update) while the combine weights
   still come from the unbiased softmax; null = no bias.
   Scales (w = d, or l for the latent layer):
   - w_dtype MOE_FP8_E4M3: W_gate / W_up / W_down hold E4M3 codes (uint8,
     same shapes) and gate_scale, up_scale [N, h], down_scale [N, w] are fp32:
     weight row r of expert i is scale[i, r] times its codes' values;
   - w_dtype MOE_MXFP4: W_gate, W_up [N, h, w/2] and W_down [N, w, h/2] hold
     packed E2M1 codes and gate_scale, up_scale [N, h, w/32], down_scale
     [N, w, h/32] are E8M0 bytes (uint8), one per 32 elements of a row;
   - any other w_dtype: all three must be null.
   With fp8 or MXFP4 all three are required. */
typedef struct moe_weights {
  const void *W_route, *W_gate, *W_up, *W_down;
  const void *W_ldown, *W_lup, *Ws_gate, *Ws_up, *Ws_down;
  const float *selection_bias;
  const void *gate_scale, *up_scale, *down_scale;
} moe_weights_t;

/* Optional outputs of moe_forward (device pointers; each may be null, the
   workspace then holds the value).  Shapes as in moe_route/moe_dispatch. */
typedef struct moe_outputs {
  int32_t *topk_idx;
  float *topk_w;
  float *stats;
  int32_t *counts, *offsets, *kept_offsets, *perm, *row_of;
  uint8_t *drop;
  float *y_perm; /* [sum_i min(L_i, C), w] fp32: the experts' outputs of the
                    kept rows (what moe_expert_ffn writes; the input of
                    moe_route_backward) */
  void *gate_up; /* [sum_i min(L_i, C), 2h] bf16: each kept row's gate sums
                    G = W_gate x (columns 0..h-1) and up sums U = W_up x
                    (columns h..2h-1), rounded to bf16, kept so that the
                    backward need not recompute them.  Only with bf16
                    activations and expert weights on the tiled path (T > 64);
                    MOE_ERR_UNSUPPORTED otherwise. */
} moe_outputs_t;

/* Sets every field of *desc to the "unset" sentinel. */
void moe_desc_init(moe_desc_t *desc);

const char *moe_status_string(moe_status_t s);

/* Bytes of workspace any entry point below needs for this layer (the same
   figure serves all of them).  *bytes receives 0 on error. */
moe_status_t moe_workspace_bytes(const moe_desc_t *desc, size_t *bytes);

/* Capacity C = ceil(c * k * T / N): with k slots per token capacity counts
   k*T dispatches (section 3.5; at k = 1 this is ceil(c T / N)).
   Returns -1 if T < 1, N < 1, k < 1 or c is not finite and positive. */
int32_t moe_capacity_from_factor(int64_t T, int32_t N, int32_t k, double c);

/* Router: scores, fp32 softmax, top-k and gate weights (section 3.2), plus
   balance statistics (section 3.4).
     u        [T, d] act_dtype (plain and latent layers both route on u)
     W_route  [N, d] router_dtype
     topk_idx [T, k] int32 out: experts of each token, by descending p (ties
              to the lower index); k distinct experts below N for any input:
              a score that is NaN ranks below every number
     topk_w   [T, k] fp32 out: combine weights a
     stats    [2N + 2] fp32 out, nullable: f_0..f_{N-1} (share of tokens whose
              argmax is i, before capacity), P_0..P_{N-1} (mean p),
              N sum f P, aux_alpha N sum f P. */
moe_status_t moe_route(const moe_desc_t *desc, const void *u, const void *W_route,
                       int32_t *topk_idx, float *topk_w, float *stats, void *ws,
                       size_t ws_bytes, moe_stream_t stream);

/* moe_route with a selection bias (page "Stable LatentMoE interactive demo",
   Quantile Balancing passage): topk_idx holds the k largest z + bias (ties to
   the lower index, by descending z + bias), topk_w the weights from the
   unbiased p (renormalised over the selected set, or p itself for
   MOE_GATE_PROB), and stats keep the unbiased arg-max for f.
     bias [N] fp32 device pointer; null gives moe_route exactly. */
moe_status_t moe_route_biased(const moe_desc_t *desc, const void *u, const void *W_route,
                              const float *bias, int32_t *topk_idx, float *topk_w,
                              float *stats, void *ws, size_t ws_bytes, moe_stream_t stream);

/* One Quantile Balancing step (same passage): with each token's cutoff a_t,
   the k-th largest z_t + bias, held fixed, expert j admits token t exactly
   when bias_j >= a_t - z_tj, so the bias that admits q tokens is the q-th
   smallest of required_tj = a_t - z_tj over the T tokens.
     u        [T, d] bf16; W_route [N, d] bf16 (the router's logits z are
              computed on the MFMA path: needs act and router dtype bf16)
     bias     [N] fp32 in, nullable (null = zeros): the current bias
     q        target tokens per expert, 1..T; q <= 0 selects round(k T / N)
     method   0: exact q-th smallest (radix select);
              1: estimate from a 256-bin histogram over each expert's
                 [min, max] of required, linear inside the bin (within one bin
                 width of the exact value)
     new_bias [N] fp32 out (may equal bias only if the caller does not need
              the old values; the update reads bias before writing new_bias)
   MOE_ERR_ARG for q > T or an unknown method; MOE_ERR_UNSUPPORTED for fp32
   activations or router weights. */
moe_status_t moe_qb_update(const moe_desc_t *desc, const void *u, const void *W_route,
                           const float *bias, int32_t q, int32_t method, float *new_bias,
                           void *ws, size_t ws_bytes, moe_stream_t stream);

/* Router backward (page "MoE: how sparse activation saves compute", §3.2
   eqs. z, p, a, y and §3.4 eq. L_aux, differentiated): the router's share of
   the gradient of L = <dy, y> + aux_scale * L_aux, with the selected sets,
   the expert outputs and the arg-max shares f held fixed.
     u, W_route        the forward's inputs (bf16)
     topk_idx, row_of  the forward's selection and row map (moe_outputs_t)
     stats             the forward's statistics; f = stats[0..N)
     y_perm            the forward's expert outputs [R, d] fp32
     dy                [T, d] bf16, the gradient of the loss at y
     aux_scale         weight of L_aux (alpha is desc->aux_alpha)
     dz                [T, N] fp32 out: gradient at the router logits
     dW_route          [N, d] fp32 out
     du                [T, d] fp32 out: the router's part of the gradient at u
                       (the experts' part is not computed here)
   Steps: da = dy_t . F per kept slot; the renorm (or prob) gate backward;
   the aux term aux_scale alpha N f_i / T on every dp; the softmax backward;
   dW_route = dz^T u; du = dz W_route.  Plain layers with bf16 activations
   and router only (MOE_ERR_UNSUPPORTED otherwise). */
moe_status_t moe_route_backward(const moe_desc_t *desc, const void *u, const void *W_route,
                                const int32_t *topk_idx, const int32_t *row_of,
                                const float *stats, const float *y_perm, const void *dy,
                                float aux_scale, float *dz, float *dW_route, float *du, void *ws,
                                size_t ws_bytes, moe_stream_t stream);

/* Workspace of moe_experts_backward (plain layer) or moe_latent_backward
   (latent layer): its own, larger than the forward's (the recomputed
   gate/up, dY/dG/dU rows and the expert-segmented transposes the weight
   gradients reduce over; for the latent layer also its per-token rows and
   the transposed operands of the T-long contractions; K-contiguous copies of
   W_down and W_gate | W_up only for experts that average more than 1024
   kept rows, which are otherwise read as stored).  Returns
   MOE_ERR_UNSUPPORTED where those entry points do. */
moe_status_t moe_backward_workspace_bytes(const moe_desc_t *desc, size_t *bytes);

/* The experts' backward (page "MoE: how sparse activation saves compute",
   §3.1 eq. F and §3.2 eq. y, differentiated): the experts' share of the
   gradient of L = <dy, y> with the combine weights held fixed (their own
   gradient is moe_route_backward's).  For each kept row of expert i with
   token t and weight a: dY = a dy_t; G = W_gate x, U = W_up x (recomputed);
   dH = W_down^T dY; (dG, dU) = act'(G, U) dH; dx_t += W_gate^T dG +
   W_up^T dU; dW_down += dY act(G, U)^T; dW_gate += dG x^T; dW_up += dU x^T.
     w         W_gate, W_up, W_down of the forward (bf16)
     u         [T, d] bf16 the forward's input (x = u for the plain layer)
     topk_w, offsets, kept_offsets, perm, row_of   the forward's (moe_outputs_t)
     gate_up   the forward's saved G | U rows (moe_outputs_t.gate_up), or
               null: G and U are then recomputed (the same values: the
               forward rounds the same fp32 sums)
     dy        [T, d] bf16
     dx        [T, d] fp32 out: the experts' part of the gradient at u
     dW_gate, dW_up [N, h, d], dW_down [N, d, h]  fp32 out, all three or
               none (null: input gradient only); experts with no kept row
               get zeros
     ws        moe_backward_workspace_bytes() bytes
   Intermediates are rounded to bf16 where they feed the MFMA GEMMs (dY, G,
   U, dG, dU); every sum is fp32.  Plain layers with bf16 activations and
   weights only (MOE_ERR_UNSUPPORTED otherwise; moe_latent_backward covers
   the latent layer). */
moe_status_t moe_experts_backward(const moe_desc_t *desc, const moe_weights_t *w, const void *u,
                                  const float *topk_w, const int32_t *offsets,
                                  const int32_t *kept_offsets, const int32_t *perm,
                                  const int32_t *row_of, const void *gate_up, const void *dy,
                                  float *dx, float *dW_gate, float *dW_up, float *dW_down,
                                  void *ws, size_t ws_bytes, moe_stream_t stream);

/* Gradients of the latent layer (device pointers, fp32, row-major; shapes
   with the weights' at moe_weights_t). */
typedef struct moe_latent_grads {
  float *du;                 /* [T, d] */
  float *dz;                 /* [T, N] gradient at the router logits */
  float *dW_route;           /* [N, d] */
  float *dW_ldown;           /* [l, d] */
  float *dW_lup;             /* [d, l] */
  float *dW_gate, *dW_up;    /* [N, h, l]; zero for an expert with no kept row */
  float *dW_down;            /* [N, l, h] */
  float *dWs_gate, *dWs_up;  /* [n_shared, h_shared, d]; unused if n_shared = 0 */
  float *dWs_down;           /* [n_shared, d, h_shared] */
} moe_latent_grads_t;

/* The LatentMoE layer's backward (page "Stable LatentMoE interactive demo":
   the layer of its width-separation, RMSNorm and SiTU-GLU passages,
   differentiated): the whole gradient of L = <dy, y> + aux_scale * L_aux
   with the selected sets, the capacity drops and f held fixed.  With
   x_l = W_ldown u, r = sum_kept a E_i(x_l), n = r / sqrt(mean(r^2) + eps)
   and y = W_lup n + sum_j S_j(u):
     dn = dy W_lup; dW_lup = dy^T n; dr = (dn - n mean(dn * n)) / rms;
     the routed experts' backward at width l driven by dr (dx_l and their
     weight gradients, as moe_experts_backward);
     the router's backward driven by dr and the expert outputs (dz, dW_route
     and its part of du, as moe_route_backward);
     du += dx_l W_ldown; dW_ldown = dx_l^T u;
     each shared expert's backward on u and dy (weight 1 for every token).
     u        [T, d] bf16, the forward's input
     fwd      the forward's outputs: topk_idx, topk_w, stats, offsets,
              kept_offsets, perm, row_of and y_perm [R, l] are required;
              gate_up [R, 2h] is used when set (the routed experts' G | U,
              otherwise recomputed)
     dy       [T, d] bf16
     g        all of its pointers (the shared ones only when n_shared > 0)
     ws       moe_backward_workspace_bytes() bytes
   x_l, dr, n and dx_l are rounded to bf16 where they feed the MFMA GEMMs;
   every sum is fp32.  bf16 activations, expert weights and router only
   (MOE_ERR_UNSUPPORTED otherwise, and for a plain layer). */
moe_status_t moe_latent_backward(const moe_desc_t *desc, const moe_weights_t *w, const void *u,
                                 const moe_outputs_t *fwd, const void *dy, float aux_scale,
                                 const moe_latent_grads_t *g, void *ws, size_t ws_bytes,
                                 moe_stream_t stream);

/* Dispatch: group the T*k (token, slot) entries e = t*k + s by expert in
   token order (sections 3.5, 3.6, 3.8).
     topk_idx     [T, k] int32 in (values in [0, N); a token names an expert once)
     counts       [N]   int32 out: L_i, entries routed to expert i (before capacity)
     offsets      [N+1] int32 out: exclusive prefix sum of L
     kept_offsets [N+1] int32 out: exclusive prefix sum of min(L_i, C)
     perm         [T*k] int32 out: entries sorted by (expert, token); the kept
                  entries of expert i are perm[offsets[i] .. offsets[i] + min(L_i, C))
     row_of       [T*k] int32 out, by entry: row kept_offsets[i] + rank of a kept
                  entry, -1 for a dropped one
     drop         [T*k] uint8 out, by entry: 1 if rank >= C */
moe_status_t moe_dispatch(const moe_desc_t *desc, const int32_t *topk_idx, int32_t *counts,
                          int32_t *offsets, int32_t *kept_offsets, int32_t *perm,
                          int32_t *row_of, uint8_t *drop, void *ws, size_t ws_bytes,
                          moe_stream_t stream);

/* Routed experts (section 3.1): for every expert i and each of its kept
   entries j (in perm order), y_perm[kept_offsets[i] + j] = F_i(x[token]).
     x        [T, w] act_dtype, w = d (plain) or l (latent: x = W_ldown u)
     W_gate, W_up [N, h, w]; W_down [N, w, h]  w_dtype
     y_perm   [sum_i min(L_i, C), w] fp32 out (rows beyond the kept total untouched)
   Only experts with at least one kept entry read their weights. */
moe_status_t moe_expert_ffn(const moe_desc_t *desc, const void *x, const int32_t *perm,
                            const int32_t *offsets, const int32_t *kept_offsets,
                            const void *W_gate, const void *W_up, const void *W_down,
                            float *y_perm, void *ws, size_t ws_bytes, moe_stream_t stream);

/* moe_expert_ffn with weight scales (the same computation, with W_gate,
   W_up, W_down expanded as described at moe_weights_t):
     gate_scale, up_scale, down_scale  device pointers in the layout
     moe_weights_t gives for w_dtype, all three required for MOE_FP8_E4M3
     and MOE_MXFP4, all three null otherwise (MOE_ERR_ARG if not). */
moe_status_t moe_expert_ffn_scaled(const moe_desc_t *desc, const void *x, const int32_t *perm,
                                   const int32_t *offsets, const int32_t *kept_offsets,
                                   const void *W_gate, const void *W_up, const void *W_down,
                                   const void *gate_scale, const void *up_scale,
                                   const void *down_scale, float *y_perm, void *ws,
                                   size_t ws_bytes, moe_stream_t stream);

/* Combine (section 3.2 eq. for y): y_t = sum_s [row_of[t*k+s] >= 0]
   topk_w[t,s] * y_perm[row_of[t*k+s]] in fp32, rounded once to act_dtype.
   Dropped slots add 0 and the other weights are not renormalised; a token
   with every slot dropped gets y_t = 0.
   Plain layer: y [T, d].  Latent layer: y [T, l] receives RMSNorm(r) (the
   input of W_lup), r the weighted sum above. */
moe_status_t moe_combine(const moe_desc_t *desc, const float *y_perm, const int32_t *row_of,
                         const float *topk_w, void *y, moe_stream_t stream);

/* Whole layer: route -> dispatch -> experts -> combine (and, for the latent
   layer, the d->l projection, shared experts, RMSNorm and l->d projection).
     u [T, d] act_dtype in; y [T, d] act_dtype out; out nullable. */
moe_status_t moe_forward(const moe_desc_t *desc, const moe_weights_t *w, const void *u,
                         void *y, const moe_outputs_t *out, void *ws, size_t ws_bytes,
                         moe_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc): moe_forward
   with the library's own scratch in place of the caller's workspace.  The
   scratch is one static device array of MOE_STATIC_SCRATCH_BYTES per GPU,
   created with the library's code object on that GPU and held until the
   process ends; the call allocates and frees nothing.  Layers whose
   moe_workspace_bytes() exceeds MOE_STATIC_SCRATCH_BYTES (64 MiB: every
   decode-sized layer of T <= 64 tokens at d = 4096, h = 14336; larger layers
   such as a 16384-token prefill) return MOE_ERR_WORKSPACE without launching.
   Every call on one GPU uses that GPU's single array: calls that may overlap
   on one GPU (different streams, or several host threads) race and must be
   serialised by the caller; calls on different GPUs do not share it.  The
   GPU is the one that runs `stream` (the current device for the null
   stream).  Other arguments, outputs and errors as moe_forward. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
moe_status_t moe_forward_noalloc(const moe_desc_t *desc, const moe_weights_t *w, const void *u,
                                 void *y, const moe_outputs_t *out, moe_stream_t stream);

/* moe_forward that also records events[0..n_events) on the stream: events[0]
   before the first kernel and events[i] after stage i, with the stages in
   the order moe_stage_name(i) lists them (i = 1..).  Extra events are
   recorded at the end; n_events may be smaller than the stage count.  The
   events are hipEvent_t handles created by the caller. */
moe_status_t moe_forward_traced(const moe_desc_t *desc, const moe_weights_t *w, const void *u,
                                void *y, const moe_outputs_t *out, void *ws, size_t ws_bytes,
                                moe_stream_t stream, void *const *events, int32_t n_events);

/* Name of stage i (1-based) of moe_forward for this layer, or null past the
   last stage; *n_stages (nullable) receives the stage count. */
const char *moe_stage_name(const moe_desc_t *desc, int32_t i, int32_t *n_stages);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
