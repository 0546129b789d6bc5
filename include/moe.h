/*
 * moe.h -- C ABI of the MI355X (gfx950) top-k routed Mixture-of-Experts layer.
 *
 * The layer (forward pass only), per token t of x[T, d]:
 *   L[t,:]  = W_r x[t] (+ b)                     router Linear, no bias in the pages
 *   p[t,:]  = softmax(L[t,:])
 *   S_t     = the k experts with the largest logits, largest first,
 *             the lower expert index first among equal logits
 *   w[t,j]  = p[t,S_j] / sum_i p[t,S_i]          renormalised top-k weights
 *   out[t]  = sum_j w[t,j] * down_e( SiLU(gate_e x[t]) * up_e x[t] ),  e = S_j
 * Sources: axonml-nn layers/moe.rs (docs.rs) -- Expert::forward,
 * MoERouter::route, MoELayer::forward; "Mixtral MoE Block" (neurarch.com) --
 * exported PyTorch _moe_forward and the Mixtral layer shapes.
 *
 * Conventions shared by every entry point
 *   - Tensors are DEVICE pointers to row-major, contiguous arrays, each
 *     aligned to 16 bytes. Weights use the nn.Linear [out, in] layout:
 *       w_router [E, d], w_gate [E, ffn, d], w_up [E, ffn, d], w_down [E, d, ffn].
 *   - dt is the storage dtype of x and of every weight (MOE_F32 or MOE_BF16);
 *     logits, probabilities, gate weights and the router bias are always fp32,
 *     expert indices int32. Arithmetic: fp32 accumulation everywhere.
 *   - The caller owns every buffer. The library never allocates or frees
 *     memory on these calls and keeps no state between them; any scratch it
 *     needs comes from the caller's workspace (see moe_workspace_size).
 *   - Each call checks its arguments on the host, enqueues its kernels on
 *     `stream` (NULL = the default stream) and returns without waiting.
 *     Outputs are valid once the caller has synchronised the stream.
 *   - On an argument error (INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL)
 *     nothing is enqueued and no output is written. MOE_HIP_ERROR means a
 *     kernel launch failed; kernels enqueued before it may still run.
 *   - T = 0 is valid: the call returns MOE_OK and launches nothing.
 *   - Non-finite inputs are outside the contract (the page's sort cannot
 *     order NaN); they are not detected on the device.
 *   - Limits (MOE_UNSUPPORTED beyond them): E <= 256, k <= 16,
 *     d % 16 == 0, ffn % 16 == 0, T * k < 2^31 - 2^20 (the permutation's
 *     per-block ranges of assignments are 32-bit), and in bytes of the
 *     storage dtype T*d, T*k*ffn and ffn*d below 2^32 (the GEMM kernels
 *     address x, the hidden activations and one expert's weights with 32-bit
 *     offsets).
 *   - Results are deterministic: no floating-point atomics are used, so two
 *     calls on the same inputs give bit-identical outputs.
 *   - Precision, MOE_BF16: bf16 operands on the bf16 MFMA with fp32
 *     accumulation, SiLU in fp32, each expert output kept to 16 significant
 *     bits (relative error at most 2^-16) until the combine, which sums in
 *     fp32.
 *     The hidden activation h = SiLU(gate) * up is the down projection's
 *     MFMA operand, so it is carried in bf16: when d >= 1024 and
 *     ffn >= 1024 as one term (its rounding to nearest even), otherwise as
 *     two bf16 terms (that rounding plus the rounding of the remainder, h to
 *     about 2^-17 of its value; the down pass then does twice the MFMA work).
 *     One term moves each output by about 1.6e-3 of its size (RMS of the bf16
 *     relative rounding error); measured against the exact layer on seeded
 *     N(0,1) inputs and N(0, 0.02^2) weights, the largest error of any output
 *     element was 1.0e-2 x output RMS at the Mixtral shape, 1.4e-2 at d=2048,
 *     ffn=1408, and at most 1.6e-2 over random shapes with both widths in
 *     1024..2048; with two terms, at most 1.5e-4 x RMS over random narrow
 *     shapes (the 16-bit expert outputs dominate there). Narrower layers
 *     with one term reached 4e-2 x RMS, which is why they take two.
 *   - Precision, MOE_F32: fp32 throughout (within 1e-4 x RMS of the exact
 *     layer): the expert GEMMs run on the fp32 MFMA (fp32 products and
 *     accumulation) in 128 x 128 tiles, SiLU with IEEE expf and division.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_INVALID_ARG = 1,          /* k<1, k>E, E<1, T<0, d<1, ffn<1, null or misaligned pointer */
  MOE_UNSUPPORTED = 2,          /* beyond the limits above, or an unknown dtype */
  MOE_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes below moe_workspace_size(...) */
  MOE_HIP_ERROR = 4             /* a kernel launch failed (hipGetLastError) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Static, human-readable name of a status code. Never NULL. */
const char* moe_status_string(moe_status s);

/* Bytes of device workspace that moe_forward and moe_expert_ffn need for this
 * shape: routing results, per-expert offsets, the permutation, the hidden
 * activations h [T*k, ffn] (in dt; twice that for a bf16 layer narrower than
 * 1024 in d or ffn, whose h takes two bf16 terms) and expert outputs
 * y [T*k, d] (as many partial sums as the down pass may cut its reduction
 * into: one per 12 steps of 64 along ffn, between one and four; 3 bytes per
 * element for bf16 layers, 4 for fp32). Returns 0 for invalid or unsupported shapes. Host-only; no
 * device access. */
size_t moe_workspace_size(int T, int d, int ffn, int E, int k, moe_dtype dt);

/* Router projection + softmax + top-k + renormalisation (one kernel).
 * Computes logits L = x W_r^T (+ router_bias) in fp32, then the same routing
 * as moe_route_logits on those logits.
 *   x [T, d] (dt), w_router [E, d] (dt), router_bias [E] fp32 or NULL
 *   (the pages' router has no bias; it exists for skewed-load workloads).
 *   logits [T, E] fp32 or NULL; probs [T, E] fp32 or NULL;
 *   topk_idx [T, k] int32, topk_w [T, k] fp32 (both required).
 * Source: axonml-nn MoERouter::route; Mixtral _moe_forward (router, softmax,
 * topk, division by the top-k sum). */
moe_status moe_route(const void* x, const void* w_router, const float* router_bias,
                     int T, int d, int E, int k, moe_dtype dt,
                     float* logits, float* probs, int32_t* topk_idx, float* topk_w,
                     hipStream_t stream);

/* Routing from given fp32 logits [T, E]: softmax, top-k selection on the
 * logits (descending; lowest index first among equal values, +0.0 == -0.0),
 * and w[t,j] = p[S_j] / sum_i p[S_i]. Selection is a comparison of the fp32
 * logits only, so it is bit-exact against any implementation fed the same
 * logits. probs [T, E] may be NULL. topk_idx [T, k] int32 and topk_w [T, k]
 * fp32 are required; slot 0 holds the largest logit.
 * Source: axonml-nn MoERouter::route (stable descending sort, take k,
 * renormalise). */
moe_status moe_route_logits(const float* logits, int T, int E, int k,
                            float* probs, int32_t* topk_idx, float* topk_w,
                            hipStream_t stream);

/* Expert histogram, exclusive prefix sum and stable permutation.
 *   topk_idx [T, k] int32 with values in [0, E) (not checked on the device;
 *   out-of-range indices are outside the contract).
 *   counts [E]: assignments per expert; offsets [E+1]: offsets[0] = 0,
 *   offsets[e+1] = offsets[e] + counts[e]; sorted_token [T*k]: the token of
 *   each permuted row, experts in ascending order and, within an expert,
 *   tokens in ascending order; inv_pos [T*k]: the row of assignment t*k+j.
 *   topk_w [T, k] fp32 and sorted_w [T*k] fp32: both NULL, or both given,
 *   then sorted_w[inv_pos[i]] = topk_w[i] (the gate weights in permuted
 *   order, copied bit for bit); one without the other is INVALID_ARG.
 * All integer; bit-exact. Source: axonml-nn MoELayer::forward (utilisation
 * counts; per-expert token lists gathered in token order).
 * ws: caller scratch of moe_permute_workspace_size(T, E, k) bytes (per-block
 * expert histograms when T*k is large; the size is 0, and ws may be NULL,
 * when one workgroup does the whole job). WORKSPACE_TOO_SMALL below it. */
size_t moe_permute_workspace_size(int T, int E, int k);
moe_status moe_permute(const int32_t* topk_idx, const float* topk_w, int T, int E, int k,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                       int32_t* inv_pos, float* sorted_w, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* The expert half of the layer for a given routing: permute, per-expert
 * SwiGLU h = SiLU(X W_g^T) * (X W_u^T), y = h W_d^T, and the weighted combine
 * out[t] = sum_{j<k} topk_w[t,j] * y[row of (t,j)], summed in slot order in
 * fp32. topk_idx [T, k] int32 holds k distinct experts per token; topk_w
 * [T, k] fp32 is used as given (not renormalised here). out [T, d] in out_dt
 * (MOE_F32 or MOE_BF16). ws: device workspace of at least
 * moe_workspace_size(T, d, ffn, E, k, dt) bytes, 256-byte aligned.
 * Source: axonml-nn Expert::forward and MoELayer::forward (gather, expert,
 * weighted scatter-add); Mixtral _moe_forward. */
moe_status moe_expert_ffn(const void* x, const int32_t* topk_idx, const float* topk_w,
                          const void* w_gate, const void* w_up, const void* w_down,
                          int T, int d, int ffn, int E, int k, moe_dtype dt,
                          void* out, moe_dtype out_dt, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* The whole layer: moe_route, then moe_expert_ffn on its routing.
 * router_bias, logits_out [T, E], probs_out [T, E] and counts_out [E] may be
 * NULL. Everything else as above.
 * Source: axonml-nn MoELayer::forward; Mixtral _moe_forward. */
moe_status moe_forward(const void* x, const void* w_router, const void* w_gate,
                       const void* w_up, const void* w_down, const float* router_bias,
                       int T, int d, int ffn, int E, int k, moe_dtype dt,
                       void* out, moe_dtype out_dt,
                       float* logits_out, float* probs_out, int32_t* counts_out,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward that also records caller-created events on `stream` between
 * its stages, for per-kernel timing: stage_events[0] before the router,
 * [1] after the router, [2] after the permutation, [3] after the gate/up
 * GEMM, [4] after the down GEMM, [5] after the combine (6 events, none NULL;
 * a bf16 batch of at most 256 assignments on the weight-streaming kernels
 * has no separate permutation, its gate/up kernel derives it, so [1] and
 * [2] are recorded back to back). Results are identical to moe_forward's. */
moe_status moe_forward_profiled(const void* x, const void* w_router, const void* w_gate,
                                const void* w_up, const void* w_down, const float* router_bias,
                                int T, int d, int ffn, int E, int k, moe_dtype dt,
                                void* out, moe_dtype out_dt,
                                float* logits_out, float* probs_out, int32_t* counts_out,
                                void* ws, size_t ws_bytes, hipStream_t stream,
                                hipEvent_t* stage_events);

/* ---- The layer without a workspace argument -----------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * computation, outputs and argument rules as moe_forward, but the workspace
 * is a fixed array of MOE_NO_ALLOC_SCRATCH_BYTES in the library's own device
 * memory (one copy per GPU the library runs on, held until the process
 * ends). The call allocates nothing: no hipMalloc, no hipFree, no allocating
 * library routine. The caller still passes inputs and outputs.
 * Limit: shapes whose moe_workspace_size(T, d, ffn, E, k, dt) exceeds
 * MOE_NO_ALLOC_SCRATCH_BYTES return MOE_WORKSPACE_TOO_SMALL and enqueue
 * nothing (at the Mixtral widths d = 4096, ffn = 14336, E = 8, k = 2 that
 * is T above 430 tokens: decode-sized batches fit). The first call on a
 * device looks up that device's copy of the array (MOE_HIP_ERROR if the
 * lookup fails). Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and give undefined
 * results; calls in order on one stream are safe. No state is carried from
 * one call to the next. */
#define MOE_NO_ALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_no_alloc(const void* x, const void* w_router, const void* w_gate,
                                const void* w_up, const void* w_down, const float* router_bias,
                                int T, int d, int ffn, int E, int k, moe_dtype dt,
                                void* out, moe_dtype out_dt,
                                float* logits_out, float* probs_out, int32_t* counts_out,
                                hipStream_t stream);

/* ---- Router statistics --------------------------------------------------
 * Source: axonml-nn layers/moe.rs (docs.rs), MoELayer::load_balancing_loss
 * (Switch Transformer form), and MoELayer::expert_utilization for counts.
 * From the routing probabilities probs [T, E] (fp32, e.g. moe_forward's
 * probs_out) and the per-expert assignment counts [E] (int32, e.g.
 * counts_out):
 *   mean_probs[e] = P_e = (1/T) sum_t probs[t, e]
 *   frac[e]       = f_e = counts[e] / T        (NULL: not written)
 *   *lb_loss      = E * sum_e f_e * P_e
 * f counts all k slots of a token, so sum_e f_e = k and a perfectly even
 * routing gives lb_loss = k (the page's convention). T = 0 writes zeros
 * (the page returns 0 before any tokens), so unlike the other entry points
 * it launches a kernel. Sums run in a fixed order (deterministic).
 * ws: caller scratch of moe_router_stats_workspace_size(T, E) bytes
 * (unused when T = 0). Errors: INVALID_ARG for T < 0, E < 1 or a null or
 * misaligned required pointer; UNSUPPORTED for E > 256;
 * WORKSPACE_TOO_SMALL. */
size_t moe_router_stats_workspace_size(int T, int E);
moe_status moe_router_stats(const float* probs, const int32_t* counts, int T, int E,
                            float* mean_probs, float* frac, float* lb_loss,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- Extended forward: the layer inside a Mixtral-style block ------------
 * Same layer as moe_forward, with options (all off when zeroed):
 *   capacity_factor  KempnerForge ModelConfig.moe_capacity_factor (0 = no
 *                    dropping). With cf > 0 each expert keeps at most
 *                    C = ceil(cf * T * k / E) assignments, the first C in
 *                    token order; a dropped assignment contributes nothing
 *                    and the token's other weights stay as routed.
 *   norm_weight      [d] in dt, or NULL. When set, the layer (router and
 *                    experts) runs on RMSNorm(x) = x / sqrt(mean(x^2) +
 *                    norm_eps) * norm_weight, the post-attention nn.RMSNorm
 *                    of the Mixtral block page; the normalised input is
 *                    stored in dt (bf16: rounded to nearest even). norm_eps
 *                    must be > 0.
 *   residual         nonzero: out = x + layer(...), with the un-normalised x
 *                    (the Mixtral block's moe_residual add), added in fp32.
 *   n_shared, shared_ffn, shared_gate [n_shared, shared_ffn, d],
 *   shared_up [n_shared, shared_ffn, d], shared_down [n_shared, d,
 *                    shared_ffn] (dt): KempnerForge moe_shared_experts,
 *                    SwiGLU experts every token passes through, added with
 *                    weight 1 after the routed experts.
 * Outputs as moe_forward; counts_out are the rows each expert kept and
 * routed_counts_out (nullable) the assignments before the capacity cut (the
 * counts the load-balancing loss uses).
 * Workspace: moe_forward_ext_workspace_size(...) bytes, 256-byte aligned.
 * Errors as moe_forward, plus INVALID_ARG for opt == NULL, a negative or
 * non-finite capacity factor, norm_eps <= 0, n_shared < 0, shared_ffn < 1
 * or a null or misaligned shared weight; UNSUPPORTED for n_shared > 16,
 * shared_ffn % 16 != 0, or shared_ffn * d or T * n_shared * shared_ffn
 * elements of dt reaching 2^32 bytes (32-bit offsets, as for the routed
 * experts). */
typedef struct {
  float capacity_factor;
  const void* norm_weight;
  float norm_eps;
  int residual;
  int n_shared;
  int shared_ffn;
  const void* shared_gate;
  const void* shared_up;
  const void* shared_down;
} moe_options;

size_t moe_forward_ext_workspace_size(int T, int d, int ffn, int E, int k, moe_dtype dt,
                                      const moe_options* opt);
moe_status moe_forward_ext(const void* x, const void* w_router, const void* w_gate,
                           const void* w_up, const void* w_down, const float* router_bias,
                           int T, int d, int ffn, int E, int k, moe_dtype dt,
                           const moe_options* opt,
                           void* out, moe_dtype out_dt,
                           float* logits_out, float* probs_out, int32_t* counts_out,
                           int32_t* routed_counts_out,
                           void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
