// C ABI of the MoE layer: argument checks, workspace carving, kernel launches.
// Every entry point validates on the host first and enqueues nothing when an
// argument is rejected. No entry point allocates or frees device memory.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "common.h"

using namespace moe;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }

// k in 1..E follows axonml-nn MoERouter::new and KempnerForge's ModelConfig
// MoE validation; the remaining limits are this library's.
moe_status check_routing(int T, int E, int k) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_INVALID_ARG;
  if (E > kMaxExperts || k > kMaxTopK) return MOE_UNSUPPORTED;
  // the permutation's per-block assignment ranges are int32: with 256 blocks
  // they reach T*k + 2^18, so 2^20 of headroom keeps them below 2^31
  if (static_cast<long long>(T) * k >= kMaxAssignments) return MOE_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_layer(int T, int d, int ffn, int E, int k, moe_dtype dt) {
  if (d < 1 || ffn < 1) return MOE_INVALID_ARG;
  moe_status st = check_routing(T, E, k);
  if (st != MOE_OK) return st;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_UNSUPPORTED;
  if (d % 16 != 0 || ffn % 16 != 0) return MOE_UNSUPPORTED;
  // the tiled kernels address x, h and one expert's weights with 32-bit
  // byte offsets
  const long long es = dt == MOE_BF16 ? 2 : 4;
  const long long lim = 1ll << 32;
  if (static_cast<long long>(T) * d * es >= lim || static_cast<long long>(T) * k * ffn * es >= lim ||
      static_cast<long long>(ffn) * d * es >= lim)
    return MOE_UNSUPPORTED;
  return MOE_OK;
}

bool ok_dtype(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16; }

// Options of the extended forward; T and d bound the shared experts' sizes.
moe_status check_options(const moe_options* o, int T, int d, moe_dtype dt) {
  if (!o) return MOE_INVALID_ARG;
  if (!(o->capacity_factor >= 0.f) || !std::isfinite(o->capacity_factor)) return MOE_INVALID_ARG;
  if (o->norm_weight && (!aligned16(o->norm_weight) || !(o->norm_eps > 0.f) ||
                         !std::isfinite(o->norm_eps)))
    return MOE_INVALID_ARG;
  if (o->n_shared < 0) return MOE_INVALID_ARG;
  if (o->n_shared > 0) {
    if (o->shared_ffn < 1 || !ok_ptr(o->shared_gate) || !ok_ptr(o->shared_up) ||
        !ok_ptr(o->shared_down))
      return MOE_INVALID_ARG;
    if (o->n_shared > kMaxShared || o->shared_ffn % 16 != 0) return MOE_UNSUPPORTED;
    if (static_cast<long long>(T) * o->n_shared >= (1ll << 31)) return MOE_UNSUPPORTED;
    const long long es = dt == MOE_BF16 ? 2 : 4;
    // h_s rows and one shared expert's weights use 32-bit byte offsets in
    // the tiled GEMMs, as the routed experts' do
    if (static_cast<long long>(T) * o->n_shared * o->shared_ffn * es >= (1ll << 32) ||
        static_cast<long long>(o->shared_ffn) * d * es >= (1ll << 32))
      return MOE_UNSUPPORTED;
  }
  return MOE_OK;
}

// Rows an expert may keep: ceil(cf * T * k / E), or T (no limit) for cf = 0.
int capacity_rows(float cf, int T, int E, int k) {
  if (cf == 0.f) return T;
  const double c = std::ceil(static_cast<double>(cf) * T * k / E);
  return c >= T ? T : static_cast<int>(c);
}

}  // namespace

// Scratch of moe_forward_no_alloc: one array per GPU, in the code object's
// device memory, so that entry point never allocates. In host code the name
// `scratch` is only a stand-in for the device array; its device address (one
// per GPU) is looked up once per device and only that address is used.
static __device__ __align__(256) char scratch[MOE_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with the device current) and kept until the process ends.
moe_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_HIP_ERROR;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_HIP_ERROR;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_INVALID_ARG: return "MOE_INVALID_ARG";
    case MOE_UNSUPPORTED: return "MOE_UNSUPPORTED";
    case MOE_WORKSPACE_TOO_SMALL: return "MOE_WORKSPACE_TOO_SMALL";
    case MOE_HIP_ERROR: return "MOE_HIP_ERROR";
  }
  return "MOE_UNKNOWN_STATUS";
}

size_t moe_workspace_size(int T, int d, int ffn, int E, int k, moe_dtype dt) {
  if (check_layer(T, d, ffn, E, k, dt) != MOE_OK) return 0;
  return carve_workspace(nullptr, T, d, ffn, E, k, dt).bytes;
}

moe_status moe_route_logits(const float* logits, int T, int E, int k, float* probs,
                            int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  moe_status st = check_routing(T, E, k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(topk_idx) || !ok_ptr(topk_w) || !ok_opt(probs))
    return MOE_INVALID_ARG;
  return launch_route_logits(logits, T, E, k, probs, topk_idx, topk_w, stream);
}

moe_status moe_route(const void* x, const void* w_router, const float* router_bias, int T, int d,
                     int E, int k, moe_dtype dt, float* logits, float* probs, int32_t* topk_idx,
                     float* topk_w, hipStream_t stream) {
  if (d < 1) return MOE_INVALID_ARG;
  moe_status st = check_routing(T, E, k);
  if (st != MOE_OK) return st;
  if (!ok_dtype(dt) || d % 16 != 0) return MOE_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(w_router) || !ok_ptr(topk_idx) || !ok_ptr(topk_w) ||
      !ok_opt(router_bias) || !ok_opt(logits) || !ok_opt(probs))
    return MOE_INVALID_ARG;
  return launch_route(x, w_router, router_bias, T, d, E, k, dt, logits, probs, topk_idx, topk_w,
                      stream);
}

size_t moe_permute_workspace_size(int T, int E, int k) {
  if (check_routing(T, E, k) != MOE_OK) return 0;
  return static_cast<size_t>(permute_blocks(T, k)) * E * sizeof(int32_t);
}

moe_status moe_permute(const int32_t* topk_idx, const float* topk_w, int T, int E, int k,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* inv_pos,
                       float* sorted_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_routing(T, E, k);
  if (st != MOE_OK) return st;
  if ((topk_w == nullptr) != (sorted_w == nullptr)) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(topk_idx) || !ok_ptr(counts) || !ok_ptr(offsets) || !ok_ptr(sorted_token) ||
      !ok_ptr(inv_pos) || !ok_opt(topk_w) || !ok_opt(sorted_w))
    return MOE_INVALID_ARG;
  const size_t need = moe_permute_workspace_size(T, E, k);
  if (need > 0 && !ok_ptr(ws)) return MOE_INVALID_ARG;
  if (ws_bytes < need) return MOE_WORKSPACE_TOO_SMALL;
  st = launch_permute(topk_idx, T, E, k, T, counts, nullptr, offsets, sorted_token, inv_pos,
                      static_cast<int32_t*>(ws), stream);
  if (st != MOE_OK || !sorted_w) return st;
  return launch_permute_weights(inv_pos, topk_w, T * k, sorted_w, stream);
}

size_t moe_router_stats_workspace_size(int T, int E) {
  if (T < 0 || E < 1 || E > kMaxExperts) return 0;
  return static_cast<size_t>(router_stats_blocks(T)) * E * sizeof(float);
}

moe_status moe_router_stats(const float* probs, const int32_t* counts, int T, int E,
                            float* mean_probs, float* frac, float* lb_loss, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || E < 1) return MOE_INVALID_ARG;
  if (E > kMaxExperts) return MOE_UNSUPPORTED;
  if (!ok_ptr(mean_probs) || !ok_ptr(lb_loss) || !ok_opt(frac)) return MOE_INVALID_ARG;
  if (T > 0 && (!ok_ptr(probs) || !ok_ptr(counts) || !ok_ptr(ws))) return MOE_INVALID_ARG;
  if (T > 0 && ws_bytes < moe_router_stats_workspace_size(T, E)) return MOE_WORKSPACE_TOO_SMALL;
  return launch_router_stats(probs, counts, T, E, mean_probs, frac, lb_loss,
                             static_cast<float*>(ws), stream);
}

// ev: NULL, or events [2..5] are recorded after the permutation, the gate/up
// GEMM, the down GEMM and the combine. A decode-sized bf16 batch has no
// separate permutation: the gate/up stream kernel derives it from the
// routing and writes the same outputs (stream_self_permute).
static moe_status run_experts(const void* x, const int32_t* topk_idx, const float* topk_w,
                              const void* w_gate, const void* w_up, const void* w_down, int T,
                              int d, int ffn, int E, int k, moe_dtype dt, void* out,
                              moe_dtype out_dt, const Workspace& ws, int32_t* counts_out,
                              hipStream_t stream, hipEvent_t* ev) {
  int32_t* counts = counts_out ? counts_out : ws.counts;
  const bool self = stream_self_permute(T * k, E, dt);
  moe_status st = MOE_OK;
  if (!self) {
    st = launch_permute(topk_idx, T, E, k, T, counts, nullptr, ws.offsets, ws.sorted_token,
                        ws.inv_pos, ws.block_counts, stream);
    if (st != MOE_OK) return st;
  }
  if (ev) hipEventRecord(ev[2], stream);
  const StreamPermute sp{topk_idx, T * k, k, counts, ws.offsets, ws.sorted_token, ws.inv_pos};
  st = launch_gate_up(x, ws.sorted_token, ws.offsets, w_gate, w_up, T, d, ffn, E, k, dt, ws.h,
                      ws.h_lo, stream, self ? &sp : nullptr);
  if (st != MOE_OK) return st;
  if (ev) hipEventRecord(ev[3], stream);
  st = launch_down(ws.h, ws.h_lo, ws.offsets, w_down, T, d, ffn, E, k, dt, ws.y, ws.split,
                   stream, ws.y_parts);
  if (st != MOE_OK) return st;
  if (ev) hipEventRecord(ev[4], stream);
  st = launch_combine(ws.y, ws.split, ws.inv_pos, topk_w, T, d, k, dt, out, out_dt, stream,
                      ws.y_parts);
  if (ev) hipEventRecord(ev[5], stream);
  return st;
}

moe_status moe_expert_ffn(const void* x, const int32_t* topk_idx, const float* topk_w,
                          const void* w_gate, const void* w_up, const void* w_down, int T, int d,
                          int ffn, int E, int k, moe_dtype dt, void* out, moe_dtype out_dt,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(T, d, ffn, E, k, dt);
  if (st != MOE_OK) return st;
  if (!ok_dtype(out_dt)) return MOE_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(topk_idx) || !ok_ptr(topk_w) || !ok_ptr(w_gate) || !ok_ptr(w_up) ||
      !ok_ptr(w_down) || !ok_ptr(out) || !ok_ptr(ws) || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return MOE_INVALID_ARG;
  const Workspace w = carve_workspace(ws, T, d, ffn, E, k, dt);
  if (ws_bytes < w.bytes) return MOE_WORKSPACE_TOO_SMALL;
  return run_experts(x, topk_idx, topk_w, w_gate, w_up, w_down, T, d, ffn, E, k, dt, out, out_dt,
                     w, nullptr, stream, nullptr);
}

// Argument checks of moe_forward apart from the workspace.
static moe_status check_forward(const void* x, const void* w_router, const void* w_gate,
                                const void* w_up, const void* w_down, const float* router_bias,
                                int T, int d, int ffn, int E, int k, moe_dtype dt, void* out,
                                moe_dtype out_dt, float* logits_out, float* probs_out,
                                int32_t* counts_out) {
  moe_status st = check_layer(T, d, ffn, E, k, dt);
  if (st != MOE_OK) return st;
  if (!ok_dtype(out_dt)) return MOE_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(w_router) || !ok_ptr(w_gate) || !ok_ptr(w_up) || !ok_ptr(w_down) ||
      !ok_ptr(out) || !ok_opt(router_bias) || !ok_opt(logits_out) || !ok_opt(probs_out) ||
      !ok_opt(counts_out))
    return MOE_INVALID_ARG;
  return MOE_OK;
}

static moe_status forward_impl(const void* x, const void* w_router, const void* w_gate,
                               const void* w_up, const void* w_down, const float* router_bias,
                               int T, int d, int ffn, int E, int k, moe_dtype dt, void* out,
                               moe_dtype out_dt, float* logits_out, float* probs_out,
                               int32_t* counts_out, void* ws, size_t ws_bytes, hipStream_t stream,
                               hipEvent_t* ev) {
  moe_status st = check_forward(x, w_router, w_gate, w_up, w_down, router_bias, T, d, ffn, E, k,
                                dt, out, out_dt, logits_out, probs_out, counts_out);
  if (st != MOE_OK || T == 0) return st;
  if (!ok_ptr(ws) || (reinterpret_cast<uintptr_t>(ws) & 255u)) return MOE_INVALID_ARG;
  const Workspace w = carve_workspace(ws, T, d, ffn, E, k, dt);
  if (ws_bytes < w.bytes) return MOE_WORKSPACE_TOO_SMALL;
  if (ev) hipEventRecord(ev[0], stream);
  st = launch_route(x, w_router, router_bias, T, d, E, k, dt, logits_out, probs_out, w.topk_idx,
                    w.topk_w, stream);
  if (st != MOE_OK) return st;
  if (ev) hipEventRecord(ev[1], stream);
  return run_experts(x, w.topk_idx, w.topk_w, w_gate, w_up, w_down, T, d, ffn, E, k, dt, out,
                     out_dt, w, counts_out, stream, ev);
}

moe_status moe_forward(const void* x, const void* w_router, const void* w_gate, const void* w_up,
                       const void* w_down, const float* router_bias, int T, int d, int ffn, int E,
                       int k, moe_dtype dt, void* out, moe_dtype out_dt, float* logits_out,
                       float* probs_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  return forward_impl(x, w_router, w_gate, w_up, w_down, router_bias, T, d, ffn, E, k, dt, out,
                      out_dt, logits_out, probs_out, counts_out, ws, ws_bytes, stream, nullptr);
}

moe_status moe_forward_profiled(const void* x, const void* w_router, const void* w_gate,
                                const void* w_up, const void* w_down, const float* router_bias,
                                int T, int d, int ffn, int E, int k, moe_dtype dt, void* out,
                                moe_dtype out_dt, float* logits_out, float* probs_out,
                                int32_t* counts_out, void* ws, size_t ws_bytes, hipStream_t stream,
                                hipEvent_t* stage_events) {
  if (!stage_events) return MOE_INVALID_ARG;
  for (int i = 0; i < 6; ++i)
    if (!stage_events[i]) return MOE_INVALID_ARG;
  return forward_impl(x, w_router, w_gate, w_up, w_down, router_bias, T, d, ffn, E, k, dt, out,
                      out_dt, logits_out, probs_out, counts_out, ws, ws_bytes, stream,
                      stage_events);
}

size_t moe_forward_ext_workspace_size(int T, int d, int ffn, int E, int k, moe_dtype dt,
                                      const moe_options* opt) {
  if (check_layer(T, d, ffn, E, k, dt) != MOE_OK || check_options(opt, T, d, dt) != MOE_OK) return 0;
  return carve_ext_workspace(nullptr, T, d, ffn, E, k, dt, opt->norm_weight != nullptr,
                             opt->n_shared, opt->shared_ffn)
      .bytes;
}

moe_status moe_forward_ext(const void* x, const void* w_router, const void* w_gate,
                           const void* w_up, const void* w_down, const float* router_bias, int T,
                           int d, int ffn, int E, int k, moe_dtype dt, const moe_options* opt,
                           void* out, moe_dtype out_dt, float* logits_out, float* probs_out,
                           int32_t* counts_out, int32_t* routed_counts_out, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(T, d, ffn, E, k, dt);
  if (st != MOE_OK) return st;
  st = check_options(opt, T, d, dt);
  if (st != MOE_OK) return st;
  if (!ok_dtype(out_dt)) return MOE_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(w_router) || !ok_ptr(w_gate) || !ok_ptr(w_up) || !ok_ptr(w_down) ||
      !ok_ptr(out) || !ok_opt(router_bias) || !ok_opt(logits_out) || !ok_opt(probs_out) ||
      !ok_opt(counts_out) || !ok_opt(routed_counts_out) || !ok_ptr(ws) ||
      (reinterpret_cast<uintptr_t>(ws) & 255u))
    return MOE_INVALID_ARG;
  const bool norm = opt->norm_weight != nullptr;
  const int S = opt->n_shared;
  const ExtWorkspace w = carve_ext_workspace(ws, T, d, ffn, E, k, dt, norm, S, opt->shared_ffn);
  if (ws_bytes < w.bytes) return MOE_WORKSPACE_TOO_SMALL;
  const Workspace& b = w.base;
  const void* xl = x;
  if (norm) {
    st = launch_rms_norm(x, opt->norm_weight, T, d, opt->norm_eps, dt, w.xn, stream);
    if (st != MOE_OK) return st;
    xl = w.xn;
  }
  st = launch_route(xl, w_router, router_bias, T, d, E, k, dt, logits_out, probs_out, b.topk_idx,
                    b.topk_w, stream);
  if (st != MOE_OK) return st;
  st = launch_permute(b.topk_idx, T, E, k, capacity_rows(opt->capacity_factor, T, E, k),
                      counts_out ? counts_out : b.counts, routed_counts_out, b.offsets,
                      b.sorted_token, b.inv_pos, b.block_counts, stream);
  if (st != MOE_OK) return st;
  st = launch_gate_up(xl, b.sorted_token, b.offsets, w_gate, w_up, T, d, ffn, E, k, dt, b.h,
                      b.h_lo, stream);
  if (st != MOE_OK) return st;
  st = launch_down(b.h, b.h_lo, b.offsets, w_down, T, d, ffn, E, k, dt, b.y, b.split, stream,
                   b.y_parts);
  if (st != MOE_OK) return st;
  if (S > 0) {
    // shared experts: S more experts that every token reaches, T rows each
    st = launch_identity_rows(T, S, w.st_s, w.off_s, stream);
    if (st != MOE_OK) return st;
    st = launch_gate_up(xl, w.st_s, w.off_s, opt->shared_gate, opt->shared_up, T, d,
                        opt->shared_ffn, S, S, dt, w.h_s, w.h_s_lo, stream);
    if (st != MOE_OK) return st;
    st = launch_down(w.h_s, w.h_s_lo, w.off_s, opt->shared_down, T, d, opt->shared_ffn, S, S, dt,
                     w.y_s, w.split_s, stream);
    if (st != MOE_OK) return st;
  }
  return launch_combine_ext(b.y, b.split, b.inv_pos, b.topk_w, T, d, k, dt, w.y_s, w.split_s, S,
                            opt->residual ? x : nullptr, dt, out, out_dt, stream, b.y_parts);
}

moe_status moe_forward_no_alloc(const void* x, const void* w_router, const void* w_gate,
                                const void* w_up, const void* w_down, const float* router_bias,
                                int T, int d, int ffn, int E, int k, moe_dtype dt, void* out,
                                moe_dtype out_dt, float* logits_out, float* probs_out,
                                int32_t* counts_out, hipStream_t stream) {
  moe_status st = check_forward(x, w_router, w_gate, w_up, w_down, router_bias, T, d, ffn, E, k,
                                dt, out, out_dt, logits_out, probs_out, counts_out);
  if (st != MOE_OK || T == 0) return st;
  const size_t need = carve_workspace(nullptr, T, d, ffn, E, k, dt).bytes;
  if (need > static_cast<size_t>(MOE_NO_ALLOC_SCRATCH_BYTES)) return MOE_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  return forward_impl(x, w_router, w_gate, w_up, w_down, router_bias, T, d, ffn, E, k, dt, out,
                      out_dt, logits_out, probs_out, counts_out, ws,
                      MOE_NO_ALLOC_SCRATCH_BYTES, stream, nullptr);
}

}  // extern "C"
