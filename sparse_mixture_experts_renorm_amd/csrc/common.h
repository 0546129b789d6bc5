// Internal helpers shared by the HIP kernels of the MoE library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;         // CDNA wavefront width
constexpr int kMaxExperts = 256;  // library limit on E
constexpr int kMaxTopK = 16;      // library limit on k
constexpr int kMaxDownSplit = 4;  // most parts the down GEMM's reduction is cut into
constexpr int kPermMaxBlocks = 256;            // most workgroups of the permutation
constexpr long long kPermBlockedFrom = 4096;   // up to this many assignments: one workgroup

typedef uint16_t bf16_t;          // bfloat16 storage (bit pattern)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Two fp32 values as packed bf16 (lo in the low half), rounded to nearest
// even by one v_cvt_pk_bf16_f32; the same rounding as f32_to_bf16.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// SiLU(z) = z * sigmoid(z), in fp32.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// SiLU for the bf16 paths, whose result is rounded to bf16 right after:
// z / (1 + 2^(-z log2 e)) with the exponential and the reciprocal on the
// transcendental unit (v_exp_f32, v_rcp_f32, about 1 ulp each), six
// instructions instead of about twenty-five for the IEEE-exact expf and
// division. The few fp32 ulps it loses are far below the bf16 rounding of
// the result. Large |z| behave: z -> +inf gives 2^-big = 0, so z; z -> -inf
// gives 1/inf = 0, so -0.
__device__ __forceinline__ float silu_fast(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.44269504088896341f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Host-side launch helpers return this when a launch failed.
inline moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}

// Layout of the caller's workspace (all regions 256-byte aligned).
struct Workspace {
  int32_t* topk_idx;      // [T*k]
  float* topk_w;          // [T*k]
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E+1]
  int32_t* sorted_token;  // [T*k]
  int32_t* inv_pos;       // [T*k]
  void* h;                // [T*k, ffn] in dt
  float* y;               // [kMaxDownSplit, T*k, d] fp32 partial sums of the down GEMM
  int32_t* split;         // [1] number of partial sums in y
  int32_t* block_counts;  // [kPermMaxBlocks * E] per-block expert histograms of the permutation
  size_t bytes;
};

inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

inline Workspace carve_workspace(void* base, int T, int d, int ffn, int E, int k, moe_dtype dt) {
  const size_t tk = static_cast<size_t>(T) * k;
  const size_t es = dt == MOE_BF16 ? 2 : 4;
  Workspace w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) { char* r = p ? p + off : nullptr; off += align256(n); return r; };
  w.topk_idx = reinterpret_cast<int32_t*>(take(tk * 4));
  w.topk_w = reinterpret_cast<float*>(take(tk * 4));
  w.counts = reinterpret_cast<int32_t*>(take(static_cast<size_t>(E) * 4));
  w.offsets = reinterpret_cast<int32_t*>(take(static_cast<size_t>(E + 1) * 4));
  w.sorted_token = reinterpret_cast<int32_t*>(take(tk * 4));
  w.inv_pos = reinterpret_cast<int32_t*>(take(tk * 4));
  w.h = take(tk * static_cast<size_t>(ffn) * es);
  w.y = reinterpret_cast<float*>(take(kMaxDownSplit * tk * static_cast<size_t>(d) * 4));
  w.split = reinterpret_cast<int32_t*>(take(4));
  w.block_counts = reinterpret_cast<int32_t*>(take(static_cast<size_t>(kPermMaxBlocks) * E * 4));
  w.bytes = off;
  return w;
}

// Extra regions of the extended forward's workspace, after the base layout.
struct ExtWorkspace {
  Workspace base;
  void* xn;               // [T, d] in dt: the normalised input (RMSNorm on)
  int32_t* st_s;          // [n_shared*T] shared experts' rows (identity)
  int32_t* off_s;         // [n_shared+1]
  void* h_s;              // [n_shared*T, shared_ffn] in dt
  float* y_s;             // [kMaxDownSplit, n_shared*T, d] fp32
  int32_t* split_s;       // [1]
  size_t bytes;
};

inline ExtWorkspace carve_ext_workspace(void* base, int T, int d, int ffn, int E, int k,
                                        moe_dtype dt, bool norm, int n_shared, int shared_ffn) {
  ExtWorkspace w{};
  w.base = carve_workspace(base, T, d, ffn, E, k, dt);
  const size_t es = dt == MOE_BF16 ? 2 : 4;
  const size_t ts = static_cast<size_t>(T) * n_shared;
  char* p = static_cast<char*>(base);
  size_t off = w.base.bytes;
  auto take = [&](size_t n) { char* r = p ? p + off : nullptr; off += align256(n); return r; };
  if (norm) w.xn = take(static_cast<size_t>(T) * d * es);
  if (n_shared > 0) {
    w.st_s = reinterpret_cast<int32_t*>(take(ts * 4));
    w.off_s = reinterpret_cast<int32_t*>(take(static_cast<size_t>(n_shared + 1) * 4));
    w.h_s = take(ts * static_cast<size_t>(shared_ffn) * es);
    w.y_s = reinterpret_cast<float*>(take(kMaxDownSplit * ts * static_cast<size_t>(d) * 4));
    w.split_s = reinterpret_cast<int32_t*>(take(4));
  }
  w.bytes = off;
  return w;
}

constexpr int kMaxShared = 16;  // library limit on shared experts

// ---- launchers (defined in the kernel files) ----
moe_status launch_route(const void* x, const void* w_router, const float* bias, int T, int d,
                        int E, int k, moe_dtype dt, float* logits, float* probs,
                        int32_t* topk_idx, float* topk_w, hipStream_t s);
moe_status launch_route_logits(const float* logits, int T, int E, int k, float* probs,
                               int32_t* topk_idx, float* topk_w, hipStream_t s);
// cap: most rows an expert keeps (>= T: no limit); routed_counts may be null.
// block_counts: [permute_blocks(T, k) * E] scratch, unused (may be null)
// when permute_blocks(T, k) == 0 (one workgroup does everything).
int permute_blocks(int T, int k);
moe_status launch_permute(const int32_t* topk_idx, int T, int E, int k, int cap, int32_t* counts,
                          int32_t* routed_counts, int32_t* offsets, int32_t* sorted_token,
                          int32_t* inv_pos, int32_t* block_counts, hipStream_t s);
moe_status launch_permute_weights(const int32_t* inv_pos, const float* topk_w, int n,
                                  float* sorted_w, hipStream_t s);
// S shared experts over all T tokens: rows s*T + t hold token t.
moe_status launch_identity_rows(int T, int S, int32_t* sorted_token, int32_t* offsets,
                                hipStream_t s);
moe_status launch_rms_norm(const void* x, const void* g, int T, int d, float eps, moe_dtype dt,
                           void* xn, hipStream_t s);
moe_status launch_gate_up(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                          const void* w_gate, const void* w_up, int T, int d, int ffn, int E,
                          int k, moe_dtype dt, void* h, hipStream_t s);
moe_status launch_down(const void* h, const int32_t* offsets, const void* w_down, int T, int d,
                       int ffn, int E, int k, moe_dtype dt, float* y, int32_t* split,
                       hipStream_t s);
moe_status launch_gate_up_stream(const void* x, const int32_t* sorted_token,
                                 const int32_t* offsets, const void* w_gate, const void* w_up,
                                 int d, int ffn, int E, int rows, void* h, hipStream_t s);
moe_status launch_down_stream(const void* h, const int32_t* offsets, const void* w_down, int d,
                              int ffn, int E, int rows, float* y, int32_t* split, hipStream_t s);
// Few rows per expert: the weight-streaming kernels replace the tiled ones.
inline bool use_stream_path(int rows, int E) { return rows <= 32 * E; }
// Router statistics (router_stats.hip): partial sums over router_stats_blocks(T)
// blocks of `partial` floats per expert.
int router_stats_blocks(int T);
moe_status launch_router_stats(const float* probs, const int32_t* counts, int T, int E,
                               float* mean_probs, float* frac, float* loss, float* partial,
                               hipStream_t s);
moe_status launch_combine(const float* y, const int32_t* split, const int32_t* inv_pos,
                          const float* topk_w, int T, int d, int k, void* out, moe_dtype out_dt,
                          hipStream_t s);
// ys: outputs of n_shared shared experts (their own split count ys_split);
// resid: [T, d] in resid_dt added last; both optional.
moe_status launch_combine_ext(const float* y, const int32_t* split, const int32_t* inv_pos,
                              const float* topk_w, int T, int d, int k, const float* ys,
                              const int32_t* ys_split, int n_shared, const void* resid,
                              moe_dtype resid_dt, void* out, moe_dtype out_dt, hipStream_t s);

}  // namespace moe
