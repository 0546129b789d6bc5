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
constexpr int kMinSplitSteps = 12;    // tiled down pass: fewest 64-wide steps per part
constexpr int kMinStreamChunks = 16;  // streaming down pass: fewest 64-wide chunks per part

// Most parts the down pass can cut a reduction of length ffn into, on either
// path (the device picks the count from the real tile count, never more):
// the workspace holds that many partial sums of y.
inline int down_split_bound(int ffn) {
  const int tiled = ((ffn + 63) / 64) / kMinSplitSteps;
  const int stream = (ffn / 64) / kMinStreamChunks;
  const int s = tiled > stream ? tiled : stream;
  return s < 1 ? 1 : (s > kMaxDownSplit ? kMaxDownSplit : s);
}
constexpr int kPermMaxBlocks = 256;            // most workgroups of the permutation
constexpr long long kPermBlockedFrom = 4096;   // up to this many assignments: one workgroup
constexpr long long kMaxAssignments = (1ll << 31) - (1ll << 20);  // T*k must stay below

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

// Four consecutive values of h, rounded to bf16 (nearest even) into hi[i..];
// with lo non-null, also the remainder h - hi (exact in fp32) rounded to
// bf16 into lo[i..], so that hi + lo holds h to about 2^-17 of its value.
__device__ __forceinline__ void store_h(bf16_t* __restrict__ hi, bf16_t* __restrict__ lo, size_t i,
                                        const float v[4]) {
  const uint32_t p0 = pack_bf16x2(v[0], v[1]), p1 = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(hi + i) = make_uint2(p0, p1);
  if (lo) {
    const float r0 = v[0] - __uint_as_float(p0 << 16), r1 = v[1] - __uint_as_float(p0 & 0xFFFF0000u);
    const float r2 = v[2] - __uint_as_float(p1 << 16), r3 = v[3] - __uint_as_float(p1 & 0xFFFF0000u);
    *reinterpret_cast<uint2*>(lo + i) = make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
  }
}

// Expert outputs y of a bf16 layer, between the down GEMM and the combine:
// each fp32 value rounded to its top 24 bits (sign, exponent and 15 mantissa
// bits, nearest with ties to even), four values in three 32-bit words. The
// relative error is at most 2^-16 (rounding h to bf16 allows 2^-8), and y's
// stores and the combine's reads move a quarter fewer bytes. fp32 layers
// keep fp32 y. Inputs are finite.
__host__ __device__ __forceinline__ uint32_t f32_to_f24(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u + 0x7Fu + ((u >> 8) & 1u)) >> 8;
}
__host__ __device__ __forceinline__ uint3 pack_f24x4(float a, float b, float c, float d) {
  const uint32_t x = f32_to_f24(a), y = f32_to_f24(b), z = f32_to_f24(c), w = f32_to_f24(d);
  return make_uint3(x | (y << 24), (y >> 8) | (z << 16), (z >> 16) | (w << 8));
}
__host__ __device__ __forceinline__ void unpack_f24x4(uint32_t w0, uint32_t w1, uint32_t w2,
                                                     float v[4]) {
  v[0] = __builtin_bit_cast(float, w0 << 8);
  v[1] = __builtin_bit_cast(float, ((w0 >> 24) | (w1 << 8)) << 8);
  v[2] = __builtin_bit_cast(float, ((w1 >> 16) | (w2 << 16)) << 8);
  v[3] = __builtin_bit_cast(float, w2 & 0xFFFFFF00u);
}
// bytes per element of y for a layer of storage dtype dt
inline size_t y_bytes(moe_dtype dt) { return dt == MOE_BF16 ? 3 : 4; }

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

// Whether a bf16 layer carries h into the down pass as two bf16 terms (the
// rounding of h and the rounding of the remainder): the down pass then does
// twice the MFMA work, and rounding h to bf16 no longer moves the output.
// Alone, that rounding moves each output by about 1.6e-3 of its size
// (relative error of bf16 rounding, RMS), and the largest of many outputs by
// several times that; with few terms per output (short expert width) or a
// narrow layer the per-token sizes spread more and the largest error reaches
// 2e-2 x RMS. Below 1024 in either width the two terms are used.
constexpr int kTwoTermBelow = 1024;
inline bool two_term_h(int d, int ffn, moe_dtype dt) {
  return dt == MOE_BF16 && (d < kTwoTermBelow || ffn < kTwoTermBelow);
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
  void* h_lo;             // [T*k, ffn] bf16: second term of h (two_term_h), else null
  void* y;                // [down_split_bound(ffn), T*k, d] partial sums of the down GEMM (y_bytes(dt) each)
  int32_t* split;         // [1] number of partial sums in y; 0: per (row, column tile) in y_parts
  uint8_t* y_parts;       // [T*k, ceil(d/256)] partial sums of each row's 256-column tile (split = 0)
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
  w.h_lo = two_term_h(d, ffn, dt) ? take(tk * static_cast<size_t>(ffn) * es) : nullptr;
  w.y = take(down_split_bound(ffn) * tk * static_cast<size_t>(d) * y_bytes(dt));
  w.split = reinterpret_cast<int32_t*>(take(4));
  w.y_parts = reinterpret_cast<uint8_t*>(take(tk * static_cast<size_t>((d + 255) / 256)));
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
  void* h_s_lo;           // second term of h_s (two_term_h for shared_ffn), else null
  void* y_s;              // [down_split_bound(shared_ffn), n_shared*T, d] (y_bytes(dt) each)
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
    w.h_s_lo = two_term_h(d, shared_ffn, dt) ? take(ts * static_cast<size_t>(shared_ffn) * es)
                                             : nullptr;
    w.y_s = take(down_split_bound(shared_ffn) * ts * static_cast<size_t>(d) * y_bytes(dt));
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
// Few rows per expert: the weight-streaming kernels replace the tiled ones.
inline bool use_stream_path(int rows, int E) { return rows <= 32 * E; }

// A decode-sized batch's permutation, derived inside the gate/up stream
// kernel instead of by launch_permute: every workgroup ranks its own
// expert's assignments in topk_idx (in assignment order, as launch_permute
// does without a capacity), and the first workgroup of each expert writes
// counts, offsets, sorted_token and inv_pos for the kernels after it. This
// saves a launch and one dependent kernel boundary per layer call.
constexpr int kSelfPermuteMax = 256;  // assignments: one per thread of a workgroup
struct StreamPermute {
  const int32_t* topk_idx;  // [n] expert ids in [0, E)
  int n, k;
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E + 1]
  int32_t* sorted_token;  // [n]
  int32_t* inv_pos;       // [n]
};
inline bool stream_self_permute(int rows, int E, moe_dtype dt) {
  return dt == MOE_BF16 && rows <= kSelfPermuteMax && use_stream_path(rows, E);
}

// h_lo: null, or (bf16 only) the second bf16 term of h, the rounding of
// h - h_hi (see store_h); the down pass then multiplies both terms.
// sp: null, or (when stream_self_permute holds) the routing from which the
// stream kernel derives sorted_token and offsets, which it then writes.
// y_parts: null, or a part table [T*k, ceil(d/256)] that a 384-row down
// pass with a long reduction fills (one byte per row and 256-column tile:
// its count of partial sums), writing 0 to *split; every other down pass
// writes its uniform count of partial sums to *split.
moe_status launch_gate_up(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                          const void* w_gate, const void* w_up, int T, int d, int ffn, int E,
                          int k, moe_dtype dt, void* h, void* h_lo, hipStream_t s,
                          const StreamPermute* sp = nullptr);
moe_status launch_down(const void* h, const void* h_lo, const int32_t* offsets, const void* w_down,
                       int T, int d, int ffn, int E, int k, moe_dtype dt, void* y, int32_t* split,
                       hipStream_t s, uint8_t* y_parts = nullptr);
// Weight-streaming kernels; experts with more than max_rows rows are skipped
// (left to a tiled launch). The down pass cuts its reduction into at most
// max_split parts.
moe_status launch_gate_up_stream(const void* x, const int32_t* sorted_token,
                                 const int32_t* offsets, const void* w_gate, const void* w_up,
                                 int d, int ffn, int E, int rows, void* h, bf16_t* h_lo,
                                 int max_rows, const StreamPermute* sp, hipStream_t s);
moe_status launch_down_stream(const void* h, const bf16_t* h_lo, const int32_t* offsets,
                              const void* w_down, int d, int ffn, int E, int rows, void* y,
                              int32_t* split, int max_rows, int max_split, hipStream_t s);
// Router statistics (router_stats.hip): partial sums over router_stats_blocks(T)
// blocks of `partial` floats per expert.
int router_stats_blocks(int T);
moe_status launch_router_stats(const float* probs, const int32_t* counts, int T, int E,
                               float* mean_probs, float* frac, float* loss, float* partial,
                               hipStream_t s);
// y (and ys) in the format of a layer of dtype dt: 24-bit for bf16, fp32.
moe_status launch_combine(const void* y, const int32_t* split, const int32_t* inv_pos,
                          const float* topk_w, int T, int d, int k, moe_dtype dt, void* out,
                          moe_dtype out_dt, hipStream_t s, const uint8_t* y_parts = nullptr);
// ys: outputs of n_shared shared experts (their own split count ys_split);
// resid: [T, d] in resid_dt added last; both optional.
moe_status launch_combine_ext(const void* y, const int32_t* split, const int32_t* inv_pos,
                              const float* topk_w, int T, int d, int k, moe_dtype dt, const void* ys,
                              const int32_t* ys_split, int n_shared, const void* resid,
                              moe_dtype resid_dt, void* out, moe_dtype out_dt, hipStream_t s,
                              const uint8_t* y_parts = nullptr);

}  // namespace moe
