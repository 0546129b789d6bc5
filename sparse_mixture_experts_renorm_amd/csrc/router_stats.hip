// Router statistics: per-expert mean routing probability P_e, routed
// fraction f_e, and the load-balancing loss E * sum_e f_e * P_e
// (axonml-nn layers/moe.rs, MoELayer::load_balancing_loss, which follows
// the Switch Transformer form). f_e = counts_e / T counts every one of the
// k slots, so the f_e add up to k, as on that page.
//
// Fixed reduction orders, so results are deterministic and no atomics or
// counters are needed. Up to kFusedElems probabilities, one block of 1024
// threads does everything (one launch: the call is latency-bound there);
// above that, two passes:
//   pass 1: block b sums the probability rows of its token range for every
//           expert into partial[b, :];
//   pass 2: one block adds the partials in block order, divides by T,
//           forms f_e and the loss (a fixed-shape tree over the experts).
// Reading probs [T, E] fp32 is the whole memory traffic: the kernels are
// bound by HBM at large T and by launch latency at small T.
#include "common.h"

namespace moe {
namespace {

constexpr int kStatThreads = 256;
constexpr int kFusedThreads = 1024;
constexpr long long kFusedElems = 1 << 16;

// Per-expert terms f_e * P_e reduced by a fixed 256-wide tree; thread e < E
// has its column sum in `colsum`. Writes mean_probs, frac and the loss.
__device__ __forceinline__ void stats_finish(float colsum, const int32_t* __restrict__ counts,
                                             int T, int E, float* __restrict__ mean_probs,
                                             float* __restrict__ frac, float* __restrict__ loss,
                                             float* term) {
  const int e = threadIdx.x;
  if (e < kStatThreads) {
    float fp = 0.f;
    if (e < E) {
      const float P = T > 0 ? colsum / static_cast<float>(T) : 0.f;
      const float f = T > 0 ? static_cast<float>(counts[e]) / static_cast<float>(T) : 0.f;
      mean_probs[e] = P;
      if (frac) frac[e] = f;
      fp = f * P;
    }
    term[e] = fp;
  }
  __syncthreads();
  for (int w = kStatThreads / 2; w > 0; w >>= 1) {
    if (e < w) term[e] += term[e + w];
    __syncthreads();
  }
  if (e == 0) *loss = static_cast<float>(E) * term[0];
}

// One block: thread i < G*E (G = 1024 / E) sums column i % E over rows
// i / E, i / E + G, ...; the G lane sums of a column are then added in lane
// order.
__global__ __launch_bounds__(kFusedThreads) void stats_fused_kernel(
    const float* __restrict__ probs, const int32_t* __restrict__ counts, int T, int E,
    float* __restrict__ mean_probs, float* __restrict__ frac, float* __restrict__ loss) {
  __shared__ float lane_sum[kFusedThreads];
  __shared__ float term[kStatThreads];
  const int G = kFusedThreads / E;
  const int i = threadIdx.x;
  float s = 0.f;
  if (i < G * E) {
    const int e = i % E, g = i / E;
    for (int t = g; t < T; t += G) s += probs[static_cast<size_t>(t) * E + e];
  }
  lane_sum[i] = s;
  __syncthreads();
  float c = 0.f;
  if (i < E)
    for (int g = 0; g < G; ++g) c += lane_sum[g * E + i];
  stats_finish(c, counts, T, E, mean_probs, frac, loss, term);
}

// Thread i < G*E (G = 256 / E row lanes) owns column e = i % E and rows
// r0 + g, r0 + g + G, ... with g = i / E; the G lane sums of a column are
// then added in lane order.
__global__ __launch_bounds__(kStatThreads) void stats_partial_kernel(
    const float* __restrict__ probs, int T, int E, int rows_per_block,
    float* __restrict__ partial) {
  __shared__ float lane_sum[kStatThreads];
  const int G = kStatThreads / E;
  const int i = threadIdx.x;
  const int r0 = blockIdx.x * rows_per_block, r1 = min(T, r0 + rows_per_block);
  float s = 0.f;
  if (i < G * E) {
    const int e = i % E, g = i / E;
    for (int t = r0 + g; t < r1; t += G) s += probs[static_cast<size_t>(t) * E + e];
  }
  lane_sum[i] = s;
  __syncthreads();
  for (int e = i; e < E; e += kStatThreads) {
    float c = 0.f;
    for (int g = 0; g < G; ++g) c += lane_sum[g * E + e];
    partial[static_cast<size_t>(blockIdx.x) * E + e] = c;
  }
}

__global__ __launch_bounds__(kStatThreads) void stats_final_kernel(
    const float* __restrict__ partial, int nblocks, const int32_t* __restrict__ counts, int T,
    int E, float* __restrict__ mean_probs, float* __restrict__ frac, float* __restrict__ loss) {
  __shared__ float term[kStatThreads];
  const int e = threadIdx.x;
  float s = 0.f;
  if (e < E)
    for (int b = 0; b < nblocks; ++b) s += partial[static_cast<size_t>(b) * E + e];
  stats_finish(s, counts, T, E, mean_probs, frac, loss, term);
}

}  // namespace

int router_stats_blocks(int T) {
  // about 64 rows per block, at most 256 blocks
  const int b = (T + 63) / 64;
  return b < 1 ? 1 : (b > 256 ? 256 : b);
}

moe_status launch_router_stats(const float* probs, const int32_t* counts, int T, int E,
                               float* mean_probs, float* frac, float* loss, float* partial,
                               hipStream_t s) {
  if (static_cast<long long>(T) * E <= kFusedElems) {
    stats_fused_kernel<<<1, kFusedThreads, 0, s>>>(probs, counts, T, E, mean_probs, frac, loss);
    return launch_status();
  }
  const int nb = router_stats_blocks(T);
  const int rows = (T + nb - 1) / nb;
  if (T > 0) {
    stats_partial_kernel<<<nb, kStatThreads, 0, s>>>(probs, T, E, rows, partial);
    const moe_status st = launch_status();
    if (st != MOE_OK) return st;
  }
  stats_final_kernel<<<1, kStatThreads, 0, s>>>(partial, T > 0 ? nb : 0, counts, T, E, mean_probs,
                                                frac, loss);
  return launch_status();
}

}  // namespace moe
