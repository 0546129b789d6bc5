// Expert histogram, exclusive prefix sum and stable token permutation.
//
// axonml-nn MoELayer::forward counts each expert's assignments and, expert
// by expert, lists the tokens that chose it in ascending token order. Here
// that list becomes a permutation of the T*k assignments: row
// offsets[e] + r holds the r-th token (ascending) that chose expert e.
// Assignment i = t*k + j is ordered by i, which within one expert is token
// order because a token chooses an expert at most once.
//
// One workgroup of 16 waves does the whole job (T*k is at most a few
// hundred thousand here, and the kernel is latency-bound):
//   1. histogram of the expert ids with integer LDS atomics (exact, so the
//      order of the atomics does not matter),
//   2. exclusive scan of the E counts by one wave (shuffle scan),
//   3. the assignments in chunks of 1024, in order: inside a wave, lanes
//      with equal expert ids are found with log2(E) ballots and ranked by
//      the lanes below them; waves are ranked through a per-chunk table of
//      per-wave counts in LDS; a running base per expert carries the rank
//      across chunks. Every position is therefore fixed by the input alone.
// Capacity (KempnerForge moe_capacity_factor): an expert keeps only the
// assignments of rank < cap (the first cap tokens that chose it); the scan
// runs over the kept counts, and a dropped assignment gets inv_pos = -1, so
// the combine adds nothing for it. cap >= T means no limit.
#include "common.h"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ idx, int n, int E, int k, int nbits, int cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ routed_counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token, int32_t* __restrict__ inv_pos) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];   // rank of the expert's next assignment
  __shared__ int start[kMaxExperts];  // first row of the expert
  __shared__ int wave_cnt[kPermWaves][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kPermThreads) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (wave == 0) {
    int c[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      c[q] = e < E ? min(cnt[e], cap) : 0;
      s += c[q];
    }
    int incl = s;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int v = __shfl_up(incl, m, kWave);
      if (lane >= m) incl += v;
    }
    int run = incl - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) {
        base[e] = 0;
        start[e] = run;
        offsets[e] = run;
        counts[e] = c[q];
        if (routed_counts) routed_counts[e] = cnt[e];
      }
      run += c[q];
    }
    if (lane == kWave - 1) offsets[E] = incl;
  }
  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < n; c0 += kPermThreads) {
    for (int q = tid; q < kPermWaves * E; q += kPermThreads) wave_cnt[q / E][q % E] = 0;
    __syncthreads();
    const int i = c0 + tid;
    int e = i < n ? idx[i] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t set = __ballot(bit);
      same &= bit ? set : ~set;
    }
    const int rank = __popcll(same & below);
    if (valid && rank == 0) wave_cnt[wave][e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int r = base[e] + rank;
      for (int w = 0; w < wave; ++w) r += wave_cnt[w][e];
      if (r < cap) {
        const int pos = start[e] + r;
        sorted_token[pos] = i / k;
        inv_pos[i] = pos;
      } else {
        inv_pos[i] = -1;
      }
    } else if (i < n) {
      inv_pos[i] = -1;
    }
    __syncthreads();
    for (int q = tid; q < E; q += kPermThreads) {
      int s = 0;
      for (int w = 0; w < kPermWaves; ++w) s += wave_cnt[w][q];
      base[q] += s;
    }
    __syncthreads();
  }
}

}  // namespace

moe_status launch_permute(const int32_t* topk_idx, int T, int E, int k, int cap, int32_t* counts,
                          int32_t* routed_counts, int32_t* offsets, int32_t* sorted_token,
                          int32_t* inv_pos, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  permute_kernel<<<1, kPermThreads, 0, s>>>(topk_idx, T * k, E, k, nbits, cap < T ? cap : T,
                                            counts, routed_counts, offsets, sorted_token, inv_pos);
  return launch_status();
}

namespace {
// Shared experts take every token: expert s owns rows s*T .. s*T + T-1,
// row s*T + t holding token t.
__global__ __launch_bounds__(256) void identity_rows_kernel(int T, int S, int32_t* sorted_token,
                                                            int32_t* offsets) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < static_cast<size_t>(T) * S) sorted_token[i] = static_cast<int32_t>(i % T);
  if (i <= static_cast<size_t>(S)) offsets[i] = static_cast<int32_t>(i * T);
}
}  // namespace

moe_status launch_identity_rows(int T, int S, int32_t* sorted_token, int32_t* offsets,
                                hipStream_t s) {
  const size_t n = static_cast<size_t>(T) * S + 1;
  identity_rows_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(T, S, sorted_token,
                                                                             offsets);
  return launch_status();
}

}  // namespace moe
