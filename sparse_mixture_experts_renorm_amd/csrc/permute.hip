// Expert histogram, exclusive prefix sum and stable token permutation.
//
// axonml-nn MoELayer::forward counts each expert's assignments and, expert
// by expert, lists the tokens that chose it in ascending token order. Here
// that list becomes a permutation of the T*k assignments: row
// offsets[e] + r holds the r-th token (ascending) that chose expert e.
// Assignment i = t*k + j is ordered by i, which within one expert is token
// order because a token chooses an expert at most once.
//
// Up to kPermBlockedFrom assignments one workgroup of 16 waves does the
// whole job in one launch (the call is latency-bound there):
//   1. histogram of the expert ids with integer LDS atomics (exact, so the
//      order of the atomics does not matter),
//   2. exclusive scan of the E counts by one wave (shuffle scan),
//   3. the assignments in chunks of 1024, in order: inside a wave, lanes
//      with equal expert ids are found with log2(E) ballots and ranked by
//      the lanes below them; waves are ranked through a per-chunk table of
//      per-wave counts in LDS; a running base per expert carries the rank
//      across chunks. Every position is therefore fixed by the input alone.
//   With at most 64 experts (permute_small_kernel) the chunks are ranked in
//   one pass, their per-wave counts kept in a table and turned into prefixes
//   afterwards, which saves the barriers between chunks.
// Above that, a count pass writes each block's expert histogram and a
// scatter pass lets every block derive the global offsets and its own rank
// bases from that table, then run step 3 on its range of assignments.
// Capacity (KempnerForge moe_capacity_factor): an expert keeps only the
// assignments of rank < cap (the first cap tokens that chose it); the scan
// runs over the kept counts, and a dropped assignment gets inv_pos = -1, so
// the combine adds nothing for it. cap >= T means no limit.
#include "common.h"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

// Wave 0 scans the kept counts min(cnt[e], cap) into start[] (first row of
// each expert); with `publish` it also writes offsets, counts and the routed
// counts. Called by every thread of the block.
__device__ __forceinline__ void scan_experts(const int* cnt, int E, int cap, bool publish,
                                             int* start, int32_t* __restrict__ counts,
                                             int32_t* __restrict__ routed_counts,
                                             int32_t* __restrict__ offsets) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < kWave) {
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
        start[e] = run;
        if (publish) {
          offsets[e] = run;
          counts[e] = c[q];
          if (routed_counts) routed_counts[e] = cnt[e];
        }
      }
      run += c[q];
    }
    if (publish && lane == kWave - 1) offsets[E] = incl;
  }
  __syncthreads();
}

// Assignments [c_begin, c_end) in chunks of 1024, in order. base[e] holds
// the rank (among all assignments to e, in assignment order) of the next
// one to e and is advanced chunk by chunk; rank r < cap lands in row
// start[e] + r, others are dropped (inv_pos = -1). Called by every thread.
__device__ __forceinline__ void rank_chunks(const int32_t* __restrict__ idx, int c_begin,
                                            int c_end, int E, int k, int nbits, int cap, int* base,
                                            const int* start, int (*wave_cnt)[kMaxExperts],
                                            int32_t* __restrict__ sorted_token,
                                            int32_t* __restrict__ inv_pos) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = c_begin; c0 < c_end; c0 += kPermThreads) {
    for (int q = tid; q < kPermWaves * E; q += kPermThreads) wave_cnt[q / E][q % E] = 0;
    __syncthreads();
    const int i = c0 + tid;
    int e = i < c_end ? idx[i] : -1;
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
    } else if (i < c_end) {
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

// One workgroup for everything (few assignments: one launch).
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ idx, int n, int E, int k, int nbits, int cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ routed_counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token, int32_t* __restrict__ inv_pos) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int start[kMaxExperts];
  __shared__ int wave_cnt[kPermWaves][kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermThreads) {
    cnt[e] = 0;
    base[e] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += kPermThreads) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  scan_experts(cnt, E, cap, true, start, counts, routed_counts, offsets);
  rank_chunks(idx, 0, n, E, k, nbits, cap, base, start, wave_cnt, sorted_token, inv_pos);
}

// Up to kPermSmallMax assignments and kPermSmallExperts experts: one
// workgroup, and every chunk of 1024 assignments ranked in the same pass
// instead of one chunk after the other. Thread tid holds assignment
// c*1024 + tid of each chunk c; in each wave the lanes with its expert id
// are found with log2(E) ballots (its rank among them, and their count);
// the counts go to a table of (chunk, wave) rows per expert, in assignment
// order; one wave per expert turns its column into exclusive prefixes (a
// shuffle scan over up to 128 rows) and a total; one wave scans the kept
// totals into the offsets. An assignment's rank is then its row's prefix
// plus its rank in the wave. Four barriers in all, against three per chunk
// (small workload: 11.4 -> 8.9 us). At 8192 assignments the two-kernel
// multi-block path is faster (11.6 against 13.8 us), so this covers the
// range one workgroup took before.
constexpr int kPermSmallMax = static_cast<int>(kPermBlockedFrom);
constexpr int kPermSmallExperts = 64;
constexpr int kPermSmallChunks = kPermSmallMax / kPermThreads;
constexpr int kPermSmallRows = kPermSmallChunks * kPermWaves;  // 128 (chunk, wave) rows
static_assert(kPermSmallRows <= 2 * kWave, "one scan of two rows per lane");

__global__ __launch_bounds__(kPermThreads) void permute_small_kernel(
    const int32_t* __restrict__ idx, int n, int E, int k, int nbits, int cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ routed_counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ inv_pos) {
  __shared__ int tbl[kPermSmallRows][kPermSmallExperts];
  __shared__ int tot[kPermSmallExperts];
  __shared__ int start[kPermSmallExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (n + kPermThreads - 1) / kPermThreads;
  for (int q = tid; q < nch * kPermWaves * kPermSmallExperts; q += kPermThreads)
    tbl[q / kPermSmallExperts][q % kPermSmallExperts] = 0;
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  int ex[kPermSmallChunks], rk[kPermSmallChunks];
#pragma unroll
  for (int c = 0; c < kPermSmallChunks; ++c) {
    ex[c] = -1;
    rk[c] = 0;
    if (c >= nch) continue;  // uniform over the workgroup
    const int i = c * kPermThreads + tid;
    const int e = i < n ? idx[i] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t set = __ballot(bit);
      same &= bit ? set : ~set;
    }
    if (valid) {
      ex[c] = e;
      rk[c] = __popcll(same & below);
      if (rk[c] == 0) tbl[c * kPermWaves + wave][e] = __popcll(same);
    }
  }
  __syncthreads();
  // column e: exclusive prefix over the rows in assignment order, and the total
  const int rows = nch * kPermWaves;
  for (int e = wave; e < E; e += kPermWaves) {
    const int v0 = lane < rows ? tbl[lane][e] : 0;
    const int v1 = lane + kWave < rows ? tbl[lane + kWave][e] : 0;
    int s0 = v0, s1 = v1;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int a0 = __shfl_up(s0, m, kWave), a1 = __shfl_up(s1, m, kWave);
      if (lane >= m) {
        s0 += a0;
        s1 += a1;
      }
    }
    const int t0 = __shfl(s0, kWave - 1, kWave);
    if (lane < rows) tbl[lane][e] = s0 - v0;
    if (lane + kWave < rows) tbl[lane + kWave][e] = t0 + s1 - v1;
    if (lane == kWave - 1) tot[e] = t0 + s1;
  }
  __syncthreads();
  if (tid < kWave) {
    // kept counts min(total, cap), scanned into each expert's first row
    const int e = lane;
    const int t = e < E ? tot[e] : 0, kept = min(t, cap);
    int incl = kept;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int v = __shfl_up(incl, m, kWave);
      if (lane >= m) incl += v;
    }
    if (e < E) {
      start[e] = incl - kept;
      offsets[e] = incl - kept;
      counts[e] = kept;
      if (routed_counts) routed_counts[e] = t;
    }
    if (lane == kWave - 1) offsets[E] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kPermSmallChunks; ++c) {
    if (c >= nch) continue;
    const int i = c * kPermThreads + tid;
    if (i >= n) continue;
    const int e = ex[c];
    if (e < 0) {
      inv_pos[i] = -1;
      continue;
    }
    const int r = tbl[c * kPermWaves + wave][e] + rk[c];
    if (r < cap) {
      const int pos = start[e] + r;
      sorted_token[pos] = i / k;
      inv_pos[i] = pos;
    } else {
      inv_pos[i] = -1;
    }
  }
}

// Many assignments: block b owns assignments [b*C, (b+1)*C) (C a multiple
// of 1024). Pass 1 writes each block's expert histogram; pass 2 gives every
// block the totals and, from the blocks before it, the rank base of each
// expert, so each block scatters its own range in order.
__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(
    const int32_t* __restrict__ idx, int n, int E, int C, int32_t* __restrict__ block_counts) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  const int c_begin = blockIdx.x * C, c_end = min(n, c_begin + C);
  for (int i = c_begin + tid; i < c_end; i += kPermThreads) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads)
    block_counts[static_cast<size_t>(blockIdx.x) * E + e] = cnt[e];
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int n, int E, int k, int nbits, int cap, int C,
    const int32_t* __restrict__ block_counts, int32_t* __restrict__ counts,
    int32_t* __restrict__ routed_counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ inv_pos) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int start[kMaxExperts];
  __shared__ int wave_cnt[kPermWaves][kMaxExperts];
  __shared__ int part_tot[kPermThreads], part_pre[kPermThreads];
  const int tid = threadIdx.x, b = blockIdx.x, nb = gridDim.x;
  // Column sums of the count table (every block's total and the blocks
  // before b): G groups of E threads, group g summing blocks g, g + G, ...
  // (independent loads, one memory round trip for up to G blocks), then E
  // threads add the G partial sums (integers: exact in any order). G is at
  // most the number of blocks, so no group sums nothing.
  const int G = min(kPermThreads / E, nb);
  if (tid < G * E) {
    const int g = tid / E, e = tid - g * E;
    int tot = 0, pre = 0;
    for (int bb = g; bb < nb; bb += G) {
      const int c = block_counts[static_cast<size_t>(bb) * E + e];
      pre += bb < b ? c : 0;
      tot += c;
    }
    part_tot[tid] = tot;
    part_pre[tid] = pre;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) {
    int tot = 0, pre = 0;
    for (int g = 0; g < G; ++g) {
      tot += part_tot[g * E + e];
      pre += part_pre[g * E + e];
    }
    cnt[e] = tot;
    base[e] = pre;
  }
  __syncthreads();
  scan_experts(cnt, E, cap, b == 0, start, counts, routed_counts, offsets);
  const int c_begin = b * C;
  rank_chunks(idx, c_begin, min(n, c_begin + C), E, k, nbits, cap, base, start, wave_cnt,
              sorted_token, inv_pos);
}

}  // namespace

int permute_blocks(int T, int k) {
  const long long n = static_cast<long long>(T) * k;
  if (n <= kPermBlockedFrom) return 0;  // one workgroup
  const long long chunks = (n + kPermThreads - 1) / kPermThreads;
  const long long per = (chunks + kPermMaxBlocks - 1) / kPermMaxBlocks;  // chunks per block
  return static_cast<int>((chunks + per - 1) / per);
}

moe_status launch_permute(const int32_t* topk_idx, int T, int E, int k, int cap, int32_t* counts,
                          int32_t* routed_counts, int32_t* offsets, int32_t* sorted_token,
                          int32_t* inv_pos, int32_t* block_counts, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int n = T * k;
  const int c = cap < T ? cap : T;
  if (n <= kPermSmallMax && E <= kPermSmallExperts) {
    permute_small_kernel<<<1, kPermThreads, 0, s>>>(topk_idx, n, E, k, nbits, c, counts,
                                                    routed_counts, offsets, sorted_token, inv_pos);
    return launch_status();
  }
  const int nb = permute_blocks(T, k);
  if (nb == 0) {
    permute_kernel<<<1, kPermThreads, 0, s>>>(topk_idx, n, E, k, nbits, c, counts, routed_counts,
                                              offsets, sorted_token, inv_pos);
    return launch_status();
  }
  const long long chunks = (static_cast<long long>(n) + kPermThreads - 1) / kPermThreads;
  const int C = static_cast<int>((chunks + nb - 1) / nb) * kPermThreads;
  permute_count_kernel<<<nb, kPermThreads, 0, s>>>(topk_idx, n, E, C, block_counts);
  moe_status st = launch_status();
  if (st != MOE_OK) return st;
  permute_scatter_kernel<<<nb, kPermThreads, 0, s>>>(topk_idx, n, E, k, nbits, c, C, block_counts,
                                                     counts, routed_counts, offsets, sorted_token,
                                                     inv_pos);
  return launch_status();
}

namespace {
// The gate weights in permuted order: sorted_w[inv_pos[i]] = topk_w[i]
// (skipping dropped assignments, inv_pos = -1).
__global__ __launch_bounds__(256) void permute_weights_kernel(const int32_t* __restrict__ inv_pos,
                                                              const float* __restrict__ topk_w,
                                                              int n, float* __restrict__ sorted_w) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int p = inv_pos[i];
  if (p >= 0) sorted_w[p] = topk_w[i];
}

// Shared experts take every token: expert s owns rows s*T .. s*T + T-1,
// row s*T + t holding token t.
__global__ __launch_bounds__(256) void identity_rows_kernel(int T, int S, int32_t* sorted_token,
                                                            int32_t* offsets) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < static_cast<size_t>(T) * S) sorted_token[i] = static_cast<int32_t>(i % T);
  if (i <= static_cast<size_t>(S)) offsets[i] = static_cast<int32_t>(i * T);
}
}  // namespace

moe_status launch_permute_weights(const int32_t* inv_pos, const float* topk_w, int n,
                                  float* sorted_w, hipStream_t s) {
  permute_weights_kernel<<<(n + 255) / 256, 256, 0, s>>>(inv_pos, topk_w, n, sorted_w);
  return launch_status();
}

moe_status launch_identity_rows(int T, int S, int32_t* sorted_token, int32_t* offsets,
                                hipStream_t s) {
  const size_t n = static_cast<size_t>(T) * S + 1;
  identity_rows_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(T, S, sorted_token,
                                                                             offsets);
  return launch_status();
}

}  // namespace moe
