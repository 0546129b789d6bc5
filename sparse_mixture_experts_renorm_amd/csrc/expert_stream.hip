// Grouped expert GEMMs for few tokens per expert (decode-sized batches).
//
// Same computation as the tiled kernels (axonml-nn Expert::forward: h =
// SiLU(X W_g^T) * (X W_u^T), y = h W_d^T over each expert's permuted rows),
// for the case where every expert holds only a handful of rows: the time is
// then the streaming of the expert weights from HBM, and each weight byte is
// used by a few MFMAs at most. Layout:
//   - v_mfma_f32_16x16x32_bf16 with the weights as the first operand: lane l
//     supplies weight row l%16 and the 8 reduction indices 8*(l/16).. of a
//     32-wide step, so the four lanes of a row read 64 contiguous bytes and
//     one load instruction covers 16 whole 64-byte pieces. (Loads whose
//     64-byte pieces are split over several instructions are fetched
//     several times and cap the stream well below the HBM rate.) The token
//     operand uses the same lane -> reduction-index map;
//   - one wave owns 16*RB weight rows of one expert (gate/up: those rows of
//     both matrices) and NB blocks of 16 token rows, accumulating all of
//     them in one pass over the weights; experts with more rows take more
//     passes;
//   - weights go straight from memory to registers, DEPTH 64-wide reduction
//     chunks ahead;
//   - the down GEMM may cut the reduction into S parts (blockIdx.z), each
//     writing its own partial (24-bit format); the combine sums the parts in
//     order;
//   - experts without rows exit at once, so their weights are never read;
//     so do experts with more than max_rows rows, which a tiled launch takes
//     (their weights would otherwise be read once per 16*NB rows);
//   - for a bf16 batch of at most 256 assignments the gate/up kernel ranks
//     each expert's assignments itself (self_permute) instead of reading a
//     permutation, and writes that permutation for the kernels after it.
// Token rows past an expert's count repeat a valid row; their results are
// never stored.
#include "common.h"

namespace moe {
namespace {

constexpr int SW = 4;     // waves per workgroup
constexpr int DEPTH = 3;  // reduction chunks in flight per wave

__device__ __forceinline__ uint4 ld16(const bf16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// lane L takes the 16 bytes lane 4*(L%16) + L/16 loaded (byte address xa)
__device__ __forceinline__ uint4 xpose(uint4 v, int xa) {
  return make_uint4(__builtin_amdgcn_ds_bpermute(xa, static_cast<int>(v.x)),
                    __builtin_amdgcn_ds_bpermute(xa, static_cast<int>(v.y)),
                    __builtin_amdgcn_ds_bpermute(xa, static_cast<int>(v.z)),
                    __builtin_amdgcn_ds_bpermute(xa, static_cast<int>(v.w)));
}

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One pass over reduction range [kbeg, kend) (kbeg a multiple of 64) for
// token rows mb .. mb + 16*NB of expert rows starting at row0; gate/up
// gathers row m's token tok[m]. TWO (down
// only): h comes as two bf16 terms, A and Alo, and both are multiplied into
// the same accumulators. GATE_UP with Clo non-null also writes the second
// term of h.
template <bool GATE_UP, int RB, int NB, bool TWO>
__device__ __forceinline__ void stream_pass(const bf16_t* __restrict__ A,
                                            const bf16_t* __restrict__ Alo,
                                            const int32_t* __restrict__ tok,
                                            const bf16_t* const (&wg)[RB],
                                            const bf16_t* const (&wu)[RB], int row0, int rows,
                                            int mb, int n0, int N, int K, int kbeg, int kend,
                                            void* __restrict__ Cv, bf16_t* __restrict__ Clo,
                                            int lane) {
  const int r16 = lane & 15, q = lane >> 4;
  const int lr = lane >> 2, lp = lane & 3;  // load layout: row lane/4, piece lane%4
  const int xa = 4 * (4 * r16 + q);
  const bf16_t* ap[NB];
  const bf16_t* apl[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    int m = mb + t * 16 + lr;
    m = m < rows ? m : mb;  // repeat a valid row past the end
    const size_t arow = GATE_UP ? static_cast<size_t>(tok[m]) : static_cast<size_t>(row0 + m);
    ap[t] = A + arow * K + lp * 8;
    apl[t] = TWO ? Alo + arow * K + lp * 8 : nullptr;
  }
  f32x4 accg[RB][NB], accu[RB][NB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) accg[r][t][i] = accu[r][t][i] = 0.f;

  // chunk = two 32-wide steps; slot s holds one chunk
  uint4 bw[DEPTH][RB][2], bu[DEPTH][RB][2], ba[DEPTH][NB][2], bl[DEPTH][TWO ? NB : 1][2];
  auto load = [&](int k0, int s) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        bw[s][r][j] = ld16(wg[r] + k0 + 32 * j);
        if (GATE_UP) bu[s][r][j] = ld16(wu[r] + k0 + 32 * j);
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        ba[s][t][j] = ld16(ap[t] + k0 + 32 * j);
        if (TWO) bl[s][t][j] = ld16(apl[t] + k0 + 32 * j);
      }
    }
  };
  auto mma = [&](int s) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint4 a[NB], al[TWO ? NB : 1];
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        a[t] = xpose(ba[s][t][j], xa);
        if (TWO) al[t] = xpose(bl[s][t][j], xa);
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const uint4 g = xpose(bw[s][r][j], xa);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          accg[r][t] = mfma16(g, a[t], accg[r][t]);
          if (TWO) accg[r][t] = mfma16(g, al[t], accg[r][t]);
        }
        if (GATE_UP) {
          const uint4 u = xpose(bu[s][r][j], xa);
#pragma unroll
          for (int t = 0; t < NB; ++t) accu[r][t] = mfma16(u, a[t], accu[r][t]);
        }
      }
    }
  };
  const int nchunks = (kend - kbeg) / 64;
#pragma unroll
  for (int s = 0; s < DEPTH; ++s)
    if (s < nchunks) load(kbeg + 64 * s, s);
  int c = 0;
  for (; c + DEPTH <= nchunks; c += DEPTH) {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
      mma(s);
      if (c + s + DEPTH < nchunks) load(kbeg + 64 * (c + s + DEPTH), s);
    }
  }
#pragma unroll
  for (int s = 0; s < DEPTH; ++s)
    if (c + s < nchunks) mma(s);
  // reduction tail (kend - kbeg not a multiple of 64): 32-wide steps whose
  // 8-element groups past kend read nothing and add zero (K % 8 == 0)
  for (int k0 = kbeg + 64 * nchunks; k0 < kend; k0 += 32) {
    const bool in = k0 + lp * 8 < kend;
    const uint4 z = make_uint4(0, 0, 0, 0);
    uint4 a[NB], al[TWO ? NB : 1];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      a[t] = xpose(in ? ld16(ap[t] + k0) : z, xa);
      if (TWO) al[t] = xpose(in ? ld16(apl[t] + k0) : z, xa);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const uint4 g = xpose(in ? ld16(wg[r] + k0) : z, xa);
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        accg[r][t] = mfma16(g, a[t], accg[r][t]);
        if (TWO) accg[r][t] = mfma16(g, al[t], accg[r][t]);
      }
      if (GATE_UP) {
        const uint4 u = xpose(in ? ld16(wu[r] + k0) : z, xa);
#pragma unroll
        for (int t = 0; t < NB; ++t) accu[r][t] = mfma16(u, a[t], accu[r][t]);
      }
    }
  }

  // acc[r][t] element i: weight row n0 + 16r + 4q + i, token row mb + 16t + r16
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int m = mb + t * 16 + r16;
    if (m >= rows) continue;
    const size_t crow = static_cast<size_t>(row0 + m) * N;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int n = n0 + 16 * r + 4 * q;
      if (n >= N) continue;  // N % 16 == 0: all four columns or none
      if (GATE_UP) {
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = silu_fast(accg[r][t][i]) * accu[r][t][i];
        store_h(static_cast<bf16_t*>(Cv), Clo, crow + n, hv);
      } else {
        *reinterpret_cast<uint3*>(static_cast<char*>(Cv) + (crow + n) * 3) =
            pack_f24x4(accg[r][t][0], accg[r][t][1], accg[r][t][2], accg[r][t][3]);
      }
    }
  }
}

// Rows of expert e = blockIdx.y derived from the routing (StreamPermute):
// one assignment per thread; two ballots per wave find the assignments to
// experts below e (their count is e's first row) and those to e (ranked by
// the assignments before them), whose tokens go to s_tok in row order.
// Workgroup x = 0 of each expert also writes the permutation's outputs; an
// id outside [0, E) (out of contract) gets inv_pos = -1, so the combine
// skips it. Every thread of the workgroup takes part (two barriers).
__device__ __forceinline__ void self_permute(const StreamPermute& sp, int e, int32_t* s_tok,
                                             int* s_cnt, int& row0, int& rows) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, E = gridDim.y;
  const int v = tid < sp.n ? sp.topk_idx[tid] : -1;
  const uint64_t below = __ballot(v >= 0 && v < e), mine = __ballot(v == e);
  if (lane == 0) {
    s_cnt[wave] = __popcll(below);
    s_cnt[SW + wave] = __popcll(mine);
  }
  __syncthreads();
  int r0 = 0, n = 0, before = 0;
#pragma unroll
  for (int w = 0; w < SW; ++w) {
    r0 += s_cnt[w];
    n += s_cnt[SW + w];
    before += w < wave ? s_cnt[SW + w] : 0;
  }
  const bool first = blockIdx.x == 0;
  if (v == e) {
    const int rank = before + __popcll(mine & ((1ull << lane) - 1));
    const int t = tid / sp.k;
    s_tok[rank] = t;
    if (first) {
      sp.sorted_token[r0 + rank] = t;
      sp.inv_pos[tid] = r0 + rank;
    }
  }
  if (first) {
    if (e == 0 && tid < sp.n && (v < 0 || v >= E)) sp.inv_pos[tid] = -1;
    if (tid == 0) {
      sp.counts[e] = n;
      sp.offsets[e] = r0;
      if (e == E - 1) sp.offsets[E] = r0 + n;
    }
  }
  __syncthreads();
  row0 = r0;
  rows = n;
}

// Grid: (ceil(N / (16 * RB * SW)), E, S). GATE_UP: A = x gathered by
// sorted_token, weight rows from w_gate and w_up, C = h (bf16; with Clo
// non-null its second term goes there). !GATE_UP: A = h rows (TWO: plus
// their second terms Alo), weights w_down, C = y (24-bit format), part z at
// element z * c_split. SELF (gate/up): the rows come from the routing in sp
// (self_permute) instead of sorted_token and offsets.
template <bool GATE_UP, int RB, int NB, bool TWO = false, bool SELF = false>
__global__ __launch_bounds__(SW * 64) void expert_stream_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ Alo,
    const int32_t* __restrict__ sorted_token, const int32_t* __restrict__ offsets,
    const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, int N, int K,
    void* __restrict__ Cv, bf16_t* __restrict__ Clo, size_t c_split,
    int32_t* __restrict__ split_out, int max_rows, StreamPermute sp) {
  static_assert(!(TWO && GATE_UP), "two terms of h are an operand of the down pass only");
  static_assert(GATE_UP || !SELF, "the down pass reads the gate/up pass's permutation");
  static_assert(SW * 64 >= kSelfPermuteMax, "self_permute takes one assignment per thread");
  const int S = gridDim.z, z = blockIdx.z;
  if (!GATE_UP && split_out && blockIdx.x == 0 && blockIdx.y == 0 && z == 0 && threadIdx.x == 0)
    *split_out = S;
  const int e = blockIdx.y;
  int row0, rows;
  const int32_t* tok = nullptr;  // gate/up: the token of each of the expert's rows
  if constexpr (SELF) {
    __shared__ int32_t s_tok[kSelfPermuteMax];
    __shared__ int s_cnt[2 * SW];
    self_permute(sp, e, s_tok, s_cnt, row0, rows);
    tok = s_tok;
  } else {
    row0 = offsets[e];
    rows = offsets[e + 1] - row0;
    if (GATE_UP) tok = sorted_token + row0;
  }
  if (rows == 0 || rows > max_rows) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * SW + wave) * 16 * RB;
  if (n0 >= N) return;
  // reduction part z: whole 64-wide chunks, the tail with the last part
  const int nch = K / 64, per = nch / S, extra = nch % S;
  const int kbeg = 64 * (z * per + min(z, extra));
  const int kend = z == S - 1 ? K : kbeg + 64 * (per + (z < extra));
  const int lr = lane >> 2, lp = lane & 3;
  const bf16_t* wg[RB];
  const bf16_t* wu[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int nrow = min(n0 + 16 * r + lr, N - 1);
    const size_t wrow = (static_cast<size_t>(e) * N + nrow) * K + lp * 8;
    wg[r] = B0 + wrow;
    wu[r] = GATE_UP ? B1 + wrow : nullptr;
  }
  void* C = GATE_UP ? Cv : static_cast<void*>(static_cast<char*>(Cv) + z * c_split * 3);
  for (int mb = 0; mb < rows; mb += 16 * NB)
    stream_pass<GATE_UP, RB, NB, TWO>(A, Alo, tok, wg, wu, row0, rows, mb, n0, N, K, kbeg, kend,
                                      C, Clo, lane);
}

// 16-row token blocks per pass: enough for the average expert of the batch.
inline int token_blocks(int rows, int E) { return rows <= 16 * E ? 1 : 2; }

// Gate/up takes one 16-row weight block per wave (more waves for the
// larger grid), down two (the grid is cut along the reduction instead).
constexpr int kRbGateUp = 1, kRbDown = 2;

}  // namespace

moe_status launch_gate_up_stream(const void* x, const int32_t* sorted_token,
                                 const int32_t* offsets, const void* w_gate, const void* w_up,
                                 int d, int ffn, int E, int rows, void* h, bf16_t* h_lo,
                                 int max_rows, const StreamPermute* sp, hipStream_t s) {
  constexpr int RB = kRbGateUp;
  dim3 grid((ffn + 16 * RB * SW - 1) / (16 * RB * SW), E, 1);
  if (sp && sp->n > kSelfPermuteMax) return MOE_UNSUPPORTED;
  const StreamPermute none{};
  auto run = [&](auto kern) {
    kern<<<grid, SW * 64, 0, s>>>(static_cast<const bf16_t*>(x), nullptr, sorted_token, offsets,
                                  static_cast<const bf16_t*>(w_gate),
                                  static_cast<const bf16_t*>(w_up), ffn, d, h, h_lo, size_t(0),
                                  nullptr, max_rows, sp ? *sp : none);
  };
  const bool one = token_blocks(rows, E) == 1;
  if (sp) {
    if (one) run(expert_stream_kernel<true, RB, 1, false, true>);
    else run(expert_stream_kernel<true, RB, 2, false, true>);
  } else {
    if (one) run(expert_stream_kernel<true, RB, 1>);
    else run(expert_stream_kernel<true, RB, 2>);
  }
  return launch_status();
}

moe_status launch_down_stream(const void* h, const bf16_t* h_lo, const int32_t* offsets,
                              const void* w_down, int d, int ffn, int E, int rows, void* y,
                              int32_t* split, int max_rows, int max_split, hipStream_t s) {
  constexpr int RB = kRbDown;
  // cut the reduction (into whole 64-wide chunks, at least 16 per part)
  // until the grid holds about two waves per SIMD
  const int nx = (d + 16 * RB * SW - 1) / (16 * RB * SW);
  int S = 1;
  while (2 * S <= max_split && nx * E * S * SW < 2048 && ffn / 64 >= 2 * S * kMinStreamChunks)
    S *= 2;
  dim3 grid(nx, E, S);
  const size_t c_split = static_cast<size_t>(rows) * d;
  auto run = [&](auto kern) {
    kern<<<grid, SW * 64, 0, s>>>(static_cast<const bf16_t*>(h), h_lo, nullptr, offsets,
                                  static_cast<const bf16_t*>(w_down), nullptr, d, ffn, y, nullptr,
                                  c_split, split, max_rows, StreamPermute{});
  };
  const bool one = token_blocks(rows, E) == 1;
  if (h_lo) {
    if (one) run(expert_stream_kernel<false, RB, 1, true>);
    else run(expert_stream_kernel<false, RB, 2, true>);
  } else {
    if (one) run(expert_stream_kernel<false, RB, 1>);
    else run(expert_stream_kernel<false, RB, 2>);
  }
  return launch_status();
}

}  // namespace moe
