// Router: logits = x W_r^T (+ b), softmax, top-k on the logits, renormalise.
//
// Routing follows axonml-nn MoERouter::route (softmax of the router Linear,
// stable descending sort, first k, divide by their sum) and the Mixtral
// page's _moe_forward (softmax, topk, division by the top-k sum). Selection
// compares the fp32 logits through an order-preserving integer key, so it is
// exact: softmax is strictly increasing, and the stable sort's tie rule
// becomes "lower expert index first", with +0.0 and -0.0 equal.
//
// Layout on gfx950: one wavefront routes one token. Lane l owns experts
// l, l+64, l+128, l+192; each of the k rounds is a 64-lane max-reduction of
// 64-bit keys (value key << 32 | ~expert) through cross-lane shuffles.
// The renormalised weight of slot j is exp(L_j - L_0) / sum_i exp(L_i - L_0),
// which equals p_j / sum_i p_i because the softmax denominator cancels.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) == 0u) b = 0u;  // -0.0 ties with +0.0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, kWave);
  uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, kWave);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Route one token whose E logits are at Lrow (LDS or global). Called by all
// 64 lanes of a wave with the same arguments.
__device__ void route_token(const float* Lrow, int E, int k, float* probs_row,
                            int32_t* idx_row, float* w_row) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[4];
  uint64_t key[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + q * kWave;
    v[q] = e < E ? Lrow[e] : -INFINITY;
    key[q] = e < E ? ((static_cast<uint64_t>(order_key(v[q])) << 32) | static_cast<uint32_t>(~e)) : 0ull;
  }
  int my_e = 0;
  float my_v = 0.f, v0;
  if (E <= kWave) {
    // One key per lane. Lane l's slot is the rank of its key (how many of the
    // E keys are larger; keys are distinct, so the ranks are 0 .. E-1; lanes
    // past E hold key 0 and rank E >= k). The keys are read out lane by lane
    // on the scalar path, then each selected lane hands its expert and logit
    // to the lane of its slot.
    const uint32_t khi = static_cast<uint32_t>(key[0] >> 32), klo = static_cast<uint32_t>(key[0]);
    int rank = 0;
    for (int m = 0; m < E; ++m) {
      const uint32_t mhi = __builtin_amdgcn_readlane(khi, m), mlo = __builtin_amdgcn_readlane(klo, m);
      rank += (mhi > khi || (mhi == khi && mlo > klo)) ? 1 : 0;
    }
    my_e = __builtin_amdgcn_ds_permute(rank * 4, lane);
    my_v = __int_as_float(__builtin_amdgcn_ds_permute(rank * 4, __float_as_int(v[0])));
    v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
  } else {
    // k rounds of a 64-lane maximum over four keys per lane
    v0 = 0.f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = key[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) best = key[q] > best ? key[q] : best;
      best = wave_max_u64(best);
      const int e = static_cast<int>(~static_cast<uint32_t>(best));
      const float ve = Lrow[e];
      if (j == 0) v0 = ve;
      if (lane == j) { my_e = e; my_v = ve; }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + q * kWave == e) key[q] = 0ull;
    }
  }
  if (probs_row) {
    // the largest logit is v0, the selected first one
    float z[4], s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      z[q] = lane + q * kWave < E ? expf(v[q] - v0) : 0.f;
      s += z[q];
    }
    s = wave_sum_f32(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + q * kWave < E) probs_row[lane + q * kWave] = z[q] * inv;
  }
  // renormalised weights over the k selected experts
  const float ex = lane < k ? expf(my_v - v0) : 0.f;
  const float s = wave_sum_f32(ex);
  if (lane < k) {
    idx_row[lane] = my_e;
    w_row[lane] = ex / s;
  }
}

// ---------------------------------------------------------------------------
// Routing from given logits: one wave per token.
__global__ __launch_bounds__(256) void route_logits_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, float* probs,
                                                           int32_t* idx, float* w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t tE = static_cast<size_t>(t) * E, tk = static_cast<size_t>(t) * k;
  route_token(logits + tE, E, k, probs ? probs + tE : nullptr, idx + tk, w + tk);
}

// ---------------------------------------------------------------------------
// bf16 router: 16 tokens per workgroup. The [16 x d] x [d x 16*NB] product
// runs on v_mfma_f32_16x16x32_bf16 with the reduction dimension split over
// the NW waves (fixed summation order afterwards, so results are
// deterministic). Operands come straight from global memory: lane l reads
// 8 consecutive bf16 (16 bytes) of row l%16 at column 8*(l/16) of each
// 32-wide slice, which is the MFMA operand layout for a K-contiguous matrix
// (A and B use the same lane-to-k assignment, so the dot products are
// complete whatever the hardware's internal k order).
template <int NB, int NW>
__global__ __launch_bounds__(NW * 64) void route_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, float* logits, float* probs, int32_t* idx, float* w) {
  constexpr int NE = 16 * NB;
  __shared__ float part[NW][16][NE];
  __shared__ float L[16][NE + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16;
  const int r = lane & 15, kq = lane >> 4;
  const bool row_ok = t0 + r < T;
  const bf16_t* xrow = x + static_cast<size_t>(row_ok ? t0 + r : 0) * d;

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each wave takes U consecutive 32-wide slices at a time and issues all
  // their loads before the first product, so a wave waits for one memory
  // round trip per U slices (this kernel is latency-bound for small T):
  // with 16 waves and U = 8 a width of 4096 takes one round trip.
  // Out-of-range rows, experts and columns load from a valid address and
  // are replaced by zeros, which keeps the loads unconditional.
  constexpr int U = NB <= 2 ? 8 : 4;  // registers: U * (1 + NB) 16-byte operands
  const int nk = (d + 31) / 32;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (int kc0 = wave * U; kc0 < nk; kc0 += NW * U) {
    uint4 a[U], b[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int col = (kc0 + u) * 32 + kq * 8;
      const bool col_ok = col < d;
      const int c = col_ok ? col : 0;
      a[u] = *reinterpret_cast<const uint4*>(xrow + c);
      if (!(row_ok && col_ok)) a[u] = zero;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int e = nb * 16 + r;
        b[u][nb] = *reinterpret_cast<const uint4*>(wr + static_cast<size_t>(min(e, E - 1)) * d + c);
        if (!(e < E && col_ok)) b[u][nb] = zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                          __builtin_bit_cast(bf16x8, b[u][nb]),
                                                          acc[nb], 0, 0, 0);
  }
  // D layout: lane l holds rows 4*(l/16)+i, column l%16
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][kq * 4 + i][nb * 16 + r] = acc[nb][i];
  __syncthreads();
  for (int q = threadIdx.x; q < 16 * NE; q += NW * 64) {
    const int m = q / NE, n = q % NE;
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) s += part[wv][m][n];
    if (n < E && bias) s += bias[n];
    L[m][n] = s;
    if (logits && n < E && t0 + m < T) logits[static_cast<size_t>(t0 + m) * E + n] = s;
  }
  __syncthreads();
  for (int m = wave; m < 16; m += NW) {
    const int t = t0 + m;
    if (t >= T) break;
    const size_t tE = static_cast<size_t>(t) * E, tk = static_cast<size_t>(t) * k;
    route_token(&L[m][0], E, k, probs ? probs + tE : nullptr, idx + tk, w + tk);
  }
}

// fp32 router: one wave per token, lanes split the width, experts in turn.
__global__ __launch_bounds__(256) void route_f32_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ wr,
                                                        const float* __restrict__ bias, int T, int d,
                                                        int E, int k, float* logits, float* probs,
                                                        int32_t* idx, float* w) {
  __shared__ float L[4][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool valid = t < T;
  const float* xr = x + static_cast<size_t>(valid ? t : 0) * d;
  for (int e = 0; e < E && valid; ++e) {
    const float* wrow = wr + static_cast<size_t>(e) * d;
    float s = 0.f;
    for (int i = lane; i < d; i += kWave) s = fmaf(xr[i], wrow[i], s);
    s = wave_sum_f32(s);
    if (bias) s += bias[e];
    if (lane == 0) L[wave][e] = s;
  }
  __syncthreads();
  if (!valid) return;
  const size_t tE = static_cast<size_t>(t) * E, tk = static_cast<size_t>(t) * k;
  if (logits)
    for (int e = lane; e < E; e += kWave) logits[tE + e] = L[wave][e];
  route_token(&L[wave][0], E, k, probs ? probs + tE : nullptr, idx + tk, w + tk);
}

template <int NB, int NW>
moe_status launch_route_bf16(const void* x, const void* wr, const float* bias, int T, int d, int E,
                             int k, float* logits, float* probs, int32_t* idx, float* w,
                             hipStream_t s) {
  dim3 grid((T + 15) / 16);
  route_bf16_kernel<NB, NW><<<grid, NW * 64, 0, s>>>(static_cast<const bf16_t*>(x),
                                                     static_cast<const bf16_t*>(wr), bias, T, d, E,
                                                     k, logits, probs, idx, w);
  return launch_status();
}

}  // namespace

moe_status launch_route_logits(const float* logits, int T, int E, int k, float* probs,
                               int32_t* topk_idx, float* topk_w, hipStream_t s) {
  route_logits_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, probs, topk_idx, topk_w);
  return launch_status();
}

moe_status launch_route(const void* x, const void* w_router, const float* bias, int T, int d,
                        int E, int k, moe_dtype dt, float* logits, float* probs,
                        int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (dt == MOE_F32) {
    route_f32_kernel<<<(T + 3) / 4, 256, 0, s>>>(static_cast<const float*>(x),
                                                 static_cast<const float*>(w_router), bias, T, d,
                                                 E, k, logits, probs, topk_idx, topk_w);
    return launch_status();
  }
  if (E <= 16) return launch_route_bf16<1, 16>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
  if (E <= 32) return launch_route_bf16<2, 16>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
  if (E <= 64) return launch_route_bf16<4, 8>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
  if (E <= 128) return launch_route_bf16<8, 4>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
  return launch_route_bf16<16, 4>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
}

}  // namespace moe
