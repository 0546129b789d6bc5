// Router: logits = x W_r^T (+ b), softmax, top-k on the logits, renormalise.
//
// Routing follows axonml-nn MoERouter::route (softmax of the router Linear,
// stable descending sort, first k, divide by their sum) and the Mixtral
// page's _moe_forward (softmax, topk, division by the top-k sum). Selection
// compares the fp32 logits through an order-preserving integer key, so it is
// exact: softmax is strictly increasing, and the stable sort's tie rule
// becomes "lower expert index first", with +0.0 and -0.0 equal.
//
// The logits come from route_bf16_kernel (16 tokens per workgroup on the
// bf16 MFMA), from route_bf16_narrow_kernel for batches of at most 64 tokens
// and 16 experts (one workgroup per token), or from route_f32_kernel.
// Routing on gfx950: one wavefront routes one token. Lane l owns experts
// l, l+64, l+128, l+192; each of the k rounds takes the largest order key
// left (a 64-lane maximum on the VALU's data-parallel moves) and, among the
// experts holding it, the lowest index (a ballot).
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

// Largest of the 64 lanes' values, in every lane: row shifts by 1, 2, 4 and
// 8 leave each 16-lane row's maximum in its lane 15, two row broadcasts
// carry it to lane 63 (all on the VALU's data-parallel moves, no LDS), and
// lane 63 is read out. Lanes a move has no source for keep their value,
// which leaves a maximum unchanged.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto mx = [](uint32_t a, int b) { return a > static_cast<uint32_t>(b) ? a : static_cast<uint32_t>(b); };
  const int iv = static_cast<int>(v);
  v = mx(v, __builtin_amdgcn_update_dpp(iv, iv, 0x111, 0xf, 0xf, false));  // row_shr:1
  int t = static_cast<int>(v);
  v = mx(v, __builtin_amdgcn_update_dpp(t, t, 0x112, 0xf, 0xf, false));   // row_shr:2
  t = static_cast<int>(v);
  v = mx(v, __builtin_amdgcn_update_dpp(t, t, 0x114, 0xf, 0xf, false));   // row_shr:4
  t = static_cast<int>(v);
  v = mx(v, __builtin_amdgcn_update_dpp(t, t, 0x118, 0xf, 0xf, false));   // row_shr:8
  t = static_cast<int>(v);
  v = mx(v, __builtin_amdgcn_update_dpp(t, t, 0x142, 0xa, 0xf, false));   // row_bcast:15
  t = static_cast<int>(v);
  v = mx(v, __builtin_amdgcn_update_dpp(t, t, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return __builtin_amdgcn_readlane(v, kWave - 1);
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
  uint32_t kv[4];  // order keys; 0 (below every finite value's key) past E
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + q * kWave;
    v[q] = e < E ? Lrow[e] : -INFINITY;
    kv[q] = e < E ? order_key(v[q]) : 0u;
  }
  // k rounds: the largest order key among the experts not yet taken (a
  // wave maximum over each lane's largest untaken key), then the lowest
  // expert holding that key (a ballot per key slot, q = 0 first: lane l,
  // slot q is expert l + 64q); it takes slot j and drops out. Order keys
  // of finite values are at least 0x007FFFFF, so 0 marks "no expert".
  int my_e = 0;
  float my_v = 0.f, v0 = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t best = kv[0];
    if (E > kWave) {
#pragma unroll
      for (int q = 1; q < 4; ++q) best = kv[q] > best ? kv[q] : best;
    }
    const uint32_t m = wave_max_u32(best);
    int e = -1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q > 0 && E <= kWave) break;
      const uint64_t b = __ballot(kv[q] == m);
      if (e < 0 && b != 0) {
        const int l = static_cast<int>(__builtin_ctzll(b));
        e = l + q * kWave;
        if (lane == l) kv[q] = 0u;
      }
    }
    const float ve = Lrow[e < 0 ? 0 : e];  // (e >= 0: m is some lane's key)
    if (j == 0) v0 = ve;
    if (lane == j) {
      my_e = e;
      my_v = ve;
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
    // every load of the slices goes out before the first product (without
    // the fence the compiler interleaves them with the products)
    __builtin_amdgcn_sched_barrier(0);
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

// bf16 router for small batches (decode): one workgroup of 256 threads per
// token, so the batch's loads spread over as many CUs as it has tokens
// instead of one CU per 16 tokens. Thread i takes 16-byte column chunks
// i, i + 256, ... of x and of every router row (EM >= E rows; the rows past
// E repeat row 0 and their sums are never used), multiplies them in fp32
// and sums per expert; the 256 partial sums are added in a fixed order
// (wave shuffles, then the four waves in turn), so the logits are
// deterministic. J chunks per thread are loaded before the first product:
// one memory round trip per 2048*J columns.
template <int EM, int J>
__global__ __launch_bounds__(256) void route_bf16_narrow_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, float* logits, float* probs, int32_t* idx, float* w) {
  __shared__ float part[4][EM];
  __shared__ float L[EM];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bf16_t* xr = x + static_cast<size_t>(t) * d;
  float acc[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) acc[e] = 0.f;
  const int nch = d / 8;  // 16-byte chunks per row
  for (int c0 = tid; c0 < nch; c0 += 256 * J) {
    uint4 a[J], b[J][EM];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = c0 + 256 * j;
      const int cc = c < nch ? c : 0;
      a[j] = *reinterpret_cast<const uint4*>(xr + 8 * cc);
      if (c >= nch) a[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < EM; ++e)
        b[j][e] = *reinterpret_cast<const uint4*>(wr + static_cast<size_t>(e < E ? e : 0) * d + 8 * cc);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t av[4] = {a[j].x, a[j].y, a[j].z, a[j].w};
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        const uint32_t bv[4] = {b[j][e].x, b[j][e].y, b[j][e].z, b[j][e].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[e] = fmaf(__uint_as_float(av[q] << 16), __uint_as_float(bv[q] << 16), acc[e]);
          acc[e] = fmaf(__uint_as_float(av[q] & 0xFFFF0000u), __uint_as_float(bv[q] & 0xFFFF0000u), acc[e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const float s = wave_sum_f32(acc[e]);
    if (lane == 0) part[wave][e] = s;
  }
  __syncthreads();
  if (wave != 0) return;
  if (lane < EM) {
    float s = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    if (lane < E && bias) s += bias[lane];
    L[lane] = s;
    if (logits && lane < E) logits[static_cast<size_t>(t) * E + lane] = s;
  }
  const size_t tE = static_cast<size_t>(t) * E, tk = static_cast<size_t>(t) * k;
  route_token(L, E, k, probs ? probs + tE : nullptr, idx + tk, w + tk);
}

// fp32 router: one wave per token (four per workgroup). Experts go in
// chunks of EC: each lane keeps EC partial sums over its columns (float4
// chunks 4l, 4l + 256, ... of x and of the EC router rows), so x is read
// once per chunk and the experts' loads go out together; then EC wave sums
// in a fixed order. Rows past E repeat row E-1 and are never stored.
template <int EC>
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
  for (int e0 = 0; e0 < E && valid; e0 += EC) {
    float acc[EC];
#pragma unroll
    for (int j = 0; j < EC; ++j) acc[j] = 0.f;
    for (int c = 4 * lane; c < d; c += 4 * kWave) {
      const float4 xv = *reinterpret_cast<const float4*>(xr + c);
#pragma unroll
      for (int j = 0; j < EC; ++j) {
        const int e = min(e0 + j, E - 1);
        const float4 wv = *reinterpret_cast<const float4*>(wr + static_cast<size_t>(e) * d + c);
        acc[j] = fmaf(xv.x, wv.x, acc[j]);
        acc[j] = fmaf(xv.y, wv.y, acc[j]);
        acc[j] = fmaf(xv.z, wv.z, acc[j]);
        acc[j] = fmaf(xv.w, wv.w, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      float s = wave_sum_f32(acc[j]);
      if (lane == 0 && e0 + j < E) {
        if (bias) s += bias[e0 + j];
        L[wave][e0 + j] = s;
      }
    }
  }
  __syncthreads();
  if (!valid) return;
  const size_t tE = static_cast<size_t>(t) * E, tk = static_cast<size_t>(t) * k;
  if (logits)
    for (int e = lane; e < E; e += kWave) logits[tE + e] = L[wave][e];
  route_token(&L[wave][0], E, k, probs ? probs + tE : nullptr, idx + tk, w + tk);
}

constexpr int kNarrowRouterTokens = 64;

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
    auto kern = E <= 4 ? route_f32_kernel<4> : (E <= 8 ? route_f32_kernel<8> : route_f32_kernel<16>);
    kern<<<(T + 3) / 4, 256, 0, s>>>(static_cast<const float*>(x),
                                     static_cast<const float*>(w_router), bias, T, d, E, k, logits,
                                     probs, topk_idx, topk_w);
    return launch_status();
  }
  // up to 64 tokens: one workgroup per token (decode batches)
  if (T <= kNarrowRouterTokens && E <= 16) {
    auto kern = E <= 8 ? route_bf16_narrow_kernel<8, 2> : route_bf16_narrow_kernel<16, 2>;
    kern<<<T, 256, 0, s>>>(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_router),
                           bias, T, d, E, k, logits, probs, topk_idx, topk_w);
    return launch_status();
  }
  if (E <= 16) return launch_route_bf16<1, 16>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
  if (E <= 32) return launch_route_bf16<2, 16>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
  if (E <= 64) return launch_route_bf16<4, 8>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
  if (E <= 128) return launch_route_bf16<8, 4>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
  return launch_route_bf16<16, 4>(x, w_router, bias, T, d, E, k, logits, probs, topk_idx, topk_w, s);
}

}  // namespace moe
