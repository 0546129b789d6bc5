// RMSNorm of the layer input (the Mixtral page's post-attention nn.RMSNorm
// ahead of the MoE block): xn[t] = x[t] / sqrt(mean_i x[t,i]^2 + eps) * g.
//
// One wave per token row. Each lane sums the squares of its 8-element
// chunks in fp32 in chunk order, a butterfly gives every lane the same row
// total (fixed shape, so deterministic), and a second pass over the row
// (now in cache) scales and stores it in the storage dtype (bf16 rounded to
// nearest even). The kernel is bound by HBM: it reads the row twice at most
// from L2 and writes it once.
#include "common.h"

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ void ld8(const T* p, float v[8]);

template <>
__device__ __forceinline__ void ld8<float>(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
__device__ __forceinline__ void ld8<bf16_t>(const bf16_t* p, float v[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

template <typename T>
__device__ __forceinline__ void st8(T* p, const float v[8]);

template <>
__device__ __forceinline__ void st8<float>(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <>
__device__ __forceinline__ void st8<bf16_t>(bf16_t* p, const float v[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

template <typename T>
__global__ __launch_bounds__(256) void rms_norm_kernel(const T* __restrict__ x,
                                                       const T* __restrict__ g, int T_, int d,
                                                       float eps, T* __restrict__ xn) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const T* row = x + static_cast<size_t>(t) * d;
  float ss = 0.f;
  for (int c = lane * 8; c < d; c += kWave * 8) {
    float v[8];
    ld8<T>(row + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) ss += __shfl_xor(ss, m, kWave);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
  T* out = xn + static_cast<size_t>(t) * d;
  for (int c = lane * 8; c < d; c += kWave * 8) {
    float v[8], w[8];
    ld8<T>(row + c, v);
    ld8<T>(g + c, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * inv * w[i];
    st8<T>(out + c, v);
  }
}

}  // namespace

moe_status launch_rms_norm(const void* x, const void* g, int T, int d, float eps, moe_dtype dt,
                           void* xn, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
  if (dt == MOE_BF16)
    rms_norm_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(x),
                                                 static_cast<const bf16_t*>(g), T, d, eps,
                                                 static_cast<bf16_t*>(xn));
  else
    rms_norm_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x),
                                                static_cast<const float*>(g), T, d, eps,
                                                static_cast<float*>(xn));
  return launch_status();
}

}  // namespace moe
