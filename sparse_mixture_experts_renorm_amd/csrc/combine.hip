// Deterministic weighted combine: out[t] = sum_{j<k} w[t,j] * y[inv_pos[t*k+j]].
//
// axonml-nn MoELayer::forward scatter-adds each expert's weighted output
// into a zero buffer; the Mixtral page's _moe_forward does the same with
// out[rows] += w * expert(x[rows]). Here each output row gathers its k
// expert rows instead, so no two threads write one element and no float
// atomics are needed; the k terms are added in slot order (j = 0..k-1) in
// fp32, which fixes the rounding independently of scheduling.
//
// y is fp32 and may hold S partial sums of the down GEMM's reduction (S is
// read from the device, where the down GEMM chose it); each expert row is
// the sum of its S parts in part order, then weighted. Each thread owns 8
// consecutive columns of one token (two 16-byte loads per term); a
// workgroup covers 2048 columns.
#include "common.h"

namespace moe {
namespace {

template <typename YT>
__device__ __forceinline__ void load8(const YT* p, float v[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename OT>
__device__ __forceinline__ void store8(OT* p, const float v[8]);

template <>
__device__ __forceinline__ void store8<float>(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float v[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

template <typename YT, typename OT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const int32_t* __restrict__ split,
                                                      size_t split_stride,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ w, int d, int k,
                                                      OT* __restrict__ out) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (col >= d) return;
  const int S = *split;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int p = inv_pos[static_cast<size_t>(t) * k + j];
    if (p < 0) continue;
    const float wj = w[static_cast<size_t>(t) * k + j];
    const YT* yp = y + static_cast<size_t>(p) * d + col;
    float v[8];
    load8<YT>(yp, v);
    for (int s = 1; s < S; ++s) {
      float u[8];
      load8<YT>(yp + s * split_stride, u);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += u[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
  }
  store8<OT>(out + static_cast<size_t>(t) * d + col, acc);
}

}  // namespace

moe_status launch_combine(const float* y, const int32_t* split, const int32_t* inv_pos,
                          const float* topk_w, int T, int d, int k, void* out, moe_dtype out_dt,
                          hipStream_t s) {
  dim3 grid(T, (d + 2047) / 2048);
  const size_t stride = static_cast<size_t>(T) * k * d;
  if (out_dt == MOE_F32)
    combine_kernel<float, float><<<grid, 256, 0, s>>>(y, split, stride, inv_pos, topk_w, d, k,
                                                      static_cast<float*>(out));
  else
    combine_kernel<float, bf16_t><<<grid, 256, 0, s>>>(y, split, stride, inv_pos, topk_w, d, k,
                                                       static_cast<bf16_t*>(out));
  return launch_status();
}

}  // namespace moe
