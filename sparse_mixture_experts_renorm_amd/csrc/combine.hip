// Deterministic weighted combine: out[t] = sum_{j<k} w[t,j] * y[inv_pos[t*k+j]].
//
// axonml-nn MoELayer::forward scatter-adds each expert's weighted output
// into a zero buffer; the Mixtral page's _moe_forward does the same with
// out[rows] += w * expert(x[rows]). Here each output row gathers its k
// expert rows instead, so no two threads write one element and no float
// atomics are needed; the k terms are added in slot order (j = 0..k-1) in
// fp32, which fixes the rounding independently of scheduling.
//
// y holds S partial sums of the down GEMM's reduction (S is read from the
// device, where the down GEMM chose it; S = 0 means the count is given per
// row and 256-column tile in a part table, where the 384-row down tiles
// record one part, or two for an XCD's tail tiles), fp32 for an fp32 layer
// and in the 24-bit format of common.h for a bf16 layer; each expert row is
// the sum of its parts in part order, then weighted. Each thread owns 8 consecutive
// columns of one token (32 or 24 bytes per term); a workgroup covers 2048
// columns.
//
// Block options (the extended forward): after the k routed terms come the
// outputs of the shared experts, each with weight 1 and in expert order
// (KempnerForge moe_shared_experts), and then the residual input (the
// Mixtral block's moe_residual add), all in fp32 before the one rounding to
// the output dtype.
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

// eight 24-bit values (24 bytes, 8-byte aligned: the column is a multiple
// of 8)
__device__ __forceinline__ void load8_f24(const char* p, float v[8]) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  const uint2 b = *reinterpret_cast<const uint2*>(p + 8);
  const uint2 c = *reinterpret_cast<const uint2*>(p + 16);
  unpack_f24x4(a.x, a.y, b.x, v);
  unpack_f24x4(b.y, c.x, c.y, v + 4);
}

// row r, columns col.. of y (element index r*d + col), in the format F24
template <bool F24>
__device__ __forceinline__ void load_y(const void* y, size_t at, float v[8]) {
  if constexpr (F24)
    load8_f24(static_cast<const char*>(y) + at * 3, v);
  else
    load8<float>(static_cast<const float*>(y) + at, v);
}

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float v[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
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

struct CombineExtra {
  const void* ys;           // shared experts' outputs: parts of [n_shared * T, d], or null
  const int32_t* ys_split;  // number of parts in ys
  size_t ys_stride;         // elements between parts
  int n_shared, T;
  const void* resid;        // residual input [T, d] (fp32 or bf16), or null
  const uint8_t* parts;     // partial sums per (y row, 256-column tile) when *split == 0
};

// RES: 0 no residual, 1 fp32 residual, 2 bf16 residual; SH: shared experts;
// F24: y and ys in the 24-bit format.
template <typename OT, int RES, bool SH, bool F24>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ split,
                                                      size_t split_stride,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ w, int d, int k,
                                                      CombineExtra ex, const uint8_t* __restrict__ parts,
                                                      OT* __restrict__ out) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (col >= d) return;
  // S partial sums for every row, or (S = 0) the count of each row's
  // 256-column tile in parts
  const int S = *split;
  const int nct = (d + 255) / 256, ct = col >> 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int p = inv_pos[static_cast<size_t>(t) * k + j];
    if (p < 0) continue;
    const float wj = w[static_cast<size_t>(t) * k + j];
    const size_t at = static_cast<size_t>(p) * d + col;
    float v[8];
    load_y<F24>(y, at, v);
    const int Sp = S > 0 ? S : parts[static_cast<size_t>(p) * nct + ct];
    for (int s = 1; s < Sp; ++s) {
      float u[8];
      load_y<F24>(y, at + s * split_stride, u);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += u[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
  }
  if constexpr (SH) {
    const int Ss = *ex.ys_split;
    for (int sh = 0; sh < ex.n_shared; ++sh) {
      const size_t at = (static_cast<size_t>(sh) * ex.T + t) * d + col;
      float v[8];
      load_y<F24>(ex.ys, at, v);
      for (int s = 1; s < Ss; ++s) {
        float u[8];
        load_y<F24>(ex.ys, at + s * ex.ys_stride, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] += u[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
  }
  if constexpr (RES != 0) {
    float r[8];
    if constexpr (RES == 1)
      load8<float>(static_cast<const float*>(ex.resid) + static_cast<size_t>(t) * d + col, r);
    else
      load8<bf16_t>(static_cast<const bf16_t*>(ex.resid) + static_cast<size_t>(t) * d + col, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += r[i];
  }
  store8<OT>(out + static_cast<size_t>(t) * d + col, acc);
}

template <typename OT, int RES, bool SH, bool F24>
void combine_launch(dim3 grid, hipStream_t s, const void* y, const int32_t* split, size_t stride,
                    const int32_t* inv_pos, const float* w, int d, int k, const CombineExtra& ex,
                    void* out) {
  combine_kernel<OT, RES, SH, F24><<<grid, 256, 0, s>>>(y, split, stride, inv_pos, w, d, k, ex,
                                                        ex.parts, static_cast<OT*>(out));
}

template <typename OT, bool F24>
void combine_dispatch(dim3 grid, hipStream_t s, const void* y, const int32_t* split,
                      size_t stride, const int32_t* inv_pos, const float* w, int d, int k,
                      const CombineExtra& ex, int res, void* out) {
  const bool sh = ex.n_shared > 0;
  if (res == 0) {
    if (sh) combine_launch<OT, 0, true, F24>(grid, s, y, split, stride, inv_pos, w, d, k, ex, out);
    else combine_launch<OT, 0, false, F24>(grid, s, y, split, stride, inv_pos, w, d, k, ex, out);
  } else if (res == 1) {
    if (sh) combine_launch<OT, 1, true, F24>(grid, s, y, split, stride, inv_pos, w, d, k, ex, out);
    else combine_launch<OT, 1, false, F24>(grid, s, y, split, stride, inv_pos, w, d, k, ex, out);
  } else {
    if (sh) combine_launch<OT, 2, true, F24>(grid, s, y, split, stride, inv_pos, w, d, k, ex, out);
    else combine_launch<OT, 2, false, F24>(grid, s, y, split, stride, inv_pos, w, d, k, ex, out);
  }
}

}  // namespace

moe_status launch_combine_ext(const void* y, const int32_t* split, const int32_t* inv_pos,
                              const float* topk_w, int T, int d, int k, moe_dtype dt,
                              const void* ys, const int32_t* ys_split, int n_shared,
                              const void* resid, moe_dtype resid_dt, void* out, moe_dtype out_dt,
                              hipStream_t s, const uint8_t* y_parts) {
  dim3 grid(T, (d + 2047) / 2048);
  const size_t stride = static_cast<size_t>(T) * k * d;
  CombineExtra ex{ys, ys_split, static_cast<size_t>(T) * n_shared * d, n_shared, T, resid, y_parts};
  const int res = resid == nullptr ? 0 : (resid_dt == MOE_F32 ? 1 : 2);
  const bool f24 = dt == MOE_BF16;
  if (out_dt == MOE_F32) {
    if (f24) combine_dispatch<float, true>(grid, s, y, split, stride, inv_pos, topk_w, d, k, ex, res, out);
    else combine_dispatch<float, false>(grid, s, y, split, stride, inv_pos, topk_w, d, k, ex, res, out);
  } else {
    if (f24) combine_dispatch<bf16_t, true>(grid, s, y, split, stride, inv_pos, topk_w, d, k, ex, res, out);
    else combine_dispatch<bf16_t, false>(grid, s, y, split, stride, inv_pos, topk_w, d, k, ex, res, out);
  }
  return launch_status();
}

moe_status launch_combine(const void* y, const int32_t* split, const int32_t* inv_pos,
                          const float* topk_w, int T, int d, int k, moe_dtype dt, void* out,
                          moe_dtype out_dt, hipStream_t s, const uint8_t* y_parts) {
  return launch_combine_ext(y, split, inv_pos, topk_w, T, d, k, dt, nullptr, nullptr, 0, nullptr,
                            MOE_F32, out, out_dt, s, y_parts);
}

}  // namespace moe
