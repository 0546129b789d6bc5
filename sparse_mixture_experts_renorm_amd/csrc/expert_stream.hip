// Grouped expert GEMMs for few tokens per expert (decode-sized batches).
//
// Same computation as the tiled kernels (axonml-nn Expert::forward: h =
// SiLU(X W_g^T) * (X W_u^T), y = h W_d^T over each expert's permuted rows),
// for the case where every expert holds only a handful of rows: the time is
// then the streaming of the expert weights from HBM, and each weight byte is
// used by at most a few MFMAs. Layout:
//   - one wave owns 32 weight rows (gate/up: 32 gate rows and the same 32
//     up rows) of one expert and all of that expert's rows, in blocks of
//     32 (v_mfma_f32_32x32x16_bf16, weights as the first operand);
//   - weights go straight from memory to registers, no LDS: per 64-wide
//     reduction chunk lane l loads 64 contiguous bytes of weight row l%32
//     (half l/32 of the 128-byte chunk) as four 16-byte loads, and MFMA i of
//     the chunk uses load i. The token operand is loaded with the same
//     lane -> reduction-index map, so every product pairs equal indices;
//   - chunks are prefetched DEPTH deep in registers so each wave keeps
//     DEPTH x 8 KB of weights in flight;
//   - experts without rows exit at once, so their weights are never read.
// Token rows past an expert's count repeat a valid row; their results are
// never stored.
#include "common.h"

namespace moe {
namespace {

constexpr int SW = 4;       // waves per workgroup
constexpr int DEPTH = 3;    // reduction chunks in flight per wave

__device__ __forceinline__ uint4 ld16(const bf16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Grid: (ceil(N / (32 * SW)), E). GATE_UP: A = x gathered by sorted_token,
// weight rows from w_gate and w_up, C = h (bf16). !GATE_UP: A = h rows,
// weights w_down, C = y (fp32).
template <bool GATE_UP>
__global__ __launch_bounds__(SW * 64) void expert_stream_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_token,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, int N, int K, void* __restrict__ Cv,
    int32_t* __restrict__ split_out) {
  if (!GATE_UP && split_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    *split_out = 1;
  const int e = blockIdx.y;
  const int row0 = offsets[e], rows = offsets[e + 1] - row0;
  if (rows == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * SW + wave) * 32;
  if (n0 >= N) return;
  const int half = lane >> 5, r32 = lane & 31;
  const int nrow = min(n0 + r32, N - 1);
  const size_t wrow = (static_cast<size_t>(e) * N + nrow) * K;
  const bf16_t* wg = B0 + wrow + half * 32;
  const bf16_t* wu = GATE_UP ? B1 + wrow + half * 32 : nullptr;
  const int nchunks = K / 64;   // K is a multiple of 16; the tail is handled below
  const int ktail = K - nchunks * 64;

  for (int mb = 0; mb < rows; mb += 32) {
    const int m = mb + r32 < rows ? mb + r32 : mb;  // repeat a valid row past the end
    const size_t arow = GATE_UP ? static_cast<size_t>(sorted_token[row0 + m])
                                : static_cast<size_t>(row0 + m);
    const bf16_t* ap = A + arow * K + half * 32;

    f32x16 acc_g, acc_u;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_g[i] = acc_u[i] = 0.f;

    uint4 bw[DEPTH][4], bu[DEPTH][4], ba[DEPTH][4];
    auto load = [&](int c, int slot) {
      const int k0 = c * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bw[slot][i] = ld16(wg + k0 + i * 8);
        if (GATE_UP) bu[slot][i] = ld16(wu + k0 + i * 8);
        ba[slot][i] = ld16(ap + k0 + i * 8);
      }
    };
    auto mma = [&](int slot) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, ba[slot][i]);
        acc_g = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bw[slot][i]), a,
                                                        acc_g, 0, 0, 0);
        if (GATE_UP)
          acc_u = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bu[slot][i]),
                                                          a, acc_u, 0, 0, 0);
      }
    };
#pragma unroll
    for (int c = 0; c < DEPTH; ++c)
      if (c < nchunks) load(c, c);
    int c = 0;
    for (; c + DEPTH <= nchunks; c += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        mma(s);
        if (c + s + DEPTH < nchunks) load(c + s + DEPTH, s);
      }
    }
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
      if (c + s < nchunks) mma(s);
    if (ktail) {
      // last K % 64 elements, in 16-wide steps: lanes of half h take the
      // 8 elements at 16*i + 8*h, with the same map for both operands
      const int k0 = nchunks * 64;
      for (int i = 0; i < ktail / 16; ++i) {
        const int kk = k0 + i * 16 + half * 8 - half * 32;  // pointers carry + half*32
        const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(ap + kk));
        acc_g = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ld16(wg + kk)),
                                                        a, acc_g, 0, 0, 0);
        if (GATE_UP)
          acc_u = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ld16(wu + kk)),
                                                          a, acc_u, 0, 0, 0);
      }
    }

    // acc element i: weight row n0 + 8*(i/4) + 4*half + i%4, token row mb + lane%32
    const int mt = mb + r32;
    if (mt < rows) {
      const size_t crow = static_cast<size_t>(row0 + mt) * N;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 8 * g + 4 * half;
        if (n >= N) continue;
        if (GATE_UP) {
          float hv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = silu(acc_g[4 * g + i]) * acc_u[4 * g + i];
          *reinterpret_cast<uint2*>(static_cast<bf16_t*>(Cv) + crow + n) =
              make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(Cv) + crow + n) =
              make_float4(acc_g[4 * g], acc_g[4 * g + 1], acc_g[4 * g + 2], acc_g[4 * g + 3]);
        }
      }
    }
  }
}

}  // namespace

moe_status launch_gate_up_stream(const void* x, const int32_t* sorted_token,
                                 const int32_t* offsets, const void* w_gate, const void* w_up,
                                 int d, int ffn, int E, void* h, hipStream_t s) {
  dim3 grid((ffn + 32 * SW - 1) / (32 * SW), E);
  expert_stream_kernel<true><<<grid, SW * 64, 0, s>>>(
      static_cast<const bf16_t*>(x), sorted_token, offsets, static_cast<const bf16_t*>(w_gate),
      static_cast<const bf16_t*>(w_up), ffn, d, h, nullptr);
  return launch_status();
}

moe_status launch_down_stream(const void* h, const int32_t* offsets, const void* w_down, int d,
                              int ffn, int E, float* y, int32_t* split, hipStream_t s) {
  dim3 grid((d + 32 * SW - 1) / (32 * SW), E);
  expert_stream_kernel<false><<<grid, SW * 64, 0, s>>>(
      static_cast<const bf16_t*>(h), nullptr, offsets, static_cast<const bf16_t*>(w_down), nullptr,
      d, ffn, y, split);
  return launch_status();
}

}  // namespace moe
