// Grouped expert GEMMs over the permuted tokens.
//
// Expert e (axonml-nn Expert::forward; skills page SwiGLU) on its rows X_e:
//   h = SiLU(X_e W_g[e]^T) * (X_e W_u[e]^T)      (gate/up pass, SiLU on gate)
//   y = h W_d[e]^T                               (down pass)
// X_e are the rows sorted_token[offsets[e] .. offsets[e+1]) of x: the gather
// is done by the tile loads, so X_e is never written out. h and y are stored
// in permuted-row order, row offsets[e] + r for the r-th token of expert e.
// h is bf16 (the down pass multiplies it on the bf16 MFMA); y stays fp32,
// because rounding y to bf16 as well would spend about half of the 2e-2 x RMS
// error budget of bf16 workloads on top of h's rounding.
//
// bf16 path (gfx950 MFMA). A workgroup of 4 waves computes one output tile
// of 128 permuted rows; the gate/up pass produces 64 columns of h from a
// 128-row weight tile (64 gate rows + the same 64 up rows), the down pass
// 128 columns of y. The reduction dimension moves through LDS in steps of
// 64 (128 bytes per row), double-buffered: the next step's global loads are
// in flight while the current one runs on v_mfma_f32_32x32x16_bf16.
// LDS rows are XOR-swizzled in 16-byte chunks (chunk c of row r is stored at
// c ^ (r & 7)) so the MFMA operand reads of 32 different rows spread over
// all banks. The MFMA takes the weight tile as its first operand, so each
// lane's accumulators hold 4 consecutive output columns of one row, which
// the epilogue writes as one 8-byte store.
//
// Tile schedule: the host sizes the grid from an upper bound on the tile
// count; each workgroup reads the per-expert offsets, counts the real tiles
// and maps itself to (expert, row tile, column tile). Workgroups are handed
// to the 8 XCDs round-robin, so consecutive tiles of the schedule are given
// to workgroups on the same XCD (sharing its L2): each XCD takes a
// contiguous eighth of the tile list. Inside an expert the list runs over
// groups of GN column tiles, and inside a group over row tiles, then
// column tiles, so a weight tile is loaded by all row tiles of the expert
// at about the same time.
#include "common.h"

namespace moe {
namespace {

constexpr int BM = 128;   // permuted rows per tile
constexpr int BNW = 128;  // weight rows per tile
constexpr int BK = 64;    // reduction step (elements)
constexpr int NT = 256;   // threads per workgroup
constexpr int GN = 8;     // column tiles per schedule group
constexpr int kXcds = 8;

struct Tile {
  int e, row0, rows, nt;
};

// Map this workgroup to a tile; returns false if it has none.
__device__ bool map_tile(const int32_t* __restrict__ offsets, int E, int nN, Tile* out) {
  __shared__ int s_tile[4];
  if (threadIdx.x == 0) {
    int total = 0;
    for (int e = 0; e < E; ++e) {
      const int m = offsets[e + 1] - offsets[e];
      total += ((m + BM - 1) / BM) * nN;
    }
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    int L = xcd * per_xcd + slot;
    int res_e = -1, res_m = 0, res_n = 0;
    if (slot < per_xcd && L < total) {
      for (int e = 0; e < E; ++e) {
        const int m = offsets[e + 1] - offsets[e];
        const int mt = (m + BM - 1) / BM;
        const int te = mt * nN;
        if (L < te) {
          const int g = L / (mt * GN);
          const int r = L % (mt * GN);
          const int gn = min(GN, nN - g * GN);
          res_e = e;
          res_m = r / gn;
          res_n = g * GN + r % gn;
          break;
        }
        L -= te;
      }
    }
    s_tile[0] = res_e;
    if (res_e >= 0) {
      const int m = offsets[res_e + 1] - offsets[res_e];
      s_tile[1] = offsets[res_e] + res_m * BM;
      s_tile[2] = min(BM, m - res_m * BM);
      s_tile[3] = res_n;
    }
  }
  __syncthreads();
  if (s_tile[0] < 0) return false;
  out->e = s_tile[0];
  out->row0 = s_tile[1];
  out->rows = s_tile[2];
  out->nt = s_tile[3];
  return true;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// GATE_UP: A = x gathered by sorted_token, B = [w_gate; w_up], C = h.
// !GATE_UP: A = h (rows in order), B = w_down, C = y.
template <bool GATE_UP>
__global__ __launch_bounds__(NT, 1) void expert_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_token,
    const int32_t* __restrict__ offsets, int E, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, int N, int K, void* __restrict__ Cv) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][BM * 128];  // [buf][A|B]
  const int nN = GATE_UP ? (N + 63) / 64 : (N + BNW - 1) / BNW;
  Tile tile;
  if (!map_tile(offsets, E, nN, &tile)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Global source of the 4 A chunks and 4 B chunks this thread stages.
  const bf16_t* a_src[4];
  const bf16_t* b_src[4];
  int lds_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = tid + NT * j;
    const int row = q >> 3, c = q & 7;
    lds_off[j] = swz(row, c);
    a_src[j] = nullptr;
    if (row < tile.rows) {
      const size_t arow = GATE_UP ? static_cast<size_t>(sorted_token[tile.row0 + row])
                                  : static_cast<size_t>(tile.row0 + row);
      a_src[j] = A + arow * K + c * 8;
    }
    b_src[j] = nullptr;
    if (GATE_UP) {
      const int n = tile.nt * 64 + (row & 63);
      if (n < N) b_src[j] = (row < 64 ? B0 : B1) + (static_cast<size_t>(tile.e) * N + n) * K + c * 8;
    } else {
      const int n = tile.nt * BNW + row;
      if (n < N) b_src[j] = B0 + (static_cast<size_t>(tile.e) * N + n) * K + c * 8;
    }
  }
  const int kc_lane = (lane >> 5);  // which 8-element half of a 16-wide k step

  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = k0 + ((tid + NT * j) & 7) * 8;
      ra[j] = (a_src[j] && kk < K) ? *reinterpret_cast<const uint4*>(a_src[j] + k0) : make_uint4(0, 0, 0, 0);
      rb[j] = (b_src[j] && kk < K) ? *reinterpret_cast<const uint4*>(b_src[j] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<uint4*>(&lds[buf][0][lds_off[j]]) = ra[j];
      *reinterpret_cast<uint4*>(&lds[buf][1][lds_off[j]]) = rb[j];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  // weight-tile row base of the wave's two 32-row blocks
  int brow[2];
  brow[0] = GATE_UP ? wn * 32 : wn * 64;
  brow[1] = GATE_UP ? 64 + wn * 32 : wn * 64 + 32;
  const int arow0 = wm * 64 + (lane & 31);

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const char* la = lds[buf][0];
    const char* lb = lds[buf][1];
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = 2 * s + kc_lane;
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        fa[mb] = *reinterpret_cast<const bf16x8*>(la + swz(arow0 + mb * 32, c));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        fb[nb] = *reinterpret_cast<const bf16x8*>(lb + swz(brow[nb] + (lane & 31), c));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nb], fa[mb], acc[nb][mb], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue. acc[nb][mb] element i: token row wm*64 + mb*32 + lane%32,
  // weight-tile row brow[nb] + 8*(i/4) + 4*(lane/32) + i%4.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = wm * 64 + mb * 32 + (lane & 31);
    if (m >= tile.rows) continue;
    const size_t crow = static_cast<size_t>(tile.row0 + m) * N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nloc = 8 * g + 4 * (lane >> 5);
      if (GATE_UP) {
        const int n = tile.nt * 64 + wn * 32 + nloc;
        if (n < N) {
          float hv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = silu(acc[0][mb][4 * g + i]) * acc[1][mb][4 * g + i];
          uint2 pk = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          *reinterpret_cast<uint2*>(static_cast<bf16_t*>(Cv) + crow + n) = pk;
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int n = tile.nt * BNW + brow[nb] + nloc;
          if (n < N)
            *reinterpret_cast<float4*>(static_cast<float*>(Cv) + crow + n) =
                make_float4(acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                            acc[nb][mb][4 * g + 3]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per output element, plain fp32 FMA loops. Only for
// the fp32 dtype (small parity workloads); grid = (rows, column blocks).
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E, int r) {
  int lo = 0, hi = E;  // largest e with offsets[e] <= r
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) void expert_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ sorted_token,
    const int32_t* __restrict__ offsets, int E, const float* __restrict__ B0,
    const float* __restrict__ B1, int N, int K, float* __restrict__ C) {
  const int r = blockIdx.x;
  const int n = blockIdx.y * 256 + threadIdx.x;
  if (r >= offsets[E] || n >= N) return;
  const int e = expert_of_row(offsets, E, r);
  const float* a = A + static_cast<size_t>(GATE_UP ? sorted_token[r] : r) * K;
  const float* b0 = B0 + (static_cast<size_t>(e) * N + n) * K;
  if (GATE_UP) {
    const float* b1 = B1 + (static_cast<size_t>(e) * N + n) * K;
    float g = 0.f, u = 0.f;
    for (int i = 0; i < K; ++i) {
      g = fmaf(a[i], b0[i], g);
      u = fmaf(a[i], b1[i], u);
    }
    C[static_cast<size_t>(r) * N + n] = silu(g) * u;
  } else {
    float s = 0.f;
    for (int i = 0; i < K; ++i) s = fmaf(a[i], b0[i], s);
    C[static_cast<size_t>(r) * N + n] = s;
  }
}

}  // namespace

// upper bound on sum_e ceil(M_e / BM) over the experts' row counts M_e
static unsigned tile_grid(int rows, int E, int nN) {
  const long long max_mt = rows / BM + (rows < E ? rows : E);
  const long long g = max_mt * nN;
  return static_cast<unsigned>((g + kXcds - 1) / kXcds * kXcds);
}

moe_status launch_gate_up(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                          const void* w_gate, const void* w_up, int T, int d, int ffn, int E,
                          int k, moe_dtype dt, void* h, hipStream_t s) {
  const int rows = T * k;
  if (dt == MOE_F32) {
    expert_gemm_f32_kernel<true><<<dim3(rows, (ffn + 255) / 256), 256, 0, s>>>(
        static_cast<const float*>(x), sorted_token, offsets, E, static_cast<const float*>(w_gate),
        static_cast<const float*>(w_up), ffn, d, static_cast<float*>(h));
    return launch_status();
  }
  expert_gemm_bf16_kernel<true><<<tile_grid(rows, E, (ffn + 63) / 64), NT, 0, s>>>(
      static_cast<const bf16_t*>(x), sorted_token, offsets, E, static_cast<const bf16_t*>(w_gate),
      static_cast<const bf16_t*>(w_up), ffn, d, h);
  return launch_status();
}

moe_status launch_down(const void* h, const int32_t* offsets, const void* w_down, int T, int d,
                       int ffn, int E, int k, moe_dtype dt, float* y, hipStream_t s) {
  const int rows = T * k;
  if (dt == MOE_F32) {
    expert_gemm_f32_kernel<false><<<dim3(rows, (d + 255) / 256), 256, 0, s>>>(
        static_cast<const float*>(h), nullptr, offsets, E, static_cast<const float*>(w_down),
        nullptr, d, ffn, y);
    return launch_status();
  }
  expert_gemm_bf16_kernel<false><<<tile_grid(rows, E, (d + BNW - 1) / BNW), NT, 0, s>>>(
      static_cast<const bf16_t*>(h), nullptr, offsets, E, static_cast<const bf16_t*>(w_down),
      nullptr, d, ffn, y);
  return launch_status();
}

}  // namespace moe
