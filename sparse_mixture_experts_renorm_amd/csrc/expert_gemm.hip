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
// bf16 path (gfx950), two tile shapes: 256 x 256 (below) and the tall
// 384 x 256 tiles further down, taken when the experts average at least 768
// rows. One workgroup of 8 waves per CU (two per SIMD)
// computes a 256 x 256 tile: 256 permuted rows against 256 weight rows
// (gate/up: 128 gate rows and the same 128 up rows, giving 128 columns of h;
// down: 256 columns of y). Each wave owns 128 token rows (four 32-row blocks,
// interleaved with the other row group's) against 64 weight rows: 8
// accumulators of v_mfma_f32_32x32x16_bf16 (128 fp32 per lane), so each
// 16-byte fragment read from LDS feeds 2 or 4 MFMAs; with two waves per SIMD
// one wave's MFMAs run while the other waits for its data. A wave skips the
// MFMAs of its blocks that lie wholly past the tile's rows. The reduction
// dimension moves in steps of 64 through two LDS stages (64 KB each): the
// loads of step s+1 go from memory straight to LDS (buffer_load_dwordx4 ...
// lds, no VGPRs) while the MFMAs of step s run, spread over the first half
// of the step. Each lane
// supplies its own 32-bit offset, which is how the token gather of the
// gate/up pass is done; when K is not a multiple of 64, global loads whose
// lanes past K read a 16-byte zero page are used instead. The step waits
// mostly on the latency of the L2 and the data it returns, not on the LDS
// or the MFMAs.
// LDS rows are 128 bytes (64 bf16); chunk c (16 bytes) of row r is stored at
// slot c ^ ((r >> 1) & 7). gfx950 serves a 16-byte-per-lane LDS read 16 lanes
// at a time over 64 four-byte banks; a fragment read sends 16 consecutive
// rows to those lanes, and the row's half of the 256-byte bank line (r & 1)
// together with its slot gives 16 distinct bank groups.
// The MFMA takes the weight fragment as its first operand, so each lane's
// accumulators hold 4 consecutive output columns of one row, which the
// epilogue writes as one 8-byte (h) or 16-byte (y) store.
//
// Tile schedule: the host sizes the grid from an upper bound on the tile
// count; each workgroup reads the per-expert offsets, counts the real tiles
// and maps itself to (expert, row tile, column tile). An expert's rows are
// cut into ceil(rows / tile height) row tiles of nearly equal height (whole
// 32-row blocks), so little of any tile is padding and the row tiles of one
// weight tile take the same time. Workgroups are handed
// to the 8 XCDs round-robin, so consecutive tiles of the schedule are given
// to workgroups on the same XCD (sharing its L2): each XCD takes a
// contiguous eighth of the tile list. Inside an expert (and split part) the
// list runs over column tiles and, for each, over its row tiles, so the row
// tiles that share a weight tile run side by side and the weights go
// through L2 about once (with the row tiles of one column tile spread over
// rounds instead, the L2 fetched a third more).
#include "common.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kXcds = 8;
constexpr int kMinSplitSteps = 12;

struct Tile {
  int e, row0, rows, nt;
  int ks, S;  // split of the reduction dimension: this tile computes part ks of S
  int half;   // -1: the whole column tile; 0 or 1: that half of its weight rows
};

// Row tiles of BM rows per expert, as a prefix: pref[e] = sum over e' < e of
// ceil(M_e' / BM), for e = 0 .. E (M_e = offsets[e+1] - offsets[e]).
// Serial form, for the host; the kernels build the same array with one wave
// (map_tile).
template <int BM>
__host__ __device__ inline void row_tile_prefix(const int32_t* __restrict__ offsets, int E,
                                                int* pref) {
  pref[0] = 0;
  for (int e = 0; e < E; ++e) pref[e + 1] = pref[e] + (offsets[e + 1] - offsets[e] + BM - 1) / BM;
}

// Tile of workgroup `block` among tiles of BM rows, given the experts' row
// offsets and their row-tile prefix pref [E+1]: res = {expert (-1: none),
// first permuted row, rows, column tile, split part, split count S, half
// (-1: whole column tile; 0 or 1: that half of its weight rows)}.
// The tile list runs over the experts in order; inside an expert over the
// split parts, and inside a part over column tiles and, for each, over its
// row tiles.
// With max_split > 1 the reduction dimension may be cut into S <= max_split
// parts, each a separate tile whose partial result goes to its own output
// slice; S is chosen from the real tile count to minimise the number of
// rounds on n_cu CUs, counted in units of a whole tile, with at least
// kMinSplitSteps of the nk reduction steps in every part (shorter parts
// would spend more on the extra partial sums than they save).
// With TAIL, an XCD whose tile count leaves a last round at most half full
// (r tiles for its n_cu/8 CUs, 2r <= n_cu/8) runs those r tiles as 2r
// half-width tiles, so its last round takes about half a tile's time
// instead of a whole one (the workgroups of the halves come last in the
// XCD's order); the grid provides n_cu/16 extra slots per XCD for them.
// Host-callable so that the assignment can be checked exhaustively on the
// CPU.
template <int BM, bool TAIL>
__host__ __device__ inline void assign_tile(const int32_t* __restrict__ offsets, const int* pref,
                                            int E, int nN, int max_split, int n_cu, int nk,
                                            int block, int* res) {
  const int base = pref[E] * nN;
  int S = 1, best_rounds = (base + n_cu - 1) / n_cu;  // rounds of S-tiles
  for (int c = 2; c <= max_split && c * kMinSplitSteps <= nk; ++c) {
    const int rounds = (base * c + n_cu - 1) / n_cu;
    if (rounds * S < best_rounds * c) {  // rounds/c < best_rounds/S
      S = c;
      best_rounds = rounds;
    }
  }
  const int total = base * S;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int xcd = block % kXcds, slot = block / kXcds;
  const int first = xcd * per_xcd;
  int cnt = total - first;  // tiles of this XCD
  cnt = cnt < 0 ? 0 : (cnt > per_xcd ? per_xcd : cnt);
  int L = -1, half = -1;
  if (TAIL) {
    const int cpx = n_cu / kXcds > 1 ? n_cu / kXcds : 1, r = cnt % cpx;
    const int nfull = (r > 0 && 2 * r <= cpx) ? cnt - r : cnt;
    if (slot < nfull) {
      L = first + slot;
    } else if (slot < nfull + 2 * (cnt - nfull)) {
      L = first + nfull + (slot - nfull) / 2;
      half = (slot - nfull) & 1;
    }
  } else if (slot < cnt) {
    L = first + slot;
  }
  res[0] = -1;
  res[5] = S;
  res[6] = half;
  if (L < 0) return;
  // the expert of tile L: the first e with pref[e+1] * nN * S > L
  const int per_row_tile = nN * S;
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pref[mid + 1] * per_row_tile > L) hi = mid; else lo = mid + 1;
  }
  const int e = lo;
  L -= pref[e] * per_row_tile;
  const int mt = pref[e + 1] - pref[e], m = offsets[e + 1] - offsets[e];
  const int te = mt * nN;  // tiles of one split part of expert e
  const int ks = L / te;
  L -= ks * te;
  // The expert's rows are cut into its mt row tiles as evenly as 32-row
  // blocks allow (block counts differ by at most one, each at most BM/32):
  // the tiles that share a weight tile then take about the same time and
  // stay in step, and no tile is mostly padding.
  const int mi = L % mt, nb = (m + 31) / 32;
  const int b0 = static_cast<int>(static_cast<long long>(mi) * nb / mt);
  const int b1 = static_cast<int>(static_cast<long long>(mi + 1) * nb / mt);
  res[0] = e;
  res[1] = offsets[e] + 32 * b0;
  res[2] = (32 * b1 < m ? 32 * b1 : m) - 32 * b0;
  res[3] = L / mt;
  res[4] = ks;
}

// LDS the tile map needs: the seven results, then the prefix.
constexpr int kMapLdsInts = 8 + kMaxExperts + 1;
static_assert(kMaxExperts <= 4 * kWave, "map_tile sums four experts per lane");

// Map this workgroup to its tile; returns false if it has none. Wave 0
// builds the row-tile prefix in LDS (lane l sums experts 4l .. 4l+3, a wave
// scan adds up the lanes: one memory round trip for any E <= 256), then
// thread 0 runs assign_tile on it. s_map: kMapLdsInts ints of LDS.
template <int BM, bool TAIL = false>
__device__ bool map_tile(const int32_t* __restrict__ offsets, int E, int nN, int max_split,
                         int n_cu, int nk, Tile* out, int* s_map) {
  int* pref = s_map + 8;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      c[q] = e < E ? (offsets[e + 1] - offsets[e] + BM - 1) / BM : 0;
      sum += c[q];
    }
    int incl = sum;
#pragma unroll
    for (int dl = 1; dl < kWave; dl <<= 1) {
      const int v = __shfl_up(incl, dl, kWave);
      if (lane >= dl) incl += v;
    }
    int run = incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      if (e < E) pref[e] = run;
      run += c[q];
    }
    if (lane == kWave - 1) pref[E] = incl;
  }
  __syncthreads();
  if (threadIdx.x == 0) assign_tile<BM, TAIL>(offsets, pref, E, nN, max_split, n_cu, nk, blockIdx.x, s_map);
  __syncthreads();
  out->S = s_map[5];
  if (s_map[0] < 0) return false;
  out->e = s_map[0];
  out->row0 = s_map[1];
  out->rows = s_map[2];
  out->nt = s_map[3];
  out->ks = s_map[4];
  out->half = s_map[6];
  return true;
}

// 16 bytes of zeros: the source of every masked lane of a direct LDS load.
__device__ __attribute__((aligned(64))) uint32_t g_zero_page[16];

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void load_lds16(const void* g, char* lds_chunk_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(lds_chunk_base), 16, 0, 0);
}

// Steps that lie wholly inside K load through a buffer resource instead:
// buffer_load_dwordx4 ... lds with the lane's 32-bit offset and the step's
// byte offset in a scalar register. The address unit takes these faster
// than 64-bit global addresses (the GEMMs run 5-10% faster), and no vector
// instruction is spent on addresses. The resource covers 4 GB from base
// (raw buffer, no range clamping in practice; every offset here is below
// 2^32 by the layer's size limits).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                                  char* lds_chunk_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lds_chunk_base), 16, voff, soff, 0, 0);
}

template <int V>
using IntC = std::integral_constant<int, V>;

constexpr int TM = 256;        // permuted rows per tile
constexpr int TW = 256;        // weight rows per tile
constexpr int TK = 64;         // reduction step (elements); one LDS row = 128 bytes
constexpr int STAGE = TM * TK * 2;  // bytes per operand and stage (32 KB)

// GATE_UP: A = x gathered by sorted_token, weights = [w_gate; w_up], C = h (bf16).
// !GATE_UP: A = h (rows in order), weights = w_down, C = y (fp32); the
// reduction may be split (see assign_tile): part ks writes C + ks * c_split,
// and workgroup 0 stores the split count S in *split_out.
// NW waves per workgroup: 4 (wave tile 128 x 128, one wave per SIMD) or 8
// (wave tile 128 x 64, two waves per SIMD, so one wave's MFMAs run while the
// other waits to issue its loads).
template <bool GATE_UP, int NW, bool KMASK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void expert_gemm_bf16_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_token,
                             const int32_t* __restrict__ offsets, int E,
                             const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, int N,
                             int K, void* __restrict__ Cv, int max_split, int n_cu,
                             size_t c_split, int32_t* __restrict__ split_out) {
  // One LDS object per stage and operand. They must be distinct objects: the
  // compiler then sees that the memory-to-LDS loads of the next stage cannot
  // alias the fragment reads of the current one, and does not make those
  // reads wait for the loads.
  __shared__ __attribute__((aligned(1024))) char lds0a[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds0b[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1a[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1b[STAGE];
  // st and op are compile-time constants at every use, so this folds away
  auto buf = [&](int st, int op) -> char* {
    return st == 0 ? (op ? lds0b : lds0a) : (op ? lds1b : lds1a);
  };
  const int nN = GATE_UP ? (N + 127) / 128 : (N + TW - 1) / TW;
  Tile tile;
  const int nk = (K + TK - 1) / TK;
  __shared__ int s_map[kMapLdsInts];
  const bool have = map_tile<TM>(offsets, E, nN, max_split, n_cu, nk, &tile, s_map);
  if (!GATE_UP && blockIdx.x == 0 && threadIdx.x == 0) *split_out = tile.S;
  if (!have) return;
  // reduction steps [kbeg, kend) of this tile
  const int kbeg = tile.ks * nk / tile.S, kend = (tile.ks + 1) * nk / tile.S;

  constexpr int IPW = 32 / NW;   // 1 KB load instructions per wave, per operand and stage
  constexpr int WN = NW / 2;     // waves along the weight rows
  constexpr int NBW = 8 / WN;    // 32-row weight blocks per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- direct-load sources. Per stage each operand is 256 rows x 128 bytes,
  // loaded by 32 instructions of 1 KB (8 rows); wave w issues instructions
  // IPW*w .. IPW*w + IPW-1 of each operand. In instruction q lane l writes
  // row r = q*8 + l/8, slot l%8, which holds chunk (l%8) ^ ((r >> 1) & 7).
  // Sources are 32-bit byte offsets from one base per operand. Rows past the
  // tile's valid rows (or past N) repeat valid rows: their products are
  // computed but never stored. With KMASK, chunks past K read the zero page.
  // Tile row r of the weight operand: gate/up rows 0-127 are gate rows
  // n0 .. n0+127, rows 128-255 the same rows of up; down rows are n0 + r.
  const int n0 = GATE_UP ? tile.nt * 128 : tile.nt * TW;
  const char* a_base = reinterpret_cast<const char*>(A);
  const size_t wexp = static_cast<size_t>(tile.e) * N * K * 2;
  auto a_row_off = [&](int r) -> uint32_t {
    // past the valid rows, spread the repeats over all valid rows (one
    // repeated row for a whole load instruction would hit one cache line)
    const int rr = r < tile.rows ? r : r % tile.rows;
    const uint32_t arow = GATE_UP ? static_cast<uint32_t>(sorted_token[tile.row0 + rr])
                                  : static_cast<uint32_t>(tile.row0 + rr);
    return arow * static_cast<uint32_t>(K) * 2u;
  };
  auto b_row_off = [&](int r) -> uint32_t {
    const int n = min(n0 + (GATE_UP ? (r & 127) : r), N - 1);
    return static_cast<uint32_t>(n) * static_cast<uint32_t>(K) * 2u;
  };
  uint32_t a_off[IPW], b_off[IPW];
  int kchunk[IPW];
  const char* b_base[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = (wave * IPW + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    kchunk[j] = c;
    a_off[j] = a_row_off(r) + c * 16u;
    b_off[j] = b_row_off(r) + c * 16u;
    b_base[j] = reinterpret_cast<const char*>((GATE_UP && r >= 128) ? B1 : B0) + wexp;
  }
  const char* zero = reinterpret_cast<const char*>(g_zero_page);
  // every b_base[j] of a wave is the same matrix (gate/up: waves 0-3 load
  // gate rows, 4-7 up rows)
  const __amdgpu_buffer_rsrc_t a_rs = buffer_rsrc(a_base), b_rs = buffer_rsrc(b_base[0]);
  // load instruction j (0 .. 2*IPW-1: A then B) of step kt into stage st;
  // without KMASK every chunk of the step lies inside K
  auto issue_one = [&](int kt, int st, int j) __attribute__((always_inline)) {
    const int k0 = kt * TK;
    const int jj = j % IPW;
    const uint32_t kb = static_cast<uint32_t>(k0) * 2u;
    const char* base = j < IPW ? a_base : b_base[jj];
    const uint32_t off = j < IPW ? a_off[jj] : b_off[jj];
    char* dst = buf(st, j < IPW ? 0 : 1) + (wave * IPW + jj) * 1024;
    if constexpr (KMASK)
      load_lds16(k0 + kchunk[jj] * 8 < K ? base + (off + kb) : zero, dst);
    else
      buffer_load_lds16(j < IPW ? a_rs : b_rs, off, kb, dst);
  };
  // ---- fragment reads: row R's chunk c is at R*128 + ((c ^ ((R >> 1) & 7)) << 4);
  // every row this lane reads has R % 32 == lane % 32.
  const int xr = ((lane & 31) >> 1) & 7, half = lane >> 5;
  // weight blocks of this wave: gate/up: NBW/2 gate blocks, then the same
  // rows of up (tile rows + 128); down: NBW consecutive blocks
  int fa_off[4], fb_off[NBW];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa_off[i] = ((wm + 2 * i) * 32 + (lane & 31)) * 128;
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int brow = GATE_UP ? (i / (NBW / 2)) * 128 + wn * (NBW / 2) * 32 + (i % (NBW / 2)) * 32
                             : wn * NBW * 32 + i * 32;
    fb_off[i] = (brow + (lane & 31)) * 128;
  }

  f32x16 acc[NBW][4];
#pragma unroll
  for (int a = 0; a < NBW; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  // One step on stage st: groups of one weight fragment times the four token
  // fragments (4 MFMAs). The fragments of group g+1 are read before the MFMAs
  // of group g, and the first half of the groups each issue a share of the
  // next step's loads, so the load instructions go out at the rate the
  // address unit takes them instead of stalling every wave at the start of
  // the step; the scheduling fences keep that order. In the last step the
  // loads re-read an in-range step into the idle stage, which keeps the
  // instruction stream free of branches.
  constexpr int kGroups = (TK / 16) * NBW;
  constexpr int kLoadGroups = kGroups / 2;
  auto run = [&](auto mac) __attribute__((always_inline)) {
    constexpr int MA = decltype(mac)::value;  // token blocks of this wave with real rows
    auto step = [&](int kt, int st) __attribute__((always_inline)) {
      const int kload = min(kt + 1, nk - 1);
      auto rd = [&](int op, int off, int s) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(buf(st, op) + off + (((2 * s + half) ^ xr) << 4));
      };
      bf16x8 fa[2][MA], fb[2];
#pragma unroll
      for (int i = 0; i < MA; ++i) fa[0][i] = rd(0, fa_off[i], 0);
      fb[0] = rd(1, fb_off[0], 0);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const int s = g / NBW, nb = g % NBW, ca = s & 1, cb = g & 1;
        if (g + 1 < kGroups) {
          const int s1 = (g + 1) / NBW, nb1 = (g + 1) % NBW;
          if (nb1 == 0) {
#pragma unroll
            for (int i = 0; i < MA; ++i) fa[ca ^ 1][i] = rd(0, fa_off[i], s1);
          }
          fb[cb ^ 1] = rd(1, fb_off[nb1], s1);
        }
        if (g < kLoadGroups) {
#pragma unroll
          for (int j = g * 2 * IPW / kLoadGroups; j < (g + 1) * 2 * IPW / kLoadGroups; ++j)
            issue_one(kload, st ^ 1, j);
        }
#pragma unroll
        for (int mb = 0; mb < MA; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cb], fa[ca][mb], acc[nb][mb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Before step kt is computed its loads must have landed in LDS (each wave
    // waits for its own); the barrier then makes every wave's loads visible
    // and guarantees that the other stage, overwritten during step kt, is no
    // longer read. Steps go in pairs (stage 0, stage 1); an odd last step runs
    // on stage 0.
    const int nsteps = kend - kbeg;
    if (nsteps > 0) {
      const int k0 = kbeg * TK;
#pragma unroll
      for (int j = 0; j < 2 * IPW; ++j) {
        const int jj = j % IPW;
        const bool kin = k0 + kchunk[jj] * 8 < K;
        const char* src = j < IPW ? a_base + (a_off[jj] + k0 * 2u) : b_base[jj] + (b_off[jj] + k0 * 2u);
        load_lds16(kin ? src : zero, buf(0, j < IPW ? 0 : 1) + (wave * IPW + jj) * 1024);
      }
    }
    for (int p = 0; p + 1 < nsteps; p += 2) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        step(kbeg + p + r, r);
      }
    }
    if (nsteps & 1) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      step(kend - 1, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  // Token block i of this wave is tile block wm + 2i (32 rows each), so the
  // blocks past the tile's rows fall on the waves, and so on the SIMDs,
  // about equally; a wave runs the step with only its MA blocks that hold
  // rows (the MFMAs of padding blocks are skipped). Every variant loads the
  // same data and meets the same barriers.
  const int nblk = (tile.rows + 31) / 32;
  const int nact = nblk - wm >= 7 ? 4 : (nblk - wm >= 5 ? 3 : (nblk - wm >= 3 ? 2 : 1));
  if (nact == 4)
    run(IntC<4>{});
  else if (nact == 3)
    run(IntC<3>{});
  else if (nact == 2)
    run(IntC<2>{});
  else
    run(IntC<1>{});

  // ---- epilogue. acc[nb][mb] element i: token row (wm + 2 mb)*32 + lane%32,
  // weight-tile row (block nb) + 8*(i/4) + 4*(lane/32) + i%4. Gate block nb
  // pairs with up block nb + NBW/2.
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = (wm + 2 * mb) * 32 + (lane & 31);
    if (m >= tile.rows) continue;
    const size_t crow = static_cast<size_t>(tile.row0 + m) * N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nloc = 8 * g + 4 * half;
      if (GATE_UP) {
#pragma unroll
        for (int nb = 0; nb < NBW / 2; ++nb) {
          const int n = tile.nt * 128 + wn * (NBW / 2) * 32 + nb * 32 + nloc;
          if (n < N) {
            float hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              hv[i] = silu_fast(acc[nb][mb][4 * g + i]) * acc[nb + NBW / 2][mb][4 * g + i];
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(Cv) + crow + n) =
                make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          }
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const int n = tile.nt * TW + wn * NBW * 32 + nb * 32 + nloc;
          if (n < N)
            *reinterpret_cast<float4*>(static_cast<float*>(Cv) + tile.ks * c_split + crow + n) =
                make_float4(acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                            acc[nb][mb][4 * g + 3]);
        }
      }
    }
  }
}

// Tall tiles: 384 permuted rows x 256 weight rows, 8 waves (two per SIMD) of
// 96 x 128 (3 x 4 accumulators of v_mfma_f32_32x32x16_bf16, 192 fp32 per
// lane; the wave's three 32-row blocks are tile blocks wm, wm + 4, wm + 8),
// two 80 KB LDS stages (the whole LDS). Each step moves 80 KB into the
// CU for 12.6 MFLOP, 17% fewer bytes per FLOP than the 256 x 256 tile; the
// cost is coarser row padding, so the host takes these tiles only when the
// experts average at least two tiles' worth of rows. The tiles of an XCD's
// last, at most half-full round run at half width (384 x 128, 96 x 64 per
// wave; see assign_tile's TAIL). Same swizzle, stages and epilogue as the
// 256 x 256 kernel. Which operand and
// which weight matrix each load instruction serves is fixed per unrolled
// index, so the compiler keeps the choice in scalar code (chosen at run
// time, the pointer selection went through scratch memory). KMASK: the
// reduction length is not a multiple of the step, so chunks past it read
// the zero page.
constexpr int TM3 = 384;              // permuted rows per tile
constexpr int STAGE_A3 = TM3 * TK * 2;  // 48 KB
constexpr int NW3 = 8;
constexpr int MBW = 3;                // 32-row token blocks per wave

template <bool GATE_UP, bool KMASK>
__global__ __launch_bounds__(NW3 * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void expert_gemm_tall_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_token,
                             const int32_t* __restrict__ offsets, int E,
                             const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, int N,
                             int K, void* __restrict__ Cv, int max_split, int n_cu,
                             size_t c_split, int32_t* __restrict__ split_out) {
  __shared__ __attribute__((aligned(1024))) char lds0a[STAGE_A3];
  __shared__ __attribute__((aligned(1024))) char lds0b[STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1a[STAGE_A3];
  __shared__ __attribute__((aligned(1024))) char lds1b[STAGE];
  auto buf = [&](int st, int op) -> char* {
    return st == 0 ? (op ? lds0b : lds0a) : (op ? lds1b : lds1a);
  };
  const int nN = GATE_UP ? (N + 127) / 128 : (N + TW - 1) / TW;
  Tile tile;
  const int nk = (K + TK - 1) / TK;
  const bool have = map_tile<TM3, true>(offsets, E, nN, max_split, n_cu, nk, &tile,
                                        reinterpret_cast<int*>(lds1a));
  __syncthreads();
  if (!GATE_UP && blockIdx.x == 0 && threadIdx.x == 0) *split_out = tile.S;
  if (!have) return;
  const int kbeg = tile.ks * nk / tile.S, kend = (tile.ks + 1) * nk / tile.S;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const char* a_base = reinterpret_cast<const char*>(A);
  const size_t wexp = static_cast<size_t>(tile.e) * N * K * 2;
  const char* g_base = reinterpret_cast<const char*>(B0) + wexp;
  const char* u_base = reinterpret_cast<const char*>(GATE_UP ? B1 : B0) + wexp;
  const char* zero = reinterpret_cast<const char*>(g_zero_page);
  const __amdgpu_buffer_rsrc_t a_rs = buffer_rsrc(a_base), g_rs = buffer_rsrc(g_base),
                               u_rs = buffer_rsrc(u_base);
  // (r >> 1) & 7 of every row a lane loads (see below) is (4*wave + l/16) & 7
  const int ch = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int xr = ((lane & 31) >> 1) & 7, half = lane >> 5;
  constexpr int JA = TM3 / 8 / NW3;  // 6 A load instructions per wave

  // The tile with NB 32-row weight blocks per wave: NB = 4 for a whole
  // column tile (256 weight rows), NB = 2 for a half one (128 rows; gate/up:
  // 64 gate rows, then the same rows of up).
  auto body = [&](auto nbc) __attribute__((always_inline)) {
    constexpr int NB = decltype(nbc)::value;
    constexpr int WR = 64 * NB;    // weight rows of the tile
    constexpr int IPW = JA + NB;   // load instructions per wave and stage
    const int n0 = GATE_UP ? tile.nt * 128 + (NB == 2 ? 64 * tile.half : 0)
                           : tile.nt * TW + (NB == 2 ? 128 * tile.half : 0);
    // instruction q = wave + 8 j: j < JA are A instructions (A rows
    // 8q .. 8q+7), j >= JA B instructions (B rows 8(wave + 8(j-JA)) ..; for
    // gate/up the first half of them are gate rows, the second half the same
    // rows of up). Lane l writes row r = 8*qq + l/8, slot l%8, holding chunk
    // (l%8) ^ ((r >> 1) & 7).
    uint32_t src_off[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const bool isA = j < JA;
      const int qq = isA ? wave + NW3 * j : wave + NW3 * (j - JA);
      const int r = qq * 8 + (lane >> 3);
      uint32_t row;
      if (isA) {
        const int rr = r < tile.rows ? r : r % tile.rows;
        row = GATE_UP ? static_cast<uint32_t>(sorted_token[tile.row0 + rr])
                      : static_cast<uint32_t>(tile.row0 + rr);
      } else {
        row = static_cast<uint32_t>(min(n0 + (GATE_UP ? (r & (WR / 2 - 1)) : r), N - 1));
      }
      src_off[j] = row * static_cast<uint32_t>(K) * 2u + ch * 16u;
    }
    auto is_up = [&](int j) { return GATE_UP && j >= JA + NB / 2; };
    // Load instruction j of step kt into stage st. Without KMASK every chunk
    // of a step lies inside K: a buffer load from the operand's resource.
    auto issue_j = [&](int kt, int st, int j, bool mask) __attribute__((always_inline)) {
      const int k0 = kt * TK;
      const uint32_t kb = static_cast<uint32_t>(k0) * 2u;
      const bool isA = j < JA;
      const int qq = isA ? wave + NW3 * j : wave + NW3 * (j - JA);
      char* dst = buf(st, isA ? 0 : 1) + qq * 1024;
      if (mask) {
        const char* base = isA ? a_base : (is_up(j) ? u_base : g_base);
        load_lds16(k0 + ch * 8 < K ? base + (src_off[j] + kb) : zero, dst);
      } else {
        buffer_load_lds16(isA ? a_rs : (is_up(j) ? u_rs : g_rs), src_off[j], kb, dst);
      }
    };
    int fa_off[MBW], fb_off[NB];
#pragma unroll
    for (int i = 0; i < MBW; ++i) fa_off[i] = ((wm + 4 * i) * 32 + (lane & 31)) * 128;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      // gate/up: blocks 0 .. NB/2-1 gate rows wn*WR/4 + 32i, then the same rows of up
      const int brow = GATE_UP ? (i / (NB / 2)) * (WR / 2) + wn * (WR / 4) + (i % (NB / 2)) * 32
                               : wn * (WR / 2) + i * 32;
      fb_off[i] = (brow + (lane & 31)) * 128;
    }
    f32x16 acc[NB][MBW];
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int y = 0; y < MBW; ++y)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[x][y][i] = 0.f;

    // One step on stage st: groups of one weight fragment times the three
    // token fragments (3 MFMAs). The fragments of group g+1 are read before the
    // MFMAs of group g, and the first half of the groups each issue a share of
    // the next step's loads, so the load instructions go out at the rate the
    // address unit takes them instead of stalling every wave at the start of
    // the step; the scheduling fences keep that order. In the last step the
    // loads re-read an in-range step into the idle stage, which keeps the
    // instruction stream free of branches.
    constexpr int kGroups = (TK / 16) * NB;
    constexpr int kLoadGroups = kGroups / 2;
    auto run = [&](auto mac) __attribute__((always_inline)) {
      constexpr int MA = decltype(mac)::value;  // token blocks of this wave with real rows
      auto step = [&](int kt, int st) __attribute__((always_inline)) {
        const int kload = min(kt + 1, nk - 1);
        auto rd = [&](int op, int off, int s) __attribute__((always_inline)) {
          return *reinterpret_cast<const bf16x8*>(buf(st, op) + off + (((2 * s + half) ^ xr) << 4));
        };
        bf16x8 fa[2][MA], fb[2];
#pragma unroll
        for (int i = 0; i < MA; ++i) fa[0][i] = rd(0, fa_off[i], 0);
        fb[0] = rd(1, fb_off[0], 0);
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          const int s = g / NB, nb = g % NB, ca = s & 1, cb = g & 1;
          if (g + 1 < kGroups) {
            const int s1 = (g + 1) / NB, nb1 = (g + 1) % NB;
            if (nb1 == 0) {
#pragma unroll
              for (int i = 0; i < MA; ++i) fa[ca ^ 1][i] = rd(0, fa_off[i], s1);
            }
            fb[cb ^ 1] = rd(1, fb_off[nb1], s1);
          }
          if (g < kLoadGroups) {
#pragma unroll
            for (int j = g * IPW / kLoadGroups; j < (g + 1) * IPW / kLoadGroups; ++j)
              issue_j(kload, st ^ 1, j, KMASK);
          }
#pragma unroll
          for (int mb = 0; mb < MA; ++mb)
            acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cb], fa[ca][mb], acc[nb][mb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      const int nsteps = kend - kbeg;
      if (nsteps > 0) {
#pragma unroll
        for (int j = 0; j < IPW; ++j) issue_j(kbeg, 0, j, true);
      }
      for (int p = 0; p + 1 < nsteps; p += 2) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          step(kbeg + p + r, r);
        }
      }
      if (nsteps & 1) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        step(kend - 1, 0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // Token block i of this wave is tile block wm + 4i (32 rows each), so the
    // blocks past the tile's rows (an expert's last row tile) fall on every
    // wave, and so on every SIMD, about equally. A wave runs the step with
    // only its MA blocks that hold rows: the MFMAs of padding blocks are
    // skipped (about a quarter of an expert's last tile at the prefill
    // shape). Every variant loads the same data and meets the same barriers.
    const int nblk = (tile.rows + 31) / 32;
    const int nact = nblk >= wm + 9 ? 3 : (nblk >= wm + 5 ? 2 : 1);
    if (nact == 3)
      run(IntC<3>{});
    else if (nact == 2)
      run(IntC<2>{});
    else
      run(IntC<1>{});

    // acc[nb][mb] element i: token row (wm + 4 mb)*32 + lane%32, weight-tile
    // row (block nb) + 8*(i/4) + 4*(lane/32) + i%4; gate block nb pairs with
    // up block nb + NB/2.
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      const int m = (wm + 4 * mb) * 32 + (lane & 31);
      if (m >= tile.rows) continue;
      const size_t crow = static_cast<size_t>(tile.row0 + m) * N;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nloc = 8 * g + 4 * half;
        if (GATE_UP) {
#pragma unroll
          for (int nb = 0; nb < NB / 2; ++nb) {
            const int n = n0 + wn * (WR / 4) + nb * 32 + nloc;
            if (n < N) {
              float hv[4];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                hv[i] = silu_fast(acc[nb][mb][4 * g + i]) * acc[nb + NB / 2][mb][4 * g + i];
              *reinterpret_cast<uint2*>(static_cast<bf16_t*>(Cv) + crow + n) =
                  make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
            }
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int n = n0 + wn * (WR / 2) + nb * 32 + nloc;
            if (n < N)
              *reinterpret_cast<float4*>(static_cast<float*>(Cv) + tile.ks * c_split + crow + n) =
                  make_float4(acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                              acc[nb][mb][4 * g + 3]);
          }
        }
      }
    }
  };
  if (tile.half < 0)
    body(IntC<4>{});
  else
    body(IntC<2>{});
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
    const float* __restrict__ B1, int N, int K, float* __restrict__ C,
    int32_t* __restrict__ split_out) {
  const int r = blockIdx.x;
  const int n = blockIdx.y * 256 + threadIdx.x;
  if (!GATE_UP && split_out && r == 0 && n == 0) *split_out = 1;
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

// upper bound on sum_e ceil(M_e / BM) over the experts' row counts M_e,
// times the column tiles and splits, rounded up to whole XCD rounds
#ifndef MOE_GEMM_WAVES
#define MOE_GEMM_WAVES 8
#endif
constexpr int kWaves = MOE_GEMM_WAVES;

unsigned tile_grid(int rows, int E, int BM, int nN, int splits) {
  const long long max_mt = rows / BM + (rows < E ? rows : E);
  const long long g = max_mt * nN * splits;
  return static_cast<unsigned>((g + kXcds - 1) / kXcds * kXcds);
}

// tile_grid plus the half-width tail tiles' extra slots (assign_tile's TAIL)
unsigned tall_grid(int rows, int E, int nN, int splits, int n_cu) {
  return tile_grid(rows, E, TM3, nN, splits) + (n_cu / kXcds / 2) * kXcds;
}

// Tall tiles pay off once the experts average two tiles' worth of rows
// (their padding is then at most a third of a tile over two or more).
bool use_tall_tiles(int rows, int E) { return rows >= 2 * TM3 * E; }

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  return n;
}

}  // namespace

moe_status launch_gate_up(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                          const void* w_gate, const void* w_up, int T, int d, int ffn, int E,
                          int k, moe_dtype dt, void* h, hipStream_t s) {
  const int rows = T * k;
  if (dt == MOE_F32) {
    expert_gemm_f32_kernel<true><<<dim3(rows, (ffn + 255) / 256), 256, 0, s>>>(
        static_cast<const float*>(x), sorted_token, offsets, E, static_cast<const float*>(w_gate),
        static_cast<const float*>(w_up), ffn, d, static_cast<float*>(h), nullptr);
    return launch_status();
  }
  if (use_stream_path(rows, E))
    return launch_gate_up_stream(x, sorted_token, offsets, w_gate, w_up, d, ffn, E, rows, h, s);
  if (use_tall_tiles(rows, E)) {
    auto kern = d % TK ? expert_gemm_tall_kernel<true, true> : expert_gemm_tall_kernel<true, false>;
    const int ncu = cu_count();
    kern<<<tall_grid(rows, E, (ffn + 127) / 128, 1, ncu), NW3 * 64, 0, s>>>(
        static_cast<const bf16_t*>(x), sorted_token, offsets, E, static_cast<const bf16_t*>(w_gate),
        static_cast<const bf16_t*>(w_up), ffn, d, h, 1, ncu, 0, nullptr);
    return launch_status();
  }
  auto kern = d % TK ? expert_gemm_bf16_kernel<true, kWaves, true> : expert_gemm_bf16_kernel<true, kWaves, false>;
  kern<<<tile_grid(rows, E, TM, (ffn + 127) / 128, 1), kWaves * 64, 0, s>>>(
      static_cast<const bf16_t*>(x), sorted_token, offsets, E, static_cast<const bf16_t*>(w_gate),
      static_cast<const bf16_t*>(w_up), ffn, d, h, 1, cu_count(), 0, nullptr);
  return launch_status();
}

moe_status launch_down(const void* h, const int32_t* offsets, const void* w_down, int T, int d,
                       int ffn, int E, int k, moe_dtype dt, float* y, int32_t* split,
                       hipStream_t s) {
  const int rows = T * k;
  if (dt == MOE_F32) {
    expert_gemm_f32_kernel<false><<<dim3(rows, (d + 255) / 256), 256, 0, s>>>(
        static_cast<const float*>(h), nullptr, offsets, E, static_cast<const float*>(w_down),
        nullptr, d, ffn, y, split);
    return launch_status();
  }
  if (use_stream_path(rows, E)) return launch_down_stream(h, offsets, w_down, d, ffn, E, rows, y, split, s);
  if (use_tall_tiles(rows, E)) {
    auto kern = ffn % TK ? expert_gemm_tall_kernel<false, true> : expert_gemm_tall_kernel<false, false>;
    const int ncu = cu_count();
    kern<<<tall_grid(rows, E, (d + TW - 1) / TW, kMaxDownSplit, ncu), NW3 * 64, 0, s>>>(
        static_cast<const bf16_t*>(h), nullptr, offsets, E, static_cast<const bf16_t*>(w_down),
        nullptr, d, ffn, y, kMaxDownSplit, ncu, static_cast<size_t>(rows) * d, split);
    return launch_status();
  }
  auto kern = ffn % TK ? expert_gemm_bf16_kernel<false, kWaves, true> : expert_gemm_bf16_kernel<false, kWaves, false>;
  kern<<<tile_grid(rows, E, TM, (d + TW - 1) / TW, kMaxDownSplit), kWaves * 64, 0, s>>>(
      static_cast<const bf16_t*>(h), nullptr, offsets, E, static_cast<const bf16_t*>(w_down),
      nullptr, d, ffn, y, kMaxDownSplit, cu_count(), static_cast<size_t>(rows) * d, split);
  return launch_status();
}

}  // namespace moe
