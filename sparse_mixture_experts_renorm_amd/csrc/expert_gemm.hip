// Grouped expert GEMMs over the permuted tokens.
//
// Expert e (axonml-nn Expert::forward; skills page SwiGLU) on its rows X_e:
//   h = SiLU(X_e W_g[e]^T) * (X_e W_u[e]^T)      (gate/up pass, SiLU on gate)
//   y = h W_d[e]^T                               (down pass)
// X_e are the rows sorted_token[offsets[e] .. offsets[e+1]) of x: the gather
// is done by the tile loads, so X_e is never written out. h and y are stored
// in permuted-row order, row offsets[e] + r for the r-th token of expert e.
// h is bf16 (the down pass multiplies it on the bf16 MFMA); y keeps 16
// significant bits (the 24-bit format of common.h), because rounding y to
// bf16 as well would spend about half of the 2e-2 x RMS error budget of bf16
// workloads on top of h's rounding.
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
// accumulators hold 4 consecutive output columns of one row. The epilogues
// turn that layout into whole rows per store instruction: through a per-wave
// LDS tile (y of both tile shapes, h of the 256 x 256 tiles) or, for h of
// the tall tiles, by an exchange between lane pairs.
//
// Tile schedule: the host sizes the grid from an upper bound on the tile
// count; each workgroup reads the per-expert offsets, counts the real tiles
// and maps itself to (expert, row tile, column tile). An expert's rows are
// cut into ceil(rows / tile height) row tiles of nearly equal height (whole
// 32-row blocks), so little of any tile is padding and the row tiles of one
// weight tile take the same time. Workgroups are handed
// to the 8 XCDs round-robin, so consecutive tiles of the schedule are given
// to workgroups on the same XCD (sharing its L2): each XCD takes a
// contiguous eighth of the tile list (of each of the two lists, heavy and
// light experts: see assign_tile). Inside an expert (and split part) the
// list runs over column tiles and, for each, over its row tiles, so the row
// tiles that share a weight tile run side by side and the weights go
// through L2 about once (with the row tiles of one column tile spread over
// rounds instead, the L2 fetched a third more).
#include "common.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kXcds = 8;

struct Tile {
  int e, row0, rows, nt;
  int ks, S;  // split of the reduction dimension: this tile computes part ks of S
  int half;   // -1: the whole column tile; 0 or 1: that half of its weight rows
};

// Row tiles of BM rows per expert, ceil(M_e / BM) (M_e = offsets[e+1] -
// offsets[e]); experts with at most min_rows rows get none (the
// weight-streaming kernel takes them).
__host__ __device__ inline int expert_row_tiles(int m, int BM, int min_rows) {
  return m > min_rows ? (m + BM - 1) / BM : 0;
}
// An expert whose rows fill at most a third of a tile is light: its one
// tile takes about 60% of a full tile's time (the loads of a whole tile,
// one token block of MFMAs per wave), so the tile list keeps the light
// experts' tiles apart and every XCD gets its share of both kinds.
__host__ __device__ inline bool light_expert(int m, int BM) { return 3 * m <= BM; }
// The row-tile prefixes, heavy experts in pref[0 .. E] and light ones in
// pref[E+1 .. 2E+1]: pref[e] = sum over heavy e' < e of their row tiles, and
// likewise for the light ones. Serial form, for the host; the kernels build
// the same arrays with one wave (map_tile).
template <int BM>
__host__ __device__ inline void row_tile_prefix(const int32_t* __restrict__ offsets, int E,
                                                int* pref, int min_rows = 0) {
  int* pl = pref + E + 1;
  pref[0] = pl[0] = 0;
  for (int e = 0; e < E; ++e) {
    const int m = offsets[e + 1] - offsets[e], t = expert_row_tiles(m, BM, min_rows);
    const bool light = light_expert(m, BM);
    pref[e + 1] = pref[e] + (light ? 0 : t);
    pl[e + 1] = pl[e] + (light ? t : 0);
  }
}

// The split count for `base` tiles per part (see assign_tile): fewest rounds
// per part, counted in whole tiles, with at least kMinSplitSteps of the nk
// reduction steps in each part.
__host__ __device__ inline int choose_split(int base, int max_split, int n_cu, int nk) {
  int S = 1, best_rounds = (base + n_cu - 1) / n_cu;  // rounds of S-tiles
  for (int c = 2; c <= max_split && c * kMinSplitSteps <= nk; ++c) {
    const int rounds = (base * c + n_cu - 1) / n_cu;
    if (rounds * S < best_rounds * c) {  // rounds/c < best_rounds/S
      S = c;
      best_rounds = rounds;
    }
  }
  return S;
}

// Tile of workgroup `block` among tiles of BM rows, given the experts' row
// offsets and their row-tile prefixes pref [2E+2]: res = {expert (-1: none),
// first permuted row, rows, column tile, split part, split count S, half
// (-1: whole column tile; 0 or 1: that half of its weight rows)}.
// There are two tile lists, of the heavy experts and of the light ones;
// each is cut into 8 contiguous ranges of equal count, and XCD x runs its
// range of the heavy list, then its range of the light one (so no XCD gets
// the light tiles of all of them while the others run only heavy tiles,
// and the heavy tiles' rounds keep their shared operands in L2; light
// tiles spread among the heavy ones were no faster and fetched 30% more).
// A list runs over its experts in order; inside an expert over the
// split parts, and inside a part over column tiles and, for each, over its
// row tiles -- or, when the expert has more rows than the operation has
// weight rows (wrows), over row tiles and, for each, over its column tiles.
// The tiles that run side by side on an XCD then share the larger operand
// through its L2, and the smaller one is what is read again per round.
// With max_split > 1 the reduction dimension may be cut into S <= max_split
// parts, each a separate tile whose partial result goes to its own output
// slice; S is chosen from the real tile count (choose_split; shorter parts
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
                                            int wrows, int block, int* res) {
  const int* pl = pref + E + 1;
  const int base_h = pref[E] * nN, base_l = pl[E] * nN;  // tiles of one split part
  const int S = choose_split(base_h + base_l, max_split, n_cu, nk);
  const int per_h = (base_h * S + kXcds - 1) / kXcds, per_l = (base_l * S + kXcds - 1) / kXcds;
  const int xcd = block % kXcds, slot = block / kXcds;
  auto share = [&](int base, int per) {  // tiles of one list on this XCD
    const int c = base * S - xcd * per;
    return c < 0 ? 0 : (c > per ? per : c);
  };
  const int cnt_h = share(base_h, per_h), cnt_l = share(base_l, per_l), cnt = cnt_h + cnt_l;
  int li = -1, half = -1;  // position in this XCD's order
  if (TAIL) {
    const int cpx = n_cu / kXcds > 1 ? n_cu / kXcds : 1, r = cnt % cpx;
    const int nfull = (r > 0 && 2 * r <= cpx) ? cnt - r : cnt;
    if (slot < nfull) {
      li = slot;
    } else if (slot < nfull + 2 * (cnt - nfull)) {
      li = nfull + (slot - nfull) / 2;
      half = (slot - nfull) & 1;
    }
  } else if (slot < cnt) {
    li = slot;
  }
  res[0] = -1;
  res[5] = S;
  res[6] = half;
  if (li < 0) return;
  // the XCD's heavy tiles first, then its light ones
  const bool light = li >= cnt_h;
  const int* pc = light ? pl : pref;
  int L = light ? xcd * per_l + (li - cnt_h) : xcd * per_h + li;
  // the expert of tile L of its list: the first e with pc[e+1] * nN * S > L
  const int per_row_tile = nN * S;
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pc[mid + 1] * per_row_tile > L) hi = mid; else lo = mid + 1;
  }
  const int e = lo;
  L -= pc[e] * per_row_tile;
  const int mt = pc[e + 1] - pc[e], m = offsets[e + 1] - offsets[e];
  const int te = mt * nN;  // tiles of one split part of expert e
  const int ks = L / te;
  L -= ks * te;
  // The expert's rows are cut into its mt row tiles as evenly as 32-row
  // blocks allow (block counts differ by at most one, each at most BM/32):
  // the tiles that share a weight tile then take about the same time and
  // stay in step, and no tile is mostly padding.
  const bool row_outer = m > wrows;
  const int mi = row_outer ? L / nN : L % mt, nb = (m + 31) / 32;
  const int b0 = static_cast<int>(static_cast<long long>(mi) * nb / mt);
  const int b1 = static_cast<int>(static_cast<long long>(mi + 1) * nb / mt);
  res[0] = e;
  res[1] = offsets[e] + 32 * b0;
  res[2] = (32 * b1 < m ? 32 * b1 : m) - 32 * b0;
  res[3] = row_outer ? L % nN : L / mt;
  res[4] = ks;
}

// LDS the tile map needs: the seven results, then the two prefixes.
constexpr int kMapLdsInts = 8 + 2 * (kMaxExperts + 1);
static_assert(kMaxExperts <= 4 * kWave, "map_tile sums four experts per lane");

// Map this workgroup to its tile; returns false if it has none. Wave 0
// builds the row-tile prefix in LDS (lane l sums experts 4l .. 4l+3, a wave
// scan adds up the lanes: one memory round trip for any E <= 256), then
// thread 0 runs assign_tile on it. s_map: kMapLdsInts ints of LDS.
template <int BM, bool TAIL = false>
__device__ bool map_tile(const int32_t* __restrict__ offsets, int E, int nN, int max_split,
                         int n_cu, int nk, int min_rows, int wrows, Tile* out, int* s_map) {
  int* pref = s_map + 8;
  int* pl = pref + E + 1;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int ch[4], cl[4], sh = 0, sl = 0;  // row tiles of heavy / light experts
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      const int m = e < E ? offsets[e + 1] - offsets[e] : 0;
      const int t = expert_row_tiles(m, BM, min_rows);
      const bool light = light_expert(m, BM);
      ch[q] = light ? 0 : t;
      cl[q] = light ? t : 0;
      sh += ch[q];
      sl += cl[q];
    }
    int ih = sh, il = sl;
#pragma unroll
    for (int dl = 1; dl < kWave; dl <<= 1) {
      const int v = __shfl_up(ih, dl, kWave);
      if (lane >= dl) ih += v;
    }
    if (__any(sl > 0)) {  // the light list's scan only when it has tiles
#pragma unroll
      for (int dl = 1; dl < kWave; dl <<= 1) {
        const int v = __shfl_up(il, dl, kWave);
        if (lane >= dl) il += v;
      }
    }
    int rh = ih - sh, rl = il - sl;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      if (e < E) {
        pref[e] = rh;
        pl[e] = rl;
      }
      rh += ch[q];
      rl += cl[q];
    }
    if (lane == kWave - 1) {
      pref[E] = ih;
      pl[E] = il;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0)
    assign_tile<BM, TAIL>(offsets, pref, E, nN, max_split, n_cu, nk, wrows, blockIdx.x, s_map);
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
// !GATE_UP: A = h (rows in order), weights = w_down, C = y (24-bit); the
// reduction may be split (see assign_tile): part ks writes C + ks * c_split,
// and workgroup 0 stores the split count S in *split_out.
// NW waves per workgroup: 4 (wave tile 128 x 128, one wave per SIMD) or 8
// (wave tile 128 x 64, two waves per SIMD, so one wave's MFMAs run while the
// other waits to issue its loads).
// TWO (down pass only): h is given as two bf16 terms, h = A + Alo (A its
// rounding to bf16, Alo the rounding of the remainder), and y = A W^T + Alo
// W^T. A tile then holds 128 rows of y: tile rows 0-127 of the token operand
// are those rows of A, tile rows 128-255 the same rows of Alo, and the
// accumulators of token block b and b + 4 (the same output rows) are added
// in the epilogue. Same loads, MFMAs and barriers per step as one term, so
// the pass takes about twice as long for the same rows.
// GATE_UP with Clo non-null writes that second term of h as well.
template <bool GATE_UP, int NW, bool KMASK, bool TWO = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void expert_gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Alo,
                             const int32_t* __restrict__ sorted_token,
                             const int32_t* __restrict__ offsets, int E,
                             const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, int N,
                             int K, void* __restrict__ Cv, bf16_t* __restrict__ Clo, int max_split,
                             int n_cu, size_t c_split, int32_t* __restrict__ split_out,
                             int min_rows) {
  static_assert(!(TWO && GATE_UP), "two terms of h are an operand of the down pass only");
  constexpr int BM = TWO ? TM / 2 : TM;  // output rows per tile
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
  const bool have = map_tile<BM>(offsets, E, nN, max_split, n_cu, nk, min_rows, GATE_UP ? 2 * N : N,
                                 &tile, s_map);
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
  // with TWO, the waves that load tile rows 128-255 read the second term
  const char* a_base = reinterpret_cast<const char*>(TWO && wave * IPW * 8 >= BM ? Alo : A);
  const size_t wexp = static_cast<size_t>(tile.e) * N * K * 2;
  auto a_row_off = [&](int r) -> uint32_t {
    if (TWO) r &= BM - 1;
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
  const int nact = TWO ? 4 : (nblk - wm >= 7 ? 4 : (nblk - wm >= 5 ? 3 : (nblk - wm >= 3 ? 2 : 1)));
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
  // With TWO, token block i < 2 of this wave is output rows (wm + 2i)*32 ..
  // and block i + 2 holds the second term of the same rows.
  // Each 32-row block goes out through a per-wave LDS tile, as whole rows
  // per store instruction (from the accumulator layout one instruction
  // wrote 16 or 32 bytes into each of 32 rows). Tile rows are padded so
  // that the LDS writes are free of bank conflicts.
  __syncthreads();  // every wave is done reading the last stage
  if constexpr (GATE_UP) {
    static_assert(NBW == 2, "one gate block of 32 columns per wave");
    constexpr int kStgH = 40;  // bf16 per tile row
    bf16_t* stg = reinterpret_cast<bf16_t*>(lds0a) + wave * (32 * kStgH);
    const int n = tile.nt * 128 + wn * 32 + (lane & 3) * 8;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int mbase = (wm + 2 * mb) * 32;
      if (mbase >= tile.rows) continue;
      uint32_t hi[4][2], lo[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = silu_fast(acc[0][mb][4 * g + i]) * acc[1][mb][4 * g + i];
        hi[g][0] = pack_bf16x2(hv[0], hv[1]);
        hi[g][1] = pack_bf16x2(hv[2], hv[3]);
        lo[g][0] = pack_bf16x2(hv[0] - __uint_as_float(hi[g][0] << 16),
                               hv[1] - __uint_as_float(hi[g][0] & 0xFFFF0000u));
        lo[g][1] = pack_bf16x2(hv[2] - __uint_as_float(hi[g][1] << 16),
                               hv[3] - __uint_as_float(hi[g][1] & 0xFFFF0000u));
      }
#pragma unroll
      for (int term = 0; term < 2; ++term) {
        if (term == 1 && !Clo) break;
        bf16_t* dst = term == 0 ? static_cast<bf16_t*>(Cv) : Clo;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(stg + (lane & 31) * kStgH + 8 * g + 4 * half) =
              term == 0 ? make_uint2(hi[g][0], hi[g][1]) : make_uint2(lo[g][0], lo[g][1]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int rr = (lane >> 2) + 16 * q, m = mbase + rr;
          const uint4 v = *reinterpret_cast<const uint4*>(stg + rr * kStgH + (lane & 3) * 8);
          if (m < tile.rows && n < N)
            *reinterpret_cast<uint4*>(dst + static_cast<size_t>(tile.row0 + m) * N + n) = v;
        }
      }
    }
  } else {
    constexpr int kStg = 36;  // floats per tile row
    float* stg = reinterpret_cast<float*>(wave < 4 ? lds0a : lds1a) + (wave & 3) * (32 * kStg);
    char* Cb = static_cast<char*>(Cv) + tile.ks * c_split * 3;  // 24-bit y
#pragma unroll
    for (int mb = 0; mb < (TWO ? 2 : 4); ++mb) {
      const int mbase = (wm + 2 * mb) * 32;
      if (mbase >= tile.rows) continue;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] = TWO ? acc[nb][mb][4 * g + i] + acc[nb][mb + 2][4 * g + i] : acc[nb][mb][4 * g + i];
          *reinterpret_cast<float4*>(stg + (lane & 31) * kStg + 8 * g + 4 * half) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
        const int n = tile.nt * TW + wn * NBW * 32 + nb * 32 + (lane & 7) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = (lane >> 3) + 8 * q, m = mbase + rr;
          const float4 v = *reinterpret_cast<const float4*>(stg + rr * kStg + (lane & 7) * 4);
          if (m < tile.rows && n < N)
            *reinterpret_cast<uint3*>(Cb + (static_cast<size_t>(tile.row0 + m) * N + n) * 3) =
                pack_f24x4(v.x, v.y, v.z, v.w);
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
// wave; see assign_tile's TAIL), except in a down pass given a part table:
// there every tile keeps its whole reduction and those tail tiles run at
// full width with their reduction in two halves (two partial sums; the
// table tells the combine which rows and 256-column tiles have two), which
// keeps the tail's bytes per FLOP and saves a tile boundary per CU and the
// second partial sum of the other tiles against a uniform split in two
// (prefill down pass 791 -> 767 us, combine 52 -> 41 us). Same swizzle,
// stages and epilogue as the
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

// Stores 32 columns (from n) of one row of h, held as an MFMA 32x32 block's
// accumulator layout: lane l has columns 8g + 4(l/32) + 0..3 of each group
// g as two packed bf16 pairs in w[g]. Lanes l and l^32 (same row) swap a
// group each (ds_bpermute, no LDS memory), so that each lane stores 8 whole
// columns: 16 contiguous bytes per lane and 32 per row pair of stores.
__device__ __forceinline__ void store_h_pairs(bf16_t* __restrict__ dst, size_t crow, int n, int N,
                                              bool ok, int half, int partner,
                                              const uint32_t w[4][2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int g0 = 2 * p, g1 = 2 * p + 1;
    // the lower half keeps group g0 and takes its partner's share of g0;
    // the upper half keeps g1
    const uint32_t s0 = half ? w[g0][0] : w[g1][0], s1 = half ? w[g0][1] : w[g1][1];
    const uint32_t r0 = __builtin_amdgcn_ds_bpermute(partner, static_cast<int>(s0));
    const uint32_t r1 = __builtin_amdgcn_ds_bpermute(partner, static_cast<int>(s1));
    const uint4 v = half ? make_uint4(r0, r1, w[g1][0], w[g1][1])
                         : make_uint4(w[g0][0], w[g0][1], r0, r1);
    const int c = n + 8 * (half ? g1 : g0);
    if (ok && c < N) *reinterpret_cast<uint4*>(dst + crow + c) = v;
  }
}

template <bool GATE_UP, bool KMASK>
__global__ __launch_bounds__(NW3 * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void expert_gemm_tall_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_token,
                             const int32_t* __restrict__ offsets, int E,
                             const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1, int N,
                             int K, void* __restrict__ Cv, bf16_t* __restrict__ Clo, int max_split,
                             int n_cu, size_t c_split, int32_t* __restrict__ split_out,
                             int min_rows, uint8_t* __restrict__ parts) {
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
  const bool have = map_tile<TM3, true>(offsets, E, nN, max_split, n_cu, nk, min_rows,
                                        GATE_UP ? 2 * N : N, &tile, reinterpret_cast<int*>(lds1a));
  __syncthreads();
  // Down pass with a part table: whole tiles keep their reduction in one
  // part, and the tail tiles an XCD's last round would run as half-width
  // tiles run whole-width with their reduction in two halves instead; each
  // tile records its part count per row in parts.
  const bool ksplit = !GATE_UP && parts != nullptr;
  if (!GATE_UP && blockIdx.x == 0 && threadIdx.x == 0) *split_out = ksplit ? 0 : tile.S;
  if (!have) return;
  if (ksplit && tile.half >= 0) {
    tile.ks = tile.half;
    tile.S = 2;
    tile.half = -1;
  }
  if (ksplit && static_cast<int>(threadIdx.x) < tile.rows)
    parts[static_cast<size_t>(tile.row0 + threadIdx.x) * nN + tile.nt] = static_cast<uint8_t>(tile.S);
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
    if constexpr (GATE_UP) {
      // h (bf16): lanes l and l^32 hold the two halves of 8 columns of one
      // row; one exchange between them (ds_bpermute, no LDS memory) gives
      // each lane 8 whole columns, so each store instruction writes 32
      // contiguous bytes into each of 32 rows, in half as many stores.
      const int partner = (lane ^ 32) << 2;
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        const int m = (wm + 4 * mb) * 32 + (lane & 31);
        const size_t crow = static_cast<size_t>(tile.row0 + m) * N;
#pragma unroll
        for (int nb = 0; nb < NB / 2; ++nb) {
          float hv[4][4];
          uint32_t w[4][2];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              hv[g][i] = silu_fast(acc[nb][mb][4 * g + i]) * acc[nb + NB / 2][mb][4 * g + i];
            w[g][0] = pack_bf16x2(hv[g][0], hv[g][1]);
            w[g][1] = pack_bf16x2(hv[g][2], hv[g][3]);
          }
          const bool ok = m < tile.rows;
          store_h_pairs(static_cast<bf16_t*>(Cv), crow, n0 + wn * (WR / 4) + nb * 32, N, ok, half,
                        partner, w);
          if (Clo) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const uint32_t p0 = w[g][0], p1 = w[g][1];
              w[g][0] = pack_bf16x2(hv[g][0] - __uint_as_float(p0 << 16),
                                    hv[g][1] - __uint_as_float(p0 & 0xFFFF0000u));
              w[g][1] = pack_bf16x2(hv[g][2] - __uint_as_float(p1 << 16),
                                    hv[g][3] - __uint_as_float(p1 & 0xFFFF0000u));
            }
            store_h_pairs(Clo, crow, n0 + wn * (WR / 4) + nb * 32, N, ok, half, partner, w);
          }
        }
      }
    } else {
      // y (24-bit format): each 32 x 32 block of the wave's accumulators goes
      // through a per-wave LDS tile and out as 8 rows x 96 contiguous bytes
      // per store instruction (stored straight from the accumulator layout,
      // one instruction wrote 32 bytes into each of 32 rows). Rows of the tile
      // are kStg floats apart, which keeps both LDS passes free of bank
      // conflicts but for one 2-way group.
      constexpr int kStg = 36;
      __syncthreads();  // every wave is done reading the last stage
      float* stg = reinterpret_cast<float*>(lds0a) + wave * (32 * kStg);
      char* Cb = static_cast<char*>(Cv) + tile.ks * c_split * 3;  // 24-bit y
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        const int mbase = (wm + 4 * mb) * 32;
        if (mbase >= tile.rows) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(stg + (lane & 31) * kStg + 8 * g + 4 * half) =
                make_float4(acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                            acc[nb][mb][4 * g + 3]);
          const int n = n0 + wn * (WR / 2) + nb * 32 + (lane & 7) * 4;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int rr = (lane >> 3) + 8 * q, m = mbase + rr;
            const float4 v = *reinterpret_cast<const float4*>(stg + rr * kStg + (lane & 7) * 4);
            if (m < tile.rows && n < N)
              *reinterpret_cast<uint3*>(Cb + (static_cast<size_t>(tile.row0 + m) * N + n) * 3) =
                  pack_f24x4(v.x, v.y, v.z, v.w);
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
// fp32 path: the same grouped GEMMs on the fp32 MFMA (v_mfma_f32_32x32x2_f32,
// fp32 products and accumulation). 128 x 128 tiles (gate/up: 64 gate rows
// and the same 64 up rows, giving 64 columns of h; down: 128 columns of y),
// scheduled by the same device-side tile map as the bf16 kernels (one
// split part: y is a single fp32 partial). Four waves, each 64 token rows x
// 64 weight rows: 2 x 2 accumulators of 32 x 32. The reduction moves in
// steps of 16 through two LDS stages filled from registers (each thread
// loads 16 bytes of two A rows and two B rows per step, stored after the
// step's MFMAs); LDS rows are 16 floats padded to 20, so the 16-byte
// fragment reads of 16 lanes (16 rows, 80 bytes apart) touch 64 distinct
// banks. In the MFMA for sub-step s, lane l supplies reduction index
// 8*(l/32) + s of its row (for both operands), so each lane reads its 8
// values of a step with two 16-byte reads.
constexpr int TMF = 128;           // token rows and weight rows per fp32 tile
constexpr int TKF = 16;            // reduction step (fp32 elements)
constexpr int LDF = TKF + 4;       // LDS row stride (floats)
typedef float f32x16f __attribute__((ext_vector_type(16)));

template <bool GATE_UP>
__global__ __launch_bounds__(256) void expert_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ sorted_token,
    const int32_t* __restrict__ offsets, int E, const float* __restrict__ B0,
    const float* __restrict__ B1, int N, int K, float* __restrict__ C, int n_cu,
    int32_t* __restrict__ split_out) {
  __shared__ __attribute__((aligned(16))) float sa[2][TMF * LDF];
  __shared__ __attribute__((aligned(16))) float sb[2][TMF * LDF];
  __shared__ int s_map[kMapLdsInts];
  const int nN = GATE_UP ? (N + 63) / 64 : (N + TMF - 1) / TMF;
  const int nk = K / TKF;  // K is a multiple of 16
  Tile tile;
  const bool have = map_tile<TMF>(offsets, E, nN, 1, n_cu, nk, 0, GATE_UP ? 2 * N : N, &tile, s_map);
  if (!GATE_UP && blockIdx.x == 0 && threadIdx.x == 0) *split_out = 1;
  if (!have) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // weight rows of the tile: gate/up rows 0-63 are gate rows n0 .. n0+63,
  // rows 64-127 the same rows of up; down rows are n0 + r
  const int n0 = GATE_UP ? tile.nt * 64 : tile.nt * TMF;
  const size_t wexp = static_cast<size_t>(tile.e) * N * K;
  // loads: thread t moves 16 bytes (4 floats, chunk t % 4) of rows t/4 and
  // t/4 + 64 of each operand per step
  const int lr = tid >> 2, lc = (tid & 3) * 4;
  const float* ap[2];
  const float* bp[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = lr + 64 * h;
    const int rr = r < tile.rows ? r : r % tile.rows;  // past the rows: repeat a valid one
    const size_t arow = GATE_UP ? static_cast<size_t>(sorted_token[tile.row0 + rr])
                                : static_cast<size_t>(tile.row0 + rr);
    ap[h] = A + arow * K + lc;
    const int n = min(n0 + (GATE_UP ? (r & 63) : r), N - 1);
    bp[h] = ((GATE_UP && r >= 64) ? B1 : B0) + wexp + static_cast<size_t>(n) * K + lc;
  }
  float4 ra[2], rb[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra[h] = *reinterpret_cast<const float4*>(ap[h] + kt * TKF);
      rb[h] = *reinterpret_cast<const float4*>(bp[h] + kt * TKF);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<float4*>(&sa[st][(lr + 64 * h) * LDF + lc]) = ra[h];
      *reinterpret_cast<float4*>(&sb[st][(lr + 64 * h) * LDF + lc]) = rb[h];
    }
  };
  // fragments: token block mb of the wave is tile rows wm*64 + 32 mb + l%32;
  // weight block nb: gate/up nb = 0 gate rows wn*32 + l%32, nb = 1 the same
  // rows of up (tile rows 64 + ...); down rows wn*64 + 32 nb + l%32
  const int kh = (lane >> 5) * 8;
  int fa[2], fb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    fa[i] = (wm * 64 + 32 * i + (lane & 31)) * LDF + kh;
    const int brow = GATE_UP ? 64 * i + wn * 32 + (lane & 31) : wn * 64 + 32 * i + (lane & 31);
    fb[i] = brow * LDF + kh;
  }
  f32x16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  gload(0);
  lstore(0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    __syncthreads();  // stage st written; stage st ^ 1 no longer read
    if (kt + 1 < nk) gload(kt + 1);
    float4 wa[2][2], tb[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        wa[i][q] = *reinterpret_cast<const float4*>(&sb[st][fb[i] + 4 * q]);
        tb[i][q] = *reinterpret_cast<const float4*>(&sa[st][fa[i] + 4 * q]);
      }
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const int q = s8 >> 2, c = s8 & 3;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[nb][q][c], tb[mb][q][c],
                                                            acc[nb][mb], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(st ^ 1);
  }

  // acc[nb][mb] element i: token row wm*64 + 32 mb + l%32, weight-tile row
  // (block nb) + 8*(i/4) + 4*(l/32) + i%4: four consecutive columns per group
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = wm * 64 + 32 * mb + (lane & 31);
    if (m >= tile.rows) continue;
    float* crow = C + static_cast<size_t>(tile.row0 + m) * N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j = 8 * g + 4 * (lane >> 5);
      if (GATE_UP) {
        const int n = n0 + wn * 32 + j;
        if (n < N)
          *reinterpret_cast<float4*>(crow + n) =
              make_float4(silu(acc[0][mb][4 * g]) * acc[1][mb][4 * g],
                          silu(acc[0][mb][4 * g + 1]) * acc[1][mb][4 * g + 1],
                          silu(acc[0][mb][4 * g + 2]) * acc[1][mb][4 * g + 2],
                          silu(acc[0][mb][4 * g + 3]) * acc[1][mb][4 * g + 3]);
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int n = n0 + wn * 64 + 32 * nb + j;
          if (n < N)
            *reinterpret_cast<float4*>(crow + n) =
                make_float4(acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                            acc[nb][mb][4 * g + 3]);
        }
      }
    }
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
  // (+1 slot per XCD: the heavy and light lists' shares each round up)
  return static_cast<unsigned>((g + kXcds - 1) / kXcds * kXcds + kXcds);
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

// Weight streaming for few rows per expert: an expert may still hold up to
// min(T, cap) rows, and the streaming kernel reads its weights once per 32
// of them; above kStreamMaxRows rows it is left to a 256 x 256 tile launch
// after the streaming one (only when T allows such an expert at all).
constexpr int kStreamMaxRows = 64;
inline bool stream_needs_tiles(int T) { return T > kStreamMaxRows; }

template <bool GATE_UP, bool TWO>
void launch_256(const bf16_t* A, const bf16_t* Alo, const int32_t* sorted_token,
                const int32_t* offsets, int E, const bf16_t* B0, const bf16_t* B1, int N, int K,
                void* C, bf16_t* Clo, int rows, int max_split, size_t c_split, int32_t* split,
                int min_rows, hipStream_t s) {
  auto kern = K % TK ? expert_gemm_bf16_kernel<GATE_UP, kWaves, true, TWO>
                     : expert_gemm_bf16_kernel<GATE_UP, kWaves, false, TWO>;
  const int nN = GATE_UP ? (N + 127) / 128 : (N + TW - 1) / TW;
  kern<<<tile_grid(rows, E, TWO ? TM / 2 : TM, nN, max_split), kWaves * 64, 0, s>>>(
      A, Alo, sorted_token, offsets, E, B0, B1, N, K, C, Clo, max_split, cu_count(), c_split,
      split, min_rows);
}

}  // namespace

moe_status launch_gate_up(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                          const void* w_gate, const void* w_up, int T, int d, int ffn, int E,
                          int k, moe_dtype dt, void* h, void* h_lo, hipStream_t s,
                          const StreamPermute* sp) {
  const int rows = T * k;
  if (sp && !stream_self_permute(rows, E, dt)) return MOE_UNSUPPORTED;
  if (dt == MOE_F32) {
    expert_gemm_f32_kernel<true><<<tile_grid(rows, E, TMF, (ffn + 63) / 64, 1), 256, 0, s>>>(
        static_cast<const float*>(x), sorted_token, offsets, E, static_cast<const float*>(w_gate),
        static_cast<const float*>(w_up), ffn, d, static_cast<float*>(h), cu_count(), nullptr);
    return launch_status();
  }
  bf16_t* hl = static_cast<bf16_t*>(h_lo);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bf16_t* wg = static_cast<const bf16_t*>(w_gate);
  const bf16_t* wu = static_cast<const bf16_t*>(w_up);
  if (use_stream_path(rows, E)) {
    const bool tiles = stream_needs_tiles(T);
    // (with sp the stream kernel writes sorted_token and offsets, which
    // the tile launch then reads)
    moe_status st = launch_gate_up_stream(x, sorted_token, offsets, w_gate, w_up, d, ffn, E, rows,
                                          h, hl, tiles ? kStreamMaxRows : T, sp, s);
    if (st != MOE_OK || !tiles) return st;
    launch_256<true, false>(xb, nullptr, sorted_token, offsets, E, wg, wu, ffn, d, h, hl, rows, 1,
                            0, nullptr, kStreamMaxRows, s);
    return launch_status();
  }
  if (use_tall_tiles(rows, E)) {
    auto kern = d % TK ? expert_gemm_tall_kernel<true, true> : expert_gemm_tall_kernel<true, false>;
    const int ncu = cu_count();
    kern<<<tall_grid(rows, E, (ffn + 127) / 128, 1, ncu), NW3 * 64, 0, s>>>(
        xb, sorted_token, offsets, E, wg, wu, ffn, d, h, hl, 1, ncu, 0, nullptr, 0, nullptr);
    return launch_status();
  }
  launch_256<true, false>(xb, nullptr, sorted_token, offsets, E, wg, wu, ffn, d, h, hl, rows, 1, 0,
                          nullptr, 0, s);
  return launch_status();
}

moe_status launch_down(const void* h, const void* h_lo, const int32_t* offsets, const void* w_down,
                       int T, int d, int ffn, int E, int k, moe_dtype dt, void* y, int32_t* split,
                       hipStream_t s, uint8_t* y_parts) {
  const int rows = T * k;
  if (dt == MOE_F32) {
    expert_gemm_f32_kernel<false><<<tile_grid(rows, E, TMF, (d + TMF - 1) / TMF, 1), 256, 0, s>>>(
        static_cast<const float*>(h), nullptr, offsets, E, static_cast<const float*>(w_down),
        nullptr, d, ffn, static_cast<float*>(y), cu_count(), split);
    return launch_status();
  }
  const bf16_t* hb = static_cast<const bf16_t*>(h);
  const bf16_t* hl = static_cast<const bf16_t*>(h_lo);
  const bf16_t* wd = static_cast<const bf16_t*>(w_down);
  const size_t c_split = static_cast<size_t>(rows) * d;
  const int max_split = down_split_bound(ffn);  // the parts the workspace holds
  if (use_stream_path(rows, E)) {
    // with a tile launch as well, both write one partial sum (the combine
    // reads one count of parts for every row)
    const bool tiles = stream_needs_tiles(T);
    moe_status st = launch_down_stream(h, hl, offsets, w_down, d, ffn, E, rows, y, split,
                                       tiles ? kStreamMaxRows : T, tiles ? 1 : max_split, s);
    if (st != MOE_OK || !tiles) return st;
    if (hl)
      launch_256<false, true>(hb, hl, nullptr, offsets, E, wd, nullptr, d, ffn, y, nullptr, rows,
                              1, c_split, split, kStreamMaxRows, s);
    else
      launch_256<false, false>(hb, nullptr, nullptr, offsets, E, wd, nullptr, d, ffn, y, nullptr,
                               rows, 1, c_split, split, kStreamMaxRows, s);
    return launch_status();
  }
  if (hl) {
    // two terms of h: 128 output rows per 256 x 256 tile
    launch_256<false, true>(hb, hl, nullptr, offsets, E, wd, nullptr, d, ffn, y, nullptr, rows,
                            max_split, c_split, split, 0, s);
    return launch_status();
  }
  if (use_tall_tiles(rows, E)) {
    auto kern = ffn % TK ? expert_gemm_tall_kernel<false, true> : expert_gemm_tall_kernel<false, false>;
    const int ncu = cu_count();
    // long reductions with a part table: one part per tile, two for the tail tiles
    const bool ksplit = y_parts != nullptr && max_split >= 2;
    const int ms = ksplit ? 1 : max_split;
    kern<<<tall_grid(rows, E, (d + TW - 1) / TW, ms, ncu), NW3 * 64, 0, s>>>(
        hb, nullptr, offsets, E, wd, nullptr, d, ffn, y, nullptr, ms, ncu, c_split, split, 0,
        ksplit ? y_parts : nullptr);
    return launch_status();
  }
  launch_256<false, false>(hb, nullptr, nullptr, offsets, E, wd, nullptr, d, ffn, y, nullptr, rows,
                           max_split, c_split, split, 0, s);
  return launch_status();
}

}  // namespace moe
