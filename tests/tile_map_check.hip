// CPU check of the grouped GEMMs' tile assignment (assign_tile on the
// row-tile prefix): over many random expert-count patterns (up to 256
// experts), shapes, split limits and CU counts, every
// tile of every expert (and split part) is handed to exactly one workgroup
// of the launched grid, whole or as both of its halves, and nothing else is.
// Built and run by test_tile_map.py; needs no GPU.
#include "../sparse_mixture_experts_renorm_amd/csrc/expert_gemm.hip"
#include "../sparse_mixture_experts_renorm_amd/csrc/expert_stream.hip"

#include <cmath>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <map>
#include <random>
#include <tuple>
#include <vector>

using namespace moe;

template <int BM, bool TAIL>
static int check(const std::vector<int32_t>& off, int E, int rows_bound, int nN, int max_split,
                 int n_cu, int nk, long long* tiles_seen, int min_rows = 0, int wrows = 1 << 30) {
  const unsigned grid = TAIL ? tall_grid(rows_bound, E, nN, max_split, n_cu)
                             : tile_grid(rows_bound, E, BM, nN, max_split);
  // key (e, row tile, column tile, part) -> counts {whole, half 0, half 1}
  std::map<std::tuple<int, int, int, int>, std::array<int, 3>> seen;
  // (e, column tile, part, first row) -> rows
  std::map<std::tuple<int, int, int, int>, int> rows_of;
  int S = -1;
  std::vector<int> pref(2 * E + 2);
  row_tile_prefix<BM>(off.data(), E, pref.data(), min_rows);
  // light experts' tiles per XCD (the halves of a split tile count once)
  std::map<std::tuple<int, int, int, int>, int> light_xcd;
  for (unsigned b = 0; b < grid; ++b) {
    int res[7];
    assign_tile<BM, TAIL>(off.data(), pref.data(), E, nN, max_split, n_cu, nk, wrows,
                          static_cast<int>(b), res);
    if (S < 0) S = res[5];
    if (res[5] != S) return printf("split count differs between workgroups\n"), 1;
    if (res[0] < 0) continue;
    const int e = res[0];
    if (e >= 0 && e < E && off[e + 1] - off[e] <= min_rows)
      return printf("expert %d with %d rows (at most %d) got a tile\n", e, off[e + 1] - off[e], min_rows), 1;
    if (e >= E || res[1] < off[e] || res[1] % 32 != off[e] % 32 || res[2] <= 0 || res[2] > BM ||
        res[1] + res[2] > off[e + 1] || res[3] < 0 || res[3] >= nN || res[4] < 0 ||
        res[4] >= S || res[6] < -1 || res[6] > 1 || (!TAIL && res[6] != -1))
      return printf("bad tile: e %d row0 %d rows %d nt %d ks %d half %d\n", e, res[1], res[2],
                    res[3], res[4], res[6]), 1;
    // key by the first row; the rows must cut the expert into its row tiles
    seen[{e, res[1], res[3], res[4]}][res[6] + 1] += 1;
    if (light_expert(off[e + 1] - off[e], BM)) light_xcd[{e, res[1], res[3], res[4]}] = b % kXcds;
    const auto key = std::make_tuple(e, res[3], res[4], res[1]);
    const auto it = rows_of.find(key);
    if (it != rows_of.end() && it->second != res[2])
      return printf("tile at row %d has %d and %d rows\n", res[1], it->second, res[2]), 1;
    rows_of[key] = res[2];
  }
  // per (expert, column tile, part): the row ranges tile [off[e], off[e+1])
  // exactly, in row tiles that differ by at most 32 rows (before the ragged
  // end of the last one)
  {
    std::map<std::tuple<int, int, int>, std::vector<std::pair<int, int>>> ranges;
    for (const auto& kv : rows_of)
      ranges[{std::get<0>(kv.first), std::get<1>(kv.first), std::get<2>(kv.first)}].push_back(
          {std::get<3>(kv.first), kv.second});
    for (auto& kv : ranges) {
      const int e = std::get<0>(kv.first);
      auto& v = kv.second;
      std::sort(v.begin(), v.end());
      int next = off[e], lo = 1 << 30, hi = 0;
      for (size_t i = 0; i < v.size(); ++i) {
        if (v[i].first != next) return printf("row tiles of expert %d leave a gap or overlap\n", e), 1;
        next += v[i].second;
        const int blocks = (v[i].second + 31) / 32;
        lo = std::min(lo, blocks);
        hi = std::max(hi, blocks);
      }
      if (next != off[e + 1]) return printf("row tiles of expert %d do not reach its end\n", e), 1;
      if (hi - lo > 1) return printf("row tiles of expert %d are uneven: %d..%d blocks\n", e, lo, hi), 1;
      if (static_cast<int>(v.size()) != expert_row_tiles(off[e + 1] - off[e], BM, min_rows))
        return printf("expert %d has %zu row tiles\n", e, v.size()), 1;
    }
  }
  long long expected = 0;
  for (int e = 0; e < E; ++e) expected += expert_row_tiles(off[e + 1] - off[e], BM, min_rows);
  expected *= static_cast<long long>(nN) * (S < 1 ? 1 : S);
  if (static_cast<long long>(seen.size()) != expected)
    return printf("%zu distinct tiles assigned, %lld expected (grid %u)\n", seen.size(), expected, grid), 1;
  for (const auto& kv : seen) {
    const auto& c = kv.second;
    // c[0]: whole (half -1), c[1], c[2]: halves 0 and 1
    const bool whole = c[0] == 1 && c[1] == 0 && c[2] == 0;
    const bool halves = c[0] == 0 && c[1] == 1 && c[2] == 1;
    if (!whole && !halves)
      return printf("tile assigned %d whole, %d + %d halves\n", c[0], c[1], c[2]), 1;
  }
  // every XCD runs at most its even share of the light experts' tiles
  {
    std::vector<int> per(kXcds, 0);
    for (const auto& kv : light_xcd) per[kv.second] += 1;
    const int share = (static_cast<int>(light_xcd.size()) + kXcds - 1) / kXcds;
    for (int x = 0; x < kXcds; ++x)
      if (per[x] > share)
        return printf("XCD %d runs %d light tiles, more than its share %d\n", x, per[x], share), 1;
  }
  *tiles_seen += expected;
  return 0;
}

// The 24-bit format of y (common.h): four values through three words and
// back are each the value rounded to 16 significant bits, nearest with ties
// to even, i.e. within 2^-16 of it relative, and exact when the low 8 bits
// are zero.
static int check_f24() {
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.f, 1.f);
  for (int it = 0; it < 200000; ++it) {
    float v[4], back[4];
    for (int i = 0; i < 4; ++i) v[i] = nd(rng) * std::ldexp(1.f, static_cast<int>(rng() % 60) - 30);
    if (it % 7 == 0) v[it % 4] = 0.f;
    if (it % 11 == 0) v[1] = -v[1];
    const uint3 w = pack_f24x4(v[0], v[1], v[2], v[3]);
    unpack_f24x4(w.x, w.y, w.z, back);
    for (int i = 0; i < 4; ++i) {
      uint32_t u;
      std::memcpy(&u, &v[i], 4);
      const uint32_t low = u & 0xFFu, keep = u >> 8;
      const uint32_t want = (low > 0x80u || (low == 0x80u && (keep & 1u))) ? (keep + 1) << 8 : keep << 8;
      uint32_t got;
      std::memcpy(&got, &back[i], 4);
      if (got != want)
        return printf("24-bit y: %a packed to %08x, want %08x\n", v[i], got, want), 1;
      if (std::fabs(back[i] - v[i]) > std::ldexp(std::fabs(v[i]), -16))
        return printf("24-bit y: %a off by more than 2^-16\n", v[i]), 1;
    }
  }
  return 0;
}

int main() {
  if (check_f24()) return 1;
  std::mt19937 rng(12345);
  long long tiles = 0;
  int cases = 0;
  const int cus[] = {256, 304, 80, 8, 1};
  for (int it = 0; it < 2000; ++it) {
    const int E = 1 + static_cast<int>(rng() % (it % 7 == 0 ? kMaxExperts : 64));
    std::vector<int32_t> off(E + 1, 0);
    for (int e = 0; e < E; ++e) {
      int m;
      switch (it % 5) {
        case 0: m = static_cast<int>(rng() % 3000); break;                         // anything
        case 1: m = (rng() % 3 == 0) ? 0 : 700 + static_cast<int>(rng() % 700);    // some empty
        case 2: m = e == 0 ? 20000 + static_cast<int>(rng() % 9000) : static_cast<int>(rng() % 60);
        case 3: m = 384 * static_cast<int>(rng() % 5) + 128 * static_cast<int>(rng() % 3);
        default: m = static_cast<int>(rng() % 40); break;                          // decode-like
      }
      off[e + 1] = off[e] + m;
    }
    const int rows_bound = off[E] + static_cast<int>(rng() % 50);  // capacity may keep fewer
    const int nN = 1 + static_cast<int>(rng() % 130);
    const int max_split = (it & 1) ? kMaxDownSplit : 1;
    const int nk = 1 + static_cast<int>(rng() % 400);
    const int n_cu = cus[it % 5];
    // the order inside an expert follows its row count against the weight
    // rows: all column-major, all row-major, or mixed
    const int wrows = (it % 3 == 0) ? 1 << 30 : (it % 3 == 1 ? 0 : 64 + static_cast<int>(rng() % 2000));
    if (check<256, false>(off, E, rows_bound, nN, max_split, n_cu, nk, &tiles, 0, wrows)) return 1;
    if (check<384, true>(off, E, rows_bound, nN, max_split, n_cu, nk, &tiles, 0, wrows)) return 1;
    // beside the weight-streaming kernel: only experts above 64 rows
    if (check<256, false>(off, E, rows_bound, nN, 1, n_cu, nk, &tiles, 64)) return 1;
    // the down pass with h in two bf16 terms: 128 output rows per tile
    if (check<128, false>(off, E, rows_bound, nN, max_split, n_cu, nk, &tiles)) return 1;
    // the fp32 kernels: 128-row tiles, one split part, either order per expert
    if (check<128, false>(off, E, rows_bound, nN, 1, n_cu, nk, &tiles, 0, wrows)) return 1;
    cases += 5;
  }
  printf("ok: %d cases, %lld tiles\n", cases, tiles);
  return 0;
}
