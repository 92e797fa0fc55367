// CPU check of the resident forward kernel's static schedule
// (vision_transformer_token_amd/csrc/lisa_resident.hpp), built by
// tests/test_schedule_cpu.py with hipcc for the host only.
//
// For each problem given on the command line as "H W T gcap" it plans the
// tiling with res_plan (as the library does) and checks, for every tile:
//   - the tiles' token slots cover every grid token exactly once;
//   - every on-grid cell of a tile token's 3x3 window is staged (res_cell does
//     not clamp it), and every clamped window cell of any slot (valid or
//     masked) is a staged cell;
//   - slot-table rows, DMA runs, the zero row, the weight runs and the
//     rescaled-Q rows stay inside their LDS regions, the regions do not
//     overlap, and the layout fits the workgroup's LDS;
//   - the sweep steps read only slots of the tile; the combine ranges of the
//     G ranks partition the statistics; the workgroup -> (group, rank) map
//     takes every rank of every group once.
// It also checks the layer projections' schedules (lisa_layer.hpp) for a set
// of row and output counts: the blocked kernel's workgroups take every
// (row block, column block) once; the streaming kernel's units take every
// (row tile, column block) once, and the units a workgroup walks share its
// column block.
// Prints one line per problem ("ok ..." or "FAIL ...") and exits non-zero on
// any failure.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "lisa_layer.hpp"
#include "lisa_resident.hpp"

using namespace lisa;

static int fails = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      if (fails < 20) {                          \
        std::printf("FAIL %s: ", #cond);         \
        std::printf(__VA_ARGS__);                \
        std::printf("\n");                       \
      }                                          \
      ++fails;                                   \
    }                                            \
  } while (0)

static void check(int H, int W, int T, int gcap) {
  ResPlan p;
  if (!res_plan(H, W, T, true, gcap, p)) {
    std::printf("none %d %d %d %d\n", H, W, T, gcap);
    return;
  }
  const int before = fails;
  const ResLayout& L = p.L;
  const int slots = p.nblk * 32;
  CHECK(p.G >= 1 && p.G <= gcap, "G %d", p.G);
  CHECK(p.nblk <= kResMaxBlocks, "nblk %d", p.nblk);
  CHECK(L.total <= kResLdsMax, "lds %d", L.total);
  // Regions in order, disjoint, and each large enough.
  const int krows = L.zrow + 1;
  CHECK(L.k == 0 && L.v >= L.k + krows * kResRowBytes, "k region");
  // The combine stages its share of all G partials (nstat floats in all) there.
  CHECK(L.v - L.k >= kResCombineFloats * 4 && kResCombineFloats % 256 == 0, "k region holds the combine's staging");
  CHECK(L.w >= L.v + krows * kResRowBytes && L.w >= L.v + slots * kResRowBytes, "v region");
  CHECK(L.tab >= L.w + res_up(slots * T, 64) * 4, "w region");
  CHECK(L.loc >= L.tab + slots * 2, "tab region");
  CHECK(L.s >= L.loc + res_loc_bytes(p.nblk) && res_loc_mask(p.nblk) >= res_loc_win(p.nblk) + p.nblk * 128 &&
            res_loc_nbr(p.nblk) >= res_loc_mask(p.nblk) + p.nblk * 8 && res_loc_hot(p.nblk) >= res_loc_nbr(p.nblk) + 256 &&
            res_loc_hot(p.nblk) % 16 == 0 && L.loc % 16 == 0,
        "loc region");
  CHECK(L.scr >= L.s + 64 * 4, "s region");
  CHECK(L.st >= L.scr + kResScratch && L.st >= L.scr + 2 * 64 * 64 * 2, "scr region");
  CHECK(L.total >= L.st + (p.G == 1 ? 2 * 64 * 64 * 4 : 0), "st region");
  CHECK(L.k % 1024 == 0 && L.v % 1024 == 0 && L.w % 256 == 0 && L.tab % 16 == 0 && L.s % 16 == 0 &&
            L.scr % 16 == 0 && L.st % 16 == 0,
        "alignment");
  std::vector<int> owner((size_t)H * W, -1);
  for (int g = 0; g < p.G; ++g) {
    const ResTile t = res_tile(p, g);
    CHECK(t.th >= 1 && t.tw >= 1, "empty tile %d", g);
    const int cells = t.SR * t.SC;
    CHECK(t.SR <= p.SR && t.SC <= p.SC && cells <= p.SR * p.SC, "staged %dx%d", t.SR, t.SC);
    CHECK(t.sr0 >= 0 && t.sc0 >= 0 && t.sr0 + t.SR <= H && t.sc0 + t.SC <= W, "staged region off grid");
    // DMA of the cells: whole 1 KB runs end before the zero row.
    CHECK(res_up(cells, 8) <= L.zrow, "dma runs reach the zero row");
    for (int s = 0; s < slots; ++s) {
      int tr, tc;
      const bool on = res_slot(p, t, s, tr, tc);
      CHECK(tr >= 0 && tc >= 0 && tr < 4 * p.BR && tc < 8 * p.BC, "slot coordinates");
      if (on) {
        const int row = t.r0 + tr, col = t.c0 + tc;
        CHECK(row < H && col < W, "slot off grid");
        int& o = owner[(size_t)row * W + col];
        CHECK(o == -1, "token %d,%d covered twice", row, col);
        o = g;
        // Every on-grid window cell is staged, at the right place.
        for (int dr = -1; dr <= 1; ++dr)
          for (int dc = -1; dc <= 1; ++dc) {
            const int r2 = row + dr, c2 = col + dc;
            if (r2 < 0 || r2 >= H || c2 < 0 || c2 >= W) continue;
            CHECK(r2 >= t.sr0 && r2 < t.sr0 + t.SR && c2 >= t.sc0 && c2 < t.sc0 + t.SC,
                  "neighbour %d,%d of %d,%d not staged", r2, c2, row, col);
            CHECK(res_cell(t, r2, c2) == (r2 - t.sr0) * t.SC + (c2 - t.sc0), "cell index");
          }
      }
      // The slot table's row and the block's window cells stay in the K / V regions.
      const int tabrow = on ? res_cell(t, t.r0 + tr, t.c0 + tc) : L.zrow;
      CHECK(tabrow >= 0 && tabrow <= L.zrow, "table row %d", tabrow);
      const int blk = s >> 5, br = blk / p.BC, bc = blk % p.BC;
      for (int c = 0; c < 64; ++c) {
        const int cc = c < 59 ? c : 59;
        const int wc = res_cell(t, t.r0 + 4 * br - 1 + cc / 10, t.c0 + 8 * bc - 1 + cc % 10);
        CHECK(wc >= 0 && wc < cells, "window cell %d", wc);
      }
    }
    // Weights: runs of 64 floats over slots * T values.
    CHECK(res_up(slots * T, 64) * 4 <= L.tab - L.w, "weight runs");
  }
  for (int r = 0; r < H; ++r)
    for (int c = 0; c < W; ++c) CHECK(owner[(size_t)r * W + c] >= 0, "token %d,%d uncovered", r, c);
  // Workgroups -> (group, rank): for the grids of 256 (and 80, 304) compute
  // units and slice counts around the XCD count, every rank of every group
  // that has a slice is taken exactly once.
  for (int grid : {256, 80, 304})
    for (int BH : {1, 7, 8, 32, 192}) {
      const int S = grid / p.G;
      if (S < 1) continue;
      std::vector<int> seen((size_t)S * p.G, 0);
      for (int w = 0; w < grid; ++w) {
        int group, g;
        res_rank_of(p.G, S, BH, w, grid, group, g);
        CHECK(group >= -1 && group < S && g >= 0 && g < p.G, "rank of workgroup %d: %d %d", w, group, g);
        if (group >= 0 && group < S && g >= 0 && g < p.G) ++seen[(size_t)group * p.G + g];
      }
      for (int k = 0; k < S * p.G; ++k) CHECK(seen[k] == 1, "grid %d BH %d: group %d rank %d taken %d times", grid, BH, k / p.G, k % p.G, seen[k]);
    }
  // Combine ranges partition the statistics, for both sizes, and each rank's
  // staging ([G][E] floats) fits the K region and its loads.
  for (int nstat : {4096, 8192}) {
    int next = 0;
    for (int g = 0; g < p.G; ++g) {
      int e0, e1;
      res_combine_range(nstat, p.G, g, e0, e1);
      CHECK(e0 == next && e1 >= e0, "combine range %d", g);
      // The staging DMA writes runs of 256 floats (16 bytes per lane, when E
      // and e0 are multiples of four) or 64 floats, the last one padded.
      const int E = e1 - e0, run = (E % 4 == 0 && e0 % 4 == 0) ? 256 : 64;
      CHECK(res_up(E * p.G, run) <= kResCombineFloats && res_up(E * p.G, run) * 4 <= L.v - L.k, "combine staging %d",
            E * p.G);
      CHECK(e1 - e0 >= 16, "combine share %d", e1 - e0);  // the float quotient q / E stays exact
      next = e1;
    }
    CHECK(next == nstat, "combine end %d", next);
  }
  if (fails == before)
    std::printf("ok %d %d %d %d: G=%d tiles %dx%d of %dx%d, %d blocks, staged %dx%d, lds %d\n", H, W, T, gcap, p.G,
                p.ty, p.tx, p.TR, p.TC, p.nblk, p.SR, p.SC, L.total);
}

static void check_proj(int M, int N) {
  const int before = fails;
  const int nct = N / 64;
  const int nrb = (M + 64 * kProjTiles - 1) / (64 * kProjTiles), nrt = (M + 63) / 64;
  std::vector<int> seen((size_t)nrb * nct, 0);
  const int grid = proj_grid(M, N);
  for (int w = 0; w < grid; ++w) {
    int rb, cb;
    proj_block(M, N, w, rb, cb);
    CHECK(rb >= -1 && rb < nrb && cb >= 0 && cb < nct, "proj block of %d: %d %d", w, rb, cb);
    if (rb >= 0 && rb < nrb && cb >= 0 && cb < nct) ++seen[(size_t)rb * nct + cb];
  }
  for (size_t k = 0; k < seen.size(); ++k) CHECK(seen[k] == 1, "M %d N %d: block %zu taken %d times", M, N, k, seen[k]);
  const int U = proj_units(M, N), G = proj_stream_grid(M, N);
  CHECK(U % (8 * nct) == 0 && G >= 1 && G <= U && (G % (8 * nct) == 0 || G == U), "stream grid %d of %d units", G, U);
  std::vector<int> tiles((size_t)nrt * nct, 0);
  for (int g = 0; g < G; ++g) {
    int rt0, cb0;
    proj_unit(N, g, rt0, cb0);
    for (int u = g; u < U; u += G) {
      int rt, cb;
      proj_unit(N, u, rt, cb);
      CHECK(cb == cb0 && cb >= 0 && cb < nct && rt >= 0, "unit %d of workgroup %d: tile %d block %d", u, g, rt, cb);
      if (rt < nrt && cb >= 0 && cb < nct) ++tiles[(size_t)rt * nct + cb];
    }
  }
  for (size_t k = 0; k < tiles.size(); ++k) CHECK(tiles[k] == 1, "M %d N %d: unit %zu taken %d times", M, N, k, tiles[k]);
  if (fails == before) std::printf("proj %d %d covered: %d workgroups, %d units on %d\n", M, N, grid, U, G);
}

int main(int argc, char** argv) {
  for (int M : {1, 63, 64, 65, 297, 1000, 37632, 51300, 100352})
    for (int N : {64, 192, 384, 576}) check_proj(M, N);
  for (int i = 1; i + 3 < argc; i += 4) check(std::atoi(argv[i]), std::atoi(argv[i + 1]), std::atoi(argv[i + 2]),
                                                std::atoi(argv[i + 3]));
  if (fails) std::printf("%d failures\n", fails);
  return fails ? 1 : 0;
}
