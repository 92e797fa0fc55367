// Static schedule of the resident forward kernel (lisa_resident.hip): how a
// (batch, head) slice's H x W token grid is cut into tiles, one per rank, and
// where a rank keeps its tile on chip.  Shared by the host planner
// (lisa_api.hip), the kernel, and a CPU check of the schedule's coverage
// (tests/test_schedule_cpu.py builds tests/schedule_check.cpp against it).
//
// Each rank owns one tile of TR x TC tokens (tiles in the last tile row or
// column may be shorter or narrower).  It stages the K and V cells of its
// tile plus a one-cell halo, clipped to the grid, in LDS once, keeps Q in
// registers, and uses them for all three uses: the KV sweep over its own
// tokens (s and phi(K)^T V), the M sweep over its own tokens (M = phi(K)^T Qt)
// and the output of its own tokens (3x3 local branch and the walk).  The
// tile's tokens are covered by BR x BC blocks of 4 x 8 tokens (the MFMA local
// branch's unit); a block's 32 token slots that fall outside the tile are
// masked.  Slot s is token s % 32 of block s / 32; block b is block row
// b / BC, block column b % BC; token j of a block is row j / 8, column j % 8.
#pragma once

#include <hip/hip_runtime.h>

namespace lisa {

constexpr int kResThreads = 512;            // 8 waves, two per SIMD (256 registers each)
constexpr int kResWaves = kResThreads / 64;
constexpr int kResMaxBlocks = 2 * kResWaves;  // 4 x 8 blocks per tile: at most two per wave
constexpr int kResMaxT = 8;                 // walk terms the resident kernel takes
constexpr int kResLdsMax = 159 * 1024;       // dynamic LDS: a gfx950 workgroup's 160 KB less the static part
constexpr int kResRowBytes = 128;           // one staged bf16 row of 64 features
// The scratch area: the second half's sweep products (four 32 x 32 fp32
// blocks and the s column), the waves' sums of the s partials, later the
// statistics fragments.
constexpr int kResScratch = 4 * 32 * 32 * 4 + 64 * 4;
// [G][E] floats staged by a rank's combine: E is nstat / G rounded up or
// down, so G * E <= nstat + G <= 8192 + 256 (a multiple of 256: the staging
// DMA's padded last run stays within it too).
constexpr int kResCombineFloats = 2 * 64 * 64 + 256;
constexpr int kResKRegionMin = kResCombineFloats * 4;

__host__ __device__ inline int res_cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int res_min(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int res_max(int a, int b) { return a > b ? a : b; }
__host__ __device__ inline int res_up(int x, int a) { return (x + a - 1) / a * a; }

// LDS byte offsets of a rank's regions.
struct ResLayout {
  int zrow;   // row index (in the K and in the V region) of a zero row
  int k;      // K cells, row r = staged cell r (swizzled 128-byte rows); later the combine's staging
  int v;      // V cells; after the local branch, row s = r_s phi(Q_s) of slot s
  int w;      // walk weights, [slot][T] fp32 (per-token weights only)
  int tab;    // [slot] uint16: staged cell of the slot's token, or zrow for a masked slot
  int loc;    // the local branch's tables: [block][64] uint16 window cells, [block][2] uint32 grid
              // masks, [64] uint32 neighbour masks, [4][64] bf16x8 one-hot operands (res_loc_*)
  int s;      // s = sum_j phi(K_j) of the slice, 64 fp32
  int scr;    // the sweeps' second-half products, the waves' s sums, later the statistics' bf16 fragments
  int st;     // one rank per slice: the statistics [phi(K)^T V | M] as fp32 rows (32 KB; else unused)
  int total;
};

struct ResPlan {
  int H, W, T, wT;    // grid; walk terms; weights per slot in LDS (T if per token, else 0)
  int TR, TC;         // tile size
  int ty, tx, G;      // tile rows and columns per slice; G = ty * tx ranks per slice
  int BR, BC, nblk;   // blocks per tile
  int SR, SC;         // staged cell rows and columns at most
  ResLayout L;
};

// One tile: its tokens and its staged cells.
struct ResTile {
  int r0, c0, th, tw;    // token rows [r0, r0 + th), columns [c0, c0 + tw)
  int sr0, sc0, SR, SC;  // staged cells: rows [sr0, sr0 + SR), columns [sc0, sc0 + SC)
};

__host__ __device__ inline ResTile res_tile(const ResPlan& p, int t) {
  ResTile x;
  const int ti = t / p.tx, tj = t % p.tx;
  x.r0 = ti * p.TR;
  x.c0 = tj * p.TC;
  x.th = res_min(p.TR, p.H - x.r0);
  x.tw = res_min(p.TC, p.W - x.c0);
  x.sr0 = res_max(x.r0 - 1, 0);
  x.sc0 = res_max(x.c0 - 1, 0);
  x.SR = res_min(x.r0 + x.th + 1, p.H) - x.sr0;
  x.SC = res_min(x.c0 + x.tw + 1, p.W) - x.sc0;
  return x;
}

// Staged cell of grid cell (row, col), clamped into the staged region: every
// cell of a tile token's 3x3 window that lies on the grid is staged; the
// window cells off the grid land on some staged cell and are masked.
__host__ __device__ inline int res_cell(const ResTile& t, int row, int col) {
  row = res_min(res_max(row, t.sr0), t.sr0 + t.SR - 1);
  col = res_min(res_max(col, t.sc0), t.sc0 + t.SC - 1);
  return (row - t.sr0) * t.SC + (col - t.sc0);
}

// The group and rank of workgroup w of a grid of `grid` (S groups of G ranks,
// BH slices; group -1: idle).  The device dispatches workgroups in index
// order, workgroup w to XCD w % 8 as the (w / 8)-th of that XCD.  Where G
// divides an XCD's share of the grid and there are at least as many slices
// as XCDs, each group sits in one XCD (group 8 (k / G) + x is the k-th G
// workgroups of XCD x): a group's tiles are neighbours, and their halo cells
// then come through one L2, while the groups with slices are spread evenly
// over the XCDs.  Otherwise a group takes consecutive indices, over all
// XCDs.  Either way each XCD starts a group's workgroups in order, after
// those of its earlier groups, so a group only waits for workgroups that
// start once earlier groups have finished.  (Ranks from an atomic ticket in
// start order, as the streaming kernel draws them, cost a round trip before
// any work and spread the workgroups' starts over 2.4 us: PVT-T stage 1 39.7
// -> 39.5 us, one 256 x 256 slice 38.4 -> 36.0, DeiT-T 224 22.0 -> 21.2.)
__host__ __device__ inline void res_rank_of(int G, int S, int BH, int w, int grid, int& group, int& g) {
  constexpr int kX = 8;  // XCDs
  const int per = grid / kX;
  if (grid % kX == 0 && per % G == 0 && BH >= kX) {
    const int x = w % kX, k = w / kX;
    group = kX * (k / G) + x;
    g = k % G;
  } else {
    group = w / G;
    g = w % G;
  }
  if (group >= S) group = -1;
}

// Tile coordinates of slot s; false when the slot lies outside the tile.
__host__ __device__ inline bool res_slot(const ResPlan& p, const ResTile& t, int s, int& tr, int& tc) {
  const int b = s >> 5, j = s & 31;
  tr = 4 * (b / p.BC) + (j >> 3);
  tc = 8 * (b % p.BC) + (j & 7);
  return tr < t.th && tc < t.tw;
}

// Elements [e0, e1) of the flattened [phi(K)^T V | M] (nstat of them: 4096
// without M, 8192 with) that rank g sums over the slice's G partials.
__host__ __device__ inline void res_combine_range(int nstat, int G, int g, int& e0, int& e1) {
  e0 = (int)((long long)g * nstat / G);
  e1 = (int)((long long)(g + 1) * nstat / G);
}

// The local branch's tables (byte offsets within the loc region, nblk blocks):
// each block's 64 window cells (uint16), its two grid masks (uint32), each
// lane's neighbour mask (uint32), each lane's one-hot operands of the four
// 16-cell steps (bf16x8).
__host__ __device__ inline int res_loc_win(int) { return 0; }
__host__ __device__ inline int res_loc_mask(int nblk) { return nblk * 64 * 2; }
__host__ __device__ inline int res_loc_nbr(int nblk) { return res_up(res_loc_mask(nblk) + nblk * 8, 16); }
__host__ __device__ inline int res_loc_hot(int nblk) { return res_loc_nbr(nblk) + 64 * 4; }
__host__ __device__ inline int res_loc_bytes(int nblk) { return res_loc_hot(nblk) + 4 * 64 * 16; }

// The LDS layout for the plan's largest tile; false if it exceeds kResLdsMax.
__host__ __device__ inline bool res_layout(ResPlan& p) {
  const int cells = p.SR * p.SC;
  const int slots = p.nblk * 32;
  // The DMA writes whole 1 KB runs (eight rows), so the zero row sits after
  // the last run of the cells; the V region also holds one row per slot.
  p.L.zrow = res_up(cells, 8);
  const int krows = p.L.zrow + 1;
  const int vrows = res_max(krows, slots);
  int o = 0;
  p.L.k = o;
  // Once the sweeps are done the K region stages the partials a rank
  // combines (its share of all G partials).
  o += res_max(res_up(krows * kResRowBytes, 1024), kResKRegionMin);
  p.L.v = o;
  o += res_up(vrows * kResRowBytes, 1024);
  p.L.w = o;
  o += res_up(slots * p.wT * 4, 256);  // the weight DMA writes 256-byte runs
  p.L.tab = o;
  o += res_up(slots * 2, 16);
  p.L.loc = o;
  o += res_loc_bytes(p.nblk);
  p.L.s = o;
  o += 64 * 4;
  p.L.scr = o;
  o += res_max(kResScratch, 2 * 64 * 64 * 2);  // fragments of phi(K)^T V and M
  // With one rank per slice the sweeps leave the statistics here directly.
  p.L.st = o;
  if (p.G == 1) o += 2 * 64 * 64 * 4;
  p.L.total = o;
  return o <= kResLdsMax;
}

// Host planner: the tiling of an H x W slice into G <= gcap tiles for the
// resident kernel, or false if none fits.  Among the tilings that fit (blocks
// per tile, LDS), the one that stages the fewest bytes per rank (K and V
// cells, Q rows, weights), counting a small cost per rank (partials and
// arrivals) and per block (masked slots compute too); ties go to fewer ranks.
inline bool res_plan(int H, int W, int T, bool per_token_weights, int gcap, ResPlan& out) {
  bool found = false;
  long best = 0;
  const int wT = per_token_weights ? T : 0;
  for (int ty = 1; ty <= res_min(H, gcap); ++ty) {
    const int TR = res_cdiv(H, ty);
    if (res_cdiv(H, TR) != ty) continue;  // the same tiles as a smaller ty
    for (int tx = 1; tx <= W && ty * tx <= gcap; ++tx) {
      const int TC = res_cdiv(W, tx);
      if (res_cdiv(W, TC) != tx) continue;
      ResPlan p{};
      p.H = H;
      p.W = W;
      p.T = T;
      p.wT = wT;
      p.TR = TR;
      p.TC = TC;
      p.ty = ty;
      p.tx = tx;
      p.G = ty * tx;
      p.BR = res_cdiv(TR, 4);
      p.BC = res_cdiv(TC, 8);
      p.nblk = p.BR * p.BC;
      if (p.nblk > kResMaxBlocks) continue;
      p.SR = res_min(TR + 2, H);
      p.SC = res_min(TC + 2, W);
      if (!res_layout(p)) continue;
      const long cost = (long)p.SR * p.SC * 2 * kResRowBytes + (long)TR * TC * (kResRowBytes + 4 * wT) +
                        512L * p.G + 256L * p.nblk;
      if (!found || cost < best) {
        found = true;
        best = cost;
        out = p;
      }
    }
  }
  return found;
}

}  // namespace lisa
