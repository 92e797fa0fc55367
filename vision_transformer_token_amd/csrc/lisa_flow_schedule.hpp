// Static schedule of the streaming forward kernel (lisa_flow.hip): which
// tokens, chunks, output tiles and statistics elements a rank of a group
// takes, in which order a rank runs its stages, and the host planner that
// picks the tiles, ranks and groups of a launch.  Shared by the kernel, the
// host planner (lisa_api.hip) and a CPU check of the schedule's coverage
// (tests/test_schedule_cpu.py builds tests/flow_schedule_check.cpp
// against it).
#pragma once

#include <hip/hip_runtime.h>

#include "lisa_kernels.hpp"

namespace lisa {

enum Phase { kPKV = 0, kPM = 1, kPC = 2, kPOut = 3, kPEnd = 4 };

// This workgroup's place in the schedule.
struct Rank {
  int group, g;       // group (-1: idle workgroup), rank within the group
  int tok0, ntok;     // token range of each slice
  int nch;            // chunks of that range
  int t0, nt;         // output tiles
  int e0, E;          // combine elements of the flattened [phi(K)^T V | M]
};

// Ranks are handed out in the order workgroups start (a ticket per XCD when
// groups stay within an XCD): a group then only ever waits for workgroups
// that are already running, so the launch makes progress as long as G
// workgroups fit on the device at once.  `ticket` comes from the launch's
// ticket counter (the one of XCD `xcd` when a.xcd_groups).
__host__ __device__ inline Rank make_rank(const FlowArgs& a, int ticket, int xcd) {
  Rank r;
  if (a.xcd_groups) {
    r.group = xcd * (a.S / kXcds) + ticket / a.G;
    if (ticket / a.G >= a.S / kXcds) r.group = -1;
  } else {
    r.group = ticket / a.G;
    if (r.group >= a.S) r.group = -1;
  }
  r.g = ticket % a.G;
  r.tok0 = (int)((long long)r.g * a.n / a.G);
  r.ntok = (int)((long long)(r.g + 1) * a.n / a.G) - r.tok0;
  r.nch = (r.ntok + a.chunk - 1) / a.chunk;
  r.t0 = (int)((long long)r.g * a.ntiles / a.G);
  r.nt = (int)((long long)(r.g + 1) * a.ntiles / a.G) - r.t0;
  r.E = 2 * kD * kD / a.G;
  r.e0 = r.g * r.E;
  return r;
}

// A stage: round r of the group's slices, phase `ph`, slice z of the round
// (slice b = group + (r Z + z) S), step j (chunk or tile index in the rank's
// range).  A round runs each phase for all its slices before the next phase,
// so a slice's dependency wait overlaps the other slices' stages.
struct Pos {
  int r, ph, z, j;
};
__host__ __device__ inline int slice_of(const FlowArgs& a, const Rank& rk, int r, int z) {
  return rk.group + (r * a.Z + z) * a.S;
}
// Slices in round r (0: past the group's last slice).
__host__ __device__ inline int round_slices(const FlowArgs& a, const Rank& rk, int r) {
  const int b0 = slice_of(a, rk, r, 0);
  if (rk.group < 0 || b0 >= a.BH) return 0;
  const int left = (a.BH - b0 + a.S - 1) / a.S;
  return a.Z < left ? a.Z : left;
}
__host__ __device__ inline int phase_len(const FlowArgs& a, const Rank& r, int ph) {
  switch (ph) {
    case kPKV: return a.do_kv ? r.nch : 0;
    case kPM: return a.do_m ? r.nch : 0;
    case kPC: return a.do_kv ? 1 : 0;
    case kPOut: return a.do_out ? r.nt : 0;
  }
  return 0;
}
// The stage after `p` (ph == kPEnd: none); empty phases are skipped.
__host__ __device__ inline Pos advance(const FlowArgs& a, const Rank& rk, Pos p) {
  if (p.ph != kPEnd) {
    if (p.j + 1 < phase_len(a, rk, p.ph)) return Pos{p.r, p.ph, p.z, p.j + 1};
    if (p.z + 1 < round_slices(a, rk, p.r)) return Pos{p.r, p.ph, p.z + 1, 0};
  }
  int r = p.r, ph = p.ph + 1;
  for (;;) {
    if (ph >= kPEnd) {
      ++r;
      ph = kPKV;
      if (round_slices(a, rk, r) == 0) return Pos{r, kPEnd, 0, 0};
    }
    if (phase_len(a, rk, ph) > 0) return Pos{r, ph, 0, 0};
    ++ph;
  }
}
__host__ __device__ inline Pos first_pos(const FlowArgs& a, const Rank& rk) {
  if (round_slices(a, rk, 0) == 0) return Pos{0, kPEnd, 0, 0};
  return advance(a, rk, Pos{-1, kPEnd, 0, 0});
}

// Output tile t's first token row and column (tiles row-major over the grid).
__host__ __device__ inline void tile_origin(const FlowArgs& a, int t, int& r0, int& c0) {
  r0 = (t / a.tiles_x) * a.TR;
  c0 = (t % a.tiles_x) * a.TC;
}

// Chunk j of the rank's range: first token and length.
__host__ __device__ inline void chunk_of(const FlowArgs& a, const Rank& r, int j, int& tok0, int& nv) {
  tok0 = r.tok0 + j * a.chunk;
  const int left = r.tok0 + r.ntok - tok0;
  nv = a.chunk < left ? a.chunk : left;
}

// ---------------------------------------------------------------------------
// Host planner.
// ---------------------------------------------------------------------------
// Output tile: TR x TC cells made of whole 4 x 8 token blocks (the MFMA
// local branch works on such blocks), at most kMaxTileTokens tokens, whose
// staged inputs (TileLayout: K and V cells with a one-cell halo, Q rows,
// per-token weights) fit one staging buffer.  Among those, the shape that
// stages the fewest bytes per slice, counting each tile as kTileOverhead
// bytes more (a stage has fixed costs), ties to the wider tile.
constexpr long kTileOverhead = 8192;

struct FlowTiles {
  int TR, TC, tiles_x, ntiles;
};

// wT: walk weights per staged token (T if per token, else 0); es: input
// element size.  False if no tile shape fits.
inline bool flow_plan_tiles(int H, int W, int wT, int es, FlowTiles& out) {
  const int stage = es == 2 ? Lds<2>::kStage : Lds<4>::kStage;
  const int h4 = (H + 3) / 4 * 4, w8 = (W + 7) / 8 * 8;
  long best = -1;
  for (int tc = (w8 < 64 ? w8 : 64); tc >= 8; tc -= 8)
    for (int tr = 4; tr <= h4 && tr * tc <= kMaxTileTokens; tr += 4) {
      const TileLayout L = tile_layout(tr, tc, wT, es);
      if (L.total > stage) break;
      const long ntiles = (long)((W + tc - 1) / tc) * ((H + tr - 1) / tr);
      const long cost = ntiles * (L.total + kTileOverhead);
      if (best < 0 || cost < best) {
        best = cost;
        out.TR = tr;
        out.TC = tc;
      }
    }
  if (best < 0) return false;
  out.tiles_x = (W + out.TC - 1) / out.TC;
  out.ntiles = out.tiles_x * ((H + out.TR - 1) / out.TR);
  return true;
}

// Workgroups per slice: `round` times as many as there are workgroups per
// slice of the grid (so that a group has that many slices to interleave), at
// most one per 128 tokens and kMaxRanks, rounded down to a power of two (the
// combine splits the 8192 statistics evenly).
inline int flow_plan_ranks(int grid, int BH, int n, int round) {
  long per = (long)round * grid / BH;
  const long tok = (n + 127) / 128;
  if (per > grid) per = grid;
  if (per > tok) per = tok;
  if (per > kMaxRanks) per = kMaxRanks;
  int G = 1;
  while (2L * G <= per) G *= 2;
  return G;
}

struct FlowGroups {
  int G, S, Z, xcd_groups;
};

// Ranks per slice (at most gmax, the ranks the workspace's partials are
// sized for), groups, slices per round, and whether groups stay within one
// XCD, for `grid` workgroups on a device of `xccs` XCDs.
// Slices per round: all of the group's slices, at most 4.  Pairs (G <= 2)
// stay on one XCD (the device hands workgroup w to XCD w % kXcds, so rank
// tickets are drawn per XCD): their many small hand-offs then start and
// finish together.  Larger groups take tickets from one counter in start
// order and so spread over all XCDs: when they were kept on one XCD, an XCD
// that fell behind in the HBM-bound KV and M phases held back every group on
// it (a PVT stage-1 forward, G = 16: 61 us on one XCD, 58 us spread; G = 4
// and 8 about even).
inline FlowGroups flow_plan_groups(int grid, int xccs, int BH, int n, int gmax, int round) {
  FlowGroups f;
  f.G = flow_plan_ranks(grid, BH, n, round);
  if (f.G > gmax) f.G = gmax;
  f.S = grid / f.G;
  const int z = (BH + f.S - 1) / f.S;
  f.Z = z < 4 ? z : 4;
  f.xcd_groups = (xccs == kXcds && f.G <= 2 && grid % kXcds == 0 && (grid / kXcds) % f.G == 0) ? 1 : 0;
  return f;
}

}  // namespace lisa
