// Internal interface between the host C ABI (lisa_api.hip) and the gfx950
// kernel (lisa_flow.hip).  Not installed; the public ABI is include/lisa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lisa {

constexpr int kD = 64;          // d_h = d_v supported by the kernel
constexpr int kMaxT = 8;        // walk terms k = 0..T-1
constexpr int kThreads = 256;   // 4 waves of 64 per workgroup
constexpr int kMaxQueues = 8;   // one work queue per XCD
constexpr int kCombineBlocks = 4;   // combine items per 64x64 matrix (16 rows each)
constexpr int kMaxTileTokens = 256;
constexpr int kCntWords = 4;    // arrival counters per (batch, head) slice: KV, M, C, OUT

// LDS of one workgroup, per element size ES: two staging buffers of kStage
// bytes that the DMA of the next stage and the compute of the current one
// alternate between, then the statistics area (the two 64x64 MFMA fragment
// sets and s) of the slice the output items work on.
template <int ES>
struct Lds {
  static constexpr int kStage = ES == 2 ? 71680 : 61440;
  static constexpr int kFragBytes = kD * kD * ES;          // one fragment set
  static constexpr int kStats = 2 * kFragBytes + 1024;    // + s (256 B, padded)
  static constexpr int kTotal = 2 * kStage + kStats;
  static constexpr int kChunk = ES == 2 ? 256 : 112;      // max tokens per KV / M item
  static constexpr int kXOff = kStage / 2 / 1024 * 1024;  // V / Q rows of a KV / M stage
};

// Byte offsets of an output tile's regions inside a staging buffer: K cells
// and V cells of the tile plus a one-cell halo, the Q rows of its token
// slots, and their walk weights (fp32, T per slot) when they are per token.
struct TileLayout {
  int cells, tokens;
  int k, v, q, w, total;
};
__host__ __device__ inline int round_kb(int x) { return (x + 1023) / 1024 * 1024; }
__host__ __device__ inline TileLayout tile_layout(int TR, int TC, int T, int es) {
  TileLayout L;
  L.cells = (TR + 2) * (TC + 2);
  L.tokens = TR * TC;
  const int rb = kD * es;
  L.k = 0;
  L.v = round_kb(L.cells * rb);
  L.q = 2 * L.v;
  L.w = L.q + round_kb(L.tokens * rb);
  L.total = L.w + round_kb(L.tokens * T * 4);
  return L;
}

// One launch of the persistent kernel processes, for every (batch, head)
// slice b, work items of four kinds in queue order:
//   KV(b, p): tokens [p*chunk, ...) -> partial s and phi(K)^T V;
//   M(b, p):  after all KV(b, *): s = fixed-order sum of the partial s, then
//             partial M = phi(K)^T Qt over the chunk;
//   C(b, q):  after all M(b, *) (all KV(b, *) when M is absent): the
//             fixed-order sum of the partials of one 16-row block of
//             phi(K)^T V (q < 4) or M (q >= 4), written as fp32 and as MFMA
//             fragments (C item 0 also writes s);
//   OUT(b, j): after all C(b, *): the run of output tiles [j R, j R + R).
// Slice b's items sit in queue b % 8 (served by the workgroups of XCD b % 8)
// when the slice count is a multiple of 8, else in a single queue.
struct FlowArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* weights;   // [BH][n][T] or nullptr (geometric)
  const float* alpha;     // [heads]
  void* Y;
  float geo[kMaxT];       // geometric weights (weights == nullptr)
  int H, W, n, T, heads, BH;
  float eps;
  float logit_scale;      // log2(e) / sqrt(d_h)
  int chunk, P;           // statistics items: tokens per item, items per slice
  int TR, TC, tiles_x, ntiles, R;  // output tiles, tiles per grid row / slice, tiles per run
  int nKV, nM, nC, nOUT;  // items per slice of each kind (0 = kind absent)
  int wait_out;           // output items wait for their slice's statistics
  int nq;                 // work queues (8 or 1)
  float* part_s;          // [BH][P][64]
  float* part_kv;         // [BH][P][64*64]
  float* part_m;          // [BH][P][64*64]
  float* fin_s;           // [BH][64]
  float* fin_kv;          // [BH][64*64]
  float* fin_m;           // [BH][64*64]
  void* frag_kv;          // [BH][64*64] elements of the input dtype
  void* frag_m;           // [BH][64*64]
  unsigned* slice_cnt;    // [BH][kCntWords]
  unsigned* queue_cnt;    // [8] tickets, [16] finished workgroups, [17] error word
  unsigned* err;
};

// dtype: 0 = fp32, 1 = bf16 (lisa_dtype).  grid = workgroups to launch.
hipError_t launch_flow(int dtype, const FlowArgs& a, int grid, hipStream_t s);

}  // namespace lisa
