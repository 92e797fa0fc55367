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
constexpr int kBufBytes = 75776;  // one LDS staging buffer (two are used)
constexpr int kMaxCells = kBufBytes / 2 / 128;   // K and V cells of a bf16 output tile
constexpr int kMaxTileTokens = 256;
constexpr int kCombineBlocks = 4;  // combine items per 64x64 matrix (16 rows each)

// One launch of the persistent kernel processes work items of four kinds for
// every (batch, head) slice b, in queue order:
//   KV(b, p): tokens [p*chunk, ...) -> partial s and phi(K)^T V;
//   M(b, p):  after all KV(b, *): s, then partial M = phi(K)^T Qt;
//   C(b, q):  after all M(b, *) (or KV(b, *) when M is absent): sums the
//             partials of one 16-row block of phi(K)^T V (q < 4) or M
//             (q >= 4) in a fixed order and writes the final fp32 values and
//             their MFMA fragments; C(b, 0) also writes s;
//   OUT(b, t): after all C(b, *): one spatial tile of Y.
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
  int TR, TC, tiles_x;    // output tile rows/cols, tiles per grid row
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
  unsigned* slice_cnt;    // [BH][4]: arrivals of KV, M, C, OUT items
  unsigned* queue_cnt;    // [8] tickets, [8] unused, [16] finished workgroups
  unsigned* err;          // set when a bounded wait gives up
};

// dtype: 0 = fp32, 1 = bf16 (lisa_dtype).  grid = workgroups to launch.
hipError_t launch_flow(int dtype, const FlowArgs& a, int grid, hipStream_t s);

}  // namespace lisa
