// Internal interface between the host C ABI (lisa_api.hip) and the gfx950
// kernels (lisa_kernels.hip).  Not installed; the public ABI is include/lisa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lisa {

constexpr int kD = 64;           // d_h = d_v supported by the kernels
constexpr int kMaxT = 8;         // walk terms k = 0..T-1
constexpr int kThreads = 256;    // every kernel runs 4 waves of 64
constexpr int kGroup = 16;       // partials summed by one level-1 combiner
constexpr int kMaxGroups = 16;   // level-1 groups summed by the level-2 combiner
constexpr int kMaxChunks = kGroup * kMaxGroups;
constexpr int kCntWords = 32;    // counter words per (batch, head): 16 groups + level 2
constexpr int kStatTile = 64;    // tokens staged per step of the statistics kernels

// One statistics sweep over the tokens of every (batch, head):
//   KV stage: partial s = sum phi(K_j) and phi(K)^T V over a token chunk;
//   M  stage: partial M = phi(K)^T Qt with Qt_j = phi(Q_j) / (phi(Q_j) . s + eps).
// Partials are summed in a fixed order by the last workgroup to finish
// (two levels when there are more than kGroup chunks), which writes the
// fp32 result and its MFMA operand fragments for the output kernel.
struct StatsArgs {
  const void* K;
  const void* X;        // V (KV stage) or Q (M stage)
  int n;                // tokens per (batch, head)
  int chunk;            // tokens per workgroup, a multiple of kStatTile
  int P;                // chunks per (batch, head) = ceil(n / chunk) <= kMaxChunks
  int ngroups;          // ceil(P / kGroup)
  float eps;
  float* part;          // [BH][P][64*64]
  float* part_s;        // [BH][P][64]        KV stage only
  float* gpart;         // [BH][ngroups][64*64]  (ngroups > 1)
  float* gpart_s;       // [BH][ngroups][64]     (ngroups > 1, KV stage)
  const float* s_in;    // [BH][64]           M stage only
  float* fin;           // [BH][64*64]
  float* fin_s;         // [BH][64]           KV stage only
  void* frag;           // [BH][64*64] elements of the input dtype
  unsigned* cnt;        // [BH][kCntWords], zero on entry, zero on exit
};

// The output pass: per spatial tile of one (batch, head), global branch from
// the fragments, 3x3 local branch from LDS-staged K/V cells, alpha mix.
struct OutArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* weights;   // [BH][n][T] or nullptr (geometric)
  const float* alpha;     // [heads]
  void* Y;
  const float* s;         // [BH][64]
  const void* frag_kv;    // [BH][64*64]
  const void* frag_m;     // [BH][64*64]
  float geo[kMaxT];       // geometric weights (weights == nullptr)
  int H, W, n, T, heads;
  int TR, TC, tiles_x;    // tile rows/cols, tiles per grid row
  float eps;
  float logit_scale;      // log2(e) / sqrt(d_h)
};

// dtype: 0 = fp32, 1 = bf16 (lisa_dtype).
hipError_t launch_stats_kv(int dtype, const StatsArgs& a, int BH, hipStream_t s);
hipError_t launch_stats_m(int dtype, const StatsArgs& a, int BH, hipStream_t s);
hipError_t launch_output(int dtype, const OutArgs& a, int BH, int ntiles, size_t lds_bytes,
                         hipStream_t s);

// LDS row stride (elements) of one staged 64-wide token row.
constexpr int kCellStride = 68;

}  // namespace lisa
