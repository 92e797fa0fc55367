// Internal interface between the host C ABI (lisa_api.hip) and the gfx950
// kernel (lisa_flow.hip).  Not installed; the public ABI is include/lisa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "lisa_resident.hpp"

namespace lisa {

// A kernel's limit on dynamic LDS beyond 64 KB, set once per device: the
// attribute belongs to the device current at the call, so each device that
// runs the kernel needs its own.  `done` is the kernel's own table (static
// storage, zero at load).  Two threads making the first call on one device
// both set it, which is harmless; devices past the table set it every call.
constexpr int kMaxDevices = 64;
inline hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<bool> (&done)[kMaxDevices]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool tracked = dev >= 0 && dev < kMaxDevices;
  if (tracked && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && tracked) done[dev].store(true, std::memory_order_release);
  return e;
}

constexpr int kD = 64;          // d_h = d_v supported by the kernel
constexpr int kMaxT = 16;       // walk terms k = 0..T-1 of the forward
constexpr int kMaxTBwd = 8;     // of the backward and the walk-weight predictor
constexpr int kThreads = 512;   // 8 waves of 64 per workgroup: 4 producers, 4 consumers
constexpr int kRoleWaves = 4;   // waves per role
constexpr int kXcds = 8;        // workgroup w runs on XCD w % 8
constexpr int kMaxRanks = 256;  // G <= 256: each rank combines >= 32 elements
constexpr int kMaxTileTokens = 256;
constexpr int kCntWords = 4;    // arrival counters per (batch, head) slice: KV, M, C (+ pad)
constexpr int kCntStride = 32;  // words between slices: each slice's counters on their own 128-byte line
// With more than kSubRanks ranks per slice, a phase's arrivals are counted per
// group of kSubRanks ranks, each group's counter on its own 128-byte line
// (slices < kMaxSubSlices, groups < kMaxSubs); a wait then reads every
// group's counter at once, one per lane (at most 64).  Arrivals on one
// counter serialise at the memory: with 256 ranks on one 256 x 256 slice,
// groups of 4 / 8 / 16 / 32 ranks gave 39.6 / 40.9 / 41.8 / 43.5 us per
// forward (one 200 x 320 slice: 42.0 / 42.8 / 43.4 / 44.8 us).
constexpr int kSubRanks = 4;
constexpr int kMaxSubSlices = 8;
constexpr int kMaxSubs = 256 / kSubRanks;
// Kernel variants (without the predictor; FlowArgs::variant): arrivals per
// group and the one-rank combine (bf16), the ELU feature map (both dtypes,
// plain arrivals and combine).
constexpr int kVarPlain = 0, kVarGrouped = 1, kVarSolo = 2, kVarElu = 3;

// q = floor(x / d) for 0 <= x < 2^20, 0 < d < 2^10, via a float reciprocal
// (inv_d = 1.0f / d): (x + 0.5) / d lies at least 0.5 / d from an integer, far
// more than the rounding error of the product.
__host__ __device__ __forceinline__ int div_small(int x, float inv_d) { return (int)(((float)x + 0.5f) * inv_d); }

// LDS of one workgroup, per element size ES: two staging buffers of kStage
// bytes that the DMA of the next stage and the compute of the current one
// alternate between, then the statistics area (the two 64x64 MFMA fragment
// sets) of the slice the output items work on.
template <int ES>
struct Lds {
  static constexpr int kStage = ES == 2 ? 71680 : 61440;
  static constexpr int kFragBytes = kD * kD * ES;          // one fragment set
  static constexpr int kStats = 2 * kFragBytes;
  static constexpr int kTotal = 2 * kStage + kStats;
  static constexpr int kChunk = ES == 2 ? 256 : 112;      // max tokens per KV / M item
  static constexpr int kXOff = kStage / 2 / 1024 * 1024;  // V / Q rows of a KV / M stage
};

// Byte offsets of an output tile's regions inside a staging buffer: K cells
// and V cells of the tile plus a one-cell halo, the Q rows of its token
// slots, their walk weights (fp32, T per slot) when they are per token, and
// r_i = 1 / (phi(Q_i) . s + eps) per slot (fp32), which the producer waves
// fill in once the Q rows have landed.
struct TileLayout {
  int cells, tokens;
  int k, v, q, w, r, total;
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
  L.r = L.w + round_kb(L.tokens * T * 4);
  L.total = L.r + round_kb(L.tokens * 4);
  return L;
}

// Static schedule of one launch.  G workgroups (ranks) share each (batch,
// head) slice; S = grid / G groups take slices b = group, group + S, ...,
// Z at a time (each phase runs for the round's Z slices before the next).
// For each slice, rank g of its group:
//   KV: sweeps its token range [g n / G, (g + 1) n / G) in chunks of at most
//       `chunk` tokens -> partial g of s and phi(K)^T V;
//   M:  after all G KV partials: s = their fixed-order sum, then partial g of
//       M = phi(K)^T Qt over the same range;
//   C:  after all G M partials (all KV partials when M is absent): elements
//       [g E, g E + E) of the flattened [phi(K)^T V | M] (E = 8192 / G), the
//       fixed-order sum of the G partials, written as fp32 and as MFMA
//       fragments (rank 0 also writes s);
//   OUT: after all G ranks' C parts: output tiles [g T / G, (g + 1) T / G).
// Each phase's completion is counted per slice (one arrival per rank).
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
  int chunk;              // tokens per KV / M stage (<= Lds::kChunk, multiple of 16)
  int G, S, Z;            // ranks per slice (a power of two), groups, slices per round
  int xcd_groups;         // groups sit within one XCD (workgroup w on XCD w % 8)
  int TR, TC, tiles_x, ntiles;  // output tiles, tiles per grid row / slice
  int do_kv, do_m, do_out;      // phases present (C runs whenever KV does)
  float* part_s;          // [BH][G][64]
  float* part_kv;         // [BH][G][64*64]
  float* part_m;          // [BH][G][64*64]
  float* fin_s;           // [BH][64]
  float* fin_kv;          // [BH][64*64]
  float* fin_m;           // [BH][64*64]
  void* frag_kv;          // [BH][64*64] elements of the input dtype
  void* frag_m;           // [BH][64*64]
  unsigned* slice_cnt;    // [BH][kCntStride], words 0..kCntWords-1 used
  unsigned* sub_cnt;      // [kMaxSubSlices][3][kMaxSubs][kCntStride], word 0 of each line used
  int variant;            // kVarPlain, kVarGrouped (arrivals per group of kSubRanks ranks, sub_cnt),
                          // kVarSolo (one rank per slice: the combine writes the statistics directly),
                          // kVarElu (phi = ELU + 1 instead of ReLU)
  unsigned* done_cnt;     // finished workgroups
  unsigned* tickets;      // [kXcds] rank tickets
  unsigned* err;          // error word (a dependency wait timed out)
  int clear_err;          // the last workgroup also clears the error word (no workspace to check it in)
  // Walk-weight predictor (weights == nullptr): w_i = softmax(W2 ReLU(W1 x_i + b1) + b2),
  // x_i = concat(Q_i, K_i), per head; W1 in the order the kernel's lanes
  // read it (launch_mlp_prep).
  const void* mlp_w1f;    // nullptr: no predictor
  const float* mlp_b1;    // [heads][hidden]
  const float* mlp_w2;    // [heads][T][hidden]
  const float* mlp_b2;    // [heads][T]
  int hidden;             // a multiple of 32, at most kMaxHidden
};

constexpr int kMaxHidden = 128;
// Floats of one head's first-layer weights as mlp_prep lays them out for the
// MFMA (bf16: [hidden/32][8 steps][64 lanes] bf16x8; fp32: [hidden/32][64 steps][64 lanes]).
__host__ __device__ inline size_t mlp_head_floats(int hidden, bool bf16) {
  return (size_t)hidden * (bf16 ? 64 : 128);
}

// The resident forward kernel (lisa_resident.hip): one tile of a slice per
// rank, staged on chip once (ResPlan).  Modes: the whole forward, the
// statistics alone (lisa_reduce), the output alone from statistics in the
// workspace (lisa_apply).
enum { kResForward = 0, kResReduce = 1, kResApply = 2 };
struct ResArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* weights;   // [BH][n][T] or nullptr (geometric: geo)
  const float* alpha;     // [heads]
  void* Y;
  float geo[kMaxT];
  int n, heads, BH;
  float eps;
  float logit_scale;      // log2(e) / sqrt(d_h)
  int S;                  // groups of G ranks
  int mode;
  int do_kv, do_m;        // statistics formed by this launch
  int per_token;          // weights per token (LDS region [slot][T]) instead of geo
  int grouped;            // arrivals counted per group of kSubRanks ranks (sub_cnt)
  ResPlan p;
  float* part_s;          // [BH][G][64]
  float* part_kv;         // [BH][G][2][64*64]: phi(K)^T V then M of each rank (the workspace's
                          // two partial regions, adjacent, as one)
  float* fin_s;           // [BH][64]
  float* fin_kv;          // [BH][64*64]
  float* fin_m;           // [BH][64*64]
  void* frag_kv;          // [BH][64*64] bf16, MFMA A-operand fragment order
  void* frag_m;
  unsigned* slice_cnt;    // [BH][kCntStride]
  unsigned* sub_cnt;      // [kMaxSubSlices][3][kMaxSubs][kCntStride]
  unsigned* done_cnt;     // XCDs whose workgroups have all finished
  unsigned* done_xcd;     // [kXcds][kCntStride]: finished workgroups of each XCD (word 0 of each line)
  unsigned* tickets;      // [kXcds] the streaming kernel's rank tickets (left at zero here too)
  unsigned* err;
  int clear_err;
  // The walk-weight predictor (forward only; nullptr: weights or geo):
  // W1 as laid out by mlp_prep (bf16 fragments), b1 [heads][hidden],
  // W2 [heads][T][hidden], b2 [heads][T].
  const void* mlp_w1f;
  const float* mlp_b1;
  const float* mlp_w2;
  const float* mlp_b2;
  int hidden;
  // A one-head layer's output projection folded into the output (forward
  // only; nullptr: Y = O): Y = O Wo^T + bo, O rounded to bf16 as the product's
  // operand.  Wo [64][64] bf16 as torch lays it out ([out][in]), bo [64].
  const void* wo;
  const float* bo;
  // Optional stage timeline: workgroup w writes the constant-clock counter
  // (s_memrealtime, 100 MHz) at stage k of its first slice to
  // stamps[w * kResPhases + k] (kResStamp*), and its group and rank to the
  // last entry.
  unsigned long long* stamps;
};
enum {
  kResStampStart = 0,   // ticket taken
  kResStampStaged,      // K, V cells, weights and Q landed
  kResStampKV,          // KV partial published
  kResStampLocal,       // local branch done
  kResStampS,           // every KV partial arrived, s formed
  kResStampM,           // M partial published
  kResStampMWait,       // every M partial arrived
  kResStampComb,        // share of the statistics written
  kResStampCWait,       // every share arrived
  kResStampFrags,       // statistics fragments in LDS
  kResStampOut,         // Y written
  kResStampEnd,         // last barrier of the workgroup
  kResStampKVSweep,     // products of the KV sweep done (before the partial is published)
  kResStampCStaged,     // the combine's share of every rank's partial in LDS
  kResStampCSummed,     // the combine's share summed
  kResPhases = 16
};
hipError_t launch_resident(const ResArgs& a, int grid, hipStream_t s);

// dtype: 0 = fp32, 1 = bf16 (lisa_dtype).  grid = workgroups to launch.
hipError_t launch_flow(int dtype, const FlowArgs& a, int grid, hipStream_t s);

// W1 [heads][hidden][2 d_h] (fp32) rearranged into the A operands of the
// predictor's first layer, per head (bf16 inputs: W1 rounded to bf16).
size_t mlp_frag_bytes(int dtype, int heads, int hidden);
hipError_t launch_mlp_prep(int dtype, const float* w1, void* block, int heads, int hidden, hipStream_t s);

// Projections of the attention layer (lisa_attention_forward):
// out[m][c] = sum_k A[m][k] Wt[c][k] + bias[c] over the K = C = 64 heads
// channels.  QKV: A = X [M][C], c < 3C goes to Q, K or V [B][heads][n][64]
// (head_elems apart); output: A = O [B][heads][n][64] merged by heads,
// out = Y [M][C].
struct ProjArgs {
  const void* A;
  const void* Wt;         // [N][K], the input dtype
  const float* bias;      // [N]
  void* out;
  int M, N, K;            // M = B n; N = 3C (QKV) or C; K = C
  int n, heads;
  size_t head_elems;      // B * heads * n * 64
};
hipError_t launch_proj(int dtype, bool out_proj, const ProjArgs& a, hipStream_t s);

// Backward pass (lisa_backward): token passes take kBwdTokens tokens per
// workgroup, one per lane; the slice statistics come from a statistics launch
// (fin_s, fin_kv, fin_m of FlowArgs) that ran before on the same stream.
constexpr int kBwdTokens = 256;

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* dY;
  const float* weights;   // [BH][n][T] or nullptr (geometric: geo)
  const float* alpha;     // [heads]
  void* dQ;
  void* dK;
  void* dV;
  float* dweights;        // [BH][n][T] or nullptr
  float* dalpha;          // [heads]
  float geo[kMaxTBwd];
  int H, W, n, T, heads, BH, nblk;  // nblk = ceil(n / kBwdTokens)
  float eps;
  const float* fin_s;     // [BH][64]
  const float* fin_kv;    // [BH][64*64]
  const float* fin_m;     // [BH][64*64]
  float* pk;              // [BH][T-1][64*64]  P_k = M^(k-1) phi(K)^T V, k = 1..T-1
  float4* tok;            // [BH][n]  per token: local max, local sum, dL_i . L_i, then (a_i -> dz_i)
  float* dp_part;         // [BH][nblk][T-1][64*64]  per-workgroup partials of dP_k
  float* da_part;         // [BH][nblk]  partials of dalpha
  float* da_slice;        // [BH]  their sums
  float* dmkv;            // [BH][2][64*64]  dM, dKV
  float* ds_part;         // [BH][nblk][64]  partials of ds
};

hipError_t launch_backward(int dtype, const BwdArgs& a, hipStream_t s);

}  // namespace lisa
