// Host side of liblisa.so: argument checks, planning, workspace layout and
// launch sequencing for the C ABI declared in include/lisa.h.  Nothing here
// touches the GPU before every argument has been checked.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "lisa.h"
#include "lisa_flow_schedule.hpp"
#include "lisa_kernels.hpp"

namespace {

using lisa::kD;
using lisa::kThreads;

constexpr size_t kAlign = 256;

// Compute units and XCDs of a device, queried once per device (attribute
// queries cost far more than a launch).  Entries are filled at most once per
// device by whichever call gets there first; a racing second fill stores the
// same values.
struct DeviceInfo {
  int cus, xccs;
};
using lisa::kMaxDevices;
std::atomic<int> g_dev_cus[kMaxDevices];
std::atomic<int> g_dev_xccs[kMaxDevices];

bool device_info(DeviceInfo& info) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev < kMaxDevices) {
    info.cus = g_dev_cus[dev].load(std::memory_order_relaxed);
    info.xccs = g_dev_xccs[dev].load(std::memory_order_relaxed);
    if (info.cus > 0) return true;
  }
  int cus = 0, xccs = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return false;
  if (hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess) xccs = 0;
  info.cus = cus;
  info.xccs = xccs;
  if (dev < kMaxDevices) {
    g_dev_xccs[dev].store(xccs, std::memory_order_relaxed);
    g_dev_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return true;
}
constexpr size_t kMaxSlices = 65535;  // batch * heads limit

size_t up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  int BH = 0, n = 0, H = 0, W = 0, T = 0, dtype = 0, heads = 0, feature = 0, schedule = 0;
  size_t esize = 0;
  int gmax = 1;                                  // ranks per slice the partials are sized for
  int grid = 0;                                  // workgroups (one per compute unit)
  int G = 1, S = 1, Z = 1, xcd_groups = 0;       // ranks per slice, groups, slices per round
  int chunk = 0;                                 // tokens per KV / M stage
  int TR = 0, TC = 0, tiles_x = 0, ntiles = 0;   // output tiles per slice
  // workspace layout (byte offsets)
  size_t slice_cnt = 0, sub_cnt = 0, done_cnt = 0, part_s = 0, part_kv = 0, part_m = 0, fin_s = 0, fin_kv = 0,
         fin_m = 0, frag_kv = 0, frag_m = 0, total = 0;
  // backward regions, after the forward's (lisa_backward_workspace_size)
  int nblk = 0;
  size_t b_pk = 0, b_tok = 0, b_dp = 0, b_da = 0, b_das = 0, b_dmkv = 0, b_ds = 0, btotal = 0;
};

lisa_status check_problem(const lisa_problem* p) {
  if (!p) return LISA_ERR_NULL;
  if (p->dtype != LISA_FP32 && p->dtype != LISA_BF16) return LISA_ERR_DTYPE;
  if (p->batch <= 0 || p->heads <= 0 || p->grid_h <= 0 || p->grid_w <= 0 || p->d_h <= 0 ||
      p->d_v <= 0)
    return LISA_ERR_SHAPE;
  if ((int64_t)p->grid_h * p->grid_w > (int64_t(1) << 24)) return LISA_ERR_SHAPE;
  if (p->d_h != kD || p->d_v != kD) return LISA_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->heads > (int64_t)kMaxSlices) return LISA_ERR_UNSUPPORTED;
  if (p->T < 1 || p->T > lisa::kMaxT) return LISA_ERR_PARAM;
  if (!std::isfinite(p->eps) || !(p->eps > 0.f)) return LISA_ERR_PARAM;
  if (p->feature != LISA_FEATURE_RELU && p->feature != LISA_FEATURE_ELU) return LISA_ERR_PARAM;
  if (p->schedule != LISA_SCHEDULE_AUTO && p->schedule != LISA_SCHEDULE_STREAMING &&
      p->schedule != LISA_SCHEDULE_RESIDENT)
    return LISA_ERR_PARAM;
  return LISA_OK;
}

// The streaming kernel's output tiles (lisa::flow_plan_tiles).
bool plan_tiles(Plan& pl, bool per_token_weights) {
  lisa::FlowTiles ft;
  if (!lisa::flow_plan_tiles(pl.H, pl.W, per_token_weights ? pl.T : 0, (int)pl.esize, ft)) return false;
  pl.TR = ft.TR;
  pl.TC = ft.TC;
  pl.tiles_x = ft.tiles_x;
  pl.ntiles = ft.ntiles;
  return true;
}

// Workgroups per slice: kRoundSlices times as many as there are workgroups
// per slice of the grid (so that a group has that many slices to
// interleave), at most one per 128 tokens and kMaxRanks, rounded down to a
// power of two (the combine splits the 8192 statistics evenly).  One slice
// per group won over two on every workload measured: fewer ranks per slice
// write fewer partials and wait for fewer arrivals, which outweighs the
// overlap of one slice's waits with another's stages (PVT stage 1, G = 8
// vs 16: 49.3 vs 50.4 us; DeiT-T 384: 63.1 vs 67.5 us).
#ifndef LISA_ROUND_SLICES
#define LISA_ROUND_SLICES 1
#endif
constexpr int kRoundSlices = LISA_ROUND_SLICES;

int plan_ranks(int grid, int BH, int n) { return lisa::flow_plan_ranks(grid, BH, n, kRoundSlices); }

// The forward's regions of a workspace, from offset 0: the launch counters
// first, sized for `counter_slices` slices, at offsets and sizes that do not
// depend on the problem (a workspace reused by problems of other shapes
// never has another problem's data written over a counter; each call leaves
// them at zero); then the rank partials for pl.gmax ranks per slice and the
// statistics.  Sets pl.total and returns it.
size_t layout_forward(Plan& pl, size_t counter_slices) {
  const size_t BH = pl.BH, G = pl.gmax;
  const size_t mat = kD * kD * sizeof(float), vec = kD * sizeof(float);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = up(o + bytes, kAlign);
    return at;
  };
  // Line 0: finished workgroups, the stall flag (word 1), rank tickets (words
  // 8..15); lines 1..8: finished workgroups per XCD (the resident kernel).
  pl.done_cnt = take((1 + lisa::kXcds) * lisa::kCntStride * sizeof(unsigned));
  pl.slice_cnt = take(counter_slices * lisa::kCntStride * sizeof(unsigned));
  pl.sub_cnt = take((size_t)lisa::kMaxSubSlices * 3 * lisa::kMaxSubs * lisa::kCntStride * sizeof(unsigned));
  pl.part_s = take(BH * G * vec);
  pl.part_kv = take(BH * G * mat);
  pl.part_m = take(BH * G * mat);
  pl.fin_s = take(BH * vec);
  pl.fin_kv = take(BH * mat);
  pl.fin_m = take(BH * mat);
  pl.frag_kv = take(BH * kD * kD * pl.esize);
  pl.frag_m = take(BH * kD * kD * pl.esize);
  pl.total = o;
  return o;
}

lisa_status make_plan(const lisa_problem* p, Plan& pl) {
  const lisa_status st = check_problem(p);
  if (st != LISA_OK) return st;
  pl.BH = p->batch * p->heads;
  pl.heads = p->heads;
  pl.H = p->grid_h;
  pl.W = p->grid_w;
  pl.n = p->grid_h * p->grid_w;
  pl.T = p->T;
  pl.dtype = p->dtype;
  pl.feature = p->feature;
  pl.schedule = p->schedule;
  pl.esize = p->dtype == LISA_BF16 ? 2 : 4;
  // The partials are sized for the most ranks any grid can give a slice
  // (the launch picks G <= gmax from the device's compute units).
  pl.gmax = plan_ranks(lisa::kMaxRanks, kRoundSlices, pl.n);
  // KV / M stages: one staging buffer holds a chunk's K rows and V (or Q)
  // rows (a multiple of 16 tokens: the MFMA sweep reads whole 16-row steps).
  pl.chunk = pl.esize == 2 ? lisa::Lds<2>::kChunk : lisa::Lds<4>::kChunk;

  size_t o = layout_forward(pl, kMaxSlices);
  const size_t BH = pl.BH;
  const size_t mat = kD * kD * sizeof(float), vec = kD * sizeof(float);
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = up(o + bytes, kAlign);
    return at;
  };
  // Backward: P_1..P_(T-1); per-token scalars; per-workgroup partials of dP_k,
  // dalpha and ds; each slice's dalpha, dM and dKV.
  const size_t T1 = pl.T > 1 ? (size_t)pl.T - 1 : 1;
  pl.nblk = (pl.n + lisa::kBwdTokens - 1) / lisa::kBwdTokens;
  const size_t nb = pl.nblk;
  pl.b_pk = take(BH * T1 * mat);
  pl.b_tok = take(BH * pl.n * 4 * sizeof(float));
  pl.b_dp = take(BH * nb * T1 * mat);
  pl.b_da = take(BH * nb * sizeof(float));
  pl.b_das = take(BH * sizeof(float));
  pl.b_dmkv = take(BH * 2 * mat);
  pl.b_ds = take(BH * nb * vec);
  pl.btotal = o;
  return LISA_OK;
}

bool misaligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

lisa_status check_workspace(const Plan& pl, const void* ws, size_t bytes) {
  if (!ws || bytes < pl.total || misaligned(ws, kAlign)) return LISA_ERR_WORKSPACE;
  return LISA_OK;
}

// Checks shared by lisa_forward and lisa_apply.
lisa_status check_forward(const lisa_problem* p, const void* Q, const void* K, const void* V,
                          const float* weights, float beta, const float* alpha, void* Y,
                          void* ws, size_t ws_bytes, Plan& pl) {
  lisa_status st = make_plan(p, pl);
  if (st != LISA_OK) return st;
  if (!weights && !(beta >= 0.f && beta < 1.f)) return LISA_ERR_PARAM;
  if (!Q || !K || !V || !alpha || !Y) return LISA_ERR_NULL;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(Y, 16) ||
      misaligned(weights, 4) || misaligned(alpha, 4))
    return LISA_ERR_ALIGN;
  st = check_workspace(pl, ws, ws_bytes);
  if (st != LISA_OK) return st;
  const size_t tensor = (size_t)pl.BH * pl.n * kD * pl.esize;
  if (overlaps(Y, tensor, Q, tensor) || overlaps(Y, tensor, K, tensor) ||
      overlaps(Y, tensor, V, tensor) || overlaps(Y, tensor, ws, pl.total))
    return LISA_ERR_PARAM;
  return LISA_OK;
}

enum class Mode { kForward, kReduce, kApply };

// Whether the resident kernel takes the problem, and its tiling: bf16 inputs,
// ReLU features, no predictor, at most kResMaxT walk terms, and a tiling
// whose tiles fit a workgroup (res_plan).  Ranks per slice: at most the
// compute units per slice, and at most the workspace's partials (one rank per
// 128 tokens).  The tiling does not depend on the weights or on the call
// (the weight region is always laid out), so lisa_forward, lisa_reduce,
// lisa_apply and the backward's statistics of one problem all cut the slices
// the same way and form the same fixed-order sums.
bool resident_fits(const Plan& pl, int cus, bool mlp, lisa::ResPlan& rp, bool* doubled = nullptr) {
  (void)mlp;  // the predictor runs inside the resident kernel too
  if (pl.dtype != LISA_BF16 || pl.feature != LISA_FEATURE_RELU || pl.T > lisa::kResMaxT) return false;
  const int gmax = plan_ranks(lisa::kMaxRanks, kRoundSlices, pl.n);
  const int gcap = std::min(std::max(1, cus / pl.BH), gmax);
  if (doubled) *doubled = false;
  if (lisa::res_plan(pl.H, pl.W, pl.T, true, gcap, rp)) return true;
  // Slices too large for one tile at the ranks the grid gives each (DeiT-T
  // 384: 192 slices of 24 x 24 on 256 CUs): twice the ranks, the groups then
  // taking the slices in two rounds.
  if (doubled) *doubled = true;
  return 2 * gcap <= gmax && lisa::res_plan(pl.H, pl.W, pl.T, true, 2 * gcap, rp);
}

// The default between the two kernels where both apply: the resident one,
// also where its tiles fit only with twice the ranks (two rounds of slices
// per group).  Measured on MI355X (256 CUs, bf16), forward of one call,
// resident against streaming: PVT-T stage 1 (32 slices of 56 x 56, T = 3)
// 38.1 / 45.6 us; DeiT-T at 224 (192 slices of 14 x 14, T = 3) 20.3 / 37.1
// us; DeiT-T at 384 (192 slices of 24 x 24, twice the ranks) 55.4 / 57.8 us;
// one 200 x 320 slice (T = 5) 36.0 / 46.6 us; one 128 x 128 slice 25.5 /
// 34.0 us; one 256 x 256 slice 34.0 / 46.8 us; one 64 x 64 slice 24.0 /
// 27.2 us.
bool resident_preferred(const lisa::ResPlan&, bool) { return true; }

// Whether the resident kernel runs the problem: where it fits, when asked
// for, and by default where it is the faster of the two kernels.
bool resident_plan(const Plan& pl, int cus, bool mlp, lisa::ResPlan& rp) {
  bool doubled = false;
  if (pl.schedule == LISA_SCHEDULE_STREAMING || !resident_fits(pl, cus, mlp, rp, &doubled)) return false;
  if (pl.schedule == LISA_SCHEDULE_RESIDENT) return true;
  return resident_preferred(rp, doubled);
}

// One launch of the resident kernel, one workgroup per compute unit.
lisa_status run_resident(const Plan& pl, const lisa::ResPlan& rp, int cus, Mode mode, const void* Q, const void* K,
                         const void* V, const float* weights, float beta, const float* alpha, void* Y, char* ws,
                         float eps, hipStream_t s, bool clear_err, unsigned long long* stamps = nullptr,
                         const lisa_weight_mlp* mlp = nullptr, const void* mlp_frag = nullptr,
                         const void* wo = nullptr, const float* bo = nullptr) {
  lisa::ResArgs a{};
  a.stamps = stamps;
  if (mode == Mode::kForward) {
    a.wo = wo;
    a.bo = bo;
  }
  if (mlp) {
    a.mlp_w1f = mlp_frag;
    a.mlp_b1 = mlp->b1;
    a.mlp_w2 = mlp->w2;
    a.mlp_b2 = mlp->b2;
    a.hidden = mlp->hidden;
  }
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.weights = weights;
  a.alpha = alpha;
  a.Y = Y;
  const double b = weights ? 0.0 : (double)beta;
  const double norm = (1.0 - b) / (1.0 - std::pow(b, pl.T));
  for (int k = 0; k < lisa::kMaxT; ++k) a.geo[k] = k < pl.T ? (float)(norm * std::pow(b, k)) : 0.f;
  a.n = pl.n;
  a.heads = pl.heads;
  a.BH = pl.BH;
  a.eps = eps;
  a.logit_scale = (float)(1.4426950408889634 / std::sqrt((double)kD));
  a.p = rp;
  a.S = cus / rp.G;
  a.mode = mode == Mode::kForward ? lisa::kResForward : mode == Mode::kReduce ? lisa::kResReduce : lisa::kResApply;
  a.do_kv = (mode == Mode::kReduce || (mode == Mode::kForward && pl.T >= 2)) ? 1 : 0;
  a.do_m = (mode == Mode::kReduce || (mode == Mode::kForward && pl.T >= 3)) ? 1 : 0;
  a.per_token = (weights != nullptr || mlp != nullptr) ? 1 : 0;
  a.grouped = (rp.G >= 64 && pl.BH <= lisa::kMaxSubSlices) ? 1 : 0;
  a.part_s = reinterpret_cast<float*>(ws + pl.part_s);
  // The rank partials as one [BH][G][2][64*64] array over the two partial
  // regions, which layout_forward places back to back (G <= gmax).
  if (pl.part_m != pl.part_kv + (size_t)pl.BH * pl.gmax * kD * kD * sizeof(float)) return LISA_ERR_WORKSPACE;
  a.part_kv = reinterpret_cast<float*>(ws + pl.part_kv);
  a.fin_s = reinterpret_cast<float*>(ws + pl.fin_s);
  a.fin_kv = reinterpret_cast<float*>(ws + pl.fin_kv);
  a.fin_m = reinterpret_cast<float*>(ws + pl.fin_m);
  a.frag_kv = ws + pl.frag_kv;
  a.frag_m = ws + pl.frag_m;
  a.slice_cnt = reinterpret_cast<unsigned*>(ws + pl.slice_cnt);
  a.sub_cnt = reinterpret_cast<unsigned*>(ws + pl.sub_cnt);
  a.done_cnt = reinterpret_cast<unsigned*>(ws + pl.done_cnt);
  a.done_xcd = a.done_cnt + lisa::kCntStride;
  a.err = a.done_cnt + 1;
  a.tickets = a.done_cnt + 8;
  a.clear_err = clear_err ? 1 : 0;
  if (lisa::launch_resident(a, cus, s) != hipSuccess) return LISA_ERR_HIP;
  return LISA_OK;
}

// One launch of the persistent kernel, one workgroup per compute unit.
lisa_status run(Plan pl, Mode mode, const void* Q, const void* K, const void* V,
                const float* weights, float beta, const float* alpha, void* Y, char* ws, float eps,
                hipStream_t s, const lisa_weight_mlp* mlp = nullptr, const void* mlp_frag = nullptr,
                bool clear_err = false, unsigned long long* stamps = nullptr, const void* wo = nullptr,
                const float* bo = nullptr) {
  lisa::FlowArgs a{};
  a.clear_err = clear_err ? 1 : 0;
  if (mlp) {
    a.mlp_w1f = mlp_frag;
    a.mlp_b1 = mlp->b1;
    a.mlp_w2 = mlp->w2;
    a.mlp_b2 = mlp->b2;
    a.hidden = mlp->hidden;
  }
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.weights = weights;
  a.alpha = alpha;
  a.Y = Y;
  // Geometric weights w_k = (1-beta) beta^k / (1-beta^T) in double, rounded once.
  const double b = weights ? 0.0 : (double)beta;
  const double norm = (1.0 - b) / (1.0 - std::pow(b, pl.T));
  for (int k = 0; k < lisa::kMaxT; ++k) a.geo[k] = k < pl.T ? (float)(norm * std::pow(b, k)) : 0.f;
  a.H = pl.H;
  a.W = pl.W;
  a.n = pl.n;
  a.T = pl.T;
  a.heads = pl.heads;
  a.BH = pl.BH;
  a.eps = eps;
  a.logit_scale = (float)(1.4426950408889634 / std::sqrt((double)kD));
  // One persistent workgroup per compute unit.
  DeviceInfo dinfo;
  if (!device_info(dinfo)) return LISA_ERR_HIP;
  lisa::ResPlan rp;
  if (resident_plan(pl, dinfo.cus, mlp != nullptr, rp))
    return run_resident(pl, rp, dinfo.cus, mode, Q, K, V, weights, beta, alpha, Y, ws, eps, s, clear_err, stamps,
                        mlp, mlp_frag, wo, bo);
  if (wo) return LISA_ERR_UNSUPPORTED;  // the folded projection is the resident kernel's
  if (pl.schedule == LISA_SCHEDULE_RESIDENT) return LISA_ERR_UNSUPPORTED;  // asked for, not applicable
  if (stamps) return LISA_ERR_UNSUPPORTED;  // the stage timeline is the resident kernel's
  if (!plan_tiles(pl, weights != nullptr || mlp != nullptr)) return LISA_ERR_UNSUPPORTED;
  pl.grid = dinfo.cus;
  const lisa::FlowGroups fg = lisa::flow_plan_groups(pl.grid, dinfo.xccs, pl.BH, pl.n, pl.gmax, kRoundSlices);
  pl.G = fg.G;
  pl.S = fg.S;
  pl.Z = fg.Z;
  pl.xcd_groups = fg.xcd_groups;
  a.chunk = pl.chunk;
  a.G = pl.G;
  a.S = pl.S;
  a.Z = pl.Z;
  a.xcd_groups = pl.xcd_groups;
  a.TR = pl.TR;
  a.TC = pl.TC;
  a.tiles_x = pl.tiles_x;
  a.ntiles = pl.ntiles;
  a.do_kv = (mode == Mode::kReduce || (mode == Mode::kForward && pl.T >= 2)) ? 1 : 0;
  a.do_m = (mode == Mode::kReduce || (mode == Mode::kForward && pl.T >= 3)) ? 1 : 0;
  a.do_out = mode == Mode::kReduce ? 0 : 1;
  a.part_s = reinterpret_cast<float*>(ws + pl.part_s);
  a.part_kv = reinterpret_cast<float*>(ws + pl.part_kv);
  a.part_m = reinterpret_cast<float*>(ws + pl.part_m);
  a.fin_s = reinterpret_cast<float*>(ws + pl.fin_s);
  a.fin_kv = reinterpret_cast<float*>(ws + pl.fin_kv);
  a.fin_m = reinterpret_cast<float*>(ws + pl.fin_m);
  a.frag_kv = ws + pl.frag_kv;
  a.frag_m = ws + pl.frag_m;
  a.slice_cnt = reinterpret_cast<unsigned*>(ws + pl.slice_cnt);
  a.sub_cnt = reinterpret_cast<unsigned*>(ws + pl.sub_cnt);
  // Kernel variant (bf16 without the predictor): arrivals per group of
  // kSubRanks ranks from 64 ranks per slice on (with 32 the one counter
  // measured faster); with one rank per slice, a combine that writes the
  // statistics in whole rows and fragment lanes.
  // The ELU feature map has kernels of its own (plain arrivals and combine).
  const bool variants = pl.dtype == LISA_BF16 && !mlp;
  a.variant = pl.feature == LISA_FEATURE_ELU                             ? lisa::kVarElu
              : (variants && pl.G >= 64 && pl.BH <= lisa::kMaxSubSlices) ? lisa::kVarGrouped
              : (variants && pl.G == 1)                                 ? lisa::kVarSolo
                                                                        : lisa::kVarPlain;
  a.done_cnt = reinterpret_cast<unsigned*>(ws + pl.done_cnt);
  a.err = a.done_cnt + 1;
  a.tickets = a.done_cnt + 8;
  if (lisa::launch_flow(pl.dtype, a, pl.grid, s) != hipSuccess) return LISA_ERR_HIP;
  return LISA_OK;
}

// ---------------------------------------------------------------------------
// Fixed scratch of lisa_forward_noalloc: the launch counters, rank partials
// and statistics that lisa_forward keeps in the caller's workspace live in
// this array instead.  Each device that runs the library holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: the device address of the current device's copy comes
// from hipGetSymbolAddress, once per device, and only that address is used.
// The array is zero when the code object loads, and every completed call
// leaves its counters (and, for this entry point, the stall flag) at zero.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr size_t kScratchSlices = 8192;  // (batch, head) slices its counters cover
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<char*> g_scratch[kMaxDevices];

// The current device's copy of `scratch` (looked up on the device's first
// call; a racing second lookup stores the same address).
lisa_status scratch_address(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LISA_ERR_HIP;
  if (dev < kMaxDevices) {
    char* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) {
      *out = p;
      return LISA_OK;
    }
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return LISA_ERR_HIP;
  if (dev < kMaxDevices) g_scratch[dev].store(static_cast<char*>(ptr), std::memory_order_release);
  *out = static_cast<char*>(ptr);
  return LISA_OK;
}

}  // namespace

extern "C" {

size_t lisa_workspace_size(const lisa_problem* p) {
  Plan pl;
  return make_plan(p, pl) == LISA_OK ? pl.total : 0;
}

lisa_status lisa_forward_schedule(const lisa_problem* p, int32_t* schedule) {
  Plan pl;
  const lisa_status st = make_plan(p, pl);
  if (st != LISA_OK) return st;
  if (!schedule) return LISA_ERR_NULL;
  DeviceInfo dinfo;
  if (!device_info(dinfo)) return LISA_ERR_HIP;
  lisa::ResPlan rp;
  if (resident_plan(pl, dinfo.cus, false, rp)) {
    *schedule = LISA_SCHEDULE_RESIDENT;
    return LISA_OK;
  }
  if (pl.schedule == LISA_SCHEDULE_RESIDENT) return LISA_ERR_UNSUPPORTED;
  *schedule = LISA_SCHEDULE_STREAMING;
  return LISA_OK;
}

lisa_status lisa_forward(const lisa_problem* p, const void* Q, const void* K, const void* V,
                         const float* weights, float beta, const float* alpha, void* Y,
                         void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  const lisa_status st = check_forward(p, Q, K, V, weights, beta, alpha, Y, workspace, workspace_bytes, pl);
  if (st != LISA_OK) return st;
  (void)hipGetLastError();  // clear a stale error so that ours are reported alone
  return run(pl, Mode::kForward, Q, K, V, weights, beta, alpha, Y, static_cast<char*>(workspace),
             p->eps, static_cast<hipStream_t>(stream));
}

lisa_status lisa_forward_phases(const lisa_problem* p, const void* Q, const void* K, const void* V,
                                const float* weights, float beta, const float* alpha, void* Y, void* workspace,
                                size_t workspace_bytes, uint64_t* stamps, size_t stamps_count, void* stream) {
  Plan pl;
  const lisa_status st = check_forward(p, Q, K, V, weights, beta, alpha, Y, workspace, workspace_bytes, pl);
  if (st != LISA_OK) return st;
  if (!stamps) return LISA_ERR_NULL;
  if (misaligned(stamps, 8)) return LISA_ERR_ALIGN;
  (void)hipGetLastError();
  DeviceInfo dinfo;
  if (!device_info(dinfo)) return LISA_ERR_HIP;
  if (stamps_count < (size_t)dinfo.cus * LISA_PHASES) return LISA_ERR_PARAM;
  // The timeline is the resident kernel's: it runs wherever it fits.
  if (pl.schedule == LISA_SCHEDULE_STREAMING) return LISA_ERR_UNSUPPORTED;
  pl.schedule = LISA_SCHEDULE_RESIDENT;
  lisa::ResPlan rp;
  if (!resident_plan(pl, dinfo.cus, false, rp)) return LISA_ERR_UNSUPPORTED;
  static_assert(LISA_PHASES == lisa::kResPhases, "stage count");
  return run(pl, Mode::kForward, Q, K, V, weights, beta, alpha, Y, static_cast<char*>(workspace), p->eps,
             static_cast<hipStream_t>(stream), nullptr, nullptr, false,
             reinterpret_cast<unsigned long long*>(stamps));
}

lisa_status lisa_forward_noalloc(const lisa_problem* p, const void* Q, const void* K, const void* V,
                                 const float* weights, float beta, const float* alpha, void* Y, void* stream) {
  Plan pl;
  lisa_status st = make_plan(p, pl);
  if (st != LISA_OK) return st;
  if (!weights && !(beta >= 0.f && beta < 1.f)) return LISA_ERR_PARAM;
  if (!Q || !K || !V || !alpha || !Y) return LISA_ERR_NULL;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(Y, 16) ||
      misaligned(weights, 4) || misaligned(alpha, 4))
    return LISA_ERR_ALIGN;
  const size_t tensor = (size_t)pl.BH * pl.n * kD * pl.esize;
  if (overlaps(Y, tensor, Q, tensor) || overlaps(Y, tensor, K, tensor) || overlaps(Y, tensor, V, tensor))
    return LISA_ERR_PARAM;
  if ((size_t)pl.BH > kScratchSlices) return LISA_ERR_SCRATCH;
  (void)hipGetLastError();
  // The partials for exactly the ranks this device's launch gives a slice
  // (run() picks the same number), not for the most any device could.
  DeviceInfo dinfo;
  if (!device_info(dinfo)) return LISA_ERR_HIP;
  lisa::ResPlan rp;
  pl.gmax = resident_plan(pl, dinfo.cus, false, rp) ? rp.G : plan_ranks(dinfo.cus, pl.BH, pl.n);
  if (layout_forward(pl, kScratchSlices) > kScratchBytes) return LISA_ERR_SCRATCH;
  char* base = nullptr;
  st = scratch_address(&base);
  if (st != LISA_OK) return st;
  return run(pl, Mode::kForward, Q, K, V, weights, beta, alpha, Y, base, p->eps, static_cast<hipStream_t>(stream),
             nullptr, nullptr, /*clear_err=*/true);
}

lisa_status lisa_reduce(const lisa_problem* p, const void* Q, const void* K, const void* V,
                        float* s_out, float* kv_out, float* m_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Plan pl;
  lisa_status st = make_plan(p, pl);
  if (st != LISA_OK) return st;
  if (!Q || !K || !V) return LISA_ERR_NULL;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(s_out, 4) ||
      misaligned(kv_out, 4) || misaligned(m_out, 4))
    return LISA_ERR_ALIGN;
  st = check_workspace(pl, workspace, workspace_bytes);
  if (st != LISA_OK) return st;
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  st = run(pl, Mode::kReduce, Q, K, V, nullptr, 0.f, nullptr, nullptr, ws, p->eps, s);
  if (st != LISA_OK) return st;
  const size_t mat = (size_t)pl.BH * kD * kD * sizeof(float), vec = (size_t)pl.BH * kD * sizeof(float);
  if (s_out && hipMemcpyAsync(s_out, ws + pl.fin_s, vec, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return LISA_ERR_HIP;
  if (kv_out && hipMemcpyAsync(kv_out, ws + pl.fin_kv, mat, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return LISA_ERR_HIP;
  if (m_out && hipMemcpyAsync(m_out, ws + pl.fin_m, mat, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return LISA_ERR_HIP;
  return LISA_OK;
}

lisa_status lisa_apply(const lisa_problem* p, const void* Q, const void* K, const void* V,
                       const float* weights, float beta, const float* alpha, void* Y,
                       void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  const lisa_status st = check_forward(p, Q, K, V, weights, beta, alpha, Y, workspace, workspace_bytes, pl);
  if (st != LISA_OK) return st;
  (void)hipGetLastError();
  return run(pl, Mode::kApply, Q, K, V, weights, beta, alpha, Y, static_cast<char*>(workspace), p->eps,
             static_cast<hipStream_t>(stream));
}

size_t lisa_forward_mlp_workspace_size(const lisa_problem* p, int32_t hidden) {
  Plan pl;
  if (make_plan(p, pl) != LISA_OK || pl.T > lisa::kMaxTBwd || pl.feature != LISA_FEATURE_RELU || hidden < 32 ||
      hidden > lisa::kMaxHidden ||
      hidden % 32 != 0)
    return 0;
  return up(pl.total, kAlign) + lisa::mlp_frag_bytes(pl.dtype, pl.heads, hidden);
}

lisa_status lisa_forward_mlp(const lisa_problem* p, const void* Q, const void* K, const void* V,
                             const lisa_weight_mlp* mlp, const float* alpha, void* Y, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!mlp) return LISA_ERR_NULL;
  Plan pl;
  lisa_status st = make_plan(p, pl);
  if (st != LISA_OK) return st;
  if (pl.T > lisa::kMaxTBwd) return LISA_ERR_PARAM;
  if (pl.feature != LISA_FEATURE_RELU) return LISA_ERR_UNSUPPORTED;
  if (mlp->hidden < 32 || mlp->hidden > lisa::kMaxHidden || mlp->hidden % 32 != 0) return LISA_ERR_PARAM;
  if (!mlp->w1 || !mlp->b1 || !mlp->w2 || !mlp->b2) return LISA_ERR_NULL;
  if (misaligned(mlp->w1, 4) || misaligned(mlp->b1, 4) || misaligned(mlp->w2, 4) || misaligned(mlp->b2, 4))
    return LISA_ERR_ALIGN;
  const size_t frag_at = up(pl.total, kAlign);
  const size_t need = frag_at + lisa::mlp_frag_bytes(pl.dtype, pl.heads, mlp->hidden);
  if (workspace_bytes < need) return LISA_ERR_WORKSPACE;
  st = check_forward(p, Q, K, V, nullptr, 0.f, alpha, Y, workspace, workspace_bytes, pl);
  if (st != LISA_OK) return st;
  const size_t tensor = (size_t)pl.BH * pl.n * kD * pl.esize;
  if (overlaps(Y, tensor, workspace, need)) return LISA_ERR_PARAM;
  (void)hipGetLastError();
  char* ws = static_cast<char*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (lisa::launch_mlp_prep(pl.dtype, mlp->w1, ws + frag_at, pl.heads, mlp->hidden, s) != hipSuccess)
    return LISA_ERR_HIP;
  return run(pl, Mode::kForward, Q, K, V, nullptr, 0.f, alpha, Y, ws, p->eps, s, mlp, ws + frag_at);
}

size_t lisa_attention_workspace_size(const lisa_problem* p) {
  Plan pl;
  if (make_plan(p, pl) != LISA_OK) return 0;
  const size_t tensor = up((size_t)pl.BH * pl.n * kD * pl.esize, kAlign);
  return up(pl.total, kAlign) + 4 * tensor;  // the operator's regions, then Q, K, V, O
}

lisa_status lisa_attention_forward(const lisa_problem* p, const void* X, const void* w_qkv,
                                   const float* b_qkv, const void* w_o, const float* b_o,
                                   const float* weights, float beta, const float* alpha, void* Y,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  lisa_status st = make_plan(p, pl);
  if (st != LISA_OK) return st;
  if (!weights && !(beta >= 0.f && beta < 1.f)) return LISA_ERR_PARAM;
  if (!X || !w_qkv || !b_qkv || !w_o || !b_o || !alpha || !Y) return LISA_ERR_NULL;
  if (misaligned(X, 16) || misaligned(w_qkv, 16) || misaligned(w_o, 16) || misaligned(Y, 16) ||
      misaligned(b_qkv, 4) || misaligned(b_o, 4) || misaligned(weights, 4) || misaligned(alpha, 4))
    return LISA_ERR_ALIGN;
  const size_t tensor = (size_t)pl.BH * pl.n * kD * pl.esize;  // one of Q, K, V, O; also X and Y
  const size_t at = up(pl.total, kAlign), step = up(tensor, kAlign);
  const size_t need = at + 4 * step;
  if (!workspace || workspace_bytes < need || misaligned(workspace, kAlign)) return LISA_ERR_WORKSPACE;
  if (overlaps(Y, tensor, X, tensor) || overlaps(Y, tensor, workspace, need) || overlaps(X, tensor, workspace, need))
    return LISA_ERR_PARAM;
  (void)hipGetLastError();
  char* ws = static_cast<char*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* q = ws + at;
  char* o = ws + at + 3 * step;
  lisa::ProjArgs pa{};
  pa.M = p->batch * pl.n;
  pa.K = pl.heads * kD;
  pa.n = pl.n;
  pa.heads = pl.heads;
  pa.head_elems = step / pl.esize;
  // [Q | K | V] = X Wqkv^T + bqkv, into the heads layout.
  pa.A = X;
  pa.Wt = w_qkv;
  pa.bias = b_qkv;
  pa.out = q;
  pa.N = 3 * pa.K;
  // One head on the resident kernel: the output projection is folded into
  // the operator's output stage (O never goes to HBM).
  bool fold = false;
  if (pl.heads == 1) {
    DeviceInfo dinfo;
    lisa::ResPlan rp;
    if (!device_info(dinfo)) return LISA_ERR_HIP;
    fold = resident_plan(pl, dinfo.cus, false, rp);
  }
  if (lisa::launch_proj(pl.dtype, false, pa, s) != hipSuccess) return LISA_ERR_HIP;
  if (fold)
    return run(pl, Mode::kForward, q, q + step, q + 2 * step, weights, beta, alpha, Y, ws, p->eps, s, nullptr,
               nullptr, false, nullptr, w_o, b_o);
  st = run(pl, Mode::kForward, q, q + step, q + 2 * step, weights, beta, alpha, o, ws, p->eps, s);
  if (st != LISA_OK) return st;
  // Y = concat_h(O_h) Wo^T + bo.
  pa.A = o;
  pa.Wt = w_o;
  pa.bias = b_o;
  pa.out = Y;
  pa.N = pa.K;
  if (lisa::launch_proj(pl.dtype, true, pa, s) != hipSuccess) return LISA_ERR_HIP;
  return LISA_OK;
}

size_t lisa_backward_workspace_size(const lisa_problem* p) {
  Plan pl;
  return make_plan(p, pl) == LISA_OK && pl.T <= lisa::kMaxTBwd && pl.feature == LISA_FEATURE_RELU ? pl.btotal : 0;
}

// The backward pass; with have_stats the slice statistics of a preceding
// forward (or reduce) of the same problem and inputs are taken from the
// workspace instead of recomputed, when that call formed all of them (T >= 3:
// with T < 3 the forward forms no M).
static lisa_status backward_common(const lisa_problem* p, const void* Q, const void* K, const void* V,
                                   const float* weights, float beta, const float* alpha, const void* dY,
                                   void* dQ, void* dK, void* dV, float* dweights, float* dalpha,
                                   void* workspace, size_t workspace_bytes, void* stream, bool have_stats) {
  Plan pl;
  lisa_status st = make_plan(p, pl);
  if (st != LISA_OK) return st;
  if (pl.T > lisa::kMaxTBwd) return LISA_ERR_PARAM;
  if (pl.feature != LISA_FEATURE_RELU) return LISA_ERR_UNSUPPORTED;
  if (!weights && !(beta >= 0.f && beta < 1.f)) return LISA_ERR_PARAM;
  if (!Q || !K || !V || !alpha || !dY || !dQ || !dK || !dV || !dalpha) return LISA_ERR_NULL;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(dY, 16) ||
      misaligned(dQ, 16) || misaligned(dK, 16) || misaligned(dV, 16) || misaligned(weights, 4) ||
      misaligned(alpha, 4) || misaligned(dweights, 4) || misaligned(dalpha, 4))
    return LISA_ERR_ALIGN;
  if (!workspace || workspace_bytes < pl.btotal || misaligned(workspace, kAlign)) return LISA_ERR_WORKSPACE;
  // Outputs overlap no input, no other output and not the workspace.
  const size_t tensor = (size_t)pl.BH * pl.n * kD * pl.esize;
  const size_t wbytes = (size_t)pl.BH * pl.n * pl.T * sizeof(float);
  const struct {
    const void* p;
    size_t n;
  } ins[] = {{Q, tensor}, {K, tensor}, {V, tensor}, {dY, tensor}, {weights, weights ? wbytes : 0},
             {alpha, (size_t)pl.heads * sizeof(float)}, {workspace, pl.btotal}},
    outs[] = {{dQ, tensor}, {dK, tensor}, {dV, tensor}, {dweights, dweights ? wbytes : 0},
              {dalpha, (size_t)pl.heads * sizeof(float)}};
  for (size_t o = 0; o < sizeof(outs) / sizeof(outs[0]); ++o) {
    for (const auto& in : ins)
      if (in.n && outs[o].n && overlaps(outs[o].p, outs[o].n, in.p, in.n)) return LISA_ERR_PARAM;
    for (size_t q = o + 1; q < sizeof(outs) / sizeof(outs[0]); ++q)
      if (outs[o].n && outs[q].n && overlaps(outs[o].p, outs[o].n, outs[q].p, outs[q].n)) return LISA_ERR_PARAM;
  }
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  // The slice statistics s, phi(K)^T V and M, as lisa_reduce forms them.
  if (!(have_stats && pl.T >= 3)) {
    st = run(pl, Mode::kReduce, Q, K, V, nullptr, 0.f, nullptr, nullptr, ws, p->eps, s);
    if (st != LISA_OK) return st;
  }
  lisa::BwdArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.dY = dY;
  a.weights = weights;
  a.alpha = alpha;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.dweights = weights ? dweights : nullptr;
  a.dalpha = dalpha;
  const double b = weights ? 0.0 : (double)beta;
  const double norm = (1.0 - b) / (1.0 - std::pow(b, pl.T));
  for (int k = 0; k < lisa::kMaxTBwd; ++k) a.geo[k] = k < pl.T ? (float)(norm * std::pow(b, k)) : 0.f;
  a.H = pl.H;
  a.W = pl.W;
  a.n = pl.n;
  a.T = pl.T;
  a.heads = pl.heads;
  a.BH = pl.BH;
  a.nblk = pl.nblk;
  a.eps = p->eps;
  a.fin_s = reinterpret_cast<const float*>(ws + pl.fin_s);
  a.fin_kv = reinterpret_cast<const float*>(ws + pl.fin_kv);
  a.fin_m = reinterpret_cast<const float*>(ws + pl.fin_m);
  a.pk = reinterpret_cast<float*>(ws + pl.b_pk);
  a.tok = reinterpret_cast<float4*>(ws + pl.b_tok);
  a.dp_part = reinterpret_cast<float*>(ws + pl.b_dp);
  a.da_part = reinterpret_cast<float*>(ws + pl.b_da);
  a.da_slice = reinterpret_cast<float*>(ws + pl.b_das);
  a.dmkv = reinterpret_cast<float*>(ws + pl.b_dmkv);
  a.ds_part = reinterpret_cast<float*>(ws + pl.b_ds);
  if (lisa::launch_backward(pl.dtype, a, s) != hipSuccess) return LISA_ERR_HIP;
  return LISA_OK;
}

lisa_status lisa_workspace_check(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return LISA_ERR_NULL;
  if (workspace_bytes < 256 || misaligned(workspace, kAlign)) return LISA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The stall flag: word 1 of the launch counters at offset 0 (the kernel's
  // error word, raised by an abandoned dependency wait).
  unsigned* flag = static_cast<unsigned*>(workspace) + 1;
  unsigned v = 0;
  if (hipMemcpyAsync(&v, flag, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return LISA_ERR_HIP;
  if (v == 0) return LISA_OK;
  if (hipMemsetAsync(flag, 0, sizeof(unsigned), s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return LISA_ERR_HIP;
  return LISA_ERR_STALLED;
}

lisa_status lisa_backward(const lisa_problem* p, const void* Q, const void* K, const void* V,
                          const float* weights, float beta, const float* alpha, const void* dY, void* dQ,
                          void* dK, void* dV, float* dweights, float* dalpha, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return backward_common(p, Q, K, V, weights, beta, alpha, dY, dQ, dK, dV, dweights, dalpha, workspace,
                         workspace_bytes, stream, false);
}

lisa_status lisa_backward_after_forward(const lisa_problem* p, const void* Q, const void* K, const void* V,
                                        const float* weights, float beta, const float* alpha, const void* dY,
                                        void* dQ, void* dK, void* dV, float* dweights, float* dalpha,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return backward_common(p, Q, K, V, weights, beta, alpha, dY, dQ, dK, dV, dweights, dalpha, workspace,
                         workspace_bytes, stream, true);
}

const char* lisa_status_str(lisa_status s) {
  switch (s) {
    case LISA_OK: return "ok";
    case LISA_ERR_NULL: return "a required pointer is NULL";
    case LISA_ERR_SHAPE: return "a dimension is <= 0 or too large";
    case LISA_ERR_PARAM: return "invalid parameter (T, beta, eps) or Y overlaps an input";
    case LISA_ERR_DTYPE: return "unknown dtype";
    case LISA_ERR_UNSUPPORTED: return "unsupported shape (d_h and d_v must be 64, batch*heads <= 65535)";
    case LISA_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case LISA_ERR_ALIGN: return "misaligned pointer (Q, K, V, Y need 16 bytes; fp32 arrays 4)";
    case LISA_ERR_HIP: return "a HIP launch or copy failed";
    case LISA_ERR_STALLED: return "a call abandoned a dependency wait; its outputs are undefined";
    case LISA_ERR_SCRATCH:
      return "problem too large for lisa_forward_noalloc's fixed 32 MiB scratch (at most 8192 slices)";
  }
  return "unknown status";
}

}  // extern "C"
