// Host side of liblisa.so: argument checks, planning, workspace layout and
// launch sequencing for the C ABI declared in include/lisa.h.  Nothing here
// touches the GPU before every argument has been checked.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "lisa.h"
#include "lisa_kernels.hpp"

namespace {

using lisa::kCellStride;
using lisa::kCntWords;
using lisa::kD;
using lisa::kGroup;
using lisa::kMaxChunks;
using lisa::kStatTile;

constexpr size_t kAlign = 256;
constexpr size_t kMaxOutLds = 64 * 1024;

size_t up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  int BH = 0, n = 0, H = 0, W = 0, T = 0, dtype = 0, heads = 0;
  size_t esize = 0;
  // statistics sweeps
  int chunk = 0, P = 0, ngroups = 0;
  // output tiles
  int TR = 0, TC = 0, tiles_x = 0, ntiles = 0;
  size_t lds = 0;
  // workspace layout (byte offsets)
  size_t cnt_kv = 0, cnt_m = 0, part_s = 0, part_kv = 0, part_m = 0, gpart_s = 0, gpart_kv = 0,
         gpart_m = 0, fin_s = 0, fin_kv = 0, fin_m = 0, frag_kv = 0, frag_m = 0, total = 0;
};

lisa_status check_problem(const lisa_problem* p) {
  if (!p) return LISA_ERR_NULL;
  if (p->dtype != LISA_FP32 && p->dtype != LISA_BF16) return LISA_ERR_DTYPE;
  if (p->batch <= 0 || p->heads <= 0 || p->grid_h <= 0 || p->grid_w <= 0 || p->d_h <= 0 ||
      p->d_v <= 0)
    return LISA_ERR_SHAPE;
  if ((int64_t)p->grid_h * p->grid_w > (int64_t(1) << 24)) return LISA_ERR_SHAPE;
  if (p->d_h != kD || p->d_v != kD) return LISA_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->heads > 65535) return LISA_ERR_UNSUPPORTED;
  if (p->T < 1 || p->T > lisa::kMaxT) return LISA_ERR_PARAM;
  if (!std::isfinite(p->eps) || !(p->eps > 0.f)) return LISA_ERR_PARAM;
  return LISA_OK;
}

// Output tile: whole grid rows when the grid is at most 64 wide, else
// 32-column strips; as many rows as fit the LDS budget (tile plus one-cell
// halo of K and V), at most 256 tokens.
void plan_tiles(Plan& pl) {
  const size_t cell_bytes = 2 * kCellStride * pl.esize;  // K and V
  const int max_cells = (int)(kMaxOutLds / cell_bytes);
  pl.TC = pl.W <= 64 ? pl.W : 32;
  if (pl.TC > max_cells / 3 - 2) pl.TC = max_cells / 3 - 2;  // at least one row with halo
  int tr = max_cells / (pl.TC + 2) - 2;
  if (tr < 1) tr = 1;
  while (tr > 1 && tr * pl.TC > 256) --tr;
  if (tr > pl.H) tr = pl.H;
  pl.TR = tr;
  pl.tiles_x = (pl.W + pl.TC - 1) / pl.TC;
  const int tiles_y = (pl.H + pl.TR - 1) / pl.TR;
  pl.ntiles = pl.tiles_x * tiles_y;
  pl.lds = (size_t)(pl.TR + 2) * (pl.TC + 2) * cell_bytes;
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
  pl.esize = p->dtype == LISA_BF16 ? 2 : 4;

  // Statistics chunks: 256 tokens per workgroup, larger when a slice would
  // need more than kMaxChunks chunks.
  int chunk = 256;
  if ((pl.n + chunk - 1) / chunk > kMaxChunks) {
    chunk = (pl.n + kMaxChunks - 1) / kMaxChunks;
    chunk = (chunk + kStatTile - 1) / kStatTile * kStatTile;
  }
  pl.chunk = chunk;
  pl.P = (pl.n + chunk - 1) / chunk;
  pl.ngroups = (pl.P + kGroup - 1) / kGroup;
  plan_tiles(pl);

  const size_t BH = pl.BH, P = pl.P, NG = pl.ngroups > 1 ? pl.ngroups : 0;
  const size_t mat = kD * kD * sizeof(float), vec = kD * sizeof(float);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = up(o + bytes, kAlign);
    return at;
  };
  pl.cnt_kv = take(BH * kCntWords * sizeof(unsigned));
  pl.cnt_m = take(BH * kCntWords * sizeof(unsigned));
  pl.part_s = take(BH * P * vec);
  pl.part_kv = take(BH * P * mat);
  pl.part_m = take(BH * P * mat);
  pl.gpart_s = take(BH * NG * vec);
  pl.gpart_kv = take(BH * NG * mat);
  pl.gpart_m = take(BH * NG * mat);
  pl.fin_s = take(BH * vec);
  pl.fin_kv = take(BH * mat);
  pl.fin_m = take(BH * mat);
  pl.frag_kv = take(BH * kD * kD * pl.esize);
  pl.frag_m = take(BH * kD * kD * pl.esize);
  pl.total = o;
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

lisa::StatsArgs stats_args(const Plan& pl, char* ws, const void* K, const void* X, float eps,
                           bool m_stage) {
  lisa::StatsArgs a{};
  a.K = K;
  a.X = X;
  a.n = pl.n;
  a.chunk = pl.chunk;
  a.P = pl.P;
  a.ngroups = pl.ngroups;
  a.eps = eps;
  a.part = reinterpret_cast<float*>(ws + (m_stage ? pl.part_m : pl.part_kv));
  a.part_s = reinterpret_cast<float*>(ws + pl.part_s);
  a.gpart = reinterpret_cast<float*>(ws + (m_stage ? pl.gpart_m : pl.gpart_kv));
  a.gpart_s = reinterpret_cast<float*>(ws + pl.gpart_s);
  a.s_in = reinterpret_cast<const float*>(ws + pl.fin_s);
  a.fin = reinterpret_cast<float*>(ws + (m_stage ? pl.fin_m : pl.fin_kv));
  a.fin_s = reinterpret_cast<float*>(ws + pl.fin_s);
  a.frag = ws + (m_stage ? pl.frag_m : pl.frag_kv);
  a.cnt = reinterpret_cast<unsigned*>(ws + (m_stage ? pl.cnt_m : pl.cnt_kv));
  return a;
}

lisa_status run_stats(const Plan& pl, const void* Q, const void* K, const void* V, char* ws,
                      float eps, bool need_m, hipStream_t s) {
  if (lisa::launch_stats_kv(pl.dtype, stats_args(pl, ws, K, V, eps, false), pl.BH, s) != hipSuccess)
    return LISA_ERR_HIP;
  if (need_m &&
      lisa::launch_stats_m(pl.dtype, stats_args(pl, ws, K, Q, eps, true), pl.BH, s) != hipSuccess)
    return LISA_ERR_HIP;
  return LISA_OK;
}

lisa_status run_output(const Plan& pl, const void* Q, const void* K, const void* V,
                       const float* weights, float beta, const float* alpha, void* Y, char* ws,
                       float eps, hipStream_t s) {
  lisa::OutArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.weights = weights;
  a.alpha = alpha;
  a.Y = Y;
  a.s = reinterpret_cast<const float*>(ws + pl.fin_s);
  a.frag_kv = ws + pl.frag_kv;
  a.frag_m = ws + pl.frag_m;
  // Geometric weights w_k = (1-beta) beta^k / (1-beta^T) in double, rounded once.
  const double b = weights ? 0.0 : (double)beta;
  const double norm = (1.0 - b) / (1.0 - std::pow(b, pl.T));
  for (int k = 0; k < lisa::kMaxT; ++k) a.geo[k] = k < pl.T ? (float)(norm * std::pow(b, k)) : 0.f;
  a.H = pl.H;
  a.W = pl.W;
  a.n = pl.n;
  a.T = pl.T;
  a.heads = pl.heads;
  a.TR = pl.TR;
  a.TC = pl.TC;
  a.tiles_x = pl.tiles_x;
  a.eps = eps;
  a.logit_scale = (float)(1.4426950408889634 / std::sqrt((double)kD));
  if (lisa::launch_output(pl.dtype, a, pl.BH, pl.ntiles, pl.lds, s) != hipSuccess) return LISA_ERR_HIP;
  return LISA_OK;
}

}  // namespace

extern "C" {

size_t lisa_workspace_size(const lisa_problem* p) {
  Plan pl;
  return make_plan(p, pl) == LISA_OK ? pl.total : 0;
}

lisa_status lisa_forward(const lisa_problem* p, const void* Q, const void* K, const void* V,
                         const float* weights, float beta, const float* alpha, void* Y,
                         void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  lisa_status st = check_forward(p, Q, K, V, weights, beta, alpha, Y, workspace, workspace_bytes, pl);
  if (st != LISA_OK) return st;
  (void)hipGetLastError();  // clear a stale error so that ours are reported alone
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (pl.T >= 2) {
    st = run_stats(pl, Q, K, V, ws, p->eps, pl.T >= 3, s);
    if (st != LISA_OK) return st;
  }
  return run_output(pl, Q, K, V, weights, beta, alpha, Y, ws, p->eps, s);
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
  st = run_stats(pl, Q, K, V, ws, p->eps, true, s);
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
  lisa_status st = check_forward(p, Q, K, V, weights, beta, alpha, Y, workspace, workspace_bytes, pl);
  if (st != LISA_OK) return st;
  (void)hipGetLastError();
  return run_output(pl, Q, K, V, weights, beta, alpha, Y, static_cast<char*>(workspace), p->eps,
                    static_cast<hipStream_t>(stream));
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
  }
  return "unknown status";
}

}  // extern "C"
