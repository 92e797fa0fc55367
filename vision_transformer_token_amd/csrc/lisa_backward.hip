// LiSA backward pass on gfx950: gradients of Y = alpha G + (1 - alpha) L
// with respect to Q, K, V, the adaptive walk weights and alpha.
//
// Source: the reading note of "LiSA: Linear Stochastic Attention for
// Long-Range Visual Modeling" trains every model it reports (§3) and picks
// the truncation T with the cost of backpropagation in mind (§2.3); it gives
// no backward formulas.  The gradients here are the exact adjoint of the
// forward pass (§2.1-§2.4), step by step:
//   G_i = w_0(i) V_i + sum_{k>=1} w_k(i) Qt_i P_k,  P_k = M^(k-1) phi(K)^T V,
//   Qt_i = r_i phi(Q_i), r_i = 1 / (phi(Q_i) . s + eps), s = sum_j phi(K_j),
//   M = phi(K)^T Qt;  L_i = softmax over the 3x3 window of q_i . k_j / 8.
// With dG = alpha dY and dL = (1 - alpha) dY:
//   dP_k = sum_i w_k(i) Qt_i^T dG_i              (token reduction, pass A)
//   dM, dKV by the power chain in d_h space      (adjoint kernel)
//   dQt_i = sum_k w_k(i) P_k dG_i + dM^T phi(K_i)
//   dz_i = -r_i^2 dQt_i . phi(Q_i),  ds = sum_i dz_i phi(Q_i)   (pass B)
//   dQ_i = (r_i dQt_i + dz_i s) [Q_i > 0] + local
//   dK_j = (dM Qt_j + dKV V_j + ds) [K_j > 0] + local
//   dV_j = w_0(j) dG_j + dKV^T phi(K_j) + local
//   dw_k(i) = dG_i . (Qt_i P_k), dw_0(i) = dG_i . V_i, dalpha = sum dY.(G - L)
// The local branch's softmax adjoint uses, per centre token i, the window's
// logit maximum m_i and sum Z_i and c_i = dL_i . L_i, which pass A keeps.
//
// Layout: the token passes take kBwdTokens tokens per workgroup, four lanes
// per token (lane quarter qd owns features 16 qd .. 16 qd + 15); dot products
// are reduced over the lane quad with DPP.  Products of token rows with the
// slice's 64 x 64 matrices (and the token reduction dP_k) run on fp32 MFMA
// (16x16x4): each wave multiplies the LDS rows of its 16 tokens by a matrix
// held in LDS, and the result returns to the quad layout through those rows.
// Everything is fp32; outputs dQ, dK, dV are written once in the input dtype.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lisa_device.hpp"
#include "lisa_kernels.hpp"

namespace lisa {
namespace {

constexpr int kBT = kBwdTokens;
constexpr int kR = kD + 1;           // padded LDS row (floats)
constexpr float kRs = 0.125f;        // 1 / sqrt(d_h), d_h = 64
constexpr int kAdjThreads = 256;

constexpr int kQ = 4;                // lanes per token
constexpr int kF = kD / kQ;          // features per lane
constexpr int kTT = kBT * kQ;        // threads of a token-pass workgroup
constexpr int kW = kMaxT + 1;        // padded LDS row of a token's walk weights

// This lane's 16 features of a row.
template <class S>
__device__ __forceinline__ void load16(const S* row, int f0, float (&x)[kF]) {
#pragma unroll
  for (int e = 0; e < kF; e += 4) load4(row + f0 + e, &x[e]);
}
template <class S>
__device__ __forceinline__ void store16(S* row, int f0, const float (&x)[kF]) {
#pragma unroll
  for (int e = 0; e < kF; e += 4) store4(row + f0 + e, &x[e]);
}
// Sum over the lane quad of a token (every lane of the quad gets it).
__device__ __forceinline__ float quad_sum(float x) { return dpp_add(dpp_add(x, 0xB1), 0x4E); }
// x . row over all 64 features (quad-reduced).
template <class S>
__device__ __forceinline__ float dot64(const S* row, int f0, const float (&x)[kF]) {
  float y[kF];
  load16(row, f0, y);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) acc += x[e] * y[e];
  return quad_sum(acc);
}
template <class S>
__device__ __forceinline__ void axpy16(float f, const S* row, int f0, float (&x)[kF]) {
  float y[kF];
  load16(row, f0, y);
#pragma unroll
  for (int e = 0; e < kF; ++e) x[e] += f * y[e];
}
// The quad's rows in LDS are written and read by lanes of one wave: order
// the LDS accesses (the compiler may not move them across this either).
__device__ __forceinline__ void quad_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
}

// MFMA 16x16x4 fp32 (exact fp32 products, fp32 sums).  Lane l = 16 h + m
// holds A[m][h] and B[h][m]; accumulator element e holds C[4 h + e][m].
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// Y += diag(sx) X M (kTr = false) or diag(sx) X M^T (kTr = true) for the
// wave's 16 tokens: X their LDS rows (stride kR), M a 64 x 64 matrix in LDS
// rows of kR floats, sx this lane's row scale (row li).  Y in accumulator
// layout: acc[ct][e] = Y[4 lk + e][16 ct + li].  Features are taken in the
// order 16 lk + kk, which keeps every operand read of the wave on 64
// distinct banks (kR = 1 mod 64).
template <bool kTr>
__device__ __forceinline__ void wave_mm(const float* X, const float* M, float sx, f32x4 (&acc)[4]) {
  const int ln = threadIdx.x % 64, li = ln % 16, lk = ln / 16;
#pragma unroll 4
  for (int kk = 0; kk < kD / 4; ++kk) {
    const int f = 16 * lk + kk;
    const float av = sx * X[li * kR + f];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      acc[ct] = mfma16(av, kTr ? M[(16 * ct + li) * kR + f] : M[f * kR + 16 * ct + li], acc[ct]);
  }
}
// Y from accumulator layout into the lane-quad layout through the wave's LDS
// rows X (overwritten): lane (token tw of the wave, quarter f0) gets
// Y[tw][f0 .. f0 + 15].
__device__ __forceinline__ void acc_to_quad(const f32x4 (&acc)[4], float* X, int tw, int f0, float (&y)[kF]) {
  const int ln = threadIdx.x % 64, li = ln % 16, lk = ln / 16;
  quad_lds_sync();
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) X[(4 * lk + e) * kR + 16 * ct + li] = acc[ct][e];
  quad_lds_sync();
#pragma unroll
  for (int e = 0; e < kF; ++e) y[e] = X[tw * kR + f0 + e];
}

// Whole workgroup: copy a 64 x 64 fp32 matrix into LDS.
__device__ __forceinline__ void load_mat(float* dst, const float* src) {
  for (int e = threadIdx.x * 4; e < kD * kD; e += blockDim.x * 4)
    *reinterpret_cast<float4*>(dst + e) = *reinterpret_cast<const float4*>(src + e);
}

// The same into rows of kR floats.
__device__ __forceinline__ void load_mat_padded(float* dst, const float* src) {
  for (int e = threadIdx.x * 4; e < kD * kD; e += blockDim.x * 4) {
    const float4 v = *reinterpret_cast<const float4*>(src + e);
    float* d = dst + (e / kD) * kR + e % kD;
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
  }
}

__device__ __forceinline__ float wgt(const BwdArgs& a, size_t tok, int k) {
  return a.weights ? a.weights[tok * a.T + k] : a.geo[k];
}

// The valid 3x3 window of token i: slot j (0..8) is the cell (row + j/3 - 1,
// col + j%3 - 1); returns its token index or -1 off the grid.
__device__ __forceinline__ int window_cell(const BwdArgs& a, int row, int col, int j) {
  const int rr = row + j / 3 - 1, cc = col + j % 3 - 1;
  return (rr >= 0 && rr < a.H && cc >= 0 && cc < a.W) ? rr * a.W + cc : -1;
}

// P_1 = phi(K)^T V, P_k = M P_(k-1) for k = 2 .. T-1: one workgroup per slice.
__global__ __launch_bounds__(kAdjThreads) void bwd_powers(BwdArgs a) {
  __shared__ float Ms[kD * kD];
  __shared__ float Ps[kD * kR];
  const int b = blockIdx.x, t = threadIdx.x;
  const int T1 = a.T - 1;
  if (T1 < 1) return;
  const float* M = a.fin_m + (size_t)b * kD * kD;
  const float* P1 = a.fin_kv + (size_t)b * kD * kD;
  float* out = a.pk + (size_t)b * T1 * kD * kD;
  load_mat(Ms, M);
  for (int e = t; e < kD * kD; e += kAdjThreads) {
    Ps[(e >> 6) * kR + (e & 63)] = P1[e];
    out[e] = P1[e];
  }
  for (int k = 2; k <= T1; ++k) {
    __syncthreads();
    float acc[kD * kD / kAdjThreads];
#pragma unroll
    for (int x = 0; x < kD * kD / kAdjThreads; ++x) {
      const int e = t + kAdjThreads * x, r = e >> 6, c = e & 63;
      float v = 0.f;
      for (int j = 0; j < kD; ++j) v += Ms[r * kD + j] * Ps[j * kR + c];
      acc[x] = v;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kD * kD / kAdjThreads; ++x) {
      const int e = t + kAdjThreads * x;
      Ps[(e >> 6) * kR + (e & 63)] = acc[x];
      out[(size_t)(k - 1) * kD * kD + e] = acc[x];
    }
  }
}

// Pass A: per token the local window statistics, dY . V_i, dY . (Qt_i P_k),
// the weight gradients and dalpha's share; per workgroup the partial sums of
// dP_k = sum_i w_k(i) alpha Qt_i^T dY_i.
template <class S>
__global__ __launch_bounds__(kTT) void bwd_token_a(BwdArgs a) {
  extern __shared__ __align__(16) float sm[];
  float* Ps = sm;                        // kD rows of kR: P_k
  float* s_sh = Ps + kD * kR;            // kD
  float* qt_sh = s_sh + kD;              // kBT rows of Qt (padded)
  float* dy_sh = qt_sh + kBT * kR;       // kBT rows of dY (padded)
  float* w_sh = dy_sh + kBT * kR;        // kBT rows of kW weights
  float* red = w_sh + kBT * kW;          // kBT
  const int b = blockIdx.y, t = threadIdx.x, blk = blockIdx.x;
  const int tk = t / kQ, qd = t % kQ, f0 = qd * kF;
  const int i = blk * kBT + tk;
  const bool on = i < a.n;
  const float alpha = a.alpha[b % a.heads];
  const size_t base = (size_t)b * a.n;
  const S* Qb = static_cast<const S*>(a.Q) + base * kD;
  const S* Kb = static_cast<const S*>(a.K) + base * kD;
  const S* Vb = static_cast<const S*>(a.V) + base * kD;
  const S* dYb = static_cast<const S*>(a.dY) + base * kD;
  if (t < kD) s_sh[t] = a.fin_s[(size_t)b * kD + t];
  if (qd == 0)
    for (int k = 0; k < kMaxT; ++k) w_sh[tk * kW + k] = (on && k < a.T) ? wgt(a, base + i, k) : 0.f;

  float q[kF], dy[kF];
  float m = 0.f, Z = 1.f, dyL = 0.f, dyv = 0.f;
  if (on) {
    load16(Qb + (size_t)i * kD, f0, q);
    load16(dYb + (size_t)i * kD, f0, dy);
    // Local branch at token i: window logits, their max and sum, dY . L_i.
    const int row = i / a.W, col = i % a.W;
    float z[9];
    m = -INFINITY;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const int c = window_cell(a, row, col, j);
      z[j] = c >= 0 ? dot64(Kb + (size_t)c * kD, f0, q) * kRs : -INFINITY;
      m = fmaxf(m, z[j]);
    }
    Z = 0.f;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const int c = window_cell(a, row, col, j);
      if (c >= 0) {
        const float e = __expf(z[j] - m);
        Z += e;
        dyL += e * dot64(Vb + (size_t)c * kD, f0, dy);
      }
    }
    dyL /= Z;
    dyv = dot64(Vb + (size_t)i * kD, f0, dy);
  } else {
#pragma unroll
    for (int e = 0; e < kF; ++e) q[e] = dy[e] = 0.f;
  }
  __syncthreads();  // s_sh, w_sh
  // Qt_i = r_i phi(Q_i).
  float den = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) {
    q[e] = fmaxf(q[e], 0.f);
    den += q[e] * s_sh[f0 + e];
  }
  const float r = 1.f / (quad_sum(den) + a.eps);
#pragma unroll
  for (int e = 0; e < kF; ++e) {
    q[e] *= r;
    qt_sh[tk * kR + f0 + e] = q[e];
    dy_sh[tk * kR + f0 + e] = dy[e];
  }
  float dyy[kMaxT];
#pragma unroll
  for (int k = 0; k < kMaxT; ++k) dyy[k] = 0.f;
  const int T1 = a.T - 1;
  // MFMA roles: wave wv holds tokens 16 wv .. 16 wv + 15 (its quads) and the
  // 16 x 16 block (ga, gc) of dP_k; lane ln = 16 lk + li.  The contractions
  // take their terms in an order (features 16 lk + kk, tokens
  // 64 (kk / 16) + 16 lk + kk % 16) under which every LDS operand read of a
  // wave hits 64 distinct banks (row stride kR = 1 mod 64).
  const int wv = t / 64, ln = t % 64, li = ln % 16, lk = ln / 16;
  const int ga = 16 * (wv / 4), gc = 16 * (wv % 4);
#pragma unroll
  for (int k = 1; k < kMaxT; ++k) {
    if (k > T1) break;
    __syncthreads();
    load_mat_padded(Ps, a.pk + ((size_t)b * T1 + (k - 1)) * kD * kD);
    __syncthreads();
    // dY_i . (Qt_i P_k): X = Qt P_k for the wave's 16 tokens (4 column
    // blocks), then each row dotted with dY_i.
    {
      f32x4 x[4] = {};
#pragma unroll 4
      for (int kk = 0; kk < kD / 4; ++kk) {
        const int f = 16 * lk + kk;
        const float av = qt_sh[(16 * wv + li) * kR + f];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) x[ct] = mfma16(av, Ps[f * kR + 16 * ct + li], x[ct]);
      }
      float part[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float* dyr = dy_sh + (16 * wv + 4 * lk + e) * kR + li;
        float v = 0.f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) v += x[ct][e] * dyr[16 * ct];
        part[e] = group_sum16(v);
      }
      // This lane's token 16 wv + ln / 4 is row 4 lk + li / 4 of the block.
      const int e = li / 4;
      dyy[k] = e == 0 ? part[0] : e == 1 ? part[1] : e == 2 ? part[2] : part[3];
    }
    // This workgroup's share of dP_k = sum_i alpha w_k(i) Qt_i^T dY_i.
    {
      f32x4 acc = {};
#pragma unroll 8
      for (int kk = 0; kk < kBT / 4; ++kk) {
        const int tt = 64 * (kk / 16) + 16 * lk + kk % 16;
        acc = mfma16(w_sh[tt * kW + k] * qt_sh[tt * kR + ga + li], dy_sh[tt * kR + gc + li], acc);
      }
      float* dst = a.dp_part + (((size_t)b * a.nblk + blk) * T1 + (k - 1)) * kD * kD;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(ga + 4 * lk + e) * kD + gc + li] = alpha * acc[e];
    }
  }
  // Scalars of the token (every lane of the quad holds them).
  float wy = 0.f;
#pragma unroll
  for (int k = 1; k < kMaxT; ++k)
    if (k <= T1) wy += w_sh[tk * kW + k] * dyy[k];
  const float dyG = w_sh[tk * kW] * dyv + wy;
  if (on && qd == 0) {
    // a_i = (sum_k w_k P_k dG_i) . phi(Q_i) = alpha / r_i * sum_k w_k dY_i . (Qt_i P_k)
    a.tok[base + i] = make_float4(m, Z, (1.f - alpha) * dyL, alpha / r * wy);
    if (a.dweights) {
      float* dw = a.dweights + (base + i) * a.T;
      dw[0] = alpha * dyv;
#pragma unroll
      for (int k = 1; k < kMaxT; ++k)
        if (k <= T1) dw[k] = alpha * dyy[k];
    }
  }
  // dalpha's share: sum_i dY_i . (G_i - L_i), fixed-order tree.
  if (qd == 0) red[tk] = on ? dyG - dyL : 0.f;
  __syncthreads();
  for (int o = kBT / 2; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  if (t == 0) a.da_part[(size_t)b * a.nblk + blk] = red[0];
}

// dP_k: the workgroups' partials summed in order, element by element, into
// the first workgroup's slot.
__global__ __launch_bounds__(kAdjThreads) void bwd_reduce_dp(BwdArgs a) {
  const int b = blockIdx.y, T1 = a.T - 1;
  const size_t per = (size_t)T1 * kD * kD;
  const size_t e = (size_t)blockIdx.x * kAdjThreads + threadIdx.x;
  if (T1 < 1 || e >= per) return;
  float* base = a.dp_part + (size_t)b * a.nblk * per + e;
  float v = 0.f;
  for (int p = 0; p < a.nblk; ++p) v += base[(size_t)p * per];
  base[0] = v;
}

// dP_k (summed by bwd_reduce_dp); then, from the last term down,
// dM += dP_k P_(k-1)^T and dP_(k-1) += M^T dP_k; dKV = dP_1.  One workgroup
// per slice; also the slice's dalpha.
__global__ __launch_bounds__(kAdjThreads) void bwd_adjoint(BwdArgs a) {
  extern __shared__ __align__(16) float sm[];
  const int b = blockIdx.x, t = threadIdx.x, T1 = a.T - 1;
  constexpr int kX = kD * kD / kAdjThreads;  // outputs per thread
  float* dP = sm;                            // T1 x 64 x 64
  float* Ms = dP + (size_t)(T1 > 0 ? T1 : 1) * kD * kD;
  float* Pp = Ms + kD * kD;                  // P_(k-1), padded rows
  float* dMo = a.dmkv + (size_t)b * 2 * kD * kD;
  float* dKVo = dMo + kD * kD;
  if (t == 0) {
    float v = 0.f;
    for (int p = 0; p < a.nblk; ++p) v += a.da_part[(size_t)b * a.nblk + p];
    a.da_slice[b] = v;
  }
  if (T1 < 1) {
    for (int e = t; e < kD * kD; e += kAdjThreads) dMo[e] = dKVo[e] = 0.f;
    return;
  }
  const size_t per = (size_t)T1 * kD * kD;
  for (size_t e = t; e < per; e += kAdjThreads) dP[e] = a.dp_part[(size_t)b * a.nblk * per + e];
  load_mat(Ms, a.fin_m + (size_t)b * kD * kD);
  float dM[kX] = {};
  for (int k = T1; k >= 2; --k) {
    __syncthreads();
    const float* Pk1 = a.pk + ((size_t)b * T1 + (k - 2)) * kD * kD;
    for (int e = t; e < kD * kD; e += kAdjThreads) Pp[(e >> 6) * kR + (e & 63)] = Pk1[e];
    __syncthreads();
    const float* dPk = dP + (size_t)(k - 1) * kD * kD;
    float up[kX];
#pragma unroll
    for (int x = 0; x < kX; ++x) {
      const int e = t + kAdjThreads * x, r = e >> 6, c = e & 63;
      float v = 0.f, u = 0.f;
      for (int j = 0; j < kD; ++j) {
        v += dPk[r * kD + j] * Pp[c * kR + j];   // (dP_k P_(k-1)^T)[r][c]
        u += Ms[j * kD + r] * dPk[j * kD + c];    // (M^T dP_k)[r][c]
      }
      dM[x] += v;
      up[x] = u;
    }
    __syncthreads();
    float* dPm = dP + (size_t)(k - 2) * kD * kD;
#pragma unroll
    for (int x = 0; x < kX; ++x) dPm[t + kAdjThreads * x] += up[x];
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < kX; ++x) {
    const int e = t + kAdjThreads * x;
    dMo[e] = dM[x];
    dKVo[e] = dP[e];
  }
}

// Pass B: dz_i = -r_i^2 (a_i + phi(K_i)^T dM phi(Q_i)) (kept in tok[i].w) and
// the workgroup's share of ds = sum_i dz_i phi(Q_i).
template <class S>
__global__ __launch_bounds__(kTT) void bwd_token_b(BwdArgs a) {
  constexpr int kG = kTT / kD;  // partial sums per feature in the ds reduction
  __shared__ float dMs[kD * kR];
  __shared__ float s_sh[kD];
  __shared__ float rows[kBT * kR];
  __shared__ float red[kG * kD];
  const int b = blockIdx.y, t = threadIdx.x, blk = blockIdx.x;
  const int tk = t / kQ, qd = t % kQ, f0 = qd * kF, tw = tk % 16;
  float* wrows = rows + (t / 64) * 16 * kR;  // this wave's 16 token rows
  const int i = blk * kBT + tk;
  const bool on = i < a.n;
  const size_t base = (size_t)b * a.n;
  load_mat_padded(dMs, a.dmkv + (size_t)b * 2 * kD * kD);
  if (t < kD) s_sh[t] = a.fin_s[(size_t)b * kD + t];
  float u[kF], kp[kF];
  if (on) {
    load16(static_cast<const S*>(a.Q) + (base + i) * kD, f0, u);
    load16(static_cast<const S*>(a.K) + (base + i) * kD, f0, kp);
  } else {
#pragma unroll
    for (int e = 0; e < kF; ++e) u[e] = kp[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < kF; ++e) rows[tk * kR + f0 + e] = fmaxf(kp[e], 0.f);
  __syncthreads();
  float den = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) {
    u[e] = fmaxf(u[e], 0.f);
    den += u[e] * s_sh[f0 + e];
  }
  const float r = 1.f / (quad_sum(den) + a.eps);
  // phi(K_i)^T dM phi(Q_i): the row phi(K_i) dM, dotted with phi(Q_i).
  f32x4 acc[4] = {};
  wave_mm<false>(wrows, dMs, 1.f, acc);
  float y[kF];
  acc_to_quad(acc, wrows, tw, f0, y);
  float bil = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) bil += y[e] * u[e];
  bil = quad_sum(bil);
  float dz = 0.f;
  if (on) {
    float4* tp = a.tok + base + i;
    const float4 v = *tp;
    dz = -r * r * (v.w + bil);
    if (qd == 0) *tp = make_float4(v.x, v.y, v.z, dz);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kF; ++e) rows[tk * kR + f0 + e] = dz * u[e];
  __syncthreads();
  // Fixed-order sums: kG groups of kBT / kG tokens, then the groups in order.
  {
    const int f = t % kD, g = t / kD;
    float v = 0.f;
    for (int tt = g * (kBT / kG); tt < (g + 1) * (kBT / kG); ++tt) v += rows[tt * kR + f];
    red[g * kD + f] = v;
  }
  __syncthreads();
  if (t < kD) {
    float v = 0.f;
#pragma unroll
    for (int g = 0; g < kG; ++g) v += red[g * kD + t];
    a.ds_part[((size_t)b * a.nblk + blk) * kD + t] = v;
  }
}

// dQ_i = (r_i dQt_i + dz_i s) [Q_i > 0] + sum_j dz_ij k_j / 8, with
// dQt_i = dM^T phi(K_i) + sum_k w_k P_k dG_i and dz_ij the softmax adjoint
// of window slot j.
template <class S>
__global__ __launch_bounds__(kTT) void bwd_token_q(BwdArgs a) {
  __shared__ float Ps[kD * kR];
  __shared__ float dMs[kD * kR];
  __shared__ float s_sh[kD];
  __shared__ float rows[kBT * kR];
  const int b = blockIdx.y, t = threadIdx.x, blk = blockIdx.x;
  const int tk = t / kQ, qd = t % kQ, f0 = qd * kF, tw = tk % 16;
  float* wrows = rows + (t / 64) * 16 * kR;
  const int i = blk * kBT + tk;
  const bool on = i < a.n;
  const size_t base = (size_t)b * a.n;
  const float alpha = a.alpha[b % a.heads];
  const S* Qb = static_cast<const S*>(a.Q) + base * kD;
  const S* Kb = static_cast<const S*>(a.K) + base * kD;
  const S* Vb = static_cast<const S*>(a.V) + base * kD;
  const S* dYb = static_cast<const S*>(a.dY) + base * kD;
  load_mat_padded(dMs, a.dmkv + (size_t)b * 2 * kD * kD);
  if (t < kD) s_sh[t] = a.fin_s[(size_t)b * kD + t];
  float x[kF];
  if (on) load16(Kb + (size_t)i * kD, f0, x);
  else
#pragma unroll
    for (int e = 0; e < kF; ++e) x[e] = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) rows[tk * kR + f0 + e] = fmaxf(x[e], 0.f);
  __syncthreads();
  // dQt rows: phi(K) dM, then + sum_k diag(alpha w_k) dY P_k^T.
  f32x4 acc[4] = {};
  wave_mm<false>(wrows, dMs, 1.f, acc);
  if (on) load16(dYb + (size_t)i * kD, f0, x);
  quad_lds_sync();
#pragma unroll
  for (int e = 0; e < kF; ++e) rows[tk * kR + f0 + e] = x[e];
  const int T1 = a.T - 1;
  // The MFMA A operand row of this lane: token 16 (t / 64) + li.
  const int ia = blk * kBT + (t / 64) * 16 + (t % 16);
  for (int k = 1; k <= T1; ++k) {
    __syncthreads();
    load_mat_padded(Ps, a.pk + ((size_t)b * T1 + (k - 1)) * kD * kD);
    __syncthreads();
    wave_mm<true>(wrows, Ps, ia < a.n ? alpha * wgt(a, base + ia, k) : 0.f, acc);
  }
  float dqt[kF];
  acc_to_quad(acc, wrows, tw, f0, dqt);
  if (!on) return;  // no barrier follows
  const float4 tp = a.tok[base + i];  // m_i, Z_i, c_i, dz_i
  float q[kF];
  load16(Qb + (size_t)i * kD, f0, q);
  float den = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) den += fmaxf(q[e], 0.f) * s_sh[f0 + e];
  const float r = 1.f / (quad_sum(den) + a.eps);
#pragma unroll
  for (int e = 0; e < kF; ++e) dqt[e] = q[e] > 0.f ? r * dqt[e] + tp.w * s_sh[f0 + e] : 0.f;
  // Local: dz_ij = p_ij ((1 - alpha) dY_i . V_j - c_i).
  const int row = i / a.W, col = i % a.W;
#pragma unroll 1
  for (int j = 0; j < 9; ++j) {
    const int c = window_cell(a, row, col, j);
    if (c < 0) continue;
    const S* kj = Kb + (size_t)c * kD;
    const float p = __expf(dot64(kj, f0, q) * kRs - tp.x) / tp.y;
    const float g = p * ((1.f - alpha) * dot64(Vb + (size_t)c * kD, f0, x) - tp.z);
    axpy16(g * kRs, kj, f0, dqt);
  }
  store16(static_cast<S*>(a.dQ) + (base + i) * kD, f0, dqt);
}

// dK_j = (dM Qt_j + dKV V_j + ds) [K_j > 0] + sum_i dz_ij q_i / 8 over the
// centres i whose window holds j (the window relation is symmetric).
template <class S>
__global__ __launch_bounds__(kTT) void bwd_token_k(BwdArgs a) {
  __shared__ float dMs[kD * kR];
  __shared__ float dKVs[kD * kR];
  __shared__ float s_sh[kD];
  __shared__ float ds_sh[kD];
  __shared__ float rows[kBT * kR];
  const int b = blockIdx.y, t = threadIdx.x, blk = blockIdx.x;
  const int tk = t / kQ, qd = t % kQ, f0 = qd * kF, tw = tk % 16;
  float* wrows = rows + (t / 64) * 16 * kR;
  const int i = blk * kBT + tk;
  const bool on = i < a.n;
  const size_t base = (size_t)b * a.n;
  const float alpha = a.alpha[b % a.heads];
  const S* Qb = static_cast<const S*>(a.Q) + base * kD;
  const S* Kb = static_cast<const S*>(a.K) + base * kD;
  const S* Vb = static_cast<const S*>(a.V) + base * kD;
  const S* dYb = static_cast<const S*>(a.dY) + base * kD;
  load_mat_padded(dMs, a.dmkv + (size_t)b * 2 * kD * kD);
  load_mat_padded(dKVs, a.dmkv + (size_t)b * 2 * kD * kD + kD * kD);
  if (t < kD) {
    s_sh[t] = a.fin_s[(size_t)b * kD + t];
    float v = 0.f;
    for (int p = 0; p < a.nblk; ++p) v += a.ds_part[((size_t)b * a.nblk + p) * kD + t];
    ds_sh[t] = v;
  }
  __syncthreads();
  // Rows Qt_j dM^T + V_j dKV^T.
  float x[kF];
  if (on) load16(Qb + (size_t)i * kD, f0, x);
  else
#pragma unroll
    for (int e = 0; e < kF; ++e) x[e] = 0.f;
  float den = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) {
    x[e] = fmaxf(x[e], 0.f);
    den += x[e] * s_sh[f0 + e];
  }
  const float r = 1.f / (quad_sum(den) + a.eps);
#pragma unroll
  for (int e = 0; e < kF; ++e) rows[tk * kR + f0 + e] = x[e] * r;
  quad_lds_sync();
  f32x4 acc[4] = {};
  wave_mm<true>(wrows, dMs, 1.f, acc);
  if (on) load16(Vb + (size_t)i * kD, f0, x);
  quad_lds_sync();
#pragma unroll
  for (int e = 0; e < kF; ++e) rows[tk * kR + f0 + e] = x[e];
  quad_lds_sync();
  wave_mm<true>(wrows, dKVs, 1.f, acc);
  float g16[kF];
  acc_to_quad(acc, wrows, tw, f0, g16);
  if (!on) return;  // no barrier follows
  float kr[kF], dk[kF];
  load16(Kb + (size_t)i * kD, f0, kr);
#pragma unroll
  for (int e = 0; e < kF; ++e) dk[e] = kr[e] > 0.f ? g16[e] + ds_sh[f0 + e] : 0.f;
  // Local: token i as the neighbour of centre c.
  const int row = i / a.W, col = i % a.W;
#pragma unroll 1
  for (int j = 0; j < 9; ++j) {
    const int c = window_cell(a, row, col, j);
    if (c < 0) continue;
    const float4 tc = a.tok[base + c];
    const S* qc = Qb + (size_t)c * kD;
    const float p = __expf(dot64(qc, f0, kr) * kRs - tc.x) / tc.y;
    const float g = p * ((1.f - alpha) * dot64(dYb + (size_t)c * kD, f0, x) - tc.z);
    axpy16(g * kRs, qc, f0, dk);
  }
  store16(static_cast<S*>(a.dK) + (base + i) * kD, f0, dk);
}

// dV_j = w_0(j) alpha dY_j + dKV^T phi(K_j) + sum_i p_ij (1 - alpha) dY_i.
template <class S>
__global__ __launch_bounds__(kTT) void bwd_token_v(BwdArgs a) {
  __shared__ float dKVs[kD * kR];
  __shared__ float rows[kBT * kR];
  const int b = blockIdx.y, t = threadIdx.x, blk = blockIdx.x;
  const int tk = t / kQ, qd = t % kQ, f0 = qd * kF, tw = tk % 16;
  float* wrows = rows + (t / 64) * 16 * kR;
  const int i = blk * kBT + tk;
  const bool on = i < a.n;
  const size_t base = (size_t)b * a.n;
  const float alpha = a.alpha[b % a.heads];
  const S* Qb = static_cast<const S*>(a.Q) + base * kD;
  const S* Kb = static_cast<const S*>(a.K) + base * kD;
  const S* dYb = static_cast<const S*>(a.dY) + base * kD;
  load_mat_padded(dKVs, a.dmkv + (size_t)b * 2 * kD * kD + kD * kD);
  float kr[kF];
  if (on) load16(Kb + (size_t)i * kD, f0, kr);
  else
#pragma unroll
    for (int e = 0; e < kF; ++e) kr[e] = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) rows[tk * kR + f0 + e] = fmaxf(kr[e], 0.f);
  __syncthreads();
  // Rows phi(K_j) dKV.
  f32x4 acc[4] = {};
  wave_mm<false>(wrows, dKVs, 1.f, acc);
  float dv[kF];
  acc_to_quad(acc, wrows, tw, f0, dv);
  if (!on) return;  // no barrier follows
  float dy[kF];
  load16(dYb + (size_t)i * kD, f0, dy);
  const float w0 = alpha * wgt(a, base + i, 0);
#pragma unroll
  for (int e = 0; e < kF; ++e) dv[e] += w0 * dy[e];
  const int row = i / a.W, col = i % a.W;
#pragma unroll 1
  for (int j = 0; j < 9; ++j) {
    const int c = window_cell(a, row, col, j);
    if (c < 0) continue;
    const float4 tc = a.tok[base + c];
    const float p = __expf(dot64(Qb + (size_t)c * kD, f0, kr) * kRs - tc.x) / tc.y;
    axpy16(p * (1.f - alpha), dYb + (size_t)c * kD, f0, dv);
  }
  store16(static_cast<S*>(a.dV) + (base + i) * kD, f0, dv);
}

// dalpha[h] = sum over the batch of the slices' shares, in batch order.
__global__ __launch_bounds__(256) void bwd_dalpha(BwdArgs a) {
  for (int h = threadIdx.x; h < a.heads; h += blockDim.x) {
    float v = 0.f;
    for (int b = h; b < a.BH; b += a.heads) v += a.da_slice[b];
    a.dalpha[h] = v;
  }
}

template <class S>
hipError_t launch_typed(const BwdArgs& a, hipStream_t s) {
  const size_t lds_a = (size_t)(kD * kR + kD + 2 * kBT * kR + kBT * kW + kBT) * sizeof(float);
  const int T1 = a.T - 1 > 0 ? a.T - 1 : 1;
  const size_t lds_adj = ((size_t)T1 * kD * kD + kD * kD + kD * kR) * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_token_a<S>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_a);
    if (e != hipSuccess) return e;
    const size_t lds_adj_max = ((size_t)(kMaxT - 1) * kD * kD + kD * kD + kD * kR) * sizeof(float);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_adjoint),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_adj_max);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 tok(a.nblk, a.BH);
  if (a.T >= 2) hipLaunchKernelGGL(bwd_powers, dim3(a.BH), dim3(kAdjThreads), 0, s, a);
  hipLaunchKernelGGL(bwd_token_a<S>, tok, dim3(kTT), lds_a, s, a);
  if (a.T >= 2)
    hipLaunchKernelGGL(bwd_reduce_dp, dim3((T1 * kD * kD + kAdjThreads - 1) / kAdjThreads, a.BH),
                       dim3(kAdjThreads), 0, s, a);
  hipLaunchKernelGGL(bwd_adjoint, dim3(a.BH), dim3(kAdjThreads), lds_adj, s, a);
  hipLaunchKernelGGL(bwd_token_b<S>, tok, dim3(kTT), 0, s, a);
  hipLaunchKernelGGL(bwd_token_q<S>, tok, dim3(kTT), 0, s, a);
  hipLaunchKernelGGL(bwd_token_k<S>, tok, dim3(kTT), 0, s, a);
  hipLaunchKernelGGL(bwd_token_v<S>, tok, dim3(kTT), 0, s, a);
  hipLaunchKernelGGL(bwd_dalpha, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(int dtype, const BwdArgs& a, hipStream_t s) {
  return dtype == 1 ? launch_typed<uint16_t>(a, s) : launch_typed<float>(a, s);
}

}  // namespace lisa
