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
constexpr int kAdjThreads = 1024;  // per-slice kernels: wave w owns rows 16 (w % 4) .., column block w / 4

constexpr int kQ = 4;                // lanes per token
constexpr int kF = kD / kQ;          // features per lane
constexpr int kTT = kBT * kQ;        // threads of a token-pass workgroup
constexpr int kW = kMaxTBwd + 1;        // padded LDS row of a token's walk weights

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
// This lane's 16 features of a row as loaded (bf16 kept packed: half the
// registers of floats), for the window gathers that hold several rows.
template <class S>
struct Piece;
template <>
struct Piece<uint16_t> {
  u32x4 w[2];
  __device__ __forceinline__ void load(const uint16_t* row, int f0) {
    w[0] = *reinterpret_cast<const u32x4*>(row + f0);
    w[1] = *reinterpret_cast<const u32x4*>(row + f0 + 8);
  }
  __device__ __forceinline__ float operator[](int e) const {  // e: a compile-time constant after unrolling
    const uint32_t x = w[e >> 3][(e & 7) >> 1];
    return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
  }
  // The loaded value is needed here: pieces loaded before and pinned
  // together are waited for together (otherwise the compiler may reuse one
  // register tuple and wait for each load before issuing the next).
  __device__ __forceinline__ void pin() { asm volatile("" : "+v"(w[0]), "+v"(w[1])); }
};
template <>
struct Piece<float> {
  float4 w[4];
  __device__ __forceinline__ void load(const float* row, int f0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const float4*>(row + f0 + 4 * j);
  }
  __device__ __forceinline__ float operator[](int e) const {
    const float4& v = w[e >> 2];
    return (e & 3) == 0 ? v.x : (e & 3) == 1 ? v.y : (e & 3) == 2 ? v.z : v.w;
  }
  __device__ __forceinline__ void pin() {}
};

// This lane's part of a . b over its 16 features.  bf16 rows: v_dot2 on the
// packed pairs (the products of two bf16 values are exact in fp32; fp32
// sums, pair by pair); fp32 rows: fused multiply-adds in feature order.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dotp(const Piece<uint16_t>& a, const Piece<uint16_t>& b) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t x = a.w[j >> 2][j & 3], y = b.w[j >> 2][j & 3];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, x), __builtin_bit_cast(bf16x2v, y), acc, false);
  }
  return acc;
}
__device__ __forceinline__ float dotp(const Piece<float>& a, const Piece<float>& b) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) acc += a[e] * b[e];
  return acc;
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
// One 16 x 16 block of X M (kTr = false) or X M^T (kTr = true): X the 16
// rows (stride kR), column block ct; same operand order as wave_mm.
template <bool kTr>
__device__ __forceinline__ f32x4 tile_mm(const float* X, const float* M, int ct, f32x4 acc) {
  const int ln = threadIdx.x % 64, li = ln % 16, lk = ln / 16;
#pragma unroll 4
  for (int kk = 0; kk < kD / 4; ++kk) {
    const int f = 16 * lk + kk;
    acc = mfma16(X[li * kR + f], kTr ? M[(16 * ct + li) * kR + f] : M[f * kR + 16 * ct + li], acc);
  }
  return acc;
}
// ---------------------------------------------------------------------------
// Token-row x matrix products of the token passes, per input type S.
//
// Each wave multiplies the rows of its 16 tokens (X, 16 x 64) by a 64 x 64
// matrix staged in LDS "B-ready": Bt[n][k] is the term of output column n
// and contraction index k, so Y = X M stages M^T and Y = X M^T stages M.
// Y comes out in accumulator layout: acc[ct][e] = Y[4 lk + e][16 ct + li]
// (lane 16 lk + li).
//  * fp32 inputs: rows and matrix in fp32 (rows of kR floats), fp32 MFMA
//    16x16x4, contraction order 16 lk + kk (every LDS read of a wave on 64
//    distinct banks).
//  * bf16 inputs: the token rows are exact bf16 values (phi(Q), phi(K), V,
//    dY); the fp32 matrix is split into bf16 high and low parts
//    (m = hi + lo + O(2^-17 m)) and Y = X hi + X lo on bf16 MFMA 16x16x32
//    with fp32 sums: rows of kRB bf16, 8 contraction slots per lane.
// ---------------------------------------------------------------------------
constexpr int kRB = kD + 8;  // bf16 row (144 bytes: 16-byte aligned, conflict-free 16-byte reads)

template <class S>
struct RowsOf {
  static constexpr bool kF32 = sizeof(S) == 4;
  static constexpr int kRowBytes = kF32 ? kR * 4 : kRB * 2;
  static constexpr int kBytes = kBT * kRowBytes;                          // all token rows
  static constexpr int kMatBytes = kF32 ? kD * kR * 4 : 2 * kD * kRB * 2;  // one staged matrix
};

// Quad lane: features f0 .. f0 + 15 of token tk into the token rows.
template <class S>
__device__ __forceinline__ void put_row(unsigned char* rows, int tk, int f0, const float (&x)[kF]) {
  if constexpr (RowsOf<S>::kF32) {
    float* r = reinterpret_cast<float*>(rows) + tk * kR + f0;
#pragma unroll
    for (int e = 0; e < kF; ++e) r[e] = x[e];
  } else {
    uint16_t* r = reinterpret_cast<uint16_t*>(rows) + tk * kRB + f0;
    u32x4 w[2];
#pragma unroll
    for (int e = 0; e < kF; e += 2) w[e / 8][(e % 8) / 2] = f2bf(x[e]) | ((uint32_t)f2bf(x[e + 1]) << 16);
    reinterpret_cast<u32x4*>(r)[0] = w[0];
    reinterpret_cast<u32x4*>(r)[1] = w[1];
  }
}

// Stage elements e .. e + 3 (one row) of a 64 x 64 fp32 matrix, v4, for
// Y = X M^T (kTr) or Y = X M (!kTr).
template <class S, bool kTr>
__device__ __forceinline__ void stage_quad(unsigned char* dst, float4 v4, int e) {
  {
    const float v[4] = {v4.x, v4.y, v4.z, v4.w};
    const int r = e / kD, c = e % kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int at = kTr ? r * (RowsOf<S>::kF32 ? kR : kRB) + c + j : (c + j) * (RowsOf<S>::kF32 ? kR : kRB) + r;
      if constexpr (RowsOf<S>::kF32) {
        reinterpret_cast<float*>(dst)[at] = v[j];
      } else {
        const uint16_t hi = f2bf(v[j]);
        reinterpret_cast<uint16_t*>(dst)[at] = hi;
        reinterpret_cast<uint16_t*>(dst)[kD * kRB + at] = f2bf(v[j] - bf2f(hi));
      }
    }
  }
}
// Whole workgroup: stage the 64 x 64 fp32 matrix src for Y = X src^T
// (kTr) or Y = X src (!kTr).
template <class S, bool kTr>
__device__ __forceinline__ void stage_mat(unsigned char* dst, const float* src) {
  for (int e = threadIdx.x * 4; e < kD * kD; e += blockDim.x * 4)
    stage_quad<S, kTr>(dst, *reinterpret_cast<const float4*>(src + e), e);
}

__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += X Bt^T for the wave's 16 token rows X (the wave's part of the rows).
template <class S>
__device__ __forceinline__ void wave_mm(const unsigned char* X, const unsigned char* Bt, f32x4 (&acc)[4]) {
  const int ln = threadIdx.x % 64, li = ln % 16, lk = ln / 16;
  if constexpr (RowsOf<S>::kF32) {
    const float* x = reinterpret_cast<const float*>(X);
    const float* m = reinterpret_cast<const float*>(Bt);
#pragma unroll 4
    for (int kk = 0; kk < kD / 4; ++kk) {
      const int f = 16 * lk + kk;
      const float av = x[li * kR + f];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] = mfma16(av, m[(16 * ct + li) * kR + f], acc[ct]);
    }
  } else {
    const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
    const uint16_t* hi = reinterpret_cast<const uint16_t*>(Bt);
    const uint16_t* lo = hi + kD * kRB;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int f = 8 * lk + 32 * h;
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(x + li * kRB + f);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int at = (16 * ct + li) * kRB + f;
        acc[ct] = mfma16_bf16(av, *reinterpret_cast<const bf16x8*>(hi + at), acc[ct]);
        acc[ct] = mfma16_bf16(av, *reinterpret_cast<const bf16x8*>(lo + at), acc[ct]);
      }
    }
  }
}

// Y from accumulator layout into the lane-quad layout through the wave's
// token rows X (overwritten): lane (token tw of the wave, quarter f0) gets
// Y[tw][f0 .. f0 + 15].  bf16 rows are too small for 16 fp32 rows: there the
// two column halves pass in turn through 16 rows of 33 floats.
template <class S>
__device__ __forceinline__ void acc_to_quad(const f32x4 (&acc)[4], unsigned char* X, int tw, int f0,
                                            float (&y)[kF]) {
  const int ln = threadIdx.x % 64, li = ln % 16, lk = ln / 16;
  float* x = reinterpret_cast<float*>(X);
  if constexpr (RowsOf<S>::kF32) {
    quad_lds_sync();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[(4 * lk + e) * kR + 16 * ct + li] = acc[ct][e];
    quad_lds_sync();
#pragma unroll
    for (int e = 0; e < kF; ++e) y[e] = x[tw * kR + f0 + e];
  } else {
    constexpr int kH = 33;
    static_assert(16 * kH * 4 <= 16 * kRB * 2, "half rows fit in the wave's bf16 rows");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      quad_lds_sync();
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[(4 * lk + e) * kH + 16 * c2 + li] = acc[2 * h + c2][e];
      quad_lds_sync();
      if (f0 / 32 == h)
#pragma unroll
        for (int e = 0; e < kF; ++e) y[e] = x[tw * kH + f0 % 32 + e];
    }
  }
}

// The wave's 16 token rows of an output (x: this lane's 16 features of its
// token, stored if `on`; tok0: the wave's first token).  bf16: through the
// wave's LDS rows, so that each store instruction writes eight whole
// 128-byte rows, nontemporally (the outputs are not read again here; dirty
// lines would be written back at the kernel's end, on the next kernel's
// time).  fp32: each lane its own 64 bytes.
template <class S>
__device__ __forceinline__ void store_rows(S* out, int tok0, int n, unsigned char* X, int tw, int f0,
                                           const float (&x)[kF], bool on) {
  if constexpr (RowsOf<S>::kF32) {
    if (on) store16(out + (size_t)(tok0 + tw) * kD, f0, x);
  } else {
    quad_lds_sync();
    if (on) put_row<S>(X, tw, f0, x);
    quad_lds_sync();
    const int lane = threadIdx.x % 64;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h + lane / 8, pc = lane % 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(X + r * RowsOf<S>::kRowBytes + 16 * pc);
      if (tok0 + r < n) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + (size_t)(tok0 + r) * kD + 8 * pc));
    }
  }
}

// Sum over the wave (butterfly of fixed shape: the same order every run).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// sum_{p < n} x[p * stride] in order of p, with 8 loads in flight.
__device__ __forceinline__ float sum_in_order(const float* x, size_t stride, int n) {
  float v = 0.f;
  for (int p0 = 0; p0 < n; p0 += 8) {
    float y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) y[u] = p0 + u < n ? x[(size_t)(p0 + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) v += y[u];
  }
  return v;
}

// Whole workgroup: copy a 64 x 64 fp32 matrix into LDS rows of kR floats.
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
  __shared__ float Ms[kD * kR];
  __shared__ float Ps[2][kD * kR];
  const int b = blockIdx.x, t = threadIdx.x, T1 = a.T - 1;
  if (T1 < 1) return;
  const int w = t / 64, li = t % 16, lk = (t % 64) / 16, r0 = 16 * (w % 4), ct = w / 4;
  const float* P1 = a.fin_kv + (size_t)b * kD * kD;
  float* out = a.pk + (size_t)b * T1 * kD * kD;
  load_mat_padded(Ms, a.fin_m + (size_t)b * kD * kD);
  load_mat_padded(Ps[0], P1);
  for (int e = t * 4; e < kD * kD; e += kAdjThreads * 4)
    *reinterpret_cast<float4*>(out + e) = *reinterpret_cast<const float4*>(P1 + e);
  for (int k = 2; k <= T1; ++k) {
    __syncthreads();
    const f32x4 y = tile_mm<false>(Ms + r0 * kR, Ps[k % 2], ct, f32x4{});
    float* Po = Ps[(k + 1) % 2];
    float* o = out + (size_t)(k - 1) * kD * kD;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Po[(r0 + 4 * lk + e) * kR + 16 * ct + li] = y[e];
      o[(r0 + 4 * lk + e) * kD + 16 * ct + li] = y[e];
    }
  }
}

// Pass A: per token the local window statistics, dY . V_i, dY . (Qt_i P_k),
// the weight gradients and dalpha's share; per workgroup the partial sums of
// dP_k = sum_i w_k(i) alpha Qt_i^T dY_i.
//
// fp32 inputs: both contractions on fp32 MFMA 16x16x4 from token rows of kR
// floats, in a term order (features 16 lk + kk, tokens
// 64 (kk / 16) + 16 lk + kk % 16) that keeps every operand read of a wave on
// 64 distinct banks.
// bf16 inputs: phi(Q) and dY are exact bf16 values, kept feature-major
// (kTS tokens per feature row) so that a lane's 8 contraction slots over
// tokens are one 16-byte read.  dY . (Qt_i P_k) = r_i dY_i . (phi(Q_i) P_k)
// with P_k split into bf16 high and low parts; dP_k's operand
// alpha w_k(i) r_i phi(Q_i) is formed per k and split the same way, against
// the exact dY.  Both on bf16 MFMA 16x16x32 with fp32 sums.
constexpr int kTS = kBT + 8;  // bf16 feature-major row: 528 bytes, 16-byte reads conflict-free

template <class S>
constexpr size_t token_a_lds() {
  if constexpr (sizeof(S) == 4)
    return (size_t)(kD * kR + kD + 2 * kBT * kR + kBT * kW + kBT) * sizeof(float);
  else
    return (size_t)4 * kD * kTS * 2 + RowsOf<S>::kMatBytes + ((kMaxTBwd - 1) * kBT + kD + kBT) * sizeof(float);
}

template <class S>
__global__ __launch_bounds__(kTT) void bwd_token_a(BwdArgs a) {
  extern __shared__ __align__(16) float sm[];
  constexpr bool kF32 = RowsOf<S>::kF32;
  // fp32 layout: P_k, Qt rows, dY rows, weights.
  float* Ps = sm;
  float* qt_sh = Ps + kD * kR;
  float* dy_sh = qt_sh + kBT * kR;
  float* w_sh = dy_sh + kBT * kR;
  // bf16 layout: split alpha w_k r phi(Q) (high, low), phi(Q), dY (all
  // feature-major), P_k staged, per-token scales alpha w_k r.
  uint16_t* sqh = reinterpret_cast<uint16_t*>(sm);
  uint16_t* sql = sqh + kD * kTS;
  uint16_t* qT = sql + kD * kTS;
  uint16_t* dyT = qT + kD * kTS;
  unsigned char* Pst = reinterpret_cast<unsigned char*>(dyT + kD * kTS);
  float* stab = reinterpret_cast<float*>(Pst + RowsOf<S>::kMatBytes);
  float* s_sh = kF32 ? w_sh + kBT * kW : stab + (kMaxTBwd - 1) * kBT;  // kD
  float* red = s_sh + kD;                                             // kBT
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
  // bf16: this thread's float4 of P_1, loaded before the window gather.
  float4 pnext = make_float4(0.f, 0.f, 0.f, 0.f);
  if (!kF32 && a.T >= 2) pnext = *reinterpret_cast<const float4*>(a.pk + (size_t)b * (a.T - 1) * kD * kD + 4 * t);
  float wk[kMaxTBwd];
#pragma unroll
  for (int k = 0; k < kMaxTBwd; ++k) wk[k] = (on && k < a.T) ? wgt(a, base + i, k) : 0.f;
  if (kF32 && qd == 0)
#pragma unroll
    for (int k = 0; k < kMaxTBwd; ++k) w_sh[tk * kW + k] = wk[k];

  float q[kF], dy[kF];
  float m = 0.f, Z = 1.f, dyL = 0.f, dyv = 0.f;
  if (on) {
    Piece<S> qp, dyp;  // raw Q_i and dY_i as loaded, for the window's dot products
    qp.load(Qb + (size_t)i * kD, f0);
    dyp.load(dYb + (size_t)i * kD, f0);
#pragma unroll
    for (int e = 0; e < kF; ++e) {
      q[e] = qp[e];
      dy[e] = dyp[e];
    }
    // Local branch at token i: window logits, their max and sum, dY . L_i.
    const int row = i / a.W, col = i % a.W;
    // The window's rows three at a time (one grid row of it), loaded without
    // branches: an off-grid cell loads token i's own row and its result is
    // masked.  Sums run over j = 0 .. 8 in order, as over the valid cells.
    int cw[9];
#pragma unroll
    for (int j = 0; j < 9; ++j) cw[j] = window_cell(a, row, col, j);
    float z[9];
    m = -INFINITY;
#pragma unroll
    for (int g0 = 0; g0 < 9; g0 += 3) {
      Piece<S> y[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) y[u].load(Kb + (size_t)(cw[g0 + u] >= 0 ? cw[g0 + u] : i) * kD, f0);
#pragma unroll
      for (int u = 0; u < 3; ++u) y[u].pin();
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const float d = quad_sum(dotp(qp, y[u]));
        z[g0 + u] = cw[g0 + u] >= 0 ? d * kRs : -INFINITY;
        m = fmaxf(m, z[g0 + u]);
      }
    }
    Z = 0.f;
#pragma unroll
    for (int g0 = 0; g0 < 9; g0 += 3) {
      Piece<S> y[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) y[u].load(Vb + (size_t)(cw[g0 + u] >= 0 ? cw[g0 + u] : i) * kD, f0);
#pragma unroll
      for (int u = 0; u < 3; ++u) y[u].pin();
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const float d = quad_sum(dotp(dyp, y[u]));
        if (cw[g0 + u] >= 0) {
          const float e = __expf(z[g0 + u] - m);
          Z += e;
          dyL += e * d;
        }
      }
    }
    dyL /= Z;
    Piece<S> vi;
    vi.load(Vb + (size_t)i * kD, f0);
    dyv = quad_sum(dotp(dyp, vi));
  } else {
#pragma unroll
    for (int e = 0; e < kF; ++e) q[e] = dy[e] = 0.f;
  }
  __syncthreads();  // s_sh, w_sh
  // r_i = 1 / (phi(Q_i) . s + eps).
  float den = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) {
    q[e] = fmaxf(q[e], 0.f);
    den += q[e] * s_sh[f0 + e];
  }
  const float r = 1.f / (quad_sum(den) + a.eps);
  float dyy[kMaxTBwd];
#pragma unroll
  for (int k = 0; k < kMaxTBwd; ++k) dyy[k] = 0.f;
  const int T1 = a.T - 1;
  // MFMA roles: wave wv holds tokens 16 wv .. 16 wv + 15 (its quads) and the
  // 16 x 16 block (ga, gc) of dP_k; lane ln = 16 lk + li.
  const int wv = t / 64, ln = t % 64, li = ln % 16, lk = ln / 16;
  const int ga = 16 * (wv / 4), gc = 16 * (wv % 4);
  if constexpr (kF32) {
#pragma unroll
    for (int e = 0; e < kF; ++e) {
      qt_sh[tk * kR + f0 + e] = q[e] * r;
      dy_sh[tk * kR + f0 + e] = dy[e];
    }
#pragma unroll
    for (int k = 1; k < kMaxTBwd; ++k) {
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
  } else {
    // Feature-major phi(Q) and dY (exact), the per-token scales.
#pragma unroll
    for (int e = 0; e < kF; ++e) {
      qT[(f0 + e) * kTS + tk] = f2bf(q[e]);
      dyT[(f0 + e) * kTS + tk] = f2bf(dy[e]);
    }
    if (qd == 0)
#pragma unroll
      for (int k = 1; k < kMaxTBwd; ++k)
        if (k <= T1) stab[(k - 1) * kBT + tk] = alpha * wk[k] * r;
    quad_lds_sync();
    // This wave's operands, fixed over k: A = phi(Q) of its 16 tokens
    // (row li, slots 8 lk + 32 h + j) and dY in accumulator layout.
    bf16x8 av[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        av[h][j] = __builtin_bit_cast(__bf16, qT[(8 * lk + 32 * h + j) * kTS + 16 * wv + li]);
    float dyd[4][4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) dyd[ct][e] = bf2f(dyT[(16 * ct + li) * kTS + 16 * wv + 4 * lk + e]);
    const uint16_t* Ph = reinterpret_cast<const uint16_t*>(Pst);
    const uint16_t* Pl = Ph + kD * kRB;
    static_assert(kTT * 4 == kD * kD, "one float4 of each P_k per thread");
#pragma unroll
    for (int k = 1; k < kMaxTBwd; ++k) {
      if (k > T1) break;
      __syncthreads();
      stage_quad<S, false>(Pst, pnext, 4 * t);
      // The next term's matrix, in flight over this term's products.
      if (k < T1) pnext = *reinterpret_cast<const float4*>(a.pk + ((size_t)b * T1 + k) * kD * kD + 4 * t);
      {
        // alpha w_k r phi(Q), split: feature t / 16, tokens 16 (t % 16) .. + 15.
        const int fa = t / 16, t0 = 16 * (t % 16);
        const float* sc = stab + (k - 1) * kBT + t0;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const u32x4 qv = *reinterpret_cast<const u32x4*>(qT + fa * kTS + t0 + 8 * hh);
          u32x4 hv, lv;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v0 = sc[8 * hh + 2 * j] * __uint_as_float(qv[j] << 16);
            const float v1 = sc[8 * hh + 2 * j + 1] * __uint_as_float(qv[j] & 0xffff0000u);
            const uint16_t h0 = f2bf(v0), h1 = f2bf(v1);
            hv[j] = h0 | ((uint32_t)h1 << 16);
            lv[j] = f2bf(v0 - bf2f(h0)) | ((uint32_t)f2bf(v1 - bf2f(h1)) << 16);
          }
          *reinterpret_cast<u32x4*>(sqh + fa * kTS + t0 + 8 * hh) = hv;
          *reinterpret_cast<u32x4*>(sql + fa * kTS + t0 + 8 * hh) = lv;
        }
      }
      __syncthreads();
      // dY_i . (Qt_i P_k) = r_i (phi(Q_i) P_k) . dY_i.
      {
        f32x4 x[4] = {};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const int at = (16 * ct + li) * kRB + 8 * lk + 32 * h;
            x[ct] = mfma16_bf16(av[h], *reinterpret_cast<const bf16x8*>(Ph + at), x[ct]);
            x[ct] = mfma16_bf16(av[h], *reinterpret_cast<const bf16x8*>(Pl + at), x[ct]);
          }
        float part[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = 0.f;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) v += x[ct][e] * dyd[ct][e];
          part[e] = group_sum16(v);
        }
        const int e = li / 4;
        dyy[k] = r * (e == 0 ? part[0] : e == 1 ? part[1] : e == 2 ? part[2] : part[3]);
      }
      // This workgroup's share of dP_k.
      {
        f32x4 acc = {};
#pragma unroll
        for (int h = 0; h < kBT / 32; ++h) {
          const int ta = (ga + li) * kTS + 8 * lk + 32 * h, tb = (gc + li) * kTS + 8 * lk + 32 * h;
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(dyT + tb);
          acc = mfma16_bf16(*reinterpret_cast<const bf16x8*>(sqh + ta), bv, acc);
          acc = mfma16_bf16(*reinterpret_cast<const bf16x8*>(sql + ta), bv, acc);
        }
        float* dst = a.dp_part + (((size_t)b * a.nblk + blk) * T1 + (k - 1)) * kD * kD;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(ga + 4 * lk + e) * kD + gc + li] = acc[e];
      }
    }
  }
  // Scalars of the token (every lane of the quad holds them).
  float wy = 0.f;
#pragma unroll
  for (int k = 1; k < kMaxTBwd; ++k)
    if (k <= T1) wy += wk[k] * dyy[k];
  const float dyG = wk[0] * dyv + wy;
  if (on && qd == 0) {
    // a_i = (sum_k w_k P_k dG_i) . phi(Q_i) = alpha / r_i * sum_k w_k dY_i . (Qt_i P_k)
    a.tok[base + i] = make_float4(m, Z, (1.f - alpha) * dyL, alpha / r * wy);
    if (a.dweights) {
      float* dw = a.dweights + (base + i) * a.T;
      dw[0] = alpha * dyv;
#pragma unroll
      for (int k = 1; k < kMaxTBwd; ++k)
        if (k <= T1) dw[k] = alpha * dyy[k];
    }
  }
  // dalpha's share: sum_i dY_i . (G_i - L_i), in a fixed order: each wave's
  // 16 tokens by a butterfly (the quad's lanes hold the same value: every
  // fourth lane takes part), then the 16 waves' sums in order.
  {
    float v = on && qd == 0 ? dyG - dyL : 0.f;
    v = wave_sum(v);
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    if (t == 0) {
      float u = 0.f;
      for (int w2 = 0; w2 < kTT / 64; ++w2) u += red[w2];
      a.da_part[(size_t)b * a.nblk + blk] = u;
    }
  }
}

// dP_k (the token workgroups' partials, summed in order); then, from the
// last term down, dM += dP_k P_(k-1)^T and dP_(k-1) += M^T dP_k; dKV = dP_1.
// One workgroup per slice.
__global__ __launch_bounds__(kAdjThreads) void bwd_adjoint(BwdArgs a) {
  extern __shared__ __align__(16) float sm[];
  const int b = blockIdx.x, t = threadIdx.x, T1 = a.T - 1;
  float* dMo = a.dmkv + (size_t)b * 2 * kD * kD;
  float* dKVo = dMo + kD * kD;
  // The slice's share of dalpha: lane-strided sums, then the wave's butterfly.
  if (t < 64) {
    float v = 0.f;
    for (int p = t; p < a.nblk; p += 64) v += a.da_part[(size_t)b * a.nblk + p];
    v = wave_sum(v);
    if (t == 0) a.da_slice[b] = v;
  }
  if (T1 < 1) {
    for (int e = t; e < kD * kD; e += kAdjThreads) dMo[e] = dKVo[e] = 0.f;
    return;
  }
  const int w = t / 64, li = t % 16, lk = (t % 64) / 16, r0 = 16 * (w % 4), ct = w / 4;
  float* dP = sm;                          // T1 blocks of kD rows of kR
  float* MT = dP + (size_t)T1 * kD * kR;   // M^T
  float* Pp = MT + kD * kR;                // P_(k-1)
  const int per = T1 * kD * kD;
  const float* part = a.dp_part + (size_t)b * a.nblk * per;
  // Each sum in workgroup order; 4 elements x 8 partials of loads in flight.
  for (int j0 = 0; j0 < per / kAdjThreads; j0 += 4) {
    float v[4] = {};
    for (int p0 = 0; p0 < a.nblk; p0 += 8) {
      float x[4][8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          x[jj][u] = p0 + u < a.nblk ? part[(size_t)(p0 + u) * per + (j0 + jj) * kAdjThreads + t] : 0.f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int u = 0; u < 8; ++u) v[jj] += x[jj][u];
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int e = (j0 + jj) * kAdjThreads + t;
      dP[(e / (kD * kD)) * kD * kR + ((e / kD) % kD) * kR + e % kD] = v[jj];
    }
  }
  const float* M = a.fin_m + (size_t)b * kD * kD;
  for (int e = t; e < kD * kD; e += kAdjThreads) MT[(e % kD) * kR + e / kD] = M[e];
  f32x4 dm = {};
  for (int k = T1; k >= 2; --k) {
    __syncthreads();
    load_mat_padded(Pp, a.pk + ((size_t)b * T1 + (k - 2)) * kD * kD);
    __syncthreads();
    const float* dPk = dP + (size_t)(k - 1) * kD * kR;
    dm = tile_mm<true>(dPk + r0 * kR, Pp, ct, dm);                   // dP_k P_(k-1)^T
    const f32x4 up = tile_mm<false>(MT + r0 * kR, dPk, ct, f32x4{});  // M^T dP_k
    float* dPm = dP + (size_t)(k - 2) * kD * kR;
#pragma unroll
    for (int e = 0; e < 4; ++e) dPm[(r0 + 4 * lk + e) * kR + 16 * ct + li] += up[e];
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; ++e) dMo[(r0 + 4 * lk + e) * kD + 16 * ct + li] = dm[e];
  for (int e = t; e < kD * kD; e += kAdjThreads) dKVo[e] = dP[(e / kD) * kR + e % kD];
}

// Pass B: dz_i = -r_i^2 (a_i + phi(K_i)^T dM phi(Q_i)) (kept in tok[i].w) and
// the workgroup's share of ds = sum_i dz_i phi(Q_i).
template <class S>
__global__ __launch_bounds__(kTT) void bwd_token_b(BwdArgs a) {
  constexpr int kG = kTT / kD;  // partial sums per feature in the ds reduction
  using RS = RowsOf<S>;
  __shared__ __align__(16) unsigned char dMs[RS::kMatBytes];
  __shared__ float s_sh[kD];
  __shared__ __align__(16) float rows[kBT * kR];  // fp32 rows for ds; first the MFMA token rows
  __shared__ float red[kG * kD];
  static_assert(RS::kBytes <= (int)sizeof(rows), "MFMA token rows fit");
  const int b = blockIdx.y, t = threadIdx.x, blk = blockIdx.x;
  const int tk = t / kQ, qd = t % kQ, f0 = qd * kF, tw = tk % 16;
  unsigned char* trows = reinterpret_cast<unsigned char*>(rows);
  unsigned char* wrows = trows + (t / 64) * 16 * RS::kRowBytes;  // this wave's 16 token rows
  const int i = blk * kBT + tk;
  const bool on = i < a.n;
  const size_t base = (size_t)b * a.n;
  stage_mat<S, false>(dMs, a.dmkv + (size_t)b * 2 * kD * kD);
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
  for (int e = 0; e < kF; ++e) kp[e] = fmaxf(kp[e], 0.f);
  put_row<S>(trows, tk, f0, kp);
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
  wave_mm<S>(wrows, dMs, acc);
  float y[kF];
  acc_to_quad<S>(acc, wrows, tw, f0, y);
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
  // dalpha[h] = sum of the slices' shares over the batch: one wave per head.
  if (b == 0 && blk == 0)
    for (int h = t / 64; h < a.heads; h += kTT / 64) {
      float v = 0.f;
      for (int bb = t % 64; bb < a.BH / a.heads; bb += 64) v += a.da_slice[(size_t)bb * a.heads + h];
      v = wave_sum(v);
      if (t % 64 == 0) a.dalpha[h] = v;
    }
}

// dQ_i = (r_i dQt_i + dz_i s) [Q_i > 0] + sum_j dz_ij k_j / 8, with
// dQt_i = dM^T phi(K_i) + sum_k w_k P_k dG_i and dz_ij the softmax adjoint
// of window slot j.
template <class S>
__global__ __launch_bounds__(kTT) void bwd_token_q(BwdArgs a) {
  using RS = RowsOf<S>;
  __shared__ __align__(16) unsigned char Ps[RS::kMatBytes];
  __shared__ __align__(16) unsigned char dMs[RS::kMatBytes];
  __shared__ float s_sh[kD];
  __shared__ __align__(16) unsigned char trows[RS::kBytes];
  const int b = blockIdx.y, t = threadIdx.x, blk = blockIdx.x;
  const int tk = t / kQ, qd = t % kQ, f0 = qd * kF, tw = tk % 16;
  unsigned char* wrows = trows + (t / 64) * 16 * RS::kRowBytes;
  const int i = blk * kBT + tk;
  const bool on = i < a.n;
  const size_t base = (size_t)b * a.n;
  const float alpha = a.alpha[b % a.heads];
  const S* Qb = static_cast<const S*>(a.Q) + base * kD;
  const S* Kb = static_cast<const S*>(a.K) + base * kD;
  const S* Vb = static_cast<const S*>(a.V) + base * kD;
  const S* dYb = static_cast<const S*>(a.dY) + base * kD;
  stage_mat<S, false>(dMs, a.dmkv + (size_t)b * 2 * kD * kD);
  if (t < kD) s_sh[t] = a.fin_s[(size_t)b * kD + t];
  // This thread's float4 of P_1 (one float4 of each P_k per thread).
  static_assert(kTT * 4 == kD * kD, "one float4 of each P_k per thread");
  float4 pnext = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.T >= 2) pnext = *reinterpret_cast<const float4*>(a.pk + (size_t)b * (a.T - 1) * kD * kD + 4 * t);
  float x[kF];
  if (on) load16(Kb + (size_t)i * kD, f0, x);
  else
#pragma unroll
    for (int e = 0; e < kF; ++e) x[e] = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) x[e] = fmaxf(x[e], 0.f);
  put_row<S>(trows, tk, f0, x);
  __syncthreads();
  // dQt rows: phi(K) dM, then + sum_k diag(alpha w_k) dY P_k^T.
  f32x4 acc[4] = {};
  wave_mm<S>(wrows, dMs, acc);
  if (on) load16(dYb + (size_t)i * kD, f0, x);
  else
#pragma unroll
    for (int e = 0; e < kF; ++e) x[e] = 0.f;
  quad_lds_sync();
  put_row<S>(trows, tk, f0, x);
  const int T1 = a.T - 1;
  // Accumulator rows 4 lk + e of this lane: tokens ib + e.
  const int ib = blk * kBT + (t / 64) * 16 + 4 * ((t % 64) / 16);
  for (int k = 1; k <= T1; ++k) {
    __syncthreads();
    stage_quad<S, true>(Ps, pnext, 4 * t);
    // The next term's matrix, in flight over this term's products.
    if (k < T1) pnext = *reinterpret_cast<const float4*>(a.pk + ((size_t)b * T1 + k) * kD * kD + 4 * t);
    __syncthreads();
    f32x4 y[4] = {};
    wave_mm<S>(wrows, Ps, y);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float f = ib + e < a.n ? alpha * wgt(a, base + ib + e, k) : 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct][e] += f * y[ct][e];
    }
  }
  float dqt[kF];
  acc_to_quad<S>(acc, wrows, tw, f0, dqt);
  if (on) {
  const float4 tp = a.tok[base + i];  // m_i, Z_i, c_i, dz_i
  Piece<S> qp, dyp;  // raw Q_i and dY_i as loaded, for the window's dot products
  qp.load(Qb + (size_t)i * kD, f0);
  dyp.load(dYb + (size_t)i * kD, f0);
  float q[kF];
#pragma unroll
  for (int e = 0; e < kF; ++e) q[e] = qp[e];
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
    Piece<S> kc, vc;
    kc.load(Kb + (size_t)c * kD, f0);
    vc.load(Vb + (size_t)c * kD, f0);
    kc.pin();
    vc.pin();
    const float p = __expf(quad_sum(dotp(kc, qp)) * kRs - tp.x) / tp.y;
    const float g = p * ((1.f - alpha) * quad_sum(dotp(vc, dyp)) - tp.z) * kRs;
#pragma unroll
    for (int e = 0; e < kF; ++e) dqt[e] += g * kc[e];
  }
  }
  store_rows<S>(static_cast<S*>(a.dQ) + base * kD, blk * kBT + (t / 64) * 16, a.n, wrows, tw, f0, dqt, on);
}

// dK_j = (dM Qt_j + dKV V_j + ds) [K_j > 0] + sum_i dz_ij q_i / 8 and
// dV_j = w_0(j) alpha dY_j + dKV^T phi(K_j) + sum_i p_ij (1 - alpha) dY_i,
// the local sums over the centres i whose window holds j (the window
// relation is symmetric); both share p_ij and the rows q_i, dY_i.
template <class S>
__global__ __launch_bounds__(kTT) void bwd_token_kv(BwdArgs a) {
  using RS = RowsOf<S>;
  __shared__ __align__(16) unsigned char dMs[RS::kMatBytes];    // for phi(Q) dM^T
  __shared__ __align__(16) unsigned char dKVt[RS::kMatBytes];   // for V dKV^T
  __shared__ __align__(16) unsigned char dKVs[RS::kMatBytes];   // for phi(K) dKV
  __shared__ float s_sh[kD];
  __shared__ float ds_sh[kD];
  __shared__ __align__(16) unsigned char trows[RS::kBytes];
  const int b = blockIdx.y, t = threadIdx.x, blk = blockIdx.x;
  const int tk = t / kQ, qd = t % kQ, f0 = qd * kF, tw = tk % 16;
  unsigned char* wrows = trows + (t / 64) * 16 * RS::kRowBytes;
  const int i = blk * kBT + tk;
  const bool on = i < a.n;
  const size_t base = (size_t)b * a.n;
  const float alpha = a.alpha[b % a.heads];
  const S* Qb = static_cast<const S*>(a.Q) + base * kD;
  const S* Kb = static_cast<const S*>(a.K) + base * kD;
  const S* Vb = static_cast<const S*>(a.V) + base * kD;
  const S* dYb = static_cast<const S*>(a.dY) + base * kD;
  const float* dM = a.dmkv + (size_t)b * 2 * kD * kD;
  stage_mat<S, true>(dMs, dM);
  stage_mat<S, true>(dKVt, dM + kD * kD);
  stage_mat<S, false>(dKVs, dM + kD * kD);
  if (t < kD) {
    s_sh[t] = a.fin_s[(size_t)b * kD + t];
    ds_sh[t] = sum_in_order(a.ds_part + (size_t)b * a.nblk * kD + t, kD, a.nblk);
  }
  float x[kF], kr[kF];
  if (on) {
    load16(Qb + (size_t)i * kD, f0, x);
    load16(Kb + (size_t)i * kD, f0, kr);
  } else {
#pragma unroll
    for (int e = 0; e < kF; ++e) x[e] = kr[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < kF; ++e) x[e] = fmaxf(x[e], 0.f);
  put_row<S>(trows, tk, f0, x);
  __syncthreads();
  // Rows Qt_j dM^T + V_j dKV^T (dK's global part) and phi(K_j) dKV (dV's);
  // Qt_j = r_j phi(Q_j), with r_j applied to the product.
  float den = 0.f;
#pragma unroll
  for (int e = 0; e < kF; ++e) den += x[e] * s_sh[f0 + e];
  const float r = 1.f / (quad_sum(den) + a.eps);
  f32x4 accq[4] = {}, acck[4] = {}, accv[4] = {};
  wave_mm<S>(wrows, dMs, accq);
  if (on) load16(Vb + (size_t)i * kD, f0, x);
  quad_lds_sync();
  put_row<S>(trows, tk, f0, x);
  quad_lds_sync();
  wave_mm<S>(wrows, dKVt, acck);
  {
    const int lk = (t % 64) / 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float re = __shfl(r, 4 * (4 * lk + e));  // r of accumulator row 4 lk + e
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acck[ct][e] += re * accq[ct][e];
    }
  }
  float kp[kF];
#pragma unroll
  for (int e = 0; e < kF; ++e) kp[e] = fmaxf(kr[e], 0.f);
  quad_lds_sync();
  put_row<S>(trows, tk, f0, kp);
  quad_lds_sync();
  wave_mm<S>(wrows, dKVs, accv);
  float dk[kF], dv[kF];
  acc_to_quad<S>(acck, wrows, tw, f0, dk);
  acc_to_quad<S>(accv, wrows, tw, f0, dv);
  if (on) {
#pragma unroll
  for (int e = 0; e < kF; ++e) dk[e] = kr[e] > 0.f ? dk[e] + ds_sh[f0 + e] : 0.f;
  {
    float dy[kF];
    load16(dYb + (size_t)i * kD, f0, dy);
    const float w0 = alpha * wgt(a, base + i, 0);
#pragma unroll
    for (int e = 0; e < kF; ++e) dv[e] += w0 * dy[e];
  }
  // Local: token i as the neighbour of centre c (x holds V_i).
  const int row = i / a.W, col = i % a.W;
#pragma unroll 1
  for (int j = 0; j < 9; ++j) {
    const int c = window_cell(a, row, col, j);
    if (c < 0) continue;
    const float4 tc = a.tok[base + c];
    float qc[kF], yc[kF];
    load16(Qb + (size_t)c * kD, f0, qc);
    load16(dYb + (size_t)c * kD, f0, yc);
    float zq = 0.f, zy = 0.f;
#pragma unroll
    for (int e = 0; e < kF; ++e) {
      zq += qc[e] * kr[e];
      zy += yc[e] * x[e];
    }
    const float p = __expf(quad_sum(zq) * kRs - tc.x) / tc.y;
    const float g = p * ((1.f - alpha) * quad_sum(zy) - tc.z) * kRs;
    const float pv = p * (1.f - alpha);
#pragma unroll
    for (int e = 0; e < kF; ++e) {
      dk[e] += g * qc[e];
      dv[e] += pv * yc[e];
    }
  }
  }
  store_rows<S>(static_cast<S*>(a.dK) + base * kD, blk * kBT + (t / 64) * 16, a.n, wrows, tw, f0, dk, on);
  store_rows<S>(static_cast<S*>(a.dV) + base * kD, blk * kBT + (t / 64) * 16, a.n, wrows, tw, f0, dv, on);
}

template <class S>
hipError_t launch_typed(const BwdArgs& a, hipStream_t s) {
  const size_t lds_a = token_a_lds<S>();
  const int T1 = a.T - 1 > 0 ? a.T - 1 : 1;
  const size_t lds_adj = ((size_t)T1 + 2) * kD * kR * sizeof(float);
  static std::atomic<bool> lds_set_a[kMaxDevices], lds_set_adj[kMaxDevices];
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&bwd_token_a<S>), (int)lds_a, lds_set_a);
  if (e != hipSuccess) return e;
  const size_t lds_adj_max = ((size_t)kMaxTBwd + 1) * kD * kR * sizeof(float);
  e = ensure_lds_limit(reinterpret_cast<const void*>(&bwd_adjoint), (int)lds_adj_max, lds_set_adj);
  if (e != hipSuccess) return e;
  const dim3 tok(a.nblk, a.BH);
  if (a.T >= 2) hipLaunchKernelGGL(bwd_powers, dim3(a.BH), dim3(kAdjThreads), 0, s, a);
  hipLaunchKernelGGL(bwd_token_a<S>, tok, dim3(kTT), lds_a, s, a);
  hipLaunchKernelGGL(bwd_adjoint, dim3(a.BH), dim3(kAdjThreads), lds_adj, s, a);
  hipLaunchKernelGGL(bwd_token_b<S>, tok, dim3(kTT), 0, s, a);
  hipLaunchKernelGGL(bwd_token_q<S>, tok, dim3(kTT), 0, s, a);
  hipLaunchKernelGGL(bwd_token_kv<S>, tok, dim3(kTT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(int dtype, const BwdArgs& a, hipStream_t s) {
  return dtype == 1 ? launch_typed<uint16_t>(a, s) : launch_typed<float>(a, s);
}

}  // namespace lisa
