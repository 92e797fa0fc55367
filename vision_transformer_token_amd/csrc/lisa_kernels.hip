// gfx950 kernels of the LiSA forward pass.
//
// Method: reading note "LiSA:面向长程视觉建模的线性随机注意力" (arXiv:2611.04216v2),
// §2.1-§2.4.  Per (batch, head) with n tokens of width 64:
//   statistics (Eq. 8): s = sum_j phi(K_j), phi(K)^T V, M = phi(K)^T Qt,
//     Qt_i = phi(Q_i) / (phi(Q_i) . s + eps), phi = ReLU;
//   output: G_i = w_0(i) V_i + r_i sum_{k=1}^{T-1} w_k(i) (phi(Q_i) M^(k-1)) (phi(K)^T V),
//     r_i = 1 / (phi(Q_i) . s + eps), which is row i of sum_k diag(w_k) S^k V;
//     L_i = 3x3 masked softmax attention; Y_i = alpha G_i + (1 - alpha) L_i.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2f32, lane l,
// m = l % 32, h = l / 32): A[m][8h + e] and B[8h + e][m] (bf16, e = 0..7) or
// A[m][h], B[h][m] (fp32); accumulator element i holds
// C[8 (i / 4) + 4 h + i % 4][m].  The contraction index may be permuted as
// long as A and B agree, which the kernels use to feed an accumulator
// straight back in as the next B operand (see dimof).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lisa_kernels.hpp"

namespace lisa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// Element traits.  EPL: contraction slots per lane in one MFMA; NQ: MFMAs
// needed to contract over 64; EPP: elements per 16-byte global piece.
struct BF16 {
  using S = uint16_t;
  using Frag = bf16x8;
  static constexpr int EPL = 8;
  static constexpr int NQ = 4;
  static constexpr int EPP = 8;
};
struct F32 {
  using S = float;
  using Frag = float;
  static constexpr int EPL = 1;
  static constexpr int NQ = 32;
  static constexpr int EPP = 4;
};

__device__ __forceinline__ void from_f(float x, uint16_t& out) {
  __bf16 h = (__bf16)x;  // round to nearest even
  out = __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ void from_f(float x, float& out) { out = x; }

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Feature dimension held in value slot v (0..31) by a lane of half h, for a
// 64-vector kept in accumulator layout: slots 0..15 are the first 32x32
// block's 16 accumulators, 16..31 the second's.
__device__ __forceinline__ int dimof(int v, int h) {
  return 32 * (v >> 4) + 8 * ((v >> 2) & 3) + 4 * h + (v & 3);
}

// 16-byte piece <-> EPP floats.
__device__ __forceinline__ void unpack16(uint4 p, float (&x)[8], BF16) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(uint4 p, float (&x)[4], F32) {
  x[0] = __uint_as_float(p.x);
  x[1] = __uint_as_float(p.y);
  x[2] = __uint_as_float(p.z);
  x[3] = __uint_as_float(p.w);
}
__device__ __forceinline__ uint4 pack16(const float (&x)[8], BF16) {
  uint16_t b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) from_f(x[i], b[i]);
  return make_uint4(b[0] | ((uint32_t)b[1] << 16), b[2] | ((uint32_t)b[3] << 16),
                    b[4] | ((uint32_t)b[5] << 16), b[6] | ((uint32_t)b[7] << 16));
}
__device__ __forceinline__ uint4 pack16(const float (&x)[4], F32) {
  return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                    __float_as_uint(x[3]));
}

// 16-byte piece into LDS at an 8-byte-aligned (bf16) or 16-byte-aligned
// (fp32) address.
__device__ __forceinline__ void lds_store16(uint16_t* dst, uint4 p) {
  uint2* d = reinterpret_cast<uint2*>(dst);
  d[0] = make_uint2(p.x, p.y);
  d[1] = make_uint2(p.z, p.w);
}
__device__ __forceinline__ void lds_store16(float* dst, uint4 p) {
  *reinterpret_cast<uint4*>(dst) = p;
}

// Four consecutive elements (8 B bf16 / 16 B fp32) <-> floats.
__device__ __forceinline__ void load4(const uint16_t* p, float* x) {
  uint2 w = *reinterpret_cast<const uint2*>(p);
  x[0] = __uint_as_float(w.x << 16);
  x[1] = __uint_as_float(w.x & 0xffff0000u);
  x[2] = __uint_as_float(w.y << 16);
  x[3] = __uint_as_float(w.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float* x) {
  float4 w = *reinterpret_cast<const float4*>(p);
  x[0] = w.x;
  x[1] = w.y;
  x[2] = w.z;
  x[3] = w.w;
}
__device__ __forceinline__ void store4(uint16_t* p, const float* x) {
  uint16_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) from_f(x[i], b[i]);
  *reinterpret_cast<uint2*>(p) = make_uint2(b[0] | ((uint32_t)b[1] << 16), b[2] | ((uint32_t)b[3] << 16));
}
__device__ __forceinline__ void store4(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// MFMA operand from EPL slots of a 32-slot fp32 vector, starting at slot q*EPL.
__device__ __forceinline__ bf16x8 operand(const float (&u)[32], int q, BF16) {
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = (__bf16)u[8 * q + e];
  return b;
}
__device__ __forceinline__ float operand(const float (&u)[32], int q, F32) { return u[q]; }

// MFMA operand of 8/EPL... gathered from an LDS tile [token][kCellStride]:
// tokens row0 + e (e < EPL), feature column col.
__device__ __forceinline__ bf16x8 gather(const uint16_t* t, int row0, int col, BF16) {
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = __builtin_bit_cast(__bf16, t[(row0 + e) * kCellStride + col]);
  return b;
}
__device__ __forceinline__ float gather(const float* t, int row0, int col, F32) {
  return t[row0 * kCellStride + col];
}

// y = x X for a 64-vector x in accumulator layout (32 slots per lane), with
// X given as A-operand fragments (see write_fragments); y in the same layout.
template <class Tr>
__device__ __forceinline__ void apply(const typename Tr::Frag (&fr)[2][Tr::NQ], const float (&x)[32],
                                      float (&y)[32]) {
  f32x16 c0 = {}, c1 = {};
#pragma unroll
  for (int q = 0; q < Tr::NQ; ++q) {
    auto b = operand(x, q, Tr{});
    c0 = mma(fr[0][q], b, c0);
    c1 = mma(fr[1][q], b, c1);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    y[i] = c0[i];
    y[16 + i] = c1[i];
  }
}

// ---------------------------------------------------------------------------
// Statistics kernels (one launch per stage).  grid = (P chunks, batch*heads),
// 4 waves.  Each chunk is swept in tiles of 64 tokens staged through LDS;
// wave w owns output block (w / 2, w % 2) of the 64x64 result and runs the
// contraction over tokens on MFMA with both operands gathered from LDS.
// ---------------------------------------------------------------------------

// Writes the A-operand fragments of the 64x64 matrix X (fp32, row-major, in
// LDS) used by apply(): fragment (mb, q, lane, e) = X[dimof(q*EPL + e, lane/32)][32 mb + lane%32].
template <class Tr>
__device__ void write_fragments(const float* X, typename Tr::S* frag) {
  for (int f = threadIdx.x; f < 4096; f += kThreads) {
    const int e = f % Tr::EPL;
    const int lane = (f / Tr::EPL) & 63;
    const int q = (f / (Tr::EPL * 64)) % Tr::NQ;
    const int mb = f / (Tr::EPL * 64 * Tr::NQ);
    const int row = dimof(q * Tr::EPL + e, lane >> 5);
    const int col = 32 * mb + (lane & 31);
    from_f(X[row * 64 + col], frag[f]);
  }
}

template <class Tr, bool kM>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a) {
  using S = typename Tr::S;
  constexpr int PPT = kD / Tr::EPP;  // 16-byte pieces per token row
  __shared__ __align__(16) S tk[kStatTile * kCellStride];
  __shared__ __align__(16) S tx[kStatTile * kCellStride];
  __shared__ __align__(16) float red[kD * kD];
  __shared__ float s_sh[kD];
  __shared__ float s_red[kThreads][Tr::EPP];
  __shared__ int last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int mb = wave >> 1, nb = wave & 1;
  const int bh = blockIdx.y, p = blockIdx.x;
  const int tok0 = p * a.chunk;
  const int tok1 = min(a.n, tok0 + a.chunk);
  const S* Kb = static_cast<const S*>(a.K) + (size_t)bh * a.n * kD;
  const S* Xb = static_cast<const S*>(a.X) + (size_t)bh * a.n * kD;

  if (kM) {
    if (tid < kD) s_sh[tid] = a.s_in[bh * kD + tid];
    __syncthreads();
  }
  const int g = tid % PPT;  // this thread's feature piece, fixed across tiles
  float sacc[Tr::EPP];
#pragma unroll
  for (int e = 0; e < Tr::EPP; ++e) sacc[e] = 0.f;
  f32x16 acc = {};

  for (int t0 = tok0; t0 < tok1; t0 += kStatTile) {
    for (int pc = tid; pc < kStatTile * PPT; pc += kThreads) {
      const int tt = pc / PPT;
      const int tok = t0 + tt;
      float kv[Tr::EPP], xv[Tr::EPP];
      uint4 kr = make_uint4(0, 0, 0, 0), xr = make_uint4(0, 0, 0, 0);
      if (tok < tok1) {
        kr = *reinterpret_cast<const uint4*>(Kb + (size_t)tok * kD + g * Tr::EPP);
        xr = *reinterpret_cast<const uint4*>(Xb + (size_t)tok * kD + g * Tr::EPP);
      }
      unpack16(kr, kv, Tr{});
      unpack16(xr, xv, Tr{});
#pragma unroll
      for (int e = 0; e < Tr::EPP; ++e) kv[e] = fmaxf(kv[e], 0.f);
      if (!kM) {
#pragma unroll
        for (int e = 0; e < Tr::EPP; ++e) sacc[e] += kv[e];
      } else {
        // r = 1 / (phi(Q) . s + eps): the PPT pieces of a token sit in PPT
        // consecutive lanes.
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < Tr::EPP; ++e) {
          xv[e] = fmaxf(xv[e], 0.f);
          part += xv[e] * s_sh[g * Tr::EPP + e];
        }
#pragma unroll
        for (int off = 1; off < PPT; off <<= 1) part += __shfl_xor(part, off);
        const float r = 1.f / (part + a.eps);
#pragma unroll
        for (int e = 0; e < Tr::EPP; ++e) xv[e] *= r;
      }
      lds_store16(tk + tt * kCellStride + g * Tr::EPP, pack16(kv, Tr{}));
      lds_store16(tx + tt * kCellStride + g * Tr::EPP, pack16(xv, Tr{}));
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kStatTile; kk += 16) {
#pragma unroll
      for (int q = 0; q < 8 / Tr::EPL; ++q) {
        const int row0 = kk + 8 * h + q * Tr::EPL;
        auto av = gather(tk, row0, 32 * mb + m, Tr{});
        auto bv = gather(tx, row0, 32 * nb + m, Tr{});
        acc = mma(av, bv, acc);
      }
    }
    __syncthreads();
  }

  // Partial of this chunk.
  float* part = a.part + ((size_t)bh * a.P + p) * (kD * kD);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3);
    part[row * kD + 32 * nb + m] = acc[i];
  }
  if (!kM) {
#pragma unroll
    for (int e = 0; e < Tr::EPP; ++e) s_red[tid][e] = sacc[e];
    __syncthreads();
    if (tid < kD) {
      const int gg = tid / Tr::EPP, e = tid % Tr::EPP;
      float t = 0.f;
      for (int u = gg; u < kThreads; u += PPT) t += s_red[u][e];
      a.part_s[((size_t)bh * a.P + p) * kD + tid] = t;
    }
  }

  // Last-arrival combine, fixed summation order.
  __threadfence();
  __syncthreads();
  const int grp = p / kGroup;
  unsigned* cnt = a.cnt + (size_t)bh * kCntWords;
  if (tid == 0) {
    const int gsize = min(kGroup, a.P - grp * kGroup);
    const unsigned old = atomicAdd(&cnt[grp], 1u);
    last = (old == (unsigned)(gsize - 1));
  }
  __syncthreads();
  if (!last) return;
  __threadfence();

  float v[16];
  float sv = 0.f;
  {
    const int p0 = grp * kGroup, p1 = min(a.P, p0 + kGroup);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = 0.f;
    for (int pp = p0; pp < p1; ++pp) {
      const float4* src = reinterpret_cast<const float4*>(a.part + ((size_t)bh * a.P + pp) * (kD * kD)) + tid * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 x = src[j];
        v[4 * j] += x.x;
        v[4 * j + 1] += x.y;
        v[4 * j + 2] += x.z;
        v[4 * j + 3] += x.w;
      }
      if (!kM && tid < kD) sv += a.part_s[((size_t)bh * a.P + pp) * kD + tid];
    }
  }
  if (tid == 0) cnt[grp] = 0u;

  if (a.ngroups > 1) {
    float4* dst = reinterpret_cast<float4*>(a.gpart + ((size_t)bh * a.ngroups + grp) * (kD * kD)) + tid * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    if (!kM && tid < kD) a.gpart_s[((size_t)bh * a.ngroups + grp) * kD + tid] = sv;
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned old = atomicAdd(&cnt[kMaxGroups], 1u);
      last = (old == (unsigned)(a.ngroups - 1));
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = 0.f;
    sv = 0.f;
    for (int gg = 0; gg < a.ngroups; ++gg) {
      const float4* src = reinterpret_cast<const float4*>(a.gpart + ((size_t)bh * a.ngroups + gg) * (kD * kD)) + tid * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 x = src[j];
        v[4 * j] += x.x;
        v[4 * j + 1] += x.y;
        v[4 * j + 2] += x.z;
        v[4 * j + 3] += x.w;
      }
      if (!kM && tid < kD) sv += a.gpart_s[((size_t)bh * a.ngroups + gg) * kD + tid];
    }
    if (tid == 0) cnt[kMaxGroups] = 0u;
  }

  // Final statistics: fp32 matrix, fp32 s, and MFMA fragments.
  float4* fin = reinterpret_cast<float4*>(a.fin + (size_t)bh * (kD * kD)) + tid * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 x = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    fin[j] = x;
    reinterpret_cast<float4*>(red)[tid * 4 + j] = x;
  }
  if (!kM && tid < kD) a.fin_s[(size_t)bh * kD + tid] = sv;
  __syncthreads();
  write_fragments<Tr>(red, static_cast<S*>(a.frag) + (size_t)bh * (kD * kD));
}

// ---------------------------------------------------------------------------
// Output kernel.  grid = (tiles, batch*heads), 4 waves.  A tile is TR x TC
// grid cells; K and V of the tile plus a one-cell halo are staged in LDS
// (cells off the grid are zero).  Each wave takes 32 tokens at a time, one
// token per lane pair (lane m and m + 32 hold 32 of the 64 features each,
// in accumulator layout), so the global branch's matrix products run on
// MFMA with no data movement between them.
// ---------------------------------------------------------------------------
template <class Tr>
__global__ __launch_bounds__(kThreads) void output_kernel(OutArgs a) {
  using S = typename Tr::S;
  using Frag = typename Tr::Frag;
  constexpr int PPT = kD / Tr::EPP;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int bh = blockIdx.y;
  const int tile = blockIdx.x;
  const int r0 = (tile / a.tiles_x) * a.TR;
  const int c0 = (tile % a.tiles_x) * a.TC;
  const int CW = a.TC + 2;
  const int ncell = (a.TR + 2) * CW;
  S* cK = reinterpret_cast<S*>(smem);
  S* cV = cK + (size_t)ncell * kCellStride;

  const size_t base = (size_t)bh * a.n * kD;
  const S* Qb = static_cast<const S*>(a.Q) + base;
  const S* Kb = static_cast<const S*>(a.K) + base;
  const S* Vb = static_cast<const S*>(a.V) + base;
  S* Yb = static_cast<S*>(a.Y) + base;

  // Stage K and V cells (tile plus halo).
  for (int pc = tid; pc < ncell * PPT; pc += kThreads) {
    const int cell = pc / PPT, g = pc % PPT;
    const int row = r0 - 1 + cell / CW;
    const int col = c0 - 1 + cell % CW;
    uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
    if (row >= 0 && row < a.H && col >= 0 && col < a.W) {
      const size_t off = (size_t)(row * a.W + col) * kD + g * Tr::EPP;
      kr = *reinterpret_cast<const uint4*>(Kb + off);
      vr = *reinterpret_cast<const uint4*>(Vb + off);
    }
    lds_store16(cK + cell * kCellStride + g * Tr::EPP, kr);
    lds_store16(cV + cell * kCellStride + g * Tr::EPP, vr);
  }

  // Per-(batch, head) statistics in registers.
  const bool global = a.T >= 2;
  float s_l[32];
  Frag fkv[2][Tr::NQ], fm[2][Tr::NQ];
  if (global) {
#pragma unroll
    for (int c = 0; c < 8; ++c) load4(a.s + (size_t)bh * kD + dimof(4 * c, h), &s_l[4 * c]);
    const Frag* gkv = reinterpret_cast<const Frag*>(static_cast<const S*>(a.frag_kv) + (size_t)bh * (kD * kD));
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < Tr::NQ; ++q) fkv[mb][q] = gkv[(mb * Tr::NQ + q) * 64 + lane];
    if (a.T >= 3) {
      const Frag* gm = reinterpret_cast<const Frag*>(static_cast<const S*>(a.frag_m) + (size_t)bh * (kD * kD));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int q = 0; q < Tr::NQ; ++q) fm[mb][q] = gm[(mb * Tr::NQ + q) * 64 + lane];
    }
  }
  const float alpha = a.alpha[bh % a.heads];
  __syncthreads();

  const int ntok = a.TR * a.TC;
  for (int t0 = 32 * wave; t0 < ntok; t0 += 32 * (kThreads / 64)) {
    const int t = t0 + m;
    int tr = t / a.TC, tc = t % a.TC;
    const int row = r0 + tr, col = c0 + tc;
    const bool valid = (t < ntok) && (row < a.H) && (col < a.W);
    if (!valid) tr = tc = 0;  // any staged cell; results are discarded
    const int i = valid ? row * a.W + col : 0;

    float q[32];
#pragma unroll
    for (int c = 0; c < 8; ++c) load4(Qb + (size_t)i * kD + dimof(4 * c, h), &q[4 * c]);
    float w[kMaxT];
    if (a.weights) {
      const float* wp = a.weights + ((size_t)bh * a.n + i) * a.T;
#pragma unroll
      for (int k = 0; k < kMaxT; ++k) w[k] = (k < a.T) ? wp[k] : 0.f;
    } else {
#pragma unroll
      for (int k = 0; k < kMaxT; ++k) w[k] = a.geo[k];
    }
    const int ccell = (tr + 1) * CW + (tc + 1);

    // Global branch.
    float G[32];
    {
      float vc[32];
#pragma unroll
      for (int c = 0; c < 8; ++c) load4(cV + ccell * kCellStride + dimof(4 * c, h), &vc[4 * c]);
#pragma unroll
      for (int v = 0; v < 32; ++v) G[v] = w[0] * vc[v];
    }
    if (global) {
      float u[32], z[32], y[32];
      float part = 0.f;
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        u[v] = fmaxf(q[v], 0.f);
        part += u[v] * s_l[v];
        z[v] = w[1] * u[v];
      }
      part += __shfl_xor(part, 32);
      const float r = 1.f / (part + a.eps);
      for (int k = 2; k < a.T; ++k) {
        apply<Tr>(fm, u, y);
#pragma unroll
        for (int v = 0; v < 32; ++v) {
          u[v] = y[v];
          z[v] += w[k] * y[v];
        }
      }
      apply<Tr>(fkv, z, y);
#pragma unroll
      for (int v = 0; v < 32; ++v) G[v] += r * y[v];
    }

    // Local branch: 3x3 window, masked, row max subtracted.
    float lg[9];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const int dr = j / 3 - 1, dc = j % 3 - 1;
      const int cell = ccell + dr * CW + dc;
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float kx[4];
        load4(cK + cell * kCellStride + dimof(4 * c, h), kx);
#pragma unroll
        for (int e = 0; e < 4; ++e) part += q[4 * c + e] * kx[e];
      }
      part += __shfl_xor(part, 32);
      const bool in = (row + dr >= 0) && (row + dr < a.H) && (col + dc >= 0) && (col + dc < a.W);
      lg[j] = in ? part * a.logit_scale : -INFINITY;
      mx = fmaxf(mx, lg[j]);
    }
    float L[32];
#pragma unroll
    for (int v = 0; v < 32; ++v) L[v] = 0.f;
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const int dr = j / 3 - 1, dc = j % 3 - 1;
      const int cell = ccell + dr * CW + dc;
      const float pj = (lg[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(lg[j] - mx);
      den += pj;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float vx[4];
        load4(cV + cell * kCellStride + dimof(4 * c, h), vx);
#pragma unroll
        for (int e = 0; e < 4; ++e) L[4 * c + e] += pj * vx[e];
      }
    }
    const float inv = 1.f / den;

    if (valid) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = alpha * G[4 * c + e] + (1.f - alpha) * (L[4 * c + e] * inv);
        store4(Yb + (size_t)i * kD + dimof(4 * c, h), o);
      }
    }
  }
}

}  // namespace

hipError_t launch_stats_kv(int dtype, const StatsArgs& a, int BH, hipStream_t s) {
  dim3 grid(a.P, BH);
  if (dtype == 1)
    hipLaunchKernelGGL((stats_kernel<BF16, false>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((stats_kernel<F32, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stats_m(int dtype, const StatsArgs& a, int BH, hipStream_t s) {
  dim3 grid(a.P, BH);
  if (dtype == 1)
    hipLaunchKernelGGL((stats_kernel<BF16, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((stats_kernel<F32, true>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_output(int dtype, const OutArgs& a, int BH, int ntiles, size_t lds_bytes,
                         hipStream_t s) {
  dim3 grid(ntiles, BH);
  if (dtype == 1)
    hipLaunchKernelGGL(output_kernel<BF16>, grid, dim3(kThreads), lds_bytes, s, a);
  else
    hipLaunchKernelGGL(output_kernel<F32>, grid, dim3(kThreads), lds_bytes, s, a);
  return hipGetLastError();
}

}  // namespace lisa
