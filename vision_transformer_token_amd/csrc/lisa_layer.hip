// The projections of a LiSA attention layer on gfx950: [Q | K | V] =
// X Wqkv^T + bqkv split into heads, and Y = concat_h(O_h) Wo^T + bo, with
// the operator (lisa_flow.hip) in between.
//
// Source: the reading note of "LiSA: Linear Stochastic Attention for
// Long-Range Visual Modeling" (arXiv:2611.04216v2) §2.1: n tokens X are
// projected to Q, K and V; the operator is a plug-in replacing the attention
// of DeiT-T and PVT-T.  The layer around it is the usual ViT attention block
// (one QKV projection with bias, heads of 64 channels in order, an output
// projection with bias).
//
// Both projections are contractions over the channels on MFMA with fp32
// sums; the head split (QKV) and merge (output) are folded into the
// addressing, so neither is a pass of its own.  A workgroup computes a
// 64 x 64 block of outputs, wave w its rows 16 w .. 16 w + 15 as four 16 x 16
// MFMA blocks; both operands are read straight from HBM / L2 with 16-byte
// loads (rows of X, of a head's O and of the torch-layout weights [out][in]
// are contiguous along the contraction).  The 64 outputs of a row in a block
// are contiguous in the output too (one head's channels of Q, K or V, or a
// stretch of a row of Y): each wave turns its accumulators into rows through
// LDS and writes them with 16-byte stores.  A workgroup takes four 64-row
// blocks of one column block, so each weight operand it reads serves four
// MFMAs and four blocks' input loads are in flight together; workgroups that
// share input rows are consecutive (the column block varies fastest), so the
// input is read from HBM about once and from L2 by the others.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lisa_device.hpp"
#include "lisa_kernels.hpp"

namespace lisa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// A[m][k]: QKV, X [M][C] row-major; output projection, O [B][heads][n][64].
template <bool kOut>
__device__ __forceinline__ size_t a_index(const ProjArgs& a, int m, int k) {
  if constexpr (!kOut) return (size_t)m * a.K + k;
  const int b = m / a.n, tok = m % a.n, h = k / kD, d = k % kD;
  return (((size_t)b * a.heads + h) * a.n + tok) * kD + d;
}
// Output (m, c): QKV, channel c of [Q | K | V] into its head-major tensor;
// output projection, Y [M][C] row-major.
template <bool kOut>
__device__ __forceinline__ size_t out_index(const ProjArgs& a, int m, int c) {
  if constexpr (kOut) return (size_t)m * a.N + c;
  const int which = c / a.K, cc = c % a.K, h = cc / kD, d = cc % kD;
  const int b = m / a.n, tok = m % a.n;
  return (size_t)which * a.head_elems + (((size_t)b * a.heads + h) * a.n + tok) * kD + d;
}

constexpr int kRowPad = 68;  // floats per LDS row: four lane groups 272 floats apart, on distinct banks
constexpr int kProjTiles = 4;  // 64-row tiles per workgroup: each weight operand read serves four

template <class S, bool kOut>
__global__ __launch_bounds__(256) void proj_gemm(ProjArgs a) {
  __shared__ __align__(16) float rows[4][16 * kRowPad];
  const int t = threadIdx.x, w = t / 64, ln = t % 64, li = ln % 16, lk = ln / 16;
  const int nct = a.N / 64;
  const int c0 = (int)(blockIdx.x % nct) * 64;
  const int mb = (int)(blockIdx.x / nct) * (64 * kProjTiles) + 16 * w;  // wave's rows in tile r: mb + 64 r + 0..15
  const S* A = static_cast<const S*>(a.A);
  const S* Wt = static_cast<const S*>(a.Wt);
  f32x4 acc[kProjTiles][4] = {};
  if constexpr (sizeof(S) == 2) {
    // bf16 MFMA 16x16x32: lane (li, lk) holds contraction slots k0 + 8 lk .. + 7.
    for (int k0 = 0; k0 < a.K; k0 += 32) {
      const int k = k0 + 8 * lk;
      bf16x8 bv[4], av[kProjTiles];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) bv[ct] = *reinterpret_cast<const bf16x8*>(Wt + (size_t)(c0 + 16 * ct + li) * a.K + k);
#pragma unroll
      for (int r = 0; r < kProjTiles; ++r) {
        const int mr = mb + 64 * r + li;
        av[r] = bf16x8{};
        if (mr < a.M) av[r] = *reinterpret_cast<const bf16x8*>(A + a_index<kOut>(a, mr, k));
      }
#pragma unroll
      for (int r = 0; r < kProjTiles; ++r)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          acc[r][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[r], bv[ct], acc[r][ct], 0, 0, 0);
    }
  } else {
    // fp32 MFMA 16x16x4: four of them per 16 inputs, lane (li, lk) taking
    // inputs k0 + 4 lk + s in the s-th (one 16-byte read each).
    for (int k0 = 0; k0 < a.K; k0 += 16) {
      const int k = k0 + 4 * lk;
      float4 bv[4], av[kProjTiles];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) bv[ct] = *reinterpret_cast<const float4*>(Wt + (size_t)(c0 + 16 * ct + li) * a.K + k);
#pragma unroll
      for (int r = 0; r < kProjTiles; ++r) {
        const int mr = mb + 64 * r + li;
        av[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (mr < a.M) av[r] = *reinterpret_cast<const float4*>(A + a_index<kOut>(a, mr, k));
      }
#pragma unroll
      for (int r = 0; r < kProjTiles; ++r)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          acc[r][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r].x, bv[ct].x, acc[r][ct], 0, 0, 0);
          acc[r][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r].y, bv[ct].y, acc[r][ct], 0, 0, 0);
          acc[r][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r].z, bv[ct].z, acc[r][ct], 0, 0, 0);
          acc[r][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r].w, bv[ct].w, acc[r][ct], 0, 0, 0);
        }
    }
  }
  // acc[r][ct][e] is output (mb + 64 r + 4 lk + e, c0 + 16 ct + li): plus the
  // bias, into the wave's 16 LDS rows; then lane ln writes columns
  // 16 (ln % 4) .. + 15 of row mb + 64 r + ln / 4.  The wave's LDS accesses
  // complete in order, so tile r + 1's writes follow tile r's reads.
  float* rw = rows[w];
  float bc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) bc[ct] = a.bias[c0 + 16 * ct + li];
  const int rr = ln / 4, q = ln % 4;
#pragma unroll
  for (int r = 0; r < kProjTiles; ++r) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) rw[(4 * lk + e) * kRowPad + 16 * ct + li] = acc[r][ct][e] + bc[ct];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 x = *reinterpret_cast<const float4*>(rw + rr * kRowPad + 16 * q + 4 * j);
      v[4 * j] = x.x;
      v[4 * j + 1] = x.y;
      v[4 * j + 2] = x.z;
      v[4 * j + 3] = x.w;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the next tile's writes
    __builtin_amdgcn_wave_barrier();
    const int m = mb + 64 * r + rr;
    if (m < a.M) {
      S* dst = static_cast<S*>(a.out) + out_index<kOut>(a, m, c0 + 16 * q);
      if constexpr (sizeof(S) == 2) {
        u32x4 o0, o1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o0[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
          o1[e] = pack_bf16x2(v[8 + 2 * e], v[8 + 2 * e + 1]);
        }
        // Streaming stores (nontemporal): the outputs are not read again by
        // this kernel (QKV 20.0 -> ~17 us at PVT-T stage 1).
        __builtin_nontemporal_store(o0, reinterpret_cast<u32x4*>(dst));
        __builtin_nontemporal_store(o1, reinterpret_cast<u32x4*>(dst) + 1);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __builtin_nontemporal_store(f32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]},
                                      reinterpret_cast<f32x4*>(dst) + j);
      }
    }
  }
}

template <class S>
hipError_t launch_proj_typed(bool out_proj, const ProjArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.M + 64 * kProjTiles - 1) / (64 * kProjTiles)) * (unsigned)(a.N / 64));
  if (out_proj)
    hipLaunchKernelGGL((proj_gemm<S, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((proj_gemm<S, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj(int dtype, bool out_proj, const ProjArgs& a, hipStream_t s) {
  return dtype == 1 ? launch_proj_typed<uint16_t>(out_proj, a, s) : launch_proj_typed<float>(out_proj, a, s);
}

}  // namespace lisa
