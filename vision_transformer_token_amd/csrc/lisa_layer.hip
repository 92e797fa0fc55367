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
// addressing, so neither is a pass of its own.  The QKV projection of a
// one-head bf16 layer streams (proj_stream_qkv, below); otherwise a
// workgroup computes a
// 64 x 64 block of outputs, wave w its rows 16 w .. 16 w + 15 as four 16 x 16
// MFMA blocks; both operands are read straight from HBM / L2 with 16-byte
// loads (rows of X, of a head's O and of the torch-layout weights [out][in]
// are contiguous along the contraction).  The 64 outputs of a row in a block
// are contiguous in the output too (one head's channels of Q, K or V, or a
// stretch of a row of Y): each wave turns its accumulators into rows through
// LDS and writes them with 16-byte stores.  A workgroup takes four 64-row
// blocks of one column block, so each weight operand it reads serves four
// MFMAs and four blocks' input loads are in flight together.  The device
// hands workgroup w to XCD w % 8, and each XCD has its own L2: the
// workgroups that share input rows (the QKV projection's column blocks) are
// the consecutive workgroups of one XCD, so the input is read from HBM about
// once and from that L2 by the others.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lisa_device.hpp"
#include "lisa_kernels.hpp"
#include "lisa_layer.hpp"

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

template <class S, bool kOut>
__global__ __launch_bounds__(256) void proj_gemm(ProjArgs a) {
  __shared__ __align__(16) float rows[4][16 * kRowPad];
  const int t = threadIdx.x, w = t / 64, ln = t % 64, li = ln % 16, lk = ln / 16;
  int rb, cb;
  proj_block(a.M, a.N, (int)blockIdx.x, rb, cb);
  if (rb < 0) return;  // no barrier in this kernel
  const int c0 = cb * 64;
  const int mb = rb * (64 * kProjTiles) + 16 * w;  // wave's rows in tile r: mb + 64 r + 0..15
  const S* A = static_cast<const S*>(a.A);
  const S* Wt = static_cast<const S*>(a.Wt);
  f32x4 acc[kProjTiles][4] = {};
  if constexpr (sizeof(S) == 2) {
    // bf16 MFMA 16x16x32: lane (li, lk) holds contraction slots k0 + 8 lk .. + 7.
    // K is a multiple of 64 (whole heads): both halves' loads are issued
    // before their products.
    for (int k0 = 0; k0 < a.K; k0 += 64) {
      bf16x8 bv[2][4], av[2][kProjTiles];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = k0 + 32 * h + 8 * lk;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          bv[h][ct] = *reinterpret_cast<const bf16x8*>(Wt + (size_t)(c0 + 16 * ct + li) * a.K + k);
#pragma unroll
        for (int r = 0; r < kProjTiles; ++r) {
          const int mr = mb + 64 * r + li;
          av[h][r] = bf16x8{};
          if (mr < a.M) av[h][r] = *reinterpret_cast<const bf16x8*>(A + a_index<kOut>(a, mr, k));
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < kProjTiles; ++r)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            acc[r][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[h][r], bv[h][ct], acc[r][ct], 0, 0, 0);
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
  // bias, into the wave's 16 LDS rows.  The wave's 16 output rows of 64
  // elements are contiguous in the output (16 tokens of one head, or 16 rows
  // of Y when it is 64 wide) or at least whole 64-element rows: each store
  // instruction writes 1 KB of them, lane ln the 16 bytes at 16 ln, so that
  // every cache line a store touches is written whole by it.  The wave's LDS
  // accesses complete in order, so tile r + 1's writes follow tile r's reads.
  float* rw = rows[w];
  float bc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) bc[ct] = a.bias[c0 + 16 * ct + li];
  constexpr int kEl = 16 / (int)sizeof(S);  // elements per 16-byte piece
  constexpr int kSt = 16 * 64 / (64 * kEl);  // store instructions per tile
#pragma unroll
  for (int r = 0; r < kProjTiles; ++r) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) rw[(4 * lk + e) * kRowPad + 16 * ct + li] = acc[r][ct][e] + bc[ct];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    // Store j: piece 64 j + ln of the 16 x 64 block, row (64 j + ln) / (64 / kEl).
    float v[kSt][kEl];
#pragma unroll
    for (int j = 0; j < kSt; ++j) {
      const int row = (64 * j + ln) / (64 / kEl), col = (ln % (64 / kEl)) * kEl;
#pragma unroll
      for (int h = 0; h < kEl; h += 4) {
        const float4 x = *reinterpret_cast<const float4*>(rw + row * kRowPad + col + h);
        v[j][h] = x.x;
        v[j][h + 1] = x.y;
        v[j][h + 2] = x.z;
        v[j][h + 3] = x.w;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the next tile's writes
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < kSt; ++j) {
      const int row = (64 * j + ln) / (64 / kEl), col = (ln % (64 / kEl)) * kEl;
      const int m = mb + 64 * r + row;
      if (m >= a.M) continue;
      S* dst = static_cast<S*>(a.out) + out_index<kOut>(a, m, c0 + col);
      // Streaming stores (nontemporal): the outputs are not read again by
      // this kernel.
      if constexpr (sizeof(S) == 2) {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(v[j][2 * e], v[j][2 * e + 1]);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst));
      } else {
        __builtin_nontemporal_store(f32x4{v[j][0], v[j][1], v[j][2], v[j][3]}, reinterpret_cast<f32x4*>(dst));
      }
    }
  }
}

// The QKV projection in bf16 with K = 64 (one head's channels in, as in a
// one-head stage): the whole contraction of a row is one 16-byte operand per
// lane and MFMA step, so a workgroup can stream.  A fixed grid of workgroups
// walks the 64 x 64 output blocks (proj_unit); a workgroup keeps one column
// block, loads its weights and bias once, and each wave loads the next
// block's 16 input rows before it works on the current one.
__global__ __launch_bounds__(256) void proj_stream_qkv(ProjArgs a) {
  __shared__ __align__(16) float rows[4][16 * kRowPad];
  const int t = threadIdx.x, w = t / 64, ln = t % 64, li = ln % 16, lk = ln / 16;
  const int nrt = (a.M + 63) / 64, U = proj_units(a.M, a.N);
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* Wt = static_cast<const uint16_t*>(a.Wt);
  const int u0 = (int)blockIdx.x;
  int rt0, cb;
  proj_unit(a.N, u0, rt0, cb);  // every unit of this workgroup has column block cb
  const int c0 = cb * 64;
  auto tile_of = [&](int u) {
    int rt, cbu;
    proj_unit(a.N, u, rt, cbu);
    return rt;
  };
  bf16x8 bv[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      bv[h][ct] = *reinterpret_cast<const bf16x8*>(Wt + (size_t)(c0 + 16 * ct + li) * 64 + 32 * h + 8 * lk);
  float bc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) bc[ct] = a.bias[c0 + 16 * ct + li];
  // The wave's operand rows of unit u (zero past the last row).
  auto load_rows = [&](int u, bf16x8 (&av)[2]) {
    const int mr = tile_of(u) * 64 + 16 * w + li;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      av[h] = bf16x8{};
      if (u < U && mr < a.M) av[h] = *reinterpret_cast<const bf16x8*>(A + a_index<false>(a, mr, 32 * h + 8 * lk));
    }
  };
  bf16x8 nxt[2];
  load_rows(u0, nxt);
  float* rw = rows[w];
  for (int u = u0; u < U; u += (int)gridDim.x) {
    bf16x8 av[2] = {nxt[0], nxt[1]};
    load_rows(u + (int)gridDim.x, nxt);
    const int rt = tile_of(u);
    if (rt >= nrt) continue;  // a padding unit (wave-uniform)
    f32x4 acc[4] = {};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[h], bv[h][ct], acc[ct], 0, 0, 0);
    // Into the wave's 16 LDS rows, then 1 KB per store instruction (lane ln
    // the 16 bytes at 16 ln of the 16 contiguous rows of 64 outputs).
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) rw[(4 * lk + e) * kRowPad + 16 * ct + li] = acc[ct][e] + bc[ct];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    u32x4 o[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 8 * j + ln / 8, col = 8 * (ln % 8);
      const float4 x0 = *reinterpret_cast<const float4*>(rw + row * kRowPad + col);
      const float4 x1 = *reinterpret_cast<const float4*>(rw + row * kRowPad + col + 4);
      o[j][0] = pack_bf16x2(x0.x, x0.y);
      o[j][1] = pack_bf16x2(x0.z, x0.w);
      o[j][2] = pack_bf16x2(x1.x, x1.y);
      o[j][3] = pack_bf16x2(x1.z, x1.w);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the next unit's writes
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = rt * 64 + 16 * w + 8 * j + ln / 8;
      if (m >= a.M) continue;
      __builtin_nontemporal_store(
          o[j], reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + out_index<false>(a, m, c0 + 8 * (ln % 8))));
    }
  }
}

template <class S>
hipError_t launch_proj_typed(bool out_proj, const ProjArgs& a, hipStream_t s) {
  // The streaming kernel pays for the QKV projection (PVT-T stage 1, 64
  // channels: 17.7 -> 15.5 us with 1024 workgroups; 256 / 512 / 768 / 1536 /
  // 2048 of them: 23.9 / 17.5 / 15.8 / 17.2 / 20.1 us); the output projection
  // takes about as long either way (8.0 -> 8.0 us at 768 workgroups, 8.8 at
  // 1024) and keeps the blocked kernel.
  if (sizeof(S) == 2 && a.K == 64 && !out_proj) {
    hipLaunchKernelGGL(proj_stream_qkv, dim3(proj_stream_grid(a.M, a.N)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid(proj_grid(a.M, a.N));
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
