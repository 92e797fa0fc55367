// The LiSA forward pass on gfx950 as one persistent, dependency-driven kernel.
//
// Method: reading note "LiSA:面向长程视觉建模的线性随机注意力" (arXiv:2611.04216v2),
// §2.1-§2.4.  Per (batch, head) slice with n tokens of width 64:
//   statistics (Eq. 8): s = sum_j phi(K_j), phi(K)^T V, M = phi(K)^T Qt with
//     Qt_j = r_j phi(Q_j), r_j = 1 / (phi(Q_j) . s + eps), phi = ReLU;
//   global branch: G_i = w_0(i) V_i + r_i sum_{k=1}^{T-1} w_k(i) (phi(Q_i) M^(k-1)) (phi(K)^T V),
//     which is row i of sum_k diag(w_k) S^k V with S = Qt phi(K)^T;
//   local branch: L_i = softmax over the clipped 3x3 window of q_i . k_j / sqrt(d_h), times V;
//   Y_i = alpha G_i + (1 - alpha) L_i.
//
// Work is split into items (see FlowArgs): KV and M items sweep token chunks
// and contract over tokens on MFMA; C items sum the chunk partials in a fixed
// order and write the statistics as MFMA fragments; OUT items produce one
// spatial tile of Y.  Each workgroup takes items from its XCD's queue (an
// atomic ticket), waits for the items an item depends on through per-slice
// arrival counters, and stages the next item's inputs into the other of two
// LDS buffers with global_load_lds while it computes the current one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lisa_device.hpp"
#include "lisa_kernels.hpp"

namespace lisa {
namespace {

enum Kind { kKV = 0, kM = 1, kC = 2, kOut = 3, kNone = 4 };
struct Item {
  int kind, b, idx;
};

__device__ __forceinline__ int queue_slices(const FlowArgs& a, int x) {
  return a.nq == 1 ? a.BH : (a.BH - x + a.nq - 1) / a.nq;
}
__device__ __forceinline__ int queue_items(const FlowArgs& a, int x) {
  return queue_slices(a, x) * (a.nKV + a.nM + a.nC + a.nOUT);
}
// Queue order: all KV items of the queue's slices (slice-major), then all M,
// then all C, then all OUT items.  An item only waits for items earlier in
// this order, which the workgroups have already taken.
__device__ __forceinline__ Item decode(const FlowArgs& a, int x, int t) {
  const int ns = queue_slices(a, x);
  const int per[4] = {a.nKV, a.nM, a.nC, a.nOUT};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int cnt = ns * per[k];
    if (t < cnt) {
      const int j = t / per[k];
      return Item{k, a.nq == 1 ? j : x + a.nq * j, t % per[k]};
    }
    t -= cnt;
  }
  return Item{kNone, 0, 0};
}

// Thread 0 only: spin until *c >= target.  The wait is bounded (about a
// second); on giving up it raises the error word, after which every later
// wait of the launch returns at once, so the launch always finishes.
__device__ void wait_for(const unsigned* c, unsigned target, unsigned* err) {
  unsigned spins = 0;
  while (get(c) < target) {
    __builtin_amdgcn_s_sleep(2);
    if ((++spins & 255u) == 0 && get(err)) break;
    if (spins > (1u << 21)) {
      put(err, 1u);
      break;
    }
  }
}

__device__ __forceinline__ void tile_origin(const FlowArgs& a, int t, int& r0, int& c0) {
  r0 = (t / a.tiles_x) * a.TR;
  c0 = (t % a.tiles_x) * a.TC;
}

// Issue the DMA of an item's inputs into `buf` (nothing for C items).
template <class Tr>
__device__ void stage(const FlowArgs& a, Item it, unsigned char* buf) {
  using S = typename Tr::S;
  if (it.kind == kKV || it.kind == kM) {
    const int tok0 = it.idx * a.chunk;
    const int nv = min(a.chunk, a.n - tok0);
    const S* Kb = static_cast<const S*>(a.K) + ((size_t)it.b * a.n + tok0) * kD;
    const S* Xb = static_cast<const S*>(it.kind == kKV ? a.V : a.Q) + ((size_t)it.b * a.n + tok0) * kD;
    dma_rows<Tr>(buf, nv, [&](int r) { return static_cast<const void*>(Kb + (size_t)r * kD); });
    dma_rows<Tr>(buf + kBufBytes / 2, nv, [&](int r) { return static_cast<const void*>(Xb + (size_t)r * kD); });
  } else if (it.kind == kOut) {
    int r0, c0;
    tile_origin(a, it.idx, r0, c0);
    const int CW = a.TC + 2, ncell = (a.TR + 2) * CW;
    const S* Kb = static_cast<const S*>(a.K) + (size_t)it.b * a.n * kD;
    const S* Vb = static_cast<const S*>(a.V) + (size_t)it.b * a.n * kD;
    // Cells off the grid fetch token 0 of the slice; they are never used.
    auto tok = [&](int r) -> size_t {
      const int row = r0 - 1 + r / CW, col = c0 - 1 + r % CW;
      return (row >= 0 && row < a.H && col >= 0 && col < a.W) ? (size_t)(row * a.W + col) : 0;
    };
    dma_rows<Tr>(buf, ncell, [&](int r) { return static_cast<const void*>(Kb + tok(r) * kD); });
    dma_rows<Tr>(buf + kBufBytes / 2, ncell, [&](int r) { return static_cast<const void*>(Vb + tok(r) * kD); });
  }
}

// Element d of staged fp32 row r.
__device__ __forceinline__ float lds_elem(const unsigned char* base, int r, int d, F32) {
  return *reinterpret_cast<const float*>(base + row_off<F32>(r, d));
}

// ---------------------------------------------------------------------------
// KV / M items: contraction over the chunk's tokens.  Wave w owns block
// (w / 2, w % 2) of the 64x64 result; A = phi(K) rows, B = V rows (KV) or
// r_j phi(Q_j) rows rounded to the input dtype (M, rescaled in LDS first).
// KV items also form s with a second MFMA against a ones operand.  Rows past
// the chunk's last token are zeroed in LDS, so the sweep needs no masks.
// ---------------------------------------------------------------------------
template <class Tr, bool kIsM, class Prefetch>
__device__ void stats_item(const FlowArgs& a, Item it, unsigned char* buf, float* s_sh,
                           Prefetch prefetch) {
  using S = typename Tr::S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, h = lane >> 5, mb = wave >> 1, nb = wave & 1;
  const int tok0 = it.idx * a.chunk;
  const int nv = min(a.chunk, a.n - tok0);
  const int nvr = (nv + 15) & ~15;
  unsigned char* bK = buf;
  unsigned char* bX = buf + kBufBytes / 2;

  if (kIsM && tid < kD) {  // s = sum of the KV items' partials, fixed order
    float t = 0.f;
    for (int p = 0; p < a.nKV; ++p) t += get(a.part_s + ((size_t)it.b * a.P + p) * kD + tid);
    s_sh[tid] = t;
  }
  prefetch();
  if (kIsM || nv < nvr) {
    if (kIsM) __syncthreads();
    for (int t = tid; t < nvr; t += kThreads) {
      if (t >= nv) {
#pragma unroll
        for (int g = 0; g < Tr::PPR; ++g) {
          *reinterpret_cast<uint4*>(bK + t * Tr::RB + g * 16) = make_uint4(0, 0, 0, 0);
          *reinterpret_cast<uint4*>(bX + t * Tr::RB + g * 16) = make_uint4(0, 0, 0, 0);
        }
      } else if (kIsM) {
        // r_t = 1 / (phi(Q_t) . s + eps); the row becomes r_t phi(Q_t).
        float x[kD];
#pragma unroll
        for (int c = 0; c < kD / 4; ++c) load4(reinterpret_cast<const S*>(bX + row_off<Tr>(t, 4 * c)), &x[4 * c]);
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < kD; ++d) {
          x[d] = fmaxf(x[d], 0.f);
          dot += x[d] * s_sh[d];
        }
        const float r = 1.f / (dot + a.eps);
#pragma unroll
        for (int d = 0; d < kD; ++d) x[d] *= r;
#pragma unroll
        for (int c = 0; c < kD / 4; ++c) store4(reinterpret_cast<S*>(bX + row_off<Tr>(t, 4 * c)), &x[4 * c]);
      }
    }
    __syncthreads();
  }

  f32x16 acc = {}, acc_s = {};
  for (int kk = 0; kk < nvr; kk += 16) {
    if constexpr (Tr::EPL == 8) {
      const bf16x8 A = as_bf16(rows_bits<true>(bK, kk, 32 * mb));
      const bf16x8 B = as_bf16(rows_bits<false>(bX, kk, 32 * nb));
      acc = mma(A, B, acc);
      if (!kIsM && nb == 0) acc_s = mma(A, as_bf16((v8s)(short)0x3f80), acc_s);  // ones: bf16 1.0
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = kk + 8 * h + q;
        const float A = fmaxf(lds_elem(bK, r, 32 * mb + m, Tr{}), 0.f);
        const float B = lds_elem(bX, r, 32 * nb + m, Tr{});
        acc = mma(A, B, acc);
        if (!kIsM && nb == 0) acc_s = mma(A, 1.f, acc_s);
      }
    }
  }

  // Partials, shared through coherent stores.
  float* part = (kIsM ? a.part_m : a.part_kv) + ((size_t)it.b * a.P + it.idx) * (kD * kD);
#pragma unroll
  for (int i = 0; i < 16; ++i) put(part + (32 * mb + 8 * (i >> 2) + 4 * h + (i & 3)) * kD + 32 * nb + m, acc[i]);
  if (!kIsM && nb == 0 && m == 0) {
    float* ps = a.part_s + ((size_t)it.b * a.P + it.idx) * kD;
#pragma unroll
    for (int i = 0; i < 16; ++i) put(ps + 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3), acc_s[i]);
  }
  wait_all();
  __syncthreads();
  if (tid == 0) {
    unsigned* cnt = a.slice_cnt + (size_t)it.b * 4;
    const unsigned old = bump(&cnt[kIsM ? kM : kKV]);
    // The last M item of a slice: every M item has passed its wait on the
    // KV count, which can now be cleared for the next launch.
    if (kIsM && old == (unsigned)(a.nM - 1)) put(&cnt[kKV], 0u);
  }
}

// ---------------------------------------------------------------------------
// C items: fixed-order sum of the P partials of rows [16 rb, 16 rb + 16) of
// phi(K)^T V (q < 4) or M (q >= 4); fp32 result plus MFMA fragments, where
// fragment (mb, q', lane, e) holds X[dimof(q' EPL + e, lane / 32)][32 mb + lane % 32].
// ---------------------------------------------------------------------------
template <class Tr, class Prefetch>
__device__ void combine_item(const FlowArgs& a, Item it, Prefetch prefetch) {
  const int tid = threadIdx.x;
  const int mat = it.idx / kCombineBlocks, rb = it.idx % kCombineBlocks;
  const float* part = (mat == 0 ? a.part_kv : a.part_m) + (size_t)it.b * a.P * (kD * kD);
  const int col = tid & 63, rp = tid >> 6;
  int rows[4];
  rows[0] = 16 * rb + 2 * rp;
  rows[1] = rows[0] + 1;
  rows[2] = 16 * rb + 2 * (rp + 4);
  rows[3] = rows[2] + 1;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  float sv = 0.f;
  const bool do_s = (it.idx == 0) && tid < kD;
  for (int p0 = 0; p0 < a.P; p0 += 8) {
    float x[8][4];
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        x[bb][j] = (p0 + bb < a.P) ? get(part + (size_t)(p0 + bb) * (kD * kD) + rows[j] * kD + col) : 0.f;
    if (p0 == 0) {
      if (do_s)
        for (int p = 0; p < a.P; ++p) sv += get(a.part_s + ((size_t)it.b * a.P + p) * kD + tid);
      prefetch();
    }
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += x[bb][j];
  }
  float* fin = (mat == 0 ? a.fin_kv : a.fin_m) + (size_t)it.b * (kD * kD);
#pragma unroll
  for (int j = 0; j < 4; ++j) fin[rows[j] * kD + col] = v[j];
  if (do_s) put(a.fin_s + (size_t)it.b * kD + tid, sv);
  void* fragv = mat == 0 ? a.frag_kv : a.frag_m;
  const int mbo = col >> 5, mm = col & 31;
#pragma unroll
  for (int j = 0; j < 4; j += 2) {
    const int r = rows[j];  // even: r and r + 1 sit in adjacent fragment slots
    const int vs = 16 * (r >> 5) + 4 * ((r & 31) >> 3) + (r & 3);
    const int hh = (r & 7) >> 2;
    const int ln = mm + 32 * hh;
    if constexpr (Tr::EPL == 8) {
      const int f = ((mbo * Tr::NQ + (vs >> 3)) * 64 + ln) * 8 + (vs & 7);
      uint32_t* w = static_cast<uint32_t*>(fragv) + (size_t)it.b * (kD * kD / 2) + (f >> 1);
      put(w, (uint32_t)f2bf(v[j]) | ((uint32_t)f2bf(v[j + 1]) << 16));
    } else {
      float* fv = static_cast<float*>(fragv) + (size_t)it.b * (kD * kD);
      put(fv + (mbo * Tr::NQ + vs) * 64 + ln, v[j]);
      put(fv + (mbo * Tr::NQ + vs + 1) * 64 + ln, v[j + 1]);
    }
  }
  wait_all();
  __syncthreads();
  if (tid == 0) {
    unsigned* cnt = a.slice_cnt + (size_t)it.b * 4;
    const unsigned old = bump(&cnt[kC]);
    if (old == (unsigned)(a.nC - 1)) {
      // Every C item of the slice has passed its wait: clear that count.
      put(&cnt[a.nM ? kM : kKV], 0u);
      if (!(a.nOUT && a.wait_out)) put(&cnt[kC], 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// OUT items: one TR x TC tile of one slice.  Each wave takes 32 tokens at a
// time, one token per lane pair (lanes m and m + 32 hold 32 features each in
// accumulator layout), so the chain u_1 = phi(Q_i), u_k = u_(k-1) M and the
// projection z (phi(K)^T V), z = sum_k w_k(i) u_k, run on MFMA with no data
// movement.  The 3x3 local branch reads K and V cells (tile plus one-cell
// halo) from the staged LDS buffer.
// ---------------------------------------------------------------------------
template <class Tr>
__device__ __forceinline__ void load_frags(const void* frag, int b, typename Tr::Frag (&fr)[2][Tr::NQ]) {
  const int lane = threadIdx.x & 63;
  using S = typename Tr::S;
  const S* base = static_cast<const S*>(frag) + (size_t)b * (kD * kD);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int q = 0; q < Tr::NQ; ++q) {
      const S* p = base + ((mb * Tr::NQ + q) * 64 + lane) * Tr::EPL;
      if constexpr (Tr::EPL == 8) {
        const uint64_t lo = get64(p), hi = get64(p + 4);
        uint32_t w[4] = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
        fr[mb][q] = __builtin_bit_cast(bf16x8, w);
      } else {
        fr[mb][q] = get(reinterpret_cast<const float*>(p));
      }
    }
}

// Local branch of one 4x8 token block on MFMA (bf16).  The block's 3x3
// windows lie in a 6x10 window of staged cells (60, padded to 64).  Logits
// C[cell][token] = K_win Q_blk^T come out with one token per lane pair and the
// cells in accumulator order; after the masked softmax, those probabilities
// are already the B operand of L^T = V_win^T P^T (the contraction index
// permuted to match), whose A operand comes from transposed LDS reads, and L
// lands in the same accumulator layout as the global branch.
__device__ __forceinline__ void local_block_mfma(const FlowArgs& a, const unsigned char* cK,
                                                 const unsigned char* cV, int CW, int r0, int c0,
                                                 int br, int bc, const bf16x8 (&qB)[4], float (&L)[32]) {
  const int lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5;
  const int i16 = lane & 15, g = lane >> 4;
  auto wcell = [&](int c) {
    c = min(c, 59);
    return (4 * br + c / 10) * CW + 8 * bc + c % 10;
  };
  // Logits: A = K rows of window cells (16-byte pieces), B = this token's queries.
  f32x16 lg[2] = {};
  const int sc0 = wcell(n), sc1 = wcell(32 + n);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(cK + row_off<BF16>(sc0, 16 * kb + 8 * h));
    const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(cK + row_off<BF16>(sc1, 16 * kb + 8 * h));
    lg[0] = mma(A0, qB[kb], lg[0]);
    lg[1] = mma(A1, qB[kb], lg[1]);
  }
  // Mask: window cell (wr, wc) is a neighbour of token (ta, tb) iff
  // wr - ta and wc - tb lie in {0, 1, 2}; and it must lie on the grid.
  const int ta = n >> 3, tb = n & 7;
  unsigned rowbits = 0, colbits = 0;
#pragma unroll
  for (int wr = 0; wr < 6; ++wr) {
    const int gr = r0 + 4 * br + wr - 1;
    rowbits |= (unsigned)(gr >= 0 && gr < a.H) << wr;
  }
#pragma unroll
  for (int wc = 0; wc < 10; ++wc) {
    const int gc = c0 + 8 * bc + wc - 1;
    colbits |= (unsigned)(gc >= 0 && gc < a.W) << wc;
  }
  float p[32];
  float mx = -INFINITY;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int cl = 32 * cb + 8 * (i >> 2) + (i & 3);  // cell of lane half 0; half 1 adds 4
      const int c = cl + 4 * h;
      const int wr = h ? (cl + 4) / 10 : cl / 10;
      const int wc = h ? (cl + 4) % 10 : cl % 10;
      const bool ok = c < 60 && (unsigned)(wr - ta) <= 2u && (unsigned)(wc - tb) <= 2u &&
                      ((rowbits >> wr) & (colbits >> wc) & 1u);
      const float l = ok ? lg[cb][i] * a.logit_scale : -INFINITY;
      p[16 * cb + i] = l;
      mx = fmaxf(mx, l);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float den = 0.f;
  bf16x8 Bp[4];
#pragma unroll
  for (int v = 0; v < 32; ++v) {
    const float e = (p[v] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(p[v] - mx);
    const __bf16 eb = (__bf16)e;
    Bp[v >> 3][v & 7] = eb;
    den += (float)eb;  // normalise by the rounded weights actually applied
  }
  den += __shfl_xor(den, 32);
  // L^T = V_win^T P^T: k-slot (h, e) of step kb is cell 16 kb + 8 (e >> 2) + 4 h + (e & 3).
  f32x16 la[2] = {};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int cA = wcell(16 * kb + 4 * (g >> 1) + (i16 >> 2));
    const int cB = wcell(16 * kb + 8 + 4 * (g >> 1) + (i16 >> 2));
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int d = 32 * db + 16 * (g & 1) + 4 * (i16 & 3);
      const bf16x8 A = as_bf16(join(tr_read(cV + row_off<BF16>(cA, d)), tr_read(cV + row_off<BF16>(cB, d))));
      la[db] = mma(A, Bp[kb], la[db]);
    }
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    L[v] = la[0][v] * inv;
    L[16 + v] = la[1][v] * inv;
  }
}

// The same local branch on VALU (fp32 inputs): each lane pair reduces the
// nine dot products of its token and accumulates the weighted values.
template <class Tr>
__device__ __forceinline__ void local_token_valu(const FlowArgs& a, const unsigned char* cK,
                                                 const unsigned char* cV, int CW, int ccell, int row,
                                                 int col, const float (&q)[32], float (&L)[32]) {
  using S = typename Tr::S;
  const int h = (threadIdx.x & 63) >> 5;
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
      load4(reinterpret_cast<const S*>(cK + row_off<Tr>(cell, dimof(4 * c, h))), kx);
#pragma unroll
      for (int e = 0; e < 4; ++e) part += q[4 * c + e] * kx[e];
    }
    part += __shfl_xor(part, 32);
    const bool in = (row + dr >= 0) && (row + dr < a.H) && (col + dc >= 0) && (col + dc < a.W);
    lg[j] = in ? part * a.logit_scale : -INFINITY;
    mx = fmaxf(mx, lg[j]);
  }
#pragma unroll
  for (int v = 0; v < 32; ++v) L[v] = 0.f;
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    const int dr = j / 3 - 1, dc = j % 3 - 1;
    const int cell = ccell + dr * CW + dc;
    const bool in = lg[j] != -INFINITY;
    const float pj = in ? __builtin_amdgcn_exp2f(lg[j] - mx) : 0.f;
    den += pj;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float vx[4];
      load4(reinterpret_cast<const S*>(cV + row_off<Tr>(cell, dimof(4 * c, h))), vx);
#pragma unroll
      for (int e = 0; e < 4; ++e) L[4 * c + e] = in ? L[4 * c + e] + pj * vx[e] : L[4 * c + e];
    }
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int v = 0; v < 32; ++v) L[v] *= inv;
}

// ---------------------------------------------------------------------------
// OUT items: one TR x TC tile (whole 4x8 token blocks) of one slice.  Each
// wave takes a block at a time, one token per lane pair: lanes m and m + 32
// hold 32 features each in accumulator layout, so the chain
// u_1 = phi(Q_i), u_k = u_(k-1) M and the projection z (phi(K)^T V),
// z = sum_k w_k(i) u_k, run on MFMA with no data movement.  K and V cells of
// the tile plus a one-cell halo are in the staged LDS buffer.
// ---------------------------------------------------------------------------
template <class Tr, class Prefetch>
__device__ void out_item(const FlowArgs& a, Item it, const unsigned char* buf, Prefetch prefetch) {
  using S = typename Tr::S;
  using Frag = typename Tr::Frag;
  constexpr bool kMfmaLocal = Tr::EPL == 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int b = it.b;
  int r0, c0;
  tile_origin(a, it.idx, r0, c0);
  const int CW = a.TC + 2;
  const int CB = a.TC / 8, nblk = (a.TR / 4) * CB;
  const unsigned char* cK = buf;
  const unsigned char* cV = buf + kBufBytes / 2;
  const size_t base = (size_t)b * a.n * kD;
  const S* Qb = static_cast<const S*>(a.Q) + base;
  S* Yb = static_cast<S*>(a.Y) + base;
  const bool global = a.T >= 2;

  // Statistics (coherent loads), then this wave's first block of queries.
  float s_l[32];
  Frag fkv[2][Tr::NQ], fm[2][Tr::NQ];
  if (global) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float* sp = a.fin_s + (size_t)b * kD + dimof(4 * c, h);
      const uint64_t lo = get64(sp), hi = get64(sp + 2);
      s_l[4 * c] = __uint_as_float((uint32_t)lo);
      s_l[4 * c + 1] = __uint_as_float((uint32_t)(lo >> 32));
      s_l[4 * c + 2] = __uint_as_float((uint32_t)hi);
      s_l[4 * c + 3] = __uint_as_float((uint32_t)(hi >> 32));
    }
    load_frags<Tr>(a.frag_kv, b, fkv);
    if (a.T >= 3) load_frags<Tr>(a.frag_m, b, fm);
  }
  const float alpha = a.alpha[b % a.heads];

  float q[32];
  bf16x8 qB[4];
  float w[kMaxT];
  int row, col, i, ccell;
  bool valid;
  auto load_block = [&](int blk) {
    const int tr = 4 * (blk / CB) + (n >> 3), tc = 8 * (blk % CB) + (n & 7);
    row = r0 + tr;
    col = c0 + tc;
    valid = row < a.H && col < a.W;
    i = valid ? row * a.W + col : 0;
    ccell = (tr + 1) * CW + (tc + 1);
    const S* qi = Qb + (size_t)i * kD;
#pragma unroll
    for (int c = 0; c < 8; ++c) load4(qi + dimof(4 * c, h), &q[4 * c]);
    if constexpr (kMfmaLocal) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qB[kb] = *reinterpret_cast<const bf16x8*>(qi + 16 * kb + 8 * h);
    }
    if (a.weights) {
      const float* wp = a.weights + ((size_t)b * a.n + i) * a.T;
#pragma unroll
      for (int k = 0; k < kMaxT; ++k) w[k] = (k < a.T) ? wp[k] : 0.f;
    } else {
#pragma unroll
      for (int k = 0; k < kMaxT; ++k) w[k] = a.geo[k];
    }
  };

  int blk = wave;
  if (blk < nblk) load_block(blk);
  prefetch();

  for (; blk < nblk; blk += kThreads / 64) {
    if (blk != wave) load_block(blk);

    // Local branch.
    float L[32];
    if constexpr (kMfmaLocal)
      local_block_mfma(a, cK, cV, CW, r0, c0, blk / CB, blk % CB, qB, L);
    else
      local_token_valu<Tr>(a, cK, cV, CW, ccell, row, col, q, L);

    // Global branch.
    float G[32];
    {
      float vc[32];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        load4(reinterpret_cast<const S*>(cV + row_off<Tr>(ccell, dimof(4 * c, h))), &vc[4 * c]);
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

    if (valid) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = alpha * G[4 * c + e] + (1.f - alpha) * L[4 * c + e];
        store4(Yb + (size_t)i * kD + dimof(4 * c, h), o);
      }
    }
  }

  if (a.wait_out) {
    __syncthreads();
    if (tid == 0) {
      unsigned* cnt = a.slice_cnt + (size_t)b * 4;
      const unsigned old = bump(&cnt[kOut]);
      if (old == (unsigned)(a.nOUT - 1)) {
        put(&cnt[kC], 0u);
        put(&cnt[kOut], 0u);
      }
    }
  }
}

template <class Tr>
__global__ __launch_bounds__(kThreads) void flow_kernel(FlowArgs a) {
  extern __shared__ __align__(1024) unsigned char smem[];
  __shared__ float s_sh[kD];
  __shared__ int sh_t[3];
  const int tid = threadIdx.x;
  const int x = blockIdx.x % a.nq;
  unsigned* qc = a.queue_cnt + x;
  const int total = queue_items(a, x);

  if (tid == 0) {
    sh_t[0] = (int)bump(qc);
    sh_t[1] = (int)bump(qc);
  }
  __syncthreads();
  int cur = sh_t[0], nxt = sh_t[1];
  int bsel = 0;
  if (cur < total) stage<Tr>(a, decode(a, x, cur), smem);

  while (cur < total) {
    const Item it = decode(a, x, cur);
    if (tid == 0) {
      const int t2 = (int)bump(qc);
      unsigned* cnt = a.slice_cnt + (size_t)it.b * 4;
      if (it.kind == kM) {
        wait_for(&cnt[kKV], a.nKV, a.err);
      } else if (it.kind == kC) {
        if (a.nM)
          wait_for(&cnt[kM], a.nM, a.err);
        else
          wait_for(&cnt[kKV], a.nKV, a.err);
      } else if (it.kind == kOut && a.wait_out) {
        wait_for(&cnt[kC], a.nC, a.err);
      }
      sh_t[2] = t2;
    }
    wait_all();  // this item's staged inputs (and the ticket)
    __syncthreads();
    const int after = sh_t[2];
    unsigned char* cb = smem + bsel * kBufBytes;
    unsigned char* nb = smem + (bsel ^ 1) * kBufBytes;
    auto prefetch = [&]() {
      if (nxt < total) stage<Tr>(a, decode(a, x, nxt), nb);
    };
    if (it.kind == kKV)
      stats_item<Tr, false>(a, it, cb, s_sh, prefetch);
    else if (it.kind == kM)
      stats_item<Tr, true>(a, it, cb, s_sh, prefetch);
    else if (it.kind == kC)
      combine_item<Tr>(a, it, prefetch);
    else
      out_item<Tr>(a, it, cb, prefetch);
    __syncthreads();
    cur = nxt;
    nxt = after;
    bsel ^= 1;
  }

  // The last workgroup to finish clears the queue tickets for the next launch.
  if (tid == 0) {
    const unsigned done = bump(a.queue_cnt + 16);
    if (done == gridDim.x - 1) {
      for (int q = 0; q < kMaxQueues; ++q) put(a.queue_cnt + q, 0u);
      put(a.queue_cnt + 16, 0u);
    }
  }
}

}  // namespace

hipError_t launch_flow(int dtype, const FlowArgs& a, int grid, hipStream_t s) {
  const size_t lds = 2 * (size_t)kBufBytes;
  static bool attr_set[2] = {false, false};
  if (dtype == 1) {
    if (!attr_set[1]) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&flow_kernel<BF16>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_set[1] = true;
    }
    hipLaunchKernelGGL(flow_kernel<BF16>, dim3(grid), dim3(kThreads), lds, s, a);
  } else {
    if (!attr_set[0]) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&flow_kernel<F32>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_set[0] = true;
    }
    hipLaunchKernelGGL(flow_kernel<F32>, dim3(grid), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace lisa
