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
// order and write the statistics as MFMA fragments; OUT items produce a run
// of spatial tiles of Y.  Each workgroup takes items from its XCD's queue (an
// atomic ticket) and waits for the items an item depends on through
// per-slice arrival counters.
//
// Every input an item reads from Q, K, V and the weights reaches LDS by
// global_load_lds DMA, one stage (a chunk, or a tile) ahead, into the other of
// two staging buffers.  Data written by other workgroups of the launch
// (partials, fragments) is read with coherent loads right after the
// dependency wait and before the next stage's DMA is issued, and barriers
// after that issue order LDS only, so the DMA of the next stage overlaps the
// whole compute of the current one.
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

template <class Tr>
using LdsOf = Lds<(int)sizeof(typename Tr::S)>;

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

template <class Tr>
__device__ __forceinline__ TileLayout layout_of(const FlowArgs& a) {
  return tile_layout(a.TR, a.TC, a.weights ? a.T : 0, (int)sizeof(typename Tr::S));
}

// ---------------------------------------------------------------------------
// Staging DMA (no wait here).
// ---------------------------------------------------------------------------
// A KV / M item's K rows, and its V (KV) or Q (M) rows.
template <class Tr>
__device__ void stage_chunk(const FlowArgs& a, Item it, unsigned char* buf) {
  using S = typename Tr::S;
  const int tok0 = it.idx * a.chunk;
  const int nv = min(a.chunk, a.n - tok0);
  const S* Kb = static_cast<const S*>(a.K) + ((size_t)it.b * a.n + tok0) * kD;
  const S* Xb = static_cast<const S*>(it.kind == kKV ? a.V : a.Q) + ((size_t)it.b * a.n + tok0) * kD;
  dma_rows<Tr>(buf, nv, [&](int r) { return static_cast<const void*>(Kb + (size_t)r * kD); });
  dma_rows<Tr>(buf + LdsOf<Tr>::kXOff, nv, [&](int r) { return static_cast<const void*>(Xb + (size_t)r * kD); });
}

// Output tile t of slice b (see TileLayout).  Cells and token slots off the
// grid fetch token 0 of the slice; they are never used.
template <class Tr>
__device__ void stage_tile(const FlowArgs& a, int b, int t, unsigned char* buf) {
  using S = typename Tr::S;
  const TileLayout L = layout_of<Tr>(a);
  int r0, c0;
  tile_origin(a, t, r0, c0);
  const int CW = a.TC + 2;
  const size_t base = (size_t)b * a.n;
  const S* Kb = static_cast<const S*>(a.K) + base * kD;
  const S* Vb = static_cast<const S*>(a.V) + base * kD;
  const S* Qb = static_cast<const S*>(a.Q) + base * kD;
  const float inv_cw = 1.f / (float)CW, inv_tc = 1.f / (float)a.TC;
  auto cell_tok = [&](int r) -> size_t {
    const int rr = div_small(r, inv_cw);
    const int row = r0 - 1 + rr, col = c0 - 1 + (r - rr * CW);
    const bool on = ((unsigned)row < (unsigned)a.H) & ((unsigned)col < (unsigned)a.W);
    return (size_t)(on ? row * a.W + col : 0);
  };
  auto slot_tok = [&](int s) -> size_t {
    const int rr = div_small(s, inv_tc);
    const int row = r0 + rr, col = c0 + (s - rr * a.TC);
    const bool on = (row < a.H) & (col < a.W);
    return (size_t)(on ? row * a.W + col : 0);
  };
  dma_rows<Tr>(buf + L.k, L.cells, [&](int r) { return static_cast<const void*>(Kb + cell_tok(r) * kD); });
  dma_rows<Tr>(buf + L.v, L.cells, [&](int r) { return static_cast<const void*>(Vb + cell_tok(r) * kD); });
  dma_rows<Tr>(buf + L.q, L.tokens, [&](int r) { return static_cast<const void*>(Qb + slot_tok(r) * kD); });
  if (a.weights) {
    // T floats per slot, 4 bytes per lane; the last instruction's spare lanes
    // repeat the last element into the region's padding.
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int cnt = L.tokens * a.T;
    const float* wb = a.weights + base * a.T;
    const float inv_t = 1.f / (float)a.T;
    for (int e0 = wave * 64; e0 < cnt; e0 += 256) {
      const int e = min(e0 + lane, cnt - 1);
      const int sl = div_small(e, inv_t);
      dma4(wb + slot_tok(sl) * a.T + (e - sl * a.T), lds_addr(buf + L.w + e0 * 4));
    }
  }
}

// The first stage of an item (C items stage nothing).
template <class Tr>
__device__ void stage_first(const FlowArgs& a, Item it, unsigned char* buf) {
  if (it.kind == kKV || it.kind == kM)
    stage_chunk<Tr>(a, it, buf);
  else if (it.kind == kOut)
    stage_tile<Tr>(a, it.b, it.idx * a.R, buf);
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
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int m = lane & 31, h = lane >> 5, mb = wave >> 1, nb = wave & 1;
  const int tok0 = it.idx * a.chunk;
  const int nv = min(a.chunk, a.n - tok0);
  const int nvr = (nv + 15) & ~15;
  unsigned char* bK = buf;
  unsigned char* bX = buf + LdsOf<Tr>::kXOff;

  if (kIsM && tid < kD) {  // s = sum of the KV items' partials, fixed order
    float t = 0.f;
    for (int p = 0; p < a.nKV; ++p) t += get(a.part_s + ((size_t)it.b * a.P + p) * kD + tid);
    s_sh[tid] = t;
  }
  wait_all();  // nothing of this item is loaded after the next stage's DMA goes out
  prefetch();
  if (kIsM || nv < nvr) {
    if (kIsM) lds_barrier();
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
    lds_barrier();
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
  lds_barrier();
  if (tid == 0) {
    unsigned* cnt = a.slice_cnt + (size_t)it.b * kCntWords;
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
template <class Tr>
__device__ void combine_item(const FlowArgs& a, Item it) {
  constexpr int kBatch = 16;
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
  for (int p0 = 0; p0 < a.P; p0 += kBatch) {
    float x[kBatch][4];
#pragma unroll
    for (int bb = 0; bb < kBatch; ++bb) {
      const int p = min(p0 + bb, a.P - 1);  // loads stay unconditional; extra ones are masked below
#pragma unroll
      for (int j = 0; j < 4; ++j) x[bb][j] = get(part + (size_t)p * (kD * kD) + rows[j] * kD + col);
    }
#pragma unroll
    for (int bb = 0; bb < kBatch; ++bb)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += (p0 + bb < a.P) ? x[bb][j] : 0.f;
  }
  const bool do_s = (it.idx == 0) && tid < kD;
  float sv = 0.f;
  if (do_s)
    for (int p = 0; p < a.P; ++p) sv += get(a.part_s + ((size_t)it.b * a.P + p) * kD + tid);

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
  lds_barrier();
  if (tid == 0) {
    unsigned* cnt = a.slice_cnt + (size_t)it.b * kCntWords;
    const unsigned old = bump(&cnt[kC]);
    if (old == (unsigned)(a.nC - 1)) {
      // Every C item of the slice has passed its wait: clear that count.
      put(&cnt[a.nM ? kM : kKV], 0u);
      if (!(a.nOUT && a.wait_out)) put(&cnt[kC], 0u);
    }
  }
}

// Window slots of the MFMA local branch: logit slot v (0..31) of lane half h
// holds window cell c = 32 (v >> 4) + 8 ((v & 15) >> 2) + (v & 3) + 4 h of
// the block's 6x10 window (cells 60..63 are padding).
__host__ __device__ constexpr int slot_cell(int v, int h) {
  return 32 * (v >> 4) + 8 * ((v & 15) >> 2) + (v & 3) + 4 * h;
}
// Slots of half h whose cell lies in window row wr / window column wc.
__host__ __device__ constexpr unsigned row_slots(int h, int wr) {
  unsigned m = 0;
  for (int v = 0; v < 32; ++v)
    if (slot_cell(v, h) < 60 && slot_cell(v, h) / 10 == wr) m |= 1u << v;
  return m;
}
__host__ __device__ constexpr unsigned col_slots(int h, int wc) {
  unsigned m = 0;
  for (int v = 0; v < 32; ++v)
    if (slot_cell(v, h) < 60 && slot_cell(v, h) % 10 == wc) m |= 1u << v;
  return m;
}

// Slots that hold the 3x3 neighbourhood of block token (ta, tb) (window
// rows ta..ta+2, columns tb..tb+2) for lane half h.
__device__ __forceinline__ unsigned neighbour_slots(int ta, int tb, int h) {
  unsigned r0 = 0, r1 = 0, k0 = 0, k1 = 0;
#pragma unroll
  for (int wr = 0; wr < 6; ++wr)
    if ((unsigned)(wr - ta) <= 2u) {
      r0 |= row_slots(0, wr);
      r1 |= row_slots(1, wr);
    }
#pragma unroll
  for (int wc = 0; wc < 10; ++wc)
    if ((unsigned)(wc - tb) <= 2u) {
      k0 |= col_slots(0, wc);
      k1 |= col_slots(1, wc);
    }
  return h ? (r1 & k1) : (r0 & k0);
}

// Slots whose cell lies on the grid, from the window's on-grid rows and
// columns (bit masks, wave-uniform).
__device__ __forceinline__ unsigned grid_slots(unsigned rowbits, unsigned colbits, int h) {
  if (rowbits == 0x3fu && colbits == 0x3ffu) return ~0u;
  unsigned r0 = 0, r1 = 0, k0 = 0, k1 = 0;
#pragma unroll
  for (int wr = 0; wr < 6; ++wr)
    if ((rowbits >> wr) & 1u) {
      r0 |= row_slots(0, wr);
      r1 |= row_slots(1, wr);
    }
#pragma unroll
  for (int wc = 0; wc < 10; ++wc)
    if ((colbits >> wc) & 1u) {
      k0 |= col_slots(0, wc);
      k1 |= col_slots(1, wc);
    }
  return h ? (r1 & k1) : (r0 & k0);
}

// Local branch of one 4x8 token block on MFMA (bf16).  The block's 3x3
// windows lie in a 6x10 window of staged cells (60, padded to 64).  Logits
// C[cell][token] = K_win Q_blk^T come out with one token per lane pair and the
// cells in accumulator order (the slots above); after the masked softmax,
// those probabilities are already the B operand of L^T = V_win^T P^T (the
// contraction index permuted to match), whose A operand comes from transposed
// LDS reads, and L lands in the same accumulator layout as the global branch.
// `nbr` = neighbour_slots of this lane's token.
__device__ __forceinline__ void local_block_mfma(const FlowArgs& a, const unsigned char* cK,
                                                 const unsigned char* cV, int CW, int r0, int c0,
                                                 int br, int bc, unsigned nbr, const bf16x8 (&qB)[4],
                                                 float scale, float (&L)[32]) {
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
  // Valid slots: the token's neighbourhood, on the grid.
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
  const unsigned valid = nbr & grid_slots(rowbits, colbits, h);
  float p[32];
  float mx = -1e30f;  // finite: a token off the grid may have no valid slot
#pragma unroll
  for (int v = 0; v < 32; ++v) {
    p[v] = (valid & (1u << v)) ? lg[v >> 4][v & 15] : -INFINITY;
    mx = fmaxf(mx, p[v]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float off = -mx * a.logit_scale;  // exp2((l - max) log2(e) / sqrt(d_h)); exp2(-inf) = 0
  bf16x8 Bp[4];
#pragma unroll
  for (int v = 0; v < 32; ++v) Bp[v >> 3][v & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(p[v], a.logit_scale, off));
  // L^T = V_win^T P^T: k-slot (h, e) of step kb is cell 16 kb + 8 (e >> 2) + 4 h + (e & 3).
  // The softmax denominator is the sum of the rounded weights actually
  // applied: a product with an all-ones A operand (every row = that sum).
  f32x16 la[2] = {}, lden = {};
  const bf16x8 ones = as_bf16((v8s)(short)0x3f80);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    lden = mma(ones, Bp[kb], lden);
    const int cA = wcell(16 * kb + 4 * (g >> 1) + (i16 >> 2));
    const int cB = wcell(16 * kb + 8 + 4 * (g >> 1) + (i16 >> 2));
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int d = 32 * db + 16 * (g & 1) + 4 * (i16 & 3);
      const bf16x8 A = as_bf16(join(tr_read(cV + row_off<BF16>(cA, d)), tr_read(cV + row_off<BF16>(cB, d))));
      la[db] = mma(A, Bp[kb], la[db]);
    }
  }
  const float inv = scale / lden[0];
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
                                                 int col, const float (&q)[32], float scale, float (&L)[32]) {
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
  const float inv = scale / den;
#pragma unroll
  for (int v = 0; v < 32; ++v) L[v] *= inv;
}

// ---------------------------------------------------------------------------
// One output tile (whole 4x8 token blocks) of slice b, all inputs in LDS.
// Each wave takes a block at a time, one token per lane pair: lanes m and
// m + 32 hold 32 features each in accumulator layout, so the chain
// u_1 = phi(Q_i), u_k = u_(k-1) M and the projection z (phi(K)^T V),
// z = sum_k w_k(i) u_k, run on MFMA with no data movement.
// ---------------------------------------------------------------------------
template <class Tr>
__device__ __forceinline__ void out_tile(const FlowArgs& a, int b, int t, const unsigned char* buf,
                                         const typename Tr::Frag (&fkv)[2][Tr::NQ],
                                         const typename Tr::Frag (&fm)[2][Tr::NQ], const float* sl,
                                         float alpha, unsigned nbr) {
  using S = typename Tr::S;
  constexpr bool kMfmaLocal = Tr::EPL == 8;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 31, h = lane >> 5;
  const TileLayout Lt = layout_of<Tr>(a);
  int r0, c0;
  tile_origin(a, t, r0, c0);
  const int CW = a.TC + 2;
  const int CB = a.TC / 8, nblk = (a.TR / 4) * CB;
  const unsigned char* cK = buf + Lt.k;
  const unsigned char* cV = buf + Lt.v;
  const unsigned char* cQ = buf + Lt.q;
  const float* cW = reinterpret_cast<const float*>(buf + Lt.w);
  S* Yb = static_cast<S*>(a.Y) + (size_t)b * a.n * kD;
  const bool global = a.T >= 2;

  for (int blk = wave; blk < nblk; blk += kThreads / 64) {
    const int br = blk / CB, bc = blk % CB;
    if (r0 + 4 * br >= a.H || c0 + 8 * bc >= a.W) continue;  // no token of the block is on the grid
    const int tr = 4 * br + (n >> 3), tc = 8 * bc + (n & 7);
    const int slot = tr * a.TC + tc;
    const int row = r0 + tr, col = c0 + tc;
    const bool valid = row < a.H && col < a.W;
    const int i = valid ? row * a.W + col : 0;
    const int ccell = (tr + 1) * CW + (tc + 1);

    float w[kMaxT];
    if (a.weights) {
#pragma unroll
      for (int k = 0; k < kMaxT; ++k) w[k] = cW[slot * a.T + min(k, a.T - 1)];  // terms k >= T are never used
    } else {
#pragma unroll
      for (int k = 0; k < kMaxT; ++k) w[k] = a.geo[k];
    }

    // acc = (1 - alpha) L_i: the local branch.
    float acc[32];
    if constexpr (kMfmaLocal) {
      bf16x8 qB[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qB[kb] = *reinterpret_cast<const bf16x8*>(cQ + row_off<BF16>(slot, 16 * kb + 8 * h));
      local_block_mfma(a, cK, cV, CW, r0, c0, br, bc, nbr, qB, 1.f - alpha, acc);
    } else {
      float q[32];
#pragma unroll
      for (int c = 0; c < 8; ++c) load4(reinterpret_cast<const S*>(cQ + row_off<Tr>(slot, dimof(4 * c, h))), &q[4 * c]);
      local_token_valu<Tr>(a, cK, cV, CW, ccell, row, col, q, 1.f - alpha, acc);
    }

    // + alpha w_0(i) V_i: the k = 0 term of the walk.
    {
      const float f = alpha * w[0];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float vc[4];
        load4(reinterpret_cast<const S*>(cV + row_off<Tr>(ccell, dimof(4 * c, h))), vc);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * c + e] += f * vc[e];
      }
    }
    // + alpha r_i sum_{k>=1} w_k(i) phi(Q_i) M^(k-1) (phi(K)^T V).
    if (global) {
      float u[32], z[32], y[32];
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float qx[4];
        load4(reinterpret_cast<const S*>(cQ + row_off<Tr>(slot, dimof(4 * c, h))), qx);
        const float4 sv = *reinterpret_cast<const float4*>(sl + dimof(4 * c, h));
        const float sx[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * c + e;
          u[v] = fmaxf(qx[e], 0.f);
          part += u[v] * sx[e];
          z[v] = w[1] * u[v];
        }
      }
      part += __shfl_xor(part, 32);
      for (int k = 2; k < a.T; ++k) {
        apply<Tr>(fm, u, y);
#pragma unroll
        for (int v = 0; v < 32; ++v) {
          u[v] = y[v];
          z[v] += w[k] * y[v];
        }
      }
      apply<Tr>(fkv, z, y);
      const float f = alpha / (part + a.eps);
#pragma unroll
      for (int v = 0; v < 32; ++v) acc[v] += f * y[v];
    }

    if (valid) {
#pragma unroll
      for (int c = 0; c < 8; ++c) store4(Yb + (size_t)i * kD + dimof(4 * c, h), &acc[4 * c]);
    }
  }
}

// OUT item: tiles [idx R, idx R + R) of slice b.  The slice's statistics are
// read once per item: fragments and s by coherent DMA into the statistics
// area, then into registers.  Tile k + 1's DMA is issued before tile k is
// computed; the last tile issues the next item's first stage.  Returns the
// staging buffer that the next item's first stage went to.
template <class Tr, class Prefetch>
__device__ int out_item(const FlowArgs& a, Item it, unsigned char* smem, int bsel, Prefetch prefetch_next) {
  using S = typename Tr::S;
  using Frag = typename Tr::Frag;
  using L = LdsOf<Tr>;
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int b = it.b;
  const int t0 = it.idx * a.R, nt = min(a.R, a.ntiles - t0);
  unsigned char* st = smem + 2 * L::kStage;

  Frag fkv[2][Tr::NQ], fm[2][Tr::NQ];
  const float* sl = reinterpret_cast<const float*>(st + 2 * L::kFragBytes);  // s, in LDS
  if (a.T >= 2) {
    dma_linear_coherent(st, static_cast<const S*>(a.frag_kv) + (size_t)b * (kD * kD), L::kFragBytes);
    if (a.T >= 3)
      dma_linear_coherent(st + L::kFragBytes, static_cast<const S*>(a.frag_m) + (size_t)b * (kD * kD), L::kFragBytes);
    dma_linear_coherent(st + 2 * L::kFragBytes, a.fin_s + (size_t)b * kD, kD * 4);
    wait_all();
    lds_barrier();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < Tr::NQ; ++q) {
        const int off = ((mb * Tr::NQ + q) * 64 + lane) * (int)sizeof(Frag);
        fkv[mb][q] = *reinterpret_cast<const Frag*>(st + off);
        fm[mb][q] = *reinterpret_cast<const Frag*>(st + L::kFragBytes + off);
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < Tr::NQ; ++q) {
        fkv[mb][q] = Frag{};
        fm[mb][q] = Frag{};
      }
  }
  const float alpha = a.alpha[b % a.heads];
  wait_all();
  const int tok = lane & 31;
  const unsigned nbr = neighbour_slots(tok >> 3, tok & 7, h);

  for (int k = 0; k < nt; ++k) {
    unsigned char* cb = smem + bsel * L::kStage;
    unsigned char* nb = smem + (bsel ^ 1) * L::kStage;
    if (k > 0) {
      wait_all();
      lds_barrier();
    }
    if (k + 1 < nt)
      stage_tile<Tr>(a, b, t0 + k + 1, nb);
    else
      prefetch_next(nb);
    out_tile<Tr>(a, b, t0 + k, cb, fkv, fm, sl, alpha, nbr);
    bsel ^= 1;
  }
  return bsel;
}

template <class Tr>
__global__ __launch_bounds__(kThreads) void flow_kernel(FlowArgs a) {
  using L = LdsOf<Tr>;
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
  if (cur < total) stage_first<Tr>(a, decode(a, x, cur), smem);

  while (cur < total) {
    const Item it = decode(a, x, cur);
    const Item nit = nxt < total ? decode(a, x, nxt) : Item{kNone, 0, 0};
    wait_all();  // this item's first stage (and everything before it)
    lds_barrier();
    unsigned char* nb = smem + (bsel ^ 1) * L::kStage;
    auto prefetch_into = [&](unsigned char* dst) {
      if (nit.kind != kNone) stage_first<Tr>(a, nit, dst);
    };
    // C items stage nothing, so the next item's inputs can go out before the wait.
    if (it.kind == kC) prefetch_into(nb);
    if (tid == 0) {
      const int t2 = (int)bump(qc);
      unsigned* cnt = a.slice_cnt + (size_t)it.b * kCntWords;
      if (it.kind == kM) {
        wait_for(&cnt[kKV], a.nKV, a.err);
      } else if (it.kind == kC) {
        if (a.nM)
          wait_for(&cnt[kM], a.nM, a.err);
        else
          wait_for(&cnt[kKV], a.nKV, a.err);
      } else if (it.kind == kOut && a.wait_out) {
        wait_for(&cnt[kC], a.nC, a.err);
        // Count the OUT items past their wait; the last clears both counts.
        const unsigned old = bump(&cnt[kOut]);
        if (old == (unsigned)(a.nOUT - 1)) {
          put(&cnt[kC], 0u);
          put(&cnt[kOut], 0u);
        }
      }
      sh_t[2] = t2;
    }
    lds_barrier();
    const int after = sh_t[2];
    unsigned char* cb = smem + bsel * L::kStage;
    auto prefetch = [&]() { prefetch_into(nb); };
    if (it.kind == kKV) {
      stats_item<Tr, false>(a, it, cb, s_sh, prefetch);
      bsel ^= 1;
    } else if (it.kind == kM) {
      stats_item<Tr, true>(a, it, cb, s_sh, prefetch);
      bsel ^= 1;
    } else if (it.kind == kC) {
      combine_item<Tr>(a, it);
      bsel ^= 1;
    } else {
      bsel = out_item<Tr>(a, it, smem, bsel, prefetch_into);
    }
    cur = nxt;
    nxt = after;
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

template <class Tr>
hipError_t launch_typed(const FlowArgs& a, int grid, hipStream_t s) {
  constexpr int lds = LdsOf<Tr>::kTotal;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&flow_kernel<Tr>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(flow_kernel<Tr>, dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_flow(int dtype, const FlowArgs& a, int grid, hipStream_t s) {
  return dtype == 1 ? launch_typed<BF16>(a, grid, s) : launch_typed<F32>(a, grid, s);
}

}  // namespace lisa
