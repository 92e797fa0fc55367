// The LiSA forward pass on gfx950 as one persistent kernel.
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
// Schedule (FlowArgs): the G ranks of a group split each slice's tokens for
// the KV and M sweeps (contractions over tokens on MFMA), its 64x64
// statistics for the combine, and its output tiles; a rank waits for the
// group's previous phase through per-slice arrival counters.
//
// A workgroup has two roles of four waves each, one wave of each per SIMD.
// Producer waves prepare the next stage (a chunk, an output tile, or the
// partials a combine sums) in the other of two LDS staging buffers: they
// issue its global_load_lds DMA (issuing stalls a wave for about as long as
// the transfer takes), wait for its dependencies, load what other
// workgroups wrote, and finish the staged data in place (the rescaled Q rows
// of an M chunk).  Consumer waves only compute on the current stage and
// publish results; they never wait for a DMA.  One workgroup barrier per
// stage hands the buffers over.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lisa_device.hpp"
#include "lisa_flow_schedule.hpp"
#include "lisa_kernels.hpp"

namespace lisa {
namespace {

template <class Tr>
using LdsOf = Lds<(int)sizeof(typename Tr::S)>;

enum Counter { kCntKV = 0, kCntM = 1, kCntC = 2 };

// The counter a rank's arrival for phase `counter` of slice b goes to.
template <int kVar>
__device__ __forceinline__ unsigned* arrival_counter(const FlowArgs& a, const Rank& rk, int b, int counter) {
  if constexpr (kVar == kVarGrouped) return a.sub_cnt + (((size_t)b * 3 + counter) * kMaxSubs + rk.g / kSubRanks) * kCntStride;
  return a.slice_cnt + (size_t)b * kCntStride + counter;
}

// A rank's arrival for one phase.  Each consumer wave, after its own stores
// have completed, counts itself in LDS (`waves`); the last of the kRoleWaves
// waves bumps the slice counter once, so a slice's counter reaches G.  That
// wave's atomic follows every other wave's completed stores (their LDS
// increments came first).  Stage barriers separate the phases, so the last
// wave's reset precedes the next phase's increments.  Nothing waits for the
// global atomic; counters only grow during a launch and the last workgroup
// clears them.
__device__ __forceinline__ void arrive(unsigned* c) {
  (void)__hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void arrive_rank(unsigned* c, int* waves) {
  if ((threadIdx.x & 63) == 0 && atomicAdd(waves, 1) == kRoleWaves - 1) {
    *waves = 0;
    arrive(c);
  }
}

template <class Tr>
__device__ __forceinline__ TileLayout layout_of(const FlowArgs& a) {
  return tile_layout(a.TR, a.TC, (a.weights || a.mlp_w1f) ? a.T : 0, (int)sizeof(typename Tr::S));
}

// ---------------------------------------------------------------------------
// Producer side (pw = producer wave, 0..3).
// ---------------------------------------------------------------------------
// DMA of a KV / M chunk: its K rows (unless the buffer still holds them),
// and its V (KV) or Q (M) rows.
template <class Tr>
__device__ void stage_chunk(const FlowArgs& a, int b, bool is_m, int tok0, int nv, unsigned char* buf, int pw,
                            bool with_k) {
  using S = typename Tr::S;
  const S* Kb = static_cast<const S*>(a.K) + ((size_t)b * a.n + tok0) * kD;
  const S* Xb = static_cast<const S*>(is_m ? a.Q : a.V) + ((size_t)b * a.n + tok0) * kD;
  if (with_k) dma_rows<Tr>(buf, nv, [&](int r) { return static_cast<const void*>(Kb + (size_t)r * kD); }, pw);
  dma_rows<Tr>(buf + LdsOf<Tr>::kXOff, nv, [&](int r) { return static_cast<const void*>(Xb + (size_t)r * kD); }, pw);
}

// DMA of output tile t of slice b (see TileLayout).  Cells and token slots
// off the grid fetch token 0 of the slice; they are never used.
template <class Tr>
__device__ void stage_tile(const FlowArgs& a, int b, int t, unsigned char* buf, int pw) {
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
  dma_rows<Tr>(buf + L.k, L.cells, [&](int r) { return static_cast<const void*>(Kb + cell_tok(r) * kD); }, pw);
  dma_rows<Tr>(buf + L.v, L.cells, [&](int r) { return static_cast<const void*>(Vb + cell_tok(r) * kD); }, pw);
  dma_rows<Tr>(buf + L.q, L.tokens, [&](int r) { return static_cast<const void*>(Qb + slot_tok(r) * kD); }, pw);
  if (a.weights) {
    // T floats per slot, 4 bytes per lane, 64 per wave instruction; the last
    // instruction's spare lanes repeat the last element into the padding.
    const int lane = threadIdx.x & 63;
    const int cnt = L.tokens * a.T;
    const float* wb = a.weights + base * a.T;
    const float inv_t = 1.f / (float)a.T;
    for (int e0 = pw * 64; e0 < cnt; e0 += 256) {
      const int e = min(e0 + lane, cnt - 1);
      const int sl = div_small(e, inv_t);
      dma4(wb + slot_tok(sl) * a.T + (e - sl * a.T), lds_addr(buf + L.w + e0 * 4));
    }
  }
}

// bf16 rows staged by dma_rows: run j (1 KB) holds rows 8 j .. 8 j + 7 and
// producer wave j % 4 issued it.  Lane l of wave pw takes slot l % 8 of row
// 8 j + l / 8 in each of its runs j = pw, pw + 4, ...; that slot holds piece
// g of the row, and since swz(r) depends only on r & 7 = l / 8 and on
// (r >> 3) & 1 = j & 1 = pw & 1, g is the same in every run of the wave.
// f(j, r, x, dot) is called per run with the run's eight elements of the
// lane's piece after the feature map (ReLU applied to the bf16 bits: a
// negative bf16 is a negative int16; ELU + 1 rounded back to bf16), and
// dot = their product with s over the row (s[8 g .. 8 g + 7] held in
// registers); runs go four at a time, all their
// LDS reads issued before the first product.  `nrun` is wave-uniform.
template <bool kElu = false, class F>
__device__ __forceinline__ void bf16_row_dots(const unsigned char* base, int nrun, const float* s, int pw, F f) {
  const int lane = threadIdx.x & 63;
  const int slot = lane & 7, sub = lane >> 3;
  const int g = (slot ^ swz(8 * pw + sub)) & 7;
  const float4 s0 = *reinterpret_cast<const float4*>(s + 8 * g);
  const float4 s1 = *reinterpret_cast<const float4*>(s + 8 * g + 4);
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  for (int j0 = pw; j0 < nrun; j0 += 16) {
    uint4 raw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j0 + 4 * u < nrun) raw[u] = *reinterpret_cast<const uint4*>(base + (8 * (j0 + 4 * u) + sub) * 128 + slot * 16);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + 4 * u;
      if (j < nrun) {
        const v8s bits = kElu ? __builtin_bit_cast(v8s, raw[u])
                              : __builtin_elementwise_max(__builtin_bit_cast(v8s, raw[u]), (v8s)0);
        const u32x4 w = __builtin_bit_cast(u32x4, bits);
        float x[8];
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
          // ELU + 1 features rounded to bf16, as the s sweep and the output's
          // u_1 take them (elu1_bits): r_j and the rows of M then use the same
          // features, and the rows of S stay stochastic.
          if (kElu) x[e] = bf2f(f2bf(elu1(x[e])));
          dot += x[e] * sv[e];
        }
        f(j, 8 * j + sub, x, group_sum8(dot));
      }
    }
  }
}

// After the wave's own DMA has landed: zero the chunk's rows [nv, nvr) (the
// sweeps read whole 16-row steps) and, for M chunks, rewrite each Q row as
// r_j phi(Q_j) with r_j = 1 / (phi(Q_j) . s + eps).  A wave only touches the
// 1 KB runs it issued itself (run j belongs to wave j % 4): each lane holds
// one 16-byte piece, and the lanes of a row reduce the dot product together.
template <class Tr, bool kIsM, bool kElu = false>
__device__ void finish_chunk(const FlowArgs& a, int nv, unsigned char* buf, const float* s, int pw) {
  constexpr int RPR = 1024 / Tr::RB;  // rows per run
  // K rows past the chunk: phi of the pad is 0 (ReLU of 0, ELU + 1 of -inf).
  constexpr unsigned kPad = !kElu ? 0u : Tr::EPP == 8 ? 0xff80ff80u : 0xff800000u;
  const int lane = threadIdx.x & 63;
  const int nvr = (nv + 15) & ~15;
  unsigned char* bK = buf;
  unsigned char* bX = buf + LdsOf<Tr>::kXOff;
  const int slot = lane % Tr::PPR;
  if constexpr (kIsM && Tr::EPP == 8) {
    bf16_row_dots<kElu>(bX, nvr / RPR, s, pw, [&](int, int r, float (&x)[8], float dot) {
      uint4* pK = reinterpret_cast<uint4*>(bK + r * Tr::RB + slot * 16);
      uint4* pX = reinterpret_cast<uint4*>(bX + r * Tr::RB + slot * 16);
      if (r < nv) {
        const float rr = __builtin_amdgcn_rcpf(dot + a.eps);
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(x[2 * e] * rr, x[2 * e + 1] * rr);
        *reinterpret_cast<u32x4*>(pX) = o;
      } else {
        *pK = make_uint4(kPad, kPad, kPad, kPad);
        *pX = make_uint4(0, 0, 0, 0);
      }
    });
    return;
  }
#pragma unroll 2
  for (int j = pw; j * RPR < nvr; j += 4) {
    if (!kIsM && (j + 1) * RPR <= nv) continue;  // nothing to zero in this run
    const int r = j * RPR + lane / Tr::PPR;
    const int g = (slot ^ swz(r)) & (Tr::PPR - 1);  // the piece in this slot
    uint4* pK = reinterpret_cast<uint4*>(bK + r * Tr::RB + slot * 16);
    uint4* pX = reinterpret_cast<uint4*>(bX + r * Tr::RB + slot * 16);
    if (kIsM) {
      float x[Tr::EPP];
      if constexpr (Tr::EPP == 8) {
        load4(reinterpret_cast<const uint16_t*>(pX), x);
        load4(reinterpret_cast<const uint16_t*>(pX) + 4, x + 4);
      } else {
        load4(reinterpret_cast<const float*>(pX), x);
      }
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < Tr::EPP; ++e) {
        x[e] = feat<kElu>(x[e]);
        dot += x[e] * s[g * Tr::EPP + e];
      }
      dot = Tr::PPR == 8 ? group_sum8(dot) : group_sum16(dot);
      const float rr = 1.f / (dot + a.eps);
#pragma unroll
      for (int e = 0; e < Tr::EPP; ++e) x[e] *= rr;
      if (r < nv) {
        if constexpr (Tr::EPP == 8) {
          store4(reinterpret_cast<uint16_t*>(pX), x);
          store4(reinterpret_cast<uint16_t*>(pX) + 4, x + 4);
        } else {
          store4(reinterpret_cast<float*>(pX), x);
        }
      }
    }
    if (r >= nv) {
      *pK = make_uint4(kPad, kPad, kPad, kPad);
      *pX = make_uint4(0, 0, 0, 0);
    }
  }
}

// After the wave's own DMA of an output tile has landed: r_j = 1 / (phi(Q_j)
// . s + eps) for the Q rows of the 1 KB runs it issued (run j belongs to
// wave j % 4), written to the tile's r region.  The lanes of a row each take
// one 16-byte piece and reduce the dot product together.
template <class Tr, bool kElu = false>
__device__ void finish_tile(const FlowArgs& a, const TileLayout& L, unsigned char* buf, const float* s, int pw) {
  constexpr int RPR = 1024 / Tr::RB;  // rows per run
  const int lane = threadIdx.x & 63;
  const int slot = lane % Tr::PPR;
  const unsigned char* bQ = buf + L.q;
  float* rr = reinterpret_cast<float*>(buf + L.r);
  if constexpr (Tr::EPP == 8) {
    bf16_row_dots<kElu>(bQ, L.tokens / RPR, s, pw, [&](int, int r, float (&)[8], float dot) {
      if (slot == 0) rr[r] = __builtin_amdgcn_rcpf(dot + a.eps);
    });
    return;
  }
#pragma unroll 2
  for (int j = pw; j * RPR < L.tokens; j += 4) {
    const int r = j * RPR + lane / Tr::PPR;
    const int g = (slot ^ swz(r)) & (Tr::PPR - 1);  // the piece in this slot
    const unsigned char* pX = bQ + r * Tr::RB + slot * 16;
    float x[Tr::EPP];
    if constexpr (Tr::EPP == 8) {
      load4(reinterpret_cast<const uint16_t*>(pX), x);
      load4(reinterpret_cast<const uint16_t*>(pX) + 4, x + 4);
    } else {
      load4(reinterpret_cast<const float*>(pX), x);
    }
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < Tr::EPP; ++e) dot += feat<kElu>(x[e]) * s[g * Tr::EPP + e];
    dot = Tr::PPR == 8 ? group_sum8(dot) : group_sum16(dot);
    if (slot == 0) rr[r] = 1.f / (dot + a.eps);
  }
}

// Lane l of a wave: s[l] = fixed-order sum over the G ranks' partials.
__device__ __forceinline__ float sum_s_partials(const FlowArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  const float* ps = a.part_s + (size_t)b * a.G * kD + lane;
  float t = 0.f;
  for (int p0 = 0; p0 < a.G; p0 += 16) {
    float x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) x[q] = get(ps + (size_t)min(p0 + q, a.G - 1) * kD);
#pragma unroll
    for (int q = 0; q < 16; ++q) t += (p0 + q < a.G) ? x[q] : 0.f;
  }
  return t;
}

// The walk-weight predictor, run by the producer waves on a staged output
// tile (its Q rows and K cells): w = softmax(W2 ReLU(W1 concat(q, k) + b1)
// + b2) per token.  The first layer runs on MFMA 32x32 as W1 x^T, 32 hidden
// units at a time, with W1 laid out by mlp_prep per head as the lanes read
// it: bf16 inputs, [hidden/32][8 steps of 16 inputs][64 lanes] bf16x8 (W1
// rounded to bf16 once, like the walk's P_k; the inputs are exact); fp32,
// [hidden/32][64 steps of 2 inputs][64 lanes] floats.  Element i of lane
// (n, h) of its accumulator is hidden unit 32 hb + 8 (i / 4) + i % 4 + 4 h of
// token n: lane halves 0 and 1 hold the two contraction slots of an fp32
// MFMA 32x32x2, so the second layer is 16 of those, A = W2 (rows past T
// zero) and B = the hidden values; its accumulator element e of lane (n, h)
// is logit 4 h + e of token n.  A lane's W2 and b1 operands are gathered
// from their natural layouts together with its W1 operands.

template <class Tr>
struct MlpRegs {
  static constexpr bool kBf16 = Tr::EPL == 8;
  bf16x8 fh[kBf16 ? 8 : 1];
  float fw[kBf16 ? 1 : 64];
  float w2[16], b1[16];
  // One hidden block's operands of this lane.
  __device__ __forceinline__ void load(const FlowArgs& a, int head, int hb) {
    const int lane = threadIdx.x & 63, m = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = 32 * hb + 8 * (i / 4) + i % 4 + 4 * h;  // hidden unit of slot h, element i
      w2[i] = m < a.T ? a.mlp_w2[((size_t)head * a.T + m) * a.hidden + j] : 0.f;
      b1[i] = a.mlp_b1[(size_t)head * a.hidden + j];
    }
    const float* blk = static_cast<const float*>(a.mlp_w1f) + (size_t)head * mlp_head_floats(a.hidden, kBf16);
    if constexpr (kBf16) {
      const bf16x8* f = reinterpret_cast<const bf16x8*>(blk) + (size_t)hb * 8 * 64;
#pragma unroll
      for (int st = 0; st < 8; ++st) fh[st] = f[st * 64 + lane];
    } else {
#pragma unroll
      for (int st = 0; st < 64; ++st) fw[st] = blk[((size_t)hb * 64 + st) * 64 + lane];
    }
  }
};

// Producer wave pw, once every producer wave's DMA of output tile t has
// landed: the predicted weights of the tile's 32-token blocks pw and pw + 4
// (blocks of 4 rows x 8 columns, as the consumers take them), into the
// tile's weight slots.  pr holds hidden block 0's operands (loaded before
// the tile's DMA was issued).
template <class Tr>
__device__ void predict_tile(const FlowArgs& a, int b, int t, unsigned char* buf, int pw, MlpRegs<Tr>& pr) {
  static_assert(kMaxTileTokens / 32 <= 2 * kRoleWaves, "at most two 32-token blocks per producer wave");
  const TileLayout L = layout_of<Tr>(a);
  int r0, c0;
  tile_origin(a, t, r0, c0);
  const int lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5, CW = a.TC + 2;
  const int CB = a.TC / 8, nblk = (a.TR / 4) * CB;
  const int head = __builtin_amdgcn_readfirstlane(b % a.heads);
  const int hidden = __builtin_amdgcn_readfirstlane(a.hidden), nhb = hidden / 32, T = a.T;
  const unsigned char* cQ = buf + L.q;
  const unsigned char* cK = buf + L.k;
  int slot[2], ccell[2];
  bool on[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int blk = pw + kRoleWaves * q, br = blk / CB, bc = blk % CB;
    on[q] = blk < nblk && r0 + 4 * br < a.H && c0 + 8 * bc < a.W;  // a token of the block is on the grid
    const int tr = 4 * br + (n >> 3), tc = 8 * bc + (n & 7);
    slot[q] = tr * a.TC + tc;
    ccell[q] = (tr + 1) * CW + (tc + 1);
  }
  f32x16 lg[2] = {};
#pragma unroll 1
  for (int hb = 0; hb < nhb; ++hb) {
    if (hb > 0) pr.load(a, head, hb);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!on[q]) continue;
      f32x16 c = {};
      if constexpr (MlpRegs<Tr>::kBf16) {
        bf16x8 xb[8];
#pragma unroll
        for (int st = 0; st < 8; ++st)
          xb[st] = *reinterpret_cast<const bf16x8*>(st < 4 ? cQ + row_off<BF16>(slot[q], 16 * st + 8 * h)
                                                           : cK + row_off<BF16>(ccell[q], 16 * (st - 4) + 8 * h));
#pragma unroll
        for (int st = 0; st < 8; ++st) c = mma(pr.fh[st], xb[st], c);
      } else {
#pragma unroll
        for (int st = 0; st < 64; ++st) {
          const unsigned char* src = st < 32 ? cQ + row_off<F32>(slot[q], 2 * st + h)
                                             : cK + row_off<F32>(ccell[q], 2 * (st - 32) + h);
          c = mma(pr.fw[st], *reinterpret_cast<const float*>(src), c);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) lg[q] = mma(pr.w2[i], fmaxf(c[i] + pr.b1[i], 0.f), lg[q]);
    }
  }
  float* cW = reinterpret_cast<float*>(buf + L.w);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (!on[q]) continue;
    float v[4], mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 4 * h + e;
      v[e] = k < T ? lg[q][e] + a.mlp_b2[head * T + k] : 0.f;
      if (k < T) mx = fmaxf(mx, v[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = 4 * h + e < T ? __expf(v[e] - mx) : 0.f;
      sum += v[e];
    }
    sum += __shfl_xor(sum, 32);
    const float inv = 1.f / sum;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * h + e < T) cW[slot[q] * T + 4 * h + e] = v[e] * inv;
  }
}

// The producer waves meet: each counts itself in `ready` and waits until all
// kRoleWaves have (every producer wave takes part in every OUT stage, so the
// count reaches the next multiple of kRoleWaves).
__device__ __forceinline__ void producers_meet(int* ready) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    const int target = (atomicAdd(ready, 1) / kRoleWaves + 1) * kRoleWaves;
    while (__atomic_load_n(ready, __ATOMIC_RELAXED) < target) __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Producer waves: make stage `p` ready for the consumers in `buf` and, at the
// start of an OUT phase, in the statistics area `st`: issue the DMA, wait for
// the dependency, load what other workgroups wrote, wait, finish.  Only
// producer wave 0 polls the arrival counter; it then posts `tag` in `dep_ok`,
// which the other producer waves watch in LDS.  `s_sl` holds s of each slice
// of the round in LDS (row z for slice z); every producer wave forms the same
// fixed-order sum and writes the same values.
template <class Tr, bool kMlp, int kVar>
__device__ void prepare(const FlowArgs& a, const Rank& rk, Pos p, unsigned char* buf, unsigned char* st,
                        float (*s_sl)[kD], volatile int* dep_ok, int* mlp_ready, int pw) {
  using S = typename Tr::S;
  using L = LdsOf<Tr>;
  const int lane = threadIdx.x & 63;
  const int b = slice_of(a, rk, p.r, p.z);
  const unsigned* cnt = a.slice_cnt + (size_t)b * kCntStride;
  const unsigned full = a.G;
  float* s_w = s_sl[p.z];
  auto dependency = [&](int counter) {
    const int tag = b * 4 + p.ph;
    if (pw == 0) {
      if constexpr (kVar == kVarGrouped) {
        wait_for_groups(a.sub_cnt + ((size_t)b * 3 + counter) * kMaxSubs * kCntStride, a.G / kSubRanks, a.err);
        if (lane == 0) *dep_ok = tag;
      } else if (lane == 0) {
        wait_for(&cnt[counter], full, a.err);
        *dep_ok = tag;
      }
    } else if (lane == 0) {
      while (*dep_ok != tag) __builtin_amdgcn_s_sleep(1);  // wave 0 always posts
    }
    // Loads of the data the dependency announces stay below the wait.
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  };
  if (p.ph == kPKV || p.ph == kPM) {
    const bool is_m = p.ph == kPM;
    int tok0, nv;
    chunk_of(a, rk, p.j, tok0, nv);
    // Stages alternate between the two buffers, and a round runs the KV
    // chunks of all its slices, then their M chunks in the same order.  When
    // the round has two KV stages (one slice of two chunks, or two slices of
    // one), M chunk j lands in the buffer that KV chunk j used two stages
    // before: its K rows (ReLU applied on read, tail rows zeroed) are still
    // there, and only the Q rows are fetched.
    const bool keep_k = is_m && rk.nch * round_slices(a, rk, p.r) == 2;
    stage_chunk<Tr>(a, b, is_m, tok0, nv, buf, pw, !keep_k);
    if (is_m && p.j == 0) {
      dependency(kCntKV);
      // s = the sum of the G partials.  Up to 16 partials: every producer
      // wave sums them all, one round of loads.  More: wave pw sums partials
      // pw, pw + 4, ..., sixteen loads in flight at a time, and the four sums
      // meet in the statistics area (free until the OUT phase), added in wave
      // order.
      float sv;
      if (a.G <= 16) {
        sv = sum_s_partials(a, b);
      } else {
        const float* ps = a.part_s + (size_t)b * a.G * kD + lane;
        const int np = (a.G - pw + kRoleWaves - 1) / kRoleWaves;  // partials of this wave
        float t = 0.f;
        for (int q0 = 0; q0 < np; q0 += 16) {
          float x[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) x[q] = get(ps + (size_t)min(pw + kRoleWaves * (q0 + q), a.G - 1) * kD);
#pragma unroll
          for (int q = 0; q < 16; ++q) t += (q0 + q < np) ? x[q] : 0.f;
        }
        float* sc = reinterpret_cast<float*>(st);
        sc[pw * kD + lane] = t;
        producers_meet(mlp_ready);
        sv = ((sc[lane] + sc[kD + lane]) + sc[2 * kD + lane]) + sc[3 * kD + lane];
      }
      s_w[lane] = sv;
      if (rk.g == 0 && pw == 0) put(a.fin_s + (size_t)b * kD + lane, sv);
    }
    wait_all();
    if (is_m)
      finish_chunk<Tr, true, kVar == kVarElu>(a, nv, buf, s_w, pw);
    else
      finish_chunk<Tr, false, kVar == kVarElu>(a, nv, buf, s_w, pw);
  } else if (p.ph == kPC) {
    dependency(a.do_m ? kCntM : kCntKV);
    if (!a.do_m && rk.g == 0 && pw == 0) put(a.fin_s + (size_t)b * kD + lane, sum_s_partials(a, b));
    // The G partials' elements [e0, e0 + E), coherent (other workgroups wrote
    // them), as [G][E] floats: 16 bytes per lane, 1 KB per wave instruction.
    const int total = a.G * rk.E;
    for (int q0 = pw * 256; q0 < total; q0 += 1024) {
      const int q = q0 + lane * 4;
      const int part = q / rk.E, f = rk.e0 + q % rk.E;
      const float* src = (f < kD * kD ? a.part_kv : a.part_m) + ((size_t)b * a.G + part) * (kD * kD) + (f % (kD * kD));
      dma16_coherent(src, lds_addr(buf + q0 * 4));
    }
    wait_all();
  } else if (p.ph == kPOut) {
    MlpRegs<Tr> pr;
    if constexpr (kMlp) pr.load(a, __builtin_amdgcn_readfirstlane(b % a.heads), 0);  // lands during the DMA
    stage_tile<Tr>(a, b, rk.t0 + p.j, buf, pw);
    // The statistics fragments, wanted once per slice.  With an M phase this
    // round, s is already in s_w (formed for the M chunks), so the tile's r_i
    // and predicted weights are computed before waiting for the combine;
    // otherwise s comes from the workspace with the fragments.
    auto load_stats = [&]() {
      dma_linear_coherent(st, static_cast<const S*>(a.frag_kv) + (size_t)b * (kD * kD), L::kFragBytes, pw);
      if (a.T >= 3)
        dma_linear_coherent(st + L::kFragBytes, static_cast<const S*>(a.frag_m) + (size_t)b * (kD * kD),
                            L::kFragBytes, pw);
    };
    const bool s_known = a.do_m;  // do_m implies do_kv and T >= 3
    if (p.j == 0 && !s_known) {
      if (a.do_kv) dependency(kCntC);
      if (a.T >= 2) {
        load_stats();
        s_w[lane] = get(a.fin_s + (size_t)b * kD + lane);  // kept for the slice's later tiles
      }
    }
    wait_all();
    if constexpr (kMlp) {
      producers_meet(mlp_ready);
      predict_tile<Tr>(a, b, rk.t0 + p.j, buf, pw, pr);
    }
    if (a.T >= 2) finish_tile<Tr, kVar == kVarElu>(a, layout_of<Tr>(a), buf, s_w, pw);
    if (p.j == 0 && s_known) {
      dependency(kCntC);
      load_stats();
      wait_all();
    }
  }
}

// Element d of staged fp32 row r.
__device__ __forceinline__ float lds_elem(const unsigned char* base, int r, int d, F32) {
  return *reinterpret_cast<const float*>(base + row_off<F32>(r, d));
}

// ---------------------------------------------------------------------------
// Consumer side (cw = consumer wave, 0..3; ct = thread index in the role).
// ---------------------------------------------------------------------------
// One chunk of a KV / M sweep, accumulated into acc (and acc_s: s, KV only).
// Wave cw owns block (cw / 2, cw % 2) of the 64x64 result; A = phi(K) rows,
// B = V rows (KV) or the rescaled Q rows (M); rows past the chunk are zero.
template <class Tr, bool kIsM, bool kElu = false>
__device__ __forceinline__ void sweep_chunk(const unsigned char* buf, int nv, int cw, f32x16& acc, f32x16& acc_s) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5, mb = cw >> 1, nb = cw & 1;
  const int nvr = (nv + 15) & ~15;
  const unsigned char* bK = buf;
  const unsigned char* bX = buf + LdsOf<Tr>::kXOff;
  if constexpr (Tr::EPL == 8) {
    // Steps of 16 rows in batches of U: every operand read of a batch is
    // issued before its first MFMA, so the LDS latency is paid once per batch.
    const bf16x8 ones = as_bf16((v8s)(short)0x3f80);  // bf16 1.0
    auto batch = [&](auto u_tag, auto s_tag, int kk) {
      constexpr int U = decltype(u_tag)::value;
      constexpr bool kS = decltype(s_tag)::value;
      v8s A[U], B[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        A[u] = rows_bits<true, kElu>(bK, kk + 16 * u, 32 * mb);
        B[u] = rows_bits<false>(bX, kk + 16 * u, 32 * nb);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc = mma(as_bf16(A[u]), as_bf16(B[u]), acc);
        if constexpr (kS) acc_s = mma(as_bf16(A[u]), ones, acc_s);
      }
    };
    auto sweep = [&](auto s_tag) {
      int kk = 0;
      for (; kk + 128 <= nvr; kk += 128) batch(std::integral_constant<int, 8>{}, s_tag, kk);
      if (kk + 64 <= nvr) {
        batch(std::integral_constant<int, 4>{}, s_tag, kk);
        kk += 64;
      }
      if (kk + 32 <= nvr) {
        batch(std::integral_constant<int, 2>{}, s_tag, kk);
        kk += 32;
      }
      if (kk < nvr) batch(std::integral_constant<int, 1>{}, s_tag, kk);
    };
    if (!kIsM && nb == 0)  // these waves also sum phi(K) (s) against a ones operand
      sweep(std::true_type{});
    else
      sweep(std::false_type{});
  } else {
    for (int kk = 0; kk < nvr; kk += 16) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = kk + 8 * h + q;
        const float A = feat<kElu>(lds_elem(bK, r, 32 * mb + m, Tr{}));
        const float B = lds_elem(bX, r, 32 * nb + m, Tr{});
        acc = mma(A, B, acc);
        if (!kIsM && nb == 0) acc_s = mma(A, 1.f, acc_s);
      }
    }
  }
}

// The KV or M phase of slice b: the rank's chunks, one stage each, then its
// partial (coherent stores) and the wave's arrival.
template <class Tr, bool kIsM, int kVar>
__device__ int consume_sweep(const FlowArgs& a, const Rank& rk, int b, unsigned char* smem, int bsel, int cw,
                             int* waves) {
  using L = LdsOf<Tr>;
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5, mb = cw >> 1, nb = cw & 1;
  f32x16 acc = {}, acc_s = {};
  for (int j = 0; j < rk.nch; ++j) {
    int tok0, nv;
    chunk_of(a, rk, j, tok0, nv);
    sweep_chunk<Tr, kIsM, kVar == kVarElu>(smem + bsel * L::kStage, nv, cw, acc, acc_s);
    if (j + 1 < rk.nch) {
      lds_barrier();
      bsel ^= 1;
    }
  }
  float* part = (kIsM ? a.part_m : a.part_kv) + ((size_t)b * a.G + rk.g) * (kD * kD);
#pragma unroll
  for (int i = 0; i < 16; ++i) put(part + (32 * mb + 8 * (i >> 2) + 4 * h + (i & 3)) * kD + 32 * nb + m, acc[i]);
  if (!kIsM && nb == 0 && m == 0) {
    float* ps = a.part_s + ((size_t)b * a.G + rk.g) * kD;
#pragma unroll
    for (int i = 0; i < 16; ++i) put(ps + 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3), acc_s[i]);
  }
  wait_all();
  arrive_rank(arrival_counter<kVar>(a, rk, b, kIsM ? kCntM : kCntKV), waves);
  lds_barrier();
  return bsel ^ 1;
}

// Store element e = 64 r + c of one statistics matrix (value v) as fp32 at
// fin[e] and in its MFMA fragment slot of frag: fragment (mb, q', lane, j)
// holds X[dimof(q' EPL + j, lane / 32)][32 mb + lane % 32].
template <class Tr>
__device__ __forceinline__ void store_stat(float* fin, void* frag, int e, float v) {
  const int r = e >> 6, c = e & 63;
  fin[e] = v;
  const int vs = 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3);
  const int ln = (c & 31) + 32 * ((r >> 2) & 1);
  const int idx = (((c >> 5) * Tr::NQ + vs / Tr::EPL) * 64 + ln) * Tr::EPL + vs % Tr::EPL;
  if constexpr (Tr::EPL == 8)
    __hip_atomic_store(static_cast<uint16_t*>(frag) + idx, f2bf(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    put(static_cast<float*>(frag) + idx, v);
}

// The C phase of slice b: elements [e0, e0 + E) of the flattened
// [phi(K)^T V | M], summed over the G staged partials in a fixed order.
// Elements go 256 at a time (one per consumer thread), which never straddle
// the two matrices, so the matrix choice stays wave-uniform.  With E < 256,
// TPE = 256 / E threads share an element (partials p = q, q + TPE, ...) and
// combine by a fixed xor tree.
template <class Tr, int kVar>
__device__ void consume_combine(const FlowArgs& a, const Rank& rk, int b, const unsigned char* buf, int ct,
                                int* waves) {
  using S = typename Tr::S;
  const float* stg = reinterpret_cast<const float*>(buf);  // [G][E]
  auto mat_base = [&](int f0, float*& fin, void*& frag) {
    const bool m = f0 >= kD * kD;
    fin = (m ? a.fin_m : a.fin_kv) + (size_t)b * (kD * kD);
    frag = static_cast<S*>(m ? a.frag_m : a.frag_kv) + (size_t)b * (kD * kD);
  };
  if constexpr (kVar == kVarSolo) {
    // One rank per slice (bf16): the staged partial is the statistics
    // themselves, [phi(K)^T V | M] row by row.  fp32 rows with 16-byte
    // stores; each fragment lane's eight bf16 (store_stat's layout) gathered
    // from LDS and written as four coherent words.  Values are formed as
    // 0 + x, as the sum over one partial elsewhere.
    for (int i = ct; i < 2 * kD * kD / 4; i += kRoleWaves * 64) {
      const int f = 4 * i;
      float* fin = (f < kD * kD ? a.fin_kv : a.fin_m) + (size_t)b * (kD * kD) + (f & (kD * kD - 1));
      const float4 x = *reinterpret_cast<const float4*>(stg + f);
      *reinterpret_cast<float4*>(fin) = make_float4(0.f + x.x, 0.f + x.y, 0.f + x.z, 0.f + x.w);
    }
    constexpr int kPieces = 2 * Tr::NQ * 64;  // per matrix: (mb, q, lane), eight elements each
    for (int pc = ct; pc < 2 * kPieces; pc += kRoleWaves * 64) {
      const int mat = pc / kPieces, rem = pc % kPieces;
      const int mb = rem / (Tr::NQ * 64), q = (rem / 64) % Tr::NQ, ln = rem % 64;
      const int c = 32 * mb + (ln & 31), h = ln >> 5;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        float x2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int vs = 8 * q + j + t;  // accumulator slot: row 32 (vs / 16) + 8 (vs / 4 % 4) + 4 h + vs % 4
          const int r = 32 * (vs >> 4) + 8 * ((vs >> 2) & 3) + 4 * h + (vs & 3);
          x2[t] = 0.f + stg[mat * (kD * kD) + r * kD + c];
        }
        w[j / 2] = pack_bf16x2(x2[0], x2[1]);
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<S*>(mat ? a.frag_m : a.frag_kv) + (size_t)b * (kD * kD)) +
                      (size_t)rem * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) put(dst + k, w[k]);
    }
  } else if (rk.E >= kRoleWaves * 64) {
    for (int e0 = 0; e0 < rk.E; e0 += kRoleWaves * 64) {
      float* fin;
      void* frag;
      mat_base(rk.e0 + e0, fin, frag);
      const int e = e0 + ct;
      float v = 0.f;
      for (int p = 0; p < a.G; ++p) v += stg[p * rk.E + e];
      store_stat<Tr>(fin, frag, (rk.e0 + e) & (kD * kD - 1), v);
    }
  } else {
    float* fin;
    void* frag;
    mat_base(rk.e0, fin, frag);
    const int tpe = kRoleWaves * 64 / rk.E;  // 2..8, consecutive lanes
    const int e = ct / tpe, q = ct % tpe;
    float v = 0.f;
    for (int p = q; p < a.G; p += tpe) v += stg[p * rk.E + e];
    for (int o = 1; o < tpe; o <<= 1) v += __shfl_xor(v, o);
    if (q == 0) store_stat<Tr>(fin, frag, (rk.e0 + e) & (kD * kD - 1), v);
  }
  wait_all();
  arrive_rank(arrival_counter<kVar>(a, rk, b, kCntC), waves);
  lds_barrier();
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
  // Valid slots: the token's neighbourhood, on the grid (window rows
  // gr0 .. gr0 + 5, columns gc0 .. gc0 + 9; wave-uniform).
  const int gr0 = r0 + 4 * br - 1, gc0 = c0 + 8 * bc - 1;
  unsigned valid = nbr;
  if (gr0 < 0 || gr0 + 6 > a.H || gc0 < 0 || gc0 + 10 > a.W) {
    unsigned rowbits = 0, colbits = 0;
#pragma unroll
    for (int wr = 0; wr < 6; ++wr) rowbits |= (unsigned)(gr0 + wr >= 0 && gr0 + wr < a.H) << wr;
#pragma unroll
    for (int wc = 0; wc < 10; ++wc) colbits |= (unsigned)(gc0 + wc >= 0 && gc0 + wc < a.W) << wc;
    valid &= grid_slots(rowbits, colbits, h);
  }
  // Invalid slots become -inf: bit v of `valid`, sign-extended, selects
  // between the logit's bits and those of -inf.
  float p[32];
  float mx = -1e30f;  // finite: a token off the grid may have no valid slot
#pragma unroll
  for (int v = 0; v < 32; ++v) {
    const unsigned keep = (unsigned)__builtin_amdgcn_sbfe((int)valid, v, 1);
    p[v] = __uint_as_float((__float_as_uint(lg[v >> 4][v & 15]) & keep) | (0xff800000u & ~keep));
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
  const float inv = scale * __builtin_amdgcn_rcpf(lden[0]);
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
// Consumer wave cw takes blocks cw, cw + 4, ..., one token per lane pair:
// lanes m and m + 32 hold 32 features each in accumulator layout, so the
// chain u_1 = phi(Q_i), u_k = u_(k-1) M and the projection z (phi(K)^T V),
// z = sum_k w_k(i) u_k, run on MFMA with no data movement.  u_1 comes from
// the token's Q operands of the local branch (re-paired across the lane
// pair), r_i from the tile's r region and `geo` holds the geometric walk
// weights, all in LDS.
// ---------------------------------------------------------------------------
template <class Tr, bool kMlp, bool kElu = false>
__device__ __forceinline__ void out_tile(const FlowArgs& a, int b, int t, const unsigned char* buf,
                                         const typename Tr::Frag (&fkv)[2][Tr::NQ],
                                         const typename Tr::Frag (&fm)[2][Tr::NQ], const float* geo,
                                         float alpha, unsigned nbr, int cw) {
  using S = typename Tr::S;
  constexpr bool kMfmaLocal = Tr::EPL == 8;
  const int lane = threadIdx.x & 63;
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
  const float* cR = reinterpret_cast<const float*>(buf + Lt.r);
  S* Yb = static_cast<S*>(a.Y) + (size_t)b * a.n * kD;
  const bool global = a.T >= 2;

  for (int blk = cw; blk < nblk; blk += kRoleWaves) {
    const int br = blk / CB, bc = blk % CB;
    if (r0 + 4 * br >= a.H || c0 + 8 * bc >= a.W) continue;  // no token of the block is on the grid
    const int tr = 4 * br + (n >> 3), tc = 8 * bc + (n & 7);
    const int slot = tr * a.TC + tc;
    const int row = r0 + tr, col = c0 + tc;
    const bool valid = row < a.H && col < a.W;
    const int i = valid ? row * a.W + col : 0;
    const int ccell = (tr + 1) * CW + (tc + 1);

    // This token's walk weights in LDS: its staged or predicted row, or the
    // geometric table.
    const float* wrow = (kMlp || a.weights) ? cW + slot * a.T : geo;
    const float w0 = wrow[0], w1 = a.T >= 2 ? wrow[1] : 0.f;

    // acc = (1 - alpha) L_i: the local branch; u1 = u_1 = phi(Q_i) in
    // accumulator slot order (bf16: as the bits of its B operands).
    float acc[32];
    using U1 = std::conditional_t<kMfmaLocal, v8s[4], float[32]>;
    U1 u1;
    if constexpr (kMfmaLocal) {
      bf16x8 qB[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qB[kb] = *reinterpret_cast<const bf16x8*>(cQ + row_off<BF16>(slot, 16 * kb + 8 * h));
      local_block_mfma(a, cK, cV, CW, r0, c0, br, bc, nbr, qB, 1.f - alpha, acc);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) u1[kb] = relu_to_slots<kElu>(__builtin_bit_cast(v8s, qB[kb]));
    } else {
      float q[32];
#pragma unroll
      for (int c = 0; c < 8; ++c) load4(reinterpret_cast<const S*>(cQ + row_off<Tr>(slot, dimof(4 * c, h))), &q[4 * c]);
      local_token_valu<Tr>(a, cK, cV, CW, ccell, row, col, q, 1.f - alpha, acc);
#pragma unroll
      for (int v = 0; v < 32; ++v) u1[v] = feat<kElu>(q[v]);
    }

    // + alpha w_0(i) V_i: the k = 0 term of the walk.
    {
      const float f = alpha * w0;
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
      float z[32], y[32];
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        if constexpr (kMfmaLocal)
          z[v] = w1 * __uint_as_float((uint32_t)(uint16_t)u1[v >> 3][v & 7] << 16);
        else
          z[v] = w1 * u1[v];
      }
      // u_k = u_(k-1) M, z += w_k u_k for k = 2 .. T-1.
      if (a.T >= 3) {
        float u[32];
        if constexpr (kMfmaLocal)
          apply_bits(fm, u1, u);
        else
          apply<Tr>(fm, u1, u);
        const float w2 = wrow[2];
#pragma unroll
        for (int v = 0; v < 32; ++v) z[v] += w2 * u[v];
        for (int k = 3; k < a.T; ++k) {
          apply<Tr>(fm, u, y);
          const float wk = wrow[k];
#pragma unroll
          for (int v = 0; v < 32; ++v) {
            u[v] = y[v];
            z[v] += wk * y[v];
          }
        }
      }
      apply<Tr>(fkv, z, y);
      const float f = alpha * cR[slot];
#pragma unroll
      for (int v = 0; v < 32; ++v) acc[v] += f * y[v];
    }

    if (valid) {
#pragma unroll
      for (int c = 0; c < 8; ++c) store4(Yb + (size_t)i * kD + dimof(4 * c, h), &acc[4 * c]);
    }
  }
}

// The OUT phase of slice b: take the slice statistics out of the statistics
// area (fragments into registers), free the area (barrier),
// then compute the rank's tiles, one stage each.  Returns the buffer index.
template <class Tr, bool kMlp, bool kElu = false>
__device__ int consume_out(const FlowArgs& a, const Rank& rk, int b, unsigned char* smem, int bsel,
                           const float* geo, int cw) {
  using Frag = typename Tr::Frag;
  using L = LdsOf<Tr>;
  const int lane = threadIdx.x & 63;
  const unsigned char* st = smem + 2 * L::kStage;
  Frag fkv[2][Tr::NQ], fm[2][Tr::NQ];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int q = 0; q < Tr::NQ; ++q) {
      const int off = ((mb * Tr::NQ + q) * 64 + lane) * (int)sizeof(Frag);
      fkv[mb][q] = *reinterpret_cast<const Frag*>(st + off);
      fm[mb][q] = *reinterpret_cast<const Frag*>(st + L::kFragBytes + off);  // unused unless T >= 3
    }
  const float alpha = a.alpha[b % a.heads];
  const int tok = lane & 31;
  const unsigned nbr = neighbour_slots(tok >> 3, tok & 7, lane >> 5);
  lds_barrier();  // the statistics area may now be refilled
  for (int k = 0; k < rk.nt; ++k) {
    out_tile<Tr, kMlp, kElu>(a, b, rk.t0 + k, smem + bsel * L::kStage, fkv, fm, geo, alpha, nbr, cw);
    lds_barrier();
    bsel ^= 1;
  }
  return bsel;
}

template <class Tr, bool kMlp, int kVar>
__global__ __launch_bounds__(kThreads) void flow_kernel(FlowArgs a) {
  using L = LdsOf<Tr>;
  extern __shared__ __align__(1024) unsigned char smem[];
  __shared__ __align__(16) float s_sl[4][kD];  // producers: s of each slice of the round (Z <= 4)
  __shared__ float geo_sh[kMaxT];        // geometric walk weights
  __shared__ int dep_ok;                 // tag of the stage whose dependency producer wave 0 has seen met
  __shared__ int last;                   // this workgroup's ticket, later: it finished last
  __shared__ int arrivals;               // consumer waves that have arrived in the current phase
  __shared__ int mlp_ready;              // producer waves that have met before predicting weights
  const int tid = threadIdx.x;
  const int wave = wave_id();
  const bool producer = wave < kRoleWaves;
  const int rw = producer ? wave : wave - kRoleWaves;  // wave index within the role
  unsigned char* st = smem + 2 * L::kStage;

  if (tid < kMaxT) geo_sh[tid] = a.geo[tid];
  if (tid == 0) {
    dep_ok = -1;
    arrivals = 0;
    mlp_ready = 0;
    last = (int)bump(a.tickets + (a.xcd_groups ? blockIdx.x % kXcds : 0));
  }
  __syncthreads();
  const Rank rk = make_rank(a, last, blockIdx.x % kXcds);
  // The roles run separate loops over the same stage sequence, with the same
  // barriers: one per stage, plus one at the start of each OUT phase.
  if (producer) {
    Pos p = first_pos(a, rk);
    if (p.ph != kPEnd) prepare<Tr, kMlp, kVar>(a, rk, p, smem, st, s_sl, &dep_ok, &mlp_ready, rw);
    lds_barrier();
    int bsel = 0;
    while (p.ph != kPEnd) {
      const Pos np = advance(a, rk, p);
      if (p.ph == kPOut && p.j == 0) lds_barrier();  // the consumers have taken the statistics
      if (np.ph != kPEnd)
        prepare<Tr, kMlp, kVar>(a, rk, np, smem + (bsel ^ 1) * L::kStage, st, s_sl, &dep_ok, &mlp_ready, rw);
      lds_barrier();
      bsel ^= 1;
      p = np;
    }
  } else {
    lds_barrier();
    int bsel = 0;
    if (rk.group >= 0) {
      // Phases are entered exactly when the producers' sequence has them.
      for (int r = 0; round_slices(a, rk, r) > 0; ++r) {
        const int nz = round_slices(a, rk, r);
        if (phase_len(a, rk, kPKV) > 0)
          for (int z = 0; z < nz; ++z)
            bsel = consume_sweep<Tr, false, kVar>(a, rk, slice_of(a, rk, r, z), smem, bsel, rw, &arrivals);
        if (phase_len(a, rk, kPM) > 0)
          for (int z = 0; z < nz; ++z)
            bsel = consume_sweep<Tr, true, kVar>(a, rk, slice_of(a, rk, r, z), smem, bsel, rw, &arrivals);
        if (phase_len(a, rk, kPC) > 0)
          for (int z = 0; z < nz; ++z) {
            consume_combine<Tr, kVar>(a, rk, slice_of(a, rk, r, z), smem + bsel * L::kStage, tid - kRoleWaves * 64,
                                &arrivals);
            bsel ^= 1;
          }
        if (phase_len(a, rk, kPOut) > 0)
          for (int z = 0; z < nz; ++z)
            bsel = consume_out<Tr, kMlp, kVar == kVarElu>(a, rk, slice_of(a, rk, r, z), smem, bsel, geo_sh, rw);
      }
    }
  }

  // The last workgroup to finish clears the arrival counters for the next
  // launch (every other workgroup's atomics have completed: each waited for
  // them before counting itself done).  The clears need no order among
  // themselves: the launch's end makes them visible to the next call.
  wait_all();
  __syncthreads();
  if (tid == 0) last = bump(a.done_cnt) == gridDim.x - 1;
  __syncthreads();
  if (last) {
    for (int i = tid; i < a.BH * kCntWords; i += kThreads)
      put(a.slice_cnt + (size_t)(i / kCntWords) * kCntStride + i % kCntWords, 0u);
    if constexpr (kVar == kVarGrouped)
      for (int i = tid; i < a.BH * 3 * kMaxSubs; i += kThreads) put(a.sub_cnt + (size_t)i * kCntStride, 0u);
    if (tid < kXcds) put(a.tickets + tid, 0u);
    if (a.clear_err && tid == 0) put(a.err, 0u);
    if (tid == 0) put(a.done_cnt, 0u);
  }
}

template <class Tr, bool kMlp, int kVar = kVarPlain>
hipError_t launch_typed(const FlowArgs& a, int grid, hipStream_t s) {
  constexpr int lds = LdsOf<Tr>::kTotal;
  static std::atomic<bool> lds_set[kMaxDevices];
  const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&flow_kernel<Tr, kMlp, kVar>), lds, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((flow_kernel<Tr, kMlp, kVar>), dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

// W1 [heads][hidden][2 d_h] rearranged per head as MlpRegs reads it: one
// thread per (head, hidden block, step, lane).
template <class Tr>
__global__ __launch_bounds__(256) void mlp_prep(const float* w1, float* out, int heads, int hidden) {
  constexpr bool kBf16 = Tr::EPL == 8;
  constexpr int kSteps = kBf16 ? 8 : 64;
  const int nhb = hidden / 32;
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id >= heads * nhb * kSteps * 64) return;
  const int lane = id % 64, st = (id / 64) % kSteps, hb = (id / (64 * kSteps)) % nhb;
  const int head = id / (64 * kSteps * nhb);
  const int m = lane % 32, h = lane / 32;
  float* blk = out + (size_t)head * mlp_head_floats(hidden, kBf16);
  const float* row = w1 + ((size_t)head * hidden + 32 * hb + m) * (2 * kD);
  if constexpr (kBf16) {
    const float4 lo4 = *reinterpret_cast<const float4*>(row + 16 * st + 8 * h);
    const float4 hi4 = *reinterpret_cast<const float4*>(row + 16 * st + 8 * h + 4);
    const float v[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[e];
    reinterpret_cast<bf16x8*>(blk)[((size_t)hb * 8 + st) * 64 + lane] = r;
  } else {
    blk[((size_t)hb * 64 + st) * 64 + lane] = row[2 * st + h];
  }
}

}  // namespace

hipError_t launch_flow(int dtype, const FlowArgs& a, int grid, hipStream_t s) {
  // The bf16 kernel's variants for many ranks per slice and for one, and the
  // ELU feature map's kernels, each a kernel of its own, so that the others
  // compile exactly as without them.
  if (a.variant == kVarGrouped) return launch_typed<BF16, false, kVarGrouped>(a, grid, s);
  if (a.variant == kVarSolo) return launch_typed<BF16, false, kVarSolo>(a, grid, s);
  if (a.variant == kVarElu)
    return dtype == 1 ? launch_typed<BF16, false, kVarElu>(a, grid, s) : launch_typed<F32, false, kVarElu>(a, grid, s);
  if (a.mlp_w1f) return dtype == 1 ? launch_typed<BF16, true>(a, grid, s) : launch_typed<F32, true>(a, grid, s);
  return dtype == 1 ? launch_typed<BF16, false>(a, grid, s) : launch_typed<F32, false>(a, grid, s);
}

size_t mlp_frag_bytes(int dtype, int heads, int hidden) {
  return (size_t)heads * mlp_head_floats(hidden, dtype == 1) * sizeof(float);
}

hipError_t launch_mlp_prep(int dtype, const float* w1, void* block, int heads, int hidden, hipStream_t s) {
  const dim3 grid((heads * (hidden / 32) * (dtype == 1 ? 8 : 64) * 64 + 255) / 256);
  float* out = static_cast<float*>(block);
  if (dtype == 1)
    hipLaunchKernelGGL(mlp_prep<BF16>, grid, dim3(256), 0, s, w1, out, heads, hidden);
  else
    hipLaunchKernelGGL(mlp_prep<F32>, grid, dim3(256), 0, s, w1, out, heads, hidden);
  return hipGetLastError();
}

}  // namespace lisa
