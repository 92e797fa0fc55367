// The LiSA forward pass on gfx950 with every rank's tile resident on chip.
//
// Method: reading note "LiSA:面向长程视觉建模的线性随机注意力" (arXiv:2611.04216v2),
// §2.1-§2.4.  Per (batch, head) slice with n tokens of width 64:
//   statistics (Eq. 8): s = sum_j phi(K_j), phi(K)^T V, M = phi(K)^T Qt with
//     Qt_j = r_j phi(Q_j), r_j = 1 / (phi(Q_j) . s + eps), phi = ReLU;
//   global branch: G_i = w_0(i) V_i + r_i sum_{k=1}^{T-1} w_k(i) (phi(Q_i) M^(k-1)) (phi(K)^T V);
//   local branch: L_i = softmax over the clipped 3x3 window of q_i . k_j / sqrt(d_h), times V;
//   Y_i = alpha G_i + (1 - alpha) L_i.
//
// Schedule (lisa_resident.hpp): the G ranks of a group cut each slice into G
// tiles.  A rank stages its tile's K and V cells (with a one-cell halo) in LDS
// and its tokens' Q in registers once, then, with no further input reads:
//   KV sweep over its tokens -> partial of s and phi(K)^T V, published;
//   local branch of its tokens and the walk's k = 0 term, kept in registers
//     (this runs while the other ranks' partials arrive);
//   after all KV partials: s, r_i, Qt rows written over the V cells, M sweep
//     over its tokens -> partial of M, published;
//   after all M partials: its share of the fixed-order sum of the partials
//     (statistics as fp32 and as MFMA fragments), published;
//   after all shares: the walk of its tokens on MFMA, Y written once (whole
//     rows per store instruction, nontemporally; for a one-head layer, after
//     the output projection applied to each block).
// All eight waves (two per SIMD, 256 registers each) do every step; waits
// on other ranks are polled by one wave while the others sit at the
// workgroup barrier.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lisa_device.hpp"
#include "lisa_kernels.hpp"
#include "lisa_resident.hpp"

namespace lisa {
namespace {

enum ResCounter { kRcKV = 0, kRcM = 1, kRcC = 2 };
constexpr int kFragBytes = kD * kD * 2;  // one 64 x 64 matrix as bf16 MFMA fragments

struct ResRank {
  int group, g;  // group (-1: idle workgroup), rank within the group (= tile of the slice)
};

// Ranks follow the workgroup index (res_rank_of).
__device__ __forceinline__ ResRank res_rank(const ResArgs& a) {
  ResRank r;
  res_rank_of(a.p.G, a.S, a.BH, (int)blockIdx.x, (int)gridDim.x, r.group, r.g);
  return r;
}

// One of two base pointers by a per-lane choice.  Both values are first
// pinned in scalar registers: left to itself the compiler selects between the
// two fields of the argument block and re-reads the pointer from memory, a
// full memory round trip, at every use.
// The result is rebuilt as a global-memory pointer, so that accesses through
// it stay global (not flat) instructions.
template <class P>
__device__ __forceinline__ P* pick(P* p0, P* p1, bool second) {
  uint64_t x0 = reinterpret_cast<uint64_t>(p0), x1 = reinterpret_cast<uint64_t>(p1);
  asm volatile("" : "+s"(x0), "+s"(x1));
  return (P*)reinterpret_cast<__attribute__((address_space(1))) P*>(second ? x1 : x0);
}

// An LDS pointer passed through an empty asm (so that nothing derived from
// it is hoisted), rebuilt as an LDS pointer: accesses through it stay LDS
// (not flat) instructions.
__device__ __forceinline__ const unsigned char* lds_launder(const unsigned char* p) {
  unsigned off = (unsigned)(uintptr_t)(lds_ptr_t)p;
  asm volatile("" : "+v"(off));
  return (const unsigned char*)reinterpret_cast<const __attribute__((address_space(3))) unsigned char*>(
      (uintptr_t)off);
}

// Row keys: k = 8 r + swz(r) for the bf16 row r of a staged region (128-byte
// rows, 16-byte pieces swizzled by row as everywhere in the library), so that
// element d of row r lies at byte ((k ^ (d / 8)) * 16 + (d % 8) * 2) of the
// region: one XOR and one shift-add per address.  The slot and window tables
// hold keys (16 bits: at most 8 K rows of 128 bytes per key unit).
__device__ __forceinline__ int res_key(int r) { return 8 * r + swz(r); }
__device__ __forceinline__ int res_at(int key, int d) { return ((key ^ (d >> 3)) << 4) + (d & 7) * 2; }

// Stage timeline (ResArgs::stamps): thread 0 of the workgroup, first slice only.
__device__ __forceinline__ void res_stamp(const ResArgs& a, bool first, int k) {
  if (a.stamps && first && threadIdx.x == 0)
    a.stamps[(size_t)blockIdx.x * kResPhases + k] = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ unsigned* res_counter(const ResArgs& a, int b, int g, int c) {
  if (a.grouped) return a.sub_cnt + (((size_t)b * 3 + c) * kMaxSubs + g / kSubRanks) * kCntStride;
  return a.slice_cnt + (size_t)b * kCntStride + c;
}

// This rank's arrival on counter c of slice b, once every wave's stores have
// completed (each wave waits for its own, then the workgroup meets).
__device__ void res_arrive(const ResArgs& a, int b, int g, int c) {
  wait_all();
  __syncthreads();
  if (threadIdx.x == 0) (void)bump(res_counter(a, b, g, c));
}

// Thread 0 counts its workgroup finished, in two levels: on its XCD's
// counter, and, for the XCD's last workgroup, on the device-wide one.  True
// for the last workgroup of the launch.  (One counter for all 256
// workgroups serialises their atomics: ~1.5 us before the last one returns.)
__device__ bool res_count_done(const ResArgs& a) {
  const int x = (int)(blockIdx.x % kXcds), grid = (int)gridDim.x;
  const unsigned on_xcd = (unsigned)((grid - x + kXcds - 1) / kXcds);
  if (bump(a.done_xcd + (size_t)x * kCntStride) != on_xcd - 1) return false;
  return bump(a.done_cnt) == (unsigned)min(grid, kXcds) - 1;
}

// Wait until all G ranks of slice b have arrived on counter c: wave 0 polls
// (lane k reads group k's counter when arrivals are counted per group of
// kSubRanks ranks), the other waves wait at the barrier.  Bounded like
// wait_for: giving up raises the error word.
__device__ void res_wait(const ResArgs& a, int b, int c) {
  if (threadIdx.x < 64) {
    if (a.grouped) {
      const int lane = threadIdx.x, ng = res_cdiv(a.p.G, kSubRanks), k = min(lane, ng - 1);
      const unsigned* cnt = a.sub_cnt + (((size_t)b * 3 + c) * kMaxSubs + k) * kCntStride;
      const unsigned target = (unsigned)min(kSubRanks, a.p.G - kSubRanks * k);
      unsigned spins = 0;
      for (;;) {
        const bool done = lane >= ng || get(cnt) >= target;
        if (__all(done)) break;
        __builtin_amdgcn_s_sleep(10);
        ++spins;
        if ((spins & 255u) == 0 && __builtin_amdgcn_readfirstlane(get(a.err))) break;
        if (spins > (1u << 21)) {
          if (lane == 0) put(a.err, 1u);
          break;
        }
      }
      asm volatile("" ::: "memory");
    } else if (threadIdx.x == 0) {
      wait_for(a.slice_cnt + (size_t)b * kCntStride + c, (unsigned)a.p.G, a.err);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Staging.
// ---------------------------------------------------------------------------
// DMA of one tensor's staged cells of tile t (staged row r = cell r of the
// SR x SC region, row-major) into swizzled 128-byte rows, 1 KB per wave
// instruction, waves taking runs in turn; the last run is padded with copies
// of the last cell.
__device__ void res_dma_cells(unsigned char* lds, const uint16_t* src, int W, const ResTile& t, int wave, int tid) {
  const int lane = tid & 63;
  const int nrow = t.SR * t.SC;
  const float inv_sc = 1.f / (float)t.SC;
  for (int base = wave * 64; base < nrow * 8; base += 64 * kResWaves) {
    const int P = base + lane;
    const int r = min(P >> 3, nrow - 1);
    const int g = ((P & 7) ^ swz(P >> 3)) & 7;  // the 16-byte piece this slot holds
    const int rr = div_small(r, inv_sc);
    const size_t tok = (size_t)(t.sr0 + rr) * W + (t.sc0 + (r - rr * t.SC));
    dma16(src + tok * kD + g * 8, lds_addr(lds + base * 16));
  }
}

// DMA of the per-token walk weights of the tile's slots ([slot][T] fp32),
// 4 bytes per lane; a masked slot takes the tile origin's row.
__device__ void res_dma_weights(unsigned char* lds, const float* wb, const ResPlan& p, const ResTile& t,
                                int wave, int tid) {
  const int lane = tid & 63;
  const int T = p.T, cnt = p.nblk * 32 * T;
  const float inv_t = 1.f / (float)T;
  for (int e0 = wave * 64; e0 < cnt; e0 += 64 * kResWaves) {
    const int e = min(e0 + lane, cnt - 1);
    const int s = div_small(e, inv_t);
    int tr, tc;
    const bool on = res_slot(p, t, s, tr, tc);
    const size_t tok = on ? (size_t)(t.r0 + tr) * p.W + (t.c0 + tc) : (size_t)t.r0 * p.W + t.c0;
    dma4(wb + tok * T + (e - s * T), lds_addr(lds + e0 * 4));
  }
}

// The row key of each slot's token's staged cell (the zero row for a masked slot).
__device__ void res_slot_table(uint16_t* tab, const ResPlan& p, const ResTile& t) {
  for (int s = threadIdx.x; s < p.nblk * 32; s += kResThreads) {
    int tr, tc;
    tab[s] = (uint16_t)res_key(res_slot(p, t, s, tr, tc) ? res_cell(t, t.r0 + tr, t.c0 + tc) : p.L.zrow);
  }
}

// The local branch's tables for tile t (the same for every slice): the row
// keys of each block's 6 x 10 window of staged cells (positions 60..63 repeat 59; a cell
// off the grid, or past the staged region, is clamped to a staged one and
// masked), each block's grid masks (the logit slots of lane half h whose cell
// lies on the grid), each lane's neighbour mask (the slots of its token's
// 3 x 3 neighbourhood) and each lane's one-hot B operands of the four 16-cell
// steps (1 at its token's own cell): against the V cells' A operands these
// give the token's own V row.
__device__ void res_local_tables(unsigned char* smem, const ResPlan& p, const ResTile& t) {
  unsigned char* loc = smem + p.L.loc;
  uint16_t* win = reinterpret_cast<uint16_t*>(loc + res_loc_win(p.nblk));
  uint32_t* msk = reinterpret_cast<uint32_t*>(loc + res_loc_mask(p.nblk));
  uint32_t* nbr = reinterpret_cast<uint32_t*>(loc + res_loc_nbr(p.nblk));
  v8s* hot = reinterpret_cast<v8s*>(loc + res_loc_hot(p.nblk));
  for (int i = threadIdx.x; i < p.nblk * 64; i += kResThreads) {
    const int blk = i >> 6, c = min(i & 63, 59), br = blk / p.BC, bc = blk % p.BC;
    win[i] = (uint16_t)res_key(res_cell(t, t.r0 + 4 * br - 1 + c / 10, t.c0 + 8 * bc - 1 + c % 10));
  }
  for (int i = threadIdx.x; i < p.nblk * 2; i += kResThreads) {
    const int blk = i >> 1, h = i & 1, br = blk / p.BC, bc = blk % p.BC;
    const int gr0 = t.r0 + 4 * br - 1, gc0 = t.c0 + 8 * bc - 1;
    unsigned rowbits = 0, colbits = 0;
    for (int wr = 0; wr < 6; ++wr) rowbits |= (unsigned)(gr0 + wr >= 0 && gr0 + wr < p.H) << wr;
    for (int wc = 0; wc < 10; ++wc) colbits |= (unsigned)(gc0 + wc >= 0 && gc0 + wc < p.W) << wc;
    msk[i] = grid_slots(rowbits, colbits, h);
  }
  if (threadIdx.x < 64) {
    const int n = threadIdx.x & 31, h = threadIdx.x >> 5;
    nbr[threadIdx.x] = neighbour_slots(n >> 3, n & 7, h);
  }
  for (int i = threadIdx.x; i < 4 * 64; i += kResThreads) {
    const int kb = i >> 6, n = i & 31, h = (i >> 5) & 1;
    const int own = (n / 8 + 1) * 10 + n % 8 + 1;  // the token's cell in its block's window
    v8s x = (v8s)0;
    for (int e = 0; e < 8; ++e)
      if (16 * kb + 8 * (e >> 2) + 4 * h + (e & 3) == own) x[e] = (short)0x3f80;  // bf16 1.0
    hot[i] = x;
  }
}

// ---------------------------------------------------------------------------
// Sweeps: contractions over the tile's token slots on MFMA.
// ---------------------------------------------------------------------------
// Operand bits of X[row(8h + e)][col0 + m], e = 0..7, for 16 slots whose
// staged rows lane (i, g) of the wave supplies (row keys ka for the first
// read, kb for the second); see rows_bits for the lane pattern of
// ds_read_b64_tr_b16.
__device__ __forceinline__ v8s rows_at(const unsigned char* base, int ka, int kb, int col) {
  return join(tr_read(base + res_at(ka, col)), tr_read(base + res_at(kb, col)));
}

// Steps [k0, k1) of 16 slots: acc += phi(K)^T X over the slots, X = the
// slots' V cells (KV sweep) or their rescaled Q rows (M sweep, by slot), and
// acc_s += phi(K)^T 1 when kWithS.  Wave output block (mb, nb) of 32 x 32.
// Steps go in batches of 4, then 2 (k1 - k0 is even): every operand
// read of a batch (slot-table rows first, then the transposed reads) is
// issued before its first MFMA, and even and odd steps accumulate into two
// chains that are added at the end.
template <bool kIsM, bool kWithS>
__device__ __forceinline__ void res_sweep(const unsigned char* smem, const ResLayout& L, int k0, int k1, int mb,
                                          int nb, f32x16& acc, f32x16& acc_s, int tid) {
  const int lane = tid & 63, i = lane & 15, g = lane >> 4;
  const int colA = 32 * mb + 16 * (g & 1) + 4 * (i & 3);
  const int colB = 32 * nb + 16 * (g & 1) + 4 * (i & 3);
  const uint16_t* tab = reinterpret_cast<const uint16_t*>(smem + L.tab);
  const unsigned char* bK = smem + L.k;
  const unsigned char* bX = smem + L.v;
  const bf16x8 ones = as_bf16((v8s)(short)0x3f80);  // bf16 1.0
  f32x16 acc2 = {}, acc_s2 = {};
  auto batch = [&](auto u_tag, int k) {
    constexpr int U = decltype(u_tag)::value;
    int ra[U], rb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s1 = 16 * (k + u) + 8 * (g >> 1) + (i >> 2);
      ra[u] = tab[s1];
      rb[u] = tab[s1 + 4];
    }
    v8s A[U], B[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s1 = 16 * (k + u) + 8 * (g >> 1) + (i >> 2);
      A[u] = __builtin_elementwise_max(rows_at(bK, ra[u], rb[u], colA), (v8s)0);  // ReLU on the bf16 bits
      B[u] = kIsM ? rows_at(bX, res_key(s1), res_key(s1 + 4), colB) : rows_at(bX, ra[u], rb[u], colB);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x16& c = (u & 1) ? acc2 : acc;
      c = mma(as_bf16(A[u]), as_bf16(B[u]), c);
      if constexpr (kWithS) {
        f32x16& cs = (u & 1) ? acc_s2 : acc_s;
        cs = mma(as_bf16(A[u]), ones, cs);
      }
    }
  };
  int k = k0;
  for (; k + 4 <= k1; k += 4) batch(std::integral_constant<int, 4>{}, k);
  if (k + 2 <= k1) batch(std::integral_constant<int, 2>{}, k);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[r] += acc2[r];
    acc_s[r] += acc_s2[r];
  }
}

// One sweep of the rank's slots and the publication of its partial:
// [phi(K)^T V or M] as fp32 rows, and s (KV sweep) as 64 fp32.  Waves w and
// w + 4 compute output block (w >> 1, w & 1) of the 64 x 64 result, over the
// first ceil(nblk / 2) blocks' slots and over the rest; the second wave
// leaves its products in the scratch area and the first adds them (first
// half + second half) and stores the block.  s comes from the waves of the
// first column block.
// arrive = false: the caller counts the arrival later (res_arrive), once it
// has other work done (the stores have then long completed).
template <bool kIsM>
__device__ void res_sweep_publish(const ResArgs& a, unsigned char* smem, int b, int g, int tid, bool arrive = true) {
  const ResLayout& L = a.p.L;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, m = lane & 31, h = lane >> 5;
  const int pw = wave & 3, half = wave >> 2;
  const int mb = pw >> 1, nb = pw & 1;
  const bool with_s = !kIsM && nb == 0;
  const int h0 = (a.p.nblk + 1) / 2;
  const int k0 = half ? 2 * h0 : 0, k1 = half ? 2 * a.p.nblk : 2 * h0;
  f32x16 acc = {}, acc_s = {};
  // The ones product (s) as a variant of its own: no branch among the MFMAs.
  if (with_s)
    res_sweep<kIsM, true>(smem, L, k0, k1, mb, nb, acc, acc_s, tid);
  else
    res_sweep<kIsM, false>(smem, L, k0, k1, mb, nb, acc, acc_s, tid);
  float* red = reinterpret_cast<float*>(smem + L.scr);  // [4][16][64], then s: [2][2][16]
  if (half) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(pw * 16 + i) * 64 + lane] = acc[i];
    if (with_s && m == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) red[4 * 16 * 64 + (mb * 2 + h) * 16 + i] = acc_s[i];
    }
  }
  lds_barrier();
  if (!kIsM) res_stamp(a, b < a.S, kResStampKVSweep);
  // One rank per slice (forward): the sum is the statistic itself, left as
  // fp32 rows in LDS for this rank's output and in the workspace for the
  // entry points that read it later; no partial, no arrival.
  const bool direct = a.p.G == 1 && a.mode == kResForward;
  if (!half) {
    // Every read of the second half's products is in flight before the first
    // add (left to itself the compiler sinks each read to its store, one LDS
    // round trip per element).
    float r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = red[(pw * 16 + i) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(r[i]));
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += r[i];
    if (direct) {
      float* dst = (kIsM ? a.fin_m : a.fin_kv) + (size_t)b * (kD * kD);
      float* st = reinterpret_cast<float*>(smem + L.st) + (kIsM ? kD * kD : 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = (32 * mb + 8 * (i >> 2) + 4 * h + (i & 3)) * kD + 32 * nb + m;
        put(dst + e, acc[i]);
        st[e] = acc[i];
      }
    } else {
      // The partial in accumulator order (res_part_index): this lane's four
      // consecutive elements of each row quartet are 16 contiguous bytes, and
      // a wave's stores cover whole 1 KB runs (4 stores per lane, not 16).
      float* dst = a.part_kv + ((size_t)b * a.p.G + g) * (2 * kD * kD) + (kIsM ? kD * kD : 0) +
                   (size_t)(mb * 2 + nb) * 1024 + lane * 4;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        put16(dst + t * 256, make_uint4(__float_as_uint(acc[4 * t]), __float_as_uint(acc[4 * t + 1]),
                                        __float_as_uint(acc[4 * t + 2]), __float_as_uint(acc[4 * t + 3])));
    }
    if (with_s && m == 0) {
      float* ps = direct ? a.fin_s + (size_t)b * kD : a.part_s + ((size_t)b * a.p.G + g) * kD;
      float* s_lds = reinterpret_cast<float*>(smem + L.s);
      float rs[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) rs[i] = red[4 * 16 * 64 + (mb * 2 + h) * 16 + i];
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(rs[i]));
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = acc_s[i] + rs[i];
      // Elements 32 mb + 8 t + 4 h + (0..3): four consecutive floats per t.
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = 32 * mb + 8 * t + 4 * h;
        put16(ps + e, make_uint4(__float_as_uint(v[4 * t]), __float_as_uint(v[4 * t + 1]),
                                 __float_as_uint(v[4 * t + 2]), __float_as_uint(v[4 * t + 3])));
        if (direct)
#pragma unroll
          for (int u = 0; u < 4; ++u) s_lds[e + u] = v[4 * t + u];
      }
    }
  }
  if (direct)
    lds_barrier();
  else if (arrive)
    res_arrive(a, b, g, kIsM ? kRcM : kRcKV);
}

// s = the fixed-order sum of the slice's G partials, into LDS.  The partials
// ([G][64] floats) are read as 16-byte pieces, every load in flight at once
// (a single round trip even at G = 256): load i of wave w takes pieces
// 64 (8 i + w) + lane, i.e. partial 4 (8 i + w) + lane / 16, elements
// 4 (lane % 16) + 0..3; coherent buffer loads (sc1; a piece past the
// partials reads as zero).  Each lane adds its loads in i order, then thread
// e < 64 adds the 32 (wave, lane / 16) sums of its element in a fixed order.
__device__ void res_sum_s(const ResArgs& a, unsigned char* smem, int b, int tid) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  constexpr int kLoads = kMaxRanks / 4 / kResWaves;  // loads per lane: 4 partials per wave instruction
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, G = a.p.G;
  float* sw = reinterpret_cast<float*>(smem + a.p.L.scr);  // [waves][64 lanes][4]
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(a.part_s + (size_t)b * G * kD, 0, G * kD * 4, 0x00020000);
  u32x4 x[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int piece = 64 * (kResWaves * i + wave) + lane;  // bytes 16 piece .. of the slice's partials
    x[i] = 16 * piece < G * kD * 4 ? __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * piece, 0, 16) : (u32x4)0u;
  }
  float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] += __uint_as_float(x[i][c]);
  *reinterpret_cast<float4*>(sw + 4 * (wave * 64 + lane)) = make_float4(t[0], t[1], t[2], t[3]);
  lds_barrier();
  if (tid < kD) {
    const int j = tid >> 2, c = tid & 3;
    float y[4 * kResWaves];
#pragma unroll
    for (int w = 0; w < kResWaves; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) y[4 * w + q] = sw[4 * (w * 64 + 16 * q + j) + c];
#pragma unroll
    for (int i = 0; i < 4 * kResWaves; ++i) asm volatile("" : "+v"(y[i]));
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 4 * kResWaves; ++i) v += y[i];
    reinterpret_cast<float*>(smem + a.p.L.s)[tid] = v;
  }
  lds_barrier();
}

// Store element e = 64 r + c of one statistics matrix as bf16 in its MFMA
// A-operand fragment slot of frag: fragment (mb, q, lane, j) holds
// X[dimof(8 q + j, lane / 32)][32 mb + lane % 32].
__device__ __forceinline__ void res_store_frag(uint16_t* frag, int e, float v) {
  const int r = e >> 6, c = e & 63;
  const int vs = 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3);
  const int ln = (c & 31) + 32 * ((r >> 2) & 1);
  const int idx = (((c >> 5) * 4 + vs / 8) * 64 + ln) * 8 + vs % 8;
  __hip_atomic_store(frag + idx, f2bf(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The rank partials of phi(K)^T V and M hold each 64 x 64 matrix in the
// sweeps' accumulator order: element (r, c), r = 32 mb + 8 t + 4 h + u,
// c = 32 nb + m, at ((2 mb + nb) 4 + t) 256 + (32 h + m) 4 + u.  The row-major
// index of partial element p:
__device__ __forceinline__ int res_part_row_major(int p) {
  const int blk = p >> 10, t = (p >> 8) & 3, ln = (p >> 2) & 63, u = p & 3;
  return (32 * (blk >> 1) + 8 * t + 4 * (ln >> 5) + u) * kD + 32 * (blk & 1) + (ln & 31);
}

// One element's total of the combine: the statistics as fp32 rows (which the
// backward and the entry points reading the statistics take) and in their
// bf16 fragment slot (which every rank's output loads).
__device__ __forceinline__ void res_combine_store(const ResArgs& a, int b, int e0, int e, float v) {
  const int f = e0 + e;
  const bool m = f >= kD * kD;
  const int x = res_part_row_major(f & (kD * kD - 1));
  put(pick(a.fin_kv, a.fin_m, m) + (size_t)b * (kD * kD) + x, v);
  res_store_frag(pick(static_cast<uint16_t*>(a.frag_kv), static_cast<uint16_t*>(a.frag_m), m) + (size_t)b * (kD * kD),
                 x, v);
}

// Rank g's share of the slice statistics: elements [e0, e1) of the flattened
// [phi(K)^T V | M] (nstat = 4096 or 8192 of them) summed over the G partials.
// The G partials' elements (G E <= nstat + G floats) are first staged in the
// K region (free after the sweeps) as [G][E] floats by coherent DMA, all in
// flight at once (a single round trip): 16 bytes per lane where E and e0 are
// multiples of four (a lane's four elements then lie in one partial), else
// 4 bytes.  Then the G partials of each element are added in an order fixed
// by G.
__device__ void res_combine(const ResArgs& a, unsigned char* smem, int b, int g, int nstat, int tid) {
  const int G = a.p.G;
  int e0, e1;
  res_combine_range(nstat, G, g, e0, e1);
  const int E = e1 - e0, total = G * E;
  float* stg = reinterpret_cast<float*>(smem + a.p.L.k);
  // q -> (partial p, element e) with p = floor(q / E): q < 8448 and E >= 16,
  // so (q + 1/2) / E in float stays well within 1/(2E) of the exact quotient.
  const float inv_e = 1.f / (float)E;
  const int wave = tid >> 6, lane = tid & 63;
  const float* part = a.part_kv + (size_t)b * G * (2 * kD * kD) + e0;
  if ((E & 3) == 0 && (e0 & 3) == 0) {
    // Runs of 256 floats; the last one is padded with copies of the last
    // four elements (G E is then a multiple of 256 at most 8448).
    for (int r = wave; 256 * r < total; r += kResWaves) {
      const int q = min(256 * r + 4 * lane, total - 4);
      const int pp = (int)(((float)q + 0.5f) * inv_e);
      dma16_coherent(part + (size_t)pp * (2 * kD * kD) + (q - pp * E), lds_addr(smem + a.p.L.k + 1024 * r));
    }
  } else {
    // Runs of 64 floats (G E rounds up to at most 8448).
    for (int r = wave; 64 * r < total; r += kResWaves) {
      const int q = min(64 * r + lane, total - 1);
      const int pp = (int)(((float)q + 0.5f) * inv_e);
      dma4_coherent(part + (size_t)pp * (2 * kD * kD) + (q - pp * E), lds_addr(smem + a.p.L.k + 256 * r));
    }
  }
  wait_all();
  __syncthreads();
  res_stamp(a, b < a.S, kResStampCStaged);
  // Consecutive threads take consecutive elements of one partial (no LDS
  // bank conflicts).  Fewer than kResThreads / 2 elements: ngrp groups of E
  // threads, group k adding partials k, k + ngrp, ... in turn; then thread e
  // adds the groups' sums in group order.  More: each thread adds all G
  // partials of its elements in turn.  Either way the order of additions
  // depends on G alone.
  if (2 * E > kResThreads) {
    // A share of whole 32 x 32 blocks (G <= 8; the partials are in
    // accumulator order) holds whole fragment pieces and whole row segments:
    // the totals go back into the staging (element e's first partial slot,
    // read by this thread only), then the pieces and the fp32 rows are
    // stored 16 bytes at a time.
    const bool whole = (E & 1023) == 0 && (e0 & 1023) == 0;
    for (int e = tid; e < E; e += kResThreads) {
      // Eight partials' reads in flight at a time (G <= 16 here), added in
      // partial order.
      float v = 0.f;
      for (int p0 = 0; p0 < G; p0 += 8) {
        float x[8];  // reads past the last partial repeat it and are not added
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = stg[min(p0 + k, G - 1) * E + e];
#pragma unroll
        for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(x[k]));
#pragma unroll
        for (int k = 0; k < 8; ++k) v += p0 + k < G ? x[k] : 0.f;
      }
      if (whole) {
        stg[e] = v;
      } else {
        res_combine_store(a, b, e0, e, v);
      }
    }
    if (whole) {
      lds_barrier();
      // Block lb of the share is the 32 x 32 block (mb, nb) = (blk / 2,
      // blk % 2), blk = beta % 4, of matrix beta / 4 (beta = e0 / 1024 + lb):
      // its totals sit at stg[1024 lb + 256 t + 4 lane + u] (row 32 mb + 8 t
      // + 4 (lane / 32) + u, column 32 nb + lane % 32).
      const int nbk = E / 1024;
      // Fragment pieces: the block holds steps q = 2 mb, 2 mb + 1 of fragment
      // half nb; piece (nb, q, lane) element j is row dimof(8 q + j, lane /
      // 32), i.e. t = 2 (q % 2) + j / 4, u = j % 4: two float4 of the staging.
      for (int pc = tid; pc < nbk * 128; pc += kResThreads) {
        const int lb = pc >> 7, beta = e0 / 1024 + lb, blk = beta & 3, qq = (pc >> 6) & 1, ln = pc & 63;
        const int q = 2 * (blk >> 1) + qq;
        const float4 lo = *reinterpret_cast<const float4*>(stg + 1024 * lb + 256 * (2 * qq) + 4 * ln);
        const float4 hi = *reinterpret_cast<const float4*>(stg + 1024 * lb + 256 * (2 * qq + 1) + 4 * ln);
        unsigned char* frag =
            pick(static_cast<unsigned char*>(a.frag_kv), static_cast<unsigned char*>(a.frag_m), beta >= 4) +
            (size_t)b * kFragBytes;
        put16(frag + (((blk & 1) * 4 + q) * 64 + ln) * 16,
              make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(hi.x, hi.y),
                         pack_bf16x2(hi.z, hi.w)));
      }
      // fp32 rows: row segment (rr, four columns from 4 cq) of the block.
      for (int sg = tid; sg < nbk * 256; sg += kResThreads) {
        const int lb = sg >> 8, beta = e0 / 1024 + lb, blk = beta & 3, rr = (sg >> 3) & 31, cq = sg & 7;
        const int t = rr >> 3, hh = (rr >> 2) & 1, u = rr & 3;
        float x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = stg[1024 * lb + 256 * t + 4 * (32 * hh + 4 * cq + k) + u];
        float* fin = pick(a.fin_kv, a.fin_m, beta >= 4) + (size_t)b * (kD * kD);
        put16(fin + (32 * (blk >> 1) + rr) * kD + 32 * (blk & 1) + 4 * cq,
              make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])));
      }
    }
  } else {
    const int ngrp = kResThreads / E, e = tid % E, pg = tid / E;
    float* sums = reinterpret_cast<float*>(smem + a.p.L.scr);  // [ngrp][E]
    if (pg < ngrp) {
      // Eight reads in flight at a time (about 16 partials per group).
      float v = 0.f;
      for (int p0 = pg; p0 < G; p0 += 8 * ngrp) {
        float x[8];  // reads past the last partial repeat it and are not added
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = stg[min(p0 + k * ngrp, G - 1) * E + e];
#pragma unroll
        for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(x[k]));
#pragma unroll
        for (int k = 0; k < 8; ++k) v += p0 + k * ngrp < G ? x[k] : 0.f;
      }
      sums[pg * E + e] = v;
    }
    lds_barrier();
    if (tid < E) {
      // ngrp <= kResThreads / 16 = 32 group sums, all read at once.
      float x[kResThreads / 16];  // reads past the last group repeat it and are not added
#pragma unroll
      for (int k = 0; k < kResThreads / 16; ++k) x[k] = sums[min(k, ngrp - 1) * E + tid];
#pragma unroll
      for (int k = 0; k < kResThreads / 16; ++k) asm volatile("" : "+v"(x[k]));
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < kResThreads / 16; ++k) v += k < ngrp ? x[k] : 0.f;
      res_combine_store(a, b, e0, tid, v);
    }
  }
  if (g == 0 && tid < kD) put(a.fin_s + (size_t)b * kD + tid, reinterpret_cast<const float*>(smem + a.p.L.s)[tid]);
  res_stamp(a, b < a.S, kResStampCSummed);
}

// The slice statistics' bf16 fragments (phi(K)^T V, then M when nmat = 2),
// as the combine wrote them, into the scratch area: coherent DMA, 1 KB per
// wave instruction, all in flight at once; no wait here.
__device__ void res_frags_dma(const ResArgs& a, unsigned char* frag, int b, int nmat, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  for (int m = 0; m < nmat; ++m) {
    const unsigned char* src = static_cast<const unsigned char*>(m ? a.frag_m : a.frag_kv) + (size_t)b * kFragBytes;
    for (int run = wave; run < kFragBytes / 1024; run += kResWaves)
      dma16_coherent(src + run * 1024 + lane * 16, lds_addr(frag + m * kFragBytes + run * 1024));
  }
}

// MFMA A-operand fragments (bf16, 8 KB) of a 64 x 64 matrix from its fp32
// rows in LDS: piece (mb, q, lane) holds X[dimof(8 q + j, lane / 32)][32 mb +
// lane % 32], j = 0..7, as 16 bytes.
__device__ void res_frags_from_rows(const float* st, unsigned char* frag, int tid) {
  uint4* dst = reinterpret_cast<uint4*>(frag);
  for (int pc = tid; pc < 512; pc += kResThreads) {
    const int mb = pc >> 8, q = (pc >> 6) & 3, ln = pc & 63;
    const int c = 32 * mb + (ln & 31), h = ln >> 5;
    float x[8];  // all eight reads in flight at once
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int vs = 8 * q + j;
      x[j] = st[(32 * (vs >> 4) + 8 * ((vs >> 2) & 3) + 4 * h + (vs & 3)) * kD + c];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(x[j]));
    dst[pc] = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                         pack_bf16x2(x[6], x[7]));
  }
}

// The folded output projection's operands, per slice: this thread's piece
// of the A-operand fragments of X = Wo^T (piece (mb, q, lane) holds
// X[dimof(8 q + j, lane / 32)][32 mb + lane % 32], j = 0..7, as above: two
// runs of four consecutive elements of row 32 mb + lane % 32 of Wo) and, for
// threads 0..15, four of the bias.  Loaded into registers, then stored into
// the K region (free in the output stage), fragments then bias.
struct ResProj {
  uint2 w[2];
  float4 b;
};
__device__ __forceinline__ ResProj res_proj_load(const ResArgs& a, int tid) {
  ResProj x;
  const int mb = tid >> 8, q = (tid >> 6) & 3, lane = tid & 63;
  const uint16_t* row = static_cast<const uint16_t*>(a.wo) + (32 * mb + (lane & 31)) * kD;
  x.w[0] = *reinterpret_cast<const uint2*>(row + dimof(8 * q, lane >> 5));
  x.w[1] = *reinterpret_cast<const uint2*>(row + dimof(8 * q + 4, lane >> 5));
  x.b = tid < 16 ? reinterpret_cast<const float4*>(a.bo)[tid] : make_float4(0.f, 0.f, 0.f, 0.f);
  return x;
}
__device__ __forceinline__ void res_proj_store(unsigned char* dst, const ResProj& x, int tid) {
  static_assert(kResThreads == 512, "one fragment piece per thread");
  reinterpret_cast<uint4*>(dst)[tid] = make_uint4(x.w[0].x, x.w[0].y, x.w[1].x, x.w[1].y);
  if (tid < 16) reinterpret_cast<float4*>(dst + kFragBytes)[tid] = x.b;
}

// ---------------------------------------------------------------------------
// Local branch and output (per 4 x 8 block; one token per lane pair, 32
// features per lane in accumulator layout).
// ---------------------------------------------------------------------------
// Local branch of block blk on MFMA, and the walk's k = 0 term:
// Lm = scale L + f V_i.  Logits C[cell][token] = K_win Q_blk^T over the
// block's 6 x 10 window of cells (60, padded to 64; the cells from the
// window table), masked softmax (grid and neighbour masks from their tables),
// then L^T = V_win^T P^T with the probabilities as the B operand and V from
// transposed LDS reads; the denominator is the same product against an
// all-ones operand, and V_i the same product against the one-hot operands.
__device__ void res_local(const ResArgs& a, const unsigned char* smem, int blk, const bf16x8 (&qB)[4], float scale,
                          float f, float (&Lm)[32], int tid) {
  const ResPlan& p = a.p;
  const int lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int i16 = lane & 15, g = lane >> 4;
  const unsigned char* cK = smem + p.L.k;
  const unsigned char* cV = smem + p.L.v;
  const unsigned char* loc = smem + p.L.loc;
  const uint16_t* win = reinterpret_cast<const uint16_t*>(loc + res_loc_win(p.nblk)) + blk * 64;
  const unsigned valid = reinterpret_cast<const uint32_t*>(loc + res_loc_nbr(p.nblk))[lane] &
                         reinterpret_cast<const uint32_t*>(loc + res_loc_mask(p.nblk))[blk * 2 + h];
  const bf16x8* hot = reinterpret_cast<const bf16x8*>(loc + res_loc_hot(p.nblk)) + lane;
  f32x16 lg[2] = {};
  const int sc0 = win[n], sc1 = win[32 + n];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(cK + res_at(sc0, 16 * kb + 8 * h));
    const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(cK + res_at(sc1, 16 * kb + 8 * h));
    lg[0] = mma(A0, qB[kb], lg[0]);
    lg[1] = mma(A1, qB[kb], lg[1]);
  }
  float pr[32];
  float mx = -1e30f;  // finite: a masked token may have no valid slot
#pragma unroll
  for (int v = 0; v < 32; ++v) {
    const unsigned keep = (unsigned)__builtin_amdgcn_sbfe((int)valid, v, 1);
    pr[v] = __uint_as_float((__float_as_uint(lg[v >> 4][v & 15]) & keep) | (0xff800000u & ~keep));
    mx = fmaxf(mx, pr[v]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float off = -mx * a.logit_scale;  // exp2((l - max) log2(e) / sqrt(d_h)); exp2(-inf) = 0
  bf16x8 Bp[4];
#pragma unroll
  for (int v = 0; v < 32; ++v)
    Bp[v >> 3][v & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(pr[v], a.logit_scale, off));
  f32x16 la[2] = {}, lv[2] = {}, lden = {};
  const bf16x8 ones = as_bf16((v8s)(short)0x3f80);
  // The window cells and one-hot operands of the four steps, read together.
  int cAB[8];
  v8s hbs[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    cAB[2 * kb] = win[16 * kb + 4 * (g >> 1) + (i16 >> 2)];
    cAB[2 * kb + 1] = win[16 * kb + 8 + 4 * (g >> 1) + (i16 >> 2)];
    hbs[kb] = __builtin_bit_cast(v8s, hot[kb * 64]);
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) asm volatile("" : "+v"(cAB[2 * kb]), "+v"(cAB[2 * kb + 1]), "+v"(hbs[kb]));
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    lden = mma(ones, Bp[kb], lden);
    const int cA = cAB[2 * kb], cB = cAB[2 * kb + 1];
    const bf16x8 hb = as_bf16(hbs[kb]);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int d = 32 * db + 16 * (g & 1) + 4 * (i16 & 3);
      const bf16x8 A = as_bf16(join(tr_read(cV + res_at(cA, d)), tr_read(cV + res_at(cB, d))));
      la[db] = mma(A, Bp[kb], la[db]);
      lv[db] = mma(A, hb, lv[db]);
    }
  }
  const float inv = scale * __builtin_amdgcn_rcpf(lden[0]);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    Lm[v] = __builtin_fmaf(f, lv[0][v], la[0][v] * inv);
    Lm[16 + v] = __builtin_fmaf(f, lv[1][v], la[1][v] * inv);
  }
}

// The walk-weight predictor for one 32-slot block (forward with the
// predictor): w = softmax(W2 ReLU(W1 concat(q, k) + b1) + b2) per token [the
// predictor of note §2.4 Eq. 10], from the slots' raw Q (qB, the B operands
// of the local branch's logits) and the K row of each token's own cell.  The
// first layer runs on MFMA 32 hidden units at a time as W1 x^T, W1 in the
// bf16 fragment order mlp_prep lays out per head; element i of lane (n, h)
// of its accumulator is hidden unit 32 hb + 8 (i / 4) + i % 4 + 4 h of token
// n, so lane halves are the two contraction slots of an fp32 MFMA 32x32x2
// and the second layer is 16 of those (A = W2, rows past T zero), whose
// element e of lane (n, h) is logit 4 h + e of token n.  The weights go to
// the slots' entries [slot][T] of the weight region.
__device__ void res_predict(const ResArgs& a, const unsigned char* cK, int slot, int cell, const bf16x8 (&qB)[4],
                            int head, float* wts, int tid) {
  const int lane = tid & 63, m = lane & 31, h = lane >> 5;
  const int T = a.p.T, hidden = a.hidden, nhb = hidden / 32;
  const bf16x8* w1 = reinterpret_cast<const bf16x8*>(static_cast<const float*>(a.mlp_w1f) +
                                                     (size_t)head * mlp_head_floats(hidden, true));
  bf16x8 xk[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) xk[kb] = *reinterpret_cast<const bf16x8*>(cK + row_off<BF16>(cell, 16 * kb + 8 * h));
  f32x16 lg = {};
#pragma unroll 1
  for (int hb = 0; hb < nhb; ++hb) {
    bf16x8 fh[8];
    float w2[16], b1[16];
#pragma unroll
    for (int st = 0; st < 8; ++st) fh[st] = w1[((size_t)hb * 8 + st) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = 32 * hb + 8 * (i / 4) + i % 4 + 4 * h;  // hidden unit of slot h, element i
      w2[i] = m < T ? a.mlp_w2[((size_t)head * T + m) * hidden + j] : 0.f;
      b1[i] = a.mlp_b1[(size_t)head * hidden + j];
    }
    f32x16 c = {};
#pragma unroll
    for (int st = 0; st < 4; ++st) c = mma(fh[st], qB[st], c);
#pragma unroll
    for (int st = 0; st < 4; ++st) c = mma(fh[4 + st], xk[st], c);
#pragma unroll
    for (int i = 0; i < 16; ++i) lg = mma(w2[i], fmaxf(c[i] + b1[i], 0.f), lg);
  }
  float v[4], b2[4], mx = -INFINITY;
  // b2 read unconditionally (a clamped index): a load under a branch is
  // waited for inside it, one round trip per load.
#pragma unroll
  for (int e = 0; e < 4; ++e) b2[e] = a.mlp_b2[head * T + min(4 * h + e, T - 1)];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k = 4 * h + e;
    v[e] = k < T ? lg[e] + b2[e] : 0.f;
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
    if (4 * h + e < T) wts[slot * T + 4 * h + e] = v[e] * inv;
}

// y += x X for X given as A-operand fragments in LDS (frag: (mb, q, lane) ->
// 16 bytes), x as the bits of its B operands (slot order), y in accumulator
// layout.
__device__ __forceinline__ void res_apply_bits(const unsigned char* frag, const v8s (&x)[4], float (&y)[32], int tid) {
  const int lane = tid & 63;
  // The fragment reads stay inside each product: hoisted out of the
  // per-block and per-term loops, the 16 operands would hold 64 registers.
  frag = lds_launder(frag);
  f32x16 c0, c1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    c0[i] = y[i];
    c1[i] = y[16 + i];
  }
  // All eight fragment reads in flight before the first product (one LDS
  // round trip, not one per product).
  v8s fa[2][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) fa[mb][q] = *reinterpret_cast<const v8s*>(frag + ((mb * 4 + q) * 64 + lane) * 16);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) asm volatile("" : "+v"(fa[mb][q]));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x8 bx = as_bf16(x[q]);
    c0 = mma(as_bf16(fa[0][q]), bx, c0);
    c1 = mma(as_bf16(fa[1][q]), bx, c1);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    y[i] = c0[i];
    y[16 + i] = c1[i];
  }
}
// The same for x in accumulator layout as fp32 (rounded to bf16 here).
__device__ __forceinline__ void res_apply(const unsigned char* frag, const float (&x)[32], float (&y)[32], int tid) {
  v8s b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) b[q] = __builtin_bit_cast(v8s, operand(x, q, BF16{}));
  res_apply_bits(frag, b, y, tid);
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
// One instantiation per mode (kResForward, kResReduce, kResApply) and
// predictor use: each carries only the code its calls run, which keeps the
// forward's code within the instruction cache a CU pair shares.
template <int kMode, bool kMlp, bool kProj>
__global__ __launch_bounds__(kResThreads) void resident_kernel(ResArgs a) {
  extern __shared__ __align__(1024) unsigned char smem[];
  __shared__ float geo[kMaxT];  // geometric walk weights
  const ResPlan& p = a.p;
  const ResLayout& L = p.L;
  const int tid0 = threadIdx.x;

  if (tid0 < kMaxT) geo[tid0] = a.geo[tid0];
  __syncthreads();
  const ResRank rk = res_rank(a);
  res_stamp(a, true, kResStampStart);
  if (a.stamps && tid0 == 0)
    a.stamps[(size_t)blockIdx.x * kResPhases + kResPhases - 1] = ((unsigned long long)(unsigned)rk.group << 32) | (unsigned)rk.g;
  constexpr bool fwd = kMode != kResReduce;  // local branch and output
  constexpr bool stats = kMode != kResApply;  // sweeps and combine

  // The workgroup counts itself done (done_cnt) once it has made its last
  // counter access, not at its end: after its last slice's C wait when it
  // takes part in hand-offs, else during its first staging (an idle
  // workgroup at once).  The atomic's round trip then overlaps a load it
  // waits for anyway, and the workgroup's end waits for nothing.
  __shared__ unsigned done_sh;
  const bool has_slice = rk.group >= 0 && rk.group < a.BH;
  const bool count_late = has_slice && stats && a.do_kv && p.G > 1;
  if (!has_slice && tid0 == 0) done_sh = res_count_done(a);

  if (rk.group >= 0) {
    res_slot_table(reinterpret_cast<uint16_t*>(smem + L.tab), p, res_tile(p, rk.g));
    if (fwd) res_local_tables(smem, p, res_tile(p, rk.g));
    constexpr int kNB = kResMaxBlocks / kResWaves;
    const int nstat = a.do_m ? 2 * kD * kD : kD * kD;
    // One rank per slice, forward: the sweeps leave the statistics in place.
    const bool direct = p.G == 1 && kMode == kResForward;

    for (int b = rk.group; b < a.BH; b += a.S) {
      // The tile is the same for every slice, but what depends on it per lane
      // (window cells, masks, token indices, operand offsets) is cheap to
      // recompute and would otherwise be held in registers across the whole
      // loop: the thread and rank indices are passed through an empty asm so
      // that nothing derived from them is hoisted out of the loop.
      int tid = tid0, gi = rk.g;
      asm volatile("" : "+v"(tid), "+s"(gi));
      const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 31, h = lane >> 5;
      // This wave's blocks: wave + 8 j, j < nown.
      const int nown = min(kNB, (p.nblk - wave + kResWaves - 1) / kResWaves);
      const ResTile t = res_tile(p, gi);
      const bool first = b == rk.group;
      const size_t base = (size_t)b * a.n;
      const uint16_t* Qb = static_cast<const uint16_t*>(a.Q) + base * kD;
      const uint16_t* Kb = static_cast<const uint16_t*>(a.K) + base * kD;
      const uint16_t* Vb = static_cast<const uint16_t*>(a.V) + base * kD;
      const float alpha = fwd ? a.alpha[b % a.heads] : 0.f;
      __syncthreads();  // the previous slice's readers of every region are done
      // Zero rows (masked slots read them in the sweeps).
      if (tid < 16) {
        reinterpret_cast<uint4*>(smem + L.k + L.zrow * kResRowBytes)[tid & 7] = make_uint4(0, 0, 0, 0);
        reinterpret_cast<uint4*>(smem + L.v + L.zrow * kResRowBytes)[tid & 7] = make_uint4(0, 0, 0, 0);
      }
      // Stage: K and V cells, the weights; Q of this wave's blocks into registers.
      res_dma_cells(smem + L.k, Kb, p.W, t, wave, tid);
      res_dma_cells(smem + L.v, Vb, p.W, t, wave, tid);
      if (fwd && a.per_token && a.weights) res_dma_weights(smem + L.w, a.weights + base * p.T, p, t, wave, tid);
      // Blocks go in pairs (two independent chains for the scheduler to
      // interleave); when the wave has an odd number of blocks, the last
      // pair's second block repeats the first: computed, never stored.
      bf16x8 qB[kNB][4];
      int slot[kNB], blkid[kNB];
      bool valid[kNB];
#pragma unroll
      for (int j = 0; j < kNB; ++j) {
        const int jj = (j < nown || (j & 1) == 0) ? j : j - 1;
        blkid[j] = wave + kResWaves * jj;
        slot[j] = blkid[j] * 32 + n;
        int tr = 0, tc = 0;
        const bool on = blkid[j] < p.nblk && res_slot(p, t, slot[j], tr, tc);
        valid[j] = j < nown && on;
        const size_t tok = on ? (size_t)(t.r0 + tr) * p.W + (t.c0 + tc) : (size_t)t.r0 * p.W + t.c0;
        if ((j & ~1) < nown) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            qB[j][kb] = *reinterpret_cast<const bf16x8*>(Qb + tok * kD + 16 * kb + 8 * h);
        }
      }
      if (!count_late && first && tid == 0) done_sh = res_count_done(a);
      wait_all();
      __syncthreads();
      res_stamp(a, first, kResStampStaged);

      // KV sweep: partials of s and phi(K)^T V.
      // With a local branch to run and arrivals on one counter per slice,
      // the KV partial's arrival is counted after it: the publication then
      // does not wait for its stores to complete before the local branch, and
      // the arrival costs no wait (PVT-T stage 1 37.1 -> 36.8 us).  With
      // arrivals counted per group (64 ranks and more, one sequence) the later
      // arrivals cost more than the wait (200 x 320: 36.3 -> 37.7 us).
      const bool defer_kv = fwd && p.G > 1 && !a.grouped;
      if (stats && a.do_kv) res_sweep_publish<false>(a, smem, b, rk.g, tid, !defer_kv);
      res_stamp(a, first, kResStampKV);

      // The predicted walk weights of this wave's slots (each wave reads only
      // its own slots' weights; LDS accesses of a wave complete in order).
      float* wts = reinterpret_cast<float*>(smem + L.w);
      if (fwd && kMlp) {
        const int head = __builtin_amdgcn_readfirstlane(b % a.heads);
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
          if (j < nown) {
            int sl = slot[j], tr, tc;
            asm volatile("" : "+v"(sl));
            const bool on = res_slot(p, t, sl, tr, tc);
            const int cell = on ? res_cell(t, t.r0 + tr, t.c0 + tc) : 0;
            res_predict(a, smem + L.k, slot[j], cell, qB[j], head, wts, tid);
          }
        }
      }

      // Local branch and the walk's k = 0 term: Lm = (1 - alpha) L_i + alpha w_0(i) V_i.
      float Lm[kNB][32];
      if (fwd) {
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
          if (j < nown) {
            const float w0 = a.per_token ? wts[slot[j] * p.T] : geo[0];
            res_local(a, smem, blkid[j], qB[j], 1.f - alpha, alpha * w0, Lm[j], tid);
          }
        }
      }
      if (stats && a.do_kv && defer_kv) res_arrive(a, b, rk.g, kRcKV);

      // s, then the rows Qt_i = r_i phi(Q_i) of this wave's slots over the V
      // cells (the local branch is done: the wait closed with a workgroup
      // barrier), zero for masked slots.  They are the B operand of the M
      // sweep and, rounded to bf16 like every operand the method derives, the
      // walk's u_1 in the output.
      res_stamp(a, first, kResStampLocal);
      const bool global = p.T >= 2;
      unsigned char* qt = smem + L.v;
      if (global || (stats && a.do_m)) {
        float* s_lds = reinterpret_cast<float*>(smem + L.s);
        if (stats) {
          // The wait (or barrier) also orders every wave's local branch,
          // which reads the V cells, before the Qt rows overwrite them.
          // (One rank, forward: the KV sweep left s in LDS.)
          if (p.G > 1)
            res_wait(a, b, kRcKV);
          else
            lds_barrier();
          if (!direct) res_sum_s(a, smem, b, tid);
          res_stamp(a, first, kResStampS);
        } else {
          __syncthreads();
          if (tid < kD) s_lds[tid] = get(a.fin_s + (size_t)b * kD + tid);
          __syncthreads();
        }
        // This lane's half of s, read once for the wave's blocks, every read
        // in flight before the first product.
        float sv[32];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 8; ++e) sv[8 * kb + e] = s_lds[16 * kb + 8 * h + e];
#pragma unroll
        for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(sv[i]));
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
          if (j < nown) {
            v8s x[4];
            float dot = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              x[kb] = __builtin_elementwise_max(__builtin_bit_cast(v8s, qB[j][kb]), (v8s)0);
#pragma unroll
              for (int e = 0; e < 8; ++e) dot += bf2f((uint16_t)x[kb][e]) * sv[8 * kb + e];
            }
            dot += __shfl_xor(dot, 32);
            const float sc = valid[j] ? __builtin_amdgcn_rcpf(dot + a.eps) : 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              uint32_t o[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                o[e] = pack_bf16x2(bf2f((uint16_t)x[kb][2 * e]) * sc, bf2f((uint16_t)x[kb][2 * e + 1]) * sc);
              *reinterpret_cast<uint4*>(qt + row_off<BF16>(slot[j], 16 * kb + 8 * h)) =
                  make_uint4(o[0], o[1], o[2], o[3]);
            }
          }
        }
        lds_barrier();
      }

      if (stats && a.do_m) res_sweep_publish<true>(a, smem, b, rk.g, tid);
      res_stamp(a, first, kResStampM);

      if (stats && a.do_kv && !direct) {
        if (p.G > 1) res_wait(a, b, a.do_m ? kRcM : kRcKV);
        res_stamp(a, first, kResStampMWait);
        res_combine(a, smem, b, rk.g, nstat, tid);
        res_stamp(a, first, kResStampComb);
        if (p.G > 1) {
          res_arrive(a, b, rk.g, kRcC);
          res_wait(a, b, kRcC);
          res_stamp(a, first, kResStampCWait);
          // The last counter access of the workgroup; with an output, the
          // count goes out with the fragments' DMA below.
          if (b + a.S >= a.BH && !(fwd && global) && tid == 0) done_sh = res_count_done(a);
        } else {
          lds_barrier();  // the totals, in LDS; their global copies complete by the launch's end
        }
      }

      if (fwd) {
        // The folded projection's operands: loads issued here, stored into
        // the K region with the statistics' fragments below.
        ResProj proj{};
        if constexpr (kProj) proj = res_proj_load(a, tid);
        if (global) {
          // The statistics (phi(K)^T V, then M) as bf16 fragments in the
          // scratch area: built from the fp32 rows the sweeps left in LDS
          // (one rank, forward), else loaded as the combine wrote them.
          if (direct) {
            const float* rows = reinterpret_cast<const float*>(smem + L.st);
            res_frags_from_rows(rows, smem + L.scr, tid);
            if (p.T >= 3) res_frags_from_rows(rows + kD * kD, smem + L.scr + kFragBytes, tid);
            if constexpr (kProj) res_proj_store(smem + L.k, proj, tid);
            lds_barrier();
          } else {
            res_frags_dma(a, smem + L.scr, b, p.T >= 3 ? 2 : 1, tid);
            if (count_late && b + a.S >= a.BH && tid == 0) done_sh = res_count_done(a);
            wait_all();
            if constexpr (kProj) res_proj_store(smem + L.k, proj, tid);
            __syncthreads();
          }
        } else if constexpr (kProj) {
          res_proj_store(smem + L.k, proj, tid);
          __syncthreads();
        }
        res_stamp(a, first, kResStampFrags);
        const unsigned char* fkv = smem + L.scr;
        const unsigned char* fm = smem + L.scr + kFragBytes;
        uint16_t* Yb = static_cast<uint16_t*>(a.Y) + base * kD;
        // One block at a time: u_1 = Qt_i from its staged row, in
        // accumulator slot order; u_k = u_(k-1) M, z = sum_k w_k(i) u_k; then
        // Lm += (alpha z) phi(K)^T V, and the block's Y is stored.
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
          if (j < nown) {
            if (global) {
              const float* wrow = a.per_token ? wts + slot[j] * p.T : geo;
              // The row and the weights w_1, w_2 read together (one LDS round
              // trip for the block).
              v8s u1[4];
#pragma unroll
              for (int kb = 0; kb < 4; ++kb) u1[kb] = *reinterpret_cast<const v8s*>(qt + row_off<BF16>(slot[j], 16 * kb + 8 * h));
              float w12[2] = {wrow[1], p.T >= 3 ? wrow[2] : 0.f};
#pragma unroll
              for (int kb = 0; kb < 4; ++kb) asm volatile("" : "+v"(u1[kb]));
              asm volatile("" : "+v"(w12[0]), "+v"(w12[1]));
#pragma unroll
              for (int kb = 0; kb < 4; ++kb) u1[kb] = relu_to_slots(u1[kb]);
              // alpha rides on the walk weights: z = sum_k (alpha w_k(i)) u_k.
              float z[32];
              const float w1 = alpha * w12[0];
#pragma unroll
              for (int v = 0; v < 32; ++v) z[v] = w1 * bf2f((uint16_t)u1[v >> 3][v & 7]);
              if (p.T >= 3) {
                float u[32];
#pragma unroll
                for (int v = 0; v < 32; ++v) u[v] = 0.f;
                res_apply_bits(fm, u1, u, tid);
                const float w2 = alpha * w12[1];
#pragma unroll
                for (int v = 0; v < 32; ++v) z[v] += w2 * u[v];
                for (int k = 3; k < p.T; ++k) {
                  float y[32];
#pragma unroll
                  for (int v = 0; v < 32; ++v) y[v] = 0.f;
                  res_apply(fm, u, y, tid);
                  const float wk = alpha * wrow[k];
#pragma unroll
                  for (int v = 0; v < 32; ++v) {
                    u[v] = y[v];
                    z[v] += wk * y[v];
                  }
                }
              }
              res_apply(fkv, z, Lm[j], tid);
            }
            if constexpr (kProj) {
              // Y = O Wo^T + bo: the bias into the accumulators, then the
              // product with O (rounded to bf16 as its operand).
              const float* bias = reinterpret_cast<const float*>(smem + L.k + kFragBytes);
              float yo[32];
#pragma unroll
              for (int c = 0; c < 8; ++c) {
                const float4 bq = *reinterpret_cast<const float4*>(bias + dimof(4 * c, h));
                yo[4 * c] = bq.x;
                yo[4 * c + 1] = bq.y;
                yo[4 * c + 2] = bq.z;
                yo[4 * c + 3] = bq.w;
              }
              res_apply(smem + L.k, Lm[j], yo, tid);
#pragma unroll
              for (int v = 0; v < 32; ++v) Lm[j][v] = yo[v];
            }
            if (global) {
              // Y through the block's own slot rows of the Qt region (its u_1
              // was read from them at the block's start; no other wave reads
              // them): written as bf16 rows, then read back so that each
              // store instruction writes one block row, 8 tokens x 128
              // contiguous bytes, as whole lines, nontemporally (Y is not
              // read again here; dirty lines would be written back at the
              // kernel's end, on the next kernel's time).
#pragma unroll
              for (int c = 0; c < 8; ++c)
                *reinterpret_cast<uint2*>(qt + row_off<BF16>(slot[j], dimof(4 * c, h))) =
                    make_uint2(pack_bf16x2(Lm[j][4 * c], Lm[j][4 * c + 1]), pack_bf16x2(Lm[j][4 * c + 2], Lm[j][4 * c + 3]));
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's rows are written
              // The block's first token row and column (one division per
              // block, on the wave-uniform block index); block row r, token
              // column lane / 8.
              int tr0, tc0;
              res_slot(p, t, __builtin_amdgcn_readfirstlane(blkid[j]) * 32, tr0, tc0);
              const int pc = lane & 7, tc = tc0 + (lane >> 3);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int sl = blkid[j] * 32 + 8 * r + (lane >> 3), tr = tr0 + r;
                const u32x4 v = *reinterpret_cast<const u32x4*>(qt + row_off<BF16>(sl, 8 * pc));
                if (tr < t.th && tc < t.tw)
                  __builtin_nontemporal_store(
                      v, reinterpret_cast<u32x4*>(Yb + ((size_t)(t.r0 + tr) * p.W + (t.c0 + tc)) * kD + 8 * pc));
              }
            } else if (valid[j]) {
              // The token index recomputed here (not kept from the Q loads).
              int sl = slot[j], tr, tc;
              asm volatile("" : "+v"(sl));
              res_slot(p, t, sl, tr, tc);
              const size_t tok = (size_t)(t.r0 + tr) * p.W + (t.c0 + tc);
#pragma unroll
              for (int c = 0; c < 8; ++c) store4(Yb + tok * kD + dimof(4 * c, h), &Lm[j][4 * c]);
            }
          }
        }
      }
    }
  }

  // The workgroup that counted itself done last clears the launch counters
  // for the next call: every workgroup counted itself after its last counter
  // access, and each of its arrivals had been seen by its own waits, so no
  // other atomic on them is still to come.  The clears need no order among
  // themselves: the launch's end makes them visible to the next call.
  if (rk.group >= 0) res_stamp(a, true, kResStampOut);
  __syncthreads();
  res_stamp(a, true, kResStampEnd);
  if (done_sh) {
    for (int i = tid0; i < a.BH * kCntWords; i += kResThreads)
      put(a.slice_cnt + (size_t)(i / kCntWords) * kCntStride + i % kCntWords, 0u);
    if (a.grouped)
      for (int i = tid0; i < a.BH * 3 * kMaxSubs; i += kResThreads) put(a.sub_cnt + (size_t)i * kCntStride, 0u);
    if (tid0 < kXcds) put(a.tickets + tid0, 0u);
    if (tid0 < kXcds) put(a.done_xcd + (size_t)tid0 * kCntStride, 0u);
    if (a.clear_err && tid0 == 0) put(a.err, 0u);
    if (tid0 == 0) put(a.done_cnt, 0u);
  }
}

}  // namespace

template <int kMode, bool kMlp, bool kProj = false>
hipError_t launch_resident_typed(const ResArgs& a, int grid, hipStream_t s) {
  static std::atomic<bool> lds_set[kMaxDevices];
  const hipError_t e =
      ensure_lds_limit(reinterpret_cast<const void*>(&resident_kernel<kMode, kMlp, kProj>), kResLdsMax, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((resident_kernel<kMode, kMlp, kProj>), dim3(grid), dim3(kResThreads), a.p.L.total, s, a);
  return hipGetLastError();
}

hipError_t launch_resident(const ResArgs& a, int grid, hipStream_t s) {
  if (a.mode == kResReduce) return launch_resident_typed<kResReduce, false>(a, grid, s);
  if (a.mode == kResApply) return launch_resident_typed<kResApply, false>(a, grid, s);
  if (a.wo) return a.mlp_w1f ? hipErrorInvalidValue : launch_resident_typed<kResForward, false, true>(a, grid, s);
  return a.mlp_w1f ? launch_resident_typed<kResForward, true>(a, grid, s)
                   : launch_resident_typed<kResForward, false>(a, grid, s);
}

}  // namespace lisa
