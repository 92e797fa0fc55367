// Device helpers shared by the gfx950 kernels: element traits, MFMA wrappers,
// the accumulator-layout feature map (dimof), conversions, swizzled LDS
// addressing for DMA-staged rows, and the fence-free cross-workgroup hand-off.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lisa_kernels.hpp"

namespace lisa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Element traits.  EPL: contraction slots per lane in one MFMA; NQ: MFMAs to
// contract over 64; EPP: elements per 16-byte piece; PPR: pieces per 64-wide
// row; RB: bytes per row.
struct BF16 {
  using S = uint16_t;
  using Frag = bf16x8;
  static constexpr int EPL = 8, NQ = 4, EPP = 8, PPR = 8, RB = 128;
};
struct F32 {
  using S = float;
  using Frag = float;
  static constexpr int EPL = 1, NQ = 32, EPP = 4, PPR = 16, RB = 256;
};

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// Two floats to two bf16 (round to nearest even) in one word, lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// MFMA 32x32 layouts (lane l, m = l % 32, h = l / 32): operand A[m][k-slot],
// B[k-slot][m] with k-slots 8h + e (bf16, e < 8) or h (fp32); accumulator
// element i holds C[8 (i / 4) + 4 h + i % 4][m].  A 64-vector is kept "in
// accumulator layout" as 32 slots per lane: slot v of a lane of half h holds
// feature dimof(v, h); slots 0..15 are the first 32x32 block's accumulators.
__device__ __forceinline__ int dimof(int v, int h) {
  return 32 * (v >> 4) + 8 * ((v >> 2) & 3) + 4 * h + (v & 3);
}

// MFMA B operand from slots q*EPL .. q*EPL+EPL-1 of a 32-slot fp32 vector.
__device__ __forceinline__ bf16x8 operand(const float (&u)[32], int q, BF16) {
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = (__bf16)u[8 * q + e];
  return b;
}
__device__ __forceinline__ float operand(const float (&u)[32], int q, F32) { return u[q]; }

// y = x X for x in accumulator layout and X given as A-operand fragments:
// fragment (mb, q, lane, e) = X[dimof(q*EPL + e, lane/32)][32 mb + lane%32].
// Because a contraction index may be permuted as long as A and B agree, the
// accumulator slots of x feed the B operand directly.
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

// Four consecutive elements (8 B bf16 / 16 B fp32) -> floats, and back.
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
  *reinterpret_cast<uint2*>(p) = make_uint2(f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16),
                                            f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16));
}
__device__ __forceinline__ void store4(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// Sums over aligned groups of 8 (16) consecutive lanes, by DPP lane moves
// within rows of 16 lanes: xor 1 and xor 2 (quad permutes), then the mirror
// within each half row (lane i <-> 7 - i), then within the row (i <-> 15 - i).
__device__ __forceinline__ float dpp_add(float x, int ctrl) {
  int y;
  switch (ctrl) {  // the control must be a constant
    case 0xB1: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true); break;
    case 0x4E: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true); break;
    case 0x141: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true); break;
    default: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true); break;
  }
  return x + __int_as_float(y);
}
__device__ __forceinline__ float group_sum8(float x) {
  x = dpp_add(x, 0xB1);   // quad_perm [1, 0, 3, 2]
  x = dpp_add(x, 0x4E);   // quad_perm [2, 3, 0, 1]
  return dpp_add(x, 0x141);  // row_half_mirror
}
__device__ __forceinline__ float group_sum16(float x) { return dpp_add(group_sum8(x), 0x140); }  // row_mirror

// Index of this thread's wave in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }


// ---------------------------------------------------------------------------
// Swizzled LDS rows.  A staged 64-wide row (a token's features, or a grid
// cell) occupies RB bytes split into PPR 16-byte pieces; piece g of row r
// sits in slot g ^ swz(r), which spreads the lanes of the gathers below over
// the LDS banks.  Rows are written by global_load_lds DMA, one 1 KB run of
// 64 pieces per wave instruction, each lane fetching the piece that belongs
// in its slot.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ (((r >> 3) & 1) << 2); }

template <class Tr>
__device__ __forceinline__ int row_off(int r, int d) {  // byte offset of element d of row r
  constexpr int SH = Tr::EPP == 8 ? 3 : 2;             // log2(elements per piece)
  constexpr int ES = (int)sizeof(typename Tr::S);
  return r * Tr::RB + ((((d >> SH) ^ swz(r)) & (Tr::PPR - 1)) << 4) + (d & (Tr::EPP - 1)) * ES;
}

// LDS DMA (global_load_lds) issued through inline assembly.  The compiler
// then neither sees the LDS writes nor inserts waits for them; if it did, it
// would wait for the whole DMA of the next stage before the first LDS access
// of the current one.  Every read of DMA-staged data therefore follows an
// explicit wait_all() and a barrier.  Lane i writes bytes [16 i, 16 i + 16)
// (dwordx4) or [4 i, 4 i + 4) (dword) after the wave-uniform LDS address
// held in M0.
__device__ __forceinline__ unsigned lds_addr(const unsigned char* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_ptr_t)p);
}
__device__ __forceinline__ void dma16(const void* g, unsigned m0) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}
// Coherent at agent scope (sc1): for data other workgroups of the launch wrote.
__device__ __forceinline__ void dma16_coherent(const void* g, unsigned m0) {
  asm volatile("global_load_lds_dwordx4 %0, off sc1" ::"v"(g), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, unsigned m0) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4_coherent(const void* g, unsigned m0) {
  asm volatile("global_load_lds_dword %0, off sc1" ::"v"(g), "{m0}"(m0) : "memory");
}

// DMA `nrow` rows into `lds` (a multiple of 1 KB is written: the last run is
// padded with copies of row nrow-1).  src(r) returns the global address of
// row r (16-byte aligned).  Run j (1 KB) is issued by wave j % 4 of the
// calling role's four waves (`wave` in 0..3); no wait here.
template <class Tr, class SrcFn>
__device__ __forceinline__ void dma_rows(unsigned char* lds, int nrow, SrcFn src, int wave) {
  const int lane = threadIdx.x & 63;
  const int npieces = nrow * Tr::PPR;
  for (int base = wave * 64; base < npieces; base += 64 * 4) {
    const int P = base + lane;
    const int r = min(P / Tr::PPR, nrow - 1);
    const int slot = P % Tr::PPR;
    const int g = (slot ^ swz(P / Tr::PPR)) & (Tr::PPR - 1);
    const unsigned char* gp = static_cast<const unsigned char*>(src(r)) + g * 16;
    dma16(gp, lds_addr(lds + base * 16));
  }
}

// Coherent DMA of `bytes` (a multiple of 16) from src to lds unchanged, 1 KB
// per wave instruction, spread over four waves (`wave` in 0..3).
__device__ __forceinline__ void dma_linear_coherent(unsigned char* lds, const void* src, int bytes, int wave) {
  const int lane = threadIdx.x & 63;
  for (int base = wave * 1024; base < bytes; base += 4096) {
    const int off = min(base + lane * 16, bytes - 16);  // spare lanes repeat the last piece
    if (base + lane * 16 < bytes) dma16_coherent(static_cast<const unsigned char*>(src) + off, lds_addr(lds + base));
  }
}

// Bytes that dma_rows writes for nrow rows.
__host__ __device__ constexpr int dma_bytes(int nrow, int row_bytes) {
  return (nrow * row_bytes + 1023) / 1024 * 1024;
}

// ---------------------------------------------------------------------------
// Operands whose contraction index runs over staged rows.  gfx950's
// ds_read_b64_tr_b16 works on groups of 16 lanes: lane i of a group receives
// element (i & 3) of the 8-byte chunks addressed by lanes (i >> 2) + 4k,
// k = 0..3.  With each source lane pointing at 4 columns of one row, two such
// reads give lane (m, h) the MFMA operand X[row0 + 8h + e][col0 + m],
// e = 0..7, of a bf16 32x32x16 product whose k runs over rows.
// ---------------------------------------------------------------------------
// Operand bits are kept in integer vectors and reinterpreted as bf16 only at
// the MFMA: element-wise work on bf16 vectors rebuilt from such reads was
// folded wrongly by the compiler in testing.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4s tr_read(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
}
__device__ __forceinline__ v4s relu4(v4s x) { return __builtin_elementwise_max(x, (v4s)0); }
// The other feature map, phi(x) = ELU(x) + 1: x + 1 above zero, e^x at or
// below it (0 at -inf, which therefore pads rows that must add nothing).
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }
template <bool kElu>
__device__ __forceinline__ float feat(float x) { return kElu ? elu1(x) : fmaxf(x, 0.f); }
// elu1 of four bf16 values given as bits, rounded back to bf16 (to nearest even).
__device__ __forceinline__ v4s elu1_bits(v4s x) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = __builtin_bit_cast(u32x2, x);
  u32x2 o;
  o[0] = pack_bf16x2(elu1(__uint_as_float(w[0] << 16)), elu1(__uint_as_float(w[0] & 0xffff0000u)));
  o[1] = pack_bf16x2(elu1(__uint_as_float(w[1] << 16)), elu1(__uint_as_float(w[1] & 0xffff0000u)));
  return __builtin_bit_cast(v4s, o);
}
__device__ __forceinline__ v8s join(v4s lo, v4s hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 as_bf16(v8s x) { return __builtin_bit_cast(bf16x8, x); }

// phi of a 64-vector held as B operands in feature order (lane (m, h) holds
// features 16 q + 8 h + e of piece q, e = 0..7), returned as B operands in
// accumulator slot order (piece q holds slots 8 q .. 8 q + 7, i.e. features
// dimof(8 q + e, h)).  Within a piece, the lower half keeps features 0..3 and
// takes 8..11 from the upper half, which takes 4..7 in exchange: the upper
// half of dwords 0, 1 trades places with the lower half of dwords 2, 3.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <bool kElu = false>
__device__ __forceinline__ v8s relu_to_slots(v8s x) {
  u32x4 w = __builtin_bit_cast(u32x4, x);
  const auto p = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
  const auto q = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
  w[0] = p[0];
  w[2] = p[1];
  w[1] = q[0];
  w[3] = q[1];
  if constexpr (kElu) {
    const v8s y = __builtin_bit_cast(v8s, w);
    return join(elu1_bits(__builtin_shufflevector(y, y, 0, 1, 2, 3)),
                elu1_bits(__builtin_shufflevector(y, y, 4, 5, 6, 7)));
  }
  return __builtin_elementwise_max(__builtin_bit_cast(v8s, w), (v8s)0);
}

// apply() for a bf16 x given as the bits of its B operands (slot order).
__device__ __forceinline__ void apply_bits(const bf16x8 (&fr)[2][4], const v8s (&x)[4], float (&y)[32]) {
  f32x16 c0 = {}, c1 = {};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x8 b = as_bf16(x[q]);
    c0 = mma(fr[0][q], b, c0);
    c1 = mma(fr[1][q], b, c1);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    y[i] = c0[i];
    y[16 + i] = c1[i];
  }
}

// Bits of X[row0 + 8h + e][col0 + m] (bf16 rows of a staged region), e = 0..7;
// with kRelu the values are clamped at zero (a negative bf16 is a negative int16),
// with kElu as well they go through elu1 instead.
template <bool kRelu, bool kElu = false>
__device__ __forceinline__ v8s rows_bits(const unsigned char* base, int row0, int col0) {
  const int L = threadIdx.x & 63, i = L & 15, g = L >> 4;
  const int col = col0 + 16 * (g & 1) + 4 * (i & 3);
  const int r = row0 + 8 * (g >> 1) + (i >> 2);
  v4s lo = tr_read(base + row_off<BF16>(r, col));
  v4s hi = tr_read(base + row_off<BF16>(r + 4, col));
  if constexpr (kRelu && kElu) {
    lo = elu1_bits(lo);
    hi = elu1_bits(hi);
  } else if (kRelu) {
    lo = relu4(lo);
    hi = relu4(hi);
  }
  return join(lo, hi);
}

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off without cache-wide fences: data shared between
// workgroups of one launch is written and read with relaxed agent-scope
// atomics (coherent accesses that bypass the non-coherent per-XCD L2), the
// writer waits for its stores to complete before bumping an arrival counter,
// and the reader reads the data only after it has observed the count.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void put(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at agent scope (sc1), for data other workgroups read: one vector
// store instruction, so a wave's pieces go out as whole lines.
__device__ __forceinline__ void put16(void* p, uint4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = {v.x, v.y, v.z, v.w};
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(x) : "memory");
}
__device__ __forceinline__ float get(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t get(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
// Wait for every outstanding memory access of this wave (the compiler may
// not move memory accesses across it).
__device__ __forceinline__ void wait_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every global load in flight, which includes the LDS DMA of the
// next stage; this one lets that DMA continue.  Each wave first waits for
// its own LDS accesses (lgkmcnt(0)).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ unsigned bump(unsigned* cnt) {
  return __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Dependency waits between the workgroups of one launch.
// ---------------------------------------------------------------------------
// Spin (one lane) until *c >= target.  The wait is bounded (about a second);
// on giving up it raises the error word, after which every later wait of the
// launch returns at once, so the launch always finishes.
__device__ inline void wait_for(const unsigned* c, unsigned target, unsigned* err) {
  unsigned spins = 0;
  // Every poll is a device-wide load of the line the arrivals update: about
  // 0.1 us between polls when at most 32 workgroups count (and poll) on it
  // (0.27 us measured 0.2 us slower at PVT-T stage 1), about 0.27 us with
  // more, where hundreds of workgroups polling one line densely slow the
  // arrivals themselves.
  const bool few = target <= 32;
  while (get(c) < target) {
    if (few)
      __builtin_amdgcn_s_sleep(4);
    else
      __builtin_amdgcn_s_sleep(10);
    if ((++spins & 255u) == 0 && get(err)) break;
    if (spins > (1u << 22)) {
      put(err, 1u);
      break;
    }
  }
  // The data the count announces is read only after this point: the
  // compiler may not move those (relaxed) loads above the poll.
  asm volatile("" ::: "memory");
}

// The same wait for a phase counted per group of kSubRanks ranks: lane k of
// the calling wave (all 64 lanes call) reads group k's counter, until every
// group's counter has reached kSubRanks; bounded like wait_for.
__device__ inline void wait_for_groups(const unsigned* base, int ngroups, unsigned* err) {
  const int lane = threadIdx.x & 63;
  const unsigned* c = base + (size_t)min(lane, ngroups - 1) * kCntStride;
  unsigned spins = 0;
  for (;;) {
    const bool done = lane >= ngroups || get(c) >= (unsigned)kSubRanks;
    if (__all(done)) break;
    __builtin_amdgcn_s_sleep(10);
    ++spins;
    if ((spins & 255u) == 0 && __builtin_amdgcn_readfirstlane(get(err))) break;
    if (spins > (1u << 21)) {
      if (lane == 0) put(err, 1u);
      break;
    }
  }
  asm volatile("" ::: "memory");  // as in wait_for
}

// ---------------------------------------------------------------------------
// The 3x3 local branch on MFMA works on blocks of 4 x 8 tokens, whose windows
// lie in a 6 x 10 window of cells; these map the MFMA's logit slots to cells.
// ---------------------------------------------------------------------------
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


}  // namespace lisa
