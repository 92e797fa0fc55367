// Static schedules of the layer's projections (lisa_layer.hip): which 64 x 64
// output blocks a workgroup of the blocked kernel (proj_gemm) or of the
// streaming QKV kernel (proj_stream_qkv) computes.  Shared by the kernels and
// a CPU check of the schedules' coverage (tests/test_schedule_cpu.py builds
// tests/schedule_check.cpp against it).  M rows, N outputs (a multiple of 64).
#pragma once

#include <hip/hip_runtime.h>

namespace lisa {

constexpr int kProjTiles = 4;      // proj_gemm: 64-row tiles per workgroup (each weight operand read serves four)
constexpr int kProjXcds = 8;       // the device hands workgroup w to XCD w % 8
constexpr int kStreamGrid = 1024;  // proj_stream_qkv: workgroups (four per CU of a 256-CU device), rounded down below

// proj_gemm: row block (kProjTiles tiles) and column block of workgroup w
// (row block -1: idle).  With several column blocks, XCD x takes row blocks
// x, x + 8, ..., each with all its column blocks in a row, so the workgroups
// that share input rows are consecutive ones of one XCD (one L2); the grid
// is padded to whole rounds of 8.
__host__ __device__ inline void proj_block(int M, int N, int w, int& rb, int& cb) {
  const int nct = N / 64, nrb = (M + 64 * kProjTiles - 1) / (64 * kProjTiles);
  if (nct == 1) {
    rb = w;
    cb = 0;
  } else {
    const int x = w % kProjXcds, k = w / kProjXcds;
    rb = x + kProjXcds * (k / nct);
    cb = k % nct;
  }
  if (rb >= nrb) rb = -1;
}
__host__ __device__ inline int proj_grid(int M, int N) {
  const int nct = N / 64, nrb = (M + 64 * kProjTiles - 1) / (64 * kProjTiles);
  return nct == 1 ? nrb : (nrb + kProjXcds - 1) / kProjXcds * kProjXcds * nct;
}

// proj_stream_qkv: unit u is the 64-row tile x + 8 (k / nct) and column block
// k % nct (x = u % 8, k = u / 8); units cover whole rounds of 8 row tiles
// (tiles past the last one are idle).  The grid is a multiple of 8 nct, so
// the units a workgroup walks (u, u + grid, ...) share its column block.
__host__ __device__ inline int proj_units(int M, int N) {
  const int nct = N / 64, nrt = (M + 63) / 64;
  return (nrt + kProjXcds - 1) / kProjXcds * kProjXcds * nct;
}
__host__ __device__ inline void proj_unit(int N, int u, int& rt, int& cb) {
  const int nct = N / 64, x = u % kProjXcds, k = u / kProjXcds;
  rt = x + kProjXcds * (k / nct);
  cb = k % nct;
}
__host__ __device__ inline int proj_stream_grid(int M, int N) {
  const int step = kProjXcds * (N / 64);
  int g = kStreamGrid / step * step;
  if (g < step) g = step;
  const int u = proj_units(M, N);
  return g < u ? g : u;
}

}  // namespace lisa
