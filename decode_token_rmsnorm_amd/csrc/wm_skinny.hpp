// wm_skinny.hpp — GEMM for few rows (decode steps, small token groups):
// C[M, N] = A[M, K] * B[N, K]^T with M <= 128.
//
// With so few rows the product is a stream of the weight matrix B and the
// time goes into memory round trips (about 1.6 us each from HBM), so the
// kernel is built to make one: every block covers a 64-row x 128-column
// output tile and one 1 KB slice of each row's k range (SKB bytes: 512 bf16
// or 256 float), and issues all of its loads before its first MFMA.  Its 8
// waves are 2 column halves x 4 k quarters; quarter q takes the 64-byte
// k-steps q, q+4, q+8, q+12 of the slice.  Fragments go from global memory
// straight into MFMA operand registers (16 bytes per lane: row or column
// lane%16, k-slice lane/16, the layout of mma16).  The quarters are summed
// through LDS in a fixed order.  With one slice (K*sizeof(T) <= SKB) the
// block then runs the epilogue functor (wm_gemm.hpp) on its tile; otherwise
// it stores the tile to a partial buffer and skinny_reduce adds the slices,
// again in a fixed order, and runs the epilogue.  Results are deterministic.
#pragma once

#include "wm_gemm.hpp"
#include "wm_host.hpp"

namespace wm {

constexpr int SKM = 64;                   // block rows
constexpr int SKT = 512;                  // threads (8 waves)
constexpr int SKP = GN + 4;               // LDS tile pitch (floats)
constexpr int SKB = kSkinnySliceBytes;    // k bytes per block
constexpr int SK_MAX_ROWS = kSkinnyRows;  // the dispatch uses this kernel up to this many rows

template <typename T, class AL, class BL, class EP>
__global__ __launch_bounds__(SKT) void gemm_skinny(AL al, BL bl, EP ep, int M, int N, int K, int S, float *partial) {
  __shared__ __attribute__((aligned(16))) float part[4 * SKM * SKP + SKM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wk = wave >> 1;  // column half, k quarter
  const int sl = blockIdx.z % S, z = blockIdx.z / S;
  const int m0 = blockIdx.y * SKM, n0 = blockIdx.x * GN;
  const int nks = (int)((int64_t)K * (int64_t)sizeof(T) / 64);
  const int st0 = sl * (SKB / 64), st1 = min(st0 + SKB / 64, nks);  // this block's k-steps
  const int kl = (lane >> 4) * 16, rl = lane & 15;

  typename AL::H ha[4];
  typename BL::H hb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ha[i] = al.row(z, m0 + i * 16 + rl, M);
    hb[i] = bl.row(z, n0, wn * 64 + i * 16 + rl, N);
  }
  // All loads first.  A step past the slice re-reads its last step and is
  // multiplied with the A fragments masked to zero, so loads and MFMAs are
  // unconditional and the waits before the MFMAs count exactly.
  u32x4 a[4][4], b[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ks = min(st0 + wk + 4 * u, st1 - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[u][i] = al.load(ha[i], ks * 64 + kl);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[u][j] = bl.load(hb[j], ks * 64 + kl);
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t mask = st0 + wk + 4 * u < st1 ? ~0u : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 am = a[u][i] & mask;
#pragma unroll
      for (int j = 0; j < 4; ++j) mma16<T>(acc[i][j], am, b[u][j]);
    }
  }

  // Quarter wk's 64 columns go to LDS tile wk; the tiles are added in order
  // into tile 0.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part[(wk * SKM + i * 16 + 4 * (lane >> 4) + e) * SKP + wn * 64 + j * 16 + rl] = acc[i][j][e];
  __syncthreads();
  if (S == 1) {
    for (int idx = tid; idx < SKM * GN; idx += SKT) {
      const int r = idx / GN, c = idx - r * GN;
      float *p = part + r * SKP + c;
      p[0] = ((p[0] + p[SKM * SKP]) + p[2 * SKM * SKP]) + p[3 * SKM * SKP];
    }
    __syncthreads();
    run_epi<T, GN / 64>(ep, z, m0, n0, part, SKP, SKM, M, N, part + 4 * SKM * SKP);
  } else {
    // partial[((z * gridDim.y + by) * gridDim.x + bx) * S + sl] is a dense
    // 64 x 128 fp32 tile.
    float *dst = partial + ((((int64_t)z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * S + sl) * (SKM * GN);
    for (int idx = tid * 4; idx < SKM * GN; idx += SKT * 4) {
      const int r = idx / GN, c = idx - r * GN;
      const float *p = part + r * SKP + c;
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = ((p[e] + p[SKM * SKP + e]) + p[2 * SKM * SKP + e]) + p[3 * SKM * SKP + e];
      *(f32x4 *)(dst + idx) = v;
    }
  }
}

// Sum of the S slice tiles of one output tile (in slice order), then the
// epilogue.  Grid (nN, nM, Z) as the GEMM's without the slices.
template <typename T, class EP>
__global__ __launch_bounds__(SKT) void skinny_reduce(EP ep, const float *partial, int M, int N, int S) {
  __shared__ __attribute__((aligned(16))) float Cs[SKM * SKP + SKM];
  const int tid = threadIdx.x, z = blockIdx.z, m0 = blockIdx.y * SKM, n0 = blockIdx.x * GN;
  const float *src = partial + (((int64_t)z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * S * (SKM * GN);
  for (int idx = tid * 4; idx < SKM * GN; idx += SKT * 4) {
    f32x4 v = *(const f32x4 *)(src + idx);
    int sl = 1;
    for (; sl + 4 <= S; sl += 4) {  // four slices' loads in flight together
      f32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = *(const f32x4 *)(src + (int64_t)(sl + u) * (SKM * GN) + idx);
#pragma unroll
      for (int u = 0; u < 4; ++u) v += w[u];
    }
    for (; sl < S; ++sl) v += *(const f32x4 *)(src + (int64_t)sl * (SKM * GN) + idx);
    const int r = idx / GN, c = idx - r * GN;
    *(f32x4 *)(Cs + r * SKP + c) = v;
  }
  __syncthreads();
  run_epi<T, GN / 64>(ep, z, m0, n0, Cs, SKP, SKM, M, N, Cs + SKM * SKP);
}

template <typename T, class AL, class BL, class EP>
hipError_t launch_skinny(const AL &al, const BL &bl, const EP &ep, int M, int N, int K, int Z, float *partial,
                         hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int S = skinny_slices((int64_t)K * (int64_t)sizeof(T));
  dim3 grid((N + GN - 1) / GN, (M + SKM - 1) / SKM, Z * S);
  hipLaunchKernelGGL((gemm_skinny<T, AL, BL, EP>), grid, dim3(SKT), 0, s, al, bl, ep, M, N, K, S, partial);
  if (S > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((skinny_reduce<T, EP>), dim3(grid.x, grid.y, Z), dim3(SKT), 0, s, ep, partial, M, N, S);
  }
  return hipGetLastError();
}

}  // namespace wm
