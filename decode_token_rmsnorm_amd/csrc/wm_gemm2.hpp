// wm_gemm2.hpp — large-tile bf16 GEMM  C[M, N] = A[M, K] * B[N, K]^T  for the
// big projections (rows >= a few thousand).
//
// Block tile 256 x 256, k-tile 64 (128 bytes per row), 256 threads = 4 wave64s
// in a 2 x 2 grid; each wave owns a 128 x 128 sub-tile of 4 x 4 MFMA
// 32x32x16 bf16 tiles (256 fp32 accumulators per lane).  Both operands are
// copied global -> LDS by the 16-byte LDS DMA (global_load_lds_dwordx4): lane
// i of a wave writes LDS bytes [16i, 16i + 16) of its 1 KB slot, so each
// instruction fills 8 rows of 128 bytes; which global 16-byte chunk a lane
// fetches is XOR-swizzled by the row, and the MFMA fragment reads undo the
// swizzle, which spreads the 32 rows a fragment read touches over all banks
// without padding.  Two LDS stages: the DMA of k-tile t+1 runs while the MFMAs
// of k-tile t execute, one barrier per k-tile.  The C tile is staged through
// LDS in two 128-row halves for the same row-wise epilogues as the 128 x 128
// kernel (wm_gemm.hpp).
#pragma once

#include "wm_gemm.hpp"

namespace wm {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int G2M = 256, G2N = 256, G2KB = 128;
constexpr int G2STAGE = (G2M + G2N) * G2KB;  // 64 KB
constexpr int G2CP = G2N + 4;                // C tile pitch (floats)
constexpr int G2CT = 128 * G2CP * 4;         // staged half C tile, bytes
constexpr int G2SMEM = (2 * G2STAGE > G2CT + 512) ? 2 * G2STAGE : G2CT + 512;

// 16-byte chunk position of logical chunk c in tile row r.
__device__ __forceinline__ int g2_swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

// Row-pointer providers (rows past the end are clamped to the last row: their
// products are computed and discarded by the epilogue).
template <typename T> struct PRows {
  const T *p;
  int64_t ld, zstride;
  int nrows;
  __device__ __forceinline__ const char *row(int z, int r) const {
    r = r < nrows ? r : nrows - 1;
    return (const char *)(p + z * zstride + (int64_t)r * ld);
  }
};
template <typename T> struct PBRows {
  PRows<T> P;
  __device__ __forceinline__ const char *row(int z, int n0, int jl) const { return P.row(z, n0 + jl); }
};
// gate/up: tile rows [0, 128) gate rows n0/2 + jl, [128, 256) the up rows.
template <typename T> struct PGateUp {
  const T *gate, *up;
  int64_t ld;
  int F;
  __device__ __forceinline__ const char *row(int z, int n0, int jl) const {
    int f = n0 / 2 + (jl & (G2N / 2 - 1));
    f = f < F ? f : F - 1;
    return (const char *)((jl < G2N / 2 ? gate : up) + (int64_t)f * ld);
  }
};
// pool projection weights: z = beta*k + j -> wk[j] / wv[j].
template <typename T> struct PKV {
  const T *wk, *wv;
  int64_t ld, mstride;
  int k, N;
  __device__ __forceinline__ const char *row(int z, int n0, int jl) const {
    int n = n0 + jl;
    n = n < N ? n : N - 1;
    int beta = z / k, j = z - beta * k;
    return (const char *)((beta == 0 ? wk : wv) + j * mstride + (int64_t)n * ld);
  }
};

__device__ __forceinline__ void dma16(const void *g, unsigned char *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// Block order: tiles are split into 8 contiguous ranges, one per XCD (blocks
// are dispatched to XCDs round-robin), and inside a range walk M-bands of 4
// tiles so that neighbouring tiles on one XCD share operand panels in its L2.
__device__ __forceinline__ void g2_tile(int b, int nM, int nN, int &tm, int &tn, int &z) {
  const int total = gridDim.x;
  const int q = total / 8, r = total % 8;
  const int x = b % 8, i = b / 8;
  int t = x * q + (x < r ? x : r) + i;
  const int per_z = nM * nN;
  z = t / per_z;
  t -= z * per_z;
  const int band = 4;
  const int g = t / (band * nN);
  const int m_first = g * band;
  const int bm = (nM - m_first) < band ? (nM - m_first) : band;
  const int tt = t - g * band * nN;
  tm = m_first + tt % bm;
  tn = tt / bm;
}

template <class AP, class BP, class EP>
__global__ __launch_bounds__(256) void gemm2_kernel(AP ap, BP bp, EP ep, int M, int N, int K, int nM, int nN) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[G2SMEM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn, z;
  g2_tile(blockIdx.x, nM, nN, tm, tn, z);
  const int m0 = tm * G2M, n0 = tn * G2N;
  const int nk = K / 64;

  // This thread's DMA sources: rows (wave*8 + j)*8 + lane/8 of each operand,
  // chunk chosen so that LDS slot (row, lane%8) holds the swizzled chunk.
  const char *pa[8], *pb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int row = (wave * 8 + j) * 8 + (lane >> 3);
    int c = g2_swz(row, lane & 7);  // the swizzle is an involution on the chunk index
    pa[j] = ap.row(z, m0 + row) + c * 16;
    pb[j] = bp.row(z, n0, row) + c * 16;
  }
  auto issue = [&](int kt, int stage) {
    unsigned char *As = smem + stage * G2STAGE, *Bs = As + G2M * G2KB;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dma16(pa[j] + kt * G2KB, As + (wave * 8 + j) * 1024);
      dma16(pb[j] + kt * G2KB, Bs + (wave * 8 + j) * 1024);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Fragments of k-step ks+1 are read from LDS while the MFMAs of step ks run.
  auto frags = [&](const unsigned char *As, const unsigned char *Bs, int ks, u32x4 *af, u32x4 *bfr) {
    const int c = 2 * ks + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = wm * 128 + i * 32 + (lane & 31);
      af[i] = *(const u32x4 *)(As + r * G2KB + g2_swz(r, c) * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int r = wn * 128 + j * 32 + (lane & 31);
      bfr[j] = *(const u32x4 *)(Bs + r * G2KB + g2_swz(r, c) * 16);
    }
  };
  issue(0, 0);
  u32x4 fa[2][4], fb[2][4];
  for (int kt = 0; kt < nk; ++kt) {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
    const unsigned char *As = smem + (kt & 1) * G2STAGE, *Bs = As + G2M * G2KB;
    frags(As, Bs, 0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) frags(As, Bs, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[ks & 1][i]),
                                                              __builtin_bit_cast(bf16x8, fb[ks & 1][j]), acc[i][j],
                                                              0, 0, 0);
    }
  }
  __syncthreads();

  // epilogue in two 128-row halves; accumulator (lane, e) of a 32x32 tile is
  // row 8*(e/4) + 4*(lane/32) + e%4, column lane%32.
  float *Cs = (float *)smem;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            Cs[(i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * G2CP + wn * 128 + j * 32 + (lane & 31)] =
                acc[i][j][e];
    }
    __syncthreads();
    run_epi<bf16, G2N / 64>(ep, z, m0 + h * 128, n0, Cs, G2CP, 128, M, N, (float *)(smem + G2CT));
    __syncthreads();
  }
}

template <class AP, class BP, class EP>
hipError_t launch_gemm2(const AP &ap, const BP &bp, const EP &ep, int M, int N, int K, int Z, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int nM = (M + G2M - 1) / G2M, nN = (N + G2N - 1) / G2N;
  hipLaunchKernelGGL((gemm2_kernel<AP, BP, EP>), dim3(nM * nN * Z), dim3(256), 0, s, ap, bp, ep, M, N, K, nM, nN);
  return hipGetLastError();
}

}  // namespace wm
