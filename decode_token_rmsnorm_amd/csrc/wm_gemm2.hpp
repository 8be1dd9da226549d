// wm_gemm2.hpp — large-tile bf16 GEMM  C[M, N] = A[M, K] * B[N, K]^T  for the
// big projections (rows >= a few thousand).
//
// Block tile 256 x 256, 256 threads = 4 wave64s in a 2 x 2 grid; each wave
// owns a 128 x 128 sub-tile of 4 x 4 MFMA 32x32x16 bf16 tiles (256 fp32
// accumulators per lane).  Both operands are copied global -> LDS by the
// 16-byte LDS DMA (global_load_lds_dwordx4): lane i of a wave writes LDS bytes
// [16i, 16i + 16) of its 1 KB slot, so one instruction fills 1 KB of rows;
// which global 16-byte chunk a lane fetches is XOR-swizzled by the row, and
// the MFMA fragment reads undo the swizzle, which spreads the 32 rows a
// fragment read touches over all banks without padding.  The k-tile is KB
// bytes per row (128 or 64) in ST LDS stages: the DMAs of the next ST-1
// k-tiles are in flight while the MFMAs of the current one run; each k-tile
// starts with a wait for its own DMAs and a bare barrier (every LDS read of a
// stage is consumed by an MFMA before the barrier that lets it be refilled, so
// no memory fence, which would also drain the prefetch, is needed).  The C
// tile is staged through LDS in two 128-row halves for the same row-wise
// epilogues as the 128 x 128 kernel (wm_gemm.hpp).
#pragma once

#include "wm_gemm.hpp"

namespace wm {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int G2M = 256, G2N = 256;
constexpr int G2CP = G2N + 4;         // C tile pitch (floats)
constexpr int G2CT = 128 * G2CP * 4;  // staged half C tile, bytes
constexpr int G2KB = 64, G2ST = 4;    // k-tile bytes per row, LDS stages
constexpr int g2_smem(int kb, int st) {
  return (st * (G2M + G2N) * kb > G2CT + 512) ? st * (G2M + G2N) * kb : G2CT + 512;
}

// 16-byte chunk position of logical chunk c in tile row r (rows of KB bytes).
template <int KB> __device__ __forceinline__ int g2_swz(int r, int c) {
  if constexpr (KB == 128) return c ^ ((r ^ (r >> 3)) & 7);
  else return c ^ (((r >> 1) ^ (r >> 3)) & 3);
}

// s_waitcnt vmcnt(n) (expcnt / lgkmcnt unconstrained), n < 64.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (N & 15));
}

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

// vanilla per-layer K/V weights stacked: rows [0, hd) of wk, then wv.
template <typename T> struct PKVL {
  const T *wk, *wv;
  int64_t ld;
  int hd, N;
  __device__ __forceinline__ const char *row(int z, int n0, int jl) const {
    int n = n0 + jl;
    n = n < N ? n : N - 1;
    return (const char *)(n < hd ? wk + (int64_t)n * ld : wv + (int64_t)(n - hd) * ld);
  }
};

__device__ __forceinline__ void dma16(const void *g, unsigned char *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// Block order. MAP bit 0: split the tiles into 8 contiguous ranges, one per
// XCD (assuming round-robin dispatch); MAP >> 1 selects M-bands of 1, 4, 8 or
// 2 tiles walked before moving along N. Measured on the gate/up shape with
// weights that do not stay cached: plain order with 4-tile bands is fastest
// (the per-XCD ranges were slowest), so MAP = 2 is the default.
template <int MAP>
__device__ __forceinline__ void g2_tile(int b, int nM, int nN, int &tm, int &tn, int &z) {
  const int total = gridDim.x;
  int t = b;
  if constexpr (MAP & 1) {  // contiguous tile range per XCD
    const int q = total / 8, r = total % 8;
    const int x = b % 8, i = b / 8;
    t = x * q + (x < r ? x : r) + i;
  }
  const int per_z = nM * nN;
  z = t / per_z;
  t -= z * per_z;
  constexpr int band = (MAP >> 1) == 0 ? 1 : (MAP >> 1) == 1 ? 4 : (MAP >> 1) == 2 ? 8 : 2;
  const int g = t / (band * nN);
  const int m_first = g * band;
  const int bm = (nM - m_first) < band ? (nM - m_first) : band;
  const int tt = t - g * band * nN;
  tm = m_first + tt % bm;
  tn = tt / bm;
}

template <int KB, int ST, int MAP, class AP, class BP, class EP>
__global__ __launch_bounds__(256) void gemm2_kernel(AP ap, BP bp, EP ep, int M, int N, int K, int nM, int nN) {
  constexpr int STAGE = (G2M + G2N) * KB;
  constexpr int RPI = 1024 / KB;          // rows per DMA instruction
  constexpr int NI = G2M / RPI / 4;       // DMA instructions per wave per operand
  constexpr int PI = 2 * NI;              // DMA instructions per wave per k-tile
  constexpr int KS = KB / 32;             // 16-deep MFMA steps per k-tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[g2_smem(KB, ST)];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn, z;
  g2_tile<MAP>(blockIdx.x, nM, nN, tm, tn, z);
  const int m0 = tm * G2M, n0 = tn * G2N;
  const int nk = K * 2 / KB;

  // This thread's DMA sources: rows (wave*NI + j)*RPI + lane/(KB/16) of each
  // operand, chunk chosen so that LDS slot (row, lane % (KB/16)) holds the
  // swizzled chunk (the swizzle is an XOR, its own inverse).
  const char *pa[NI], *pb[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    int row = (wave * NI + j) * RPI + lane / (KB / 16);
    int c = g2_swz<KB>(row, lane % (KB / 16));
    pa[j] = ap.row(z, m0 + row) + c * 16;
    pb[j] = bp.row(z, n0, row) + c * 16;
  }
  auto issue = [&](int kt, int stage) {
    unsigned char *As = smem + stage * STAGE, *Bs = As + G2M * KB;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      dma16(pa[j] + kt * KB, As + (wave * NI + j) * 1024);
      dma16(pb[j] + kt * KB, Bs + (wave * NI + j) * 1024);
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
      af[i] = *(const u32x4 *)(As + r * KB + g2_swz<KB>(r, c) * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int r = wn * 128 + j * 32 + (lane & 31);
      bfr[j] = *(const u32x4 *)(Bs + r * KB + g2_swz<KB>(r, c) * 16);
    }
  };
  // Wait until at most `later` k-tiles after the awaited one are in flight.
  auto wait_tiles = [&](int later) {
    if constexpr (ST >= 4) {
      if (later >= 2) wait_vmcnt<2 * PI>();
      else if (later == 1) wait_vmcnt<PI>();
      else wait_vmcnt<0>();
    } else if constexpr (ST == 3) {
      if (later >= 1) wait_vmcnt<PI>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
  };
  auto mfmas = [&](const u32x4 *af, const u32x4 *bfr) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                            __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j], 0, 0, 0);
  };
  // 2 MFMAs : 1 fragment read, so LDS latency hides under the MFMAs.
  auto interleave = [&]() {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
  };

  // Prologue: k-tiles 0..ST-2 in flight; wait for tile 0, then refill and read
  // its first fragments.
#pragma unroll
  for (int t = 0; t < ST - 1; ++t)
    if (t < nk) issue(t, t);
  wait_tiles(min(ST - 2, nk - 1));
  __builtin_amdgcn_s_barrier();
  if (ST - 1 < nk) issue(ST - 1, (ST - 1) % ST);
  u32x4 fa[2][4], fb[2][4];
  frags(smem, smem + G2M * KB, 0, fa[0], fb[0]);

  // Steady state. The barrier that makes k-tile kt+1 visible (and frees the
  // stage of tile kt for tile kt+ST) sits before the last MFMA step of tile
  // kt, so tile kt+1's first fragments load while that step's MFMAs run.
  for (int kt = 0; kt < nk; ++kt) {
    const unsigned char *As = smem + (kt % ST) * STAGE, *Bs = As + G2M * KB;
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      frags(As, Bs, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      mfmas(fa[ks & 1], fb[ks & 1]);
      interleave();
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of tile kt are done
    if (kt + 1 < nk) wait_tiles(min(ST - 2, nk - kt - 2));
    __builtin_amdgcn_s_barrier();
    if (kt + ST < nk) issue(kt + ST, (kt + ST) % ST);
    {  // (on the last k-tile this reads a stale stage; the values are unused)
      const unsigned char *An = smem + ((kt + 1) % ST) * STAGE;
      frags(An, An + G2M * KB, 0, fa[KS & 1], fb[KS & 1]);
    }
    mfmas(fa[(KS - 1) & 1], fb[(KS - 1) & 1]);
    __builtin_amdgcn_sched_group_barrier(0x020, 2 * NI, 0);  // DMA issue first
    interleave();
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

template <int KB = G2KB, int ST = G2ST, int MAP = 2, class AP, class BP, class EP>
hipError_t launch_gemm2(const AP &ap, const BP &bp, const EP &ep, int M, int N, int K, int Z, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int nM = (M + G2M - 1) / G2M, nN = (N + G2N - 1) / G2N;
  hipLaunchKernelGGL((gemm2_kernel<KB, ST, MAP, AP, BP, EP>), dim3(nM * nN * Z), dim3(256), 0, s, ap, bp, ep, M, N,
                     K, nM, nN);
  return hipGetLastError();
}

}  // namespace wm
