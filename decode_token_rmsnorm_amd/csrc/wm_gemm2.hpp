// wm_gemm2.hpp — large-tile bf16 GEMM  C[M, N] = A[M, K] * B[N, K]^T  for the
// big projections (rows >= a few thousand).
//
// Block tile 256 x 256, 256 threads = 4 wave64s in a 2 x 2 grid (or 512 threads =
// 8 waves, two per SIMD: G2Shape below); each wave
// owns a 128 x 128 sub-tile of 4 x 4 MFMA 32x32x16 bf16 tiles (256 fp32
// accumulators per lane); or 256 x 224, with wave sub-tiles of 64 x 224,
// 32 x 224 or 64 x 112 (the last on 16x16x32 MFMA tiles; G2Shape below).
// Both operands are copied global -> LDS by the
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

#include <type_traits>
#include <utility>

#include "wm_gemm.hpp"

namespace wm {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int G2M = 256, G2N = 256;
constexpr int kComputeUnits = 256;    // MI355X
constexpr int G2CP = G2N + 4;         // C tile pitch (floats)
constexpr int G2CT = 128 * G2CP * 4;  // staged half C tile, bytes
constexpr int G2KB = 128, G2ST = 2;  // k-tile bytes per row, LDS stages
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

// Wave arrangements of the 256-row block tile. SH 0: 2 x 2 waves of 128 x 128
// (4 x 4 MFMA tiles), 256 columns. SH 1: 4 x 1 waves of 64 x 224 (2 x 7 MFMA
// tiles), 224 columns: a 1792-column product then has 8 column tiles, and
// 8192 rows give 256 blocks, one per compute unit, where 256 columns give 224.
// SH 2: 2 x 4 waves of 128 x 64 (4 x 2 MFMA tiles), 256 columns, and SH 3:
// 8 x 1 waves of 32 x 224 (1 x 7 MFMA tiles), 224 columns: two waves per SIMD
// with 128 or 112 accumulators each, so one wave's LDS reads and DMA waits
// overlap the other's MFMAs.  SH 4: 4 x 2 waves of 64 x 112 on the 16x16x32
// MFMA (4 x 7 tiles of 16 x 16), 224 columns: the same 112 accumulators as
// SH 3, but a wave reads 176 instead of 256 fragment rows per k-step, which
// matters because the 224-column kernel is bound by its LDS reads.
template <int SH> struct G2Shape {
  static constexpr int NW = SH >= 2 ? 8 : 4;                                          // waves per block
  static constexpr int MF = SH == 4 ? 16 : 32;                                        // MFMA tile edge
  static constexpr int WN = SH == 1 || SH == 3 ? 1 : SH == 2 ? 4 : 2;                 // waves along N
  static constexpr int TI = SH == 1 ? 2 : SH == 3 ? 1 : 4;                            // MF-row MFMA tiles per wave
  static constexpr int TJ = SH == 1 || SH == 3 || SH == 4 ? 7 : SH == 2 ? 2 : 4;      // MF-column tiles per wave
  static constexpr int BN = MF * TJ * WN;
};

// Scheduling groups: NR fragment reads spread evenly over NMF MFMAs.
template <int NMF, int NR, int... G> __device__ __forceinline__ void g2_spread(std::integer_sequence<int, G...>) {
  ((__builtin_amdgcn_sched_group_barrier(0x008, (G + 1) * NMF / NR - G * NMF / NR, 0),
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0)),
   ...);
}

template <int KB, int ST, int MAP, int SH, class AP, class BP, class EP>
__global__ __launch_bounds__(64 * G2Shape<SH>::NW) void gemm2_kernel(AP ap, BP bp, EP ep, int M, int N, int K, int nM,
                                                                     int nN) {
  using S = G2Shape<SH>;
  constexpr int NW = S::NW, TI = S::TI, TJ = S::TJ, BN = S::BN, MF = S::MF;
  using Acc = typename std::conditional<MF == 32, f32x16, f32x4>::type;
  constexpr int STAGE = (G2M + BN) * KB;
  constexpr int RPI = 1024 / KB;          // rows per DMA instruction
  constexpr int NI = G2M / RPI / NW;      // A DMA instructions per wave
  constexpr int NBT = BN / RPI;           // B DMA instructions per block
  constexpr int NIB = (NBT + NW - 1) / NW;     // B DMA slots per wave
  constexpr int NBF = NBT - NW * (NIB - 1);  // waves [0, NBF) fill all NIB slots
  constexpr int PI = NI + NIB;            // DMA instructions per wave per k-tile (waves < NBF)
  constexpr int PI1 = NBF == NW ? PI : PI - 1;  // (waves >= NBF)
  constexpr int KS = KB * MF / 1024;      // MFMA k-steps per k-tile (32 or 64 bytes deep)
  static_assert(BN % RPI == 0 && TI * MF * (NW / S::WN) == G2M && G2M % (RPI * NW) == 0, "tile shape");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[g2_smem(KB, ST)];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WN, wn = wave % S::WN;
  const bool bfull = NBF == NW || wave < NBF;
  int tm, tn, z;
  g2_tile<MAP>(blockIdx.x, nM, nN, tm, tn, z);
  const int m0 = tm * G2M, n0 = tn * BN;
  const int nk = K * 2 / KB;

  // This thread's DMA sources: A rows (wave*NI + j)*RPI + lane/(KB/16), B row
  // blocks wave*NIB + j (256 columns) or NW*j + wave (224 columns, the last
  // slot of waves >= NBF unused), chunk chosen so that LDS slot (row,
  // lane % (KB/16)) holds the swizzled chunk (the swizzle is an XOR, its own
  // inverse).
  auto bblk = [&](int j) { return BN == 224 ? NW * j + wave : wave * NIB + j; };
  const char *pa[NI], *pb[NIB];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    int row = (wave * NI + j) * RPI + lane / (KB / 16);
    pa[j] = ap.row(z, m0 + row) + g2_swz<KB>(row, lane % (KB / 16)) * 16;
  }
#pragma unroll
  for (int j = 0; j < NIB; ++j) {
    int row = (bblk(j) < NBT ? bblk(j) : NBT - 1) * RPI + lane / (KB / 16);
    pb[j] = bp.row(z, n0, row) + g2_swz<KB>(row, lane % (KB / 16)) * 16;
  }
  auto issue = [&](int kt, int stage) {
    unsigned char *As = smem + stage * STAGE, *Bs = As + G2M * KB;
#pragma unroll
    for (int j = 0; j < NIB; ++j) {
      if (j < NI) dma16(pa[j] + kt * KB, As + (wave * NI + j) * 1024);
      if (j + 1 < NIB || bfull) dma16(pb[j] + kt * KB, Bs + bblk(j) * 1024);
    }
#pragma unroll
    for (int j = NIB; j < NI; ++j) dma16(pa[j] + kt * KB, As + (wave * NI + j) * 1024);
  };

  Acc acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = Acc{};

  // Fragments of k-step ks+1 are read from LDS while the MFMAs of step ks run.
  // A 32x32x16 operand: lane row lane % 32, 16-byte k chunk lane / 32; a
  // 16x16x32 operand: row lane % 16, chunk lane / 16.
  auto frags = [&](const unsigned char *As, const unsigned char *Bs, int ks, u32x4 *af, u32x4 *bfr) {
    const int c = (64 / MF) * ks + lane / MF;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      int r = wm * TI * MF + i * MF + lane % MF;
      af[i] = *(const u32x4 *)(As + r * KB + g2_swz<KB>(r, c) * 16);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      int r = wn * TJ * MF + j * MF + lane % MF;
      bfr[j] = *(const u32x4 *)(Bs + r * KB + g2_swz<KB>(r, c) * 16);
    }
  };
  // Wait until at most `later` k-tiles after the awaited one are in flight
  // (counts per wave: the waves issue PI or PI1 DMAs per k-tile).
  auto wait_tiles = [&](int later) {
    if constexpr (ST >= 4) {
      if (later >= 2) {
        if (bfull) wait_vmcnt<2 * PI>();
        else wait_vmcnt<2 * PI1>();
      } else if (later == 1) {
        if (bfull) wait_vmcnt<PI>();
        else wait_vmcnt<PI1>();
      } else {
        wait_vmcnt<0>();
      }
    } else if constexpr (ST == 3) {
      if (later >= 1) {
        if (bfull) wait_vmcnt<PI>();
        else wait_vmcnt<PI1>();
      } else {
        wait_vmcnt<0>();
      }
    } else {
      wait_vmcnt<0>();
    }
  };
  auto mfmas = [&](const u32x4 *af, const u32x4 *bfr) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if constexpr (MF == 32)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                              __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                              __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j], 0, 0, 0);
      }
  };
  // Fragment reads spread over the MFMAs (2 : 1 where there are enough
  // MFMAs), so LDS latency hides under them.
  auto interleave = [&]() {
    // NR reads among NMF MFMAs: N2 groups of 2 MFMAs + 1 read, then N1 of 1 + 1
    // (with fewer MFMAs than reads the last reads are left to the compiler)
    constexpr int NR = TI + TJ, NMF = TI * TJ;
    if constexpr (NMF > 2 * NR) {
      // (more than two MFMAs per read: the reads spread evenly)
      g2_spread<NMF, NR>(std::make_integer_sequence<int, NR>{});
    } else {
      constexpr int N2 = NMF > NR ? NMF - NR : 0, N1 = NMF > NR ? NR - N2 : NMF;
#pragma unroll
      for (int g = 0; g < N2; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
#pragma unroll
      for (int g = 0; g < N1; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
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
  u32x4 fa[2][TI], fb[2][TJ];
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
    __builtin_amdgcn_sched_group_barrier(0x020, PI1, 0);  // DMA issue first
    interleave();
  }
  __syncthreads();

  // epilogue in two 128-row halves; accumulator (lane, e) of a 32x32 tile is
  // row 8*(e/4) + 4*(lane/32) + e%4, column lane%32; of a 16x16 tile row
  // 4*(lane/16) + e, column lane%16.
  constexpr int CP = BN + 4;  // C tile pitch (floats)
  float *Cs = (float *)smem;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r0 = wm * TI * MF - h * 128;  // this wave's first row within the half
    if (r0 >= 0 && r0 < 128) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          if constexpr (MF == 32) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              Cs[(r0 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * CP + wn * TJ * 32 + j * 32 +
                 (lane & 31)] = acc[i][j][e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              Cs[(r0 + i * 16 + 4 * (lane >> 4) + e) * CP + wn * TJ * 16 + j * 16 + (lane & 15)] = acc[i][j][e];
          }
        }
    }
    __syncthreads();
    if constexpr (BN == G2N)
      run_epi<bf16, G2N / 64>(ep, z, m0 + h * 128, n0, Cs, CP, 128, M, N, (float *)(smem + G2CT));
    else  // (only epilogues that take a tile width)
      run_epi<bf16, 4>(ep, z, m0 + h * 128, n0, Cs, CP, 128, M, N, (float *)(smem + G2CT), BN);
    __syncthreads();
  }
}

template <int KB = G2KB, int ST = G2ST, int MAP = 2, int SH = 0, class AP, class BP, class EP>
hipError_t launch_gemm2(const AP &ap, const BP &bp, const EP &ep, int M, int N, int K, int Z, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  constexpr int BN = G2Shape<SH>::BN;
  const int nM = (M + G2M - 1) / G2M, nN = (N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm2_kernel<KB, ST, MAP, SH, AP, BP, EP>), dim3(nM * nN * Z), dim3(64 * G2Shape<SH>::NW), 0, s,
                     ap, bp, ep, M, N, K, nM, nN);
  return hipGetLastError();
}

// Column tile of the residual products: 224 where that needs fewer rounds of
// blocks over the compute units than 256 (e.g. 1792 columns over 8192 rows:
// 256 blocks instead of 224), counted in column-tile widths per unit.
inline int g2_resid_bn(int M, int N, int cus) {
  const long nM = (M + G2M - 1) / G2M;
  const long r256 = (nM * ((N + 255) / 256) + cus - 1) / cus, r224 = (nM * ((N + 223) / 224) + cus - 1) / cus;
  return r224 * 224 < r256 * 256 ? 224 : 256;
}

}  // namespace wm
