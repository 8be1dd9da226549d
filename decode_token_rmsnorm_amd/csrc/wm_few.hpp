// wm_few.hpp — GEMM for few rows (decode steps, small token groups):
// C[M, N] = A[M, K] * B[N, K]^T with M <= kFewRows.
//
// With so few rows the product streams the weight matrix B once, and the
// time goes into memory round trips (about 1.6 us each from HBM) and into how
// many loads each compute unit can keep in flight, not into bandwidth or
// MFMA.  So the work is cut into many small blocks: a block owns 16 rows x TN
// columns (TN = 16..128) over the whole of K, its NWK waves (4..16) split K
// into contiguous ranges, and every wave issues all loads of a round of up to
// R 64-byte k-steps before its first MFMA, so a typical product costs one
// memory round trip.  Fragments go from global memory straight into the
// 16x16x32 MFMA operand registers (row or column lane%16, k-slice lane/16).
// The waves' partial tiles are summed through LDS in wave order (results are
// deterministic) and the block then runs a narrow-tile epilogue on its
// 16 x TN tile.
//
// Narrow-tile epilogues: thread t of the block takes tile row t / (TN/4) and
// the 4 contiguous columns 4*(t % (TN/4)), so the TN/4 lanes of a row are
// adjacent in one wave and row reductions are shuffles among them.  Epilogues
// that normalise per attention head (q, cached keys) use TN = head dim.
#pragma once

#include "wm_gemm.hpp"
#include "wm_host.hpp"

namespace wm {

constexpr int FM = 16;  // rows per block

template <int TN> struct FewCfg {
  static constexpr int NWK = TN == 128 ? 8 : 16;  // most waves per block
  static constexpr int R = TN == 128 ? 2 : 4;     // k-steps per wave and round
  static constexpr int P = TN + 4;                // LDS tile pitch (floats)
};

// B operand of the fused gate/up projection on a TN-wide tile: tile rows
// [0, TN/2) are gate rows, [TN/2, TN) the matching up rows.
template <typename T> struct FGateUp {
  const T *gate, *up;
  int64_t ld;
  int F, half;
  typedef const char *H;
  __device__ __forceinline__ H row(int z, int n0, int jl, int N) const {
    const bool g = jl < half;
    int f = n0 / 2 + (g ? jl : jl - half);
    f = f < F ? f : F - 1;
    return (const char *)((g ? gate : up) + (int64_t)f * ld);
  }
  __device__ __forceinline__ u32x4 load(H h, int kbyte) const { return *(const u32x4 *)(h + kbyte); }
};

// ---------------------------------------------------------------- epilogues
// run_epi_few(ep, z, m0, n0, Cs, P, M, N, rowbuf): Cs = the 16 x TN fp32 tile
// (pitch P), tile row rl = output row m0 + rl, first column n0.  Every thread
// of the block calls it (row-scale set-up synchronises the block).

// h += C; hb = h * gain_next; optionally S_next = h; the row's sum of squares
// over the tile's columns -> ss_out[r, n0 / TN].
template <typename T, int TN>
__device__ __forceinline__ void run_epi_few(const EpiResid<T> &e, int z, int m0, int n0, const float *Cs, int P,
                                            int M, int N, float *rowbuf) {
  constexpr int LPR = TN / 4;
  for (int t = threadIdx.x; t < FM * LPR; t += blockDim.x) {
    const int rl = t / LPR, cq = t - rl * LPR, c = n0 + 4 * cq, r = m0 + rl;
    const bool on = c < N, ok = on && r < M;
    const int cl = on ? c : N - 4;
    const int rc = r < M ? r : M - 1;
    float g[4], hv[4], x[4], xb[4];
    ldf<4>(g, e.gain_next + cl);
    ldf<4>(hv, e.h + (int64_t)rc * N + cl);
    ldf<4>(x, Cs + rl * P + 4 * cq);
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] += hv[i];
      xb[i] = x[i] * g[i];
      sq += x[i] * x[i];
    }
    if (ok) {
      const int64_t o = (int64_t)r * N + c;
      stf<4>(e.h + o, x);
      stT<T, 4>(e.hb + o, xb);
      if (e.S_next) stT<T, 4>(e.S_next + o, x);
    } else {
      sq = 0.f;
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) sq += __shfl_xor(sq, o);
    if (cq == 0 && r < M) e.ss_out[(int64_t)r * e.nparts_out + n0 / TN] = sq;
  }
}

// act[r, n0/2 + f] = silu(rs * gate) * (rs * up); gate columns [0, TN/2) of
// the tile, up columns [TN/2, TN).
template <typename T, int TN>
__device__ __forceinline__ void run_epi_few(const EpiSwiGLU<T> &e, int z, int m0, int n0, const float *Cs, int P,
                                            int M, int N, float *rowbuf) {
  constexpr int LPR = TN / 8;  // 4 outputs per thread
  fill_rowbuf_parts(rowbuf, e.ss, nullptr, e.nparts, e.invD, e.eps, m0, FM, M);
  for (int t = threadIdx.x; t < FM * LPR; t += blockDim.x) {
    const int rl = t / LPR, cq = t - rl * LPR, f = n0 / 2 + 4 * cq, r = m0 + rl;
    if (r >= M || f >= e.F) continue;
    const float rs = rowbuf[rl];
    float gt[4], up[4], y[4];
    ldf<4>(gt, Cs + rl * P + 4 * cq);
    ldf<4>(up, Cs + rl * P + TN / 2 + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = silu(gt[i] * rs) * (up[i] * rs);
    stT<T, 4>(e.act + (int64_t)r * e.F + f, y);
  }
}

// q = RoPE(RMSNorm_head(rinv_row * C; q_norm)); TN = head dim.
template <typename T, int TN>
__device__ __forceinline__ void run_epi_few(const EpiQ<T> &e, int z, int m0, int n0, const float *Cs, int P, int M,
                                            int N, float *rowbuf) {
  constexpr int LPR = TN / 4;
  fill_rowbuf_parts(rowbuf, e.ss, nullptr, e.nparts, e.invD, e.eps, m0, FM, M);
  const int lane = threadIdx.x & 63;
  for (int t = threadIdx.x; t < FM * LPR; t += blockDim.x) {  // whole waves: FM * LPR is a multiple of 64
    const int rl = t / LPR, cq = t - rl * LPR, r = m0 + rl;
    const int rc = r < M ? r : M - 1;
    float g[4], cs[1][4], sn[1][4], x[1][4];
    ldf<4>(g, e.qnorm + 4 * cq);
    rope_entries<4>(cs[0], sn[0], e.cosT, e.sinT, e.rp.pos(rc), lane, TN);
    ldf<4>(x[0], Cs + rl * P + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[0][i] *= rowbuf[rl];
    head_norm_rope<4, 1>(x, lane, TN, e.eps, g, cs, sn);
    if (r < M) stT<T, 4>(e.q + (int64_t)r * N + n0 + 4 * cq, x[0]);
  }
}

// Pool projection, z = beta*k + j: rows scaled by the channel's 1/rms; keys
// get the per-head key norm and RoPE; both go to cache[j, b, h, pos, :].
// TN = head dim, so the block's columns are head n0 / TN.
template <typename T, int TN>
__device__ __forceinline__ void run_epi_few(const EpiKV<T> &e, int z, int m0, int n0, const float *Cs, int P, int M,
                                            int N, float *rowbuf) {
  constexpr int LPR = TN / 4;
  const int beta = z / e.k, j = z - beta * e.k, hh = n0 / TN;
  for (int rl = threadIdx.x; rl < FM; rl += blockDim.x) {
    const int r = m0 + rl;
    rowbuf[rl] = r < M ? e.rinvM[(int64_t)z * e.rows + r] : 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  T *base = beta == 0 ? e.Kc : e.Vc;
  for (int t = threadIdx.x; t < FM * LPR; t += blockDim.x) {  // whole waves
    const int rl = t / LPR, cq = t - rl * LPR, r = m0 + rl;
    const int rc = r < M ? r : M - 1;
    float x[1][4];
    ldf<4>(x[0], Cs + rl * P + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[0][i] *= rowbuf[rl];
    if (beta == 0) {
      float g[4], cs[1][4], sn[1][4];
      ldf<4>(g, e.knorm + (int64_t)j * TN + 4 * cq);
      rope_entries<4>(cs[0], sn[0], e.cosT, e.sinT, e.rp.pos(rc), lane, TN);
      head_norm_rope<4, 1>(x, lane, TN, e.eps, g, cs, sn);
    }
    if (r < M) {
      const int pos = e.rp.pos(r), b = e.rp.seq(r);
      stT<T, 4>(base + ((((int64_t)j * e.B + b) * e.Hkv + hh) * e.T_max + pos) * TN + 4 * cq, x[0]);
    }
  }
}

// out[(map ? map[r] : r) * ldo + c] (+ z * zstride) = rs * C, rs from
// partial sums of squares when ss is given.
template <typename T, int TN>
__device__ __forceinline__ void run_epi_few(const EpiStoreF32 &e, int z, int m0, int n0, const float *Cs, int P,
                                            int M, int N, float *rowbuf) {
  constexpr int LPR = TN / 4;
  if (e.ss) fill_rowbuf_parts(rowbuf, e.ss, e.ss_rows, e.nparts, e.invD, e.eps, m0, FM, M);
  const bool vec = ((e.ldo | e.zstride) & 3) == 0;
  for (int t = threadIdx.x; t < FM * LPR; t += blockDim.x) {
    const int rl = t / LPR, cq = t - rl * LPR, c = n0 + 4 * cq, r = m0 + rl;
    if (r >= M || c >= N) continue;
    const float rs = e.ss ? rowbuf[rl] : 1.f;
    const int64_t orow = e.out_rows ? e.out_rows[r] : r;
    float *dst = e.out + z * e.zstride + orow * e.ldo + c;
    float x[4];
    ldf<4>(x, Cs + rl * P + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= rs;
    if (vec && c + 4 <= N) {
      stf<4>(dst, x);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c + i < N) dst[i] = x[i];
    }
  }
}

// ---------------------------------------------------------------- kernel
// Grid (ceil(N / TN), ceil(M / FM), Z); block 64 * nwk threads, nwk <= NWK.
template <typename T, int TN, class AL, class BL, class EP>
__global__ __launch_bounds__(64 * FewCfg<TN>::NWK) void gemm_few(AL al, BL bl, EP ep, int M, int N, int K) {
  constexpr int NJ = TN / 16, R = FewCfg<TN>::R, P = FewCfg<TN>::P;
  __shared__ __attribute__((aligned(16))) float part[FewCfg<TN>::NWK * FM * P + FM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwk = blockDim.x >> 6;
  const int z = blockIdx.z, m0 = blockIdx.y * FM, n0 = blockIdx.x * TN;
  const int rl = lane & 15, kl = (lane >> 4) * 16;
  const int nks = (int)((int64_t)K * (int64_t)sizeof(T) / 64);
  const int per = (nks + nwk - 1) / nwk, s0 = min(wave * per, nks), s1 = min(s0 + per, nks);

  const typename AL::H ha = al.row(z, m0 + rl, M);
  typename BL::H hb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) hb[j] = bl.row(z, n0, j * 16 + rl, N);
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s1; s += R) {
    // a round: R k-steps, all loads first; a step past the range re-reads the
    // last one and is multiplied with its A fragment masked to zero
    u32x4 a[R], b[R][NJ];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int kb = min(s + u, s1 - 1) * 64 + kl;
      a[u] = al.load(ha, kb);
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[u][j] = bl.load(hb[j], kb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const u32x4 am = a[u] & (s + u < s1 ? ~0u : 0u);
#pragma unroll
      for (int j = 0; j < NJ; ++j) mma16<T>(acc[j], am, b[u][j]);
    }
  }

  // wave partials -> LDS, summed in wave order into tile 0
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) part[(wave * FM + 4 * (lane >> 4) + e) * P + j * 16 + rl] = acc[j][e];
  __syncthreads();
  for (int idx = tid * 4; idx < FM * TN; idx += blockDim.x * 4) {
    const int r = idx / TN, c = idx - r * TN;
    f32x4 v = *(const f32x4 *)(&part[r * P + c]);
    for (int w = 1; w < nwk; ++w) v += *(const f32x4 *)(&part[(w * FM + r) * P + c]);
    *(f32x4 *)(&part[r * P + c]) = v;
  }
  __syncthreads();
  run_epi_few<T, TN>(ep, z, m0, n0, part, P, M, N, part + FewCfg<TN>::NWK * FM * P);
}

// Waves per block: enough for one round of R k-steps each, 4 at least.
template <int TN> inline int few_waves(int nks) {
  int w = (nks + FewCfg<TN>::R - 1) / FewCfg<TN>::R;
  w = w < 4 ? 4 : w;
  return w > FewCfg<TN>::NWK ? FewCfg<TN>::NWK : w;
}

// A loader's view of the tile width (the gate/up split sits at TN/2).
template <class BL> inline BL few_bind(const BL &b, int) { return b; }
template <typename T> inline FGateUp<T> few_bind(const FGateUp<T> &b, int tn) {
  FGateUp<T> r = b;
  r.half = tn / 2;
  return r;
}

template <typename T, int TN, class AL, class BL, class EP>
hipError_t launch_few_tn(const AL &al, const BL &bl, const EP &ep, int M, int N, int K, int Z, hipStream_t s) {
  const int nks = (int)((int64_t)K * (int64_t)sizeof(T) / 64);
  dim3 grid((N + TN - 1) / TN, (M + FM - 1) / FM, Z);
  hipLaunchKernelGGL((gemm_few<T, TN, AL, BL, EP>), grid, dim3(64 * few_waves<TN>(nks)), 0, s, al, few_bind(bl, TN), ep,
                     M, N, K);
  return hipGetLastError();
}

// Tile width of an epilogue that works per attention head: its head dim.
template <class EP> struct FewHead {
  static constexpr bool value = false;
  static int width(const EP &) { return 0; }
};
template <typename T> struct FewHead<EpiQ<T>> {
  static constexpr bool value = true;
  static int width(const EpiQ<T> &e) { return e.d; }
};
template <typename T> struct FewHead<EpiKV<T>> {
  static constexpr bool value = true;
  static int width(const EpiKV<T> &e) { return e.d; }
};

// Tile width for other epilogues: the narrowest of 16, 32, 64 that keeps the
// grid within about one block per compute unit.
inline int few_width(int M, int N, int Z) {
  int tn = 16;
  while (tn < 64 && (int64_t)((N + tn - 1) / tn) * ((M + FM - 1) / FM) * Z > 256) tn *= 2;
  return tn;
}

// Number of partial sums of squares a residual epilogue writes per row.
inline int few_parts(int M, int N) {
  const int tn = few_width(M, N, 1);
  return (N + tn - 1) / tn;
}

template <typename T, class AL, class BL, class EP>
hipError_t launch_few(const AL &al, const BL &bl, const EP &ep, int M, int N, int K, int Z, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  // (k in whole 64-byte steps; the model's widths make every other output
  // width a multiple of 4, the plain store handles any)
  if (((int64_t)K * (int64_t)sizeof(T)) % 64 != 0) return hipErrorInvalidValue;
  if constexpr (FewHead<EP>::value) {
    switch (FewHead<EP>::width(ep)) {
      case 32: return launch_few_tn<T, 32>(al, bl, ep, M, N, K, Z, s);
      case 64: return launch_few_tn<T, 64>(al, bl, ep, M, N, K, Z, s);
      case 128: return launch_few_tn<T, 128>(al, bl, ep, M, N, K, Z, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (few_width(M, N, Z)) {
      case 16: return launch_few_tn<T, 16>(al, bl, ep, M, N, K, Z, s);
      case 32: return launch_few_tn<T, 32>(al, bl, ep, M, N, K, Z, s);
      default: return launch_few_tn<T, 64>(al, bl, ep, M, N, K, Z, s);
    }
  }
}

}  // namespace wm
