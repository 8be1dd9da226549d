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
// adjacent in one wave and row reductions are shuffles among them.  Each
// epilogue issues the global loads it needs (residual rows, gains, RoPE table
// entries, the row's partial sums of squares) before the main loop, so they
// travel with the operand loads and the epilogue itself makes no round trip.
// A row's RMSNorm scale comes from its partial sums spread over the row's
// lanes and added with shuffles.  Epilogues that normalise per attention head
// (q, cached keys) use TN = head dim.
#pragma once

#include "wm_gemm.hpp"
#include "wm_host.hpp"

namespace wm {

constexpr int FM = 16;  // rows per MFMA block

// TR row blocks of 16 per block (4 only for wide plain stores, where the
// weight matrix is then read once instead of once per 16 rows).
template <int TN, int TR> struct FewCfg {
  static constexpr int NWK = (TN >= 64 || TR > 1) ? 8 : 16;  // most waves per block
  static constexpr int R = 4;                                // k-steps per wave and round
  static constexpr int P = TN + 4;                           // LDS tile pitch (floats)
  static constexpr int ROWS = FM * TR;
};

// Sum over the partial sums of squares p < nparts of one row, spread over the
// LPR lanes of the row (lane cq loads p = cq, cq + LPR, ...; the first 8*LPR
// parts are loaded ahead, more are added when summed), then added across the
// lanes with shuffles; every lane of the row gets the sum.
template <int LPR> struct PartSum {
  static constexpr int NL = 8;
  float v[NL];
  const float *row;
  int np, cq;
  __device__ __forceinline__ void load(const float *ss, int64_t ssrow, int nparts, int lane_cq) {
    row = ss + ssrow * nparts;
    np = nparts;
    cq = lane_cq;
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = row[min(cq + LPR * i, np - 1)];
  }
  __device__ __forceinline__ float sum() const {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) s += cq + LPR * i < np ? v[i] : 0.f;
    for (int p = cq + LPR * NL; p < np; p += LPR) s += row[p];
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
    return s;
  }
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
// FewEpi<EP, T, TN, ROWS>: load(...) before the main loop, run(...) on the
// reduced ROWS x TN tile Cs (pitch P) in LDS; tile row rl is output row
// m0 + rl, first column n0.  Thread t < NT = ROWS * LPR owns one (row, 4
// columns) item, and blocks have at least NT threads.
template <class EP, typename T, int TN, int ROWS> struct FewEpi;

// h += C; hb = h * gain_next; optionally S_next = h; the row's sum of squares
// over the tile's columns -> ss_out[r, n0 / TN].
template <typename T, int TN, int ROWS> struct FewEpi<EpiResid<T>, T, TN, ROWS> {
  static constexpr int LPR = TN / 4, NT = ROWS * LPR;
  float g[4], hv[4];
  __device__ __forceinline__ void load(const EpiResid<T> &e, int z, int m0, int n0, int M, int N) {
    const int t = min((int)threadIdx.x, NT - 1), rl = t / LPR, cq = t - rl * LPR, c = n0 + 4 * cq;
    const int cl = c < N ? c : N - 4, rc = min(m0 + rl, M - 1);
    ldf<4>(g, e.gain_next + cl);
    ldf<4>(hv, e.h + (int64_t)rc * N + cl);
  }
  __device__ __forceinline__ void run(const EpiResid<T> &e, int z, int m0, int n0, const float *Cs, int P, int M,
                                      int N) {
    const int t = threadIdx.x;
    if (t >= NT) return;  // (whole waves: NT is a multiple of 64 or the block's only wave)
    const int rl = t / LPR, cq = t - rl * LPR, c = n0 + 4 * cq, r = m0 + rl;
    const bool ok = c < N && r < M;
    float x[4], xb[4];
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
};

// act[r, n0/2 + f] = silu(rs * gate) * (rs * up); gate columns [0, TN/2) of
// the tile, up columns [TN/2, TN); 4 outputs per thread.
template <typename T, int TN, int ROWS> struct FewEpi<EpiSwiGLU<T>, T, TN, ROWS> {
  static constexpr int LPR = TN / 8, NT = ROWS * LPR;
  PartSum<LPR> ps;
  __device__ __forceinline__ void load(const EpiSwiGLU<T> &e, int z, int m0, int n0, int M, int N) {
    const int t = min((int)threadIdx.x, NT - 1), rl = t / LPR, cq = t - rl * LPR;
    ps.load(e.ss, min(m0 + rl, M - 1), e.nparts, cq);
  }
  __device__ __forceinline__ void run(const EpiSwiGLU<T> &e, int z, int m0, int n0, const float *Cs, int P, int M,
                                      int N) {
    const int t = threadIdx.x;
    if (t >= NT) return;
    const int rl = t / LPR, cq = t - rl * LPR, f = n0 / 2 + 4 * cq, r = m0 + rl;
    const float rs = rsqrtf(ps.sum() * e.invD + e.eps);  // (shuffles: all lanes of the row)
    if (r >= M || f >= e.F) return;
    float gt[4], up[4], y[4];
    ldf<4>(gt, Cs + rl * P + 4 * cq);
    ldf<4>(up, Cs + rl * P + TN / 2 + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = silu(gt[i] * rs) * (up[i] * rs);
    stT<T, 4>(e.act + (int64_t)r * e.F + f, y);
  }
};

// q = RoPE(RMSNorm_head(rinv_row * C; q_norm)); TN = head dim.
template <typename T, int TN, int ROWS> struct FewEpi<EpiQ<T>, T, TN, ROWS> {
  static constexpr int LPR = TN / 4, NT = ROWS * LPR;
  PartSum<LPR> ps;
  float g[4], cs[1][4], sn[1][4];
  __device__ __forceinline__ void load(const EpiQ<T> &e, int z, int m0, int n0, int M, int N) {
    const int t = min((int)threadIdx.x, NT - 1), rl = t / LPR, cq = t - rl * LPR, rc = min(m0 + rl, M - 1);
    ps.load(e.ss, rc, e.nparts, cq);
    ldf<4>(g, e.qnorm + 4 * cq);
    rope_entries<4>(cs[0], sn[0], e.cosT, e.sinT, e.rp.pos(rc), threadIdx.x & 63, TN);
  }
  __device__ __forceinline__ void run(const EpiQ<T> &e, int z, int m0, int n0, const float *Cs, int P, int M,
                                      int N) {
    const int t = threadIdx.x;
    if (t >= NT) return;
    const int rl = t / LPR, cq = t - rl * LPR, r = m0 + rl;
    const float rs = rsqrtf(ps.sum() * e.invD + e.eps);
    float x[1][4];
    ldf<4>(x[0], Cs + rl * P + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[0][i] *= rs;
    head_norm_rope<4, 1>(x, t & 63, TN, e.eps, g, cs, sn);
    if (r < M) stT<T, 4>(e.q + (int64_t)r * N + n0 + 4 * cq, x[0]);
  }
};

// The q epilogue on its own, for few-row Q products with 128-dim heads, whose
// fused form (one 128-column head per block) leaves most compute units idle
// at the 1.3B widths (14 column tiles): the product then runs on narrow tiles
// into a raw fp32 buffer C [rows, Hq*d], and one wave per (row, head) applies
// q = RoPE(RMSNorm_head(rinv_row * C; q_norm)), two elements per lane.
template <typename T>
__global__ __launch_bounds__(256) void q_epi128(const float *C, T *q, const float *ss, int nparts, float invD,
                                                float eps, const float *qnorm, const float *cosT, const float *sinT,
                                                RowPos rp, int rows, int Hq) {
  constexpr int D = 128, CPL = 2;
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wv >= rows * Hq) return;  // (a whole wave)
  const int r = wv / Hq, hd = wv - r * Hq, c = CPL * lane;
  const float rs = rinv_from_parts(ss, r, nparts, invD, eps);
  float x[1][CPL], g[CPL], cs[1][CPL], sn[1][CPL];
  ldf<CPL>(x[0], C + ((int64_t)r * Hq + hd) * D + c);
  ldf<CPL>(g, qnorm + c);
  rope_entries<CPL>(cs[0], sn[0], cosT, sinT, rp.pos(r), lane, D);
#pragma unroll
  for (int i = 0; i < CPL; ++i) x[0][i] *= rs;
  head_norm_rope<CPL, 1>(x, lane, D, eps, g, cs, sn);
  stT<T, CPL>(q + ((int64_t)r * Hq + hd) * D + c, x[0]);
}

// Pool projection, z = beta*k + j: rows scaled by the channel's 1/rms; keys
// get the per-head key norm and RoPE; both go to cache[j, b, h, pos, :].
// TN = head dim, so the block's columns are head n0 / TN.
template <typename T, int TN, int ROWS> struct FewEpi<EpiKV<T>, T, TN, ROWS> {
  static constexpr int LPR = TN / 4, NT = ROWS * LPR;
  float rs, g[4], cs[1][4], sn[1][4];
  __device__ __forceinline__ void load(const EpiKV<T> &e, int z, int m0, int n0, int M, int N) {
    const int t = min((int)threadIdx.x, NT - 1), rl = t / LPR, cq = t - rl * LPR, rc = min(m0 + rl, M - 1);
    const int beta = z / e.k, j = z - beta * e.k;
    rs = e.rinvM[(int64_t)z * e.rows + rc];
    ldf<4>(g, e.knorm + (int64_t)j * TN + 4 * cq);
    rope_entries<4>(cs[0], sn[0], e.cosT, e.sinT, e.rp.pos(rc), threadIdx.x & 63, TN);
  }
  __device__ __forceinline__ void run(const EpiKV<T> &e, int z, int m0, int n0, const float *Cs, int P, int M,
                                      int N) {
    const int t = threadIdx.x;
    if (t >= NT) return;
    const int rl = t / LPR, cq = t - rl * LPR, r = m0 + rl;
    const int beta = z / e.k, j = z - beta * e.k, hh = n0 / TN;
    float x[1][4];
    ldf<4>(x[0], Cs + rl * P + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[0][i] *= rs;
    if (beta == 0) head_norm_rope<4, 1>(x, t & 63, TN, e.eps, g, cs, sn);
    if (r < M) {
      const int pos = e.rp.pos(r), b = e.rp.seq(r);
      T *base = beta == 0 ? e.Kc : e.Vc;
      stT<T, 4>(base + ((((int64_t)j * e.B + b) * e.Hkv + hh) * e.T_max + pos) * TN + 4 * cq, x[0]);
    }
  }
};

// Vanilla per-layer K/V projection; TN = head dim, the block's columns are
// one head: a key head (key norm, RoPE) when n0 < Hkv*d, else a value head.
template <typename T, int TN, int ROWS> struct FewEpi<EpiKVL<T>, T, TN, ROWS> {
  static constexpr int LPR = TN / 4, NT = ROWS * LPR;
  PartSum<LPR> ps;
  float g[4], cs[1][4], sn[1][4];
  __device__ __forceinline__ void load(const EpiKVL<T> &e, int z, int m0, int n0, int M, int N) {
    const int t = min((int)threadIdx.x, NT - 1), rl = t / LPR, cq = t - rl * LPR, rc = min(m0 + rl, M - 1);
    ps.load(e.ss, rc, e.nparts, cq);
    ldf<4>(g, e.knorm + 4 * cq);
    rope_entries<4>(cs[0], sn[0], e.cosT, e.sinT, e.rp.pos(rc), threadIdx.x & 63, TN);
  }
  __device__ __forceinline__ void run(const EpiKVL<T> &e, int z, int m0, int n0, const float *Cs, int P, int M,
                                      int N) {
    const int t = threadIdx.x;
    if (t >= NT) return;
    const int rl = t / LPR, cq = t - rl * LPR, r = m0 + rl;
    const int hd = e.Hkv * TN;
    const bool isK = n0 < hd;
    const int hh = (isK ? n0 : n0 - hd) / TN;
    const float rs = rsqrtf(ps.sum() * e.invD + e.eps);
    float x[1][4];
    ldf<4>(x[0], Cs + rl * P + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[0][i] *= rs;
    if (isK) head_norm_rope<4, 1>(x, t & 63, TN, e.eps, g, cs, sn);
    if (r < M) {
      const int pos = e.rp.pos(r), b = e.rp.seq(r);
      stT<T, 4>((isK ? e.Kc : e.Vc) + (((int64_t)b * e.Hkv + hh) * e.T_max + pos) * TN + 4 * cq, x[0]);
    }
  }
};

// out[(map ? map[r] : r) * ldo + c] (+ z * zstride) = rs * C, rs from the
// row's partial sums of squares when ss is given (ss row = ss_rows[r] when
// that map is given).
template <typename T, int TN, int ROWS> struct FewEpi<EpiStoreF32, T, TN, ROWS> {
  static constexpr int LPR = TN / 4, NT = ROWS * LPR;
  PartSum<LPR> ps;
  int64_t orow;
  __device__ __forceinline__ void load(const EpiStoreF32 &e, int z, int m0, int n0, int M, int N) {
    const int t = min((int)threadIdx.x, NT - 1), rl = t / LPR, cq = t - rl * LPR, rc = min(m0 + rl, M - 1);
    orow = e.out_rows ? e.out_rows[rc] : rc;
    if (e.ss) ps.load(e.ss, e.ss_rows ? e.ss_rows[rc] : rc, e.nparts, cq);
  }
  __device__ __forceinline__ void run(const EpiStoreF32 &e, int z, int m0, int n0, const float *Cs, int P, int M,
                                      int N) {
    const int t = threadIdx.x;
    if (t >= NT) return;
    const int rl = t / LPR, cq = t - rl * LPR, c = n0 + 4 * cq, r = m0 + rl;
    const float rs = e.ss ? rsqrtf(ps.sum() * e.invD + e.eps) : 1.f;
    if (r >= M || c >= N) return;
    float *dst = e.out + z * e.zstride + orow * e.ldo + c;
    float x[4];
    ldf<4>(x, Cs + rl * P + 4 * cq);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= rs;
    if (((e.ldo | e.zstride) & 3) == 0 && c + 4 <= N) {
      stf<4>(dst, x);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c + i < N) dst[i] = x[i];
    }
  }
};

// ---------------------------------------------------------------- kernel
// Grid (ceil(N / TN), ceil(M / ROWS), Z); block 64 * nwk threads with
// NT / 64 <= nwk <= NWK.
template <typename T, int TN, int TR, class AL, class BL, class EP>
__global__ __launch_bounds__((64 * FewCfg<TN, TR>::NWK)) void gemm_few(AL al, BL bl, EP ep, int M, int N, int K) {
  using C = FewCfg<TN, TR>;
  constexpr int NJ = TN / 16, R = C::R, P = C::P, ROWS = C::ROWS;
  __shared__ __attribute__((aligned(16))) float part[C::NWK * ROWS * P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwk = blockDim.x >> 6;
  const int z = blockIdx.z, m0 = blockIdx.y * ROWS, n0 = blockIdx.x * TN;
  const int rl = lane & 15, kl = (lane >> 4) * 16;
  const int nks = (int)((int64_t)K * (int64_t)sizeof(T) / 64);
  const int per = (nks + nwk - 1) / nwk, s0 = min(wave * per, nks), s1 = min(s0 + per, nks);

  FewEpi<EP, T, TN, ROWS> epi;
  epi.load(ep, z, m0, n0, M, N);  // in flight during the main loop

  typename AL::H ha[TR];
#pragma unroll
  for (int i = 0; i < TR; ++i) ha[i] = al.row(z, m0 + i * FM + rl, M);
  typename BL::H hb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) hb[j] = bl.row(z, n0, j * 16 + rl, N);
  f32x4 acc[TR][NJ];
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s1; s += R) {
    // a round: R k-steps, all loads first; a step past the range re-reads the
    // last one and is multiplied with its A fragments masked to zero
    u32x4 a[R][TR], b[R][NJ];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int kb = min(s + u, s1 - 1) * 64 + kl;
#pragma unroll
      for (int i = 0; i < TR; ++i) a[u][i] = al.load(ha[i], kb);
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[u][j] = bl.load(hb[j], kb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const uint32_t msk = s + u < s1 ? ~0u : 0u;
#pragma unroll
      for (int i = 0; i < TR; ++i) {
        const u32x4 am = a[u][i] & msk;
#pragma unroll
        for (int j = 0; j < NJ; ++j) mma16<T>(acc[i][j], am, b[u][j]);
      }
    }
  }

  // wave partials -> LDS, summed in wave order into tile 0
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part[(wave * ROWS + i * FM + 4 * (lane >> 4) + e) * P + j * 16 + rl] = acc[i][j][e];
  __syncthreads();
  for (int idx = tid * 4; idx < ROWS * TN; idx += blockDim.x * 4) {
    const int r = idx / TN, c = idx - r * TN;
    f32x4 v = *(const f32x4 *)(&part[r * P + c]);
    for (int w = 1; w < nwk; ++w) v += *(const f32x4 *)(&part[(w * ROWS + r) * P + c]);
    *(f32x4 *)(&part[r * P + c]) = v;
  }
  __syncthreads();
  epi.run(ep, z, m0, n0, part, P, M, N);
}

// ---------------------------------------------------------------- wide outputs
// C = A B^T for at most 64 rows and many columns (the vocabulary projection),
// stored as fp32 by EpiStoreF32.  A block of 8 waves owns 64 rows x 128
// columns; it stages the 64 A rows of a k chunk in LDS once (so the weight
// matrix B is the only stream from memory and is read once), each wave takes
// 16 columns: its B fragments come straight from global memory, all loads of
// the chunk issued before the first MFMA, and the A fragments of its 4 row
// blocks from LDS.  The row scales (RMSNorm from partial sums of squares) are
// loaded before the main loop and reduced over 8 lanes per row.
constexpr int WM_ROWS = 64, WM_COLS = 128, WM_KC = 1024;  // rows, columns, k bytes per chunk and row
constexpr int WM_AP = WM_KC + 16;                        // LDS row pitch (bytes)

template <typename T, class AL, class BL>
__global__ __launch_bounds__(512) void gemm_wide(AL al, BL bl, EpiStoreF32 ep, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) char As[WM_ROWS * WM_AP];
  __shared__ float rsc[WM_ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int z = blockIdx.z, m0 = blockIdx.y * WM_ROWS, n0 = blockIdx.x * WM_COLS + 16 * wave;
  const int rl = lane & 15, kl = (lane >> 4) * 16;
  const int64_t kbytes = (int64_t)K * (int64_t)sizeof(T);
  // row scales: 8 lanes per row
  {
    const int row = tid >> 3, rc = min(m0 + row, M - 1);
    PartSum<8> ps;
    if (ep.ss) ps.load(ep.ss, ep.ss_rows ? ep.ss_rows[rc] : rc, ep.nparts, tid & 7);
    const float s = ep.ss ? ps.sum() : 0.f;
    if ((tid & 7) == 0) rsc[row] = ep.ss ? rsqrtf(s * ep.invD + ep.eps) : 1.f;
  }
  // A rows of a chunk: 64 rows x WM_KC bytes, 16 bytes per load, WM_KC / 128 per thread
  const int arow = tid >> 3;
  const typename AL::H ha = al.row(z, m0 + arow, M);
  const typename BL::H hb = bl.row(z, blockIdx.x * WM_COLS, 16 * wave + rl, N);
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < kbytes; k0 += WM_KC) {
    const int nst = (int)min((int64_t)WM_KC, kbytes - k0) / 64;  // 64-byte k-steps in the chunk
    constexpr int NA = WM_KC / 128;
    u32x4 b[WM_KC / 64], a[NA];
#pragma unroll
    for (int u = 0; u < WM_KC / 64; ++u) b[u] = bl.load(hb, (int)(k0 + min(u, nst - 1) * 64 + kl));
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int off = min(16 * ((tid & 7) + 8 * i), nst * 64 - 16);
      a[i] = al.load(ha, (int)(k0 + off));
    }
    __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
    for (int i = 0; i < NA; ++i)
      *(u32x4 *)(&As[arow * WM_AP + min(16 * ((tid & 7) + 8 * i), nst * 64 - 16)]) = a[i];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < WM_KC / 64; ++u) {
      if (u < nst) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          mma16<T>(acc[i], *(const u32x4 *)(&As[(16 * i + rl) * WM_AP + u * 64 + kl]), b[u]);
      }
    }
  }
  // lane: rows 16i + 4(lane/16) + e, column n0 + lane%16
  const int c = n0 + rl;
  if (c >= N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = 16 * i + 4 * (lane >> 4) + e, r = m0 + rr;
      if (r < M) {
        const int64_t orow = ep.out_rows ? ep.out_rows[r] : r;
        ep.out[z * ep.zstride + orow * ep.ldo + c] = acc[i][e] * rsc[rr];
      }
    }
}

// Waves per block: enough for one round of R k-steps each, and at least 4
// and enough for one epilogue item per thread.
template <int TN, int TR, int NT> inline int few_waves(int nks) {
  using C = FewCfg<TN, TR>;
  static_assert(NT <= 64 * C::NWK, "epilogue items exceed the block");
  int w = (nks + C::R - 1) / C::R;
  const int lo = NT / 64 > 4 ? NT / 64 : 4;
  w = w < lo ? lo : w;
  return w > C::NWK ? C::NWK : w;
}

// A loader's view of the tile width (the gate/up split sits at TN/2).
template <class BL> inline BL few_bind(const BL &b, int) { return b; }
template <typename T> inline FGateUp<T> few_bind(const FGateUp<T> &b, int tn) {
  FGateUp<T> r = b;
  r.half = tn / 2;
  return r;
}

template <typename T, int TN, int TR, class AL, class BL, class EP>
hipError_t launch_few_tn(const AL &al, const BL &bl, const EP &ep, int M, int N, int K, int Z, hipStream_t s) {
  constexpr int ROWS = FewCfg<TN, TR>::ROWS;
  const int nks = (int)((int64_t)K * (int64_t)sizeof(T) / 64);
  const int nX = (N + TN - 1) / TN, nY = (M + ROWS - 1) / ROWS;
  int nw = few_waves<TN, TR, FewEpi<EP, T, TN, ROWS>::NT>(nks);
  // more blocks than compute units: the fewest waves the epilogue allows, so
  // that more blocks are resident at once (at 8 waves, blocks whose
  // registers admit 12 waves per CU run one per CU; the 1.3B-shape decode's
  // gate/up product, 608 blocks: 37.5 -> 34.3 us)
  {
    constexpr int NT = FewEpi<EP, T, TN, ROWS>::NT, lo = NT / 64 > 4 ? NT / 64 : 4;
    if ((int64_t)nX * nY * Z > 256 && nw > lo) nw = lo;
  }
  hipLaunchKernelGGL((gemm_few<T, TN, TR, AL, BL, EP>), dim3(nX, nY, Z), dim3(64 * nw), 0, s, al, few_bind(bl, TN), ep,
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
template <typename T> struct FewHead<EpiKVL<T>> {
  static constexpr bool value = true;
  static int width(const EpiKVL<T> &e) { return e.d; }
};

// Tile width for other epilogues: the narrowest of 16, 32, 64 that keeps the
// grid within about one block per compute unit.
inline int few_width(int M, int N, int Z) {
  int tn = 16;
  while (tn < 64 && (int64_t)((N + tn - 1) / tn) * ((M + FM - 1) / FM) * Z > 256) tn *= 2;
  return tn;
}

// Outputs wide enough that 16-row blocks of 64 columns would pass 1024 blocks.
inline bool few_wide(int M, int N, int Z) {
  return (int64_t)((N + 63) / 64) * ((M + FM - 1) / FM) * Z > 1024;
}

// Residual products of at least kFewTallRows rows over at least kFewTallK
// of k run on 64-row blocks (4 row blocks of 16, 32 columns), which read
// their weight columns once per 64 rows instead of 16 (the small model's
// 1024-row down product, k = 1536: 24.9 -> 18.6 us; its 512-deep O product
// is faster on 16-row blocks, 10.7 against 12.0 us).
constexpr int kFewTallRows = 512, kFewTallK = 1024;
inline bool few_tall(int M, int K) { return M >= kFewTallRows && K >= kFewTallK; }

// Number of partial sums of squares a residual epilogue writes per row (the
// product's k range decides its tile shape).
inline int few_parts(int M, int N, int K) {
  if (few_tall(M, K)) return (N + 31) / 32;
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
      case 32: return launch_few_tn<T, 32, 1>(al, bl, ep, M, N, K, Z, s);
      case 64: return launch_few_tn<T, 64, 1>(al, bl, ep, M, N, K, Z, s);
      case 128: return launch_few_tn<T, 128, 1>(al, bl, ep, M, N, K, Z, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    if constexpr (std::is_same<EP, EpiStoreF32>::value) {
      // wide outputs over more than 16 rows: 64-row blocks, the weights read once
      if (M > FM && few_wide(M, N, Z)) {
        dim3 grid((N + WM_COLS - 1) / WM_COLS, (M + WM_ROWS - 1) / WM_ROWS, Z);
        hipLaunchKernelGGL((gemm_wide<T, AL, BL>), grid, dim3(512), 0, s, al, bl, ep, M, N, K);
        return hipGetLastError();
      }
    }
    if constexpr (std::is_same<EP, EpiResid<T>>::value) {
      if (few_tall(M, K)) return launch_few_tn<T, 32, 4>(al, bl, ep, M, N, K, Z, s);
    }
    switch (few_width(M, N, Z)) {
      case 16: return launch_few_tn<T, 16, 1>(al, bl, ep, M, N, K, Z, s);
      case 32: return launch_few_tn<T, 32, 1>(al, bl, ep, M, N, K, Z, s);
      default: return launch_few_tn<T, 64, 1>(al, bl, ep, M, N, K, Z, s);
    }
  }
}

}  // namespace wm
