// wm_gemm.hpp — tiled MFMA GEMM  C[M, N] = A[M, K] * B[N, K]^T  with pluggable
// operand loaders and fused epilogues.
//
// Block tile 128 x 128, k-tile of 128 bytes (64 bf16 / 32 float), 256 threads
// = 4 wave64s in a 2 x 2 grid, each wave a 64 x 64 sub-tile of 4 x 4 MFMA
// 16x16 tiles.  Operands go global -> registers -> LDS (rows padded by 16 B so
// the 16-lane fragment reads hit distinct banks), two LDS stages, the next
// k-tile's global loads in flight while the current one is multiplied.  After
// the k loop the fp32 C tile is staged in LDS and an epilogue functor walks
// it row by row (one wave per row, lane owns columns lane and lane + 64),
// which keeps stores coalesced and lets row / head reductions (RMSNorm, key
// and query norms, RoPE partners, residual sums of squares) be done in place.
#pragma once

#include "wm_common.hpp"

#include <type_traits>

namespace wm {

constexpr int GM = 128;            // block rows
constexpr int GN = 128;            // block columns
constexpr int GKB = 128;           // k-tile, bytes
constexpr int GROW = GKB + 16;     // LDS row pitch, bytes
constexpr int GTHREADS = 256;
constexpr int GSTAGE = 2 * GM * GROW;  // A + B tile bytes of one stage
constexpr int GCP = GN + 4;        // C tile pitch in floats
static_assert(2 * GSTAGE >= GM * GCP * 4 + GM * 4, "C tile and row scales must fit in the operand LDS");

// Position of row r of a token set (row r = b*M + m sits at s0 + m*step).
// With s0p set (a decode step whose position lives in device memory), s0 is
// read from *s0p when the kernel runs, clamped to [0, tmax).
struct RowPos {
  int M, s0, step;
  const int32_t *s0p = nullptr;
  int tmax = 1;
  __device__ __forceinline__ int base() const { return s0p ? min(max(*s0p, 0), tmax - 1) : s0; }
  __device__ __forceinline__ int pos(int r) const { return base() + (r % M) * step; }
  __device__ __forceinline__ int seq(int r) const { return r / M; }
};

// 1 / sqrt(mean(x^2) + eps) of a row from `nparts` partial sums of squares,
// added in part order; the loads go out 8 at a time (one memory round trip for
// up to 8 parts instead of one per part).
__device__ __forceinline__ float rinv_from_parts(const float *ss, int row, int nparts, float invD, float eps) {
  const float *p = ss + (int64_t)row * nparts;
  float s = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[min(p0 + i, nparts - 1)];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += p0 + i < nparts ? v[i] : 0.f;
  }
  return rsqrtf(s * invD + eps);
}

// ---------------------------------------------------------------- loaders
// A loader resolves a tile row once, before the k loop (row(...) -> handle),
// and then fetches 16-byte chunks of it (load(handle, kbyte)).  Rows past the
// end are clamped to the last row: their products land in tile rows or
// columns that every epilogue skips, and no load depends on a branch (a
// conditional load makes the compiler wait for every load in flight).

// Plain row-major operand [rows, K] with leading dimension ld (elements), an
// optional row gather and a per-blockIdx.z offset.
template <typename T> struct LoadRows {
  const T *p;
  int64_t ld, zstride;
  const int *gather;  // nullable: logical row r reads row gather[r]
  typedef const char *H;
  __device__ __forceinline__ H row(int z, int r, int nrows) const {
    r = r < nrows ? r : nrows - 1;
    const int64_t rr = gather ? gather[r] : r;
    return (const char *)(p + z * zstride + rr * ld);
  }
  __device__ __forceinline__ u32x4 load(H h, int kbyte) const { return *(const u32x4 *)(h + kbyte); }
};

// B operand of the fused gate/up projection: tile-local rows [0, GN/2) are
// gate rows, [GN/2, GN) the matching up rows, so that gate and up of one
// output column sit GN/2 apart in the C tile.
template <typename T> struct LoadGateUp {
  const T *gate, *up;
  int64_t ld;
  int F;
  typedef const char *H;
  __device__ __forceinline__ H row(int n0, int jl) const {
    int f = n0 / 2 + (jl & (GN / 2 - 1));
    f = f < F ? f : F - 1;
    return (const char *)((jl < GN / 2 ? gate : up) + (int64_t)f * ld);
  }
  __device__ __forceinline__ u32x4 load(H h, int kbyte) const { return *(const u32x4 *)(h + kbyte); }
};

// ---------------------------------------------------------------- epilogues
// Every epilogue walks a staged fp32 C tile in LDS: `nrows` rows of pitch
// `pitch` floats, tile row rl being output row m0 + rl, 64*CPL columns wide,
// first column = output column n0.  Lane l owns the CPL contiguous columns
// CPL*l .. CPL*l + CPL-1, so global loads and stores are 8- or 16-byte
// vectors.  First every thread computes per-row scales (RMSNorm 1/rms from
// partial sums of squares) into `rowbuf` in LDS; then each wave takes blocks
// of ER rows and issues all of their global loads (residual values, RoPE
// table entries) before using any, so the loads of a block are in flight
// together.  Output widths are multiples of 64, so a lane's CPL columns are
// either all inside the output or all outside.
constexpr int ER = 8;    // rows per wave per step (epilogues with RoPE tables)
constexpr int ERS = 16;  // rows per wave per step (SwiGLU epilogue)
constexpr int ERR = 16;  // rows per wave per step (residual epilogue)

template <int CPL> struct VecF;
template <> struct VecF<2> { typedef float __attribute__((ext_vector_type(2))) t; };
template <> struct VecF<4> { typedef float __attribute__((ext_vector_type(4))) t; };

template <int CPL> __device__ __forceinline__ void ldf(float *x, const float *p) {
  typename VecF<CPL>::t v = *(const typename VecF<CPL>::t *)p;
#pragma unroll
  for (int i = 0; i < CPL; ++i) x[i] = v[i];
}
template <int CPL> __device__ __forceinline__ void stf(float *p, const float *x) {
  typename VecF<CPL>::t v;
#pragma unroll
  for (int i = 0; i < CPL; ++i) v[i] = x[i];
  *(typename VecF<CPL>::t *)p = v;
}
// Store CPL values converted to T (float: 8/16 B, bf16: 4/8 B).
template <typename T, int CPL> __device__ __forceinline__ void stT(T *p, const float *x) {
  if constexpr (std::is_same<T, float>::value) {
    stf<CPL>((float *)p, x);
  } else {
    uint32_t w[CPL / 2];
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i)
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x[2 * i]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)x[2 * i + 1]) << 16);
    if constexpr (CPL == 4) *(u32x2 *)p = u32x2{w[0], w[1]};
    else *(uint32_t *)p = w[0];
  }
}

// Waves in the block (the epilogues run on 256- and 512-thread blocks).
__device__ __forceinline__ int nwaves() { return (int)(blockDim.x >> 6); }

// Row scale helpers.
__device__ __forceinline__ void fill_rowbuf_parts(float *rowbuf, const float *ss, const int *ss_rows, int nparts,
                                                  float invD, float eps, int m0, int nrows, int M) {
  for (int rl = threadIdx.x; rl < nrows; rl += blockDim.x) {
    int r = m0 + rl;
    rowbuf[rl] = r < M ? rinv_from_parts(ss, ss_rows ? ss_rows[r] : r, nparts, invD, eps) : 0.f;
  }
  __syncthreads();
}

// RMSNorm over heads of d columns (d/CPL lanes each), then RoPE, for NR rows
// at once (their lane reductions and exchanges overlap instead of forming one
// long chain per row): element m of a head pairs with m + d/2, which sits
// d/(2*CPL) lanes away at the same position in the lane.  g = gains, cs/sn =
// RoPE table entries of the lane's columns per row.
template <int CPL, int NR>
__device__ __forceinline__ void head_norm_rope(float (&x)[NR][CPL], int lane, int d, float eps, const float *g,
                                               const float (&cs)[NR][CPL], const float (&sn)[NR][CPL]) {
  const int width = d / CPL;
  float sq[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    sq[u] = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) sq[u] += x[u][i] * x[u][i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
    if (o < width) {
#pragma unroll
      for (int u = 0; u < NR; ++u) sq[u] += __shfl_xor(sq[u], o);
    }
  float y[NR][CPL], pr[NR][CPL];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const float sc = rsqrtf(sq[u] / d + eps);
#pragma unroll
    for (int i = 0; i < CPL; ++i) y[u][i] = x[u][i] * sc * g[i];
  }
#pragma unroll
  for (int u = 0; u < NR; ++u)
#pragma unroll
    for (int i = 0; i < CPL; ++i) pr[u][i] = __shfl_xor(y[u][i], d / (2 * CPL));
  const bool first = ((CPL * lane) & (d - 1)) < d / 2;
#pragma unroll
  for (int u = 0; u < NR; ++u)
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      x[u][i] = first ? y[u][i] * cs[u][i] - pr[u][i] * sn[u][i] : pr[u][i] * sn[u][i] + y[u][i] * cs[u][i];
}

template <int CPL>
__device__ __forceinline__ void rope_entries(float *cs, float *sn, const float *cosT, const float *sinT, int pos,
                                             int lane, int d) {
  const int half = d / 2, m = (CPL * lane) & (half - 1);
  ldf<CPL>(cs, cosT + (int64_t)pos * half + m);
  ldf<CPL>(sn, sinT + (int64_t)pos * half + m);
}

// q = RoPE(RMSNorm_head(rinv_row * C; q_norm)) -> q [rows, Hq*d].
template <typename T> struct EpiQ {
  T *q;
  const float *ss;
  int nparts;
  float invD, eps;
  const float *qnorm;  // [d]
  const float *cosT, *sinT;
  int d;
  RowPos rp;
};

// Rows per wave per step of the q epilogue: 4, so that it fits the
// two-waves-per-SIMD register budget of the 8-wave Q product (with 8 it
// spilled 55 registers there; on 4 waves 4 and 8 rows measure the same).
constexpr int ERQ = 4;

template <typename T, int CPL>
__device__ __forceinline__ void run_epi(const EpiQ<T> &e, int z, int m0, int n0, const float *Cs, int pitch,
                                        int nrows, int M, int N, float *rowbuf) {
  constexpr int ER = ERQ;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  fill_rowbuf_parts(rowbuf, e.ss, nullptr, e.nparts, e.invD, e.eps, m0, nrows, M);
  const int c0 = n0 + CPL * lane;
  if (c0 >= N) return;  // no __syncthreads below
  float g[CPL];
  ldf<CPL>(g, e.qnorm + ((CPL * lane) & (e.d - 1)));
  for (int rb = wave * ER; rb < nrows; rb += nwaves() * ER) {
    float cs[ER][CPL], sn[ER][CPL];
#pragma unroll
    for (int u = 0; u < ER; ++u) {
      int r = m0 + rb + u;
      rope_entries<CPL>(cs[u], sn[u], e.cosT, e.sinT, e.rp.pos(r < M ? r : M - 1), lane, e.d);
    }
    float x[ER][CPL];
#pragma unroll
    for (int u = 0; u < ER; ++u) {
      const int rl = rb + u < nrows ? rb + u : nrows - 1;
      ldf<CPL>(x[u], Cs + rl * pitch + CPL * lane);
#pragma unroll
      for (int i = 0; i < CPL; ++i) x[u][i] *= rowbuf[rl];
    }
    head_norm_rope<CPL, ER>(x, lane, e.d, e.eps, g, cs, sn);
#pragma unroll
    for (int u = 0; u < ER; ++u) {
      const int r = m0 + rb + u;
      if (rb + u < nrows && r < M) stT<T, CPL>(e.q + (int64_t)r * N + c0, x[u]);
    }
  }
}

// Residual: h += C; hb = h * gain_next; optionally S_next = h; and the row's
// sum of squares over this tile's columns -> ss_out[r, n0 / tile width]
// (tile width tw: 64 * CPL, or fewer columns with the lanes past it idle).
template <typename T> struct EpiResid {
  float *h;
  T *hb;
  const float *gain_next;  // [N]
  T *S_next;               // nullable, [rows, N]
  float *ss_out;
  int nparts_out;
};

template <typename T, int CPL>
__device__ __forceinline__ void run_epi(const EpiResid<T> &e, int z, int m0, int n0, const float *Cs, int pitch,
                                        int nrows, int M, int N, float *rowbuf, int tw = 64 * CPL) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = n0 + CPL * lane;
  const bool on = c0 < N && CPL * lane < tw;
  const int cl = on ? c0 : N - CPL;  // (off lanes read a valid column and store nothing)
  float g[CPL];
  ldf<CPL>(g, e.gain_next + cl);
  for (int rb = wave * ERR; rb < nrows; rb += nwaves() * ERR) {
    float hv[ERR][CPL], sq[ERR];
#pragma unroll
    for (int u = 0; u < ERR; ++u) {
      const int r = m0 + rb + u;
      ldf<CPL>(hv[u], e.h + (int64_t)(r < M ? r : M - 1) * N + cl);
    }
#pragma unroll
    for (int u = 0; u < ERR; ++u) {
      const int rl = rb + u, r = m0 + rl;
      const bool ok = on && rl < nrows && r < M;
      float x[CPL], xb[CPL];
      ldf<CPL>(x, Cs + (rl < nrows ? rl : nrows - 1) * pitch + CPL * lane);
      sq[u] = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        x[i] += hv[u][i];
        xb[i] = x[i] * g[i];
        sq[u] += ok ? x[i] * x[i] : 0.f;
      }
      if (ok) {
        const int64_t o = (int64_t)r * N + c0;
        stf<CPL>(e.h + o, x);
        stT<T, CPL>(e.hb + o, xb);
        if (e.S_next) stT<T, CPL>(e.S_next + o, x);
      }
    }
    // the rows' sums over the wave, reduced together
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
#pragma unroll
      for (int u = 0; u < ERR; ++u) sq[u] += __shfl_xor(sq[u], o);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < ERR; ++u) {
        const int r = m0 + rb + u;
        if (rb + u < nrows && r < M) e.ss_out[(int64_t)r * e.nparts_out + n0 / tw] = sq[u];
      }
    }
  }
}

// SwiGLU: tile columns [0, 32*CPL) are gate, [32*CPL, 64*CPL) the matching up
// columns; each lane takes CPL/2 consecutive gate columns and reads their up
// partners from the staged tile: act[r, n0/2 + c] = silu(rs*gate) * (rs*up).
template <typename T> struct EpiSwiGLU {
  T *act;
  const float *ss;
  int nparts;
  float invD, eps;
  int F;
};

template <typename T, int CPL>
__device__ __forceinline__ void run_epi(const EpiSwiGLU<T> &e, int z, int m0, int n0, const float *Cs, int pitch,
                                        int nrows, int M, int N, float *rowbuf) {
  constexpr int OPL = CPL / 2;  // outputs per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  fill_rowbuf_parts(rowbuf, e.ss, nullptr, e.nparts, e.invD, e.eps, m0, nrows, M);
  const int f0 = n0 / 2 + OPL * lane;
  if (f0 >= e.F) return;  // no __syncthreads below
  // ERS rows per wave and step: every LDS read of the step before any use
  for (int rb = wave * ERS; rb < nrows; rb += nwaves() * ERS) {
    float gt[ERS][OPL], up[ERS][OPL], rs[ERS];
#pragma unroll
    for (int u = 0; u < ERS; ++u) {
      const int rl = rb + u < nrows ? rb + u : nrows - 1;
      rs[u] = rowbuf[rl];
      const float *row = Cs + rl * pitch + OPL * lane;
#pragma unroll
      for (int i = 0; i < OPL; ++i) {
        gt[u][i] = row[i];
        up[u][i] = row[i + 32 * CPL];
      }
    }
#pragma unroll
    for (int u = 0; u < ERS; ++u) {
      const int r = m0 + rb + u;
      float y[OPL];
#pragma unroll
      for (int i = 0; i < OPL; ++i) y[i] = silu(gt[u][i] * rs[u]) * (up[u][i] * rs[u]);
      if (rb + u < nrows && r < M) {
        T *dst = e.act + (int64_t)r * e.F + f0;
        if constexpr (OPL == 2) {
          stT<T, 2>(dst, y);
        } else {
          dst[0] = from_f<T>(y[0]);
        }
      }
    }
  }
}

// Plain fp32 store with an optional row scale from partial sums and an
// optional output row map: out[(map ? map[r] : r) * ldo + c] (per z offset).
// (Element-wise: the router's output width L*k need not be a multiple of 4.)
struct EpiStoreF32 {
  float *out;
  int64_t ldo, zstride;
  const int *out_rows;  // nullable
  const float *ss;      // nullable: no row scale
  const int *ss_rows;   // nullable: ss row = ss_rows[r]
  int nparts;
  float invD, eps;
};

template <typename T, int CPL>
__device__ __forceinline__ void run_epi(const EpiStoreF32 &e, int z, int m0, int n0, const float *Cs, int pitch,
                                        int nrows, int M, int N, float *rowbuf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (e.ss) fill_rowbuf_parts(rowbuf, e.ss, e.ss_rows, e.nparts, e.invD, e.eps, m0, nrows, M);
  for (int rl = wave; rl < nrows; rl += nwaves()) {
    int r = m0 + rl;
    if (r >= M) break;
    float rs = e.ss ? rowbuf[rl] : 1.f;
    int64_t orow = e.out_rows ? e.out_rows[r] : r;
    float *dst = e.out + z * e.zstride + orow * e.ldo;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      int c = n0 + lane + 64 * i;
      if (c < N) dst[c] = Cs[rl * pitch + lane + 64 * i] * rs;
    }
  }
}

// Pool projection, blockIdx.z = beta*k + j: rows scaled by the channel's
// 1/rms (rinvM [2k, rows]); keys then get the per-head key norm (k_norm[j])
// and RoPE, values stay raw; both go to cache[j, b, h, pos, :].
template <typename T> struct EpiKV {
  T *Kc, *Vc;  // [k, B, Hkv, T_max, d]
  const float *rinvM;
  const float *knorm;  // [k, d]
  const float *cosT, *sinT;
  int k, B, Hkv, T_max, d, rows;
  float eps;
  RowPos rp;
};

template <typename T, int CPL>
__device__ __forceinline__ void run_epi(const EpiKV<T> &e, int z, int m0, int n0, const float *Cs, int pitch,
                                        int nrows, int M, int N, float *rowbuf) {
  constexpr int ER = ERQ;  // (4 rows per step: the 8-wave K/V projection's register budget)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int beta = z / e.k, j = z - beta * e.k;
  for (int rl = threadIdx.x; rl < nrows; rl += blockDim.x) {
    int r = m0 + rl;
    rowbuf[rl] = r < M ? e.rinvM[(int64_t)z * e.rows + r] : 0.f;
  }
  __syncthreads();
  const int c0 = n0 + CPL * lane;
  if (c0 >= N) return;  // no __syncthreads below
  const int h = c0 / e.d, dd = c0 - h * e.d;
  float g[CPL];
  ldf<CPL>(g, e.knorm + (int64_t)j * e.d + ((CPL * lane) & (e.d - 1)));
  T *base = beta == 0 ? e.Kc : e.Vc;
  for (int rb = wave * ER; rb < nrows; rb += nwaves() * ER) {
    float cs[ER][CPL], sn[ER][CPL];
    if (beta == 0) {
#pragma unroll
      for (int u = 0; u < ER; ++u) {
        int r = m0 + rb + u;
        rope_entries<CPL>(cs[u], sn[u], e.cosT, e.sinT, e.rp.pos(r < M ? r : M - 1), lane, e.d);
      }
    }
    float x[ER][CPL];
#pragma unroll
    for (int u = 0; u < ER; ++u) {
      const int rl = rb + u < nrows ? rb + u : nrows - 1;
      ldf<CPL>(x[u], Cs + rl * pitch + CPL * lane);
#pragma unroll
      for (int i = 0; i < CPL; ++i) x[u][i] *= rowbuf[rl];
    }
    if (beta == 0) head_norm_rope<CPL, ER>(x, lane, e.d, e.eps, g, cs, sn);
#pragma unroll
    for (int u = 0; u < ER; ++u) {
      const int r = m0 + rb + u;
      if (rb + u < nrows && r < M) {
        const int pos = e.rp.pos(r), b = e.rp.seq(r);
        stT<T, CPL>(base + ((((int64_t)j * e.B + b) * e.Hkv + h) * e.T_max + pos) * e.d + dd, x[u]);
      }
    }
  }
}

// Per-layer K/V projection of the vanilla comparison model: output columns
// [0, hd) are keys (per-head key norm, RoPE), [hd, 2*hd) values (hd = Hkv*d);
// rows scaled by their RMSNorm factor from partial sums of squares; both go to
// the layer's cache slices Kc / Vc [B, Hkv, T_max, d] at the row's position.
template <typename T> struct EpiKVL {
  T *Kc, *Vc;
  const float *ss;
  int nparts;
  float invD, eps;
  const float *knorm;  // [d]
  const float *cosT, *sinT;
  int Hkv, d, T_max;
  RowPos rp;
};

template <typename T, int CPL>
__device__ __forceinline__ void run_epi(const EpiKVL<T> &e, int z, int m0, int n0, const float *Cs, int pitch,
                                        int nrows, int M, int N, float *rowbuf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  fill_rowbuf_parts(rowbuf, e.ss, nullptr, e.nparts, e.invD, e.eps, m0, nrows, M);
  const int c0 = n0 + CPL * lane;
  if (c0 >= N) return;  // no __syncthreads below
  const int hd = e.Hkv * e.d;
  const bool isK = c0 < hd;  // (heads never straddle the key/value boundary)
  const int cc = isK ? c0 : c0 - hd, hh = cc / e.d, dd = cc - hh * e.d;
  float g[CPL];
  ldf<CPL>(g, e.knorm + ((CPL * lane) & (e.d - 1)));
  T *base = isK ? e.Kc : e.Vc;
  for (int rb = wave * ER; rb < nrows; rb += nwaves() * ER) {
    float cs[ER][CPL], sn[ER][CPL];
#pragma unroll
    for (int u = 0; u < ER; ++u) {
      int r = m0 + rb + u;
      rope_entries<CPL>(cs[u], sn[u], e.cosT, e.sinT, e.rp.pos(r < M ? r : M - 1), lane, e.d);
    }
    float x[ER][CPL];
#pragma unroll
    for (int u = 0; u < ER; ++u) {
      const int rl = rb + u < nrows ? rb + u : nrows - 1;
      ldf<CPL>(x[u], Cs + rl * pitch + CPL * lane);
#pragma unroll
      for (int i = 0; i < CPL; ++i) x[u][i] *= rowbuf[rl];
    }
    if (isK) head_norm_rope<CPL, ER>(x, lane, e.d, e.eps, g, cs, sn);
#pragma unroll
    for (int u = 0; u < ER; ++u) {
      const int r = m0 + rb + u;
      if (rb + u < nrows && r < M) {
        const int pos = e.rp.pos(r), b = e.rp.seq(r);
        stT<T, CPL>(base + (((int64_t)b * e.Hkv + hh) * e.T_max + pos) * e.d + dd, x[u]);
      }
    }
  }
}

// ---------------------------------------------------------------- B loaders
// row(z, n0, jl, N): tile row jl of the block whose first output column is n0.
template <typename T> struct BRows {
  LoadRows<T> L;
  typedef const char *H;
  __device__ __forceinline__ H row(int z, int n0, int jl, int N) const { return L.row(z, n0 + jl, N); }
  __device__ __forceinline__ u32x4 load(H h, int kbyte) const { return L.load(h, kbyte); }
};
template <typename T> struct BGateUp {
  LoadGateUp<T> L;
  typedef const char *H;
  __device__ __forceinline__ H row(int z, int n0, int jl, int N) const { return L.row(n0, jl); }
  __device__ __forceinline__ u32x4 load(H h, int kbyte) const { return L.load(h, kbyte); }
};
// Vanilla per-layer K/V weights stacked: rows [0, hd) of wk, then rows of wv.
template <typename T> struct BKVL {
  const T *wk, *wv;
  int64_t ld;
  int hd;
  typedef const char *H;
  __device__ __forceinline__ H row(int z, int n0, int jl, int N) const {
    int n = n0 + jl;
    n = n < N ? n : N - 1;
    return (const char *)(n < hd ? wk + (int64_t)n * ld : wv + (int64_t)(n - hd) * ld);
  }
  __device__ __forceinline__ u32x4 load(H h, int kbyte) const { return *(const u32x4 *)(h + kbyte); }
};
// Pool projection weights: z = beta*k + j -> wk[j] or wv[j].
template <typename T> struct BKV {
  const T *wk, *wv;
  int64_t ld, mstride;
  int k;
  typedef const char *H;
  __device__ __forceinline__ H row(int z, int n0, int jl, int N) const {
    int n = n0 + jl;
    n = n < N ? n : N - 1;
    const int beta = z / k, j = z - beta * k;
    return (const char *)((beta == 0 ? wk : wv) + j * mstride + (int64_t)n * ld);
  }
  __device__ __forceinline__ u32x4 load(H h, int kbyte) const { return *(const u32x4 *)(h + kbyte); }
};

// ---------------------------------------------------------------- kernel
template <typename T, class AL, class BL, class EP>
__global__ __launch_bounds__(GTHREADS) void gemm_kernel(AL al, BL bl, EP ep, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * GSTAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int z = blockIdx.z;
  const int m0 = blockIdx.y * GM, n0 = blockIdx.x * GN;
  const int nk = (int)((int64_t)K * (int64_t)sizeof(T) / GKB);

  u32x4 ra[4], rb[4];
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  typename AL::H ha[4];
  typename BL::H hb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid + GTHREADS * i) >> 3;
    ha[i] = al.row(z, m0 + r, M);
    hb[i] = bl.row(z, n0, r, N);
  }
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cb = (tid + GTHREADS * i) & 7;
      ra[i] = al.load(ha[i], kt * GKB + cb * 16);
      rb[i] = bl.load(hb[i], kt * GKB + cb * 16);
    }
  };
  auto sstore = [&](int buf) {
    unsigned char *As = smem + buf * GSTAGE, *Bs = As + GM * GROW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + GTHREADS * i, r = c >> 3, cb = c & 7;
      *(u32x4 *)(As + r * GROW + cb * 16) = ra[i];
      *(u32x4 *)(Bs + r * GROW + cb * 16) = rb[i];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
    const unsigned char *As = smem + (kt & 1) * GSTAGE, *Bs = As + GM * GROW;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *(const u32x4 *)(As + (wm * 64 + i * 16 + (lane & 15)) * GROW + ks * 64 + (lane >> 4) * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *(const u32x4 *)(Bs + (wn * 64 + j * 16 + (lane & 15)) * GROW + ks * 64 + (lane >> 4) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma16<T>(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < nk) sstore((kt + 1) & 1);
    __syncthreads();
  }

  float *Cs = (float *)smem;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Cs[(wm * 64 + i * 16 + (lane >> 4) * 4 + e) * GCP + wn * 64 + j * 16 + (lane & 15)] = acc[i][j][e];
  __syncthreads();
  run_epi<T, GN / 64>(ep, z, m0, n0, Cs, GCP, GM, M, N, (float *)(smem + GM * GCP * 4));
}

template <typename T, class AL, class BL, class EP>
hipError_t launch_gemm(const AL &al, const BL &bl, const EP &ep, int M, int N, int K, int Z, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  dim3 grid((N + GN - 1) / GN, (M + GM - 1) / GM, Z);
  hipLaunchKernelGGL((gemm_kernel<T, AL, BL, EP>), grid, dim3(GTHREADS), 0, s, al, bl, ep, M, N, K);
  return hipGetLastError();
}

}  // namespace wm
