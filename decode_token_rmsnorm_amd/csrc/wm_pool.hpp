// wm_pool.hpp — the streaming parts of the cross-layer KV pool and small
// helper kernels.
//
//  state_rinv   1/rms of every (layer, row) of the state stack S [L, rows, D]
//  pool_mix     for both branches and every channel j of one token:
//                 m_j = sum_l A[l, j] * rinv_l * (gamma_l (.) S[l])   (signed A)
//               stores rho_j (.) m_j (channel gain folded in; the channel's
//               1/rms is applied after the projection, which is linear) and
//               1/rms(m_j) for the projection epilogue.
//  router_input the router's normalised input rows, written out (the
//               feedback-free variant's channel steps)
//  rinv_router_input  state_rinv and router_input in one launch (few rows)
//  state_rinv_u state_rinv plus the normalised router-layer rows (many rows)
//  fold_router  router weights times the source gains
//  embed_rows   h_0 = E[token] (+ the first state, the next GEMM's operand and
//               its sum of squares, and the LM head's row lists)
//  rope_table   cos/sin of s * base^(-2m/d), double precision, rounded
#pragma once

#include "wm_common.hpp"

namespace wm {

// One wave per (layer, row): rinv[l*rows + r] = 1/sqrt(mean(S^2) + eps).
template <typename T>
__global__ __launch_bounds__(256) void state_rinv(const T *S, float *rinv, int64_t nrowsL, int D, float eps) {
  int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (w >= nrowsL) return;
  constexpr int E = Elt<T>::E16;
  const T *x = S + w * D;
  float s = 0.f;
  for (int c = lane * E; c < D; c += 64 * E) {
    float f[E];
    unpack16<T>(*(const u32x4 *)(x + c), f);
#pragma unroll
    for (int e = 0; e < E; ++e) s += f[e] * f[e];
  }
  s = wave_sum(s);
  if (lane == 0) rinv[w] = rsqrtf(s / D + eps);
}

// state_rinv plus, for the router's layers (layer % p == 0), the normalised
// router input u[r, (layer/p)*D + c] = S[layer, r, c] * rinv (source gains are
// folded into the router weights instead).  One wave per (layer, row).
template <typename T>
__global__ __launch_bounds__(256) void state_rinv_u(const T *S, float *rinv, T *u, int rows, int L, int p, int R,
                                                    int D, float eps) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= (int64_t)L * rows) return;
  const int layer = (int)(w / rows), r = (int)(w - (int64_t)layer * rows);
  constexpr int E = Elt<T>::E16;
  const T *x = S + w * D;
  float s = 0.f;
  for (int c = lane * E; c < D; c += 64 * E) {
    float f[E];
    unpack16<T>(*(const u32x4 *)(x + c), f);
#pragma unroll
    for (int e = 0; e < E; ++e) s += f[e] * f[e];
  }
  s = wave_sum(s);
  const float ri = rsqrtf(s / D + eps);
  if (lane == 0) rinv[w] = ri;
  if (layer % p) return;
  T *dst = u + (int64_t)r * R * D + (int64_t)(layer / p) * D;
  for (int c = lane * E; c < D; c += 64 * E) {
    float f[E];
    unpack16<T>(*(const u32x4 *)(x + c), f);
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] *= ri;
    *(u32x4 *)(dst + c) = pack16<T>(f);
  }
}

// Router weights with the source gains folded in, both branches stacked:
// Wf[o, s*D + c] = W[o, s*D + c] * gain[o / Lk, s*p, c]  (W is [2*Lk, R*D]).
template <typename T>
__global__ __launch_bounds__(256) void fold_router(const T *W, const float *gain, T *Wf, int Lk, int L, int p, int R,
                                                   int D) {
  constexpr int E = Elt<T>::E16;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * E;
  const int64_t RD = (int64_t)R * D;
  if (i >= 2 * (int64_t)Lk * RD) return;
  const int o = (int)(i / RD);
  const int kk = (int)(i - (int64_t)o * RD), sg = kk / D, c = kk - sg * D;
  const float *g = gain + ((int64_t)(o / Lk) * L + (int64_t)sg * p) * D + c;
  float f[E];
  unpack16<T>(*(const u32x4 *)(W + i), f);
#pragma unroll
  for (int e = 0; e < E; ++e) f[e] *= g[e];
  *(u32x4 *)(Wf + i) = pack16<T>(f);
}

// One block per token row; thread owns columns tid, tid + 256, ...
// Router output A: element (z, beta, row, l*k + j) at z*az + beta*ab +
// row*ar + l*k + j, summed over Z partials; S [L, rows, D]; mb [2, k, rows,
// D]; rinvM [2, k, rows].
// src_gain / chan_gain: element (beta, l, c) at beta*sgb + l*D + c and
// (beta, j, c) at beta*cgb + j*D + c.
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void pool_mix(const T *S, const float *rinvS, const float *A, int Z, int64_t az,
                                                int64_t ab, int64_t ar, const float *src_gain, int64_t sgb,
                                                const float *chan_gain, int64_t cgb, T *mb, float *rinvM, int rows,
                                                int L, int k, int D, float eps) {
  __shared__ float Aw[2][32][KMAX];  // L <= 32
  __shared__ float red[4][2 * KMAX];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 2 * L * k; i += 256) {
    int beta = i / (L * k), rem = i - beta * L * k, l = rem / k, j = rem - l * k;
    float v = 0.f;
    for (int z = 0; z < Z; ++z) v += A[z * az + beta * ab + r * ar + rem];
    Aw[beta][l][j] = v * rinvS[(int64_t)l * rows + r];
  }
  __syncthreads();
  float ss[2][KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) ss[0][j] = ss[1][j] = 0.f;
  for (int c = tid; c < D; c += 256) {
    float acc[2][KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) acc[0][j] = acc[1][j] = 0.f;
    for (int l = 0; l < L; ++l) {
      float x = to_f(S[((int64_t)l * rows + r) * D + c]);
      float xk = x * src_gain[(int64_t)l * D + c];
      float xv = x * src_gain[sgb + (int64_t)l * D + c];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          acc[0][j] += Aw[0][l][j] * xk;
          acc[1][j] += Aw[1][l][j] * xv;
        }
      }
    }
#pragma unroll
    for (int beta = 0; beta < 2; ++beta)
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          float m = acc[beta][j];
          ss[beta][j] += m * m;
          mb[(((int64_t)beta * k + j) * rows + r) * D + c] = from_f<T>(m * chan_gain[beta * cgb + (int64_t)j * D + c]);
        }
      }
  }
#pragma unroll
  for (int beta = 0; beta < 2; ++beta)
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      float v = wave_sum(ss[beta][j]);
      if (lane == 0) red[wave][beta * KMAX + j] = v;
    }
  __syncthreads();
  if (tid < 2 * k) {
    int beta = tid / k, j = tid - beta * k;
    float v = red[0][beta * KMAX + j] + red[1][beta * KMAX + j] + red[2][beta * KMAX + j] + red[3][beta * KMAX + j];
    rinvM[((int64_t)beta * k + j) * rows + r] = rsqrtf(v / D + eps);
  }
}

// Router input, both branches, blocks b0 <= b < b1 of R:
// u[beta, r, b*D + c] = S[b*p, r, c] * rinvS[b*p, r] * gain[beta, b*p, c].
template <typename T>
__global__ __launch_bounds__(256) void router_input(const T *S, const float *rinvS, const float *gain, T *u, int rows,
                                                    int L, int p, int R, int D, int b0, int b1) {
  constexpr int E = Elt<T>::E16;
  const int r = blockIdx.x, beta = blockIdx.y;
  for (int b = b0; b < b1; ++b) {
    const int l = b * p;
    const float s = rinvS[(int64_t)l * rows + r];
    const T *src = S + ((int64_t)l * rows + r) * D;
    const float *g = gain + ((int64_t)beta * L + l) * D;
    T *dst = u + ((int64_t)beta * rows + r) * R * D + (int64_t)b * D;
    for (int c = threadIdx.x * E; c < D; c += 256 * E) {
      float f[E];
      unpack16<T>(*(const u32x4 *)(src + c), f);
#pragma unroll
      for (int e = 0; e < E; ++e) f[e] *= s * g[c + e];
      *(u32x4 *)(dst + c) = pack16<T>(f);
    }
  }
}

// Gather/scatter row lists of the LM head, n entries (rows_in null: none):
// mode 1: rows_in[b] = b*M + m_sel, rows_out[b] = b;
// mode 2: rows_in[r] = r, rows_out[r] = b*T + s0 + m*step (r = b*M + m).
struct RowMap {
  int *rows_in, *rows_out;
  int n, mode, m_sel, T, s0, step;
  __device__ __forceinline__ void fill(int i, int M) const {
    if (mode == 1) {
      rows_in[i] = i * M + m_sel;
      rows_out[i] = i;
    } else {
      const int b = i / M, m = i - b * M;
      rows_in[i] = i;
      rows_out[i] = b * T + s0 + m * step;
    }
  }
};

// state_rinv and router_input in one launch for steps of few rows: block
// (r, beta) computes the row scales of all L states of row r (the same wave
// sums as state_rinv; the beta = 0 block stores them), then writes the row's
// gained router input of branch beta.  The launch is latency-bound (a few MB
// per step), so each wave issues the loads of four layers before it reduces
// any of them, and the router input is written by all 256 threads, four
// 16-byte pieces each per round, every load of a round issued before its
// stores.
template <typename T>
__global__ __launch_bounds__(256) void rinv_router_input(const T *S, float *rinvS, const float *gain, T *u, int rows,
                                                         int L, int p, int R, int D, float eps) {
  constexpr int E = Elt<T>::E16;
  constexpr int LB = 4;  // layers in flight per wave
  const int r = blockIdx.x, beta = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ float rs[32];  // (L <= 32)
  for (int l0 = wave; l0 < L; l0 += 4 * LB) {
    float s[LB] = {};
    for (int c = lane * E; c < D; c += 64 * E) {
      u32x4 v[LB] = {};
#pragma unroll
      for (int j = 0; j < LB; ++j)
        if (l0 + 4 * j < L) v[j] = *(const u32x4 *)(S + ((int64_t)(l0 + 4 * j) * rows + r) * D + c);
#pragma unroll
      for (int j = 0; j < LB; ++j) {
        float f[E];
        unpack16<T>(v[j], f);
#pragma unroll
        for (int e = 0; e < E; ++e) s[j] += f[e] * f[e];
      }
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int l = l0 + 4 * j;
      if (l >= L) break;  // wave-uniform
      const float v = rsqrtf(wave_sum(s[j]) / D + eps);
      if (lane == 0) {
        rs[l] = v;
        if (beta == 0) rinvS[(int64_t)l * rows + r] = v;
      }
    }
  }
  __syncthreads();
  constexpr int PU = 4;  // 16-byte pieces per thread and round
  const int npc = D / E, n = R * npc;
  T *urow = u + ((int64_t)beta * rows + r) * R * D;
  for (int i0 = threadIdx.x; i0 < n; i0 += 256 * PU) {
    u32x4 v[PU] = {};
    float g[PU][E];
#pragma unroll
    for (int j = 0; j < PU; ++j) {
      const int i = i0 + 256 * j;
      if (i >= n) break;
      const int b = i / npc, c = (i - b * npc) * E, l = b * p;
      v[j] = *(const u32x4 *)(S + ((int64_t)l * rows + r) * D + c);
      const float *gp = gain + ((int64_t)beta * L + l) * D + c;
#pragma unroll
      for (int e = 0; e < E; ++e) g[j][e] = gp[e];
    }
#pragma unroll
    for (int j = 0; j < PU; ++j) {
      const int i = i0 + 256 * j;
      if (i >= n) break;
      const int b = i / npc, c = (i - b * npc) * E;
      const float sc = rs[b * p];
      float f[E];
      unpack16<T>(v[j], f);
#pragma unroll
      for (int e = 0; e < E; ++e) f[e] *= sc * g[j][e];
      *(u32x4 *)(urow + (int64_t)b * D + c) = pack16<T>(f);
    }
  }
}

// Row r = b*M + m reads token tokens[b*tstride + toff + m*tstep].  Writes
// h = E[tok] (fp32), S0 = E[tok], hb = E[tok] * gain, and the row's sum of
// squares (one part).  A token id outside [0, V) reads nothing and makes the
// row NaN, so the error shows in everything computed from it.
template <typename T>
__global__ __launch_bounds__(256) void embed_rows(const int32_t *tokens, const T *E, const float *gain, float *h, T *hb,
                                                  T *S0, float *ss, int M, int tstride, int toff, int tstep, int V,
                                                  int D, RowMap map) {
  const int r = blockIdx.x, tid = threadIdx.x;
  if (tid == 0 && map.rows_in && r < map.n) map.fill(r, M);
  const int b = r / M, m = r - b * M;
  const int tok = tokens[(int64_t)b * tstride + toff + (int64_t)m * tstep];
  const bool valid = tok >= 0 && tok < V;
  float s = 0.f;
  for (int c = tid; c < D; c += 256) {
    const T e = valid ? E[(int64_t)tok * D + c] : from_f<T>(__builtin_nanf(""));
    const float v = to_f(e);
    h[(int64_t)r * D + c] = v;
    S0[(int64_t)r * D + c] = e;
    hb[(int64_t)r * D + c] = from_f<T>(v * gain[c]);
    s += v * v;
  }
  __shared__ float red[4];
  s = wave_sum(s);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) ss[r] = red[0] + red[1] + red[2] + red[3];
}

__global__ void rope_table(float *cosT, float *sinT, int T_max, int half, double base, int d) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T_max * half) return;
  int s = (int)(i / half), m = (int)(i - (int64_t)s * half);
  double ang = (double)s * pow(base, -2.0 * m / d);
  cosT[i] = (float)cos(ang);
  sinT[i] = (float)sin(ang);
}


}  // namespace wm
