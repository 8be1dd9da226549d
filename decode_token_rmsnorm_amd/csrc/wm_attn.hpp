// wm_attn.hpp — strict-causal channel attention over a strided token set.
//
// Grid (row blocks, B*Hkv, splits).  The rows of one (sequence b, KV head hk)
// pair are the (m, g) products of the token set's M queries and the G = Hq/Hkv
// query heads sharing hk, row rho = m*G + g at position s0 + m*step.  A block
// of NW waves owns NW*NQ*16 such rows and walks 64-key tiles of the cache
// channel, staged in LDS (keys row-major, values transposed) and shared by its
// waves; each wave keeps NQ 16-row query tiles in registers.
//
// Scores are computed transposed, S^T = K Q^T, so that a lane's accumulator
// holds 4 keys of ONE query: the online-softmax rescale of the output is then
// lane-local, and the probabilities P^T are already in the B-operand layout of
// O^T += V^T P^T (the MFMA k index only has to agree between the V^T fragment
// read from LDS and the P^T fragment taken from the accumulators).  The mask
// (key < position of the row's token) and the group stride are applied in the
// tile loop.  With several splits each writes unnormalised (o, max, sum)
// partials and attn_combine merges them.
#pragma once

#include "wm_common.hpp"

namespace wm {

constexpr int AKT = 64;  // keys per tile

struct AttnArgs {
  const void *q;       // [B*M, Hq, d]
  void *out;           // [B*M, Hq*d]
  const void *Kc, *Vc; // channel base: [B, Hkv, T_max, d]
  float *part_o;       // [splits, B*M, Hq, d]
  float *part_ml;      // [splits, B*M, Hq, 2]
  int B, M, s0, step, Hq, Hkv, G, T_max, nsplit;
  float scale_log2;    // log2(e) / sqrt(d)
};

template <typename T, int DH, int NW, int NQ>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  constexpr int E = Elt<T>::E16;       // elements per 16-byte fragment
  constexpr int KCH = 4 * E;           // k (head dim) per MFMA step
  constexpr int NCH = DH / KCH;        // MFMA steps over the head dim
  constexpr int KP = DH + 16 / (int)sizeof(T) * 1;  // key-row pitch (elements), +16 B
  constexpr int VP = AKT + 16 / (int)sizeof(T);     // transposed value pitch (elements)
  constexpr int PVK = 4 * E;           // keys per PV MFMA step
  constexpr int RB = NW * NQ * 16;     // rows per block
  __shared__ __attribute__((aligned(16))) T Ks[AKT * KP];
  __shared__ __attribute__((aligned(16))) T Vt[DH * VP];

  const T *qp = (const T *)a.q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = blockIdx.y, b = pair / a.Hkv, hk = pair - b * a.Hkv;
  const int nrows = a.M * a.G;
  const int rb0 = blockIdx.x * RB;
  if (rb0 >= nrows) return;
  const int last = min(nrows, rb0 + RB) - 1;
  int kmax = a.s0 + (last / a.G) * a.step;  // keys s < kmax for the block
  kmax = min(kmax, a.T_max);
  const int ntile = (kmax + AKT - 1) / AKT;
  const int tps = (ntile + a.nsplit - 1) / a.nsplit;
  const int t0 = blockIdx.z * tps, t1 = min(ntile, t0 + tps);

  // this lane's query row per nq (column lane%16 of the S^T tiles)
  int rpos[NQ], rrow[NQ], rhead[NQ];
  bool rvalid[NQ];
  u32x4 qf[NQ][NCH];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    int rho = rb0 + wave * NQ * 16 + nq * 16 + (lane & 15);
    rvalid[nq] = rho < nrows;
    int m = rvalid[nq] ? rho / a.G : 0, g = rvalid[nq] ? rho - m * a.G : 0;
    rpos[nq] = rvalid[nq] ? a.s0 + m * a.step : 0;
    rrow[nq] = b * a.M + m;
    rhead[nq] = hk * a.G + g;
    const T *src = qp + ((int64_t)rrow[nq] * a.Hq + rhead[nq]) * DH;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      qf[nq][c] = rvalid[nq] ? *(const u32x4 *)(src + c * KCH + (lane >> 4) * E) : u32x4{0, 0, 0, 0};
  }

  f32x4 o[DH / 16][NQ];
  float mrun[NQ], lrun[NQ];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    mrun[nq] = -INFINITY;
    lrun[nq] = 0.f;
#pragma unroll
    for (int u = 0; u < DH / 16; ++u) o[u][nq] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const T *Kb = (const T *)a.Kc + ((int64_t)b * a.Hkv + hk) * a.T_max * DH;
  const T *Vb = (const T *)a.Vc + ((int64_t)b * a.Hkv + hk) * a.T_max * DH;

  for (int t = t0; t < t1; ++t) {
    const int key0 = t * AKT;
    // keys: 16-byte chunks, row-major with padding
    for (int c = tid; c < AKT * DH / E; c += NW * 64) {
      int kr = c / (DH / E), cc = c - kr * (DH / E);
      int key = key0 + kr;
      u32x4 v = key < kmax ? *(const u32x4 *)(Kb + (int64_t)key * DH + cc * E) : u32x4{0, 0, 0, 0};
      *(u32x4 *)(Ks + kr * KP + cc * E) = v;
    }
    // values: 4 keys x E columns per item, written transposed
    for (int c = tid; c < (AKT / 4) * (DH / E); c += NW * 64) {
      int kq = c / (DH / E), cc = c - kq * (DH / E);
      float f[4][E];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int key = key0 + 4 * kq + i;
        u32x4 v = key < kmax ? *(const u32x4 *)(Vb + (int64_t)key * DH + cc * E) : u32x4{0, 0, 0, 0};
        unpack16<T>(v, f[i]);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        T *dst = Vt + (cc * E + e) * VP + 4 * kq;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = from_f<T>(f[i][e]);
      }
    }
    __syncthreads();

    // S^T = K Q^T for 4 key sub-tiles
    f32x4 s[4][NQ];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) s[kt][nq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        u32x4 kf = *(const u32x4 *)(Ks + (kt * 16 + (lane & 15)) * KP + c * KCH + (lane >> 4) * E);
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) mma16<T>(s[kt][nq], kf, qf[nq][c]);
      }
    }

    // mask, online softmax
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int key = key0 + kt * 16 + (lane >> 4) * 4 + e;
          float v = (key < rpos[nq]) ? s[kt][nq][e] * a.scale_log2 : -INFINITY;
          s[kt][nq][e] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      float mnew = fmaxf(mrun[nq], tmax);
      float alpha = mnew == -INFINITY ? 1.f : exp2f(mrun[nq] - mnew);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv = mnew == -INFINITY ? 0.f : exp2f(s[kt][nq][e] - mnew);
          s[kt][nq][e] = pv;
          psum += pv;
        }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      lrun[nq] = lrun[nq] * alpha + psum;
      mrun[nq] = mnew;
#pragma unroll
      for (int u = 0; u < DH / 16; ++u) o[u][nq] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < AKT / PVK; ++kc) {
      u32x4 pf[NQ];
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) {
        float pv[E];
#pragma unroll
        for (int part = 0; part < E / 4; ++part)
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[part * 4 + e] = s[kc * (E / 4) + part][nq][e];
        pf[nq] = pack16<T>(pv);
      }
#pragma unroll
      for (int u = 0; u < DH / 16; ++u) {
        const T *vrow = Vt + (u * 16 + (lane & 15)) * VP + kc * PVK + (lane >> 4) * 4;
        u32x4 vf;
        if constexpr (E == 8) {
          u32x2 lo = *(const u32x2 *)vrow, hi = *(const u32x2 *)(vrow + 16);
          vf = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          vf = *(const u32x4 *)vrow;
        }
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) mma16<T>(o[u][nq], vf, pf[nq]);
      }
    }
    __syncthreads();
  }

  // write out (lane: query lane%16, head dims u*16 + 4*(lane/16) + e)
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    if (!rvalid[nq]) continue;
    if (a.nsplit == 1) {
      float inv = lrun[nq] > 0.f ? 1.f / lrun[nq] : 0.f;
      T *dst = (T *)a.out + (int64_t)rrow[nq] * a.Hq * DH + rhead[nq] * DH;
#pragma unroll
      for (int u = 0; u < DH / 16; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[u * 16 + (lane >> 4) * 4 + e] = from_f<T>(o[u][nq][e] * inv);
    } else {
      int64_t base = ((int64_t)blockIdx.z * a.B * a.M + rrow[nq]) * a.Hq + rhead[nq];
      float *dst = a.part_o + base * DH;
#pragma unroll
      for (int u = 0; u < DH / 16; ++u)
        *(f32x4 *)(dst + u * 16 + (lane >> 4) * 4) = o[u][nq];
      if ((lane >> 4) == 0) {
        a.part_ml[base * 2] = mrun[nq];
        a.part_ml[base * 2 + 1] = lrun[nq];
      }
    }
  }
}

// Merge split partials: o = sum_s o_s 2^(m_s - m) / sum_s l_s 2^(m_s - m).
template <typename T>
__global__ void attn_combine(const float *part_o, const float *part_ml, void *out, int rows, int Hq, int d,
                             int nsplit) {
  int r = blockIdx.x;
  for (int i = threadIdx.x; i < Hq * d; i += blockDim.x) {
    int h = i / d;
    float mx = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, part_ml[(((int64_t)s * rows + r) * Hq + h) * 2]);
    float l = 0.f, acc = 0.f;
    if (mx != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        int64_t base = ((int64_t)s * rows + r) * Hq + h;
        float ms = part_ml[base * 2];
        if (ms == -INFINITY) continue;
        float w = exp2f(ms - mx);
        l += part_ml[base * 2 + 1] * w;
        acc += part_o[base * d + (i - h * d)] * w;
      }
    }
    ((T *)out)[(int64_t)r * Hq * d + i] = from_f<T>(l > 0.f ? acc / l : 0.f);
  }
}

}  // namespace wm
