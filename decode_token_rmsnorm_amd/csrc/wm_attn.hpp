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
  const int32_t *s0p;  // when set: s0 = *s0p read at run time, clamped to [0, T_max)
};

__device__ __forceinline__ int attn_s0(const AttnArgs &a) {
  return a.s0p ? min(max(*a.s0p, 0), a.T_max - 1) : a.s0;
}

// Transposed value tile: row dd (head dim), 64 keys in 16 quads of 4. Quad q
// of row dd is stored at quad position q ^ (dd / E % 16) (E = elements per 16
// bytes), which makes both the transposing stores (16 lanes writing 16 rows of
// one quad) and the MFMA fragment reads (16 lanes reading 16 consecutive rows)
// hit distinct banks.
__device__ __forceinline__ int vswz(int q, int chunk) { return q ^ (chunk & 15); }

// Raw element e of a 16-byte fragment, as bits (no conversion).
template <typename T> __device__ __forceinline__ uint32_t elt_bits(const u32x4 &v, int e);
template <> __device__ __forceinline__ uint32_t elt_bits<float>(const u32x4 &v, int e) { return v[e]; }
template <> __device__ __forceinline__ uint32_t elt_bits<bf16>(const u32x4 &v, int e) {
  return (v[e >> 1] >> (16 * (e & 1))) & 0xffffu;
}
// Store element e of four keys' fragments as 4 consecutive elements.
template <typename T> __device__ __forceinline__ void store4(T *dst, const u32x4 *v, int e);
template <> __device__ __forceinline__ void store4<float>(float *dst, const u32x4 *v, int e) {
  *(u32x4 *)dst = u32x4{v[0][e], v[1][e], v[2][e], v[3][e]};
}
template <> __device__ __forceinline__ void store4<bf16>(bf16 *dst, const u32x4 *v, int e) {
  *(u32x2 *)dst = u32x2{elt_bits<bf16>(v[0], e) | (elt_bits<bf16>(v[1], e) << 16),
                        elt_bits<bf16>(v[2], e) | (elt_bits<bf16>(v[3], e) << 16)};
}

template <typename T, int DH, int NW, int NQ>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  constexpr int E = Elt<T>::E16;       // elements per 16-byte fragment
  constexpr int KCH = 4 * E;           // k (head dim) per MFMA step
  constexpr int NCH = DH / KCH;        // MFMA steps over the head dim
  constexpr int KP = DH + 16 / (int)sizeof(T);  // key-row pitch (elements), +16 B
  constexpr int VP = AKT + 16 / (int)sizeof(T); // transposed value pitch (elements)
  constexpr int PVK = 4 * E;           // keys per PV MFMA step
  constexpr int RB = NW * NQ * 16;     // rows per block
  constexpr int NT = NW * 64;
  constexpr int CPR = DH / E;          // 16-byte chunks per key row
  constexpr int KPT = (AKT * CPR + NT - 1) / NT;        // key chunks per thread
  constexpr int VPT = ((AKT / 4) * CPR + NT - 1) / NT;  // 4-key value items per thread
  __shared__ __attribute__((aligned(16))) T Ks[2][AKT * KP];
  __shared__ __attribute__((aligned(16))) T Vt[2][DH * VP];

  const T *qp = (const T *)a.q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = blockIdx.y, b = pair / a.Hkv, hk = pair - b * a.Hkv;
  const int nrows = a.M * a.G;
  const int rb0 = blockIdx.x * RB;
  if (rb0 >= nrows) return;
  const int last = min(nrows, rb0 + RB) - 1;
  const int s0 = attn_s0(a);
  int kmax = s0 + (last / a.G) * a.step;  // keys s < kmax for the block
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
    rpos[nq] = rvalid[nq] ? s0 + m * a.step : 0;
    rrow[nq] = b * a.M + m;
    rhead[nq] = hk * a.G + g;
    const T *src = qp + ((int64_t)rrow[nq] * a.Hq + rhead[nq]) * DH;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      qf[nq][c] = rvalid[nq] ? *(const u32x4 *)(src + c * KCH + (lane >> 4) * E) : u32x4{0, 0, 0, 0};
  }
  // Wait for the query fragments here, so the compiler knows they are
  // resident and does not drain the in-flight K/V prefetch to read them.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  int wave_minpos = 0x7fffffff;
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) wave_minpos = min(wave_minpos, rvalid[nq] ? rpos[nq] : 0x7fffffff);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wave_minpos = min(wave_minpos, __shfl_xor(wave_minpos, off));

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

  // Tile t: global -> registers. Loads are unconditional (addresses clamped
  // to the last valid key, so no branch stalls the prefetch); keys past kmax
  // are zeroed when the registers are written to LDS.
  u32x4 kreg[KPT], vreg[VPT][4];
  int kmaxk = kmax - 1;
  auto gload = [&](int t) {
    const int key0 = t * AKT;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int c = min(tid + NT * i, AKT * CPR - 1), kr = c / CPR, cc = c - kr * CPR;
      int key = min(key0 + kr, kmaxk);
      kreg[i] = *(const u32x4 *)(Kb + (int64_t)key * DH + cc * E);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int c = min(tid + NT * i, (AKT / 4) * CPR - 1), kq = c / CPR, cc = c - kq * CPR;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int key = min(key0 + 4 * kq + q, kmaxk);
        vreg[i][q] = *(const u32x4 *)(Vb + (int64_t)key * DH + cc * E);
      }
    }
  };
  // ... registers -> LDS stage st (keys row-major, values transposed).
  auto sstore = [&](int st, int t) {
    const int key0 = t * AKT;
    const u32x4 zero{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int c = tid + NT * i, kr = c / CPR, cc = c - kr * CPR;
      if (c < AKT * CPR) *(u32x4 *)(&Ks[st][kr * KP + cc * E]) = key0 + kr <= kmaxk ? kreg[i] : zero;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int c = tid + NT * i, kq = c / CPR, cc = c - kq * CPR;
      if (c < (AKT / 4) * CPR) {
        u32x4 v4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v4[q] = key0 + 4 * kq + q <= kmaxk ? vreg[i][q] : zero;
#pragma unroll
        for (int e = 0; e < E; ++e) store4<T>(&Vt[st][(cc * E + e) * VP + 4 * vswz(kq, cc)], v4, e);
      }
    }
  };

  if (t0 < t1) {
    gload(t0);
    sstore(0, t0);
  }
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    const int st = (t - t0) & 1;
    const int key0 = t * AKT;
    if (t + 1 < t1) gload(t + 1);

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
        u32x4 kf = *(const u32x4 *)(&Ks[st][(kt * 16 + (lane & 15)) * KP + c * KCH + (lane >> 4) * E]);
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) mma16<T>(s[kt][nq], kf, qf[nq][c]);
      }
    }

    // online softmax. Tiles whose keys all precede every row of this wave need
    // no mask; the max is taken on raw scores (the scale is positive) and the
    // scale folded into one fma before the exponential.
    const bool full = key0 + AKT <= wave_minpos;
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      if (!full) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            int key = key0 + kt * 16 + (lane >> 4) * 4 + e;
            if (key >= rpos[nq]) s[kt][nq][e] = -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, s[kt][nq][e]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(mrun[nq], tmax * a.scale_log2);
      const bool none = mnew == -INFINITY;
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(mrun[nq] - mnew);
      const float nm = none ? 0.f : -mnew;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv = __builtin_amdgcn_exp2f(fmaf(s[kt][nq][e], a.scale_log2, nm));
          s[kt][nq][e] = pv;
          psum += pv;
        }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      lrun[nq] = lrun[nq] * alpha + psum;
      mrun[nq] = mnew;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int u = 0; u < DH / 16; ++u) o[u][nq] *= alpha;
      }
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
        const int dd = u * 16 + (lane & 15), q0 = kc * (PVK / 4) + (lane >> 4);
        const T *vrow = &Vt[st][dd * VP];
        u32x4 vf;
        if constexpr (E == 8) {
          u32x2 lo = *(const u32x2 *)(vrow + 4 * vswz(q0, dd / E)),
                hi = *(const u32x2 *)(vrow + 4 * vswz(q0 + 4, dd / E));
          vf = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          vf = *(const u32x4 *)(vrow + 4 * vswz(q0, dd / E));
        }
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) mma16<T>(o[u][nq], vf, pf[nq]);
      }
    }
    if (t + 1 < t1) sstore(st ^ 1, t + 1);
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
// One thread per output element; every split's values are loaded before any
// is used (nsplit <= ACS), so a thread waits for memory once.
constexpr int ACS = 16;  // most splits the attention dispatch makes
template <typename T>
__global__ __launch_bounds__(256) void attn_combine(const float *part_o, const float *part_ml, void *out, int rows,
                                                    int Hq, int d, int nsplit) {
  const int64_t n = (int64_t)rows * Hq * d;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t rh = i / d, plane = (int64_t)rows * Hq;
  const int dd = (int)(i - rh * d);
  float ms[ACS], ls[ACS], os[ACS];
#pragma unroll
  for (int s = 0; s < ACS; ++s) {
    if (s < nsplit) {
      const int64_t base = s * plane + rh;
      ms[s] = part_ml[base * 2];
      ls[s] = part_ml[base * 2 + 1];
      os[s] = part_o[base * d + dd];
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < ACS; ++s)
    if (s < nsplit) mx = fmaxf(mx, ms[s]);
  float l = 0.f, acc = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int s = 0; s < ACS; ++s) {
      if (s < nsplit && ms[s] != -INFINITY) {
        const float w = exp2f(ms[s] - mx);
        l += ls[s] * w;
        acc += os[s] * w;
      }
    }
  }
  ((T *)out)[i] = from_f<T>(l > 0.f ? acc / l : 0.f);
}

}  // namespace wm
