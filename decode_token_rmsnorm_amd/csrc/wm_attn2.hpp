// wm_attn2.hpp — strict-causal channel attention, bf16, for token sets with
// many query rows per (sequence, KV head) pair (prefill group steps).
//
// Same contract as attn_kernel (wm_attn.hpp), rows rho = m*G + g of one
// (b, hk) pair at position s0 + m*step, keys s < position, partials for the
// split combine, except for the grid: (B*Hkv, row blocks, splits) with
// blockIdx.y = 0 the pair's last row block.  A block's work grows with its
// last position, so the longest blocks of every pair are dispatched first and
// the short ones fill in behind them.  A block is 4 waves of
// 32*QB query rows; 64-key tiles of K and V are staged row-major in LDS,
// double buffered, and shared by the waves.
//
// Both products use 32x32x16 MFMAs, so every K and V element read from LDS
// serves 32 queries.  Scores are computed transposed, S^T = K Q^T, one 32x32
// accumulator per 32-key half of the tile: a lane holds 16 of the half's keys
// for one query (column lane%32) and lane ^ 32 the other 16, so the
// online-softmax statistics need one exchange and the output rescale is
// lane-local (the halves' order is described at the tile loop).  The probabilities feed O^T += V^T P^T straight from the
// accumulators: the MFMA k slot j of lane half h stands for key 4h + j
// (j < 4) or 8 + 4h + (j - 4) of each 16-key slice.  V stays row-major in
// LDS and its transposed fragments come from the LDS transpose read
// (ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4 of
// the 8-byte rows addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12), with
// lane i addressing key 4h + i/4 (+ slice offset) at head dims 4(i%4) of its
// 16-dim half; two reads give the 8 slots.
//
// LDS layouts (rows padded, not swizzled, so every fragment address is a
// per-lane base plus an immediate offset):
//  K tile: row = key, DH bf16 + 16 bytes; the 32-row fragment reads and the
//          row-wise stores are conflict-free in a 64-bank model.
//  V tile: row = key, DH bf16 + 64 bytes, so the 4 keys x 32 bytes read by a
//          16-lane group and the other half of the head dims fall on disjoint
//          banks.
#pragma once

#include "wm_attn.hpp"
#include "wm_gemm.hpp"

namespace wm {

typedef float f32x16 __attribute__((ext_vector_type(16)));


// QB 32-row query blocks per wave (block = 4 waves = 128*QB rows): with QB = 2
// every K and V fragment read from LDS feeds two MFMAs.
template <int DH, int QB>
__global__ __launch_bounds__(256, 3 - QB) void attn2_kernel(AttnArgs a) {
  static_assert(DH == 64 || DH == 128, "head dim");
  static_assert(QB == 1 || QB == 2, "query blocks per wave");
  constexpr int KT = 64;                          // keys per tile
  constexpr int NCH = DH / 16;                    // 16-deep MFMA steps over the head dim
  constexpr int CPR = DH / 8;                     // 16-byte chunks per key row
  constexpr int ND = DH / 32;                     // 32-row blocks of O^T
  constexpr int KP = DH + 8;                      // K row pitch (elements)
  constexpr int VP = DH + 32;                     // V row pitch (elements)
  constexpr int RB = 128 * QB;                    // rows per block
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][KT * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][KT * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, ql = lane & 31;
  const int pair = blockIdx.x, b = pair / a.Hkv, hk = pair - b * a.Hkv;
  const int nrows = a.M * a.G;
  const int rb0 = (gridDim.y - 1 - blockIdx.y) * RB;
  if (rb0 >= nrows) return;
  const int last = min(nrows, rb0 + RB) - 1;
  const int s0 = attn_s0(a);
  const int kmax = min(s0 + (last / a.G) * a.step, a.T_max);  // keys s < kmax for the block
  const int ntile = (kmax + KT - 1) / KT;
  const int tps = (ntile + a.nsplit - 1) / a.nsplit;
  const int t0 = blockIdx.z * tps, t1 = min(ntile, t0 + tps);

  // this lane's query in each block qb (rows past the end read the last row
  // and store nothing)
  bool rvalid[QB];
  int rpos[QB], rrow[QB], rhead[QB];
  u32x4 qf[QB][NCH];
  int minpos = 0x7fffffff, maxpos = 0;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int rho_raw = rb0 + wave * 32 * QB + qb * 32 + ql;
    rvalid[qb] = rho_raw < nrows;
    const int rho = rvalid[qb] ? rho_raw : nrows - 1;
    const int m = rho / a.G, g = rho - m * a.G;
    rpos[qb] = s0 + m * a.step;
    rrow[qb] = b * a.M + m;
    rhead[qb] = hk * a.G + g;
    const bf16 *src = (const bf16 *)a.q + ((int64_t)rrow[qb] * a.Hq + rhead[qb]) * DH + 8 * h;
#pragma unroll
    for (int c = 0; c < NCH; ++c) qf[qb][c] = *(const u32x4 *)(src + 16 * c);
    if (rvalid[qb]) {
      minpos = min(minpos, rpos[qb]);
      maxpos = max(maxpos, rpos[qb]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): queries resident before the K/V prefetch starts
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    minpos = min(minpos, __shfl_xor(minpos, off));
    maxpos = max(maxpos, __shfl_xor(maxpos, off));
  }
  minpos = __builtin_amdgcn_readfirstlane(minpos);  // (wave-uniform: branches on them stay scalar)
  maxpos = __builtin_amdgcn_readfirstlane(maxpos);

  f32x16 o[QB][ND];
  float mrun[QB], lrun[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrun[qb] = -INFINITY;
    lrun[qb] = 0.f;
#pragma unroll
    for (int u = 0; u < ND; ++u) o[qb][u] = f32x16{};
  }

  const bf16 *Kb = (const bf16 *)a.Kc + ((int64_t)b * a.Hkv + hk) * a.T_max * DH;
  const bf16 *Vb = (const bf16 *)a.Vc + ((int64_t)b * a.Hkv + hk) * a.T_max * DH;
  const int klast = kmax - 1;

  // global -> registers (addresses clamped to the last key, no branches)
  constexpr int RPT = KT * CPR / 256;  // 16-byte chunks per thread of each of K and V
  u32x4 kreg[RPT], vreg[RPT];
  auto gload = [&](int t) {
    const int key0 = t * KT;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = tid + 256 * i, kr = c / CPR, cc = c - kr * CPR;
      const int64_t off = (int64_t)min(key0 + kr, klast) * DH + 8 * cc;
      kreg[i] = *(const u32x4 *)(Kb + off);
      vreg[i] = *(const u32x4 *)(Vb + off);
    }
  };
  // registers -> LDS stage st
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = tid + 256 * i, kr = c / CPR, cc = c - kr * CPR;
      *(u32x4 *)(&Ks[st][kr * KP + 8 * cc]) = kreg[i];
      *(u32x4 *)(&Vs[st][kr * VP + 8 * cc]) = vreg[i];
    }
  };
  // transpose-read base of this lane: key 4h + (lane%16)/4, head dim 16*((lane/16)%2) + 4*(lane%4)
  const int vbase = (4 * h + ((lane & 15) >> 2)) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
  typedef __attribute__((address_space(3))) v4s lds_v4s;

  if (t0 < t1) {
    gload(t0);
    sstore(0);
  }
  __syncthreads();
  const float sc = a.scale_log2;
  for (int t = t0; t < t1; ++t) {
    const int st = (t - t0) & 1;
    const int key0 = t * KT;
    if (t + 1 < t1) gload(t + 1);

    const bf16 *vst = &Vs[st][vbase];
    // The tile in two 32-key halves kb: S^T = K Q^T (each K fragment feeds QB
    // MFMAs), online softmax, then O^T += V^T P^T over the half's two 16-key
    // slices (each V fragment feeds QB MFMAs).  Half 1's scores are computed
    // and masked before half 0's PV products, so that half 1's softmax, which
    // has no branch, is issued among those MFMAs (it does not feed them; its
    // rescale of O waits for them).  O sees the same operations in the same
    // order as a half-by-half walk.
    auto qk = [&](int kb, f32x16 (&sc_)[QB]) {
      // K fragments first (each read would otherwise sit just before its
      // MFMA and wait out the LDS latency); the head-dim steps accumulate in
      // one chain
      u32x4 kf[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) kf[c] = *(const u32x4 *)(&Ks[st][(32 * kb + ql) * KP + 16 * c + 8 * h]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc_[qb] = f32x16{};
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc_[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[c]),
                                                            __builtin_bit_cast(bf16x8, qf[qb][c]), sc_[qb], 0, 0, 0);
    };
    // element i of sc_[qb] is key key0 + 32*kb + 8*(i/4) + 4h + i%4; keys at
    // or past the query's position get -inf (only halves that reach past the
    // wave's first query need it)
    auto mask = [&](int kb, f32x16 (&sc_)[QB]) {
      const int kb0 = key0 + 32 * kb;
      if (kb0 + 32 > minpos) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb0 + 8 * (i >> 2) + 4 * h + (i & 3) >= rpos[qb]) sc_[qb][i] = -INFINITY;
      }
    };
    // scores -> probabilities in place, running max and sum; alpha = the
    // factor O must be rescaled by before this half's PV products.  Lazy
    // rescaling: the reference max moves only when the half's max exceeds it
    // by more than 2^8, so probabilities stay <= 256 and O is rescaled
    // rarely; numerator and denominator share the reference, so the result
    // is unchanged.  Selects instead of branches: alpha = 2^(m_old - m_new)
    // when the reference moves (0 on the first finite max), else 1; a row
    // with no unmasked key so far keeps m = -inf and gets p = 0.
    auto softmax = [&](f32x16 (&sc_)[QB], float (&alpha)[QB]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc_[qb][i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float tm = tmax * sc;
        const bool upd = tm > mrun[qb] + 8.f;
        const float mnew = upd ? tm : mrun[qb];
        const float e = __builtin_amdgcn_exp2f(mrun[qb] - mnew);
        alpha[qb] = upd ? e : 1.f;
        const float nm = mnew == -INFINITY ? 0.f : -mnew;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc_[qb][i], sc, nm));
          sc_[qb][i] = p;
          psum += p;
        }
        psum += __shfl_xor(psum, 32);
        lrun[qb] = lrun[qb] * alpha[qb] + psum;
        mrun[qb] = mnew;
      }
    };
    auto rescale = [&](const float (&alpha)[QB]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        if (__any(alpha[qb] != 1.f)) {
#pragma unroll
          for (int u = 0; u < ND; ++u) o[qb][u] *= alpha[qb];
        }
    };
    // probabilities of a half as bf16 MFMA operands, one per 16-key slice
    auto pack = [&](const f32x16 (&p_)[QB], u32x4 (&pf)[2][QB]) {
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float pv_[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) pv_[j] = p_[qb][8 * half + j];
          pf[half][qb] = pack16<bf16>(pv_);
        }
    };
    auto pv = [&](int kb, const u32x4 (&pf)[2][QB]) {
      // V^T fragments of the half's two 16-key slices, all read before the MFMAs
      u32x4 vf[2][ND];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int u = 0; u < ND; ++u) {
          const int sl = 2 * kb + half;  // 16-key slice of the tile
          const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vst + 16 * sl * VP + 32 * u));
          const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vst + (16 * sl + 8) * VP + 32 * u));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          vf[half][u] = u32x4{l2[0], l2[1], h2[0], h2[1]};
        }
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int u = 0; u < ND; ++u)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[half][u]),
                                                               __builtin_bit_cast(bf16x8, pf[half][qb]), o[qb][u], 0,
                                                               0, 0);
    };
    // A tile whose keys all lie at or past every query of this wave adds
    // nothing (its probabilities are 0 and the running max stays), so the
    // wave skips it; the block still stages every tile up to its own last
    // query, which the other waves may need.  (Half 1 of the last tile a
    // wave takes may be fully masked; it runs and adds zeros.)
    if (key0 < maxpos) {
      f32x16 sc0[QB], sc1[QB];
      float al0[QB], al1[QB];
      u32x4 pf0[2][QB], pf1[2][QB];
      qk(0, sc0);
      mask(0, sc0);
      softmax(sc0, al0);
      pack(sc0, pf0);
      qk(1, sc1);
      mask(1, sc1);
      rescale(al0);
      pv(0, pf0);
      softmax(sc1, al1);
      pack(sc1, pf1);
      rescale(al1);
      pv(1, pf1);
    }
    if (t + 1 < t1) sstore(st ^ 1);
    __syncthreads();
  }

  // write out: lane holds query ql of block qb, head dims u*32 + 8*(i/4) + 4h + i%4
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (!rvalid[qb]) continue;
    if (a.nsplit == 1) {
      const float inv = lrun[qb] > 0.f ? 1.f / lrun[qb] : 0.f;
      bf16 *dst = (bf16 *)a.out + (int64_t)rrow[qb] * a.Hq * DH + rhead[qb] * DH;
#pragma unroll
      for (int u = 0; u < ND; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[qb][u][4 * j + e] * inv;
          stT<bf16, 4>(dst + u * 32 + 8 * j + 4 * h, v);
        }
    } else {
      const int64_t base = ((int64_t)blockIdx.z * a.B * a.M + rrow[qb]) * a.Hq + rhead[qb];
      float *dst = a.part_o + base * DH;
#pragma unroll
      for (int u = 0; u < ND; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(f32x4 *)(dst + u * 32 + 8 * j + 4 * h) =
              f32x4{o[qb][u][4 * j], o[qb][u][4 * j + 1], o[qb][u][4 * j + 2], o[qb][u][4 * j + 3]};
      if (h == 0) {
        a.part_ml[base * 2] = mrun[qb];
        a.part_ml[base * 2 + 1] = lrun[qb];
      }
    }
  }
}

// Few query rows per (sequence, KV head) pair (decode steps, small group
// steps): attn_few.  A block of NW waves takes one (pair, key split, block of
// 32 query rows; blockIdx.z = 0 is the pair's last row block, the longest);
// wave w walks the split's 32-key tiles w, w+NW, ... with the block's query
// rows as the columns of S^T = K Q^T (32x32x16 MFMA; columns past the pair's
// rows are padding that is computed and never stored).  The K fragments of a tile are loaded straight
// from global memory in the MFMA operand layout (lane: key lane%32, head dims
// 8*(lane/32) of each 16-dim step); the V tile goes through a wave-private LDS
// buffer for the transpose reads of O^T += V^T P^T, as in attn2_kernel.  The
// next tile's loads are issued before the current tile is multiplied.  At the
// end the waves' (o, m, l) are merged through LDS in wave order, so one launch
// covers a pair without a combine kernel unless the keys are split further.
template <int DH, int NW>
__global__ __launch_bounds__(64 * NW) void attn_few(AttnArgs a) {
  static_assert(DH == 64 || DH == 128, "head dim");
  constexpr int KT = 32;                // keys per tile
  constexpr int NCH = DH / 16;          // 16-deep MFMA steps over the head dim
  constexpr int ND = DH / 32;           // 32-row blocks of O^T
  constexpr int VP = DH + 32;           // V row pitch (elements), as in attn2_kernel
  constexpr int VC = KT * DH / 8 / 64;  // 16-byte V chunks per lane per tile
  constexpr int OP = DH + 4;            // merge buffer pitch (floats)
  constexpr int VBYTES = NW * KT * VP * 2, OBYTES = NW * 32 * OP * 4;
  __shared__ __attribute__((aligned(16))) char smem[VBYTES > OBYTES ? VBYTES : OBYTES];
  __shared__ float mls[NW][2][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, ql = lane & 31;
  bf16 *Vs = (bf16 *)smem + wave * KT * VP;
  const int split = blockIdx.x, pair = blockIdx.y, b = pair / a.Hkv, hk = pair - b * a.Hkv;
  const int rb0 = (gridDim.z - 1 - blockIdx.z) * 32;  // first row of the block
  const int nrows = min(32, a.M * a.G - rb0);         // rows of the block
  const int s0 = attn_s0(a);
  const int kmax = min(s0 + ((rb0 + nrows - 1) / a.G) * a.step, a.T_max);
  const int ntile = (kmax + KT - 1) / KT;
  const int tps = (ntile + a.nsplit - 1) / a.nsplit;
  const int t0 = split * tps, t1 = min(ntile, t0 + tps);

  const bool rvalid = ql < nrows;
  const int rho = rb0 + (rvalid ? ql : nrows - 1);
  const int m = rho / a.G, g = rho - m * a.G;
  const int rpos = s0 + m * a.step;
  const int rrow = b * a.M + m, rhead = hk * a.G + g;
  u32x4 qf[NCH];
  {
    const bf16 *src = (const bf16 *)a.q + ((int64_t)rrow * a.Hq + rhead) * DH + 8 * h;
#pragma unroll
    for (int c = 0; c < NCH; ++c) qf[c] = *(const u32x4 *)(src + 16 * c);
  }
  int minpos = rvalid ? rpos : 0x7fffffff;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) minpos = min(minpos, __shfl_xor(minpos, off));

  f32x16 o[ND];
#pragma unroll
  for (int u = 0; u < ND; ++u) o[u] = f32x16{};
  float mrun = -INFINITY, lrun = 0.f;
  const bf16 *Kb = (const bf16 *)a.Kc + ((int64_t)b * a.Hkv + hk) * a.T_max * DH;
  const bf16 *Vb = (const bf16 *)a.Vc + ((int64_t)b * a.Hkv + hk) * a.T_max * DH;
  const int klast = max(kmax - 1, 0);

  u32x4 kf[NCH], vr[VC];
  auto gload = [&](int t) {  // addresses clamped to the last key: no branches
    const int key0 = t * KT;
    const bf16 *kr = Kb + (int64_t)min(key0 + ql, klast) * DH + 8 * h;
#pragma unroll
    for (int c = 0; c < NCH; ++c) kf[c] = *(const u32x4 *)(kr + 16 * c);
#pragma unroll
    for (int i = 0; i < VC; ++i) {
      const int ch = lane + 64 * i, key = ch / (DH / 8), cc = ch - key * (DH / 8);
      vr[i] = *(const u32x4 *)(Vb + (int64_t)min(key0 + key, klast) * DH + 8 * cc);
    }
  };
  const int vbase = (4 * h + ((lane & 15) >> 2)) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const float sc = a.scale_log2;

  int t = t0 + wave;
  if (t < t1) gload(t);
  for (; t < t1; t += NW) {
    const int key0 = t * KT;
    u32x4 kc[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) kc[c] = kf[c];
#pragma unroll
    for (int i = 0; i < VC; ++i) {
      const int ch = lane + 64 * i, key = ch / (DH / 8), cc = ch - key * (DH / 8);
      *(u32x4 *)(&Vs[key * VP + 8 * cc]) = vr[i];
    }
    if (t + NW < t1) gload(t + NW);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's V stores landed
    __builtin_amdgcn_wave_barrier();

    f32x16 sa = f32x16{}, sb = f32x16{};
#pragma unroll
    for (int c = 0; c < NCH; c += 2) {
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kc[c]), __builtin_bit_cast(bf16x8, qf[c]),
                                                   sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kc[c + 1]),
                                                   __builtin_bit_cast(bf16x8, qf[c + 1]), sb, 0, 0, 0);
    }
    f32x16 s = sa + sb;
    // element i is key key0 + 8*(i/4) + 4h + i%4 of query column ql
    if (key0 + KT > minpos) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + 8 * (i >> 2) + 4 * h + (i & 3) >= rpos) s[i] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // lazy rescaling, as in attn2_kernel
    const float tm = tmax * sc;
    const bool upd = tm > mrun + 8.f;
    const float mnew = upd ? tm : mrun;
    const float alpha = upd && mrun != -INFINITY ? __builtin_amdgcn_exp2f(mrun - mnew) : (upd ? 0.f : 1.f);
    const float nm = mnew == -INFINITY ? 0.f : -mnew;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[i], sc, nm));
      s[i] = p;
      psum += p;
    }
    psum += __shfl_xor(psum, 32);
    lrun = lrun * alpha + psum;
    mrun = mnew;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int u = 0; u < ND; ++u) o[u] *= alpha;
    }
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = s[8 * sl + j];
      const u32x4 pf = pack16<bf16>(pv);
#pragma unroll
      for (int u = 0; u < ND; ++u) {
        const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(&Vs[vbase + 16 * sl * VP + 32 * u]));
        const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(&Vs[vbase + (16 * sl + 8) * VP + 32 * u]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 vf{l2[0], l2[1], h2[0], h2[1]};
        o[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf), __builtin_bit_cast(bf16x8, pf),
                                                       o[u], 0, 0, 0);
      }
    }
    // the next tile's V stores must not overtake this tile's transpose reads
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
  }

  // merge of the waves, in wave order: M = max m_w, o = sum o_w 2^(m_w - M),
  // l = sum l_w 2^(m_w - M)
  if (h == 0) {
    mls[wave][0][ql] = mrun;
    mls[wave][1][ql] = lrun;
  }
  __syncthreads();  // also: every wave is done with its V buffer
  float mmax = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) mmax = fmaxf(mmax, mls[w][0][ql]);
  const float f = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - mmax);
  float *Os = (float *)smem;
  if (rvalid) {
#pragma unroll
    for (int u = 0; u < ND; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(f32x4 *)(&Os[(wave * 32 + ql) * OP + u * 32 + 8 * j + 4 * h]) =
            f32x4{o[u][4 * j] * f, o[u][4 * j + 1] * f, o[u][4 * j + 2] * f, o[u][4 * j + 3] * f};
  }
  __syncthreads();
  // thread -> (query row, 4 head dims)
  for (int item = tid; item < nrows * (DH / 4); item += 64 * NW) {
    const int q = item / (DH / 4), d4 = 4 * (item - q * (DH / 4));
    float lsum = 0.f, mq = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mq = fmaxf(mq, mls[w][0][q]);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = mls[w][0][q];
      lsum += mw == -INFINITY ? 0.f : mls[w][1][q] * __builtin_amdgcn_exp2f(mw - mq);
      acc += *(const f32x4 *)(&Os[(w * 32 + q) * OP + d4]);
    }
    const int mm = (rb0 + q) / a.G, gg = rb0 + q - mm * a.G;
    const int orow = b * a.M + mm, ohead = hk * a.G + gg;
    if (a.nsplit == 1) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      float v[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
      stT<bf16, 4>((bf16 *)a.out + (int64_t)orow * a.Hq * DH + ohead * DH + d4, v);
    } else {
      const int64_t base = ((int64_t)split * a.B * a.M + orow) * a.Hq + ohead;
      *(f32x4 *)(a.part_o + base * DH + d4) = acc;
      if (d4 == 0) {
        a.part_ml[base * 2] = mq;
        a.part_ml[base * 2 + 1] = lsum;
      }
    }
  }
}

}  // namespace wm
