// wm_pool2.hpp — the pool mix of bf16 state stacks on MFMA.
//
// For one token row and one branch the mix is a small product,
//   m[j, c] = sum_l W[j, l] * (gamma_l[c] * S_l[c]),   W[j, l] = A[l, j] * rinv_l,
// channels j (k <= 16*KB) by layers l (L <= 32) times layers by columns c.
// A block takes RT token rows and walks the columns in 64-wide chunks; each
// of its 4 waves owns one 16-column slice of the chunk and, for every row,
// runs one 16x16x32 MFMA per branch and channel block: A = W (16 channels x
// 32 layers, bf16, built once per block into LDS), B = the gained states (32
// layers x 16 columns).  The states of the chunk are staged row-major in LDS
// ([row][layer][64 columns], 192-byte pitch) and the B fragments (8
// consecutive layers of one column per lane) come from the LDS transpose read
// ds_read_b64_tr_b16: in each 16-lane group lane i receives element i%4 of
// the 8-byte rows addressed by lanes i/4 + 4e, so lane i addresses layer
// i/4 (+4) at column 4*(i%4) and receives 4 layers of column i per read.  The
// source gains multiply the fragment in fp32 before it is rounded to bf16, so
// one staged chunk serves both branches, and each wave loads its slice's gains
// once per chunk for all RT rows.  The output m * rho (channel gain folded, its
// 1/rms applied after the projection) is stored as bf16; the per-channel sums
// of squares are reduced in a fixed order into rinvM.
//
// With k <= 8 and L <= 16 (PB) the two branches share one MFMA per row and
// slice: A is block diagonal (lane row li = 8 beta + j is channel j of branch
// beta; k chunks 0-1 = branch 0's 16 layers, 2-3 = branch 1's),
// and the B fragment's chunks 2-3 carry the same states as 0-1 under branch
// 1's source gains.  That removes the channel and layer padding of the
// per-branch MFMAs (half of M and half of K) and half of the gain loads,
// products and output writes.
#pragma once

#include "wm_common.hpp"

namespace wm {

constexpr int PM_RT4 = 4;   // token rows per block with one channel block (k <= 16)
constexpr int PM_RTPB = 4;  // token rows per block with both branches in one MFMA
constexpr int PM_CW = 64;   // columns per chunk
constexpr int PM_SP = 96;   // staged row pitch (elements): 64 columns + 64 bytes

// Router output A: element (z, beta, row, l*k + j) at z*zstride +
// beta*bstride + row*rstride + l*k + j, summed over the Z split partials;
// S [L, rows, D]; mb [2, k, rows, D]; rinvM [2, k, rows].
// (gains: src_gain (beta, l, c) at beta*sgb + l*D + c, chan_gain (beta, j, c)
// at beta*cgb + j*D + c)
template <int KB, int LMAX, bool PB = false, int RT = 0>
__global__ __launch_bounds__(256, 2) void pool_mix2(const bf16 *S, const float *rinvS, const float *A, int Z,
                                                 int64_t zstride, int64_t bstride, int64_t rstride,
                                                 const float *src_gain, int64_t sgb, const float *chan_gain,
                                                 int64_t cgb, bf16 *mb, float *rinvM, int rows, int L, int k, int D,
                                                 float eps) {
  static_assert(!PB || (KB == 1 && LMAX == 16), "branches share an MFMA only for k <= 8 and L <= 16");
  // token rows per block (RT > 0: set by the caller, one row for the few-row
  // steps of decoding, whose 64 rows would otherwise fill only 16 blocks)
  constexpr int PM_RT = RT > 0 ? RT : PB ? PM_RTPB : PM_RT4 / KB;
  constexpr int NB = PB ? 1 : 2;                       // MFMA A operands per row and channel block
  constexpr int CH = PB ? 8 : 16 * KB;                 // staged output channels per branch and row
  constexpr int NPT = (PM_RT * LMAX * 8 + 255) / 256;  // 16-byte pieces per thread and chunk (L <= LMAX)
  __shared__ __attribute__((aligned(16))) bf16 Sl[PM_RT * LMAX * PM_SP];
  __shared__ __attribute__((aligned(16))) u32x4 Wl[PM_RT][NB][KB][64];
  __shared__ float red[4][PM_RT][2][KB][16];
  // output chunk [beta][row][channel][64 columns], 144-byte rows: the four
  // lane groups of a wave write channels 16 banks apart
  constexpr int OP = 72;
  __shared__ __attribute__((aligned(16))) bf16 Ol[2 * PM_RT * CH * OP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int r0 = blockIdx.x * PM_RT;

  // W fragments: lane holds channel 16*kb + li, layers 8*g .. 8*g + 7
  // (PB: one fragment per row, block diagonal: lane row li is channel li % 8
  // of branch li / 8, k chunk g holds layers 8 (g % 2) .. + 7 of branch g / 2)
  for (int item = wave; item < (PB ? PM_RT : PM_RT * 2 * KB); item += 4) {
    const int rr = PB ? item : item / (2 * KB), beta = PB ? li >> 3 : (item / KB) & 1, kb = PB ? 0 : item % KB;
    const int lb = PB ? 8 * (g & 1) : 8 * g;  // first layer of the lane's k chunk
    const bool own = !PB || (g >> 1) == beta;  // (PB: the chunk belongs to the lane's branch)
    const int row = min(r0 + rr, rows - 1), j = PB ? (li & 7) : 16 * kb + li;
    // (every load of the item is issued before any is used: Z <= 4 partials
    // of 8 layers plus their row scales, addresses clamped into range)
    const int jc = min(j, k - 1);
    float part[4][8], rs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int lc = min(lb + e, L - 1);
#pragma unroll
      for (int z = 0; z < 4; ++z)
        part[z][e] = A[min(z, Z - 1) * zstride + beta * bstride + row * rstride + lc * k + jc];
      rs[e] = rinvS[(int64_t)lc * rows + row];
    }
    float wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = part[0][e];
#pragma unroll
      for (int z = 1; z < 4; ++z)
        if (z < Z) a += part[z][e];
      wv[e] = (own && j < k && lb + e < L) ? a * rs[e] : 0.f;
    }
    Wl[rr][PB ? 0 : beta][kb][lane] = pack16<bf16>(wv);
  }

  // staging of one chunk: piece q = (rr, layer, p), 16 bytes, layer < L; the
  // loads of the next PD chunks are in flight (a register ring; addresses
  // past the last chunk re-read it, so every load is unconditional)
  constexpr int PD = 1;
  const int npieces = PM_RT * L * 8;
  const int nchunk = D / PM_CW;
  u32x4 pre[PD][NPT];
  auto gload = [&](u32x4 (&buf)[NPT], int chunk) {
    chunk = min(chunk, nchunk - 1);
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int q = min(tid + 256 * i, npieces - 1);
      const int rr = q / (L * 8), rem = q - rr * L * 8, l = rem >> 3, p = rem & 7;
      const int row = min(r0 + rr, rows - 1);
      buf[i] = *(const u32x4 *)(S + ((int64_t)l * rows + row) * D + chunk * PM_CW + 8 * p);
    }
  };
  auto sstore = [&](const u32x4 (&buf)[NPT]) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int q = tid + 256 * i;
      if (q < npieces) {
        const int rr = q / (L * 8), rem = q - rr * L * 8, l = rem >> 3, p = rem & 7;
        *(u32x4 *)(&Sl[(rr * LMAX + l) * PM_SP + 8 * p]) = buf[i];
      }
    }
  };

  float ss[PM_RT][2][KB][4];
#pragma unroll
  for (int rr = 0; rr < PM_RT; ++rr)
#pragma unroll
    for (int beta = 0; beta < 2; ++beta)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss[rr][beta][kb][i] = 0.f;

  // transpose-read sources of this lane: layers 8g + li/4 and 8g + 4 + li/4
  // (clamped to L-1: rows past L are never staged; their weights are zero),
  // column 4*(li%4) of the wave's slice
  typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const int gl = PB ? (g & 1) : g;  // the lane's layer chunk
  const int tr_lo = min(8 * gl + (li >> 2), L - 1) * PM_SP + 16 * wave + 4 * (li & 3);
  const int tr_hi = min(8 * gl + 4 + (li >> 2), L - 1) * PM_SP + 16 * wave + 4 * (li & 3);

  // one token row per block (RT = 1, both branches on their own MFMAs): the
  // gains of the next chunk are loaded while the current one is computed, in
  // flight with its staged states, so a chunk waits for one memory round
  // trip instead of two (no other rows' work hides them); with more rows
  // per block the registers this takes would cost a block per CU
  constexpr bool GP = !PB && PM_RT == 1;
  float gsn[2][8], grn[2][KB][4];
  auto gainload = [&](int chunk) {
    chunk = min(chunk, nchunk - 1);
    const int col = chunk * PM_CW + 16 * wave + li;
#pragma unroll
    for (int beta = 0; beta < 2; ++beta) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gsn[beta][e] = src_gain[beta * sgb + (int64_t)min(8 * g + e, L - 1) * D + col];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          grn[beta][kb][i] = chan_gain[beta * cgb + (int64_t)min(16 * kb + 4 * g + i, k - 1) * D + col];
    }
  };

#pragma unroll
  for (int u = 0; u < PD; ++u) gload(pre[u], u);
  if constexpr (GP) gainload(0);
  for (int c0 = 0; c0 < nchunk; c0 += PD)
#pragma unroll
  for (int u = 0; u < PD; ++u) {
    const int chunk = c0 + u;
    if (chunk >= nchunk) break;
    __syncthreads();  // the previous chunk's reads of Sl are done
    sstore(pre[u]);
    gload(pre[u], chunk + PD);
    __syncthreads();
    const int col = chunk * PM_CW + 16 * wave + li;
    // gains of this lane's column: source gains for layers 8g..8g+7, channel
    // gains for channels 16kb + 4g + i
    if constexpr (PB) {
      // the lane's branch g / 2: source gains of its 8 layers, channel gains
      // of its 4 output channels 4 (g % 2) + i
      const int bl = g >> 1;
      float gs[8], gr[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) gs[e] = src_gain[bl * sgb + (int64_t)min(8 * (g & 1) + e, L - 1) * D + col];
#pragma unroll
      for (int i = 0; i < 4; ++i) gr[i] = chan_gain[bl * cgb + (int64_t)min(4 * (g & 1) + i, k - 1) * D + col];
#pragma unroll
      for (int rr = 0; rr < PM_RT; ++rr) {
        const bf16 *base = &Sl[rr * LMAX * PM_SP];
        const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + tr_lo));
        const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + tr_hi));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        float x[8];
        unpack16<bf16>(u32x4{l2[0], l2[1], h2[0], h2[1]}, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= gs[e];
        f32x4 m = f32x4{0.f, 0.f, 0.f, 0.f};
        mma16<bf16>(m, Wl[rr][0][0][lane], pack16<bf16>(x));
        // accumulator row 4g + i: channel 4 (g % 2) + i of branch g / 2
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ss[rr][0][0][i] += m[i] * m[i];
          Ol[((bl * PM_RT + rr) * CH + 4 * (g & 1) + i) * OP + 16 * wave + li] = (bf16)(m[i] * gr[i]);
        }
      }
    } else {
    // (GP: the gains loaded during the previous chunk)
    if constexpr (!GP) gainload(chunk);
    float gs[2][8], gr[2][KB][4];
#pragma unroll
    for (int beta = 0; beta < 2; ++beta) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gs[beta][e] = gsn[beta][e];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) gr[beta][kb][i] = grn[beta][kb][i];
    }
    if constexpr (GP) gainload(chunk + 1);
#pragma unroll
    for (int rr = 0; rr < PM_RT; ++rr) {
      const int row = r0 + rr;
      const bf16 *base = &Sl[rr * LMAX * PM_SP];
      const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + tr_lo));
      const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + tr_hi));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      float x[8];
      unpack16<bf16>(u32x4{l2[0], l2[1], h2[0], h2[1]}, x);
#pragma unroll
      for (int beta = 0; beta < 2; ++beta) {
        float y[8];
        (void)row;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[e] * gs[beta][e];
        const u32x4 bfr = pack16<bf16>(y);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          f32x4 m = f32x4{0.f, 0.f, 0.f, 0.f};
          mma16<bf16>(m, Wl[rr][beta][kb][lane], bfr);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ss[rr][beta][kb][i] += m[i] * m[i];
            Ol[((beta * PM_RT + rr) * CH + 16 * kb + 4 * g + i) * OP + 16 * wave + li] =
                (bf16)(m[i] * gr[beta][kb][i]);
          }
        }
      }
    }
    }
    // the chunk's outputs: 16-byte pieces of 128-byte rows
    __syncthreads();
    for (int q = tid; q < 2 * PM_RT * k * 8; q += 256) {
      const int pc = q & 7, t = q >> 3, j = t % k, br = t / k, rr = br % PM_RT, beta = br / PM_RT;
      const int row = r0 + rr;
      if (row < rows)
        *(u32x4 *)(mb + (((int64_t)beta * k + j) * rows + row) * D + chunk * PM_CW + 8 * pc) =
            *(const u32x4 *)(&Ol[((beta * PM_RT + rr) * CH + j) * OP + 8 * pc]);
    }
  }

  // sums of squares: over the 16 columns of the slice (lanes of a group),
  // then over the 4 slices in wave order
#pragma unroll
  for (int o = 8; o > 0; o >>= 1)
#pragma unroll
    for (int rr = 0; rr < PM_RT; ++rr)
#pragma unroll
      for (int beta = 0; beta < (PB ? 1 : 2); ++beta)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) ss[rr][beta][kb][i] += __shfl_xor(ss[rr][beta][kb][i], o);
  if (li == 0) {
    if constexpr (PB) {
#pragma unroll
      for (int rr = 0; rr < PM_RT; ++rr)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][rr][g >> 1][0][4 * (g & 1) + i] = ss[rr][0][0][i];
    } else {
#pragma unroll
      for (int rr = 0; rr < PM_RT; ++rr)
#pragma unroll
        for (int beta = 0; beta < 2; ++beta)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][rr][beta][kb][4 * g + i] = ss[rr][beta][kb][i];
    }
  }
  __syncthreads();
  for (int item = tid; item < PM_RT * 2 * KB * 16; item += 256) {
    const int rr = item / (2 * KB * 16), rem = item % (2 * KB * 16), beta = rem / (KB * 16), kb = (rem / 16) % KB,
              jj = rem % 16;
    const int j = 16 * kb + jj, row = r0 + rr;
    if (j < k && row < rows) {
      const float v = ((red[0][rr][beta][kb][jj] + red[1][rr][beta][kb][jj]) + red[2][rr][beta][kb][jj]) +
                      red[3][rr][beta][kb][jj];
      rinvM[((int64_t)beta * k + j) * rows + row] = rsqrtf(v / D + eps);
    }
  }
}

}  // namespace wm
