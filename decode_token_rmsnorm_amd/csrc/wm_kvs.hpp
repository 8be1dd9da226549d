// wm_kvs.hpp — per-channel K/V projection of the pool for model width 512 and
// 4 KV heads of 64, with the projection matrix held in registers.
//
// Each channel's projection (z = beta*k + j) is a [rows x 512] by [512 x 256]
// product: short in k and narrow in n, so a tiled GEMM spends much of each
// tile in its prologue and epilogue, and every tile re-reads the 256 KB
// matrix.  Here a block of 8 waves owns one channel and a contiguous range of
// 32-row chunks: wave w keeps columns [32w, 32w + 32) of the channel's matrix
// for the whole launch as B fragments of the 32x32x16 bf16 MFMA (128 VGPRs
// per lane), and the mixed rows stream through a ring of 4 LDS stages of one
// chunk each (32 rows x 1 KB), two chunks ahead of the MFMAs.
//
// Wave roles keep each wave's vector-memory counter in issue order: waves
// 0-3 issue the 16-byte LDS DMAs (8 rows of each chunk, and for keys those
// rows' RoPE table entries one chunk ahead) and nothing else that goes to
// global memory after their matrix loads, so counting their outstanding
// DMAs tells them when a chunk has landed; waves 4-7 run the epilogue (row
// scale, key norm and RoPE for keys, cache scatter) of the previous chunk,
// reading only LDS and one register of row scales loaded an iteration ahead,
// while the DMA waves, one per SIMD beside them, run their MFMAs.  Every wave
// runs the MFMAs of its 32 columns.
//
// LDS rows are 1 KB; global 16-byte chunk c of chunk row r sits at position
// c ^ (r & 15), so the 16 rows a quarter-wave fragment read touches fall on
// distinct banks.  After its MFMAs a stage is reused for the fp32 C tile of
// the same chunk (32 rows x 256 columns, 32 KB), read by the epilogue one
// iteration later.
//
// Per chunk the MFMAs accumulate k in ascending 16-wide steps into one
// accumulator, the order of the large-tile GEMM.
#pragma once

#include "wm_gemm2.hpp"

namespace wm {

// v from the lane that DPP control CTRL selects (all rows and banks on).
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

constexpr int KVS_D = 512;     // model width (k of the product)
constexpr int KVS_HD = 64;     // head dim
constexpr int KVS_N = 256;     // Hkv * d (output columns per channel)
constexpr int KVS_CR = 32;     // rows per chunk
constexpr int KVS_STG = 4;     // LDS stages of rows
constexpr int KVS_RST = 3;     // LDS stages of RoPE entries
constexpr int KVS_RB = KVS_D * 2;          // bytes per staged row
constexpr int KVS_SB = KVS_CR * KVS_RB;    // bytes per row stage
constexpr int KVS_RSB = KVS_CR * KVS_HD * 4;  // bytes per RoPE stage: [cos | sin][32 rows][32]
static_assert(KVS_CR * KVS_N * 4 == KVS_SB, "the C tile of a chunk fills one stage");

// mb [2k, rows, 512] bf16 (z = beta*k + j); wk / wv [k, 256, 512] bf16; the
// epilogue arguments are those of the tiled projection (EpiKV, d = 64).
// Grid: 2k * P blocks; block b serves channel z = b / P and chunk range b % P.
__global__ __launch_bounds__(512, 1) void kv_stream(const bf16 *mb, const bf16 *wk, const bf16 *wv, EpiKV<bf16> e,
                                                    int rows, int P) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[KVS_STG * KVS_SB + KVS_RST * KVS_RSB];
  unsigned char *rope = smem + KVS_STG * KVS_SB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int z = blockIdx.x / P, p = blockIdx.x - z * P;
  const int nch = (rows + KVS_CR - 1) / KVS_CR, cpb = (nch + P - 1) / P;
  const int cbeg = p * cpb, n = min(nch, cbeg + cpb) - cbeg;
  if (n <= 0) return;  // (the whole block: no barrier is reached)
  const int beta = z / e.k, j = z - beta * e.k;
  const bool isK = beta == 0;
  const bf16 *W = (isK ? wk : wv) + (int64_t)j * KVS_N * KVS_D;
  const bf16 *A = mb + (int64_t)z * rows * KVS_D;
  const bool dw = wave < 4;      // DMA waves (wave-uniform)
  const int pbase = e.rp.base();  // (read before any DMA is in flight)
  auto posof = [&](int r) { return pbase + (r % e.rp.M) * e.rp.step; };

  // matrix fragments: column 32*wave + lane%32, k = 16 s + 8 (lane/32) .. + 7
  u32x4 wf[KVS_D / 16];
  {
    const bf16 *wr = W + (int64_t)(32 * wave + (lane & 31)) * KVS_D + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < KVS_D / 16; ++s) wf[s] = *(const u32x4 *)(wr + 16 * s);
  }

  // DMA waves: chunk c's rows 8*wave .. 8*wave+7 into row stage c%4, and
  // (keys) the cos and sin entries of those rows' positions into RoPE stage
  // c%3: lane l carries 16 bytes of row 8*wave + l/8
  auto issue_rows = [&](int c) {
    unsigned char *st = smem + (c % KVS_STG) * KVS_SB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * wave + i;
      const int grow = min((cbeg + c) * KVS_CR + r, rows - 1);
      dma16(A + (int64_t)grow * KVS_D + 8 * (lane ^ (r & 15)), st + r * KVS_RB);
    }
  };
  auto issue_rope = [&](int c) {
    unsigned char *rs = rope + (c % KVS_RST) * KVS_RSB;
    const int grow = min((cbeg + c) * KVS_CR + 8 * wave + (lane >> 3), rows - 1);
    const int64_t off = (int64_t)posof(grow) * (KVS_HD / 2) + 4 * (lane & 7);
    dma16(e.cosT + off, rs + wave * 1024);
    dma16(e.sinT + off, rs + KVS_RSB / 2 + wave * 1024);
  };
  // the last batch issued (chunk c+1's rows and, for keys, chunk c's RoPE
  // entries) may stay in flight while chunk c is used
  auto wait_batch = [&](bool rows_pending) {
    if (isK) {
      if (rows_pending) wait_vmcnt<10>();
      else wait_vmcnt<2>();
    } else {
      if (rows_pending) wait_vmcnt<8>();
      else wait_vmcnt<0>();
    }
  };

  // epilogue of chunk c from the C tile in row stage c%4 (waves 4-7, 8 rows
  // each, 2 per step): the EpiKV arithmetic of the tiled projection, with the
  // row scales in rv (lane i%32: row i of the chunk) and the RoPE entries in
  // LDS.  Lane l owns columns 4l .. 4l+3, so a head is one 16-lane DPP row:
  // the head's sum of squares is a row rotation by 8, 4, 2, 1 (each step adds
  // the value the xor-by-8, 4, 2, 1 exchange would bring, so the sum is the
  // same as the shuffle tree's) and RoPE's partner element sits 8 lanes away.
  const int cc = 4 * lane, hh = cc / KVS_HD, dd = cc - hh * KVS_HD;
  const bool first_half = dd < KVS_HD / 2;
  bf16 *obase = isK ? e.Kc : e.Vc;
  float g[4];
  ldf<4>(g, e.knorm + (int64_t)j * KVS_HD + dd);
  auto epi = [&](int c, float rv) {
    constexpr int ER4 = 2;
    const float *Cs = (const float *)(smem + (c % KVS_STG) * KVS_SB);
    const float *rc = (const float *)(rope + (c % KVS_RST) * KVS_RSB);
    const int mrope = dd & (KVS_HD / 2 - 1);
    const int rb0 = (wave - 4) * 8, r0 = (cbeg + c) * KVS_CR + rb0;
    int b = r0 / e.rp.M, rem = r0 - b * e.rp.M;  // sequence and index of row r0
#pragma unroll
    for (int rb = rb0; rb < rb0 + 8; rb += ER4) {
      float cs[ER4][4], sn[ER4][4], x[ER4][4];
#pragma unroll
      for (int u = 0; u < ER4; ++u) {
        const float rs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rv), rb + u));
        ldf<4>(x[u], Cs + (rb + u) * KVS_N + cc);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[u][i] *= rs;
        if (isK) {
          ldf<4>(cs[u], rc + (rb + u) * (KVS_HD / 2) + mrope);
          ldf<4>(sn[u], rc + KVS_RSB / 8 + (rb + u) * (KVS_HD / 2) + mrope);
        }
      }
      if (isK) {
        float sq[ER4];
#pragma unroll
        for (int u = 0; u < ER4; ++u) {
          sq[u] = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) sq[u] += x[u][i] * x[u][i];
          sq[u] += dpp_f<0x128>(sq[u]);  // row_ror:8
          sq[u] += dpp_f<0x124>(sq[u]);  // row_ror:4
          sq[u] += dpp_f<0x122>(sq[u]);  // row_ror:2
          sq[u] += dpp_f<0x121>(sq[u]);  // row_ror:1
        }
#pragma unroll
        for (int u = 0; u < ER4; ++u) {
          const float sc = rsqrtf(sq[u] / KVS_HD + e.eps);
          float y[4], pr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = x[u][i] * sc * g[i];
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[i] = dpp_f<0x128>(y[i]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            x[u][i] = first_half ? y[i] * cs[u][i] - pr[i] * sn[u][i] : pr[i] * sn[u][i] + y[i] * cs[u][i];
        }
      }
#pragma unroll
      for (int u = 0; u < ER4; ++u) {
        if (rb + u > rb0 && ++rem == e.rp.M) {
          rem = 0;
          ++b;
        }
        if (r0 + (rb + u - rb0) < rows) {
          const int pos = pbase + rem * e.rp.step;
          stT<bf16, 4>(obase + ((((int64_t)j * e.B + b) * e.Hkv + hh) * e.T_max + pos) * KVS_HD + dd, x[u]);
        }
      }
    }
  };
  auto load_rv = [&](int c) { return e.rinvM[(int64_t)z * e.rows + min((cbeg + c) * KVS_CR + (lane & 31), rows - 1)]; };

  // the matrix loads were issued first, so once no more than this wave's
  // DMAs are outstanding the fragments are in registers
  if (dw) {
    issue_rows(0);
    if (n > 1) issue_rows(1);
    if (isK) issue_rope(0);
    if (n > 1) {
      if (isK) wait_vmcnt<18>();
      else wait_vmcnt<16>();
    } else {
      if (isK) wait_vmcnt<10>();
      else wait_vmcnt<8>();
    }
  } else {
    wait_vmcnt<0>();
  }

  // MFMAs of chunk c (stage c%4) for this wave's 32 columns, then, once every
  // wave has read the stage, the accumulators into the stage as the chunk's
  // C tile
  const int fr = lane & 31;  // fragment row within the chunk
  auto mfma_chunk = [&](int c) {
    const unsigned char *As = smem + (c % KVS_STG) * KVS_SB;
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < KVS_D / 16; ++s) {
      const u32x4 af = *(const u32x4 *)(As + fr * KVS_RB + (((2 * s + (lane >> 5)) ^ (fr & 15)) << 4));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af), __builtin_bit_cast(bf16x8, wf[s]),
                                                    acc, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    float *Cs = (float *)(smem + (c % KVS_STG) * KVS_SB);
#pragma unroll
    for (int q = 0; q < 16; ++q)
      Cs[(8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * KVS_N + 32 * wave + (lane & 31)] = acc[q];
  };
  // Each iteration starts with a barrier that publishes chunk c's rows and
  // chunk c-1's C tile and RoPE entries (the DMA waves first wait for their
  // own DMAs of them), and frees row stage (c+2)%4 and RoPE stage (c+1)%3,
  // whose contents were consumed before it.  The two roles run separate
  // loops with the same barriers, so each loop's memory counters only see its
  // own kind of access.
  if (dw) {
    for (int c = 0; c < n; ++c) {
      wait_batch(c + 1 < n);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_s_barrier();
      if (c + 2 < n) issue_rows(c + 2);
      if (isK && c + 1 < n) issue_rope(c + 1);
      mfma_chunk(c);
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
  } else {
    float rv = 0.f;
    for (int c = 0; c < n; ++c) {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_s_barrier();
      if (c > 0) epi(c - 1, rv);
      rv = load_rv(c);
      mfma_chunk(c);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    epi(n - 1, rv);
  }
}

// Blocks per channel: enough for about one block per compute unit.
inline int kvs_blocks_per_channel(int nz) { return nz >= kComputeUnits ? 1 : (kComputeUnits + nz - 1) / nz; }

}  // namespace wm
