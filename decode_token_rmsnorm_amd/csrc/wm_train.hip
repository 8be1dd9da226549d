// wm_train.hip — one training step with truncated backpropagation, float32.
//
// The step (onedev.kr "What differs": in training, gradients flow only
// through the last n_g passes; "How used": one cyclic pass without gradients,
// then two with; paperlayer.ai §3 "Execution schedules": training solves the
// feedback as a fixed point by passes): from the zero cache, n_nograd cyclic
// passes without gradient, then n_grad passes with it; the loss is the mean
// next-token cross-entropy of the last pass's logits (position i < T-1 of
// sequence b predicts token i+1); the gradient of every parameter is taken
// with the cache left by the no-gradient passes held constant.
//
// Plan.  The cache lives in the workspace in float32 [k, B, Hkv, T, d].  The
// forward runs every group step of every pass in order; before a gradient
// pass's group step overwrites its entries, the old values go to an undo
// log (one slot per gradient step).  The backward walks the gradient steps in
// reverse.  For each it takes the gradient of the entries the step wrote from
// dCache (an array shaped like the cache that collects, for every entry, the
// gradient of the value it holds at that point of the walk), clears it there,
// puts the old values back (so the cache is as the step found it), takes
// the step's forward intermediates (kept from the forward pass in a slot of
// the workspace when it holds one per gradient step, else recomputed from
// the restored cache; both give the same bits), and runs the step's
// backward: the pool first (the written keys/values back to the layer inputs
// and the pool parameters), then the layers from the top, where the
// attention of layer l adds the gradient of every cache entry it read into
// dCache.  A step reads the entries of earlier groups of its own pass and of
// later groups of the previous pass; both writers come later in the reverse
// walk, so each finds its gradient complete.  What the first gradient pass
// reads from the no-gradient cache is left in dCache and dropped.
//
// Every kernel here computes in float32, written for correctness at training
// shapes first: a tiled GEMM with optional transposes on float32 MFMAs, row
// RMSNorm forward/backward and gain gradients (chunked, summed in order),
// RoPE and its inverse, strict-causal attention forward (with its softmax
// statistics) and backward (queries per row; keys and values per key, so no
// atomics), SwiGLU, the pool's mix and its two backward products, the
// embedding gather and its backward (rows that share a token summed along
// a chain in row order), cross-entropy.  All reductions run in a fixed
// order, so a step is deterministic.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "../../include/wm.h"
#include "wm_common.hpp"
#include "wm_host.hpp"

namespace wm {
namespace tr {

#define TR_TRY(expr)                                                               \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess) {                                                        \
      set_error("%s failed: %s", #expr, hipGetErrorString(e_));                    \
      return WM_ERR_HIP;                                                           \
    }                                                                              \
  } while (0)

#define TR_CHECK(cond, code, ...) \
  do {                            \
    if (!(cond)) {                \
      set_error(__VA_ARGS__);     \
      return code;                \
    }                             \
  } while (0)

// Rows of a group step: row n = b*M + m is position s0 + m*step of sequence b.
struct Rows {
  int M, s0, step;
  __host__ __device__ int pos(int n) const { return s0 + (n % M) * step; }
  __host__ __device__ int seq(int n) const { return n / M; }
};

__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// ------------------------------------------------------------------ elementwise
__global__ void k_fill(float *p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}
__global__ void k_copy(float *dst, const float *src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}
__global__ void k_add(float *y, const float *x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    y[i] += x[i];
}

// act = silu(G) * U
__global__ void k_swiglu(const float *G, const float *U, float *act, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float g = G[i], sg = 1.f / (1.f + expf(-g));
    act[i] = g * sg * U[i];
  }
}
// dG = dact * U * silu'(G), dU = dact * silu(G); silu'(x) = s (1 + x (1 - s)).
__global__ void k_swiglu_bwd(const float *G, const float *U, const float *dact, float *dG, float *dU, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float g = G[i], sg = 1.f / (1.f + expf(-g)), da = dact[i];
    dG[i] = da * U[i] * sg * (1.f + g * (1.f - sg));
    dU[i] = da * g * sg;
  }
}

// ------------------------------------------------------------------ GEMM
// C[z] = alpha * op(A[z]) op(B[z]) + beta * C[z], op(A) [M, K], op(B) [K, N],
// row-major.  TA: A is stored [K, M] (leading dim lda), else [M, K].  TB: B
// is stored [N, K], else [K, N].  beta = 0 never reads C.  64 x 64 tiles,
// k in steps of 32 through two LDS buffers: the next step's operands are
// loaded into registers while the current buffer feeds the MFMAs, then
// stored into the other buffer (one barrier per step).  An operand stored
// with k contiguous keeps that layout in LDS ([row][k], pitch 36); one
// stored with k as the outer index keeps [k][row] (pitch 80); both pitches
// put a read's 64 lanes on distinct banks.  4 waves of 32 x 32, each on
// 2 x 2 float32 16x16x4 MFMAs (lane: A row lane % 16 and B column lane % 16
// at k lane / 16; in a 16-k chunk c, step e takes k = 16c + 4 (lane / 16)
// + e, so that a [row][k] operand gives a lane its four steps in one
// 16-byte read).  With splits > 1, blockIdx.z = batch * splits + split: the
// block sums k in [split * kchunk, (split + 1) * kchunk) and C[blockIdx.z]
// is a partial (k_split_sum adds them).
constexpr int GT = 64, GK = 32;

// 4 consecutive floats p[0..3], index idx of p[0] along a dimension of
// extent lim: past-the-end elements read as 0; one 16-byte load when vec
// (the caller's strides and base allow it) and all four are in range.
__device__ __forceinline__ f32x4 ld4(const float *p, int idx, int lim, bool vec) {
  if (vec && idx + 3 < lim) return *(const f32x4 *)p;
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = idx + e < lim ? p[e] : 0.f;
  return r;
}

// One operand's k-step: 2 runs of 4 floats per thread, in registers, and
// their place in LDS.  KO: k is the outer index in memory ([K, rows]).
template <bool KO>
struct GOp {
  static constexpr int P = KO ? GT + 16 : GK + 4, SZ = KO ? GK * P : GT * P;
  static constexpr int NV = GT * GK / 4 / 256;  // 16-byte runs per thread
  // thread -> run v: k-row (tid / 16) + 16 v, rows 4 (tid % 16) .. + 3 when
  // k is the outer index; else row (tid / (GK / 4)) + (1024 / GK) v, k
  // 4 (tid % (GK / 4)) .. + 3
  static constexpr int KQ = GK / 4, RS = 256 / KQ;
  f32x4 r[NV];
  __device__ __forceinline__ void load(const float *X, int64_t ld, int r0, int R, int k0, int ke, bool vec, int tid) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if (KO) {
        const int kk = (tid >> 4) + 16 * v, rr = 4 * (tid & 15);
        r[v] = k0 + kk < ke ? ld4(X + (int64_t)(k0 + kk) * ld + r0 + rr, r0 + rr, R, vec) : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        const int rr = tid / KQ + RS * v, kk = 4 * (tid % KQ);
        r[v] = r0 + rr < R ? ld4(X + (int64_t)(r0 + rr) * ld + k0 + kk, k0 + kk, ke, vec) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  __device__ __forceinline__ void store(float *S, int tid) const {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if (KO)
        *(f32x4 *)&S[((tid >> 4) + 16 * v) * P + 4 * (tid & 15)] = r[v];
      else
        *(f32x4 *)&S[(tid / KQ + RS * v) * P + 4 * (tid % KQ)] = r[v];
    }
  }
  // operand values of row `row` (of the tile) for the 4 steps of chunk c
  __device__ __forceinline__ static f32x4 frag(const float *S, int row, int c, int lj) {
    if (KO) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = S[(16 * c + 4 * lj + e) * P + row];
      return x;
    }
    return *(const f32x4 *)&S[row * P + 16 * c + 4 * lj];
  }
};

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void k_gemm(const float *A, int64_t lda, int64_t sA, const float *B, int64_t ldb,
                                              int64_t sB, float *C, int64_t ldc, int64_t sC, const float *Cr, int M,
                                              int N, int K, float alpha, float beta, int splits, int kchunk, int vecA,
                                              int vecB) {
  typedef GOp<TA> OA;
  typedef GOp<!TB> OB;
  __shared__ __attribute__((aligned(16))) float As[2][OA::SZ];
  __shared__ __attribute__((aligned(16))) float Bs[2][OB::SZ];
  const int batch = blockIdx.z / splits, split = blockIdx.z - batch * splits;
  A += batch * sA;
  B += batch * sB;
  C += blockIdx.z * sC;
  Cr += blockIdx.z * sC;  // (read only when splits == 1: then blockIdx.z is the batch)
  const int kb = split * kchunk, ke = min(K, kb + kchunk);
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lj = lane >> 4, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  OA oa;
  OB ob;
  oa.load(A, lda, m0, M, kb, ke, vecA, tid);
  ob.load(B, ldb, n0, N, kb, ke, vecB, tid);
  oa.store(As[0], tid);
  ob.store(Bs[0], tid);
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += GK, buf ^= 1) {
    const bool more = k0 + GK < ke;
    if (more) {
      oa.load(A, lda, m0, M, k0 + GK, ke, vecA, tid);
      ob.load(B, ldb, n0, N, k0 + GK, ke, vecB, tid);
    }
#pragma unroll
    for (int c = 0; c < GK / 16; ++c) {
      f32x4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = OA::frag(As[buf], wm * 32 + i * 16 + li, c, lj);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = OB::frag(Bs[buf], wn * 32 + j * 16 + li, c, lj);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
    }
    if (more) {
      oa.store(As[buf ^ 1], tid);
      ob.store(Bs[buf ^ 1], tid);
    }
    __syncthreads();
  }
  // accumulator (lane, e): row 4 * (lane / 16) + e, column lane % 16 of its tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + wn * 32 + j * 16 + li;
      if (gn >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gm = m0 + wm * 32 + i * 16 + 4 * lj + e;
        if (gm >= M) continue;
        const int64_t off = (int64_t)gm * ldc + gn;
        const float v = acc[i][j][e];
        C[off] = beta == 0.f ? alpha * v : alpha * v + beta * Cr[off];
      }
    }
}

// C[z] = beta * Cr[z] + sum over the splits (in order) of part[z * splits + s], [M, N]
__global__ void k_split_sum(const float *part, int splits, float *C, const float *Cr, int64_t ldc, int64_t sC, int M,
                            int N, int Z, float beta) {
  const int64_t MN = (int64_t)M * N, total = MN * Z;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t z = i / MN, e = i - z * MN;
    const int m = (int)(e / N), n = (int)(e - (int64_t)m * N);
    float t = 0.f;
    for (int sp = 0; sp < splits; ++sp) t += part[(z * splits + sp) * MN + e];
    const int64_t off = z * sC + (int64_t)m * ldc + n;
    C[off] = beta == 0.f ? t : t + beta * Cr[off];
  }
}

// ------------------------------------------------------------------ RMSNorm
// y = x * r * gain[r / rpg], r = 1 / sqrt(mean(x^2) + eps) per row of D.
__global__ __launch_bounds__(64) void k_rms(const float *x, const float *gain, int rpg, float *y, float *rinv, int D,
                                            float eps) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const float *xr = x + (int64_t)r * D;
  float ss = 0.f;
  for (int c = lane; c < D; c += 64) ss += xr[c] * xr[c];
  const float rs = 1.f / sqrtf(wave_sum(ss) / D + eps);
  const float *g = gain + (int64_t)(r / rpg) * D;
  for (int c = lane; c < D; c += 64) y[(int64_t)r * D + c] = xr[c] * rs * g[c];
  if (lane == 0) rinv[r] = rs;
}
// k_rms of x = sum over the splits (in order) of part[s] (+ beta * Cin),
// the rows of a split-k product whose sum was left to this kernel; x is
// stored too (exactly what k_split_sum would have written).  part[s] holds
// the rows at s * ps.
__global__ __launch_bounds__(64) void k_rms_parts(const float *part, int splits, int64_t ps, const float *Cin,
                                                  float beta, float *x, const float *gain, int rpg, float *y,
                                                  float *rinv, int D, float eps) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int64_t ro = (int64_t)r * D;
  float ss = 0.f;
  for (int c = lane; c < D; c += 64) {
    float t = 0.f;
    for (int sp = 0; sp < splits; ++sp) t += part[sp * ps + ro + c];
    if (beta != 0.f) t = t + beta * Cin[ro + c];
    x[ro + c] = t;
    ss += t * t;
  }
  const float rs = 1.f / sqrtf(wave_sum(ss) / D + eps);
  const float *g = gain + (int64_t)(r / rpg) * D;
  for (int c = lane; c < D; c += 64) y[ro + c] = x[ro + c] * rs * g[c];  // (this lane's own stores)
  if (lane == 0) rinv[r] = rs;
}
// dx (+)= r * (g dy) - x r^3 sum(g dy x) / D
__global__ __launch_bounds__(64) void k_rms_bwd(const float *x, const float *gain, int rpg, const float *rinv,
                                                const float *dy, float *dx, int accumulate, int D) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const float *xr = x + (int64_t)r * D, *dyr = dy + (int64_t)r * D, *g = gain + (int64_t)(r / rpg) * D;
  float dot = 0.f;
  for (int c = lane; c < D; c += 64) dot += g[c] * dyr[c] * xr[c];
  dot = wave_sum(dot);
  const float rs = rinv[r], k3 = rs * rs * rs * dot / D;
  for (int c = lane; c < D; c += 64) {
    const float v = rs * g[c] * dyr[c] - xr[c] * k3;
    float *o = dx + (int64_t)r * D + c;
    *o = accumulate ? *o + v : v;
  }
}
// dgain[gi, c] += sum over the rows r of group gi of dy[r, c] x[r, c] rinv[r],
// in two passes: k_gain_part sums chunks of GCH rows (block: 64 columns x 16
// row slices, slice j taking rows j, j + 16, ... of the chunk, the slices
// added in order) into part[gi, chunk, c]; k_gain_sum adds the chunks in
// order.
constexpr int GCH = 256;
__global__ __launch_bounds__(1024) void k_gain_part(const float *x, const float *dy, const float *rinv, float *part,
                                                    int rpg, int D) {
  __shared__ float sl[16][64];
  const int cl = threadIdx.x & 63, j = threadIdx.x >> 6, c = blockIdx.x * 64 + cl, gi = blockIdx.y, ch = blockIdx.z;
  const int nch = gridDim.z;
  float s = 0.f;
  if (c < D) {
    const int64_t r0 = (int64_t)gi * rpg + (int64_t)ch * GCH, r1 = (int64_t)gi * rpg + min(rpg, (ch + 1) * GCH);
    for (int64_t r = r0 + j; r < r1; r += 16) s += dy[r * D + c] * x[r * D + c] * rinv[r];
  }
  sl[j][cl] = s;
  __syncthreads();
  if (j == 0 && c < D) {
    float t = 0.f;
    for (int i = 0; i < 16; ++i) t += sl[i][cl];
    part[((int64_t)gi * nch + ch) * D + c] = t;
  }
}
__global__ void k_gain_sum(const float *part, float *dg, int nch, int D, int ngain) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= ngain * D) return;
  const int gi = i / D, c = i - gi * D;
  float t = 0.f;
  for (int ch = 0; ch < nch; ++ch) t += part[((int64_t)gi * nch + ch) * D + c];
  dg[i] += t;
}

// ------------------------------------------------------------------ RoPE
// x [rows, H, d], row r at position pos(r % N); element m turns with m + d/2
// by the angle of the table; inverse = the opposite turn (its own transpose).
__global__ void k_rope(float *x, Rows rm, int N, int H, int d, const float *cosT, const float *sinT, int inverse,
                       int64_t total) {
  const int half = d / 2;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(i % half);
    const int64_t rh = i / half;  // (row, head)
    const int r = (int)(rh / H);
    const int p = rm.pos(r % N);
    const float c = cosT[(int64_t)p * half + m], s = inverse ? -sinT[(int64_t)p * half + m] : sinT[(int64_t)p * half + m];
    float *v = x + rh * d;
    const float x1 = v[m], x2 = v[m + half];
    v[m] = x1 * c - x2 * s;
    v[m + half] = x1 * s + x2 * c;
  }
}

// ------------------------------------------------------------------ embedding
__global__ void k_embed(const int32_t *tokens, int T, Rows rm, const float *E, float *h, int N, int D, int V) {
  const int n = blockIdx.x;
  const int tok = tokens[(int64_t)rm.seq(n) * T + rm.pos(n)];
  const bool ok = tok >= 0 && tok < V;
  for (int c = threadIdx.x; c < D; c += blockDim.x) h[(int64_t)n * D + c] = ok ? E[(int64_t)tok * D + c] : NAN;
}
// Rows sharing a token, as chains in row order: nxt[n] = the next row with
// the same token (-1 at the end), head[n] = 1 for the first row of a token.
__global__ __launch_bounds__(64) void k_embed_chains(const int32_t *tokens, int T, Rows rm, int N, int *nxt,
                                                     int *head) {
  // the step's tokens pass through LDS in chunks; every lane of a wave reads
  // the same entry (a broadcast) while comparing it with its own row's token
  constexpr int CH = 2048;
  __shared__ int tl[CH];
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int tok = n < N ? tokens[(int64_t)rm.seq(n) * T + rm.pos(n)] : 0;
  int first = 1, next = -1;
  for (int m0 = 0; m0 < N; m0 += CH) {
    const int cnt = min(CH, N - m0);
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) tl[i] = tokens[(int64_t)rm.seq(m0 + i) * T + rm.pos(m0 + i)];
    __syncthreads();
    for (int i = 0; i < cnt; ++i) {
      const int m = m0 + i;
      if (tl[i] != tok) continue;
      if (m < n) first = 0;
      if (m > n && next < 0) next = m;
    }
  }
  if (n < N) {
    nxt[n] = next;
    head[n] = first;
  }
}
// dE[token] += sum of dh over the token's chain, in row order (one block per
// chain head; ids outside [0, V) are skipped: their rows are NaN already)
__global__ void k_embed_bwd(const int32_t *tokens, int T, Rows rm, const float *dh, const int *nxt, const int *head,
                            float *dE, int D, int V) {
  const int n = blockIdx.x;
  if (!head[n]) return;
  const int tok = tokens[(int64_t)rm.seq(n) * T + rm.pos(n)];
  if (tok < 0 || tok >= V) return;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float s = 0.f;
    for (int m = n; m >= 0; m = nxt[m]) s += dh[(int64_t)m * D + c];
    dE[(int64_t)tok * D + c] += s;
  }
}

// ------------------------------------------------------------------ attention
// Strict causal attention of row n (position i), head h to keys s < i of the
// channel (K, V: [B, Hkv, Tc, d]), on float32 16x16x4 MFMAs in tiles of 16
// keys x 16 query slots.  A query slot (m, g) of sequence b and KV head hk is
// row b*M + m at head hk*G + g (slot = m*G + g); the slots of a tile share
// the tile's keys, so GQA heads reuse every K/V load.
//
// MFMA operand lanes (l = lane, li = l % 16, lj = l / 16): A row li and B
// column li, both at k = lj; accumulator element e: row 4*lj + e, column
// li.  Products over the head dim take dims 16t + 4*lj + e at step (t, e),
// so that a lane's four steps read one 16-byte run of a K, V, q or dout
// row; products over keys (or slots) take key (slot) 4*lj + e at step e,
// the row of the accumulator element e that feeds them, so scores and
// probabilities go from accumulators to operands without moving.
//
// Forward and query side: a block of 8 waves takes 16 slots; wave w takes
// the 16-key tiles w, w + 8, ... below the block's last position, loading
// its K and V rows from memory into registers one tile ahead of use, and
// keeps its own running max, sum and output; the block then merges the 8
// waves' partial results in wave order.  Scores are kept transposed (keys
// x slots: S^T = K q^T), so that each lane holds one slot, its statistics
// included.
constexpr int ATQ = 16;  // query slots per block (forward and query side)
constexpr int NWF = 8;   // waves per block (forward and query side)

struct Slot {
  bool act;
  int ipos;
  int64_t so;  // (row, head) index
};
__device__ __forceinline__ Slot slot_of(int slot, int nslot, Rows rm, int b, int hk, int G, int Hq) {
  Slot r;
  r.act = slot < nslot;
  const int m = r.act ? slot / G : 0, n = b * rm.M + m, h = hk * G + (r.act ? slot - m * G : 0);
  r.ipos = r.act ? rm.pos(n) : 0;
  r.so = (int64_t)n * Hq + h;
  return r;
}
__device__ __forceinline__ f32x4 mf4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Scores and probabilities of out = softmax(scale q K^T over s < i) V.  Keeps
// the scaled-score max m and the sum l of exp(score - m) for the backward
// (a slot with no key: m = -inf, l = 0, output 0).  Blocks run longest
// (last slots) first.
template <int DH>
__global__ __launch_bounds__(64 * NWF) void k_attn(const float *q, const float *Kc, const float *Vc, Rows rm, int Hq,
                                              int Hkv, int Tc, float scale, float *out, float *mst, float *lst) {
  constexpr int NT = DH / 16;
  __shared__ float cm[NWF][ATQ], cl[NWF][ATQ], co[NWF][DH][ATQ + 1];
  const int pair = blockIdx.x, b = pair / Hkv, hk = pair - b * Hkv, G = Hq / Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lj = lane >> 4;
  const int nslot = rm.M * G, sb = (gridDim.y - 1 - blockIdx.y) * ATQ;
  const int imax = rm.pos(b * rm.M + min(sb + ATQ - 1, nslot - 1) / G);
  const Slot me = slot_of(sb + li, nslot, rm, b, hk, G, Hq);
  const float *K = Kc + ((int64_t)b * Hkv + hk) * Tc * DH, *V = Vc + ((int64_t)b * Hkv + hk) * Tc * DH;
  f32x4 qf[NT], o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    qf[t] = me.act ? *(const f32x4 *)&q[me.so * DH + 16 * t + 4 * lj] : f32x4{0.f, 0.f, 0.f, 0.f};
    o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float mx = -INFINITY, ls = 0.f;
  f32x4 kn[NT];
  float vn[NT][4];
  auto fetch = [&](int k0) {
    const int kr = min(k0 + li, Tc - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) kn[t] = *(const f32x4 *)&K[(int64_t)kr * DH + 16 * t + 4 * lj];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int vr = min(k0 + 4 * lj + e, Tc - 1);
#pragma unroll
      for (int i = 0; i < NT; ++i) vn[i][e] = V[(int64_t)vr * DH + 16 * i + li];
    }
  };
  if (16 * wave < imax) fetch(16 * wave);
  for (int k0 = 16 * wave; k0 < imax; k0 += 16 * NWF) {
    f32x4 kf[NT];
    float vf[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) kf[t] = kn[t];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) vf[i][e] = vn[i][e];
    if (k0 + 16 * NWF < imax) fetch(k0 + 16 * NWF);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mf4(kf[t][e], qf[t][e], s);
    float sc[4], ml = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[e] = k0 + 4 * lj + e < me.ipos ? s[e] * scale : -INFINITY;
      ml = fmaxf(ml, sc[e]);
    }
    ml = fmaxf(ml, __shfl_xor(ml, 16));
    ml = fmaxf(ml, __shfl_xor(ml, 32));
    const float mn = fmaxf(mx, ml), al = mn == -INFINITY ? 1.f : expf(mx - mn);
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = sc[e] == -INFINITY ? 0.f : expf(sc[e] - mn);
    ls = ls * al + ((p[0] + p[1]) + (p[2] + p[3]));
    mx = mn;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      o[i] *= al;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[i] = mf4(vf[i][e], p[e], o[i]);  // O^T += V^T P^T
    }
  }
  ls += __shfl_xor(ls, 16);
  ls += __shfl_xor(ls, 32);
  if (lj == 0) {
    cm[wave][li] = mx;
    cl[wave][li] = ls;
  }
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) co[wave][16 * i + 4 * lj + e][li] = o[i][e];
  __syncthreads();
  for (int x = threadIdx.x; x < ATQ * DH; x += 64 * NWF) {
    const int sl = x / DH, d = x - sl * DH;
    const Slot r = slot_of(sb + sl, nslot, rm, b, hk, G, Hq);
    if (!r.act) continue;
    float M = -INFINITY, L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NWF; ++w) M = fmaxf(M, cm[w][sl]);
    if (M != -INFINITY)
#pragma unroll
      for (int w = 0; w < NWF; ++w) {
        const float f = cm[w][sl] == -INFINITY ? 0.f : expf(cm[w][sl] - M);
        L += f * cl[w][sl];
        O += f * co[w][d][sl];
      }
    out[r.so * DH + d] = L > 0.f ? O / L : 0.f;
    if (d == 0) {
      mst[r.so] = M;
      lst[r.so] = L;
    }
  }
}

// dq of row n, head h: dS_t = p_t (dP_t - Dn) with dP_t = dout . V_t and
// Dn = dout . out (out: the forward's attention output, which equals
// sum_t p_t V_t, so Dn = sum_t p_t dP_t); dq = scale * sum_t dS_t K_t.  Keeps
// Dn for the key-side kernel.  Blocks, waves and key tiles as in k_attn;
// each wave walks its tiles once (S^T and dP^T, then dq^T = K^T dS^T) and
// the waves' dq are added in wave order.
template <int DH>
__global__ __launch_bounds__(64 * NWF) void k_attn_dq(const float *q, const float *Kc, const float *Vc,
                                                      const float *dout, const float *outf, const float *mst,
                                                      const float *lst, Rows rm, int Hq, int Hkv, int Tc, float scale,
                                                      float *dq, float *Dst) {
  constexpr int NT = DH / 16;
  __shared__ float cg[NWF][DH][ATQ + 1];
  const int pair = blockIdx.x, b = pair / Hkv, hk = pair - b * Hkv, G = Hq / Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lj = lane >> 4;
  const int nslot = rm.M * G, sb = (gridDim.y - 1 - blockIdx.y) * ATQ;
  const int imax = rm.pos(b * rm.M + min(sb + ATQ - 1, nslot - 1) / G);
  const Slot me = slot_of(sb + li, nslot, rm, b, hk, G, Hq);
  const float *K = Kc + ((int64_t)b * Hkv + hk) * Tc * DH, *V = Vc + ((int64_t)b * Hkv + hk) * Tc * DH;
  f32x4 qf[NT], df[NT];
  float Dp = 0.f;  // (the lane's dims of dout . out; summed over the lane groups below)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    qf[t] = me.act ? *(const f32x4 *)&q[me.so * DH + 16 * t + 4 * lj] : z;
    df[t] = me.act ? *(const f32x4 *)&dout[me.so * DH + 16 * t + 4 * lj] : z;
    const f32x4 of = me.act ? *(const f32x4 *)&outf[me.so * DH + 16 * t + 4 * lj] : z;
#pragma unroll
    for (int e = 0; e < 4; ++e) Dp = fmaf(df[t][e], of[e], Dp);
  }
  Dp += __shfl_xor(Dp, 16);
  const float Dn = Dp + __shfl_xor(Dp, 32);
  const float mrow = me.act ? mst[me.so] : 0.f, lr = me.act ? lst[me.so] : 0.f, invl = lr > 0.f ? 1.f / lr : 0.f;
  // a tile's K and V rows k0 + li as A operands (16-byte runs), loaded one
  // tile ahead
  f32x4 kn[NT], vn[NT];
  auto fetch = [&](int k0) {
    const int kr = min(k0 + li, Tc - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      kn[t] = *(const f32x4 *)&K[(int64_t)kr * DH + 16 * t + 4 * lj];
      vn[t] = *(const f32x4 *)&V[(int64_t)kr * DH + 16 * t + 4 * lj];
    }
  };
  f32x4 g[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) g[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (16 * wave < imax) fetch(16 * wave);
  for (int k0 = 16 * wave; k0 < imax; k0 += 16 * NWF) {
    // K rows k0 + 4 lj + e as the A operand of dq^T (used after the S and dP products)
    float kt[NT][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = min(k0 + 4 * lj + e, Tc - 1);
#pragma unroll
      for (int i = 0; i < NT; ++i) kt[i][e] = K[(int64_t)r * DH + 16 * i + li];
    }
    f32x4 kf[NT], vf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      kf[t] = kn[t];
      vf[t] = vn[t];
    }
    if (k0 + 16 * NWF < imax) fetch(k0 + 16 * NWF);
    f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc = mf4(kf[t][e], qf[t][e], sc);  // S^T = K q^T
        dP = mf4(vf[t][e], df[t][e], dP);  // dP^T = V dout^T
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = k0 + 4 * lj + e < me.ipos ? expf(sc[e] * scale - mrow) * invl : 0.f;
      const float dS = p * (dP[e] - Dn);
#pragma unroll
      for (int i = 0; i < NT; ++i) g[i] = mf4(kt[i][e], dS, g[i]);  // dq^T += K^T dS^T
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) cg[wave][16 * i + 4 * lj + e][li] = g[i][e];
  __syncthreads();
  for (int x = threadIdx.x; x < ATQ * DH; x += 64 * NWF) {
    const int sl = x / DH, d = x - sl * DH;
    const Slot r = slot_of(sb + sl, nslot, rm, b, hk, G, Hq);
    if (!r.act) continue;
    float gs = 0.f;
#pragma unroll
    for (int w = 0; w < NWF; ++w) gs += cg[w][d][sl];
    dq[r.so * DH + d] = gs * scale;
  }
  if (wave == 0 && lj == 0 && me.act) Dst[me.so] = Dn;
}

// dK_t += scale * sum dS q, dV_t += sum p dout over the rows n of sequence b
// with position > t and the heads of KV head hk.  A block of 4 waves takes
// 64 keys of (b, hk), 16 per wave, with the wave's K and V rows in registers;
// it walks the query slots from the first row past its first key in tiles
// of 16, staged in LDS (q, dout and each slot's m, 1/l, Dn and position;
// two buffers, the next tile loaded into registers while the current one is
// used, one barrier per tile).  Per tile a wave forms S = q K^T and
// dP = dout V^T (slots x keys, so the slot is the k index of the products
// that follow), p and dS, then dV^T += dout^T P and dK^T += q^T dS.
template <int DH>
__global__ __launch_bounds__(256) void k_attn_dkv(const float *q, const float *Kc, const float *Vc, const float *dout,
                                                  const float *mst, const float *lst, const float *Dst, Rows rm,
                                                  int Hq, int Hkv, int Tc, float scale, float *dK, float *dV) {
  constexpr int NT = DH / 16, QP = DH + 4, NV = (ATQ * DH / 4 + 255) / 256;
  __shared__ __attribute__((aligned(16))) float qs[2][ATQ][QP], ds[2][ATQ][QP];
  __shared__ __attribute__((aligned(16))) float sst[2][4][ATQ];  // m, 1/l, Dn, position
  const int pair = blockIdx.x, b = pair / Hkv, hk = pair - b * Hkv, G = Hq / Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lj = lane >> 4;
  const int t0 = blockIdx.y * 64, kb = t0 + 16 * wave, nslot = rm.M * G;
  const int64_t base = ((int64_t)b * Hkv + hk) * Tc * DH;
  // first row whose position is past the block's first key (positions grow with m)
  int m0 = 0;
  while (m0 < rm.M && rm.pos(b * rm.M + m0) <= t0) ++m0;
  if (m0 >= rm.M) return;  // (block-uniform)
  const int s0 = m0 * G, ntile = (nslot - s0 + ATQ - 1) / ATQ;
  f32x4 kf[NT], vf[NT], ak[NT], av[NT];
  {
    const int kr = min(kb + li, Tc - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      kf[t] = *(const f32x4 *)&Kc[base + (int64_t)kr * DH + 16 * t + 4 * lj];
      vf[t] = *(const f32x4 *)&Vc[base + (int64_t)kr * DH + 16 * t + 4 * lj];
      ak[t] = av[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // staging of tile i: thread x holds float4 runs x, x + 256, ... of q and
  // dout ([16 slots][DH / 4 runs]); threads 0..15 the statistics of slot x
  f32x4 rq[NV], rd[NV];
  float rst[4];
  auto fetch = [&](int i) {
    const int st = s0 + i * ATQ;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int x = threadIdx.x + 256 * v, sl = x / (DH / 4), c = 4 * (x - sl * (DH / 4));
      rq[v] = rd[v] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (sl < ATQ) {
        const Slot r = slot_of(st + sl, nslot, rm, b, hk, G, Hq);
        if (r.act) {
          rq[v] = *(const f32x4 *)&q[r.so * DH + c];
          rd[v] = *(const f32x4 *)&dout[r.so * DH + c];
        }
      }
    }
    if (threadIdx.x < ATQ) {
      const Slot r = slot_of(st + threadIdx.x, nslot, rm, b, hk, G, Hq);
      const float l = r.act ? lst[r.so] : 0.f;
      rst[0] = r.act ? mst[r.so] : 0.f;
      rst[1] = l > 0.f ? 1.f / l : 0.f;
      rst[2] = r.act ? Dst[r.so] : 0.f;
      rst[3] = (float)r.ipos;  // (exact: positions < 2^24)
    }
  };
  fetch(0);
  for (int i = 0; i < ntile; ++i) {
    const int buf = i & 1;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int x = threadIdx.x + 256 * v, sl = x / (DH / 4), c = 4 * (x - sl * (DH / 4));
      if (sl < ATQ) {
        *(f32x4 *)&qs[buf][sl][c] = rq[v];
        *(f32x4 *)&ds[buf][sl][c] = rd[v];
      }
    }
    if (threadIdx.x < ATQ)
#pragma unroll
      for (int j = 0; j < 4; ++j) sst[buf][j][threadIdx.x] = rst[j];
    __syncthreads();  // (tile i staged; every wave is past tile i - 1, so buffer !buf is free)
    if (i + 1 < ntile) fetch(i + 1);
    // the tile's last position (positions grow with the slot) past the wave's first key?
    const int st = s0 + i * ATQ;
    if (rm.pos(b * rm.M + min(st + ATQ - 1, nslot - 1) / G) <= kb) continue;
    f32x4 s = {0.f, 0.f, 0.f, 0.f}, dP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 qa = *(const f32x4 *)&qs[buf][li][16 * t + 4 * lj];
      const f32x4 da = *(const f32x4 *)&ds[buf][li][16 * t + 4 * lj];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = mf4(qa[e], kf[t][e], s);    // S = q K^T
        dP = mf4(da[e], vf[t][e], dP);  // dP = dout V^T
      }
    }
    const f32x4 sm = *(const f32x4 *)&sst[buf][0][4 * lj], sil = *(const f32x4 *)&sst[buf][1][4 * lj];
    const f32x4 sD = *(const f32x4 *)&sst[buf][2][4 * lj], sp = *(const f32x4 *)&sst[buf][3][4 * lj];
    float p[4], dS[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = (float)(kb + li) < sp[e] ? expf(s[e] * scale - sm[e]) * sil[e] : 0.f;
      dS[e] = p[e] * (dP[e] - sD[e]);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        av[j] = mf4(ds[buf][4 * lj + e][16 * j + li], p[e], av[j]);   // dV^T += dout^T P
        ak[j] = mf4(qs[buf][4 * lj + e][16 * j + li], dS[e], ak[j]);  // dK^T += q^T dS
      }
  }
  // accumulator element e of lane l: dim 16 j + 4 lj + e of key kb + li
  if (kb + li < Tc)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t a = base + (int64_t)(kb + li) * DH + 16 * j + 4 * lj;
      f32x4 xk = *(f32x4 *)&dK[a], xv = *(f32x4 *)&dV[a];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xk[e] += ak[j][e] * scale;
        xv[e] += av[j][e];
      }
      *(f32x4 *)&dK[a] = xk;
      *(f32x4 *)&dV[a] = xv;
    }
}

// ------------------------------------------------------------------ pool
// u[n, r*D + c] = nsrc[r*p, n, c]
__global__ void k_router_in(const float *nsrc, float *u, int p, int R, int N, int D) {
  const int64_t total = (int64_t)N * R * D;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % D);
    const int64_t nr = i / D;
    const int r = (int)(nr % R), n = (int)(nr / R);
    u[i] = nsrc[((int64_t)r * p * N + n) * D + c];
  }
}
// m[j, n, c] = sum_l A[n, l*k + j] * nsrc[l, n, c] (l ascending)
__global__ void k_mix(const float *A, const float *nsrc, float *m, int L, int k, int N, int D) {
  const int64_t total = (int64_t)k * N * D;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % D);
    const int64_t jn = i / D;
    const int n = (int)(jn % N), j = (int)(jn / N);
    float s = 0.f;
    for (int l = 0; l < L; ++l) s += A[((int64_t)n * L + l) * k + j] * nsrc[((int64_t)l * N + n) * D + c];
    m[i] = s;
  }
}
// dA[n, l*k + j] = dm[j, n, :] . nsrc[l, n, :]; one wave per (n, l, j)
__global__ __launch_bounds__(64) void k_mix_dA(const float *dm, const float *nsrc, float *dA, int L, int k, int N,
                                               int D) {
  const int n = blockIdx.x, lj = blockIdx.y, l = lj / k, j = lj - l * k, lane = threadIdx.x;
  const float *a = dm + ((int64_t)j * N + n) * D, *b = nsrc + ((int64_t)l * N + n) * D;
  float s = 0.f;
  for (int c = lane; c < D; c += 64) s += a[c] * b[c];
  s = wave_sum(s);
  if (lane == 0) dA[(int64_t)n * L * k + lj] = s;
}
// dn[l, n, c] = sum_j A[n, l*k + j] dm[j, n, c]
__global__ void k_mix_dn(const float *A, const float *dm, float *dn, int L, int k, int N, int D) {
  const int64_t total = (int64_t)L * N * D;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % D);
    const int64_t ln = i / D;
    const int n = (int)(ln % N), l = (int)(ln / N);
    float s = 0.f;
    for (int j = 0; j < k; ++j) s += A[((int64_t)n * L + l) * k + j] * dm[((int64_t)j * N + n) * D + c];
    dn[i] = s;
  }
}
// dn[r*p, n, c] += du[n, r*D + c]
__global__ void k_router_in_bwd(const float *du, float *dn, int p, int R, int N, int D) {
  const int64_t total = (int64_t)N * R * D;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % D);
    const int64_t nr = i / D;
    const int r = (int)(nr % R), n = (int)(nr / R);
    dn[((int64_t)r * p * N + n) * D + c] += du[i];
  }
}

// ------------------------------------------------------------------ cache entries
// Entries (j, b, h, pos(n), :) of the cache [k, B, Hkv, Tc, d] against a
// row-ordered array [k, N, Hkv, d].  mode 0: array = cache; 1: cache = array;
// 2: array = cache, then cache = 0.
__global__ void k_entries(float *cache, float *arr, Rows rm, int k, int B, int N, int Hkv, int Tc, int d, int mode) {
  const int64_t total = (int64_t)k * N * Hkv * d;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % d);
    int64_t r = i / d;
    const int h = (int)(r % Hkv);
    r /= Hkv;
    const int n = (int)(r % N), j = (int)(r / N);
    float *e = cache + ((((int64_t)j * B + rm.seq(n)) * Hkv + h) * Tc + rm.pos(n)) * d + c;
    if (mode == 1) {
      *e = arr[i];
    } else {
      arr[i] = *e;
      if (mode == 2) *e = 0.f;
    }
  }
}

// ------------------------------------------------------------------ loss
__device__ float block_reduce(float v, bool is_max, float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = is_max ? wmax(v) : wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < nw; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}
// Row n of the last pass: loss = logsumexp(z) - z[target] when position
// i < T-1 (target = token i+1), written to lossrow[b*T + i] (0 otherwise);
// dz = (softmax(z) - onehot(target)) * inv_count.
__global__ __launch_bounds__(256) void k_ce(const float *logits, const int32_t *tokens, int T, Rows rm, int V,
                                            float inv_count, float *lossrow, float *dlogits) {
  __shared__ float red[4];
  const int n = blockIdx.x, b = rm.seq(n), i = rm.pos(n);
  const bool has = i < T - 1;
  const int tgt = has ? tokens[(int64_t)b * T + i + 1] : -1;
  const float *z = logits + (int64_t)n * V;
  float mx = -INFINITY;
  for (int c = threadIdx.x; c < V; c += blockDim.x) mx = fmaxf(mx, z[c]);
  mx = block_reduce(mx, true, red);
  float se = 0.f;
  for (int c = threadIdx.x; c < V; c += blockDim.x) se += expf(z[c] - mx);
  se = block_reduce(se, false, red);
  const float inv = 1.f / se;
  for (int c = threadIdx.x; c < V; c += blockDim.x)
    dlogits[(int64_t)n * V + c] = has ? (expf(z[c] - mx) * inv - (c == tgt ? 1.f : 0.f)) * inv_count : 0.f;
  if (threadIdx.x == 0)
    lossrow[(int64_t)b * T + i] = has ? (tgt >= 0 && tgt < V ? logf(se) + mx - z[tgt] : NAN) : 0.f;
}
// *loss = sum(lossrow) * inv_count, in a fixed order (one block)
__global__ __launch_bounds__(256) void k_loss_sum(const float *lossrow, int64_t n, float inv_count, float *loss) {
  __shared__ float red[4];
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) s += lossrow[i];
  s = block_reduce(s, false, red);
  if (threadIdx.x == 0) *loss = s * inv_count;
}

// ------------------------------------------------------------------ host side
// b - a in floats, for batching products over buffers of different allocations
inline int64_t fdist(const float *a, const float *b) {
  return (int64_t)(((intptr_t)b - (intptr_t)a) / (intptr_t)sizeof(float));
}

inline unsigned grid1(int64_t n, int per = 256) {
  int64_t g = (n + per - 1) / per;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(g, 65536));
}

struct Layout {
  size_t total = 0;
  size_t take(size_t floats) {
    const size_t o = total;
    total += (floats * 4 + 255) & ~(size_t)255;
    return o;
  }
};

// Float offsets into the workspace (bytes / 4 after Layout).
struct Ws {
  size_t cK, cV, dK, dV, undo, undo_slot;
  // tape of one step
  size_t S, rA, a, qraw, rQ, q, o, mst, lst, h1, rF, bn, G, U, act, hL, rL, xf, logits;
  // pool (one branch at a time)
  size_t nsrc, rS, u, A, m, rM, c, kraw, rK, Kn, Vn;
  // backward
  size_t dh, dS, da, dq, dout, dG, dU, dact, db, Dst, dKn, dVn, dkraw, dc, dm, dA, dn, du, dz, dxf, lossrow;
  size_t enext, ehead;  // (int arrays)
  size_t split, split_cap;  // split-k partials (floats)
  size_t gpart;             // gain-gradient chunk sums
  // The step tape (S .. hL) is one slot of tape_stride floats at its fields'
  // offsets; with nslot > 1 the gradient steps keep their tapes in slots
  // 1 .. nslot - 1, from extra0 on, and the reverse walk does not recompute
  // their forward.
  size_t tape0, tape_stride, extra0;
  int nslot;
  size_t bytes;
  Ws slot(int i) const {
    Ws w = *this;
    const size_t sh = i == 0 ? 0 : extra0 + (size_t)(i - 1) * tape_stride - tape0;
    for (size_t *f : {&w.S, &w.rA, &w.a, &w.qraw, &w.rQ, &w.q, &w.o, &w.mst, &w.lst, &w.h1, &w.rF, &w.bn, &w.G,
                      &w.U, &w.act, &w.hL})
      *f += sh;
    return w;
  }
};

// Gradient-step tapes are kept when the whole workspace stays within this
// many bytes (a quarter of the device's HBM at the sizes benchmarked here);
// beyond it the reverse walk recomputes each step's forward instead.
constexpr size_t kTapeBudget = (size_t)64 << 30;

inline Ws layout(const wm_config &c, int B, int T, int g, int n_grad, bool tapes = true) {
  const size_t L = c.L, D = c.D, QD = (size_t)c.Hq * c.d, KD = (size_t)c.Hkv * c.d, F = c.F, k = c.k, V = c.V;
  const size_t R = (c.L + c.p - 1) / c.p, ng = std::min(g, T);
  const size_t N = (size_t)B * ((T + g - 1) / g), cache = k * B * KD * T;
  Layout l;
  Ws w{};
  auto t = [&](size_t n) { return l.take(n) / 4; };
  w.cK = t(cache);
  w.cV = t(cache);
  w.dK = t(cache);
  w.dV = t(cache);
  w.undo_slot = ((2 * k * N * KD * 4 + 255) & ~(size_t)255) / 4;
  w.undo = t(w.undo_slot * (size_t)n_grad * ng);
  w.tape0 = l.total / 4;
  w.S = t(L * N * D);
  w.rA = t(L * N);
  w.a = t(L * N * D);
  w.qraw = t(L * N * QD);
  w.rQ = t(L * N * c.Hq);
  w.q = t(L * N * QD);
  w.o = t(L * N * QD);
  w.mst = t(L * N * c.Hq);
  w.lst = t(L * N * c.Hq);
  w.h1 = t(L * N * D);
  w.rF = t(L * N);
  w.bn = t(L * N * D);
  w.G = t(L * N * F);
  w.U = t(L * N * F);
  w.act = t(L * N * F);
  w.hL = t(N * D);
  w.tape_stride = l.total / 4 - w.tape0;
  w.rL = t(N);
  w.xf = t(N * D);
  w.logits = t(N * V);
  w.nsrc = t(L * N * D);
  w.rS = t(L * N);
  w.u = t(N * R * D);
  w.A = t(N * L * k);
  w.m = t(k * N * D);
  w.rM = t(k * N);
  w.c = t(k * N * D);
  w.kraw = t(k * N * KD);
  w.rK = t(k * N * c.Hkv);
  w.Kn = t(k * N * KD);
  w.Vn = t(k * N * KD);
  w.dh = t(N * D);
  w.dS = t(L * N * D);
  w.da = t(N * D);
  w.dq = t(N * QD);
  w.dout = t(N * QD);
  w.dG = t(N * F);
  w.dU = t(N * F);
  w.dact = t(N * F);
  w.db = t(N * D);
  w.Dst = t(N * c.Hq);
  w.dKn = t(k * N * KD);
  w.dVn = t(k * N * KD);
  w.dkraw = t(k * N * KD);
  w.dc = t(k * N * D);
  w.dm = t(k * N * D);
  w.dA = t(N * L * k);
  w.dn = t(L * N * D);
  w.du = t(N * R * D);
  w.dz = t(N * V);
  w.dxf = t(N * D);
  w.lossrow = t((size_t)B * T);
  w.enext = t(N);
  w.ehead = t(N);
  // split-k partials: up to 8 of the largest product other than the LM head's
  const size_t wide = std::max({F, D, QD, R * D, L * k, KD});
  w.split_cap = 8 * std::max({N * wide, D * F, QD * D, L * k * R * D, k * KD * D, k * N * D});
  w.split = t(w.split_cap);
  // gain-gradient chunks: ngain * ceil(rows per gain / 256) * width, largest
  // for the source states [L*N, D], channels [k*N, D], key heads [k*N*Hkv, d]
  // and query heads [N*Hq, d]
  auto chunks = [](size_t rows, size_t ngain) { return rows / 256 + ngain; };
  w.gpart = t(std::max({chunks(L * N, L) * D, chunks(k * N, k) * D, chunks(k * N * c.Hkv, k) * c.d,
                        chunks(N * c.Hq, 1) * c.d, chunks(N, 1) * D}));
  const size_t extra = (size_t)n_grad * ng * w.tape_stride;
  w.nslot = 1;
  w.extra0 = 0;
  if (tapes && l.total + extra * 4 <= kTapeBudget) {
    w.extra0 = t(extra);
    w.nslot = 1 + n_grad * (int)ng;
  }
  w.bytes = l.total;
  return w;
}

// A split-k product whose partial sum was left to the consumer of its rows:
// C = sum over the splits of the partials (ps floats apart) + beta * Cin.
struct Pending {
  int splits = 1;  // (1: nothing pending)
  int64_t ps = 0;
  float *C = nullptr;
  const float *Cin = nullptr;
  float beta = 0.f;
};

struct Trainer {
  const wm_config &c;
  const wm_weights &w;
  const wm_grads &gr;
  const int32_t *tokens;
  int B, T, g;
  float *base;
  Ws o;
  hipStream_t s;
  int L, D, QD, KD, F, k, V, R;

  Trainer(const wm_config &c_, const wm_weights &w_, const wm_grads &g_, const int32_t *tok, int B_, int T_, int gg,
          int n_grad, bool tapes, void *ws, hipStream_t st)
      : c(c_), w(w_), gr(g_), tokens(tok), B(B_), T(T_), g(gg), base((float *)ws), s(st) {
    o = layout(c, B, T, g, n_grad, tapes);
    L = c.L;
    D = c.D;
    QD = c.Hq * c.d;
    KD = c.Hkv * c.d;
    F = c.F;
    k = c.k;
    V = c.V;
    R = (L + c.p - 1) / c.p;
  }
  float *P(size_t off) const { return base + off; }
  static const float *W(const void *p) { return (const float *)p; }

  hipError_t fill(float *p, int64_t n, float v) {
    hipLaunchKernelGGL(k_fill, dim3(grid1(n)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
  }
  hipError_t copy(float *d, const float *x, int64_t n) {
    hipLaunchKernelGGL(k_copy, dim3(grid1(n)), dim3(256), 0, s, d, x, n);
    return hipGetLastError();
  }
  hipError_t add(float *y, const float *x, int64_t n) {
    hipLaunchKernelGGL(k_add, dim3(grid1(n)), dim3(256), 0, s, y, x, n);
    return hipGetLastError();
  }
  // C = op(A) op(B) + beta Cin (Cin = C unless given; laid out as C), batched
  // over Z with element strides.  Grids of fewer tiles than compute units
  // split k (chunks of at least 128, up to 8 splits) into partials in the
  // workspace, summed in split order.
  hipError_t gemm(bool ta, bool tb, const float *A, int64_t lda, const float *B_, int64_t ldb, float *C, int64_t ldc,
                  int M, int N, int K, float beta, int Z = 1, int64_t sA = 0, int64_t sB = 0, int64_t sC = 0,
                  const float *Cin = nullptr, Pending *defer = nullptr) {
    if (defer) *defer = Pending{};
    if (M <= 0 || N <= 0) return hipSuccess;
    const int64_t tiles = (int64_t)((N + GT - 1) / GT) * ((M + GT - 1) / GT) * Z;
    int splits = 1;
    if (tiles < 256) {
      splits = (int)std::min<int64_t>(8, std::min<int64_t>((256 + tiles - 1) / tiles, K / 128));
      if (splits < 2 || (size_t)splits * Z * M * N > o.split_cap) splits = 1;
    }
    const int kchunk = splits > 1 ? ((K + splits - 1) / splits + GK - 1) / GK * GK : K;
    if (splits > 1) splits = (K + kchunk - 1) / kchunk;
    float *Cd = splits > 1 ? P(o.split) : C;
    const float *Cr = Cin ? Cin : C;  // (the beta term's source, laid out as C)
    const int64_t ldd = splits > 1 ? N : ldc, sD = splits > 1 ? (int64_t)M * N : sC;
    const float bd = splits > 1 ? 0.f : beta;
    dim3 grid((N + GT - 1) / GT, (M + GT - 1) / GT, Z * splits);
    // 16-byte loads where every row and batch starts on a 16-byte boundary
    const int va = ((uintptr_t)A % 16 == 0 && lda % 4 == 0 && sA % 4 == 0) ? 1 : 0;
    const int vb = ((uintptr_t)B_ % 16 == 0 && ldb % 4 == 0 && sB % 4 == 0) ? 1 : 0;
    if (!ta && !tb)
      hipLaunchKernelGGL((k_gemm<false, false>), grid, dim3(256), 0, s, A, lda, sA, B_, ldb, sB, Cd, ldd, sD, Cr, M, N,
                         K, 1.f, bd, splits, kchunk, va, vb);
    else if (!ta && tb)
      hipLaunchKernelGGL((k_gemm<false, true>), grid, dim3(256), 0, s, A, lda, sA, B_, ldb, sB, Cd, ldd, sD, Cr, M, N, K,
                         1.f, bd, splits, kchunk, va, vb);
    else if (ta && !tb)
      hipLaunchKernelGGL((k_gemm<true, false>), grid, dim3(256), 0, s, A, lda, sA, B_, ldb, sB, Cd, ldd, sD, Cr, M, N, K,
                         1.f, bd, splits, kchunk, va, vb);
    else
      hipLaunchKernelGGL((k_gemm<true, true>), grid, dim3(256), 0, s, A, lda, sA, B_, ldb, sB, Cd, ldd, sD, Cr, M, N, K,
                         1.f, bd, splits, kchunk, va, vb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    if (defer && Z == 1 && ldc == N) {  // (the sum is left to the rows' consumer: rms_in)
      *defer = Pending{splits, (int64_t)M * N, C, Cr, beta};
      return hipSuccess;
    }
    const int64_t total = (int64_t)M * N * Z;
    hipLaunchKernelGGL(k_split_sum, dim3(grid1(total)), dim3(256), 0, s, P(o.split), splits, C, Cr, ldc, sC, M, N, Z, beta);
    return hipGetLastError();
  }
  hipError_t rms(const float *x, const float *gain, int rpg, float *y, float *rinv, int rows, int width) {
    hipLaunchKernelGGL(k_rms, dim3(rows), dim3(64), 0, s, x, gain, rpg, y, rinv, width, c.eps);
    return hipGetLastError();
  }
  // rms of x, or, when x's split-k sum was left pending, of that sum (which
  // is also written to x: pd.C == x)
  hipError_t rms_in(const Pending &pd, const float *x, const float *gain, int rpg, float *y, float *rinv, int rows,
                    int width) {
    if (pd.splits <= 1) return rms(x, gain, rpg, y, rinv, rows, width);
    hipLaunchKernelGGL(k_rms_parts, dim3(rows), dim3(64), 0, s, P(o.split), pd.splits, pd.ps, pd.Cin, pd.beta, pd.C,
                       gain, rpg, y, rinv, width, c.eps);
    return hipGetLastError();
  }
  // dx (+)= RMSNorm backward; dgain (ngain rows of width) += its gain gradient
  hipError_t rms_bwd(const float *x, const float *gain, float *dgain, int rpg, int ngain, const float *rinv,
                     const float *dy, float *dx, bool acc, int rows, int width) {
    hipLaunchKernelGGL(k_rms_bwd, dim3(rows), dim3(64), 0, s, x, gain, rpg, rinv, dy, dx, acc ? 1 : 0, width);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nch = (rpg + GCH - 1) / GCH;
    hipLaunchKernelGGL(k_gain_part, dim3((width + 63) / 64, ngain, nch), dim3(1024), 0, s, x, dy, rinv, P(o.gpart),
                       rpg, width);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gain_sum, dim3((ngain * width + 255) / 256), dim3(256), 0, s, P(o.gpart), dgain, nch, width,
                       ngain);
    return hipGetLastError();
  }
  hipError_t rope(float *x, Rows rm, int N, int rows, int H, bool inverse) {
    const int64_t total = (int64_t)rows * H * (c.d / 2);
    hipLaunchKernelGGL(k_rope, dim3(grid1(total)), dim3(256), 0, s, x, rm, N, H, c.d, w.rope_cos, w.rope_sin,
                       inverse ? 1 : 0, total);
    return hipGetLastError();
  }
  hipError_t entries(float *cache, float *arr, Rows rm, int N, int mode) {
    const int64_t total = (int64_t)k * N * KD;
    hipLaunchKernelGGL(k_entries, dim3(grid1(total)), dim3(256), 0, s, cache, arr, rm, k, B, N, c.Hkv, T, c.d, mode);
    return hipGetLastError();
  }
  float *chanK(size_t cacheoff, int ch) const { return P(cacheoff) + (size_t)ch * B * KD * T; }
  hipError_t attn_fwd(const float *q, const float *K, const float *Vv, Rows rm, int N, float scale, float *out,
                      float *mst, float *lst) {
    dim3 grid(B * c.Hkv, (rm.M * (c.Hq / c.Hkv) + ATQ - 1) / ATQ);
    if (c.d == 32)
      hipLaunchKernelGGL(k_attn<32>, grid, dim3(64 * NWF), 0, s, q, K, Vv, rm, c.Hq, c.Hkv, T, scale, out, mst, lst);
    else if (c.d == 64)
      hipLaunchKernelGGL(k_attn<64>, grid, dim3(64 * NWF), 0, s, q, K, Vv, rm, c.Hq, c.Hkv, T, scale, out, mst, lst);
    else
      hipLaunchKernelGGL(k_attn<128>, grid, dim3(64 * NWF), 0, s, q, K, Vv, rm, c.Hq, c.Hkv, T, scale, out, mst, lst);
    return hipGetLastError();
  }
  hipError_t attn_dkv(const float *q, const float *K, const float *Vv, const float *dout, const float *mst,
                      const float *lst, const float *Dst, Rows rm, float scale, float *dK, float *dV) {
    dim3 grid(B * c.Hkv, (T + 63) / 64);
    if (c.d == 32)
      hipLaunchKernelGGL(k_attn_dkv<32>, grid, dim3(256), 0, s, q, K, Vv, dout, mst, lst, Dst, rm, c.Hq, c.Hkv, T,
                         scale, dK, dV);
    else if (c.d == 64)
      hipLaunchKernelGGL(k_attn_dkv<64>, grid, dim3(256), 0, s, q, K, Vv, dout, mst, lst, Dst, rm, c.Hq, c.Hkv, T,
                         scale, dK, dV);
    else
      hipLaunchKernelGGL(k_attn_dkv<128>, grid, dim3(256), 0, s, q, K, Vv, dout, mst, lst, Dst, rm, c.Hq, c.Hkv, T,
                         scale, dK, dV);
    return hipGetLastError();
  }
  hipError_t attn_dq(const float *q, const float *K, const float *Vv, const float *dout, const float *outf,
                     const float *mst, const float *lst, Rows rm, int N, float scale, float *dq, float *Dst) {
    dim3 grid(B * c.Hkv, (rm.M * (c.Hq / c.Hkv) + ATQ - 1) / ATQ);
    if (c.d == 32)
      hipLaunchKernelGGL(k_attn_dq<32>, grid, dim3(64 * NWF), 0, s, q, K, Vv, dout, outf, mst, lst, rm, c.Hq, c.Hkv, T, scale, dq,
                         Dst);
    else if (c.d == 64)
      hipLaunchKernelGGL(k_attn_dq<64>, grid, dim3(64 * NWF), 0, s, q, K, Vv, dout, outf, mst, lst, rm, c.Hq, c.Hkv, T, scale, dq,
                         Dst);
    else
      hipLaunchKernelGGL(k_attn_dq<128>, grid, dim3(64 * NWF), 0, s, q, K, Vv, dout, outf, mst, lst, rm, c.Hq, c.Hkv, T,
                         scale, dq, Dst);
    return hipGetLastError();
  }

  // The pool of one branch for the rows of the step (S from the tape):
  // nsrc, rS, u, A, m, rM, c; keys also kraw, rK and K_new (normed, turned);
  // values V_new.
  wm_status pool_fwd(int beta, Rows rm, int N) {
    TR_TRY(rms(P(o.S), w.src_norm + (size_t)beta * L * D, N, P(o.nsrc), P(o.rS), L * N, D));
    hipLaunchKernelGGL(k_router_in, dim3(grid1((int64_t)N * R * D)), dim3(256), 0, s, P(o.nsrc), P(o.u), c.p, R, N,
                       D);
    TR_TRY(hipGetLastError());
    TR_TRY(gemm(false, true, P(o.u), (int64_t)R * D, W(w.router) + (size_t)beta * L * k * R * D, (int64_t)R * D,
                P(o.A), (int64_t)L * k, N, L * k, R * D, 0.f));
    hipLaunchKernelGGL(k_mix, dim3(grid1((int64_t)k * N * D)), dim3(256), 0, s, P(o.A), P(o.nsrc), P(o.m), L, k, N,
                       D);
    TR_TRY(hipGetLastError());
    TR_TRY(rms(P(o.m), w.chan_norm + (size_t)beta * k * D, N, P(o.c), P(o.rM), k * N, D));
    if (beta == 0) {
      TR_TRY(gemm(false, true, P(o.c), D, W(w.wk), D, P(o.kraw), KD, N, KD, D, 0.f, k, (int64_t)N * D,
                  (int64_t)KD * D, (int64_t)N * KD));
      TR_TRY(rms(P(o.kraw), w.k_norm, N * c.Hkv, P(o.Kn), P(o.rK), k * N * c.Hkv, c.d));
      TR_TRY(rope(P(o.Kn), rm, N, k * N, c.Hkv, false));
    } else {
      TR_TRY(gemm(false, true, P(o.c), D, W(w.wv), D, P(o.Vn), KD, N, KD, D, 0.f, k, (int64_t)N * D,
                  (int64_t)KD * D, (int64_t)N * KD));
    }
    return WM_OK;
  }

  // Forward of one group step with every intermediate kept.  The cache is
  // only read.  want_logits: logits, and the loss rows with their gradient.
  wm_status step_fwd(Rows rm, int N, bool want_logits, float inv_count, bool with_pool = true) {
    const float scale = 1.f / sqrtf((float)c.d);
    hipLaunchKernelGGL(k_embed, dim3(N), dim3(256), 0, s, tokens, T, rm, W(w.embed), P(o.S), N, D, V);
    TR_TRY(hipGetLastError());
    // (split-k sums of Q, O and down are left to the RMSNorm that reads them)
    Pending pd;
    for (int l = 0; l < L; ++l) {
      const size_t nd = (size_t)N * D, nq = (size_t)N * QD, nf = (size_t)N * F;
      float *S = P(o.S) + l * nd, *a = P(o.a) + l * nd, *qraw = P(o.qraw) + l * nq, *q = P(o.q) + l * nq;
      float *out = P(o.o) + l * nq, *h1 = P(o.h1) + l * nd, *bn = P(o.bn) + l * nd;
      float *G = P(o.G) + l * nf, *U = P(o.U) + l * nf, *act = P(o.act) + l * nf;
      TR_TRY(rms_in(pd, S, w.attn_norm + (size_t)l * D, N, a, P(o.rA) + (size_t)l * N, N, D));
      TR_TRY(gemm(false, true, a, D, W(w.wq) + (size_t)l * QD * D, D, qraw, QD, N, QD, D, 0.f, 1, 0, 0, 0, nullptr,
                  &pd));
      TR_TRY(rms_in(pd, qraw, w.q_norm + (size_t)l * c.d, N * c.Hq, q, P(o.rQ) + (size_t)l * N * c.Hq, N * c.Hq,
                    c.d));
      TR_TRY(rope(q, rm, N, N, c.Hq, false));
      const int ch = l % k;
      TR_TRY(attn_fwd(q, chanK(o.cK, ch), chanK(o.cV, ch), rm, N, scale, out, P(o.mst) + (size_t)l * N * c.Hq,
                      P(o.lst) + (size_t)l * N * c.Hq));
      TR_TRY(gemm(false, true, out, QD, W(w.wo) + (size_t)l * D * QD, QD, h1, D, N, D, QD, 1.f, 1, 0, 0, 0, S, &pd));
      TR_TRY(rms_in(pd, h1, w.ffn_norm + (size_t)l * D, N, bn, P(o.rF) + (size_t)l * N, N, D));
      // gate and up in one launch (z = 0, 1: the two weight matrices and outputs)
      const float *Wg = W(w.w_gate) + (size_t)l * F * D, *Wu = W(w.w_up) + (size_t)l * F * D;
      TR_TRY(gemm(false, true, bn, D, Wg, D, G, F, N, F, D, 0.f, 2, 0, fdist(Wg, Wu), fdist(G, U)));
      hipLaunchKernelGGL(k_swiglu, dim3(grid1(nf)), dim3(256), 0, s, G, U, act, (int64_t)nf);
      TR_TRY(hipGetLastError());
      float *next = l + 1 < L ? P(o.S) + (l + 1) * nd : P(o.hL);
      TR_TRY(gemm(false, true, act, F, W(w.w_down) + (size_t)l * D * F, F, next, D, N, D, F, 1.f, 1, 0, 0, 0, h1,
                  l + 1 < L ? &pd : nullptr));
    }
    if (with_pool) {
      wm_status st = pool_fwd(0, rm, N);
      if (st != WM_OK) return st;
      st = pool_fwd(1, rm, N);
      if (st != WM_OK) return st;
    }
    return want_logits ? head_fwd(rm, N, inv_count) : WM_OK;
  }
  // final norm, logits, the loss rows and their gradient dz
  wm_status head_fwd(Rows rm, int N, float inv_count) {
    TR_TRY(rms(P(o.hL), w.final_norm, N, P(o.xf), P(o.rL), N, D));
    TR_TRY(gemm(false, true, P(o.xf), D, W(w.lm_head), D, P(o.logits), V, N, V, D, 0.f));
    hipLaunchKernelGGL(k_ce, dim3(N), dim3(256), 0, s, P(o.logits), tokens, T, rm, V, inv_count, P(o.lossrow),
                       P(o.dz));
    TR_TRY(hipGetLastError());
    return WM_OK;
  }

  // Backward of one branch of the pool: dout [k, N, KD] = gradient of the
  // written keys (beta 0, as stored: normed and turned) or values; adds the
  // gradient of the layer inputs into dS and the branch's parameter
  // gradients.  Recomputes the branch's forward first.
  wm_status pool_bwd(int beta, Rows rm, int N, float *dout) {
    wm_status st = pool_fwd(beta, rm, N);
    if (st != WM_OK) return st;
    const int64_t zA = (int64_t)N * KD, zB = (int64_t)KD * D, zC = (int64_t)N * D;
    if (beta == 0) {
      TR_TRY(rope(dout, rm, N, k * N, c.Hkv, true));
      TR_TRY(rms_bwd(P(o.kraw), w.k_norm, gr.k_norm, N * c.Hkv, k, P(o.rK), dout, P(o.dkraw), false, k * N * c.Hkv,
                     c.d));
      // dc_j = dkraw_j W_K^j ; dW_K^j += dkraw_j^T c_j
      TR_TRY(gemm(false, false, P(o.dkraw), KD, W(w.wk), D, P(o.dc), D, N, D, KD, 0.f, k, zA, zB, zC));
      TR_TRY(gemm(true, false, P(o.dkraw), KD, P(o.c), D, gr.wk, D, KD, D, N, 1.f, k, zA, zC, zB));
    } else {
      TR_TRY(gemm(false, false, dout, KD, W(w.wv), D, P(o.dc), D, N, D, KD, 0.f, k, zA, zB, zC));
      TR_TRY(gemm(true, false, dout, KD, P(o.c), D, gr.wv, D, KD, D, N, 1.f, k, zA, zC, zB));
    }
    TR_TRY(rms_bwd(P(o.m), w.chan_norm + (size_t)beta * k * D, gr.chan_norm + (size_t)beta * k * D, N, k, P(o.rM),
                   P(o.dc), P(o.dm), false, k * N, D));
    hipLaunchKernelGGL(k_mix_dA, dim3(N, L * k), dim3(64), 0, s, P(o.dm), P(o.nsrc), P(o.dA), L, k, N, D);
    TR_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_mix_dn, dim3(grid1((int64_t)L * N * D)), dim3(256), 0, s, P(o.A), P(o.dm), P(o.dn), L, k, N,
                       D);
    TR_TRY(hipGetLastError());
    const float *Wr = W(w.router) + (size_t)beta * L * k * R * D;
    TR_TRY(gemm(true, false, P(o.dA), (int64_t)L * k, P(o.u), (int64_t)R * D, gr.router + (size_t)beta * L * k * R * D,
                (int64_t)R * D, L * k, R * D, N, 1.f));
    TR_TRY(gemm(false, false, P(o.dA), (int64_t)L * k, Wr, (int64_t)R * D, P(o.du), (int64_t)R * D, N, R * D, L * k,
                0.f));
    hipLaunchKernelGGL(k_router_in_bwd, dim3(grid1((int64_t)N * R * D)), dim3(256), 0, s, P(o.du), P(o.dn), c.p, R, N,
                       D);
    TR_TRY(hipGetLastError());
    TR_TRY(rms_bwd(P(o.S), w.src_norm + (size_t)beta * L * D, gr.src_norm + (size_t)beta * L * D, N, L, P(o.rS),
                   P(o.dn), P(o.dS), true, L * N, D));
    return WM_OK;
  }

  // Backward of one group step whose forward is in the tape; dKn / dVn hold
  // the gradient of its written entries.
  wm_status step_bwd(Rows rm, int N, bool last_pass) {
    const float scale = 1.f / sqrtf((float)c.d);
    const size_t nd = (size_t)N * D, nq = (size_t)N * QD, nf = (size_t)N * F;
    float *dh = P(o.dh);
    if (last_pass) {
      TR_TRY(gemm(false, false, P(o.dz), V, W(w.lm_head), D, P(o.dxf), D, N, D, V, 0.f));
      TR_TRY(gemm(true, false, P(o.dz), V, P(o.xf), D, gr.lm_head, D, V, D, N, 1.f));
      TR_TRY(rms_bwd(P(o.hL), w.final_norm, gr.final_norm, N, 1, P(o.rL), P(o.dxf), dh, false, N, D));
    } else {
      TR_TRY(fill(dh, nd, 0.f));
    }
    TR_TRY(fill(P(o.dS), (int64_t)L * nd, 0.f));
    wm_status st = pool_bwd(0, rm, N, P(o.dKn));
    if (st != WM_OK) return st;
    st = pool_bwd(1, rm, N, P(o.dVn));
    if (st != WM_OK) return st;
    for (int l = L - 1; l >= 0; --l) {
      float *S = P(o.S) + l * nd, *a = P(o.a) + l * nd, *qraw = P(o.qraw) + l * nq, *q = P(o.q) + l * nq;
      float *out = P(o.o) + l * nq, *h1 = P(o.h1) + l * nd, *bn = P(o.bn) + l * nd;
      float *G = P(o.G) + l * nf, *U = P(o.U) + l * nf, *act = P(o.act) + l * nf;
      float *mst = P(o.mst) + (size_t)l * N * c.Hq, *lst = P(o.lst) + (size_t)l * N * c.Hq;
      // FFN: h_out = h1 + act W_down^T
      TR_TRY(gemm(false, false, dh, D, W(w.w_down) + (size_t)l * D * F, F, P(o.dact), F, N, F, D, 0.f));
      TR_TRY(gemm(true, false, dh, D, act, F, gr.w_down + (size_t)l * D * F, F, D, F, N, 1.f));
      hipLaunchKernelGGL(k_swiglu_bwd, dim3(grid1(nf)), dim3(256), 0, s, G, U, P(o.dact), P(o.dG), P(o.dU),
                         (int64_t)nf);
      TR_TRY(hipGetLastError());
      TR_TRY(gemm(false, false, P(o.dG), F, W(w.w_gate) + (size_t)l * F * D, D, P(o.db), D, N, D, F, 0.f));
      TR_TRY(gemm(false, false, P(o.dU), F, W(w.w_up) + (size_t)l * F * D, D, P(o.db), D, N, D, F, 1.f));
      {  // the gate and up weight gradients in one launch
        float *gg = gr.w_gate + (size_t)l * F * D, *gu = gr.w_up + (size_t)l * F * D;
        TR_TRY(gemm(true, false, P(o.dG), F, bn, D, gg, D, F, D, N, 1.f, 2, fdist(P(o.dG), P(o.dU)), 0,
                    fdist(gg, gu)));
      }
      TR_TRY(rms_bwd(h1, w.ffn_norm + (size_t)l * D, gr.ffn_norm + (size_t)l * D, N, 1, P(o.rF) + (size_t)l * N,
                     P(o.db), dh, true, N, D));
      // attention: h1 = h_l + out W_O^T
      TR_TRY(gemm(false, false, dh, D, W(w.wo) + (size_t)l * D * QD, QD, P(o.dout), QD, N, QD, D, 0.f));
      TR_TRY(gemm(true, false, dh, D, out, QD, gr.wo + (size_t)l * D * QD, QD, D, QD, N, 1.f));
      const int ch = l % k;
      TR_TRY(attn_dq(q, chanK(o.cK, ch), chanK(o.cV, ch), P(o.dout), out, mst, lst, rm, N, scale, P(o.dq),
                     P(o.Dst)));
      TR_TRY(attn_dkv(q, chanK(o.cK, ch), chanK(o.cV, ch), P(o.dout), mst, lst, P(o.Dst), rm, scale,
                      chanK(o.dK, ch), chanK(o.dV, ch)));
      TR_TRY(rope(P(o.dq), rm, N, N, c.Hq, true));
      // (the head-norm backward's output goes to dout, free again)
      TR_TRY(rms_bwd(qraw, w.q_norm + (size_t)l * c.d, gr.q_norm + (size_t)l * c.d, N * c.Hq, 1,
                     P(o.rQ) + (size_t)l * N * c.Hq, P(o.dq), P(o.dout), false, N * c.Hq, c.d));
      TR_TRY(gemm(false, false, P(o.dout), QD, W(w.wq) + (size_t)l * QD * D, D, P(o.da), D, N, D, QD, 0.f));
      TR_TRY(gemm(true, false, P(o.dout), QD, a, D, gr.wq + (size_t)l * QD * D, D, QD, D, N, 1.f));
      TR_TRY(rms_bwd(S, w.attn_norm + (size_t)l * D, gr.attn_norm + (size_t)l * D, N, 1, P(o.rA) + (size_t)l * N,
                     P(o.da), dh, true, N, D));
      // the block input also feeds the pool
      TR_TRY(add(dh, P(o.dS) + l * nd, nd));
    }
    int *nxt = (int *)P(o.enext), *head = (int *)P(o.ehead);
    hipLaunchKernelGGL(k_embed_chains, dim3((N + 63) / 64), dim3(64), 0, s, tokens, T, rm, N, nxt, head);
    TR_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_embed_bwd, dim3(N), dim3(256), 0, s, tokens, T, rm, dh, nxt, head, gr.embed, D, V);
    TR_TRY(hipGetLastError());
    return WM_OK;
  }

  // Group step of a forward pass: keep the old entries (undo != null), run
  // the stack and the pool, write the new entries.
  wm_status fwd_write(Rows rm, int N, float *undo) {
    if (undo) {
      TR_TRY(entries(P(o.cK), undo, rm, N, 0));
      TR_TRY(entries(P(o.cV), undo + (size_t)k * N * KD, rm, N, 0));
    }
    wm_status st = step_fwd(rm, N, false, 0.f);
    if (st != WM_OK) return st;
    TR_TRY(entries(P(o.cK), P(o.Kn), rm, N, 1));
    TR_TRY(entries(P(o.cV), P(o.Vn), rm, N, 1));
    return WM_OK;
  }

  wm_status run(int n_nograd, int n_grad, float *loss) {
    const int64_t cache = (int64_t)k * B * KD * T;
    const int ng = std::min(g, T);
    const float inv_count = 1.f / ((float)B * (T - 1));
    TR_TRY(fill(P(o.cK), cache, 0.f));
    TR_TRY(fill(P(o.cV), cache, 0.f));
    TR_TRY(fill(P(o.dK), cache, 0.f));
    TR_TRY(fill(P(o.dV), cache, 0.f));
    TR_TRY(fill(P(o.lossrow), (int64_t)B * T, 0.f));
    // gradients start at zero
    struct G2 {
      float *p;
      int64_t n;
    };
    const int64_t Ld = (int64_t)L * D;
    const G2 gz[] = {{gr.embed, (int64_t)V * D},
                     {gr.lm_head, (int64_t)V * D},
                     {gr.final_norm, D},
                     {gr.attn_norm, Ld},
                     {gr.wq, (int64_t)L * QD * D},
                     {gr.q_norm, (int64_t)L * c.d},
                     {gr.wo, (int64_t)L * D * QD},
                     {gr.ffn_norm, Ld},
                     {gr.w_gate, (int64_t)L * F * D},
                     {gr.w_up, (int64_t)L * F * D},
                     {gr.w_down, (int64_t)L * D * F},
                     {gr.src_norm, 2 * Ld},
                     {gr.router, (int64_t)2 * L * k * R * D},
                     {gr.chan_norm, (int64_t)2 * k * D},
                     {gr.wk, (int64_t)k * KD * D},
                     {gr.wv, (int64_t)k * KD * D},
                     {gr.k_norm, (int64_t)k * c.d}};
    for (const G2 &z : gz) TR_TRY(fill(z.p, z.n, 0.f));
    // forward: passes without gradient, then the gradient passes with undo
    // (and, when they fit, each gradient step's tape in its own slot)
    const Ws base = o;
    const bool keep = base.nslot > 1;
    for (int pass = 0; pass < n_nograd + n_grad; ++pass) {
      const int gp = pass - n_nograd;
      for (int q = 0; q < ng; ++q) {
        const int M = (T - q + g - 1) / g;
        const Rows rm{M, q, g};
        float *undo = gp >= 0 ? P(o.undo) + ((size_t)gp * ng + q) * o.undo_slot : nullptr;
        o = keep && gp >= 0 ? base.slot(1 + gp * ng + q) : base;
        wm_status st = fwd_write(rm, B * M, undo);
        o = base;
        if (st != WM_OK) return st;
      }
    }
    // backward over the gradient steps in reverse: the step's tape (kept, or
    // recomputed from the cache as the step found it; the pool's forward is
    // redone branch by branch in its backward either way)
    for (int gp = n_grad - 1; gp >= 0; --gp) {
      for (int q = ng - 1; q >= 0; --q) {
        const int M = (T - q + g - 1) / g, N = B * M;
        const Rows rm{M, q, g};
        float *undo = P(o.undo) + ((size_t)gp * ng + q) * o.undo_slot;
        TR_TRY(entries(P(o.dK), P(o.dKn), rm, N, 2));
        TR_TRY(entries(P(o.dV), P(o.dVn), rm, N, 2));
        TR_TRY(entries(P(o.cK), undo, rm, N, 1));
        TR_TRY(entries(P(o.cV), undo + (size_t)k * N * KD, rm, N, 1));
        const bool last = gp == n_grad - 1;
        wm_status st = WM_OK;
        if (keep) {
          o = base.slot(1 + gp * ng + q);
          if (last) st = head_fwd(rm, N, inv_count);
        } else {
          st = step_fwd(rm, N, last, inv_count, false);
        }
        if (st == WM_OK) st = step_bwd(rm, N, last);
        o = base;
        if (st != WM_OK) return st;
      }
    }
    hipLaunchKernelGGL(k_loss_sum, dim3(1), dim3(256), 0, s, P(o.lossrow), (int64_t)B * T, inv_count, loss);
    TR_TRY(hipGetLastError());
    return WM_OK;
  }
};

}  // namespace tr
}  // namespace wm

using namespace wm;

extern "C" {

size_t wm_train_workspace_bytes(const wm_config *cfg, int32_t B, int32_t T, int32_t g, int32_t n_grad) {
  if (!cfg || wm_check_config(cfg) != WM_OK || B < 1 || T < 2 || g < 1 || n_grad < 1) return 0;
  return tr::layout(*cfg, B, T, g, n_grad, true).bytes;
}

size_t wm_train_workspace_min_bytes(const wm_config *cfg, int32_t B, int32_t T, int32_t g, int32_t n_grad) {
  if (!cfg || wm_check_config(cfg) != WM_OK || B < 1 || T < 2 || g < 1 || n_grad < 1) return 0;
  return tr::layout(*cfg, B, T, g, n_grad, false).bytes;
}

wm_status wm_train_step(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t B, int32_t T,
                        int32_t g, int32_t n_nograd, int32_t n_grad, const wm_grads *grads, float *loss, void *ws,
                        size_t ws_bytes, wm_stream stream) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  TR_CHECK(cfg->dtype == WM_F32, WM_ERR_DTYPE, "the training step runs in float32 only (dtype %d)", cfg->dtype);
  TR_CHECK(B >= 1, WM_ERR_SHAPE, "B = %d must be >= 1", B);
  TR_CHECK(T >= 2 && T <= cfg->T_max, WM_ERR_RANGE, "T = %d outside [2, T_max = %d]", T, cfg->T_max);
  TR_CHECK(g >= 1, WM_ERR_SHAPE, "g = %d must be >= 1", g);
  TR_CHECK(n_nograd >= 0 && n_grad >= 1, WM_ERR_ARG, "n_nograd = %d must be >= 0 and n_grad = %d >= 1", n_nograd,
           n_grad);
  TR_CHECK(w && tokens && grads && loss && ws, WM_ERR_ARG, "weights, tokens, grads, loss or workspace is NULL");
  TR_CHECK(w->static_mix == nullptr, WM_ERR_ARG, "static_mix must be NULL: the training step trains the router");
  const void *wp[] = {w->embed,  w->lm_head, w->final_norm, w->attn_norm, w->wq,        w->q_norm,
                      w->wo,     w->ffn_norm, w->w_gate,    w->w_up,      w->w_down,    w->src_norm,
                      w->router, w->chan_norm, w->wk,       w->wv,        w->k_norm,    w->rope_cos,
                      w->rope_sin};
  for (const void *p : wp) TR_CHECK(p, WM_ERR_ARG, "a weight pointer or the rope table is NULL");
  const float *gp[] = {grads->embed, grads->lm_head, grads->final_norm, grads->attn_norm, grads->wq,
                       grads->q_norm, grads->wo,     grads->ffn_norm,   grads->w_gate,    grads->w_up,
                       grads->w_down, grads->src_norm, grads->router,   grads->chan_norm, grads->wk,
                       grads->wv,     grads->k_norm};
  for (const float *p : gp) TR_CHECK(p, WM_ERR_ARG, "a gradient pointer is NULL");
  // the kept-tape layout when the workspace holds it, else the recomputing one
  const bool tapes = ws_bytes >= tr::layout(*cfg, B, T, g, n_grad, true).bytes;
  const size_t need = tr::layout(*cfg, B, T, g, n_grad, false).bytes;
  TR_CHECK(ws_bytes >= need, WM_ERR_WORKSPACE, "workspace of %zu bytes, the training step needs %zu", ws_bytes,
           need);
  tr::Trainer t(*cfg, *w, *grads, tokens, B, T, g, n_grad, tapes, ws, (hipStream_t)stream);
  return t.run(n_nograd, n_grad, loss);
}

}  // extern "C"
