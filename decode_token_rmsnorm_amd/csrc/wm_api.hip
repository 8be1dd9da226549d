// wm_api.hip — device entry points of the C ABI (include/wm.h): argument
// checks, then the kernel sequence of each call on the caller's stream.
#include "../../include/wm.h"
#include "wm_attn.hpp"
#include "wm_gemm.hpp"
#include "wm_gemm2.hpp"
#include "wm_host.hpp"
#include "wm_pool.hpp"
#include "wm_few.hpp"
#include "wm_attn2.hpp"
#include "wm_pool2.hpp"
#include "wm_kvs.hpp"

#include <mutex>
#include <type_traits>
#include <vector>

namespace wm {

// Group steps of at most this many rows run the layer stack's products with
// one output row block per 16 rows (Q, O, down, LM head, the vanilla model's
// K/V) on the few-row kernel: at 1024 rows it launches ~512 blocks where the
// 128 x 128 kernel launches 32, and Q and O take 10.7 instead of 20.8 and
// 18.9 us, down 24.8 instead of 33.6 (small model, D512).  The fused gate/up
// product, 6x wider, stays on the 128 x 128 kernel above kFewRows rows (15.5
// against 34 us there).
constexpr int kFewStackRows = 1024;
// bf16 channel attention with at most this many query rows per (sequence, KV
// head) pair runs on attn_few in blocks of 32 rows (no key split, so no
// combine launch, where attn2_kernel's 128-row blocks would need splits to
// fill the GPU).
constexpr int kFewAttnRows = 512;

// ------------------------------------------------------------ launch timing
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
struct ProfState {
  uint32_t mask = 0;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<ProfRec> recs;
};
static ProfState g_prof;

static hipEvent_t prof_event() {
  if (g_prof.used == g_prof.pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_prof.pool.push_back(e);
  }
  return g_prof.pool[g_prof.used++];
}

// Brackets the launches of one kernel kind with events while profiling.
struct ProfScope {
  int kind;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(int k, hipStream_t st) : kind(k), s(st) {
    if (g_prof.mask & (1u << k)) {
      a = prof_event();
      b = prof_event();
      if (a && b) (void)hipEventRecord(a, s);
    }
  }
  ~ProfScope() {
    if (a && b) {
      (void)hipEventRecord(b, s);
      g_prof.recs.push_back({kind, a, b});
    }
  }
};

#define WM_TRY(expr)                                                               \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess) {                                                        \
      set_error("%s failed: %s", #expr, hipGetErrorString(e_));                    \
      return WM_ERR_HIP;                                                           \
    }                                                                              \
  } while (0)

#define WM_CHECK(cond, code, ...) \
  do {                            \
    if (!(cond)) {                \
      set_error(__VA_ARGS__);     \
      return code;                \
    }                             \
  } while (0)

// Everything one call needs, resolved from the C structs.
template <typename T> struct Run {
  const wm_config &c;
  const wm_weights *w;
  const wm_cache *cache;
  unsigned char *ws;
  WsLayout lay;
  hipStream_t s;
  int R;
  int rows_cap;  // rows the workspace was laid out for
  // The vanilla comparison model: per-layer K/V projection (cache slot l =
  // layer l, k = L) appended before the layer's attention, which then includes
  // the query's own position (s <= i); no state stack and no pool.
  bool vanilla = false;
  // The feedback-free variant (k = L): channel l mixes the states 0..l of its
  // token only, so it is built at layer l, before that layer's (strict)
  // attention, from the states already in place; no pool after the stack.
  bool ff = false;

  Run(const wm_config &c_, const wm_weights *w_, const wm_cache *ca, void *ws_, int rows, hipStream_t st)
      : c(c_), w(w_), cache(ca), ws((unsigned char *)ws_), lay(ws_layout(c_, rows)), s(st), R((c_.L + c_.p - 1) / c_.p),
        rows_cap(rows) {}

  template <typename P> P *at(size_t off) const { return (P *)(ws + off); }
  // The 256 x 256 kernel (bf16 only) for steps with enough rows to fill the chip.
  static constexpr bool kBig = std::is_same<T, bf16>::value;
  bool big(int M) const { return kBig && M >= 2048; }
  // rows from which the pool's width-512 K/V projection streams past a
  // register-held matrix (below, the tiled kernels)
  static constexpr int kKvsMinRows = 256;
  // column tile of the residual products on M rows
  int resid_bn(int M, int N) const { return big(M) ? g2_resid_bn(M, N, kComputeUnits) : GN; }
  // partial sums of squares per row written by a residual epilogue on M rows
  int parts(int M, int N, int K) const {
    if (M <= kFewStackRows) return few_parts(M, N, K);
    return (N + resid_bn(M, N) - 1) / resid_bn(M, N);
  }
  // Decode steps whose position lives in device memory: read by the kernels
  // when they run (RowPos::s0p, AttnArgs::s0p).
  const int32_t *pos_dev = nullptr;
  RowPos rowpos(const wm_tokset &ts) const { return RowPos{ts.M, ts.s0, ts.s_step, pos_dev, c.T_max}; }
  T *Kch(int ch) const { return (T *)cache->k + (int64_t)ch * cache->B * c.Hkv * c.T_max * c.d; }
  T *Vch(int ch) const { return (T *)cache->v + (int64_t)ch * cache->B * c.Hkv * c.T_max * c.d; }

  // Block order of the Q, O and down products (about one round of blocks over
  // the compute units at the 1.3B shapes): 8-tile M-bands, about 1% faster
  // there than the 4-tile bands the five-round gate/up product runs best with.
  static constexpr int kOneRoundMap = 4;
  // Wave arrangement of the large-tile products (G2Shape): gate/up and Q on 2
  // x 4 waves of 128 x 64 and the residual products on 224-column tiles of 4 x
  // 2 waves of 64 x 112 on the 16x16x32 MFMA (two waves per SIMD: gate/up
  // 309.6 -> 279.3 us, Q 87 -> 71.5 with its epilogue at 4 rows per step, on
  // the 1.3B shapes; the pool's router and K/V projection 66 -> 54 and 173 ->
  // 149 us on the mix-only workload; O 85.5 -> 79.1 -> 74.8 and down 170.3 ->
  // 157.3 -> 144.1 us through 8 x 1 waves of 32 x 224 to the 4 x 2 waves,
  // whose fragment reads are 31% fewer; A/B on one GPU each).
  static constexpr int kGUShape = 2, kQShape = 2, kR224Shape = 4, kR256Shape = 0, kPoolShape = 2;
  // A [M, K] (row-major, lda) times B [N, K]^T on the large-tile kernel.
  template <class EP>
  hipError_t gemm2_rows(const T *A, int64_t lda, const T *B, int64_t ldb, const EP &ep, int M, int N, int K) {
    if constexpr (kBig) {
      return launch_gemm2<G2KB, G2ST, kOneRoundMap, kQShape>(PRows<T>{A, lda, 0, M}, PBRows<T>{PRows<T>{B, ldb, 0, N}},
                                                             ep, M, N, K, 1, s);
    } else {
      return hipErrorInvalidValue;
    }
  }
  // The same for the residual products, on the column tile resid_bn(M, N).
  hipError_t gemm2_resid(const T *A, int64_t lda, const T *B, int64_t ldb, const EpiResid<T> &ep, int M, int N,
                         int K) {
    if constexpr (kBig) {
      const PRows<T> a{A, lda, 0, M};
      const PBRows<T> b{PRows<T>{B, ldb, 0, N}};
      if (resid_bn(M, N) == G2Shape<1>::BN)
        return launch_gemm2<G2KB, G2ST, kOneRoundMap, kR224Shape>(a, b, ep, M, N, K, 1, s);
      return launch_gemm2<G2KB, G2ST, kOneRoundMap, kR256Shape>(a, b, ep, M, N, K, 1, s);
    } else {
      return hipErrorInvalidValue;
    }
  }

  // A product of the layer stack below the large-tile size: the few-row
  // kernel up to kFewStackRows rows, otherwise the 128 x 128 tiled one.
  template <class AL, class BL, class EP>
  hipError_t gemm_s(const AL &al, const BL &bl, const EP &ep, int M, int N, int K) {
    if (M <= kFewStackRows) return launch_few<T>(al, bl, ep, M, N, K, 1, s);
    return launch_gemm<T>(al, bl, ep, M, N, K, 1, s);
  }

  // Few rows: the few-row kernel; otherwise the 128 x 128 tiled one.
  template <class AL, class BL, class EP>
  hipError_t gemm1(const AL &al, const BL &bl, const EP &ep, int M, int N, int K, int Z) {
    if constexpr (!std::is_same<BL, BGateUp<T>>::value) {  // (few-row gate/up: FGateUp)
      if (M <= kFewRows) return launch_few<T>(al, bl, ep, M, N, K, Z, s);
    }
    return launch_gemm<T>(al, bl, ep, M, N, K, Z, s);
  }

  // -------------------------------------------------------- channel attention
  template <int DH> wm_status attn_dh(int layer, const T *q, wm_tokset ts, T *out) {
    const int ch = layer % c.k, G = c.Hq / c.Hkv, rows = ts.B * ts.M;
    const int rows_pair = ts.M * G;
    const bool large = rows_pair >= 128;
    constexpr bool bfd = std::is_same<T, bf16>::value && DH >= 64;
    // bf16 with up to kFewAttnRows rows per pair: a block of waves per (pair,
    // split, 32 query rows), the waves splitting the keys and merging in LDS
    // (attn_few); with more: 4 waves of 32 rows on 32x32 MFMAs sharing LDS
    // tiles (attn2_kernel)
    const bool few = bfd && rows_pair <= kFewAttnRows;
    const bool v2 = large && bfd && !few;
    constexpr int few_nw = DH == 64 ? 8 : 4;
    const int rb = few ? 32 : large ? 128 : 16, nw = v2 ? 4 : few ? few_nw : large ? 8 : 1;
    const int nrb = (rows_pair + rb - 1) / rb;
    const int blocks = nrb * ts.B * c.Hkv;
    int64_t kmax = (int64_t)ts.s0 + (int64_t)(ts.M - 1) * ts.s_step;
    if (kmax > c.T_max) kmax = c.T_max;
    const int kt = few ? 32 : AKT;
    const int ntile = (int)((kmax + kt - 1) / kt);
    // waves in flight; attn_few keeps at least 4 tiles per wave.  (Many-row
    // steps: 1024 waves; with 2048 the small model's 1024-row group steps
    // took 8 key splits and a combine, 25.1 against 23.4 us per layer-step;
    // with 512, 30.4.  The 1.3B steps reach 1024 waves without splitting.)
    const int64_t target = large ? 1024 : few ? 1024 : 4096;
    int ns = 1;
    while ((int64_t)blocks * nw * ns < target && ns * 2 <= ACS && ntile / (ns * 2 * (few ? few_nw : 1)) >= (few ? 4 : 2) &&
           (int64_t)(ns * 2) * rows <= part_rows_cap(rows_cap))
      ns *= 2;
    AttnArgs a;
    a.q = q;
    a.out = out;
    a.Kc = Kch(ch);
    a.Vc = Vch(ch);
    a.part_o = at<float>(lay.part_o);
    a.part_ml = at<float>(lay.part_ml);
    a.B = ts.B;
    a.M = ts.M;
    a.s0 = ts.s0;
    a.step = ts.s_step;
    a.Hq = c.Hq;
    a.Hkv = c.Hkv;
    a.G = G;
    a.T_max = c.T_max;
    a.nsplit = ns;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)c.d);
    a.s0p = pos_dev;
    dim3 grid(nrb, ts.B * c.Hkv, ns);
    ProfScope prof(WM_K_ATTN, s);
    if constexpr (bfd) {
      if (v2) hipLaunchKernelGGL((attn2_kernel<DH, 1>), dim3(ts.B * c.Hkv, nrb, ns), dim3(256), 0, s, a);
      if (few) hipLaunchKernelGGL((attn_few<DH, few_nw>), dim3(ns, ts.B * c.Hkv, nrb), dim3(64 * few_nw), 0, s, a);
    }
    if (v2 || few)
      ;
    else if (large)
      hipLaunchKernelGGL((attn_kernel<T, DH, 8, 1>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((attn_kernel<T, DH, 1, 1>), grid, dim3(64), 0, s, a);
    WM_TRY(hipGetLastError());
    if (ns > 1) {
      const int64_t nout = (int64_t)rows * c.Hq * c.d;
      hipLaunchKernelGGL((attn_combine<T>), dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, s, a.part_o, a.part_ml,
                         (void *)out, rows, c.Hq, c.d, ns);
      WM_TRY(hipGetLastError());
    }
    return WM_OK;
  }

  wm_status attn(int layer, const T *q, wm_tokset ts, T *out) {
    switch (c.d) {
      case 32: return attn_dh<32>(layer, q, ts, out);
      case 64: return attn_dh<64>(layer, q, ts, out);
      default: return attn_dh<128>(layer, q, ts, out);
    }
  }

  // -------------------------------------------------------- KV pool
  // Router output layout (see pool): element (z, beta, row, l*k + j) at
  // z*az + beta*ab + row*ar + l*k + j, Z split partials.
  struct RouterOut {
    int Z;
    int64_t az, ab, ar;
  };

  // Mix of kk channels over the first LL source states; the gains are the
  // model's (beta strides L*D and k*D) from src_norm / cg0.
  template <int KMAX> wm_status mix(const T *S, int rows, RouterOut ro, const float *A) {
    return mix_g<KMAX>(S, rows, ro, A, c.L, c.k, w->chan_norm);
  }
  template <int KMAX>
  wm_status mix_g(const T *S, int rows, RouterOut ro, const float *A, int LL, int kk, const float *cg0) {
    const int64_t sgb = (int64_t)c.L * c.D, cgb = (int64_t)c.k * c.D;
    if constexpr (std::is_same<T, bf16>::value) {  // MFMA mix (wm_pool2.hpp)
      // (template: channel blocks of 16, layers staged per chunk at most 16 or 32)
      auto go = [&](auto kern, int rt) {
        hipLaunchKernelGGL(kern, dim3((rows + rt - 1) / rt), dim3(256), 0, s, S, at<float>(lay.rinvS), A, ro.Z,
                           ro.az, ro.ab, ro.ar, w->src_norm, sgb, cg0, cgb, at<T>(lay.mb), at<float>(lay.rinvM), rows,
                           LL, kk, c.D, c.eps);
      };
      // (up to kFewRows rows: one row per block)
      const bool one = rows <= kFewRows;
      if (kk <= 8 && LL <= 16)  // both branches' channels in one MFMA
        one ? go(pool_mix2<1, 16, true, 1>, 1) : go(pool_mix2<1, 16, true>, PM_RTPB);
      else if (kk <= 16)
        one ? (LL <= 16 ? go(pool_mix2<1, 16, false, 1>, 1) : go(pool_mix2<1, 32, false, 1>, 1))
            : (LL <= 16 ? go(pool_mix2<1, 16>, PM_RT4) : go(pool_mix2<1, 32>, PM_RT4));
      else
        LL <= 16 ? go(pool_mix2<2, 16>, PM_RT4 / 2) : go(pool_mix2<2, 32>, PM_RT4 / 2);
    } else {
      hipLaunchKernelGGL((pool_mix<T, KMAX>), dim3(rows), dim3(256), 0, s, S, at<float>(lay.rinvS), A, ro.Z, ro.az,
                         ro.ab, ro.ar, w->src_norm, sgb, cg0, cgb, at<T>(lay.mb), at<float>(lay.rinvM), rows, LL, kk,
                         c.D, c.eps);
    }
    WM_TRY(hipGetLastError());
    return WM_OK;
  }

  // Router weights with the source gains folded in, for steps with more than
  // kFewRows rows (once per call; the workspace keeps them).
  wm_status prep_router() {
    if (rows_cap <= kFewRows || w->static_mix) return WM_OK;
    const int64_t n = 2 * (int64_t)c.L * c.k * R * c.D / Elt<T>::E16;
    hipLaunchKernelGGL((fold_router<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const T *)w->router,
                       w->src_norm, at<T>(lay.wf), c.L * c.k, c.L, c.p, R, c.D);
    WM_TRY(hipGetLastError());
    return WM_OK;
  }

  wm_status pool(const T *S, wm_tokset ts) {
    const int rows = ts.B * ts.M;
    const int64_t nl = (int64_t)c.L * rows;
    const int Lk = c.L * c.k;
    const int64_t RD = (int64_t)R * c.D;
    RouterOut ro;
    const float *Amix = at<float>(lay.Aw);
    if (w->static_mix) {
      // static mixing: every row mixes with the constant [2, L, k] weights
      // (row stride 0); only the source row scales are needed
      ProfScope prof(WM_K_MIX, s);
      hipLaunchKernelGGL((state_rinv<T>), dim3((unsigned)((nl + 3) / 4)), dim3(256), 0, s, S, at<float>(lay.rinvS),
                         nl, c.D, c.eps);
      WM_TRY(hipGetLastError());
      ro = RouterOut{1, 0, Lk, 0};
      Amix = w->static_mix;
    } else if (rows <= kFewRows) {
      // few rows: row scales and per-branch gained router input in one launch,
      // then the few-row GEMM, Z = branch
      ProfScope prof(WM_K_ROUTER, s);
      hipLaunchKernelGGL((rinv_router_input<T>), dim3(rows, 2), dim3(256), 0, s, S, at<float>(lay.rinvS), w->src_norm,
                         at<T>(lay.u), rows, c.L, c.p, R, c.D, c.eps);
      WM_TRY(hipGetLastError());
      LoadRows<T> ua{at<T>(lay.u), RD, (int64_t)rows * RD, nullptr};
      BRows<T> rb{LoadRows<T>{(const T *)w->router, RD, (int64_t)Lk * RD, nullptr}};
      EpiStoreF32 re{at<float>(lay.Aw), Lk, (int64_t)rows * Lk, nullptr, nullptr, nullptr, 0, 0.f, 0.f};
      WM_TRY((gemm1(ua, rb, re, rows, Lk, (int)RD, 2)));
      ro = RouterOut{1, 0, (int64_t)rows * Lk, Lk};
    } else {
      // many rows: one normalised router input (gains folded into the
      // weights), both branches in one GEMM, k split in Zs ranges whose
      // partials the mix adds
      {
        ProfScope prof(WM_K_MIX, s);
        hipLaunchKernelGGL((state_rinv_u<T>), dim3((unsigned)((nl + 3) / 4)), dim3(256), 0, s, S, at<float>(lay.rinvS),
                           at<T>(lay.u), rows, c.L, c.p, R, c.D, c.eps);
        WM_TRY(hipGetLastError());
      }
      const int N = 2 * Lk;
      const bool g2 = big(rows);
      const int64_t tiles = g2 ? (int64_t)((rows + G2M - 1) / G2M) * ((N + G2N - 1) / G2N)
                               : (int64_t)((rows + GM - 1) / GM) * ((N + GN - 1) / GN);
      int Zs = 1;
      while (Zs < kRouterMaxSplits && tiles * Zs < 256 && RD % (2 * Zs * 64) == 0) Zs *= 2;
      const int64_t Kz = RD / Zs;
      EpiStoreF32 re{at<float>(lay.Aw), N, (int64_t)rows * N, nullptr, nullptr, nullptr, 0, 0.f, 0.f};
      ProfScope prof(WM_K_ROUTER, s);
      bool done = false;
      if constexpr (kBig) {
        if (g2) {
          PRows<T> a2{at<T>(lay.u), RD, Kz, rows};
          PBRows<T> b2{PRows<T>{at<T>(lay.wf), RD, Kz, N}};
          WM_TRY((launch_gemm2<G2KB, G2ST, 2, kPoolShape>(a2, b2, re, rows, N, (int)Kz, Zs, s)));
          done = true;
        }
      }
      if (!done) {
        LoadRows<T> ua{at<T>(lay.u), RD, Kz, nullptr};
        BRows<T> rb{LoadRows<T>{at<T>(lay.wf), RD, Kz, nullptr}};
        WM_TRY((gemm1(ua, rb, re, rows, N, (int)Kz, Zs)));
      }
      ro = RouterOut{Zs, (int64_t)rows * N, Lk, N};
    }
    wm_status st;
    {
      ProfScope prof(WM_K_MIX, s);
      st = c.k <= 4    ? mix<4>(S, rows, ro, Amix)
           : c.k <= 8  ? mix<8>(S, rows, ro, Amix)
           : c.k <= 16 ? mix<16>(S, rows, ro, Amix)
                       : mix<32>(S, rows, ro, Amix);
    }
    if (st != WM_OK) return st;
    // per-channel projection, z = beta*k + j
    LoadRows<T> pa{at<T>(lay.mb), c.D, (int64_t)rows * c.D, nullptr};
    BKV<T> pb{(const T *)w->wk, (const T *)w->wv, c.D, (int64_t)c.Hkv * c.d * c.D, c.k};
    EpiKV<T> pe{(T *)cache->k, (T *)cache->v, at<float>(lay.rinvM), w->k_norm, w->rope_cos, w->rope_sin, c.k,
                cache->B, c.Hkv, c.T_max, c.d, rows, c.eps, rowpos(ts)};
    ProfScope prof(WM_K_KVPROJ, s);
    if constexpr (kBig) {
      if (c.D == KVS_D && c.d == KVS_HD && c.Hkv * c.d == KVS_N && rows >= kKvsMinRows) {
        // width 512, 4 KV heads of 64: the matrix stays in registers
        // and the mixed rows stream past it (wm_kvs.hpp)
        const int P = kvs_blocks_per_channel(2 * c.k);
        hipLaunchKernelGGL(kv_stream, dim3(2 * c.k * P), dim3(512), 0, s, (const bf16 *)at<T>(lay.mb),
                           (const bf16 *)w->wk, (const bf16 *)w->wv, pe, rows, P);
        WM_TRY(hipGetLastError());
        return WM_OK;
      }
      if (big(rows)) {
        PRows<T> a2{at<T>(lay.mb), c.D, (int64_t)rows * c.D, rows};
        PKV<T> b2{(const T *)w->wk, (const T *)w->wv, c.D, (int64_t)c.Hkv * c.d * c.D, c.k, c.Hkv * c.d};
        WM_TRY((launch_gemm2<G2KB, G2ST, 2, kPoolShape>(a2, b2, pe, rows, c.Hkv * c.d, c.D, 2 * c.k, s)));
        return WM_OK;
      }
    }
    WM_TRY((gemm1(pa, pb, pe, rows, c.Hkv * c.d, c.D, 2 * c.k)));
    return WM_OK;
  }

  // -------------------------------------------------------- feedback-free channel
  // Channel l of the step's rows from their states 0..l (S[0..l] in place):
  // row scale of state l, its block of the gained router input when it is a
  // router layer (l % p == 0), router weights of sources 0..l for channel l
  // (router rows src*k + l over the first l/p + 1 input blocks), mix,
  // channel norm, K/V projection and append into cache channel l.
  wm_status ff_channel(int l, const T *S, wm_tokset ts) {
    const int rows = ts.B * ts.M, D = c.D, Nl = l + 1, Rl = l / c.p + 1, Lk = c.L * c.k;
    const int64_t RD = (int64_t)R * D, HD = (int64_t)c.Hkv * c.d;
    {
      ProfScope prof(WM_K_MIX, s);
      hipLaunchKernelGGL((state_rinv<T>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                         S + (int64_t)l * rows * D, at<float>(lay.rinvS) + (int64_t)l * rows, (int64_t)rows, D, c.eps);
      WM_TRY(hipGetLastError());
      if (l % c.p == 0) {
        hipLaunchKernelGGL((router_input<T>), dim3(rows, 2), dim3(256), 0, s, S, at<float>(lay.rinvS), w->src_norm,
                           at<T>(lay.u), rows, c.L, c.p, R, D, l / c.p, l / c.p + 1);
        WM_TRY(hipGetLastError());
      }
    }
    float *Aw = at<float>(lay.Aw);
    {
      ProfScope prof(WM_K_ROUTER, s);
      LoadRows<T> ua{at<T>(lay.u), RD, (int64_t)rows * RD, nullptr};
      BRows<T> rb{LoadRows<T>{(const T *)w->router + (int64_t)l * RD, (int64_t)c.k * RD, (int64_t)Lk * RD, nullptr}};
      EpiStoreF32 re{Aw, Nl, (int64_t)rows * Nl, nullptr, nullptr, nullptr, 0, 0.f, 0.f};
      WM_TRY((gemm1(ua, rb, re, rows, Nl, Rl * D, 2)));
    }
    {
      ProfScope prof(WM_K_MIX, s);
      wm_status st = mix_g<4>(S, rows, RouterOut{1, 0, (int64_t)rows * Nl, Nl}, Aw, Nl, 1,
                              w->chan_norm + (int64_t)l * D);
      if (st != WM_OK) return st;
    }
    const T *wkl = (const T *)w->wk + (int64_t)l * HD * D, *wvl = (const T *)w->wv + (int64_t)l * HD * D;
    EpiKV<T> pe{Kch(l), Vch(l), at<float>(lay.rinvM), w->k_norm + (int64_t)l * c.d, w->rope_cos, w->rope_sin, 1,
                cache->B, c.Hkv, c.T_max, c.d, rows, c.eps, rowpos(ts)};
    ProfScope prof(WM_K_KVPROJ, s);
    if constexpr (kBig) {
      if (big(rows)) {
        WM_TRY((launch_gemm2(PRows<T>{at<T>(lay.mb), D, (int64_t)rows * D, rows},
                             PKV<T>{wkl, wvl, D, HD * D, 1, (int)HD}, pe, rows, (int)HD, D, 2, s)));
        return WM_OK;
      }
    }
    WM_TRY((gemm1(LoadRows<T>{at<T>(lay.mb), D, (int64_t)rows * D, nullptr}, BKV<T>{wkl, wvl, D, HD * D, 1}, pe,
                  rows, (int)HD, D, 2)));
    return WM_OK;
  }

  // -------------------------------------------------------- one group step
  // Rows of ts; row r = b*M + m takes token tokens[b*tstride + toff + m*tstep].
  // logit_mode 0: none; 1: row m_sel of every sequence -> logits[b]; 2: all
  // rows -> logits[b*T + pos].
  wm_status group_step(const int32_t *tokens, int tstride, int toff, int tstep, wm_tokset ts, int logit_mode,
                       int m_sel, int Tseq, float *logits) {
    const int rows = ts.B * ts.M, D = c.D, L = c.L, QD = c.Hq * c.d;
    const float invD = 1.0f / D;
    float *h = at<float>(lay.h), *ss = at<float>(lay.ss);
    T *hb = at<T>(lay.hb), *q = at<T>(lay.q), *o = at<T>(lay.o), *act = at<T>(lay.act), *S = at<T>(lay.S);
    const T *wq = (const T *)w->wq, *wo = (const T *)w->wo, *wg = (const T *)w->w_gate, *wu = (const T *)w->w_up,
            *wd = (const T *)w->w_down;
    const RowPos rp = rowpos(ts);
    // (the LM head's row lists are written by the embedding launch)
    const int nlog = logit_mode == 1 ? ts.B : rows;
    int *rin = at<int>(lay.rowmap), *rout = rin + rows;
    const RowMap rmap{logit_mode ? rin : nullptr, rout, nlog, logit_mode, m_sel, Tseq, ts.s0, ts.s_step};
    {
    ProfScope prof(WM_K_EMBED, s);
    hipLaunchKernelGGL((embed_rows<T>), dim3(rows), dim3(256), 0, s, tokens, (const T *)w->embed, w->attn_norm, h, hb,
                       S, ss, ts.M, tstride, toff, tstep, c.V, D, rmap);
    WM_TRY(hipGetLastError());
    }
    int nparts = 1;
    for (int l = 0; l < L; ++l) {
      // q = RoPE(qnorm(W_Q RMSNorm(h)))
      {
        LoadRows<T> a{hb, D, 0, nullptr};
        BRows<T> b{LoadRows<T>{wq + (int64_t)l * QD * D, D, 0, nullptr}};
        EpiQ<T> e{q, ss, nparts, invD, c.eps, w->q_norm + (int64_t)l * c.d, w->rope_cos, w->rope_sin, c.d, rp};
        ProfScope prof(WM_K_QPROJ, s);
        if (big(rows)) {
          WM_TRY(gemm2_rows(hb, D, wq + (int64_t)l * QD * D, D, e, rows, QD, D));
        } else if (rows <= kFewRows && c.d == 128) {
          // (128-dim heads, few rows: the product on narrow tiles into a raw
          // buffer, then the q epilogue; the attention partials' region is
          // free until the attention below)
          float *qraw = at<float>(lay.part_o);
          EpiStoreF32 er{qraw, QD, 0, nullptr, nullptr, nullptr, 0, 0.f, 0.f};
          WM_TRY((gemm_s(a, b, er, rows, QD, D)));
          hipLaunchKernelGGL((q_epi128<T>), dim3((unsigned)((rows * c.Hq + 3) / 4)), dim3(256), 0, s, qraw, q, ss,
                             nparts, invD, c.eps, w->q_norm + (int64_t)l * c.d, w->rope_cos, w->rope_sin, rp, rows,
                             c.Hq);
          WM_TRY(hipGetLastError());
        } else {
          WM_TRY((gemm_s(a, b, e, rows, QD, D)));
        }
      }
      if (vanilla) {
        // K/V of the step's rows for layer l, written before the attention
        const int hd = c.Hkv * c.d;
        const T *wkl = (const T *)w->wk + (int64_t)l * hd * D, *wvl = (const T *)w->wv + (int64_t)l * hd * D;
        EpiKVL<T> e{Kch(l), Vch(l), ss, nparts, invD, c.eps, w->k_norm + (int64_t)l * c.d, w->rope_cos, w->rope_sin,
                    c.Hkv, c.d, c.T_max, rp};
        ProfScope prof(WM_K_KVPROJ, s);
        bool done = false;
        if constexpr (kBig) {
          if (big(rows)) {
            WM_TRY((launch_gemm2(PRows<T>{hb, D, 0, rows}, PKVL<T>{wkl, wvl, D, hd, 2 * hd}, e, rows, 2 * hd, D, 1, s)));
            done = true;
          }
        }
        if (!done) WM_TRY((gemm_s(LoadRows<T>{hb, D, 0, nullptr}, BKVL<T>{wkl, wvl, D, hd}, e, rows, 2 * hd, D)));
      }
      if (ff) {
        wm_status st = ff_channel(l, S, ts);
        if (st != WM_OK) return st;
      }
      // (vanilla: keys s <= i, i.e. the strict mask one position further)
      wm_tokset tsa = ts;
      if (vanilla) tsa.s0 += 1;
      wm_status st = attn(l, q, tsa, o);
      if (st != WM_OK) return st;
      // h += W_O o; hb = h * ffn_norm
      {
        LoadRows<T> a{o, QD, 0, nullptr};
        BRows<T> b{LoadRows<T>{wo + (int64_t)l * D * QD, QD, 0, nullptr}};
        EpiResid<T> e{h, hb, w->ffn_norm + (int64_t)l * D, nullptr, ss, parts(rows, D, QD)};
        ProfScope prof(WM_K_OPROJ, s);
        if (big(rows))
          WM_TRY(gemm2_resid(o, QD, wo + (int64_t)l * D * QD, QD, e, rows, D, QD));
        else
          WM_TRY((gemm_s(a, b, e, rows, D, QD)));
        nparts = parts(rows, D, QD);
      }
      // act = silu(W_gate b) * (W_up b), b = RMSNorm(h)
      {
        LoadRows<T> a{hb, D, 0, nullptr};
        BGateUp<T> b{LoadGateUp<T>{wg + (int64_t)l * c.F * D, wu + (int64_t)l * c.F * D, D, c.F}};
        EpiSwiGLU<T> e{act, ss, nparts, invD, c.eps, c.F};
        ProfScope prof(WM_K_GATEUP, s);
        bool done = false;
        if constexpr (kBig) {
          if (big(rows)) {
            PRows<T> a2{hb, D, 0, rows};
            PGateUp<T> b2{wg + (int64_t)l * c.F * D, wu + (int64_t)l * c.F * D, D, c.F};
            WM_TRY((launch_gemm2<G2KB, G2ST, 2, kGUShape>(a2, b2, e, rows, 2 * c.F, D, 1, s)));
            done = true;
          }
        }
        if (!done && rows <= kFewRows) {
          FGateUp<T> bf{wg + (int64_t)l * c.F * D, wu + (int64_t)l * c.F * D, D, c.F, 0};
          WM_TRY((launch_few<T>(a, bf, e, rows, 2 * c.F, D, 1, s)));
        } else if (!done) {
          WM_TRY((launch_gemm<T>(a, b, e, rows, 2 * c.F, D, 1, s)));
        }
      }
      // h += W_down act; next state, next norm operand
      {
        LoadRows<T> a{act, c.F, 0, nullptr};
        BRows<T> b{LoadRows<T>{wd + (int64_t)l * D * c.F, c.F, 0, nullptr}};
        const float *gnext = l + 1 < L ? w->attn_norm + (int64_t)(l + 1) * D : w->final_norm;
        T *Snext = l + 1 < L && !vanilla ? S + (int64_t)(l + 1) * rows * D : nullptr;
        EpiResid<T> e{h, hb, gnext, Snext, ss, parts(rows, D, c.F)};
        ProfScope prof(WM_K_DOWN, s);
        if (big(rows))
          WM_TRY(gemm2_resid(act, c.F, wd + (int64_t)l * D * c.F, c.F, e, rows, D, c.F));
        else
          WM_TRY((gemm_s(a, b, e, rows, D, c.F)));
      }
      nparts = parts(rows, D, c.F);
    }
    if (!vanilla && !ff) {
      wm_status st = pool(S, ts);
      if (st != WM_OK) return st;
    }
    if (logit_mode) {
      const int n = nlog;
      LoadRows<T> a{hb, D, 0, rin};
      BRows<T> b{LoadRows<T>{(const T *)w->lm_head, D, 0, nullptr}};
      EpiStoreF32 e{logits, c.V, 0, rout, ss, rin, nparts, invD, c.eps};
      ProfScope prof(WM_K_LMHEAD, s);
      WM_TRY((gemm_s(a, b, e, n, c.V, D)));
    }
    return WM_OK;
  }
};

static bool weights_ok(const wm_weights *w, bool stack) {
  if (!w) return false;
  // (static mixing: constant weights instead of the router)
  bool pool = w->src_norm && (w->router || w->static_mix) && w->chan_norm && w->wk && w->wv && w->k_norm &&
              w->rope_cos && w->rope_sin;
  if (!stack) return pool;
  return pool && w->embed && w->lm_head && w->final_norm && w->attn_norm && w->wq && w->q_norm && w->wo &&
         w->ffn_norm && w->w_gate && w->w_up && w->w_down;
}

static bool vanilla_weights_ok(const wm_weights *w) {
  return w && w->embed && w->lm_head && w->final_norm && w->attn_norm && w->wq && w->q_norm && w->wo && w->ffn_norm &&
         w->w_gate && w->w_up && w->w_down && w->wk && w->wv && w->k_norm && w->rope_cos && w->rope_sin;
}

static wm_status check_common(const wm_config *cfg, const wm_cache *cache, void *ws, size_t ws_bytes, int rows) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  WM_CHECK(cache && cache->k && cache->v, WM_ERR_ARG, "cache or its k/v pointer is NULL");
  WM_CHECK(cache->B >= 1, WM_ERR_SHAPE, "cache->B = %d must be >= 1", cache->B);
  WM_CHECK(rows >= 1, WM_ERR_SHAPE, "no rows to process");
  size_t need = ws_layout(*cfg, rows).total;
  WM_CHECK(ws && ws_bytes >= need, WM_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for %d rows", ws_bytes, need,
           rows);
  return WM_OK;
}

static wm_status check_tokset(const wm_config *cfg, const wm_cache *cache, wm_tokset ts, int64_t pos_limit) {
  WM_CHECK(ts.B >= 1 && ts.B <= cache->B, WM_ERR_SHAPE, "token set B = %d outside [1, cache->B = %d]", ts.B,
           cache->B);
  WM_CHECK(ts.M >= 1, WM_ERR_SHAPE, "token set M = %d must be >= 1", ts.M);
  WM_CHECK(ts.s0 >= 0 && (ts.M == 1 || ts.s_step >= 1), WM_ERR_RANGE, "token set s0 = %d / step = %d invalid", ts.s0,
           ts.s_step);
  int64_t last = (int64_t)ts.s0 + (int64_t)(ts.M - 1) * (ts.M == 1 ? 0 : ts.s_step);
  WM_CHECK(last <= pos_limit, WM_ERR_RANGE, "last position %lld beyond %lld", (long long)last, (long long)pos_limit);
  return WM_OK;
}

template <typename T>
static wm_status prefill_impl(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int Tseq, int g,
                              const wm_cache *cache, float *logits, int mode, void *ws, int rows, hipStream_t s) {
  Run<T> r(*cfg, w, cache, ws, rows, s);
  wm_status pst = r.prep_router();
  if (pst != WM_OK) return pst;
  const int B = cache->B, ng = g < Tseq ? g : Tseq;
  for (int q = 0; q < ng; ++q) {
    int Mq = (Tseq - q + g - 1) / g;
    wm_tokset ts{B, Mq, q, g};
    int lm = 0, msel = 0;
    if (mode == 2) lm = 2;
    if (mode == 1 && (Tseq - 1) % g == q) {
      lm = 1;
      msel = (Tseq - 1 - q) / g;
    }
    wm_status st = r.group_step(tokens, Tseq, q, g, ts, lm, msel, Tseq, logits);
    if (st != WM_OK) return st;
  }
  return WM_OK;
}

// The vanilla comparison model over positions [0, T): steps of `chunk`
// consecutive positions in order, each appending its K/V before attending.
template <typename T>
static wm_status chunked_prefill_impl(bool vanilla, const wm_config *cfg, const wm_weights *w, const int32_t *tokens,
                                      int Tseq, int chunk, const wm_cache *cache, float *logits, int mode, void *ws,
                                      int rows, hipStream_t s) {
  Run<T> r(*cfg, w, cache, ws, rows, s);
  r.vanilla = vanilla;
  r.ff = !vanilla;
  const int B = cache->B;
  for (int p0 = 0; p0 < Tseq; p0 += chunk) {
    const int Mc = Tseq - p0 < chunk ? Tseq - p0 : chunk;
    wm_tokset ts{B, Mc, p0, 1};
    int lm = mode == 2 ? 2 : 0, msel = 0;
    if (mode == 1 && Tseq - 1 < p0 + Mc) {
      lm = 1;
      msel = Tseq - 1 - p0;
    }
    wm_status st = r.group_step(tokens, Tseq, p0, 1, ts, lm, msel, Tseq, logits);
    if (st != WM_OK) return st;
  }
  return WM_OK;
}

// ------------------------------------------------ allocation-free decode step
// Scratch of wm_decode_step_static: a static device array, one copy per GPU
// (each device holds it from the library's load until the process ends).  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address reaches a kernel.  No
// kernel of the decode path reads a scratch element before writing it in the
// same call, so nothing is cleared between calls.
static __device__ __align__(256) unsigned char scratch[WM_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device.
static wm_status scratch_address(void **out) {
  int dev = -1;
  WM_TRY(hipGetDevice(&dev));
  WM_CHECK(dev >= 0 && dev < kMaxDevices, WM_ERR_ARG, "device index %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    WM_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    WM_CHECK(p != nullptr, WM_ERR_HIP, "hipGetSymbolAddress returned NULL for the static scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WM_OK;
}

}  // namespace wm

using namespace wm;

extern "C" {

wm_status wm_rope_table(const wm_config *cfg, float *cosT, float *sinT, wm_stream stream) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  WM_CHECK(cosT && sinT, WM_ERR_ARG, "rope table pointer is NULL");
  int half = cfg->d / 2;
  int64_t n = (int64_t)cfg->T_max * half;
  hipLaunchKernelGGL(rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, cosT, sinT,
                     cfg->T_max, half, (double)cfg->rope_base, cfg->d);
  WM_TRY(hipGetLastError());
  return WM_OK;
}

wm_status wm_mix_kv(const wm_config *cfg, const wm_weights *w, const void *states, wm_tokset ts, const wm_cache *cache,
                    void *ws, size_t ws_bytes, wm_stream stream) {
  WM_CHECK(cfg, WM_ERR_ARG, "config is NULL");
  wm_status st = check_common(cfg, cache, ws, ws_bytes, ts.B * ts.M);
  if (st != WM_OK) return st;
  WM_CHECK(weights_ok(w, false) && states, WM_ERR_ARG, "a pool weight, the rope table or states is NULL");
  st = check_tokset(cfg, cache, ts, (int64_t)cfg->T_max - 1);
  if (st != WM_OK) return st;
  if (ts.M == 1) ts.s_step = 1;
  int rows = ts.B * ts.M;
  if (cfg->dtype == WM_BF16) {
    Run<bf16> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
    st = r.prep_router();
    return st != WM_OK ? st : r.pool((const bf16 *)states, ts);
  }
  Run<float> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
  st = r.prep_router();
  return st != WM_OK ? st : r.pool((const float *)states, ts);
}

wm_status wm_channel_attn(const wm_config *cfg, int32_t layer, const void *q, wm_tokset ts, const wm_cache *cache,
                          void *out, void *ws, size_t ws_bytes, wm_stream stream) {
  WM_CHECK(cfg, WM_ERR_ARG, "config is NULL");
  wm_status st = check_common(cfg, cache, ws, ws_bytes, ts.B * ts.M);
  if (st != WM_OK) return st;
  WM_CHECK(q && out, WM_ERR_ARG, "q or out is NULL");
  WM_CHECK(layer >= 0 && layer < cfg->L, WM_ERR_RANGE, "layer %d outside [0, L = %d)", layer, cfg->L);
  st = check_tokset(cfg, cache, ts, cfg->T_max);
  if (st != WM_OK) return st;
  if (ts.M == 1) ts.s_step = 1;
  int rows = ts.B * ts.M;
  if (cfg->dtype == WM_BF16) {
    Run<bf16> r(*cfg, nullptr, cache, ws, rows, (hipStream_t)stream);
    return r.attn(layer, (const bf16 *)q, ts, (bf16 *)out);
  }
  Run<float> r(*cfg, nullptr, cache, ws, rows, (hipStream_t)stream);
  return r.attn(layer, (const float *)q, ts, (float *)out);
}

wm_status wm_cyclic_prefill_pass(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t T,
                                 int32_t g, const wm_cache *cache, float *logits, int32_t logits_mode, void *ws,
                                 size_t ws_bytes, wm_stream stream) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  WM_CHECK(cache && cache->k && cache->v && cache->B >= 1, WM_ERR_ARG, "cache, its pointers or B invalid");
  WM_CHECK(g >= 1, WM_ERR_SHAPE, "g = %d must be >= 1", g);
  WM_CHECK(T >= 1 && T <= cfg->T_max, WM_ERR_RANGE, "T = %d outside [1, T_max = %d]", T, cfg->T_max);
  WM_CHECK(logits_mode >= 0 && logits_mode <= 2, WM_ERR_ARG, "logits_mode %d not in {0, 1, 2}", logits_mode);
  WM_CHECK(logits_mode == 0 || logits, WM_ERR_ARG, "logits is NULL but logits_mode = %d", logits_mode);
  WM_CHECK(tokens && weights_ok(w, true), WM_ERR_ARG, "tokens or a weight pointer is NULL");
  int rows = cache->B * ((T + g - 1) / g);
  st = check_common(cfg, cache, ws, ws_bytes, rows);
  if (st != WM_OK) return st;
  if (cfg->dtype == WM_BF16)
    return prefill_impl<bf16>(cfg, w, tokens, T, g, cache, logits, logits_mode, ws, rows, (hipStream_t)stream);
  return prefill_impl<float>(cfg, w, tokens, T, g, cache, logits, logits_mode, ws, rows, (hipStream_t)stream);
}

wm_status wm_decode_step(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t t,
                         const wm_cache *cache, float *logits, void *ws, size_t ws_bytes, wm_stream stream) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  WM_CHECK(cache && cache->k && cache->v && cache->B >= 1, WM_ERR_ARG, "cache, its pointers or B invalid");
  WM_CHECK(t >= 0 && t < cfg->T_max, WM_ERR_RANGE, "t = %d outside [0, T_max = %d)", t, cfg->T_max);
  WM_CHECK(tokens && logits && weights_ok(w, true), WM_ERR_ARG, "tokens, logits or a weight pointer is NULL");
  int rows = cache->B;
  st = check_common(cfg, cache, ws, ws_bytes, rows);
  if (st != WM_OK) return st;
  wm_tokset ts{cache->B, 1, t, 1};
  // (more than kFewRows sequences: the pool reads the gain-folded router
  // weights, which prep_router writes into the workspace)
  if (cfg->dtype == WM_BF16) {
    Run<bf16> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
    st = r.prep_router();
    if (st != WM_OK) return st;
    return r.group_step(tokens, 1, 0, 0, ts, 1, 0, 1, logits);
  }
  Run<float> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
  st = r.prep_router();
  if (st != WM_OK) return st;
  return r.group_step(tokens, 1, 0, 0, ts, 1, 0, 1, logits);
}

wm_status wm_decode_step_at(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, const int32_t *t,
                            const wm_cache *cache, float *logits, void *ws, size_t ws_bytes, wm_stream stream) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  WM_CHECK(cache && cache->k && cache->v && cache->B >= 1, WM_ERR_ARG, "cache, its pointers or B invalid");
  WM_CHECK(t && tokens && logits && weights_ok(w, true), WM_ERR_ARG,
           "t, tokens, logits or a weight pointer is NULL");
  int rows = cache->B;
  st = check_common(cfg, cache, ws, ws_bytes, rows);
  if (st != WM_OK) return st;
  // (host-side choices that depend on the position, the key splits of the
  // attention, are made for the last position; the kernels read *t)
  wm_tokset ts{cache->B, 1, cfg->T_max - 1, 1};
  if (cfg->dtype == WM_BF16) {
    Run<bf16> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
    r.pos_dev = t;
    st = r.prep_router();
    if (st != WM_OK) return st;
    return r.group_step(tokens, 1, 0, 0, ts, 1, 0, 1, logits);
  }
  Run<float> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
  r.pos_dev = t;
  st = r.prep_router();
  if (st != WM_OK) return st;
  return r.group_step(tokens, 1, 0, 0, ts, 1, 0, 1, logits);
}

wm_status wm_decode_step_static(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t t,
                                const wm_cache *cache, float *logits, wm_stream stream) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  WM_CHECK(cache && cache->k && cache->v && cache->B >= 1, WM_ERR_ARG, "cache, its pointers or B invalid");
  WM_CHECK(t >= 0 && t < cfg->T_max, WM_ERR_RANGE, "t = %d outside [0, T_max = %d)", t, cfg->T_max);
  WM_CHECK(tokens && logits && weights_ok(w, true), WM_ERR_ARG, "tokens, logits or a weight pointer is NULL");
  const size_t need = ws_layout(*cfg, cache->B).total;
  WM_CHECK(need <= (size_t)WM_STATIC_SCRATCH_BYTES, WM_ERR_WORKSPACE,
           "a decode step of %d sequences needs %zu bytes of scratch; the static scratch holds %zu", cache->B, need,
           (size_t)WM_STATIC_SCRATCH_BYTES);
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != WM_OK) return st;
  return wm_decode_step(cfg, w, tokens, t, cache, logits, ws, need, stream);
}

wm_status wm_vanilla_prefill(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t T,
                             int32_t chunk, const wm_cache *cache, float *logits, int32_t logits_mode, void *ws,
                             size_t ws_bytes, wm_stream stream) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  WM_CHECK(cfg->k == cfg->L, WM_ERR_SHAPE, "the vanilla model needs one cache slot per layer: k = %d, L = %d",
           cfg->k, cfg->L);
  WM_CHECK(cache && cache->k && cache->v && cache->B >= 1, WM_ERR_ARG, "cache, its pointers or B invalid");
  WM_CHECK(chunk >= 1, WM_ERR_SHAPE, "chunk = %d must be >= 1", chunk);
  WM_CHECK(T >= 1 && T <= cfg->T_max, WM_ERR_RANGE, "T = %d outside [1, T_max = %d]", T, cfg->T_max);
  WM_CHECK(logits_mode >= 0 && logits_mode <= 2, WM_ERR_ARG, "logits_mode %d not in {0, 1, 2}", logits_mode);
  WM_CHECK(logits_mode == 0 || logits, WM_ERR_ARG, "logits is NULL but logits_mode = %d", logits_mode);
  WM_CHECK(tokens && vanilla_weights_ok(w), WM_ERR_ARG, "tokens or a weight pointer is NULL");
  const int rows = cache->B * (chunk < T ? chunk : T);
  st = check_common(cfg, cache, ws, ws_bytes, rows);
  if (st != WM_OK) return st;
  if (cfg->dtype == WM_BF16)
    return chunked_prefill_impl<bf16>(true, cfg, w, tokens, T, chunk, cache, logits, logits_mode, ws, rows,
                                      (hipStream_t)stream);
  return chunked_prefill_impl<float>(true, cfg, w, tokens, T, chunk, cache, logits, logits_mode, ws, rows,
                                     (hipStream_t)stream);
}

wm_status wm_vanilla_decode_step(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t t,
                                 const wm_cache *cache, float *logits, void *ws, size_t ws_bytes, wm_stream stream) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  WM_CHECK(cfg->k == cfg->L, WM_ERR_SHAPE, "the vanilla model needs one cache slot per layer: k = %d, L = %d",
           cfg->k, cfg->L);
  WM_CHECK(cache && cache->k && cache->v && cache->B >= 1, WM_ERR_ARG, "cache, its pointers or B invalid");
  WM_CHECK(t >= 0 && t < cfg->T_max, WM_ERR_RANGE, "t = %d outside [0, T_max = %d)", t, cfg->T_max);
  WM_CHECK(tokens && logits && vanilla_weights_ok(w), WM_ERR_ARG, "tokens, logits or a weight pointer is NULL");
  const int rows = cache->B;
  st = check_common(cfg, cache, ws, ws_bytes, rows);
  if (st != WM_OK) return st;
  wm_tokset ts{cache->B, 1, t, 1};
  if (cfg->dtype == WM_BF16) {
    Run<bf16> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
    r.vanilla = true;
    return r.group_step(tokens, 1, 0, 0, ts, 1, 0, 1, logits);
  }
  Run<float> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
  r.vanilla = true;
  return r.group_step(tokens, 1, 0, 0, ts, 1, 0, 1, logits);
}

static wm_status ff_checks(const wm_config *cfg, const wm_weights *w, const wm_cache *cache) {
  wm_status st = wm_check_config(cfg);
  if (st != WM_OK) return st;
  WM_CHECK(cfg->k == cfg->L, WM_ERR_SHAPE, "the feedback-free model has one channel per layer: k = %d, L = %d",
           cfg->k, cfg->L);
  WM_CHECK(cache && cache->k && cache->v && cache->B >= 1, WM_ERR_ARG, "cache, its pointers or B invalid");
  WM_CHECK(w && w->router && !w->static_mix, WM_ERR_ARG,
           "the feedback-free model needs the router (and no static mixing weights)");
  return WM_OK;
}

wm_status wm_feedback_free_prefill(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t T,
                                   int32_t chunk, const wm_cache *cache, float *logits, int32_t logits_mode,
                                   void *ws, size_t ws_bytes, wm_stream stream) {
  wm_status st = ff_checks(cfg, w, cache);
  if (st != WM_OK) return st;
  WM_CHECK(chunk >= 1, WM_ERR_SHAPE, "chunk = %d must be >= 1", chunk);
  WM_CHECK(T >= 1 && T <= cfg->T_max, WM_ERR_RANGE, "T = %d outside [1, T_max = %d]", T, cfg->T_max);
  WM_CHECK(logits_mode >= 0 && logits_mode <= 2, WM_ERR_ARG, "logits_mode %d not in {0, 1, 2}", logits_mode);
  WM_CHECK(logits_mode == 0 || logits, WM_ERR_ARG, "logits is NULL but logits_mode = %d", logits_mode);
  WM_CHECK(tokens && weights_ok(w, true), WM_ERR_ARG, "tokens or a weight pointer is NULL");
  const int rows = cache->B * (chunk < T ? chunk : T);
  st = check_common(cfg, cache, ws, ws_bytes, rows);
  if (st != WM_OK) return st;
  if (cfg->dtype == WM_BF16)
    return chunked_prefill_impl<bf16>(false, cfg, w, tokens, T, chunk, cache, logits, logits_mode, ws, rows,
                                      (hipStream_t)stream);
  return chunked_prefill_impl<float>(false, cfg, w, tokens, T, chunk, cache, logits, logits_mode, ws, rows,
                                     (hipStream_t)stream);
}

wm_status wm_feedback_free_decode_step(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t t,
                                       const wm_cache *cache, float *logits, void *ws, size_t ws_bytes,
                                       wm_stream stream) {
  wm_status st = ff_checks(cfg, w, cache);
  if (st != WM_OK) return st;
  WM_CHECK(t >= 0 && t < cfg->T_max, WM_ERR_RANGE, "t = %d outside [0, T_max = %d)", t, cfg->T_max);
  WM_CHECK(tokens && logits && weights_ok(w, true), WM_ERR_ARG, "tokens, logits or a weight pointer is NULL");
  const int rows = cache->B;
  st = check_common(cfg, cache, ws, ws_bytes, rows);
  if (st != WM_OK) return st;
  wm_tokset ts{cache->B, 1, t, 1};
  if (cfg->dtype == WM_BF16) {
    Run<bf16> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
    r.ff = true;
    return r.group_step(tokens, 1, 0, 0, ts, 1, 0, 1, logits);
  }
  Run<float> r(*cfg, w, cache, ws, rows, (hipStream_t)stream);
  r.ff = true;
  return r.group_step(tokens, 1, 0, 0, ts, 1, 0, 1, logits);
}

wm_status wm_profile_begin(uint32_t kind_mask) {
  g_prof.mask = kind_mask;
  g_prof.used = 0;
  g_prof.recs.clear();
  return WM_OK;
}

wm_status wm_profile_read(int64_t *counts, double *total_ms) {
  WM_CHECK(counts && total_ms, WM_ERR_ARG, "counts or total_ms is NULL");
  for (int i = 0; i < WM_K_COUNT; ++i) {
    counts[i] = 0;
    total_ms[i] = 0.0;
  }
  for (const ProfRec &r : g_prof.recs) {
    WM_TRY(hipEventSynchronize(r.b));
    float ms = 0.f;
    WM_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    counts[r.kind] += 1;
    total_ms[r.kind] += ms;
  }
  return WM_OK;
}

wm_status wm_profile_end(void) {
  g_prof.mask = 0;
  for (hipEvent_t e : g_prof.pool) (void)hipEventDestroy(e);
  g_prof.pool.clear();
  g_prof.used = 0;
  g_prof.recs.clear();
  return WM_OK;
}

}  // extern "C"
