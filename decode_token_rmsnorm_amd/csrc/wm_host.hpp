// wm_host.hpp — host-side shape checks, workspace layout and the error
// string; plain C++ (no HIP), shared by the C ABI entry points.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/wm.h"

namespace wm {

void set_error(const char *fmt, ...);

// Attention partials are kept for at most max(rows, 16384) split-rows.
inline int64_t part_rows_cap(int rows) {
  int64_t c = rows > 16384 ? rows : 16384;
  int64_t m = 16 * (int64_t)rows;
  return c < m ? c : m;
}

// Steps with at most this many rows run their GEMMs on the k-split skinny
// kernel and build the router input explicitly (workspace region u).  That
// kernel gives each block one k slice of this many bytes per row; with more
// than one slice the 64 x 128 fp32 tile of every (tile, slice) goes through
// the workspace region skp.
constexpr int kSkinnyRows = 128;
constexpr int kSkinnySliceBytes = 1024;
inline int skinny_slices(int64_t k_bytes) { return (int)((k_bytes + kSkinnySliceBytes - 1) / kSkinnySliceBytes); }
// Partial tiles (floats) one skinny GEMM [rows, N, K] x Z needs (0 with one slice).
inline size_t skinny_partial_floats(int rows, int N, int64_t k_bytes, int Z) {
  const int S = skinny_slices(k_bytes);
  if (S <= 1) return 0;
  const size_t nM = (size_t)(rows + 63) / 64, nN = (size_t)(N + 127) / 128;
  return (size_t)Z * nM * nN * S * 64 * 128;
}

// Router split-K partials kept for steps with more rows than kSkinnyRows.
constexpr int kRouterMaxSplits = 4;

struct WsLayout {
  size_t h, hb, ss, q, o, act, S, rinvS, Aw, mb, rinvM, u, wf, skp, part_o, part_ml, rowmap, total;
  int ssp;  // partial sums of squares per row
};

inline WsLayout ws_layout(const wm_config &c, int rows) {
  WsLayout w{};
  size_t es = c.dtype == WM_BF16 ? 2 : 4, off = 0, R = (size_t)rows;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  w.ssp = (c.D + 127) / 128;
  size_t qd = (size_t)c.Hq * c.d;
  w.h = take(R * c.D * 4);
  w.hb = take(R * c.D * es);
  w.ss = take(R * w.ssp * 4);
  w.q = take(R * qd * es);
  w.o = take(R * qd * es);
  w.act = take(R * c.F * es);
  w.S = take((size_t)c.L * R * c.D * es);
  w.rinvS = take((size_t)c.L * R * 4);
  w.Aw = take((rows > kSkinnyRows ? (size_t)kRouterMaxSplits : 1) * 2 * R * c.L * c.k * 4);
  w.mb = take(2 * (size_t)c.k * R * c.D * es);
  w.rinvM = take(2 * (size_t)c.k * R * 4);
  const size_t nR = (size_t)(c.L + c.p - 1) / c.p;
  const int sr = rows < kSkinnyRows ? rows : kSkinnyRows;
  // router input: two gained copies of few rows, or one normalised copy
  const size_t urows = 2 * (size_t)sr > R ? 2 * (size_t)sr : R;
  w.u = take(urows * nR * c.D * es);
  w.wf = take(rows > kSkinnyRows ? 2 * (size_t)c.L * c.k * nR * c.D * es : 0);
  {  // the largest split GEMM of a few-row step
    const int64_t D = c.D, F = c.F, QD = (int64_t)c.Hq * c.d, KVD = (int64_t)c.Hkv * c.d, LK = (int64_t)c.L * c.k;
    size_t m = skinny_partial_floats(sr, (int)QD, D * es, 1);
    auto mx = [&](size_t v) { m = v > m ? v : m; };
    mx(skinny_partial_floats(sr, (int)D, QD * es, 1));
    mx(skinny_partial_floats(sr, (int)(2 * F), D * es, 1));
    mx(skinny_partial_floats(sr, (int)D, F * es, 1));
    mx(skinny_partial_floats(sr, (int)LK, (int64_t)nR * D * es, 2));
    mx(skinny_partial_floats(sr, (int)KVD, D * es, 2 * c.k));
    mx(skinny_partial_floats(sr, c.V, D * es, 1));
    w.skp = take(m * 4);
  }
  size_t cap = (size_t)part_rows_cap(rows);
  w.part_o = take(cap * qd * 4);
  w.part_ml = take(cap * c.Hq * 2 * 4);
  w.rowmap = take(2 * R * 4);
  w.total = off;
  return w;
}

}  // namespace wm
