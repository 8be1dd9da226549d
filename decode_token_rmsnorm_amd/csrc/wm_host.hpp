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

// Steps with at most this many rows run their GEMMs on the few-row kernel
// (16-row blocks over the whole k range) and build the router input
// explicitly (workspace region u).
constexpr int kFewRows = 128;
// Partial sums of squares per row: a residual epilogue writes one per output
// tile, and the narrowest tile is 16 columns wide.
constexpr int kMinTileCols = 16;

// Router split-K partials kept for steps with more rows than kFewRows.
constexpr int kRouterMaxSplits = 4;

struct WsLayout {
  size_t h, hb, ss, q, o, act, S, rinvS, Aw, mb, rinvM, u, wf, part_o, part_ml, rowmap, total;
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
  w.ssp = (c.D + kMinTileCols - 1) / kMinTileCols;
  size_t qd = (size_t)c.Hq * c.d;
  w.h = take(R * c.D * 4);
  w.hb = take(R * c.D * es);
  w.ss = take(R * w.ssp * 4);
  w.q = take(R * qd * es);
  w.o = take(R * qd * es);
  w.act = take(R * c.F * es);
  w.S = take((size_t)c.L * R * c.D * es);
  w.rinvS = take((size_t)c.L * R * 4);
  w.Aw = take((rows > kFewRows ? (size_t)kRouterMaxSplits : 1) * 2 * R * c.L * c.k * 4);
  w.mb = take(2 * (size_t)c.k * R * c.D * es);
  w.rinvM = take(2 * (size_t)c.k * R * 4);
  const size_t nR = (size_t)(c.L + c.p - 1) / c.p;
  // router input: two gained copies (few-row steps and the feedback-free
  // variant), or one normalised copy (many rows)
  const size_t urows = 2 * R;
  w.u = take(urows * nR * c.D * es);
  w.wf = take(rows > kFewRows ? 2 * (size_t)c.L * c.k * nR * c.D * es : 0);
  size_t cap = (size_t)part_rows_cap(rows);
  w.part_o = take(cap * qd * 4);
  w.part_ml = take(cap * c.Hq * 2 * 4);
  w.rowmap = take(2 * R * 4);
  w.total = off;
  return w;
}

}  // namespace wm
