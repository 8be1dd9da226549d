// wm_host.cpp — host-only part of the C ABI: shape checks, the group schedule,
// channel selection, cache and workspace sizes, the thread-local error string.
// Plain C++; callable without a GPU.
#include "wm_host.hpp"

#include <stdarg.h>
#include <stdio.h>

namespace wm {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

}  // namespace wm

using wm::set_error;

extern "C" {

const char *wm_last_error(void) { return wm::g_err; }

wm_status wm_check_config(const wm_config *c) {
  if (!c) {
    set_error("config is NULL");
    return WM_ERR_ARG;
  }
  if (c->dtype != WM_F32 && c->dtype != WM_BF16) {
    set_error("dtype %d is neither WM_F32 nor WM_BF16", c->dtype);
    return WM_ERR_DTYPE;
  }
  if (c->L < 1 || c->L > 32) {
    set_error("L = %d outside [1, 32]", c->L);
    return WM_ERR_SHAPE;
  }
  if (c->k < 1 || c->k > c->L) {
    set_error("k = %d outside [1, L = %d]", c->k, c->L);
    return WM_ERR_SHAPE;
  }
  if (c->p < 1 || c->p > c->L) {
    set_error("p = %d outside [1, L = %d]", c->p, c->L);
    return WM_ERR_SHAPE;
  }
  if (c->Hq < 1 || c->Hkv < 1 || c->Hq % c->Hkv != 0) {
    set_error("Hq = %d must be a positive multiple of Hkv = %d", c->Hq, c->Hkv);
    return WM_ERR_SHAPE;
  }
  if (c->d != 32 && c->d != 64 && c->d != 128) {
    set_error("head dim d = %d not in {32, 64, 128}", c->d);
    return WM_ERR_SHAPE;
  }
  if (c->D < 64 || c->D % 64 || c->F < 64 || c->F % 64 || (c->Hq * c->d) % 64) {
    set_error("D = %d, F = %d and Hq*d = %d must be positive multiples of 64", c->D, c->F, c->Hq * c->d);
    return WM_ERR_SHAPE;
  }
  if (c->V < 1 || c->T_max < 1) {
    set_error("V = %d and T_max = %d must be >= 1", c->V, c->T_max);
    return WM_ERR_SHAPE;
  }
  if (!(c->eps > 0.f) || !(c->rope_base > 1.f)) {
    set_error("eps must be > 0 and rope_base > 1");
    return WM_ERR_ARG;
  }
  return WM_OK;
}

int32_t wm_group_positions(int32_t T, int32_t g, int32_t q, int32_t *out) {
  if (T < 0 || g < 1 || q < 0 || q >= g) return -1;
  int32_t n = 0;
  for (int32_t i = q; i < T; i += g) {
    if (out) out[n] = i;
    ++n;
  }
  return n;
}

int32_t wm_channel_of_layer(int32_t layer, int32_t k) {
  if (k < 1 || layer < 0) return -1;
  return layer % k;
}

int64_t wm_cache_elems(const wm_config *c, int32_t B) {
  if (wm_check_config(c) != WM_OK || B < 1) return -1;
  return (int64_t)c->k * B * c->Hkv * c->T_max * c->d;
}

size_t wm_workspace_bytes(const wm_config *c, int32_t rows) {
  if (wm_check_config(c) != WM_OK || rows < 1) return 0;
  return wm::ws_layout(*c, rows).total;
}

}  // extern "C"
