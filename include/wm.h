/*
 * wm.h — C ABI of the WhiteMatter KV-pool library for MI355X (gfx950).
 *
 * WhiteMatter (arXiv 2608.18486) replaces per-layer K/V projections by a
 * cross-layer KV pool: for each token the L per-layer hidden states are
 * RMSNorm'd, a router that reads every p-th of them emits signed weights for
 * all L layers and k channels, the mixed channels are RMSNorm'd again and
 * projected by per-channel K/V matrices; keys get a per-channel norm and RoPE
 * before they are cached. Consumer layer l attends strictly causally (s < i)
 * to channel l mod k. Sources: the paperlayer.ai summary, §3 Method
 * ("Cross-layer KV pool", "Per-layer channel selection", "Execution
 * schedules"), and the onedev.kr summary, sections "How it works" and "What
 * differs" (order of the pool's steps, G_q groups, strict causality).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host).
 *  - The caller owns and allocates every buffer: weights, caches, workspace,
 *    outputs. The library allocates no device memory (the one exception,
 *    wm_decode_step_static's scratch, is a static array of its code object).
 *  - Compute calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream). Arguments are validated on the host before anything is
 *    launched; on error nothing is launched or written, a negative wm_status
 *    is returned and wm_last_error() holds the reason. A launch failure
 *    returns WM_ERR_HIP; a fault inside a kernel shows at the caller's next
 *    synchronisation of the stream.
 *  - Matrices and state/cache/activation tensors have the element type of
 *    cfg->dtype (WM_F32: float, WM_BF16: bfloat16, bit layout of the upper
 *    half of an IEEE float). Norm gains and RoPE tables are always float.
 *  - Matrices are row-major [out, in]. Index 0 of a leading "2" axis is the
 *    key branch, 1 the value branch.
 *  - Calls that write one cache must not overlap; calls on distinct caches
 *    and workspaces may run concurrently on different streams.
 *
 * Shape limits (checked; WM_ERR_SHAPE otherwise): 1 <= k <= L, 1 <= p <= L,
 * Hq % Hkv == 0, d in {32, 64, 128}, D % 64 == 0, F % 64 == 0,
 * (Hq*d) % 64 == 0, T_max >= 1, V >= 1.
 */
#ifndef WM_H
#define WM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WM_OK = 0,
  WM_ERR_ARG = -1,       /* null pointer or bad enum value                     */
  WM_ERR_SHAPE = -2,     /* shape outside the limits above                     */
  WM_ERR_DTYPE = -3,     /* unknown element type                               */
  WM_ERR_WORKSPACE = -4, /* workspace smaller than wm_workspace_bytes()        */
  WM_ERR_RANGE = -5,     /* a position or index outside the cache / sequence   */
  WM_ERR_HIP = -6        /* a HIP runtime call or launch failed                */
} wm_status;

typedef enum { WM_F32 = 0, WM_BF16 = 1 } wm_dtype;

/* Model shape. R = ceil(L / p) layers (0, p, 2p, ...) feed the router. */
typedef struct {
  int32_t L;      /* layers; also the number of pooled source states        */
  int32_t D;      /* model width                                            */
  int32_t Hq;     /* query heads                                            */
  int32_t Hkv;    /* key/value heads per cache channel                      */
  int32_t d;      /* head dimension                                         */
  int32_t F;      /* SwiGLU hidden width                                    */
  int32_t k;      /* cache channels (k <= L); layer l reads channel l mod k */
  int32_t p;      /* router stride                                          */
  int32_t V;      /* vocabulary                                             */
  int32_t T_max;  /* positions per sequence in the cache                    */
  float eps;      /* RMSNorm epsilon (1e-6)                                 */
  float rope_base;/* RoPE base (1e6)                                        */
  int32_t dtype;  /* wm_dtype                                               */
} wm_config;

/* Parameters (caller-owned, device). Shapes with R = ceil(L/p):
 *   embed [V, D], lm_head [V, D], final_norm [D] (float)
 *   attn_norm [L, D] (float), wq [L, Hq*d, D], q_norm [L, d] (float),
 *   wo [L, D, Hq*d], ffn_norm [L, D] (float), w_gate [L, F, D], w_up [L, F, D],
 *   w_down [L, D, F]
 *   src_norm [2, L, D] (float)   source-state RMSNorm gains per branch/layer
 *   router   [2, L*k, R*D]       row l*k + j = weight of source layer l in
 *                                channel j; column block r = layer r*p
 *   chan_norm [2, k, D] (float)  channel RMSNorm gains
 *   wk [k, Hkv*d, D], wv [k, Hkv*d, D], k_norm [k, d] (float)
 *   rope_cos, rope_sin [T_max, d/2] (float), filled by wm_rope_table().
 *   static_mix [2, L, k] (float), nullable: when set, the static-mixing
 *                                variant runs (paperlayer.ai §5 analysis,
 *                                "Dynamic routing"): every token mixes its
 *                                normalised states with these constant signed
 *                                weights (element (b, l, j) = weight of source
 *                                layer l in channel j of branch b) and the
 *                                router is not read (it may be NULL).      */
typedef struct {
  const void *embed, *lm_head;
  const float *final_norm;
  const float *attn_norm;
  const void *wq;
  const float *q_norm;
  const void *wo;
  const float *ffn_norm;
  const void *w_gate, *w_up, *w_down;
  const float *src_norm;
  const void *router;
  const float *chan_norm;
  const void *wk, *wv;
  const float *k_norm;
  const float *rope_cos, *rope_sin;
  const float *static_mix;
} wm_weights;

/* Shared KV cache: key and value arrays, each [k, B, Hkv, T_max, d] of
 * cfg->dtype. Entry (j, b, h, s, :) is channel j, sequence b, KV head h,
 * position s. Keys are stored after key norm and RoPE, values raw. */
typedef struct {
  void *k;
  void *v;
  int32_t B;
} wm_cache;

/* A set of rows: row r = b*M + m (b < B, m < M) is position s0 + m*s_step of
 * sequence b. A cyclic group G_q is (B, M_q, q, g); a decode step is
 * (B, 1, t, 1). */
typedef struct {
  int32_t B, M, s0, s_step;
} wm_tokset;

typedef void *wm_stream; /* a hipStream_t */

/* ---- host-only helpers (no GPU needed) --------------------------------- */

/* Reason for the last error returned on this thread ("" if none). */
const char *wm_last_error(void);

/* Checks the shape limits listed above. */
wm_status wm_check_config(const wm_config *cfg);

/* G_q = {i in [0, T) : i mod g = q} in ascending order, written to out (host,
 * room for ceil(T/g) entries; may be NULL to only count). Returns |G_q|, or
 * -1 when T < 0, g < 1 or q is outside [0, g). (onedev.kr, "What differs".) */
int32_t wm_group_positions(int32_t T, int32_t g, int32_t q, int32_t *out);

/* Channel read by consumer layer `layer`: layer mod k, or -1 when k < 1 or
 * layer < 0. (paperlayer.ai §3, "Per-layer channel selection".) */
int32_t wm_channel_of_layer(int32_t layer, int32_t k);

/* Elements of ONE of the two caches: k * B * Hkv * T_max * d (k/L of an
 * L-layer cache). -1 on a bad config or B < 1. (paperlayer.ai §3.) */
int64_t wm_cache_elems(const wm_config *cfg, int32_t B);

/* Workspace bytes needed by calls that process at most `rows` rows per group
 * step (rows = B * max_q |G_q| for a prefill pass, B for a decode step,
 * B*M for wm_mix_kv / wm_channel_attn). 0 on a bad config or rows < 1. */
size_t wm_workspace_bytes(const wm_config *cfg, int32_t rows);

/* ---- device entry points ------------------------------------------------ */

/* Fills rope_cos/rope_sin [T_max, d/2] with cos/sin(s * base^(-2m/d)),
 * computed on the device in double and rounded to float. Element m of a
 * head rotates together with element m + d/2. */
wm_status wm_rope_table(const wm_config *cfg, float *rope_cos, float *rope_sin, wm_stream stream);

/* Cross-layer KV pool + append for the rows of `ts` (paperlayer.ai §3
 * "Cross-layer KV pool"; onedev.kr "How it works"): for each branch, RMSNorm
 * each of the L states (src_norm), router over layers 0, p, 2p, ... -> signed
 * [L, k] weights, mix, channel RMSNorm (chan_norm), per-channel projection
 * (wk / wv); keys get a per-head RMSNorm (k_norm) and RoPE at their position.
 * states [L, B*M, D] (cfg->dtype): state l of row r is the input of block l.
 * Writes cache entries (j, b, :, s0 + m*s_step, :) for every j; reads no
 * cache entry. Positions must be < T_max (WM_ERR_RANGE). */
wm_status wm_mix_kv(const wm_config *cfg, const wm_weights *w, const void *states, wm_tokset ts,
                    const wm_cache *cache, void *ws, size_t ws_bytes, wm_stream stream);

/* Strict-causal channel attention of consumer layer `layer` (paperlayer.ai
 * §3 "Per-layer channel selection"; onedev.kr "What differs"): the row at
 * position i, query head h, attends to positions s < i of channel
 * layer mod k, KV head h / (Hq/Hkv), with softmax(q.k / sqrt(d)). A row at
 * position 0 gets 0. q [B*M, Hq, d] is already normed and rotated; out
 * [B*M, Hq*d]. Both cfg->dtype. Positions must be <= T_max. */
wm_status wm_channel_attn(const wm_config *cfg, int32_t layer, const void *q, wm_tokset ts,
                          const wm_cache *cache, void *out, void *ws, size_t ws_bytes,
                          wm_stream stream);

/* One cyclic Gauss-Seidel prefill pass (onedev.kr "What differs";
 * paperlayer.ai §3 "Execution schedules"): for q = 0 .. min(g, T)-1 in order,
 * every token of G_q = {i < T : i mod g = q} of every sequence runs the full
 * L-layer stack against the cache as it stands when the group starts, then
 * the group's pooled K/V are written, so later groups of the same pass read
 * them. g = 1 is a Jacobi pass, g >= T is exact autoregressive execution.
 * tokens [B, T] int32, ids in [0, V): an id outside that range is not read
 * from the embedding; its row becomes NaN, and so does everything computed
 * from it (its cache entries, its logits, and the later positions of its
 * sequence that attend to it). The cache must hold B = cache->B sequences
 * and T <= T_max.
 * logits_mode 0: none (logits may be NULL); 1: logits [B, V] float of
 * position T-1; 2: logits [B, T, V] float of every position. Logits of a
 * position come from its own group step of this pass.
 * Workspace: wm_workspace_bytes(cfg, B * ceil(T/g)). */
wm_status wm_cyclic_prefill_pass(const wm_config *cfg, const wm_weights *w, const int32_t *tokens,
                                 int32_t T, int32_t g, const wm_cache *cache, float *logits,
                                 int32_t logits_mode, void *ws, size_t ws_bytes, wm_stream stream);

/* One decode step (paperlayer.ai §3 "Execution schedules": a token's pooled
 * channels are appended after its own layer stack): the token tokens[b] at
 * position t of every sequence b < cache->B attends to positions s < t,
 * then its K/V are written at slot t. logits [B, V] float. Requires
 * 0 <= t < T_max. tokens [B] int32 in [0, V); an id outside it makes that
 * sequence's logits and appended entries NaN. Workspace:
 * wm_workspace_bytes(cfg, B). */
wm_status wm_decode_step(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t t,
                         const wm_cache *cache, float *logits, void *ws, size_t ws_bytes,
                         wm_stream stream);

/* One decode step whose position is read from device memory when the kernels
 * run (*t, int32) instead of being passed by value; otherwise the step of
 * wm_decode_step (same kernels and arguments). A caller can capture it once
 * into a HIP graph and replay the graph at successive positions, writing the
 * next position and tokens into the same device buffers between replays
 * (paperlayer.ai §3 "Execution schedules": decoding appends one token's
 * channels per step). *t must lie in [0, T_max); the kernels clamp a value
 * outside that range into it. The host cannot read *t, so the attention's
 * key splits are chosen for position T_max - 1 (splits past the position do
 * no work), and results at other positions may differ from wm_decode_step's
 * in the order of the final sums (rounding only). Launches no memset and no
 * host synchronisation. Workspace: wm_workspace_bytes(cfg, B). */
wm_status wm_decode_step_at(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, const int32_t *t,
                            const wm_cache *cache, float *logits, void *ws, size_t ws_bytes, wm_stream stream);

/* ---- allocation-free decode step ---------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * step as wm_decode_step (same arguments, kernels and results), with its
 * scratch taken from a static device array of WM_STATIC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends, instead
 * of a caller workspace.  The caller still owns the weights, the cache, the
 * tokens and the logits.  Returns WM_ERR_WORKSPACE, launching nothing, when
 * wm_workspace_bytes(cfg, cache->B) exceeds WM_STATIC_SCRATCH_BYTES (64 MiB:
 * up to 128 sequences at the 1.3B shape L28 D1792 F4864, up to 256 at
 * L16 D512 F1536).  Calls no
 * allocating routine.  All calls on one GPU share its array, which keeps the
 * last call's contents (no kernel reads an element before writing it in the
 * same call); calls that overlap on one GPU (several streams or threads) race
 * on it and must be serialised by the caller. */
#define WM_STATIC_SCRATCH_BYTES (64u << 20)
wm_status wm_decode_step_static(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t t,
                                const wm_cache *cache, float *logits, wm_stream stream);

/* ---- the vanilla comparison model --------------------------------------
 * The decoder the pages measure WhiteMatter against (paperlayer.ai §3 and
 * onedev.kr "What differs": the per-layer KV cache that the pool replaces):
 * block l projects its own normed input to keys and values with W_K^l, W_V^l
 * (keys: per-head key norm k_norm[l], RoPE) and its queries attend causally
 * to positions s <= i of layer l. It runs on the same kernels; cfg->k must
 * equal cfg->L (WM_ERR_SHAPE otherwise): wk / wv / k_norm hold one entry per
 * layer and the cache one slot per layer (slot l = layer l). Weights used:
 * every stack weight plus wk, wv, k_norm and the RoPE tables (src_norm,
 * router and chan_norm are not read). */

/* One causal pass over positions [0, T) of tokens [B, T] (int32), in steps
 * of `chunk` consecutive positions taken in order; each step appends its
 * keys and values before attending, so every chunk >= 1 gives the same
 * result. logits_mode as for wm_cyclic_prefill_pass. Requires T <= T_max.
 * Workspace: wm_workspace_bytes(cfg, B * min(chunk, T)). */
wm_status wm_vanilla_prefill(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t T,
                             int32_t chunk, const wm_cache *cache, float *logits, int32_t logits_mode, void *ws,
                             size_t ws_bytes, wm_stream stream);

/* One vanilla decode step: the token at position t of every sequence writes
 * its keys and values at slot t of each layer and attends to s <= t.
 * logits [B, V] float. Requires 0 <= t < T_max. Workspace:
 * wm_workspace_bytes(cfg, B). */
wm_status wm_vanilla_decode_step(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t t,
                                 const wm_cache *cache, float *logits, void *ws, size_t ws_bytes,
                                 wm_stream stream);

/* ---- the feedback-free variant -------------------------------------------
 * paperlayer.ai §5 analysis ("Deep-to-shallow feedback") and onedev.kr's
 * ablations: layer l sees only the states 0..l, so there is no deep-to-
 * shallow feedback and no iteration. Reading: cfg->k must equal cfg->L
 * (WM_ERR_SHAPE); consumer layer l reads channel l; channel l of a token
 * mixes its normalised states 0..l with router weights computed from the
 * sampled states r <= l (r = 0, p, 2p, ...) and router rows src*k + l, then
 * channel norm, projection, key norm and RoPE as in wm_mix_kv; attention is
 * strictly causal (s < i). Channel l is appended at layer l, before that
 * layer's attention, so one layer-synchronous pass computes the model. Needs
 * the router; static_mix must be NULL (WM_ERR_ARG). */

/* One pass over positions [0, T) of tokens [B, T] in steps of `chunk`
 * consecutive positions (every chunk >= 1 gives the same result);
 * logits_mode as for wm_cyclic_prefill_pass. Workspace:
 * wm_workspace_bytes(cfg, B * min(chunk, T)). */
wm_status wm_feedback_free_prefill(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t T,
                                   int32_t chunk, const wm_cache *cache, float *logits, int32_t logits_mode,
                                   void *ws, size_t ws_bytes, wm_stream stream);

/* One decode step of the feedback-free model at position t (channels of the
 * token appended at slot t layer by layer; attention to s < t). logits
 * [B, V] float. Requires 0 <= t < T_max. Workspace: wm_workspace_bytes(cfg, B). */
wm_status wm_feedback_free_decode_step(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t t,
                                       const wm_cache *cache, float *logits, void *ws, size_t ws_bytes,
                                       wm_stream stream);

/* ---- training step with truncated backpropagation -----------------------
 * onedev.kr "What differs": in training, gradients flow only through the last
 * n_g passes; "How used": WhiteMatter trains with one cyclic pass without
 * gradients followed by two passes with gradients; paperlayer.ai §3
 * "Execution schedules": training treats the feedback as a fixed-point
 * problem solved by passes.
 *
 * From the zero cache, n_nograd cyclic passes over tokens [B, T] (groups
 * G_q, as wm_cyclic_prefill_pass) run without gradient, then n_grad passes
 * with it. The loss is the mean next-token cross-entropy of the last pass's
 * logits: position i < T-1 of sequence b predicts tokens[b, i+1], over the
 * B*(T-1) predictions. Its gradient with respect to every parameter is
 * written to `grads`, with the cache left by the no-gradient passes held
 * constant; inside the gradient passes it flows through every cache entry a
 * group step reads, back to the group step that wrote it.
 *
 * float32 only: cfg->dtype must be WM_F32 (WM_ERR_DTYPE). The weights are
 * those of wm_weights (float), the RoPE tables included; static_mix must be
 * NULL (WM_ERR_ARG). tokens [B, T] int32 (device), 2 <= T <= T_max
 * (WM_ERR_RANGE), g >= 1, n_nograd >= 0, n_grad >= 1 (WM_ERR_ARG). An id
 * outside [0, V) makes the loss and the gradients NaN. grads: float device
 * buffers of the parameters' shapes, overwritten (not accumulated); *loss is
 * a device float. The cache and every intermediate live in the caller's
 * workspace. wm_train_workspace_bytes(cfg, B, T, g, n_grad) bytes (0 on bad
 * arguments) hold, besides, the intermediates of every gradient group step
 * from the forward passes, so the reverse walk does not recompute them,
 * whenever that total stays within 64 GiB (else it equals the minimum);
 * wm_train_workspace_min_bytes gives the least the step accepts
 * (WM_ERR_WORKSPACE below it), with which it recomputes each gradient step's
 * forward during the reverse walk. Both layouts give bit-identical results.
 * Deterministic: the same inputs give bit-identical results. */
typedef struct {
  float *embed, *lm_head, *final_norm, *attn_norm, *wq, *q_norm, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
  float *src_norm, *router, *chan_norm, *wk, *wv, *k_norm;
} wm_grads;

size_t wm_train_workspace_bytes(const wm_config *cfg, int32_t B, int32_t T, int32_t g, int32_t n_grad);
size_t wm_train_workspace_min_bytes(const wm_config *cfg, int32_t B, int32_t T, int32_t g, int32_t n_grad);
wm_status wm_train_step(const wm_config *cfg, const wm_weights *w, const int32_t *tokens, int32_t B, int32_t T,
                        int32_t g, int32_t n_nograd, int32_t n_grad, const wm_grads *grads, float *loss, void *ws,
                        size_t ws_bytes, wm_stream stream);

/* ---- per-kernel timing (measurement support) ---------------------------
 * Kernel kinds launched by the calls above. */
typedef enum {
  WM_K_QPROJ = 0,   /* query projection + q-norm + RoPE GEMM            */
  WM_K_ATTN = 1,    /* channel attention (and its split combine)        */
  WM_K_OPROJ = 2,   /* output projection + residual GEMM                */
  WM_K_GATEUP = 3,  /* fused gate/up projection + SwiGLU GEMM           */
  WM_K_DOWN = 4,    /* down projection + residual GEMM                  */
  WM_K_ROUTER = 5,  /* pool router GEMM                                 */
  WM_K_MIX = 6,     /* pool mix (and the source-state row norms)        */
  WM_K_KVPROJ = 7,  /* pool K/V projection + key norm + RoPE + append   */
  WM_K_LMHEAD = 8,  /* final norm + LM head GEMM                        */
  WM_K_EMBED = 9,   /* embedding gather                                 */
  WM_K_COUNT = 10
} wm_kernel_kind;

/* While `kind_mask` has bit (1 << kind) set, every launch of that kind on
 * any stream is bracketed by two hipEvents recorded on the same stream.
 * wm_profile_read() synchronises those events and returns, per kind, the
 * launch count and the summed elapsed milliseconds since the last
 * wm_profile_begin(); both arrays (host) have WM_K_COUNT entries. Events are
 * created by the library and kept for reuse until wm_profile_end(). Not
 * thread-safe; intended for benchmarks. */
wm_status wm_profile_begin(uint32_t kind_mask);
wm_status wm_profile_read(int64_t *counts, double *total_ms);
wm_status wm_profile_end(void);

/* ---- device peaks (measurement support) ---------------------------------
 * Not part of the method: what the current device reaches on plain
 * streaming and on dense bf16 MFMA work, so that a kernel's roofline fraction
 * can be stated against a peak measured on the same GPU beside the datasheet
 * figures (8 TB/s HBM, 2.5 PFLOP/s dense bf16 on an MI355X).  Both calls run
 * one untimed launch, then time `iters` (>= 1, WM_ERR_SHAPE otherwise)
 * launches with hipEvents on `stream` and wait for them (the call blocks).
 *
 * wm_peak_stream: reads `bytes` from device buffer `src` and, when `dst` is
 * not NULL, writes them to device buffer `dst` (16-byte chunks, grid-stride,
 * coalesced).  bytes > 0 and a multiple of 16, both buffers 16-byte aligned
 * (WM_ERR_SHAPE otherwise); src and dst must not overlap (WM_ERR_ARG).
 * *gb_per_s (host) = bytes moved per second / 1e9, where a copy moves
 * 2 * bytes (read + write) and a read moves bytes.  The caller owns both
 * buffers; dst's contents become a copy of src.
 *
 * wm_peak_mfma_bf16: two blocks of four waves per compute unit, each wave
 * running 32x32x16 bf16 MFMAs on register-resident operands that keep
 * changing; no memory traffic.  *tflop_per_s (host) = 2*32*32*16 flop per
 * MFMA times MFMAs per second / 1e12. */
wm_status wm_peak_stream(const void *src, void *dst, int64_t bytes, int32_t iters, wm_stream stream,
                         double *gb_per_s);
wm_status wm_peak_mfma_bf16(int32_t iters, wm_stream stream, double *tflop_per_s);

#ifdef __cplusplus
}
#endif

#endif /* WM_H */
