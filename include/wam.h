/*
 * wam.h -- C-ABI of the KV-cached action-denoising library (libwam.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (the "Long-WAM", "Fast-WAM" and "Faster-WAM" pages):
 *   1. a video expert fills a per-layer K/V cache once, with block-causal
 *      attention over history latents and future latents that are partially
 *      denoised to sigma* ("Long-WAM: Scaling the Context of World-Action
 *      Models | Summary", section 3.2; Long-WAM code close-reading, section 04);
 *   2. Faster-WAM's Interval KV-Fusion may collapse each depth interval of
 *      video layers into one softmax-weighted K/V pair ("世界模型之Faster-WAM详解",
 *      section 3.3);
 *   3. an action expert runs N flow-matching Euler steps over a 32-token
 *      action chunk; at every step the action queries attend over
 *      [video cache ; action K/V] and video tokens never read actions
 *      ("Fast-WAM 精读", section 七; Long-WAM Summary, section 3.2).
 *
 * Conventions (all calls):
 *   - Every buffer is owned by the caller.  The library never allocates or
 *     frees device memory inside these calls; scratch comes from the caller's
 *     workspace ``ws`` (size from the matching *_workspace_bytes call).
 *   - Device pointers must be 16-byte aligned and contiguous in the layouts
 *     stated below.  Host arrays are read before the call returns.
 *   - Work is enqueued asynchronously on ``stream`` (a hipStream_t passed as
 *     void*, NULL = default stream).  Argument errors are detected on the host
 *     before anything is enqueued; the call then returns a negative status and
 *     enqueues nothing.  ``wam_last_error()`` gives a message (thread-local).
 *   - Matrices are out-major: W[out_features][in_features] (y = x W^T).
 *   - dtype WAM_BF16: weight matrices, latent tokens, noise and K/V are bf16;
 *     residual stream, softmax, accumulators, latents and actions are fp32.
 *     dtype WAM_F32: everything fp32.  RMSNorm gains are always fp32.
 *   - Results are deterministic: identical inputs give bitwise-identical
 *     outputs (no floating-point atomics; split reductions merge in a fixed
 *     order).  Calls on disjoint buffers and workspaces may run concurrently.
 */
#ifndef WAM_H
#define WAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WAM_ABI_VERSION 4
#define WAM_MAX_FRAMES 256   /* latent frames per episode (history + future) */
#define WAM_MAX_BATCH 64     /* episodes per call */
#define WAM_MAX_FUSE 32      /* fused pairs per wam_fuse_interval_kv call */
#define WAM_MAX_INTERVAL 8   /* layers per fusion interval */
#define WAM_MAX_STEPS 64     /* Euler steps per call */

enum {
  WAM_OK = 0,
  WAM_E_ARG = -1,        /* null pointer, bad enum, out-of-range scalar */
  WAM_E_SHAPE = -2,      /* inconsistent or unsupported dimensions */
  WAM_E_DTYPE = -3,      /* dtype mismatch between arguments */
  WAM_E_ALIGN = -4,      /* device pointer not 16-byte aligned */
  WAM_E_WORKSPACE = -5,  /* workspace missing or too small */
  WAM_E_HIP = -6         /* a HIP runtime call failed (see wam_last_error) */
};

/* WAM_FP8 is a K/V cache type only (see wam_quantize_kv_fp8): OCP E4M3 codes
 * with one power-of-two fp32 scale per (layer, episode, head, 64-key tile)
 * for K and one for V.  Every other tensor of a WAM_BF16 model stays bf16. */
enum { WAM_F32 = 0, WAM_BF16 = 1, WAM_FP8 = 2 };

/* Shapes of the two experts.  Layer count, heads and head dim are shared, so
 * that video layer i pairs with action layer i over one attention interface of
 * Hh heads x dh ("Fast-WAM 精读" section 四.4: both branches project to 24 x 128
 * whatever their own widths, 3072 and 1024). */
typedef struct {
  int L;      /* layers per expert */
  int D;      /* video expert width; D == Hh * dh */
  int Hh;     /* attention heads */
  int dh;     /* head dim: 64 or 128 (scores scaled by 1/sqrt(dh)) */
  int Fm;     /* video expert MLP inner width */
  int Cv;     /* channels per video latent token */
  int A;      /* action dims per action token */
  int H;      /* action tokens per chunk; must be 32 */
  int P;      /* tokens per latent frame */
  int dtype;  /* WAM_F32 or WAM_BF16 */
  int Da;     /* action expert width (0: D); its Wqkv is [3 Hh dh][Da], Wo [Da][Hh dh] */
  int Fma;    /* action expert MLP inner width (0: Fm) */
  int rope;   /* 0: no position embedding (C1-C6); 1: rotary option, below */
  int Tc;     /* condition tokens per episode (Tc - 1 text + 1 proprio); 0: none */
  int Ct;     /* condition width (the text encoder's output width), multiple of 64 */
  int S;      /* robot state dims the proprio encoder reads (0: A) */
} wam_dims;

/* Text/state condition (Tc > 0).  The language instruction enters as text
 * tokens of width Ct (the text encoder's output, an input here) and the robot
 * state as one more token of the same width made by a linear layer (the
 * proprio encoder), appended after the text ("Fast-WAM 精读" section 四.5).
 * Video and action tokens read this condition sequence through
 * cross-attention ("Fast-WAM 精读" section 五, step 3): every layer of both
 * experts gains, after its self-attention,
 *   X += Attn(RMSNorm(X; gx) Wqx^T ; K_c, V_c) Wox^T,
 * with K_c, V_c = ctx Wkx^T, ctx Wvx^T per expert layer.  K_c, V_c depend on
 * nothing that changes across denoising steps: wam_prefill_condition_kv
 * computes them once per call (text/state KV reuse, Long-WAM Summary section
 * 4.2) into a wam_kv per expert, which the calls running that expert's
 * layers read through wam_expert_w.cond.  No rotary positions there. */

/* Rotary option (rope = 1).  The pages say only that rotary position tables
 * are computed once per inference call and reused across the denoising steps
 * (Long-WAM Summary section 4.2).  Here, in both experts, every layer rotates
 * Q and K after the projection (K before it is cached): pair j of a head,
 * x[2j] + i x[2j+1], is multiplied by exp(i p w_j), w_j = 10000^(-2j/dh),
 * where p is the token's index in its episode's joint sequence
 * [cached rows in cache order ; the action chunk]: cache row r is at p = r,
 * action token i at p = len[b] + i (i alone where no cache is given).
 * Angles, sines and cosines in float64, rounded to float32 once. */

/* One layer: Y = RMSNorm(X; g1); [Q K V] = Y Wqkv^T; X += Attn Wo^T;
 * X += GELU(RMSNorm(X; g2) W1^T) W2^T.  No biases.  RMSNorm eps = 1e-6. */
typedef struct {
  const float* g1;   /* [D] fp32 */
  const void* wqkv;  /* [3D][D]; rows 0..D-1 = Wq, D..2D-1 = Wk, 2D..3D-1 = Wv */
  const void* wo;    /* [D][D] */
  const float* g2;   /* [D] fp32 */
  const void* w1;    /* [Fm][D] */
  const void* w2;    /* [D][Fm] */
  /* cross-attention to the condition (read only when Tc > 0, else may be NULL) */
  const float* gx;   /* [D] fp32 */
  const void* wqx;   /* [Hh dh][D] */
  const void* wkvx;  /* [2 Hh dh][Ct]: rows 0..Hh dh-1 = Wkx, the rest Wvx */
  const void* wox;   /* [D][Hh dh] */
} wam_layer_w;

/* An expert: X = x W_in^T + emb(sigma); layers; v = RMSNorm(X; g_out) W_out^T.
 * emb(sigma) = [cos(t w_i), sin(t w_i)], t = 1000 sigma, w_i = 10000^(-i/(D/2)).
 * C = Cv for the video expert, A for the action expert. */
struct wam_kv_s;
typedef struct {
  const void* w_in;            /* [D][C] */
  const float* g_out;          /* [D] fp32 */
  const void* w_out;           /* [C][D] */
  const wam_layer_w* layers;   /* host array of n_layers */
  int n_layers;
  /* Tc > 0: this expert's condition K/V for the call (n_layers layers, the
   * call's B episodes, len[b] == Tc), from wam_prefill_condition_kv; NULL
   * without a condition */
  const struct wam_kv_s* cond;
} wam_expert_w;

/* Per-layer K/V cache of B episodes.
 *   k: [n_layers][B][Hh][cap][dh]   (token-major within a head)
 *   v: [n_layers][B][Hh][dh][cap]   (transposed: tokens contiguous)
 * Rows 0..len[b]-1 of episode b are valid: the valid history frames in frame
 * order, then the future frames.  cap must be a multiple of 64.
 * dtype WAM_FP8 (one byte per element; written by wam_quantize_kv_fp8 only):
 *   within each K row, with U = dh/64 and g = 0..3, u = 0..U-1, bytes
 *   16(Ug+u)..+7 hold dims 64u+8g..+7 and bytes 16(Ug+u)+8..+15 dims
 *   64u+32+8g..+7 (dh = 64: bytes 16g.. dims 8g.., bytes 16g+8.. dims
 *   32+8g..); within each 64-key tile of
 *   a V row, bytes 16g..16g+7 hold keys 8g..8g+7 of the tile and bytes
 *   16g+8..16g+15 keys 32+8g..32+8g+7.  k_scale, v_scale: device
 *   [n_layers][B][Hh][cap/64] fp32, each a power of two; a value is
 *   E4M3(code) * scale of its tile.  NULL for the other dtypes. */
typedef struct wam_kv_s {
  void* k;
  void* v;
  int n_layers, B, Hh, dh, cap, dtype;
  int32_t* len;                /* host [B] */
  float* k_scale;
  float* v_scale;
} wam_kv;

/* ---------------------------------------------------------------------------
 * wam_prefill_video_cache -- the video expert's side of one chunk
 * ("prefill_video_cache", Fast-WAM 精读 section 七.1; imagine-then-cache,
 * Long-WAM code close-reading section 04 and Summary section 3.2; one-shot
 * future at video time 1, Faster-WAM section 3.1).
 *
 * Per episode b:
 *   - history frames with hist_valid[b][f] != 0 (all if hist_valid is NULL)
 *     are embedded at sigma = 0 and run through the L layers; a query token
 *     of frame f sees key tokens of valid frames g with
 *     frame_block[g] <= frame_block[f]; each layer's K, V are stored;
 *   - video_steps >= 1: future latents z start at fut_noise and take
 *     video_steps Euler steps over sigma_k = sigma_star + (1 - sigma_star) *
 *     phi(1 - k/video_steps), phi(u) = s u / (1 + (s-1) u) with s = shift,
 *     attending to [history cache ; future] under the same block rule; then
 *     one more pass at sigma_star stores the future K, V;
 *   - video_steps == 0: one pass of the noise at sigma = 1 stores the future
 *     K, V.  Ff == 0: history only.
 * The last layer of a caching pass computes K, V only.  Episodes whose
 * compacted frame tables are equal take their video steps and caching pass
 * together (one launch per product for all their future rows); an episode's
 * results never depend on another episode's inputs.
 *
 *   hist       device [B][Fh][P][Cv] dtype     history / anchor latents
 *   hist_valid host [B][Fh] uint8 or NULL
 *   fut_noise  device [B][Ff][P][Cv] dtype     (may be NULL iff Ff == 0)
 *   frame_block host [Fh + Ff] int32, non-decreasing
 *   cache      device k/v per wam_kv; n_layers == L; cache->len (host) is written
 *   fut_latents_out device [B][Ff][P][Cv] fp32 or NULL: z after the video steps
 *   ws         wam_prefill_workspace_bytes(d, B, Fh, Ff) bytes, 16-byte aligned
 *              (it holds one episode's history rows or all B episodes' future rows)
 * Errors: WAM_E_SHAPE if a frame table is not monotone, an episode has no
 * token at all, or cap is too small.
 * ------------------------------------------------------------------------- */
size_t wam_prefill_workspace_bytes(const wam_dims* d, int B, int Fh, int Ff);
int wam_prefill_video_cache(const wam_dims* d, const wam_expert_w* video,
                            const void* hist, const uint8_t* hist_valid, int B, int Fh,
                            const void* fut_noise, int Ff, const int32_t* frame_block,
                            int video_steps, double sigma_star, double shift,
                            wam_kv* cache, float* fut_latents_out,
                            void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Streaming the history (the observation encoding runs as frames arrive, not
 * when the window is complete: the Long-WAM tutorial section 三, Long-WAM
 * Summary section 4.1).  A decision then costs the new frames and the future
 * instead of the whole window:
 *   1. after a chunk, set cache->len[b] back to the valid history rows (the
 *      future rows are recomputed at every decision);
 *   2. wam_extend_history_cache appends the frames that arrived;
 *   3. wam_prefill_future adds the future rows; then fuse / denoise as usual.
 * The result equals wam_prefill_video_cache over the whole window (the
 * block rule: no frame reads a later block).  Appending is exact only while
 * frames are appended in whole temporal blocks and no frame leaves the
 * window: eviction or a change of the temporal positions invalidates the
 * cached rows (Long-WAM Summary appendix B.2) and needs a new prefill.
 *
 * wam_extend_history_cache -- history frames Fh_old .. Fh_old+Fn-1 (at
 * sigma = 0) through the L layers with keys [cached rows ; new rows] under
 * the block rule; their valid rows are appended to the cache.
 *   hist_new    device [B][Fn][P][Cv] dtype
 *   hist_valid  host [B][Fh_old + Fn] uint8 or NULL (validity of every frame)
 *   frame_block host [Fh_old + Fn], non-decreasing
 *   cache       in: len[b] = valid rows of frames 0..Fh_old-1; out: + new rows
 *   ws          wam_prefill_workspace_bytes(d, B, Fn, 0)
 * Errors: WAM_E_SHAPE if len does not match, if a new valid frame shares a
 * temporal block with a cached frame, or if cap is too small.
 * ------------------------------------------------------------------------- */
int wam_extend_history_cache(const wam_dims* d, const wam_expert_w* video,
                             const void* hist_new, const uint8_t* hist_valid, int B,
                             int Fh_old, int Fn, const int32_t* frame_block, wam_kv* cache,
                             void* ws, size_t ws_bytes, void* stream);

/* wam_prefill_future -- the future part of wam_prefill_video_cache over a
 * cache that holds the valid history rows (len[b] checked): video_steps
 * imagine steps to sigma_star and one caching pass, or (video_steps = 0) one
 * pass of the noise at sigma = 1.  Arguments as wam_prefill_video_cache;
 * Ff >= 1; ws: wam_prefill_workspace_bytes(d, B, 0, Ff). */
int wam_prefill_future(const wam_dims* d, const wam_expert_w* video,
                       const uint8_t* hist_valid, int B, int Fh, const void* fut_noise,
                       int Ff, const int32_t* frame_block, int video_steps,
                       double sigma_star, double shift, wam_kv* cache,
                       float* fut_latents_out, void* ws, size_t ws_bytes, void* stream);

/* Asynchronous execution (Long-WAM Summary section 4.1): of each H-step
 * chunk the first R steps may execute and inference triggers every S control
 * steps, with R/2 <= S < R <= H, leaving an overlap O = R - S.
 * wam_async_check returns WAM_OK or WAM_E_ARG for (H, R, S).
 * wam_async_handoff: a chunk triggered `elapsed` control steps ago is handed
 * over by discarding its first `elapsed` actions and executing the aligned
 * suffix; *first = elapsed, *count = R - elapsed actions of it may run.
 * Returns WAM_E_ARG if (H, R, S) is invalid or elapsed < 0, and WAM_E_SHAPE
 * if elapsed > O: the chunk missed its deadline (T_ready <= O control
 * steps) and the robot has waited. */
int wam_async_check(int H, int R, int S);
int wam_async_handoff(int H, int R, int S, int elapsed, int* first, int* count);

/* ---------------------------------------------------------------------------
 * wam_fuse_interval_kv -- Interval KV-Fusion ("世界模型之Faster-WAM详解",
 * section 3.3): for m < M,
 *   (Kbar_m, Vbar_m) = sum_{j < count[m]} w_{m,j} (K_{start[m]+j}, V_{start[m]+j}),
 *   w_m = softmax(logits[m*logits_stride + 0 .. count[m]-1])   (host, float64;
 *   -INFINITY gives an exact 0 weight).
 * One scalar per (m, j) for K and V, all heads and tokens; fp32 accumulation,
 * output rounded once to the cache dtype.  The fused pair has one layer's
 * length.  dst->n_layers >= M; dst->len is set to src->len.
 * ------------------------------------------------------------------------- */
int wam_fuse_interval_kv(const wam_kv* src, int M, const int32_t* start,
                         const int32_t* count, const float* logits, int logits_stride,
                         wam_kv* dst, void* stream);

/* ---------------------------------------------------------------------------
 * wam_quantize_kv_fp8 -- an option that departs from the pages' bf16 cache
 * (Long-WAM keeps bf16 KV storage, Long-WAM Summary section 4.2; the
 * LongLive-2.0 stack under it quantises its KV cache block by block, the
 * Long-WAM tutorial section 三): the bf16 cache src becomes an E4M3 cache dst
 * that the action layers read (wam_action_layer, wam_denoise_chunk) at half
 * the HBM bytes.
 * For every layer, episode b, head and 64-key tile of rows [0, len[b]) of K,
 * and likewise of V: e = the smallest integer with max|x| <= 448 * 2^e over
 * the tile's valid rows (0 for an all-zero tile), code = E4M3(x / 2^e)
 * rounded to nearest even, scale = 2^e.  Codes of rows >= len[b] in the last
 * tile are 0; later tiles are not written.  dst->len is set to src->len.
 *   src: dtype WAM_BF16; dst: dtype WAM_FP8 with the same n_layers, B, Hh,
 *   dh (64 or 128) and cap, k_scale and v_scale set.
 * ------------------------------------------------------------------------- */
int wam_quantize_kv_fp8(const wam_kv* src, wam_kv* dst, void* stream);

/* ---------------------------------------------------------------------------
 * wam_prefill_condition_kv -- the text/state condition of a call: per
 * episode b the condition sequence ctx_b = [text_b ; state_b Wp^T] (Tc rows of
 * width Ct; the proprio token rounded once to the model dtype), then for every
 * layer l of each given expert K_c, V_c = ctx_b Wkx^T, ctx_b Wvx^T written to
 * rows 0..Tc-1 of that expert's condition cache, len[b] = Tc.
 *   proprio_w  device [Ct][S] dtype      the proprio encoder (S = dims.S or A)
 *   text       device [B][Tc-1][Ct] dtype
 *   state      device [B][S] fp32
 *   video, action   either may be NULL (that side is not computed); the
 *              other arguments are the experts' weights (cond is not read)
 *   cond_video, cond_action  wam_kv of dtype dims.dtype, n_layers == L,
 *              cap >= Tc; NULL where the matching expert is NULL
 *   ws         wam_condition_workspace_bytes(d, B)
 * Errors: WAM_E_SHAPE if Tc == 0 or a cache does not fit.
 * ------------------------------------------------------------------------- */
size_t wam_condition_workspace_bytes(const wam_dims* d, int B);
int wam_prefill_condition_kv(const wam_dims* d, const wam_expert_w* video,
                             const wam_expert_w* action, const void* proprio_w,
                             const void* text, const float* state, int B, wam_kv* cond_video,
                             wam_kv* cond_action, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * wam_action_layer -- one action-expert layer on the chunk, in place
 * (forward_action_with_video_cache for one layer): the B*H action queries of
 * episode b attend over [kv layer kv_layer of episode b ; the chunk's own H
 * keys], or over the chunk alone when kv is NULL (SparseMoT action-only
 * layers, Faster-WAM section 3.2).  No mask among action tokens.
 *   x  device [B][H][D] fp32, updated in place.
 *   cond, cond_layer  with dims.Tc > 0: the action expert's condition cache
 *      and the layer of it this layer reads (cross-attention); else NULL.
 * ------------------------------------------------------------------------- */
size_t wam_action_workspace_bytes(const wam_dims* d, int B, const wam_kv* kv);
int wam_action_layer(const wam_dims* d, const wam_layer_w* w, float* x,
                     const wam_kv* kv, int kv_layer, const wam_kv* cond, int cond_layer,
                     int B, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * wam_flow_euler_step -- x <- x + (sigma_next - sigma) * v, elementwise fp32
 * (the flow path x_sigma = (1-sigma) x + sigma eps has velocity eps - x, Long-WAM
 * code close-reading section 03).  n >= 0; x and v device fp32.
 * ------------------------------------------------------------------------- */
int wam_flow_euler_step(float* x, const float* v, int64_t n, float sigma,
                        float sigma_next, void* stream);

/* ---------------------------------------------------------------------------
 * wam_denoise_chunk -- N Euler steps of the action flow from t=1 to t=0 over
 * t_k = phi(1 - k/N), re-reading the cached video K/V at every step
 * ("Fast-WAM 精读" section 七.2-七.3).  Step k: X = a W_in^T + emb(t_k); layer l
 * reads kv layer read_map[l] (or nothing if read_map[l] < 0); v = head(X);
 * a += (t_{k+1} - t_k) v.
 *   read_map   host [L] int32
 *   eps        device [B][H][A] fp32   initial noise
 *   actions_out device [B][H][A] fp32
 *   vhat_out   device [N][B][H][A] fp32 or NULL
 * kv may be NULL only if every read_map entry is negative.  With a WAM_BF16
 * model kv may be a WAM_FP8 cache (wam_quantize_kv_fp8); the same holds for
 * wam_action_layer.
 * ------------------------------------------------------------------------- */
size_t wam_denoise_workspace_bytes(const wam_dims* d, int B, const wam_kv* kv);
int wam_denoise_chunk(const wam_dims* d, const wam_expert_w* action, const wam_kv* kv,
                      const int32_t* read_map, const float* eps, int B, int N,
                      double shift, float* actions_out, float* vhat_out,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * wam_denoise_chunk_noalloc -- wam_denoise_chunk for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and kernels, but no
 * workspace argument.  Its scratch is a static device array of
 * WAM_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU it
 * runs on until the process ends; the call allocates nothing and frees
 * nothing.  Returns WAM_E_WORKSPACE, before enqueuing anything, when the
 * chunk needs more scratch than that (wam_denoise_workspace_bytes(d, B, kv),
 * e.g. 4 episodes of 16 heads x 64 or one of 24 heads x 128 fit).  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  No part
 * of the scratch needs to start at any value.
 * ------------------------------------------------------------------------- */
#define WAM_NOALLOC_SCRATCH_BYTES (64u << 20)
#define WAM_MAX_DEVICES 64
int wam_denoise_chunk_noalloc(const wam_dims* d, const wam_expert_w* action, const wam_kv* kv,
                              const int32_t* read_map, const float* eps, int B, int N,
                              double shift, float* actions_out, float* vhat_out, void* stream);

/* ---------------------------------------------------------------------------
 * wam_codenoise_chunk -- co-denoising (CoD): the future video latents and the
 * action chunk take N Euler steps together (Long-WAM Summary section 3.2 and
 * Figure 2; the joint call creates and returns both latents, "Fast-WAM 精读"
 * section 03).  Video levels sigma_k = sigma_video_end + (1 - sigma_video_end)
 * phi(1 - k/N), action levels t_k = phi(1 - k/N).  Step k:
 *   1. per episode, z at sigma_k runs through the L video layers with keys
 *      [history rows ; future] under the block rule of wam_prefill_video_cache
 *      (video rows never read actions); every layer writes its future K, V to
 *      cache rows [len_h[b], len_h[b] + Ff*P) and v_video = head(X);
 *   2. the action expert at t_k, layer l attending over cache layer l rows
 *      [0, len_h[b] + Ff*P) (history and the future at sigma_k) and the
 *      chunk's own keys;
 *   3. z += (sigma_{k+1} - sigma_k) v_video, a += (t_{k+1} - t_k) v_action.
 * Step 1 before step 2 is the same as one joint pass over [history ; future ;
 * actions], since video rows read no action token.
 *   cache       in: the history rows only, as wam_prefill_video_cache leaves
 *               them with Ff = 0 (len[b] must equal valid history frames * P);
 *               out: plus the future rows at the last video level, len updated.
 *               n_layers == L; the action layers pair with it densely.
 *   hist_valid  host [B][Fh] uint8 or NULL, frame_block host [Fh + Ff]: the
 *               tables of the history prefill
 *   fut_noise   device [B][Ff][P][Cv] dtype      video noise at sigma_0 = 1
 *   eps         device [B][H][A] fp32            action noise at t_0 = 1
 *   actions_out device [B][H][A] fp32
 *   fut_latents_out device [B][Ff][P][Cv] fp32  (required: holds z during the
 *               call; z at sigma_N on return)
 *   vhat_out    device [N][B][H][A] fp32 or NULL (action velocity per step)
 * Requires Ff >= 1, 1 <= N <= WAM_MAX_STEPS, 0 <= sigma_video_end < 1.
 * ------------------------------------------------------------------------- */
size_t wam_codenoise_workspace_bytes(const wam_dims* d, int B, int Ff, const wam_kv* cache);
int wam_codenoise_chunk(const wam_dims* d, const wam_expert_w* video,
                        const wam_expert_w* action, const uint8_t* hist_valid, int B, int Fh,
                        const void* fut_noise, int Ff, const int32_t* frame_block,
                        const float* eps, int N, double sigma_video_end, double shift,
                        wam_kv* cache, float* actions_out, float* fut_latents_out,
                        float* vhat_out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Auxiliary calls.
 * ------------------------------------------------------------------------- */
int wam_abi_version(void);
const char* wam_status_str(int status);
const char* wam_last_error(void);

/* sigma_k = sigma_end + (1 - sigma_end) * phi(1 - k/steps), k = 0..steps,
 * computed in float64 and rounded to float32 (host only; out has steps+1). */
int wam_schedule(int steps, double sigma_end, double shift, float* out);

/* Host-side frame table of one episode: compacted frames (valid history in
 * order, then future), and for each compacted frame i the end (exclusive,
 * in tokens) of the key prefix its queries see.  src_frame/kend: host
 * [WAM_MAX_FRAMES].  Returns the number of compacted frames or < 0. */
int wam_frame_table(const int32_t* frame_block, const uint8_t* valid, int Fh, int Ff,
                    int P, int32_t* src_frame, int32_t* kend);

/* Visibility matrix evaluated on the GPU by the same predicate the attention
 * kernels use: vis[q][k] (uncompacted tokens, F = Fh + Ff frames of P) is 1
 * iff both tokens are valid and k is visible to q.  vis: device [F*P][F*P]. */
int wam_debug_visibility(const int32_t* frame_block, const uint8_t* valid, int Fh, int Ff,
                         int P, uint8_t* vis, void* stream);

/* Kernel-level attention entries (the kernels the calls above use).
 * Query contract: fp32 q holds the queries; bf16 q holds the queries times
 * log2(e) / sqrt(dh), rounded to bf16 once (the projection epilogue of the
 * calls above writes Q that way), so that the bf16 kernels' score MFMAs give
 * scores in log2 units with no second rounding of q.
 * Action attention: q [B][Hh][H][dh], ka [B][Hh][H][dh], va [B][Hh][dh][H]
 * (the chunk's own keys; NULL with n_act = 0 to leave them out), cache layer
 * kc [B][Hh][cap][dh], vc [B][Hh][dh][cap] with len[b] (host) rows, or
 * kc = vc = NULL.  out [B][H][Hh*dh] dtype.  splits_hint in 1..63 forces
 * the number of cache-key splits per (episode, head); 0 = automatic:
 * (compute units / Hh) - 1 splits of whole 64-key tiles, at most 63, which
 * depends on the episode's length, Hh and the device but not on B, so an
 * episode's result does not depend on the batch it is in.
 * ws: wam_action_workspace_bytes of a matching dims. */
int wam_attention_action(int dtype, int B, int Hh, int dh, int H, const void* q,
                         const void* ka, const void* va, int n_act,
                         const void* kc, const void* vc, int cap, const int32_t* len,
                         void* out, int splits_hint, void* ws, size_t ws_bytes, void* stream);
/* dh is 64 or 128 in both attention entries; WAM_E_SHAPE otherwise.
 * The same over an E4M3 cache layer (layouts and scales [B][Hh][cap/64] as
 * in wam_kv with dtype WAM_FP8); q, ka, va, out bf16.  ws as
 * above (bf16). */
int wam_attention_action_fp8(int B, int Hh, int dh, int H, const void* q, const void* ka,
                             const void* va, int n_act, const void* kc8, const void* vc8,
                             const float* k_scale, const float* v_scale, int cap,
                             const int32_t* len, void* out, int splits_hint, void* ws,
                             size_t ws_bytes, void* stream);

/* Block-causal prefill attention for rows row0..row0+nq-1 of one episode's
 * cache layer: q [Hh][nq][dh], kc [Hh][cap][dh], vc [Hh][dh][cap];
 * query row r (cache position row0 + r) sees cache rows 0..kend[(row0+r)/P]-1
 * (kend from wam_frame_table).  out [nq][Hh*dh] dtype; dh 64 or 128. */
int wam_attention_prefill(int dtype, int Hh, int dh, int nq, int row0, int P,
                          const int32_t* kend, int n_frames, const void* q,
                          const void* kc, const void* vc, int cap, void* out, void* stream);

/* Measurement: per-kernel-class durations from HIP events recorded around
 * every launch while timing is on (wam_timing(1) also clears earlier
 * records), with the algorithmic bytes and flops of those launches.
 * wam_timing_report waits for the recorded events and returns the number of
 * classes written to out (at most max). */
typedef struct {
  char name[32];
  int launches;
  double ms;     /* sum of launch durations */
  double bytes;  /* algorithmic HBM bytes of those launches */
  double flops;  /* algorithmic flops of those launches */
} wam_kernel_stat;
int wam_timing(int enable);
int wam_timing_report(wam_kernel_stat* out, int max);

#ifdef __cplusplus
}
#endif
#endif /* WAM_H */
