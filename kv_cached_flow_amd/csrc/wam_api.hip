// C-ABI of libwam: argument validation, schedules, frame tables, workspace
// planning and the stream-ordered launch sequence of each call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "wam_internal.h"

using namespace wam;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIPCK(x)                                                                 \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess)                                                        \
      return fail(WAM_E_HIP, "%s failed: %s", #x, hipGetErrorString(e_));       \
  } while (0)

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t esz(int dt) { return dt == WAM_FP8 ? 1 : (dt == WAM_BF16 ? 2 : 4); }

// Carves a caller-provided workspace (base == nullptr: sizing pass).
struct Arena {
  char* base;
  size_t off = 0;
  explicit Arena(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

// Multiplier of the Q columns in the QKV epilogue: bf16 models keep Q as
// Q log2(e) / sqrt(dh), rounded once, and the bf16 attention kernels take
// their scores in log2 units straight from the MFMAs; the fp32 kernels scale
// the scores themselves.
float qkv_q_scale(const wam_dims* d) {
  return d->dtype == WAM_BF16 ? (float)(1.4426950408889634 / sqrt((double)d->dh)) : 1.0f;
}

int check_dims(const wam_dims* d) {
  if (!d) return fail(WAM_E_ARG, "dims is NULL");
  if (d->dtype != WAM_F32 && d->dtype != WAM_BF16) return fail(WAM_E_ARG, "bad dtype %d", d->dtype);
  if (d->L < 1 || d->D < 1 || d->Hh < 1 || d->Fm < 1 || d->P < 1)
    return fail(WAM_E_SHAPE, "non-positive dimension");
  if (d->dh != 64 && d->dh != 128) return fail(WAM_E_SHAPE, "head dim must be 64 or 128 (got %d)", d->dh);
  if (d->D != d->Hh * d->dh) return fail(WAM_E_SHAPE, "D (%d) != Hh*dh (%d)", d->D, d->Hh * d->dh);
  if (d->D % 64 || d->Fm % 64) return fail(WAM_E_SHAPE, "D and Fm must be multiples of 64");
  if (d->Da < 0 || d->Da % 64 || d->Fma < 0 || d->Fma % 64)
    return fail(WAM_E_SHAPE, "Da and Fma must be 0 or positive multiples of 64");
  if (d->D > 4096 || d->Da > 4096) return fail(WAM_E_SHAPE, "expert widths above 4096 are not supported");
  if (d->H != 32) return fail(WAM_E_SHAPE, "action chunk length must be 32 (got %d)", d->H);
  if (d->rope != 0 && d->rope != 1) return fail(WAM_E_ARG, "rope must be 0 or 1");
  if (d->Cv < 1 || d->Cv > 64 || d->A < 1 || d->A > 64)
    return fail(WAM_E_SHAPE, "Cv and A must be in [1, 64]");
  if (d->Tc < 0 || d->Tc > 4096) return fail(WAM_E_SHAPE, "Tc must be in [0, 4096]");
  if (d->Tc > 0) {
    if (d->Ct < 64 || d->Ct > 8192 || d->Ct % 64)
      return fail(WAM_E_SHAPE, "Ct must be a multiple of 64 in [64, 8192]");
    if (d->S < 0 || d->S > 64) return fail(WAM_E_SHAPE, "S must be in [0, 64]");
  }
  return WAM_OK;
}

inline int state_dims(const wam_dims* d) { return d->S ? d->S : d->A; }

// The action expert's shapes: width Da and MLP width Fma in D and Fm (the
// attention interface Hh x dh is unchanged).
wam_dims action_view(const wam_dims* d) {
  wam_dims a = *d;
  if (d->Da) a.D = d->Da;
  if (d->Fma) a.Fm = d->Fma;
  return a;
}

int check_expert(const wam_dims* d, const wam_expert_w* e, const char* name) {
  if (!e || !e->w_in || !e->g_out || !e->w_out || !e->layers)
    return fail(WAM_E_ARG, "%s expert has a NULL pointer", name);
  if (e->n_layers != d->L) return fail(WAM_E_SHAPE, "%s expert has %d layers, dims say %d", name, e->n_layers, d->L);
  if (!aligned16(e->w_in) || !aligned16(e->w_out) || !aligned16(e->g_out))
    return fail(WAM_E_ALIGN, "%s expert pointer not 16-byte aligned", name);
  for (int l = 0; l < e->n_layers; l++) {
    const wam_layer_w& w = e->layers[l];
    if (!w.g1 || !w.wqkv || !w.wo || !w.g2 || !w.w1 || !w.w2)
      return fail(WAM_E_ARG, "%s layer %d has a NULL pointer", name, l);
    if (!aligned16(w.g1) || !aligned16(w.wqkv) || !aligned16(w.wo) || !aligned16(w.g2) ||
        !aligned16(w.w1) || !aligned16(w.w2))
      return fail(WAM_E_ALIGN, "%s layer %d pointer not 16-byte aligned", name, l);
    if (d->Tc > 0) {
      if (!w.gx || !w.wqx || !w.wkvx || !w.wox)
        return fail(WAM_E_ARG, "%s layer %d has a NULL cross-attention pointer", name, l);
      if (!aligned16(w.gx) || !aligned16(w.wqx) || !aligned16(w.wkvx) || !aligned16(w.wox))
        return fail(WAM_E_ALIGN, "%s layer %d cross-attention pointer not 16-byte aligned", name, l);
    }
  }
  return WAM_OK;
}

// A condition cache (wam_prefill_condition_kv's output) that L layers of B
// episodes of this model can read: Tc rows per episode.
int check_cond_kv(const wam_dims* d, const wam_kv* c, int B, int L, const char* name) {
  if (!c || !c->k || !c->v || !c->len) return fail(WAM_E_ARG, "%s condition cache missing", name);
  if (!aligned16(c->k) || !aligned16(c->v))
    return fail(WAM_E_ALIGN, "%s condition cache not 16-byte aligned", name);
  if (c->dtype != d->dtype) return fail(WAM_E_DTYPE, "%s condition cache dtype differs", name);
  if (c->n_layers != L || c->B != B || c->Hh != d->Hh || c->dh != d->dh)
    return fail(WAM_E_SHAPE, "%s condition cache shape does not match", name);
  if (c->cap < d->Tc || c->cap % 64)
    return fail(WAM_E_SHAPE, "%s condition cache cap %d: need a multiple of 64 >= Tc", name, c->cap);
  return WAM_OK;
}

// The expert's condition for a call of B episodes (nothing to check without one).
int check_cond(const wam_dims* d, const wam_expert_w* e, int B, const char* name) {
  if (d->Tc == 0) return WAM_OK;
  int st;
  if ((st = check_cond_kv(d, e->cond, B, e->n_layers, name))) return st;
  for (int b = 0; b < B; b++)
    if (e->cond->len[b] != d->Tc)
      return fail(WAM_E_SHAPE, "%s condition cache len[%d] = %d, Tc is %d", name, b,
                  e->cond->len[b], d->Tc);
  return WAM_OK;
}

// fp8_ok: the caller only reads kv through the action attention, which takes
// an E4M3 cache next to a bf16 model.
int check_kv(const wam_dims* d, const wam_kv* kv, int B, const char* name, bool fp8_ok = false) {
  if (!kv->k || !kv->v || !kv->len) return fail(WAM_E_ARG, "%s has a NULL pointer", name);
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(WAM_E_ALIGN, "%s not 16-byte aligned", name);
  if (kv->dtype == WAM_FP8) {
    if (!fp8_ok || d->dtype != WAM_BF16)
      return fail(WAM_E_DTYPE, "%s: an E4M3 cache is read only by the action layers of a bf16 model",
                  name);
    if (!kv->k_scale || !kv->v_scale) return fail(WAM_E_ARG, "%s has no tile scales", name);
  } else if (kv->dtype != d->dtype) {
    return fail(WAM_E_DTYPE, "%s dtype differs from dims", name);
  }
  if (kv->B != B || kv->Hh != d->Hh || kv->dh != d->dh)
    return fail(WAM_E_SHAPE, "%s shape (B=%d Hh=%d dh=%d) does not match", name, kv->B, kv->Hh, kv->dh);
  if (kv->cap < 64 || kv->cap % 64) return fail(WAM_E_SHAPE, "%s cap must be a positive multiple of 64", name);
  if (kv->n_layers < 1) return fail(WAM_E_SHAPE, "%s has no layer", name);
  return WAM_OK;
}

double phi(double u, double shift) {
  if (u == 0.0) return 0.0;
  if (u == 1.0) return 1.0;
  if (shift == 1.0) return u;
  return shift * u / (1.0 + (shift - 1.0) * u);
}

#pragma clang fp contract(off)
void schedule(int steps, double sigma_end, double shift, float* out) {
  for (int k = 0; k <= steps; k++) {
    double u = 1.0 - (double)k / (double)steps;
    double p = phi(u, shift);
    double s = sigma_end + (1.0 - sigma_end) * p;
    out[k] = (float)s;
  }
}
#pragma clang fp contract(on)

// Compacted frames (valid history in order, then future) and key prefix ends.
int frame_table(const int32_t* block, const uint8_t* valid, int Fh, int Ff, int P,
                int* src, int* kend) {
  int n = 0;
  std::vector<int> blk;
  for (int f = 0; f < Fh + Ff; f++) {
    if (f < Fh && valid && !valid[f]) continue;
    src[n++] = f;
    blk.push_back(block[f]);
  }
  for (int i = 0; i < n; i++) {
    int j = i;
    while (j + 1 < n && blk[j + 1] <= blk[i]) j++;
    kend[i] = (j + 1) * P;
  }
  return n;
}

int check_blocks(const int32_t* block, int F) {
  for (int f = 1; f < F; f++)
    if (block[f] < block[f - 1])
      return fail(WAM_E_SHAPE, "frame_block must be non-decreasing (frame %d)", f);
  return WAM_OK;
}

struct Bufs {
  float* X;
  void* Y;
  void* Q;
  void* Ka;
  void* Va;
  void* O;
  void* Hb;
  float* Yh;
  float* emb;
  float* part;  // split partial products (action path; prefill rows that split)
  size_t part_bytes;
  int pend;     // splits of a product not yet added to X (0: none)
  void* attn;
  size_t attn_bytes;
  float* pattn;  // split partials of the prefill attention
  size_t pattn_bytes;
};

// ----------------------------------------------------------------- layers
struct Layer {
  hipStream_t s;
  const wam_dims* d;
  Bufs* b;
};

int norm_rows(const Layer& c, int odt, const float* g, void* y, int M);
int video_resid(const Layer& c, int M, int N, int K, const void* A, const void* W);
int action_resid(const Layer& c, int M, int N, int K, const void* A, const void* W);

// Condition K/V one layer reads (k == nullptr: no condition).  For a video
// pass they point at one episode's rows, for the action rows at episode 0 of
// the layer (the kernels step by cap per episode).
struct CondRef {
  const void* k = nullptr;
  const void* v = nullptr;
  int cap = 0;
  long long ep = 0;  // elements from one episode's condition rows to the next
};

CondRef cond_ref(const wam_dims* d, const wam_kv* c, int l, int b) {
  CondRef r;
  if (d->Tc == 0 || !c) return r;
  const size_t es = c->dtype == WAM_F32 ? 4 : 2;
  const size_t ls = (size_t)c->B * c->Hh * c->cap * c->dh * es;
  const size_t ep = b > 0 ? (size_t)b * c->Hh * c->cap * c->dh * es : 0;
  r.k = (const char*)c->k + l * ls + ep;
  r.v = (const char*)c->v + l * ls + ep;
  r.cap = c->cap;
  r.ep = (long long)c->Hh * c->cap * c->dh;
  return r;
}

// Cross-attention of n video rows (nep episodes of n / nep rows, episode-
// major, the condition of the first at cr) to their condition:
// X += Attn(RMSNorm(X; gx) Wqx^T ; K_c, V_c) Wox^T.  Every row sees the Tc
// condition rows: one frame of the table whose key prefix ends at Tc.
int video_cross(const Layer& c, const wam_layer_w& w, int n, const CondRef& cr, int nep) {
  const wam_dims* d = c.d;
  const int dt = d->dtype, D = d->D, Dq = d->Hh * d->dh, rpg = n / nep;
  Bufs& b = *c.b;
  int st;
  if ((st = norm_rows(c, dt, w.gx, b.Y, n))) return st;
  EpiArgs e{};
  e.q = b.Q;
  e.D = Dq;
  e.dh = d->dh;
  e.rpg = rpg;
  e.q_gs = (long long)d->Hh * rpg * d->dh;
  e.q_hs = (long long)rpg * d->dh;
  e.q_scale = qkv_q_scale(d);
  HIPCK(gemm(c.s, dt, dt, dt, EPI_QKV, n, Dq, D, b.Y, D, w.wqx, D, e));
  FrameTab ct;
  ct.n = 1;
  ct.P = 1 << 30;
  ct.kend[0] = d->Tc;
  HIPCK(attn_prefill(c.s, dt, d->Hh, d->dh, rpg, 0, ct, b.Q, cr.k, cr.v, cr.cap, b.O, b.pattn,
                     b.pattn_bytes, nep, cr.ep));
  return video_resid(c, n, D, Dq, b.O, w.wox);
}

// The same for the B*H action rows (c.d is the action view: D = its width).
int action_cross(const Layer& c, const wam_layer_w& w, int B, const CondRef& cr) {
  const wam_dims* d = c.d;
  const int dt = d->dtype, D = d->D, Dq = d->Hh * d->dh, H = d->H, M = B * H;
  Bufs& b = *c.b;
  int st;
  if ((st = norm_rows(c, dt, w.gx, b.Y, M))) return st;
  EpiArgs e{};
  e.q = b.Q;
  e.D = Dq;
  e.dh = d->dh;
  e.rpg = H;
  e.q_gs = (long long)d->Hh * H * d->dh;
  e.q_hs = (long long)H * d->dh;
  e.q_scale = qkv_q_scale(d);
  HIPCK(gemm(c.s, dt, dt, dt, EPI_QKV, M, Dq, D, b.Y, D, w.wqx, D, e));
  ActLens cl{};
  for (int i = 0; i < B; i++) cl.len[i] = d->Tc;
  // a few condition tiles per (episode, head): one split
  HIPCK(attn_action(c.s, dt, B, d->Hh, H, d->dh, b.Q, nullptr, nullptr, 0, cr.k, cr.v, cr.cap, cl,
                    b.O, 1, b.attn, b.attn_bytes));
  return action_resid(c, M, D, Dq, b.O, w.wox);
}

// One video layer for rows row0.. of nep episodes that share a frame table:
// n rows, episode-major (n / nep per episode), episode e's cache layer at
// (kl, vl) + e kv_ep elements.
int video_layer(const Layer& c, const wam_layer_w& w, int n, int row0, const FrameTab& tab,
                void* kl, void* vl, int cap, bool kv_only, const CondRef& cr = CondRef(),
                int nep = 1, long long kv_ep = 0) {
  const wam_dims* d = c.d;
  const int dt = d->dtype, D = d->D, rpg = n / nep;
  Bufs& b = *c.b;
  int st;
  if ((st = norm_rows(c, dt, w.g1, b.Y, n))) return st;
  EpiArgs e{};
  e.q = b.Q;
  e.k = kl;
  e.v = vl;
  e.D = D;
  e.dh = d->dh;
  e.rpg = rpg;
  e.q_gs = (long long)d->Hh * rpg * d->dh;
  e.q_hs = (long long)rpg * d->dh;
  e.k_gs = e.v_gs = kv_ep;
  e.k_hs = (long long)cap * d->dh;
  e.v_hs = (long long)d->dh * cap;
  e.k_row0 = row0;
  e.v_ld = cap;
  e.v_col0 = row0;
  e.q_scale = qkv_q_scale(d);
  // rotary option: Q rows and the K rows just cached sit at positions row0 ..
  RopeRows rb{};
  for (int i = 0; i < nep; i++) rb.base[i] = row0;
  void* krows = (char*)kl + (size_t)row0 * d->dh * esz(dt);
  if (kv_only) {
    e.n_begin = D;
    HIPCK(gemm(c.s, dt, dt, dt, EPI_QKV, n, 2 * D, D, b.Y, D,
               (const char*)w.wqkv + (size_t)D * D * esz(dt), D, e));
    if (d->rope)
      HIPCK(rope_qk(c.s, dt, krows, kv_ep, e.k_hs, nullptr, 0, 0, nep, rpg, d->Hh, d->dh, rb));
    return WAM_OK;
  }
  HIPCK(gemm(c.s, dt, dt, dt, EPI_QKV, n, 3 * D, D, b.Y, D, w.wqkv, D, e));
  if (d->rope)
    HIPCK(rope_qk(c.s, dt, b.Q, e.q_gs, e.q_hs, krows, kv_ep, e.k_hs, nep, rpg, d->Hh, d->dh, rb));
  HIPCK(attn_prefill(c.s, dt, d->Hh, d->dh, rpg, row0, tab, b.Q, kl, vl, cap, b.O, b.pattn,
                     b.pattn_bytes, nep, kv_ep));
  if ((st = video_resid(c, n, D, D, b.O, w.wo))) return st;
  if (cr.k && (st = video_cross(c, w, n, cr, nep))) return st;
  if ((st = norm_rows(c, dt, w.g2, b.Y, n))) return st;
  EpiArgs gl{};
  gl.out = b.Hb;
  gl.ldo = d->Fm;
  HIPCK(gemm(c.s, dt, dt, dt, EPI_GELU, n, d->Fm, D, b.Y, D, w.w1, D, gl));
  return video_resid(c, n, D, d->Fm, b.Hb, w.w2);
}

// X += A W^T for the action rows, as split partials that the next RMSNorm adds
// (bf16 shapes the split GEMM supports), else directly.
int action_resid(const Layer& c, int M, int N, int K, const void* A, const void* W) {
  const wam_dims* d = c.d;
  Bufs& b = *c.b;
  if (d->dtype == WAM_BF16 && gemm_partial_splits(M, N, K) > 0) {
    int ks = 0;
    HIPCK(gemm_partial(c.s, M, N, K, A, K, W, K, b.part, &ks));
    b.pend = ks;
    return WAM_OK;
  }
  EpiArgs r{};
  r.out = b.X;
  r.ldo = N;
  HIPCK(gemm(c.s, d->dtype, d->dtype, WAM_F32, EPI_RESID, M, N, K, A, K, W, K, r));
  b.pend = 0;
  return WAM_OK;
}

// X += A W^T for video rows: as split partials (b.pend) where the rows are
// too few to fill the CUs with output tiles and the workspace holds them,
// else directly.  The next RMSNorm adds pending partials to X.
int video_resid(const Layer& c, int M, int N, int K, const void* A, const void* W) {
  const wam_dims* d = c.d;
  Bufs& b = *c.b;
  const int ks = d->dtype == WAM_BF16 && b.part ? gemm_big_splits(M, N, K) : 1;
  if (ks > 1 && (size_t)ks * M * N * 4 <= b.part_bytes) {
    HIPCK(gemm_big_partial(c.s, M, N, K, A, K, W, K, b.part, ks));
    b.pend = ks;
    return WAM_OK;
  }
  EpiArgs r{};
  r.out = b.X;
  r.ldo = N;
  HIPCK(gemm(c.s, d->dtype, d->dtype, WAM_F32, EPI_RESID, M, N, K, A, K, W, K, r));
  b.pend = 0;
  return WAM_OK;
}

// y = RMSNorm(X; g) (odt), first adding pending split partials to X.
int norm_rows(const Layer& c, int odt, const float* g, void* y, int M) {
  Bufs& b = *c.b;
  if (b.pend > 0) {
    HIPCK(rmsnorm_accum(c.s, odt, b.X, b.part, b.pend, g, y, M, c.d->D));
    b.pend = 0;
  } else {
    HIPCK(rmsnorm(c.s, odt, b.X, g, y, M, c.d->D));
  }
  return WAM_OK;
}

// One action layer on the B*H rows in b.X; kc/vc: that layer's cache for all
// episodes (or NULL).  May leave the W2 product pending (b.pend).
int action_layer(const Layer& c, const wam_layer_w& w, int B, const void* kc, const void* vc,
                 int cap, const ActLens& lens, const float* ksc = nullptr,
                 const float* vsc = nullptr, const CondRef& cr = CondRef()) {
  const wam_dims* d = c.d;  // the action view: D = the action width
  const int dt = d->dtype, D = d->D, Dq = d->Hh * d->dh, H = d->H, M = B * H;
  Bufs& b = *c.b;
  int st;
  EpiArgs e{};
  e.q = b.Q;
  e.k = b.Ka;
  e.v = b.Va;
  e.D = Dq;
  e.dh = d->dh;
  e.rpg = H;
  e.q_gs = e.k_gs = (long long)d->Hh * H * d->dh;
  e.q_hs = e.k_hs = (long long)H * d->dh;
  e.v_gs = (long long)d->Hh * d->dh * H;
  e.v_hs = (long long)d->dh * H;
  e.v_ld = H;
  e.q_scale = qkv_q_scale(d);
  if ((st = norm_rows(c, dt, w.g1, b.Y, M))) return st;
  HIPCK(gemm(c.s, dt, dt, dt, EPI_QKV, M, 3 * Dq, D, b.Y, D, w.wqkv, D, e));
  if (d->rope) {
    // action token i of episode b follows that episode's cached rows
    RopeRows rb{};
    for (int i = 0; i < B; i++) rb.base[i] = lens.len[i];
    HIPCK(rope_qk(c.s, dt, b.Q, e.q_gs, e.q_hs, b.Ka, e.k_gs, e.k_hs, B, H, d->Hh, d->dh, rb));
  }
  HIPCK(attn_action(c.s, dt, B, d->Hh, H, d->dh, b.Q, b.Ka, b.Va, H, kc, vc, cap, lens, b.O, 0, b.attn,
                    b.attn_bytes, ksc, vsc));
  if ((st = action_resid(c, M, D, Dq, b.O, w.wo))) return st;
  if (cr.k && (st = action_cross(c, w, B, cr))) return st;
  if ((st = norm_rows(c, dt, w.g2, b.Y, M))) return st;
  EpiArgs gl{};
  gl.out = b.Hb;
  gl.ldo = d->Fm;
  HIPCK(gemm(c.s, dt, dt, dt, EPI_GELU, M, d->Fm, D, b.Y, D, w.w1, D, gl));
  return action_resid(c, M, D, d->Fm, b.Hb, w.w2);
}

// pending partials of the last layer -> X (before the step boundary)
int flush_pending(const Layer& c, const float* g, int M) {
  Bufs& b = *c.b;
  if (b.pend == 0) return WAM_OK;
  return norm_rows(c, c.d->dtype, g, b.Y, M);
}

// workspace of the action path (rows M = B*H); d is the action view
void plan_action(Arena& a, const wam_dims* d, int B, int max_len, bool with_emb, Bufs& b) {
  const int M = B * d->H;
  const size_t e = esz(d->dtype), Dq = (size_t)d->Hh * d->dh;
  b.emb = with_emb ? (float*)a.take((size_t)WAM_MAX_STEPS * d->D * 4) : nullptr;
  b.X = (float*)a.take((size_t)M * d->D * 4);
  b.Y = a.take((size_t)M * d->D * e);
  b.Q = a.take((size_t)M * Dq * e);
  b.Ka = a.take((size_t)M * Dq * e);
  b.Va = a.take((size_t)M * Dq * e);
  b.O = a.take((size_t)M * Dq * e);
  b.Hb = a.take((size_t)M * d->Fm * e);
  b.Yh = (float*)a.take((size_t)M * d->D * 4);
  b.part_bytes = (size_t)4 * M * d->D * 4;
  b.part = (float*)a.take(b.part_bytes);
  b.pend = 0;
  b.attn_bytes = attn_action_scratch_bytes(B, d->Hh, d->H, d->dh, max_len, 0);
  b.attn = a.take(b.attn_bytes);
  b.pattn = nullptr;
  b.pattn_bytes = 0;
}

// Workspace of a video call: rows for one episode's history and future, or
// for the future rows of nb episodes denoised together.
void plan_prefill(Arena& a, const wam_dims* d, int nb, int Fh, int Ff, Bufs& b, float** z) {
  const size_t e = esz(d->dtype);
  // history and future rows share one pass when the future is not denoised
  const size_t Tf = (size_t)nb * Ff * d->P;
  const size_t T = std::max<size_t>((size_t)(Fh + Ff) * d->P, Tf);
  b.emb = (float*)a.take((size_t)(WAM_MAX_STEPS + 2) * d->D * 4);
  b.X = (float*)a.take(T * d->D * 4);
  b.Y = a.take(T * d->D * e);
  b.Q = a.take(T * d->D * e);
  b.O = a.take(T * d->D * e);
  b.Hb = a.take(T * d->Fm * e);
  b.Yh = (float*)a.take(std::max<size_t>(Tf, 1) * d->D * 4);
  *z = (float*)a.take(std::max<size_t>(Tf, 1) * d->Cv * 4);
  b.Ka = b.Va = nullptr;
  // residual products of row counts that leave CUs idle split k 4 ways at most,
  // and only while their 128x128 tiles number at most one per CU
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  b.part_bytes = (size_t)4 * std::min(T * d->D, (size_t)n_cu * 128 * 128 + (size_t)128 * d->D) * 4;
  b.part = (float*)a.take(b.part_bytes);
  b.pend = 0;
  b.attn = nullptr;
  b.attn_bytes = 0;
  b.pattn_bytes = attn_prefill_split_bytes(d->Hh, d->dh, (int)T);
  b.pattn = (float*)a.take(b.pattn_bytes);
}

size_t layer_stride(const wam_kv* kv) {
  return (size_t)kv->B * kv->Hh * kv->cap * kv->dh * esz(kv->dtype);
}

// Tile scales of layer l of an E4M3 cache (NULL for the other dtypes).
const float* layer_scales(const wam_kv* kv, const float* base, int l) {
  if (kv->dtype != WAM_FP8) return nullptr;
  return base + (size_t)l * kv->B * kv->Hh * (kv->cap / 64);
}

}  // namespace

// =================================================================== C-ABI
extern "C" {

int wam_abi_version(void) { return WAM_ABI_VERSION; }

const char* wam_status_str(int st) {
  switch (st) {
    case WAM_OK: return "ok";
    case WAM_E_ARG: return "invalid argument";
    case WAM_E_SHAPE: return "invalid or inconsistent shape";
    case WAM_E_DTYPE: return "dtype mismatch";
    case WAM_E_ALIGN: return "pointer not 16-byte aligned";
    case WAM_E_WORKSPACE: return "workspace missing or too small";
    case WAM_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* wam_last_error(void) { return g_err.c_str(); }

int wam_schedule(int steps, double sigma_end, double shift, float* out) {
  if (!out) return fail(WAM_E_ARG, "out is NULL");
  if (steps < 1 || steps > 4096) return fail(WAM_E_ARG, "steps must be in [1, 4096]");
  if (!(sigma_end >= 0.0 && sigma_end < 1.0)) return fail(WAM_E_ARG, "sigma_end must be in [0, 1)");
  if (!(shift > 0.0)) return fail(WAM_E_ARG, "shift must be > 0");
  schedule(steps, sigma_end, shift, out);
  return WAM_OK;
}

int wam_frame_table(const int32_t* frame_block, const uint8_t* valid, int Fh, int Ff, int P,
                    int32_t* src_frame, int32_t* kend) {
  if (!frame_block || !src_frame || !kend) return fail(WAM_E_ARG, "NULL pointer");
  if (Fh < 0 || Ff < 0 || Fh + Ff > WAM_MAX_FRAMES || P < 1)
    return fail(WAM_E_SHAPE, "bad frame counts");
  int st = check_blocks(frame_block, Fh + Ff);
  if (st) return st;
  return frame_table(frame_block, valid, Fh, Ff, P, src_frame, kend);
}

size_t wam_prefill_workspace_bytes(const wam_dims* d, int B, int Fh, int Ff) {
  (void)B;
  if (check_dims(d)) return 0;
  Arena a(nullptr);
  Bufs b;
  float* z;
  plan_prefill(a, d, std::max(B, 1), Fh, Ff, b, &z);
  return a.off + 256;
}

namespace {

// Frame tables of every episode of a call, validated before anything is
// enqueued: the compacted table (valid history in order, then the future),
// the gather map of the valid history frames (rows of the history input,
// b * Fh + frame) and the number of valid history frames.
struct Tables {
  std::vector<FrameTab> tab;
  std::vector<RowMap> hmap;
  std::vector<int> nh;
};

int build_tables(const int32_t* frame_block, const uint8_t* hist_valid, int B, int Fh, int Ff,
                 int P, int cap, Tables& t) {
  t.tab.assign(B, FrameTab{});
  t.hmap.assign(B, RowMap{});
  t.nh.assign(B, 0);
  for (int b = 0; b < B; b++) {
    int src[WAM_MAX_FRAMES], kend[WAM_MAX_FRAMES];
    const uint8_t* v = hist_valid ? hist_valid + (size_t)b * Fh : nullptr;
    const int n = frame_table(frame_block, v, Fh, Ff, P, src, kend);
    if (n == 0) return fail(WAM_E_SHAPE, "episode %d has no valid frame", b);
    if ((long long)n * P > cap)
      return fail(WAM_E_SHAPE, "episode %d needs %d cache rows, cap is %d", b, n * P, cap);
    t.tab[b].n = n;
    t.tab[b].P = P;
    for (int i = 0; i < n; i++) t.tab[b].kend[i] = kend[i];
    t.nh[b] = n - Ff;
    t.hmap[b].n = t.nh[b];
    t.hmap[b].P = P;
    for (int i = 0; i < t.nh[b]; i++) t.hmap[b].src[i] = b * Fh + src[i];
  }
  return WAM_OK;
}

// History rows [row0, row0 + n) of one episode at sigma = 0 (emb0), gathered
// from `hist` by `map`, through the L layers; their K/V go to the cache rows.
// The last layer computes K/V only.
int history_rows(const Layer& c, const wam_expert_w* video, int ep, const void* hist,
                 const RowMap& map, const float* emb0, const FrameTab& tab, int row0, int n,
                 char* k, char* v, size_t ls, int cap) {
  const wam_dims* d = c.d;
  Bufs& b = *c.b;
  int st;
  HIPCK(embed(c.s, d->dtype, d->dtype, hist, map, video->w_in, emb0, b.X, n, d->D, d->Cv));
  for (int l = 0; l < d->L; l++)
    if ((st = video_layer(c, video->layers[l], n, row0, tab, k + l * ls, v + l * ls, cap,
                          l == d->L - 1, cond_ref(d, video->cond, l, ep))))
      return st;
  return WAM_OK;
}

// The future rows [Th, Th + Tf) of episodes ep .. ep + nep - 1, which share
// one frame table, over their cached history: video_steps Euler steps of z
// over sig (embeddings emb_steps[k]) attending to [history ; future], then
// one caching pass at emb_last; z (fp32, [nep][Tf][Cv]) starts as
// fut_noise_b (dtype, the same layout).  video_steps == 0: the caching pass
// of the noise.  k / v: episode ep's cache, episode ep + i at + i kv_ep elements.
int future_rows(const Layer& c, const wam_expert_w* video, int ep, const void* fut_noise_b,
                float* z, const std::vector<float>& sig, int video_steps, const float* emb_steps,
                const float* emb_last, const FrameTab& tab, int Th, int Tf, char* k, char* v,
                size_t ls, int cap, int nep = 1, long long kv_ep = 0) {
  const wam_dims* d = c.d;
  Bufs& b = *c.b;
  const int D = d->D, dt = d->dtype, n = nep * Tf;
  int st;
  RowMap zmap;
  zmap.n = 1;
  zmap.P = n;
  zmap.src[0] = 0;
  HIPCK(copy_cvt_f32(c.s, dt, fut_noise_b, z, (int64_t)n * d->Cv));
  for (int s = 0; s < video_steps; s++) {
    HIPCK(embed(c.s, WAM_F32, dt, z, zmap, video->w_in, emb_steps + (size_t)s * D, b.X, n, D,
                d->Cv));
    for (int l = 0; l < d->L; l++)
      if ((st = video_layer(c, video->layers[l], n, Th, tab, k + l * ls, v + l * ls, cap, false,
                            cond_ref(d, video->cond, l, ep), nep, kv_ep)))
        return st;
    if ((st = flush_pending(c, video->g_out, n))) return st;  // X whole for the head
    HIPCK(step_boundary(c.s, dt, b.X, video->g_out, video->w_out, z, sig[s + 1] - sig[s], nullptr,
                        nullptr, nullptr, n, D, d->Cv, true));
  }
  HIPCK(embed(c.s, WAM_F32, dt, z, zmap, video->w_in, emb_last, b.X, n, D, d->Cv));
  for (int l = 0; l < d->L; l++)
    if ((st = video_layer(c, video->layers[l], n, Th, tab, k + l * ls, v + l * ls, cap,
                          l == d->L - 1, cond_ref(d, video->cond, l, ep), nep, kv_ep)))
      return st;
  return WAM_OK;
}

// True when every episode of the call has the same compacted frame table
// (then their future rows can be denoised together).
bool same_tables(const Tables& t) {
  for (size_t b = 1; b < t.tab.size(); b++) {
    if (t.tab[b].n != t.tab[0].n || t.nh[b] != t.nh[0]) return false;
    for (int i = 0; i < t.tab[0].n; i++)
      if (t.tab[b].kend[i] != t.tab[0].kend[i]) return false;
  }
  return true;
}

// Time embeddings of a video call into emb: [0 (history), sigma_0 ..
// sigma_{V-1} (imagine steps), sigma_V (V >= 1) | 1 (V = 0) (caching pass)].
void video_schedule(int video_steps, double sigma_star, double shift, std::vector<float>& sig,
                    std::vector<float>& embs) {
  sig.assign(video_steps + 1, 0.f);
  if (video_steps > 0) schedule(video_steps, sigma_star, shift, sig.data());
  embs.clear();
  embs.push_back(0.f);
  if (video_steps > 0)
    for (int k = 0; k <= video_steps; k++) embs.push_back(sig[k]);
  else
    embs.push_back(1.f);
}

int check_video_call(const wam_dims* d, const wam_expert_w* video, int B, int Fh, int Ff,
                     const int32_t* frame_block, const wam_kv* cache) {
  int st;
  if ((st = check_dims(d))) return st;
  if ((st = check_expert(d, video, "video"))) return st;
  if (B < 1 || B > WAM_MAX_BATCH) return fail(WAM_E_SHAPE, "B must be in [1, %d]", WAM_MAX_BATCH);
  if (Fh < 0 || Ff < 0 || Fh + Ff < 1 || Fh + Ff > WAM_MAX_FRAMES)
    return fail(WAM_E_SHAPE, "frame counts out of range");
  if (!frame_block) return fail(WAM_E_ARG, "frame_block is NULL");
  if ((st = check_blocks(frame_block, Fh + Ff))) return st;
  if (!cache) return fail(WAM_E_ARG, "cache is NULL");
  if ((st = check_kv(d, cache, B, "cache"))) return st;
  if (cache->n_layers != d->L) return fail(WAM_E_SHAPE, "cache must hold L layers");
  return check_cond(d, video, B, "video");
}

int check_future_args(int video_steps, double sigma_star, double shift) {
  if (video_steps < 0 || video_steps > WAM_MAX_STEPS)
    return fail(WAM_E_ARG, "video_steps must be in [0, %d]", WAM_MAX_STEPS);
  if (video_steps > 0 && !(sigma_star > 0.0 && sigma_star < 1.0))
    return fail(WAM_E_ARG, "sigma_star must be in (0, 1)");
  if (!(shift > 0.0)) return fail(WAM_E_ARG, "shift must be > 0");
  return WAM_OK;
}

}  // namespace

int wam_prefill_video_cache(const wam_dims* d, const wam_expert_w* video, const void* hist,
                            const uint8_t* hist_valid, int B, int Fh, const void* fut_noise,
                            int Ff, const int32_t* frame_block, int video_steps,
                            double sigma_star, double shift, wam_kv* cache,
                            float* fut_latents_out, void* ws, size_t ws_bytes, void* stream) {
  int st;
  if ((st = check_video_call(d, video, B, Fh, Ff, frame_block, cache))) return st;
  if (Fh > 0 && !hist) return fail(WAM_E_ARG, "hist is NULL");
  if (Ff > 0 && !fut_noise) return fail(WAM_E_ARG, "fut_noise is NULL");
  if ((hist && !aligned16(hist)) || (fut_noise && !aligned16(fut_noise)) ||
      (fut_latents_out && !aligned16(fut_latents_out)))
    return fail(WAM_E_ALIGN, "input pointer not 16-byte aligned");
  if ((st = check_future_args(video_steps, sigma_star, shift))) return st;
  if (!ws || !aligned16(ws)) return fail(WAM_E_WORKSPACE, "workspace NULL or unaligned");
  if (ws_bytes < wam_prefill_workspace_bytes(d, B, Fh, Ff))
    return fail(WAM_E_WORKSPACE, "workspace too small (%zu < %zu)", ws_bytes,
                wam_prefill_workspace_bytes(d, B, Fh, Ff));
  const int P = d->P;
  Tables t;
  if ((st = build_tables(frame_block, hist_valid, B, Fh, Ff, P, cache->cap, t))) return st;

  hipStream_t s = (hipStream_t)stream;
  Arena a(ws);
  Bufs bufs;
  float* z;
  plan_prefill(a, d, B, Fh, Ff, bufs, &z);
  std::vector<float> sig, embs;
  video_schedule(video_steps, sigma_star, shift, sig, embs);
  const int D = d->D;
  HIPCK(time_embedding(s, embs.data(), (int)embs.size(), D, bufs.emb));
  const float* emb_hist = bufs.emb;
  const float* emb_last = bufs.emb + (size_t)(embs.size() - 1) * D;

  const int dt = d->dtype;
  const size_t ls = layer_stride(cache);
  const size_t ep = (size_t)d->Hh * cache->cap * d->dh * esz(dt);  // one episode in a layer
  Layer c{s, d, &bufs};
  const int Tf = Ff * P;
  // imagined futures of episodes with one frame table go through the layers together
  const bool together = video_steps > 0 && Ff > 0 && B > 1 && same_tables(t);
  for (int b = 0; b < B; b++) {
    const int Th = t.nh[b] * P;
    char* kb = (char*)cache->k + b * ep;
    char* vb = (char*)cache->v + b * ep;
    const void* fut_b = Ff > 0 ? (const char*)fut_noise + (size_t)b * Tf * d->Cv * esz(dt) : nullptr;
    if (video_steps == 0 && Ff > 0) {
      // No video denoising: the history rows and the future rows go through
      // the same layers, so one pass over all of them (history rows see only
      // history keys through the block-causal frame table) replaces the
      // history pass plus the future cache pass.
      if (Th > 0)
        HIPCK(embed(s, dt, dt, hist, t.hmap[b], video->w_in, emb_hist, bufs.X, Th, D, d->Cv));
      RowMap zmap;
      zmap.n = 1;
      zmap.P = Tf;
      zmap.src[0] = 0;
      HIPCK(copy_cvt_f32(s, dt, fut_b, z, (int64_t)Tf * d->Cv));
      HIPCK(embed(s, WAM_F32, dt, z, zmap, video->w_in, emb_last, bufs.X + (size_t)Th * D, Tf, D,
                  d->Cv));
      for (int l = 0; l < d->L; l++)
        if ((st = video_layer(c, video->layers[l], Th + Tf, 0, t.tab[b], kb + l * ls, vb + l * ls,
                              cache->cap, l == d->L - 1, cond_ref(d, video->cond, l, b))))
          return st;
    } else {
      if (Th > 0 && (st = history_rows(c, video, b, hist, t.hmap[b], emb_hist, t.tab[b], 0, Th, kb,
                                        vb, ls, cache->cap)))
        return st;
      if (Ff > 0 && !together &&
          (st = future_rows(c, video, b, fut_b, z, sig, video_steps, bufs.emb + D, emb_last,
                            t.tab[b], Th, Tf, kb, vb, ls, cache->cap)))
        return st;
    }
    if (Ff > 0 && fut_latents_out && !together)
      HIPCK(hipMemcpyAsync(fut_latents_out + (size_t)b * Tf * d->Cv, z, (size_t)Tf * d->Cv * 4,
                           hipMemcpyDeviceToDevice, s));
    cache->len[b] = t.tab[b].n * P;
  }
  if (together) {
    if ((st = future_rows(c, video, 0, fut_noise, z, sig, video_steps, bufs.emb + D, emb_last,
                          t.tab[0], t.nh[0] * P, Tf, (char*)cache->k, (char*)cache->v, ls,
                          cache->cap, B, (long long)(ep / esz(dt)))))
      return st;
    if (fut_latents_out)
      HIPCK(hipMemcpyAsync(fut_latents_out, z, (size_t)B * Tf * d->Cv * 4, hipMemcpyDeviceToDevice,
                           s));
  }
  return WAM_OK;
}

int wam_extend_history_cache(const wam_dims* d, const wam_expert_w* video, const void* hist_new,
                             const uint8_t* hist_valid, int B, int Fh_old, int Fn,
                             const int32_t* frame_block, wam_kv* cache, void* ws, size_t ws_bytes,
                             void* stream) {
  int st;
  if (Fh_old < 0 || Fn < 1) return fail(WAM_E_SHAPE, "need Fh_old >= 0 and Fn >= 1");
  if ((st = check_video_call(d, video, B, Fh_old + Fn, 0, frame_block, cache))) return st;
  if (!hist_new) return fail(WAM_E_ARG, "hist_new is NULL");
  if (!aligned16(hist_new)) return fail(WAM_E_ALIGN, "hist_new not 16-byte aligned");
  if (!ws || !aligned16(ws) || ws_bytes < wam_prefill_workspace_bytes(d, B, Fn, 0))
    return fail(WAM_E_WORKSPACE, "workspace missing or too small");
  const int P = d->P, Fh = Fh_old + Fn;
  std::vector<FrameTab> tab(B);
  std::vector<RowMap> map(B);
  std::vector<int> n_old(B), n_all(B);
  for (int b = 0; b < B; b++) {
    int src[WAM_MAX_FRAMES], kend[WAM_MAX_FRAMES];
    const uint8_t* v = hist_valid ? hist_valid + (size_t)b * Fh : nullptr;
    const int n = frame_table(frame_block, v, Fh, 0, P, src, kend);
    int no = 0;
    while (no < n && src[no] < Fh_old) no++;
    if ((long long)n * P > cache->cap)
      return fail(WAM_E_SHAPE, "episode %d needs %d cache rows, cap is %d", b, n * P, cache->cap);
    if (cache->len[b] != no * P)
      return fail(WAM_E_SHAPE, "episode %d: cache holds %d rows, its %d valid old frames %d", b,
                  cache->len[b], no, no * P);
    // frames of one block read each other: the new frames must start a block
    if (no > 0 && no < n && frame_block[src[no]] <= frame_block[src[no - 1]])
      return fail(WAM_E_SHAPE,
                  "episode %d: new frame %d shares temporal block %d with a cached frame", b,
                  src[no], frame_block[src[no]]);
    tab[b].n = n;
    tab[b].P = P;
    for (int i = 0; i < n; i++) tab[b].kend[i] = kend[i];
    map[b].n = n - no;
    map[b].P = P;
    for (int i = no; i < n; i++) map[b].src[i - no] = b * Fn + (src[i] - Fh_old);
    n_old[b] = no;
    n_all[b] = n;
  }

  hipStream_t s = (hipStream_t)stream;
  Arena a(ws);
  Bufs bufs;
  float* z;
  plan_prefill(a, d, 1, Fn, 0, bufs, &z);
  const float zero = 0.f;
  HIPCK(time_embedding(s, &zero, 1, d->D, bufs.emb));
  const size_t ls = layer_stride(cache);
  const size_t ep = (size_t)d->Hh * cache->cap * d->dh * esz(d->dtype);
  Layer c{s, d, &bufs};
  for (int b = 0; b < B; b++) {
    const int rows = (n_all[b] - n_old[b]) * P;
    if (rows > 0 &&
        (st = history_rows(c, video, b, hist_new, map[b], bufs.emb, tab[b], n_old[b] * P, rows,
                           (char*)cache->k + b * ep, (char*)cache->v + b * ep, ls, cache->cap)))
      return st;
    cache->len[b] = n_all[b] * P;
  }
  return WAM_OK;
}

int wam_prefill_future(const wam_dims* d, const wam_expert_w* video, const uint8_t* hist_valid,
                       int B, int Fh, const void* fut_noise, int Ff, const int32_t* frame_block,
                       int video_steps, double sigma_star, double shift, wam_kv* cache,
                       float* fut_latents_out, void* ws, size_t ws_bytes, void* stream) {
  int st;
  if (Ff < 1) return fail(WAM_E_SHAPE, "Ff must be >= 1");
  if ((st = check_video_call(d, video, B, Fh, Ff, frame_block, cache))) return st;
  if (!fut_noise) return fail(WAM_E_ARG, "fut_noise is NULL");
  if (!aligned16(fut_noise) || (fut_latents_out && !aligned16(fut_latents_out)))
    return fail(WAM_E_ALIGN, "pointer not 16-byte aligned");
  if ((st = check_future_args(video_steps, sigma_star, shift))) return st;
  if (!ws || !aligned16(ws) || ws_bytes < wam_prefill_workspace_bytes(d, B, 0, Ff))
    return fail(WAM_E_WORKSPACE, "workspace missing or too small");
  const int P = d->P;
  Tables t;
  if ((st = build_tables(frame_block, hist_valid, B, Fh, Ff, P, cache->cap, t))) return st;
  for (int b = 0; b < B; b++)
    if (cache->len[b] != t.nh[b] * P)
      return fail(WAM_E_SHAPE, "episode %d: cache holds %d rows, its valid history has %d", b,
                  cache->len[b], t.nh[b] * P);

  hipStream_t s = (hipStream_t)stream;
  Arena a(ws);
  Bufs bufs;
  float* z;
  plan_prefill(a, d, B, 0, Ff, bufs, &z);
  std::vector<float> sig, embs;
  video_schedule(video_steps, sigma_star, shift, sig, embs);
  const int D = d->D, dt = d->dtype;
  HIPCK(time_embedding(s, embs.data(), (int)embs.size(), D, bufs.emb));
  const size_t ls = layer_stride(cache);
  const size_t ep = (size_t)d->Hh * cache->cap * d->dh * esz(dt);
  Layer c{s, d, &bufs};
  const int Tf = Ff * P;
  const float* emb_last = bufs.emb + (size_t)(embs.size() - 1) * D;
  if (video_steps > 0 && B > 1 && same_tables(t)) {
    // every episode's future through the layers together
    if ((st = future_rows(c, video, 0, fut_noise, z, sig, video_steps, bufs.emb + D, emb_last,
                          t.tab[0], t.nh[0] * P, Tf, (char*)cache->k, (char*)cache->v, ls,
                          cache->cap, B, (long long)(ep / esz(dt)))))
      return st;
    if (fut_latents_out)
      HIPCK(hipMemcpyAsync(fut_latents_out, z, (size_t)B * Tf * d->Cv * 4, hipMemcpyDeviceToDevice,
                           s));
    for (int b = 0; b < B; b++) cache->len[b] = t.tab[b].n * P;
    return WAM_OK;
  }
  for (int b = 0; b < B; b++) {
    const void* fut_b = (const char*)fut_noise + (size_t)b * Tf * d->Cv * esz(dt);
    if ((st = future_rows(c, video, b, fut_b, z, sig, video_steps, bufs.emb + D, emb_last,
                          t.tab[b], t.nh[b] * P, Tf, (char*)cache->k + b * ep,
                          (char*)cache->v + b * ep, ls, cache->cap)))
      return st;
    if (fut_latents_out)
      HIPCK(hipMemcpyAsync(fut_latents_out + (size_t)b * Tf * d->Cv, z, (size_t)Tf * d->Cv * 4,
                           hipMemcpyDeviceToDevice, s));
    cache->len[b] = t.tab[b].n * P;
  }
  return WAM_OK;
}

int wam_async_check(int H, int R, int S) {
  if (!(0 < S && S < R && R <= H) || 2 * S < R)
    return fail(WAM_E_ARG, "asynchronous execution needs R/2 <= S < R <= H (H=%d R=%d S=%d)", H, R,
                S);
  return WAM_OK;
}

int wam_async_handoff(int H, int R, int S, int elapsed, int* first, int* count) {
  int st;
  if ((st = wam_async_check(H, R, S))) return st;
  if (!first || !count) return fail(WAM_E_ARG, "NULL pointer");
  if (elapsed < 0) return fail(WAM_E_ARG, "elapsed must be >= 0");
  if (elapsed > R - S)
    return fail(WAM_E_SHAPE, "chunk ready %d steps after its trigger, the overlap is %d", elapsed,
                R - S);
  *first = elapsed;
  *count = R - elapsed;
  return WAM_OK;
}

int wam_fuse_interval_kv(const wam_kv* src, int M, const int32_t* start, const int32_t* count,
                         const float* logits, int logits_stride, wam_kv* dst, void* stream) {
  if (!src || !dst || !start || !count || !logits) return fail(WAM_E_ARG, "NULL pointer");
  if (!src->k || !src->v || !dst->k || !dst->v || !src->len || !dst->len)
    return fail(WAM_E_ARG, "NULL cache pointer");
  if (!aligned16(src->k) || !aligned16(src->v) || !aligned16(dst->k) || !aligned16(dst->v))
    return fail(WAM_E_ALIGN, "cache not 16-byte aligned");
  if (src->dtype != dst->dtype) return fail(WAM_E_DTYPE, "src and dst dtypes differ");
  if (src->dtype != WAM_F32 && src->dtype != WAM_BF16) return fail(WAM_E_ARG, "bad dtype");
  if (src->B != dst->B || src->Hh != dst->Hh || src->dh != dst->dh || src->cap != dst->cap)
    return fail(WAM_E_SHAPE, "src and dst shapes differ");
  if (src->B < 1 || src->B > WAM_MAX_BATCH) return fail(WAM_E_SHAPE, "bad B");
  if (M < 1 || M > WAM_MAX_FUSE || dst->n_layers < M)
    return fail(WAM_E_SHAPE, "M must be in [1, %d] and fit dst", WAM_MAX_FUSE);
  if (logits_stride < 1) return fail(WAM_E_ARG, "logits_stride must be >= 1");
  FuseArgs fa;
  fa.M = M;
  for (int m = 0; m < M; m++) {
    if (count[m] < 1 || count[m] > WAM_MAX_INTERVAL || count[m] > logits_stride)
      return fail(WAM_E_SHAPE, "interval %d has %d layers", m, count[m]);
    if (start[m] < 0 || start[m] + count[m] > src->n_layers)
      return fail(WAM_E_SHAPE, "interval %d outside the source layers", m);
    const float* lg = logits + (size_t)m * logits_stride;
    double mx = -INFINITY;
    for (int j = 0; j < count[m]; j++) mx = std::max(mx, (double)lg[j]);
    if (!(mx > -INFINITY) || std::isnan(mx)) return fail(WAM_E_ARG, "interval %d logits are all -inf or NaN", m);
    double e[WAM_MAX_INTERVAL], sum = 0.0;
    for (int j = 0; j < count[m]; j++) {
      e[j] = exp((double)lg[j] - mx);
      sum += e[j];
    }
    fa.start[m] = start[m];
    fa.count[m] = count[m];
    for (int j = 0; j < count[m]; j++) fa.w[m][j] = (float)(e[j] / sum);
  }
  hipStream_t s = (hipStream_t)stream;
  const long long le = (long long)src->B * src->Hh * src->cap * src->dh;
  HIPCK(fuse_kv(s, src->dtype, src->k, dst->k, le, fa));
  HIPCK(fuse_kv(s, src->dtype, src->v, dst->v, le, fa));
  for (int b = 0; b < src->B; b++) dst->len[b] = src->len[b];
  return WAM_OK;
}

static int max_len_of(const wam_kv* kv, int B) {
  int m = 0;
  if (kv)
    for (int b = 0; b < B; b++) m = std::max(m, (int)kv->len[b]);
  return m;
}

size_t wam_action_workspace_bytes(const wam_dims* d, int B, const wam_kv* kv) {
  if (check_dims(d) || B < 1 || B > WAM_MAX_BATCH) return 0;
  const wam_dims dav = action_view(d);
  d = &dav;
  Arena a(nullptr);
  Bufs b;
  plan_action(a, d, B, kv ? std::max(max_len_of(kv, B), kv->cap) : 0, false, b);
  return a.off + 256;
}

size_t wam_denoise_workspace_bytes(const wam_dims* d, int B, const wam_kv* kv) {
  if (check_dims(d) || B < 1 || B > WAM_MAX_BATCH) return 0;
  const wam_dims dav = action_view(d);
  d = &dav;
  Arena a(nullptr);
  Bufs b;
  plan_action(a, d, B, kv ? std::max(max_len_of(kv, B), kv->cap) : 0, true, b);
  return a.off + 256;
}

static int check_lens(const wam_kv* kv, int B, ActLens* lens) {
  for (int b = 0; b < B; b++) {
    if (kv->len[b] < 0 || kv->len[b] > kv->cap)
      return fail(WAM_E_SHAPE, "len[%d] = %d outside [0, cap]", b, kv->len[b]);
    lens->len[b] = kv->len[b];
  }
  return WAM_OK;
}

int wam_action_layer(const wam_dims* d, const wam_layer_w* w, float* x, const wam_kv* kv,
                     int kv_layer, const wam_kv* cond, int cond_layer, int B, void* ws,
                     size_t ws_bytes, void* stream) {
  int st;
  if ((st = check_dims(d))) return st;
  const wam_dims* d_in = d;
  const wam_dims dav = action_view(d);
  d = &dav;  // the action expert's shapes from here on
  if (!w || !x) return fail(WAM_E_ARG, "NULL pointer");
  if (!w->g1 || !w->wqkv || !w->wo || !w->g2 || !w->w1 || !w->w2)
    return fail(WAM_E_ARG, "layer has a NULL pointer");
  if (!aligned16(x)) return fail(WAM_E_ALIGN, "x not 16-byte aligned");
  if (B < 1 || B > WAM_MAX_BATCH) return fail(WAM_E_SHAPE, "bad B");
  if (d->Tc > 0) {
    if (!w->gx || !w->wqx || !w->wkvx || !w->wox)
      return fail(WAM_E_ARG, "layer has a NULL cross-attention pointer");
    if (!cond) return fail(WAM_E_ARG, "Tc > 0 needs the condition cache");
    if ((st = check_cond_kv(d, cond, B, cond->n_layers, "action"))) return st;
    if (cond_layer < 0 || cond_layer >= cond->n_layers) return fail(WAM_E_ARG, "cond_layer out of range");
    for (int i = 0; i < B; i++)
      if (cond->len[i] != d->Tc) return fail(WAM_E_SHAPE, "condition cache len[%d] != Tc", i);
  }
  ActLens lens{};
  if (kv) {
    if ((st = check_kv(d, kv, B, "kv", true))) return st;
    if (kv_layer < 0 || kv_layer >= kv->n_layers) return fail(WAM_E_ARG, "kv_layer out of range");
    if ((st = check_lens(kv, B, &lens))) return st;
  }
  if (!ws || !aligned16(ws) || ws_bytes < wam_action_workspace_bytes(d_in, B, kv))
    return fail(WAM_E_WORKSPACE, "workspace missing or too small");
  hipStream_t s = (hipStream_t)stream;
  Arena a(ws);
  Bufs b;
  plan_action(a, d, B, kv ? std::max(max_len_of(kv, B), kv->cap) : 0, false, b);
  const size_t bytes = (size_t)B * d->H * d->D * 4;
  HIPCK(hipMemcpyAsync(b.X, x, bytes, hipMemcpyDeviceToDevice, s));
  Layer c{s, d, &b};
  const void* kc = kv ? (const char*)kv->k + kv_layer * layer_stride(kv) : nullptr;
  const void* vc = kv ? (const char*)kv->v + kv_layer * layer_stride(kv) : nullptr;
  if ((st = action_layer(c, *w, B, kc, vc, kv ? kv->cap : 0, lens,
                         kv ? layer_scales(kv, kv->k_scale, kv_layer) : nullptr,
                         kv ? layer_scales(kv, kv->v_scale, kv_layer) : nullptr,
                         cond_ref(d, cond, cond_layer, 0))))
    return st;
  if ((st = flush_pending(c, w->g1, B * d->H))) return st;
  HIPCK(hipMemcpyAsync(x, b.X, bytes, hipMemcpyDeviceToDevice, s));
  return WAM_OK;
}

int wam_flow_euler_step(float* x, const float* v, int64_t n, float sigma, float sigma_next,
                        void* stream) {
  if (n < 0) return fail(WAM_E_ARG, "n < 0");
  if (n == 0) return WAM_OK;
  if (!x || !v) return fail(WAM_E_ARG, "NULL pointer");
  HIPCK(euler((hipStream_t)stream, x, v, n, sigma_next - sigma));
  return WAM_OK;
}

int wam_denoise_chunk(const wam_dims* d, const wam_expert_w* action, const wam_kv* kv,
                      const int32_t* read_map, const float* eps, int B, int N, double shift,
                      float* actions_out, float* vhat_out, void* ws, size_t ws_bytes,
                      void* stream) {
  int st;
  if ((st = check_dims(d))) return st;
  const wam_dims* d_in = d;
  const wam_dims dav = action_view(d);
  d = &dav;  // the action expert's shapes from here on
  if ((st = check_expert(d, action, "action"))) return st;
  if (!read_map || !eps || !actions_out) return fail(WAM_E_ARG, "NULL pointer");
  if (B >= 1 && B <= WAM_MAX_BATCH && (st = check_cond(d, action, B, "action"))) return st;
  if (!aligned16(eps) || !aligned16(actions_out) || (vhat_out && !aligned16(vhat_out)))
    return fail(WAM_E_ALIGN, "pointer not 16-byte aligned");
  if (B < 1 || B > WAM_MAX_BATCH) return fail(WAM_E_SHAPE, "bad B");
  if (N < 1 || N > WAM_MAX_STEPS) return fail(WAM_E_ARG, "N must be in [1, %d]", WAM_MAX_STEPS);
  if (!(shift > 0.0)) return fail(WAM_E_ARG, "shift must be > 0");
  ActLens lens{};
  bool any = false;
  for (int l = 0; l < d->L; l++) any |= read_map[l] >= 0;
  if (any) {
    if (!kv) return fail(WAM_E_ARG, "read_map reads a cache but kv is NULL");
    if ((st = check_kv(d, kv, B, "kv", true))) return st;
    if ((st = check_lens(kv, B, &lens))) return st;
    for (int l = 0; l < d->L; l++)
      if (read_map[l] >= kv->n_layers) return fail(WAM_E_ARG, "read_map[%d] out of range", l);
  }
  if (!ws || !aligned16(ws) || ws_bytes < wam_denoise_workspace_bytes(d_in, B, any ? kv : nullptr))
    return fail(WAM_E_WORKSPACE, "workspace missing or too small");

  hipStream_t s = (hipStream_t)stream;
  Arena a(ws);
  Bufs b;
  plan_action(a, d, B, any ? std::max(max_len_of(kv, B), kv->cap) : 0, true, b);
  float t[WAM_MAX_STEPS + 1];  // no host allocation on this path
  schedule(N, 0.0, shift, t);
  HIPCK(time_embedding(s, t, N, d->D, b.emb));
  const int M = B * d->H;
  HIPCK(hipMemcpyAsync(actions_out, eps, (size_t)M * d->A * 4, hipMemcpyDeviceToDevice, s));
  Layer c{s, d, &b};
  const size_t ls = any ? layer_stride(kv) : 0;
  // X = eps W_in^T + emb(t_0); then per step: layers, and one step-boundary
  // kernel doing head + Euler + the next step's embedding
  HIPCK(step_boundary(s, d->dtype, b.X, nullptr, nullptr, actions_out, 0.f, nullptr, action->w_in,
                      b.emb, M, d->D, d->A, false));
  for (int k = 0; k < N; k++) {
    for (int l = 0; l < d->L; l++) {
      const int r = read_map[l];
      const void* kc = r >= 0 ? (const char*)kv->k + r * ls : nullptr;
      const void* vc = r >= 0 ? (const char*)kv->v + r * ls : nullptr;
      if ((st = action_layer(c, action->layers[l], B, kc, vc, r >= 0 ? kv->cap : 0, lens,
                             r >= 0 ? layer_scales(kv, kv->k_scale, r) : nullptr,
                             r >= 0 ? layer_scales(kv, kv->v_scale, r) : nullptr,
                             cond_ref(d, action->cond, l, 0))))
        return st;
    }
    const bool last = (k + 1 == N);
    if ((st = flush_pending(c, action->g_out, M))) return st;
    HIPCK(step_boundary(s, d->dtype, b.X, action->g_out, action->w_out, actions_out,
                        t[k + 1] - t[k], vhat_out ? vhat_out + (size_t)k * M * d->A : nullptr,
                        last ? nullptr : action->w_in,
                        last ? nullptr : b.emb + (size_t)(k + 1) * d->D, M, d->D, d->A, true));
  }
  return WAM_OK;
}

// ----------------------------------------------------------------- no allocation
// Scratch of wam_denoise_chunk_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes `scratch`
// itself (its host-side name is not the device address): the address comes
// from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) char scratch[WAM_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[WAM_MAX_DEVICES] = {};

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WAM_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= WAM_MAX_DEVICES) return fail(WAM_E_ARG, "device %d beyond %d", dev, WAM_MAX_DEVICES);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(WAM_E_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WAM_OK;
}
}  // namespace

int wam_denoise_chunk_noalloc(const wam_dims* d, const wam_expert_w* action, const wam_kv* kv,
                              const int32_t* read_map, const float* eps, int B, int N, double shift,
                              float* actions_out, float* vhat_out, void* stream) {
  int st;
  if ((st = check_dims(d))) return st;
  if (!read_map) return fail(WAM_E_ARG, "NULL pointer");
  bool any = false;
  for (int l = 0; l < d->L; l++) any |= read_map[l] >= 0;
  const size_t need = wam_denoise_workspace_bytes(d, B, any ? kv : nullptr);
  if (need > WAM_NOALLOC_SCRATCH_BYTES)
    return fail(WAM_E_WORKSPACE,
                "this chunk needs %zu bytes of scratch; the static scratch holds %zu (use "
                "wam_denoise_chunk with a workspace)",
                need, (size_t)WAM_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return wam_denoise_chunk(d, action, kv, read_map, eps, B, N, shift, actions_out, vhat_out, ws,
                           WAM_NOALLOC_SCRATCH_BYTES, stream);
}

// ----------------------------------------------------------------- co-denoising
size_t wam_codenoise_workspace_bytes(const wam_dims* d, int B, int Ff, const wam_kv* cache) {
  if (check_dims(d) || B < 1 || B > WAM_MAX_BATCH || Ff < 1 || !cache) return 0;
  Arena a(nullptr);
  Bufs vb, ab;
  float* z;
  plan_prefill(a, d, 1, 0, Ff, vb, &z);
  const wam_dims da = action_view(d);
  plan_action(a, &da, B, cache->cap, true, ab);
  return a.off + 256;
}

int wam_codenoise_chunk(const wam_dims* d, const wam_expert_w* video, const wam_expert_w* action,
                        const uint8_t* hist_valid, int B, int Fh, const void* fut_noise, int Ff,
                        const int32_t* frame_block, const float* eps, int N,
                        double sigma_video_end, double shift, wam_kv* cache, float* actions_out,
                        float* fut_latents_out, float* vhat_out, void* ws, size_t ws_bytes,
                        void* stream) {
  int st;
  if ((st = check_dims(d))) return st;
  if ((st = check_expert(d, video, "video"))) return st;
  if ((st = check_expert(d, action, "action"))) return st;
  if (B < 1 || B > WAM_MAX_BATCH) return fail(WAM_E_SHAPE, "B must be in [1, %d]", WAM_MAX_BATCH);
  if ((st = check_cond(d, video, B, "video")) || (st = check_cond(d, action, B, "action"))) return st;
  if (Fh < 0 || Ff < 1 || Fh + Ff > WAM_MAX_FRAMES)
    return fail(WAM_E_SHAPE, "co-denoising needs Ff >= 1 and Fh + Ff <= %d", WAM_MAX_FRAMES);
  if (!fut_noise || !eps || !actions_out || !fut_latents_out || !frame_block)
    return fail(WAM_E_ARG, "NULL pointer");
  if (!aligned16(fut_noise) || !aligned16(eps) || !aligned16(actions_out) ||
      !aligned16(fut_latents_out) || (vhat_out && !aligned16(vhat_out)))
    return fail(WAM_E_ALIGN, "pointer not 16-byte aligned");
  if ((st = check_blocks(frame_block, Fh + Ff))) return st;
  if (N < 1 || N > WAM_MAX_STEPS) return fail(WAM_E_ARG, "N must be in [1, %d]", WAM_MAX_STEPS);
  if (!(sigma_video_end >= 0.0 && sigma_video_end < 1.0))
    return fail(WAM_E_ARG, "sigma_video_end must be in [0, 1)");
  if (!(shift > 0.0)) return fail(WAM_E_ARG, "shift must be > 0");
  if (!cache) return fail(WAM_E_ARG, "cache is NULL");
  if ((st = check_kv(d, cache, B, "cache"))) return st;
  if (cache->n_layers != d->L) return fail(WAM_E_SHAPE, "cache must hold L layers");
  if (!ws || !aligned16(ws) || ws_bytes < wam_codenoise_workspace_bytes(d, B, Ff, cache))
    return fail(WAM_E_WORKSPACE, "workspace missing or too small");

  // frame tables; the cache must hold exactly the valid history rows
  const int P = d->P;
  std::vector<FrameTab> tabs(B);
  std::vector<int> nh(B);
  ActLens lens{};
  for (int b = 0; b < B; b++) {
    int src[WAM_MAX_FRAMES], kend[WAM_MAX_FRAMES];
    const uint8_t* v = hist_valid ? hist_valid + (size_t)b * Fh : nullptr;
    const int n = frame_table(frame_block, v, Fh, Ff, P, src, kend);
    if (n == 0) return fail(WAM_E_SHAPE, "episode %d has no valid frame", b);
    if ((long long)n * P > cache->cap)
      return fail(WAM_E_SHAPE, "episode %d needs %d cache rows, cap is %d", b, n * P, cache->cap);
    nh[b] = n - Ff;
    if (cache->len[b] != nh[b] * P)
      return fail(WAM_E_SHAPE, "episode %d: cache holds %d rows, its valid history has %d", b,
                  cache->len[b], nh[b] * P);
    tabs[b].n = n;
    tabs[b].P = P;
    for (int i = 0; i < n; i++) tabs[b].kend[i] = kend[i];
    lens.len[b] = n * P;
  }

  hipStream_t s = (hipStream_t)stream;
  Arena a(ws);
  Bufs vb, ab;
  float* zs;
  plan_prefill(a, d, 1, 0, Ff, vb, &zs);
  const wam_dims da = action_view(d);
  plan_action(a, &da, B, cache->cap, true, ab);
  std::vector<float> sv(N + 1), ta(N + 1);
  schedule(N, sigma_video_end, shift, sv.data());
  schedule(N, 0.0, shift, ta.data());
  const int D = d->D, dt = d->dtype, M = B * d->H, Tf = Ff * P;
  HIPCK(time_embedding(s, sv.data(), N, D, vb.emb));
  HIPCK(time_embedding(s, ta.data(), N, da.D, ab.emb));
  for (int b = 0; b < B; b++)
    HIPCK(copy_cvt_f32(s, dt, (const char*)fut_noise + (size_t)b * Tf * d->Cv * esz(dt),
                       fut_latents_out + (size_t)b * Tf * d->Cv, (int64_t)Tf * d->Cv));
  HIPCK(hipMemcpyAsync(actions_out, eps, (size_t)M * d->A * 4, hipMemcpyDeviceToDevice, s));
  HIPCK(step_boundary(s, dt, ab.X, nullptr, nullptr, actions_out, 0.f, nullptr, action->w_in,
                      ab.emb, M, da.D, d->A, false));

  Layer cv{s, d, &vb}, ca{s, &da, &ab};
  const size_t ls = layer_stride(cache);
  const size_t ep = (size_t)d->Hh * cache->cap * d->dh * esz(dt);  // one episode in a layer
  RowMap zmap;
  zmap.n = 1;
  zmap.P = Tf;
  zmap.src[0] = 0;
  for (int k = 0; k < N; k++) {
    // 1. the video pass at sigma_k of every episode (future K/V into the cache)
    for (int b = 0; b < B; b++) {
      float* z = fut_latents_out + (size_t)b * Tf * d->Cv;
      const int Th = nh[b] * P;
      HIPCK(embed(s, WAM_F32, dt, z, zmap, video->w_in, vb.emb + (size_t)k * D, vb.X, Tf, D,
                  d->Cv));
      for (int l = 0; l < d->L; l++) {
        char* kl = (char*)cache->k + l * ls + b * ep;
        char* vl = (char*)cache->v + l * ls + b * ep;
        if ((st = video_layer(cv, video->layers[l], Tf, Th, tabs[b], kl, vl, cache->cap, false,
                              cond_ref(d, video->cond, l, b))))
          return st;
      }
      if ((st = flush_pending(cv, video->g_out, Tf))) return st;
      HIPCK(step_boundary(s, dt, vb.X, video->g_out, video->w_out, z, sv[k + 1] - sv[k], nullptr,
                          nullptr, nullptr, Tf, D, d->Cv, true));
    }
    // 2. the action pass at t_k over [history ; future at sigma_k], 3. Euler
    for (int l = 0; l < d->L; l++) {
      const void* kc = (const char*)cache->k + l * ls;
      const void* vc = (const char*)cache->v + l * ls;
      if ((st = action_layer(ca, action->layers[l], B, kc, vc, cache->cap, lens, nullptr, nullptr,
                             cond_ref(d, action->cond, l, 0))))
        return st;
    }
    const bool last = (k + 1 == N);
    if ((st = flush_pending(ca, action->g_out, M))) return st;
    HIPCK(step_boundary(s, dt, ab.X, action->g_out, action->w_out, actions_out, ta[k + 1] - ta[k],
                        vhat_out ? vhat_out + (size_t)k * M * d->A : nullptr,
                        last ? nullptr : action->w_in,
                        last ? nullptr : ab.emb + (size_t)(k + 1) * da.D, M, da.D, d->A, true));
  }
  for (int b = 0; b < B; b++) cache->len[b] = lens.len[b];
  return WAM_OK;
}

size_t wam_condition_workspace_bytes(const wam_dims* d, int B) {
  if (check_dims(d) || B < 1 || B > WAM_MAX_BATCH || d->Tc < 1) return 0;
  return (size_t)B * d->Tc * d->Ct * esz(d->dtype) + 256;
}

int wam_prefill_condition_kv(const wam_dims* d, const wam_expert_w* video, const wam_expert_w* action,
                             const void* proprio_w, const void* text, const float* state, int B,
                             wam_kv* cond_video, wam_kv* cond_action, void* ws, size_t ws_bytes,
                             void* stream) {
  int st;
  if ((st = check_dims(d))) return st;
  if (d->Tc < 1) return fail(WAM_E_SHAPE, "no condition (Tc = 0)");
  if (B < 1 || B > WAM_MAX_BATCH) return fail(WAM_E_SHAPE, "bad B");
  if (!video && !action) return fail(WAM_E_ARG, "no expert given");
  if (!proprio_w || !state || (d->Tc > 1 && !text)) return fail(WAM_E_ARG, "NULL pointer");
  if (!aligned16(proprio_w) || !aligned16(state) || (text && !aligned16(text)))
    return fail(WAM_E_ALIGN, "pointer not 16-byte aligned");
  const wam_dims dav = action_view(d);
  if (video) {
    if ((st = check_expert(d, video, "video"))) return st;
    if ((st = check_cond_kv(d, cond_video, B, video->n_layers, "video"))) return st;
  }
  if (action) {
    if ((st = check_expert(&dav, action, "action"))) return st;
    if ((st = check_cond_kv(d, cond_action, B, action->n_layers, "action"))) return st;
  }
  if (!ws || !aligned16(ws) || ws_bytes < wam_condition_workspace_bytes(d, B))
    return fail(WAM_E_WORKSPACE, "workspace missing or too small");
  hipStream_t s = (hipStream_t)stream;
  const int dt = d->dtype, Tc = d->Tc, Ct = d->Ct, S = state_dims(d), Dq = d->Hh * d->dh;
  const size_t es = esz(dt);
  char* ctx = (char*)ws;  // [B][Tc][Ct]: text rows, then the proprio token
  if (Tc > 1)
    HIPCK(hipMemcpy2DAsync(ctx, (size_t)Tc * Ct * es, text, (size_t)(Tc - 1) * Ct * es,
                           (size_t)(Tc - 1) * Ct * es, B, hipMemcpyDeviceToDevice, s));
  EpiArgs pe{};
  pe.out = ctx + (size_t)(Tc - 1) * Ct * es;
  pe.ldo = Tc * Ct;
  HIPCK(gemm(s, WAM_F32, dt, dt, EPI_STORE, B, Ct, S, state, S, proprio_w, S, pe));
  const wam_expert_w* ex[2] = {video, action};
  wam_kv* cc[2] = {cond_video, cond_action};
  for (int i = 0; i < 2; i++) {
    if (!ex[i]) continue;
    wam_kv* c = cc[i];
    const size_t ls = layer_stride(c);
    for (int l = 0; l < ex[i]->n_layers; l++) {
      EpiArgs e{};
      e.k = (char*)c->k + l * ls;
      e.v = (char*)c->v + l * ls;
      e.D = Dq;
      e.dh = d->dh;
      e.rpg = Tc;
      e.n_begin = Dq;  // the K and V parts of [Q | K | V]
      e.q_scale = 1.0f;
      e.k_gs = e.v_gs = (long long)d->Hh * c->cap * d->dh;
      e.k_hs = (long long)c->cap * d->dh;
      e.v_hs = (long long)d->dh * c->cap;
      e.v_ld = c->cap;
      HIPCK(gemm(s, dt, dt, dt, EPI_QKV, B * Tc, 2 * Dq, Ct, ctx, Ct, ex[i]->layers[l].wkvx, Ct, e));
    }
    for (int b = 0; b < B; b++) c->len[b] = Tc;
  }
  return WAM_OK;
}

int wam_debug_visibility(const int32_t* frame_block, const uint8_t* valid, int Fh, int Ff, int P,
                         uint8_t* vis, void* stream) {
  if (!frame_block || !vis) return fail(WAM_E_ARG, "NULL pointer");
  if (Fh < 0 || Ff < 0 || Fh + Ff < 1 || Fh + Ff > WAM_MAX_FRAMES || P < 1)
    return fail(WAM_E_SHAPE, "bad frame counts");
  int st;
  if ((st = check_blocks(frame_block, Fh + Ff))) return st;
  int src[WAM_MAX_FRAMES], kend[WAM_MAX_FRAMES];
  int n = frame_table(frame_block, valid, Fh, Ff, P, src, kend);
  FrameTab tab;
  tab.n = n;
  tab.P = P;
  for (int i = 0; i < n; i++) tab.kend[i] = kend[i];
  int comp[WAM_MAX_FRAMES];
  for (int f = 0; f < Fh + Ff; f++) comp[f] = -1;
  for (int i = 0; i < n; i++) comp[src[i]] = i;
  HIPCK(debug_visibility((hipStream_t)stream, tab, comp, Fh + Ff, vis));
  return WAM_OK;
}

static int attention_action_entry(int dtype, int B, int Hh, int dh, int H, const void* q,
                                  const void* ka, const void* va, int n_act, const void* kc,
                                  const void* vc, const float* ksc, const float* vsc, int cap,
                                  const int32_t* len, void* out, int splits_hint, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (dtype != WAM_F32 && dtype != WAM_BF16) return fail(WAM_E_ARG, "bad dtype");
  if (ksc && (!kc || !vsc)) return fail(WAM_E_ARG, "an E4M3 cache needs kc, vc and both scales");
  if ((dh != 64 && dh != 128) || H != 32) return fail(WAM_E_SHAPE, "dh must be 64 or 128 and H 32");
  if (B < 1 || B > WAM_MAX_BATCH || Hh < 1) return fail(WAM_E_SHAPE, "bad B or Hh");
  if (!q || !out) return fail(WAM_E_ARG, "NULL pointer");
  if (n_act < 0 || n_act > H || (n_act > 0 && (!ka || !va)))
    return fail(WAM_E_ARG, "bad own keys");
  if ((kc == nullptr) != (vc == nullptr)) return fail(WAM_E_ARG, "kc and vc must both be set");
  if (splits_hint < 0 || splits_hint > 63) return fail(WAM_E_ARG, "splits_hint must be in [0, 63]");
  ActLens lens{};
  int max_len = 0;
  if (kc) {
    if (!len) return fail(WAM_E_ARG, "len is NULL");
    if (cap < 64 || cap % 64) return fail(WAM_E_SHAPE, "cap must be a multiple of 64");
    for (int b = 0; b < B; b++) {
      if (len[b] < 0 || len[b] > cap) return fail(WAM_E_SHAPE, "len out of range");
      lens.len[b] = len[b];
      max_len = std::max(max_len, (int)len[b]);
    }
  }
  for (int b = 0; b < B; b++)
    if ((kc ? lens.len[b] : 0) + n_act == 0) return fail(WAM_E_SHAPE, "episode %d has no key", b);
  const void* ptrs[] = {q, ka, va, kc, vc, out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(WAM_E_ALIGN, "pointer not 16-byte aligned");
  size_t need = dtype == WAM_BF16 ? attn_action_scratch_bytes(B, Hh, H, dh, max_len, splits_hint) : 0;
  if (need && (!ws || ws_bytes < need)) return fail(WAM_E_WORKSPACE, "workspace too small (%zu)", need);
  HIPCK(attn_action((hipStream_t)stream, dtype, B, Hh, H, dh, q, ka, va, n_act, kc, vc, cap, lens, out,
                    splits_hint, ws, ws_bytes, ksc, vsc));
  return WAM_OK;
}

int wam_attention_action(int dtype, int B, int Hh, int dh, int H, const void* q, const void* ka,
                         const void* va, int n_act, const void* kc, const void* vc, int cap,
                         const int32_t* len, void* out, int splits_hint, void* ws,
                         size_t ws_bytes, void* stream) {
  return attention_action_entry(dtype, B, Hh, dh, H, q, ka, va, n_act, kc, vc, nullptr, nullptr,
                                cap, len, out, splits_hint, ws, ws_bytes, stream);
}

int wam_attention_action_fp8(int B, int Hh, int dh, int H, const void* q, const void* ka,
                             const void* va, int n_act, const void* kc8, const void* vc8,
                             const float* k_scale, const float* v_scale, int cap,
                             const int32_t* len, void* out, int splits_hint, void* ws,
                             size_t ws_bytes, void* stream) {
  if (!kc8 || !vc8 || !k_scale || !v_scale) return fail(WAM_E_ARG, "NULL cache pointer");
  return attention_action_entry(WAM_BF16, B, Hh, dh, H, q, ka, va, n_act, kc8, vc8, k_scale,
                                v_scale, cap, len, out, splits_hint, ws, ws_bytes, stream);
}

int wam_quantize_kv_fp8(const wam_kv* src, wam_kv* dst, void* stream) {
  if (!src || !dst) return fail(WAM_E_ARG, "NULL pointer");
  if (!src->k || !src->v || !src->len || !dst->k || !dst->v || !dst->len || !dst->k_scale ||
      !dst->v_scale)
    return fail(WAM_E_ARG, "NULL cache pointer");
  if (!aligned16(src->k) || !aligned16(src->v) || !aligned16(dst->k) || !aligned16(dst->v))
    return fail(WAM_E_ALIGN, "cache not 16-byte aligned");
  if (src->dtype != WAM_BF16 || dst->dtype != WAM_FP8)
    return fail(WAM_E_DTYPE, "src must be WAM_BF16 and dst WAM_FP8");
  if (src->n_layers != dst->n_layers || src->B != dst->B || src->Hh != dst->Hh ||
      src->dh != dst->dh || src->cap != dst->cap)
    return fail(WAM_E_SHAPE, "src and dst shapes differ");
  if (src->dh != 64 && src->dh != 128) return fail(WAM_E_SHAPE, "dh must be 64 or 128");
  if (src->n_layers < 1 || src->Hh < 1) return fail(WAM_E_SHAPE, "bad n_layers or Hh");
  if (src->B < 1 || src->B > WAM_MAX_BATCH) return fail(WAM_E_SHAPE, "bad B");
  if (src->cap < 64 || src->cap % 64) return fail(WAM_E_SHAPE, "cap must be a positive multiple of 64");
  ActLens lens{};
  for (int b = 0; b < src->B; b++) {
    if (src->len[b] < 0 || src->len[b] > src->cap)
      return fail(WAM_E_SHAPE, "len[%d] = %d outside [0, cap]", b, src->len[b]);
    lens.len[b] = src->len[b];
  }
  HIPCK(quantize_kv_fp8((hipStream_t)stream, src->k, src->v, dst->k, dst->v, dst->k_scale,
                        dst->v_scale, src->n_layers, src->B, src->Hh, src->dh, src->cap, lens));
  for (int b = 0; b < src->B; b++) dst->len[b] = src->len[b];
  return WAM_OK;
}

int wam_attention_prefill(int dtype, int Hh, int dh, int nq, int row0, int P, const int32_t* kend,
                          int n_frames, const void* q, const void* kc, const void* vc, int cap,
                          void* out, void* stream) {
  if (dtype != WAM_F32 && dtype != WAM_BF16) return fail(WAM_E_ARG, "bad dtype");
  if ((dh != 64 && dh != 128) || Hh < 1 || nq < 0 || row0 < 0 || P < 1)
    return fail(WAM_E_SHAPE, "bad shape");
  if (!kend || !q || !kc || !vc || !out) return fail(WAM_E_ARG, "NULL pointer");
  if (n_frames < 1 || n_frames > WAM_MAX_FRAMES) return fail(WAM_E_SHAPE, "bad n_frames");
  if (cap < 64 || cap % 64) return fail(WAM_E_SHAPE, "cap must be a multiple of 64");
  if ((row0 + nq + P - 1) / P > n_frames) return fail(WAM_E_SHAPE, "query rows beyond the frame table");
  FrameTab tab;
  tab.n = n_frames;
  tab.P = P;
  for (int i = 0; i < n_frames; i++) {
    if (kend[i] < 1 || kend[i] > cap || (i && kend[i] < kend[i - 1]))
      return fail(WAM_E_SHAPE, "kend must be non-decreasing in [1, cap]");
    tab.kend[i] = kend[i];
  }
  const void* ptrs[] = {q, kc, vc, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(WAM_E_ALIGN, "pointer not 16-byte aligned");
  HIPCK(attn_prefill((hipStream_t)stream, dtype, Hh, dh, nq, row0, tab, q, kc, vc, cap, out, nullptr, 0));
  return WAM_OK;
}

}  // extern "C"
