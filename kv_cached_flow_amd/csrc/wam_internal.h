// Internal declarations of libwam: device helpers, kernel-argument structs
// and the launchers the C-ABI layer calls.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/wam.h"

namespace wam {

typedef uint16_t bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

// ---------------------------------------------------------------- bf16
__host__ __device__ inline float bf2f(bf16_t h) {
  union { uint32_t u; float f; } x;
  x.u = (uint32_t)h << 16;
  return x.f;
}

// Round to nearest even; NaN stays NaN.
__host__ __device__ inline bf16_t f2bf(float f) {
  union { uint32_t u; float f; } x;
  x.f = f;
  uint32_t u = x.u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ inline float to_f(T v);
template <> __device__ inline float to_f<float>(float v) { return v; }
template <> __device__ inline float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

// Device conversion to bf16 uses the gfx950 v_cvt_pk_bf16_f32 instruction
// (round to nearest even, like f2bf).
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 hbf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float hfloat2;
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  hfloat2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hbf16x2));
}
__device__ inline bf16_t dev_f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename T> __device__ inline T from_f(float v);
template <> __device__ inline float from_f<float>(float v) { return v; }
template <> __device__ inline bf16_t from_f<bf16_t>(float v) { return dev_f2bf(v); }

__device__ inline float gelu_f(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

// Wait until every vector-memory load of this wave has completed, including
// global_load_lds transfers into LDS.  A barrier alone does not imply this:
// its lowering waits for LDS instructions but not necessarily for those
// transfers.  (s_waitcnt vmcnt(0), expcnt and lgkmcnt left free.)
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// GELU for results rounded to bf16 next: x Phi(x) with the normal tail
// 1 - Phi(|x|) = erfc(z)/2, z = |x|/sqrt 2, from Abramowitz & Stegun 7.1.26,
// erfc(z) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1/(1 + p z),
// absolute error <= 1.5e-7 (some 2^-22, far below the 2^-9 bf16 step).  The
// tail is used directly for x < 0, so small Phi keeps its relative accuracy.
__device__ inline float gelu_bf16out(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float poly = fmaf(t, 1.061405429f, -1.453152027f);
  poly = fmaf(t, poly, 1.421413741f);
  poly = fmaf(t, poly, -0.284496736f);
  poly = fmaf(t, poly, 0.254829592f);
  // exp(-z^2) = 2^(-z^2 log2 e); the argument underflows cleanly to 0 for large z
  const float e = __builtin_amdgcn_exp2f(-(z * z) * 1.44269504088896341f);
  const float tail = 0.5f * t * poly * e;  // 1 - Phi(|x|)
  return x * (x >= 0.f ? 1.0f - tail : tail);
}

// ---------------------------------------------------------------- block table
// Compacted frames of one episode: tokens of compacted frame i occupy cache
// rows [i*P, (i+1)*P); a query in compacted frame i sees rows [0, kend[i]).
struct FrameTab {
  int n;
  int P;
  int kend[WAM_MAX_FRAMES];
};

// The one visibility predicate of the block-causal attention (query cache
// row qr sees key cache row kr).  Used by the attention kernels and the
// debug export.
__device__ inline int kend_of_row(const FrameTab& t, int qr) { return t.kend[qr / t.P]; }
__device__ inline bool visible(const FrameTab& t, int qr, int kr) { return kr < kend_of_row(t, qr); }

// ---------------------------------------------------------------- GEMM epilogues
enum EpiKind {
  EPI_STORE = 0,   // out[m*ldo + n] = v                    (out type TO)
  EPI_GELU = 1,    // out[m*ldo + n] = GELU(v)              (out type TO)
  EPI_RESID = 2,   // X[m*ldo + n] += v                     (fp32)
  EPI_QKV = 3      // scatter to Q / K cache / V^T cache    (out type TO)
};

struct EpiArgs {
  void* out;      // STORE/GELU/RESID destination
  int ldo;
  // QKV: column n_begin + n of [Q | K | V] (each D wide), row m -> group g = m / rpg, t = m % rpg
  void* q;
  void* k;
  void* v;
  int D, dh, rpg, n_begin;
  // Q part: the fp32 accumulator is multiplied by q_scale before its one
  // rounding to the output type (bf16 models: log2(e) / sqrt(dh), so that the
  // attention kernels' score MFMAs yield log2-domain scores; fp32 models: 1)
  float q_scale;
  long long q_gs, q_hs;          // q[g*q_gs + h*q_hs + t*dh + d]
  long long k_gs, k_hs;          // k[g*k_gs + h*k_hs + (k_row0 + t)*dh + d]
  long long v_gs, v_hs;          // v[g*v_gs + h*v_hs + d*v_ld + v_col0 + t]
  int k_row0, v_ld, v_col0;
};

template <int EPI, typename TO>
__device__ inline void epi_store(const EpiArgs& e, int m, int n, float v) {
  if constexpr (EPI == EPI_STORE) {
    ((TO*)e.out)[(long long)m * e.ldo + n] = from_f<TO>(v);
  } else if constexpr (EPI == EPI_GELU) {
    ((TO*)e.out)[(long long)m * e.ldo + n] =
        from_f<TO>(sizeof(TO) == 2 ? gelu_bf16out(v) : gelu_f(v));
  } else if constexpr (EPI == EPI_RESID) {
    ((float*)e.out)[(long long)m * e.ldo + n] += v;
  } else {
    int nn = e.n_begin + n;
    int part = nn / e.D;
    int c = nn - part * e.D;
    int h = c / e.dh, d = c - h * e.dh;
    int g = m / e.rpg, t = m - g * e.rpg;
    if (part == 0)
      ((TO*)e.q)[g * e.q_gs + h * e.q_hs + (long long)t * e.dh + d] = from_f<TO>(v * e.q_scale);
    else if (part == 1)
      ((TO*)e.k)[g * e.k_gs + h * e.k_hs + (long long)(e.k_row0 + t) * e.dh + d] = from_f<TO>(v);
    else
      ((TO*)e.v)[g * e.v_gs + h * e.v_hs + (long long)d * e.v_ld + e.v_col0 + t] = from_f<TO>(v);
  }
}

// ---------------------------------------------------------------- launchers
// C[M][N] = A[M][K] * B[N][K]^T with the epilogue; adt/bdt/odt are WAM_F32 or
// WAM_BF16 (A, B and epilogue output element types).
hipError_t gemm(hipStream_t s, int adt, int bdt, int odt, int epi, int M, int N, int K,
                const void* A, int lda, const void* B, int ldb, const EpiArgs& e);

// bf16 action rows (M <= 128): raw fp32 split-K partials part[ks][M][N],
// ks < *ks_out; the consumer adds them in ks order (rmsnorm_accum does).
int gemm_partial_splits(int M, int N, int K);
hipError_t gemm_partial(hipStream_t s, int M, int N, int K, const void* A, int lda, const void* B,
                        int ldb, float* part, int* ks_out);

// bf16 rows whose tiles leave CUs idle (M in the thousands): the same split
// partials with the large-tile kernel; gemm_big_splits gives the split count
// (1: do not split).
int gemm_big_splits(int M, int N, int K);
hipError_t gemm_big_partial(hipStream_t s, int M, int N, int K, const void* A, int lda,
                            const void* B, int ldb, float* part, int ks);

hipError_t rmsnorm(hipStream_t s, int odt, const float* x, const float* g, void* y, int M, int D);
// x[m] += sum_{ks < KS} part[ks][m] (in ks order), then y = RMSNorm(x; g).
hipError_t rmsnorm_accum(hipStream_t s, int odt, float* x, const float* part, int KS,
                         const float* g, void* y, int M, int D);

// X[m][n] = sum_c x[row(m)][c] * w_in[n][c] + emb[n]; rows are gathered by
// frame: m -> frame src[m / P], token m % P, of a [*][P][C] input.
struct RowMap {
  int n;
  int P;
  int src[WAM_MAX_FRAMES];
};
hipError_t embed(hipStream_t s, int xdt, int wdt, const void* x, const RowMap& map,
                 const void* w_in, const float* emb, float* X, int M, int D, int C);

// emb[i][0..D) for sigma[i], i < n (float64 on the device, stored fp32).
hipError_t time_embedding(hipStream_t s, const float* sigma_host, int n, int D, float* emb);

hipError_t euler(hipStream_t s, float* x, const float* v, int64_t n, float dt);

// Step boundary of the flow, one workgroup per row: optionally the velocity
// head and Euler update (z += dt * RMSNorm(X; g_out) W_out^T, vhat = the
// velocity), then optionally the next embedding X = z W_in^T + emb_next.
hipError_t step_boundary(hipStream_t s, int wdt, float* X, const float* g_out, const void* w_out,
                         float* z, float dt, float* vhat, const void* w_in, const float* emb_next,
                         int M, int D, int C, bool do_head);
hipError_t copy_cvt_f32(hipStream_t s, int sdt, const void* src, float* dst, int64_t n);

struct FuseArgs {
  int M;
  int count[WAM_MAX_FUSE];
  int start[WAM_MAX_FUSE];
  float w[WAM_MAX_FUSE][WAM_MAX_INTERVAL];
};
hipError_t fuse_kv(hipStream_t s, int dt, const void* src, void* dst, long long layer_elems,
                   const FuseArgs& a);

// part / part_bytes: workspace for split partials (bf16 launches with few
// query tiles split their keys and merge; NULL: never split).
// dh is 64 or 128.  n_ep episodes with the same frame table in one launch:
// episode e's queries at q + e Hh nq dh, its output rows at out + e nq Hh dh,
// its cache at kc / vc + e kv_ep (elements).
hipError_t attn_prefill(hipStream_t s, int dt, int Hh, int dh, int nq, int row0,
                        const FrameTab& tab, const void* q, const void* kc, const void* vc, int cap,
                        void* out, float* part, size_t part_bytes, int n_ep = 1,
                        long long kv_ep = 0);
// Partial workspace a prefill of up to max_rows query rows can use.
size_t attn_prefill_split_bytes(int Hh, int dh, int max_rows);

struct ActLens {
  int len[WAM_MAX_BATCH];
};
size_t attn_action_scratch_bytes(int B, int Hh, int H, int dh, int max_len, int splits_hint);
// ksc/vsc non-NULL: kc/vc is an E4M3 cache layer (bf16 model) with these
// per-(episode, head, 64-key tile) scales, [B][Hh][cap/64].
hipError_t attn_action(hipStream_t s, int dt, int B, int Hh, int H, int dh, const void* q,
                       const void* ka, const void* va, int n_act, const void* kc,
                       const void* vc, int cap, const ActLens& lens, void* out,
                       int splits_hint, void* scratch, size_t scratch_bytes,
                       const float* ksc = nullptr, const float* vsc = nullptr);

// bf16 cache (n_layers x B episodes) -> E4M3 cache with power-of-two tile
// scales, rows [0, len[b]) of every episode.
// Rotary position embedding in place on x0 (and x1 unless NULL), layout
// [G][Hh][rows][dh] with group stride gs and head stride hs (elements); row r
// of group g sits at position base[g] + r.
struct RopeRows {
  int base[WAM_MAX_BATCH];
};
hipError_t rope_qk(hipStream_t s, int dt, void* x0, long long gs0, long long hs0, void* x1,
                   long long gs1, long long hs1, int G, int rows, int Hh, int dh,
                   const RopeRows& rb);

hipError_t quantize_kv_fp8(hipStream_t s, const void* k, const void* v, void* k8, void* v8,
                           float* ks, float* vs, int n_layers, int B, int Hh, int dh, int cap,
                           const ActLens& lens);

hipError_t debug_visibility(hipStream_t s, const FrameTab& tab, const int* comp_of_frame,
                            int F, uint8_t* vis);

// ---------------------------------------------------------------- timing
enum KClass {
  KC_GEMM_BIG, KC_GEMM_SKINNY, KC_GEMM_SIMPLE, KC_ATTN_PREFILL, KC_ATTN_ACTION,
  KC_ATTN_MERGE, KC_RMSNORM, KC_EMBED, KC_FUSE, KC_QUANT, KC_MISC, KC_COUNT
};
// RAII event pair around the launches of one kernel class (no-op unless
// wam_timing(1) was called); bytes/flops are the algorithmic work.
class TimingScope {
 public:
  TimingScope(hipStream_t s, int cls, double bytes, double flops);
  ~TimingScope();

 private:
  hipStream_t s_;
  int cls_;
  double bytes_, flops_;
  void* a_;
};

}  // namespace wam
