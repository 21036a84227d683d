// Elementwise and row-wise kernels: RMSNorm, token embedding (+ time
// embedding), Euler update, dtype conversion, Interval KV-Fusion.
#include "wam_internal.h"

namespace wam {

// ------------------------------------------------------------ RMSNorm
// One wavefront per row: (optionally x += sum of split partials, written
// back), then y = x * (mean(x^2) + 1e-6)^(-1/2) * g.
template <typename TO, bool ACC, int MAXV = 8>  // D <= 256 MAXV
__global__ __launch_bounds__(256) void rmsnorm_kernel(float* __restrict__ x,
                                                      const float* __restrict__ part, int KS,
                                                      const float* __restrict__ g,
                                                      TO* __restrict__ y, int M, int D) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  float* xr = x + (long long)row * D;
  float4 v[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV; j++) {
    const int i = lane * 4 + 256 * j;
    if (i < D) {
      float4 t = *(const float4*)(xr + i);
      if (ACC) {
        for (int k = 0; k < KS; k++) {
          float4 p = *(const float4*)(part + ((long long)k * M + row) * D + i);
          t.x += p.x;
          t.y += p.y;
          t.z += p.z;
          t.w += p.w;
        }
        *(float4*)(xr + i) = t;
      }
      v[j] = t;
      ss = fmaf(t.x, t.x, ss);
      ss = fmaf(t.y, t.y, ss);
      ss = fmaf(t.z, t.z, ss);
      ss = fmaf(t.w, t.w, ss);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float r = 1.0f / sqrtf(ss / (float)D + 1e-6f);
  TO* yr = y + (long long)row * D;
#pragma unroll
  for (int j = 0; j < MAXV; j++) {
    const int i = lane * 4 + 256 * j;
    if (i < D) {
      float4 gg = *(const float4*)(g + i);
      TO o4[4] = {from_f<TO>(v[j].x * r * gg.x), from_f<TO>(v[j].y * r * gg.y),
                  from_f<TO>(v[j].z * r * gg.z), from_f<TO>(v[j].w * r * gg.w)};
      if constexpr (sizeof(TO) == 2)
        *(uint2*)(yr + i) = *(uint2*)o4;
      else
        *(float4*)(yr + i) = *(float4*)o4;
    }
  }
}

// One workgroup per row (small M): thread t owns columns 4t..4t+3 (+1024 j),
// D <= 1024 NJ; all loads of a thread are issued before any reduction.
template <typename TO, bool ACC, int NJ = 2>
__global__ __launch_bounds__(256) void rmsnorm_row_kernel(float* __restrict__ x,
                                                          const float* __restrict__ part, int KS,
                                                          const float* __restrict__ g,
                                                          TO* __restrict__ y, int M, int D) {
  __shared__ float wss[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* xr = x + (long long)row * D;
  float4 v[NJ];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    const int i = 4 * tid + 1024 * j;
    if (i < D) {
      float4 t = *(const float4*)(xr + i);
      if (ACC) {
        float4 p[4];
#pragma unroll
        for (int k = 0; k < 4; k++)
          if (k < KS) p[k] = *(const float4*)(part + ((long long)k * M + row) * D + i);
#pragma unroll
        for (int k = 0; k < 4; k++)
          if (k < KS) {
            t.x += p[k].x;
            t.y += p[k].y;
            t.z += p[k].z;
            t.w += p[k].w;
          }
        *(float4*)(xr + i) = t;
      }
      v[j] = t;
      ss = fmaf(t.x, t.x, ss);
      ss = fmaf(t.y, t.y, ss);
      ss = fmaf(t.z, t.z, ss);
      ss = fmaf(t.w, t.w, ss);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) wss[w] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((((wss[0] + wss[1]) + wss[2]) + wss[3]) / (float)D + 1e-6f);
  TO* yr = y + (long long)row * D;
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    const int i = 4 * tid + 1024 * j;
    if (i < D) {
      const float4 gg = *(const float4*)(g + i);
      TO o4[4] = {from_f<TO>(v[j].x * r * gg.x), from_f<TO>(v[j].y * r * gg.y),
                  from_f<TO>(v[j].z * r * gg.z), from_f<TO>(v[j].w * r * gg.w)};
      if constexpr (sizeof(TO) == 2)
        *(uint2*)(yr + i) = *(uint2*)o4;
      else
        *(float4*)(yr + i) = *(float4*)o4;
    }
  }
}

template <bool ACC>
static hipError_t rmsnorm_launch(hipStream_t s, int odt, float* x, const float* part, int KS,
                                 const float* g, void* y, int M, int D) {
  if (M <= 0) return hipSuccess;
  if (D > 4096 || D % 4 || KS > 4) return hipErrorInvalidValue;
  const bool wide = D > 2048;
  TimingScope ts(s, KC_RMSNORM,
                 (double)M * D * ((ACC ? 8 + 4 * KS : 4) + (odt == WAM_BF16 ? 2 : 4)), 0.0);
  if (M <= 512) {  // latency bound: a workgroup per row
    if (odt == WAM_BF16 && !wide)
      hipLaunchKernelGGL((rmsnorm_row_kernel<bf16_t, ACC>), dim3(M), dim3(256), 0, s, x, part, KS,
                         g, (bf16_t*)y, M, D);
    else if (odt == WAM_BF16)
      hipLaunchKernelGGL((rmsnorm_row_kernel<bf16_t, ACC, 4>), dim3(M), dim3(256), 0, s, x, part,
                         KS, g, (bf16_t*)y, M, D);
    else if (!wide)
      hipLaunchKernelGGL((rmsnorm_row_kernel<float, ACC>), dim3(M), dim3(256), 0, s, x, part, KS,
                         g, (float*)y, M, D);
    else
      hipLaunchKernelGGL((rmsnorm_row_kernel<float, ACC, 4>), dim3(M), dim3(256), 0, s, x, part,
                         KS, g, (float*)y, M, D);
    return hipGetLastError();
  }
  dim3 grid((M + 3) / 4);
  if (odt == WAM_BF16 && !wide)
    hipLaunchKernelGGL((rmsnorm_kernel<bf16_t, ACC>), grid, dim3(256), 0, s, x, part, KS, g,
                       (bf16_t*)y, M, D);
  else if (odt == WAM_BF16)
    hipLaunchKernelGGL((rmsnorm_kernel<bf16_t, ACC, 16>), grid, dim3(256), 0, s, x, part, KS, g,
                       (bf16_t*)y, M, D);
  else if (!wide)
    hipLaunchKernelGGL((rmsnorm_kernel<float, ACC>), grid, dim3(256), 0, s, x, part, KS, g,
                       (float*)y, M, D);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<float, ACC, 16>), grid, dim3(256), 0, s, x, part, KS, g,
                       (float*)y, M, D);
  return hipGetLastError();
}

hipError_t rmsnorm(hipStream_t s, int odt, const float* x, const float* g, void* y, int M, int D) {
  return rmsnorm_launch<false>(s, odt, const_cast<float*>(x), nullptr, 0, g, y, M, D);
}

hipError_t rmsnorm_accum(hipStream_t s, int odt, float* x, const float* part, int KS,
                         const float* g, void* y, int M, int D) {
  return rmsnorm_launch<true>(s, odt, x, part, KS, g, y, M, D);
}

// ------------------------------------------------------------ embedding
// X[m][n] = sum_c x[row(m)][c] * w_in[n][c] + emb[n]  (C <= 64, fp32 FMA in c order)
//
// A workgroup computes a 64-row x 128-column tile: x rows and the W_in slice
// (transposed, so a thread reads its 4 columns as one float4) are staged in
// LDS as fp32; each thread accumulates an 8 x 4 register tile and writes
// 16-byte rows.
constexpr int EMB_MAXC = 64, EMB_BM = 64, EMB_BN = 128;

// four consecutive elements as fp32 (8- or 16-byte load; p 8/16-byte aligned)
__device__ inline void load4(const float* p, float (&v)[4]) {
  const float4 a = *(const float4*)p;
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
__device__ inline void load4(const bf16_t* p, float (&v)[4]) {
  const uint2 a = *(const uint2*)p;
  v[0] = __uint_as_float(a.x << 16);
  v[1] = __uint_as_float(a.x & 0xFFFF0000u);
  v[2] = __uint_as_float(a.y << 16);
  v[3] = __uint_as_float(a.y & 0xFFFF0000u);
}

template <typename TX, typename TW>
__global__ __launch_bounds__(256) void embed_kernel(const TX* __restrict__ x, RowMap map,
                                                    const TW* __restrict__ w_in,
                                                    const float* __restrict__ emb,
                                                    float* __restrict__ X, int M, int D, int C) {
  __shared__ __attribute__((aligned(16))) float xs[EMB_BM][EMB_MAXC + 4];
  __shared__ __attribute__((aligned(16))) float ws[EMB_MAXC][EMB_BN];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * EMB_BM, n0 = blockIdx.y * EMB_BN;
  if (C % 16 == 0) {
    // four threads per x row (C/4 values each, whole 16-byte pieces), one
    // row-map lookup per thread; all loads independent
    const int r = tid >> 2, q = tid & 3, cq = C / 4, m = m0 + r;
    if (m < M) {
      const int f = m / map.P, t = m - f * map.P;
      const TX* xr = x + ((long long)map.src[f] * map.P + t) * C + q * cq;
      for (int c = 0; c < cq; c += 4) {
        float v[4];
        load4(xr + c, v);
#pragma unroll
        for (int j = 0; j < 4; j++) xs[r][q * cq + c + j] = v[j];
      }
    } else {
      for (int c = 0; c < cq; c++) xs[r][q * cq + c] = 0.f;
    }
    // two threads per weight row; consecutive lanes hold consecutive columns
    // n, so the transposed LDS writes of a wave hit consecutive banks
    const int n = tid & (EMB_BN - 1), half = tid >> 7, ch = C / 2;
    const TW* wr = w_in + (long long)(n0 + n) * C + half * ch;
    const bool ok = n0 + n < D;
    for (int c = 0; c < ch; c += 4) {
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (ok) load4(wr + c, v);
#pragma unroll
      for (int j = 0; j < 4; j++) ws[half * ch + c + j][n] = v[j];
    }
  } else {
    for (int i = tid; i < EMB_BM * C; i += 256) {
      const int r = i / C, c = i - r * C, m = m0 + r;
      float v = 0.f;
      if (m < M) {
        const int f = m / map.P, t = m - f * map.P;
        v = to_f<TX>(x[((long long)map.src[f] * map.P + t) * C + c]);
      }
      xs[r][c] = v;
    }
    for (int i = tid; i < EMB_BN * C; i += 256) {
      const int n = i & (EMB_BN - 1), c = i / EMB_BN;
      ws[c][n] = (n0 + n < D) ? to_f<TW>(w_in[(long long)(n0 + n) * C + c]) : 0.f;
    }
  }
  __syncthreads();
  const int cg = tid & 31, rg = tid >> 5;  // columns 4cg..4cg+3, rows 8rg..8rg+7
  float acc[8][4];
#pragma unroll
  for (int r = 0; r < 8; r++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[r][j] = 0.f;
  auto step = [&](int c, float xv[8]) {
    const float4 wv = *(const float4*)&ws[c][4 * cg];
#pragma unroll
    for (int r = 0; r < 8; r++) {
      acc[r][0] = fmaf(xv[r], wv.x, acc[r][0]);
      acc[r][1] = fmaf(xv[r], wv.y, acc[r][1]);
      acc[r][2] = fmaf(xv[r], wv.z, acc[r][2]);
      acc[r][3] = fmaf(xv[r], wv.w, acc[r][3]);
    }
  };
  int c = 0;
  for (; c + 4 <= C; c += 4) {  // x values of 8 rows x 4 c as 16-byte reads
    float4 xq[8];
#pragma unroll
    for (int r = 0; r < 8; r++) xq[r] = *(const float4*)&xs[8 * rg + r][c];
    float xv[8];
#pragma unroll
    for (int r = 0; r < 8; r++) xv[r] = xq[r].x;
    step(c, xv);
#pragma unroll
    for (int r = 0; r < 8; r++) xv[r] = xq[r].y;
    step(c + 1, xv);
#pragma unroll
    for (int r = 0; r < 8; r++) xv[r] = xq[r].z;
    step(c + 2, xv);
#pragma unroll
    for (int r = 0; r < 8; r++) xv[r] = xq[r].w;
    step(c + 3, xv);
  }
  for (; c < C; c++) {
    float xv[8];
#pragma unroll
    for (int r = 0; r < 8; r++) xv[r] = xs[8 * rg + r][c];
    step(c, xv);
  }
  const int n = n0 + 4 * cg;
  if (n >= D) return;  // D is a multiple of 4
  const float4 e = *(const float4*)(emb + n);
#pragma unroll
  for (int r = 0; r < 8; r++) {
    const int m = m0 + 8 * rg + r;
    if (m < M)
      *(float4*)(X + (long long)m * D + n) =
          float4{acc[r][0] + e.x, acc[r][1] + e.y, acc[r][2] + e.z, acc[r][3] + e.w};
  }
}

hipError_t embed(hipStream_t s, int xdt, int wdt, const void* x, const RowMap& map,
                 const void* w_in, const float* emb, float* X, int M, int D, int C) {
  if (M <= 0) return hipSuccess;
  if (C > EMB_MAXC || D % 4) return hipErrorInvalidValue;
  dim3 grid((M + EMB_BM - 1) / EMB_BM, (D + EMB_BN - 1) / EMB_BN);
  TimingScope ts(s, KC_EMBED, (double)M * D * 4, 2.0 * M * D * C);
#define EMB(TX, TW)                                                                          \
  hipLaunchKernelGGL((embed_kernel<TX, TW>), grid, dim3(256), 0, s, (const TX*)x, map,       \
                     (const TW*)w_in, emb, X, M, D, C)
  if (xdt == WAM_F32 && wdt == WAM_F32) EMB(float, float);
  else if (xdt == WAM_F32 && wdt == WAM_BF16) EMB(float, bf16_t);
  else if (xdt == WAM_BF16 && wdt == WAM_BF16) EMB(bf16_t, bf16_t);
  else return hipErrorInvalidValue;
#undef EMB
  return hipGetLastError();
}

// ------------------------------------------------------------ time embedding
struct SigmaList {
  float v[WAM_MAX_STEPS + 8];
};

// emb[i] = [cos(t w_j), sin(t w_j)], t = 1000 sigma_i, w_j = 10000^(-j/(D/2)),
// evaluated in float64 and rounded to fp32.
__global__ void time_embedding_kernel(SigmaList sig, int D, float* __restrict__ emb) {
  const int i = blockIdx.y;
  const int half = D / 2;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < half; j += gridDim.x * blockDim.x) {
    double t = 1000.0 * (double)sig.v[i];
    double w = pow(10000.0, -(double)j / (double)half);
    double a = t * w;
    emb[(long long)i * D + j] = (float)cos(a);
    emb[(long long)i * D + half + j] = (float)sin(a);
  }
}

hipError_t time_embedding(hipStream_t s, const float* sigma_host, int n, int D, float* emb) {
  if (n <= 0) return hipSuccess;
  if (n > WAM_MAX_STEPS + 8) return hipErrorInvalidValue;
  SigmaList l;
  for (int i = 0; i < n; i++) l.v[i] = sigma_host[i];
  dim3 grid((D / 2 + 255) / 256, n);
  hipLaunchKernelGGL(time_embedding_kernel, grid, dim3(256), 0, s, l, D, emb);
  return hipGetLastError();
}

// ------------------------------------------------------------ Euler / copy
__global__ void euler_kernel(float* __restrict__ x, const float* __restrict__ v, int64_t n, float dt) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    x[i] = fmaf(dt, v[i], x[i]);
}

hipError_t euler(hipStream_t s, float* x, const float* v, int64_t n, float dt) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(euler_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, v, n, dt);
  return hipGetLastError();
}

template <typename T>
__global__ void cvt_kernel(const T* __restrict__ src, float* __restrict__ dst, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = to_f<T>(src[i]);
}

hipError_t copy_cvt_f32(hipStream_t s, int sdt, const void* src, float* dst, int64_t n) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (sdt == WAM_BF16)
    hipLaunchKernelGGL(cvt_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const bf16_t*)src, dst, n);
  else
    hipLaunchKernelGGL(cvt_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const float*)src, dst, n);
  return hipGetLastError();
}


// ------------------------------------------------------------ step boundary
// One workgroup per row m (D <= 1024 NJ, C <= 64):
//   head:  y = RMSNorm(X[m]; g_out); v[n] = y . W_out[n] for n < C;
//          z[m][n] += dt v[n]; vhat[m][n] = v[n]      (the flow update)
//   next:  X[m][:] = z[m][:] W_in^T + emb_next[:]       (the next embedding)
// Either part may be switched off (do_head = 0 / w_in = nullptr).
template <typename TW, int NJ = 2>
__global__ __launch_bounds__(256) void step_kernel(float* __restrict__ X,
                                                   const float* __restrict__ g_out,
                                                   const TW* __restrict__ w_out,
                                                   float* __restrict__ z, float dt,
                                                   float* __restrict__ vhat,
                                                   const TW* __restrict__ w_in,
                                                   const float* __restrict__ emb_next, int D, int C,
                                                   int do_head) {
  __shared__ float red[4][64];
  __shared__ float wss[4];
  __shared__ float zs[64];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* xr = X + (long long)m * D;
  float* zr = z + (long long)m * C;
  if (do_head) {
    float4 y[NJ];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int i = 4 * tid + 1024 * j;
      y[j] = (i < D) ? *(const float4*)(xr + i) : float4{0.f, 0.f, 0.f, 0.f};
      ss = fmaf(y[j].x, y[j].x, ss);
      ss = fmaf(y[j].y, y[j].y, ss);
      ss = fmaf(y[j].z, y[j].z, ss);
      ss = fmaf(y[j].w, y[j].w, ss);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) wss[w] = ss;
    __syncthreads();
    const float r = 1.0f / sqrtf((((wss[0] + wss[1]) + wss[2]) + wss[3]) / (float)D + 1e-6f);
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int i = 4 * tid + 1024 * j;
      if (i < D) {
        const float4 gg = *(const float4*)(g_out + i);
        y[j].x *= r * gg.x;
        y[j].y *= r * gg.y;
        y[j].z *= r * gg.z;
        y[j].w *= r * gg.w;
      }
    }
    for (int n = 0; n < C; n++) {
      float p = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; j++) {
        const int i = 4 * tid + 1024 * j;
        if (i < D) {
          const TW* wr = w_out + (long long)n * D + i;
          p = fmaf(y[j].x, to_f<TW>(wr[0]), p);
          p = fmaf(y[j].y, to_f<TW>(wr[1]), p);
          p = fmaf(y[j].z, to_f<TW>(wr[2]), p);
          p = fmaf(y[j].w, to_f<TW>(wr[3]), p);
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) p += __shfl_xor(p, o, 64);
      if (lane == 0) red[w][n] = p;
    }
    __syncthreads();
    if (tid < C) {
      const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
      const float zn = fmaf(dt, v, zr[tid]);
      zr[tid] = zn;
      if (vhat) vhat[(long long)m * C + tid] = v;
      zs[tid] = zn;
    }
  } else if (tid < C) {
    zs[tid] = zr[tid];
  }
  if (w_in == nullptr) return;
  __syncthreads();
  for (int col = tid; col < D; col += 256) {
    float acc = 0.f;
    for (int c = 0; c < C; c++) acc = fmaf(zs[c], to_f<TW>(w_in[(long long)col * C + c]), acc);
    xr[col] = acc + emb_next[col];
  }
}

hipError_t step_boundary(hipStream_t s, int wdt, float* X, const float* g_out, const void* w_out,
                         float* z, float dt, float* vhat, const void* w_in, const float* emb_next,
                         int M, int D, int C, bool do_head) {
  if (M <= 0) return hipSuccess;
  if (D > 4096 || D % 4 || C > 64) return hipErrorInvalidValue;
  TimingScope ts(s, KC_MISC,
                 (double)M * ((do_head ? D * 4.0 + 2.0 * C * 4 : 0.0) + (w_in ? D * 4.0 : 0.0)),
                 (double)M * ((do_head ? 2.0 * C * D : 0.0) + (w_in ? 2.0 * C * D : 0.0)));
  const bool wide = D > 2048;
  if (wdt == WAM_BF16 && !wide)
    hipLaunchKernelGGL(step_kernel<bf16_t>, dim3(M), dim3(256), 0, s, X, g_out,
                       (const bf16_t*)w_out, z, dt, vhat, (const bf16_t*)w_in, emb_next, D, C,
                       do_head ? 1 : 0);
  else if (wdt == WAM_BF16)
    hipLaunchKernelGGL((step_kernel<bf16_t, 4>), dim3(M), dim3(256), 0, s, X, g_out,
                       (const bf16_t*)w_out, z, dt, vhat, (const bf16_t*)w_in, emb_next, D, C,
                       do_head ? 1 : 0);
  else if (!wide)
    hipLaunchKernelGGL(step_kernel<float>, dim3(M), dim3(256), 0, s, X, g_out, (const float*)w_out,
                       z, dt, vhat, (const float*)w_in, emb_next, D, C, do_head ? 1 : 0);
  else
    hipLaunchKernelGGL((step_kernel<float, 4>), dim3(M), dim3(256), 0, s, X, g_out,
                       (const float*)w_out, z, dt, vhat, (const float*)w_in, emb_next, D, C,
                       do_head ? 1 : 0);
  return hipGetLastError();
}

// ------------------------------------------------------------ Interval KV-Fusion
// dst[m][i] = sum_{j < count_m} w[m][j] * src[start_m + j][i], fp32 accumulate in
// j order, one rounding to the storage type.  8 elements per thread (16-byte
// bf16 loads); layer_elems is a multiple of 8.
template <typename T>
__global__ __launch_bounds__(256) void fuse_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                   long long layer_elems, FuseArgs a) {
  const int m = blockIdx.y;
  const int cnt = a.count[m];
  const T* base = src + (long long)a.start[m] * layer_elems;
  T* out = dst + (long long)m * layer_elems;
  for (long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 8; i < layer_elems;
       i += (long long)gridDim.x * 256 * 8) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = 0.f;
    for (int j = 0; j < cnt; j++) {
      const float wj = a.w[m][j];
      T v[8];
      if constexpr (sizeof(T) == 2) {
        *(u32x4*)v = __builtin_nontemporal_load((const u32x4*)(base + j * layer_elems + i));
      } else {
        *(u32x4*)v = __builtin_nontemporal_load((const u32x4*)(base + j * layer_elems + i));
        *(u32x4*)(v + 4) = __builtin_nontemporal_load((const u32x4*)(base + j * layer_elems + i + 4));
      }
#pragma unroll
      for (int e = 0; e < 8; e++) acc[e] = fmaf(wj, to_f<T>(v[e]), acc[e]);
    }
    T o[8];
#pragma unroll
    for (int e = 0; e < 8; e++) o[e] = from_f<T>(acc[e]);
    if constexpr (sizeof(T) == 2) {
      *(u32x4*)(out + i) = *(u32x4*)o;
    } else {
      *(u32x4*)(out + i) = *(u32x4*)o;
      *(u32x4*)(out + i + 4) = *(u32x4*)(o + 4);
    }
  }
}

hipError_t fuse_kv(hipStream_t s, int dt, const void* src, void* dst, long long layer_elems,
                   const FuseArgs& a) {
  if (a.M <= 0 || layer_elems <= 0) return hipSuccess;
  if (layer_elems % 8) return hipErrorInvalidValue;
  long long per = (layer_elems / 8 + 255) / 256;
  unsigned bx = (unsigned)(per < 1024 ? per : 1024);
  dim3 grid(bx, a.M);
  int reads = 0;
  for (int m = 0; m < a.M; m++) reads += a.count[m];
  TimingScope ts(s, KC_FUSE, (double)(reads + a.M) * layer_elems * (dt == WAM_BF16 ? 2 : 4),
                 2.0 * reads * layer_elems);
  if (dt == WAM_BF16)
    hipLaunchKernelGGL(fuse_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)src,
                       (bf16_t*)dst, layer_elems, a);
  else
    hipLaunchKernelGGL(fuse_kernel<float>, grid, dim3(256), 0, s, (const float*)src,
                       (float*)dst, layer_elems, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ E4M3 cache
// One 64-key tile of one (layer, episode, head) per workgroup: K when
// blockIdx.z is even, V^T when odd.  Thread t takes row t/4 of the tile (a
// key of K, a head-dim row of V^T) and the 16 elements that go to bytes
// 16g..16g+15 of that row, g = t%4: elements 8g..8g+7 and 32+8g..32+8g+7
// (dims of K, keys of the V^T tile).  The tile exponent is exact: with
// amax = m 2^q (m in [0.5, 1)), the smallest e with amax <= 448 2^e =
// 0.875 2^(9+e) is q-9 when m <= 0.875, else q-8, and at least -126.  Scaling
// by 2^-e is exact, and v_cvt_pk_fp8_f32 rounds to nearest even
// (|x 2^-e| <= 448).
template <int DH>
__global__ __launch_bounds__(256) void quantize_kv_kernel(const bf16_t* __restrict__ k,
                                                          const bf16_t* __restrict__ v,
                                                          uint8_t* __restrict__ k8,
                                                          uint8_t* __restrict__ v8,
                                                          float* __restrict__ ks,
                                                          float* __restrict__ vs, int B, int Hh,
                                                          int cap, ActLens lens) {
  // NU units of 16 elements per thread: K row r, dims 64u + {8g.., 32 + 8g..};
  // V^T rows r + 64u, keys {8g.., 32 + 8g..} of the tile
  constexpr int NU = DH / 64;
  __shared__ float wmax[4];
  const int t = blockIdx.x, h = blockIdx.y, which = blockIdx.z & 1, lb = blockIdx.z >> 1;
  const int len = lens.len[lb % B];
  if (t * 64 >= len) return;
  const int tid = threadIdx.x, r = tid >> 2, g = tid & 3;
  const long long head = ((long long)lb * Hh + h) * cap * DH;  // one head's elements
  float x[16 * NU];
  long long dst[NU];
  if (which == 0) {
    const int key = t * 64 + r;
#pragma unroll
    for (int u = 0; u < NU; u++) {
      // a lane group's NU * 16 bytes of a K row are contiguous
      dst[u] = head + (long long)key * DH + 16 * NU * g + 16 * u;
      if (key < len) {
        const bf16x8 a = *(const bf16x8*)(k + head + (long long)key * DH + 64 * u + 8 * g);
        const bf16x8 b = *(const bf16x8*)(k + head + (long long)key * DH + 64 * u + 32 + 8 * g);
#pragma unroll
        for (int j = 0; j < 8; j++) {
          x[16 * u + j] = bf2f((bf16_t)a[j]);
          x[16 * u + 8 + j] = bf2f((bf16_t)b[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; j++) x[16 * u + j] = 0.f;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < NU; u++) {
      const long long row = head + (long long)(r + 64 * u) * cap + t * 64;
      dst[u] = row + 16 * g;
      const bf16x8 a = *(const bf16x8*)(v + row + 8 * g);
      const bf16x8 b = *(const bf16x8*)(v + row + 32 + 8 * g);
#pragma unroll
      for (int j = 0; j < 8; j++) {
        x[16 * u + j] = (t * 64 + 8 * g + j < len) ? bf2f((bf16_t)a[j]) : 0.f;
        x[16 * u + 8 + j] = (t * 64 + 32 + 8 * g + j < len) ? bf2f((bf16_t)b[j]) : 0.f;
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 16 * NU; j++) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  int e = 0;
  if (amax > 0.f) {
    int q;
    const float m = frexpf(amax, &q);
    e = (m <= 0.875f) ? q - 9 : q - 8;
    // the scale stays a normal float32 number (and 2^-e finite): tiles
    // below 448 * 2^-127 keep e = -126, their codes then stay under 224
    e = e < -126 ? -126 : e;
  }
  const float inv = ldexpf(1.0f, -e);
#pragma unroll
  for (int u = 0; u < NU; u++) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const float* y = x + 16 * u + 4 * w;
      unsigned word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0] * inv, y[1] * inv, 0u, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2] * inv, y[3] * inv, word, true);
      o[w] = word;
    }
    *(u32x4*)((which == 0 ? k8 : v8) + dst[u]) = o;
  }
  if (tid == 0) (which == 0 ? ks : vs)[((long long)lb * Hh + h) * (cap / 64) + t] = ldexpf(1.0f, e);
}

hipError_t quantize_kv_fp8(hipStream_t s, const void* k, const void* v, void* k8, void* v8,
                           float* ks, float* vs, int n_layers, int B, int Hh, int dh, int cap,
                           const ActLens& lens) {
  int maxlen = 0;
  double rows = 0.0;
  for (int b = 0; b < B; b++) {
    maxlen = lens.len[b] > maxlen ? lens.len[b] : maxlen;
    rows += lens.len[b];
  }
  if (maxlen == 0 || n_layers <= 0) return hipSuccess;
  if (cap % 64 || maxlen > cap || (dh != 64 && dh != 128)) return hipErrorInvalidValue;
  const double elems = 2.0 * n_layers * Hh * dh * rows;  // K and V
  TimingScope ts(s, KC_QUANT, elems * 3.0, 0.0);
  dim3 grid((maxlen + 63) / 64, Hh, 2 * n_layers * B);
  if (dh == 64)
    hipLaunchKernelGGL(quantize_kv_kernel<64>, grid, dim3(256), 0, s, (const bf16_t*)k,
                       (const bf16_t*)v, (uint8_t*)k8, (uint8_t*)v8, ks, vs, B, Hh, cap, lens);
  else
    hipLaunchKernelGGL(quantize_kv_kernel<128>, grid, dim3(256), 0, s, (const bf16_t*)k,
                       (const bf16_t*)v, (uint8_t*)k8, (uint8_t*)v8, ks, vs, B, Hh, cap, lens);
  return hipGetLastError();
}

// ---------------------------------------------------------------- rotary option
// Rotary position embedding in place on one or two tensors of layout
// [G][Hh][rows][dh] (group stride gs, head stride hs): row r of group g is the
// token at position base[g] + r, and pair j = (x[2j], x[2j+1]) of every head
// is multiplied, as x[2j] + i x[2j+1], by exp(i p w_j), w_j = 10000^(-2j/dh).
// One thread per (row, pair, group of RH heads) computes the angle and its
// sine and cosine in float64, rounds them to float32 once, loads the pair of
// each of its heads in both tensors, then rotates and stores them: the loads
// are all in flight together.
constexpr int RH = 4;
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ x0, long long gs0, long long hs0,
                                                   T* __restrict__ x1, long long gs1, long long hs1,
                                                   int rows, int Hh, int dh, RopeRows rb) {
  const int half = dh >> 1, g = blockIdx.y, h0 = blockIdx.z * RH;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)rows * half) return;
  const int r = (int)(i / half), j = (int)(i - (long long)r * half);
  const double w = pow(10000.0, -2.0 * j / dh);
  double sd, cd;
  sincos((double)(rb.base[g] + r) * w, &sd, &cd);
  const float c = (float)cd, sn = (float)sd;
  const long long off = (long long)r * dh + 2 * j;
  T* p0[RH];
  T* p1[RH];
  float a0[RH], b0[RH], a1[RH], b1[RH];
#pragma unroll
  for (int u = 0; u < RH; u++) {
    const int h = min(h0 + u, Hh - 1);  // heads past Hh repeat the last one and store nothing
    p0[u] = x0 + g * gs0 + h * hs0 + off;
    p1[u] = x1 ? x1 + g * gs1 + h * hs1 + off : p0[u];
    a0[u] = to_f<T>(p0[u][0]);
    b0[u] = to_f<T>(p0[u][1]);
    a1[u] = to_f<T>(p1[u][0]);
    b1[u] = to_f<T>(p1[u][1]);
  }
#pragma unroll
  for (int u = 0; u < RH; u++) {
    if (h0 + u >= Hh) break;
    p0[u][0] = from_f<T>(a0[u] * c - b0[u] * sn);
    p0[u][1] = from_f<T>(a0[u] * sn + b0[u] * c);
    if (x1) {
      p1[u][0] = from_f<T>(a1[u] * c - b1[u] * sn);
      p1[u][1] = from_f<T>(a1[u] * sn + b1[u] * c);
    }
  }
}

hipError_t rope_qk(hipStream_t s, int dt, void* x0, long long gs0, long long hs0, void* x1,
                   long long gs1, long long hs1, int G, int rows, int Hh, int dh,
                   const RopeRows& rb) {
  if (rows <= 0 || G <= 0) return hipSuccess;
  if (G > WAM_MAX_BATCH || dh % 2) return hipErrorInvalidValue;
  const double es = dt == WAM_BF16 ? 2.0 : 4.0;
  TimingScope ts(s, KC_MISC, (x1 ? 4.0 : 2.0) * G * Hh * (double)rows * dh * es, 0.0);
  dim3 grid((unsigned)(((long long)rows * (dh / 2) + 255) / 256), G, (Hh + RH - 1) / RH);
  if (dt == WAM_BF16)
    hipLaunchKernelGGL(rope_kernel<bf16_t>, grid, dim3(256), 0, s, (bf16_t*)x0, gs0, hs0,
                       (bf16_t*)x1, gs1, hs1, rows, Hh, dh, rb);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(256), 0, s, (float*)x0, gs0, hs0,
                       (float*)x1, gs1, hs1, rows, Hh, dh, rb);
  return hipGetLastError();
}

}  // namespace wam
