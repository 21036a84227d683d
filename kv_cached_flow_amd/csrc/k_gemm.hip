// GEMM kernels: C[M][N] = A[M][K] * B[N][K]^T with fused epilogues.
//
//  * gemm_big    bf16 MFMA (v_mfma_f32_16x16x32_bf16), 128x128x64 tiles, LDS
//                staged with register prefetch; the prefill / imagine
//                projections (M = thousands of tokens).
//  * gemm_skinny bf16 MFMA for M <= 128 (the 32*B action rows): weight
//                streaming, A staged once in LDS, split-K across workgroups
//                merged by the last-arriving workgroup in a fixed order.
//  * gemm_simple fp32-accumulate FMA tiles for any type/size: the fp32
//                workload and the narrow heads (N = Cv or A).
#include "wam_internal.h"

namespace wam {

// ============================================================ simple (FMA)
template <typename TA, typename TB, typename TO, int EPI>
__global__ __launch_bounds__(256) void gemm_simple_kernel(const TA* __restrict__ A, int lda,
                                                          const TB* __restrict__ B, int ldb,
                                                          int M, int N, int K, EpiArgs e) {
  constexpr int T = 64, BK = 16;
  __shared__ float As[BK][T + 4];
  __shared__ float Bs[BK][T + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  const int tx = tid % 16, ty = tid / 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < K; k0 += BK) {
    // 64 rows x 16 k per operand: 1024 elements, 4 per thread
#pragma unroll
    for (int r = 0; r < 4; r++) {
      int idx = tid + 256 * r;
      int row = idx / BK, kk = idx % BK;
      int gm = m0 + row, gn = n0 + row, gk = k0 + kk;
      As[kk][row] = (gm < M && gk < K) ? to_f<TA>(A[(long long)gm * lda + gk]) : 0.f;
      Bs[kk][row] = (gn < N && gk < K) ? to_f<TB>(B[(long long)gn * ldb + gk]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk++) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; i++) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; j++) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      int n = n0 + tx + 16 * j;
      if (n < N) epi_store<EPI, TO>(e, m, n, acc[i][j]);
    }
  }
}

// ============================================================ big MFMA
namespace big {
constexpr int BM = 128, BN = 128, BK = 64, LDS_LD = BK + 8;  // padded row (bf16 elements)
}

__device__ inline int swizzle_tile(int bid, int nb, int ntm, int ntn, int* tm, int* tn) {
  // Blocks are dealt round-robin to the 8 XCDs; make consecutive logical ids
  // land on one XCD so that neighbouring tiles share an L2, then walk tiles
  // in groups of 8 row-panels.
  int lid = bid;
  if ((nb & 7) == 0) lid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int GM = 8;
  int per_group = GM * ntn;
  int g = lid / per_group;
  int first = g * GM;
  int gsz = min(ntm - first, GM);
  int r = lid - g * per_group;
  *tm = first + r % gsz;
  *tn = r / gsz;
  return lid;
}

template <int EPI, typename TO>
__global__ __launch_bounds__(256) void gemm_big_kernel(const bf16_t* __restrict__ A, int lda,
                                                       const bf16_t* __restrict__ B, int ldb,
                                                       int M, int N, int K, EpiArgs e) {
  using namespace big;
  __shared__ __attribute__((aligned(16))) bf16_t sA[BM * LDS_LD];
  __shared__ __attribute__((aligned(16))) bf16_t sB[BN * LDS_LD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ntm = (M + BM - 1) / BM, ntn = N / BN;
  int tm, tn;
  swizzle_tile(blockIdx.x, gridDim.x, ntm, ntn, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm = w >> 1, wn = w & 1;

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // global -> register staging: 4 chunks of 8 bf16 per operand per thread
  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      int c = tid + 256 * r;
      int row = c >> 3, ch = c & 7;
      int gm = m0 + row;
      if (gm < M)
        ra[r] = *(const u32x4*)(A + (long long)gm * lda + k0 + ch * 8);
      else
        ra[r] = u32x4{0u, 0u, 0u, 0u};
      rb[r] = *(const u32x4*)(B + (long long)(n0 + row) * ldb + k0 + ch * 8);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      int c = tid + 256 * r;
      int row = c >> 3, ch = c & 7;
      *(u32x4*)(sA + row * LDS_LD + ch * 8) = ra[r];
      *(u32x4*)(sB + row * LDS_LD + ch * 8) = rb[r];
    }
  };

  gload(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    lstore();
    __syncthreads();
    if (k0 + BK < K) gload(k0 + BK);
#pragma unroll
    for (int s = 0; s < 2; s++) {
      bf16x8 af[4], bfr[4];
      const int kk = s * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; i++)
        af[i] = *(const bf16x8*)(sA + (wm * 64 + i * 16 + (lane & 15)) * LDS_LD + kk);
#pragma unroll
      for (int j = 0; j < 4; j++)
        bfr[j] = *(const bf16x8*)(sB + (wn * 64 + j * 16 + (lane & 15)) * LDS_LD + kk);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // C layout of 16x16 MFMA: lane holds column lane%16, rows 4*(lane/16)+r
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      int m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        int n = n0 + wn * 64 + j * 16 + (lane & 15);
        epi_store<EPI, TO>(e, m, n, acc[i][j][r]);
      }
    }
}

// ============================================================ skinny MFMA (M <= 128)
namespace skinny {
constexpr int NT = 16;   // columns per workgroup
constexpr int MAXM = 128;
constexpr int MAXKS = 8;
}

// Workgroup (kt, ks) computes columns [16kt, 16kt+16) over the k range
// [ks*kr, (ks+1)*kr); its four waves take consecutive quarters of that range
// and are summed through LDS in wave order.  No inter-workgroup
// synchronisation: with gridDim.y > 1 each workgroup writes its raw fp32
// partial to part[ks][M][N] and the consumer sums the partials in ks order.
// k is visited 64 at a time; lane group g = lane/16 owns k offsets
// 16g..16g+15 of each 64-wide step, split over two MFMAs (a dot product may
// permute k freely as long as A and B agree), so each weight row segment is
// one 128-byte contiguous read.
template <int EPI, typename TO, int MT>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const bf16_t* __restrict__ A, int lda,
                                                          const bf16_t* __restrict__ B, int ldb,
                                                          int M, int N, int K, int kr, EpiArgs e,
                                                          float* __restrict__ part) {
  constexpr int U = MT <= 2 ? 4 : (MT <= 4 ? 2 : 1);
  __shared__ float red[4][MT * 16][17];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int n0 = blockIdx.x * skinny::NT;
  const int kw = kr / 4;
  const int kb = blockIdx.y * kr + w * kw;
  const bf16_t* brow = B + (long long)(n0 + c16) * ldb + kb + 16 * g;
  const bf16_t* arow = A + (long long)c16 * lda + kb + 16 * g;

  floatx4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; i++) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int nsteps = kw / 64;
  for (int st = 0; st < nsteps; st += U) {
    bf16x8 b0[U], b1[U], a0[U][MT], a1[U][MT];
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (st + u < nsteps) {
        b0[u] = *(const bf16x8*)(brow + (st + u) * 64);
        b1[u] = *(const bf16x8*)(brow + (st + u) * 64 + 8);
#pragma unroll
        for (int i = 0; i < MT; i++) {
          const bf16_t* ap = arow + (long long)(16 * i) * lda + (st + u) * 64;
          a0[u][i] = *(const bf16x8*)ap;
          a1[u][i] = *(const bf16x8*)(ap + 8);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (st + u < nsteps) {
#pragma unroll
        for (int i = 0; i < MT; i++) {
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[u][i], b0[u], acc[i], 0, 0, 0);
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[u][i], b1[u], acc[i], 0, 0, 0);
        }
      }
    }
  }
  // C layout: lane holds column c16, rows 16i + 4g + r
#pragma unroll
  for (int i = 0; i < MT; i++)
#pragma unroll
    for (int r = 0; r < 4; r++) red[w][16 * i + 4 * g + r][c16] = acc[i][r];
  __syncthreads();
  for (int idx = tid; idx < M * 16; idx += 256) {
    const int m = idx >> 4, c = idx & 15;
    const float v = ((red[0][m][c] + red[1][m][c]) + red[2][m][c]) + red[3][m][c];
    if (gridDim.y == 1)
      epi_store<EPI, TO>(e, m, n0 + c, v);
    else
      part[((long long)blockIdx.y * M + m) * N + n0 + c] = v;
  }
}

// ============================================================ dispatch
// Algorithmic HBM bytes of one GEMM: read A and B once, write C once (read
// and write for the accumulate-into epilogues).
template <int EPI>
static double gemm_bytes(int M, int N, int K, int ea, int eb, int eo) {
  double out = (double)M * N * ((EPI == EPI_RESID || EPI == EPI_EULER) ? 8.0 : (double)eo);
  return (double)M * K * ea + (double)N * K * eb + out;
}

template <int EPI, typename TO>
static hipError_t launch_big(hipStream_t s, int M, int N, int K, const void* A, int lda,
                             const void* B, int ldb, const EpiArgs& e) {
  int ntm = (M + big::BM - 1) / big::BM, ntn = N / big::BN;
  TimingScope ts(s, KC_GEMM_BIG, gemm_bytes<EPI>(M, N, K, 2, 2, sizeof(TO)), 2.0 * M * N * K);
  hipLaunchKernelGGL((gemm_big_kernel<EPI, TO>), dim3(ntm * ntn), dim3(256), 0, s,
                     (const bf16_t*)A, lda, (const bf16_t*)B, ldb, M, N, K, e);
  return hipGetLastError();
}

// k range of one workgroup: a multiple of 256 (64 per wave) dividing K.
static bool skinny_ok(int M, int N, int K) {
  return M >= 16 && M <= skinny::MAXM && M % 16 == 0 && N % skinny::NT == 0 && K % 256 == 0;
}

template <int EPI, typename TO>
static hipError_t launch_skinny(hipStream_t s, int M, int N, int K, const void* A, int lda,
                                const void* B, int ldb, const EpiArgs& e, int KS, float* part) {
  const int kr = K / KS;
  dim3 grid(N / skinny::NT, KS);
  TimingScope ts(s, KC_GEMM_SKINNY, gemm_bytes<EPI>(M, N, K, 2, 2, KS > 1 ? 4 * KS : sizeof(TO)),
                 2.0 * M * N * K);
  const bf16_t* a = (const bf16_t*)A;
  const bf16_t* b = (const bf16_t*)B;
  switch (M / 16) {
#define SK(mt)                                                                              \
  case mt:                                                                                  \
    hipLaunchKernelGGL((gemm_skinny_kernel<EPI, TO, mt>), grid, dim3(256), 0, s, a, lda, b, \
                       ldb, M, N, K, kr, e, part);                                          \
    break;
    SK(1) SK(2) SK(3) SK(4) SK(5) SK(6) SK(7) SK(8)
#undef SK
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int gemm_partial_splits(int M, int N, int K) {
  if (!skinny_ok(M, N, K)) return 0;
  int ks = 1;
  while (ks < skinny::MAXKS && (N / skinny::NT) * ks < 256 && K % (256 * ks * 2) == 0) ks *= 2;
  return ks;
}

hipError_t gemm_partial(hipStream_t s, int M, int N, int K, const void* A, int lda, const void* B,
                        int ldb, float* part, int* ks_out) {
  const int ks = gemm_partial_splits(M, N, K);
  if (ks == 0) return hipErrorInvalidValue;
  *ks_out = ks;
  EpiArgs e{};
  e.out = part;
  e.ldo = N;
  return launch_skinny<EPI_STORE, float>(s, M, N, K, A, lda, B, ldb, e, ks, part);
}

template <typename TA, typename TB, int EPI, typename TO>
static hipError_t launch_simple(hipStream_t s, int M, int N, int K, const void* A, int lda,
                                const void* B, int ldb, const EpiArgs& e) {
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  TimingScope ts(s, KC_GEMM_SIMPLE, gemm_bytes<EPI>(M, N, K, sizeof(TA), sizeof(TB), sizeof(TO)),
                 2.0 * M * N * K);
  hipLaunchKernelGGL((gemm_simple_kernel<TA, TB, TO, EPI>), grid, dim3(256), 0, s,
                     (const TA*)A, lda, (const TB*)B, ldb, M, N, K, e);
  return hipGetLastError();
}

template <int EPI, typename TO>
static hipError_t gemm_epi(hipStream_t s, int adt, int bdt, int M, int N, int K, const void* A,
                           int lda, const void* B, int ldb, const EpiArgs& e,
                           int /*unused*/ = 0) {
  const bool aligned = ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0) && (lda % 8 == 0) &&
                       (ldb % 8 == 0);
  if (adt == WAM_BF16 && bdt == WAM_BF16 && aligned && K % 64 == 0) {
    if (skinny_ok(M, N, K)) return launch_skinny<EPI, TO>(s, M, N, K, A, lda, B, ldb, e, 1, nullptr);
    if (N % big::BN == 0) return launch_big<EPI, TO>(s, M, N, K, A, lda, B, ldb, e);
  }
  if (adt == WAM_F32 && bdt == WAM_F32)
    return launch_simple<float, float, EPI, TO>(s, M, N, K, A, lda, B, ldb, e);
  if (adt == WAM_F32 && bdt == WAM_BF16)
    return launch_simple<float, bf16_t, EPI, TO>(s, M, N, K, A, lda, B, ldb, e);
  if (adt == WAM_BF16 && bdt == WAM_BF16)
    return launch_simple<bf16_t, bf16_t, EPI, TO>(s, M, N, K, A, lda, B, ldb, e);
  return hipErrorInvalidValue;
}

hipError_t gemm(hipStream_t s, int adt, int bdt, int odt, int epi, int M, int N, int K,
                const void* A, int lda, const void* B, int ldb, const EpiArgs& e) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const bool ob = (odt == WAM_BF16);
  switch (epi) {
    case EPI_STORE:
      return ob ? gemm_epi<EPI_STORE, bf16_t>(s, adt, bdt, M, N, K, A, lda, B, ldb, e)
                : gemm_epi<EPI_STORE, float>(s, adt, bdt, M, N, K, A, lda, B, ldb, e);
    case EPI_GELU:
      return ob ? gemm_epi<EPI_GELU, bf16_t>(s, adt, bdt, M, N, K, A, lda, B, ldb, e)
                : gemm_epi<EPI_GELU, float>(s, adt, bdt, M, N, K, A, lda, B, ldb, e);
    case EPI_RESID:
      return gemm_epi<EPI_RESID, float>(s, adt, bdt, M, N, K, A, lda, B, ldb, e);
    case EPI_EULER:
      return gemm_epi<EPI_EULER, float>(s, adt, bdt, M, N, K, A, lda, B, ldb, e);
    case EPI_QKV:
      return ob ? gemm_epi<EPI_QKV, bf16_t>(s, adt, bdt, M, N, K, A, lda, B, ldb, e)
                : gemm_epi<EPI_QKV, float>(s, adt, bdt, M, N, K, A, lda, B, ldb, e);
  }
  return hipErrorInvalidValue;
}

}  // namespace wam
