// GEMM kernels: C[M][N] = A[M][K] * B[N][K]^T with fused epilogues.
//
//  * gemm_big    bf16 MFMA (v_mfma_f32_16x16x32_bf16), 128x128x64 tiles, LDS
//                staged with register prefetch; the prefill / imagine
//                projections (M = thousands of tokens).
//  * gemm_skinny bf16 MFMA for M <= 128 (the 32*B action rows): weight
//                streaming, A and B fragments loaded straight into registers,
//                k split over the waves of a workgroup (summed through LDS in
//                wave order) and, for the residual products, over workgroups
//                (fp32 partials that the next RMSNorm adds in split order).
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

__device__ inline int swizzle_tile(int bid, int nb, int ntm, int ntn, int* tm, int* tn, int GM = 8) {
  // Blocks are dealt round-robin to the 8 XCDs; make consecutive logical ids
  // land on one XCD so that neighbouring tiles share an L2, then walk tiles
  // in groups of GM row-panels.
  int lid = bid;
  if ((nb & 7) == 0) lid = (bid & 7) * (nb >> 3) + (bid >> 3);
  int per_group = GM * ntn;
  int g = lid / per_group;
  int first = g * GM;
  int gsz = min(ntm - first, GM);
  int r = lid - g * per_group;
  *tm = first + r % gsz;
  *tn = r / gsz;
  return lid;
}

// Epilogue on 4 consecutive columns n..n+3 of row m (n % 4 == 0).
template <int EPI, typename TO>
__device__ inline void epi_row4(const EpiArgs& e, int m, int n, float4 v) {
  if constexpr (EPI == EPI_STORE || EPI == EPI_GELU) {
    if (EPI == EPI_GELU) {
      if constexpr (sizeof(TO) == 2) {
        v.x = gelu_bf16out(v.x);
        v.y = gelu_bf16out(v.y);
        v.z = gelu_bf16out(v.z);
        v.w = gelu_bf16out(v.w);
      } else {
        v.x = gelu_f(v.x);
        v.y = gelu_f(v.y);
        v.z = gelu_f(v.z);
        v.w = gelu_f(v.w);
      }
    }
    TO* p = (TO*)e.out + (long long)m * e.ldo + n;
    if constexpr (sizeof(TO) == 2)
      *(uint2*)p = uint2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
    else
      *(float4*)p = v;
  } else if constexpr (EPI == EPI_RESID) {
    float4* p = (float4*)((float*)e.out + (long long)m * e.ldo + n);
    float4 x = *p;
    x.x += v.x;
    x.y += v.y;
    x.z += v.z;
    x.w += v.w;
    *p = x;
  } else {  // QKV, Q or K part: 4 consecutive head dims
    const int nn = e.n_begin + n;
    const int part = nn / e.D, c = nn - part * e.D;
    const int h = c / e.dh, d = c - h * e.dh;
    const int g = m / e.rpg, t = m - g * e.rpg;
    TO* p = part == 0 ? (TO*)e.q + g * e.q_gs + h * e.q_hs + (long long)t * e.dh + d
                      : (TO*)e.k + g * e.k_gs + h * e.k_hs + (long long)(e.k_row0 + t) * e.dh + d;
    if (part == 0) {
      v.x *= e.q_scale;
      v.y *= e.q_scale;
      v.z *= e.q_scale;
      v.w *= e.q_scale;
    }
    if constexpr (sizeof(TO) == 2)
      *(uint2*)p = uint2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
    else
      *(float4*)p = v;
  }
}

// QKV V part: rows m..m+3 (all < M) of column n go to 4 consecutive tokens of V^T.
template <typename TO>
__device__ inline void epi_vt4(const EpiArgs& e, int m, int n, float4 v) {
  const int nn = e.n_begin + n;
  const int c = nn - 2 * e.D;
  const int h = c / e.dh, d = c - h * e.dh;
  const int g = m / e.rpg, t = m - g * e.rpg;
  const long long off = g * e.v_gs + h * e.v_hs + (long long)d * e.v_ld + e.v_col0 + t;
  TO* p = (TO*)e.v + off;
  if (((e.v_col0 + t) & 3) == 0 && t + 3 < e.rpg) {
    if constexpr (sizeof(TO) == 2)
      *(uint2*)p = uint2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
    else
      *(float4*)p = v;
  } else {
    epi_store<EPI_QKV, TO>(e, m, n, v.x);
    epi_store<EPI_QKV, TO>(e, m + 1, n, v.y);
    epi_store<EPI_QKV, TO>(e, m + 2, n, v.z);
    epi_store<EPI_QKV, TO>(e, m + 3, n, v.w);
  }
}

// BM x 128 x 64 tiles, 4 waves, two workgroups per CU.  BM = 128: waves in a
// 2x2 grid, each 64 x 64; BM = 144 (9 row tiles of 16): waves side by side,
// each 144 x 32.  The host picks the height that fills the CUs in whole
// rounds (e.g. 9216 rows = 64 x 144: exactly 2 x 256 tiles for N = 1024).
// Operand tiles go from global memory straight into LDS (global_load_lds:
// lane i of a wave fills bytes [16i, 16i+16) of the destination), two stages
// deep.  A 64-wide k slice of one row is 128 bytes = 8 chunks of 16 bytes;
// chunk c of row r is stored at slot c ^ (r & 7), so each lane picks the
// global chunk that belongs at its LDS slot, and the 16-byte fragment reads of
// 8 consecutive rows hit distinct banks.  The fragment reads of a k step are
// issued before its MFMAs.  The C tile is transposed through LDS (a pass of
// 2048 values per wave at a time) so that the epilogue issues 8/16-byte
// accesses.
namespace big2 {
constexpr int BN = 128, BK = 64;
}
typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int BM>
struct BigGeom {
  static constexpr int NWM = BM == 144 ? 1 : 2, NWN = 4 / NWM;
  static constexpr int WM = BM / NWM, WN = big2::BN / NWN;  // wave tile
  static constexpr int MI = WM / 16, NI = WN / 16;
  static constexpr int ACH = BM / 8, BCH = big2::BN / 8;    // 1 KB chunks per stage
  static constexpr int AL = (ACH + 3) / 4;                   // A load instructions per wave
  static constexpr int STAGE = (BM + big2::BN) * 128;        // bytes
  static constexpr int RP = BM == 144 ? 48 : 32;            // epilogue rows per pass
  static constexpr int PASSES = WM / RP, TPP = RP / 16;      // passes, row tiles per pass
  static constexpr int ITEMS = RP * WN / 256;                // float4 items per lane per pass
  static_assert(BM == 128 || BM == 144, "tile height");
  static_assert(WM % RP == 0 && RP % 16 == 0, "epilogue passes");
};

template <int BM, int EPI, typename TO>
__global__ __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_big_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B, int ldb, int M, int N,
    int K, EpiArgs e) {
  using G = BigGeom<BM>;
  using namespace big2;
  constexpr int MI = G::MI, NI = G::NI, WM = G::WM, WN = G::WN, STAGE = G::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  // k split (gridDim.y > 1, plain fp32 stores only): workgroup (., ks) takes
  // k range [ks K, (ks + 1) K) and writes its partial to out + ks M ldo.
  if constexpr (EPI == EPI_STORE) {
    const int ks = blockIdx.y;
    A += (long long)ks * K;
    B += (long long)ks * K;
    e.out = (TO*)e.out + (long long)ks * M * e.ldo;
  }
  const int ntm = (M + BM - 1) / BM, ntn = N / BN;
  int tm, tn;
  // groups of 16 row panels where K is long and the rows many: measured 10 %
  // faster on 25 520 x 1024 x 4096, neutral or slower on the other shapes
  swizzle_tile(blockIdx.x, gridDim.x, ntm, ntn, &tm, &tn, K >= 4096 && ntm >= 128 ? 16 : 8);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm = w / G::NWN, wn = w % G::NWN;

  // Load instruction i of wave w fills LDS rows 8(4i + w) .. +7 of an
  // operand; lane l covers row 8(4i + w) + l/8, slot l%8.  Rows past M are
  // clamped (their products land in accumulator rows never stored).
  const int lrow = lane >> 3, lkc = (lane & 7) ^ lrow;
  const bf16_t* asrc[G::AL];
  const bf16_t* bsrc[4];
#pragma unroll
  for (int i = 0; i < G::AL; i++) {
    const int row = min((4 * i + w) * 8, BM - 8) + lrow;
    asrc[i] = A + (long long)min(m0 + row, M - 1) * lda + lkc * 8;
  }
#pragma unroll
  for (int i = 0; i < 4; i++) bsrc[i] = B + (long long)(n0 + (4 * i + w) * 8 + lrow) * ldb + lkc * 8;
  auto issue = [&](int kt, int buf) {
    char* sa = smem + buf * STAGE;
    char* sb = sa + BM * 128;
#pragma unroll
    for (int i = 0; i < G::AL; i++)
      if (4 * i + w < G::ACH)
        __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + kt * BK),
                                         (lds_ptr_t)(sa + (4 * i + w) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; i++)
      __builtin_amdgcn_global_load_lds((const void*)(bsrc[i] + kt * BK),
                                       (lds_ptr_t)(sb + (4 * i + w) * 1024), 16, 0, 0);
  };

  floatx4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; i++)
#pragma unroll
    for (int j = 0; j < NI; j++) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // epilogue item `it` of pass `p`: row it*(64/(WN/4)) + lane/(WN/4) of the
  // pass, columns 4*(lane%(WN/4)) .. +3
  constexpr int CPL = WN / 4, RPI = 64 / CPL;  // lanes per row, rows per item step
  const int nk = K / BK, x7 = c16 & 7;
  // residual epilogue: this lane's X values, loaded a few k steps before the
  // end so that the read overlaps the MFMAs; rows past M are clamped and never
  // stored
  float4 xr[G::PASSES][G::ITEMS];
  auto xload = [&] {
#pragma unroll
    for (int p = 0; p < G::PASSES; p++)
#pragma unroll
      for (int it = 0; it < G::ITEMS; it++) {
        const int m = min(m0 + wm * WM + p * G::RP + it * RPI + lane / CPL, M - 1);
        xr[p][it] = *(const float4*)((const float*)e.out + (long long)m * e.ldo + n0 + wn * WN +
                                     (lane % CPL) * 4);
      }
  };
  const int kx = max(nk - 4, 0);
  // every issued stage is waited for inside the loop (no LDS write may land
  // after the workgroup has left)
  if (nk > 0) issue(0, 0);
  for (int kt = 0; kt < nk; kt++) {
    if constexpr (EPI == EPI_RESID)
      if (kt == kx) xload();
    wait_vmem();      // this wave's transfers of stage kt have landed in LDS,
    __syncthreads();  // then everyone's
    const char* sa = smem + (kt & 1) * STAGE;
    const char* sb = sa + BM * 128;
    if constexpr (EPI != EPI_RESID) {
      bf16x8 af[2][MI], bfr[2][NI];
#pragma unroll
      for (int s = 0; s < 2; s++) {
        const int slot = ((4 * s + g) ^ x7) * 16;
#pragma unroll
        for (int i = 0; i < MI; i++) af[s][i] = *(const bf16x8*)(sa + (wm * WM + i * 16 + c16) * 128 + slot);
#pragma unroll
        for (int j = 0; j < NI; j++) bfr[s][j] = *(const bf16x8*)(sb + (wn * WN + j * 16 + c16) * 128 + slot);
      }
      __builtin_amdgcn_sched_barrier(0);
      // the other buffer was last read in step kt - 1, which every wave has left
      if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int i = 0; i < MI; i++)
#pragma unroll
          for (int j = 0; j < NI; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][i], bfr[s][j], acc[i][j], 0, 0, 0);
    } else {
      // the prefetched X tile holds registers: fragments one 32-wide k half at a time
      if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
#pragma unroll
      for (int s = 0; s < 2; s++) {
        const int slot = ((4 * s + g) ^ x7) * 16;
        bf16x8 af[MI], bfr[NI];
#pragma unroll
        for (int i = 0; i < MI; i++) af[i] = *(const bf16x8*)(sa + (wm * WM + i * 16 + c16) * 128 + slot);
#pragma unroll
        for (int j = 0; j < NI; j++) bfr[j] = *(const bf16x8*)(sb + (wn * WN + j * 16 + c16) * 128 + slot);
#pragma unroll
        for (int i = 0; i < MI; i++)
#pragma unroll
          for (int j = 0; j < NI; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // operand buffers become the C staging area

  // epilogue: RP rows x WN columns of the wave tile per pass
  constexpr int CLD = WN + 4;
  float* ct = (float*)smem + w * G::RP * CLD;
  bool vt = false;
  if constexpr (EPI == EPI_QKV) vt = (e.n_begin + n0 + wn * WN) / e.D == 2;
#pragma unroll
  for (int p = 0; p < G::PASSES; p++) {
#pragma unroll
    for (int ii = 0; ii < G::TPP; ii++)
#pragma unroll
      for (int j = 0; j < NI; j++)
#pragma unroll
        for (int r = 0; r < 4; r++)
          ct[(16 * ii + 4 * g + r) * CLD + 16 * j + c16] = acc[p * G::TPP + ii][j][r];
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    const int mb = m0 + wm * WM + p * G::RP, nb = n0 + wn * WN;
    if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int it = 0; it < G::ITEMS; it++) {
        const int row = it * RPI + lane / CPL, c4 = (lane % CPL) * 4;
        if (mb + row < M) {
          const float4 v = *(const float4*)(ct + row * CLD + c4);
          float4 x = xr[p][it];
          x.x += v.x;
          x.y += v.y;
          x.z += v.z;
          x.w += v.w;
          *(float4*)((float*)e.out + (long long)(mb + row) * e.ldo + nb + c4) = x;
        }
      }
    } else if (!vt) {
#pragma unroll 2
      for (int it = 0; it < G::ITEMS; it++) {
        const int row = it * RPI + lane / CPL, c4 = (lane % CPL) * 4;
        if (mb + row < M) epi_row4<EPI, TO>(e, mb + row, nb + c4, *(const float4*)(ct + row * CLD + c4));
      }
    } else {
      if constexpr (EPI == EPI_QKV) {
        // V^T: lanes walk 4-row groups of one column, so a column's keys are
        // written contiguously
        constexpr int RG = G::RP / 4;  // 4-row groups per column
#pragma unroll 2
        for (int it = 0; it < G::ITEMS; it++) {
          const int idx = it * 64 + lane;
          const int col = idx / RG, r4 = (idx % RG) * 4;
          const int m = mb + r4;
          if (m + 3 < M) {
            float4 v = {ct[r4 * CLD + col], ct[(r4 + 1) * CLD + col], ct[(r4 + 2) * CLD + col],
                        ct[(r4 + 3) * CLD + col]};
            epi_vt4<TO>(e, m, nb + col, v);
          } else {
            for (int r = 0; r < 4; r++)
              if (m + r < M) epi_store<EPI, TO>(e, m + r, nb + col, ct[(r4 + r) * CLD + col]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
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
template <int EPI, typename TO, int MT, int NW, int U = (MT <= 2 ? 4 : (MT <= 4 ? 2 : 1))>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_kernel(const bf16_t* __restrict__ A, int lda,
                                                          const bf16_t* __restrict__ B, int ldb,
                                                          int M, int N, int K, int kr, EpiArgs e,
                                                          float* __restrict__ part) {
  __shared__ float red[NW][MT * 16][17];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int n0 = blockIdx.x * skinny::NT;
  const int kw = kr / NW;
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
  for (int idx = tid; idx < M * 16; idx += 64 * NW) {
    const int m = idx >> 4, c = idx & 15;
    float v = red[0][m][c];
#pragma unroll
    for (int ww = 1; ww < NW; ww++) v += red[ww][m][c];
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
  double out = (double)M * N * (EPI == EPI_RESID ? 8.0 : (double)eo);
  return (double)M * K * ea + (double)N * K * eb + out;
}

template <int EPI, typename TO>
static hipError_t launch_big(hipStream_t s, int M, int N, int K, const void* A, int lda,
                             const void* B, int ldb, const EpiArgs& e) {
  const int ntn = N / big2::BN;
  TimingScope ts(s, KC_GEMM_BIG, gemm_bytes<EPI>(M, N, K, 2, 2, sizeof(TO)), 2.0 * M * N * K);
  // Tile height: fewest rounds (two resident workgroups per CU) weighted by
  // the measured time of one round: a 144-row round takes about 1.4x a
  // 128-row one (side-by-side waves read more LDS per MFMA), so 144 pays
  // only where it removes many rounds (9216 x 1024: 2 rounds -> 1).
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  const long long slots = 2ll * n_cu;
  auto rounds = [&](int bm) {
    const long long tiles = (long long)((M + bm - 1) / bm) * ntn;
    return (tiles + slots - 1) / slots;
  };
  if (rounds(144) * 7 < rounds(128) * 5) {
    const int ntm = (M + 143) / 144;
    hipLaunchKernelGGL((gemm_big_kernel<144, EPI, TO>), dim3(ntm * ntn), dim3(256), 0, s,
                       (const bf16_t*)A, lda, (const bf16_t*)B, ldb, M, N, K, e);
  } else {
    const int ntm = (M + 127) / 128;
    hipLaunchKernelGGL((gemm_big_kernel<128, EPI, TO>), dim3(ntm * ntn), dim3(256), 0, s,
                       (const bf16_t*)A, lda, (const bf16_t*)B, ldb, M, N, K, e);
  }
  return hipGetLastError();
}

// Split-K for row counts whose 128x128 tiles leave CUs idle: ks partial
// products part[ks][M][N] (raw fp32, 128-row tiles), summed by the consumer
// in ks order.  1 where the tiles fill the CUs or K does not split evenly.
int gemm_big_splits(int M, int N, int K) {
  if (N % big2::BN || K % big2::BK) return 1;
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  const long long tiles = (long long)((M + 127) / 128) * (N / big2::BN);
  int ks = 1;
  while (ks < 4 && tiles * ks * 2 <= n_cu * 2 && K % (ks * 2 * big2::BK) == 0) ks *= 2;
  return ks;
}

hipError_t gemm_big_partial(hipStream_t s, int M, int N, int K, const void* A, int lda,
                            const void* B, int ldb, float* part, int ks) {
  if (ks < 1 || K % (ks * big2::BK) || N % big2::BN) return hipErrorInvalidValue;
  TimingScope ts(s, KC_GEMM_BIG, gemm_bytes<EPI_STORE>(M, N, K, 2, 2, 4 * ks), 2.0 * M * N * K);
  EpiArgs e{};
  e.out = part;
  e.ldo = N;
  const int ntm = (M + 127) / 128, ntn = N / big2::BN;
  hipLaunchKernelGGL((gemm_big_kernel<128, EPI_STORE, float>), dim3(ntm * ntn, ks), dim3(256), 0, s,
                     (const bf16_t*)A, lda, (const bf16_t*)B, ldb, M, N, K / ks, e);
  return hipGetLastError();
}

// k range of one workgroup: a multiple of 64 per wave dividing K.
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
  // long k ranges: 8 waves so that each wave's loads stay few
  const bool w8 = (kr % 512 == 0) && kr >= 2048;
  switch (M / 16) {
#define SK(mt)                                                                                    \
  case mt:                                                                                        \
    if (w8)                                                                                       \
      hipLaunchKernelGGL((gemm_skinny_kernel<EPI, TO, mt, 8>), grid, dim3(512), 0, s, a, lda, b,  \
                         ldb, M, N, K, kr, e, part);                                              \
    else                                                                                          \
      hipLaunchKernelGGL((gemm_skinny_kernel<EPI, TO, mt, 4>), grid, dim3(256), 0, s, a, lda, b,  \
                         ldb, M, N, K, kr, e, part);                                              \
    break;
    SK(1) SK(2) SK(3) SK(4) SK(5) SK(6) SK(7) SK(8)
#undef SK
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Split-K partial products for the action rows: part[ks][M][N] (raw fp32,
// summed by the consumer in ks order).  Four splits measured best for the
// 1024-wide outputs at M = 32 (each workgroup then reads a quarter of A).
int gemm_partial_splits(int M, int N, int K) {
  if (!skinny_ok(M, N, K)) return 0;
  int ks = 1;
  while (ks < 4 && (N / skinny::NT) * ks < 256 && K % (256 * ks * 2) == 0) ks *= 2;
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
    if (N % big2::BN == 0) return launch_big<EPI, TO>(s, M, N, K, A, lda, B, ldb, e);
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
    case EPI_QKV:
      return ob ? gemm_epi<EPI_QKV, bf16_t>(s, adt, bdt, M, N, K, A, lda, B, ldb, e)
                : gemm_epi<EPI_QKV, float>(s, adt, bdt, M, N, K, A, lda, B, ldb, e);
  }
  return hipErrorInvalidValue;
}

}  // namespace wam
