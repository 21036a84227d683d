// Attention kernels.
//
//  * attn_prefill  block-causal video attention (flash style): bf16 MFMA
//    (v_mfma_f32_16x16x32_bf16) with K and V^T tiles staged in LDS, fp32
//    online softmax in the log2 domain.  A query in cache row r sees cache
//    rows [0, kend(r)) (own and earlier temporal blocks; padded frames are
//    compacted out of the cache).
//  * attn_action   32 action queries per (episode, head) over [cache ; own
//    keys]: split-K over the cache tokens, K and V^T streamed straight from
//    HBM into MFMA operands with 16-byte loads, per-wave online softmax, a
//    fixed-order merge inside the workgroup and a fixed-order merge of the
//    splits in a second kernel.  The chunk's own keys are one more split.
//
// Both compute S^T = K Q^T so that a lane owns one query column: row maxima
// and sums are per-lane plus two cross-lane steps.  Key rows are permuted
// inside each 32-key window so that the S^T output layout is exactly the
// B-operand layout of the P V MFMA (no data movement between the two):
// in window w, S subtile 2w row r is key 8*(r/4) + r%4, subtile 2w+1 row r is
// key 8*(r/4) + 4 + r%4, so lane group g ends up holding keys 8g..8g+7.
//
// fp32 variants (one thread per query, plain FMA) serve the fp32 workload.
#include <algorithm>
#include <type_traits>

#include "wam_internal.h"

namespace wam {


// Reductions over the four lanes {c, c+16, c+32, c+48} that hold one query
// column, with the gfx950 lane-swap instructions (VALU, no LDS traffic).
__device__ inline float wave_max16x4(float v) {
  const unsigned u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned w = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float wave_sum16x4(float v) {
  const unsigned u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned w = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// key index (0..63) inside a 64-key tile of S^T subtile `sub` (0..3), row r (0..15)
__device__ inline int perm_key(int sub, int r) {
  return 32 * (sub >> 1) + 8 * (r >> 2) + (r & 3) + 4 * (sub & 1);
}
// Running softmax state of one wave: 32 queries (two 16-column tiles).
// o[0..3][t] are the O^T accumulators (head dim x query); o[4][t] row 0 holds
// the row sums, accumulated by the same P V MFMA against a row of ones, so
// numerator and denominator use the same bf16 probabilities.  Scores are in
// log2 units (the bf16 queries arrive as Q log2(e) / sqrt(dh), scaled in the
// projection's fp32 epilogue before their one rounding), and m is the
// reference max in those units, a whole number.  The score MFMA starts from
// -m instead of 0, so it yields s - m directly and p = exp2(s - m) costs one
// exponential and no FMA.  The reference max is raised, by whole units, only
// when a score exceeds it by more than 2^8 in probability, so rescaling is
// rare; P < 512 stays finite in bf16 and the result does not depend on the
// reference.
// DH: head dim (64 or 128); o[0 .. DH/16 - 1] hold O^T, o[DH/16] the row sums.
template <int DH>
struct WaveAccT {
  static constexpr int ND = DH / 16;  // 16-row head-dim tiles of O^T
  static constexpr int NS = DH / 32;  // 32-dim k steps of a score MFMA chain
  floatx4 o[ND + 1][2];
  float m[2];
};

template <int DH>
__device__ inline void acc_init(WaveAccT<DH>& a) {
#pragma unroll
  for (int d = 0; d <= WaveAccT<DH>::ND; d++)
#pragma unroll
    for (int t = 0; t < 2; t++) a.o[d][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  a.m[0] = a.m[1] = -INFINITY;
}

// bf16 operand of the ones row (head-dim row 0 of the fifth tile)
__device__ inline bf16x8 ones_row(int c16) {
  const short one = c16 == 0 ? (short)0x3F80 : (short)0;
  return bf16x8{one, one, one, one, one, one, one, one};
}

// Row sum of query column (lane & 15) after the last tile (all lanes).
template <int DH>
__device__ inline float acc_rowsum(const WaveAccT<DH>& a, int t) {
  // row 0 of the sums tile lives in lane group 0, register 0
  const float v = a.o[WaveAccT<DH>::ND][t][0];
  return __shfl(v, threadIdx.x & 15, 64);
}

constexpr float kLazyLog2 = 8.0f;

// Scores of keys kbase + index >= kq[t] become -inf (probability 0), in place.
__device__ inline void tile_mask(floatx4 (&sacc)[4][2], int kbase, const int (&kq)[2], int g) {
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int sub = 0; sub < 4; sub++)
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (kbase + 32 * (sub >> 1) + 8 * g + 4 * (sub & 1) + r >= kq[t]) sacc[sub][t][r] = -INFINITY;
}

// One 64-key tile: online softmax of sacc = s - m (S^T in log2 units,
// permuted key rows, masked scores already -inf), then
// O^T += V^T P^T with the V^T operands from vop(d, wd).  `first` (wave-
// uniform) marks a wave's first tile, where every query has a visible key:
// there m is the tile max itself.  Inlined once per kernel: a second inlined
// copy makes the register allocator shuffle the accumulators at the join.
template <int DH, typename VOp>
__device__ inline void tile_update(WaveAccT<DH>& a, floatx4 (&sacc)[4][2], bool first,
                                   const bf16x8& ones, VOp vop) {
  constexpr int ND = WaveAccT<DH>::ND;
  bf16x8 pf[2][2];
#pragma unroll
  for (int t = 0; t < 2; t++) {
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 4; sub++)
#pragma unroll
      for (int r = 0; r < 4; r++) mx = fmaxf(mx, sacc[sub][t][r]);
    // Some column's tile max exceeds the threshold iff some lane's does, so
    // the check needs no cross-lane step; the column max (relative to m, or
    // to 0 on the first tile) is formed only when the reference moves.
    if (first || __any(mx > kLazyLog2)) {
      mx = wave_max16x4(mx);
      const bool need = mx > kLazyLog2;
      // The reference moves by whole units only: every probability is then
      // bf16(2^s) scaled by an exact power of two, whatever keys a split or
      // tile saw first, and rescales and split merges multiply by exact powers
      // of two, so split plans differ only in fp32 summation order.
      const float step = floorf(mx);
      float delta;
      if (first) {
        a.m[t] = step;
        delta = step;
      } else {
        const float mnew = need ? a.m[t] + step : a.m[t];
        const float alpha = __builtin_amdgcn_exp2f(a.m[t] - mnew);
        a.m[t] = mnew;
#pragma unroll
        for (int d = 0; d <= ND; d++) a.o[d][t] *= alpha;
        delta = need ? step : 0.f;  // rows without a new max keep their reference
      }
#pragma unroll
      for (int sub = 0; sub < 4; sub++)
#pragma unroll
        for (int r = 0; r < 4; r++) sacc[sub][t][r] -= delta;
    }
#pragma unroll
    for (int wd = 0; wd < 2; wd++) {
      float p[8];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        p[r] = __builtin_amdgcn_exp2f(sacc[2 * wd][t][r]);
        p[4 + r] = __builtin_amdgcn_exp2f(sacc[2 * wd + 1][t][r]);
      }
      const u32x4 u = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                       pack_bf16x2(p[6], p[7])};
      pf[wd][t] = __builtin_bit_cast(bf16x8, u);
    }
  }
#pragma unroll
  for (int wd = 0; wd < 2; wd++) {
#pragma unroll
    for (int d = 0; d < ND; d++) {
      const bf16x8 v = vop(d, wd);
#pragma unroll
      for (int t = 0; t < 2; t++)
        a.o[d][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pf[wd][t], a.o[d][t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 2; t++)
      a.o[ND][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[wd][t], a.o[ND][t], 0, 0, 0);
  }
}

// S^T - m for one 64-key tile from K operands kop(sub, s) (16 keys x 32
// dims): the first MFMA of each subtile starts from -m (from 0 on a wave's
// first tile, where m is not set yet).
template <int DH, typename KOp>
__device__ inline void tile_scores(floatx4 (&sacc)[4][2], const bf16x8 (&qf)[2][DH / 32],
                                   const WaveAccT<DH>& a, bool first, KOp kop) {
  constexpr int NS = WaveAccT<DH>::NS;
  floatx4 init[2];
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const float b = first ? 0.f : -a.m[t];
    init[t] = floatx4{b, b, b, b};
  }
#pragma unroll
  for (int sub = 0; sub < 4; sub++) {
    bf16x8 kk[NS];
#pragma unroll
    for (int s = 0; s < NS; s++) kk[s] = kop(sub, s);
#pragma unroll
    for (int t = 0; t < 2; t++) {
      sacc[sub][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[0], qf[t][0], init[t], 0, 0, 0);
#pragma unroll
      for (int s = 1; s < NS; s++)
        sacc[sub][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[s], qf[t][s], sacc[sub][t], 0, 0, 0);
    }
  }
}

// ====================================================================== prefill
namespace pf {
constexpr int QW = 32, NW = 4, QT = QW * NW;  // queries per wave / per workgroup
constexpr int KT = 64;                        // keys per tile
constexpr int MAX_SPLIT = 4;                  // key splits per (query tile, head)
}

// Workgroups are dealt round-robin to the 8 XCDs.  Give every XCD whole heads
// and let it work through them one at a time, each head's longest (latest)
// query tiles first: the workgroups resident on an XCD then stream one head's
// K/V through its L2.  j in [0, nj) numbers the (query tile, key split) units
// of a head, longest first.
__device__ inline void prefill_block(int bid, int Hh, int nj, int* h, int* j) {
  if ((Hh & 7) == 0) {
    const int x = bid & 7, i = bid >> 3;
    *h = x + 8 * (i / nj);
    *j = nj - 1 - i % nj;
  } else {
    *h = bid % Hh;
    *j = nj - 1 - bid / Hh;
  }
}

// Key range of split sp of a query tile whose keys end at kend_max: whole
// 64-key tiles, as even as the tile count allows.
__device__ __host__ inline void prefill_split_range(int kend_max, int sp, int nsplit, int* k_lo,
                                                    int* k_hi) {
  const int ntile = (kend_max + pf::KT - 1) / pf::KT;
  *k_lo = (sp * ntile / nsplit) * pf::KT;
  const int hi = ((sp + 1) * ntile / nsplit) * pf::KT;
  *k_hi = hi < kend_max ? hi : kend_max;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One 16-byte-per-lane buffer load into LDS (64 lanes fill 1 KiB at lds).
// A plain function, so that template kernels never hand dependent operands
// to the builtin (the host pass drops such kernels' launch stubs).
__device__ inline void buffer_lds16(__amdgpu_buffer_rsrc_t rs, char* lds, unsigned voff, unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// K and V^T tiles go from global memory straight into LDS (global_load_lds:
// lane i of a wave fills bytes [16i, 16i+16) of the destination).  Both use
// 128-byte rows of 8 16-byte chunks, chunk c of row r stored at slot
// c ^ (r & 7): the 16-byte fragment reads of 16 consecutive rows are then
// free of bank conflicts.  K row j of the tile holds the key whose S^T slot is
// j, so each lane fetches the key that belongs at its LDS position.  Two
// stages, one barrier per tile.
template <int DH>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    bf16_t* __restrict__ out, int nq, int row0, int cap, int Hh, FrameTab tab, int nsplit,
    float* __restrict__ part, int n_ep, long long kv_ep) {
  using namespace pf;
  static_assert(DH == 64 || DH == 128, "head dim");
  // A K tile is DH/64 halves of 64 keys x 64 dims (128-byte rows), a V^T
  // tile DH rows of 64 keys: both DH * 128 bytes.
  constexpr int NS = DH / 32, ND = DH / 16, TB = KT * DH * 2;
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TB];  // [stage][K | V^T]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int ntq = (nq + QT - 1) / QT, HE = Hh * n_ep;
  // (episode, head) pairs are scheduled as HE heads; episode ep's queries,
  // output rows and cache sit at their own offsets, with the same frame table
  int hx, j;
  prefill_block(blockIdx.x, HE, ntq * nsplit, &hx, &j);
  const int ep = hx / Hh, h = hx - ep * Hh;
  q += (long long)ep * Hh * nq * DH;
  kc += ep * kv_ep;
  vc += ep * kv_ep;
  out += (long long)ep * nq * Hh * DH;
  const int qt = j / nsplit, sp = j % nsplit;
  const int q0 = qt * QT;
  const int qlast = min(q0 + QT, nq) - 1;
  const int kend_min = kend_of_row(tab, row0 + q0);
  const int kend_max = kend_of_row(tab, row0 + qlast);
  // This workgroup's keys: [k_lo, k_hi).  The host splits only where the first
  // tile of every split holds a visible key for every query of the tile.
  int k_lo, k_hi;
  prefill_split_range(kend_max, sp, nsplit, &k_lo, &k_hi);
  const bf16_t* kh = kc + (long long)h * cap * DH;
  const bf16_t* vh = vc + (long long)h * DH * cap;

  int kq[2];
  bf16x8 qf[2][NS];
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int qi = q0 + w * QW + 16 * t + c16;
    const bool ok = qi < nq;
    kq[t] = ok ? kend_of_row(tab, row0 + qi) : kend_max;
#pragma unroll
    for (int s = 0; s < NS; s++)
      qf[t][s] = ok ? *(const bf16x8*)(q + ((long long)h * nq + qi) * DH + 32 * s + 8 * g)
                    : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  WaveAccT<DH> acc;
  acc_init(acc);
  const bf16x8 ones = ones_row(c16);

  // Load instruction i of wave w fills tile rows 8(4i + w) .. +7; lane l
  // covers row 8(4i + w) + l/8, slot l%8, i.e. chunk (l%8) ^ (row & 7).
  // K rows stay inside the cache (kt + 64 <= cap); rows past kend_max are
  // masked, V^T columns past kend_max are zeroed after the tile lands.
  // The tiles come in through buffer loads into LDS: a per-head descriptor,
  // a fixed per-lane byte offset and the tile's offset in a scalar register,
  // so issuing a tile costs no vector arithmetic.  Offsets stay below 2 GiB
  // (cap * 128 bytes per head).
  // K half hf (dims 64 hf ..) of tile row `row` holds key perm_key(row): load
  // (hf, i) fills half hf, rows 8(4i + w) .. +7; V^T load i fills rows 8(4i + w) ..
  const int lrow = lane >> 3, lkc = (lane & 7) ^ lrow;
  constexpr int KH = DH / 64, VL = DH / 32;
  unsigned koff[KH][2], voff[VL];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int row = (4 * i + w) * 8 + lrow;
#pragma unroll
    for (int hf = 0; hf < KH; hf++)
      koff[hf][i] = (unsigned)(perm_key(row >> 4, row & 15) * DH + 64 * hf + lkc * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < VL; i++) voff[i] = (unsigned)(((4 * i + w) * 8 + lrow) * cap + lkc * 8) * 2u;
  const auto krs = __builtin_amdgcn_make_buffer_rsrc((void*)kh, (short)0, 0x7FFFFFFF, 0x00020000);
  const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vh, (short)0, 0x7FFFFFFF, 0x00020000);
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the LDS destinations are scalar
  auto issue = [&](int kt, int buf) {
    char* sk = smem + buf * 2 * TB;
    char* sv = sk + TB;
#pragma unroll
    for (int hf = 0; hf < KH; hf++)
#pragma unroll
      for (int i = 0; i < 2; i++)
        buffer_lds16(krs, sk + hf * 8192 + (4 * i + wu) * 1024, koff[hf][i], (unsigned)kt * (2u * DH));
#pragma unroll
    for (int i = 0; i < VL; i++) buffer_lds16(vrs, sv + (4 * i + wu) * 1024, voff[i], (unsigned)kt * 2u);
  };

  const int x7 = c16 & 7;
  // every issued tile is waited for inside the loop (no LDS write may land
  // after the workgroup has left)
  if (k_lo < k_hi) issue(k_lo, (k_lo / KT) & 1);
  // One tile; FIRST (tile 0, where every query sees a key) is a compile-time
  // flag so that the later tiles carry no test of it.
  auto tile = [&](int kt, auto first_tag) {
    constexpr bool FIRST = decltype(first_tag)::value;
    const int buf = (kt / KT) & 1;
    char* sk = smem + buf * 2 * TB;
    char* sv = sk + TB;
    wait_vmem();      // this wave's transfers of the tile have landed in LDS,
    __syncthreads();  // then everyone's
    if (kt + KT > kend_max) {
      // tail tile: V^T columns past kend_max may hold anything (0 * NaN)
#pragma unroll
      for (int i = 0; i < DH / 32; i++) {
        const int c = tid + 256 * i, row = c >> 3, slot = c & 7, ch = slot ^ (row & 7);
        const int k0 = kt + 8 * ch;
        if (k0 + 8 > kend_max) {
          bf16x8* p = (bf16x8*)(sv + row * 128 + slot * 16);
          bf16x8 x = *p;
#pragma unroll
          for (int j = 0; j < 8; j++)
            if (k0 + j >= kend_max) x[j] = 0;
          *p = x;
        }
      }
      __syncthreads();
    }
    bf16x8 kf[4][NS], vf[ND][2];
    auto read_v = [&] {
#pragma unroll
      for (int d = 0; d < ND; d++)
#pragma unroll
        for (int wd = 0; wd < 2; wd++)
          vf[d][wd] = *(const bf16x8*)(sv + (16 * d + c16) * 128 + (((4 * wd + g) ^ x7) * 16));
    };
#pragma unroll
    for (int sub = 0; sub < 4; sub++)
#pragma unroll
      for (int s = 0; s < NS; s++)
        kf[sub][s] = *(const bf16x8*)(sk + (s >> 1) * 8192 + (16 * sub + c16) * 128 +
                                      (((4 * (s & 1) + g) ^ x7) * 16));
    // dh = 64: every fragment read of the tile before its MFMAs; dh = 128
    // reads V^T after the scores so that K and V^T fragments are never live
    // together
    if constexpr (DH == 64) read_v();
    __builtin_amdgcn_sched_barrier(0);
    // the other stage was last read in the previous tile, which every wave has left
    if (kt + KT < k_hi) issue(kt + KT, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    floatx4 sacc[4][2];
    tile_scores(sacc, qf, acc, FIRST, [&](int sub, int s) { return kf[sub][s]; });
    if constexpr (DH != 64) read_v();
    if (kt + KT > kend_min) tile_mask(sacc, kt, kq, g);
    tile_update(acc, sacc, FIRST, ones, [&](int d, int wd) { return vf[d][wd]; });
  };
  if (k_lo < k_hi) tile(k_lo, std::true_type{});
  for (int kt = k_lo + KT; kt < k_hi; kt += KT) tile(kt, std::false_type{});
  const int D = Hh * DH;
  if (part != nullptr) {
    // split partial (log2-domain max m, row sum l, unnormalised O), heads
    // numbered ep * Hh + h: m [nsplit][HE][nq], l [nsplit][HE][nq], o [nsplit][HE][nq][DH]
    const long long plane = (long long)nsplit * HE * nq;
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const float l = acc_rowsum(acc, t);
      const int qi = q0 + w * QW + 16 * t + c16;
      if (qi >= nq) continue;
      const long long pi = ((long long)sp * HE + hx) * nq + qi;
      if (g == 0) {
        part[pi] = acc.m[t];
        part[plane + pi] = l;
      }
#pragma unroll
      for (int d = 0; d < ND; d++)
        *(floatx4*)(part + 2 * plane + pi * DH + 16 * d + 4 * g) = acc.o[d][t];
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const float l = acc_rowsum(acc, t);
    const int qi = q0 + w * QW + 16 * t + c16;
    if (qi >= nq) continue;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < ND; d++) {
      uint2 v = {pack_bf16x2(acc.o[d][t][0] * inv, acc.o[d][t][1] * inv),
                 pack_bf16x2(acc.o[d][t][2] * inv, acc.o[d][t][3] * inv)};
      *(uint2*)(out + (long long)qi * D + h * DH + 16 * d + 4 * g) = v;
    }
  }
}

// Merge of the key splits of one launch: one wavefront per (query, head),
// lane = head-dim index, splits combined in a fixed order.
template <int DH>
__global__ __launch_bounds__(256) void attn_prefill_merge_kernel(const float* __restrict__ part,
                                                                 int nsplit, int Hh, int nq,
                                                                 bf16_t* __restrict__ out, int n_ep) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int HE = Hh * n_ep;
  if (wv >= nq * HE) return;
  const int qi = wv / HE, hx = wv - qi * HE, ep = hx / Hh, h = hx - ep * Hh;
  const long long plane = (long long)nsplit * HE * nq;
  float mv[pf::MAX_SPLIT], lv[pf::MAX_SPLIT], ov[pf::MAX_SPLIT][DH / 64];
#pragma unroll
  for (int s = 0; s < pf::MAX_SPLIT; s++) {
    if (s < nsplit) {
      const long long pi = ((long long)s * HE + hx) * nq + qi;
      mv[s] = part[pi];
      lv[s] = part[plane + pi];
#pragma unroll
      for (int r = 0; r < DH / 64; r++) ov[s][r] = part[2 * plane + pi * DH + 64 * r + lane];
    }
  }
  float M = mv[0];
#pragma unroll
  for (int s = 1; s < pf::MAX_SPLIT; s++)
    if (s < nsplit) M = fmaxf(M, mv[s]);
  float L = 0.f, O[DH / 64];
#pragma unroll
  for (int r = 0; r < DH / 64; r++) O[r] = 0.f;
#pragma unroll
  for (int s = 0; s < pf::MAX_SPLIT; s++) {
    if (s < nsplit) {
      const float f = __builtin_amdgcn_exp2f(mv[s] - M);
      L = fmaf(lv[s], f, L);
#pragma unroll
      for (int r = 0; r < DH / 64; r++) O[r] = fmaf(ov[s][r], f, O[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < DH / 64; r++)
    out[((long long)ep * nq + qi) * Hh * DH + h * DH + 64 * r + lane] = dev_f2bf(O[r] / L);
}

// fp32: one thread per (query, head)
template <int DH>
__global__ __launch_bounds__(64) void attn_prefill_f32_kernel(const float* __restrict__ q,
                                                              const float* __restrict__ kc,
                                                              const float* __restrict__ vc,
                                                              float* __restrict__ out, int nq,
                                                              int row0, int cap, int Hh,
                                                              FrameTab tab, float scale,
                                                              long long kv_ep) {
  const int h = blockIdx.y, ep = blockIdx.z;
  const int qi = blockIdx.x * 64 + threadIdx.x;
  if (qi >= nq) return;
  q += (long long)ep * Hh * nq * DH;
  out += (long long)ep * nq * Hh * DH;
  const float* qr = q + ((long long)h * nq + qi) * DH;
  const float* kh = kc + ep * kv_ep + (long long)h * cap * DH;
  const float* vh = vc + ep * kv_ep + (long long)h * DH * cap;
  float qv[DH], o[DH];
#pragma unroll
  for (int d = 0; d < DH; d++) { qv[d] = qr[d]; o[d] = 0.f; }
  const int kend = kend_of_row(tab, row0 + qi);
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < kend; j++) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DH; d++) s = fmaf(qv[d], kh[(long long)j * DH + d], s);
    float mn, a, p;
    {
      // the scaled score is rounded once and never fused into s - mn: the
      // largest key then weighs exactly 1
#pragma clang fp contract(off)
      s = s * scale;
      mn = fmaxf(m, s);
      a = expf(m - mn);
      p = expf(s - mn);
    }
    l = l * a + p;
#pragma unroll
    for (int d = 0; d < DH; d++) o[d] = fmaf(p, vh[(long long)d * cap + j], o[d] * a);
    m = mn;
  }
  const float inv = 1.0f / l;
  float* orow = out + (long long)qi * Hh * DH + h * DH;
#pragma unroll
  for (int d = 0; d < DH; d++) orow[d] = o[d] * inv;
}

static int device_cus() {
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  return n_cu;
}

size_t attn_prefill_split_bytes(int Hh, int dh, int max_rows) {
  // a launch splits only below 2 workgroups per CU, so splits x workgroups
  // stays below 4 per CU: at most 4 n_cu QT (query, head, split) partials
  const long long n = std::min<long long>((long long)pf::MAX_SPLIT * Hh * max_rows,
                                          4ll * device_cus() * pf::QT);
  return (size_t)n * (dh + 2) * sizeof(float);
}

// Key splits of a launch: enough (query tile, head, split) workgroups for two
// per CU, at most MAX_SPLIT, and only where, for every query tile, the first
// tile of every split holds a key that every query of the tile sees (the
// tile loop takes a split's first tile as setting the reference max).  Under
// the block-causal mask a query sees a key prefix, so that holds when the
// last split starts below the tile's smallest prefix end.
static int prefill_splits(int Hh, int dh, int nq, int row0, const FrameTab& tab, size_t part_bytes) {
  const int ntq = (nq + pf::QT - 1) / pf::QT, n_cu = device_cus();
  const long long g = (long long)ntq * Hh;
  if (g >= 2ll * n_cu) return 1;
  int S = (int)std::min<long long>(pf::MAX_SPLIT, (2ll * n_cu + g - 1) / g);
  for (; S > 1; S--) {
    if ((size_t)S * Hh * nq * (dh + 2) * sizeof(float) > part_bytes) continue;
    bool ok = true;
    for (int qt = 0; qt < ntq && ok; qt++) {
      const int q0 = qt * pf::QT, ql = std::min(q0 + pf::QT, nq) - 1;
      const int kmin = tab.kend[(row0 + q0) / tab.P], kmax = tab.kend[(row0 + ql) / tab.P];
      int lo, hi;
      prefill_split_range(kmax, S - 1, S, &lo, &hi);
      ok = (kmax + pf::KT - 1) / pf::KT >= S && lo < kmin;
    }
    if (ok) break;
  }
  return S;
}

hipError_t attn_prefill(hipStream_t s, int dt, int Hh, int dh, int nq, int row0,
                        const FrameTab& tab, const void* q, const void* kc, const void* vc, int cap,
                        void* out, float* part, size_t part_bytes, int n_ep, long long kv_ep) {
  if (nq <= 0 || n_ep <= 0) return hipSuccess;
  if (dh != 64 && dh != 128) return hipErrorInvalidValue;
  const float scale = dh == 64 ? 0.125f : 0.08838834764831845f;  // 1 / sqrt(dh)
  double pairs = 0.0;  // visible (query, key) pairs of one episode
  for (int r = row0; r < row0 + nq;) {
    int f = r / tab.P, e = std::min(row0 + nq, (f + 1) * tab.P);
    pairs += (double)(e - r) * tab.kend[f];
    r = e;
  }
  const int es = dt == WAM_BF16 ? 2 : 4;
  const int kmax = tab.kend[(row0 + nq - 1) / tab.P];
  const int HE = Hh * n_ep;  // (episode, head) pairs
  if (dt == WAM_BF16) {
    const int nsplit = part ? prefill_splits(HE, dh, nq, row0, tab, part_bytes) : 1;
    {
      TimingScope ts(s, KC_ATTN_PREFILL, (double)HE * dh * es * (2.0 * nq + 2.0 * kmax),
                     4.0 * dh * HE * pairs);
      dim3 grid(((nq + pf::QT - 1) / pf::QT) * HE * nsplit);
      if (dh == 64)
        hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, dim3(256), 0, s, (const bf16_t*)q,
                           (const bf16_t*)kc, (const bf16_t*)vc, (bf16_t*)out, nq, row0, cap, Hh,
                           tab, nsplit, nsplit > 1 ? part : nullptr, n_ep, kv_ep);
      else
        hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, dim3(256), 0, s, (const bf16_t*)q,
                           (const bf16_t*)kc, (const bf16_t*)vc, (bf16_t*)out, nq, row0, cap, Hh,
                           tab, nsplit, nsplit > 1 ? part : nullptr, n_ep, kv_ep);
    }
    if (nsplit > 1) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      TimingScope ts(s, KC_ATTN_MERGE,
                     (double)nsplit * HE * nq * (dh + 2) * 4 + (double)nq * HE * dh * es, 0.0);
      if (dh == 64)
        hipLaunchKernelGGL(attn_prefill_merge_kernel<64>, dim3((nq * HE + 3) / 4), dim3(256), 0, s,
                           (const float*)part, nsplit, Hh, nq, (bf16_t*)out, n_ep);
      else
        hipLaunchKernelGGL(attn_prefill_merge_kernel<128>, dim3((nq * HE + 3) / 4), dim3(256), 0,
                           s, (const float*)part, nsplit, Hh, nq, (bf16_t*)out, n_ep);
    }
  } else {
    TimingScope ts(s, KC_ATTN_PREFILL, (double)HE * dh * es * (2.0 * nq + 2.0 * kmax),
                   4.0 * dh * HE * pairs);
    dim3 grid((nq + 63) / 64, Hh, n_ep);
    if (dh == 64)
      hipLaunchKernelGGL(attn_prefill_f32_kernel<64>, grid, dim3(64), 0, s, (const float*)q,
                         (const float*)kc, (const float*)vc, (float*)out, nq, row0, cap, Hh, tab,
                         scale, kv_ep);
    else
      hipLaunchKernelGGL(attn_prefill_f32_kernel<128>, grid, dim3(64), 0, s, (const float*)q,
                         (const float*)kc, (const float*)vc, (float*)out, nq, row0, cap, Hh, tab,
                         scale, kv_ep);
  }
  return hipGetLastError();
}

// ====================================================================== action
namespace act {
constexpr int H = 32;            // queries per (episode, head)
constexpr int KT = 64;           // keys per wave tile
constexpr int MAX_SPLITS = 64;   // splits per (episode, head), own keys included
}

struct ActGeom {
  int B, Hh, cap, n_act, S;  // S = max splits per (b, h) incl. the own-key split
  ActLens lens;
  int kc[WAM_MAX_BATCH];     // cache keys per split of episode b (0: no cache)
};

// Eight E4M3 codes (two words) -> eight bf16 operand values times a
// power-of-two scale (v_cvt_scalef32_pk_bf16_fp8, exact for such scales).
__device__ inline bf16x8 e4m3x8_bf16(unsigned lo, unsigned hi, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false));
  r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true));
  r[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false));
  r[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true));
  return __builtin_bit_cast(bf16x8, r);
}

// One 64-key tile of bf16 K rows (A of S^T) and V^T rows (A of P V), all
// loads unconditional so that they are in flight together: K rows past key1
// read row key1 - 1 (their scores are masked to -inf), V^T chunks that start
// past key1 read the row's first chunk (zeroed by the caller).
template <int DH>
__device__ inline void bf16_k_tile(bf16x8 (&ak)[4][DH / 32], const bf16_t* kb, int kt, int key1,
                                   int c16, int g) {
#pragma unroll
  for (int sub = 0; sub < 4; sub++) {
    const int key = min(kt + perm_key(sub, c16), key1 - 1);
#pragma unroll
    for (int ss = 0; ss < DH / 32; ss++)
      ak[sub][ss] = *(const bf16x8*)(kb + (long long)key * DH + 32 * ss + 8 * g);
  }
}
template <int DH>
__device__ inline void bf16_v_tile(bf16x8 (&av)[DH / 16][2], const bf16_t* vb, int kt, int key0,
                                   int key1, int vld, int c16, int g) {
#pragma unroll
  for (int d = 0; d < DH / 16; d++)
#pragma unroll
    for (int wd = 0; wd < 2; wd++) {
      const int k0 = kt + 32 * wd + 8 * g;
      av[d][wd] = *(const bf16x8*)(vb + (long long)(16 * d + c16) * vld + (k0 < key1 ? k0 : key0));
    }
}
template <int DH>
__device__ inline void bf16_tiles(bf16x8 (&ak)[4][DH / 32], bf16x8 (&av)[DH / 16][2],
                                  const bf16_t* kb, const bf16_t* vb, int kt, int key0, int key1,
                                  int vld, int c16, int g) {
  bf16_k_tile<DH>(ak, kb, kt, key1, c16, g);
  bf16_v_tile<DH>(av, vb, kt, key0, key1, vld, c16, g);
}
// P is zero past key1, but 0 * V must not meet a non-finite V
template <int DH>
__device__ inline void zero_v_tail(bf16x8 (&av)[DH / 16][2], int kt, int key1, int g) {
#pragma unroll
  for (int wd = 0; wd < 2; wd++) {
    const int k0 = kt + 32 * wd + 8 * g;
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (k0 + j >= key1)
#pragma unroll
        for (int d = 0; d < DH / 16; d++) av[d][wd][j] = 0;
  }
}

// Split (b, h, s): cache keys [s*kc[b], min(len, (s+1)*kc[b])) for s < ncs(b),
// the chunk's own keys for s == ncs(b).  Writes the split's (m, l, o) in the
// log2 domain: m [32], l [32], o [32][64] (unnormalised).
// F8: the cache is E4M3 (kc, vc bytes; ksc, vsc tile scales [B][Hh][cap/64]).
// Its rows are stored in the order the lanes consume them, so one 16-byte
// load gives a lane two 8-element fragments of a K row (dims 64u + 8g.. and
// 64u + 32 + 8g.., lane group g's DH/4 bytes contiguous) or of a V^T row
// (keys 8g.. and 32+8g.. of the tile); converted with the tile's scale they
// are the bf16 operands of the same MFMAs.  The chunk's own keys stay bf16.
template <bool F8, int DH>
__global__ __launch_bounds__(256, 2) void attn_action_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ ka, const bf16_t* __restrict__ va,
    const void* __restrict__ kc, const void* __restrict__ vc, const float* __restrict__ ksc,
    const float* __restrict__ vsc, ActGeom G, float* __restrict__ part) {
  using namespace act;
  static_assert(DH == 64 || DH == 128, "head dim");
  constexpr int NS = DH / 32, ND = DH / 16;
  __shared__ float sm[4][H], sl[4][H];
  __shared__ float so[4][H][DH + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int len = G.lens.len[b];
  const int chunk = G.kc[b];
  const int ncs = (kc != nullptr && chunk > 0) ? (len + chunk - 1) / chunk : 0;
  const bool own = (s == ncs);
  if (s > ncs || (own && G.n_act == 0)) return;
  const bf16_t* kb;
  const bf16_t* vb;
  const uint8_t* k8 = nullptr;
  const uint8_t* v8 = nullptr;
  const float* ksh = nullptr;
  const float* vsh = nullptr;
  int key0, key1, vld;
  if (!own) {
    const long long hb = (long long)b * G.Hh + h;
    kb = (const bf16_t*)kc + hb * G.cap * DH;
    vb = (const bf16_t*)vc + hb * DH * G.cap;
    if constexpr (F8) {
      k8 = (const uint8_t*)kc + hb * G.cap * DH;
      v8 = (const uint8_t*)vc + hb * DH * G.cap;
      ksh = ksc + hb * (G.cap / 64);
      vsh = vsc + hb * (G.cap / 64);
    }
    key0 = s * chunk;
    key1 = min(len, key0 + chunk);
    vld = G.cap;
  } else {
    kb = ka + ((long long)b * G.Hh + h) * H * DH;
    vb = va + ((long long)b * G.Hh + h) * DH * H;
    key0 = 0;
    key1 = G.n_act;
    vld = H;
  }
  // queries: B operand of S^T = K Q^T
  bf16x8 qf[2][NS];
  const bf16_t* qb = q + ((long long)b * G.Hh + h) * H * DH;
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int ss = 0; ss < NS; ss++)
      qf[t][ss] = *(const bf16x8*)(qb + (16 * t + c16) * DH + 32 * ss + 8 * g);

  WaveAccT<DH> acc;
  acc_init(acc);
  const bf16x8 ones = ones_row(c16);
  const int kq[2] = {key1, key1};
  for (int kt = key0 + w * KT; kt < key1; kt += 4 * KT) {
    if constexpr (DH == 128) {
      // 128-wide heads: the V^T tile is loaded after the scores, so that the
      // K and V^T fragments (64 registers each) are never live together
      const bool tail = kt + KT > key1;  // wave-uniform
      const bool first = kt == key0 + w * KT;
      floatx4 sacc[4][2];
      bf16x8 ak[4][NS], av[ND][2];
      const bool f8 = F8 && !own;  // an E4M3 split (kt is then a multiple of 64)
      if (f8) {
        const float sk = ksh[kt >> 6];
        u32x4 rk[4][2];
#pragma unroll
        for (int sub = 0; sub < 4; sub++) {
          const int key = min(kt + perm_key(sub, c16), key1 - 1);
#pragma unroll
          for (int u = 0; u < 2; u++) rk[sub][u] = *(const u32x4*)(k8 + (long long)key * DH + 32 * g + 16 * u);
        }
#pragma unroll
        for (int sub = 0; sub < 4; sub++)
#pragma unroll
          for (int u = 0; u < 2; u++) {
            ak[sub][2 * u] = e4m3x8_bf16(rk[sub][u][0], rk[sub][u][1], sk);
            ak[sub][2 * u + 1] = e4m3x8_bf16(rk[sub][u][2], rk[sub][u][3], sk);
          }
      } else {
        bf16_k_tile<DH>(ak, kb, kt, key1, c16, g);
      }
      tile_scores(sacc, qf, acc, first, [&](int sub, int ss) { return ak[sub][ss]; });
      if (f8) {
        const float sv = vsh[kt >> 6];
        u32x4 rv[ND];
#pragma unroll
        for (int d = 0; d < ND; d++)
          rv[d] = *(const u32x4*)(v8 + (long long)(16 * d + c16) * G.cap + kt + 16 * g);
#pragma unroll
        for (int d = 0; d < ND; d++) {
          av[d][0] = e4m3x8_bf16(rv[d][0], rv[d][1], sv);
          av[d][1] = e4m3x8_bf16(rv[d][2], rv[d][3], sv);
        }
      } else {
        bf16_v_tile<DH>(av, vb, kt, key0, key1, vld, c16, g);
      }
      if (tail) {
        zero_v_tail<DH>(av, kt, key1, g);
        tile_mask(sacc, kt, kq, g);
      }
      tile_update(acc, sacc, first, ones, [&](int d, int wd) { return av[d][wd]; });
    } else {
    // ---- loads: K rows (A of S^T) and V^T rows (A of P V).  All loads are
    // unconditional so that they are in flight together: K rows past key1
    // read row key1 - 1 (their scores are masked to -inf), V^T chunks that
    // start past key1 read the row's first chunk and are zeroed below.
    bf16x8 ak[4][NS], av[ND][2];
    if constexpr (F8) {
    if (!own) {
      // E4M3 tile: kt is a multiple of 64 (splits are whole tiles), and the
      // 16-byte V^T reads stay inside the tile, hence below cap; keys past
      // key1 are zeroed below like the bf16 ones
      const float sk = ksh[kt >> 6], sv = vsh[kt >> 6];
      u32x4 rk[4], rv[4];
#pragma unroll
      for (int sub = 0; sub < 4; sub++) {
        const int key = min(kt + perm_key(sub, c16), key1 - 1);
        rk[sub] = *(const u32x4*)(k8 + (long long)key * 64 + 16 * g);
      }
#pragma unroll
      for (int d = 0; d < 4; d++)
        rv[d] = *(const u32x4*)(v8 + (long long)(16 * d + c16) * G.cap + kt + 16 * g);
#pragma unroll
      for (int sub = 0; sub < 4; sub++) {
        ak[sub][0] = e4m3x8_bf16(rk[sub][0], rk[sub][1], sk);
        ak[sub][1] = e4m3x8_bf16(rk[sub][2], rk[sub][3], sk);
      }
#pragma unroll
      for (int d = 0; d < 4; d++) {
        av[d][0] = e4m3x8_bf16(rv[d][0], rv[d][1], sv);
        av[d][1] = e4m3x8_bf16(rv[d][2], rv[d][3], sv);
      }
    } else {
      bf16_tiles<DH>(ak, av, kb, vb, kt, key0, key1, vld, c16, g);
    }
    } else {
      bf16_tiles<DH>(ak, av, kb, vb, kt, key0, key1, vld, c16, g);
    }
    const bool tail = kt + KT > key1;  // wave-uniform
    if (tail) {
      // P is zero past key1, but 0 * V must not meet a non-finite V
#pragma unroll
      for (int wd = 0; wd < 2; wd++) {
        const int k0 = kt + 32 * wd + 8 * g;
#pragma unroll
        for (int j = 0; j < 8; j++)
          if (k0 + j >= key1)
#pragma unroll
            for (int d = 0; d < ND; d++) av[d][wd][j] = 0;
      }
    }
    // ---- S^T, softmax, P V
    floatx4 sacc[4][2];
    tile_scores(sacc, qf, acc, kt == key0 + w * KT, [&](int sub, int ss) { return ak[sub][ss]; });
    auto vop = [&](int d, int wd) { return av[d][wd]; };
    if (tail) tile_mask(sacc, kt, kq, g);
    tile_update(acc, sacc, kt == key0 + w * KT, ones, vop);
    }
  }
  // ---- per-wave state to LDS (waves without keys hold m = -inf, l = 0, o = 0)
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const float l = acc_rowsum(acc, t);
    const int qi = 16 * t + c16;
    if (g == 0) {
      sm[w][qi] = acc.m[t];
      sl[w][qi] = l;
    }
#pragma unroll
    for (int d = 0; d < ND; d++)
#pragma unroll
      for (int r = 0; r < 4; r++) so[w][qi][16 * d + 4 * g + r] = acc.o[d][t][r];
  }
  __syncthreads();
  // ---- merge the 4 waves in a fixed order, write the split's partial
  const long long pidx = (((long long)b * G.Hh + h) * G.S + s);
  float* pm = part + pidx * H;
  float* pl = part + (long long)G.B * G.Hh * G.S * H + pidx * H;
  float* po = part + 2ll * G.B * G.Hh * G.S * H + pidx * H * DH;
  for (int i = tid; i < H * DH; i += 256) {
    const int qi = i / DH, d = i % DH;
    float M = sm[0][qi];
#pragma unroll
    for (int ww = 1; ww < 4; ww++) M = fmaxf(M, sm[ww][qi]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ww++) {
      const float f =
          (sm[ww][qi] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sm[ww][qi] - M);
      L += sl[ww][qi] * f;
      O += so[ww][qi][d] * f;
    }
    po[qi * DH + d] = O;
    if (d == 0) {
      pm[qi] = M;  // log2 units, as the split merge expects
      pl[qi] = L;
    }
  }
}

// Merge splits 0..ns-1 of (b, h) (ns <= 64): one wavefront per (query, head,
// episode).  Lane j reads split j's (m, l); lane d reads every split's o[d];
// all loads are issued before any arithmetic.  Fixed reduction order.
template <typename TO, int DH>
__global__ __launch_bounds__(64) void attn_action_merge_kernel(const float* __restrict__ part,
                                                               ActGeom G, TO* __restrict__ out) {
  using namespace act;
  const int qi = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int len = G.lens.len[b];
  const int ncs = G.kc[b] > 0 ? (len + G.kc[b] - 1) / G.kc[b] : 0;
  const int ns = ncs + (G.n_act > 0 ? 1 : 0);
  const long long base = ((long long)b * G.Hh + h) * G.S;
  const float* pm = part + base * H + qi;
  const float* pl = part + (long long)G.B * G.Hh * G.S * H + base * H + qi;
  const float mj = lane < ns ? pm[lane * H] : -INFINITY;
  const float lj = lane < ns ? pl[lane * H] : 0.f;
  float M = mj;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  const float wj = lane < ns ? __builtin_amdgcn_exp2f(mj - M) : 0.f;
  float L = lj * wj;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
  // lane d takes head dims d, d + 64, ..
#pragma unroll
  for (int r = 0; r < DH / 64; r++) {
    const float* po =
        part + 2ll * G.B * G.Hh * G.S * H + (base * H + qi) * DH + 64 * r + lane;
    float ov[MAX_SPLITS];
#pragma unroll
    for (int j = 0; j < MAX_SPLITS; j++) ov[j] = (j < ns) ? po[(long long)j * H * DH] : 0.f;
    float O = 0.f;
#pragma unroll
    for (int j = 0; j < MAX_SPLITS; j++)
      if (j < ns) O = fmaf(__shfl(wj, j, 64), ov[j], O);
    out[((long long)b * H + qi) * G.Hh * DH + h * DH + 64 * r + lane] = from_f<TO>(O / L);
  }
}

// fp32: one thread per (episode, head, query)
template <int DH>
__global__ __launch_bounds__(64) void attn_action_f32_kernel(const float* __restrict__ q,
                                                             const float* __restrict__ ka,
                                                             const float* __restrict__ va,
                                                             const float* __restrict__ kc,
                                                             const float* __restrict__ vc,
                                                             ActGeom G, float* __restrict__ out,
                                                             float scale) {
  using namespace act;
  const int h = blockIdx.x, b = blockIdx.y, qi = threadIdx.x;
  if (qi >= H) return;
  const float* qr = q + (((long long)b * G.Hh + h) * H + qi) * DH;
  float qv[DH], o[DH];
#pragma unroll
  for (int d = 0; d < DH; d++) { qv[d] = qr[d]; o[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int part = 0; part < 2; part++) {
    const float* kb;
    const float* vb;
    int n, ld;
    if (part == 0) {
      if (!kc) continue;
      kb = kc + ((long long)b * G.Hh + h) * G.cap * DH;
      vb = vc + ((long long)b * G.Hh + h) * DH * G.cap;
      n = G.lens.len[b];
      ld = G.cap;
    } else {
      kb = ka + ((long long)b * G.Hh + h) * H * DH;
      vb = va + ((long long)b * G.Hh + h) * DH * H;
      n = G.n_act;
      ld = H;
    }
    for (int j = 0; j < n; j++) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DH; d++) s = fmaf(qv[d], kb[(long long)j * DH + d], s);
      float mn, a, p;
      {
        // the scaled score is rounded once and never fused into s - mn: the
        // largest key then weighs exactly 1
#pragma clang fp contract(off)
        s = s * scale;
        mn = fmaxf(m, s);
        a = expf(m - mn);
        p = expf(s - mn);
      }
      l = l * a + p;
#pragma unroll
      for (int d = 0; d < DH; d++) o[d] = fmaf(p, vb[(long long)d * ld + j], o[d] * a);
      m = mn;
    }
  }
  const float inv = 1.0f / l;
  float* orow = out + ((long long)b * H + qi) * G.Hh * DH + h * DH;
#pragma unroll
  for (int d = 0; d < DH; d++) orow[d] = o[d] * inv;
}

// Keys per split for one episode: a function of that episode's length, the
// head count and the device only, so an episode is split identically
// whatever the batch (batch independence is bitwise).  Measured on MI355X,
// about one workgroup per CU for a single episode is best: n_cu / Hh - 1
// cache splits (plus the own-key split) of whole 64-key tiles, at most 63.
// An explicit hint (tests) asks for a split count instead.
static int action_chunk(int len, int Hh, int splits_hint) {
  if (len <= 0) return 0;
  int splits = splits_hint;
  if (splits <= 0) {
    int dev = 0, n_cu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n_cu = 256;
    splits = std::max(1, std::min(act::MAX_SPLITS - 1, n_cu / std::max(Hh, 1) - 1));
  }
  const int kc = (len + splits - 1) / splits;
  return (kc + act::KT - 1) / act::KT * act::KT;
}

size_t attn_action_scratch_bytes(int B, int Hh, int H, int dh, int max_len, int splits_hint) {
  (void)max_len;
  (void)splits_hint;
  return (size_t)B * Hh * act::MAX_SPLITS * H * (dh + 2) * sizeof(float);
}

hipError_t attn_action(hipStream_t s, int dt, int B, int Hh, int H, int dh, const void* q,
                       const void* ka, const void* va, int n_act, const void* kc,
                       const void* vc, int cap, const ActLens& lens, void* out,
                       int splits_hint, void* scratch, size_t scratch_bytes, const float* ksc,
                       const float* vsc) {
  const bool f8 = ksc != nullptr;
  if (f8 && (dt != WAM_BF16 || !vsc || !kc)) return hipErrorInvalidValue;
  if (H != act::H || (dh != 64 && dh != 128)) return hipErrorInvalidValue;
  const float scale = dh == 64 ? 0.125f : 0.08838834764831845f;  // 1 / sqrt(dh)
  ActGeom G;
  G.B = B;
  G.Hh = Hh;
  G.cap = cap;
  G.n_act = n_act;
  G.lens = lens;
  if (!kc)
    for (int b = 0; b < B; b++) G.lens.len[b] = 0;
  double keys = 0.0;
  for (int b = 0; b < B; b++) keys += (double)G.lens.len[b] + n_act;
  const int es = dt == WAM_BF16 ? 2 : 4;
  const double ces = f8 ? 1.0 : es;  // bytes per cached element
  if (splits_hint >= act::MAX_SPLITS) return hipErrorInvalidValue;
  for (int b = 0; b < B; b++) G.kc[b] = kc ? action_chunk(G.lens.len[b], Hh, splits_hint) : 0;
  if (dt == WAM_F32) {
    G.S = 0;
    TimingScope ts(s, KC_ATTN_ACTION, keys * Hh * dh * 2 * es + 2.0 * B * H * Hh * dh * es,
                   4.0 * dh * Hh * H * keys);
    if (dh == 64)
      hipLaunchKernelGGL(attn_action_f32_kernel<64>, dim3(Hh, B), dim3(64), 0, s, (const float*)q,
                         (const float*)ka, (const float*)va, (const float*)kc, (const float*)vc,
                         G, (float*)out, scale);
    else
      hipLaunchKernelGGL(attn_action_f32_kernel<128>, dim3(Hh, B), dim3(64), 0, s, (const float*)q,
                         (const float*)ka, (const float*)va, (const float*)kc, (const float*)vc,
                         G, (float*)out, scale);
    return hipGetLastError();
  }
  G.S = 1;
  for (int b = 0; b < B; b++)
    if (G.kc[b] > 0) G.S = std::max(G.S, (G.lens.len[b] + G.kc[b] - 1) / G.kc[b] + 1);
  if (scratch_bytes < (size_t)B * Hh * G.S * H * (dh + 2) * sizeof(float)) return hipErrorInvalidValue;
  {
    double cached = 0.0;
    for (int b = 0; b < B; b++) cached += G.lens.len[b];
    const double kv_bytes = cached * Hh * dh * 2 * ces + (double)B * n_act * Hh * dh * 2 * es +
                            (f8 ? 2.0 * 4 * Hh * (cached / 64.0) : 0.0);
    TimingScope ts(s, KC_ATTN_ACTION, kv_bytes + 1.0 * B * H * Hh * dh * es,
                   4.0 * dh * Hh * H * keys);
    if (f8 && dh == 64)
      hipLaunchKernelGGL((attn_action_kernel<true, 64>), dim3(G.S, Hh, B), dim3(256), 0, s,
                         (const bf16_t*)q, (const bf16_t*)ka, (const bf16_t*)va, kc, vc, ksc, vsc,
                         G, (float*)scratch);
    else if (f8)
      hipLaunchKernelGGL((attn_action_kernel<true, 128>), dim3(G.S, Hh, B), dim3(256), 0, s,
                         (const bf16_t*)q, (const bf16_t*)ka, (const bf16_t*)va, kc, vc, ksc, vsc,
                         G, (float*)scratch);
    else if (dh == 64)
      hipLaunchKernelGGL((attn_action_kernel<false, 64>), dim3(G.S, Hh, B), dim3(256), 0, s,
                         (const bf16_t*)q, (const bf16_t*)ka, (const bf16_t*)va, kc, vc,
                         (const float*)nullptr, (const float*)nullptr, G, (float*)scratch);
    else
      hipLaunchKernelGGL((attn_action_kernel<false, 128>), dim3(G.S, Hh, B), dim3(256), 0, s,
                         (const bf16_t*)q, (const bf16_t*)ka, (const bf16_t*)va, kc, vc,
                         (const float*)nullptr, (const float*)nullptr, G, (float*)scratch);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TimingScope ts(s, KC_ATTN_MERGE,
                 (double)B * Hh * G.S * H * (dh + 2) * 4 + (double)B * H * Hh * dh * es, 0.0);
  if (dh == 64)
    hipLaunchKernelGGL((attn_action_merge_kernel<bf16_t, 64>), dim3(H, Hh, B), dim3(64), 0, s,
                       (const float*)scratch, G, (bf16_t*)out);
  else
    hipLaunchKernelGGL((attn_action_merge_kernel<bf16_t, 128>), dim3(H, Hh, B), dim3(64), 0, s,
                       (const float*)scratch, G, (bf16_t*)out);
  return hipGetLastError();
}

// ====================================================================== debug
struct FrameComp {
  int F, P;
  int comp[WAM_MAX_FRAMES];
};

__global__ void visibility_kernel(FrameTab tab, FrameComp fc, uint8_t* __restrict__ vis) {
  const long long n = (long long)fc.F * fc.P;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n * n;
       i += (long long)gridDim.x * blockDim.x) {
    const int qt = (int)(i / n), kt = (int)(i % n);
    const int cq = fc.comp[qt / fc.P], ck = fc.comp[kt / fc.P];
    uint8_t v = 0;
    if (cq >= 0 && ck >= 0) v = visible(tab, cq * fc.P + qt % fc.P, ck * fc.P + kt % fc.P) ? 1 : 0;
    vis[i] = v;
  }
}

hipError_t debug_visibility(hipStream_t s, const FrameTab& tab, const int* comp_of_frame,
                            int F, uint8_t* vis) {
  FrameComp fc;
  fc.F = F;
  fc.P = tab.P;
  for (int f = 0; f < F; f++) fc.comp[f] = comp_of_frame[f];
  long long n = (long long)F * tab.P;
  long long blocks = (n * n + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(visibility_kernel, dim3((unsigned)blocks), dim3(256), 0, s, tab, fc, vis);
  return hipGetLastError();
}

}  // namespace wam
