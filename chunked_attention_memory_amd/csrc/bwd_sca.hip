// Backward of sliding chunk attention, bf16 inputs, fp32 accumulation, gfx950
// MFMA.
//
// Forward (Gecko summary, paper.rainbus.top, "Method steps" (2)-(3)): for
// query i of chunk s, P_ij = softmax_j(q_i . k_j) over the keys of chunks s-1
// and s with j <= i, O_i = sum_j P_ij v_j, q = kappa_q z + nu_q,
// k = kappa_k z + nu_k. For L = sum(dO * O), with l_ij = q_i . k_j:
//   dL/dv_j    = sum_i P_ij dO_i
//   dS_ij      = dL/dl_ij = P_ij (dO_i . v_j - D_i),   D_i = dO_i . O_i
//   dL/dq_i    = sum_j dS_ij k_j = kappa_k * sum_j dS_ij z_j
//                (the nu_k part vanishes: sum_j dS_ij = 0)
//   dL/dk_j    = sum_i dS_ij q_i = kappa_q * sum_i dS_ij z_i + nu_q sum_i dS_ij
// As in the forward kernel, the logits are formed as q'_i . z_j with
// q' = q * kappa_k * log2(e) rounded to bf16 (a per-row shift by q_i . nu_k,
// which softmax ignores), so P = 2^(q'_i . z_j - lse2_i) with lse2_i the
// log2-sum-exp of the row's scaled logits.
//
// Kernels:
//  * prep: q' (bf16); dO in bf16 when it comes as float32.
//  * dq: one workgroup = 256 queries of one chunk (8 waves x 32), streaming
//    the key window in 64-key tiles twice (once with saved statistics). Per
//    32-key half and wave,
//      S^T = Z_keys q'^T, dP^T = V dO^T,
//    then (first pass) the row statistics lse2_i and D_i = sum_j P_ij dP_ij,
//    or (second pass) dS^T and U^T += Z_keys^T dS^T; dL/dq = kappa_k * U.
//  * dkdv: one workgroup = 32 keys per wave of one chunk, streaming the
//    queries that see them (the rest of their chunk, the next chunk) in
//    64-query tiles; per 32-query half and wave,
//      S = q' Z_keys^T, dP = dO V^T, dV^T += dO^T P, Y^T += Z_q^T dS
//    and dL/dk = kappa_q * Y + nu_q * colsum(dS) at the end: one kernel of 4
//    waves (one per SIMD: with dv = 256 the dV and dK accumulators take a
//    wave's whole register file), or as a build option dV (S, P, dV) and dK
//    (S, dP, dS, Y) as two kernels of 8 waves.
// Key (query) tiles go from HBM straight into LDS (buffer loads writing LDS),
// two stages; all operands come from LDS through lds_row / lds_tr.
#include <algorithm>

#include "bwd_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

constexpr int kT = 64;  // rows per staged tile

// Waves per workgroup of the dq kernel, and the dk dv layout at dv = 256:
// 0 one kernel for both accumulators, 4 waves of one key block (one wave per
// SIMD: the dV and dK accumulators together need its whole register file);
// 1 separate dV and dK kernels of 4 waves of GECKO_BWD_QB key blocks; 2
// separate kernels of 8 waves of one block (two waves per SIMD, so that one
// wave's exponentials overlap the other's MFMAs). Eight waves fit the
// registers only with the two 32-row halves of a tile processed in a loop
// rather than unrolled. With the XCD-aware workgroup order, 0 is the fastest
// at 128K tokens (5.9 ms against 6.3 ms for 2): it forms S and reads each
// query tile once for both products.
#ifndef GECKO_BWD_DQ_NW
#define GECKO_BWD_DQ_NW 8
#endif
#ifndef GECKO_BWD_KV256
#define GECKO_BWD_KV256 0
#endif
// Operand reads from LDS run GECKO_BWD_AHEAD MFMAs ahead of their use;
// GECKO_BWD_SCHED pins that interleave with scheduling group barriers.
#ifndef GECKO_BWD_SCHED
#define GECKO_BWD_SCHED 1
#endif
#ifndef GECKO_BWD_AHEAD
#define GECKO_BWD_AHEAD 2
#endif

// Pin `n` MFMAs each preceded by `per` LDS reads, after `ahead` leading
// reads (the chains below read their operands that far ahead).
template <int N, int PER, int AH, int MF>
__device__ __forceinline__ void sched_chain() {
#if GECKO_BWD_SCHED
  __builtin_amdgcn_sched_group_barrier(0x100, PER * AH, 0);
#pragma unroll
  for (int i = 0; i < N - AH; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, MF * AH, 0);
#endif
}

// 32-row blocks per wave: queries in dq, keys in the split dk dv kernels
#ifndef GECKO_BWD_DQ_QB
#define GECKO_BWD_DQ_QB 1
#endif
#ifndef GECKO_BWD_QB
#define GECKO_BWD_QB 1
#endif

// ---------------------------------------------------------------- prep
struct PrepArgs {
  const uint16_t* z;
  const float* kq; const float* nq; const float* kk;
  uint16_t* qp;
  int64_t rows, n;
  int H;
};

// q' = (kappa_q z + nu_q) kappa_k log2(e) in bf16, the forward kernel's
// expression; 16 threads per row, features 8 t + [0, 8)
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(PrepArgs a) {
  static_assert(D == 128, "one 16-byte chunk of features per thread");
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  if (row >= a.rows) return;
  const int h = (int)((row / a.n) % a.H);
  const int f0 = 8 * t;
  const float* kq = a.kq + h * D + f0;
  const float* nq = a.nq + h * D + f0;
  const float* kk = a.kk + h * D + f0;
  float x[8];
  unpack8(ld16(a.z + row * D + f0), x);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (kq[i] * x[i] + nq[i]) * (kk[i] * kLog2e);
  st16(a.qp + row * D + f0, pack8(x));
}

// dO (float32) rounded to bf16, the operand precision of every product
__global__ __launch_bounds__(256) void bwd_dout_bf16_kernel(const float* __restrict__ d, uint16_t* __restrict__ o,
                                                            int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(d + 8 * i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(d + 8 * i + 4);
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    st16(o + 8 * i, pack8(x));
  }
}

// Workgroups are dealt to the 8 XCDs round-robin (block b to XCD b mod 8),
// and each XCD has its own L2. Logical block (b mod 8) per_xcd + b / 8 gives
// every XCD a contiguous run of (batch*head, chunk) pairs, so the tiles that
// read the same key window meet in one L2 instead of each XCD streaming the
// whole window from HBM.
#ifndef GECKO_BWD_XCD
#define GECKO_BWD_XCD 1
#endif
__device__ __forceinline__ uint32_t logical_block(uint32_t per_xcd) {
#if GECKO_BWD_XCD
  return (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
#else
  (void)per_xcd;
  return blockIdx.x;
#endif
}

inline unsigned xcd_grid(int64_t nblocks, int64_t* per_xcd) {
#if GECKO_BWD_XCD
  *per_xcd = (nblocks + 7) / 8;
  return (unsigned)(8 * *per_xcd);
#else
  *per_xcd = nblocks;
  return (unsigned)nblocks;
#endif
}

// ---------------------------------------------------------------- saved statistics
// From the forward's per-query offset m and sum l of its bf16 weights
// 2^(s - m) (log2 units, as the PV product used them) and its float32
// attention output O: the attention kernels' dO operand dO' = bf16(dO / l)
// and, per query, (m, D') with D' = dO' . O. Then
//   2^(s_ij - m_i) (dO'_i . v_j - D'_i) = P_ij (dP_ij - D_i)
// for the forward's own weights P_ij = bf16(2^(s_ij - m_i)) / l_i (up to the
// bf16 rounding of dO / l), and sum_j P_ij dP_ij = D_i holds to float32
// rounding because O is the forward's product of those same weights: the
// kernels use (m, D') where they would use their own (lse2, D).
struct SavedArgs {
  const void* dout;     // bf16 or float32 [rows][dv]
  const float* o;       // [rows][dv]
  const float* stats;   // [rows][2]: (m, l)
  uint16_t* dos;        // [rows][dv]
  float* ld;            // [rows][2]: (m, D')
  int64_t rows;
  int out_f32;
};

// DV / 8 threads per row, 8 values each; a row's threads are consecutive
// lanes of one wave (DV / 8 divides 64)
template <int DV>
__global__ __launch_bounds__(256) void bwd_saved_prep_kernel(SavedArgs a) {
  constexpr int TPR = DV / 8, RPB = 256 / TPR;
  static_assert(64 % TPR == 0, "a row's threads within one wave");
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  // rows past the end repeat the last row (every lane takes part in the
  // shuffles) and store nothing
  const int64_t r = row < a.rows ? row : a.rows - 1;
  const float2 st = *reinterpret_cast<const float2*>(a.stats + 2 * r);
  const float inv = 1.f / st.y;
  float x[8];
  if (a.out_f32) {
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.dout) + r * DV + 8 * t);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = x0[i];
      x[4 + i] = x1[i];
    }
  } else {
    unpack8(ld16(static_cast<const uint16_t*>(a.dout) + r * DV + 8 * t), x);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] *= inv;
  const u32x4 pk = pack8(x);
  unpack8(pk, x);  // the rounded values the products use
  const f32x4* orow = reinterpret_cast<const f32x4*>(a.o + r * DV + 8 * t);
  const f32x4 o0 = orow[0], o1 = orow[1];
  float dsum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) dsum += x[i] * o0[i] + x[4 + i] * o1[i];
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) dsum += __shfl_xor(dsum, off, 64);
  if (row < a.rows) {
    st16(a.dos + row * DV + 8 * t, pk);
    if (t == 0) *reinterpret_cast<float2*>(a.ld + 2 * row) = make_float2(st.x, dsum);
  }
}

// ---------------------------------------------------------------- dq
struct DqArgs {
  const uint16_t* qp;
  const uint16_t* z;
  const uint16_t* v;
  const uint16_t* dO;
  const float* kk;
  float* ld;   // written: (lse2, D) per query, for the dk dv kernels (read instead when saved)
  float* dq;
  int64_t n;
  int c, nchunks, qtiles, H, prev;
  int saved;   // (m, D') of the forward's statistics already in ld: no statistics pass
  uint32_t nblocks, per_xcd;
};

// Running softmax statistics of one lane's keys for its query: max m (log2
// units), sum l of 2^(s - m) and sum a of 2^(s - m) dP.
struct RowStats {
  float m, l, a;
};

// NW waves, QB 32-query blocks per wave: each K / V operand read from LDS
// serves QB MFMAs, and a workgroup of 32 NW QB queries reuses every staged
// key tile that many times (the staging, not the MFMAs, bounds a workgroup of
// fewer queries).
template <int D, int DV, int NW, int QB>
struct DqLoop {
  static constexpr int THREADS = 64 * NW;
  static constexpr int ZB = kT * D * 2, VB = kT * DV * 2;
  static constexpr int STAGE = ZB + VB;
  static constexpr int ZL = ZB / 16 / THREADS, VL = VB / 16 / THREADS;
  static constexpr int KS = D / 16, VS = DV / 16, NF = D / 32;
  // LDS stages: three where they fit (tile k + 2 loads while tile k is
  // computed), else two
  static constexpr int NS = 3 * STAGE <= 160 * 1024 ? 3 : 2;
  static constexpr int LOADS = ZL + VL;  // staging loads per lane and tile
  const uint16_t* zbh;
  const uint16_t* vbh;
  char* sb[3];
  int n, kbeg, ntiles, wave_first, wave_last, w, lane, g, lq;
  int myq[QB];
  float lse2[QB], dd[QB];
  uint32_t zoff[ZL], voff[VL];
  u32x4 qf[QB][KS], df[QB][VS];
  RowReader<D> zr;
  RowReader<DV> vr;
  TrReader<D> zt;

  __device__ __forceinline__ void stage(int kt, int slot) const {
    const int row0 = kbeg + kt * kT;
    stage_rows(zbh, row0, n, D, sb[slot], NW, w, zoff, ZL);
    stage_rows(vbh, row0, n, DV, sb[slot] + ZB, NW, w, voff, VL);
  }

  // S^T and dP^T of one 32-key half of the tile in `slot`, every query block
  __device__ __forceinline__ void scores(int mb, int slot, f32x16 (&sc)[QB], f32x16 (&dp)[QB]) const {
    const char* Zs = sb[slot];
    const char* Vs = sb[slot] + ZB;
    const int row0 = 32 * mb;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      sc[qb] = f32x16{};
      dp[qb] = f32x16{};
    }
    // one stream of KS K-row and VS V-row operands, read AH ahead
    constexpr int NI = KS + VS, AH = GECKO_BWD_AHEAD;
    u32x4 op[AH + 1];
#pragma unroll
    for (int i = 0; i < AH; ++i) op[i] = i < KS ? zr.read(Zs, row0, i) : vr.read(Vs, row0, i - KS);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = i + AH;
      if (j < NI) op[j % (AH + 1)] = j < KS ? zr.read(Zs, row0, j) : vr.read(Vs, row0, j - KS);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (i < KS)
          sc[qb] = mfma_bf16(op[i % (AH + 1)], qf[qb][i], sc[qb]);
        else
          dp[qb] = mfma_bf16(op[i % (AH + 1)], df[qb][i - KS], dp[qb]);
      }
    }
    sched_chain<NI, 1, AH, QB>();
  }

  // whether every key of the half at kb is visible to every query of the
  // wave (its last key at or before the wave's first query): no mask
  __device__ __forceinline__ bool all_visible(int kb) const { return kb + 31 <= wave_first; }

  // statistics pass: fold this half's visible keys into (m, l, a). Without
  // kMax the offset is fixed at 0 (2^s summed directly: bf16 and fp32 share
  // the exponent range, so only the final sums need checking); with kMax it
  // follows the running maximum.
  template <bool kMax>
  __device__ __forceinline__ void stats_half(int kt, int mb, int slot, RowStats (&st)[QB]) const {
    f32x16 sc[QB], dp[QB];
    scores(mb, slot, sc, dp);
    const int kb = kbeg + kt * kT + 32 * mb;
    const bool full = all_visible(kb);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float e[16];
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = sc[qb][r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + (r & 7) + 8 * g + 16 * (r >> 3);
          e[r] = key <= myq[qb] ? sc[qb][r] : kNegInf;
        }
      }
      if constexpr (kMax) {
        float mx = e[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, e[r]);
        if (mx > st[qb].m) {  // rescale to the new maximum (a first finite maximum scales 0 by 0)
          const float f = st[qb].m == kNegInf ? 0.f : exp2_fast(st[qb].m - mx);
          st[qb].l *= f;
          st[qb].a *= f;
          st[qb].m = mx;
        }
        // a lane half with no visible key yet keeps m = -inf: offset 0 (its
        // exponentials are all 0), not -inf - (-inf)
        const float ms = st[qb].m == kNegInf ? 0.f : st[qb].m;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] -= ms;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = exp2_fast(e[r]);
        st[qb].l += x;
        st[qb].a += x * dp[qb][r];
      }
    }
  }

  // gradient pass: dS and U^T += Z^T dS^T for one half; sig gathers the row
  // sums of the bf16 dS that the products use
  __device__ __forceinline__ void grad_half(int kt, int mb, int slot, f32x16 (&U)[QB][NF], float (&sig)[QB]) const {
    f32x16 sc[QB], dp[QB];
    scores(mb, slot, sc, dp);
    const char* Zs = sb[slot];
    const int kb = kbeg + kt * kT + 32 * mb;
    const bool full = all_visible(kb);
    u32x4 d0[QB], d1[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float ds[16];
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = exp2_fast(sc[qb][r] - lse2[qb]) * (dp[qb][r] - dd[qb]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + (r & 7) + 8 * g + 16 * (r >> 3);
          const float p = key <= myq[qb] ? exp2_fast(sc[qb][r] - lse2[qb]) : 0.f;
          ds[r] = p * (dp[qb][r] - dd[qb]);
        }
      }
      d0[qb] = pack8(ds);
      d1[qb] = pack8(ds + 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) sig[qb] = sum2_bf16(d0[qb][i], sum2_bf16(d1[qb][i], sig[qb]));
    }
    // operand i = (fb, k-half) of Z^T, read AH ahead
    constexpr int NI = 2 * NF, AH = GECKO_BWD_AHEAD;
    u32x4 op[AH + 1];
#pragma unroll
    for (int i = 0; i < AH; ++i) op[i] = zt.read(Zs, 32 * mb + 16 * (i & 1), i >> 1);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = i + AH;
      if (j < NI) op[j % (AH + 1)] = zt.read(Zs, 32 * mb + 16 * (j & 1), j >> 1);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        U[qb][i >> 1] = mfma_bf16(op[i % (AH + 1)], (i & 1) ? d1[qb] : d0[qb], U[qb][i >> 1]);
    }
    sched_chain<NI, 2, AH, QB>();
  }

  // Tile kt in stage SLOT: stage tile kt + NS - 1 into the stage tile kt - 1
  // used (every wave is past it), compute, wait for this wave's share of
  // tile kt + 1 (tile kt + 2's loads may stay in flight) and end at the barrier.
  // kPass: 0 statistics with a fixed offset, 1 statistics with the running
  // maximum, 2 gradients
  template <int SLOT, int kPass>
  __device__ __forceinline__ void tile(int kt, RowStats (&st)[QB], f32x16 (&U)[QB][NF], float (&sig)[QB]) const {
    const bool ahead = kt + NS - 1 < ntiles;
    if (ahead) stage(kt + NS - 1, (SLOT + NS - 1) % NS);
#pragma unroll 1
    for (int mb = 0; mb < 2; ++mb) {
      if (kbeg + kt * kT + 32 * mb <= wave_last) {
        if constexpr (kPass < 2)
          stats_half<kPass == 1>(kt, mb, SLOT, st);
        else
          grad_half(kt, mb, SLOT, U, sig);
      }
    }
    if (NS == 3 && ahead)
      wait_vmem_leave<LOADS>();
    else
      wait_vmem();
    barrier_lds();
  }

  template <int kPass>
  __device__ __forceinline__ void pass(RowStats (&st)[QB], f32x16 (&U)[QB][NF], float (&sig)[QB]) const {
    stage(0, 0);
    if (NS == 3 && ntiles > 1) {
      stage(1, 1);
      wait_vmem_leave<LOADS>();
    } else {
      wait_vmem();
    }
    barrier_lds();
    for (int kt = 0; kt < ntiles; kt += NS) {
      tile<0, kPass>(kt, st, U, sig);
      if (kt + 1 < ntiles) tile<1, kPass>(kt + 1, st, U, sig);
      if (NS == 3 && kt + 2 < ntiles) tile<2 % NS, kPass>(kt + 2, st, U, sig);
    }
  }
};

// Two passes over the key window. The first gathers, per query, the
// log2-sum-exp of its scaled logits and D_i = sum_j P_ij dP_ij with the same
// fp32 P and dP that the second pass uses, so that sum_j dS_ij = 0 holds to
// fp32 rounding. (D_i from the bf16 forward output, or a normaliser from the
// forward's bf16-rounded weights, would be off by 2^-9 of dP; under a peaked
// softmax, where dS_ii = P_ii (dP_ii - D_i) is a small difference of large
// terms, that error exceeds dS itself.) The second pass forms dS and U.
template <int D, int DV, int NW, int QB>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dq_kernel(DqArgs a) {
  using L = DqLoop<D, DV, NW, QB>;
  constexpr int NF = L::NF;
  constexpr int kBlk = 32 * NW * QB;
  __shared__ __attribute__((aligned(16))) char S0[L::STAGE];
  __shared__ __attribute__((aligned(16))) char S1[L::STAGE];
  __shared__ __attribute__((aligned(16))) char S2[L::NS == 3 ? L::STAGE : 16];
  // within a chunk the last query tiles have the longest key windows: they
  // start first, so the workgroups left at the end of the grid are short
  const uint32_t lb = logical_block(a.per_xcd);
  if (lb >= a.nblocks) return;
  const int qt = a.qtiles - 1 - (int)(lb % (unsigned)a.qtiles);
  const int rest = (int)(lb / (unsigned)a.qtiles);
  const int s = rest % a.nchunks;
  const int bh = rest / a.nchunks;
  const int n = (int)a.n, c = a.c;
  const int q0 = s * c + qt * kBlk;
  const int cend = min((s + 1) * c, n);
  if (q0 >= cend) return;
  const int qend = min(q0 + kBlk, cend);
  const int h = bh % a.H;

  L l;
  const int tid = threadIdx.x;
  l.lane = tid & 63;
  l.g = l.lane >> 5;
  l.lq = l.lane & 31;
  l.w = __builtin_amdgcn_readfirstlane(tid >> 6);
  l.n = n;
  const int wq0 = q0 + 32 * QB * l.w;
  l.wave_first = wq0;
  l.wave_last = wq0 < qend ? min(wq0 + 32 * QB, qend) - 1 : -1;
  const size_t base = (size_t)bh * (size_t)n;
  l.zbh = a.z + base * D;
  l.vbh = a.v + base * DV;
  l.sb[0] = S0;
  l.sb[1] = S1;
  l.sb[2] = S2;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l.myq[qb] = wq0 + 32 * qb + l.lq;
    const size_t qrow = base + (size_t)min(l.myq[qb], qend - 1);
#pragma unroll
    for (int ks = 0; ks < L::KS; ++ks) l.qf[qb][ks] = ld16(a.qp + qrow * D + 16 * ks + 8 * l.g);
#pragma unroll
    for (int ks = 0; ks < L::VS; ++ks) l.df[qb][ks] = ld16(a.dO + qrow * DV + 16 * ks + 8 * l.g);
  }
  l.kbeg = (a.prev && s > 0) ? (s - 1) * c : s * c;
  l.ntiles = (qend - l.kbeg + kT - 1) / kT;
  stage_offsets<D>(l.zoff, NW, l.w, l.lane);
  stage_offsets<DV>(l.voff, NW, l.w, l.lane);
  l.zr.init(l.lane);
  l.vr.init(l.lane);
  l.zt.init(l.lane);

  f32x16 U[QB][NF];
  RowStats st[QB];
  float sig[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    st[qb] = RowStats{0.f, 0.f, 0.f};
    sig[qb] = 0.f;
#pragma unroll
    for (int fb = 0; fb < NF; ++fb) U[qb][fb] = f32x16{};
  }
  if (a.saved) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float2 v = *reinterpret_cast<const float2*>(a.ld + 2 * (base + (size_t)min(l.myq[qb], qend - 1)));
      l.lse2[qb] = v.x;
      l.dd[qb] = v.y;
    }
  } else {
    // First without an offset; if a valid query's sum lies outside
    // [2^-60, 2^63] (some 2^s overflowed, or every term is tiny), the workgroup
    // redoes the statistics with the running maximum.
    l.template pass<0>(st, U, sig);
    bool redo = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = other_half_sum(st[qb].l);
      redo = redo || (l.myq[qb] < qend && !(lt >= 0x1p-60f && lt <= 0x1p63f));
    }
    if (__syncthreads_or(redo)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) st[qb] = RowStats{kNegInf, 0.f, 0.f};
      l.template pass<1>(st, U, sig);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // merge the two lane halves (each saw half of every 32-key block); each
      // swap result holds this lane's value and the other half's, in the same
      // order for the three, and the merge is symmetric in the two
      const auto sm = __builtin_amdgcn_permlane32_swap(__float_as_uint(st[qb].m), __float_as_uint(st[qb].m), false, false);
      const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(st[qb].l), __float_as_uint(st[qb].l), false, false);
      const auto sa = __builtin_amdgcn_permlane32_swap(__float_as_uint(st[qb].a), __float_as_uint(st[qb].a), false, false);
      const float m0 = __uint_as_float(sm[0]), m1 = __uint_as_float(sm[1]);
      const float l0 = __uint_as_float(sl[0]), l1 = __uint_as_float(sl[1]);
      const float a0 = __uint_as_float(sa[0]), a1 = __uint_as_float(sa[1]);
      const float m = fmaxf(m0, m1);
      const float f0 = m0 == kNegInf ? 0.f : exp2_fast(m0 - m);
      const float f1 = m1 == kNegInf ? 0.f : exp2_fast(m1 - m);
      const float lt = l0 * f0 + l1 * f1, at = a0 * f0 + a1 * f1;
      const bool any = m != kNegInf && lt > 0.f;
      l.lse2[qb] = any ? m + log2f(lt) : 0.f;
      l.dd[qb] = any ? at / lt : 0.f;
      if (l.g == 0 && l.myq[qb] < qend)
        *reinterpret_cast<float2*>(a.ld + 2 * (base + (size_t)l.myq[qb])) = make_float2(l.lse2[qb], l.dd[qb]);
    }
  }
  // after a statistics pass every wave is past its last barrier: the stages are free
  l.template pass<2>(st, U, sig);

  // dq = kappa_k * sum_j dS_ij z_j relies on sum_j dS_ij = 0; the bf16 dS
  // that the products use sum to a rounding residue sigma, which a component
  // shared by all keys would multiply. Moving the residue onto the diagonal
  // key (U - sigma z_i) makes the sum exactly zero, so shared components
  // cancel as they do in exact arithmetic.
  const float* kk = a.kk + h * D;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float sg = other_half_sum(sig[qb]);
    if (l.myq[qb] >= qend) continue;
    const uint16_t* zq = a.z + (base + (size_t)l.myq[qb]) * D;
    // register r of block fb holds feature 32 fb + 16 (r >> 3) + 8 g + (r & 7)
    float* dst = a.dq + (base + (size_t)l.myq[qb]) * D;
#pragma unroll
    for (int fb = 0; fb < NF; ++fb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int f = 32 * fb + 16 * hh + 8 * l.g;
        float zf[8];
        unpack8(ld16(zq + f), zf);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 k4 = *reinterpret_cast<const f32x4*>(kk + f + 4 * q);
          const int r = 8 * hh + 4 * q;
          f32x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = k4[i] * (U[qb][fb][r + i] - sg * zf[4 * q + i]);
          *reinterpret_cast<f32x4*>(dst + f + 4 * q) = o;
        }
      }
  }
}

// ---------------------------------------------------------------- dk, dv
struct KvArgs {
  const uint16_t* qp;
  const uint16_t* z;
  const uint16_t* v;
  const uint16_t* dO;
  const float* ld;
  const float* kq;
  const float* nq;
  float* dk;
  float* dv;
  int64_t n;
  int c, nchunks, ktiles, H, prev, accum;
  uint32_t nblocks, per_xcd;
};

// NW waves, KB 32-key blocks per wave. MODE 0: dK and dV; 1: dV only (P
// alone, no dP); 2: dK only.
template <int D, int DV, int NW, int KB, int MODE>
struct KvLoop {
  static constexpr bool kDV = MODE != 2, kDK = MODE != 1;
  static constexpr int THREADS = 64 * NW;
  static constexpr int QB_ = kT * D * 2, VB = kT * DV * 2, LB = 1024;
  // q' tile, z tile (dK only), dO tile, (lse2, D) of 128 rows
  static constexpr int ZOFF = QB_, DOFF = kDK ? 2 * QB_ : QB_, LOFF = DOFF + VB;
  static constexpr int STAGE = LOFF + LB;
  static constexpr int QL = QB_ / 16 / THREADS, VL = VB / 16 / THREADS;
  static constexpr int KS = D / 16, VS = DV / 16, NF = D / 32, NMV = DV / 32;
  static constexpr int NY = kDK ? NF : 1, NV = kDV ? NMV : 1;
  static constexpr int NS = 3 * STAGE <= 160 * 1024 ? 3 : 2;
  static constexpr int LOADS = QL * (kDK ? 2 : 1) + VL;  // staging loads per lane and tile (wave 0: one more)
  const uint16_t* qbh;
  const uint16_t* zbh;
  const uint16_t* dbh;
  const uint16_t* lbh;  // (lse2, D) pairs as 4 bf16-sized units per row
  char* sb[3];
  int n, ta, nb0, ntiles, j0, wj0, has, w, lane, g, lq;
  int own_end, next_end;  // ends of the two query ranges (a tile may reach past them)
  int myk[KB];
  uint32_t qoff[QL], doff[VL];
  u32x4 kf[KB][KS], vf[KB][kDK ? VS : 1];
  RowReader<D> qr;
  RowReader<DV> dr;
  TrReader<DV> dt;
  TrReader<D> zt;

  __device__ __forceinline__ int qbase(int kt) const { return kt < ta ? j0 + kt * kT : nb0 + (kt - ta) * kT; }

  __device__ __forceinline__ void stage(int kt, int slot) const {
    const int row0 = qbase(kt);
    stage_rows(qbh, row0, n, D, sb[slot], NW, w, qoff, QL);
    if constexpr (kDK) stage_rows(zbh, row0, n, D, sb[slot] + ZOFF, NW, w, qoff, QL);
    stage_rows(dbh, row0, n, DV, sb[slot] + DOFF, NW, w, doff, VL);
    if (w == 0) {
      const uint32_t lo[1] = {(uint32_t)lane * 16u};
      stage_rows(lbh, row0, n, 4, sb[slot] + LOFF, 1, 0, lo, 1);
    }
  }

  // one 32-query half of the tile in `slot`, every key block
  __device__ __forceinline__ void half(int kt, int mq, int slot, f32x16 (&Y)[KB][NY], f32x16 (&dV)[KB][NV],
                                       float (&sig)[KB]) const {
    const char* Qs = sb[slot];
    const char* Zq = sb[slot] + ZOFF;
    const char* Ds = sb[slot] + DOFF;
    const float* Ls = reinterpret_cast<const float*>(sb[slot] + LOFF);
    const bool own = kt < ta;
    const int qb = qbase(kt) + 32 * mq;
    const int row0 = 32 * mq;
    f32x16 sc[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sc[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
    {
      // one stream of KS q'-row and (dK) VS dO-row operands, read AH ahead
      constexpr int NI = KS + (kDK ? VS : 0), AH = GECKO_BWD_AHEAD;
      u32x4 op[AH + 1];
#pragma unroll
      for (int i = 0; i < AH; ++i) op[i] = i < KS ? qr.read(Qs, row0, i) : dr.read(Ds, row0, i - KS);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = i + AH;
        if (j < NI) op[j % (AH + 1)] = j < KS ? qr.read(Qs, row0, j) : dr.read(Ds, row0, j - KS);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if (i < KS)
            sc[kb] = mfma_bf16(op[i % (AH + 1)], kf[kb][i], sc[kb]);
          else if constexpr (kDK)
            dp[kb] = mfma_bf16(op[i % (AH + 1)], vf[kb][i - KS], dp[kb]);
        }
      }
      sched_chain<NI, 1, AH, KB>();
    }
    // no mask when every query of the half sees every key of the wave:
    // the half lies inside its range and (own chunk) after the wave's keys
    const bool full = own ? (qb >= wj0 + 32 * KB - 1 && qb + 31 < own_end) : qb + 31 < next_end;
    u32x4 pk[KB][2], dk[KB][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      // queries 32 mq + 16 hh + 8 g + [0, 8): (lse2, D) pairs, 64 bytes
      const float* lp = Ls + 2 * (32 * mq + 16 * hh + 8 * g);
      float2 st[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) st[j] = *reinterpret_cast<const float2*>(lp + 2 * j);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float p[8], ds[8];
        if (full) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            p[j] = exp2_fast(sc[kb][8 * hh + j] - st[j].x);
            ds[j] = p[j] * (dp[kb][8 * hh + j] - st[j].y);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = 8 * hh + j;
            const int q = qb + 16 * hh + 8 * g + j;
            const bool vis = own ? (q < own_end && q >= myk[kb]) : q < next_end;
            p[j] = vis ? exp2_fast(sc[kb][r] - st[j].x) : 0.f;
            ds[j] = p[j] * (dp[kb][r] - st[j].y);
          }
        }
        pk[kb][hh] = pack8(p);
        dk[kb][hh] = pack8(ds);
      }
    }
    if constexpr (kDV) {
      // operand i = (mv, k-half) of dO^T, read AH ahead
      constexpr int NI = 2 * NMV, AH = GECKO_BWD_AHEAD;
      u32x4 op[AH + 1];
#pragma unroll
      for (int i = 0; i < AH; ++i) op[i] = dt.read(Ds, 32 * mq + 16 * (i & 1), i >> 1);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = i + AH;
        if (j < NI) op[j % (AH + 1)] = dt.read(Ds, 32 * mq + 16 * (j & 1), j >> 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) dV[kb][i >> 1] = mfma_bf16(op[i % (AH + 1)], pk[kb][i & 1], dV[kb][i >> 1]);
      }
      sched_chain<NI, 2, AH, KB>();
    }
    if constexpr (kDK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sig[kb] = sum2_bf16(dk[kb][0][i], sum2_bf16(dk[kb][1][i], sig[kb]));
      // operand i = (fb, k-half) of Z_q^T, read AH ahead
      constexpr int NI = 2 * NF, AH = GECKO_BWD_AHEAD;
      u32x4 op[AH + 1];
#pragma unroll
      for (int i = 0; i < AH; ++i) op[i] = zt.read(Zq, 32 * mq + 16 * (i & 1), i >> 1);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = i + AH;
        if (j < NI) op[j % (AH + 1)] = zt.read(Zq, 32 * mq + 16 * (j & 1), j >> 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) Y[kb][i >> 1] = mfma_bf16(op[i % (AH + 1)], dk[kb][i & 1], Y[kb][i >> 1]);
      }
      sched_chain<NI, 2, AH, KB>();
    }
  }

  // wait until only the newest tile's loads may be in flight
  __device__ __forceinline__ void wait_all_but_one_tile() const {
    if (w == 0)
      wait_vmem_leave<LOADS + 1>();
    else
      wait_vmem_leave<LOADS>();
  }

  template <int SLOT>
  __device__ __forceinline__ void tile(int kt, f32x16 (&Y)[KB][NY], f32x16 (&dV)[KB][NV], float (&sig)[KB]) const {
    const bool ahead = kt + NS - 1 < ntiles;
    if (ahead) stage(kt + NS - 1, (SLOT + NS - 1) % NS);
    const int qb0 = qbase(kt);
#pragma unroll 1
    for (int mq = 0; mq < 2; ++mq) {
      const int qb = qb0 + 32 * mq;
      // skip halves past the sequence, or (own chunk) wholly before the wave's keys
      if (has && qb < n && !(kt < ta && qb + 31 < wj0)) half(kt, mq, SLOT, Y, dV, sig);
    }
    if (NS == 3 && ahead)
      wait_all_but_one_tile();
    else
      wait_vmem();
    barrier_lds();
  }

  __device__ __forceinline__ void run(f32x16 (&Y)[KB][NY], f32x16 (&dV)[KB][NV], float (&sig)[KB]) const {
    stage(0, 0);
    if (NS == 3 && ntiles > 1) {
      stage(1, 1);
      wait_all_but_one_tile();
    } else {
      wait_vmem();
    }
    barrier_lds();
    for (int kt = 0; kt < ntiles; kt += NS) {
      tile<0>(kt, Y, dV, sig);
      if (kt + 1 < ntiles) tile<1>(kt + 1, Y, dV, sig);
      if (NS == 3 && kt + 2 < ntiles) tile<2 % NS>(kt + 2, Y, dV, sig);
    }
  }
};

template <int D, int DV, int NW, int KB, int MODE>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dkdv_kernel(KvArgs a) {
  using L = KvLoop<D, DV, NW, KB, MODE>;
  constexpr int NF = L::NF, NMV = L::NMV, NY = L::NY, NV = L::NV;
  constexpr int kBlk = 32 * NW * KB;
  __shared__ __attribute__((aligned(16))) char S0[L::STAGE];
  __shared__ __attribute__((aligned(16))) char S1[L::STAGE];
  __shared__ __attribute__((aligned(16))) char S2[L::NS == 3 ? L::STAGE : 16];
  // the first key tiles of a chunk have the most queries: they start first
  const uint32_t lb = logical_block(a.per_xcd);
  if (lb >= a.nblocks) return;
  const int kt_ = (int)(lb % (unsigned)a.ktiles);
  const int rest = (int)(lb / (unsigned)a.ktiles);
  const int s = rest % a.nchunks;
  const int bh = rest / a.nchunks;
  const int n = (int)a.n, c = a.c;
  const int j0 = s * c + kt_ * kBlk;
  const int cend = min((s + 1) * c, n);
  if (j0 >= cend) return;
  const int jend = min(j0 + kBlk, cend);
  const int h = bh % a.H;

  L l;
  const int tid = threadIdx.x;
  l.lane = tid & 63;
  l.g = l.lane >> 5;
  l.lq = l.lane & 31;
  l.w = __builtin_amdgcn_readfirstlane(tid >> 6);
  l.n = n;
  l.j0 = j0;
  l.wj0 = j0 + 32 * KB * l.w;
  l.has = l.wj0 < jend;
  const size_t base = (size_t)bh * (size_t)n;
  l.qbh = a.qp + base * D;
  l.zbh = a.z + base * D;
  l.dbh = a.dO + base * DV;
  l.lbh = reinterpret_cast<const uint16_t*>(a.ld + 2 * base);
  l.sb[0] = S0;
  l.sb[1] = S1;
  l.sb[2] = S2;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    l.myk[kb] = l.wj0 + 32 * kb + l.lq;
    const size_t krow = base + (size_t)min(l.myk[kb], jend - 1);
#pragma unroll
    for (int ks = 0; ks < L::KS; ++ks) l.kf[kb][ks] = ld16(a.z + krow * D + 16 * ks + 8 * l.g);
    if constexpr (L::kDK) {
#pragma unroll
      for (int ks = 0; ks < L::VS; ++ks) l.vf[kb][ks] = ld16(a.v + krow * DV + 16 * ks + 8 * l.g);
    }
  }
  // queries that see these keys: the rest of chunk s, then all of chunk s + 1
  l.ta = (cend - j0 + kT - 1) / kT;
  l.nb0 = (s + 1) * c;
  const int nbq = (a.prev && l.nb0 < n) ? min(l.nb0 + c, n) - l.nb0 : 0;
  l.own_end = cend;
  l.next_end = l.nb0 + nbq;
  l.ntiles = l.ta + (nbq + kT - 1) / kT;
  stage_offsets<D>(l.qoff, NW, l.w, l.lane);
  stage_offsets<DV>(l.doff, NW, l.w, l.lane);
  l.qr.init(l.lane);
  l.dr.init(l.lane);
  l.dt.init(l.lane);
  l.zt.init(l.lane);

  f32x16 Y[KB][NY], dV[KB][NV];
  float sig[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    sig[kb] = 0.f;
#pragma unroll
    for (int fb = 0; fb < NY; ++fb) Y[kb][fb] = f32x16{};
#pragma unroll
    for (int mv = 0; mv < NV; ++mv) dV[kb][mv] = f32x16{};
  }
  l.run(Y, dV, sig);

  const float* kq = a.kq + h * D;
  const float* nq = a.nq + h * D;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const float sg = other_half_sum(sig[kb]);
    const int myk = l.myk[kb];
    if (myk >= jend) continue;
    if constexpr (L::kDK) {
      float* dk = a.dk + (base + (size_t)myk) * D;
#pragma unroll
      for (int fb = 0; fb < NF; ++fb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int f = 32 * fb + 16 * hh + 8 * l.g;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const f32x4 k4 = *reinterpret_cast<const f32x4*>(kq + f + 4 * q);
            const f32x4 n4 = *reinterpret_cast<const f32x4*>(nq + f + 4 * q);
            const int r = 8 * hh + 4 * q;
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = k4[i] * Y[kb][fb][r + i] + n4[i] * sg;
            *reinterpret_cast<f32x4*>(dk + f + 4 * q) = o;
          }
        }
    }
    if constexpr (L::kDV) {
      float* dv = a.dv + (base + (size_t)myk) * DV;
#pragma unroll
      for (int mv = 0; mv < NMV; ++mv)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int col = 32 * mv + 16 * hh + 8 * l.g;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int r = 8 * hh + 4 * q;
            f32x4 o{dV[kb][mv][r], dV[kb][mv][r + 1], dV[kb][mv][r + 2], dV[kb][mv][r + 3]};
            f32x4* p = reinterpret_cast<f32x4*>(dv + col + 4 * q);
            if (a.accum) o += *p;
            *p = o;
          }
        }
    }
  }
}

const uint16_t* dout16(const BwdProblem& p, const BwdWorkspace& w) {
  return w.do16 ? w.do16 : static_cast<const uint16_t*>(p.dout);
}

// the attention kernels' dO operand: dO / l per query with saved statistics
const uint16_t* attn_dout(const BwdProblem& p, const BwdWorkspace& w) { return p.saved ? w.dos : dout16(p, w); }

}  // namespace

bool bwd_shape_built(int64_t d, int64_t dv) { return d == 128 && (dv == 256 || dv == 128); }

hipError_t launch_bwd_prep(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s) {
  PrepArgs a;
  a.z = static_cast<const uint16_t*>(p.f.z);
  a.kq = p.f.kappa_q; a.nq = p.f.nu_q; a.kk = p.f.kappa_k;
  a.qp = w.qp;
  a.rows = p.f.B * p.f.H * p.f.n;
  a.n = p.f.n; a.H = (int)p.f.H;
  hipLaunchKernelGGL((bwd_prep_kernel<128>), dim3((unsigned)((a.rows + 15) / 16)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dout16(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s) {
  const int64_t n8 = p.f.B * p.f.H * p.f.n * p.f.dv / 8;
  const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, 4096);
  hipLaunchKernelGGL(bwd_dout_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const float*>(p.dout), w.do16, n8);
  return hipGetLastError();
}

hipError_t launch_bwd_saved_prep(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s) {
  SavedArgs a;
  a.dout = p.dout;
  a.o = p.o_sca;
  a.stats = p.stats;
  a.dos = w.dos;
  a.ld = w.ld;
  a.rows = p.f.B * p.f.H * p.f.n;
  a.out_f32 = p.out_f32 ? 1 : 0;
  if (p.f.dv == 256) {
    hipLaunchKernelGGL((bwd_saved_prep_kernel<256>), dim3((unsigned)((a.rows + 7) / 8)), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_saved_prep_kernel<128>), dim3((unsigned)((a.rows + 15) / 16)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s) {
  constexpr int NW = GECKO_BWD_DQ_NW, QB = GECKO_BWD_DQ_QB;
  DqArgs a;
  a.qp = w.qp;
  a.z = static_cast<const uint16_t*>(p.f.z);
  a.v = static_cast<const uint16_t*>(p.f.v);
  a.dO = attn_dout(p, w);
  a.ld = w.ld; a.kk = p.f.kappa_k; a.dq = w.dq;
  a.saved = p.saved ? 1 : 0;
  a.n = p.f.n;
  const int64_t cc = p.f.c < p.f.n ? p.f.c : p.f.n;
  a.c = (int)cc; a.nchunks = (int)p.f.nchunks; a.H = (int)p.f.H; a.prev = (int)p.f.prev;
  a.qtiles = (int)((cc + 32 * NW * QB - 1) / (32 * NW * QB));
  const int64_t nblocks = p.f.B * p.f.H * p.f.nchunks * a.qtiles;
  int64_t per_xcd = 0;
  const dim3 grid(xcd_grid(nblocks, &per_xcd));
  a.nblocks = (uint32_t)nblocks;
  a.per_xcd = (uint32_t)per_xcd;
  if (p.f.dv == 256)
    hipLaunchKernelGGL((bwd_dq_kernel<128, 256, NW, QB>), grid, dim3(64 * NW), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<128, 128, NW, QB>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int DV, int NW, int KB, int MODE>
hipError_t launch_kv(KvArgs a, const BwdProblem& p, hipStream_t s) {
  const int64_t cc = p.f.c < p.f.n ? p.f.c : p.f.n;
  a.ktiles = (int)((cc + 32 * NW * KB - 1) / (32 * NW * KB));
  const int64_t nblocks = p.f.B * p.f.H * p.f.nchunks * a.ktiles;
  int64_t per_xcd = 0;
  const dim3 grid(xcd_grid(nblocks, &per_xcd));
  a.nblocks = (uint32_t)nblocks;
  a.per_xcd = (uint32_t)per_xcd;
  hipLaunchKernelGGL((bwd_dkdv_kernel<128, DV, NW, KB, MODE>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdProblem& p, const BwdWorkspace& w, bool accumulate_dv, hipStream_t s) {
  KvArgs a;
  a.qp = w.qp;
  a.z = static_cast<const uint16_t*>(p.f.z);
  a.v = static_cast<const uint16_t*>(p.f.v);
  a.dO = attn_dout(p, w);
  a.ld = w.ld; a.kq = p.f.kappa_q; a.nq = p.f.nu_q; a.dk = w.dk; a.dv = p.dv;
  a.n = p.f.n;
  const int64_t cc = p.f.c < p.f.n ? p.f.c : p.f.n;
  a.c = (int)cc; a.nchunks = (int)p.f.nchunks; a.H = (int)p.f.H; a.prev = (int)p.f.prev;
  a.accum = accumulate_dv ? 1 : 0;
  a.ktiles = 0;
  if (p.f.dv == 128) return launch_kv<128, 4, 1, 0>(a, p, s);
#if GECKO_BWD_KV256 == 0
  return launch_kv<256, 4, 1, 0>(a, p, s);
#else
  // dv = 256 as two kernels (GECKO_BWD_KV256 1 or 2, see above)
  constexpr int NW = GECKO_BWD_KV256 == 2 ? 8 : 4, KB = GECKO_BWD_KV256 == 2 ? 1 : GECKO_BWD_QB;
  hipError_t e = launch_kv<256, NW, KB, 1>(a, p, s);
  if (e != hipSuccess) return e;
  return launch_kv<256, NW, KB, 2>(a, p, s);
#endif
}

}  // namespace gecko
