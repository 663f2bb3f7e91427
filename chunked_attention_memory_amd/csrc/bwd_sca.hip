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
//  * dq: one workgroup = 128 queries of one chunk (4 waves x 32), streaming
//    the key window in 64-key tiles twice. Per 32-key half and wave,
//      S^T = Z_keys q'^T, dP^T = V dO^T,
//    then (first pass) the row statistics lse2_i and D_i = sum_j P_ij dP_ij,
//    or (second pass) dS^T and U^T += Z_keys^T dS^T; dL/dq = kappa_k * U.
//  * dkdv: one workgroup = 128 keys of one chunk (4 waves x 32), streaming
//    the queries that see them (the rest of their chunk, the next chunk) in
//    64-query tiles; per 32-query half and wave,
//      S = q' Z_keys^T, dP = dO V^T, dV^T += dO^T P, Y^T += Z_q^T dS
//    and dL/dk = kappa_q * Y + nu_q * colsum(dS) at the end.
// Key (query) tiles go from HBM straight into LDS (buffer loads writing LDS),
// two stages; all operands come from LDS through lds_row / lds_tr.
#include <algorithm>

#include "bwd_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

constexpr int kNW = 4;  // one wave per SIMD: the accumulators need more than half the register file
constexpr int kThreads = 64 * kNW;
constexpr int kBlk = 32 * kNW;  // queries (dq) or keys (dkdv) per workgroup
constexpr int kT = 64;          // rows per staged tile

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

// ---------------------------------------------------------------- dq
struct DqArgs {
  const uint16_t* qp;
  const uint16_t* z;
  const uint16_t* v;
  const uint16_t* dO;
  const float* kk;
  float* ld;   // written: (lse2, D) per query, for the dk dv kernel
  float* dq;
  int64_t n;
  int c, nchunks, qtiles, H, prev;
};

// Running softmax statistics of one lane's keys for its query: max m (log2
// units), sum l of 2^(s - m) and sum a of 2^(s - m) dP.
struct RowStats {
  float m, l, a;
};

template <int D, int DV>
struct DqLoop {
  static constexpr int ZB = kT * D * 2, VB = kT * DV * 2;
  static constexpr int STAGE = ZB + VB;
  static constexpr int ZL = ZB / 16 / kThreads, VL = VB / 16 / kThreads;
  static constexpr int KS = D / 16, VS = DV / 16, NF = D / 32;
  const uint16_t* zbh;
  const uint16_t* vbh;
  char* sb[2];
  int n, kbeg, ntiles, myq, wave_last, w, lane, g, lq;
  float lse2, dd;
  uint32_t zoff[ZL], voff[VL];
  u32x4 qf[KS], df[VS];

  __device__ __forceinline__ void stage(int kt, int slot) const {
    const int row0 = kbeg + kt * kT;
    stage_rows(zbh, row0, n, D, sb[slot], kNW, w, zoff, ZL);
    stage_rows(vbh, row0, n, DV, sb[slot] + ZB, kNW, w, voff, VL);
  }

  // S^T and dP^T of one 32-key half of the tile in `slot`
  __device__ __forceinline__ void scores(int mb, int slot, f32x16& sc, f32x16& dp) const {
    const char* Zs = sb[slot];
    const char* Vs = sb[slot] + ZB;
    const int arow = 32 * mb + perm_row(lq);
    sc = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma_bf16(lds_row<D>(Zs, arow, 2 * ks + g), qf[ks], sc);
#pragma unroll
    for (int ks = 0; ks < VS; ++ks) dp = mfma_bf16(lds_row<DV>(Vs, arow, 2 * ks + g), df[ks], dp);
  }

  // statistics pass: fold this half's visible keys into (m, l, a)
  __device__ __forceinline__ void stats_half(int kt, int mb, int slot, RowStats& st) const {
    f32x16 sc, dp;
    scores(mb, slot, sc, dp);
    const int kb = kbeg + kt * kT + 32 * mb;
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + (r & 7) + 8 * g + 16 * (r >> 3);
      mx = fmaxf(mx, key <= myq ? sc[r] : kNegInf);
    }
    if (mx > st.m) {  // rescale to the new maximum (a first finite maximum scales 0 by 0)
      const float f = st.m == kNegInf ? 0.f : exp2_fast(st.m - mx);
      st.l *= f;
      st.a *= f;
      st.m = mx;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + (r & 7) + 8 * g + 16 * (r >> 3);
      const float e = key <= myq ? exp2_fast(sc[r] - st.m) : 0.f;
      st.l += e;
      st.a += e * dp[r];
    }
  }

  // gradient pass: dS and U^T += Z^T dS^T for one half
  __device__ __forceinline__ void grad_half(int kt, int mb, int slot, f32x16 (&U)[NF]) const {
    f32x16 sc, dp;
    scores(mb, slot, sc, dp);
    const char* Zs = sb[slot];
    const int kb = kbeg + kt * kT + 32 * mb;
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + (r & 7) + 8 * g + 16 * (r >> 3);
      const float p = key <= myq ? exp2_fast(sc[r] - lse2) : 0.f;
      ds[r] = p * (dp[r] - dd);
    }
    const u32x4 d0 = pack8(ds), d1 = pack8(ds + 8);
#pragma unroll
    for (int fb = 0; fb < NF; ++fb) {
      U[fb] = mfma_bf16(lds_tr<D>(Zs, 32 * mb, 32 * fb, lane), d0, U[fb]);
      U[fb] = mfma_bf16(lds_tr<D>(Zs, 32 * mb + 16, 32 * fb, lane), d1, U[fb]);
    }
  }

  template <int SLOT, bool kStats>
  __device__ __forceinline__ void tile(int kt, RowStats& st, f32x16 (&U)[NF]) const {
    if (kt + 1 < ntiles) stage(kt + 1, SLOT ^ 1);  // every wave is past tile kt - 1
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (kbeg + kt * kT + 32 * mb <= wave_last) {
        if constexpr (kStats)
          stats_half(kt, mb, SLOT, st);
        else
          grad_half(kt, mb, SLOT, U);
      }
    }
    wait_vmem();
    barrier_lds();
  }

  template <bool kStats>
  __device__ __forceinline__ void pass(RowStats& st, f32x16 (&U)[NF]) const {
    stage(0, 0);
    wait_vmem();
    barrier_lds();
    for (int kt = 0; kt < ntiles; kt += 2) {
      tile<0, kStats>(kt, st, U);
      if (kt + 1 < ntiles) tile<1, kStats>(kt + 1, st, U);
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
template <int D, int DV>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(DqArgs a) {
  using L = DqLoop<D, DV>;
  constexpr int NF = L::NF;
  __shared__ __attribute__((aligned(16))) char S0[L::STAGE];
  __shared__ __attribute__((aligned(16))) char S1[L::STAGE];
  const int qt = (int)(blockIdx.x % (unsigned)a.qtiles);
  const int rest = (int)(blockIdx.x / (unsigned)a.qtiles);
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
  const int wq0 = q0 + 32 * l.w;
  l.myq = wq0 + l.lq;
  l.wave_last = wq0 < qend ? min(wq0 + 32, qend) - 1 : -1;
  const size_t base = (size_t)bh * (size_t)n;
  l.zbh = a.z + base * D;
  l.vbh = a.v + base * DV;
  l.sb[0] = S0;
  l.sb[1] = S1;
  const size_t qrow = base + (size_t)min(l.myq, qend - 1);
#pragma unroll
  for (int ks = 0; ks < L::KS; ++ks) l.qf[ks] = ld16(a.qp + qrow * D + 16 * ks + 8 * l.g);
#pragma unroll
  for (int ks = 0; ks < L::VS; ++ks) l.df[ks] = ld16(a.dO + qrow * DV + 16 * ks + 8 * l.g);
  l.kbeg = (a.prev && s > 0) ? (s - 1) * c : s * c;
  l.ntiles = (qend - l.kbeg + kT - 1) / kT;
  stage_offsets<D>(l.zoff, kNW, l.w, l.lane);
  stage_offsets<DV>(l.voff, kNW, l.w, l.lane);

  f32x16 U[NF];
#pragma unroll
  for (int fb = 0; fb < NF; ++fb) U[fb] = f32x16{};
  RowStats st{kNegInf, 0.f, 0.f};
  l.template pass<true>(st, U);
  {
    // merge the two lane halves (each saw half of every 32-key block)
    const auto sm = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.m), __float_as_uint(st.m), false, false);
    const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.l), __float_as_uint(st.l), false, false);
    const auto sa = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.a), __float_as_uint(st.a), false, false);
    // each swap result holds this lane's value and the other half's, in the
    // same order for the three; the merge is symmetric in the two
    const float m0 = __uint_as_float(sm[0]), m1 = __uint_as_float(sm[1]);
    const float l0 = __uint_as_float(sl[0]), l1 = __uint_as_float(sl[1]);
    const float a0 = __uint_as_float(sa[0]), a1 = __uint_as_float(sa[1]);
    const float m = fmaxf(m0, m1);
    const float f0 = m0 == kNegInf ? 0.f : exp2_fast(m0 - m);
    const float f1 = m1 == kNegInf ? 0.f : exp2_fast(m1 - m);
    const float lt = l0 * f0 + l1 * f1, at = a0 * f0 + a1 * f1;
    const bool any = m != kNegInf && lt > 0.f;
    l.lse2 = any ? m + log2f(lt) : 0.f;
    l.dd = any ? at / lt : 0.f;
  }
  if (l.g == 0 && l.myq < qend)
    *reinterpret_cast<float2*>(a.ld + 2 * (base + (size_t)l.myq)) = make_float2(l.lse2, l.dd);
  // every wave is past the statistics pass's last barrier: its stages are free
  l.template pass<false>(st, U);

  if (l.myq < qend) {
    // register r of block fb holds feature 32 fb + 16 (r >> 3) + 8 g + (r & 7)
    const float* kk = a.kk + h * D;
    float* dst = a.dq + (base + (size_t)l.myq) * D;
#pragma unroll
    for (int fb = 0; fb < NF; ++fb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int f = 32 * fb + 16 * hh + 8 * l.g;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 k4 = *reinterpret_cast<const f32x4*>(kk + f + 4 * q);
          const int r = 8 * hh + 4 * q;
          *reinterpret_cast<f32x4*>(dst + f + 4 * q) =
              f32x4{k4[0] * U[fb][r], k4[1] * U[fb][r + 1], k4[2] * U[fb][r + 2], k4[3] * U[fb][r + 3]};
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
};

template <int D, int DV>
struct KvLoop {
  static constexpr int QB_ = kT * D * 2, VB = kT * DV * 2, LB = 1024;
  static constexpr int STAGE = 2 * QB_ + VB + LB;  // q' tile, z tile, dO tile, (lse2, D) of 128 rows
  static constexpr int QL = QB_ / 16 / kThreads, VL = VB / 16 / kThreads;
  static constexpr int KS = D / 16, VS = DV / 16, NF = D / 32, NMV = DV / 32;
  const uint16_t* qbh;
  const uint16_t* zbh;
  const uint16_t* dbh;
  const uint16_t* lbh;  // (lse2, D) pairs as 4 bf16-sized units per row
  char* sb[2];
  int n, ta, nb0, ntiles, j0, myk, wj0, has, w, lane, g, lq;
  int own_end, next_end;  // ends of the two query ranges (a tile may reach past them)
  uint32_t qoff[QL], doff[VL];
  u32x4 kf[KS], vf[VS];

  __device__ __forceinline__ int qbase(int kt) const { return kt < ta ? j0 + kt * kT : nb0 + (kt - ta) * kT; }

  __device__ __forceinline__ void stage(int kt, int slot) const {
    const int row0 = qbase(kt);
    stage_rows(qbh, row0, n, D, sb[slot], kNW, w, qoff, QL);
    stage_rows(zbh, row0, n, D, sb[slot] + QB_, kNW, w, qoff, QL);
    stage_rows(dbh, row0, n, DV, sb[slot] + 2 * QB_, kNW, w, doff, VL);
    if (w == 0) {
      const uint32_t lo[1] = {(uint32_t)lane * 16u};
      stage_rows(lbh, row0, n, 4, sb[slot] + 2 * QB_ + VB, 1, 0, lo, 1);
    }
  }

  // one 32-query half of the tile in `slot`
  __device__ __forceinline__ void half(int kt, int mq, int slot, f32x16 (&Y)[NF], f32x16 (&dV)[NMV],
                                       float& sig) const {
    const char* Qs = sb[slot];
    const char* Zq = sb[slot] + QB_;
    const char* Ds = sb[slot] + 2 * QB_;
    const float* Ls = reinterpret_cast<const float*>(sb[slot] + 2 * QB_ + VB);
    const bool own = kt < ta;
    const int qb = qbase(kt) + 32 * mq;
    const int arow = 32 * mq + perm_row(lq);
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma_bf16(lds_row<D>(Qs, arow, 2 * ks + g), kf[ks], sc);
#pragma unroll
    for (int ks = 0; ks < VS; ++ks) dp = mfma_bf16(lds_row<DV>(Ds, arow, 2 * ks + g), vf[ks], dp);
    u32x4 pk[2], dk[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      // queries 32 mq + 16 hh + 8 g + [0, 8): (lse2, D) pairs, 64 bytes
      const float* lp = Ls + 2 * (32 * mq + 16 * hh + 8 * g);
      float p[8], ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * hh + j;
        const int q = qb + 16 * hh + 8 * g + j;
        const float2 st = *reinterpret_cast<const float2*>(lp + 2 * j);
        const bool vis = own ? (q < own_end && q >= myk) : q < next_end;
        p[j] = vis ? exp2_fast(sc[r] - st.x) : 0.f;
        ds[j] = p[j] * (dp[r] - st.y);
      }
      pk[hh] = pack8(p);
      dk[hh] = pack8(ds);
    }
    const u32x4 p0 = pk[0], p1 = pk[1], d0 = dk[0], d1 = dk[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) sig = sum2_bf16(d0[i], sum2_bf16(d1[i], sig));
#pragma unroll
    for (int mv = 0; mv < NMV; ++mv) {
      dV[mv] = mfma_bf16(lds_tr<DV>(Ds, 32 * mq, 32 * mv, lane), p0, dV[mv]);
      dV[mv] = mfma_bf16(lds_tr<DV>(Ds, 32 * mq + 16, 32 * mv, lane), p1, dV[mv]);
    }
#pragma unroll
    for (int fb = 0; fb < NF; ++fb) {
      Y[fb] = mfma_bf16(lds_tr<D>(Zq, 32 * mq, 32 * fb, lane), d0, Y[fb]);
      Y[fb] = mfma_bf16(lds_tr<D>(Zq, 32 * mq + 16, 32 * fb, lane), d1, Y[fb]);
    }
  }

  template <int SLOT>
  __device__ __forceinline__ void tile(int kt, f32x16 (&Y)[NF], f32x16 (&dV)[NMV], float& sig) const {
    if (kt + 1 < ntiles) stage(kt + 1, SLOT ^ 1);
    const int qb0 = qbase(kt);
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      const int qb = qb0 + 32 * mq;
      // skip halves past the sequence, or (own chunk) wholly before the wave's keys
      if (has && qb < n && !(kt < ta && qb + 31 < wj0)) half(kt, mq, SLOT, Y, dV, sig);
    }
    wait_vmem();
    barrier_lds();
  }
};

template <int D, int DV>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(KvArgs a) {
  using L = KvLoop<D, DV>;
  constexpr int NF = L::NF, NMV = L::NMV;
  __shared__ __attribute__((aligned(16))) char S0[L::STAGE];
  __shared__ __attribute__((aligned(16))) char S1[L::STAGE];
  const int kt_ = (int)(blockIdx.x % (unsigned)a.ktiles);
  const int rest = (int)(blockIdx.x / (unsigned)a.ktiles);
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
  l.wj0 = j0 + 32 * l.w;
  l.myk = l.wj0 + l.lq;
  l.has = l.wj0 < jend;
  const size_t base = (size_t)bh * (size_t)n;
  l.qbh = a.qp + base * D;
  l.zbh = a.z + base * D;
  l.dbh = a.dO + base * DV;
  l.lbh = reinterpret_cast<const uint16_t*>(a.ld + 2 * base);
  l.sb[0] = S0;
  l.sb[1] = S1;
  const size_t krow = base + (size_t)min(l.myk, jend - 1);
#pragma unroll
  for (int ks = 0; ks < L::KS; ++ks) l.kf[ks] = ld16(a.z + krow * D + 16 * ks + 8 * l.g);
#pragma unroll
  for (int ks = 0; ks < L::VS; ++ks) l.vf[ks] = ld16(a.v + krow * DV + 16 * ks + 8 * l.g);
  // queries that see these keys: the rest of chunk s, then all of chunk s + 1
  l.ta = (cend - j0 + kT - 1) / kT;
  l.nb0 = (s + 1) * c;
  const int nbq = (a.prev && l.nb0 < n) ? min(l.nb0 + c, n) - l.nb0 : 0;
  l.own_end = cend;
  l.next_end = l.nb0 + nbq;
  l.ntiles = l.ta + (nbq + kT - 1) / kT;
  stage_offsets<D>(l.qoff, kNW, l.w, l.lane);
  stage_offsets<DV>(l.doff, kNW, l.w, l.lane);

  f32x16 Y[NF], dV[NMV];
#pragma unroll
  for (int fb = 0; fb < NF; ++fb) Y[fb] = f32x16{};
#pragma unroll
  for (int mv = 0; mv < NMV; ++mv) dV[mv] = f32x16{};
  float sig = 0.f;
  l.stage(0, 0);
  wait_vmem();
  barrier_lds();
  for (int kt = 0; kt < l.ntiles; kt += 2) {
    l.template tile<0>(kt, Y, dV, sig);
    if (kt + 1 < l.ntiles) l.template tile<1>(kt + 1, Y, dV, sig);
  }
  sig = other_half_sum(sig);

  if (l.myk < jend) {
    const float* kq = a.kq + h * D;
    const float* nq = a.nq + h * D;
    float* dk = a.dk + (base + (size_t)l.myk) * D;
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
          for (int i = 0; i < 4; ++i) o[i] = k4[i] * Y[fb][r + i] + n4[i] * sig;
          *reinterpret_cast<f32x4*>(dk + f + 4 * q) = o;
        }
      }
    float* dv = a.dv + (base + (size_t)l.myk) * DV;
#pragma unroll
    for (int mv = 0; mv < NMV; ++mv)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 32 * mv + 16 * hh + 8 * l.g;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int r = 8 * hh + 4 * q;
          f32x4 o{dV[mv][r], dV[mv][r + 1], dV[mv][r + 2], dV[mv][r + 3]};
          f32x4* p = reinterpret_cast<f32x4*>(dv + col + 4 * q);
          if (a.accum) o += *p;
          *p = o;
        }
      }
  }
}

const uint16_t* dout16(const BwdProblem& p, const BwdWorkspace& w) {
  return w.do16 ? w.do16 : static_cast<const uint16_t*>(p.dout);
}

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

hipError_t launch_bwd_dq(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s) {
  DqArgs a;
  a.qp = w.qp;
  a.z = static_cast<const uint16_t*>(p.f.z);
  a.v = static_cast<const uint16_t*>(p.f.v);
  a.dO = dout16(p, w);
  a.ld = w.ld; a.kk = p.f.kappa_k; a.dq = w.dq;
  a.n = p.f.n;
  const int64_t cc = p.f.c < p.f.n ? p.f.c : p.f.n;
  a.c = (int)cc; a.nchunks = (int)p.f.nchunks; a.H = (int)p.f.H; a.prev = (int)p.f.prev;
  a.qtiles = (int)((cc + kBlk - 1) / kBlk);
  const dim3 grid((unsigned)(p.f.B * p.f.H * p.f.nchunks * a.qtiles));
  if (p.f.dv == 256)
    hipLaunchKernelGGL((bwd_dq_kernel<128, 256>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<128, 128>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdProblem& p, const BwdWorkspace& w, bool accumulate_dv, hipStream_t s) {
  KvArgs a;
  a.qp = w.qp;
  a.z = static_cast<const uint16_t*>(p.f.z);
  a.v = static_cast<const uint16_t*>(p.f.v);
  a.dO = dout16(p, w);
  a.ld = w.ld; a.kq = p.f.kappa_q; a.nq = p.f.nu_q; a.dk = w.dk; a.dv = p.dv;
  a.n = p.f.n;
  const int64_t cc = p.f.c < p.f.n ? p.f.c : p.f.n;
  a.c = (int)cc; a.nchunks = (int)p.f.nchunks; a.H = (int)p.f.H; a.prev = (int)p.f.prev;
  a.ktiles = (int)((cc + kBlk - 1) / kBlk);
  a.accum = accumulate_dv ? 1 : 0;
  const dim3 grid((unsigned)(p.f.B * p.f.H * p.f.nchunks * a.ktiles));
  if (p.f.dv == 256)
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, 256>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, 128>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace gecko
