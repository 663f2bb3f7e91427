// Backward of the adaptive working memory, bf16 inputs, gfx950.
//
// Forward (Gecko summary, paper.rainbus.top, "Method steps" (4)-(5) and
// "Core method"; initial state from the paperlayer.ai summary, Appendix A),
// with t the 0-based chunk entering the memory and S_t the state after it
// (S_{-1} = 0):
//   z_t = z_{t-1} + colsum(exp K_t),  Phi_t = exp(K_t) / z_t,  D_t = z_{t-1} / z_t,
//   Psi_t = psi(K_t) (feature softmax of each row),
//   S_t = D_t * S_{t-1} + Phi_t^T (V_t - Psi_t S_{t-1}) = A_t S_{t-1} + Phi_t^T V_t,
//   A_t = diag(D_t) - Phi_t^T Psi_t,
// and chunk s reads O_m = psi(Q_s) S_{s-lag} (lag 2, or 1 without sliding
// chunks). For L = sum(dO * O_m), dS_t = dL/dS_t:
//   dS_t = R_t + A_{t+1}^T dS_{t+1},  R_t = psi(Q_s)^T dO_s  (s = t + lag)
// (the reverse scan), and per chunk, with X_t = dS_t S_{t-1}^T:
//   dV_t   = Phi_t dS_t
//   dPhi_t = (V_t - Psi_t S_{t-1}) dS_t^T = V_t dS_t^T - Psi_t X_t^T
//   dPsi_t = -Phi_t X_t
//   dK_t   = Phi_t * (dPhi_t + zeta_t) + Psi_t * (dPsi_t - rowsum(dPsi_t * Psi_t))
// where zeta_t = z_t dL/dz_t per feature. Collecting the paths of z_t
// (Phi_t, D_t, D_{t+1}, z_{t+1}) and using Phi_t^T (V_t - Psi_t S_{t-1}) =
// S_t - D_t S_{t-1} gives the backward recurrence
//   zeta_t = D_{t+1} (zeta_{t+1} + rowsum(dS_{t+1} * S_t)) - rowsum(dS_t * S_t)
// (zeta and D at t = nmem taken as 0). With the scan step
// dS_t = R_t + D_{t+1} dS_{t+1} - C_t, C_t = (Phi_{t+1}^T Psi_{t+1})^T dS_{t+1},
// the two D_{t+1} rowsum(dS_{t+1} * S_t) terms cancel exactly, leaving
//   zeta_t = D_{t+1} zeta_{t+1} - rowsum(R_t * S_t) + rowsum(C_t * S_t),
// which is what is evaluated (the form above subtracts two large rowsums). On the query side,
//   dQ_m = psi(Q) * (dPsi_Q - rowsum(dPsi_Q * psi(Q))),  dPsi_Q = dO S_{s-lag}^T,
// where rowsum(dPsi_Q * psi(Q)) is dO . O_m.
//
// The memory chunk pass and scan of the forward are run again first (their
// snapshots S_t are the chunk-boundary states the backward needs), unless a
// training forward kept them; then:
//  rpass   R_t^T per chunk (like the forward's E^T V product, psi(Q) for E)
//  htrans  H_t (Phi_t^T Psi_t up to the per-feature factor) in the order the
//          reverse scan reads it
//  rscan   the reverse scan over t, one workgroup per (b h, 32 values); writes
//          dS_t (bf16) and per-slice rowsums of R_t * S_t and C_t * S_t
//  zscan   zeta_t per (b h, feature)
//  xpass   X_t per chunk
//  qside   dQ_m per token
//  kside   dV and dK_m per token
#include "bwd_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

constexpr int kTT = 64;  // tokens per tile of the readout-gradient pass

// ---------------------------------------------------------------- rpass
struct RArgs {
  const uint16_t* z;
  const uint16_t* dO;
  const float* eta_q;
  const float* rho_q;
  float* r;  // [bh][t][dv/32][d/32][64][16]
  int64_t n, c, nmem;
  int H, lag;
};

// One workgroup per (b h, t): chunk s = t + lag, 4 waves, wave w owns
// features 32 w + [0, 32) of R^T = dO^T psi(Q) (dv x d). Per 64-token tile:
// Z' and dO go to LDS, the psi phase writes psi(Q_m) of the tile's tokens to
// LDS (4 threads per token), and the MFMA phase reads both transposed.
template <int D, int DV>
__global__ __launch_bounds__(2 * D, 1) void bwd_rpass_kernel(RArgs a) {
  constexpr int NW = D / 32, THREADS = 64 * NW, NMV = DV / 32;
  constexpr int ZB = kTT * D * 2, VB = kTT * DV * 2;
  constexpr int ZL = ZB / 16 / THREADS, VL = VB / 16 / THREADS;
  constexpr int PARTS = THREADS / kTT, FPT = D / PARTS;  // psi phase: threads per token, features per thread
  static_assert(PARTS == 4 && FPT % 8 == 0, "psi phase split");
  __shared__ __attribute__((aligned(16))) char S0[ZB + VB];
  __shared__ __attribute__((aligned(16))) char S1[ZB + VB];
  __shared__ __attribute__((aligned(16))) char PS[ZB];
  const int64_t bh = blockIdx.x / a.nmem;
  const int64_t t = blockIdx.x % a.nmem;
  const int h = (int)(bh % a.H);
  const int n = (int)a.n;
  const int cbeg = (int)((t + a.lag) * a.c);
  const int cend = (int)min((int64_t)cbeg + a.c, a.n);
  const int ntiles = (cend - cbeg + kTT - 1) / kTT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t* zbh = a.z + (size_t)bh * n * D;
  const uint16_t* dbh = a.dO + (size_t)bh * n * DV;
  uint32_t zoff[ZL], voff[VL];
  stage_offsets<D>(zoff, NW, w, lane);
  stage_offsets<DV>(voff, NW, w, lane);
  // psi phase: thread -> token tk, features FPT q + [0, FPT)
  const int tk = tid / PARTS, q = tid % PARTS;
  float eq[FPT], rq[FPT];
#pragma unroll
  for (int i = 0; i < FPT; ++i) {
    eq[i] = a.eta_q[h * D + FPT * q + i] * kLog2e;
    rq[i] = a.rho_q[h * D + FPT * q + i] * kLog2e;
  }
  f32x16 acc[NMV];
#pragma unroll
  for (int mv = 0; mv < NMV; ++mv) acc[mv] = f32x16{};

  stage_rows(zbh, cbeg, n, D, S0, NW, w, zoff, ZL);
  stage_rows(dbh, cbeg, n, DV, S0 + ZB, NW, w, voff, VL);
  wait_vmem();
  barrier_lds();
  for (int it = 0; it < ntiles; ++it) {
    char* cur = (it & 1) ? S1 : S0;
    char* nxt = (it & 1) ? S0 : S1;
    if (it + 1 < ntiles) {
      const int r0 = cbeg + (it + 1) * kTT;
      stage_rows(zbh, r0, n, D, nxt, NW, w, zoff, ZL);
      stage_rows(dbh, r0, n, DV, nxt + ZB, NW, w, voff, VL);
    }
    {
      float x[FPT];
#pragma unroll
      for (int k = 0; k < FPT / 8; ++k) unpack8(lds_row<D>(cur, tk, FPT / 8 * q + k), x + 8 * k);
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        x[i] = eq[i] * x[i] + rq[i];
        mx = fmaxf(mx, x[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
      float sm = 0.f;
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        x[i] = exp2_fast(x[i] - mx);
        sm += x[i];
      }
      sm += __shfl_xor(sm, 1, 64);
      sm += __shfl_xor(sm, 2, 64);
      // tokens past the chunk (a chunk length that is not a multiple of the
      // tile) or the sequence enter with weight zero
      const float inv = cbeg + it * kTT + tk < cend ? 1.f / sm : 0.f;
#pragma unroll
      for (int i = 0; i < FPT; ++i) x[i] *= inv;
#pragma unroll
      for (int k = 0; k < FPT / 8; ++k) {
        const int ch = FPT / 8 * q + k;
        *reinterpret_cast<u32x4*>(PS + tk * (D * 2) + 16 * (ch ^ sw16(tk))) = pack8(x + 8 * k);
      }
    }
    barrier_lds();
#pragma unroll
    for (int ks = 0; ks < kTT / 16; ++ks) {
      const u32x4 b = lds_tr<D, false>(PS, 16 * ks, 32 * w, lane);
#pragma unroll
      for (int mv = 0; mv < NMV; ++mv) acc[mv] = mfma_bf16(lds_tr<DV, false>(cur + ZB, 16 * ks, 32 * mv, lane), b, acc[mv]);
    }
    wait_vmem();
    barrier_lds();
  }
  const int64_t row = bh * a.nmem + t;
#pragma unroll
  for (int mv = 0; mv < NMV; ++mv) {
    f32x4* o = reinterpret_cast<f32x4*>(a.r + ((((row * NMV + mv) * NW + w) * 64) + lane) * 16);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) o[qq] = f32x4{acc[mv][4 * qq], acc[mv][4 * qq + 1], acc[mv][4 * qq + 2], acc[mv][4 * qq + 3]};
  }
}

// ---------------------------------------------------------------- htrans
// hm (the forward chunk pass) holds H_t[32 w + lq][f'] at [t][ks][w][lane][e],
// f' = 16 ks + 8 (e >> 2) + 4 g + (e & 3). The reverse scan needs H_t[f'][f]
// at the same position with f = 32 w + lq.
template <int D>
__global__ __launch_bounds__(256) void bwd_htrans_kernel(const uint16_t* __restrict__ hm, uint16_t* __restrict__ ht) {
  constexpr int NW = D / 32;
  const int64_t base = (int64_t)blockIdx.x * D * D;
  for (int o = threadIdx.x; o < D * D; o += 256) {
    const int e = o & 7, lane = (o >> 3) & 63, w = (o >> 9) % NW, ks = (o >> 9) / NW;
    const int g = lane >> 5, lq = lane & 31;
    const int fa = 16 * ks + 8 * (e >> 2) + 4 * g + (e & 3);  // row index of H (the E feature)
    const int fb = 32 * w + lq;                               // column index (the psi feature)
    // position of H_t[fa][fb] in hm
    const int rem = fb & 15;
    const int es = 4 * (rem >> 3) + (rem & 3), gs = (rem >> 2) & 1;
    const int src = (((fb >> 4) * NW + (fa >> 5)) * 64 + 32 * gs + (fa & 31)) * 8 + es;
    ht[base + o] = hm[base + src];
  }
}

// ---------------------------------------------------------------- rscan
struct RScanArgs {
  const float* r;       // [bh][t][dv/32][d/32][64][16]
  const uint16_t* ht;   // [bh][t][d/16][d/32][64][8]
  const float* decay;   // [bh][t][d]
  const float* wscale;  // [bh][t][d]
  const float* s32;     // [bh][t][d][dv]: S_t in float32
  uint16_t* ds;         // [bh][t][d][dv]
  float* part;          // [bh][t][dv/32][d][2]: rowsum(R_t * S_t), rowsum(C_t * S_t) over the slice
  int64_t nmem;
};

template <int D>
struct RStep {
  static constexpr int KS = D / 16;
  f32x4 rv[4];     // R_t^T cells of this lane
  u32x4 hf[KS];    // H_{t+1} in B-operand order
  f32x4 sv[4];     // S_t cells
  float dn, ws;    // D_{t+1}[f], wscale_t[f]
};

// Workgroup per (b h, 32-value slice j), 4 waves. Lane (w, lq, g) holds
// dS^T[v][f] for f = 32 w + lq and v = 32 j + 8 (r >> 2) + 4 g + (r & 3), the
// layout of the forward scan. Step t:
//   dS_t^T = R_t^T + D_{t+1} dS_{t+1}^T - (wscale_{t+1} dS_{t+1})^T H_{t+1}
// the last term one MFMA chain with A = a bf16 LDS copy of
// wscale_{t+1} * dS_{t+1} ([f][v], read transposed as in the forward scan)
// and B = H_{t+1} in transposed order.
template <int D, int DV, bool kNoDelta>
__global__ __launch_bounds__(2 * D, 1) void bwd_rscan_kernel(RScanArgs a) {
  constexpr int NMV = DV / 32, NW = D / 32, KS = D / 16, kDepth = 3;
  __shared__ __attribute__((aligned(16))) uint16_t mt[2][D * 32];
  const int64_t BH = gridDim.x / NMV;
  const int64_t bh = blockIdx.x % BH;
  const int j = (int)(blockIdx.x / BH);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, lq = lane & 31;
  const int f = 32 * w + lq;
  const int64_t nmem = a.nmem;
  const int sl = lane & 15, grp2 = (lane >> 4) & 1;
  const int trb = (4 * g + (sl >> 2)) * 64 + (16 * grp2 + 4 * (sl & 3)) * 2;

  // operands of step t in three parts: H_{t+1}; R_t and S_t; the decay and
  // scale. A wave waits while its loads are issued (64 KiB a step through
  // the CU's load path), so each step issues them at its own waits (see step)
  auto load = [&](int64_t t, RStep<D>& q, int part) {
    const int64_t row = bh * nmem + t;
    if (part == 0) {
      const int64_t t1 = t + 1 < nmem ? t + 1 : t;  // (unused at the last step)
      const uint16_t* hp = a.ht + (bh * nmem + t1) * (int64_t)D * D + ((int64_t)w * 64 + lane) * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) q.hf[ks] = ld16(hp + (int64_t)ks * NW * 64 * 8);
    } else if (part == 1) {
      const f32x4* rt = reinterpret_cast<const f32x4*>(a.r + ((((row * NMV + j) * NW + w) * 64) + lane) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) q.rv[i] = rt[i];
      const float* sp = a.s32 + row * (int64_t)D * DV + (int64_t)f * DV + 32 * j + 4 * g;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) q.sv[qq] = *reinterpret_cast<const f32x4*>(sp + 8 * qq);
    } else {
      q.dn = t + 1 < nmem ? a.decay[(bh * nmem + t + 1) * D + f] : 0.f;
      q.ws = a.wscale[row * D + f];
    }
  };

  f32x16 cur = f32x16{};  // dS_{t+1}^T
  int buf = 0;
  // step t (in decreasing t) fills nxt, the slot the step before it in the
  // loop used, with the operands of step tn
  auto step = [&](int64_t t, const RStep<D>& q, RStep<D>& nxt, int64_t tn) {
    f32x16 p0 = f32x16{}, p1 = f32x16{};
    if constexpr (!kNoDelta) {
      if (t + 1 < nmem) {  // mt[buf] holds wscale_{t+1} dS_{t+1}
        const char* mb = reinterpret_cast<const char*>(mt[buf]) + trb;
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) {
          const u32x2 a0 = lds_read_tr(mb + (16 * ks) * 64), a1 = lds_read_tr(mb + (16 * ks + 8) * 64);
          const u32x2 b0 = lds_read_tr(mb + (16 * ks + 16) * 64), b1 = lds_read_tr(mb + (16 * ks + 24) * 64);
          p0 = mfma_bf16(u32x4{a0[0], a0[1], a1[0], a1[1]}, q.hf[ks], p0);
          p1 = mfma_bf16(u32x4{b0[0], b0[1], b1[0], b1[1]}, q.hf[ks + 1], p1);
        }
      }
    }
    load(tn, nxt, 0);
    // rowsums of R_t * S_t and C_t * S_t over this lane's cells (zeta)
    float s_r = 0.f, s_c = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float sv = q.sv[r >> 2][r & 3], rv = q.rv[r >> 2][r & 3], cv = p0[r] + p1[r];
      s_r += rv * sv;
      s_c += cv * sv;
      cur[r] = rv + q.dn * cur[r] - cv;
    }
    load(tn, nxt, 1);
    s_r = other_half_sum(s_r);
    s_c = other_half_sum(s_c);
    if (g == 0)
      *reinterpret_cast<float2*>(a.part + (((bh * nmem + t) * NMV + j) * D + f) * 2) = make_float2(s_r, s_c);
    // dS_t (bf16) to HBM: row f, values 32 j + 8 qq + 4 g + [0, 4)
    uint16_t* dp = a.ds + (bh * nmem + t) * (int64_t)D * DV + (int64_t)f * DV + 32 * j + 4 * g;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      *reinterpret_cast<u32x2*>(dp + 8 * qq) =
          u32x2{pack2(cur[4 * qq], cur[4 * qq + 1]), pack2(cur[4 * qq + 2], cur[4 * qq + 3])};
    // scaled copy for step t - 1
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      *reinterpret_cast<u32x2*>(&mt[buf ^ 1][f * 32 + 8 * qq + 4 * g]) =
          u32x2{pack2(q.ws * cur[4 * qq], q.ws * cur[4 * qq + 1]), pack2(q.ws * cur[4 * qq + 2], q.ws * cur[4 * qq + 3])};
    __syncthreads();
    load(tn, nxt, 2);
    buf ^= 1;
  };

  // loop step i (t = nmem - 1 - i) uses slot i mod kDepth and fills slot
  // (i - 1) mod kDepth, done with, for step i + kDepth - 1; loads past the
  // last step re-read it (unused)
  RStep<D> ring[kDepth];
#pragma unroll
  for (int k = 0; k < kDepth - 1; ++k)
#pragma unroll
    for (int part = 0; part < 3; ++part) load(max(nmem - 1 - k, (int64_t)0), ring[k], part);
  int64_t k0 = 0;
  for (; k0 + kDepth <= nmem; k0 += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k)
      step(nmem - 1 - (k0 + k), ring[k], ring[(k + kDepth - 1) % kDepth],
           max(nmem - 1 - (k0 + k + kDepth - 1), (int64_t)0));
  }
#pragma unroll
  for (int k = 0; k < kDepth; ++k)
    if (k0 + k < nmem)
      step(nmem - 1 - (k0 + k), ring[k], ring[(k + kDepth - 1) % kDepth],
           max(nmem - 1 - (k0 + k + kDepth - 1), (int64_t)0));
}

// ---------------------------------------------------------------- zscan
__global__ void bwd_zeta_kernel(const float* __restrict__ part, const float* __restrict__ decay,
                                float* __restrict__ zeta, int64_t nmem, int D, int nsl) {
  const int f = threadIdx.x;
  if (f >= D) return;
  const int64_t bh = blockIdx.x;
  float z = 0.f;
  // the loads do not depend on the recurrence: unrolled, they run ahead of it
#pragma unroll 4
  for (int64_t t = nmem - 1; t >= 0; --t) {
    const int64_t row = bh * nmem + t;
    float pr = 0.f, pc = 0.f;
#pragma unroll 8
    for (int j = 0; j < nsl; ++j) {
      const float2 pp = *reinterpret_cast<const float2*>(part + ((row * nsl + j) * D + f) * 2);
      pr += pp.x;
      pc += pp.y;
    }
    z = (t + 1 < nmem ? decay[(row + 1) * D + f] * z : 0.f) - pr + pc;
    zeta[row * D + f] = z;
  }
}

// ---------------------------------------------------------------- xpass
// X_t = dS_t S_{t-1}^T (d x d, bf16 row-major); X_0 = 0. Wave w: rows 32 w + [0, 32).
template <int D, int DV>
__global__ __launch_bounds__(2 * D) void bwd_xpass_kernel(const uint16_t* __restrict__ ds,
                                                         const uint16_t* __restrict__ snap,
                                                         uint16_t* __restrict__ x, int64_t nmem) {
  constexpr int NW = D / 32, VS = DV / 16;
  __shared__ __attribute__((aligned(16))) uint16_t xs[D * D];
  const int64_t row = blockIdx.x;
  const int64_t t = row % nmem;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, lq = lane & 31;
  uint16_t* dst = x + row * (int64_t)D * D;
  if (t == 0) {
    for (int e = tid; e < D * D / 8; e += 2 * D) st16(dst + 8 * e, u32x4{0u, 0u, 0u, 0u});
    return;
  }
  const uint16_t* dsr = ds + row * (int64_t)D * DV + (int64_t)(32 * w + lq) * DV + 8 * g;
  const uint16_t* sp = snap + (row - 1) * (int64_t)D * DV + (int64_t)lq * DV + 8 * g;
  f32x16 acc[NW];
#pragma unroll
  for (int cb = 0; cb < NW; ++cb) acc[cb] = f32x16{};
#pragma unroll 4
  for (int ks = 0; ks < VS; ++ks) {
    const u32x4 av = ld16(dsr + 16 * ks);
#pragma unroll
    for (int cb = 0; cb < NW; ++cb) acc[cb] = mfma_bf16(av, ld16(sp + (int64_t)32 * cb * DV + 16 * ks), acc[cb]);
  }
  // C[f][f'']: lane column f'' = 32 cb + lq, register r row f = 32 w + 8 (r >> 2) + 4 g + (r & 3)
#pragma unroll
  for (int cb = 0; cb < NW; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int fr = 32 * w + 8 * (r >> 2) + 4 * g + (r & 3);
      xs[fr * D + 32 * cb + lq] = (uint16_t)(pack2(acc[cb][r], 0.f) & 0xFFFFu);
    }
  __syncthreads();
  for (int e = tid; e < D * D / 8; e += 2 * D) st16(dst + 8 * e, *reinterpret_cast<const u32x4*>(&xs[8 * e]));
}

// ---------------------------------------------------------------- token passes
struct SideArgs {
  const uint16_t* z;
  const uint16_t* v;
  const uint16_t* dO;
  const float* eta_q; const float* rho_q; const float* eta_k; const float* rho_k;
  const uint16_t* snap;   // [bh][t][d][dv]
  const float* s32;       // [bh][t][d][dv]
  const uint16_t* ds;     // [bh][t][d][dv]
  const uint16_t* x;      // [bh][t][d][d]
  const float* cmax;      // [bh][t][d]
  const float* wscale;    // [bh][t][d]
  const float* zeta;      // [bh][t][d]
  float* dqm;             // [bh][n][d]
  float* dkm;             // [bh][n][d]
  float* dv;              // [bh][n][dv]
  int64_t n, c, nmem;
  int nchunks, blocks_per_chunk, H, lag;
  uint32_t nblocks, per_xcd;
};

// Per-token gradients leave the side kernels through a wave-private LDS
// block: their MFMA accumulators hold one token per lane, so storing them
// directly writes 16 bytes into each of 64 different rows per instruction.
// block_store takes a 32-token x 32-column float32 block in accumulator
// order (lane (lq, g): token lq, column 16 (r >> 3) + 8 g + (r & 7) for
// element r), and stores it so that each instruction writes eight whole
// 128-byte row pieces. Rows are padded to kTS floats (conflict-free writes).
// LDS accesses of one wave are processed in order, so neither the read after
// the write nor the next block's write after this block's read needs a wait
// of its own.
constexpr int kTS = 36;
__device__ __forceinline__ void block_store(float* buf, const float (&x)[16], int lane, float* dst, int64_t ld,
                                            int nvalid) {
  const int lq = lane & 31, g = lane >> 5;
  float* wp = buf + lq * kTS + 8 * g;
  *reinterpret_cast<f32x4*>(wp) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(wp + 4) = f32x4{x[4], x[5], x[6], x[7]};
  *reinterpret_cast<f32x4*>(wp + 16) = f32x4{x[8], x[9], x[10], x[11]};
  *reinterpret_cast<f32x4*>(wp + 20) = f32x4{x[12], x[13], x[14], x[15]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = (lane >> 3) + 8 * i, c4 = 4 * (lane & 7);
    const f32x4 y = *reinterpret_cast<const f32x4*>(buf + tr * kTS + c4);
    if (tr < nvalid) *reinterpret_cast<f32x4*>(dst + tr * ld + c4) = y;
  }
}

// Workgroups go to the 8 XCDs round-robin, each with its own L2; logical
// block (b mod 8) per_xcd + b / 8 keeps the blocks of one chunk (which all
// stage that chunk's state-sized operands) on one XCD.
__device__ __forceinline__ uint32_t side_block(const SideArgs& a) {
  return (blockIdx.x & 7u) * a.per_xcd + (blockIdx.x >> 3);
}

// features of lane half g in B-operand order: k-step ks, element e -> 16 ks + 8 g + e
template <int D>
__device__ __forceinline__ void row_features(const uint16_t* zr, const float* sc, const float* sh, int g,
                                             float (&x)[D / 2]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int f0 = 16 * ks + 8 * g;
    float zz[8];
    unpack8(ld16(zr + f0), zz);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[8 * ks + i] = (sc[f0 + i] * zz[i] + sh[f0 + i]) * kLog2e;
  }
}

// feature softmax of a row held half by each lane half (log2-scaled logits), in place
template <int N>
__device__ __forceinline__ void softmax2(float (&x)[N]) {
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < N; ++i) mx = fmaxf(mx, x[i]);
  mx = other_half_max(mx);
  float sm = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    x[i] = exp2_fast(x[i] - mx);
    sm += x[i];
  }
  const float inv = 1.f / other_half_sum(sm);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] *= inv;
}

// Query side: one workgroup per (b h, chunk s, 256 tokens), wave = 32 tokens
// (lane = token). dPsi^T = S_{s-lag} dO^T with the state staged in LDS.
template <int D, int DV>
__global__ __launch_bounds__(512, 1) void bwd_qside_kernel(SideArgs a) {
  constexpr int NF = D / 32, VS = DV / 16, KS = D / 16;
  constexpr int MB = D * DV * 2;
  __shared__ __attribute__((aligned(16))) char Ms[MB];
  __shared__ float CS[512];
  __shared__ __attribute__((aligned(16))) float TB[8][32 * kTS];
  const uint32_t lb = side_block(a);
  if (lb >= a.nblocks) return;
  const int blk = (int)(lb % (unsigned)a.blocks_per_chunk);
  const int rest = (int)(lb / (unsigned)a.blocks_per_chunk);
  const int s = rest % a.nchunks;
  const int64_t bh = rest / a.nchunks;
  const int h = (int)(bh % a.H);
  const int64_t n = a.n;
  const int64_t cbeg = s * a.c, cend = min(cbeg + a.c, n);
  const int64_t t0 = cbeg + 256 * blk;
  if (t0 >= cend) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tok = t0 + 32 * w + lq;
  const bool valid = tok < cend;
  const int64_t trow = bh * n + min(tok, cend - 1);
  const bool reads = s >= a.lag;
  if (!reads) {  // chunks before the first memory read
    if (valid) {
      float* o = a.dqm + trow * D;
      for (int f = 8 * g; f < D; f += 16) {
        *reinterpret_cast<f32x4*>(o + f) = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(o + f + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }
  {
    // M = S_{s-lag} from the float32 states with each column centred on its
    // mean over the features, then rounded to bf16. dQ_m depends on dPsi only
    // through dPsi - rowsum(dPsi * psi), which a row added to every feature of
    // M leaves unchanged (psi sums to one); centring keeps the differences
    // between features, small next to M itself when the memory's rows are
    // alike, at bf16 precision.
    constexpr int TPC = 512 / DV, RPT = D / TPC;  // threads per column, rows per thread
    const float* m32 = a.s32 + (bh * a.nmem + (s - a.lag)) * (int64_t)D * DV;
    const int col = tid % DV, part = tid / DV;
    float mv[RPT];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      mv[i] = m32[(int64_t)(part * RPT + i) * DV + col];
      sum += mv[i];
    }
    CS[tid] = sum;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < TPC; ++k) tot += CS[k * DV + col];
    const float mean = tot * (1.f / D);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int f = part * RPT + i;
      *reinterpret_cast<uint16_t*>(Ms + f * (DV * 2) + 16 * ((col >> 3) ^ sw16(f)) + 2 * (col & 7)) =
          (uint16_t)(pack2(mv[i] - mean, 0.f) & 0xFFFFu);
    }
  }
  float psi[D / 2];
  row_features<D>(a.z + trow * D, a.eta_q + h * D, a.rho_q + h * D, g, psi);
  softmax2(psi);
  u32x4 df[VS];
#pragma unroll
  for (int ks = 0; ks < VS; ++ks) df[ks] = ld16(a.dO + trow * DV + 16 * ks + 8 * g);
  wait_vmem();
  barrier_lds();
  f32x16 acc[NF];
#pragma unroll
  for (int fb = 0; fb < NF; ++fb) {
    acc[fb] = f32x16{};
    const int arow = 32 * fb + perm_row(lq);
#pragma unroll
    for (int ks = 0; ks < VS; ++ks) acc[fb] = mfma_bf16(lds_row<DV>(Ms, arow, 2 * ks + g), df[ks], acc[fb]);
  }
  // register r of block fb: feature 32 fb + 16 (r >> 3) + 8 g + (r & 7) = psi index 8 (2 fb + (r >> 3)) + (r & 7)
  float rs = 0.f;
#pragma unroll
  for (int fb = 0; fb < NF; ++fb)
#pragma unroll
    for (int r = 0; r < 16; ++r) rs += acc[fb][r] * psi[16 * fb + r];
  rs = other_half_sum(rs);
  (void)KS;
  {
    // rows t0 + 32 w + [0, 32) of dQ_m, those before cend
    const int64_t w0 = t0 + 32 * w;
    const int nvalid = (int)min((int64_t)32, cend - w0);
    float* o = a.dqm + (bh * n + w0) * D;
#pragma unroll
    for (int fb = 0; fb < NF; ++fb) {
      float y[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) y[r] = psi[16 * fb + r] * (acc[fb][r] - rs);
      block_store(TB[w], y, lane, o + 32 * fb, D, nvalid);
    }
  }
}

// Key side: one workgroup per (b h, chunk t, 256 tokens), wave = 32 tokens
// (lane = token); dS_t and X_t staged in LDS. Chunks that never enter the
// memory write zeros.
template <int D, int DV, bool kNoDelta>
__global__ __launch_bounds__(512, 1) void bwd_kside_kernel(SideArgs a) {
  constexpr int NF = D / 32, VS = DV / 16, KS = D / 16, NMV = DV / 32;
  constexpr int DSB = D * DV * 2, XB = D * D * 2;
  constexpr int DSL = DSB / 16 / 512, XL = XB / 16 / 512;
  __shared__ __attribute__((aligned(16))) char DSs[DSB];
  __shared__ __attribute__((aligned(16))) char Xs[kNoDelta ? 16 : XB];
  __shared__ __attribute__((aligned(16))) float FV[2 * D];  // log2 z_t, zeta_t
  __shared__ __attribute__((aligned(16))) float TB[8][32 * kTS];
  const uint32_t lb = side_block(a);
  if (lb >= a.nblocks) return;
  const int blk = (int)(lb % (unsigned)a.blocks_per_chunk);
  const int rest = (int)(lb / (unsigned)a.blocks_per_chunk);
  const int t = rest % a.nchunks;
  const int64_t bh = rest / a.nchunks;
  const int h = (int)(bh % a.H);
  const int64_t n = a.n;
  const int64_t cbeg = t * a.c, cend = min(cbeg + a.c, n);
  const int64_t t0 = cbeg + 256 * blk;
  if (t0 >= cend) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tok = t0 + 32 * w + lq;
  const bool valid = tok < cend;
  const int64_t trow = bh * n + min(tok, cend - 1);
  if (t >= a.nmem) {
    if (valid) {
      float* o = a.dkm + trow * D;
      for (int f = 4 * g; f < D; f += 8) *reinterpret_cast<f32x4*>(o + f) = f32x4{0.f, 0.f, 0.f, 0.f};
      float* ov = a.dv + trow * DV;
      for (int f = 4 * g; f < DV; f += 8) *reinterpret_cast<f32x4*>(ov + f) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int64_t crow = bh * a.nmem + t;
  {
    uint32_t off[DSL];
    stage_offsets<DV>(off, 8, w, lane);
    stage_rows(a.ds + crow * (int64_t)D * DV, 0, D, DV, DSs, 8, w, off, DSL);
    if constexpr (!kNoDelta) {
      uint32_t xo[XL];
      stage_offsets<D>(xo, 8, w, lane);
      stage_rows(a.x + crow * (int64_t)D * D, 0, D, D, Xs, 8, w, xo, XL);
    }
  }
  if (tid < D) {
    FV[tid] = a.cmax[crow * D + tid] - log2f(a.wscale[crow * D + tid]);
    FV[D + tid] = a.zeta[crow * D + tid];
  }
  float km[D / 2];
  row_features<D>(a.z + trow * D, a.eta_k + h * D, a.rho_k + h * D, g, km);
  wait_vmem();
  barrier_lds();
  // Phi = 2^(k - log2 z_t) and psi(K) in B-operand order, bf16
  u32x4 phf[KS], psf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = exp2_fast(km[8 * ks + i] - FV[16 * ks + 8 * g + i]);
    phf[ks] = pack8(e);
  }
  if constexpr (!kNoDelta) {
    softmax2(km);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) psf[ks] = pack8(km + 8 * ks);
  }
  // rows t0 + 32 w + [0, 32) of dV and dK_m, those before cend
  const int64_t w0 = t0 + 32 * w;
  const int nvalid = (int)min((int64_t)32, cend - w0);
  // dV^T = dS_t^T Phi^T, block by block
  {
    float* ov = a.dv + (bh * n + w0) * DV;
#pragma unroll
    for (int mv = 0; mv < NMV; ++mv) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16(lds_tr<DV>(DSs, 16 * ks, 32 * mv, lane), phf[ks], acc);
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = acc[r];
      block_store(TB[w], x, lane, ov + 32 * mv, DV, nvalid);
    }
  }
  // dPhi^T = dS_t V^T - X_t Psi^T,  dPsi^T = -X_t^T Phi^T
  f32x16 dph[NF], dps[NF];
  const uint16_t* vr = a.v + trow * DV + 8 * g;
#pragma unroll
  for (int fb = 0; fb < NF; ++fb) {
    dph[fb] = f32x16{};
    dps[fb] = f32x16{};
  }
#pragma unroll 4
  for (int ks = 0; ks < VS; ++ks) {
    const u32x4 vb = ld16(vr + 16 * ks);
#pragma unroll
    for (int fb = 0; fb < NF; ++fb)
      dph[fb] = mfma_bf16(lds_row<DV>(DSs, 32 * fb + perm_row(lq), 2 * ks + g), vb, dph[fb]);
  }
  if constexpr (!kNoDelta) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 np = neg8(psf[ks]), nf = neg8(phf[ks]);
#pragma unroll
      for (int fb = 0; fb < NF; ++fb) {
        dph[fb] = mfma_bf16(lds_row<D>(Xs, 32 * fb + perm_row(lq), 2 * ks + g), np, dph[fb]);
        dps[fb] = mfma_bf16(lds_tr<D>(Xs, 16 * ks, 32 * fb, lane), nf, dps[fb]);
      }
    }
  }
  // dK_m = Phi (dPhi + zeta) + Psi (dPsi - rowsum(dPsi Psi)); register r of
  // block fb is feature 32 fb + 16 (r >> 3) + 8 g + (r & 7), operand k-step
  // 2 fb + (r >> 3), element r & 7
  float rs = 0.f;
  if constexpr (!kNoDelta) {
#pragma unroll
    for (int fb = 0; fb < NF; ++fb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float ps[8];
        unpack8(psf[2 * fb + hh], ps);
#pragma unroll
        for (int i = 0; i < 8; ++i) rs += dps[fb][8 * hh + i] * ps[i];
      }
    rs = other_half_sum(rs);
  }
  {
    float* o = a.dkm + (bh * n + w0) * D;
#pragma unroll
    for (int fb = 0; fb < NF; ++fb) {
      float y[16];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int f = 32 * fb + 16 * hh + 8 * g;
        float ph[8], ps[8];
        unpack8(phf[2 * fb + hh], ph);
        if constexpr (!kNoDelta) unpack8(psf[2 * fb + hh], ps);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          y[8 * hh + i] = ph[i] * (dph[fb][8 * hh + i] + FV[D + f + i]);
          if constexpr (!kNoDelta) y[8 * hh + i] += ps[i] * (dps[fb][8 * hh + i] - rs);
        }
      }
      block_store(TB[w], y, lane, o + 32 * fb, D, nvalid);
    }
  }
}

const uint16_t* dout16(const BwdProblem& p, const BwdWorkspace& w) {
  return w.do16 ? w.do16 : static_cast<const uint16_t*>(p.dout);
}

template <int D, int DV>
hipError_t launch_all(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s) {
  const Problem& f = p.f;
  const int64_t BH = f.B * f.H;
  const bool no_delta = (f.flags & GECKO_AWM_NO_DELTA_BIT) != 0;
  const uint16_t* dO = dout16(p, w);
  hipError_t e;
  if (f.nmem > 0) {
    // the forward memory pass, denominator prefix and scan (snapshots S_t),
    // unless the training forward kept them
    if (!p.mem_saved) {
      if ((e = launch_awm_chunk_bf16(f, w.fw, s)) != hipSuccess) return e;
      if ((e = launch_awm_zscan(f, w.fw, s)) != hipSuccess) return e;
      if ((e = launch_awm_scan_bf16(f, w.fw, s)) != hipSuccess) return e;
    }
    RArgs ra;
    ra.z = static_cast<const uint16_t*>(f.z);
    ra.dO = dO;
    ra.eta_q = f.eta_q; ra.rho_q = f.rho_q; ra.r = w.r;
    ra.n = f.n; ra.c = f.c; ra.nmem = f.nmem; ra.H = (int)f.H; ra.lag = (int)f.lag;
    hipLaunchKernelGGL((bwd_rpass_kernel<D, DV>), dim3((unsigned)(BH * f.nmem)), dim3(2 * D), 0, s, ra);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!no_delta) {
      hipLaunchKernelGGL((bwd_htrans_kernel<D>), dim3((unsigned)(BH * f.nmem)), dim3(256), 0, s,
                         static_cast<const uint16_t*>(w.fw.h), w.ht);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    RScanArgs sa;
    sa.r = w.r; sa.ht = w.ht; sa.decay = w.fw.decay; sa.wscale = w.fw.wscale;
    sa.s32 = w.s32; sa.ds = w.ds; sa.part = w.part; sa.nmem = f.nmem;
    const dim3 sgrid((unsigned)(BH * (DV / 32)));
    if (no_delta)
      hipLaunchKernelGGL((bwd_rscan_kernel<D, DV, true>), sgrid, dim3(2 * D), 0, s, sa);
    else
      hipLaunchKernelGGL((bwd_rscan_kernel<D, DV, false>), sgrid, dim3(2 * D), 0, s, sa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_zeta_kernel, dim3((unsigned)BH), dim3(D), 0, s, w.part, w.fw.decay, w.zeta, f.nmem,
                       D, DV / 32);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!no_delta) {
      hipLaunchKernelGGL((bwd_xpass_kernel<D, DV>), dim3((unsigned)(BH * f.nmem)), dim3(2 * D), 0, s, w.ds,
                         static_cast<const uint16_t*>(w.fw.snap), w.x, f.nmem);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  SideArgs sa;
  sa.z = static_cast<const uint16_t*>(f.z);
  sa.v = static_cast<const uint16_t*>(f.v);
  sa.dO = dO;
  sa.eta_q = f.eta_q; sa.rho_q = f.rho_q; sa.eta_k = f.eta_k; sa.rho_k = f.rho_k;
  sa.snap = static_cast<const uint16_t*>(w.fw.snap);
  sa.s32 = w.s32;
  sa.ds = w.ds; sa.x = w.x; sa.cmax = w.fw.cmax; sa.wscale = w.fw.wscale; sa.zeta = w.zeta;
  sa.dqm = w.dqm; sa.dkm = w.dkm; sa.dv = p.dv;
  const int64_t cc = f.c < f.n ? f.c : f.n;
  sa.n = f.n; sa.c = cc; sa.nmem = f.nmem;
  sa.nchunks = (int)f.nchunks;
  sa.blocks_per_chunk = (int)((cc + 255) / 256);
  sa.H = (int)f.H; sa.lag = (int)f.lag;
  const int64_t nblocks = BH * f.nchunks * sa.blocks_per_chunk;
  sa.nblocks = (uint32_t)nblocks;
  sa.per_xcd = (uint32_t)((nblocks + 7) / 8);
  const dim3 grid((unsigned)(8 * sa.per_xcd));
  hipLaunchKernelGGL((bwd_qside_kernel<D, DV>), grid, dim3(512), 0, s, sa);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (no_delta)
    hipLaunchKernelGGL((bwd_kside_kernel<D, DV, true>), grid, dim3(512), 0, s, sa);
  else
    hipLaunchKernelGGL((bwd_kside_kernel<D, DV, false>), grid, dim3(512), 0, s, sa);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_awm(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s) {
  if (p.f.d == 128 && p.f.dv == 256) return launch_all<128, 256>(p, w, s);
  if (p.f.d == 128 && p.f.dv == 128) return launch_all<128, 128>(p, w, s);
  return hipErrorInvalidValue;
}

}  // namespace gecko
