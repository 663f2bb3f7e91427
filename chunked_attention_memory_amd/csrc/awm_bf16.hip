// Adaptive working memory for bf16 inputs on gfx950: the chunk-parallel pass
// and the sequential state scan.
//
// The memory update (Gecko summary, paper.rainbus.top, "Method steps" (4) and
// "Core method"; initial state from the paperlayer.ai summary, Appendix A) is,
// with 0-based chunk t entering the state M'_{t+1} -> M'_{t+2}:
//   M'_{t+2} = (z^{t-1}/z^t) * M'_{t+1} + phi^t(K_t)^T (V_t - psi(K_t) M'_{t+1})
// where z^t is the per-feature exp-sum of the memory keys over chunks 0..t,
// phi^t(k) = exp(k)/z^t and psi is the feature softmax of a row.
//
// Reassociation used here: with m_t the (per-feature) max of K_t and
// E_t = exp(K_t - m_t), phi^t(K_t)^T = diag(exp(m_t)/z^t) E_t^T, so
//   M'_{t+2} = decay_t * M'_{t+1} + wscale_t * (G_t - H_t M'_{t+1})
// with G_t = E_t^T V_t (d x dv), H_t = E_t^T psi(K_t) (d x d),
// decay_t = z^{t-1}/z^t and wscale_t = exp(m_t)/z^t (both per row). G_t, H_t,
// m_t and the column sums l_t of E_t depend on chunk t alone (chunk-parallel
// pass); decay and wscale come from a running log-space prefix of (m_t, l_t);
// the product H_t M'_{t+1} is the only sequential part (scan).
// All maxima and logarithms are kept in base 2 (exp2 on the hardware).
#include "gecko_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

constexpr int kBT = 64;          // tokens per tile of the chunk pass
constexpr float kLazy = 8.0f;    // rescale accumulators only when the max grows by > 2^8

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// reduction over aligned groups of G lanes (G = 8 or 16) with DPP lane swaps
template <int G>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  if constexpr (G == 16) x = fmaxf(x, dpp<0x140>(x));  // row_mirror
  return x;
}
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  if constexpr (G == 16) x += dpp<0x140>(x);
  return x;
}

template <int D, int DV>
struct ChunkTile {
  static constexpr int ROW = kBT + 8;  // LDS row (bf16 elements) of Z^T, psi^T and V^T
  static constexpr int ZELEMS = D * ROW;
  static constexpr int PELEMS = D * ROW;
  static constexpr int VELEMS = DV * ROW;
  static constexpr size_t LDS_BYTES = (size_t)(ZELEMS + PELEMS + VELEMS) * sizeof(uint16_t);
  static constexpr int THREADS = 2 * D;  // D / 32 waves, one 32-feature block each
};

struct ChunkArgs {
  const uint16_t* z;
  const uint16_t* v;
  const float* eta_k;
  const float* rho_k;
  float* g;          // [bh][t][dv/32][d][32]
  uint16_t* hm;      // [bh][t][d][d]
  float* cmax;       // [bh][t][d] (log2 units)
  float* csum;       // [bh][t][d]
  int64_t n, c, nmem;
  int H;
};

// One workgroup per (batch*head, chunk t). Wave w owns key features
// [32 w, 32 w + 32) and accumulates, transposed,
//   G^T (dv x 32) += V^T E and H^T (d x 32) += psi^T E
// over 64-token tiles, with E = exp(K_m - m) under a running per-feature max.
template <int D, int DV>
__global__ __launch_bounds__(2 * D, 1) void awm_chunk_bf16_kernel(ChunkArgs a) {
  using T = ChunkTile<D, DV>;
  constexpr int NMV = DV / 32;
  constexpr int NMF = D / 32;
  constexpr int FG = D / 8;   // 8-feature groups per token row
  constexpr int VG = DV / 8;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* Zt = lds;                 // [d][ROW]  raw z, token-contiguous
  uint16_t* Pt = Zt + T::ZELEMS;      // [d][ROW]  psi(K_m)^T
  uint16_t* Vt = Pt + T::PELEMS;      // [dv][ROW] V^T

  const int64_t bh = blockIdx.x / a.nmem;
  const int64_t t = blockIdx.x % a.nmem;
  const int h = (int)(bh % a.H);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, lq = lane & 31;
  const int64_t n = a.n;
  const int64_t cbeg = t * a.c;
  const int64_t cend = cbeg + a.c;  // chunks 0..nmem-1 are full
  const uint16_t* zbh = a.z + bh * n * D;
  const uint16_t* vbh = a.v + bh * n * DV;
  const float* ek = a.eta_k + h * D;
  const float* rk = a.rho_k + h * D;

  // this lane's feature in the MFMA phase
  const int f = 32 * w + lq;
  const float ekf = ek[f] * kLog2e, rkf = rk[f] * kLog2e;

  f32x16 accg[NMV], acch[NMF];
#pragma unroll
  for (int i = 0; i < NMV; ++i) accg[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < NMF; ++i) acch[i] = f32x16{};
  float mrun = kNegInf, lrun = 0.f;

  const int ntiles = (int)((a.c + kBT - 1) / kBT);
  for (int it = 0; it < ntiles; ++it) {
    const int64_t tb = cbeg + (int64_t)it * kBT;
    __syncthreads();  // previous tile's LDS reads are done
    // ---- stage Z^T and psi^T: thread b < D owns 8 tokens x 8 features
    if (tid < D) {
      const int tg = tid / FG, fg = tid % FG;
      u32x4 raw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t tok = tb + 8 * tg + i;
        raw[i] = tok < cend ? ld16(zbh + tok * D + 8 * fg) : u32x4{};
      }
      u32x4 tr[8];
      transpose8x8(raw, tr);
#pragma unroll
      for (int j = 0; j < 8; ++j) st16(Zt + (8 * fg + j) * T::ROW + 8 * tg, tr[j]);
      // memory keys of this block (log2 units) and the row softmax psi
      float e2[8], r2[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e2[j] = ek[8 * fg + j] * kLog2e;
        r2[j] = rk[8 * fg + j] * kLog2e;
      }
      u32x4 prow[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float km[8];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          km[2 * jj] = e2[2 * jj] * bf_lo(raw[i][jj]) + r2[2 * jj];
          km[2 * jj + 1] = e2[2 * jj + 1] * bf_hi(raw[i][jj]) + r2[2 * jj + 1];
        }
        float mx = km[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, km[j]);
        mx = group_max<FG>(mx);
        float sm = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          km[j] = exp2_fast(km[j] - mx);
          sm += km[j];
        }
        sm = group_sum<FG>(sm);
        const float inv = 1.f / sm;
        prow[i] = u32x4{pack2(km[0] * inv, km[1] * inv), pack2(km[2] * inv, km[3] * inv),
                        pack2(km[4] * inv, km[5] * inv), pack2(km[6] * inv, km[7] * inv)};
      }
      transpose8x8(prow, tr);
#pragma unroll
      for (int j = 0; j < 8; ++j) st16(Pt + (8 * fg + j) * T::ROW + 8 * tg, tr[j]);
    }
    // ---- stage V^T: 8x8 blocks spread over all threads
    for (int b = (tid + D) % (2 * D); b < DV; b += 2 * D) {
      const int vtg = b / VG, vg = b % VG;
      u32x4 raw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t tok = tb + 8 * vtg + i;
        raw[i] = tok < cend ? ld16(vbh + tok * DV + 8 * vg) : u32x4{};
      }
      u32x4 tr[8];
      transpose8x8(raw, tr);
#pragma unroll
      for (int j = 0; j < 8; ++j) st16(Vt + (8 * vg + j) * T::ROW + 8 * vtg, tr[j]);
    }
    __syncthreads();

    // ---- E fragments for feature f: tokens 16 ks + 8 g + [0, 8)
    float km[32];
    float tmax = kNegInf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 zr = ld16(Zt + f * T::ROW + 16 * ks + 8 * g);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        km[8 * ks + 2 * jj] = ekf * bf_lo(zr[jj]) + rkf;
        km[8 * ks + 2 * jj + 1] = ekf * bf_hi(zr[jj]) + rkf;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (tb + 16 * ks + 8 * g + i >= cend) km[8 * ks + i] = kNegInf;
        tmax = fmaxf(tmax, km[8 * ks + i]);
      }
    }
    tmax = fmaxf(tmax, wave_xor32(tmax));
    const float mnew = fmaxf(mrun, tmax);
    if (__any(mnew > mrun + kLazy)) {
      const float alpha = (mnew == kNegInf) ? 1.f : exp2_fast(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int i = 0; i < NMV; ++i) accg[i] *= alpha;
#pragma unroll
      for (int i = 0; i < NMF; ++i) acch[i] *= alpha;
      mrun = mnew;
    }
    const float msub = (mrun == kNegInf) ? 0.f : mrun;
    u32x4 ef[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = exp2_fast(km[8 * ks + i] - msub);
        lrun += e[i];
      }
      ef[ks] = u32x4{pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mv = 0; mv < NMV; ++mv) {
        const u32x4 af = ld16(Vt + (32 * mv + lq) * T::ROW + 16 * ks + 8 * g);
        accg[mv] = mfma_bf16(af, ef[ks], accg[mv]);
      }
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf) {
        const u32x4 af = ld16(Pt + (32 * mf + lq) * T::ROW + 16 * ks + 8 * g);
        acch[mf] = mfma_bf16(af, ef[ks], acch[mf]);
      }
    }
  }

  const float ltot = lrun + wave_xor32(lrun);
  const int64_t row = bh * a.nmem + t;
  if (g == 0) {
    a.cmax[row * D + f] = mrun;
    a.csum[row * D + f] = ltot;
  }
  // accumulator (block, r): column f, row 8 (r >> 2) + 4 g + (r & 3) of the block
  float* gt = a.g + row * (int64_t)NMV * D * 32;
#pragma unroll
  for (int mv = 0; mv < NMV; ++mv)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 val{accg[mv][4 * q], accg[mv][4 * q + 1], accg[mv][4 * q + 2], accg[mv][4 * q + 3]};
      *reinterpret_cast<f32x4*>(gt + ((int64_t)mv * D + f) * 32 + 8 * q + 4 * g) = val;
    }
  uint16_t* ht = a.hm + row * (int64_t)D * D + (int64_t)f * D;
#pragma unroll
  for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x2 val{pack2(acch[mf][4 * q], acch[mf][4 * q + 1]), pack2(acch[mf][4 * q + 2], acch[mf][4 * q + 3])};
      *reinterpret_cast<u32x2*>(ht + 32 * mf + 8 * q + 4 * g) = val;
    }
}

// ---------------------------------------------------------------- z prefix
// One thread per (batch*head, feature): running z^t = 2^M L in log2 space.
__global__ void awm_zscan_kernel(const float* cmax, const float* csum, float* decay, float* wscale,
                                 int64_t nmem, int D) {
  const int64_t bh = blockIdx.x;
  const int f = threadIdx.x;
  if (f >= D) return;
  float M = kNegInf, L = 0.f;
  const int64_t base = bh * nmem * D + f;
  for (int64_t t = 0; t < nmem; ++t) {
    const float m = cmax[base + t * D];
    const float l = csum[base + t * D];
    const float Mn = fmaxf(M, m);
    const float old = (M == kNegInf) ? 0.f : L * exp2_fast(M - Mn);
    const float cur = l * exp2_fast(m - Mn);
    const float Ln = old + cur;
    decay[base + t * D] = old / Ln;              // z^{t-1} / z^t
    wscale[base + t * D] = exp2_fast(m - Mn) / Ln;  // 2^{m_t} / z^t
    M = Mn;
    L = Ln;
  }
}

// ---------------------------------------------------------------- scan
struct ScanArgs {
  const float* g;
  const uint16_t* hm;
  const float* decay;
  const float* wscale;
  uint16_t* snap;  // [bh][t][dv][d]
  int64_t nmem;
  int no_delta;    // drop the H_t M' term (test variant)
};

// One workgroup per (batch*head, 32-column slice of M'). Wave w keeps rows
// [32 w, 32 w + 32) of the slice in fp32 registers (MFMA accumulator layout);
// a bf16 copy of the whole slice goes through LDS each step as the B operand
// of H_t M' and is written out as the snapshot that chunk t + 2 reads.
template <int D, int DV>
__global__ __launch_bounds__(2 * D, 1) void awm_scan_bf16_kernel(ScanArgs a) {
  constexpr int NMV = DV / 32;
  constexpr int KS = D / 16;
  constexpr int MROW = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t mt[2][32 * MROW];

  const int64_t bh = blockIdx.x / NMV;
  const int j = (int)(blockIdx.x % NMV);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, lq = lane & 31;
  const int64_t nmem = a.nmem;

  f32x16 mst = f32x16{};
  // operands of step t, loaded one step ahead
  u32x4 hf[KS];
  float gv[16], dc[16], ws[16];
  auto load_step = [&](int64_t t, u32x4 (&hq)[KS], float (&gq)[16], float (&dq)[16], float (&wq)[16]) {
    const int64_t row = bh * nmem + t;
    const uint16_t* ht = a.hm + row * (int64_t)D * D + (int64_t)(32 * w + lq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) hq[ks] = ld16(ht + 16 * ks + 8 * g);
    const float* gt = a.g + ((row * NMV + j) * D) * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int fr = 32 * w + 8 * (r >> 2) + 4 * g + (r & 3);
      gq[r] = gt[(int64_t)fr * 32 + lq];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int fr = 32 * w + 8 * q + 4 * g;
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(a.decay + row * D + fr);
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(a.wscale + row * D + fr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dq[4 * q + i] = d4[i];
        wq[4 * q + i] = w4[i];
      }
    }
  };

  load_step(0, hf, gv, dc, ws);
  int buf = 0;
  for (int64_t t = 0; t < nmem; ++t) {
    u32x4 hn[KS];
    float gn[16], dn[16], wn[16];
    if (t + 1 < nmem) load_step(t + 1, hn, gn, dn, wn);

    f32x16 p0 = f32x16{}, p1 = f32x16{};
    if (t > 0 && !a.no_delta) {
#pragma unroll
      for (int ks = 0; ks < KS; ks += 2) {
        p0 = mfma_bf16(hf[ks], ld16(&mt[buf][lq * MROW + 16 * ks + 8 * g]), p0);
        p1 = mfma_bf16(hf[ks + 1], ld16(&mt[buf][lq * MROW + 16 * (ks + 1) + 8 * g]), p1);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) mst[r] = dc[r] * mst[r] + ws[r] * (gv[r] - (p0[r] + p1[r]));
    // bf16 copy: row v = lq of the slice, features 32 w + 8 q + 4 g + [0, 4)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x2 pk{pack2(mst[4 * q], mst[4 * q + 1]), pack2(mst[4 * q + 2], mst[4 * q + 3])};
      *reinterpret_cast<u32x2*>(&mt[buf ^ 1][lq * MROW + 32 * w + 8 * q + 4 * g]) = pk;
    }
    __syncthreads();
    // snapshot rows 32 j .. 32 j + 31 of M'_{t+2}^T
    uint16_t* sn = a.snap + ((bh * nmem + t) * DV + 32 * j) * D;
    for (int e = tid; e < 32 * D / 8; e += 2 * D) {
      const int r = e / (D / 8), cc = (e % (D / 8)) * 8;
      st16(sn + (int64_t)r * D + cc, ld16(&mt[buf ^ 1][r * MROW + cc]));
    }
    buf ^= 1;
    if (t + 1 < nmem) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) hf[ks] = hn[ks];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        gv[r] = gn[r];
        dc[r] = dn[r];
        ws[r] = wn[r];
      }
    }
  }
}

template <int D, int DV>
hipError_t launch_chunk(const ChunkArgs& a, int64_t BH, hipStream_t s) {
  auto kern = awm_chunk_bf16_kernel<D, DV>;
  const size_t lds = ChunkTile<D, DV>::LDS_BYTES;
  if (lds > 65536) {
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(BH * a.nmem)), dim3(ChunkTile<D, DV>::THREADS), lds, s, a);
  return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_scan(const ScanArgs& a, int64_t BH, hipStream_t s) {
  hipLaunchKernelGGL((awm_scan_bf16_kernel<D, DV>), dim3((unsigned)(BH * (DV / 32))), dim3(2 * D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_awm_chunk_bf16(const Problem& p, const Workspace& w, hipStream_t s) {
  ChunkArgs a;
  a.z = static_cast<const uint16_t*>(p.z);
  a.v = static_cast<const uint16_t*>(p.v);
  a.eta_k = p.eta_k; a.rho_k = p.rho_k;
  a.g = w.g; a.hm = static_cast<uint16_t*>(w.h); a.cmax = w.cmax; a.csum = w.csum;
  a.n = p.n; a.c = p.c; a.nmem = p.nmem; a.H = (int)p.H;
  const int64_t BH = p.B * p.H;
  if (p.d == 128 && p.dv == 256) return launch_chunk<128, 256>(a, BH, s);
  if (p.d == 128 && p.dv == 128) return launch_chunk<128, 128>(a, BH, s);
  if (p.d == 64 && p.dv == 128) return launch_chunk<64, 128>(a, BH, s);
  if (p.d == 64 && p.dv == 64) return launch_chunk<64, 64>(a, BH, s);
  return hipErrorInvalidValue;
}

hipError_t launch_awm_zscan(const Problem& p, const Workspace& w, hipStream_t s) {
  const int64_t BH = p.B * p.H;
  hipLaunchKernelGGL(awm_zscan_kernel, dim3((unsigned)BH), dim3(128), 0, s, w.cmax, w.csum, w.decay,
                     w.wscale, p.nmem, (int)p.d);
  return hipGetLastError();
}

hipError_t launch_awm_scan_bf16(const Problem& p, const Workspace& w, hipStream_t s) {
  ScanArgs a;
  a.g = w.g; a.hm = static_cast<const uint16_t*>(w.h); a.decay = w.decay; a.wscale = w.wscale;
  a.snap = static_cast<uint16_t*>(w.snap); a.nmem = p.nmem;
  a.no_delta = (p.flags & GECKO_AWM_NO_DELTA_BIT) ? 1 : 0;
  const int64_t BH = p.B * p.H;
  if (p.d == 128 && p.dv == 256) return launch_scan<128, 256>(a, BH, s);
  if (p.d == 128 && p.dv == 128) return launch_scan<128, 128>(a, BH, s);
  if (p.d == 64 && p.dv == 128) return launch_scan<64, 128>(a, BH, s);
  if (p.d == 64 && p.dv == 64) return launch_scan<64, 64>(a, BH, s);
  return hipErrorInvalidValue;
}

}  // namespace gecko
