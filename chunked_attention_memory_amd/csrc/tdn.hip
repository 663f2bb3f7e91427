// Timestep decay normalisation (TDN) on gfx950.
//
// Per group g of F = D / G consecutive features of token t (Gecko summary on
// paper.rainbus.top, "Novelty"; paperlayer.ai summary, 2.2 and 3.1):
//   mu_t, s2_t = mean and variance of the token's values in the group
//   m_t = b1 m_{t-1} + (1 - b1) mu_t,   v_t = b2 v_{t-1} + (1 - b2) s2_t
//   m_hat = m_t / (1 - b1^t),           v_hat = v_t / (1 - b2^t)
//   y = gamma (x - m_hat) / sqrt(v_hat + eps) + shift      (per feature)
// t counts tokens of the sequence from 1; (m, v, t) may continue an earlier
// call.
//
// Four kernels, each bound by HBM traffic or latency, none by arithmetic:
//   stats: one 256-thread block per sub-chunk of 16 tokens; per token the
//     group mean and variance (two passes over registers, reduced across
//     lanes, or through LDS where a group does not fit one wave's lanes), and
//     per group the decayed sums from zero at the sub-chunk's first token,
//     written per token, with the sub-chunk's end sums;
//   chunk / carry: the same recurrence over the sub-chunk sums (decay b^16
//     per sub-chunk): chunks of them from zero in parallel, the sums entering
//     each chunk carried across chunks, then the sums entering every
//     sub-chunk, all in double;
//   apply: 8 token rows per block; each token's sums are its within-sub-chunk
//     sums plus the entering ones decayed to it, then bias correction and the
//     affine output, 16-byte loads and stores.
// x is read twice (stats, apply) and y written once.
#include <algorithm>

#include "gecko_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

template <bool kBf16>
__device__ __forceinline__ void store8(void* base, int64_t i, const float (&v)[8]) {
  if constexpr (kBf16) {
    st16(static_cast<uint16_t*>(base) + i, u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]),
                                                 pack2(v[6], v[7])});
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + i);
    p[0] = f32x4{v[0], v[1], v[2], v[3]};
    p[1] = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// Sum over aligned runs of cpg lanes (a power of two up to 64), the result in
// every lane of the run: DPP lane moves within a row of 16 lanes (swap
// neighbours, swap pairs, mirror each half-row, mirror the row: after each
// step all lanes of a run of 2, 4, 8, 16 hold the same value), then lane
// exchanges across rows.
__device__ __forceinline__ float dpp_add(float s, int ctrl_sel) {
  int t;
  const int si = __float_as_int(s);
  switch (ctrl_sel) {
    case 0: t = __builtin_amdgcn_mov_dpp(si, 0xB1, 0xF, 0xF, true); break;   // quad_perm [1, 0, 3, 2]
    case 1: t = __builtin_amdgcn_mov_dpp(si, 0x4E, 0xF, 0xF, true); break;   // quad_perm [2, 3, 0, 1]
    case 2: t = __builtin_amdgcn_mov_dpp(si, 0x141, 0xF, 0xF, true); break;  // row_half_mirror
    default: t = __builtin_amdgcn_mov_dpp(si, 0x140, 0xF, 0xF, true); break; // row_mirror
  }
  return s + __int_as_float(t);
}

__device__ __forceinline__ float run_sum(float s, int cpg) {
  if (cpg >= 2) s = dpp_add(s, 0);
  if (cpg >= 4) s = dpp_add(s, 1);
  if (cpg >= 8) s = dpp_add(s, 2);
  if (cpg >= 16) s = dpp_add(s, 3);
  for (int o = 16; o < cpg; o <<= 1) s += __shfl_xor(s, o);
  return s;
}

constexpr int kT = 256;   // threads per row block
constexpr int kR = 16;    // tokens per statistics block (one sub-chunk of the sequence)
constexpr int kGPT = 4;   // groups per thread at most (G <= D / 8 <= 1024 = kGPT kT)

// One block per sub-chunk of kR tokens of a batch row. Per token: the group
// (mean, variance) from 16-byte loads, mean then variance (two passes over
// registers); then, per group, the decayed sums from a zero start at the
// sub-chunk's first token,
//   m = b1 m + (1 - b1) mu,  v = b2 v + (1 - b2) s2   (double),
// written per token to st, and the sums after its last token to agg. Rows
// r + 1 .. r + kRing - 1 are loading while row r is reduced. kShfl: a group
// is a power-of-two run of at most 64 lanes of one wave (cpg lanes), reduced
// with lane exchanges, and its first lane keeps the group's sums: no
// barriers. Otherwise the partials go through LDS, alternating between two
// buffers by row so that three barriers per row suffice, and thread g keeps
// the sums of groups g + j kT.
constexpr int kRing = 4;

template <bool kBf16, int CPT, bool kShfl>
__global__ __launch_bounds__(kT) void tdn_stats_kernel(const void* x, float2* st, float2* agg, int64_t n,
                                                       int64_t nsub, int D, int G, float b1, float b2) {
  extern __shared__ float sm[];
  const int nch = D / 8, cpg = (D / G) / 8;  // chunks per row, per group
  const int64_t b = blockIdx.x / nsub;
  const int64_t k = blockIdx.x % nsub;
  const int64_t row0 = b * n + k * kR;  // first token row of the sub-chunk
  const int rows = (int)min((int64_t)kR, n - k * kR);
  const float invF = 1.f / (float)(D / G);
  const double d1 = b1, d2 = b2, e1 = 1.0 - d1, e2 = 1.0 - d2;
  constexpr int NS = kShfl ? CPT : kGPT;  // sums kept per thread
  double m[NS], v[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) m[j] = v[j] = 0.0;

  // raw rows in flight: loads are unconditional (lanes past the row re-read
  // its last chunk, unused) and converted where used, so the compiler keeps
  // them in flight instead of waiting inside a branch
  constexpr int RW = kBf16 ? 1 : 2;  // 16-byte words per 8-feature chunk
  auto load_row = [&](int r, u32x4 (&dst)[CPT][RW]) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = min((int)threadIdx.x + q * kT, nch - 1);
      const int64_t e = (row0 + r) * D + 8 * c;
      if constexpr (kBf16) {
        dst[q][0] = ld16(static_cast<const uint16_t*>(x) + e);
      } else {
        const u32x4* pw = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + e);
        dst[q][0] = pw[0];
        dst[q][1] = pw[1];
      }
    }
  };
  // one token row from its raw words: statistics, then the sums
  auto do_row = [&](int r, const u32x4 (&raw)[CPT][RW]) {
    float cur[CPT][8];
#pragma unroll
    for (int q = 0; q < CPT; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (kBf16) {
          const uint32_t wd = raw[q][0][j / 2];
          cur[q][j] = (j & 1) ? bf_hi(wd) : bf_lo(wd);
        } else {
          cur[q][j] = __uint_as_float(raw[q][j / 4][j % 4]);
        }
      }
    if constexpr (kShfl) {
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = threadIdx.x + q * kT;
        const bool on = c < nch;
        float s = 0.f;
        if (on) {
#pragma unroll
          for (int j = 0; j < 8; ++j) s += cur[q][j];
        }
        s = run_sum(s, cpg);
        const float mu = s * invF;
        float sq = 0.f;
        if (on) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sq = fmaf(cur[q][j] - mu, cur[q][j] - mu, sq);
        }
        sq = run_sum(sq, cpg);
        if (on && c % cpg == 0) {
          m[q] = fma(d1, m[q], e1 * (double)mu);
          v[q] = fma(d2, v[q], e2 * (double)(sq * invF));
          st[(row0 + r) * G + c / cpg] = make_float2((float)m[q], (float)v[q]);
        }
      }
    } else {
      float* part = sm + (r & 1) * nch;
      float* gmean = sm + 2 * nch + (r & 1) * G;
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = threadIdx.x + q * kT;
        if (c < nch) {
          float s = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) s += cur[q][j];
          part[c] = s;
        }
      }
      __syncthreads();
      for (int g = threadIdx.x; g < G; g += kT) {
        float s = 0.f;
        for (int i = 0; i < cpg; ++i) s += part[g * cpg + i];
        gmean[g] = s * invF;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = threadIdx.x + q * kT;
        if (c < nch) {
          const float mu = gmean[c / cpg];
          float s = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) s = fmaf(cur[q][j] - mu, cur[q][j] - mu, s);
          part[c] = s;
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kGPT; ++j) {
        const int g = threadIdx.x + j * kT;
        if (g < G) {
          float s = 0.f;
          for (int i = 0; i < cpg; ++i) s += part[g * cpg + i];
          m[j] = fma(d1, m[j], e1 * (double)gmean[g]);
          v[j] = fma(d2, v[j], e2 * (double)(s * invF));
          st[(row0 + r) * G + g] = make_float2((float)m[j], (float)v[j]);
        }
      }
    }
  };
  if (rows == kR) {
    // a whole sub-chunk: straight-line code with constant ring slots, so
    // the compiler's memory-counter waits leave kRing - 1 rows in flight
    u32x4 xr[kRing][CPT][RW];
#pragma unroll
    for (int u = 0; u + 1 < kRing; ++u) load_row(u, xr[u]);
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      if (r + kRing - 1 < kR) load_row(r + kRing - 1, xr[(r + kRing - 1) % kRing]);
      do_row(r, xr[r % kRing]);
    }
  } else {
    for (int r = 0; r < rows; ++r) {
      u32x4 one[CPT][RW];
      load_row(r, one);
      do_row(r, one);
    }
  }
  float2* ag = agg + (b * nsub + k) * G;
  if constexpr (kShfl) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = threadIdx.x + q * kT;
      if (c < nch && c % cpg == 0) ag[c / cpg] = make_float2((float)m[q], (float)v[q]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kGPT; ++j) {
      const int g = threadIdx.x + j * kT;
      if (g < G) ag[g] = make_float2((float)m[j], (float)v[j]);
    }
  }
}

// Decayed sums over the sub-chunks [c Ls, (c + 1) Ls) of row b, one thread
// per group (consecutive threads read consecutive groups). The sums after
// sub-chunk k are S_k = b^len_k S_{k-1} + agg_k, len_k its token count (kR
// but for the sequence's last). kFinal = 0 (phase A): from zero, write the
// chunk's end sums to carry[b][c][g]. kFinal = 1 (phase C): from the entering
// sums in carry[b][c][g] (phase B), replace each agg_k by the sums entering
// sub-chunk k; the last chunk also writes the final sums. In double.
template <bool kFinal>
__global__ __launch_bounds__(256) void tdn_chunk_kernel(float2* ag, float2* carry, float* m_out, float* v_out,
                                                       int64_t n, int64_t nsub, int G, int64_t Ls, int NC, float b1,
                                                       float b2) {
  const int64_t b = blockIdx.x / NC;
  const int c = (int)(blockIdx.x % NC);
  const int64_t ka = (int64_t)c * Ls, kb = std::min<int64_t>(ka + Ls, nsub);
  const double f1 = pow((double)b1, (double)kR), f2 = pow((double)b2, (double)kR);
  const double lastlen = (double)(n - (nsub - 1) * kR);
  const double l1 = pow((double)b1, lastlen), l2 = pow((double)b2, lastlen);
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    double m = 0.0, v = 0.0;
    if constexpr (kFinal) {
      const float2 e = carry[(b * NC + c) * G + g];
      m = e.x;
      v = e.y;
    }
    float2* s = ag + b * nsub * G + g;
    // kB sub-chunks per step: their loads are issued together, then the sums run
    constexpr int kB = 16;
    for (int64_t k0 = ka; k0 < kb; k0 += kB) {
      float2 a[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (k0 + u < kb) a[u] = s[(k0 + u) * G];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (k0 + u < kb) {
          if constexpr (kFinal) s[(k0 + u) * G] = make_float2((float)m, (float)v);
          const bool last = k0 + u == nsub - 1;
          m = fma(last ? l1 : f1, m, (double)a[u].x);
          v = fma(last ? l2 : f2, v, (double)a[u].y);
        }
      }
    }
    if constexpr (kFinal) {
      if (c == NC - 1) {
        if (m_out) m_out[b * G + g] = (float)m;
        if (v_out) v_out[b * G + g] = (float)v;
      }
    } else {
      carry[(b * NC + c) * G + g] = make_float2((float)m, (float)v);
    }
  }
}

// Phase B: one thread per (b, g); the sums entering each chunk, in double,
// written over the chunk end sums: enter(c + 1) = b^L enter(c) + end(c),
// L the tokens of a chunk.
__global__ void tdn_carry_kernel(float2* carry, const float* m0, const float* v0, int64_t B, int G, int64_t L,
                                 int NC, float b1, float b2) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * G) return;
  const int64_t b = i / G;
  const int g = (int)(i % G);
  const double d1 = b1 > 0.f ? pow((double)b1, (double)L) : 0.0;
  const double d2 = b2 > 0.f ? pow((double)b2, (double)L) : 0.0;
  double m = m0 ? m0[i] : 0.0, v = v0 ? v0[i] : 0.0;
  // the last chunk's end sums are not needed; the others are read 16 at a time
  constexpr int kB = 16;
  for (int c0 = 0; c0 < NC; c0 += kB) {
    float2 end[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (c0 + k < NC - 1) end[k] = carry[(b * NC + c0 + k) * G + g];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      if (c0 + k < NC) {
        carry[(b * NC + c0 + k) * G + g] = make_float2((float)m, (float)v);
        if (c0 + k < NC - 1) {
          m = d1 * m + end[k].x;
          v = d2 * v + end[k].y;
        }
      }
    }
  }
}

constexpr int kRows = 8;  // token rows per apply block (gamma and shift stay in registers)

// y for kRows token rows. Token t of row b, i = t mod kR tokens into its
// sub-chunk k: the sums are m = st_t + b1^(i+1) enter_k (v alike), and with
// tau = t0 + t + 1 tokens of the sequence so far, m_hat = m / (1 - b1^tau),
// v_hat = v / (1 - b2^tau); 1 - b^tau is -expm1(tau ln b), accurate for b
// near 1.
template <bool kIn, bool kOut, int CPT>
__global__ __launch_bounds__(kT) void tdn_apply_kernel(const void* x, const float2* st, const float2* ent,
                                                       const float* gamma, const float* shift, void* y, int64_t n,
                                                       int64_t nsub, int64_t rows, int D, int G, int64_t t0,
                                                       float b1, float b2, float eps) {
  const int nch = D / 8, cpg = (D / G) / 8;
  float gm[CPT][8], sh[CPT][8];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = min((int)threadIdx.x + k * kT, nch - 1);
    const f32x4* gp = reinterpret_cast<const f32x4*>(gamma + 8 * c);
    const f32x4* sp = reinterpret_cast<const f32x4*>(shift + 8 * c);
    const f32x4 g0 = gp[0], g1 = gp[1], s0 = sp[0], s1 = sp[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      gm[k][j] = g0[j];
      gm[k][4 + j] = g1[j];
      sh[k][j] = s0[j];
      sh[k][4 + j] = s1[j];
    }
  }
  const float lg1 = log2f(b1), lg2 = log2f(b2);  // -inf at b = 0
  const float ln1 = logf(b1), ln2 = logf(b2);
  constexpr int RW = kIn ? 1 : 2;  // 16-byte words per 8-feature chunk
  // kA rows at a time: every load of the batch is issued before the first
  // is used (unconditional loads: lanes past the row re-read its last chunk,
  // unused), so the compiler's memory-counter waits keep them in flight
  constexpr int kA = 4;
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  const int64_t r1 = min(r0 + kRows, rows);
  for (int64_t ra = r0; ra < r1; ra += kA) {
    const int na = (int)min((int64_t)kA, r1 - ra);
    u32x4 raw[kA][CPT][RW];
    float2 sv[kA][CPT], ev[kA][CPT];
    int64_t tok[kA];
#pragma unroll
    for (int u = 0; u < kA; ++u) {
      const int64_t row = ra + min(u, na - 1);
      const int64_t b = row / n, t = row - b * n;
      tok[u] = t;
      const float2* ek = ent + (b * nsub + t / kR) * G;
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = min((int)threadIdx.x + q * kT, nch - 1);
        const int64_t e = row * D + 8 * c;
        if constexpr (kIn) {
          raw[u][q][0] = ld16(static_cast<const uint16_t*>(x) + e);
        } else {
          const u32x4* pw = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + e);
          raw[u][q][0] = pw[0];
          raw[u][q][1] = pw[1];
        }
        sv[u][q] = st[row * G + c / cpg];
        ev[u][q] = ek[c / cpg];
      }
    }
#pragma unroll
    for (int u = 0; u < kA; ++u) {
      if (u >= na) break;
      const int64_t row = ra + u, t = tok[u];
      const float i1 = (float)(t % kR + 1);
      const float p1 = exp2f(lg1 * i1), p2 = exp2f(lg2 * i1);
      const float tau = (float)(t0 + t + 1);
      const float iu1 = 1.f / -expm1f(tau * ln1), iu2 = 1.f / -expm1f(tau * ln2);
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = threadIdx.x + q * kT;
        if (c < nch) {
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if constexpr (kIn) {
              const uint32_t wd = raw[u][q][0][j / 2];
              v[j] = (j & 1) ? bf_hi(wd) : bf_lo(wd);
            } else {
              v[j] = __uint_as_float(raw[u][q][j / 4][j % 4]);
            }
          }
          const float mh = fmaf(p1, ev[u][q].x, sv[u][q].x) * iu1;
          const float rs = rsqrtf(fmaf(p2, ev[u][q].y, sv[u][q].y) * iu2 + eps);
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = fmaf(gm[q][j] * rs, v[j] - mh, sh[q][j]);
          store8<kOut>(y, row * D + 8 * c, v);
        }
      }
    }
  }
}

template <bool kIn, bool kOut, int CPT>
hipError_t launch_cpt(const TdnProblem& p, char* ws, hipStream_t s) {
  const TdnPlan pl = tdn_plan(p.B, p.n, p.G);
  float2* st = reinterpret_cast<float2*>(ws);
  float2* sub = reinterpret_cast<float2*>(ws + pl.off_sub);
  float2* carry = reinterpret_cast<float2*>(ws + pl.off_carry);
  const int64_t cpg = p.D / p.G / 8;
  const dim3 sgrid((unsigned)(p.B * pl.nsub));
  if (cpg <= 64 && (cpg & (cpg - 1)) == 0) {
    hipLaunchKernelGGL((tdn_stats_kernel<kIn, CPT, true>), sgrid, dim3(kT), 0, s, p.x, st, sub, p.n, pl.nsub,
                       (int)p.D, (int)p.G, p.beta1, p.beta2);
  } else {
    const size_t lds = (size_t)(2 * (p.D / 8) + 2 * p.G) * sizeof(float);
    hipLaunchKernelGGL((tdn_stats_kernel<kIn, CPT, false>), sgrid, dim3(kT), lds, s, p.x, st, sub, p.n, pl.nsub,
                       (int)p.D, (int)p.G, p.beta1, p.beta2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // scan over the sub-chunk sums: chunks of Ls sub-chunks in parallel,
  // carries across chunks
  const unsigned blocks = (unsigned)(p.B * pl.NC);
  const unsigned cthreads = (unsigned)std::min<int64_t>(256, (p.G + 63) / 64 * 64);  // one thread per group
  if (pl.NC > 1) {
    hipLaunchKernelGGL((tdn_chunk_kernel<false>), dim3(blocks), dim3(cthreads), 0, s, sub, carry, p.m_out, p.v_out,
                       p.n, pl.nsub, (int)p.G, pl.Ls, (int)pl.NC, p.beta1, p.beta2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {  // with one chunk this only writes the given (or zero) sums as its entering ones
    const int64_t th = p.B * p.G;
    hipLaunchKernelGGL(tdn_carry_kernel, dim3((unsigned)((th + 255) / 256)), dim3(256), 0, s, carry, p.m0, p.v0,
                       p.B, (int)p.G, pl.Ls * kR, (int)pl.NC, p.beta1, p.beta2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((tdn_chunk_kernel<true>), dim3(blocks), dim3(cthreads), 0, s, sub, carry, p.m_out, p.v_out, p.n,
                     pl.nsub, (int)p.G, pl.Ls, (int)pl.NC, p.beta1, p.beta2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t rows = p.B * p.n;
  hipLaunchKernelGGL((tdn_apply_kernel<kIn, kOut, CPT>), dim3((unsigned)((rows + kRows - 1) / kRows)), dim3(kT), 0,
                     s, p.x, st, sub, p.gamma, p.shift, p.y, p.n, pl.nsub, rows, (int)p.D, (int)p.G, p.t0, p.beta1,
                     p.beta2, p.eps);
  return hipGetLastError();
}

template <bool kIn, bool kOut>
hipError_t launch_io(const TdnProblem& p, char* ws, hipStream_t s) {
  const int64_t cpt = (p.D / 8 + kT - 1) / kT;
  if (cpt <= 1) return launch_cpt<kIn, kOut, 1>(p, ws, s);
  if (cpt <= 2) return launch_cpt<kIn, kOut, 2>(p, ws, s);
  return launch_cpt<kIn, kOut, 4>(p, ws, s);
}

}  // namespace

TdnPlan tdn_plan(int64_t B, int64_t n, int64_t G) {
  TdnPlan p{};
  p.nsub = (n + kR - 1) / kR;
  // about sqrt(nsub) chunks of as many sub-chunks: the two chunk passes and
  // the carry each run that many dependent steps
  int64_t nc = 1;
  while ((nc + 1) * (nc + 1) <= p.nsub) ++nc;
  p.Ls = (p.nsub + nc - 1) / nc;
  p.NC = (p.nsub + p.Ls - 1) / p.Ls;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t stats = (size_t)B * (size_t)n * (size_t)G * sizeof(float2);
  p.off_sub = up(stats);
  p.off_carry = up(p.off_sub + (size_t)B * (size_t)p.nsub * (size_t)G * sizeof(float2));
  p.bytes = p.off_carry + (size_t)B * (size_t)p.NC * (size_t)G * sizeof(float2);
  return p;
}

hipError_t launch_tdn(const TdnProblem& p, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  if (p.in_bf16) return p.out_bf16 ? launch_io<true, true>(p, w, s) : launch_io<true, false>(p, w, s);
  return p.out_bf16 ? launch_io<false, true>(p, w, s) : launch_io<false, false>(p, w, s);
}

}  // namespace gecko
