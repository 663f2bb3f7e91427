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
// Three kernels, each bound by HBM traffic or latency, none by arithmetic:
//   stats: one 256-thread block per token row; 16-byte loads of 8 features,
//     per-group mean then variance (two passes over registers) through LDS;
//   scan: the tokens cut into chunks; one thread per (batch, chunk, group)
//     computes the chunk's decayed sums from zero, the sums entering each
//     chunk are carried across chunks (b^L per chunk), and a second pass from
//     the entering sums writes (m_hat, 1 / sqrt(v_hat + eps)) in place of the
//     statistics; the sums run in double (1 - b^t by its own recurrence);
//   apply: one block per token row, 16-byte loads and stores.
#include <algorithm>

#include "gecko_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

template <bool kBf16>
__device__ __forceinline__ void load8(const void* base, int64_t i, float (&v)[8]) {
  if constexpr (kBf16) {
    const u32x4 r = ld16(static_cast<const uint16_t*>(base) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf_lo(r[j]);
      v[2 * j + 1] = bf_hi(r[j]);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
}

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

constexpr int kT = 256;  // threads per row block

// stats[(b n + t) G + g] = (mean, variance) of the group. CPT 8-feature
// chunks per thread (D <= 8 CPT kT); part holds one partial per chunk.
template <bool kBf16, int CPT>
__global__ __launch_bounds__(kT) void tdn_stats_kernel(const void* x, float2* stats, int D, int G) {
  extern __shared__ float sm[];
  float* part = sm;              // [D / 8]
  float* gmean = sm + D / 8;     // [G]
  const int64_t row = blockIdx.x;
  const int nch = D / 8, cpg = (D / G) / 8;  // chunks per row, per group
  const float invF = 1.f / (float)(D / G);
  float v[CPT][8];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = threadIdx.x + k * kT;
    if (c < nch) {
      load8<kBf16>(x, row * D + 8 * c, v[k]);
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) s += v[k][j];
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
  for (int k = 0; k < CPT; ++k) {
    const int c = threadIdx.x + k * kT;
    if (c < nch) {
      const float mu = gmean[c / cpg];
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) s = fmaf(v[k][j] - mu, v[k][j] - mu, s);
      part[c] = s;
    }
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += kT) {
    float s = 0.f;
    for (int i = 0; i < cpg; ++i) s += part[g * cpg + i];
    stats[row * G + g] = make_float2(gmean[g], s * invF);
  }
}

// Decayed statistics over the tokens of chunk c of row b, one thread per
// group (consecutive threads read consecutive groups of a token). kFinal = 0
// (phase A): from zero, write the chunk's end sums to carry[b][c][g].
// kFinal = 1 (phase C): from the entering sums in carry[b][c][g] (phase B),
// replace each token's (mean, variance) by (m_hat, 1 / sqrt(v_hat + eps));
// the last chunk also writes the final sums.
template <bool kFinal>
__global__ __launch_bounds__(256) void tdn_chunk_kernel(float2* st, float2* carry, const float* m0, const float* v0,
                                                       float* m_out, float* v_out, int64_t n, int G, int64_t L,
                                                       int NC, int64_t t0, float b1, float b2, float eps) {
  const int64_t b = blockIdx.x / NC;
  const int c = (int)(blockIdx.x % NC);
  const int64_t ta = (int64_t)c * L, tb = std::min<int64_t>(ta + L, n);
  // The sums run in double: with b near 1 a float32 sum settles about
  // 2^-25 / (1 - b) away from its exact value (3e-4 relative at b = 0.9999).
  // 1 - b^t follows u_t = b u_{t-1} + (1 - b) and runs beside them, from its
  // value before the chunk.
  const double d1 = b1, d2 = b2, e1 = 1.0 - d1, e2 = 1.0 - d2;
  const double tp = (double)(t0 + ta);  // tokens of the sequence before the chunk
  const double u1s = tp > 0.0 ? -expm1(tp * log(d1)) : 0.0, u2s = tp > 0.0 ? -expm1(tp * log(d2)) : 0.0;
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    double m = 0.0, v = 0.0, u1 = u1s, u2 = u2s;
    if constexpr (kFinal) {
      const float2 e = carry[(b * NC + c) * G + g];
      m = e.x;
      v = e.y;
    }
    float2* s = st + b * n * G + g;
    // kB tokens per step: their loads are issued together, then the sums run
    constexpr int kB = 16;
    int64_t t = ta;
    for (; t + kB <= tb; t += kB) {
      float2 x[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) x[k] = s[(t + k) * G];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        m = fma(d1, m, e1 * x[k].x);
        v = fma(d2, v, e2 * x[k].y);
        if constexpr (kFinal) {
          u1 = fma(d1, u1, e1);
          u2 = fma(d2, u2, e2);
          s[(t + k) * G] = make_float2((float)(m / u1), rsqrtf((float)(v / u2) + eps));
        }
      }
    }
    for (; t < tb; ++t) {
      const float2 x = s[t * G];
      m = fma(d1, m, e1 * x.x);
      v = fma(d2, v, e2 * x.y);
      if constexpr (kFinal) {
        u1 = fma(d1, u1, e1);
        u2 = fma(d2, u2, e2);
        s[t * G] = make_float2((float)(m / u1), rsqrtf((float)(v / u2) + eps));
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
// written over the chunk end sums: enter(c + 1) = b^L enter(c) + end(c).
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

template <bool kIn, bool kOut, int CPT>
__global__ __launch_bounds__(kT) void tdn_apply_kernel(const void* x, const float2* nrm, const float* gamma,
                                                       const float* shift, void* y, int64_t rows, int D, int G) {
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
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  const int64_t r1 = min(r0 + kRows, rows);
  for (int64_t row = r0; row < r1; ++row) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = threadIdx.x + k * kT;
      if (c < nch) {
        float v[8];
        load8<kIn>(x, row * D + 8 * c, v);
        const float2 q = nrm[row * G + c / cpg];  // (m_hat, 1 / sqrt(v_hat + eps))
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = fmaf(gm[k][j] * q.y, v[j] - q.x, sh[k][j]);
        store8<kOut>(y, row * D + 8 * c, v);
      }
    }
  }
}

template <bool kIn, bool kOut, int CPT>
hipError_t launch_cpt(const TdnProblem& p, float2* st, hipStream_t s) {
  const unsigned rows = (unsigned)(p.B * p.n);
  const size_t lds = (size_t)(p.D / 8 + p.G) * sizeof(float);
  hipLaunchKernelGGL((tdn_stats_kernel<kIn, CPT>), dim3(rows), dim3(kT), lds, s, p.x, st, (int)p.D, (int)p.G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // statistics scan: chunks of L tokens in parallel, carries across chunks
  const TdnPlan pl = tdn_plan(p.B, p.n, p.G);
  float2* carry = reinterpret_cast<float2*>(reinterpret_cast<char*>(st) + pl.off_carry);
  const unsigned blocks = (unsigned)(p.B * pl.NC);
  const unsigned cthreads = (unsigned)std::min<int64_t>(256, (p.G + 63) / 64 * 64);  // one thread per group
  if (pl.NC > 1) {
    hipLaunchKernelGGL((tdn_chunk_kernel<false>), dim3(blocks), dim3(cthreads), 0, s, st, carry, p.m0, p.v0, p.m_out,
                       p.v_out, p.n, (int)p.G, pl.L, (int)pl.NC, p.t0, p.beta1, p.beta2, p.eps);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {  // with one chunk this only writes the given (or zero) sums as its entering ones
    const int64_t th = p.B * p.G;
    hipLaunchKernelGGL(tdn_carry_kernel, dim3((unsigned)((th + 255) / 256)), dim3(256), 0, s, carry, p.m0, p.v0,
                       p.B, (int)p.G, pl.L, (int)pl.NC, p.beta1, p.beta2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((tdn_chunk_kernel<true>), dim3(blocks), dim3(cthreads), 0, s, st, carry, p.m0, p.v0, p.m_out,
                     p.v_out, p.n, (int)p.G, pl.L, (int)pl.NC, p.t0, p.beta1, p.beta2, p.eps);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((tdn_apply_kernel<kIn, kOut, CPT>), dim3((unsigned)((rows + kRows - 1) / kRows)), dim3(kT), 0,
                     s, p.x, st, p.gamma, p.shift, p.y, (int64_t)rows, (int)p.D, (int)p.G);
  return hipGetLastError();
}

template <bool kIn, bool kOut>
hipError_t launch_io(const TdnProblem& p, float2* st, hipStream_t s) {
  const int64_t cpt = (p.D / 8 + kT - 1) / kT;
  if (cpt <= 1) return launch_cpt<kIn, kOut, 1>(p, st, s);
  if (cpt <= 2) return launch_cpt<kIn, kOut, 2>(p, st, s);
  return launch_cpt<kIn, kOut, 4>(p, st, s);
}

}  // namespace

TdnPlan tdn_plan(int64_t B, int64_t n, int64_t G) {
  TdnPlan p{};
  // chunks of at least 512 tokens; up to 2048 blocks in all
  const int64_t want = std::max<int64_t>(1, 2048 / B);
  p.NC = std::max<int64_t>(1, std::min(want, n / 512));
  p.L = (n + p.NC - 1) / p.NC;
  p.NC = (n + p.L - 1) / p.L;
  const size_t stats = (size_t)B * (size_t)n * (size_t)G * sizeof(float2);
  p.off_carry = (stats + 255) / 256 * 256;
  p.bytes = p.off_carry + (size_t)B * (size_t)p.NC * (size_t)G * sizeof(float2);
  return p;
}

hipError_t launch_tdn(const TdnProblem& p, void* ws, hipStream_t s) {
  float2* st = static_cast<float2*>(ws);
  if (p.in_bf16) return p.out_bf16 ? launch_io<true, true>(p, st, s) : launch_io<true, false>(p, st, s);
  return p.out_bf16 ? launch_io<false, true>(p, st, s) : launch_io<false, false>(p, st, s);
}

}  // namespace gecko
