// float32 path of the forward: plain vector-ALU kernels (no MFMA), written
// for the tight-tolerance workloads (small d, dv and c). Same decomposition as
// the bf16 path (chunk pass, log2-space denominator prefix shared with it,
// sequential state scan, attention with the readout in its epilogue). Stored
// intermediates are float32; long sums are accumulated in double.
//
// Source of the arithmetic: the Gecko summary on paper.rainbus.top, "Method
// steps" (2)-(5) and "Core method"; initial state M'_1 = 0 from the
// paperlayer.ai summary, Appendix A.
#include "gecko_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

// per-token (max, sum) of the memory-key row in log2 units, for psi(K_m)
// (Grids are one-dimensional, block = (batch*head, part): the y and z grid
// dimensions stop at 65535.)
__global__ void f32_rowstat_kernel(const float* z, const float* eta_k, const float* rho_k, float* rowstat,
                                   int64_t n, int64_t ntok, int d, int H, int64_t nblk) {
  const int64_t bh = blockIdx.x / nblk;
  const int64_t i = (int64_t)(blockIdx.x % nblk) * blockDim.x + threadIdx.x;
  if (i >= ntok) return;
  const int h = (int)(bh % H);
  const float* zr = z + (bh * n + i) * d;
  float mx = kNegInf;
  for (int f = 0; f < d; ++f) mx = fmaxf(mx, (eta_k[h * d + f] * zr[f] + rho_k[h * d + f]) * kLog2e);
  float sm = 0.f;
  for (int f = 0; f < d; ++f) sm += exp2_fast((eta_k[h * d + f] * zr[f] + rho_k[h * d + f]) * kLog2e - mx);
  rowstat[(bh * n + i) * 2] = mx;
  rowstat[(bh * n + i) * 2 + 1] = sm;
}

// per (bh, chunk t, feature f): max over the chunk of K_m (log2) and the sum of
// 2^(K_m - max)
__global__ void f32_colstat_kernel(const float* z, const float* eta_k, const float* rho_k, float* cmax,
                                   float* csum, int64_t n, int64_t c, int64_t nmem, int d, int H) {
  const int64_t row = blockIdx.x;  // bh * nmem + t
  const int64_t bh = row / nmem, t = row % nmem;
  const int f = threadIdx.x;
  if (f >= d) return;
  const int h = (int)(bh % H);
  const float e = eta_k[h * d + f] * kLog2e, r = rho_k[h * d + f] * kLog2e;
  const float* zc = z + (bh * n + t * c) * d + f;
  float mx = kNegInf;
  for (int64_t i = 0; i < c; ++i) mx = fmaxf(mx, e * zc[i * d] + r);
  float sm = 0.f;
  for (int64_t i = 0; i < c; ++i) sm += exp2_fast(e * zc[i * d] + r - mx);
  cmax[row * d + f] = mx;
  csum[row * d + f] = sm;
}

// G[f][x] = sum_i E[i][f] V[i][x] and H[f][f'] = sum_i E[i][f] psi(K_m)[i][f'],
// one thread per output element of one chunk.
__global__ void f32_products_kernel(const float* z, const float* v, const float* eta_k, const float* rho_k,
                                    const float* rowstat, const float* cmax, float* gout, float* hout,
                                    int64_t n, int64_t c, int64_t nmem, int d, int dv, int H, int64_t nblk) {
  const int64_t row = blockIdx.x / nblk;  // bh * nmem + t
  const int64_t bh = row / nmem, t = row % nmem;
  const int h = (int)(bh % H);
  const int64_t e = (int64_t)(blockIdx.x % nblk) * blockDim.x + threadIdx.x;
  const int width = dv + d;
  if (e >= (int64_t)d * width) return;
  const int f = (int)(e / width), x = (int)(e % width);
  const float ef = eta_k[h * d + f] * kLog2e, rf = rho_k[h * d + f] * kLog2e;
  const float m = cmax[row * d + f];
  const int64_t t0 = t * c;
  double acc = 0.0;
  if (x < dv) {
    for (int64_t i = 0; i < c; ++i) {
      const int64_t tok = bh * n + t0 + i;
      acc += exp2_fast(ef * z[tok * d + f] + rf - m) * v[tok * dv + x];
    }
    // same layout as the bf16 path: [t][x / 32][f][x % 32]
    gout[((row * (dv / 32) + x / 32) * d + f) * 32 + (x % 32)] = (float)acc;
  } else {
    const int fp = x - dv;
    const float ep = eta_k[h * d + fp] * kLog2e, rp = rho_k[h * d + fp] * kLog2e;
    for (int64_t i = 0; i < c; ++i) {
      const int64_t tok = bh * n + t0 + i;
      const float psi = exp2_fast(ep * z[tok * d + fp] + rp - rowstat[tok * 2]) / rowstat[tok * 2 + 1];
      acc += exp2_fast(ef * z[tok * d + f] + rf - m) * psi;
    }
    hout[(row * d + f) * d + fp] = (float)acc;
  }
}

// One workgroup per bh; the state lives in the snapshot slots ([t][dv][d]).
__global__ void f32_scan_kernel(const float* g, const float* hm, const float* decay, const float* wscale,
                                float* snap, int64_t nmem, int d, int dv, int no_delta) {
  const int64_t bh = blockIdx.x;
  const int nel = d * dv;
  for (int64_t t = 0; t < nmem; ++t) {
    const int64_t row = bh * nmem + t;
    const float* prev = t > 0 ? snap + (row - 1) * nel : nullptr;  // M'_{t+1}^T
    float* cur = snap + row * nel;                                  // M'_{t+2}^T
    for (int e = threadIdx.x; e < nel; e += blockDim.x) {
      const int x = e / d, f = e % d;  // element (f, x) of M', stored at [x][f]
      double p = 0.0, old = 0.0;
      if (prev) {
        const float* hr = hm + (row * d + f) * d;
        const float* mc = prev + (int64_t)x * d;
        if (!no_delta)
          for (int k = 0; k < d; ++k) p += (double)hr[k] * mc[k];
        old = mc[f];
      }
      const double gv = g[((row * (dv / 32) + x / 32) * d + f) * 32 + (x % 32)];
      cur[e] = (float)((double)decay[row * d + f] * old + (double)wscale[row * d + f] * (gv - p));
    }
    __syncthreads();
  }
}

// One thread per (query, 32-column slice of the output). Logits, weights and
// sums are carried in double so the float32 result is rounded once.
__global__ void f32_sca_kernel(Problem p, const float* snap, int mode, int64_t nqblk) {
  const int d = (int)p.d, dv = (int)p.dv;
  const int64_t slices = dv / 32;
  const int64_t bh = blockIdx.x / (slices * nqblk);
  const int h = (int)(bh % p.H);
  const int x0 = 32 * (int)((blockIdx.x / nqblk) % slices);
  const int64_t i = (int64_t)(blockIdx.x % nqblk) * blockDim.x + threadIdx.x;
  if (i >= p.n) return;
  const float* z = static_cast<const float*>(p.z) + bh * p.n * d;
  const float* v = static_cast<const float*>(p.v) + bh * p.n * dv;
  float* out = static_cast<float*>(p.out) + (bh * p.n + i) * dv + x0;
  const int64_t s = i / p.c;
  double acc[32];
  for (int k = 0; k < 32; ++k) acc[k] = 0.0;

  if (mode & 1) {
    double q[128];
    for (int f = 0; f < d; ++f) q[f] = (double)p.kappa_q[h * d + f] * z[i * d + f] + p.nu_q[h * d + f];
    const int64_t kbeg = (p.prev && s > 0) ? (s - 1) * p.c : s * p.c;  // previous chunk, if sliding
    double m = -__builtin_inf(), l = 0.0;
    for (int64_t j = kbeg; j <= i; ++j) {
      double logit = 0.0;
      for (int f = 0; f < d; ++f) logit += q[f] * ((double)p.kappa_k[h * d + f] * z[j * d + f] + p.nu_k[h * d + f]);
      const double mn = fmax(m, logit);
      const double alpha = exp(m - mn);  // 0 on the first key
      const double pj = exp(logit - mn);
      l = l * alpha + pj;
      for (int k = 0; k < 32; ++k) acc[k] = acc[k] * alpha + pj * v[j * dv + x0 + k];
      m = mn;
    }
    for (int k = 0; k < 32; ++k) acc[k] /= l;
  }
  if ((mode & 2) && s >= p.first_read) {  // the state after chunks <= s - lag
    double qm[128];
    double mx = -__builtin_inf();
    for (int f = 0; f < d; ++f) {
      qm[f] = (double)p.eta_q[h * d + f] * z[i * d + f] + p.rho_q[h * d + f];
      mx = fmax(mx, qm[f]);
    }
    double sm = 0.0;
    for (int f = 0; f < d; ++f) {
      qm[f] = exp(qm[f] - mx);
      sm += qm[f];
    }
    const float* sn = snap + (bh * p.nmem + (s - p.lag)) * (int64_t)dv * d;
    for (int k = 0; k < 32; ++k) {
      double r = 0.0;
      for (int f = 0; f < d; ++f) r += qm[f] * sn[(int64_t)(x0 + k) * d + f];
      acc[k] += r / sm;
    }
  }
  for (int k = 0; k < 32; ++k) out[k] = (float)acc[k];
}

}  // namespace

hipError_t launch_awm_chunk_f32(const Problem& p, const Workspace& w, hipStream_t s) {
  const int64_t BH = p.B * p.H;
  const float* z = static_cast<const float*>(p.z);
  const float* v = static_cast<const float*>(p.v);
  const int64_t ntok = p.nmem * p.c;
  const int64_t rblk = (ntok + 127) / 128;
  hipLaunchKernelGGL(f32_rowstat_kernel, dim3((unsigned)(rblk * BH)), dim3(128), 0, s,
                     z, p.eta_k, p.rho_k, w.rowstat, p.n, ntok, (int)p.d, (int)p.H, rblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(f32_colstat_kernel, dim3((unsigned)(BH * p.nmem)), dim3(128), 0, s, z, p.eta_k, p.rho_k,
                     w.cmax, w.csum, p.n, p.c, p.nmem, (int)p.d, (int)p.H);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t outs = p.d * (p.dv + p.d);
  const int64_t pblk = (outs + 255) / 256;
  hipLaunchKernelGGL(f32_products_kernel, dim3((unsigned)(pblk * BH * p.nmem)), dim3(256),
                     0, s, z, v, p.eta_k, p.rho_k, w.rowstat, w.cmax, w.g, static_cast<float*>(w.h), p.n, p.c,
                     p.nmem, (int)p.d, (int)p.dv, (int)p.H, pblk);
  return hipGetLastError();
}

hipError_t launch_awm_scan_f32(const Problem& p, const Workspace& w, hipStream_t s) {
  const int64_t BH = p.B * p.H;
  hipLaunchKernelGGL(f32_scan_kernel, dim3((unsigned)BH), dim3(256), 0, s, w.g, static_cast<const float*>(w.h),
                     w.decay, w.wscale, static_cast<float*>(w.snap), p.nmem, (int)p.d, (int)p.dv,
                     (p.flags & GECKO_AWM_NO_DELTA_BIT) ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_sca_f32(const Problem& p, const Workspace& w, int mode, hipStream_t s) {
  const int64_t BH = p.B * p.H;
  const int64_t qblk = (p.n + 63) / 64;
  hipLaunchKernelGGL(f32_sca_kernel, dim3((unsigned)(qblk * (p.dv / 32) * BH)), dim3(64), 0, s, p,
                     static_cast<const float*>(w.snap), mode, qblk);
  return hipGetLastError();
}

}  // namespace gecko
