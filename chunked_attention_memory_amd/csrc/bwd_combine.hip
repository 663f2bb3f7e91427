// Last step of the backward: the four per-token gradients with respect to
// Q, K (attention) and Q_m, K_m (memory) go back through the affine maps of
// the Gecko summary (paper.rainbus.top, "Method steps" (2) and (4)):
//   dL/dZ'     = kappa_q dQ + kappa_k dK + eta_q dQ_m + eta_k dK_m
//   dL/dkappa_q = sum over (batch, token) of Z' dQ,  dL/dnu_q = sum of dQ,
// and likewise for (kappa_k, nu_k), (eta_q, rho_q) and (eta_k, rho_k).
// One thread per feature, one workgroup per run of rows of one (batch, head);
// the per-workgroup sums go to a partial array that a second kernel reduces
// (in a fixed order) over the runs and the batch.
#include "gecko_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

struct CombineArgs {
  const uint16_t* z;
  const float* g[4];    // dQ, dK, dQ_m, dK_m ([bh][n][d]) or null
  const float* aff[8];  // kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k
  float* dz;
  float* apart;         // [bh][nblk][8][d]
  int64_t n, rows_per_blk;
  int nblk, H, D;
};

__global__ __launch_bounds__(128) void bwd_combine_kernel(CombineArgs a) {
  const int f = threadIdx.x;
  if (f >= a.D) return;
  const int64_t bh = blockIdx.x / a.nblk;
  const int blk = (int)(blockIdx.x % a.nblk);
  const int h = (int)(bh % a.H);
  const int D = a.D;
  float coef[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) coef[i] = a.g[i] ? a.aff[2 * i][h * D + f] : 0.f;
  const int64_t r0 = blk * a.rows_per_blk;
  const int64_t r1 = min(r0 + a.rows_per_blk, a.n);
  float sums[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sums[i] = 0.f;
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t e = (bh * a.n + r) * D + f;
    const float zf = __uint_as_float((uint32_t)a.z[e] << 16);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gi = a.g[i] ? a.g[i][e] : 0.f;
      acc += coef[i] * gi;
      sums[2 * i] += zf * gi;
      sums[2 * i + 1] += gi;
    }
    a.dz[e] = acc;
  }
  float* out = a.apart + ((bh * a.nblk + blk) * 8) * (int64_t)D + f;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[(int64_t)i * D] = sums[i];
}

// daff[i][h][f] = sum over b and runs of apart[b h][run][i][f]: kSplit
// threads per feature, each summing a contiguous share of the runs with
// eight partial sums in flight (a single thread per feature waits on one
// load after another: 512 runs at 128K tokens), then the shares added in
// LDS. The order of every addition is fixed, so the result does not depend
// on timing.
constexpr int kSplit = 8;
__global__ __launch_bounds__(1024) void bwd_affine_reduce_kernel(const float* __restrict__ apart,
                                                                float* __restrict__ daff, int64_t B, int H,
                                                                int nblk, int D) {
  __shared__ float red[kSplit][128];
  const int f = threadIdx.x % D, sp = threadIdx.x / D;  // D <= 128, blockDim.x = kSplit * D
  const int i = blockIdx.x % 8;
  const int h = blockIdx.x / 8;
  const int per = (nblk + kSplit - 1) / kSplit;
  const int k0 = sp * per, k1 = min(k0 + per, nblk);
  float s = 0.f;
  for (int64_t b = 0; b < B; ++b) {
    const float* p = apart + (((b * H + h) * nblk) * 8 + i) * (int64_t)D + f;
    float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int k = k0;
    for (; k + 8 <= k1; k += 8)
#pragma unroll
      for (int u = 0; u < 8; ++u) s8[u] += p[(int64_t)(k + u) * 8 * D];
    for (; k < k1; ++k) s8[0] += p[(int64_t)k * 8 * D];
    red[sp][f] = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
    __syncthreads();
    if (sp == 0) {
#pragma unroll
      for (int q = 0; q < kSplit; ++q) s += red[q][f];
    }
    __syncthreads();
  }
  if (sp == 0) daff[((int64_t)i * H + h) * D + f] = s;
}

}  // namespace

hipError_t launch_bwd_combine(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s) {
  CombineArgs a;
  a.z = static_cast<const uint16_t*>(p.f.z);
  a.g[0] = p.sca ? w.dq : nullptr;
  a.g[1] = p.sca ? w.dk : nullptr;
  a.g[2] = p.awm ? w.dqm : nullptr;
  a.g[3] = p.awm ? w.dkm : nullptr;
  const float* aff[8] = {p.f.kappa_q, p.f.nu_q, p.f.kappa_k, p.f.nu_k, p.f.eta_q, p.f.rho_q, p.f.eta_k, p.f.rho_k};
  for (int i = 0; i < 8; ++i) a.aff[i] = aff[i];
  a.dz = p.dz;
  a.apart = w.apart;
  a.n = p.f.n;
  a.rows_per_blk = w.rows_per_blk;
  a.nblk = (int)w.nblk;
  a.H = (int)p.f.H;
  a.D = (int)p.f.d;
  const int64_t BH = p.f.B * p.f.H;
  hipLaunchKernelGGL(bwd_combine_kernel, dim3((unsigned)(BH * w.nblk)), dim3(128), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.f.d > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_affine_reduce_kernel, dim3((unsigned)(8 * p.f.H)), dim3((unsigned)(kSplit * p.f.d)), 0, s,
                     w.apart, p.daff, p.f.B, (int)p.f.H, (int)w.nblk, (int)p.f.d);
  return hipGetLastError();
}

}  // namespace gecko
