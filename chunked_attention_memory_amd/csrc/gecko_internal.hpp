// Host-side interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gecko {

// same bit as GECKO_AWM_NO_DELTA in gecko.h
constexpr unsigned GECKO_AWM_NO_DELTA_BIT = 1u << 0;

// Per-launch description of one forward. All pointers are device pointers.
struct Problem {
  const void* z;        // [BH][n][d]   in dtype
  const void* v;        // [BH][n][dv]  in dtype
  void* out;            // [BH][n][dv]  out dtype
  const float* kappa_q; const float* nu_q; const float* kappa_k; const float* nu_k;
  const float* eta_q; const float* rho_q; const float* eta_k; const float* rho_k;
  int64_t B, H, n, d, dv, c;
  int64_t nchunks;      // N = ceil(n / c)
  int64_t nmem;         // chunks written into the memory that some chunk reads: max(N - 2, 0)
  unsigned flags;
  bool out_f32;         // output dtype (bf16 inputs may write float32 output)
};

// Workspace carve-up (byte offsets from the workspace base). Every array is
// indexed [bh][t] with t = 0..nmem-1 the 0-based chunk that is written.
struct Workspace {
  float* g;        // memory-write product E^T V, fp32: bf16 path [bh][t][dv/32][d/32][64][16]
                   //   (MFMA accumulator layout), fp32 path [bh][t][dv/32][d][32]
  void* h;         // correction product E^T psi(K_m)   [bh][t][d][d]  (bf16 or fp32)
  float* cmax;     // per-feature max of K_m over the chunk   [bh][t][d]
  float* csum;     // per-feature sum of exp(K_m - cmax)     [bh][t][d]
  float* decay;    // z^{t-1} / z^t (fp32 path)              [bh][t][d]
  float* wscale;   // exp(cmax) / z^t (fp32 path)            [bh][t][d]
  void* snap;      // state read by chunk t+2: bf16 [bh][t][d][dv], fp32 [bh][t][dv][d]
  float* rowstat;  // fp32 path only: per-token (max, sum) of K_m rows  [bh][n][2]
  size_t bytes;
};

Workspace carve_workspace(void* base, int64_t BH, int64_t n, int64_t d, int64_t dv,
                          int64_t nmem, bool bf16);

// Launchers (stream-ordered, asynchronous). Each returns the launch status.
hipError_t launch_awm_chunk_bf16(const Problem& p, const Workspace& w, hipStream_t s);
hipError_t launch_awm_zscan(const Problem& p, const Workspace& w, hipStream_t s);
hipError_t launch_awm_scan_bf16(const Problem& p, const Workspace& w, hipStream_t s);
// mode bit 0: attention, bit 1: memory readout
hipError_t launch_sca_bf16(const Problem& p, const Workspace& w, int mode, hipStream_t s);

hipError_t launch_awm_chunk_f32(const Problem& p, const Workspace& w, hipStream_t s);
hipError_t launch_awm_scan_f32(const Problem& p, const Workspace& w, hipStream_t s);
hipError_t launch_sca_f32(const Problem& p, const Workspace& w, int mode, hipStream_t s);

bool bf16_shape_built(int64_t d, int64_t dv);

}  // namespace gecko
