// CEMA (complex multi-dimensional damped EMA, the layer that produces
// X' = CEMA(X) before Z') on gfx950.
//
// Per input dimension d and hidden dimension j (Gecko summary on
// paper.rainbus.top, "Prerequisites / EMA"; paperlayer.ai summary, 2.1 and
// Appendix B.1):
//   h_t = alpha beta x_t + M_t q h_{t-1},   q = (1 - alpha delta) e^{i theta},
//   y_t = Re(sum_j eta_j h_t,j),
// with M_t = 0 on a document reset (h_t = alpha beta x_t) and h_0 given (or 0).
//
// Work decomposition: one lane per input dimension d, holding its H complex
// states and per-j constants in registers; a wave covers 64 consecutive
// dimensions, so every load of x and store of y is 64 contiguous elements.
// The work per token is plain FMA arithmetic (no contraction), so the kernel
// is bound by the vector ALU. The sequence is cut into C chunks so that there
// are enough waves to fill the chip:
//   phase A (chunks 0..C-2): each chunk's end state from a zero start;
//   phase B: per (b, d, j), the states entering every chunk, carried across
//     chunks in double: h_in(c+1) = (reset in c ? 0 : q^L) h_in(c) + S(c);
//   phase C (every chunk): the chunk again from its entering state, writing y
//     (and the final state for the last chunk).
// With C = 1 only phase C runs, from h_0.
#include <algorithm>

#include "gecko_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

constexpr int kU = 8;  // tokens per unrolled step (loads issued together)

struct CemaArgs {
  const void* x;        // [B][n][D]
  void* y;              // [B][n][D]
  const float* alpha;   // [D][H]
  const float* delta;
  const float* theta;
  const float* beta;
  const float* eta;     // [D][H][2]
  const uint8_t* reset; // [B][n] or null
  const float* h0;      // [B][D][H][2] or null
  float* hfin;          // [B][D][H][2] or null
  float2* S;            // [B][C][H][D] chunk end states from zero (phase A)
  float2* Hin;          // [B][C][H][D] states entering each chunk (phase B)
  int* flag;            // [B][C] a reset inside the chunk
  int64_t n, L;         // tokens, chunk length (a multiple of kU)
  int D, C, nwd;        // dimensions, chunks, waves per (b, chunk)
};

template <bool kBf16>
__device__ __forceinline__ float load_x(const void* base, int64_t i) {
  if constexpr (kBf16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
  else
    return static_cast<const float*>(base)[i];
}

template <bool kBf16>
__device__ __forceinline__ void store_y(void* base, int64_t i, float v) {
  if constexpr (kBf16)
    static_cast<uint16_t*>(base)[i] = (uint16_t)(pack2(v, 0.f) & 0xffffu);
  else
    static_cast<float*>(base)[i] = v;
}

// The per-lane constants of dimension d: multiplier q, input weight w = alpha
// beta, projection eta.
template <int H>
struct CemaLane {
  float qr[H], qi[H], w[H], er[H], ei[H];

  __device__ __forceinline__ void load(const CemaArgs& a, int d) {
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int k = d * H + j;
      const float al = a.alpha[k], de = a.delta[k];
      float s, c;
      sincosf(a.theta[k], &s, &c);
      const float r = 1.f - al * de;
      qr[j] = r * c;
      qi[j] = r * s;
      w[j] = al * a.beta[k];
      er[j] = a.eta[2 * k];
      ei[j] = a.eta[2 * k + 1];
    }
  }

  // one token: h <- w x + (keep ? q h : 0); returns Re(eta . h) if kOut
  template <bool kOut>
  __device__ __forceinline__ float step(float x, bool reset, float (&hr)[H], float (&hi)[H]) const {
    float out = 0.f;
    if (reset) {
#pragma unroll
      for (int j = 0; j < H; ++j) hr[j] = hi[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const float nr = fmaf(qr[j], hr[j], fmaf(-qi[j], hi[j], w[j] * x));
      const float ni = fmaf(qr[j], hi[j], qi[j] * hr[j]);
      hr[j] = nr;
      hi[j] = ni;
      if constexpr (kOut) out = fmaf(er[j], nr, fmaf(-ei[j], ni, out));
    }
    return out;
  }
};

// Phases A and C: one wave per (b, 64 dimensions, chunk). kOut: phase C.
template <int H, bool kInBf16, bool kOutBf16, bool kOut>
__global__ __launch_bounds__(64) void cema_chunk_kernel(CemaArgs a) {
  const int blk = blockIdx.x;
  const int c = blk % a.C;
  const int wd = (blk / a.C) % a.nwd;
  const int64_t b = blk / (a.C * a.nwd);
  const int d = wd * 64 + (int)threadIdx.x;
  const bool live = d < a.D;
  const int dd = live ? d : a.D - 1;  // lanes past D compute a copy, store nothing
  CemaLane<H> P;
  P.load(a, dd);

  float hr[H], hi[H];
  if constexpr (kOut) {
    if (a.C > 1) {
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const float2 v = a.Hin[((b * a.C + c) * H + j) * a.D + dd];
        hr[j] = v.x;
        hi[j] = v.y;
      }
    } else if (a.h0) {
#pragma unroll
      for (int j = 0; j < H; ++j) {
        hr[j] = a.h0[((b * a.D + dd) * H + j) * 2];
        hi[j] = a.h0[((b * a.D + dd) * H + j) * 2 + 1];
      }
    } else {
#pragma unroll
      for (int j = 0; j < H; ++j) hr[j] = hi[j] = 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < H; ++j) hr[j] = hi[j] = 0.f;
  }

  const int64_t t0 = (int64_t)c * a.L;
  const int64_t t1 = std::min<int64_t>(t0 + a.L, a.n);
  const int64_t D = a.D;
  const int64_t base = b * a.n * D + dd;
  const uint8_t* rs = a.reset ? a.reset + b * a.n : nullptr;
  int any_reset = 0;
  int64_t t = t0;
  for (; t + kU <= t1; t += kU) {
    float xv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) xv[u] = load_x<kInBf16>(a.x, base + (t + u) * D);
    uint64_t rb = 0;  // reset bytes of the kU tokens (wave-uniform)
    if (rs) {
#pragma unroll
      for (int u = 0; u < kU; ++u) rb |= (uint64_t)(rs[t + u] != 0) << (8 * u);
    }
    any_reset |= rb != 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float o = P.template step<kOut>(xv[u], (rb >> (8 * u)) & 1u, hr, hi);
      if constexpr (kOut) {
        if (live) store_y<kOutBf16>(a.y, base + (t + u) * D, o);
      }
    }
  }
  for (; t < t1; ++t) {  // ragged end of the sequence
    const bool r = rs && rs[t] != 0;
    any_reset |= r;
    const float o = P.template step<kOut>(load_x<kInBf16>(a.x, base + t * D), r, hr, hi);
    if constexpr (kOut) {
      if (live) store_y<kOutBf16>(a.y, base + t * D, o);
    }
  }

  if constexpr (!kOut) {
    if (live) {
#pragma unroll
      for (int j = 0; j < H; ++j) a.S[((b * a.C + c) * H + j) * a.D + d] = make_float2(hr[j], hi[j]);
    }
    if (wd == 0 && threadIdx.x == 0) a.flag[b * a.C + c] = any_reset;
  } else {
    if (c == a.C - 1 && a.hfin && live) {
#pragma unroll
      for (int j = 0; j < H; ++j) {
        a.hfin[((b * a.D + d) * H + j) * 2] = hr[j];
        a.hfin[((b * a.D + d) * H + j) * 2 + 1] = hi[j];
      }
    }
  }
}

// Phase B: one thread per (b, d, j); the chunk-entering states, in double.
__global__ void cema_carry_kernel(CemaArgs a, int H) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = blockIdx.y;
  if (i >= (int64_t)a.D * H) return;
  const int d = (int)(i / H), j = (int)(i % H);
  const int k = d * H + j;
  // q^L by repeated squaring (L = chunk length)
  const double r = 1.0 - (double)a.alpha[k] * (double)a.delta[k];
  const double th = (double)a.theta[k];
  double pr = 1.0, pi = 0.0, br = r * cos(th), bi = r * sin(th);
  for (int64_t e = a.L; e > 0; e >>= 1) {
    if (e & 1) {
      const double tr = pr * br - pi * bi;
      pi = pr * bi + pi * br;
      pr = tr;
    }
    const double sr = br * br - bi * bi;
    bi = 2.0 * br * bi;
    br = sr;
  }
  double hr = 0.0, hi = 0.0;
  if (a.h0) {
    hr = a.h0[((b * a.D + d) * H + j) * 2];
    hi = a.h0[((b * a.D + d) * H + j) * 2 + 1];
  }
  for (int c = 0; c < a.C; ++c) {
    a.Hin[((b * a.C + c) * H + j) * a.D + d] = make_float2((float)hr, (float)hi);
    if (c == a.C - 1) break;
    const float2 s = a.S[((b * a.C + c) * H + j) * a.D + d];
    if (a.flag[b * a.C + c]) {
      hr = s.x;
      hi = s.y;
    } else {
      const double nr = pr * hr - pi * hi + s.x;
      hi = pr * hi + pi * hr + s.y;
      hr = nr;
    }
  }
}

template <int H, bool kIn, bool kOut>
hipError_t launch_h(const CemaArgs& a, int64_t B, hipStream_t s) {
  const unsigned blocks = (unsigned)(B * a.nwd * a.C);
  if (a.C > 1) {
    hipLaunchKernelGGL((cema_chunk_kernel<H, kIn, kOut, false>), dim3(blocks), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)a.D * H;
    hipLaunchKernelGGL(cema_carry_kernel, dim3((unsigned)((threads + 255) / 256), (unsigned)B), dim3(256), 0, s, a,
                       H);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((cema_chunk_kernel<H, kIn, kOut, true>), dim3(blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <bool kIn, bool kOut>
hipError_t launch_dt(const CemaArgs& a, int64_t B, int H, hipStream_t s) {
  switch (H) {
    case 1: return launch_h<1, kIn, kOut>(a, B, s);
    case 2: return launch_h<2, kIn, kOut>(a, B, s);
    case 4: return launch_h<4, kIn, kOut>(a, B, s);
    case 8: return launch_h<8, kIn, kOut>(a, B, s);
    case 16: return launch_h<16, kIn, kOut>(a, B, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

CemaPlan cema_plan(int64_t B, int64_t n, int64_t D, int64_t H) {
  CemaPlan p{};
  const int64_t nwd = (D + 63) / 64;
  // enough waves for 256 CUs x 4 SIMDs x 4, chunks of at least 512 tokens
  const int64_t want = std::max<int64_t>(1, (4096 + B * nwd - 1) / (B * nwd));
  const int64_t most = std::max<int64_t>(1, n / 512);
  const int64_t C0 = std::min(want, most);
  p.L = ((n + C0 - 1) / C0 + kU - 1) / kU * kU;
  p.C = (n + p.L - 1) / p.L;
  p.nwd = nwd;
  const size_t states = p.C > 1 ? (size_t)B * (size_t)p.C * (size_t)H * (size_t)D * sizeof(float2) : 0;
  p.off_hin = (states + 255) / 256 * 256;
  p.off_flag = p.off_hin + (states + 255) / 256 * 256;
  p.bytes = p.C > 1 ? p.off_flag + (size_t)B * (size_t)p.C * sizeof(int) : 0;
  return p;
}

hipError_t launch_cema(const CemaProblem& q, const CemaPlan& plan, void* ws, hipStream_t s) {
  CemaArgs a;
  a.x = q.x; a.y = q.y;
  a.alpha = q.alpha; a.delta = q.delta; a.theta = q.theta; a.beta = q.beta; a.eta = q.eta;
  a.reset = q.reset; a.h0 = q.h0; a.hfin = q.hfin;
  a.S = static_cast<float2*>(ws);
  a.Hin = reinterpret_cast<float2*>(static_cast<char*>(ws) + plan.off_hin);
  a.flag = reinterpret_cast<int*>(static_cast<char*>(ws) + plan.off_flag);
  a.n = q.n; a.L = plan.L; a.D = (int)q.D; a.C = (int)plan.C; a.nwd = (int)plan.nwd;
  if (q.in_bf16)
    return q.out_bf16 ? launch_dt<true, true>(a, q.B, (int)q.H, s) : launch_dt<true, false>(a, q.B, (int)q.H, s);
  return q.out_bf16 ? launch_dt<false, true>(a, q.B, (int)q.H, s) : launch_dt<false, false>(a, q.B, (int)q.H, s);
}

}  // namespace gecko
