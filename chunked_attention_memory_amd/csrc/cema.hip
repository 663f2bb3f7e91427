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
// Tokens are taken in groups (four at a time for the end states, two at a
// time for the outputs) with powers of q computed once per lane.
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

// Phase A advances four tokens at a time: h <- q^4 h + (q^3 w) x_1 + (q^2 w) x_2
// + (q w) x_3 + w x_4, with the complex factors per (d, j) computed once (about
// 2.75 operations per token and j instead of 5).
template <int H>
struct CemaQuad {
  float q4r[H], q4i[H], c3r[H], c3i[H], c2r[H], c2i[H], c1r[H], c1i[H], w[H];

  __device__ __forceinline__ void load(const CemaArgs& a, int d) {
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int k = d * H + j;
      const float al = a.alpha[k], de = a.delta[k];
      float sn, cs;
      sincosf(a.theta[k], &sn, &cs);
      const float r = 1.f - al * de;
      const float qr = r * cs, qi = r * sn;
      w[j] = al * a.beta[k];
      const float q2r = qr * qr - qi * qi, q2i = 2.f * qr * qi;
      const float q3r = q2r * qr - q2i * qi, q3i = q2r * qi + q2i * qr;
      q4r[j] = q2r * q2r - q2i * q2i;
      q4i[j] = 2.f * q2r * q2i;
      c1r[j] = qr * w[j];
      c1i[j] = qi * w[j];
      c2r[j] = q2r * w[j];
      c2i[j] = q2i * w[j];
      c3r[j] = q3r * w[j];
      c3i[j] = q3i * w[j];
    }
  }

  // four tokens x[0..3]; reset bits r (bit u: M = 0 at token u). A reset at
  // u drops the state and every input before u, so only the last one counts.
  // kReset = false: r is known to be 0 (no state scaling).
  template <bool kReset>
  __device__ __forceinline__ void step4(const float* xin, uint32_t r, float (&hr)[H], float (&hi)[H]) const {
    float x[4] = {xin[0], xin[1], xin[2], xin[3]};
    float keep = 1.f;
    if (kReset && r) {
      const int u = 31 - __builtin_clz(r);  // the last reset of the four
      keep = 0.f;
#pragma unroll
      for (int k = 0; k < 3; ++k) x[k] = k < u ? 0.f : x[k];
    }
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const float pr = kReset ? keep * hr[j] : hr[j], pi = kReset ? keep * hi[j] : hi[j];
      float nr = fmaf(q4r[j], pr, fmaf(-q4i[j], pi, w[j] * x[3]));
      float ni = fmaf(q4r[j], pi, q4i[j] * pr);
      nr = fmaf(c3r[j], x[0], fmaf(c2r[j], x[1], fmaf(c1r[j], x[2], nr)));
      ni = fmaf(c3i[j], x[0], fmaf(c2i[j], x[1], fmaf(c1i[j], x[2], ni)));
      hr[j] = nr;
      hi[j] = ni;
    }
  }
};

// Phase C advances two tokens at a time from the entering state h:
//   y_t     = sum_j Re((eta q)_j h_j) + K0 x_t
//   y_{t+1} = sum_j Re((eta q^2)_j h_j) + K1 x_t + K0 x_{t+1}
//   h      <- q^2 h + (q w) x_t + w x_{t+1}
// with K0 = sum_j Re(eta_j) w_j and K1 = sum_j Re(eta_j q_j) w_j (about 5.5
// operations per token and j instead of 7). A reset at t drops h; a reset at
// t + 1 drops h and x_t from the second token on.
template <int H>
struct CemaPair {
  float aqr[H], aqi[H], bqr[H], bqi[H], q2r[H], q2i[H], cwr[H], cwi[H], w[H], qr[H], qi[H];
  float K0, K1;

  __device__ __forceinline__ void load(const CemaArgs& a, int d) {
    K0 = K1 = 0.f;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int k = d * H + j;
      const float al = a.alpha[k], de = a.delta[k];
      float sn, cs;
      sincosf(a.theta[k], &sn, &cs);
      const float r = 1.f - al * de;
      qr[j] = r * cs;
      qi[j] = r * sn;
      w[j] = al * a.beta[k];
      const float er = a.eta[2 * k], ei = a.eta[2 * k + 1];
      q2r[j] = qr[j] * qr[j] - qi[j] * qi[j];
      q2i[j] = 2.f * qr[j] * qi[j];
      aqr[j] = er * qr[j] - ei * qi[j];  // eta q
      aqi[j] = er * qi[j] + ei * qr[j];
      bqr[j] = er * q2r[j] - ei * q2i[j];  // eta q^2
      bqi[j] = er * q2i[j] + ei * q2r[j];
      cwr[j] = qr[j] * w[j];
      cwi[j] = qi[j] * w[j];
      K0 = fmaf(er, w[j], K0);
      K1 = fmaf(aqr[j], w[j], K1);
    }
  }

  // kReset = false: r0 and r1 are known to be false (no state scaling)
  template <bool kReset>
  __device__ __forceinline__ void step2(float x0, float x1, bool r0, bool r1, float (&hr)[H], float (&hi)[H],
                                        float& y0, float& y1) const {
    const float keep = r0 ? 0.f : 1.f, keep1 = r1 ? 0.f : keep, xa = r1 ? 0.f : x0;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      s0 = fmaf(aqr[j], hr[j], fmaf(-aqi[j], hi[j], s0));
      s1 = fmaf(bqr[j], hr[j], fmaf(-bqi[j], hi[j], s1));
      const float pr = kReset ? keep1 * hr[j] : hr[j], pi = kReset ? keep1 * hi[j] : hi[j];
      const float nr = fmaf(q2r[j], pr, fmaf(-q2i[j], pi, fmaf(cwr[j], xa, w[j] * x1)));
      const float ni = fmaf(q2r[j], pi, fmaf(q2i[j], pr, cwi[j] * xa));
      hr[j] = nr;
      hi[j] = ni;
    }
    y0 = fmaf(keep, s0, K0 * x0);
    y1 = fmaf(keep1, s1, fmaf(K1, xa, K0 * x1));
  }

  // one token (an odd last token of the sequence): y_t and the state after it
  __device__ __forceinline__ float step1(float x, bool r, float (&hr)[H], float (&hi)[H]) const {
    const float keep = r ? 0.f : 1.f;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      s = fmaf(aqr[j], hr[j], fmaf(-aqi[j], hi[j], s));
      const float pr = keep * hr[j], pi = keep * hi[j];
      const float nr = fmaf(qr[j], pr, fmaf(-qi[j], pi, w[j] * x));
      hi[j] = fmaf(qr[j], pi, qi[j] * pr);
      hr[j] = nr;
    }
    return fmaf(keep, s, K0 * x);
  }
};

// The kU tokens of one loop step (reset bytes rb, byte u for token u),
// written to y at element i0 + u D in phase C. kReset = false: no reset
// among them, so the steps skip the state scaling that a reset needs.
template <bool kReset, bool kOutBf16, bool kOut, int HP, int HQ>
__device__ __forceinline__ void steps(const CemaPair<HP>& P, const CemaQuad<HQ>& Q, const float (&xv)[kU], uint64_t rb,
                                      bool live, int64_t i0, int64_t D, float (&hr)[kOut ? HP : HQ],
                                      float (&hi)[kOut ? HP : HQ], void* y) {
  if constexpr (kOut) {
#pragma unroll
    for (int u = 0; u < kU; u += 2) {
      float y0, y1;
      P.template step2<kReset>(xv[u], xv[u + 1], (rb >> (8 * u)) & 1u, (rb >> (8 * u + 8)) & 1u, hr, hi, y0, y1);
      if (live) {
        store_y<kOutBf16>(y, i0 + u * D, y0);
        store_y<kOutBf16>(y, i0 + (u + 1) * D, y1);
      }
    }
  } else {  // four tokens at a time; reset byte u of rb becomes bit u
#pragma unroll
    for (int u = 0; u < kU; u += 4) {
      const uint32_t r4 = (uint32_t)((rb >> (8 * u)) & 0x01010101u);
      const uint32_t bits = (r4 & 1u) | ((r4 >> 7) & 2u) | ((r4 >> 14) & 4u) | ((r4 >> 21) & 8u);
      Q.template step4<kReset>(xv + u, bits, hr, hi);
    }
  }
}

// Phases A and C: one wave per (b, 64 dimensions, chunk). kOut: phase C.
// kReset: a reset array is given (without one, no step scales the state).
template <int H, bool kInBf16, bool kOutBf16, bool kOut, bool kReset>
__global__ __launch_bounds__(64) void cema_chunk_kernel(CemaArgs a) {
  const int blk = blockIdx.x;
  const int c = blk % a.C;
  const int wd = (blk / a.C) % a.nwd;
  const int64_t b = blk / (a.C * a.nwd);
  const int d = wd * 64 + (int)threadIdx.x;
  const bool live = d < a.D;
  const int dd = live ? d : a.D - 1;  // lanes past D compute a copy, store nothing
  // phase C: two-token steps with the projection; phase A: four-token steps
  CemaPair<kOut ? H : 1> P;
  CemaQuad<kOut ? 1 : H> Q;
  if constexpr (kOut)
    P.load(a, dd);
  else
    Q.load(a, dd);

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
    if constexpr (kReset) {
#pragma unroll
      for (int u = 0; u < kU; ++u) rb |= (uint64_t)(rs[t + u] != 0) << (8 * u);
    }
    any_reset |= rb != 0;
    steps<kReset, kOutBf16, kOut>(P, Q, xv, rb, live, base + t * D, D, hr, hi, a.y);
  }
  for (; t < t1; ++t) {  // ragged end of the sequence
    const bool r = kReset && rs[t] != 0;
    any_reset |= r;
    const float xt = load_x<kInBf16>(a.x, base + t * D);
    if constexpr (kOut) {  // phase A covers full chunks only (L is a multiple of kU)
      const float o = P.step1(xt, r, hr, hi);
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

template <int H, bool kIn, bool kOut, bool kReset>
hipError_t launch_hr(const CemaArgs& a, int64_t B, hipStream_t s) {
  const unsigned blocks = (unsigned)(B * a.nwd * a.C);
  if (a.C > 1) {
    hipLaunchKernelGGL((cema_chunk_kernel<H, kIn, kOut, false, kReset>), dim3(blocks), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)a.D * H;
    hipLaunchKernelGGL(cema_carry_kernel, dim3((unsigned)((threads + 255) / 256), (unsigned)B), dim3(256), 0, s, a,
                       H);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((cema_chunk_kernel<H, kIn, kOut, true, kReset>), dim3(blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int H, bool kIn, bool kOut>
hipError_t launch_h(const CemaArgs& a, int64_t B, hipStream_t s) {
  return a.reset ? launch_hr<H, kIn, kOut, true>(a, B, s) : launch_hr<H, kIn, kOut, false>(a, B, s);
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
