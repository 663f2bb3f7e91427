// Sliding chunk attention with the memory readout fused into its epilogue,
// bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Computes, for every query row i of chunk s (Gecko summary, paper.rainbus.top,
// "Method steps" (3) and (5)):
//   O_i = softmax_j(q_i . k_j) v_j over keys j of chunks s-1 and s with j <= i
//         + psi(Q_m,i) M'_{s-1}            (readout; chunks s >= 3, 1-based)
//
// Work decomposition: one workgroup = 128 consecutive queries of one chunk of
// one (batch, head); 4 waves x 32 queries. The key window [(s-1)c, last query]
// is streamed in tiles of 64 keys through double-buffered LDS.
//
// Per tile and wave:
//   S^T (64 keys x 32 queries) = K_tile Q^T       (A = K from LDS, B = Q in VGPRs)
//   online softmax over keys, lane-local per query (a query's 64 keys are
//   split between lane l and lane l ^ 32)
//   O^T (dv x 32 queries) += V^T P^T               (A = V^T from LDS, B = P in VGPRs)
// Holding O transposed keeps each query's accumulator column, its running max
// and its running sum in the same lane, so rescaling never crosses lanes.
//
// Algebra used to drop the key-side affine map: q . (kappa_k * z_j + nu_k)
// = (q * kappa_k) . z_j + q . nu_k. The second term is the same for every key
// of query i, and softmax is invariant to a per-row shift, so the kernel uses
// q' = (kappa_q * z_i + nu_q) * kappa_k * log2(e) against the raw z_j. The
// log2(e) factor lets the exponentials run on the hardware exp2.
#include "gecko_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

constexpr int kBM = 128;       // queries per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 waves
constexpr float kLazy = 8.0f;  // rescale only when the running max grows by > 2^8

template <int D, int DV>
struct ScaTile {
  static constexpr int KROW = D + 8;    // LDS row of K (bf16 elements), +16 B pad
  static constexpr int VROW = kBN + 8;  // LDS row of V^T
  static constexpr int KELEMS = kBN * KROW;
  static constexpr int VELEMS = DV * VROW;
  static constexpr int STAGE = KELEMS + VELEMS;
  static constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(uint16_t);
  static constexpr int KPIECES = kBN * D / 8 / kThreads;  // 16-byte pieces per thread
};

struct ScaArgs {
  const uint16_t* z;
  const uint16_t* v;
  void* out;  // bf16 or float32 [bh][n][dv]
  const float* kappa_q;
  const float* nu_q;
  const float* kappa_k;
  const float* eta_q;
  const float* rho_q;
  const uint16_t* snap;  // [bh][nmem][dv][d]; slot t is the state read by chunk t + 2 (0-based)
  int64_t n, c, nchunks, nmem, qtiles, nblocks, per_xcd;
  int H;
};

template <int D, int DV, bool kSca, bool kRead, bool kOutF32>
__global__ __launch_bounds__(kThreads, 1) void sca_bf16_kernel(ScaArgs a) {
  using T = ScaTile<D, DV>;
  constexpr int KS = D / 16;   // 16-feature k-steps of Q K^T
  constexpr int NMV = DV / 32; // 32-row blocks of O^T
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  // Blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous
  // run of logical blocks so the q-tiles of one chunk share an L2.
  const int64_t bid = blockIdx.x;
  const int64_t lb = (bid & 7) * a.per_xcd + (bid >> 3);
  if (lb >= a.nblocks) return;
  const int qt = (int)(a.qtiles - 1 - lb % a.qtiles);  // longest q-tiles first
  const int64_t rest = lb / a.qtiles;
  const int64_t s = rest % a.nchunks;
  const int64_t bh = rest / a.nchunks;
  const int h = (int)(bh % a.H);
  const int64_t n = a.n, c = a.c;
  const int64_t q0 = s * c + (int64_t)qt * kBM;
  const int64_t cend = min((s + 1) * c, n);
  if (q0 >= cend) return;
  const int64_t qend = min(q0 + (int64_t)kBM, cend);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, lq = lane & 31;
  const int64_t myq = q0 + w * 32 + lq;
  const bool qvalid = myq < qend;
  const int64_t qrow = qvalid ? myq : qend - 1;
  const uint16_t* zbh = a.z + bh * n * D;

  f32x16 oacc[NMV];
#pragma unroll
  for (int i = 0; i < NMV; ++i) oacc[i] = f32x16{};

  if constexpr (kSca) {
    const uint16_t* vbh = a.v + bh * n * DV;
    // ---- query fragments: lane holds query lq, features 16 ks + 8 g + [0, 8)
    u32x4 qf[KS];
    {
      const float* kq = a.kappa_q + h * D;
      const float* nq = a.nu_q + h * D;
      const float* kk = a.kappa_k + h * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int f0 = 16 * ks + 8 * g;
        const u32x4 raw = ld16(zbh + qrow * D + f0);
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = bf_lo(raw[j]);
          x[2 * j + 1] = bf_hi(raw[j]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (kq[f0 + i] * x[i] + nq[f0 + i]) * (kk[f0 + i] * kLog2e);
        qf[ks] = u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
      }
    }

    const int64_t kbeg = s > 0 ? (s - 1) * c : 0;
    const int64_t kend = qend;
    const int ntiles = (int)((kend - kbeg + kBN - 1) / kBN);
    const int64_t wave_q0 = q0 + w * 32;

    u32x4 kreg[T::KPIECES];
    u32x4 vreg[8];
    // V is staged as 8x8 blocks: block (kg, vg) covers tile positions
    // [8 kg, 8 kg + 8) and value columns [8 vg, 8 vg + 8).
    constexpr int VG = DV / 8;
    const bool vthread = tid < 8 * VG;
    const int kg = tid / VG, vg = tid % VG;

    auto load_tile = [&](int kt) {
      const int64_t kb = kbeg + (int64_t)kt * kBN;
#pragma unroll
      for (int i = 0; i < T::KPIECES; ++i) {
        const int p = tid + kThreads * i;
        const int row = p / (D / 8), col = (p % (D / 8)) * 8;
        const int64_t key = kb + row;
        kreg[i] = key < n ? ld16(zbh + key * D + col) : u32x4{};
      }
      if (vthread) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // tile position 8 kg + i holds key perm_row(8 kg + i): inside each
          // 16-key group, bits 2 and 3 of the key index are swapped, which is
          // the order the S^T accumulator hands P to the P V product.
          const int64_t key = kb + perm_row(8 * kg + i);
          vreg[i] = key < n ? ld16(vbh + key * DV + 8 * vg) : u32x4{};
        }
      }
    };
    auto store_tile = [&](int buf) {
      uint16_t* Ks = lds + buf * T::STAGE;
      uint16_t* Vs = Ks + T::KELEMS;
#pragma unroll
      for (int i = 0; i < T::KPIECES; ++i) {
        const int p = tid + kThreads * i;
        const int row = p / (D / 8), col = (p % (D / 8)) * 8;
        st16(Ks + row * T::KROW + col, kreg[i]);
      }
      if (vthread) {
        u32x4 tr[8];
        transpose8x8(vreg, tr);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const int vcol = 8 * vg + cc;
          // value column v lives in LDS row perm_row(v) of its 32-block, so a
          // lane reading row l of the block gets v = perm_row(l): accumulator
          // rows then come out as 8 consecutive values per lane half.
          const int vrow = (vcol & ~31) | perm_row(vcol & 31);
          st16(Vs + vrow * T::VROW + 8 * kg, tr[cc]);
        }
      }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    float mrun = kNegInf;  // running max of the row (log2 units), same in lanes l and l^32
    float lrun = 0.f;      // this lane's share of the running exp-sum
    for (int kt = 0; kt < ntiles; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < ntiles) load_tile(kt + 1);
      const uint16_t* Ks = lds + buf * T::STAGE;
      const uint16_t* Vs = Ks + T::KELEMS;

      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const u32x4 af = ld16(Ks + (32 * mb + lq) * T::KROW + 16 * ks + 8 * g);
          sacc[mb] = mfma_bf16(af, qf[ks], sacc[mb]);
        }
      }

      // accumulator (mb, r) holds key kb + 32 mb + 8 (r >> 2) + 4 g + (r & 3)
      const int64_t kb = kbeg + (int64_t)kt * kBN;
      if (kb + kBN - 1 > wave_q0 || kb + kBN > kend) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t key = kb + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key > myq || key >= kend) sacc[mb][r] = kNegInf;
          }
      }

      float tmax = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[mb][r]);
      tmax = fmaxf(tmax, wave_xor32(tmax));
      const float mnew = fmaxf(mrun, tmax);
      if (__any(mnew > mrun + kLazy)) {
        const float alpha = (mnew == kNegInf) ? 1.f : exp2_fast(mrun - mnew);
        lrun *= alpha;
#pragma unroll
        for (int i = 0; i < NMV; ++i) oacc[i] *= alpha;
        mrun = mnew;
      }
      const float msub = (mrun == kNegInf) ? 0.f : mrun;
      float psum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(sacc[mb][r] - msub);
          sacc[mb][r] = p;
          psum += p;
        }
      lrun += psum;

#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x16& sp = sacc[mb];
          const u32x4 pf{pack2(sp[8 * hh + 0], sp[8 * hh + 1]), pack2(sp[8 * hh + 2], sp[8 * hh + 3]),
                         pack2(sp[8 * hh + 4], sp[8 * hh + 5]), pack2(sp[8 * hh + 6], sp[8 * hh + 7])};
#pragma unroll
          for (int mv = 0; mv < NMV; ++mv) {
            const u32x4 af = ld16(Vs + (32 * mv + lq) * T::VROW + 32 * mb + 16 * hh + 8 * g);
            oacc[mv] = mfma_bf16(af, pf, oacc[mv]);
          }
        }

      if (kt + 1 < ntiles) store_tile(buf ^ 1);
      __syncthreads();
    }
    const float ltot = lrun + wave_xor32(lrun);
    const float inv = 1.f / ltot;
#pragma unroll
    for (int i = 0; i < NMV; ++i) oacc[i] *= inv;
  }

  if constexpr (kRead) {
    if (s >= 2) {
      // psi(Q_m) of this lane's query, features 16 ks + 8 g + [0, 8)
      const float* eq = a.eta_q + h * D;
      const float* rq = a.rho_q + h * D;
      float qm[KS * 8];
      float mx = kNegInf;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int f0 = 16 * ks + 8 * g;
        const u32x4 raw = ld16(zbh + qrow * D + f0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qm[8 * ks + 2 * j] = eq[f0 + 2 * j] * bf_lo(raw[j]) + rq[f0 + 2 * j];
          qm[8 * ks + 2 * j + 1] = eq[f0 + 2 * j + 1] * bf_hi(raw[j]) + rq[f0 + 2 * j + 1];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, qm[8 * ks + i]);
      }
      mx = fmaxf(mx, wave_xor32(mx));
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < KS * 8; ++i) {
        qm[i] = exp2_fast((qm[i] - mx) * kLog2e);
        sum += qm[i];
      }
      sum += wave_xor32(sum);
      const float inv = 1.f / sum;
      const uint16_t* sn = a.snap + ((bh * a.nmem + (s - 2)) * DV) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float* e = qm + 8 * ks;
        const u32x4 pf{pack2(e[0] * inv, e[1] * inv), pack2(e[2] * inv, e[3] * inv),
                       pack2(e[4] * inv, e[5] * inv), pack2(e[6] * inv, e[7] * inv)};
#pragma unroll
        for (int mv = 0; mv < NMV; ++mv) {
          const int vrow = 32 * mv + perm_row(lq);
          const u32x4 af = ld16(sn + vrow * D + 16 * ks + 8 * g);
          oacc[mv] = mfma_bf16(af, pf, oacc[mv]);
        }
      }
    }
  }

  // accumulator register r of block mv holds value column
  // 32 mv + 16 (r >> 3) + 8 g + (r & 7): two runs of 8 per lane
  if (qvalid) {
    if constexpr (kOutF32) {
      float* orow = static_cast<float*>(a.out) + (bh * n + myq) * DV;
#pragma unroll
      for (int mv = 0; mv < NMV; ++mv)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x16& o = oacc[mv];
          float* dst = orow + 32 * mv + 16 * hh + 8 * g;
          *reinterpret_cast<f32x4*>(dst) = f32x4{o[8 * hh + 0], o[8 * hh + 1], o[8 * hh + 2], o[8 * hh + 3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[8 * hh + 4], o[8 * hh + 5], o[8 * hh + 6], o[8 * hh + 7]};
        }
    } else {
      uint16_t* orow = static_cast<uint16_t*>(a.out) + (bh * n + myq) * DV;
#pragma unroll
      for (int mv = 0; mv < NMV; ++mv)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x16& o = oacc[mv];
          const u32x4 pk{pack2(o[8 * hh + 0], o[8 * hh + 1]), pack2(o[8 * hh + 2], o[8 * hh + 3]),
                         pack2(o[8 * hh + 4], o[8 * hh + 5]), pack2(o[8 * hh + 6], o[8 * hh + 7])};
          st16(orow + 32 * mv + 16 * hh + 8 * g, pk);
        }
    }
  }
}

template <int D, int DV, bool kSca, bool kRead, bool kOutF32>
hipError_t launch_one(const ScaArgs& a, hipStream_t stream) {
  auto kern = sca_bf16_kernel<D, DV, kSca, kRead, kOutF32>;
  const size_t lds = kSca ? ScaTile<D, DV>::LDS_BYTES : 0;
  if (lds > 65536) {
    static bool attr_set = false;  // per instantiation
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  const dim3 grid((unsigned)(8 * a.per_xcd));
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int D, int DV, bool kOutF32>
hipError_t launch_mode(const ScaArgs& a, int mode, hipStream_t s) {
  switch (mode) {
    case 1: return launch_one<D, DV, true, false, kOutF32>(a, s);
    case 2: return launch_one<D, DV, false, true, kOutF32>(a, s);
    case 3: return launch_one<D, DV, true, true, kOutF32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int DV>
hipError_t launch_shape(const ScaArgs& a, int mode, bool out_f32, hipStream_t s) {
  return out_f32 ? launch_mode<D, DV, true>(a, mode, s) : launch_mode<D, DV, false>(a, mode, s);
}

}  // namespace

bool bf16_shape_built(int64_t d, int64_t dv) {
  return (d == 128 && (dv == 256 || dv == 128)) || (d == 64 && (dv == 128 || dv == 64));
}

hipError_t launch_sca_bf16(const Problem& p, const Workspace& w, int mode, hipStream_t stream) {
  ScaArgs a;
  a.z = static_cast<const uint16_t*>(p.z);
  a.v = static_cast<const uint16_t*>(p.v);
  a.out = p.out;
  a.kappa_q = p.kappa_q; a.nu_q = p.nu_q; a.kappa_k = p.kappa_k;
  a.eta_q = p.eta_q; a.rho_q = p.rho_q;
  a.snap = static_cast<const uint16_t*>(w.snap);
  a.n = p.n; a.c = p.c; a.nchunks = p.nchunks; a.nmem = p.nmem; a.H = (int)p.H;
  a.qtiles = (min(p.c, p.n) + kBM - 1) / kBM;
  a.nblocks = p.B * p.H * p.nchunks * a.qtiles;
  a.per_xcd = (a.nblocks + 7) / 8;
  if (p.d == 128 && p.dv == 256) return launch_shape<128, 256>(a, mode, p.out_f32, stream);
  if (p.d == 128 && p.dv == 128) return launch_shape<128, 128>(a, mode, p.out_f32, stream);
  if (p.d == 64 && p.dv == 128) return launch_shape<64, 128>(a, mode, p.out_f32, stream);
  if (p.d == 64 && p.dv == 64) return launch_shape<64, 64>(a, mode, p.out_f32, stream);
  return hipErrorInvalidValue;
}

}  // namespace gecko
