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
#include <algorithm>

#include "gecko_device.hpp"
#include "gecko_internal.hpp"

namespace gecko {
namespace {

// Chunk pass: tokens per tile and LDS stages (tile i + kNS - 1 loads while
// tile i is computed)
#ifndef GECKO_CHUNK_BT
#define GECKO_CHUNK_BT 32
#endif
#ifndef GECKO_CHUNK_NS
#define GECKO_CHUNK_NS 4
#endif
constexpr int kBT = GECKO_CHUNK_BT;
constexpr int kNS = GECKO_CHUNK_NS;
static_assert(kNS >= 4 && kNS <= 6 && kNS % 2 == 0, "chunk pass stages");
// operands of the chunk pass's MFMAs read from LDS this many MFMAs ahead
#ifndef GECKO_CHUNK_AH
#define GECKO_CHUNK_AH 2
#endif
constexpr float kOverflow = 0x1p63f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// reductions over aligned groups of P = 2, 4 or 8 consecutive lanes
template <int P>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));                        // quad_perm [1,0,3,2]
  if constexpr (P >= 4) x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  if constexpr (P >= 8) x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  return x;
}
template <int P>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);
  if constexpr (P >= 4) x += dpp<0x4E>(x);
  if constexpr (P >= 8) x += dpp<0x141>(x);
  return x;
}

// XOR swizzle of the 16-byte chunks of a staged Z' (and psi) row, chosen so
// that both the row reads of the psi phase (16 lanes x 16 bytes per pass) and
// the 4-row transpose reads of the MFMA phase (32 lanes x 8 bytes per pass)
// touch each of the 64 LDS banks once.
template <int D>
__device__ __forceinline__ int zswz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | (r & 3);
  if constexpr (D == 32) return (r >> 2) & 3;  // rows of 64 bytes: 4 chunks
  const int rho = (r >> 1) & 3;
  return rho ^ ((rho & 1) << 2);
}

template <int D, int DV>
struct ChunkTile {
  static constexpr int NW = D / 32;          // one wave per 32 key features
  static constexpr int THREADS = 64 * NW;
  static constexpr int ZBYTES = kBT * D * 2;
  static constexpr int VBYTES = kBT * DV * 2;
  // 16-byte loads per thread per tile, at least one (with fewer 1 KiB
  // pieces than waves, waves share pieces; see stage_rows)
  static constexpr int ZPIECES = ZBYTES / 1024;
  static constexpr int VPIECES = VBYTES / 1024;
  static constexpr int ZLOADS = ZBYTES / 16 / THREADS > 0 ? ZBYTES / 16 / THREADS : 1;
  static constexpr int VLOADS = VBYTES / 16 / THREADS > 0 ? VBYTES / 16 / THREADS : 1;
  static constexpr int ZMOD = ZPIECES < NW * ZLOADS ? ZPIECES : 0;  // piece count for stage_rows (0: no sharing)
  static constexpr int VMOD = VPIECES < NW * VLOADS ? VPIECES : 0;
  static constexpr int PARTS = THREADS / kBT;  // threads per token row in the psi phase
  static constexpr int FPT = D / PARTS;        // features per thread in the psi phase
  static constexpr int KT = kBT / 16;          // 16-token k-steps per tile
  static_assert(FPT % 8 == 0 && FPT <= 16 && (PARTS == 2 || PARTS == 4 || PARTS == 8), "psi phase split");
  static constexpr int STAGE = ZBYTES + VBYTES;
  static constexpr int LOADS = ZLOADS + VLOADS;  // staging loads per lane and tile
  // kNS (Z', V) stages, then two psi tiles
  static constexpr size_t LDS_BYTES = kNS * (size_t)STAGE + 2 * (size_t)ZBYTES;
};

struct ChunkArgs {
  const uint16_t* z;
  const uint16_t* v;
  const float* eta_k;
  const float* rho_k;
  float* g;          // G^T accumulators, [bh][t][dv/32][d/32][64 lanes][16]
  uint16_t* hm;      // H^T accumulators in scan-operand order, [bh][t][d/16][d/32][64 lanes][8]
  float* cmax;       // [bh][t][d] (log2 units)
  float* csum;       // [bh][t][d]
  const uint16_t* zprev;  // streaming: chunk t = 0 is the carried chunk [bh][c][d] / [bh][c][dv]
  const uint16_t* vprev;
  int64_t n, c, nmem;
  int H, has_prev;
};

// One workgroup per (batch*head, chunk t). Wave w owns key features
// [32 w, 32 w + 32) and accumulates, transposed,
//   G^T (dv x 32) += V^T E  and  H^T (d x 32) += psi^T E
// over 64-token tiles, E = 2^(K_m log2(e) - m) with m fixed per feature at the
// exact maximum over the chunk's first tile (a final exp-sum above 2^63 sends
// the workgroup through an exact-maximum recompute). Per tile: Z' and V are
// staged straight into LDS; the psi phase writes psi(K_m) for the tile's 64
// tokens into LDS (computed once, shared by the waves); the MFMA phase forms
// E from transpose reads of Z' and reads V^T and psi^T with transpose reads.
// Member functions rather than lambdas: lambdas in a kernel are compiled for
// the host too, where the buffer and LDS builtins do not exist.
template <int D, int DV>
struct ChunkLoop {
  using T = ChunkTile<D, DV>;
  static constexpr int NMV = DV / 32;
  static constexpr int NMF = D / 32;
  const uint16_t* zbh;
  const uint16_t* vbh;
  // stage s: Z' tile at sb[s], V tile after it; psi tiles at psb. Separate LDS
  // variables, so that the compiler sees that the reads of one stage do not
  // alias the loads filling the other (it would wait for them otherwise).
  char* sb[kNS];
  char* psb[2];  // psi of tiles with even / odd index
  int n, cbeg, cend, ntiles, w, lane, g, lq;
  float ekf, rkf;  // this lane's feature
  // eta_k, rho_k (log2-scaled) of this thread's features in the psi phase
  float pe[T::FPT], pr[T::FPT];
  uint32_t zoff[T::ZLOADS], voff[T::VLOADS];
  // Transpose-read bases (byte offsets within a stage / the psi tile) for
  // read jj of block blk at k-step 0; k-step ks adds 16 ks rows. See tr_base.
  int zb[2], vb[2][NMV], pb[2][NMF];
  int poff[T::FPT / 8];  // psi phase: this thread's 16-byte chunks of its token row

  __device__ __forceinline__ void init(const ChunkArgs& a, int64_t bh, int64_t t, char* const (&stages)[kNS],
                                       char* ps0, char* ps1) {
    const int h = (int)(bh % a.H);
    // chunk t of the virtual sequence [carried chunk (streaming)] + this
    // call's chunks; every chunk entered into the memory is full
    if (a.has_prev && t == 0) {
      n = (int)a.c;
      cbeg = 0;
      zbh = a.zprev + (size_t)bh * (size_t)a.c * D;
      vbh = a.vprev + (size_t)bh * (size_t)a.c * DV;
    } else {
      n = (int)a.n;
      cbeg = (int)((t - a.has_prev) * a.c);
      zbh = a.z + (size_t)bh * (size_t)n * D;
      vbh = a.v + (size_t)bh * (size_t)n * DV;
    }
    cend = cbeg + (int)a.c;
    ntiles = (int)((a.c + kBT - 1) / kBT);
    const int tid = threadIdx.x;
    lane = tid & 63;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    g = lane >> 5;
    lq = lane & 31;
#pragma unroll
    for (int i = 0; i < kNS; ++i) sb[i] = stages[i];
    psb[0] = ps0;
    psb[1] = ps1;
    {
      const int f0 = T::FPT * (tid % T::PARTS);
#pragma unroll
      for (int i = 0; i < T::FPT; ++i) {
        pe[i] = a.eta_k[h * D + f0 + i] * kLog2e;
        pr[i] = a.rho_k[h * D + f0 + i] * kLog2e;
      }
    }
    const int f = 32 * w + lq;
    ekf = a.eta_k[h * D + f] * kLog2e;
    rkf = a.rho_k[h * D + f] * kLog2e;
#pragma unroll
    for (int i = 0; i < T::ZLOADS; ++i) {
      const int P = stage_piece(T::NW, w, i, T::ZMOD) * 64 + lane;
      const int r = P / (D / 8), p = P % (D / 8);
      zoff[i] = (uint32_t)(r * D + 8 * (p ^ zswz<D>(r))) * 2u;
    }
#pragma unroll
    for (int i = 0; i < T::VLOADS; ++i) {
      const int P = stage_piece(T::NW, w, i, T::VMOD) * 64 + lane;
      const int r = P / (DV / 8), p = P % (DV / 8);
      voff[i] = (uint32_t)(r * DV + 8 * (p ^ vswz<DV>(r))) * 2u;
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      zb[jj] = tr_base<D, true>(w, jj);
#pragma unroll
      for (int mv = 0; mv < NMV; ++mv) vb[jj][mv] = tr_base<DV, false>(mv, jj);
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf) pb[jj][mf] = tr_base<D, true>(mf, jj);
    }
    {
      const int tk = tid / T::PARTS, q = tid % T::PARTS;
#pragma unroll
      for (int k = 0; k < T::FPT / 8; ++k) poff[k] = tk * D * 2 + 16 * ((T::FPT / 8 * q + k) ^ zswz<D>(tk));
    }
  }

  // Transpose-read operand: element j of lane (lq, g) is M[16 ks + 8 g + j][32 blk + lq]
  // for a row-major staged tile M with WIDTH columns and its chunk swizzle.
  // Read jj supplies j = 4 jj + j': source lane s of each 16-lane group points
  // at row 16 ks + 8 g + 4 jj + s / 4 and columns 32 blk + 16 (group % 2) + 4 (s % 4).
  // Both swizzles depend on row bits 0..2 only, so k-step ks adds 16 ks rows
  // to the offset computed here for ks = 0.
  template <int WIDTH, bool kZ>
  __device__ __forceinline__ int tr_base(int blk, int jj) const {
    const int sl = lane & 15, g2 = (lane >> 4) & 1;
    const int r = 8 * g + 4 * jj + (sl >> 2);
    const int col = 32 * blk + 16 * g2 + 4 * (sl & 3);
    const int sw = kZ ? zswz<D>(r) : vswz<DV>(r);
    return r * WIDTH * 2 + 16 * ((col >> 3) ^ sw) + 2 * (col & 7);
  }
  template <int WIDTH>
  __device__ __forceinline__ u32x4 tr_operand(const char* base, int b0, int b1, int ks) const {
    const u32x2 lo = lds_read_tr(base + b0 + 16 * ks * WIDTH * 2);
    const u32x2 hi = lds_read_tr(base + b1 + 16 * ks * WIDTH * 2);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }

  __device__ __forceinline__ const char* zs(int slot) const { return sb[slot]; }
  __device__ __forceinline__ const char* vs(int slot) const { return sb[slot] + T::ZBYTES; }
  __device__ __forceinline__ void stage_z(int it, int slot) const {
    stage_rows(zbh, cbeg + it * kBT, n, D, sb[slot], T::NW, w, zoff, T::ZLOADS, T::ZMOD);
  }
  __device__ __forceinline__ void stage_v(int it, int slot) const {
    stage_rows(vbh, cbeg + it * kBT, n, DV, sb[slot] + T::ZBYTES, T::NW, w, voff, T::VLOADS, T::VMOD);
  }

  // eta_k z + shift for this lane's feature (log2 units) and tokens
  // 16 ks + 8 g + [0, 8) of the tile in `slot`: K_m itself for
  // shift = rho_k log2(e), K_m less an offset m for shift = rho_k log2(e) - m
  __device__ __forceinline__ void keys(int slot, int ks, float shift, float (&k)[8]) const {
    const u32x4 zr = tr_operand<D>(zs(slot), zb[0], zb[1], ks);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      k[2 * j] = ekf * bf_lo(zr[j]) + shift;
      k[2 * j + 1] = ekf * bf_hi(zr[j]) + shift;
    }
  }

  // maximum of this lane's keys over the valid tokens of tile it, staged in `slot`
  __device__ __forceinline__ float tile_max(int it, int slot) const {
    const int valid = cend - (cbeg + it * kBT);  // tokens of the tile inside the chunk
    float mx = kNegInf;
#pragma unroll
    for (int ks = 0; ks < T::KT; ++ks) {
      float k[8];
      keys(slot, ks, rkf, k);
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, 16 * ks + 8 * g + j < valid ? k[j] : kNegInf);
    }
    return mx;
  }

  // psi(K_m) for the tokens of the tile in `slot` into the psi buffer `pd`:
  // thread -> token tid / PARTS, features FPT (tid % PARTS) + [0, FPT). psi
  // is a softmax over the row, so any per-row offset gives the same result:
  // without kMax the offset is 0 and a valid row whose exp-sum leaves
  // [2^-60, 2^63] sets `bad` (the workgroup then redoes the pass with kMax,
  // offset = the row maximum).
  template <bool kMax>
  __device__ __forceinline__ void psi_phase(int slot, char* pd, int valid, bool& bad) const {
    constexpr int FPT = T::FPT, CH = FPT / 8;
    float x[FPT];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(zs(slot) + poff[k]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * k + 2 * j] = pe[8 * k + 2 * j] * bf_lo(raw[j]) + pr[8 * k + 2 * j];
        x[8 * k + 2 * j + 1] = pe[8 * k + 2 * j + 1] * bf_hi(raw[j]) + pr[8 * k + 2 * j + 1];
      }
    }
    if constexpr (kMax) {
      float mx = x[0];
#pragma unroll
      for (int f = 1; f < FPT; ++f) mx = fmaxf(mx, x[f]);
      mx = group_max<T::PARTS>(mx);
#pragma unroll
      for (int f = 0; f < FPT; ++f) x[f] -= mx;
    }
    float sm = 0.f;
#pragma unroll
    for (int f = 0; f < FPT; ++f) {
      x[f] = exp2_fast(x[f]);
      sm += x[f];
    }
    sm = group_sum<T::PARTS>(sm);
    if constexpr (!kMax) {
      if ((int)threadIdx.x / T::PARTS < valid && !(sm >= 0x1p-60f && sm <= kOverflow)) bad = true;
    }
    const float inv = 1.f / sm;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const float* y = x + 8 * k;
      const u32x4 pk{pack2(y[0] * inv, y[1] * inv), pack2(y[2] * inv, y[3] * inv), pack2(y[4] * inv, y[5] * inv),
                     pack2(y[6] * inv, y[7] * inv)};
      *reinterpret_cast<u32x4*>(pd + poff[k]) = pk;
    }
  }

  // E of this lane's feature for every k-step of the tile in `slot` (its sum
  // accumulated into lsum), as the MFMA B operands. rkm = rho_k log2(e) less
  // the feature's offset; tokens from `valid` on belong to no chunk entry:
  // E = 0 there.
  __device__ __forceinline__ void e_phase(int slot, int valid, float rkm, float& lsum, u32x4 (&ef)[T::KT]) const {
    const bool full = valid >= kBT;
#pragma unroll
    for (int ks = 0; ks < T::KT; ++ks) {
      float e[8];
      keys(slot, ks, rkm, e);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e[j] = full || 16 * ks + 8 * g + j < valid ? exp2_fast(e[j]) : 0.f;
        lsum += e[j];
      }
      ef[ks] = u32x4{pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
    }
  }

  // the two products of the tile in `slot` with psi from `psr`: G^T += V^T E
  // and H^T += psi^T E; the operand of MFMA i + AH is read from LDS before
  // MFMA i
  __device__ __forceinline__ void products(int slot, const char* psr, const u32x4 (&ef)[T::KT],
                                           f32x16 (&accg)[NMV], f32x16 (&acch)[NMF]) const {
    constexpr int NB = NMV + NMF, NI = T::KT * NB, AH = GECKO_CHUNK_AH;
    const char* vsb = vs(slot);
    u32x4 op[AH + 1];
#pragma unroll
    for (int i = 0; i < NI + AH; ++i) {
      if (i < NI) {
        const int ks = i / NB, b = i % NB;
        op[i % (AH + 1)] = b < NMV ? tr_operand<DV>(vsb, vb[0][b], vb[1][b], ks)
                                   : tr_operand<D>(psr, pb[0][b - NMV], pb[1][b - NMV], ks);
      }
      if (i >= AH) {
        const int m = i - AH, ks = m / NB, b = m % NB;
        if (b < NMV) accg[b] = mfma_bf16(op[m % (AH + 1)], ef[ks], accg[b]);
        else acch[b - NMV] = mfma_bf16(op[m % (AH + 1)], ef[ks], acch[b - NMV]);
      }
    }
  }

  // wait until this lane's staging loads have landed except those of the
  // last k tiles issued (k >= 0, uniform)
  __device__ __forceinline__ void wait_leaving(int k) const {
    if constexpr (kNS >= 6) if (k >= 3) { wait_vmem_leave<3 * T::LOADS>(); return; }
    if constexpr (kNS >= 5) if (k >= 2) { wait_vmem_leave<2 * T::LOADS>(); return; }
    if constexpr (kNS >= 4) if (k >= 1) { wait_vmem_leave<T::LOADS>(); return; }
    wait_vmem();
  }

  // Tile it in LDS stage SLOT (a constant, so LDS offsets fold into the
  // reads), psi(it) in buffer SLOT & 1 (kNS is even, so that is it & 1) and
  // E(it) in ef: stage tile it + kNS - 1 into the stage of tile it - 1; the
  // products of tile it, and in the same stretch of code (no barrier
  // between, so that the VALU work runs under the MFMAs) psi and E of tile
  // it + 1 (landed), into the other psi buffer and ef. Past the last tile
  // that second part reads a stale stage with every token outside the chunk
  // (E = 0, no range check), and its psi is never read. Then wait for tile
  // it + 2 and end at the barrier.
  template <int SLOT, bool kMax>
  __device__ __forceinline__ void tile(int it, float rkm, float& lsum, f32x16 (&accg)[NMV], f32x16 (&acch)[NMF],
                                       u32x4 (&ef)[T::KT], bool& bad) const {
    if (it + kNS - 1 < ntiles) {
      stage_z(it + kNS - 1, (SLOT + kNS - 1) % kNS);
      stage_v(it + kNS - 1, (SLOT + kNS - 1) % kNS);
    }
    u32x4 efn[T::KT];
    const int valid1 = cend - (cbeg + (it + 1) * kBT);
    products(SLOT, psb[SLOT & 1], ef, accg, acch);
    psi_phase<kMax>((SLOT + 1) % kNS, psb[(SLOT + 1) & 1], valid1, bad);
    e_phase((SLOT + 1) % kNS, valid1, rkm, lsum, efn);
    // tiles issued after tile it + 2: it + 3 .. min(it + kNS - 1, ntiles - 1)
    wait_leaving(min(kNS - 3, ntiles - 3 - it));
    barrier_lds();  // psi(it + 1) written; tile it + 2 landed; stage of tile it free
#pragma unroll
    for (int ks = 0; ks < T::KT; ++ks) ef[ks] = efn[ks];
  }

  template <int S, bool kMax>
  __device__ __forceinline__ void tiles_from(int it, float rkm, float& lsum, f32x16 (&accg)[NMV],
                                             f32x16 (&acch)[NMF], u32x4 (&ef)[T::KT], bool& bad) const {
    if (it + S < ntiles) {
      tile<S, kMax>(it + S, rkm, lsum, accg, acch, ef, bad);
      if constexpr (S + 1 < kNS) tiles_from<S + 1, kMax>(it, rkm, lsum, accg, acch, ef, bad);
    }
  }

  // one pass over the chunk with a fixed per-feature offset msub for E and
  // (kMax) the row maximum or (otherwise) no offset for psi; returns the
  // exp-sum of E and sets `bad` as psi_phase does. Expects tile 0 staged in
  // stage 0 and landed (every wave past a barrier); stages tiles
  // 1 .. kNS - 2 itself.
  template <bool kMax>
  __device__ __forceinline__ float pass(float msub, f32x16 (&accg)[NMV], f32x16 (&acch)[NMF], bool& bad) const {
#pragma unroll
    for (int i = 1; i < kNS - 1; ++i)
      if (i < ntiles) {
        stage_z(i, i);
        stage_v(i, i);
      }
    const float rkm = rkf - msub;
    float lsum = 0.f;
    u32x4 ef[T::KT];
    psi_phase<kMax>(0, psb[0], cend - cbeg, bad);
    e_phase(0, cend - cbeg, rkm, lsum, ef);
    // tiles issued after tile 1: 2 .. min(kNS - 2, ntiles - 1)
    wait_leaving(min(kNS - 3, ntiles - 2));
    barrier_lds();  // psi(0) written; tile 1 landed
    for (int it = 0; it < ntiles; it += kNS) tiles_from<0, kMax>(it, rkm, lsum, accg, acch, ef, bad);
    return other_half_sum(lsum);
  }
};

template <int D, int DV>
__global__ __launch_bounds__(2 * D, 1) void awm_chunk_bf16_kernel(ChunkArgs a) {
  using T = ChunkTile<D, DV>;
  constexpr int NMV = DV / 32;
  constexpr int NMF = D / 32;
  // each stage its own LDS variable (see ChunkLoop::sb)
  __shared__ __attribute__((aligned(16))) char S0[T::STAGE];
  __shared__ __attribute__((aligned(16))) char S1[T::STAGE];
  __shared__ __attribute__((aligned(16))) char S2[kNS > 2 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char S3[kNS > 3 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char S4[kNS > 4 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char S5[kNS > 5 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char PS0[T::ZBYTES];
  __shared__ __attribute__((aligned(16))) char PS1[T::ZBYTES];
  const int64_t bh = blockIdx.x / a.nmem;
  const int64_t t = blockIdx.x % a.nmem;
  ChunkLoop<D, DV> L;
  char* const all[6] = {S0, S1, S2, S3, S4, S5};
  char* stages[kNS];
#pragma unroll
  for (int i = 0; i < kNS; ++i) stages[i] = all[i];
  L.init(a, bh, t, stages, PS0, PS1);

  f32x16 accg[NMV], acch[NMF];
#pragma unroll
  for (int i = 0; i < NMV; ++i) accg[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < NMF; ++i) acch[i] = f32x16{};

  L.stage_z(0, 0);
  L.stage_v(0, 0);
  wait_vmem();
  __syncthreads();
  float m = other_half_max(L.tile_max(0, 0));  // the first token is always valid
  bool psi_bad = false;
  float ltot = L.template pass<false>(m, accg, acch, psi_bad);
  const bool e_bad = !(ltot <= kOverflow);
  if (__syncthreads_or(e_bad || psi_bad)) {
    // the offset-free psi left its range, or a key exceeded the first tile's
    // maximum by 2^63: redo with the row maxima in psi and (for the latter)
    // the exact per-feature maximum in E
    if (__syncthreads_or(e_bad)) {
      float mx = kNegInf;
      for (int it = 0; it < L.ntiles; ++it) {
        L.stage_z(it, 0);
        wait_vmem();
        __syncthreads();
        mx = fmaxf(mx, L.tile_max(it, 0));
        __syncthreads();
      }
      m = other_half_max(mx);
    }
#pragma unroll
    for (int i = 0; i < NMV; ++i) accg[i] = f32x16{};
#pragma unroll
    for (int i = 0; i < NMF; ++i) acch[i] = f32x16{};
    L.stage_z(0, 0);
    L.stage_v(0, 0);
    wait_vmem();
    __syncthreads();
    ltot = L.template pass<true>(m, accg, acch, psi_bad);
  }

  const int f = 32 * L.w + L.lq;
  const int g = L.g;
  const int64_t row = bh * a.nmem + t;
  if (g == 0) {
    a.cmax[row * D + f] = m;
    a.csum[row * D + f] = ltot;
  }
  // G^T accumulators as they are: block mv, wave w, lane, 16 registers
  // (column f, value rows 32 mv + 8 (r >> 2) + 4 g + (r & 3)); the scan reads
  // them back in the same layout
#pragma unroll
  for (int mv = 0; mv < NMV; ++mv) {
    f32x4* gt = reinterpret_cast<f32x4*>(a.g + ((((row * NMV + mv) * T::NW + L.w) * 64) + L.lane) * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) gt[q] = f32x4{accg[mv][4 * q], accg[mv][4 * q + 1], accg[mv][4 * q + 2], accg[mv][4 * q + 3]};
  }
  // H^T accumulators (column f, rows f' = 32 mf + 8 (r >> 2) + 4 g + (r & 3)) as
  // the scan's B operand: k-step ks = 2 mf + p holds registers 8 p .. 8 p + 7,
  // i.e. f' = 32 mf + 16 p + 8 (e >> 2) + 4 g + (e & 3) for element e; stored
  // [ks][wave][lane][8] so that a scan load of 16 bytes per lane is contiguous
  uint16_t* ht = a.hm + row * (int64_t)D * D;
#pragma unroll
  for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const f32x16& x = acch[mf];
      const int o = 8 * pp;
      const u32x4 val{pack2(x[o], x[o + 1]), pack2(x[o + 2], x[o + 3]), pack2(x[o + 4], x[o + 5]),
                      pack2(x[o + 6], x[o + 7])};
      st16(ht + ((int64_t)((2 * mf + pp) * T::NW + L.w) * 64 + L.lane) * 8, val);
    }
}

// ---------------------------------------------------------------- z prefix
// One thread per (batch*head, feature): running z^t = 2^M L in log2 space.
// Loads are batched ahead of the dependent recurrence.
__global__ void awm_zscan_kernel(const float* __restrict__ cmax, const float* __restrict__ csum,
                                 float* __restrict__ decay, float* __restrict__ wscale, int64_t nmem, int D) {
  constexpr int kBatch = 8;
  const int f = threadIdx.x;
  if (f >= D) return;
  const int64_t off = (int64_t)blockIdx.x * nmem * D + f;
  const float* pm = cmax + off;
  const float* pl = csum + off;
  float* pd = decay + off;
  float* pw = wscale + off;
  float M = kNegInf, L = 0.f;
  for (int64_t t0 = 0; t0 < nmem; t0 += kBatch) {
    const int cnt = (int)min((int64_t)kBatch, nmem - t0);
    float mb[kBatch], lb[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      mb[j] = j < cnt ? pm[j * D] : 0.f;
      lb[j] = j < cnt ? pl[j * D] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j < cnt) {
        const float Mn = fmaxf(M, mb[j]);
        const float old = (M == kNegInf) ? 0.f : L * exp2_fast(M - Mn);
        const float cur = exp2_fast(mb[j] - Mn);
        const float Ln = old + lb[j] * cur;
        pd[j * D] = old / Ln;  // z^{t-1} / z^t
        pw[j * D] = cur / Ln;  // 2^{m_t} / z^t
        M = Mn;
        L = Ln;
      }
    }
    pm += kBatch * D;
    pl += kBatch * D;
    pd += kBatch * D;
    pw += kBatch * D;
  }
}

// ---------------------------------------------------------------- scan
struct ScanArgs {
  const float* g;      // chunk-pass accumulators of G^T, [bh][t][dv/32][d/32][64 lanes][16]
  const uint16_t* hm;  // [bh][t][d/16][d/32][64 lanes][8] bf16, see the chunk pass
  const float* cmax;   // [bh][t][d] (log2 units)
  const float* csum;   // [bh][t][d]
  uint16_t* snap;      // [bh][nsnap][d][dv]: slot t + has_prev holds the state after step t
  float* mstate;       // streaming: fp32 M'^T in this kernel's register layout
                       //   [bh][dv/32][d/32][64 lanes][16]; read if has_prev, written if stream
  const float* zstate; // streaming: (M, L) per feature before the call [bh][d][2], read if has_prev
  float* zfinal;       // streaming: (M, L) per feature after the call [bh][d][2], written if stream
  float* snap32;       // optional: every snapshot again in float32 [bh][nsnap][d][dv]
  int64_t nmem, nsnap;
  int no_delta;        // drop the H_t M' term (test variant)
  int has_prev, stream;
};

// Operands of one scan step for one lane, loaded ahead of use.
template <int D>
struct ScanStep {
  static constexpr int KS = D / 16;
  u32x4 hf[KS];  // H_t[f][f'] for k-step ks: f' = 16 ks + 8 (e >> 2) + 4 g + (e & 3)
  f32x4 gv[4];   // G_t^T of this lane's 16 accumulator cells
  float cm, cs;  // max (log2) and exp-sum of feature f over chunk t
};

// One workgroup per (batch*head, 32-value slice j of M'), working on the
// transpose: wave w holds M'^T[v][f] for features f = 32 w + lq (one per
// lane, both halves of the wave) and the slice's values v in MFMA
// accumulator layout (register r: v = 8 (r >> 2) + 4 g + (r & 3)), which is
// also the layout in which the chunk pass stored G^T, so a lane's G_t is 64
// contiguous bytes. A step is
//   M'^T <- decay_f M'^T + wscale_f (G_t^T - M'^T H_t^T)
// with decay_f = z^{t-1}/z^t and wscale_f = 2^{m_t}/z^t from the running
// per-feature exp-sum z^t = 2^M L (kept in log2 form by each lane for its
// feature). M'^T H_t^T is one MFMA chain: A = M'^T read (transposed) from a
// bf16 copy of the slice in LDS ([f][v]), B = rows of H_t from HBM. The copy
// is also the snapshot that chunk t + 2 reads. Step operands are prefetched
// kDepth - 1 steps ahead; block b handles slice b / BH of batch*head b % BH, so
// with BH a multiple of 8 all slices of a head run on one XCD.
template <int D, int DV, bool kNoDelta>
__global__ __launch_bounds__(2 * D, 1) void awm_scan_bf16_kernel(ScanArgs a) {
  constexpr int NMV = DV / 32;
  constexpr int NW = D / 32;
  constexpr int KS = D / 16;
  constexpr int kDepth = 4;
  __shared__ __attribute__((aligned(16))) uint16_t mt[2][D * 32];  // [f][v] bf16

  const int64_t BH = gridDim.x / NMV;
  const int64_t bh = blockIdx.x % BH;
  const int j = (int)(blockIdx.x / BH);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, lq = lane & 31;
  const int f = 32 * w + lq;
  const int64_t nmem = a.nmem;
  // transpose read of the copy, in the k order of the H operand: element e =
  // 4 jj + e' of lane (lq, g) at k-step ks is mt[16 ks + 8 jj + 4 g + e'][lq];
  // source lane s of each 16-lane group points at row 16 ks + 8 jj + 4 g +
  // s / 4, columns 16 (group % 2) + 4 (s % 4) + [0, 4). Rows are 64 bytes, so
  // the 32 lanes of a pass read 4 whole rows: every LDS bank once.
  const int sl = lane & 15, grp2 = (lane >> 4) & 1;
  const int trb = (4 * g + (sl >> 2)) * 64 + (16 * grp2 + 4 * (sl & 3)) * 2;

  ScanStep<D> ring[kDepth];
  // operands of step t in three parts: H_t k-steps [0, KS / 2), [KS / 2, KS);
  // then G_t^T and the chunk's max and sum
  auto load_part = [&](int64_t t, ScanStep<D>& q, int part) {
    const int64_t row = bh * nmem + t;
    if (part < 2) {
      const uint16_t* ht = a.hm + row * (int64_t)D * D + ((int64_t)w * 64 + lane) * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        if (ks / (KS / 2) == part) q.hf[ks] = ld16(ht + (int64_t)ks * NW * 64 * 8);
    } else {
      const f32x4* gt = reinterpret_cast<const f32x4*>(a.g + ((((row * NMV + j) * NW + w) * 64) + lane) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) q.gv[i] = gt[i];
      q.cm = a.cmax[row * D + f];
      q.cs = a.csum[row * D + f];
    }
  };

  f32x16 mst = f32x16{};
  float zM = kNegInf, zL = 0.f;
  int buf = 0;
  // this lane's 16 cells of the state in the streaming state arrays
  const int64_t scell = (((bh * NMV + j) * NW + w) * 64 + lane) * 16;
  const int hp = a.has_prev;
  // one 32-value slice of a snapshot from the bf16 copy in LDS
  auto write_snap = [&](int64_t slot, const uint16_t* src) {
    uint16_t* sn = a.snap + (bh * a.nsnap + slot) * (int64_t)D * DV + 32 * j;
#pragma unroll
    for (int e = tid; e < D * 4; e += 2 * D) {
      const int r = e >> 2, cc = (e & 3) * 8;
      st16(sn + (int64_t)r * DV + cc, ld16(&src[r * 32 + cc]));
    }
  };
  const int64_t last = nmem - 1;
  // nxt: the ring slot that the operands of step t + kDepth - 1 go into. A
  // wave waits while its loads are issued (about 900 cycles for a step's
  // 48 KiB through the CU's load path), so they are issued in three parts
  // at the step's own waits: after the products are issued, after the state
  // copy is written and after the snapshot is stored. (All at the end of the
  // step the scan took 89 us at 128K tokens, in three parts 78 us.)
  auto step = [&](int64_t t, const ScanStep<D>& q, ScanStep<D>& nxt) {
    // running denominator of feature f
    const float Mn = fmaxf(zM, q.cm);
    const float old = zM == kNegInf ? 0.f : zL * exp2_fast(zM - Mn);
    const float cur = exp2_fast(q.cm - Mn);
    const float Ln = old + q.cs * cur;
    const float inv = 1.f / Ln;
    const float dc = old * inv, ws = cur * inv;
    zM = Mn;
    zL = Ln;
    f32x16 p0 = f32x16{}, p1 = f32x16{};
    if constexpr (!kNoDelta) {  // at t = 0 the copy holds M'_1 = 0
      const char* mb = reinterpret_cast<const char*>(mt[buf]) + trb;
#pragma unroll
      for (int ks = 0; ks < KS; ks += 2) {
        const u32x2 a0 = lds_read_tr(mb + (16 * ks) * 64), a1 = lds_read_tr(mb + (16 * ks + 8) * 64);
        const u32x2 b0 = lds_read_tr(mb + (16 * ks + 16) * 64), b1 = lds_read_tr(mb + (16 * ks + 24) * 64);
        p0 = mfma_bf16(u32x4{a0[0], a0[1], a1[0], a1[1]}, q.hf[ks], p0);
        p1 = mfma_bf16(u32x4{b0[0], b0[1], b1[0], b1[1]}, q.hf[ks + 1], p1);
      }
    }
    const int64_t tn = min(t + kDepth - 1, last);
    load_part(tn, nxt, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) mst[r] = dc * mst[r] + ws * (q.gv[r >> 2][r & 3] - (p0[r] + p1[r]));
    // bf16 copy: column f, values 8 qq + 4 g + [0, 4)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const u32x2 pk{pack2(mst[4 * qq], mst[4 * qq + 1]), pack2(mst[4 * qq + 2], mst[4 * qq + 3])};
      *reinterpret_cast<u32x2*>(&mt[buf ^ 1][f * 32 + 8 * qq + 4 * g]) = pk;
    }
    load_part(tn, nxt, 1);
    __syncthreads();
    // snapshot rows f of the state after step t, values 32 j .. 32 j + 31:
    // 64 bytes per row
    write_snap(t + hp, mt[buf ^ 1]);
    load_part(tn, nxt, 2);
    if (a.snap32) {  // float32 copy: row f, values 32 j + 8 qq + 4 g + [0, 4)
      float* s32 = a.snap32 + (bh * a.nsnap + t + hp) * (int64_t)D * DV + (int64_t)f * DV + 32 * j + 4 * g;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        *reinterpret_cast<f32x4*>(s32 + 8 * qq) = f32x4{mst[4 * qq], mst[4 * qq + 1], mst[4 * qq + 2], mst[4 * qq + 3]};
    }
    buf ^= 1;
  };

  if (hp) {
    // continue a sequence: the state and the running denominator carried
    // over from the previous call; its bf16 copy is both the first MFMA
    // operand and snapshot slot 0 (read by the call's first chunk)
    const f32x4* ms = reinterpret_cast<const f32x4*>(a.mstate + scell);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = ms[q];
#pragma unroll
      for (int i = 0; i < 4; ++i) mst[4 * q + i] = x[i];
    }
    zM = a.zstate[(bh * D + f) * 2];
    zL = a.zstate[(bh * D + f) * 2 + 1];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const u32x2 pk{pack2(mst[4 * qq], mst[4 * qq + 1]), pack2(mst[4 * qq + 2], mst[4 * qq + 3])};
      *reinterpret_cast<u32x2*>(&mt[0][f * 32 + 8 * qq + 4 * g]) = pk;
    }
    __syncthreads();
    write_snap(0, mt[0]);
  } else {
    // M'_1 = 0
    for (int e = tid; e < D * 32 / 8; e += 2 * D) st16(&mt[0][8 * e], u32x4{0u, 0u, 0u, 0u});
    __syncthreads();
  }
  // Steady state without branches, so that the compiler can count the loads
  // in flight exactly; loads past the last step re-read it (unused). Step t
  // uses slot t mod kDepth and fills slot (t - 1) mod kDepth, which step
  // t - 1 is done with, with the operands of step t + kDepth - 1.
#pragma unroll
  for (int k = 0; k < kDepth - 1; ++k)
#pragma unroll
    for (int part = 0; part < 3; ++part) load_part(min((int64_t)k, last), ring[k], part);
  int64_t t0 = 0;
  for (; t0 + kDepth <= nmem; t0 += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) step(t0 + k, ring[k], ring[(k + kDepth - 1) % kDepth]);
  }
#pragma unroll
  for (int k = 0; k < kDepth; ++k)
    if (t0 + k < nmem) step(t0 + k, ring[k], ring[(k + kDepth - 1) % kDepth]);

  if (a.stream) {  // the state after the last step, for the next call
    f32x4* ms = reinterpret_cast<f32x4*>(a.mstate + scell);
#pragma unroll
    for (int q = 0; q < 4; ++q) ms[q] = f32x4{mst[4 * q], mst[4 * q + 1], mst[4 * q + 2], mst[4 * q + 3]};
    if (j == 0 && g == 0) {
      a.zfinal[(bh * D + f) * 2] = zM;
      a.zfinal[(bh * D + f) * 2 + 1] = zL;
    }
  }
}

// ---------------------------------------------------------------- streaming state
// A new sequence whose first call enters no chunk into the memory: M' = 0 and
// an empty running denominator (M, L) = (-inf, 0).
__global__ void stream_reset_kernel(float* __restrict__ mstate, float* __restrict__ zstate, int64_t mcells,
                                    int64_t zfeat) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mcells; i += stride) mstate[i] = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < zfeat; i += stride) {
    zstate[2 * i] = kNegInf;
    zstate[2 * i + 1] = 0.f;
  }
}

// End of a streaming call, after every kernel that reads the old carried
// chunk: rows [row0, row0 + rows) of each (b, h) slab of Z' and V become the
// carried chunk, and the scan's final running denominator the carried one.
// Block b serves slab b / per_bh; 16-byte copies (d and dv are multiples of 8).
__global__ void stream_finish_kernel(const uint16_t* __restrict__ z, const uint16_t* __restrict__ v,
                                     uint16_t* __restrict__ zc, uint16_t* __restrict__ vc,
                                     const float* __restrict__ zfinal, float* __restrict__ zstate, int64_t n,
                                     int64_t c, int d, int dv, int64_t row0, int64_t rows, int per_bh) {
  const int64_t bh = blockIdx.x / per_bh;
  const int part = (int)(blockIdx.x % per_bh);
  const int64_t zch = rows * d / 8, vch = rows * dv / 8;
  const u32x4* zs = reinterpret_cast<const u32x4*>(z + (bh * n + row0) * d);
  const u32x4* vs = reinterpret_cast<const u32x4*>(v + (bh * n + row0) * dv);
  u32x4* zd = reinterpret_cast<u32x4*>(zc + bh * c * d);
  u32x4* vd = reinterpret_cast<u32x4*>(vc + bh * c * dv);
  const int64_t stride = (int64_t)per_bh * blockDim.x;
  for (int64_t i = (int64_t)part * blockDim.x + threadIdx.x; i < zch + vch; i += stride) {
    if (i < zch)
      zd[i] = zs[i];
    else
      vd[i - zch] = vs[i - zch];
  }
  if (zfinal && part == 0)
    for (int k = threadIdx.x; k < 2 * d; k += blockDim.x) zstate[bh * 2 * d + k] = zfinal[bh * 2 * d + k];
}

template <int D, int DV>
hipError_t launch_chunk(const ChunkArgs& a, int64_t BH, hipStream_t s) {
  static_assert(ChunkTile<D, DV>::LDS_BYTES <= 160 * 1024, "LDS per workgroup");  // all static
  hipLaunchKernelGGL((awm_chunk_bf16_kernel<D, DV>), dim3((unsigned)(BH * a.nmem)), dim3(ChunkTile<D, DV>::THREADS),
                     0, s, a);
  return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_scan(const ScanArgs& a, int64_t BH, hipStream_t s) {
  const dim3 grid((unsigned)(BH * (DV / 32)));
  if (a.no_delta)
    hipLaunchKernelGGL((awm_scan_bf16_kernel<D, DV, true>), grid, dim3(2 * D), 0, s, a);
  else
    hipLaunchKernelGGL((awm_scan_bf16_kernel<D, DV, false>), grid, dim3(2 * D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_awm_chunk_bf16(const Problem& p, const Workspace& w, hipStream_t s) {
  ChunkArgs a;
  a.z = static_cast<const uint16_t*>(p.z);
  a.v = static_cast<const uint16_t*>(p.v);
  a.eta_k = p.eta_k; a.rho_k = p.rho_k;
  a.g = w.g; a.hm = static_cast<uint16_t*>(w.h); a.cmax = w.cmax; a.csum = w.csum;
  a.zprev = static_cast<const uint16_t*>(p.zprev);
  a.vprev = static_cast<const uint16_t*>(p.vprev);
  a.n = p.n; a.c = p.c; a.nmem = p.nmem; a.H = (int)p.H; a.has_prev = p.has_prev ? 1 : 0;
  const int64_t BH = p.B * p.H;
  switch (p.d * 1000 + p.dv) {
#define GECKO_AWM_SHAPE(D_, DV_) \
  case D_ * 1000 + DV_:          \
    return launch_chunk<D_, DV_>(a, BH, s);
    GECKO_BF16_SHAPES(GECKO_AWM_SHAPE)
#undef GECKO_AWM_SHAPE
  }
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
  a.g = w.g; a.hm = static_cast<const uint16_t*>(w.h); a.cmax = w.cmax; a.csum = w.csum;
  a.snap = static_cast<uint16_t*>(w.snap); a.nmem = p.nmem; a.nsnap = p.nsnap;
  a.no_delta = (p.flags & GECKO_AWM_NO_DELTA_BIT) ? 1 : 0;
  a.mstate = p.mstate; a.zstate = p.zstate; a.zfinal = w.zfinal; a.snap32 = w.snap32;
  a.has_prev = p.has_prev ? 1 : 0; a.stream = p.stream ? 1 : 0;
  const int64_t BH = p.B * p.H;
  switch (p.d * 1000 + p.dv) {
#define GECKO_AWM_SHAPE(D_, DV_) \
  case D_ * 1000 + DV_:          \
    return launch_scan<D_, DV_>(a, BH, s);
    GECKO_BF16_SHAPES(GECKO_AWM_SHAPE)
#undef GECKO_AWM_SHAPE
  }
  return hipErrorInvalidValue;
}

hipError_t launch_stream_reset(float* mstate, float* zstate, int64_t BH, int64_t d, int64_t dv, hipStream_t s) {
  const int64_t mcells = BH * d * dv, zfeat = BH * d;
  const int64_t blocks = std::min<int64_t>((mcells + 255) / 256, 1024);
  hipLaunchKernelGGL(stream_reset_kernel, dim3((unsigned)blocks), dim3(256), 0, s, mstate, zstate, mcells, zfeat);
  return hipGetLastError();
}

hipError_t launch_stream_finish(const Problem& p, const Workspace& w, void* zcarry, void* vcarry, float* zstate,
                                int64_t row0, int64_t rows, hipStream_t s) {
  const int64_t BH = p.B * p.H;
  const int64_t chunks16 = rows * (p.d + p.dv) / 8;
  const int per_bh = (int)std::max<int64_t>(1, std::min<int64_t>((chunks16 + 255) / 256, 32));
  hipLaunchKernelGGL(stream_finish_kernel, dim3((unsigned)(BH * per_bh)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(p.z), static_cast<const uint16_t*>(p.v),
                     static_cast<uint16_t*>(zcarry), static_cast<uint16_t*>(vcarry),
                     p.nmem > 0 ? w.zfinal : nullptr, zstate, p.n, p.c, (int)p.d, (int)p.dv, row0, rows, per_bh);
  return hipGetLastError();
}

}  // namespace gecko
