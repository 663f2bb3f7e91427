// Sliding chunk attention with the memory readout fused into its epilogue,
// bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Computes, for every query row i of chunk s (Gecko summary, paper.rainbus.top,
// "Method steps" (3) and (5)):
//   O_i = softmax_j(q_i . k_j) v_j over keys j of chunks s-1 and s with j <= i
//         + psi(Q_m,i) M'_{s-1}            (readout; chunks s >= 3, 1-based)
//
// Work decomposition: one workgroup = 256 consecutive queries of one chunk of
// one (batch, head). With dv = 256: 8 waves x 32 queries, two waves per SIMD
// so that one wave's exponentials overlap the other's matrix instructions;
// with dv <= 128: 4 waves x 64 queries, one wave per SIMD, each K / V operand
// read serving two MFMAs. The key window [(s-1)c, last query] is streamed in
// tiles of 32 keys; a wave skips the tiles that lie past all of its queries.
// (64-key tiles processed as two halves measured 1.4% slower at 128K tokens:
// twice the workgroup barriers, but each wave waits less at each.)
//
// Per 32-key tile and wave:
//   S^T (32 keys x 32 queries) = K Q^T            (A = K from LDS, B = Q in VGPRs)
//   P^T = exp2(S^T - m), lane-local per query (a query's 32 keys are split
//   between lane l and lane l ^ 32)
//   O^T (dv x 32 queries) += V^T P^T               (A = V^T from LDS, B = P in VGPRs)
// Holding O transposed keeps each query's accumulator column and its
// exp-sum in the same lane.
//
// Staging: K and V tiles go from HBM straight into LDS with buffer loads that
// write LDS (no registers, out-of-range rows read as zero). Rows are stored
// dense with their 16-byte chunks XOR-swizzled by row, so that the MFMA
// operand reads below hit each of the 64 LDS banks once per pass. V stays row-major
// in LDS; its transposed MFMA operand comes from the gfx950 LDS transpose
// read (ds_read_b64_tr_b16: in each 16-lane group, lane i receives column i
// of a 4-row x 16-column block).
//
// Pipeline: three LDS stages, one LDS array (the memory state for the
// readout goes there after the loop); tile kt+2 is loaded while tile kt is
// computed, and the wait at the end of a tile leaves tile kt+2's loads in
// flight. Operand reads from LDS run a few MFMAs ahead of their use, and the
// loop is unrolled by three tiles so every LDS address is a per-lane base
// plus a constant offset.
//
// Softmax offset: the first pass uses none (P = 2^s; bf16 and fp32 share the
// exponent range, so P keeps its relative precision at any scale). The final
// row sum shows whether that was safe: outside [2^-60, 2^63] (an overflow, or
// every term tiny) the workgroup finds the exact row maxima with a max-only
// pass and recomputes with them. No accumulator is ever rescaled inside the
// loop, and the row sums add the bf16 P values that multiply V.
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

// Scheduling of LDS operand reads: KAHEAD (VAHEAD) K (V) operands are read
// ahead of the MFMA that consumes them; SCHED adds group barriers that keep
// the compiler to that interleave.
#ifndef GECKO_SCA_SCHED
#define GECKO_SCA_SCHED 1
#endif
#ifndef GECKO_SCA_KAHEAD
#define GECKO_SCA_KAHEAD 2
#endif
#ifndef GECKO_SCA_VAHEAD
#define GECKO_SCA_VAHEAD 2
#endif
// (batch*head, chunk) pairs per group of the workgroup order (see the kernel)
#ifndef GECKO_SCA_GROUP
#define GECKO_SCA_GROUP 2
#endif

constexpr int kBM = 256;               // queries per workgroup
constexpr int kBN = 32;                // keys per tile
constexpr float kOverflow = 0x1p63f;   // row-sum range of the offset-free pass
constexpr float kUnderflow = 0x1p-60f;

// QB 32-query blocks per wave, NW waves per workgroup (32 QB NW = kBM).
// QB = 2 reads each K / V operand from LDS once for two MFMAs and gives a
// wave the whole register file of its SIMD (one wave per SIMD); QB = 1 runs
// two waves per SIMD with half the registers each.
template <int D, int DV, int QB>
struct ScaTile {
  static constexpr int NW = kBM / (32 * QB);
  static constexpr int THREADS = 64 * NW;
  static constexpr int KBYTES = kBN * D * 2;   // dense rows, chunk-swizzled
  static constexpr int VBYTES = kBN * DV * 2;
  // (K, V) stages in LDS: tile k + 2 is loaded while tile k is computed
  static constexpr int NSTAGE = 3;
  static constexpr size_t STAGE1 = (size_t)KBYTES + (size_t)VBYTES;  // one stage: K tile, then V tile
  static constexpr size_t STAGE_BYTES = NSTAGE * STAGE1;
  static constexpr size_t SNAP_BYTES = (size_t)D * DV * 2;  // the memory state for the readout
  // With the attention the state goes into the stage memory after the loop
  // (staged at kernel start into a region of its own it measured slower);
  // without it, into a region of its own at kernel start.
  static_assert(STAGE_BYTES >= SNAP_BYTES, "the state fits the stage memory");
  static constexpr size_t lds_bytes(bool sca, bool read) {
    return sca ? STAGE_BYTES : (read ? SNAP_BYTES : 0);
  }
  // 1 KiB pieces of a tile, and 16-byte loads per thread per tile (at least
  // one: with fewer pieces than waves, waves share pieces; see stage_rows)
  static constexpr int KPIECES = KBYTES / 1024;
  static constexpr int VPIECES = VBYTES / 1024;
  static constexpr int KLOADS = KBYTES / 16 / THREADS > 0 ? KBYTES / 16 / THREADS : 1;
  static constexpr int VLOADS = VBYTES / 16 / THREADS > 0 ? VBYTES / 16 / THREADS : 1;
  // the piece count handed to stage_rows: 0 (no sharing) unless the waves
  // have more loads than the tile has pieces
  static constexpr int KMOD = KPIECES < NW * KLOADS ? KPIECES : 0;
  static constexpr int VMOD = VPIECES < NW * VLOADS ? VPIECES : 0;
  static constexpr int LOADS = KLOADS + VLOADS;  // staging loads per lane and tile
  static_assert(32 * QB * NW == kBM, "tile shape");
};

// query blocks per wave for each built shape: with DV = 256, two blocks'
// accumulators (256 registers) plus the scores exceed the accumulator
// registers and the compiler shuttles values between register files.
template <int D, int DV>
struct ScaShape {
  static constexpr int QB = DV >= 256 ? 1 : 2;
};

// XOR swizzle of the 16-byte chunks of a staged K row, chosen so that the
// 16-byte operand reads below touch each of the 64 LDS banks once per pass of
// 16 lanes (V rows use vswz, for the 8-byte transpose reads).
template <int D>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (D == 128) return r & 15;
  if constexpr (D == 64) return (r >> 1) & 7;
  return (r >> 2) & 3;  // rows of 64 bytes: 4 chunks
}

struct ScaArgs {
  const uint16_t* z;
  const uint16_t* v;
  void* out;  // bf16 or float32 [bh][n][dv]
  const float* kappa_q;
  const float* nu_q;
  const float* kappa_k;
  const float* nu_k;   // read only when lse is set
  float* lse;          // optional [bh][n]: natural log-sum-exp of each query's logits
  float* o_sca;        // optional [bh][n][dv] float32: the attention output alone
  float* stats;        // optional [bh][n][2]: offset m and sum l of the bf16 weights 2^(s - m)
  const float* eta_q;
  const float* rho_q;
  const uint16_t* snap;  // [bh][nsnap][d][dv]; chunk s reads slot s - 2 + 2 has_prev (0-based)
  // streaming: the chunk before this call's first one (keys at rows -c .. -1)
  const uint16_t* zprev;   // [bh][c][d]
  const uint16_t* vprev;   // [bh][c][dv]
  int64_t n;
  int c, nchunks, nsnap, qtiles, nblocks, per_xcd, H, has_prev;
  int first_read;  // chunks before it read no memory (the sequence's first lag chunks)
  int lag;         // chunk s reads the state after chunks <= s - lag (2, or 1 for the chunk-wise variant)
  int prev;        // 1: the window holds the previous chunk; 0: the current chunk only
};

// The attention loop of one workgroup. Member functions rather than lambdas:
// lambdas inside a kernel are compiled for the host too, where the buffer and
// LDS builtins used here do not exist.
template <int D, int DV, int QB>
struct ScaLoop {
  using T = ScaTile<D, DV, QB>;
  static constexpr int NW = T::NW;
  static constexpr int KS = D / 16;   // 16-feature k-steps of Q K^T
  static constexpr int NMV = DV / 32; // 32-row blocks of O^T
  static constexpr int KCH = D / 8;   // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;  // 16-byte chunks per V row

  const uint16_t* zbh;
  const uint16_t* vbh;
  const uint16_t* zpv;  // carried chunk (keys at negative rows), streaming only
  const uint16_t* vpv;
  int cl;               // chunk length
  // stage i: K tile at sb[i], V tile at sb[i] + KBYTES (consecutive parts
  // of one LDS array).
  char* sb[T::NSTAGE];
  int n, kbeg, kend, ntiles, myq0, wave_q0, wave_last, w, g, lq;
  u32x4 qf[QB][KS];
  uint32_t koff[T::KLOADS], voff[T::VLOADS];
  int ka[KS];    // K operand byte offset in a stage for k-step ks, key block 0
  int va[NMV];   // V transpose-read byte offset in a stage for value block mv, key row 0

  __device__ __forceinline__ void init(const ScaArgs& a, uint32_t bh, int h, int n_, int s, int c, int q0,
                                       int qend, int w_, int lane, char* s0, char* s1, char* s2,
                                       const int (&va_)[NMV]) {
    n = n_;
    w = w_;
    wave_q0 = q0 + 32 * QB * w;
    g = lane >> 5;
    lq = lane & 31;
    myq0 = wave_q0 + lq;
    zbh = a.z + (size_t)bh * (size_t)n * D;
    vbh = a.v + (size_t)bh * (size_t)n * DV;
    cl = c;
    zpv = a.has_prev ? a.zprev + (size_t)bh * (size_t)c * D : nullptr;
    vpv = a.has_prev ? a.vprev + (size_t)bh * (size_t)c * DV : nullptr;
    sb[0] = s0;
    sb[1] = s1;
    sb[2] = s2;

    // query fragments: lane holds query 32 qb + lq of the wave, features
    // 16 ks + 8 g + [0, 8); rows past the tile repeat its last query
    const float* kq = a.kappa_q + h * D;
    const float* nq = a.nu_q + h * D;
    const float* kk = a.kappa_k + h * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = min(myq0 + 32 * qb, qend - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int f0 = 16 * ks + 8 * g;
        const u32x4 raw = ld16(zbh + (size_t)qrow * D + f0);
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = bf_lo(raw[j]);
          x[2 * j + 1] = bf_hi(raw[j]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (kq[f0 + i] * x[i] + nq[f0 + i]) * (kk[f0 + i] * kLog2e);
        qf[qb][ks] = u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
      }
    }

    // key window: the previous chunk (rows -c .. -1 are the carried chunk of
    // a streaming call; none in the chunk-wise variant) and this chunk up to
    // its last query
    kbeg = (a.prev && (s > 0 || a.has_prev)) ? (s - 1) * c : s * c;
    kend = qend;
    ntiles = (kend - kbeg + kBN - 1) / kBN;
    // last key any query of this wave can see; -1 (every key tile skipped)
    // if the wave holds no query of the tile
    wave_last = wave_q0 < kend ? min(wave_q0 + 32 * QB, kend) - 1 : -1;

    // staging offsets (constant over tiles). Load i of wave w covers the
    // 1 KiB piece NW i + w of the tile; lane l writes LDS chunk
    // (NW i + w) 64 + l, which is physical chunk p of row r holding
    // logical chunk p ^ swz(r).
#pragma unroll
    for (int i = 0; i < T::KLOADS; ++i) {
      const int P = stage_piece(NW, w, i, T::KMOD) * 64 + lane;
      const int r = P / KCH, p = P % KCH;
      koff[i] = (uint32_t)(r * D + 8 * (p ^ kswz<D>(r))) * 2u;
    }
#pragma unroll
    for (int i = 0; i < T::VLOADS; ++i) {
      const int P = stage_piece(NW, w, i, T::VMOD) * 64 + lane;
      const int r = P / VCH, p = P % VCH;
      voff[i] = (uint32_t)(r * DV + 8 * (p ^ vswz<DV>(r))) * 2u;
    }
    // Operand reads. K: lane reads row 32 mb + lq, logical chunk 2 ks + g;
    // the swizzle of row r depends on r mod 16 only, so mb adds a constant.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = lq * (D * 2) + 16 * ((2 * ks + g) ^ kswz<D>(lq));
    // V operand bases va[mv]: see v_operand_base.
#pragma unroll
    for (int mv = 0; mv < NMV; ++mv) va[mv] = va_[mv];
  }

  __device__ __forceinline__ void stage(int kt, int slot) const {
    // rows below 0 are the carried chunk (c is a multiple of the tile, so no
    // tile straddles); scalar selects, one load sequence
    const int row0 = kbeg + kt * kBN;
    const bool carried = row0 < 0;
    const int r = carried ? row0 + cl : row0;
    const int lim = carried ? cl : n;
    stage_rows(carried ? zpv : zbh, r, lim, D, sb[slot], NW, w, koff, T::KLOADS, T::KMOD);
    stage_rows(carried ? vpv : vbh, r, lim, DV, sb[slot] + T::KBYTES, NW, w, voff, T::VLOADS, T::VMOD);
  }

  __device__ __forceinline__ int k_addr(int mb, int ks) const { return ka[ks] + 32 * mb * (D * 2); }
  __device__ __forceinline__ int v_addr(int mv, int mb, int hh, int jj) const {
    return va[mv] + (32 * mb + 16 * hh + 8 * jj) * (DV * 2);
  }

  // S^T for keys 32 mb + [0, 32) of the tile in `slot`, every query block:
  // register r holds key 32 mb + 8 (r >> 2) + 4 g + (r & 3)
  __device__ __forceinline__ void qk(int slot, int mb, f32x16 (&sc)[QB]) const {
    const char* Kb = sb[slot];
    constexpr int AH = GECKO_SCA_KAHEAD;
    u32x4 op[AH + 1];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) sc[qb] = f32x16{};
#pragma unroll
    for (int i = 0; i < AH; ++i) op[i] = *reinterpret_cast<const u32x4*>(Kb + k_addr(mb, i));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + AH < KS) op[(ks + AH) % (AH + 1)] = *reinterpret_cast<const u32x4*>(Kb + k_addr(mb, ks + AH));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb] = mfma_bf16(op[ks % (AH + 1)], qf[qb][ks], sc[qb]);
    }
#if GECKO_SCA_SCHED
    __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
    for (int ks = 0; ks < KS - AH; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, QB * AH, 0);
#endif
  }

  __device__ __forceinline__ u32x4 v_operand(const char* Vb, int i, int mb) const {
    const int hh = i / NMV, mv = i % NMV;
    const u32x2 l2 = lds_read_tr(Vb + v_addr(mv, mb, hh, 0));
    const u32x2 h2 = lds_read_tr(Vb + v_addr(mv, mb, hh, 1));
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }

  // O^T += V^T P^T for the 32 keys of half mb; the V operand of MFMA i + AH
  // is read from LDS before MFMA i is issued.
  __device__ __forceinline__ void pv(int slot, int mb, const u32x4 (&pf)[QB][2], f32x16 (&oacc)[QB][NMV]) const {
    const char* Vb = sb[slot] + T::KBYTES;
    constexpr int NI = 2 * NMV;
    constexpr int AH = GECKO_SCA_VAHEAD;
    u32x4 op[AH + 1];
#pragma unroll
    for (int i = 0; i < AH; ++i) op[i] = v_operand(Vb, i, mb);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i + AH < NI) op[(i + AH) % (AH + 1)] = v_operand(Vb, i + AH, mb);
      const int hh = i / NMV, mv = i % NMV;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[qb][mv] = mfma_bf16(op[i % (AH + 1)], pf[qb][hh], oacc[qb][mv]);
    }
#if GECKO_SCA_SCHED
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);
#pragma unroll
    for (int i = 0; i < NI - AH; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, QB * AH, 0);
#endif
  }

  // last visible key offset within tile kt for query block qb of this lane
  __device__ __forceinline__ int last_visible(int kt, int qb) const {
    return min(myq0 + 32 * qb, kend - 1) - (kbeg + kt * kBN);
  }
  __device__ __forceinline__ bool needs_mask(int kt) const {
    const int kb = kbeg + kt * kBN;
    return kb + kBN - 1 > wave_q0 || kb + kBN > kend;
  }

  __device__ __forceinline__ float masked_max(const f32x16& sc, int kt, int mb, int qb) const {
    const int lim = last_visible(kt, qb);
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ko = 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
      mx = fmaxf(mx, ko > lim ? kNegInf : sc[r]);
    }
    return mx;
  }

  // whether half mb of key tile kt has a key some query of this wave sees
  // (wave-uniform)
  __device__ __forceinline__ bool live(int kt, int mb) const {
    return kt < ntiles && kbeg + kt * kBN + 32 * mb <= wave_last;
  }

  // P = 2^(S - m) (m = 0 unless kSub) for half mb of tile kt, packed as the
  // B operand of V^T P^T, and the row sums of the bf16 P that multiply V
  template <bool kSub>
  __device__ __forceinline__ void softmax_half(int kt, int mb, const float (&msub)[QB], const f32x16 (&sc)[QB],
                                               float (&lrun)[QB], u32x4 (&pf)[QB][2]) const {
    const bool masked = needs_mask(kt);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = exp2_fast(kSub ? sc[qb][r] - msub[qb] : sc[qb][r]);
      if (masked) {
        const int lim = last_visible(kt, qb);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
          e[r] = ko > lim ? 0.f : e[r];
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float* x = e + 8 * hh;
        pf[qb][hh] = u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
#pragma unroll
        for (int i = 0; i < 4; ++i) lrun[qb] = sum2_bf16(pf[qb][hh][i], lrun[qb]);
      }
    }
  }

  // S^T, softmax and O^T += V^T P^T for half mb of tile kt (in stage STG)
  template <int STG, bool kSub>
  __device__ __forceinline__ void half(int kt, int mb, const float (&msub)[QB], float (&lrun)[QB],
                                       f32x16 (&oacc)[QB][NMV]) const {
    f32x16 sc[QB];
    qk(STG, mb, sc);
    u32x4 pf[QB][2];
    softmax_half<kSub>(kt, mb, msub, sc, lrun, pf);
    pv(STG, mb, pf, oacc);
  }

  // Tile k of a pass in stage STG = k mod 3 (a constant, so that operand
  // addresses fold into the read offsets): stage this wave's share of tile
  // k + 2 into the stage tile k - 1 used (every wave is past it), compute the
  // halves of tile k that some query of the wave sees, wait for this wave's
  // share of tile k + 1 (tile k + 2's loads may stay in flight) and end at
  // the barrier.
  template <int STG, bool kSub>
  __device__ __forceinline__ void tile(int k, const float (&msub)[QB], float (&lrun)[QB],
                                       f32x16 (&oacc)[QB][NMV]) const {
    const bool ahead = k + 2 < ntiles;
    if (ahead) stage(k + 2, (STG + 2) % T::NSTAGE);
    if (live(k, 0)) half<STG, kSub>(k, 0, msub, lrun, oacc);
    if constexpr (kBN > 32)
      if (live(k, 1)) half<STG, kSub>(k, 1, msub, lrun, oacc);
    if (ahead)
      wait_vmem_leave<T::LOADS>();
    else
      wait_vmem();
    barrier_lds();  // tile k + 1 is in LDS for every wave; tile k + 2 may still be loading
  }

  // full pass with fixed softmax offsets; returns the row exp-sums
  template <bool kSub>
  __device__ __forceinline__ void pass(const float (&msub)[QB], float (&ltot)[QB], f32x16 (&oacc)[QB][NMV]) const {
    static_assert(T::NSTAGE == 3, "the tile loop is unrolled by the stage count");
    stage(0, 0);
    if (ntiles > 1) {
      stage(1, 1);
      wait_vmem_leave<T::LOADS>();
    } else {
      wait_vmem();
    }
    barrier_lds();
    float lrun[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lrun[qb] = 0.f;
    for (int k = 0; k < ntiles; k += 3) {
      tile<0, kSub>(k, msub, lrun, oacc);
      if (k + 1 < ntiles) tile<1, kSub>(k + 1, msub, lrun, oacc);
      if (k + 2 < ntiles) tile<2, kSub>(k + 2, msub, lrun, oacc);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ltot[qb] = other_half_sum(lrun[qb]);
  }

  // OR of a per-lane flag over the workgroup, through a word of the stage
  // memory (free between passes; every wave is past the pass's last barrier)
  __device__ __forceinline__ bool block_any(bool x) const {
    volatile int* flag = reinterpret_cast<volatile int*>(sb[0]);
    if (threadIdx.x == 0) *flag = 0;
    __syncthreads();
    if (x) *flag = 1;
    __syncthreads();
    const bool any = *flag != 0;
    __syncthreads();
    return any;
  }

  // O^T for the wave's queries, not yet divided by the row sums (lsum); the
  // row sums hold 2^(s - mout) summed over the visible keys
  __device__ __forceinline__ void run(f32x16 (&oacc)[QB][NMV], float (&lsum)[QB], float (&mout)[QB]) const {
    // First pass without an offset: P = 2^s. The row sums show whether that
    // was safe: if a valid query's sum lies outside [2^-60, 2^63] (some 2^s
    // overflowed, or every term is tiny), the workgroup finds the exact row
    // maxima with a max-only pass and redoes the pass with them.
    float msub[QB], ltot[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) msub[qb] = 0.f;
    pass<false>(msub, ltot, oacc);
    bool redo = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      redo = redo || (myq0 + 32 * qb < kend && !(ltot[qb] >= kUnderflow && ltot[qb] <= kOverflow));
    if (block_any(redo)) {
      float mx[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mx[qb] = kNegInf;
      for (int kt = 0; kt < ntiles; ++kt) {
        stage(kt, 0);
        wait_vmem();
        __syncthreads();
#pragma unroll
        for (int mb = 0; mb < kBN / 32; ++mb) {
          f32x16 sc[QB];
          qk(0, mb, sc);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) mx[qb] = fmaxf(mx[qb], masked_max(sc[qb], kt, mb, qb));
        }
        __syncthreads();
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        msub[qb] = other_half_max(mx[qb]);
#pragma unroll
        for (int i = 0; i < NMV; ++i) oacc[qb][i] = f32x16{};
      }
      pass<true>(msub, ltot, oacc);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      lsum[qb] = ltot[qb];
      mout[qb] = msub[qb];
    }
  }
};

// A operand i of the readout (value block mv = i / (2 NFB), feature block
// fb = (i / 2) % NFB, half hh = i % 2) from the staged state: the V^T
// transpose reads of ScaLoop::v_addr with features in the role of keys.
// A plain device function: a lambda in a kernel is compiled for the host too.
// The staged state at sa holds the feature blocks in order (32 rows of DV
// values per block).
template <int D, int DV>
__device__ __forceinline__ u32x4 snap_operand(const char* sa, const int (&va)[DV / 32], int i) {
  constexpr int NFB = D / 32;
  const int mv = i / (2 * NFB), fb = (i / 2) % NFB, hh = i % 2;
  const char* base = sa + 32 * fb * (DV * 2) + va[mv];
  const u32x2 l2 = lds_read_tr(base + (16 * hh) * (DV * 2));
  const u32x2 h2 = lds_read_tr(base + (16 * hh + 8) * (DV * 2));
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// Stage the memory state [D][DV] (bf16, feature rows) into LDS at sa with
// the V tiles' layout and swizzle.
template <int D, int DV, int THREADS>
__device__ __forceinline__ void stage_snapshot(const uint16_t* sn, char* sa, int w, int lane) {
  constexpr int NW = THREADS / 64;
  constexpr int RB = 32;  // rows per staging call: one feature block
  constexpr int SPIECES = RB * DV * 2 / 1024;
  constexpr int SLOADS = SPIECES * 64 >= THREADS ? SPIECES * 64 / THREADS : 1;
  constexpr int SMOD = SPIECES < NW * SLOADS ? SPIECES : 0;
  static_assert(SPIECES >= 1 && SLOADS * 16 * THREADS >= RB * DV * 2, "snapshot staging shape");
  constexpr int VCH = DV / 8;
  uint32_t soff[SLOADS];
#pragma unroll
  for (int i = 0; i < SLOADS; ++i) {
    const int P = stage_piece(NW, w, i, SMOD) * 64 + lane;
    const int r = P / VCH, p = P % VCH;
    soff[i] = (uint32_t)(r * DV + 8 * (p ^ vswz<DV>(r))) * 2u;
  }
#pragma unroll
  for (int rb = 0; rb < D / RB; ++rb) stage_rows(sn, rb * RB, D, DV, sa + rb * RB * DV * 2, NW, w, soff, SLOADS, SMOD);
}

// Byte offset, in a staged V tile (rows of DV values), of the transpose read
// for O rows 32 mv + [0, 32), key row 0. The V^T block for O rows
// 32 mv + [0, 32) and the P keys of k-step (mb, hh) needs, at element j of
// lane (lq, g), V[32 mb + 16 hh + 8 (j >> 2) + 4 g + (j & 3)][32 mv + perm_row(lq)].
// Transpose read jj supplies j = 4 jj + j': source lane sl of each 16-lane
// group points at key 32 mb + 16 hh + 8 jj + 4 g + sl / 4 and at values
// 32 mv + 16 (group % 2) + 4 perm2(sl % 4) + [0, 4), perm2 swapping two bits.
// The V swizzle depends on the row mod 4 = sl / 4 only, so (mb, hh, jj) add
// a constant to this base.
template <int DV>
__device__ __forceinline__ int v_operand_base(int lane, int mv) {
  const int g = lane >> 5, sl = lane & 15, grp2 = (lane >> 4) & 1;
  const int perm2 = ((sl & 3) >> 1) | ((sl & 1) << 1);
  const int col = 32 * mv + 16 * grp2 + 4 * perm2;
  return (4 * g + (sl >> 2)) * (DV * 2) + 16 * ((col >> 3) ^ vswz<DV>(sl >> 2)) + 2 * (col & 7);
}

// Output rows through LDS. A lane holds one query's row of O, so a store
// straight from the accumulators writes 16 or 32 bytes into each of 32 rows
// per instruction. With the stage memory free, each wave instead passes its
// 32 rows, CPR columns at a time, through its own part of that memory and
// stores whole row pieces of CPR elements. Accumulator register r of block
// mv holds column 32 mv + 16 (r >> 3) + 8 g + (r & 7) (two runs of 8 per
// lane). CPR is the most columns (a power of two, at most DV) for which the
// waves' rows fit the stage memory, with 16 bytes of padding per row.
template <int D, int DV, int QB, int EB>
struct OutStage {
  using T = ScaTile<D, DV, QB>;
  static constexpr bool fits(int cpr) { return (size_t)T::NW * 32 * (EB * cpr + 16) <= T::STAGE_BYTES; }
  // (shapes whose stage memory is too small store straight from the accumulators)
  static constexpr bool kUse = fits(32);
  static constexpr int CPR = fits(DV) ? DV : fits(DV / 2) ? DV / 2 : fits(DV / 4) ? DV / 4 : 32;
  static constexpr int RW = EB * CPR + 16;  // row pitch in LDS
  static constexpr int PPR = EB * CPR / 16, RPI = 64 / PPR;  // 16-byte pieces per row, rows per instruction
  static_assert(!kUse || (CPR >= 32 && fits(CPR) && RPI >= 1 && 32 % RPI == 0), "output staging shape");
  static constexpr size_t wave_bytes() { return (size_t)32 * RW; }

  // rows [row0, row0 + nvalid) of orow's matrix (row pitch DV elements,
  // bf16 for EB = 2, float32 for EB = 4), scaled by `scale`; buf is the
  // wave's part. A wave's LDS accesses are processed in order: the reads see
  // the writes before them, and the next piece's writes follow the reads.
  template <typename E>
  __device__ __forceinline__ static void store(char* buf, const f32x16 (&o)[DV / 32], float scale, E* orow,
                                               int nvalid, int lane) {
    static_assert(sizeof(E) == EB, "element size");
    const int lq = lane & 31, g = lane >> 5;
#pragma unroll
    for (int m0 = 0; m0 < DV / 32; m0 += CPR / 32) {
#pragma unroll
      for (int mv = m0; mv < m0 + CPR / 32; ++mv)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          char* dst = buf + lq * RW + EB * (32 * (mv - m0) + 16 * hh + 8 * g);
          const f32x16& x = o[mv];
          if constexpr (EB == 2) {
            *reinterpret_cast<u32x4*>(dst) =
                u32x4{pack2(x[8 * hh + 0] * scale, x[8 * hh + 1] * scale), pack2(x[8 * hh + 2] * scale, x[8 * hh + 3] * scale),
                      pack2(x[8 * hh + 4] * scale, x[8 * hh + 5] * scale), pack2(x[8 * hh + 6] * scale, x[8 * hh + 7] * scale)};
          } else {
            *reinterpret_cast<f32x4*>(dst) =
                f32x4{x[8 * hh + 0] * scale, x[8 * hh + 1] * scale, x[8 * hh + 2] * scale, x[8 * hh + 3] * scale};
            *reinterpret_cast<f32x4*>(dst + 16) =
                f32x4{x[8 * hh + 4] * scale, x[8 * hh + 5] * scale, x[8 * hh + 6] * scale, x[8 * hh + 7] * scale};
          }
        }
#pragma unroll
      for (int k = 0; k < 32 / RPI; ++k) {
        const int r = lane / PPR + RPI * k, cb = 16 * (lane % PPR);
        const u32x4 v = *reinterpret_cast<const u32x4*>(buf + r * RW + cb);
        if (r < nvalid) st16(reinterpret_cast<char*>(orow + (size_t)r * DV + 32 * m0) + cb, v);
      }
    }
  }
};

template <int D, int DV, bool kSca, bool kRead, bool kOutF32>
__global__ __launch_bounds__((ScaTile<D, DV, ScaShape<D, DV>::QB>::THREADS), 1) void sca_bf16_kernel(ScaArgs a) {
  constexpr int QB = ScaShape<D, DV>::QB;
  constexpr int KS = D / 16;   // 16-feature k-steps of the readout
  constexpr int NMV = DV / 32; // 32-row blocks of O^T

  // Blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous
  // run of logical blocks so the q-tiles of one chunk share an L2.
  const uint32_t bid = blockIdx.x;
  const uint32_t lb = (bid & 7u) * (uint32_t)a.per_xcd + (bid >> 3);
  if (lb >= (uint32_t)a.nblocks) return;
  // Within an XCD, groups of GECKO_SCA_GROUP consecutive (batch*head, chunk)
  // pairs run their longest q-tiles first, so the workgroups left at the end
  // of the grid are short ones.
  const uint32_t qtiles = (uint32_t)a.qtiles, nchunks = (uint32_t)a.nchunks;
  const uint32_t npairs = (uint32_t)a.nblocks / qtiles;
  const uint32_t grp = lb / (GECKO_SCA_GROUP * qtiles);
  const uint32_t base = grp * GECKO_SCA_GROUP;
  const uint32_t gsize = min((uint32_t)GECKO_SCA_GROUP, npairs - base);
  const uint32_t within = lb - base * qtiles;
  const int qt = (int)(qtiles - 1 - within / gsize);
  const uint32_t rest = base + within % gsize;
  const int s = (int)(rest % nchunks);
  const uint32_t bh = rest / nchunks;
  const int h = (int)(bh % (uint32_t)a.H);
  const int n = (int)a.n, c = a.c;  // n * max(d, dv) * 2 < 2^32 (validated on the host)
  const int q0 = s * c + qt * kBM;
  const int cend = min((s + 1) * c, n);
  if (q0 >= cend) return;
  const int qend = min(q0 + kBM, cend);

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int myq0 = q0 + 32 * QB * w + lq;  // query of block qb: myq0 + 32 qb
  const uint16_t* zbh = a.z + (size_t)bh * (size_t)n * D;

  f32x16 oacc[QB][NMV];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < NMV; ++i) oacc[qb][i] = f32x16{};

  // LDS: the three (K, V) stages, and the memory state M'_{s-1} ([d][dv],
  // feature rows) with the V tiles' layout and swizzle (the readout
  // psi(Q_m) M' is the PV product with features in the role of keys). The
  // state is final before this kernel starts; with the attention it goes
  // into the stage memory after the loop, without it into its own region
  // now.
  using T = ScaTile<D, DV, QB>;
  constexpr int NFB = D / 32;
  constexpr bool kEarly = !kSca;
  __shared__ __attribute__((aligned(16))) char SM[kSca ? T::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char SN[kRead && kEarly ? T::SNAP_BYTES : 16];
  char* const S0 = SM;
  char* const S1 = SM + (kSca ? T::STAGE1 : 0);
  char* const S2 = SM + (kSca ? 2 * T::STAGE1 : 0);
  char* const snap_a = kEarly ? SN : SM;
  // chunk s reads the state holding the chunks before its previous one
  // (chunk-wise variant: the chunks before it): snapshot slot
  // s - lag + 2 has_prev (with a carried chunk, slot 0 is the incoming
  // state); the first lag chunks of a sequence read nothing
  const int rslot = s - a.lag + 2 * a.has_prev;
  const bool reads = s >= a.first_read;
  const uint16_t* sn = a.snap + ((size_t)bh * a.nsnap + rslot) * (size_t)(D * DV);
  if constexpr (kRead && kEarly) {
    if (reads) stage_snapshot<D, DV, T::THREADS>(sn, snap_a, w, lane);
  }

  // attention row sums: O = oacc / lsum (+ readout)
  float lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) lsum[qb] = 1.f;
  int va[NMV];  // V / state transpose-read bases, shared by the loop and the readout
#pragma unroll
  for (int mv = 0; mv < NMV; ++mv) va[mv] = v_operand_base<DV>(lane, mv);
  if constexpr (kSca) {
    ScaLoop<D, DV, QB> L;
    L.init(a, bh, h, n, s, c, q0, qend, w, lane, S0, S1, S2, va);
    float msub[QB];
    L.run(oacc, lsum, msub);
    // training outputs: O_SCA = oacc / lsum in float32 (accumulator register
    // r of block mv holds value column 32 mv + 16 (r >> 3) + 8 g + (r & 7)),
    // and per query the offset and the sum of the bf16 weights the PV product
    // used, from which a backward pass rebuilds exactly those weights
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int myq = myq0 + 32 * qb;
      if (myq < qend && a.stats && g == 0)
        *reinterpret_cast<float2*>(a.stats + 2 * ((size_t)bh * n + myq)) = make_float2(msub[qb], lsum[qb]);
    }
    if (a.o_sca) {
      using OS = OutStage<D, DV, QB, 4>;
      if constexpr (OS::kUse) {  // the stage memory is free: every wave is past the loop's last barrier
        char* buf = SM + w * OS::wave_bytes();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int row0 = q0 + 32 * QB * w + 32 * qb;
          const int nvalid = min(32, qend - row0);
          if (nvalid > 0)
            OS::store(buf, oacc[qb], 1.f / lsum[qb], a.o_sca + ((size_t)bh * n + row0) * DV, nvalid, lane);
        }
        __syncthreads();  // the readout's state may go into the stage memory now
      } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int myq = myq0 + 32 * qb;
          if (myq >= qend) continue;
          const float inv = 1.f / lsum[qb];
          float* orow = a.o_sca + ((size_t)bh * n + myq) * DV;
#pragma unroll
          for (int mv = 0; mv < NMV; ++mv)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const f32x16& o = oacc[qb][mv];
              float* dst = orow + 32 * mv + 16 * hh + 8 * g;
              *reinterpret_cast<f32x4*>(dst) =
                  f32x4{o[8 * hh + 0] * inv, o[8 * hh + 1] * inv, o[8 * hh + 2] * inv, o[8 * hh + 3] * inv};
              *reinterpret_cast<f32x4*>(dst + 4) =
                  f32x4{o[8 * hh + 4] * inv, o[8 * hh + 5] * inv, o[8 * hh + 6] * inv, o[8 * hh + 7] * inv};
            }
        }
      }
    }
    if (a.lse) {
      // the kernel's logits are log2(e) (q_i . k_j - q_i . nu_k) (see the
      // header), so log sum_j exp(q_i . k_j) = ln 2 (msub + log2 lsum) + q_i . nu_k
      const float* kq = a.kappa_q + h * D;
      const float* nq = a.nu_q + h * D;
      const float* nk = a.nu_k + h * D;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int myq = myq0 + 32 * qb;
        const uint16_t* zq = zbh + (size_t)min(myq, qend - 1) * D;
        float qn = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int f0 = 16 * ks + 8 * g;
          float x[8];
          const u32x4 raw = ld16(zq + f0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[2 * j] = bf_lo(raw[j]);
            x[2 * j + 1] = bf_hi(raw[j]);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) qn += (kq[f0 + i] * x[i] + nq[f0 + i]) * nk[f0 + i];
        }
        qn = other_half_sum(qn);
        if (g == 0 && myq < qend)
          a.lse[(size_t)bh * n + myq] = 0.6931471805599453f * (msub[qb] + log2f(lsum[qb])) + qn;
      }
    }
  }
  if constexpr (kRead && !kEarly) {  // every wave is past the loop's last barrier
    if (reads) stage_snapshot<D, DV, T::THREADS>(sn, snap_a, w, lane);
  }

  if constexpr (kRead) {
    if (reads) {
      // psi(Q_m) as the B operand: element e of lane (lq, g) in k-step
      // (fb, hh) is feature 32 fb + 16 hh + 8 (e >> 2) + 4 g + (e & 3). It is
      // packed unnormalised (2^(x - max)); the accumulators are scaled by the
      // psi row sum before the readout MFMAs and divided by it afterwards, so
      // that O = attention / lsum + psi M'.
      const float* eq = a.eta_q + h * D;
      const float* rq = a.rho_q + h * D;
      u32x4 pf[QB][NFB][2];
      float psum[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const uint16_t* zq = zbh + (size_t)min(myq0 + 32 * qb, qend - 1) * D + 4 * g;
        float mx = kNegInf;
#pragma unroll
        for (int k = 0; k < 4 * NFB; ++k) {  // k = 4 fb + 2 hh + jh: features 8 k + 4 g + [0, 4)
          const u32x2 raw = *reinterpret_cast<const u32x2*>(zq + 8 * k);
          const f32x4 e4 = *reinterpret_cast<const f32x4*>(eq + 8 * k + 4 * g);
          const f32x4 r4 = *reinterpret_cast<const f32x4*>(rq + 8 * k + 4 * g);
          mx = fmaxf(mx, fmaxf(fmaxf(e4[0] * bf_lo(raw[0]) + r4[0], e4[1] * bf_hi(raw[0]) + r4[1]),
                               fmaxf(e4[2] * bf_lo(raw[1]) + r4[2], e4[3] * bf_hi(raw[1]) + r4[3])));
        }
        mx = other_half_max(mx) * kLog2e;
        float sum = 0.f;
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            uint32_t wd[4];
#pragma unroll
            for (int jh = 0; jh < 2; ++jh) {
              const int k = 4 * fb + 2 * hh + jh;
              const u32x2 raw = *reinterpret_cast<const u32x2*>(zq + 8 * k);
              const f32x4 e4 = *reinterpret_cast<const f32x4*>(eq + 8 * k + 4 * g);
              const f32x4 r4 = *reinterpret_cast<const f32x4*>(rq + 8 * k + 4 * g);
              const float x0 = exp2_fast((e4[0] * bf_lo(raw[0]) + r4[0]) * kLog2e - mx);
              const float x1 = exp2_fast((e4[1] * bf_hi(raw[0]) + r4[1]) * kLog2e - mx);
              const float x2 = exp2_fast((e4[2] * bf_lo(raw[1]) + r4[2]) * kLog2e - mx);
              const float x3 = exp2_fast((e4[3] * bf_hi(raw[1]) + r4[3]) * kLog2e - mx);
              wd[2 * jh] = pack2(x0, x1);
              wd[2 * jh + 1] = pack2(x2, x3);
              sum = sum2_bf16(wd[2 * jh], sum2_bf16(wd[2 * jh + 1], sum));
            }
            pf[qb][fb][hh] = u32x4{wd[0], wd[1], wd[2], wd[3]};
          }
        psum[qb] = other_half_sum(sum);
        const float scale = psum[qb] / lsum[qb];
#pragma unroll
        for (int i = 0; i < NMV; ++i) oacc[qb][i] *= scale;
        lsum[qb] = psum[qb];
      }
      wait_vmem();
      __syncthreads();
      // A operand: V^T-style transpose reads of the staged M' (see
      // ScaLoop::v_addr), read AH MFMA operands ahead
      constexpr int NI = NMV * NFB * 2, AH = 2;
      u32x4 op[AH + 1];
#pragma unroll
      for (int i = 0; i < AH; ++i) op[i] = snap_operand<D, DV>(snap_a, va, i);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i + AH < NI) op[(i + AH) % (AH + 1)] = snap_operand<D, DV>(snap_a, va, i + AH);
        const int mv = i / (2 * NFB), fb = (i / 2) % NFB, hh = i % 2;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][mv] = mfma_bf16(op[i % (AH + 1)], pf[qb][fb][hh], oacc[qb][mv]);
      }
    }
  }

  // divide by the row sums (attention's, or psi's after the readout)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.f / lsum[qb];
#pragma unroll
    for (int i = 0; i < NMV; ++i) oacc[qb][i] *= inv;
  }

  // accumulator register r of block mv holds value column
  // 32 mv + 16 (r >> 3) + 8 g + (r & 7): two runs of 8 per lane. A lane
  // holds one query, so a bf16 store straight from the accumulators writes
  // 32 bytes into each of 32 rows per instruction; with the stage memory
  // free, each wave instead passes its 32 x CPR-column pieces of O through
  // its own part of it and stores whole 2 CPR-byte row pieces.
  if constexpr (kSca && !kOutF32 && OutStage<D, DV, QB, 2>::kUse) {
    using OS = OutStage<D, DV, QB, 2>;
    __syncthreads();  // every wave is past its reads of the stage memory
    char* buf = SM + w * OS::wave_bytes();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row0 = q0 + 32 * QB * w + 32 * qb;
      const int nvalid = min(32, qend - row0);
      if (nvalid > 0)
        OS::store(buf, oacc[qb], 1.f, static_cast<uint16_t*>(a.out) + ((size_t)bh * n + row0) * DV, nvalid, lane);
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int myq = myq0 + 32 * qb;
    if (myq >= qend) continue;
    if constexpr (kOutF32) {
      float* orow = static_cast<float*>(a.out) + ((size_t)bh * n + myq) * DV;
#pragma unroll
      for (int mv = 0; mv < NMV; ++mv)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x16& o = oacc[qb][mv];
          float* dst = orow + 32 * mv + 16 * hh + 8 * g;
          *reinterpret_cast<f32x4*>(dst) = f32x4{o[8 * hh + 0], o[8 * hh + 1], o[8 * hh + 2], o[8 * hh + 3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[8 * hh + 4], o[8 * hh + 5], o[8 * hh + 6], o[8 * hh + 7]};
        }
    } else {
      uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)bh * n + myq) * DV;
#pragma unroll
      for (int mv = 0; mv < NMV; ++mv)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x16& o = oacc[qb][mv];
          const u32x4 pk{pack2(o[8 * hh + 0], o[8 * hh + 1]), pack2(o[8 * hh + 2], o[8 * hh + 3]),
                         pack2(o[8 * hh + 4], o[8 * hh + 5]), pack2(o[8 * hh + 6], o[8 * hh + 7])};
          st16(orow + 32 * mv + 16 * hh + 8 * g, pk);
        }
    }
  }
}

template <int D, int DV, bool kSca, bool kRead, bool kOutF32>
hipError_t launch_one(const ScaArgs& a, hipStream_t stream) {
  using T = ScaTile<D, DV, ScaShape<D, DV>::QB>;
  // all LDS is static (per-stage variables, sized by lds_bytes)
  static_assert(T::lds_bytes(kSca, kRead) <= 160 * 1024, "LDS per workgroup");
  const dim3 grid((unsigned)(8 * a.per_xcd));
  hipLaunchKernelGGL((sca_bf16_kernel<D, DV, kSca, kRead, kOutF32>), grid, dim3(T::THREADS), 0, stream, a);
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
  switch (d * 1000 + dv) {
#define GECKO_SCA_SHAPE(D_, DV_) \
  case D_ * 1000 + DV_:          \
    return true;
    GECKO_BF16_SHAPES(GECKO_SCA_SHAPE)
#undef GECKO_SCA_SHAPE
  }
  return false;
}

hipError_t launch_sca_bf16(const Problem& p, const Workspace& w, int mode, hipStream_t stream) {
  ScaArgs a;
  a.z = static_cast<const uint16_t*>(p.z);
  a.v = static_cast<const uint16_t*>(p.v);
  a.out = p.out;
  a.kappa_q = p.kappa_q; a.nu_q = p.nu_q; a.kappa_k = p.kappa_k;
  a.nu_k = p.nu_k; a.lse = p.lse;
  a.o_sca = p.o_sca; a.stats = p.stats;
  a.eta_q = p.eta_q; a.rho_q = p.rho_q;
  a.snap = static_cast<const uint16_t*>(w.snap);
  a.zprev = static_cast<const uint16_t*>(p.zprev);
  a.vprev = static_cast<const uint16_t*>(p.vprev);
  a.has_prev = p.has_prev ? 1 : 0;
  a.first_read = (int)p.first_read;
  a.lag = (int)p.lag;
  a.prev = (int)p.prev;
  a.n = p.n;
  // the host validated n * max(d, dv) * 2 < 2^32 and the block count < 2^31;
  // without a carried chunk, a chunk longer than the sequence is the sequence
  const int64_t cc = min(p.c, p.n);
  a.c = (int)(p.has_prev ? p.c : cc);
  a.nchunks = (int)p.nchunks; a.nsnap = (int)p.nsnap; a.H = (int)p.H;
  a.qtiles = (int)((cc + kBM - 1) / kBM);
  const int64_t nblocks = p.B * p.H * p.nchunks * a.qtiles;
  a.nblocks = (int)nblocks;
  a.per_xcd = (int)((nblocks + 7) / 8);
  switch (p.d * 1000 + p.dv) {
#define GECKO_SCA_SHAPE(D_, DV_) \
  case D_ * 1000 + DV_:          \
    return launch_shape<D_, DV_>(a, mode, p.out_f32, stream);
    GECKO_BF16_SHAPES(GECKO_SCA_SHAPE)
#undef GECKO_SCA_SHAPE
  }
  return hipErrorInvalidValue;
}

}  // namespace gecko
