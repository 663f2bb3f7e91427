// Host-side interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gecko {

// same bits as GECKO_AWM_NO_DELTA and GECKO_CHUNKWISE in gecko.h
constexpr unsigned GECKO_AWM_NO_DELTA_BIT = 1u << 0;
constexpr unsigned GECKO_CHUNKWISE_BIT = 1u << 1;

// Per-launch description of one forward. All pointers are device pointers.
struct Problem {
  const void* z;        // [BH][n][d]   in dtype
  const void* v;        // [BH][n][dv]  in dtype
  void* out;            // [BH][n][dv]  out dtype
  const float* kappa_q; const float* nu_q; const float* kappa_k; const float* nu_k;
  const float* eta_q; const float* rho_q; const float* eta_k; const float* rho_k;
  int64_t B, H, n, d, dv, c;
  int64_t nchunks;      // N = ceil(n / c) chunks of this call
  int64_t nmem;         // chunks entered into the memory by this call (scan steps):
                        //   one call: max(N - lag, 0); streaming: has_prev + N - 1
  unsigned flags;
  bool out_f32;         // output dtype (bf16 inputs may write float32 output)
  // Streaming (bf16 only). The memory pass and the scan see a virtual
  // sequence [carried chunk (if has_prev)] + this call's chunks; attention
  // and output cover this call's tokens. Chunk s of the call reads scan
  // output r = s - 2 + has_prev, stored in snapshot slot r + has_prev; slot 0
  // of a call with has_prev holds the incoming state (r = -1).
  int64_t nsnap;        // snapshot slots per (b, h): nmem + has_prev
  int64_t first_read;   // first chunk of the call that reads the memory: the
                        //   sequence's first lag chunks read none (lag - chunks before, at least 0)
  int64_t lag;          // chunk s reads the state after chunks <= s - lag (one call: scan output s - lag);
                        //   2 with sliding chunks, 1 for the chunk-wise variant
  int64_t prev;         // attention window: 1 = previous chunk + current chunk, 0 = current chunk only
  bool stream;          // keep the memory state after this call (mstate, zfinal)
  bool has_prev;        // tokens were processed before: a carried chunk and an incoming state
  const void* zprev;    // [BH][c][d]  carried chunk (the last chunk of the previous call)
  const void* vprev;    // [BH][c][dv]
  float* mstate;        // [BH][dv/32][d/32][64][16] fp32 state M'^T (scan accumulator layout), in/out
  const float* zstate;  // [BH][d][2] running (M, L) per feature (log2 max, scaled sum) before this call
  float* lse;           // bf16 attention only, may be null: [BH][n] natural log-sum-exp of each query's logits
  float* o_sca;         // bf16 attention only, may be null: [BH][n][dv] float32 attention output alone
  float* stats;         // bf16 attention only, may be null: [BH][n][2] offset and sum of the bf16 weights
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
  void* snap;      // state read by chunk t+2: bf16 [bh][nsnap][d][dv], fp32 [bh][t][dv][d]
  float* rowstat;  // fp32 path only: per-token (max, sum) of K_m rows  [bh][n][2]
  float* zfinal;   // streaming: running (M, L) per feature after the call  [bh][d][2]
  float* snap32;   // optional (bf16 scan): the snapshots again in float32 [bh][nsnap][d][dv] (set by the backward)
  size_t bytes;
};

Workspace carve_workspace(void* base, int64_t BH, int64_t n, int64_t d, int64_t dv,
                          int64_t nmem, int64_t nsnap, bool bf16, bool stream);

// The memory pass a training forward keeps for its backward: the bf16
// Workspace w of a one-call forward, then every state S_t again in float32
// [bh][t][d][dv] (what the backward's reverse scan and readout reads),
// 256-byte aligned. 0 bytes when no chunk reads the memory.
size_t kept_memory_bytes(const Workspace& w, int64_t BH, int64_t nmem, int64_t d, int64_t dv);
float* kept_states(const void* base, const Workspace& w);

// The library's own scratch array (noalloc.hip): its size, and the device
// address of `device`'s copy (looked up once per device, with that device
// current; never the array's host-side name).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(int device, void** ptr);

// The (d, dv) pairs the bf16 kernels are built for: every pair of
// d in {32, 64, 128} and dv in {32, 64, 128, 256}.
#define GECKO_BF16_SHAPES(X)                                      \
  X(128, 256) X(128, 128) X(128, 64) X(128, 32) X(64, 256) X(64, 128) \
  X(64, 64) X(64, 32) X(32, 256) X(32, 128) X(32, 64) X(32, 32)

// Launchers (stream-ordered, asynchronous). Each returns the launch status.
hipError_t launch_awm_chunk_bf16(const Problem& p, const Workspace& w, hipStream_t s);
hipError_t launch_awm_zscan(const Problem& p, const Workspace& w, hipStream_t s);
hipError_t launch_awm_scan_bf16(const Problem& p, const Workspace& w, hipStream_t s);
// mode bit 0: attention, bit 1: memory readout
hipError_t launch_sca_bf16(const Problem& p, const Workspace& w, int mode, hipStream_t s);

hipError_t launch_awm_chunk_f32(const Problem& p, const Workspace& w, hipStream_t s);
hipError_t launch_awm_scan_f32(const Problem& p, const Workspace& w, hipStream_t s);
hipError_t launch_sca_f32(const Problem& p, const Workspace& w, int mode, hipStream_t s);
// Streaming state. reset: M' = 0 and (M, L) = (-inf, 0) for a sequence whose
// first call enters nothing into the memory. finish (after the attention
// kernel, which reads the old carried chunk): the last chunk of this call
// (`rows` rows starting at row0) becomes the carried chunk, and zfinal the
// running denominator.
hipError_t launch_stream_reset(float* mstate, float* zstate, int64_t BH, int64_t d, int64_t dv, hipStream_t s);
hipError_t launch_stream_finish(const Problem& p, const Workspace& w, void* zcarry, void* vcarry, float* zstate,
                                int64_t row0, int64_t rows, hipStream_t s);

bool bf16_shape_built(int64_t d, int64_t dv);

// ---------------------------------------------------------------- backward
// Gradients of L = sum(dO * O) (bf16 inputs, d = 128, dv in {128, 256}).
struct BwdProblem {
  Problem f;            // the forward (z, v, affine vectors, sizes, nmem, lag, prev)
  const void* dout;     // [BH][n][dv], bf16 or float32
  float* dz;            // [BH][n][d]
  float* dv;            // [BH][n][dv]
  float* daff;          // [8][H][d]: kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k
  bool sca, awm, out_f32;
  // saved attention statistics of the forward (gecko_backward_saved), else null
  bool saved;
  const float* o_sca;   // [BH][n][dv] float32 attention output
  const float* stats;   // [BH][n][2] offset m and sum l of the bf16 weights 2^(s - m)
  // the training forward's memory pass and scan (kept_memory_bytes, laid out
  // as a Workspace followed by the states in float32), else null: recomputed
  const void* mem_saved;
};

// Backward workspace. Arrays indexed [bh][t] have t = 0..nmem-1, the chunk
// entering the memory (scan step t).
struct BwdWorkspace {
  Workspace fw;         // forward memory pass and scan, recomputed
  uint16_t* qp;         // scaled queries (kappa_q z + nu_q) kappa_k log2(e), bf16 [BH][n][d]
  float* ld;            // per query: (log2-sum-exp of the scaled logits, sum_j P_ij dP_ij) [BH][n][2]
  uint16_t* do16;       // dO in bf16 [BH][n][dv] when dO is float32 (else null: dO itself)
  uint16_t* dos;        // saved statistics: bf16(dO / l) per query, the attention kernels' dO [BH][n][dv]
  float* dq;            // dL/dQ, dL/dK, dL/dQ_m, dL/dK_m, each [BH][n][d]
  float* dk;
  float* dqm;
  float* dkm;
  float* r;             // readout gradient reaching state t: psi(Q_m)^T dO of the chunk that reads it,
                        //   transposed, in the scan's accumulator layout [BH][t][dv/32][d/32][64][16]
  uint16_t* ht;         // H_t transposed, scan B-operand order [BH][t][d/16][d/32][64][8]
  uint16_t* ds;         // dL/dS_t (state after step t), bf16 [BH][t][d][dv]
  float* part;          // per 32-value slice: rowsum(R_t * S_t), rowsum(C_t * S_t) [BH][t][dv/32][d][2]
  float* zeta;          // z^t * dL/dz^t per feature [BH][t][d]
  uint16_t* x;          // dS_t S_{t-1}^T, bf16 [BH][t][d][d]
  float* s32;           // the states S_t in float32 [BH][t][d][dv] (forward scan, backward mode)
  float* apart;         // affine-gradient partial sums [BH][nblk][8][d]
  int64_t nblk, rows_per_blk;
  size_t bytes;
};

BwdWorkspace carve_bwd_workspace(void* base, const BwdProblem& p);
bool bwd_shape_built(int64_t d, int64_t dv);
hipError_t launch_bwd_prep(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s);
hipError_t launch_bwd_dout16(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s);
hipError_t launch_bwd_saved_prep(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s);
hipError_t launch_bwd_dq(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdProblem& p, const BwdWorkspace& w, bool accumulate_dv, hipStream_t s);
hipError_t launch_bwd_awm(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s);
hipError_t launch_bwd_combine(const BwdProblem& p, const BwdWorkspace& w, hipStream_t s);

// CEMA (cema.hip). All pointers are device pointers.
struct CemaProblem {
  const void* x;        // [B][n][D], bf16 or float32
  void* y;              // [B][n][D], bf16 or float32
  const float* alpha; const float* delta; const float* theta; const float* beta;  // [D][H]
  const float* eta;     // [D][H][2]
  const uint8_t* reset; // [B][n] or null
  const float* h0;      // [B][D][H][2] or null
  float* hfin;          // [B][D][H][2] or null
  int64_t B, n, D, H;
  bool in_bf16, out_bf16;
};

// Chunking of the sequence and the workspace it needs: chunk end states and
// entering states ([B][C][H][D] float2 each) and per-chunk reset flags.
struct CemaPlan {
  int64_t C, L, nwd;
  size_t off_hin, off_flag, bytes;
};

CemaPlan cema_plan(int64_t B, int64_t n, int64_t D, int64_t H);

// Timestep decay normalisation (tdn.hip).
struct TdnProblem {
  const void* x;        // [B][n][D]
  void* y;              // [B][n][D]
  const float* gamma; const float* shift;  // [D]
  const float* m0; const float* v0;        // [B][G] or null (zero)
  float* m_out; float* v_out;              // [B][G] or null
  int64_t B, n, D, G, t0;                  // t0: tokens of the sequence before this call
  float beta1, beta2, eps;
  bool in_bf16, out_bf16;
};
// workspace: per-token decayed sums within each sub-chunk [B][n][G] float2,
// the sums of each sub-chunk (then the sums entering it) [B][nsub][G] float2,
// then the chunk carries [B][NC][G] float2 (chunks of Ls sub-chunks)
struct TdnPlan {
  int64_t nsub, NC, Ls;
  size_t off_sub, off_carry, bytes;
};
TdnPlan tdn_plan(int64_t B, int64_t n, int64_t G);
hipError_t launch_tdn(const TdnProblem& p, void* ws, hipStream_t s);
hipError_t launch_cema(const CemaProblem& q, const CemaPlan& plan, void* ws, hipStream_t s);

}  // namespace gecko
