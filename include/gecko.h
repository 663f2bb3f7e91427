/*
 * gecko.h - C ABI of the MI355X (gfx950) Gecko per-layer forward:
 * sliding chunk attention (SCA) plus adaptive working memory (AWM).
 *
 * Operation (sources: the Gecko summary on paper.rainbus.top, sections
 * "Method steps" (2)-(5) and "Core method"; the paperlayer.ai summary,
 * sections 3.2, 3.3 and Appendix A):
 *
 *   Q   = kappa_q * Z' + nu_q     K   = kappa_k * Z' + nu_k      (per feature)
 *   Q_m = eta_q   * Z' + rho_q    K_m = eta_k   * Z' + rho_k
 *   O_SCA rows of chunk s = softmax(Q_s [K_{s-1}; K_s]^T) [V_{s-1}; V_s],
 *       causal inside chunk s, logits unscaled;
 *   z^s = per-feature sum of exp(K_m) over chunks 1..s;  phi^s(k) = exp(k)/z^s;
 *   psi = softmax over the features of a row;
 *   M'_1 = 0;  M'_s = (z^{s-2}/z^{s-1}) * M'_{s-1}
 *                    + phi^{s-1}(K_m,{s-1})^T (V_{s-1} - psi(K_m,{s-1}) M'_{s-1});
 *   O_m rows of chunk s = psi(Q_m,s) M'_{s-1}   (zero for chunks 1 and 2);
 *   O = O_SCA + O_m.
 *
 * Layout: every tensor is dense row-major. Z' is [B][H][n][d], V and O are
 * [B][H][n][dv], each affine vector is [H][d] float32. Chunks are consecutive
 * runs of c tokens; the last one may be shorter; c >= n means one chunk.
 *
 * Memory: all data pointers are DEVICE pointers owned by the caller. The
 * library allocates nothing on these calls and keeps no state between them.
 * Inputs are read-only; O must not alias any input or the workspace.
 * Calls are asynchronous and ordered on the given HIP stream (a hipStream_t
 * passed as void*; NULL means the default stream). No host synchronisation.
 *
 * Errors: arguments are validated on the host before any launch. Nothing is
 * launched when a call returns an error. No C++ exception crosses this ABI.
 * gecko_last_error() gives a thread-local text for the last failing call.
 */
#ifndef GECKO_H
#define GECKO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GECKO_OK = 0,
    GECKO_EINVAL = 1,       /* null/misaligned pointer, size < 1, inconsistent arguments */
    GECKO_EUNSUPPORTED = 2, /* valid but not built: d, dv or dtype combination */
    GECKO_EWORKSPACE = 3,   /* workspace pointer null or smaller than gecko_workspace_size() */
    GECKO_EHIP = 4          /* a HIP runtime call or kernel launch failed */
} gecko_status;

typedef enum { GECKO_F32 = 0, GECKO_BF16 = 1 } gecko_dtype;

/* flags */
enum {
    /* Test variant: drop the -psi(K_m) M' term of the update, leaving plain
     * linear attention with the online-softmax kernel. Not the method. */
    GECKO_AWM_NO_DELTA = 1u << 0,
    /* Ablation variant without sliding chunks: the chunk-wise attention
     * Gecko replaces (paperlayer.ai summary, section 2.3: attention inside
     * each chunk only, causal) and the memory without sliding chunks
     * (Appendix A: M_0 = 0, the same update, and chunk s reads the state
     * holding chunks 1..s-1, i.e. one chunk earlier than with sliding
     * chunks). Not accepted by the streaming forward. */
    GECKO_CHUNKWISE = 1u << 1
};

/*
 * Supported shapes: d in {32, 64, 128}; dv in {32, 64, 128, 256}; the bf16
 * and the float32 kernels are built for every pair of the two sets.
 * float32 input writes float32 output; bf16 input writes bf16 output
 * (round to nearest even of the fp32 accumulator) or float32 output (the
 * accumulator itself). n >= 1, c >= 1, B >= 1, H >= 1. z, v and out must be
 * 16-byte aligned, the workspace 256-byte aligned, the affine vectors 4-byte
 * aligned.
 */

/* Bytes of device workspace gecko_sca_awm_forward / gecko_awm_forward need
 * for these sizes (0 if none, (size_t)-1 if the sizes are invalid).
 * It holds, per (batch, head) and per chunk 1..N-2, the chunk's memory-write
 * and correction products, its key statistics, its decay factors and the
 * memory-state snapshots that the readout uses. */
size_t gecko_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                            int64_t c, gecko_dtype in_dtype);

/* The same for a given set of flags (GECKO_CHUNKWISE stores one more chunk
 * per (batch, head)); gecko_workspace_size is this with flags = 0. */
size_t gecko_workspace_size_for(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                                int64_t c, gecko_dtype in_dtype, unsigned flags);

/* O = O_SCA + O_m (the whole forward). Workspace: gecko_workspace_size()
 * bytes of caller-owned device memory; its contents on entry do not matter
 * and are clobbered. */
gecko_status gecko_sca_awm_forward(
    const void* z,
    const float* kappa_q, const float* nu_q, const float* kappa_k, const float* nu_k,
    const float* eta_q, const float* rho_q, const float* eta_k, const float* rho_k,
    const void* v, void* out,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
    gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * gecko_sca_awm_forward (same arguments, same kernels, bit-identical output)
 * without the workspace: the memory pass and the scan use a scratch array
 * that the library holds on each GPU it runs on, GECKO_NOALLOC_SCRATCH_BYTES
 * bytes per GPU from the first call there until the process ends. The call
 * allocates and frees nothing; the caller passes inputs and outputs as for
 * gecko_sca_awm_forward. Sizes whose workspace (gecko_workspace_size_for)
 * exceeds GECKO_NOALLOC_SCRATCH_BYTES are refused with GECKO_EWORKSPACE
 * before anything reaches the device (B1 H8, 131072 tokens, c 2048, d 128,
 * dv 256 in bf16 needs 109.5 MiB and fits).
 *
 * The scratch array is shared by every call on one GPU and keeps whatever
 * the last call left in it (nothing in it needs to start at zero). Calls
 * that overlap in time on one GPU (on different streams, or from different
 * threads without ordering) race on it and give undefined results: order
 * them on one stream. The stream must belong to the current device
 * (GECKO_EINVAL otherwise); NULL is the current device's null stream.
 */
#define GECKO_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gecko_status gecko_sca_awm_forward_noalloc(
    const void* z,
    const float* kappa_q, const float* nu_q, const float* kappa_k, const float* nu_k,
    const float* eta_q, const float* rho_q, const float* eta_k, const float* rho_k,
    const void* v, void* out,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
    gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags, void* stream);

/* O = O_SCA only (needs no workspace; the memory vectors are not read). */
gecko_status gecko_sca_forward(
    const void* z,
    const float* kappa_q, const float* nu_q, const float* kappa_k, const float* nu_k,
    const void* v, void* out,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
    gecko_dtype in_dtype, gecko_dtype out_dtype, void* stream);

/* O = O_m only (exact zeros on chunks 1 and 2). Workspace as above. */
gecko_status gecko_awm_forward(
    const void* z,
    const float* eta_q, const float* rho_q, const float* eta_k, const float* rho_k,
    const void* v, void* out,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
    gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Streaming forward (bf16 inputs only): one sequence handed over in
 * consecutive calls. The pages present Gecko as a model for sequences of
 * arbitrary length whose memory is updated chunk by chunk and carries what
 * the attention window no longer sees (chatpaper.ai abstract; paperlayer.ai
 * summary, section 3.3). The output rows of each call are exactly the rows
 * that one gecko_sca_awm_forward call over the whole sequence would give for
 * the same tokens (chunks are counted from the start of the sequence).
 *
 * State: gecko_stream_state_size() bytes of caller-owned device memory,
 * 256-byte aligned, one per sequence (all B*H heads of it). It holds the
 * float32 memory state, the running per-feature denominator of the memory
 * keys and the last chunk of Z' and V. Its contents are opaque; a call with
 * pos == 0 ignores them, every call rewrites them. Sizes (B, H, d, dv, c)
 * and the affine vectors must be the same on every call of a sequence.
 *
 * pos: tokens of this sequence given to earlier calls; 0 starts a new
 * sequence. pos must be a multiple of c, and every call but the last of a
 * sequence must hold a multiple of c tokens (a call with n % c != 0 ends the
 * sequence; the library cannot detect a later call, whose result would then
 * be undefined). c must be a multiple of 64. n >= 1 may be smaller than c.
 *
 * Workspace: gecko_stream_workspace_size() bytes (clobbered). The state must
 * not alias z, v, out or the workspace. Errors as for gecko_sca_awm_forward
 * (GECKO_EINVAL for a bad pos or a missing or small state). Calls of one
 * sequence are ordered by the stream they are issued on.
 */
size_t gecko_stream_state_size(int64_t B, int64_t H, int64_t d, int64_t dv, int64_t c, gecko_dtype in_dtype);
size_t gecko_stream_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                                   gecko_dtype in_dtype);
gecko_status gecko_sca_awm_forward_stream(
    const void* z,
    const float* kappa_q, const float* nu_q, const float* kappa_k, const float* nu_k,
    const float* eta_q, const float* rho_q, const float* eta_k, const float* rho_k,
    const void* v, void* out,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c, int64_t pos,
    gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
    void* state, size_t state_bytes, void* workspace, size_t workspace_bytes, void* stream);

/*
 * CEMA: the complex multi-dimensional damped EMA that produces X' = CEMA(X)
 * ahead of Z' (Gecko summary on paper.rainbus.top, "Prerequisites / EMA" and
 * "Method steps" (1); paperlayer.ai summary, 2.1 and Appendix B.1). Per input
 * dimension d and hidden dimension j < h:
 *
 *   h_t[d,j] = alpha[d,j] beta[d,j] x_t[d]
 *              + M_t (1 - alpha[d,j] delta[d,j]) e^{i theta[d,j]} h_{t-1}[d,j]
 *   y_t[d]   = Re(sum_j eta[d,j] h_t[d,j])
 *
 * with M_t = 0 where reset[t] != 0 (a document boundary: h_t restarts from
 * the input) and h_0 = h0 (zero if h0 is NULL). Readings of what the pages
 * leave open: the expansion of x into h dimensions is the real scale beta;
 * the projection back to one output is Re(eta . h) with complex eta.
 *
 * Layout: x [B][n][D] (in_dtype), y [B][n][D] (out_dtype), dense row-major;
 * alpha, delta, theta, beta [D][h] float32; eta [D][h][2] float32 (re, im);
 * reset [B][n] bytes or NULL; h0 and h_final [B][D][h][2] float32 (re, im),
 * each may be NULL. h in {1, 2, 4, 8, 16}. Pointers 4-byte aligned, the
 * workspace 256-byte aligned (gecko_cema_workspace_size bytes; 0 when the
 * sequence is short enough to run in one piece). h_final receives the state
 * after the last token, so that a later call with h0 = h_final continues the
 * sequence. Device pointers, caller-owned; asynchronous on `stream`.
 */
size_t gecko_cema_workspace_size(int64_t B, int64_t n, int64_t D, int64_t h);
gecko_status gecko_cema_forward(
    const void* x,
    const float* alpha, const float* delta, const float* theta, const float* beta, const float* eta,
    const uint8_t* reset, const float* h0, void* y, float* h_final,
    int64_t B, int64_t n, int64_t D, int64_t h, gecko_dtype in_dtype, gecko_dtype out_dtype,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Timestep decay normalisation (TDN), the normalisation Gecko uses in place
 * of Megalodon's timestep normalisation (Gecko summary on paper.rainbus.top,
 * "Novelty"; paperlayer.ai summary, 2.2 and 3.1). For each of G equal groups
 * of the D features of token t (t counted from 1 over the whole sequence):
 *
 *   mu_t, s2_t = mean and variance of the group's values at token t
 *   m_t = beta1 m_{t-1} + (1 - beta1) mu_t,  v_t = beta2 v_{t-1} + (1 - beta2) s2_t
 *   y_t = gamma * (x_t - m_t / (1 - beta1^t)) / sqrt(v_t / (1 - beta2^t) + eps) + shift
 *
 * with m_0 = v_0 = 0 unless a call continues a sequence: then m0, v0 are the
 * sums after the previous call (m_out, v_out of that call) and t0 the tokens
 * before this call. Readings of what the pages leave open: the statistics are
 * the current token's group mean and variance; the decayed sums start at 0
 * and are bias-corrected as in Adam; the output is normalised per group and
 * scaled and shifted per feature.
 *
 * Layout: x, y [B][n][D] (bf16 or float32, 16-byte aligned); gamma, shift [D]
 * float32 (16-byte aligned); m0, v0, m_out, v_out [B][G] float32 or NULL.
 * D % G == 0, D / G a multiple of 8, D <= 8192, 0 <= beta < 1, eps > 0.
 * Workspace: gecko_tdn_workspace_size() bytes, 256-byte aligned (per-token
 * group statistics). Device pointers, caller-owned; asynchronous on `stream`.
 */
size_t gecko_tdn_workspace_size(int64_t B, int64_t n, int64_t D, int64_t G);
gecko_status gecko_tdn_forward(
    const void* x, const float* gamma, const float* shift,
    const float* m0, const float* v0, int64_t t0,
    void* y, float* m_out, float* v_out,
    int64_t B, int64_t n, int64_t D, int64_t G, float beta1, float beta2, float eps,
    gecko_dtype in_dtype, gecko_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Measurement helper: HIP events recorded between the kernels of a forward.
 * gecko_timer_create allocates the host object and `capacity` event sets;
 * each gecko_sca_awm_forward_timed call records one set (calls beyond the
 * capacity are not recorded). gecko_timer_read waits for the recorded events
 * and writes, per stage, the summed milliseconds over the recorded calls:
 * ms[0] memory chunk pass, ms[1] denominator prefix, ms[2] memory scan,
 * ms[3] attention + readout kernel; *calls receives the number of calls.
 * The events are created with hipEventDisableSystemFence: they carry timing
 * only, and recording one flushes no cache between the kernels. */
typedef struct gecko_timer gecko_timer;
gecko_status gecko_timer_create(int capacity, gecko_timer** timer);
gecko_status gecko_timer_reset(gecko_timer* timer);
gecko_status gecko_timer_read(gecko_timer* timer, float* ms4, int* calls);
gecko_status gecko_timer_destroy(gecko_timer* timer);

/* gecko_sca_awm_forward that also records one event set into `timer` (may be NULL). */
gecko_status gecko_sca_awm_forward_timed(
    const void* z,
    const float* kappa_q, const float* nu_q, const float* kappa_k, const float* nu_k,
    const float* eta_q, const float* rho_q, const float* eta_k, const float* rho_k,
    const void* v, void* out,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
    gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
    void* workspace, size_t workspace_bytes, void* stream, gecko_timer* timer);

/*
 * Training: the backward (bf16 inputs only; (d, dv) in {(128, 256),
 * (128, 128)}) and a forward that also returns the attention normaliser.
 *
 * The pages define the forward only; the backward computes the derivatives
 * of L = sum(dO * O) with respect to Z', V and the eight affine vectors, O
 * being the output of the same parts of the layer (O_SCA, O_m or both) with
 * the same flags. Following the training setup the pages describe
 * (paperlayer.ai summary, Appendix B.1: what the backward needs is recomputed
 * from chunk-boundary states instead of being stored), the backward keeps
 * nothing from the forward: it reruns the memory's chunk pass and scan and
 * the attention's row statistics itself.
 *
 * parts: GECKO_PART_SCA, GECKO_PART_AWM or both (O = O_SCA + O_m).
 */
enum { GECKO_PART_SCA = 1, GECKO_PART_AWM = 2 };

/* gecko_sca_awm_forward (parts = SCA | AWM) or gecko_sca_forward (parts =
 * SCA) that also writes lse [B][H][n] float32: for each query i,
 * log sum_j exp(q_i . k_j) over its attention window (natural log), the
 * softmax normaliser (e.g. for a caller's own attention backward). parts
 * must hold GECKO_PART_SCA; the workspace is needed with GECKO_PART_AWM
 * (gecko_workspace_size_for bytes). bf16 inputs only (GECKO_EUNSUPPORTED
 * otherwise). lse must be 4-byte aligned and alias nothing else. */
gecko_status gecko_forward_lse(
    const void* z,
    const float* kappa_q, const float* nu_q, const float* kappa_k, const float* nu_k,
    const float* eta_q, const float* rho_q, const float* eta_k, const float* rho_k,
    const void* v, void* out, float* lse,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
    gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags, unsigned parts,
    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace gecko_backward needs ((size_t)-1 if the
 * arguments are invalid or not built). It holds the recomputed memory pass
 * and scan, the scaled queries and their row statistics, per-token
 * gradients with respect to Q, K, Q_m and K_m (float32), the state gradients
 * per chunk and partial sums. out_dtype is the dtype of dout. */
size_t gecko_backward_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                                     gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags, unsigned parts);

/* Gradients of L = sum(dout * O), O the output of `parts` with `flags`.
 *   z, v, affine vectors: the forward's inputs (z, v bf16, 16-byte aligned;
 *       the affine vectors of the parts used, 16-byte aligned).
 *   dout: dL/dO, [B][H][n][dv] in out_dtype (bf16 or float32; float32 is
 *       rounded to bf16, the operand precision of every product).
 *   dz [B][H][n][d], dv_out [B][H][n][dv], daff [8][H][d] (float32, fully
 *       overwritten): daff holds, in this order, the gradients of kappa_q,
 *       nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k summed over the batch
 *       (zero for the vectors of a part not selected).
 * The outputs must not alias each other, an input or the workspace. flags:
 * GECKO_AWM_NO_DELTA and GECKO_CHUNKWISE as in the forward. */
gecko_status gecko_backward(
    const void* z,
    const float* kappa_q, const float* nu_q, const float* kappa_k, const float* nu_k,
    const float* eta_q, const float* rho_q, const float* eta_k, const float* rho_k,
    const void* v, const void* dout,
    float* dz, float* dv_out, float* daff,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
    gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags, unsigned parts,
    void* workspace, size_t workspace_bytes, void* stream);

/* Training forward: out exactly as gecko_forward_lse / gecko_sca_awm_forward
 * with the same arguments, plus what gecko_backward_saved reuses in place of
 * recomputing (the quantities are those of the attention step,
 * paper.rainbus.top, "Method steps" (3), and the memory's chunk-boundary
 * states, paperlayer.ai summary, Appendix B.1, "Method steps" (4)-(5); the
 * pages' training recomputes the memory from such states; keeping the
 * attention's per-query statistics as well is this library's choice):
 *   o_sca: [B][H][n][dv] float32, 16-byte aligned, caller-owned, fully
 *       overwritten: the attention output O_SCA alone.
 *   stats: [B][H][n][2] float32, 8-byte aligned, fully overwritten: per query
 *       the offset m and the sum l of the weights 2^(s - m) rounded to bf16,
 *       as the attention's value product used them; s is the query's logit
 *       less q . nu_k, times log2(e) (a shift shared by the query's keys).
 *       O_SCA = (sum_j bf16(2^(s_j - m)) v_j) / l.
 *   mem_saved: null, or (with GECKO_PART_AWM) a 256-byte aligned device
 *       buffer of mem_saved_bytes >= gecko_memory_saved_size bytes,
 *       caller-owned: the memory pass writes its results there (every
 *       chunk's write and correction products, denominator steps and the
 *       states S_t in bf16 and float32), and the call then uses no
 *       workspace (workspace may be null). Ignored without GECKO_PART_AWM or
 *       when no chunk reads the memory (n <= 2c, or n <= c chunk-wise).
 * bf16 inputs, (d, dv) in {(128, 256), (128, 128)}; parts must include
 * GECKO_PART_SCA. o_sca and stats must not alias each other, an input, the
 * output, mem_saved or the workspace, nor mem_saved an input or the output
 * (GECKO_EINVAL); mem_saved too small: GECKO_EWORKSPACE. Without mem_saved,
 * workspace as gecko_workspace_size. */
gecko_status gecko_forward_train(
    const void* z,
    const float* kappa_q, const float* nu_q, const float* kappa_k, const float* nu_k,
    const float* eta_q, const float* rho_q, const float* eta_k, const float* rho_k,
    const void* v, void* out, float* o_sca, float* stats,
    void* mem_saved, size_t mem_saved_bytes,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
    gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags, unsigned parts,
    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the memory pass gecko_forward_train keeps in mem_saved for these
 * sizes and flags (0 when no chunk reads the memory; (size_t)-1 if the
 * arguments are invalid or not built: bf16 inputs and (d, dv) in
 * {(128, 256), (128, 128)} only). */
size_t gecko_memory_saved_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                               gecko_dtype in_dtype, unsigned flags);

/* Bytes of device workspace gecko_backward_saved needs: gecko_backward's
 * plus the per-query scaled copy of dO ((size_t)-1 if the arguments are
 * invalid, not built, or parts lacks GECKO_PART_SCA). With mem_saved the
 * call needs less (the recomputed memory pass and its float32 states are not
 * taken from the workspace); this size is enough either way. */
size_t gecko_backward_saved_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                                           gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
                                           unsigned parts);

/* gecko_backward with the attention statistics of gecko_forward_train of the
 * same inputs, c, parts and flags (o_sca, stats as written there; read only,
 * not aliasing an output or the workspace): the same gradients, with the
 * attention weights taken as the forward's own bf16-rounded ones, and no
 * statistics pass over the key window. mem_saved: null (the memory pass and
 * scan are run again), or the buffer that forward filled (read only,
 * mem_saved_bytes >= gecko_memory_saved_size, 256-byte aligned, not aliasing
 * an output or the workspace): the backward reads the memory pass there,
 * with bit-identical results. Ignored without GECKO_PART_AWM or when no
 * chunk reads the memory. parts must include GECKO_PART_SCA; other
 * arguments and errors as gecko_backward. */
gecko_status gecko_backward_saved(
    const void* z,
    const float* kappa_q, const float* nu_q, const float* kappa_k, const float* nu_k,
    const float* eta_q, const float* rho_q, const float* eta_k, const float* rho_k,
    const void* v, const void* dout, const float* o_sca, const float* stats,
    const void* mem_saved, size_t mem_saved_bytes,
    float* dz, float* dv_out, float* daff,
    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
    gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags, unsigned parts,
    void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* gecko_status_string(gecko_status status);

/* Thread-local description of the last error returned on this thread
 * ("" if none). Valid until the next call on the same thread. */
const char* gecko_last_error(void);

/* ABI version (major * 100 + minor). */
int gecko_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GECKO_H */
