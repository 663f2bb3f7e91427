// C ABI of the Gecko SCA + AWM forward (declarations and contract in
// include/gecko.h): argument validation, workspace carve-up and the launch
// sequence on the caller's stream.
#include "gecko.h"

#include <stdarg.h>
#include <stdio.h>

#include <new>
#include <string>
#include <vector>

#include "gecko_internal.hpp"

namespace {

thread_local std::string g_last_error;

gecko_status fail(gecko_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gecko_status hip_fail(hipError_t e, const char* what) {
  return fail(GECKO_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_d(int64_t d) { return d == 32 || d == 64 || d == 128; }
bool valid_dv(int64_t dv) { return dv == 32 || dv == 64 || dv == 128 || dv == 256; }

int64_t nchunks_of(int64_t n, int64_t c) { return (n + c - 1) / c; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

enum Mode { kModeSca = 1, kModeAwm = 2 };

}  // namespace

namespace gecko {

Workspace carve_workspace(void* base, int64_t BH, int64_t n, int64_t d, int64_t dv, int64_t nmem, int64_t nsnap,
                          bool bf16, bool stream) {
  Workspace w{};
  const size_t rows = (size_t)BH * (size_t)nmem;
  const size_t e16 = bf16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return static_cast<char*>(base) + at;
  };
  w.g = reinterpret_cast<float*>(take(rows * d * dv * 4));
  w.h = take(rows * d * d * e16);
  w.cmax = reinterpret_cast<float*>(take(rows * d * 4));
  w.csum = reinterpret_cast<float*>(take(rows * d * 4));
  w.decay = reinterpret_cast<float*>(take(rows * d * 4));
  w.wscale = reinterpret_cast<float*>(take(rows * d * 4));
  w.snap = take((size_t)BH * (size_t)nsnap * dv * d * e16);
  w.rowstat = bf16 ? nullptr : reinterpret_cast<float*>(take((size_t)BH * n * 2 * 4));
  w.zfinal = stream ? reinterpret_cast<float*>(take((size_t)BH * d * 2 * 4)) : nullptr;
  w.bytes = nmem > 0 ? off : 0;
  return w;
}

size_t kept_memory_bytes(const Workspace& w, int64_t BH, int64_t nmem, int64_t d, int64_t dv) {
  return nmem > 0 ? align_up(w.bytes) + (size_t)BH * (size_t)nmem * (size_t)d * (size_t)dv * 4 : 0;
}

float* kept_states(const void* base, const Workspace& w) {
  return reinterpret_cast<float*>(const_cast<char*>(static_cast<const char*>(base)) + align_up(w.bytes));
}

// Streaming state (caller-owned device memory, 256-byte aligned arrays):
// the fp32 memory state M'^T in the scan's register layout, the running
// denominator (M, L) per feature, and the carried chunk of Z' and V.
struct StreamState {
  float* mstate;   // [BH][dv/32][d/32][64][16]
  float* zstate;   // [BH][d][2]
  void* zcarry;    // [BH][c][d]  bf16
  void* vcarry;    // [BH][c][dv] bf16
  size_t bytes;
};

StreamState carve_state(void* base, int64_t BH, int64_t d, int64_t dv, int64_t c) {
  StreamState t{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return static_cast<char*>(base) + at;
  };
  t.mstate = reinterpret_cast<float*>(take((size_t)BH * d * dv * 4));
  t.zstate = reinterpret_cast<float*>(take((size_t)BH * d * 2 * 4));
  t.zcarry = take((size_t)BH * c * d * 2);
  t.vcarry = take((size_t)BH * c * dv * 2);
  t.bytes = off;
  return t;
}

}  // namespace gecko

struct gecko_timer {
  std::vector<hipEvent_t> ev;  // 5 per recorded call
  int capacity = 0;
  int used = 0;
};

namespace {

struct Call {
  const void* z; const void* v; void* out;
  const float* aff[8];
  int64_t B, H, n, d, dv, c;
  gecko_dtype in_dtype, out_dtype;
  unsigned flags;
  void* ws; size_t ws_bytes;
  void* stream;
  int mode;
  gecko_timer* timer;
  // streaming (gecko_sca_awm_forward_stream)
  bool streaming;
  int64_t pos;
  void* state; size_t state_bytes;
  // gecko_forward_lse: per-query attention log-sum-exp output (bf16 only)
  float* lse;
  // gecko_forward_train: float32 attention output and per-query (m, l) (bf16 only)
  float* o_sca;
  float* stats;
  // gecko_sca_awm_forward_noalloc: the workspace is the library's scratch array
  bool noalloc;
  // gecko_forward_train with mem_saved: ws is mem_saved, which also receives
  // the states in float32 and the denominator steps the backward reads
  bool keep;
};

// memory steps and snapshot slots of a call (see gecko::Problem); lag 2 with
// sliding chunks, 1 for the chunk-wise variant (one call only)
void mem_counts(int64_t N, bool stream, bool has_prev, int64_t lag, int64_t& nmem, int64_t& nsnap) {
  if (stream) {
    nmem = (has_prev ? 1 : 0) + N - 1;
    nsnap = nmem + (has_prev ? 1 : 0);
  } else {
    nmem = N > lag ? N - lag : 0;
    nsnap = nmem;
  }
}

int64_t lag_of(unsigned flags) { return (flags & GECKO_CHUNKWISE) ? 1 : 2; }

gecko_status validate(const Call& k, gecko::Problem& p, bool& bf16) {
  if (k.B < 1 || k.H < 1 || k.n < 1 || k.c < 1)
    return fail(GECKO_EINVAL, "sizes must be >= 1 (B=%lld H=%lld n=%lld c=%lld)", (long long)k.B, (long long)k.H,
                (long long)k.n, (long long)k.c);
  if (k.d < 1 || k.dv < 1) return fail(GECKO_EINVAL, "d and dv must be >= 1");
  if (k.in_dtype != GECKO_F32 && k.in_dtype != GECKO_BF16) return fail(GECKO_EINVAL, "unknown input dtype %d", (int)k.in_dtype);
  if (k.out_dtype != GECKO_F32 && k.out_dtype != GECKO_BF16) return fail(GECKO_EINVAL, "unknown output dtype %d", (int)k.out_dtype);
  if (k.flags & ~(unsigned)(GECKO_AWM_NO_DELTA | GECKO_CHUNKWISE))
    return fail(GECKO_EINVAL, "unknown flag bits 0x%x", k.flags);
  if (k.streaming && (k.flags & GECKO_CHUNKWISE))
    return fail(GECKO_EUNSUPPORTED, "the streaming forward is built for sliding chunks only");
  if (!k.z || !k.v || !k.out) return fail(GECKO_EINVAL, "z, v and out must be non-null");
  if (!aligned16(k.z) || !aligned16(k.v) || !aligned16(k.out))
    return fail(GECKO_EINVAL, "z, v and out must be 16-byte aligned");
  const bool need_sca = k.mode & kModeSca, need_awm = k.mode & kModeAwm;
  for (int i = 0; i < 8; ++i) {
    const bool needed = (i < 4) ? need_sca : need_awm;
    if (needed && !k.aff[i]) return fail(GECKO_EINVAL, "affine vector %d is null", i);
    if (needed && (reinterpret_cast<uintptr_t>(k.aff[i]) & 3u)) return fail(GECKO_EINVAL, "affine vector %d misaligned", i);
  }
  if (!valid_d(k.d) || !valid_dv(k.dv))
    return fail(GECKO_EUNSUPPORTED, "unsupported (d, dv) = (%lld, %lld): d in {32,64,128}, dv in {32,64,128,256}",
                (long long)k.d, (long long)k.dv);
  bf16 = k.in_dtype == GECKO_BF16;
  if (!bf16 && k.out_dtype != GECKO_F32) return fail(GECKO_EUNSUPPORTED, "float32 input needs float32 output");
  if (bf16 && !gecko::bf16_shape_built(k.d, k.dv))
    return fail(GECKO_EUNSUPPORTED, "no bf16 kernels for (d, dv) = (%lld, %lld)", (long long)k.d, (long long)k.dv);
  if (k.B > (1 << 20) || k.H > (1 << 20) || k.n > (int64_t(1) << 40))
    return fail(GECKO_EINVAL, "sizes out of range");
  const int64_t BH = k.B * k.H;
  const int64_t N = nchunks_of(k.n, k.c);
  const bool has_prev = k.streaming && k.pos > 0;
  int64_t nmem = 0, nsnap = 0;
  const int64_t lag = lag_of(k.flags);
  mem_counts(N, k.streaming, has_prev, lag, nmem, nsnap);
  if (k.streaming) {
    if (!bf16) return fail(GECKO_EUNSUPPORTED, "the streaming forward is built for bf16 inputs only");
    if (k.c % 64) return fail(GECKO_EUNSUPPORTED, "the streaming forward needs c to be a multiple of 64");
    if (k.pos < 0 || k.pos % k.c)
      return fail(GECKO_EINVAL, "pos (%lld) must be a non-negative multiple of c (%lld)", (long long)k.pos,
                  (long long)k.c);
  }
  if (bf16) {
    // the bf16 kernels address one (batch, head) slab with 32-bit byte offsets
    const int64_t widest = k.d > k.dv ? k.d : k.dv;
    if ((k.n + 512) * widest * 2 > (int64_t)0xFFFFFFFF)
      return fail(GECKO_EUNSUPPORTED, "bf16 path needs n * max(d, dv) * 2 < 4 GiB per (batch, head) slab");
    const int64_t cc = k.c < k.n ? k.c : k.n;
    if (BH * N * ((cc + 127) / 128) >= ((int64_t)1 << 31) || BH * nmem >= ((int64_t)1 << 31) ||
        BH * (k.dv / 32) >= ((int64_t)1 << 31) || (k.streaming && k.c * k.dv * 2 > (int64_t)0xFFFFFFFF))
      return fail(GECKO_EUNSUPPORTED, "too many workgroups for one launch");
  }
  if (!bf16) {
    // one-dimensional grids (the fp32 kernels): fewer than 2^31 blocks each
    const int64_t lim = (int64_t)1 << 31;
    const int64_t ntok = nmem * k.c;
    if (BH * ((k.n + 63) / 64) * (k.dv / 32) >= lim || BH * ((ntok + 127) / 128) >= lim ||
        BH * nmem * ((k.d * (k.d + k.dv) + 255) / 256) >= lim)
      return fail(GECKO_EUNSUPPORTED, "too many workgroups for one launch");
  }
  const size_t esz = bf16 ? 2 : 4;
  const size_t osz = k.out_dtype == GECKO_BF16 ? 2 : 4;
  const size_t zb = (size_t)BH * k.n * k.d * esz, vb = (size_t)BH * k.n * k.dv * esz;
  const size_t ob = (size_t)BH * k.n * k.dv * osz;
  if (overlaps(k.out, ob, k.z, zb) || overlaps(k.out, ob, k.v, vb)) return fail(GECKO_EINVAL, "out aliases an input");
  if (k.streaming) {
    const gecko::StreamState t = gecko::carve_state(nullptr, BH, k.d, k.dv, k.c);
    if (!k.state) return fail(GECKO_EINVAL, "streaming state is null (need %zu bytes)", t.bytes);
    if (k.state_bytes < t.bytes)
      return fail(GECKO_EINVAL, "streaming state too small: %zu < %zu bytes", k.state_bytes, t.bytes);
    if (reinterpret_cast<uintptr_t>(k.state) & (kAlign - 1))
      return fail(GECKO_EINVAL, "streaming state must be 256-byte aligned");
    if (overlaps(k.state, t.bytes, k.z, zb) || overlaps(k.state, t.bytes, k.v, vb) ||
        overlaps(k.state, t.bytes, k.out, ob))
      return fail(GECKO_EINVAL, "streaming state aliases an input or the output");
    if (k.ws && overlaps(k.state, t.bytes, k.ws, k.ws_bytes))
      return fail(GECKO_EINVAL, "streaming state aliases the workspace");
  }
  if (need_awm && nmem > 0 && k.noalloc) {
    const gecko::Workspace w = gecko::carve_workspace(nullptr, BH, k.n, k.d, k.dv, nmem, nsnap, bf16, k.streaming);
    if (w.bytes > gecko::noalloc_scratch_bytes())
      return fail(GECKO_EWORKSPACE,
                  "these sizes need %zu bytes of scratch, more than the %zu bytes the allocation-free forward "
                  "holds per GPU; use gecko_sca_awm_forward with a caller workspace",
                  w.bytes, gecko::noalloc_scratch_bytes());
  } else if (need_awm && nmem > 0) {
    const gecko::Workspace w = gecko::carve_workspace(nullptr, BH, k.n, k.d, k.dv, nmem, nsnap, bf16, k.streaming);
    const size_t need = k.keep ? gecko::kept_memory_bytes(w, BH, nmem, k.d, k.dv) : w.bytes;
    const char* what = k.keep ? "mem_saved" : "workspace";
    if (!k.ws) return fail(GECKO_EWORKSPACE, "%s is null (need %zu bytes)", what, need);
    if (k.ws_bytes < need) return fail(GECKO_EWORKSPACE, "%s too small: %zu < %zu bytes", what, k.ws_bytes, need);
    if (reinterpret_cast<uintptr_t>(k.ws) & (kAlign - 1)) return fail(GECKO_EINVAL, "%s must be 256-byte aligned", what);
    if (overlaps(k.out, ob, k.ws, need)) return fail(GECKO_EINVAL, "out aliases the %s", what);
    // the chunk pass and the scan write the workspace before the attention
    // kernel reads z, v and the affine vectors
    if (overlaps(k.ws, need, k.z, zb) || overlaps(k.ws, need, k.v, vb))
      return fail(GECKO_EINVAL, "the %s aliases z or v", what);
    for (int i = 0; i < 8; ++i)
      if (k.aff[i] && overlaps(k.ws, need, k.aff[i], (size_t)k.H * k.d * 4))
        return fail(GECKO_EINVAL, "the %s aliases affine vector %d", what, i);
    if (k.lse && overlaps(k.ws, need, k.lse, (size_t)BH * k.n * 4))
      return fail(GECKO_EINVAL, "the %s aliases the log-sum-exp output", what);
    if (k.o_sca && overlaps(k.ws, need, k.o_sca, (size_t)BH * k.n * k.dv * 4))
      return fail(GECKO_EINVAL, "the %s aliases the attention output", what);
    if (k.stats && overlaps(k.ws, need, k.stats, (size_t)BH * k.n * 8))
      return fail(GECKO_EINVAL, "the %s aliases the attention statistics", what);
  }
  p.z = k.z; p.v = k.v; p.out = k.out;
  p.kappa_q = k.aff[0]; p.nu_q = k.aff[1]; p.kappa_k = k.aff[2]; p.nu_k = k.aff[3];
  p.eta_q = k.aff[4]; p.rho_q = k.aff[5]; p.eta_k = k.aff[6]; p.rho_k = k.aff[7];
  p.B = k.B; p.H = k.H; p.n = k.n; p.d = k.d; p.dv = k.dv; p.c = k.c;
  p.nchunks = N; p.nmem = nmem; p.nsnap = nsnap; p.flags = k.flags;
  {
    const int64_t before = k.streaming ? k.pos / k.c : 0;  // chunks of the sequence before this call
    p.first_read = before >= lag ? 0 : lag - before;
  }
  p.lag = lag;
  p.prev = (k.flags & GECKO_CHUNKWISE) ? 0 : 1;
  p.out_f32 = k.out_dtype == GECKO_F32;
  p.stream = k.streaming;
  p.has_prev = has_prev;
  p.zprev = p.vprev = nullptr;
  p.mstate = nullptr;
  p.zstate = nullptr;
  p.lse = k.lse;
  p.o_sca = k.o_sca;
  p.stats = k.stats;
  if (k.streaming) {
    const gecko::StreamState t = gecko::carve_state(k.state, BH, k.d, k.dv, k.c);
    p.mstate = t.mstate;
    p.zstate = t.zstate;
    if (has_prev) {
      p.zprev = t.zcarry;
      p.vprev = t.vcarry;
    }
  }
  return GECKO_OK;
}

gecko_status run(const Call& k) {
  gecko::Problem p;
  bool bf16 = false;
  gecko_status st = validate(k, p, bf16);
  if (st != GECKO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(k.stream);
  const bool do_awm = (k.mode & kModeAwm) && p.nmem > 0;
  void* ws = k.ws;
  if (k.noalloc && do_awm) {
    // the current device's copy of the scratch array; the stream must belong to it
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (s) {
      int sdev = -1;
      if ((e = hipStreamGetDevice(s, &sdev)) != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
      if (sdev != dev)
        return fail(GECKO_EINVAL, "the stream belongs to device %d, but device %d is current", sdev, dev);
    }
    if ((e = gecko::noalloc_scratch(dev, &ws)) != hipSuccess) return hip_fail(e, "scratch address lookup");
  }
  gecko::Workspace w{};
  if (do_awm) w = gecko::carve_workspace(ws, p.B * p.H, p.n, p.d, p.dv, p.nmem, p.nsnap, bf16, p.stream);
  if (do_awm && k.keep) w.snap32 = gecko::kept_states(ws, w);

  hipEvent_t* ev = nullptr;
  if (k.timer && k.timer->used < k.timer->capacity) ev = &k.timer->ev[5 * k.timer->used++];
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };

  hipError_t e = mark(0);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (do_awm) {
    e = bf16 ? gecko::launch_awm_chunk_bf16(p, w, s) : gecko::launch_awm_chunk_f32(p, w, s);
    if (e != hipSuccess) return hip_fail(e, "memory chunk pass launch");
    if ((e = mark(1)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if (!bf16 || k.keep) {  // the bf16 scan keeps the running denominator itself
      e = gecko::launch_awm_zscan(p, w, s);
      if (e != hipSuccess) return hip_fail(e, "denominator prefix launch");
    }
    if ((e = mark(2)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    e = bf16 ? gecko::launch_awm_scan_bf16(p, w, s) : gecko::launch_awm_scan_f32(p, w, s);
    if (e != hipSuccess) return hip_fail(e, "memory scan launch");
    if ((e = mark(3)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  } else {
    for (int i = 1; i <= 3; ++i)
      if ((e = mark(i)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  // attention (bit 0) and readout (bit 1). With at most two chunks no chunk
  // reads the memory and the readout writes its exact zeros.
  const int mode = (k.mode & kModeSca ? 1 : 0) | (k.mode & kModeAwm ? 2 : 0);
  e = bf16 ? gecko::launch_sca_bf16(p, w, mode, s) : gecko::launch_sca_f32(p, w, mode, s);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  if ((e = mark(4)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (p.stream) {
    // a sequence whose first call enters nothing: empty memory state
    const gecko::StreamState t = gecko::carve_state(k.state, p.B * p.H, p.d, p.dv, p.c);
    if (p.nmem == 0 && (e = gecko::launch_stream_reset(t.mstate, t.zstate, p.B * p.H, p.d, p.dv, s)) != hipSuccess)
      return hip_fail(e, "stream state reset launch");
    // the last chunk of this call is carried to the next one
    const int64_t row0 = (p.nchunks - 1) * p.c;
    e = gecko::launch_stream_finish(p, w, t.zcarry, t.vcarry, t.zstate, row0, p.n - row0, s);
    if (e != hipSuccess) return hip_fail(e, "stream state update launch");
  }
  g_last_error.clear();
  return GECKO_OK;
}

}  // namespace

extern "C" {

size_t gecko_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c, gecko_dtype in_dtype) {
  if (B < 1 || H < 1 || n < 1 || c < 1 || !valid_d(d) || !valid_dv(dv)) return (size_t)-1;
  if (in_dtype != GECKO_F32 && in_dtype != GECKO_BF16) return (size_t)-1;
  return gecko_workspace_size_for(B, H, n, d, dv, c, in_dtype, 0u);
}

size_t gecko_workspace_size_for(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                                gecko_dtype in_dtype, unsigned flags) {
  if (B < 1 || H < 1 || n < 1 || c < 1 || !valid_d(d) || !valid_dv(dv)) return (size_t)-1;
  if (in_dtype != GECKO_F32 && in_dtype != GECKO_BF16) return (size_t)-1;
  if (flags & ~(unsigned)(GECKO_AWM_NO_DELTA | GECKO_CHUNKWISE)) return (size_t)-1;
  int64_t nmem = 0, nsnap = 0;
  mem_counts(nchunks_of(n, c), false, false, lag_of(flags), nmem, nsnap);
  return gecko::carve_workspace(nullptr, B * H, n, d, dv, nmem, nsnap, in_dtype == GECKO_BF16, false).bytes;
}

size_t gecko_memory_saved_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                               gecko_dtype in_dtype, unsigned flags) {
  if (B < 1 || H < 1 || n < 1 || c < 1 || in_dtype != GECKO_BF16 || !gecko::bwd_shape_built(d, dv)) return (size_t)-1;
  if (flags & ~(unsigned)(GECKO_AWM_NO_DELTA | GECKO_CHUNKWISE)) return (size_t)-1;
  int64_t nmem = 0, nsnap = 0;
  mem_counts(nchunks_of(n, c), false, false, lag_of(flags), nmem, nsnap);
  const gecko::Workspace w = gecko::carve_workspace(nullptr, B * H, n, d, dv, nmem, nsnap, true, false);
  return gecko::kept_memory_bytes(w, B * H, nmem, d, dv);
}

gecko_status gecko_sca_awm_forward_timed(const void* z, const float* kappa_q, const float* nu_q,
                                         const float* kappa_k, const float* nu_k, const float* eta_q,
                                         const float* rho_q, const float* eta_k, const float* rho_k, const void* v,
                                         void* out, int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                                         gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags, void* workspace,
                                         size_t workspace_bytes, void* stream, gecko_timer* timer) {
  try {
    Call k{z, v, out, {kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k}, B, H, n, d, dv, c,
           in_dtype, out_dtype, flags, workspace, workspace_bytes, stream, kModeSca | kModeAwm, timer};
    return run(k);
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

gecko_status gecko_sca_awm_forward(const void* z, const float* kappa_q, const float* nu_q, const float* kappa_k,
                                   const float* nu_k, const float* eta_q, const float* rho_q, const float* eta_k,
                                   const float* rho_k, const void* v, void* out, int64_t B, int64_t H, int64_t n,
                                   int64_t d, int64_t dv, int64_t c, gecko_dtype in_dtype, gecko_dtype out_dtype,
                                   unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  return gecko_sca_awm_forward_timed(z, kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k, v, out, B, H, n, d,
                                     dv, c, in_dtype, out_dtype, flags, workspace, workspace_bytes, stream, nullptr);
}

gecko_status gecko_sca_awm_forward_noalloc(const void* z, const float* kappa_q, const float* nu_q,
                                           const float* kappa_k, const float* nu_k, const float* eta_q,
                                           const float* rho_q, const float* eta_k, const float* rho_k, const void* v,
                                           void* out, int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                                           int64_t c, gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
                                           void* stream) {
  try {
    Call k{z, v, out, {kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k}, B, H, n, d, dv, c,
           in_dtype, out_dtype, flags, nullptr, 0, stream, kModeSca | kModeAwm, nullptr};
    k.noalloc = true;
    return run(k);
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

gecko_status gecko_sca_forward(const void* z, const float* kappa_q, const float* nu_q, const float* kappa_k,
                               const float* nu_k, const void* v, void* out, int64_t B, int64_t H, int64_t n, int64_t d,
                               int64_t dv, int64_t c, gecko_dtype in_dtype, gecko_dtype out_dtype, void* stream) {
  try {
    Call k{z, v, out, {kappa_q, nu_q, kappa_k, nu_k, nullptr, nullptr, nullptr, nullptr}, B, H, n, d, dv, c,
           in_dtype, out_dtype, 0u, nullptr, 0, stream, kModeSca, nullptr};
    return run(k);
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

gecko_status gecko_awm_forward(const void* z, const float* eta_q, const float* rho_q, const float* eta_k,
                               const float* rho_k, const void* v, void* out, int64_t B, int64_t H, int64_t n, int64_t d,
                               int64_t dv, int64_t c, gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
                               void* workspace, size_t workspace_bytes, void* stream) {
  try {
    Call k{z, v, out, {nullptr, nullptr, nullptr, nullptr, eta_q, rho_q, eta_k, rho_k}, B, H, n, d, dv, c,
           in_dtype, out_dtype, flags, workspace, workspace_bytes, stream, kModeAwm, nullptr};
    return run(k);
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

size_t gecko_cema_workspace_size(int64_t B, int64_t n, int64_t D, int64_t h) {
  if (B < 1 || n < 1 || D < 1 || !(h == 1 || h == 2 || h == 4 || h == 8 || h == 16)) return (size_t)-1;
  return gecko::cema_plan(B, n, D, h).bytes;
}

gecko_status gecko_cema_forward(const void* x, const float* alpha, const float* delta, const float* theta,
                                const float* beta, const float* eta, const uint8_t* reset, const float* h0, void* y,
                                float* h_final, int64_t B, int64_t n, int64_t D, int64_t h, gecko_dtype in_dtype,
                                gecko_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (B < 1 || n < 1 || D < 1) return fail(GECKO_EINVAL, "sizes must be >= 1");
    if (!(h == 1 || h == 2 || h == 4 || h == 8 || h == 16))
      return fail(GECKO_EUNSUPPORTED, "hidden dimensions per input dimension must be 1, 2, 4, 8 or 16 (got %lld)",
                  (long long)h);
    if ((in_dtype != GECKO_F32 && in_dtype != GECKO_BF16) || (out_dtype != GECKO_F32 && out_dtype != GECKO_BF16))
      return fail(GECKO_EINVAL, "unknown dtype");
    if (!x || !y || !alpha || !delta || !theta || !beta || !eta)
      return fail(GECKO_EINVAL, "x, y and the parameter vectors must be non-null");
    const void* ptrs[] = {x, y, alpha, delta, theta, beta, eta, h0, h_final};
    for (const void* q : ptrs)
      if (reinterpret_cast<uintptr_t>(q) & 3u) return fail(GECKO_EINVAL, "pointers must be 4-byte aligned");
    if (B > 65535 || n > (int64_t(1) << 40) || D > (1 << 24)) return fail(GECKO_EINVAL, "sizes out of range");
    const size_t ib = in_dtype == GECKO_BF16 ? 2 : 4, ob = out_dtype == GECKO_BF16 ? 2 : 4;
    const size_t xb = (size_t)B * n * D * ib, yb = (size_t)B * n * D * ob, sb = (size_t)B * D * h * 8;
    if (overlaps(y, yb, x, xb)) return fail(GECKO_EINVAL, "y aliases x");
    if (h_final && (overlaps(h_final, sb, y, yb) || overlaps(h_final, sb, x, xb) || (h0 && overlaps(h_final, sb, h0, sb))))
      return fail(GECKO_EINVAL, "h_final aliases another buffer");
    const gecko::CemaPlan plan = gecko::cema_plan(B, n, D, h);
    if (B * plan.nwd * plan.C >= ((int64_t)1 << 31)) return fail(GECKO_EUNSUPPORTED, "too many workgroups for one launch");
    if (plan.bytes > 0) {
      if (!workspace) return fail(GECKO_EWORKSPACE, "workspace is null (need %zu bytes)", plan.bytes);
      if (workspace_bytes < plan.bytes)
        return fail(GECKO_EWORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, plan.bytes);
      if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
        return fail(GECKO_EINVAL, "workspace must be 256-byte aligned");
      if (overlaps(workspace, plan.bytes, y, yb) || (h_final && overlaps(workspace, plan.bytes, h_final, sb)))
        return fail(GECKO_EINVAL, "workspace aliases an output");
    }
    gecko::CemaProblem q;
    q.x = x; q.y = y; q.alpha = alpha; q.delta = delta; q.theta = theta; q.beta = beta; q.eta = eta;
    q.reset = reset; q.h0 = h0; q.hfin = h_final;
    q.B = B; q.n = n; q.D = D; q.H = h;
    q.in_bf16 = in_dtype == GECKO_BF16;
    q.out_bf16 = out_dtype == GECKO_BF16;
    const hipError_t e = gecko::launch_cema(q, plan, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "CEMA kernel launch");
    g_last_error.clear();
    return GECKO_OK;
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

size_t gecko_tdn_workspace_size(int64_t B, int64_t n, int64_t D, int64_t G) {
  if (B < 1 || n < 1 || D < 1 || G < 1 || D % G || (D / G) % 8 || D > 8192) return (size_t)-1;
  return gecko::tdn_plan(B, n, G).bytes;
}

gecko_status gecko_tdn_forward(const void* x, const float* gamma, const float* shift, const float* m0,
                               const float* v0, int64_t t0, void* y, float* m_out, float* v_out, int64_t B,
                               int64_t n, int64_t D, int64_t G, float beta1, float beta2, float eps,
                               gecko_dtype in_dtype, gecko_dtype out_dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  try {
    if (B < 1 || n < 1 || D < 1 || G < 1 || t0 < 0) return fail(GECKO_EINVAL, "sizes must be >= 1 and t0 >= 0");
    if (D % G || (D / G) % 8)
      return fail(GECKO_EUNSUPPORTED, "groups must split D into equal runs of a multiple of 8 features");
    if (D > 8192) return fail(GECKO_EUNSUPPORTED, "D up to 8192");
    if (!(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f) || !(eps > 0.f))
      return fail(GECKO_EINVAL, "decay factors must lie in [0, 1) and eps must be > 0");
    if ((in_dtype != GECKO_F32 && in_dtype != GECKO_BF16) || (out_dtype != GECKO_F32 && out_dtype != GECKO_BF16))
      return fail(GECKO_EINVAL, "unknown dtype");
    if (!x || !y || !gamma || !shift) return fail(GECKO_EINVAL, "x, y, gamma and shift must be non-null");
    if (!aligned16(x) || !aligned16(y) || !aligned16(gamma) || !aligned16(shift))
      return fail(GECKO_EINVAL, "x, y, gamma and shift must be 16-byte aligned");
    const void* small[] = {m0, v0, m_out, v_out};
    for (const void* q : small)
      if (reinterpret_cast<uintptr_t>(q) & 3u) return fail(GECKO_EINVAL, "state pointers must be 4-byte aligned");
    if (B * n >= ((int64_t)1 << 31) || B > 65535) return fail(GECKO_EUNSUPPORTED, "B * n must stay below 2^31");
    const size_t ib = in_dtype == GECKO_BF16 ? 2 : 4, ob = out_dtype == GECKO_BF16 ? 2 : 4;
    const size_t xb = (size_t)B * n * D * ib, yb = (size_t)B * n * D * ob;
    if (overlaps(y, yb, x, xb)) return fail(GECKO_EINVAL, "y aliases x");
    const gecko::TdnPlan plan = gecko::tdn_plan(B, n, G);
    if (!workspace) return fail(GECKO_EWORKSPACE, "workspace is null (need %zu bytes)", plan.bytes);
    if (workspace_bytes < plan.bytes)
      return fail(GECKO_EWORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, plan.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
      return fail(GECKO_EINVAL, "workspace must be 256-byte aligned");
    if (overlaps(workspace, plan.bytes, y, yb) || overlaps(workspace, plan.bytes, x, xb))
      return fail(GECKO_EINVAL, "workspace aliases x or y");
    gecko::TdnProblem p;
    p.x = x; p.y = y; p.gamma = gamma; p.shift = shift; p.m0 = m0; p.v0 = v0; p.m_out = m_out; p.v_out = v_out;
    p.B = B; p.n = n; p.D = D; p.G = G; p.t0 = t0;
    p.beta1 = beta1; p.beta2 = beta2; p.eps = eps;
    p.in_bf16 = in_dtype == GECKO_BF16;
    p.out_bf16 = out_dtype == GECKO_BF16;
    const hipError_t e = gecko::launch_tdn(p, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "TDN kernel launch");
    g_last_error.clear();
    return GECKO_OK;
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

size_t gecko_stream_state_size(int64_t B, int64_t H, int64_t d, int64_t dv, int64_t c, gecko_dtype in_dtype) {
  if (B < 1 || H < 1 || c < 1 || !valid_d(d) || !valid_dv(dv) || in_dtype != GECKO_BF16) return (size_t)-1;
  return gecko::carve_state(nullptr, B * H, d, dv, c).bytes;
}

size_t gecko_stream_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                                   gecko_dtype in_dtype) {
  if (B < 1 || H < 1 || n < 1 || c < 1 || !valid_d(d) || !valid_dv(dv) || in_dtype != GECKO_BF16) return (size_t)-1;
  int64_t nmem = 0, nsnap = 0;
  mem_counts(nchunks_of(n, c), true, true, 2, nmem, nsnap);  // the larger case: a carried chunk
  return gecko::carve_workspace(nullptr, B * H, n, d, dv, nmem, nsnap, true, true).bytes;
}

gecko_status gecko_sca_awm_forward_stream(const void* z, const float* kappa_q, const float* nu_q,
                                          const float* kappa_k, const float* nu_k, const float* eta_q,
                                          const float* rho_q, const float* eta_k, const float* rho_k, const void* v,
                                          void* out, int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                                          int64_t c, int64_t pos, gecko_dtype in_dtype, gecko_dtype out_dtype,
                                          unsigned flags, void* state, size_t state_bytes, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  try {
    Call k{z, v, out, {kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k}, B, H, n, d, dv, c,
           in_dtype, out_dtype, flags, workspace, workspace_bytes, stream, kModeSca | kModeAwm, nullptr,
           true, pos, state, state_bytes};
    return run(k);
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

gecko_status gecko_forward_lse(const void* z, const float* kappa_q, const float* nu_q, const float* kappa_k,
                               const float* nu_k, const float* eta_q, const float* rho_q, const float* eta_k,
                               const float* rho_k, const void* v, void* out, float* lse, int64_t B, int64_t H,
                               int64_t n, int64_t d, int64_t dv, int64_t c, gecko_dtype in_dtype,
                               gecko_dtype out_dtype, unsigned flags, unsigned parts, void* workspace,
                               size_t workspace_bytes, void* stream) {
  try {
    if (!(parts & GECKO_PART_SCA) || (parts & ~3u))
      return fail(GECKO_EINVAL, "parts must hold GECKO_PART_SCA (and may hold GECKO_PART_AWM)");
    if (in_dtype != GECKO_BF16) return fail(GECKO_EUNSUPPORTED, "the log-sum-exp output is built for bf16 inputs only");
    if (!lse) return fail(GECKO_EINVAL, "lse must be non-null");
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(GECKO_EINVAL, "lse must be 4-byte aligned");
    if (B >= 1 && H >= 1 && n >= 1 && dv >= 1 && out && B <= (1 << 20) && H <= (1 << 20) && n <= (int64_t(1) << 40)) {
      const size_t lb = (size_t)B * H * n * 4;
      const size_t ob = (size_t)B * H * n * dv * (out_dtype == GECKO_BF16 ? 2 : 4);
      if (overlaps(lse, lb, out, ob) || (workspace && overlaps(lse, lb, workspace, workspace_bytes)))
        return fail(GECKO_EINVAL, "lse aliases the output or the workspace");
    }
    const int mode = (parts & GECKO_PART_SCA ? kModeSca : 0) | (parts & GECKO_PART_AWM ? kModeAwm : 0);
    Call k{z, v, out, {kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k}, B, H, n, d, dv, c,
           in_dtype, out_dtype, flags, workspace, workspace_bytes, stream, mode, nullptr};
    k.lse = lse;
    return run(k);
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

gecko_status gecko_forward_train(const void* z, const float* kappa_q, const float* nu_q, const float* kappa_k,
                                 const float* nu_k, const float* eta_q, const float* rho_q, const float* eta_k,
                                 const float* rho_k, const void* v, void* out, float* o_sca, float* stats,
                                 void* mem_saved, size_t mem_saved_bytes, int64_t B, int64_t H, int64_t n, int64_t d,
                                 int64_t dv, int64_t c, gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
                                 unsigned parts, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!(parts & GECKO_PART_SCA) || (parts & ~3u))
      return fail(GECKO_EINVAL, "parts must hold GECKO_PART_SCA (and may hold GECKO_PART_AWM)");
    if (in_dtype != GECKO_BF16) return fail(GECKO_EUNSUPPORTED, "the training forward is built for bf16 inputs only");
    if (!gecko::bwd_shape_built(d, dv))
      return fail(GECKO_EUNSUPPORTED, "the training forward is built for (d, dv) in {(128, 256), (128, 128)}");
    if (!o_sca || !stats) return fail(GECKO_EINVAL, "o_sca and stats must be non-null");
    if (!aligned16(o_sca) || (reinterpret_cast<uintptr_t>(stats) & 7u))
      return fail(GECKO_EINVAL, "o_sca must be 16-byte and stats 8-byte aligned");
    // with mem_saved, the memory pass writes there (and the workspace goes unused)
    const bool keep = mem_saved && (parts & GECKO_PART_AWM);
    if (keep) {
      workspace = mem_saved;
      workspace_bytes = mem_saved_bytes;
    }
    if (B >= 1 && H >= 1 && n >= 1 && out && B <= (1 << 20) && H <= (1 << 20) && n <= (int64_t(1) << 40)) {
      const size_t BH = (size_t)B * H;
      const size_t sb = BH * n * 8, ab = BH * n * dv * 4;
      const size_t ob = BH * n * dv * (out_dtype == GECKO_BF16 ? 2 : 4);
      const void* in[] = {z, v};
      const size_t ib[] = {BH * n * d * 2, BH * n * dv * 2};
      if (overlaps(o_sca, ab, stats, sb) || overlaps(o_sca, ab, out, ob) || overlaps(stats, sb, out, ob) ||
          (workspace && (overlaps(o_sca, ab, workspace, workspace_bytes) ||
                         overlaps(stats, sb, workspace, workspace_bytes))))
        return fail(GECKO_EINVAL, "o_sca and stats must not alias each other, the output or the %s",
                    keep ? "mem_saved" : "workspace");
      for (int i = 0; i < 2; ++i)
        if (in[i] && (overlaps(o_sca, ab, in[i], ib[i]) || overlaps(stats, sb, in[i], ib[i])))
          return fail(GECKO_EINVAL, "o_sca and stats must not alias an input");
    }
    const int mode = (parts & GECKO_PART_SCA ? kModeSca : 0) | (parts & GECKO_PART_AWM ? kModeAwm : 0);
    Call k{z, v, out, {kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k}, B, H, n, d, dv, c,
           in_dtype, out_dtype, flags, workspace, workspace_bytes, stream, mode, nullptr};
    k.o_sca = o_sca;
    k.stats = stats;
    k.keep = keep;
    return run(k);
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

}  // extern "C"

namespace {

// the forward description the backward kernels share (one call, no stream)
gecko_status bwd_problem(const void* z, const float* const (&aff)[8], const void* v, const void* dout, float* dz,
                         float* dv_out, float* daff, int64_t B,
                         int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c, gecko_dtype in_dtype,
                         gecko_dtype out_dtype, unsigned flags, unsigned parts, bool check_ptrs,
                         gecko::BwdProblem& p) {
  if (B < 1 || H < 1 || n < 1 || c < 1 || d < 1 || dv < 1)
    return fail(GECKO_EINVAL, "sizes must be >= 1");
  if (B > (1 << 20) || H > (1 << 20) || n > (int64_t(1) << 40)) return fail(GECKO_EINVAL, "sizes out of range");
  if (in_dtype != GECKO_F32 && in_dtype != GECKO_BF16) return fail(GECKO_EINVAL, "unknown input dtype %d", (int)in_dtype);
  if (out_dtype != GECKO_F32 && out_dtype != GECKO_BF16) return fail(GECKO_EINVAL, "unknown output dtype %d", (int)out_dtype);
  if (flags & ~(unsigned)(GECKO_AWM_NO_DELTA | GECKO_CHUNKWISE)) return fail(GECKO_EINVAL, "unknown flag bits 0x%x", flags);
  if (parts < 1 || parts > 3) return fail(GECKO_EINVAL, "parts must be GECKO_PART_SCA, GECKO_PART_AWM or both");
  if (in_dtype != GECKO_BF16) return fail(GECKO_EUNSUPPORTED, "the backward is built for bf16 inputs only");
  if (!gecko::bwd_shape_built(d, dv))
    return fail(GECKO_EUNSUPPORTED, "the backward is built for (d, dv) in {(128, 256), (128, 128)}");
  if ((n + 512) * (d > dv ? d : dv) * 2 > (int64_t)0xFFFFFFFF)
    return fail(GECKO_EUNSUPPORTED, "the backward needs n * max(d, dv) * 2 < 4 GiB per (batch, head) slab");
  const int64_t BH = B * H;
  const int64_t N = nchunks_of(n, c);
  const int64_t cc = c < n ? c : n;
  if (BH * N * ((cc + 255) / 256) >= ((int64_t)1 << 31) || BH * ((n + 255) / 256) >= ((int64_t)1 << 31))
    return fail(GECKO_EUNSUPPORTED, "too many workgroups for one launch");
  const bool sca = parts & GECKO_PART_SCA, awm = parts & GECKO_PART_AWM;
  if (check_ptrs) {
    if (!z || !v || !dout || !dz || !dv_out || !daff) return fail(GECKO_EINVAL, "z, v, dout, dz, dv and daff must be non-null");
    const void* a16[] = {z, v, dout, dz, dv_out};
    for (const void* q : a16)
      if (reinterpret_cast<uintptr_t>(q) & 15u) return fail(GECKO_EINVAL, "z, v, dout, dz and dv must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(daff) & 3u) return fail(GECKO_EINVAL, "daff must be 4-byte aligned");
    for (int i = 0; i < 8; ++i) {
      const bool needed = i < 4 ? sca : awm;
      if (needed && !aff[i]) return fail(GECKO_EINVAL, "affine vector %d is null", i);
      if (needed && (reinterpret_cast<uintptr_t>(aff[i]) & 15u))
        return fail(GECKO_EINVAL, "affine vector %d must be 16-byte aligned", i);
    }
    const size_t osz = out_dtype == GECKO_BF16 ? 2 : 4;
    const size_t zb = (size_t)BH * n * d * 2, vb = (size_t)BH * n * dv * 2, ob = (size_t)BH * n * dv * osz;
    const size_t dzb = (size_t)BH * n * d * 4, dvb = (size_t)BH * n * dv * 4, ab = (size_t)8 * H * d * 4;
    struct R { const void* p; size_t b; } outs[] = {{dz, dzb}, {dv_out, dvb}, {daff, ab}};
    struct R ins[] = {{z, zb}, {v, vb}, {dout, ob}};
    for (int i = 0; i < 3; ++i) {
      for (const R& r : ins)
        if (r.p && overlaps(outs[i].p, outs[i].b, r.p, r.b)) return fail(GECKO_EINVAL, "a gradient output aliases an input");
      for (int j = i + 1; j < 3; ++j)
        if (overlaps(outs[i].p, outs[i].b, outs[j].p, outs[j].b)) return fail(GECKO_EINVAL, "gradient outputs overlap");
    }
  }
  gecko::Problem& f = p.f;
  f = gecko::Problem{};
  f.z = z; f.v = v; f.out = nullptr;
  f.kappa_q = aff[0]; f.nu_q = aff[1]; f.kappa_k = aff[2]; f.nu_k = aff[3];
  f.eta_q = aff[4]; f.rho_q = aff[5]; f.eta_k = aff[6]; f.rho_k = aff[7];
  f.B = B; f.H = H; f.n = n; f.d = d; f.dv = dv; f.c = c;
  f.nchunks = N;
  const int64_t lag = lag_of(flags);
  int64_t nmem = 0, nsnap = 0;
  mem_counts(N, false, false, lag, nmem, nsnap);
  f.nmem = nmem; f.nsnap = nsnap; f.flags = flags;
  f.first_read = lag; f.lag = lag; f.prev = (flags & GECKO_CHUNKWISE) ? 0 : 1;
  f.out_f32 = out_dtype == GECKO_F32;
  f.stream = false; f.has_prev = false;
  p.dout = dout; p.dz = dz; p.dv = dv_out; p.daff = daff;
  p.sca = sca; p.awm = awm; p.out_f32 = out_dtype == GECKO_F32;
  p.saved = false; p.o_sca = nullptr; p.stats = nullptr; p.mem_saved = nullptr;
  return GECKO_OK;
}

}  // namespace

namespace gecko {

BwdWorkspace carve_bwd_workspace(void* base, const BwdProblem& p) {
  BwdWorkspace w{};
  const Problem& f = p.f;
  const size_t BH = (size_t)(f.B * f.H), n = (size_t)f.n, d = (size_t)f.d, dv = (size_t)f.dv;
  const size_t nm = (size_t)f.nmem;
  size_t off = 0;
  const bool mem = p.awm && f.nmem > 0;
  const bool kept = mem && p.mem_saved;  // the training forward's memory pass, read in place
  if (mem) {
    w.fw = carve_workspace(kept ? const_cast<void*>(p.mem_saved) : base, f.B * f.H, f.n, f.d, f.dv, f.nmem, f.nsnap,
                           true, false);
    if (!kept) off = align_up(w.fw.bytes);
  }
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return static_cast<char*>(base) + at;
  };
  if (p.sca) {
    w.qp = reinterpret_cast<uint16_t*>(take(BH * n * d * 2));
    w.ld = reinterpret_cast<float*>(take(BH * n * 8));
    w.dq = reinterpret_cast<float*>(take(BH * n * d * 4));
    w.dk = reinterpret_cast<float*>(take(BH * n * d * 4));
  }
  if (p.out_f32) w.do16 = reinterpret_cast<uint16_t*>(take(BH * n * dv * 2));
  if (p.saved && p.sca) w.dos = reinterpret_cast<uint16_t*>(take(BH * n * dv * 2));
  if (p.awm) {
    w.dqm = reinterpret_cast<float*>(take(BH * n * d * 4));
    w.dkm = reinterpret_cast<float*>(take(BH * n * d * 4));
  }
  if (mem) {
    w.r = reinterpret_cast<float*>(take(BH * nm * d * dv * 4));
    w.ht = reinterpret_cast<uint16_t*>(take(BH * nm * d * d * 2));
    w.ds = reinterpret_cast<uint16_t*>(take(BH * nm * d * dv * 2));
    w.part = reinterpret_cast<float*>(take(BH * nm * (dv / 32) * d * 2 * 4));
    w.zeta = reinterpret_cast<float*>(take(BH * nm * d * 4));
    w.x = reinterpret_cast<uint16_t*>(take(BH * nm * d * d * 2));
    w.s32 = kept ? kept_states(p.mem_saved, w.fw) : reinterpret_cast<float*>(take(BH * nm * d * dv * 4));
    w.fw.snap32 = w.s32;
  }
  w.rows_per_blk = 256;
  w.nblk = (f.n + w.rows_per_blk - 1) / w.rows_per_blk;
  w.apart = reinterpret_cast<float*>(take(BH * (size_t)w.nblk * 8 * d * 4));
  w.bytes = off;
  return w;
}

}  // namespace gecko

extern "C" {

size_t gecko_backward_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                                     gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags, unsigned parts) {
  const float* none[8] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  gecko::BwdProblem p;
  const std::string saved = g_last_error;
  if (bwd_problem(nullptr, none, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, n, d, dv, c, in_dtype, out_dtype,
                  flags, parts, false, p) != GECKO_OK) {
    g_last_error = saved;
    return (size_t)-1;
  }
  return gecko::carve_bwd_workspace(nullptr, p).bytes;
}

size_t gecko_backward_saved_workspace_size(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int64_t c,
                                           gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
                                           unsigned parts) {
  const float* none[8] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  gecko::BwdProblem p;
  const std::string saved = g_last_error;
  if (bwd_problem(nullptr, none, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, n, d, dv, c, in_dtype, out_dtype,
                  flags, parts, false, p) != GECKO_OK || !p.sca) {
    g_last_error = saved;
    return (size_t)-1;
  }
  p.saved = true;
  return gecko::carve_bwd_workspace(nullptr, p).bytes;
}

}  // extern "C"

namespace {

// workspace and alias checks, then the launch sequence of both backward entry points
gecko_status run_backward(const gecko::BwdProblem& p, void* workspace, size_t workspace_bytes, void* stream) {
  const gecko::BwdWorkspace need = gecko::carve_bwd_workspace(nullptr, p);
  if (!workspace) return fail(GECKO_EWORKSPACE, "workspace is null (need %zu bytes)", need.bytes);
  if (workspace_bytes < need.bytes)
    return fail(GECKO_EWORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
    return fail(GECKO_EINVAL, "workspace must be 256-byte aligned");
  {
    const gecko::Problem& f = p.f;
    const size_t BH = (size_t)(f.B * f.H), n = (size_t)f.n, d = (size_t)f.d, dv = (size_t)f.dv;
    const void* o[] = {f.z, f.v, p.dout, p.dz, p.dv, p.daff, p.o_sca, p.stats};
    const size_t ob = BH * n * dv * (p.out_f32 ? 4 : 2);
    const size_t b[] = {BH * n * d * 2, BH * n * dv * 2, ob, BH * n * d * 4, BH * n * dv * 4,
                        (size_t)8 * f.H * d * 4, BH * n * dv * 4, BH * n * 8};
    for (int i = 0; i < 8; ++i)
      if (o[i] && overlaps(workspace, need.bytes, o[i], b[i]))
        return fail(GECKO_EINVAL, "the workspace aliases an input or an output");
    if (p.saved)
      for (int i = 6; i < 8; ++i)
        for (int j = 3; j < 6; ++j)
          if (o[j] && overlaps(o[i], b[i], o[j], b[j]))
            return fail(GECKO_EINVAL, "o_sca and stats must not alias an output");
    if (p.mem_saved) {
      const gecko::Workspace mw = gecko::carve_workspace(nullptr, f.B * f.H, f.n, f.d, f.dv, f.nmem, f.nsnap, true, false);
      const size_t mb = gecko::kept_memory_bytes(mw, f.B * f.H, f.nmem, f.d, f.dv);
      if (overlaps(p.mem_saved, mb, workspace, need.bytes))
        return fail(GECKO_EINVAL, "mem_saved aliases the workspace");
      for (int j = 3; j < 6; ++j)
        if (o[j] && overlaps(p.mem_saved, mb, o[j], b[j])) return fail(GECKO_EINVAL, "mem_saved aliases an output");
    }
  }
  const gecko::BwdWorkspace w = gecko::carve_bwd_workspace(workspace, p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p.out_f32 && (e = gecko::launch_bwd_dout16(p, w, s)) != hipSuccess) return hip_fail(e, "dO conversion launch");
  if (p.awm && (e = gecko::launch_bwd_awm(p, w, s)) != hipSuccess) return hip_fail(e, "memory backward launch");
  if (p.sca) {
    if ((e = gecko::launch_bwd_prep(p, w, s)) != hipSuccess) return hip_fail(e, "attention backward prep launch");
    if (p.saved && (e = gecko::launch_bwd_saved_prep(p, w, s)) != hipSuccess)
      return hip_fail(e, "saved statistics launch");
    if ((e = gecko::launch_bwd_dq(p, w, s)) != hipSuccess) return hip_fail(e, "attention dQ launch");
    if ((e = gecko::launch_bwd_dkdv(p, w, p.awm, s)) != hipSuccess) return hip_fail(e, "attention dK dV launch");
  }
  if ((e = gecko::launch_bwd_combine(p, w, s)) != hipSuccess) return hip_fail(e, "gradient combine launch");
  g_last_error.clear();
  return GECKO_OK;
}

}  // namespace

extern "C" {

gecko_status gecko_backward(const void* z, const float* kappa_q, const float* nu_q, const float* kappa_k,
                            const float* nu_k, const float* eta_q, const float* rho_q, const float* eta_k,
                            const float* rho_k, const void* v, const void* dout, float* dz, float* dv_out,
                            float* daff, int64_t B, int64_t H, int64_t n, int64_t d,
                            int64_t dv, int64_t c, gecko_dtype in_dtype, gecko_dtype out_dtype, unsigned flags,
                            unsigned parts, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    const float* aff[8] = {kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k};
    gecko::BwdProblem p;
    gecko_status st = bwd_problem(z, aff, v, dout, dz, dv_out, daff, B, H, n, d, dv, c, in_dtype, out_dtype, flags,
                                  parts, true, p);
    if (st != GECKO_OK) return st;
    return run_backward(p, workspace, workspace_bytes, stream);
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

gecko_status gecko_backward_saved(const void* z, const float* kappa_q, const float* nu_q, const float* kappa_k,
                                  const float* nu_k, const float* eta_q, const float* rho_q, const float* eta_k,
                                  const float* rho_k, const void* v, const void* dout, const float* o_sca,
                                  const float* stats, const void* mem_saved, size_t mem_saved_bytes, float* dz,
                                  float* dv_out, float* daff, int64_t B, int64_t H,
                                  int64_t n, int64_t d, int64_t dv, int64_t c, gecko_dtype in_dtype,
                                  gecko_dtype out_dtype, unsigned flags, unsigned parts, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  try {
    const float* aff[8] = {kappa_q, nu_q, kappa_k, nu_k, eta_q, rho_q, eta_k, rho_k};
    gecko::BwdProblem p;
    gecko_status st = bwd_problem(z, aff, v, dout, dz, dv_out, daff, B, H, n, d, dv, c, in_dtype, out_dtype, flags,
                                  parts, true, p);
    if (st != GECKO_OK) return st;
    if (!p.sca) return fail(GECKO_EINVAL, "saved statistics belong to the attention part: parts must hold it");
    if (!o_sca || !stats) return fail(GECKO_EINVAL, "o_sca and stats must be non-null");
    if (!aligned16(o_sca) || (reinterpret_cast<uintptr_t>(stats) & 7u))
      return fail(GECKO_EINVAL, "o_sca must be 16-byte and stats 8-byte aligned");
    p.saved = true;
    p.o_sca = o_sca;
    p.stats = stats;
    if (mem_saved && p.awm && p.f.nmem > 0) {
      const gecko::Problem& f = p.f;
      const gecko::Workspace mw = gecko::carve_workspace(nullptr, f.B * f.H, f.n, f.d, f.dv, f.nmem, f.nsnap, true, false);
      const size_t mb = gecko::kept_memory_bytes(mw, f.B * f.H, f.nmem, f.d, f.dv);
      if (mem_saved_bytes < mb)
        return fail(GECKO_EWORKSPACE, "mem_saved too small: %zu < %zu bytes", mem_saved_bytes, mb);
      if (reinterpret_cast<uintptr_t>(mem_saved) & (kAlign - 1))
        return fail(GECKO_EINVAL, "mem_saved must be 256-byte aligned");
      p.mem_saved = mem_saved;
    }
    return run_backward(p, workspace, workspace_bytes, stream);
  } catch (...) {
    return fail(GECKO_EHIP, "internal error");
  }
}

#ifndef GECKO_TIMER_EVENT_FLAGS
#define GECKO_TIMER_EVENT_FLAGS hipEventDisableSystemFence
#endif

gecko_status gecko_timer_create(int capacity, gecko_timer** timer) {
  if (!timer || capacity < 1 || capacity > (1 << 20)) return fail(GECKO_EINVAL, "bad timer arguments");
  gecko_timer* t = new (std::nothrow) gecko_timer;
  if (!t) return fail(GECKO_EINVAL, "out of host memory");
  t->capacity = capacity;
  t->ev.resize((size_t)capacity * 5);
  // The events only time the stages: without the system-scope fence an event
  // record writes back and invalidates no cache, so the kernel after it
  // starts with the L2 the one before it left (what an untimed call sees).
  // The elapsed times are read after the last event of a call has completed.
  for (size_t i = 0; i < t->ev.size(); ++i) {
    hipError_t e = hipEventCreateWithFlags(&t->ev[i], GECKO_TIMER_EVENT_FLAGS);
    if (e != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(t->ev[j]);
      delete t;
      return hip_fail(e, "hipEventCreate");
    }
  }
  *timer = t;
  return GECKO_OK;
}

gecko_status gecko_timer_reset(gecko_timer* timer) {
  if (!timer) return fail(GECKO_EINVAL, "null timer");
  timer->used = 0;
  return GECKO_OK;
}

gecko_status gecko_timer_read(gecko_timer* timer, float* ms4, int* calls) {
  if (!timer || !ms4 || !calls) return fail(GECKO_EINVAL, "null argument");
  for (int i = 0; i < 4; ++i) ms4[i] = 0.f;
  for (int k = 0; k < timer->used; ++k) {
    hipEvent_t* ev = &timer->ev[5 * k];
    hipError_t e = hipEventSynchronize(ev[4]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    for (int i = 0; i < 4; ++i) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, ev[i], ev[i + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      ms4[i] += ms;
    }
  }
  *calls = timer->used;
  return GECKO_OK;
}

gecko_status gecko_timer_destroy(gecko_timer* timer) {
  if (!timer) return GECKO_OK;
  for (hipEvent_t e : timer->ev) (void)hipEventDestroy(e);
  delete timer;
  return GECKO_OK;
}

const char* gecko_status_string(gecko_status status) {
  switch (status) {
    case GECKO_OK: return "GECKO_OK: success";
    case GECKO_EINVAL: return "GECKO_EINVAL: invalid argument";
    case GECKO_EUNSUPPORTED: return "GECKO_EUNSUPPORTED: shape or dtype not supported";
    case GECKO_EWORKSPACE: return "GECKO_EWORKSPACE: workspace missing or too small";
    case GECKO_EHIP: return "GECKO_EHIP: HIP runtime error";
  }
  return "unknown gecko_status";
}

const char* gecko_last_error(void) { return g_last_error.c_str(); }

int gecko_version(void) { return 104; }

}  // extern "C"
