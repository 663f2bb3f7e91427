"""ctypes binding of libgecko.so (declared in include/gecko.h).

Argument marshalling only: every step of the forward and the backward runs in
the HIP library.
Tensors are torch tensors on the GPU (torch provides device memory and the
stream); shapes are taken from them. Importing this module loads the library
and raises if it has not been built (``python -m chunked_attention_memory_amd.build``).
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libgecko.so")

GECKO_OK, GECKO_EINVAL, GECKO_EUNSUPPORTED, GECKO_EWORKSPACE, GECKO_EHIP = range(5)
GECKO_F32, GECKO_BF16 = 0, 1
GECKO_AWM_NO_DELTA = 1 << 0
GECKO_CHUNKWISE = 1 << 1
GECKO_PART_SCA, GECKO_PART_AWM = 1, 2

EXPORTED = (
    "gecko_workspace_size", "gecko_sca_awm_forward", "gecko_sca_forward", "gecko_awm_forward",
    "gecko_timer_create", "gecko_timer_reset", "gecko_timer_read", "gecko_timer_destroy",
    "gecko_sca_awm_forward_timed", "gecko_status_string", "gecko_last_error", "gecko_version",
    "gecko_stream_state_size", "gecko_stream_workspace_size", "gecko_sca_awm_forward_stream",
    "gecko_workspace_size_for", "gecko_cema_workspace_size", "gecko_cema_forward",
    "gecko_tdn_workspace_size", "gecko_tdn_forward",
    "gecko_forward_lse", "gecko_backward_workspace_size", "gecko_backward",
    "gecko_forward_train", "gecko_memory_saved_size", "gecko_backward_saved_workspace_size", "gecko_backward_saved",
    "gecko_sca_awm_forward_noalloc",
)

# bytes of the scratch array gecko_sca_awm_forward_noalloc holds per GPU (GECKO_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20


class GeckoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [status {status}]")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m chunked_attention_memory_amd.build`")
    # torch first: its HIP runtime is then the one libgecko.so binds to (same
    # soname), so the process has a single HIP runtime and torch's device
    # memory and stream handles are valid in the library. Loading libgecko.so
    # first would map a second HIP runtime beside torch's.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    P, F, I64, U, SZ = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint, ctypes.c_size_t
    I = ctypes.c_int
    lib.gecko_workspace_size.restype = SZ
    lib.gecko_workspace_size.argtypes = [I64] * 6 + [I]
    lib.gecko_workspace_size_for.restype = SZ
    lib.gecko_workspace_size_for.argtypes = [I64] * 6 + [I, U]
    fwd = [P] + [F] * 8 + [P, P] + [I64] * 6 + [I, I, U, P, SZ, P]
    lib.gecko_sca_awm_forward.restype = I
    lib.gecko_sca_awm_forward.argtypes = fwd
    lib.gecko_sca_awm_forward_timed.restype = I
    lib.gecko_sca_awm_forward_timed.argtypes = fwd + [P]
    lib.gecko_sca_awm_forward_noalloc.restype = I
    lib.gecko_sca_awm_forward_noalloc.argtypes = [P] + [F] * 8 + [P, P] + [I64] * 6 + [I, I, U, P]
    lib.gecko_sca_forward.restype = I
    lib.gecko_sca_forward.argtypes = [P] + [F] * 4 + [P, P] + [I64] * 6 + [I, I, P]
    lib.gecko_awm_forward.restype = I
    lib.gecko_awm_forward.argtypes = [P] + [F] * 4 + [P, P] + [I64] * 6 + [I, I, U, P, SZ, P]
    lib.gecko_timer_create.restype = I
    lib.gecko_timer_create.argtypes = [I, ctypes.POINTER(P)]
    lib.gecko_timer_reset.restype = I
    lib.gecko_timer_reset.argtypes = [P]
    lib.gecko_timer_read.restype = I
    lib.gecko_timer_read.argtypes = [P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(I)]
    lib.gecko_timer_destroy.restype = I
    lib.gecko_timer_destroy.argtypes = [P]
    lib.gecko_status_string.restype = ctypes.c_char_p
    lib.gecko_status_string.argtypes = [I]
    lib.gecko_last_error.restype = ctypes.c_char_p
    lib.gecko_last_error.argtypes = []
    lib.gecko_version.restype = I
    lib.gecko_version.argtypes = []
    lib.gecko_cema_workspace_size.restype = SZ
    lib.gecko_cema_workspace_size.argtypes = [I64] * 4
    lib.gecko_cema_forward.restype = I
    lib.gecko_cema_forward.argtypes = [P] + [F] * 5 + [P, P, P, P] + [I64] * 4 + [I, I, P, SZ, P]
    lib.gecko_tdn_workspace_size.restype = SZ
    lib.gecko_tdn_workspace_size.argtypes = [I64] * 4
    lib.gecko_tdn_forward.restype = I
    lib.gecko_tdn_forward.argtypes = ([P, F, F, F, F, I64, P, F, F] + [I64] * 4
                                      + [ctypes.c_float] * 3 + [I, I, P, SZ, P])
    lib.gecko_stream_state_size.restype = SZ
    lib.gecko_stream_state_size.argtypes = [I64] * 5 + [I]
    lib.gecko_stream_workspace_size.restype = SZ
    lib.gecko_stream_workspace_size.argtypes = [I64] * 6 + [I]
    lib.gecko_sca_awm_forward_stream.restype = I
    lib.gecko_sca_awm_forward_stream.argtypes = [P] + [F] * 8 + [P, P] + [I64] * 7 + [I, I, U, P, SZ, P, SZ, P]
    lib.gecko_forward_lse.restype = I
    lib.gecko_forward_lse.argtypes = [P] + [F] * 8 + [P, P, P] + [I64] * 6 + [I, I, U, U, P, SZ, P]
    lib.gecko_backward_workspace_size.restype = SZ
    lib.gecko_backward_workspace_size.argtypes = [I64] * 6 + [I, I, U, U]
    lib.gecko_backward.restype = I
    lib.gecko_backward.argtypes = [P] + [F] * 8 + [P, P, P, P, P] + [I64] * 6 + [I, I, U, U, P, SZ, P]
    lib.gecko_forward_train.restype = I
    lib.gecko_forward_train.argtypes = [P] + [F] * 8 + [P, P, P, P, P, SZ] + [I64] * 6 + [I, I, U, U, P, SZ, P]
    lib.gecko_memory_saved_size.restype = SZ
    lib.gecko_memory_saved_size.argtypes = [I64] * 6 + [I, U]
    lib.gecko_backward_saved_workspace_size.restype = SZ
    lib.gecko_backward_saved_workspace_size.argtypes = [I64] * 6 + [I, I, U, U]
    lib.gecko_backward_saved.restype = I
    lib.gecko_backward_saved.argtypes = [P] + [F] * 8 + [P] * 5 + [SZ] + [P] * 3 + [I64] * 6 + [I, I, U, U, P, SZ, P]
    return lib


lib = _load()


def _check(status: int) -> None:
    if status != GECKO_OK:
        msg = lib.gecko_last_error().decode() or lib.gecko_status_string(status).decode()
        raise GeckoError(status, msg)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return GECKO_BF16
    if t.dtype == torch.float32:
        return GECKO_F32
    raise GeckoError(GECKO_EUNSUPPORTED, f"unsupported tensor dtype {t.dtype}")


def _empty(shape, dtype, device, stream):
    """torch.empty allocated on the stream the kernels are launched on.

    The caching allocator hands a freed block to the next allocation on the
    stream that allocated it without waiting for other streams; a buffer that
    this module allocates and frees again (a workspace) must therefore belong
    to the launch stream, or a later allocation on the current stream could
    reuse it while the kernels still write it."""
    import torch

    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _shape(z, v):
    if z.dim() != 4 or v.dim() != 4:
        raise GeckoError(GECKO_EINVAL, "z and v must be [B, H, n, d] / [B, H, n, dv]")
    B, H, n, d = z.shape
    if tuple(v.shape[:3]) != (B, H, n):
        raise GeckoError(GECKO_EINVAL, "z and v disagree on (B, H, n)")
    for t in (z, v):
        if not t.is_contiguous() or not t.is_cuda:
            raise GeckoError(GECKO_EINVAL, "z and v must be contiguous device tensors")
    return B, H, n, d, v.shape[3]


def gecko_version() -> int:
    return lib.gecko_version()


def gecko_status_string(status: int) -> str:
    return lib.gecko_status_string(status).decode()


def gecko_workspace_size(B, H, n, d, dv, c, dtype_code, flags=0) -> int:
    r = lib.gecko_workspace_size_for(B, H, n, d, dv, c, dtype_code, flags)
    if r == ctypes.c_size_t(-1).value:
        raise GeckoError(GECKO_EINVAL, "invalid sizes for gecko_workspace_size")
    return r


def alloc_workspace(z, v, c, flags=0, stream=None):
    """Device workspace (uint8 tensor, 256-byte aligned by torch) for a forward on z, v,
    allocated on ``stream`` (default: the current stream)."""
    import torch

    B, H, n, d, dv = _shape(z, v)
    nbytes = gecko_workspace_size(B, H, n, d, dv, c, _dtype_code(z), flags)
    return _empty(max(nbytes, 256), torch.uint8, z.device, stream)


def _params(p, names, device, H, d):
    import torch

    out = []
    for k in names:
        t = p[k]
        if t.device != device or t.dtype != torch.float32 or t.numel() != H * d or not t.is_contiguous():
            raise GeckoError(GECKO_EINVAL, f"affine vector {k} must be a contiguous float32 [H, d] device tensor")
        out.append(_ptr(t))
    return out


Q_NAMES = ("kappa_q", "nu_q", "kappa_k", "nu_k")
M_NAMES = ("eta_q", "rho_q", "eta_k", "rho_k")


def gecko_sca_awm_forward(z, params, v, c, out=None, out_dtype=None, flags=0, workspace=None, stream=None, timer=None):
    """O = O_SCA + O_m. ``params`` maps the eight affine-vector names to float32 [H, d] tensors."""
    import torch

    B, H, n, d, dv = _shape(z, v)
    if out is None:
        out = _empty((B, H, n, dv), out_dtype or z.dtype, z.device, stream)
    if workspace is None:
        workspace = alloc_workspace(z, v, c, flags, stream)
    dt = _dtype_code(z)
    args = [_ptr(z), *_params(params, Q_NAMES + M_NAMES, z.device, H, d), _ptr(v), _ptr(out),
            B, H, n, d, dv, c, dt, _dtype_code(out), flags, _ptr(workspace), workspace.numel(), _stream(stream)]
    if timer is not None:
        _check(lib.gecko_sca_awm_forward_timed(*args, timer.handle))
    else:
        _check(lib.gecko_sca_awm_forward(*args))
    return out


def gecko_sca_awm_forward_noalloc(z, params, v, c, out, flags=0, stream=None):
    """O = O_SCA + O_m into the caller's ``out`` (bf16 or float32 [B, H, n, dv]),
    with the library's own scratch memory in place of a workspace: nothing is
    allocated, here or in the library. Calls on one GPU must not overlap in time."""
    B, H, n, d, dv = _shape(z, v)
    if tuple(out.shape) != (B, H, n, dv) or not out.is_contiguous() or out.device != z.device:
        raise GeckoError(GECKO_EINVAL, "out must be a contiguous [B, H, n, dv] tensor on z's device")
    _check(lib.gecko_sca_awm_forward_noalloc(
        _ptr(z), *_params(params, Q_NAMES + M_NAMES, z.device, H, d), _ptr(v), _ptr(out),
        B, H, n, d, dv, c, _dtype_code(z), _dtype_code(out), flags, _stream(stream)))
    return out


def gecko_sca_forward(z, params, v, c, out=None, out_dtype=None, stream=None):
    """O = O_SCA only."""
    import torch

    B, H, n, d, dv = _shape(z, v)
    if out is None:
        out = _empty((B, H, n, dv), out_dtype or z.dtype, z.device, stream)
    _check(lib.gecko_sca_forward(_ptr(z), *_params(params, Q_NAMES, z.device, H, d), _ptr(v), _ptr(out),
                                 B, H, n, d, dv, c, _dtype_code(z), _dtype_code(out), _stream(stream)))
    return out


def gecko_awm_forward(z, params, v, c, out=None, out_dtype=None, flags=0, workspace=None, stream=None):
    """O = O_m only (exact zeros on chunks 1 and 2)."""
    import torch

    B, H, n, d, dv = _shape(z, v)
    if out is None:
        out = _empty((B, H, n, dv), out_dtype or z.dtype, z.device, stream)
    if workspace is None:
        workspace = alloc_workspace(z, v, c, flags, stream)
    _check(lib.gecko_awm_forward(_ptr(z), *_params(params, M_NAMES, z.device, H, d), _ptr(v), _ptr(out),
                                 B, H, n, d, dv, c, _dtype_code(z), _dtype_code(out), flags,
                                 _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def gecko_stream_state_size(B, H, d, dv, c, dtype_code) -> int:
    r = lib.gecko_stream_state_size(B, H, d, dv, c, dtype_code)
    if r == ctypes.c_size_t(-1).value:
        raise GeckoError(GECKO_EINVAL, "invalid sizes for gecko_stream_state_size")
    return r


def gecko_stream_workspace_size(B, H, n, d, dv, c, dtype_code) -> int:
    r = lib.gecko_stream_workspace_size(B, H, n, d, dv, c, dtype_code)
    if r == ctypes.c_size_t(-1).value:
        raise GeckoError(GECKO_EINVAL, "invalid sizes for gecko_stream_workspace_size")
    return r


def gecko_sca_awm_forward_stream(z, params, v, c, pos, state, out=None, out_dtype=None, flags=0, workspace=None,
                                 stream=None):
    """One call of a streamed sequence: rows pos .. pos + n of O = O_SCA + O_m.
    ``state`` is a uint8 device tensor of gecko_stream_state_size() bytes."""
    import torch

    B, H, n, d, dv = _shape(z, v)
    if out is None:
        out = _empty((B, H, n, dv), out_dtype or z.dtype, z.device, stream)
    dt = _dtype_code(z)
    if workspace is None:
        nbytes = gecko_stream_workspace_size(B, H, n, d, dv, c, dt)
        workspace = _empty(max(nbytes, 256), torch.uint8, z.device, stream)
    _check(lib.gecko_sca_awm_forward_stream(
        _ptr(z), *_params(params, Q_NAMES + M_NAMES, z.device, H, d), _ptr(v), _ptr(out),
        B, H, n, d, dv, c, pos, dt, _dtype_code(out), flags, _ptr(state), state.numel(),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


CEMA_NAMES = ("alpha", "delta", "theta", "beta")


def gecko_cema_workspace_size(B, n, D, h) -> int:
    r = lib.gecko_cema_workspace_size(B, n, D, h)
    if r == ctypes.c_size_t(-1).value:
        raise GeckoError(GECKO_EINVAL, "invalid sizes for gecko_cema_workspace_size")
    return r


def gecko_cema_forward(x, params, reset=None, h0=None, out=None, out_dtype=None, want_state=False,
                       workspace=None, stream=None):
    """y = CEMA(x) for x [B, n, D]. ``params``: alpha, delta, theta, beta float32 [D, h] and
    eta float32 [D, h, 2] (re, im). ``reset``: uint8 [B, n] or None; ``h0``: float32
    [B, D, h, 2] or None. Returns y, or (y, h_final) with ``want_state``."""
    import torch

    if x.dim() != 3 or not x.is_cuda or not x.is_contiguous():
        raise GeckoError(GECKO_EINVAL, "x must be a contiguous [B, n, D] device tensor")
    B, n, D = x.shape
    h = params["alpha"].shape[-1]
    for k in CEMA_NAMES + ("eta",):
        t = params[k]
        shape = (D, h, 2) if k == "eta" else (D, h)
        if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous() or t.device != x.device:
            raise GeckoError(GECKO_EINVAL, f"CEMA parameter {k} must be a contiguous float32 {shape} device tensor")
    if out is None:
        out = _empty((B, n, D), out_dtype or x.dtype, x.device, stream)
    hfin = _empty((B, D, h, 2), torch.float32, x.device, stream) if want_state else None
    for t, name in ((reset, "reset"), (h0, "h0")):
        if t is not None and (not t.is_contiguous() or t.device != x.device):
            raise GeckoError(GECKO_EINVAL, f"{name} must be a contiguous device tensor")
    if reset is not None and (reset.dtype != torch.uint8 or tuple(reset.shape) != (B, n)):
        raise GeckoError(GECKO_EINVAL, "reset must be uint8 [B, n]")
    if h0 is not None and (h0.dtype != torch.float32 or tuple(h0.shape) != (B, D, h, 2)):
        raise GeckoError(GECKO_EINVAL, "h0 must be float32 [B, D, h, 2]")
    if workspace is None:
        nbytes = gecko_cema_workspace_size(B, n, D, h)
        workspace = _empty(max(nbytes, 256), torch.uint8, x.device, stream)
    _check(lib.gecko_cema_forward(
        _ptr(x), *[_ptr(params[k]) for k in CEMA_NAMES], _ptr(params["eta"]), _ptr(reset), _ptr(h0), _ptr(out),
        _ptr(hfin), B, n, D, h, _dtype_code(x), _dtype_code(out), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return (out, hfin) if want_state else out


def gecko_tdn_workspace_size(B, n, D, G) -> int:
    r = lib.gecko_tdn_workspace_size(B, n, D, G)
    if r == ctypes.c_size_t(-1).value:
        raise GeckoError(GECKO_EINVAL, "invalid sizes for gecko_tdn_workspace_size")
    return r


def gecko_tdn_forward(x, gamma, shift, G, beta1, beta2, eps=1e-5, state=None, out=None, out_dtype=None,
                      want_state=False, workspace=None, stream=None):
    """Timestep decay normalisation of x [B, n, D] in G groups. ``state`` is
    (m, v, t0) from an earlier call of the same sequence (m, v float32 [B, G]).
    Returns y, or (y, (m, v, t)) with ``want_state``."""
    import torch

    if x.dim() != 3 or not x.is_cuda or not x.is_contiguous():
        raise GeckoError(GECKO_EINVAL, "x must be a contiguous [B, n, D] device tensor")
    B, n, D = x.shape
    for t, name in ((gamma, "gamma"), (shift, "shift")):
        if t.dtype != torch.float32 or t.numel() != D or not t.is_contiguous() or t.device != x.device:
            raise GeckoError(GECKO_EINVAL, f"{name} must be a contiguous float32 [D] device tensor")
    m0 = v0 = None
    t0 = 0
    if state is not None:
        m0, v0, t0 = state
    if out is None:
        out = _empty((B, n, D), out_dtype or x.dtype, x.device, stream)
    m_out = _empty((B, G), torch.float32, x.device, stream) if want_state else None
    v_out = _empty((B, G), torch.float32, x.device, stream) if want_state else None
    if workspace is None:
        workspace = _empty(max(gecko_tdn_workspace_size(B, n, D, G), 256), torch.uint8, x.device, stream)
    _check(lib.gecko_tdn_forward(_ptr(x), _ptr(gamma), _ptr(shift), _ptr(m0), _ptr(v0), int(t0), _ptr(out),
                                 _ptr(m_out), _ptr(v_out), B, n, D, G, float(beta1), float(beta2), float(eps),
                                 _dtype_code(x), _dtype_code(out), _ptr(workspace), workspace.numel(),
                                 _stream(stream)))
    return (out, (m_out, v_out, t0 + n)) if want_state else out


class Stream:
    """A sequence handed to the streaming forward in consecutive calls. Keeps
    the device state and the token count; refuses a call after one that ended
    inside a chunk."""

    def __init__(self, B, H, d, dv, c, params, device="cuda", flags=0):
        import torch

        self.B, self.H, self.d, self.dv, self.c = B, H, d, dv, c
        self.params, self.flags = params, flags
        nbytes = gecko_stream_state_size(B, H, d, dv, c, GECKO_BF16)
        self.state = _empty(nbytes, torch.uint8, device, None)
        self.pos = 0

    def forward(self, z, v, out=None, out_dtype=None, workspace=None, stream=None):
        if self.pos % self.c:
            raise GeckoError(GECKO_EINVAL, "the previous call of this sequence ended inside a chunk")
        if tuple(z.shape[:2]) != (self.B, self.H) or z.shape[3] != self.d or v.shape[3] != self.dv:
            raise GeckoError(GECKO_EINVAL, "z and v do not match the stream's (B, H, d, dv)")
        out = gecko_sca_awm_forward_stream(z, self.params, v, self.c, self.pos, self.state, out=out,
                                           out_dtype=out_dtype, flags=self.flags, workspace=workspace,
                                           stream=stream)
        self.pos += z.shape[2]
        return out


class Timer:
    """HIP events between the kernels of gecko_sca_awm_forward (see gecko_timer_* in gecko.h)."""

    STAGES = ("awm_chunk", "awm_zscan", "awm_scan", "sca_readout")

    def __init__(self, capacity: int):
        h = ctypes.c_void_p()
        _check(lib.gecko_timer_create(capacity, ctypes.byref(h)))
        self.handle = h

    def reset(self):
        _check(lib.gecko_timer_reset(self.handle))

    def read(self):
        ms = (ctypes.c_float * 4)()
        calls = ctypes.c_int()
        _check(lib.gecko_timer_read(self.handle, ms, ctypes.byref(calls)))
        return {k: ms[i] for i, k in enumerate(self.STAGES)}, calls.value

    def close(self):
        if self.handle:
            lib.gecko_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def to_device_inputs(host: dict, device="cuda"):
    """Move inputs from ``inputs.make_inputs`` (float32, dtype-exact) to the device in the run dtype."""
    import torch

    tdt = torch.bfloat16 if host["dtype"] == "bf16" else torch.float32
    z = torch.from_numpy(host["z"]).to(device=device).to(tdt).contiguous()
    v = torch.from_numpy(host["v"]).to(device=device).to(tdt).contiguous()
    params = {k: torch.from_numpy(a).to(device=device, dtype=torch.float32).contiguous()
              for k, a in host["params"].items()}
    return z, v, params


def _part_params(params, parts, device, H, d):
    q = _params(params, Q_NAMES, device, H, d) if parts & GECKO_PART_SCA else [None] * 4
    m = _params(params, M_NAMES, device, H, d) if parts & GECKO_PART_AWM else [None] * 4
    return q + m


def gecko_forward_lse(z, params, v, c, parts=GECKO_PART_SCA | GECKO_PART_AWM, out=None, lse=None, out_dtype=None,
                      flags=0, workspace=None, stream=None):
    """O of the selected parts and the attention log-sum-exp per query ([B, H, n] float32)."""
    import torch

    B, H, n, d, dv = _shape(z, v)
    if out is None:
        out = _empty((B, H, n, dv), out_dtype or z.dtype, z.device, stream)
    if lse is None:
        lse = _empty((B, H, n), torch.float32, z.device, stream)
    if workspace is None and parts & GECKO_PART_AWM:
        workspace = alloc_workspace(z, v, c, flags, stream)
    _check(lib.gecko_forward_lse(_ptr(z), *_part_params(params, parts, z.device, H, d), _ptr(v), _ptr(out), _ptr(lse),
                                 B, H, n, d, dv, c, _dtype_code(z), _dtype_code(out), flags, parts,
                                 _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, lse


def gecko_forward_train(z, params, v, c, parts=GECKO_PART_SCA | GECKO_PART_AWM, out=None, o_sca=None, stats=None,
                        out_dtype=None, flags=0, workspace=None, keep_memory=False, mem_saved=None, stream=None):
    """O of the selected parts, the attention output alone (``o_sca`` [B, H, n, dv] float32) and the per-query
    offset and bf16-weight sum (``stats`` [B, H, n, 2] float32) that gecko_backward_saved reuses. With
    ``keep_memory`` (or a ``mem_saved`` uint8 tensor of gecko_memory_saved_size bytes) the memory pass is
    written to that buffer, returned fourth, for gecko_backward_saved to read instead of recomputing it."""
    import torch

    B, H, n, d, dv = _shape(z, v)
    if out is None:
        out = _empty((B, H, n, dv), out_dtype or z.dtype, z.device, stream)
    if o_sca is None:
        o_sca = _empty((B, H, n, dv), torch.float32, z.device, stream)
    if stats is None:
        stats = _empty((B, H, n, 2), torch.float32, z.device, stream)
    keep = keep_memory or mem_saved is not None
    if mem_saved is not None and (mem_saved.dtype != torch.uint8 or not mem_saved.is_contiguous()):
        raise GeckoError(GECKO_EINVAL, "mem_saved must be a contiguous uint8 tensor")
    if keep and mem_saved is None:
        nbytes = gecko_memory_saved_size(B, H, n, d, dv, c, _dtype_code(z), flags)
        mem_saved = _empty(max(nbytes, 256), torch.uint8, z.device, stream)
    if workspace is None and parts & GECKO_PART_AWM and not keep:
        workspace = alloc_workspace(z, v, c, flags, stream)
    _check(lib.gecko_forward_train(_ptr(z), *_part_params(params, parts, z.device, H, d), _ptr(v), _ptr(out),
                                   _ptr(o_sca), _ptr(stats), _ptr(mem_saved),
                                   0 if mem_saved is None else mem_saved.numel(), B, H, n, d, dv, c, _dtype_code(z),
                                   _dtype_code(out), flags, parts, _ptr(workspace),
                                   0 if workspace is None else workspace.numel(), _stream(stream)))
    return (out, o_sca, stats, mem_saved) if keep else (out, o_sca, stats)


def gecko_memory_saved_size(B, H, n, d, dv, c, in_code=None, flags=0) -> int:
    r = lib.gecko_memory_saved_size(B, H, n, d, dv, c, GECKO_BF16 if in_code is None else in_code, flags)
    if r == ctypes.c_size_t(-1).value:
        raise GeckoError(GECKO_EINVAL, "invalid or unsupported arguments for gecko_memory_saved_size")
    return r


def gecko_backward_workspace_size(B, H, n, d, dv, c, in_code, out_code, flags=0,
                                  parts=GECKO_PART_SCA | GECKO_PART_AWM) -> int:
    r = lib.gecko_backward_workspace_size(B, H, n, d, dv, c, in_code, out_code, flags, parts)
    if r == ctypes.c_size_t(-1).value:
        raise GeckoError(GECKO_EINVAL, "invalid or unsupported arguments for gecko_backward_workspace_size")
    return r


def gecko_backward(z, params, v, dout, c, parts=GECKO_PART_SCA | GECKO_PART_AWM, flags=0, dz=None, dv=None,
                   daff=None, workspace=None, stream=None):
    """Gradients of sum(dout * O): dict with ``dz`` [B, H, n, d], ``dv`` [B, H, n, dv] (float32) and one
    float32 [H, d] tensor per affine name (views of ``daff`` [8, H, d])."""
    import torch

    B, H, n, d, dvs = _shape(z, v)
    if tuple(dout.shape) != (B, H, n, dvs) or not dout.is_contiguous():
        raise GeckoError(GECKO_EINVAL, "dout must be a contiguous [B, H, n, dv] tensor")
    if dz is None:
        dz = _empty((B, H, n, d), torch.float32, z.device, stream)
    if dv is None:
        dv = _empty((B, H, n, dvs), torch.float32, z.device, stream)
    if daff is None:
        daff = _empty((8, H, d), torch.float32, z.device, stream)
    if workspace is None:
        nbytes = gecko_backward_workspace_size(B, H, n, d, dvs, c, _dtype_code(z), _dtype_code(dout), flags, parts)
        workspace = _empty(max(nbytes, 256), torch.uint8, z.device, stream)
    _check(lib.gecko_backward(_ptr(z), *_part_params(params, parts, z.device, H, d), _ptr(v), _ptr(dout),
                              _ptr(dz), _ptr(dv), _ptr(daff), B, H, n, d, dvs, c, _dtype_code(z),
                              _dtype_code(dout), flags, parts, _ptr(workspace), workspace.numel(), _stream(stream)))
    res = {"dz": dz, "dv": dv}
    for i, k in enumerate(Q_NAMES + M_NAMES):
        res["d" + k] = daff[i]
    return res


def gecko_backward_saved_workspace_size(B, H, n, d, dv, c, in_code, out_code, flags=0,
                                        parts=GECKO_PART_SCA | GECKO_PART_AWM) -> int:
    r = lib.gecko_backward_saved_workspace_size(B, H, n, d, dv, c, in_code, out_code, flags, parts)
    if r == ctypes.c_size_t(-1).value:
        raise GeckoError(GECKO_EINVAL, "invalid or unsupported arguments for gecko_backward_saved_workspace_size")
    return r


def gecko_backward_saved(z, params, v, dout, o_sca, stats, c, parts=GECKO_PART_SCA | GECKO_PART_AWM, flags=0,
                         dz=None, dv=None, daff=None, workspace=None, mem_saved=None, stream=None):
    """gecko_backward with the attention statistics of gecko_forward_train (same inputs, c, parts and flags),
    and its memory pass when ``mem_saved`` (that forward's kept buffer) is given."""
    import torch

    B, H, n, d, dvs = _shape(z, v)
    if tuple(dout.shape) != (B, H, n, dvs) or not dout.is_contiguous():
        raise GeckoError(GECKO_EINVAL, "dout must be a contiguous [B, H, n, dv] tensor")
    if (tuple(o_sca.shape) != (B, H, n, dvs) or o_sca.dtype != torch.float32 or not o_sca.is_contiguous()
            or tuple(stats.shape) != (B, H, n, 2) or stats.dtype != torch.float32 or not stats.is_contiguous()):
        raise GeckoError(GECKO_EINVAL, "o_sca must be float32 [B, H, n, dv] and stats float32 [B, H, n, 2]")
    if mem_saved is not None and (mem_saved.dtype != torch.uint8 or not mem_saved.is_contiguous()):
        raise GeckoError(GECKO_EINVAL, "mem_saved must be a contiguous uint8 tensor")
    if dz is None:
        dz = _empty((B, H, n, d), torch.float32, z.device, stream)
    if dv is None:
        dv = _empty((B, H, n, dvs), torch.float32, z.device, stream)
    if daff is None:
        daff = _empty((8, H, d), torch.float32, z.device, stream)
    if workspace is None:
        nbytes = gecko_backward_saved_workspace_size(B, H, n, d, dvs, c, _dtype_code(z), _dtype_code(dout), flags,
                                                     parts)
        workspace = _empty(max(nbytes, 256), torch.uint8, z.device, stream)
    _check(lib.gecko_backward_saved(_ptr(z), *_part_params(params, parts, z.device, H, d), _ptr(v), _ptr(dout),
                                    _ptr(o_sca), _ptr(stats), _ptr(mem_saved),
                                    0 if mem_saved is None else mem_saved.numel(), _ptr(dz), _ptr(dv), _ptr(daff),
                                    B, H, n, d, dvs, c,
                                    _dtype_code(z), _dtype_code(dout), flags, parts, _ptr(workspace),
                                    workspace.numel(), _stream(stream)))
    res = {"dz": dz, "dv": dv}
    for i, k in enumerate(Q_NAMES + M_NAMES):
        res["d" + k] = daff[i]
    return res
