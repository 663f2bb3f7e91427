"""CPU tier: the C-ABI library loads, exports what include/gecko.h declares, and
rejects bad arguments on the host before launching anything. No call here
reaches a device: every call fails validation first."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gecko.h")


@pytest.fixture(scope="module")
def g():
    from chunked_attention_memory_amd import build

    lib = os.path.join(ROOT, "chunked_attention_memory_amd", "_lib", "libgecko.so")
    if not os.path.exists(lib):
        build.build()
    from chunked_attention_memory_amd import gecko

    return gecko


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gecko_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(g):
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(g.lib, name), name
    assert set(names) == set(g.EXPORTED)


def test_version_and_status_strings(g):
    assert g.gecko_version() == 104
    for s in range(5):
        assert g.gecko_status_string(s).startswith("GECKO_")
    assert "unknown" in g.gecko_status_string(99)


def test_workspace_size(g):
    # at most two chunks: nothing to store
    assert g.gecko_workspace_size(1, 1, 100, 128, 256, 50, g.GECKO_BF16) == 0
    a = g.gecko_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16)
    rows = 8 * 62
    expect_min = rows * (128 * 256 * 4 + 128 * 128 * 2 + 4 * 128 * 4 + 256 * 128 * 2)
    assert expect_min <= a <= expect_min + 7 * 256
    # doubling the heads doubles the workspace (up to alignment)
    b = g.gecko_workspace_size(2, 8, 131072, 128, 256, 2048, g.GECKO_BF16)
    assert abs(b - 2 * a) <= 7 * 256
    f = g.gecko_workspace_size(1, 1, 256, 32, 32, 64, g.GECKO_F32)
    assert f >= 2 * (32 * 32 * 4 * 2 + 4 * 32 * 4 + 32 * 32 * 4) + 256 * 2 * 4
    with pytest.raises(g.GeckoError):
        g.gecko_workspace_size(1, 1, 0, 128, 256, 64, g.GECKO_BF16)
    with pytest.raises(g.GeckoError):
        g.gecko_workspace_size(1, 1, 10, 48, 256, 64, g.GECKO_BF16)


FAKE = 1 << 20  # an aligned non-null address; never dereferenced (validation fails first)


def call_full(g, **kw):
    a = dict(z=FAKE, aff=[FAKE + 64 * i for i in range(8)], v=2 * FAKE, out=3 * FAKE, B=1, H=1, n=1000,
             d=128, dv=256, c=100, din=g.GECKO_BF16, dout=g.GECKO_BF16, flags=0, ws=0, wsb=0)
    a.update(kw)
    st = g.lib.gecko_sca_awm_forward(a["z"], *a["aff"], a["v"], a["out"], a["B"], a["H"], a["n"], a["d"], a["dv"],
                                     a["c"], a["din"], a["dout"], a["flags"], a["ws"], a["wsb"], None)
    return st, g.lib.gecko_last_error().decode()


def test_validation_errors(g):
    st, msg = call_full(g, z=0)
    assert st == g.GECKO_EINVAL and "non-null" in msg
    st, _ = call_full(g, n=0)
    assert st == g.GECKO_EINVAL
    st, _ = call_full(g, c=0)
    assert st == g.GECKO_EINVAL
    st, _ = call_full(g, z=FAKE + 2)
    assert st == g.GECKO_EINVAL
    st, _ = call_full(g, aff=[FAKE] * 7 + [0])
    assert st == g.GECKO_EINVAL
    st, _ = call_full(g, flags=1 << 5)
    assert st == g.GECKO_EINVAL
    st, _ = call_full(g, d=96)
    assert st == g.GECKO_EUNSUPPORTED
    st, msg = call_full(g, d=32, dv=32)  # a built bf16 shape: validation reaches the missing workspace
    assert st == g.GECKO_EWORKSPACE and "null" in msg
    st, _ = call_full(g, din=g.GECKO_F32, dout=g.GECKO_BF16)
    assert st == g.GECKO_EUNSUPPORTED
    st, _ = call_full(g, din=7)
    assert st == g.GECKO_EINVAL
    st, msg = call_full(g)  # N = 10 chunks and no workspace
    assert st == g.GECKO_EWORKSPACE and "null" in msg
    st, msg = call_full(g, ws=8 * FAKE, wsb=1024)
    assert st == g.GECKO_EWORKSPACE and "too small" in msg
    st, msg = call_full(g, out=FAKE + 4096)  # overlaps z
    assert st == g.GECKO_EINVAL and "alias" in msg
    # more than 65535 (batch, head) pairs: the float32 path takes them (its
    # grids are one-dimensional); here validation stops at the missing workspace
    big = 1 << 40  # widely spaced fake addresses, so that nothing aliases
    st, msg = call_full(g, din=g.GECKO_F32, dout=g.GECKO_F32, B=70000, H=1, n=10, c=1, d=32, dv=32, z=big,
                        v=2 * big, out=3 * big, aff=[4 * big + (1 << 30) * i for i in range(8)])
    assert st == g.GECKO_EWORKSPACE and "null" in msg, msg


def test_workspace_must_not_alias_inputs(g):
    """The chunk pass and the scan write the workspace before the attention
    kernel reads z, v and the affine vectors: a workspace over any of them is
    refused before any launch."""
    wsb = g.gecko_workspace_size(1, 1, 1000, 128, 256, 100, g.GECKO_BF16)
    assert wsb > FAKE  # so that a workspace at 16 FAKE covers affine vectors placed there
    st, msg = call_full(g, ws=FAKE, wsb=wsb)
    assert st == g.GECKO_EINVAL and "aliases z or v" in msg
    st, msg = call_full(g, ws=(2 * FAKE + 4096 - wsb) & ~255, wsb=wsb)  # ends inside v, before out
    assert st == g.GECKO_EINVAL and "aliases z or v" in msg
    st, msg = call_full(g, ws=16 * FAKE, wsb=wsb, aff=[16 * FAKE + 64 * i for i in range(8)])
    assert st == g.GECKO_EINVAL and "affine vector 0" in msg
    st, msg = call_full(g, ws=16 * FAKE, wsb=wsb, aff=[FAKE + 64 * i for i in range(7)] + [16 * FAKE + 4096])
    assert st == g.GECKO_EINVAL and "affine vector 7" in msg


def test_noalloc_forward_size_limit(g):
    """The allocation-free forward states its scratch size in the header and
    refuses sizes whose workspace exceeds it before touching the device."""
    text = open(HEADER).read()
    m = re.search(r"#define GECKO_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == g.NOALLOC_SCRATCH_BYTES
    big = 1 << 40  # widely spaced fake addresses: nothing aliases, nothing is dereferenced

    def call(n, H=8, **kw):
        a = dict(z=big, v=2 * big, out=3 * big)
        a.update(kw)
        st = g.lib.gecko_sca_awm_forward_noalloc(a["z"], *[4 * big + 256 * i for i in range(8)], a["v"], a["out"],
                                                 1, H, n, 128, 256, 2048, g.GECKO_BF16, g.GECKO_BF16, 0, None)
        return st, g.lib.gecko_last_error().decode()

    need = g.gecko_workspace_size(1, 8, 262144, 128, 256, 2048, g.GECKO_BF16)
    assert need > g.NOALLOC_SCRATCH_BYTES
    st, msg = call(262144)
    assert st == g.GECKO_EWORKSPACE and "scratch" in msg and str(need) in msg
    st, msg = call(131072, z=0)
    assert st == g.GECKO_EINVAL and "non-null" in msg
    st, msg = call(131072, out=big + 4096)
    assert st == g.GECKO_EINVAL and "alias" in msg


def test_sca_and_awm_entry_validation(g):
    st = g.lib.gecko_sca_forward(FAKE, FAKE, FAKE, FAKE, 0, 2 * FAKE, 3 * FAKE, 1, 1, 10, 128, 256, 4,
                                 g.GECKO_BF16, g.GECKO_BF16, None)
    assert st == g.GECKO_EINVAL
    st = g.lib.gecko_awm_forward(FAKE, FAKE, FAKE, FAKE, FAKE, 2 * FAKE, 3 * FAKE, 1, 1, 100, 128, 256, 4,
                                 g.GECKO_BF16, g.GECKO_BF16, 0, 0, 0, None)
    assert st == g.GECKO_EWORKSPACE


def test_timer_argument_errors(g):
    h = ctypes.c_void_p()
    assert g.lib.gecko_timer_create(0, ctypes.byref(h)) == g.GECKO_EINVAL
    assert g.lib.gecko_timer_reset(None) == g.GECKO_EINVAL
    assert g.lib.gecko_timer_destroy(None) == g.GECKO_OK


def call_stream(g, **kw):
    a = dict(z=FAKE, aff=[FAKE + 64 * i for i in range(8)], v=2 * FAKE, out=3 * FAKE, B=1, H=1, n=1000,
             d=128, dv=256, c=128, pos=0, din=g.GECKO_BF16, dout=g.GECKO_BF16, flags=0, st=16 * FAKE,
             stb=1 << 30, ws=32 * FAKE, wsb=1 << 30)
    a.update(kw)
    st = g.lib.gecko_sca_awm_forward_stream(a["z"], *a["aff"], a["v"], a["out"], a["B"], a["H"], a["n"], a["d"],
                                            a["dv"], a["c"], a["pos"], a["din"], a["dout"], a["flags"], a["st"],
                                            a["stb"], a["ws"], a["wsb"], None)
    return st, g.lib.gecko_last_error().decode()


def test_stream_validation_errors(g):
    st, msg = call_stream(g, pos=64)
    assert st == g.GECKO_EINVAL and "multiple of c" in msg
    st, _ = call_stream(g, pos=-128)
    assert st == g.GECKO_EINVAL
    st, msg = call_stream(g, c=100)
    assert st == g.GECKO_EUNSUPPORTED and "multiple of 64" in msg
    st, msg = call_stream(g, din=g.GECKO_F32, dout=g.GECKO_F32, d=32, dv=32)
    assert st == g.GECKO_EUNSUPPORTED and "bf16" in msg
    st, msg = call_stream(g, st=0)
    assert st == g.GECKO_EINVAL and "state" in msg
    st, msg = call_stream(g, stb=1024)
    assert st == g.GECKO_EINVAL and "too small" in msg
    st, msg = call_stream(g, st=16 * FAKE + 16)
    assert st == g.GECKO_EINVAL and "aligned" in msg
    st, msg = call_stream(g, st=FAKE)  # overlaps z
    assert st == g.GECKO_EINVAL and "alias" in msg
    st, msg = call_stream(g, wsb=1024)
    assert st == g.GECKO_EWORKSPACE


def test_stream_sizes(g):
    s = g.gecko_stream_state_size(1, 8, 128, 256, 2048, g.GECKO_BF16)
    expect = 8 * (128 * 256 * 4 + 128 * 2 * 4 + 2048 * 128 * 2 + 2048 * 256 * 2)
    assert expect <= s <= expect + 4 * 256
    with pytest.raises(g.GeckoError):
        g.gecko_stream_state_size(1, 8, 128, 256, 2048, g.GECKO_F32)
    # a call with a carried chunk stores one more memory step and one more snapshot
    one = g.gecko_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16)
    st = g.gecko_stream_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16)
    per_step = 8 * (128 * 256 * 4 + 128 * 128 * 2 + 4 * 128 * 4 + 256 * 128 * 2)
    extra = 8 * 128 * 256 * 2 + 8 * 128 * 2 * 4  # one more snapshot slot, the final denominator
    assert one + 2 * per_step + extra <= st <= one + 2 * per_step + extra + 10 * 256


def test_chunkwise_flag_host_checks(g):
    # accepted by validation (fails later on the missing workspace), refused by the streaming entry
    st, msg = call_full(g, flags=g.GECKO_CHUNKWISE)
    assert st == g.GECKO_EWORKSPACE
    st, msg = call_stream(g, flags=g.GECKO_CHUNKWISE)
    assert st == g.GECKO_EUNSUPPORTED and "sliding" in msg
    # one more memory chunk per (batch, head) than the sliding form
    a = g.gecko_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16)
    b = g.gecko_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16, g.GECKO_CHUNKWISE)
    per_step = 8 * (128 * 256 * 4 + 128 * 128 * 2 + 4 * 128 * 4 + 256 * 128 * 2)
    assert per_step <= b - a <= per_step + 8 * 256
    # two chunks: the chunk-wise form already stores the first
    assert g.gecko_workspace_size(1, 1, 100, 128, 256, 50, g.GECKO_BF16) == 0
    assert g.gecko_workspace_size(1, 1, 100, 128, 256, 50, g.GECKO_BF16, g.GECKO_CHUNKWISE) > 0
    assert g.lib.gecko_workspace_size_for(1, 1, 100, 128, 256, 50, g.GECKO_BF16, 1 << 7) == ctypes.c_size_t(-1).value


def test_one_hip_runtime_per_process(g):
    """Importing the binding before torch must still leave one HIP runtime
    mapped (torch's), so torch's memory and streams are valid in the library."""
    import subprocess
    import sys

    code = ("import chunked_attention_memory_amd.gecko\nimport torch\n"
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    mapped = eval(out.stdout.strip().splitlines()[-1])
    assert len(mapped) == 1, mapped


def test_cema_host_checks(g):
    assert g.gecko_cema_workspace_size(1, 100, 64, 16) == 0          # one chunk: no workspace
    assert g.gecko_cema_workspace_size(1, 131072, 4096, 16) > 0
    assert g.lib.gecko_cema_workspace_size(1, 100, 64, 3) == ctypes.c_size_t(-1).value
    aff = [FAKE + 256 * i for i in range(5)]
    args = lambda **k: [k.get("x", FAKE * 8), *aff, 0, 0, k.get("y", FAKE * 16), 0, 1, k.get("n", 100), 64,
                        k.get("h", 16), g.GECKO_BF16, g.GECKO_BF16, 0, 0, None]
    assert g.lib.gecko_cema_forward(*args(h=3)) == g.GECKO_EUNSUPPORTED
    assert g.lib.gecko_cema_forward(*args(x=0)) == g.GECKO_EINVAL
    assert g.lib.gecko_cema_forward(*args(y=FAKE * 8 + 64)) == g.GECKO_EINVAL     # y aliases x
    assert g.lib.gecko_cema_forward(*args(n=131072, y=FAKE * 64)) == g.GECKO_EWORKSPACE  # chunked, no workspace


def test_tdn_host_checks(g):
    assert g.gecko_tdn_workspace_size(1, 100, 64, 8) > 0
    assert g.lib.gecko_tdn_workspace_size(1, 100, 64, 3) == ctypes.c_size_t(-1).value   # uneven groups
    assert g.lib.gecko_tdn_workspace_size(1, 100, 16384, 64) == ctypes.c_size_t(-1).value
    F = ctypes.c_float
    base = dict(x=FAKE * 8, gamma=FAKE, shift=FAKE + 4096, y=FAKE * 16, D=64, G=8, b1=0.9, b2=0.99, eps=1e-5,
                ws=FAKE * 32, wsb=1 << 30)

    def call(**k):
        a = dict(base)
        a.update(k)
        return g.lib.gecko_tdn_forward(a["x"], a["gamma"], a["shift"], 0, 0, 0, a["y"], 0, 0, 1, 100, a["D"],
                                       a["G"], F(a["b1"]), F(a["b2"]), F(a["eps"]), g.GECKO_BF16, g.GECKO_BF16,
                                       a["ws"], a["wsb"], None)
    assert call(G=3) == g.GECKO_EUNSUPPORTED
    assert call(b1=1.0) == g.GECKO_EINVAL
    assert call(eps=0.0) == g.GECKO_EINVAL
    assert call(x=FAKE * 8 + 2) == g.GECKO_EINVAL
    assert call(ws=0) == g.GECKO_EWORKSPACE


def call_bwd(g, **kw):
    a = dict(z=FAKE, aff=[FAKE + 64 * i for i in range(8)], v=2 * FAKE, dout=5 * FAKE, dz=6 * FAKE, dv=7 * FAKE,
             daff=8 * FAKE, B=1, H=1, n=1000, d=128, dvs=256, c=128, din=g.GECKO_BF16, dtype=g.GECKO_BF16, flags=0,
             parts=3, ws=0, wsb=0)
    a.update(kw)
    st = g.lib.gecko_backward(a["z"], *a["aff"], a["v"], a["dout"], a["dz"], a["dv"], a["daff"],
                              a["B"], a["H"], a["n"], a["d"], a["dvs"], a["c"], a["din"], a["dtype"], a["flags"],
                              a["parts"], a["ws"], a["wsb"], None)
    return st, g.lib.gecko_last_error().decode()


def test_backward_host_checks(g):
    st, msg = call_bwd(g)
    assert st == g.GECKO_EWORKSPACE and "workspace" in msg
    st, msg = call_bwd(g, din=g.GECKO_F32)
    assert st == g.GECKO_EUNSUPPORTED and "bf16" in msg
    st, msg = call_bwd(g, d=64, dvs=128)
    assert st == g.GECKO_EUNSUPPORTED
    st, msg = call_bwd(g, parts=0)
    assert st == g.GECKO_EINVAL and "parts" in msg
    st, msg = call_bwd(g, flags=8)
    assert st == g.GECKO_EINVAL
    st, msg = call_bwd(g, dout=0)
    assert st == g.GECKO_EINVAL and "non-null" in msg
    # without the memory part its vectors may be null (the workspace is still needed)
    st, msg = call_bwd(g, aff=[FAKE + 64 * i for i in range(4)] + [0] * 4, parts=g.GECKO_PART_SCA)
    assert st == g.GECKO_EWORKSPACE
    st, msg = call_bwd(g, aff=[FAKE + 64 * i for i in range(4)] + [0] * 4)
    assert st == g.GECKO_EINVAL and "affine" in msg
    st, msg = call_bwd(g, dz=FAKE + 8)
    assert st == g.GECKO_EINVAL and "aligned" in msg
    st, msg = call_bwd(g, dz=FAKE)  # dz on top of z
    assert st == g.GECKO_EINVAL and "alias" in msg
    st, msg = call_bwd(g, dv=6 * FAKE + 4096)  # dv inside dz
    assert st == g.GECKO_EINVAL and ("overlap" in msg or "alias" in msg)
    st, msg = call_bwd(g, n=0)
    assert st == g.GECKO_EINVAL


def test_backward_workspace_size(g):
    full = g.gecko_backward_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16, g.GECKO_BF16)
    sca = g.gecko_backward_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16, g.GECKO_BF16,
                                          parts=g.GECKO_PART_SCA)
    awm = g.gecko_backward_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16, g.GECKO_BF16,
                                          parts=g.GECKO_PART_AWM)
    rows = 8 * 131072
    # attention: q' (bf16), row statistics, dQ and dK (fp32) per token
    assert sca >= rows * (128 * 2 + 8 + 2 * 128 * 4)
    # memory: dQ_m, dK_m per token plus per-chunk state gradients
    assert awm >= rows * 2 * 128 * 4 + 8 * 62 * (128 * 256 * (4 + 2) + 2 * 128 * 128 * 2)
    assert full >= max(sca, awm)
    f32 = g.gecko_backward_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16, g.GECKO_F32)
    assert f32 >= full + rows * 256 * 2  # a bf16 copy of a float32 dO
    with pytest.raises(g.GeckoError):
        g.gecko_backward_workspace_size(1, 1, 100, 64, 64, 32, g.GECKO_BF16, g.GECKO_BF16)
    with pytest.raises(g.GeckoError):
        g.gecko_backward_workspace_size(1, 1, 100, 128, 256, 32, g.GECKO_F32, g.GECKO_F32)


def test_forward_lse_host_checks(g):
    def call(**kw):
        a = dict(parts=3, lse=4 * FAKE, din=g.GECKO_BF16, ws=0, wsb=0)
        a.update(kw)
        st = g.lib.gecko_forward_lse(FAKE, *[FAKE + 64 * i for i in range(8)], 2 * FAKE, 3 * FAKE, a["lse"], 1, 1,
                                     1000, 128, 256, 100, a["din"], g.GECKO_BF16, 0, a["parts"], a["ws"], a["wsb"],
                                     None)
        return st, g.lib.gecko_last_error().decode()

    st, msg = call(parts=g.GECKO_PART_AWM)
    assert st == g.GECKO_EINVAL and "GECKO_PART_SCA" in msg
    st, msg = call(din=g.GECKO_F32)
    assert st == g.GECKO_EUNSUPPORTED
    st, msg = call(lse=0)
    assert st == g.GECKO_EINVAL
    st, msg = call(lse=3 * FAKE + 64)  # inside out
    assert st == g.GECKO_EINVAL and "alias" in msg
    st, msg = call()  # the memory part needs the workspace
    assert st == g.GECKO_EWORKSPACE

def test_memory_saved_size(g):
    # no chunk reads the memory at n <= 2c (sliding) or n <= c (chunk-wise)
    assert g.gecko_memory_saved_size(1, 2, 256, 128, 256, 128) == 0
    assert g.gecko_memory_saved_size(1, 2, 128, 128, 256, 128, flags=g.GECKO_CHUNKWISE) == 0
    one = g.gecko_memory_saved_size(1, 2, 257, 128, 256, 128)  # one memory step
    assert one > 0
    # at least the float32 states, the bf16 snapshots and the float32 write products
    BH, d, dv = 2, 128, 256
    assert one >= BH * d * dv * (4 + 2 + 4)
    two = g.gecko_memory_saved_size(1, 2, 385, 128, 256, 128)
    assert two > one
    assert g.gecko_memory_saved_size(2, 1, 385, 128, 256, 128) == two  # only B * H matters
    assert g.gecko_memory_saved_size(1, 2, 385, 128, 128, 128) < two
    for bad in (dict(in_code=g.GECKO_F32), dict(flags=1 << 7)):
        with pytest.raises(g.GeckoError):
            g.gecko_memory_saved_size(1, 2, 385, 128, 256, 128, **bad)
    with pytest.raises(g.GeckoError):
        g.gecko_memory_saved_size(1, 2, 385, 64, 64, 128)  # no backward built for this pair


def test_forward_train_host_checks(g):
    def call(**kw):
        a = dict(parts=3, o=4 * FAKE, stats=5 * FAKE, din=g.GECKO_BF16, d=128, dvs=256, ws=0, wsb=0, mem=0, memb=0)
        a.update(kw)
        st = g.lib.gecko_forward_train(FAKE, *[FAKE + 64 * i for i in range(8)], 2 * FAKE, 3 * FAKE, a["o"],
                                       a["stats"], a["mem"], a["memb"], 1, 1, 1000, a["d"], a["dvs"], 100, a["din"],
                                       g.GECKO_BF16, 0, a["parts"], a["ws"], a["wsb"], None)
        return st, g.lib.gecko_last_error().decode()

    st, msg = call(parts=g.GECKO_PART_AWM)
    assert st == g.GECKO_EINVAL and "GECKO_PART_SCA" in msg
    st, msg = call(din=g.GECKO_F32)
    assert st == g.GECKO_EUNSUPPORTED
    st, msg = call(d=64, dvs=128)
    assert st == g.GECKO_EUNSUPPORTED
    st, msg = call(o=0)
    assert st == g.GECKO_EINVAL and "non-null" in msg
    st, msg = call(stats=5 * FAKE + 4)
    assert st == g.GECKO_EINVAL and "aligned" in msg
    st, msg = call(o=3 * FAKE + 64)  # inside out
    assert st == g.GECKO_EINVAL and "alias" in msg
    st, msg = call(stats=FAKE + 256)  # inside z
    assert st == g.GECKO_EINVAL and "alias" in msg
    st, msg = call()  # the memory part needs the workspace
    assert st == g.GECKO_EWORKSPACE
    # mem_saved in place of the workspace: size, alignment, aliasing
    need = g.gecko_memory_saved_size(1, 1, 1000, 128, 256, 100)
    st, msg = call(mem=6 * FAKE, memb=need - 1)
    assert st == g.GECKO_EWORKSPACE and "mem_saved too small" in msg
    st, msg = call(mem=6 * FAKE + 16, memb=need)
    assert st == g.GECKO_EINVAL and "mem_saved must be 256-byte aligned" in msg
    far = dict(o=64 * FAKE, stats=80 * FAKE, memb=need)
    st, msg = call(mem=3 * FAKE - 256, **far)  # runs into out
    assert st == g.GECKO_EINVAL and "out aliases the mem_saved" in msg
    st, msg = call(mem=80 * FAKE - 256, **far)  # runs into stats
    assert st == g.GECKO_EINVAL and "alias" in msg and "mem_saved" in msg
    st, msg = call(mem=FAKE, **far)  # on top of z
    assert st == g.GECKO_EINVAL and "alias" in msg and "mem_saved" in msg
    # without the memory part, mem_saved is not used
    st, msg = call(parts=g.GECKO_PART_SCA, mem=6 * FAKE + 16, memb=1)
    assert st != g.GECKO_EINVAL or "mem_saved" not in msg

    # mem_saved in place of the workspace: size, alignment, aliasing
    need = g.gecko_memory_saved_size(1, 1, 1000, 128, 256, 100)
    st, msg = call(mem=6 * FAKE, memb=need - 1)
    assert st == g.GECKO_EWORKSPACE and "mem_saved too small" in msg
    st, msg = call(mem=6 * FAKE + 16, memb=need)
    assert st == g.GECKO_EINVAL and "mem_saved must be 256-byte aligned" in msg
    far = dict(o=64 * FAKE, stats=80 * FAKE, memb=need)
    st, msg = call(mem=3 * FAKE - 256, **far)  # runs into out
    assert st == g.GECKO_EINVAL and "out aliases the mem_saved" in msg
    st, msg = call(mem=80 * FAKE - 256, **far)  # runs into stats
    assert st == g.GECKO_EINVAL and "alias" in msg and "mem_saved" in msg
    st, msg = call(mem=FAKE, **far)  # on top of z
    assert st == g.GECKO_EINVAL and "alias" in msg and "mem_saved" in msg
    # without the memory part, mem_saved is not used
    st, msg = call(parts=g.GECKO_PART_SCA, mem=6 * FAKE + 16, memb=1)
    assert st != g.GECKO_EINVAL or "mem_saved" not in msg


def test_memory_saved_size(g):
    # no chunk reads the memory at n <= 2c (sliding) or n <= c (chunk-wise)
    assert g.gecko_memory_saved_size(1, 2, 256, 128, 256, 128) == 0
    assert g.gecko_memory_saved_size(1, 2, 128, 128, 256, 128, flags=g.GECKO_CHUNKWISE) == 0
    one = g.gecko_memory_saved_size(1, 2, 257, 128, 256, 128)  # one memory step
    assert one > 0
    # at least the float32 states, the bf16 snapshots and the float32 write products
    BH, d, dv = 2, 128, 256
    assert one >= BH * d * dv * (4 + 2 + 4)
    two = g.gecko_memory_saved_size(1, 2, 385, 128, 256, 128)
    assert two > one
    assert g.gecko_memory_saved_size(2, 1, 385, 128, 256, 128) == two  # only B * H matters
    assert g.gecko_memory_saved_size(1, 2, 385, 128, 128, 128) < two
    for bad in (dict(in_code=g.GECKO_F32), dict(flags=1 << 7)):
        with pytest.raises(g.GeckoError):
            g.gecko_memory_saved_size(1, 2, 385, 128, 256, 128, **bad)
    with pytest.raises(g.GeckoError):
        g.gecko_memory_saved_size(1, 2, 385, 64, 64, 128)  # no backward built for this pair


def call_bwd_saved(g, **kw):
    a = dict(z=FAKE, aff=[FAKE + 64 * i for i in range(8)], v=2 * FAKE, dout=5 * FAKE, o=3 * FAKE, stats=4 * FAKE,
             dz=6 * FAKE, dv=7 * FAKE, daff=8 * FAKE, parts=3, ws=0, wsb=0, mem=0, memb=0)
    a.update(kw)
    st = g.lib.gecko_backward_saved(a["z"], *a["aff"], a["v"], a["dout"], a["o"], a["stats"], a["mem"], a["memb"],
                                    a["dz"], a["dv"], a["daff"], 1, 1, 1000, 128, 256, 128, g.GECKO_BF16,
                                    g.GECKO_BF16, 0, a["parts"], a["ws"], a["wsb"], None)
    return st, g.lib.gecko_last_error().decode()


def test_backward_saved_host_checks(g):
    st, msg = call_bwd_saved(g)
    assert st == g.GECKO_EWORKSPACE and "workspace" in msg
    st, msg = call_bwd_saved(g, parts=g.GECKO_PART_AWM)
    assert st == g.GECKO_EINVAL and "attention" in msg
    st, msg = call_bwd_saved(g, o=0)
    assert st == g.GECKO_EINVAL and "non-null" in msg
    st, msg = call_bwd_saved(g, stats=4 * FAKE + 4)
    assert st == g.GECKO_EINVAL and "aligned" in msg
    st, msg = call_bwd_saved(g, o=FAKE + 8)
    assert st == g.GECKO_EINVAL and "aligned" in msg
    # with a workspace, the alias checks (every case below fails before any launch)
    ws = 16 * FAKE
    st, msg = call_bwd_saved(g, o=6 * FAKE, ws=ws, wsb=1 << 40)  # o_sca on top of dz
    assert st == g.GECKO_EINVAL and "alias" in msg
    st, msg = call_bwd_saved(g, stats=ws + 4096, ws=ws, wsb=1 << 40)  # stats inside the workspace
    assert st == g.GECKO_EINVAL and "alias" in msg
    # the training forward's kept memory pass: size, alignment, aliasing
    need = g.gecko_memory_saved_size(1, 1, 1000, 128, 256, 128)
    st, msg = call_bwd_saved(g, mem=64 * FAKE, memb=need - 1)
    assert st == g.GECKO_EWORKSPACE and "mem_saved too small" in msg
    st, msg = call_bwd_saved(g, mem=64 * FAKE + 128, memb=need)
    assert st == g.GECKO_EINVAL and "mem_saved must be 256-byte aligned" in msg
    st, msg = call_bwd_saved(g, mem=ws, memb=need, ws=ws, wsb=1 << 40)
    assert st == g.GECKO_EINVAL and "mem_saved aliases the workspace" in msg
    st, msg = call_bwd_saved(g, mem=7 * FAKE - 256, memb=need, ws=ws, wsb=1 << 40)  # runs into dv
    assert st == g.GECKO_EINVAL and "mem_saved aliases an output" in msg
    # ignored without the memory part: the call goes on to its workspace check
    st, msg = call_bwd_saved(g, parts=g.GECKO_PART_SCA, mem=64 * FAKE + 128, memb=1)
    assert st == g.GECKO_EWORKSPACE and "mem_saved" not in msg


def test_backward_saved_workspace_size(g):
    rows = 8 * 131072
    plain = g.gecko_backward_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16, g.GECKO_BF16)
    saved = g.gecko_backward_saved_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16, g.GECKO_BF16)
    assert saved >= plain + rows * 256 * 2  # the per-query scaled dO (bf16)
    with pytest.raises(g.GeckoError):
        g.gecko_backward_saved_workspace_size(1, 8, 131072, 128, 256, 2048, g.GECKO_BF16, g.GECKO_BF16,
                                              parts=g.GECKO_PART_AWM)


def test_launch_failure_without_a_device(g):
    """Arguments that pass validation on a machine with no HIP device: the
    first launch fails and the call returns GECKO_EHIP with the runtime's
    message, no exception crosses the ABI. Runs only where there is no
    device, so that nothing is ever launched with these placeholder
    addresses."""
    import torch

    if torch.cuda.device_count() != 0:
        pytest.skip("a HIP device is present: the call would launch kernels on placeholder addresses")
    big = 1 << 40
    # attention only (no workspace): B1 H1, 100 tokens in one chunk, (d, dv) = (128, 256)
    st = g.lib.gecko_sca_forward(big, big + 4096, big + 8192, big + 12288, big + 16384, 2 * big, 3 * big,
                                 1, 1, 100, 128, 256, 100, g.GECKO_BF16, g.GECKO_BF16, None)
    msg = g.lib.gecko_last_error().decode()
    assert st == g.GECKO_EHIP, (st, msg)
    assert "launch" in msg
