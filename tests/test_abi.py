"""The C ABI library without a GPU: it loads, exports every symbol the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import exact_attention_online_softmax_amd as osm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "osm.h")

FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation


def _hip_device_count():
    """Devices that the HIP runtime libosm.so is bound to sees (0 when it
    reports none, or on any error).  The runtime is the instance already
    mapped into this process (loading the library loads it), so no second
    instance is started."""
    try:
        osm.load_library()
        path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln), None)
        if path is None:
            return 0
        hip = ctypes.CDLL(path)
    except OSError:
        return 0
    n = ctypes.c_int(0)
    err = hip.hipGetDeviceCount(ctypes.byref(n))
    return n.value if err == 0 else 0


def _has_gpu():
    """True when either the HIP runtime or torch sees a device: the
    fake-pointer tests below must never reach a launch on a real GPU."""
    if _hip_device_count() > 0:
        return True
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


no_gpu_only = pytest.mark.skipif(_has_gpu(), reason="fake-pointer checks run only without a GPU")


@pytest.fixture(scope="module")
def lib():
    return osm.load_library()


def test_header_symbols_exported(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(osm_[a-z0-9_]+)\s*\(", text))
    assert declared == set(osm.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in osm.STATUS.items():
        assert osm.status_str(code).startswith(name)
    assert osm.status_str(99) == "OSM_ERR_UNKNOWN"


def test_workspace_bytes(lib):
    # m, l: rows * C floats each; O~: rows * C * d floats; each 256-byte aligned
    rows, C, d = 16 * 32, 128, 128
    al = lambda n: (n + 255) // 256 * 256
    assert osm.decode_workspace_bytes(16, 32, 32768, 128, 256) == 2 * al(rows * C * 4) + al(rows * C * d * 4)
    assert osm.decode_workspace_bytes(1, 1, 4096, 64, 64) == 2 * al(64 * 4) + al(64 * 64 * 4)
    assert osm.decode_workspace_bytes(1, 1, 4097, 64, 64) == 2 * al(65 * 4) + al(65 * 64 * 4)
    assert osm.decode_workspace_bytes(0, 1, 1, 64, 64) == 0
    assert osm.decode_workspace_bytes(1, 1, 1, 64, 0) == 0


@no_gpu_only
def test_softmax_validation(lib):
    s = None
    assert lib.osm_softmax_rows(FAKE, FAKE, -1, 4, 4, 4, None, None, s) == 2
    assert lib.osm_softmax_rows(FAKE, FAKE, 2, 4, 3, 4, None, None, s) == 2     # ld_x < cols
    assert lib.osm_softmax_rows(FAKE, FAKE, 2, 4, 4, 3, None, None, s) == 2
    assert lib.osm_softmax_rows(None, FAKE, 2, 4, 4, 4, None, None, s) == 1
    assert lib.osm_softmax_rows(FAKE, None, 2, 4, 4, 4, None, None, s) == 1
    assert lib.osm_softmax_rows(None, None, 0, 4, 4, 4, None, None, s) == 0     # nothing to do
    f = lib.osm_softmax_rows_twopass
    assert f(FAKE, FAKE, -1, 4, 4, 4, None, None, s) == 2
    assert f(FAKE, FAKE, 2, 4, 3, 4, None, None, s) == 2
    assert f(FAKE, FAKE, 2, 4, 4, 3, None, None, s) == 2
    assert f(None, FAKE, 2, 4, 4, 4, None, None, s) == 1
    assert f(FAKE, None, 2, 4, 4, 4, None, None, s) == 1
    assert f(None, None, 0, 4, 4, 4, None, None, s) == 0
    assert f(None, None, 3, 0, 0, 0, None, None, s) == 0                       # no columns, no stats


@no_gpu_only
def test_attn_fwd_validation(lib):
    def call(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=osm.OSM_BF16, B=1, Hq=2, Hkv=1, Nq=8, Nk=8,
             d=128, scale=0.1, causal=0):
        return lib.osm_attn_fwd(q, k, v, o, None, dtype, B, Hq, Hkv, Nq, Nk, d, None, None,
                                scale, causal, None)
    assert call(B=0) == 2
    assert call(Hq=3, Hkv=2) == 2
    assert call(Nq=-1) == 2
    assert call(scale=0.0) == 2
    assert call(scale=float("inf")) == 2
    assert call(scale=float("nan")) == 2
    assert call(causal=2) == 2
    assert call(dtype=osm.OSM_F32) == 3
    assert call(d=96) == 3
    assert call(d=64, q=None) == 1                  # head dim 64 is supported: fails only at the NULL check
    assert call(Nk=1 << 23) == 3                    # one head's K rows would span 2 GiB
    assert call(d=64, Nk=1 << 23, q=None) == 1      # at head dim 64 the same keys span 1 GiB
    assert call(d=64, Nk=1 << 24) == 3
    assert call(Nq=1 << 23) == 3                    # one head's Q (and O) rows would span 2 GiB
    assert call(Nq=(1 << 23) - 1, q=None) == 1      # just below: accepted as far as the NULL check
    assert call(q=None) == 1
    assert call(o=None) == 1
    assert call(k=None) == 1
    # no keys: k and v may be NULL (the request then fails only at the
    # alignment check that follows the NULL check, before any launch)
    assert call(k=None, v=None, Nk=0, o=ctypes.c_void_p(0x10008)) == 3
    assert call(q=None, Nq=0) == 0                  # nothing to compute
    assert call(q=ctypes.c_void_p(0x10002)) == 3    # not 16-byte aligned
    assert call(o=ctypes.c_void_p(0x10008)) == 3
    assert call(B=65536, Hq=32768) == 3             # 2^31 (batch, head) pairs


@no_gpu_only
def test_decode_validation(lib):
    ws_ok = osm.decode_workspace_bytes(2, 8, 1000, 128, 256)

    def call(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, dtype=osm.OSM_BF16, B=2, Hq=8, Hkv=2, L=1000,
             d=128, sk=FAKE, scale=0.1, split=256, ws=FAKE, wsb=ws_ok):
        return lib.osm_attn_decode_splitkv(q, kc, vc, o, None, dtype, B, Hq, Hkv, L, d, sk, scale,
                                           split, ws, wsb, None)
    assert call(B=0) == 2
    assert call(Hq=6, Hkv=4) == 2
    assert call(split=0) == 2
    assert call(scale=-1.0) == 2
    assert call(d=96) == 3
    assert call(Hq=6, Hkv=2) == 3                   # group of 3
    assert call(split=100) == 3                     # not a multiple of 64
    assert call(split=8192 + 64) == 3
    assert call(Hq=16, Hkv=2, split=4096) == 3      # 8 * 4096 scores exceed the LDS budget
    assert call(dtype=7) == 3
    assert call(sk=None) == 1
    assert call(q=None) == 1
    assert call(ws=None) == 4
    assert call(wsb=ws_ok - 1) == 4
    assert call(ws=ctypes.c_void_p(0x10010)) == 4   # not 256-byte aligned
    assert call(kc=ctypes.c_void_p(0x10008)) == 3   # not 16-byte aligned
    assert call(B=65536, Hq=32768, Hkv=4096) == 3   # 2^31 (batch, head) pairs


@no_gpu_only
def test_decode_noalloc_validation(lib):
    """The allocation-free decode checks its arguments like the workspace
    entry point, and rejects partials larger than the library's 64 MiB
    scratch array with OSM_ERR_WORKSPACE, before any HIP call."""
    def call(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, dtype=osm.OSM_BF16, B=16, Hq=32, Hkv=8, L=32768,
             d=128, sk=FAKE, scale=0.1, split=256):
        return lib.osm_attn_decode_splitkv_noalloc(q, kc, vc, o, None, dtype, B, Hq, Hkv, L, d, sk, scale,
                                                   split, None)
    assert call(B=0) == 2
    assert call(split=0) == 2
    assert call(d=96) == 3
    assert call(split=100) == 3
    assert call(sk=None) == 1
    assert call(kc=ctypes.c_void_p(0x10008)) == 3
    assert lib.osm_decode_workspace_bytes(64, 32, 32768, 128, 256) > (64 << 20)
    assert call(B=64) == 4                          # 136 MiB of partials
    assert call(B=16, L=131072) == 4


@no_gpu_only
def test_merge_validation(lib):
    def call(pm=FAKE, pl=FAKE, po=FAKE, rows=4, C=3, d=64, o=FAKE, dt=osm.OSM_F32):
        return lib.osm_merge_partials(pm, pl, po, rows, C, d, o, dt, None, None)
    assert call(rows=-1) == 2
    assert call(C=0) == 2
    assert call(d=0) == 2
    assert call(d=513) == 3
    assert call(dt=9) == 3
    assert call(pm=None) == 1
    assert call(o=None) == 1
    assert call(pm=None, rows=0) == 0


@no_gpu_only
def test_merge_lse_validation(lib):
    def call(op=FAKE, lp=FAKE, rows=4, S=3, d=128, it=osm.OSM_BF16, o=FAKE, ot=osm.OSM_BF16):
        return lib.osm_merge_lse(op, lp, rows, S, d, it, o, ot, None, None)
    assert call(rows=-1) == 2
    assert call(S=0) == 2
    assert call(d=0) == 2
    assert call(d=1026) == 3
    assert call(d=513) == 3                         # odd head_dim is limited to 511
    assert call(it=9) == 3
    assert call(ot=9) == 3
    assert call(op=None) == 1
    assert call(lp=None) == 1
    assert call(o=None) == 1
    assert call(op=None, rows=0) == 0
    assert call(op=ctypes.c_void_p(0x10008)) == 3    # pieces not 16-byte aligned
    assert call(o=ctypes.c_void_p(0x10004)) == 3     # output not 16-byte aligned


@no_gpu_only
def test_extend_validation(lib):
    ws_ok = lib.osm_decode_workspace_bytes(1, 2, 100, 128, 64)
    def call(q=FAKE, k=FAKE, v=FAKE, dt=osm.OSM_BF16, B=1, Hq=2, Hkv=1, n=100, d=128, scale=0.1,
             sm=FAKE, sl=FAKE, so=FAKE, split=64, ws=FAKE, wsb=ws_ok):
        return lib.osm_attn_extend(q, k, v, dt, B, Hq, Hkv, n, d, scale, sm, sl, so, split, ws, wsb, None)
    assert call(B=0) == 2
    assert call(n=-1) == 2
    assert call(Hq=3, Hkv=2) == 2
    assert call(scale=float("nan")) == 2
    assert call(d=96) == 3
    assert call(dt=9) == 3
    assert call(split=100) == 3
    assert call(Hq=16, Hkv=1) == 3                  # group 16
    assert call(sm=None) == 1
    assert call(so=None) == 1
    assert call(n=0, q=None, k=None, v=None) == 0   # no new keys: nothing to do
    assert call(q=None) == 1
    assert call(wsb=ws_ok - 1) == 4
    assert call(ws=ctypes.c_void_p(0x10004)) == 4    # not 256-byte aligned
    assert call(v=ctypes.c_void_p(0x10004)) == 3     # not 16-byte aligned
    assert call(B=65536, Hq=32768, Hkv=32768) == 3   # 2^31 (batch, head) pairs


def test_attn_fwd_fp8_validation(lib):
    def call(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=128, scale=0.1,
             vs=1.0, causal=0):
        return lib.osm_attn_fwd_fp8(q, k, v, o, None, B, Hq, Hkv, Nq, Nk, d, None, None, scale, vs,
                                    causal, None)
    assert call(B=0) == 2
    assert call(Hq=3, Hkv=2) == 2
    assert call(scale=-1.0) == 2
    assert call(vs=float("nan")) == 2
    assert call(causal=3) == 2
    assert call(d=64) == 3
    assert call(Nk=1 << 24) == 3
    assert call(Nq=1 << 23) == 3                     # one head's bf16 O rows would span 2 GiB
    assert call(Nq=(1 << 23) - 1, q=None) == 1
    assert call(Nq=0, q=None) == 0
    assert call(q=None) == 1
    assert call(v=None) == 1
    assert call(o=ctypes.c_void_p(0x10001)) == 3     # not 16-byte aligned
    assert call(B=65536, Hq=32768) == 3              # 2^31 (batch, head) pairs


def test_attn_bwd_validation(lib):
    ws_ok = lib.osm_attn_bwd_workspace_bytes(1, 2, 8)
    assert ws_ok == 1 * 2 * 8 * 8
    assert lib.osm_attn_bwd_workspace_bytes(0, 2, 8) == 0

    def call(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             dtype=osm.OSM_BF16, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=128, scale=0.1, causal=0,
             ws=FAKE, wsb=ws_ok):
        return lib.osm_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, dtype, B, Hq, Hkv, Nq, Nk, d,
                                None, None, scale, causal, ws, wsb, None)
    assert call(B=0) == 2
    assert call(Nq=-1) == 2
    assert call(Hq=3, Hkv=2) == 2
    assert call(scale=0.0) == 2
    assert call(scale=float("inf")) == 2
    assert call(causal=2) == 2
    assert call(d=96) == 3
    assert call(d=256) == 3
    assert call(dtype=osm.OSM_F32) == 3
    assert call(Nk=1 << 23) == 3                    # one head's rows span 2 GiB
    assert call(d=64, q=None) == 1                  # head dim 64 is supported: fails only at the NULL check
    assert call(d=64, Nk=1 << 23, q=None) == 1      # at head dim 64 the same keys span 1 GiB
    assert call(d=64, Nq=1 << 24) == 3
    assert call(Nq=0, Nk=0, q=None, k=None) == 0    # nothing to do
    for name in ("q", "o", "do", "lse", "dq", "k", "v", "dk", "dv"):
        assert call(**{name: None}) == 1, name
    assert call(dk=ctypes.c_void_p(0x10008)) == 3   # not 16-byte aligned
    assert call(B=65536, Hq=32768) == 3             # 2^31 (batch, head) pairs
    assert call(wsb=ws_ok - 1) == 4
    assert call(ws=None) == 4
    assert call(ws=ctypes.c_void_p(0x10010)) == 4   # not 256-byte aligned


@no_gpu_only
def test_no_device_reports_hip_error(lib):
    """A fully valid request in a process without a GPU fails cleanly with
    OSM_ERR_HIP (the launch is refused by the runtime, nothing is read)."""
    rc = lib.osm_merge_partials(FAKE, FAKE, FAKE, 4, 3, 64, FAKE, osm.OSM_F32, None, None)
    assert rc == 5
    rc = lib.osm_softmax_rows(FAKE, FAKE, 2, 4, 4, 4, None, None, None)
    assert rc == 5
    rc = lib.osm_merge_lse(FAKE, FAKE, 4, 3, 128, osm.OSM_BF16, FAKE, osm.OSM_BF16, None, None)
    assert rc == 5
