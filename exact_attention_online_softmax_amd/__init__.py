"""Exact softmax attention via the online-softmax recurrence, for MI355X.

Thin ctypes binding of ``libosm.so`` (C ABI declared in ``include/osm.h``).
This module only marshals arguments: every step of every operation runs in
the library's HIP kernels on the GPU.  PyTorch supplies device memory and
the current stream.  There is no CPU fallback: if ``libosm.so`` is missing
or a call fails, an exception is raised.

Entry points (same names as the C ABI, without the ``osm_`` prefix):

* ``softmax_rows(x, return_stats=False, two_pass=False)``
* ``attn_fwd(q, k, v, *, scale=None, causal=False, seqlens_q=None, seqlens_k=None)``
* ``attn_decode_splitkv(q, k_cache, v_cache, seqlens_k, *, scale=None, split_size=256)``
* ``merge_partials(part_m, part_l, part_o, out_dtype=torch.float32)``
* ``decode_workspace_bytes(batch, heads_q, max_seqlen_k, head_dim, split_size)``
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libosm.so")

OSM_F32 = 0
OSM_BF16 = 1
STATUS = {0: "OSM_OK", 1: "OSM_ERR_NULL", 2: "OSM_ERR_SHAPE", 3: "OSM_ERR_UNSUPPORTED",
          4: "OSM_ERR_WORKSPACE", 5: "OSM_ERR_HIP"}
EXPORTS = ("osm_status_str", "osm_softmax_rows", "osm_softmax_rows_twopass", "osm_attn_fwd", "osm_decode_workspace_bytes",
           "osm_attn_decode_splitkv", "osm_merge_partials", "osm_merge_lse", "osm_attn_extend",
           "osm_attn_bwd_workspace_bytes", "osm_attn_bwd", "osm_attn_fwd_fp8",
           "osm_attn_decode_splitkv_noalloc")


class OsmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


_lib = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libosm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m exact_attention_online_softmax_amd.build`")
    # torch first: its HIP runtime then satisfies libosm.so's dependency on
    # libamdhip64.so.7, so the library and the tensors and streams it is given
    # share one runtime.  Loaded the other way round, the process would hold
    # two runtime instances, and the library's would not see torch's device
    # memory or streams.
    _torch()
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.osm_status_str.argtypes = [ctypes.c_int]
    lib.osm_status_str.restype = ctypes.c_char_p
    lib.osm_softmax_rows.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp]
    lib.osm_softmax_rows_twopass.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp]
    lib.osm_attn_fwd.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i32, i32, i32, i32, i32, i32,
                                 vp, vp, f32, i32, vp]
    lib.osm_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.osm_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.osm_attn_decode_splitkv.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i32, i32, i32, i32,
                                            i32, vp, f32, i32, vp, ctypes.c_size_t, vp]
    lib.osm_attn_decode_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i32, i32, i32, i32,
                                                    i32, vp, f32, i32, vp]
    lib.osm_merge_partials.argtypes = [vp, vp, vp, i64, i32, i32, vp, ctypes.c_int, vp, vp]
    lib.osm_merge_lse.argtypes = [vp, vp, i64, i32, i32, ctypes.c_int, vp, ctypes.c_int, vp, vp]
    lib.osm_attn_extend.argtypes = [vp, vp, vp, ctypes.c_int, i32, i32, i32, i32, i32, f32, vp, vp, vp,
                                    i32, vp, ctypes.c_size_t, vp]
    lib.osm_attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, f32, f32,
                                     i32, vp]
    lib.osm_attn_bwd_workspace_bytes.argtypes = [i32, i32, i32]
    lib.osm_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.osm_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i32, i32, i32, i32,
                                 i32, i32, vp, vp, f32, i32, vp, ctypes.c_size_t, vp]
    for name in ("osm_softmax_rows", "osm_softmax_rows_twopass", "osm_attn_fwd", "osm_attn_decode_splitkv",
                 "osm_merge_partials", "osm_merge_lse", "osm_attn_extend", "osm_attn_bwd",
                 "osm_attn_fwd_fp8", "osm_attn_decode_splitkv_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load_library().osm_status_str(code).decode()


def _check(code: int) -> None:
    if code != 0:
        raise OsmError(code, status_str(code))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _device_tensor(t, name, dtypes):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out_tensor(t, name, shape, dtype, device):
    """A caller-supplied output: the kernels write exactly ``shape`` contiguous
    elements of ``dtype`` through its pointer, so anything else is refused
    before the launch."""
    _device_tensor(t, name, (dtype,))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    return t


def _workspace(ws, nbytes, device):
    """The caller's device workspace (bytes), or a new one of ``nbytes``; the
    library checks its size, this checks that it is device memory."""
    torch = _torch()
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _device_tensor(ws, "workspace", (torch.uint8,))
    if ws.device != device:
        raise ValueError(f"workspace must be on {device} (got {ws.device})")
    return ws


def _dtype_code(dt):
    torch = _torch()
    return {torch.float32: OSM_F32, torch.bfloat16: OSM_BF16}[dt]


def _lengths(t, name, batch, device):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        t = torch.as_tensor(t, dtype=torch.int32)
    t = t.to(device=device, dtype=torch.int32).contiguous()
    if t.numel() != batch:
        raise ValueError(f"{name} must have {batch} entries")
    return t


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def softmax_rows(x, return_stats: bool = False, out=None, two_pass: bool = False):
    """Row softmax of a 2-D fp32 GPU tensor (two-pass online normalizer).
    Returns y, or (y, row_max, row_sum) with ``return_stats``.  With
    ``two_pass`` every row is read twice from memory
    (``osm_softmax_rows_twopass``); otherwise rows of up to 65536 columns stay
    on chip between the passes."""
    torch = _torch()
    lib = load_library()
    _device_tensor(x, "x", (torch.float32,))
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    y = torch.empty_like(x) if out is None else _device_tensor(out, "out", (torch.float32,))
    if y.shape != x.shape:
        raise ValueError("out has the wrong shape")
    mx = sm = None
    if return_stats:
        mx = torch.empty(rows, dtype=torch.float32, device=x.device)
        sm = torch.empty(rows, dtype=torch.float32, device=x.device)
    fn = lib.osm_softmax_rows_twopass if two_pass else lib.osm_softmax_rows
    _check(fn(_ptr(x), _ptr(y), rows, cols, cols, cols, _ptr(mx), _ptr(sm), _stream()))
    return (y, mx, sm) if return_stats else y


def attn_fwd(q, k, v, *, scale=None, causal=False, seqlens_q=None, seqlens_k=None, out=None,
             lse=None):
    """Fused attention forward.  q [B, Hq, Nq, d], k/v [B, Hkv, Nk, d] bf16.
    Returns (o [B, Hq, Nq, d] bf16, lse [B, Hq, Nq] fp32)."""
    torch = _torch()
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _device_tensor(t, name, (torch.bfloat16,))
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, heads, positions, head_dim]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k, v shapes are inconsistent")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else _out_tensor(out, "out", q.shape, q.dtype, q.device)
    lse_t = (torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None
             else _out_tensor(lse, "lse", (B, Hq, Nq), torch.float32, q.device))
    sq = _lengths(seqlens_q, "seqlens_q", B, q.device)
    sk = _lengths(seqlens_k, "seqlens_k", B, q.device)
    _check(lib.osm_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t),
                            _dtype_code(q.dtype), B, Hq, Hkv, Nq, Nk, d, _ptr(sq), _ptr(sk),
                            float(scale), int(bool(causal)), _stream()))
    return o, lse_t


def attn_fwd_fp8(q, k, v, *, scale=None, v_scale=1.0, causal=False, seqlens_q=None, seqlens_k=None,
                 out=None, lse=None):
    """Fused attention forward with FP8 E4M3 inputs (torch.float8_e4m3fn, or
    uint8 tensors of E4M3 codes).  q [B, Hq, Nq, d], k/v [B, Hkv, Nk, d].
    Returns (o [B, Hq, Nq, d] bf16, lse [B, Hq, Nq] fp32)."""
    torch = _torch()
    lib = load_library()
    fp8 = tuple(t for t in (getattr(torch, "float8_e4m3fn", None), torch.uint8) if t is not None)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _device_tensor(t, name, fp8)
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, heads, positions, head_dim]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k, v shapes are inconsistent")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = (torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q.device) if out is None
         else _out_tensor(out, "out", (B, Hq, Nq, d), torch.bfloat16, q.device))
    lse_t = (torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None
             else _out_tensor(lse, "lse", (B, Hq, Nq), torch.float32, q.device))
    sq = _lengths(seqlens_q, "seqlens_q", B, q.device)
    sk = _lengths(seqlens_k, "seqlens_k", B, q.device)
    _check(lib.osm_attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, Hq, Hkv, Nq, Nk, d,
                                _ptr(sq), _ptr(sk), float(scale), float(v_scale), int(bool(causal)),
                                _stream()))
    return o, lse_t


def attn_bwd_workspace_bytes(batch, heads_q, seqlen_q):
    return int(load_library().osm_attn_bwd_workspace_bytes(batch, heads_q, seqlen_q))


def attn_bwd(q, k, v, o, lse, dout, *, scale=None, causal=False, seqlens_q=None, seqlens_k=None,
             workspace=None, dq=None, dk=None, dv=None):
    """Attention backward from the forward's o and lse.  q, o, dout
    [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d] bf16; lse [B, Hq, Nq] fp32.
    Returns (dq, dk, dv) shaped like q, k, v."""
    torch = _torch()
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _device_tensor(t, name, (torch.bfloat16,))
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, heads, positions, head_dim]")
    _device_tensor(lse, "lse", (torch.float32,))
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk_ = k.shape
    if (Bk != B or dk_ != d or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape)
            or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Nq)):
        raise ValueError("q, k, v, o, lse, dout shapes are inconsistent")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sq = _lengths(seqlens_q, "seqlens_q", B, q.device)
    sk = _lengths(seqlens_k, "seqlens_k", B, q.device)
    workspace = _workspace(workspace, attn_bwd_workspace_bytes(B, Hq, Nq), q.device)
    dq = torch.empty_like(q) if dq is None else _out_tensor(dq, "dq", q.shape, q.dtype, q.device)
    dk = torch.empty_like(k) if dk is None else _out_tensor(dk, "dk", k.shape, k.dtype, q.device)
    dv = torch.empty_like(v) if dv is None else _out_tensor(dv, "dv", v.shape, v.dtype, q.device)
    _check(lib.osm_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                            _ptr(dk), _ptr(dv), _dtype_code(q.dtype), B, Hq, Hkv, Nq, Nk, d, _ptr(sq),
                            _ptr(sk), float(scale), int(bool(causal)), _ptr(workspace),
                            workspace.numel(), _stream()))
    return dq, dk, dv


def decode_workspace_bytes(batch, heads_q, max_seqlen_k, head_dim, split_size=256):
    return int(load_library().osm_decode_workspace_bytes(batch, heads_q, max_seqlen_k, head_dim,
                                                           split_size))


def attn_decode_splitkv(q, k_cache, v_cache, seqlens_k, *, scale=None, split_size=256,
                        workspace=None, out=None, lse=None):
    """Split-KV decode.  q [B, Hq, d]; caches [B, Hkv, Lmax, d] (bf16 or fp32);
    seqlens_k int32 [B].  Returns (o [B, Hq, d], lse [B, Hq] fp32)."""
    torch = _torch()
    lib = load_library()
    dts = (torch.bfloat16, torch.float32)
    _device_tensor(q, "q", dts)
    _device_tensor(k_cache, "k_cache", (q.dtype,))
    _device_tensor(v_cache, "v_cache", (q.dtype,))
    if q.dim() != 3 or k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q must be [B, Hq, d]; caches [B, Hkv, Lmax, d]")
    B, Hq, d = q.shape
    Bk, Hkv, Lmax, dk_ = k_cache.shape
    if Bk != B or dk_ != d:
        raise ValueError("the caches' batch and head_dim must match q's")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sk = _lengths(seqlens_k, "seqlens_k", B, q.device)
    workspace = _workspace(workspace, decode_workspace_bytes(B, Hq, Lmax, d, split_size), q.device)
    o = torch.empty_like(q) if out is None else _out_tensor(out, "out", q.shape, q.dtype, q.device)
    lse_t = (torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None
             else _out_tensor(lse, "lse", (B, Hq), torch.float32, q.device))
    _check(lib.osm_attn_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o),
                                       _ptr(lse_t), _dtype_code(q.dtype), B, Hq, Hkv, Lmax, d,
                                       _ptr(sk), float(scale), int(split_size), _ptr(workspace),
                                       workspace.numel(), _stream()))
    return o, lse_t


def merge_partials(part_m, part_l, part_o, out_dtype=None):
    """Merge partial summaries: part_m, part_l [rows, C] fp32, part_o
    [rows, C, d] fp32.  Returns (o [rows, d], lse [rows])."""
    torch = _torch()
    lib = load_library()
    for name, t in (("part_m", part_m), ("part_l", part_l), ("part_o", part_o)):
        _device_tensor(t, name, (torch.float32,))
    rows, C = part_m.shape
    d = part_o.shape[-1]
    if tuple(part_l.shape) != (rows, C) or tuple(part_o.shape) != (rows, C, d):
        raise ValueError("partials shapes are inconsistent")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    o = torch.empty((rows, d), dtype=out_dtype, device=part_m.device)
    lse = torch.empty(rows, dtype=torch.float32, device=part_m.device)
    _check(lib.osm_merge_partials(_ptr(part_m), _ptr(part_l), _ptr(part_o), rows, C, d, _ptr(o),
                                  _dtype_code(out_dtype), _ptr(lse), _stream()))
    return o, lse


def merge_lse(o_parts, lse_parts, out_dtype=None, out=None, lse=None):
    """Combine normalized results of disjoint key sets in log-sum-exp form:
    o_parts [S, rows, d] (fp32 or bf16), lse_parts [S, rows] fp32.  Returns
    (o [rows, d], lse [rows])."""
    torch = _torch()
    lib = load_library()
    _device_tensor(o_parts, "o_parts", (torch.float32, torch.bfloat16))
    _device_tensor(lse_parts, "lse_parts", (torch.float32,))
    if o_parts.dim() != 3 or lse_parts.dim() != 2:
        raise ValueError("o_parts must be [S, rows, d] and lse_parts [S, rows]")
    S, rows, d = o_parts.shape
    if tuple(lse_parts.shape) != (S, rows):
        raise ValueError("lse_parts shape does not match o_parts")
    out_dtype = o_parts.dtype if out_dtype is None else out_dtype
    o = (torch.empty((rows, d), dtype=out_dtype, device=o_parts.device) if out is None
         else _out_tensor(out, "out", (rows, d), out_dtype, o_parts.device))
    lse_t = (torch.empty(rows, dtype=torch.float32, device=o_parts.device) if lse is None
             else _out_tensor(lse, "lse", (rows,), torch.float32, o_parts.device))
    _check(lib.osm_merge_lse(_ptr(o_parts), _ptr(lse_parts), rows, S, d, _dtype_code(o_parts.dtype),
                             _ptr(o), _dtype_code(out_dtype), _ptr(lse_t), _stream()))
    return o, lse_t


def attn_state(batch, heads_q, head_dim, device="cuda"):
    """A fresh streaming summary (the empty set): m = -inf, l = 0, O~ = 0,
    shaped [batch * heads_q], [batch * heads_q], [batch * heads_q, head_dim]."""
    torch = _torch()
    rows = batch * heads_q
    return (torch.full((rows,), float("-inf"), dtype=torch.float32, device=device),
            torch.zeros(rows, dtype=torch.float32, device=device),
            torch.zeros((rows, head_dim), dtype=torch.float32, device=device))


def attn_extend(q, k_new, v_new, state, *, scale=None, split_size=512, workspace=None):
    """Fold new keys k_new, v_new [B, Hkv, n, d] into the streaming summary
    `state` = (m, l, O~) of the queries q [B, Hq, d], in place."""
    torch = _torch()
    lib = load_library()
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        _device_tensor(t, name, (torch.float32, torch.bfloat16))
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise TypeError("q, k_new and v_new must have one dtype")
    if q.dim() != 3 or k_new.dim() != 4 or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("q must be [B, Hq, d]; k_new, v_new [B, Hkv, n, d]")
    B, Hq, d = q.shape
    Bk, Hkv, n, dk_ = k_new.shape
    if Bk != B or dk_ != d:
        raise ValueError("k_new's batch and head_dim must match q's")
    sm, sl, so = state
    for name, t, shape in (("state_m", sm, (B * Hq,)), ("state_l", sl, (B * Hq,)), ("state_o", so, (B * Hq, d))):
        _out_tensor(t, name, shape, torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    workspace = _workspace(workspace, decode_workspace_bytes(B, Hq, max(n, 1), d, split_size), q.device)
    _check(lib.osm_attn_extend(_ptr(q), _ptr(k_new), _ptr(v_new), _dtype_code(q.dtype), B, Hq, Hkv, n, d,
                               float(scale), _ptr(sm), _ptr(sl), _ptr(so), int(split_size),
                               _ptr(workspace), workspace.numel(), _stream()))
    return state


def attn_state_finalize(state, out_dtype=None):
    """o = O~ / l and LSE = m + log l of a streaming summary (the state is
    not modified)."""
    torch = _torch()
    sm, sl, so = state
    rows, d = so.shape
    return merge_partials(sm.reshape(rows, 1), sl.reshape(rows, 1), so.reshape(rows, 1, d), out_dtype=out_dtype)
