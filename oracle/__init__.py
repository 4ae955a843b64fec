"""CPU fp64 oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does: the
two share no code.  The arithmetic lives in ``osm_oracle.c`` (plain fp64, the
pages' definitions written out); this module only marshals numpy arrays.

Functions that follow a definition on the pages (all pinned by tests under
``tests/test_oracle_*.py`` against printed values, closed forms, invariants
and brute force):

* ``softmax_rows``       safe softmax, three passes
* ``online_normalizer``  the scalar (m, l) recurrence, every step
* ``summary``            the (m, l, o~) triple of a set of scores
* ``merge``              the merge of partial triples, then o = o~/l
* ``attention``          naive attention materializing each score row
* ``merge_lse``          the log-sum-exp form of the merge
* ``attention_bwd``      gradients of naive attention (chain rule through the
                         forward definition; the pages print no backward)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "osm_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def compile_oracle(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, OpenMP over rows)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def _i64_or_null(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), a


def _i32_or_null(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), a


class Oracle:
    """ctypes view of one compiled oracle library (the default one, or a
    variant a test compiled from edited source)."""

    def __init__(self, path: str = LIBRARY):
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_softmax_rows.argtypes = [_f32p, i64, i64, vp, i64, _f64p, vp, vp]
        lib.oracle_online_normalizer.argtypes = [_f64p, i64, _f64p, _f64p]
        lib.oracle_summary.argtypes = [_f64p, _f64p, i64, i64, vp, vp, _f64p]
        lib.oracle_merge.argtypes = [_f32p, _f32p, _f32p, i64, i64, i64, _f64p, _f64p]
        lib.oracle_attention.argtypes = [_f32p, _f32p, _f32p, i64, i64, i64, i64, i64, i64,
                                         vp, vp, ctypes.c_double, ctypes.c_int, vp, i64,
                                         _f64p, _f64p]
        lib.oracle_merge_lse.argtypes = [_f64p, _f64p, _f64p, _f64p, i64, i64, _f64p, _f64p]
        lib.oracle_attention_bwd.argtypes = [_f32p, _f32p, _f32p, _f32p, i64, i64, i64, i64, i64,
                                             i64, vp, vp, ctypes.c_double, ctypes.c_int,
                                             _f64p, _f64p, _f64p]
        for f in (lib.oracle_softmax_rows, lib.oracle_online_normalizer, lib.oracle_summary,
                  lib.oracle_merge, lib.oracle_attention, lib.oracle_merge_lse,
                  lib.oracle_attention_bwd):
            f.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # -- softmax -----------------------------------------------------------
    def softmax_rows(self, x, rows=None):
        """Safe softmax of the rows of a 2-D fp32 array (or of ``rows`` only).
        Returns (y, m, l) in fp64."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        if x.ndim == 1:
            x = x[None, :]
        R, C = x.shape
        sel = _i64_or_null(rows)
        nsel = R if rows is None else len(sel[1])
        y = np.empty((nsel, C), np.float64)
        m = np.empty(nsel, np.float64)
        l = np.empty(nsel, np.float64)
        rc = self.lib.oracle_softmax_rows(
            x, C, C, None if sel is None else ctypes.cast(sel[0], ctypes.c_void_p), nsel, y,
            m.ctypes.data_as(ctypes.c_void_p), l.ctypes.data_as(ctypes.c_void_p))
        if rc:
            raise RuntimeError(f"oracle_softmax_rows failed ({rc})")
        return y, m, l

    def online_normalizer(self, s):
        """Running (m_j, l_j) after each score of the scalar recurrence."""
        s = np.ascontiguousarray(s, dtype=np.float64)
        m = np.empty(len(s), np.float64)
        l = np.empty(len(s), np.float64)
        if self.lib.oracle_online_normalizer(s, len(s), m, l):
            raise RuntimeError("oracle_online_normalizer failed")
        return m, l

    def summary(self, s, v):
        """The (m, l, o~) triple of scores ``s`` [n] and values ``v`` [n, d]."""
        s = np.ascontiguousarray(s, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        d = v.shape[-1] if v.ndim > 1 else 1
        v = v.reshape(len(s), d)
        m = ctypes.c_double()
        l = ctypes.c_double()
        o = np.empty(d, np.float64)
        if self.lib.oracle_summary(s, v, len(s), d, ctypes.byref(m), ctypes.byref(l), o):
            raise RuntimeError("oracle_summary failed")
        return m.value, l.value, o

    def merge(self, part_m, part_l, part_o):
        """Merge partial triples: part_m, part_l [rows, C]; part_o [rows, C, d].
        Returns (o [rows, d], lse [rows])."""
        part_m = np.ascontiguousarray(part_m, dtype=np.float32)
        part_l = np.ascontiguousarray(part_l, dtype=np.float32)
        part_o = np.ascontiguousarray(part_o, dtype=np.float32)
        rows, C = part_m.shape
        d = part_o.shape[-1]
        o = np.empty((rows, d), np.float64)
        lse = np.empty(rows, np.float64)
        if self.lib.oracle_merge(part_m, part_l, part_o, rows, C, d, o, lse):
            raise RuntimeError("oracle_merge failed")
        return o, lse

    def attention(self, q, k, v, *, scale, causal=False, seqlens_q=None, seqlens_k=None,
                  rows=None):
        """Naive attention.  q [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d] (fp32 or
        anything numpy widens exactly to fp32).  Returns (o, lse) in fp64,
        shaped [B, Hq, Nq, d] / [B, Hq, Nq], or [len(rows), d] / [len(rows)]
        when ``rows`` (flat query-row ids) is given."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        B, Hq, Nq, d = q.shape
        _, Hkv, Nk, _ = k.shape
        sq = _i32_or_null(seqlens_q)
        sk = _i32_or_null(seqlens_k)
        sel = _i64_or_null(rows)
        nsel = B * Hq * Nq if rows is None else len(sel[1])
        o = np.empty((nsel, d), np.float64)
        lse = np.empty(nsel, np.float64)
        cv = lambda p: None if p is None else ctypes.cast(p[0], ctypes.c_void_p)
        rc = self.lib.oracle_attention(q, k, v, B, Hq, Hkv, Nq, Nk, d, cv(sq), cv(sk),
                                       float(scale), int(bool(causal)), cv(sel), nsel, o, lse)
        if rc:
            raise RuntimeError(f"oracle_attention failed ({rc})")
        if rows is None:
            return o.reshape(B, Hq, Nq, d), lse.reshape(B, Hq, Nq)
        return o, lse

    def merge_lse(self, o_a, lse_a, o_b, lse_b):
        """Log-sum-exp form of the merge of two (o, lse) results."""
        o_a = np.ascontiguousarray(o_a, dtype=np.float64)
        o_b = np.ascontiguousarray(o_b, dtype=np.float64)
        lse_a = np.ascontiguousarray(lse_a, dtype=np.float64)
        lse_b = np.ascontiguousarray(lse_b, dtype=np.float64)
        rows, d = o_a.shape
        o = np.empty((rows, d), np.float64)
        lse = np.empty(rows, np.float64)
        if self.lib.oracle_merge_lse(o_a, lse_a, o_b, lse_b, rows, d, o, lse):
            raise RuntimeError("oracle_merge_lse failed")
        return o, lse


    def attention_bwd(self, q, k, v, dout, *, scale, causal=False, seqlens_q=None,
                      seqlens_k=None):
        """Gradients (dq, dk, dv) in fp64 of attention(q, k, v) against the
        output gradient ``dout`` [B, Hq, Nq, d]; shapes as ``attention``."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        dout = np.ascontiguousarray(dout, dtype=np.float32)
        B, Hq, Nq, d = q.shape
        _, Hkv, Nk, _ = k.shape
        if dout.shape != q.shape:
            raise ValueError("dout must be shaped like q")
        sq = _i32_or_null(seqlens_q)
        sk = _i32_or_null(seqlens_k)
        dq = np.empty((B, Hq, Nq, d), np.float64)
        dk = np.empty((B, Hkv, Nk, d), np.float64)
        dv = np.empty((B, Hkv, Nk, d), np.float64)
        cv = lambda p: None if p is None else ctypes.cast(p[0], ctypes.c_void_p)
        rc = self.lib.oracle_attention_bwd(q, k, v, dout, B, Hq, Hkv, Nq, Nk, d, cv(sq), cv(sk),
                                           float(scale), int(bool(causal)), dq, dk, dv)
        if rc:
            raise RuntimeError(f"oracle_attention_bwd failed ({rc})")
        return dq, dk, dv


_default = None


def load(build_if_missing: bool = True) -> Oracle:
    """The oracle compiled from ``osm_oracle.c`` (compiled here if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or (
                os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE) and build_if_missing):
            if not build_if_missing and not os.path.exists(LIBRARY):
                raise FileNotFoundError(LIBRARY)
            compile_oracle()
        _default = Oracle(LIBRARY)
    return _default
