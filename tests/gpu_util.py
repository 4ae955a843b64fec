"""Helpers for the GPU parity tests: device tensors from the seeded host
inputs, and the tolerance checks against the oracle."""
from __future__ import annotations

import numpy as np

FLT_MIN = 2.0 ** -126


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def torch_mod():
    import torch
    return torch


def dev_f32(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def dev_bf16(bits: np.ndarray):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to("cuda")


def dev_input(a: np.ndarray, dtype: str):
    return dev_bf16(a) if dtype == "bf16" else dev_f32(a)


def dev_i32(a):
    torch = torch_mod()
    return torch.as_tensor(np.asarray(a, np.int32)).to("cuda")


def host(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().to(torch.float64).cpu().numpy()


def host_bits(t) -> np.ndarray:
    """Raw bits of a device tensor (for bit-exactness checks)."""
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


def check_softmax(y, m, l, y_ref, m_ref, l_ref, rtol=1e-5):
    """Elementwise |y - y_ref| <= rtol |y_ref| + FLT_MIN; (m, l) within rtol;
    each row sums to 1 within rtol (rows with any visible entry)."""
    err = np.abs(y - y_ref)
    bad = err > rtol * np.abs(y_ref) + FLT_MIN
    assert not bad.any(), f"softmax: {bad.sum()} bad, worst rel {np.max(err / (np.abs(y_ref) + FLT_MIN))}"
    if m is not None:
        assert np.array_equal(np.isneginf(m), np.isneginf(m_ref))
        fin = np.isfinite(m_ref)
        assert np.all(np.abs(m[fin] - m_ref[fin]) <= rtol * np.abs(m_ref[fin]) + 1e-30)
        assert np.all(np.abs(l - l_ref) <= rtol * np.abs(l_ref)), np.max(np.abs(l - l_ref) / np.maximum(l_ref, 1e-30))
    live = np.isfinite(m_ref) if m_ref is not None else np.ones(len(y), bool)
    assert np.all(np.abs(y[live].sum(1) - 1.0) <= rtol)


def check_attn(o, lse, o_ref, lse_ref, dtype: str):
    """bf16: max |o - o_ref| <= 2e-2, |lse - lse_ref| <= 1e-3, and the
    stricter normwise ||o - o_ref||_F / ||o_ref||_F <= 1e-2.
    fp32: per row max|o - o_ref| <= 1e-5 max|o_ref|, |lse - lse_ref| <= 1e-5 |lse_ref|.
    Rows with no visible key must be exactly o = 0, lse = -inf."""
    o = o.reshape(-1, o.shape[-1])
    o_ref = o_ref.reshape(-1, o_ref.shape[-1])
    lse = lse.reshape(-1)
    lse_ref = lse_ref.reshape(-1)
    dead = np.isneginf(lse_ref)
    assert np.all(np.isneginf(lse[dead])), "fully masked rows must have lse = -inf"
    assert np.all(o[dead] == 0.0), "fully masked rows must be exactly 0"
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "NaN in output"
    live = ~dead
    if not live.any():
        return
    if dtype == "bf16":
        ea = np.abs(o[live] - o_ref[live]).max()
        assert ea <= 2e-2, f"max abs err {ea}"
        el = np.abs(lse[live] - lse_ref[live]).max()
        assert el <= 1e-3, f"lse err {el}"
        nw = np.linalg.norm(o[live] - o_ref[live]) / max(np.linalg.norm(o_ref[live]), 1e-30)
        assert nw <= 1e-2, f"normwise err {nw}"
    else:
        rowmax = np.abs(o_ref[live]).max(1)
        err = np.abs(o[live] - o_ref[live]).max(1)
        assert np.all(err <= 1e-5 * rowmax), f"worst normwise row err {np.max(err / rowmax)}"
        el = np.abs(lse[live] - lse_ref[live])
        assert np.all(el <= 1e-5 * np.abs(lse_ref[live]) + 1e-6), f"lse err {el.max()}"
