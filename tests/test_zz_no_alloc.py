"""osm_attn_decode_splitkv_noalloc (the decode entry point that allocates
nothing: its piece summaries go to the library's per-GPU scratch array)
against osm_attn_decode_splitkv with a caller workspace, through the C ABI:
two calls in a row, the second smaller, each bit-identical to the workspace
call (same kernels), plus the oracle's tolerance on the first."""
import ctypes

import numpy as np
import pytest

import exact_attention_online_softmax_amd as osm
from exact_attention_online_softmax_amd import inputs
from gpu_util import announce, check_attn, dev_i32, dev_input, host, host_bits

pytestmark = pytest.mark.gpu


def _call(lib, noalloc, q, kc, vc, lens, dtype, split, scale):
    torch = __import__("torch")
    B, Hq, d = q.shape
    _, Hkv, Lmax, _ = kc.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    code = osm.OSM_BF16 if dtype == "bf16" else osm.OSM_F32
    if noalloc:
        st = lib.osm_attn_decode_splitkv_noalloc(osm._ptr(q), osm._ptr(kc), osm._ptr(vc), osm._ptr(o),
                                                 osm._ptr(lse), code, B, Hq, Hkv, Lmax, d, osm._ptr(lens),
                                                 float(scale), split, osm._stream())
    else:
        nbytes = lib.osm_decode_workspace_bytes(B, Hq, Lmax, d, split)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        st = lib.osm_attn_decode_splitkv(osm._ptr(q), osm._ptr(kc), osm._ptr(vc), osm._ptr(o), osm._ptr(lse),
                                         code, B, Hq, Hkv, Lmax, d, osm._ptr(lens), float(scale), split,
                                         osm._ptr(ws), ctypes.c_size_t(nbytes), osm._stream())
    assert st == 0, lib.osm_status_str(st)
    torch.cuda.synchronize()
    return o, lse


def _case(inp, split):
    q = dev_input(inp.q[:, :, 0, :], inp.dtype)
    kc = dev_input(inp.k, inp.dtype)
    vc = dev_input(inp.v, inp.dtype)
    return q, kc, vc, dev_i32(inp.seqlens_k)


def test_noalloc_equals_workspace_decode(orc):
    lib = osm.load_library()
    # 1: the measured decode configuration (34 MB of partials in the scratch)
    announce("decode noalloc: B16 Hq32 Hkv8 L<=32768 d128 bf16 split 256")
    inp = inputs.config5()
    q, kc, vc, lens = _case(inp, 256)
    o1, l1 = _call(lib, True, q, kc, vc, lens, "bf16", 256, inp.scale)
    o2, l2 = _call(lib, False, q, kc, vc, lens, "bf16", 256, inp.scale)
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert np.array_equal(host_bits(l1), host_bits(l2))
    qw, kw, vw = inp.widened()
    o_ref, lse_ref = orc.attention(qw, kw, vw, scale=inp.scale, seqlens_k=inp.seqlens_k)
    check_attn(host(o1), host(l1), o_ref[:, :, 0, :], lse_ref[:, :, 0], "bf16")
    del inp, q, kc, vc

    # 2: a smaller call right after it: fp32, head_dim 64, an empty sequence,
    # so the scratch still holds the first call's partials where this one
    # writes none
    announce("decode noalloc: second, smaller call (f32 d64, B3 Hq8 Hkv2 L<=1000 split 64)")
    lens_np = np.array([0, 1000, 517], np.int32)
    inp = inputs.attention_inputs(3, 8, 2, 1, 1000, 64, seed=4242, dtype="f32", seqlens_k=lens_np,
                                  poison=True)
    q, kc, vc, lens = _case(inp, 64)
    o1, l1 = _call(lib, True, q, kc, vc, lens, "f32", 64, inp.scale)
    o2, l2 = _call(lib, False, q, kc, vc, lens, "f32", 64, inp.scale)
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert np.array_equal(host_bits(l1), host_bits(l2))
    qw, kw, vw = inp.widened()
    o_ref, lse_ref = orc.attention(qw, kw, vw, scale=inp.scale, seqlens_k=inp.seqlens_k)
    check_attn(host(o1), host(l1), o_ref[:, :, 0, :], lse_ref[:, :, 0], "f32")
