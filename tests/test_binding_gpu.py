"""The Python binding refuses, before any launch, caller-supplied outputs,
workspaces and operands whose shape, dtype or device does not match what the
kernels will write or read through their pointers (the C ABI sees only
pointers and sizes and cannot tell)."""
import pytest
import torch

import exact_attention_online_softmax_amd as osm
from gpu_util import announce

pytestmark = pytest.mark.gpu


def _bf16(*shape):
    return torch.randn(*shape, device="cuda").to(torch.bfloat16)


def test_forward_outputs():
    announce("binding: forward outputs")
    q, k, v = _bf16(1, 2, 64, 128), _bf16(1, 2, 64, 128), _bf16(1, 2, 64, 128)
    with pytest.raises(ValueError, match="out must have shape"):
        osm.attn_fwd(q, k, v, out=_bf16(1, 2, 63, 128))
    with pytest.raises(TypeError):
        osm.attn_fwd(q, k, v, lse=torch.empty(1, 2, 64, device="cuda", dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be on the GPU"):
        osm.attn_fwd(q, k, v, lse=torch.empty(1, 2, 64))
    with pytest.raises(ValueError, match="contiguous"):
        osm.attn_fwd(q, k, v, out=_bf16(1, 2, 128, 64).transpose(2, 3))
    q8 = torch.zeros(1, 2, 64, 128, dtype=torch.uint8, device="cuda")
    with pytest.raises(TypeError):
        osm.attn_fwd_fp8(q8, q8, q8, out=torch.empty(1, 2, 64, 128, device="cuda"))


def test_backward_outputs_and_workspace():
    announce("binding: backward outputs and workspace")
    q, k, v = _bf16(1, 4, 64, 64), _bf16(1, 2, 64, 64), _bf16(1, 2, 64, 64)
    o, lse = osm.attn_fwd(q, k, v)
    do = _bf16(1, 4, 64, 64)
    with pytest.raises(ValueError, match="dk must have shape"):
        osm.attn_bwd(q, k, v, o, lse, do, dk=_bf16(1, 4, 64, 64))
    with pytest.raises(ValueError, match="must be on the GPU"):
        osm.attn_bwd(q, k, v, o, lse, do, workspace=torch.empty(1 << 16, dtype=torch.uint8))
    with pytest.raises(TypeError):
        osm.attn_bwd(q, k, v, o, lse, do, workspace=torch.empty(1 << 14, device="cuda"))
    torch.cuda.synchronize()


def test_decode_and_extend_shapes():
    announce("binding: decode and extend shapes")
    q = _bf16(2, 4, 128)
    kc = _bf16(2, 2, 300, 64)
    lens = torch.tensor([300, 200], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="batch and head_dim"):
        osm.attn_decode_splitkv(q, kc, kc, lens)
    kc = _bf16(2, 2, 300, 128)
    with pytest.raises(ValueError, match="lse must have shape"):
        osm.attn_decode_splitkv(q, kc, kc, lens, lse=torch.empty(2, 3, device="cuda"))
    st = osm.attn_state(2, 4, 128)
    with pytest.raises(ValueError, match="batch and head_dim"):
        osm.attn_extend(q, _bf16(1, 2, 100, 128), _bf16(1, 2, 100, 128), st)
    with pytest.raises(ValueError, match="state_o must have shape"):
        osm.attn_extend(q, _bf16(2, 2, 100, 128), _bf16(2, 2, 100, 128), osm.attn_state(2, 4, 64))
    with pytest.raises(TypeError):
        osm.attn_extend(q, _bf16(2, 2, 100, 128), torch.randn(2, 2, 100, 128, device="cuda"), st)


def test_merge_lse_outputs():
    announce("binding: merge_lse outputs")
    op = torch.randn(3, 10, 128, device="cuda")
    lp = torch.randn(3, 10, device="cuda")
    with pytest.raises(ValueError, match="out must have shape"):
        osm.merge_lse(op, lp, out=torch.empty(10, 64, device="cuda"))
    with pytest.raises(TypeError):
        osm.merge_lse(op, lp, out_dtype=torch.bfloat16, out=torch.empty(10, 128, device="cuda"))
