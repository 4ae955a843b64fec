"""osm_attn_extend (streaming attention over arriving keys) on the GPU: the
finalized state after every chunk equals the oracle's attention over all the
keys seen so far."""
import numpy as np
import pytest

import exact_attention_online_softmax_amd as osm
from exact_attention_online_softmax_amd import inputs
from gpu_util import announce, check_attn, dev_i32, dev_input, host, host_bits, torch_mod

pytestmark = pytest.mark.gpu


def stream(orc, B, Hq, Hkv, d, dtype, chunks, seed, split=64, check_every=True):
    total = int(sum(chunks))
    inp = inputs.attention_inputs(B, Hq, Hkv, 1, max(total, 1), d, seed, dtype=dtype)
    q = dev_input(inp.q[:, :, 0, :], dtype)
    k = dev_input(inp.k, dtype)
    v = dev_input(inp.v, dtype)
    state = osm.attn_state(B, Hq, d)
    qw, kw, vw = inp.widened()
    seen = 0
    for i, n in enumerate(chunks):
        osm.attn_extend(q, k[:, :, seen:seen + n].contiguous(), v[:, :, seen:seen + n].contiguous(),
                        state, scale=inp.scale, split_size=split)
        seen += n
        if check_every or i == len(chunks) - 1:
            o, lse = osm.attn_state_finalize(state)
            o_ref, lse_ref = orc.attention(qw, kw[:, :, :seen], vw[:, :, :seen], scale=inp.scale)
            check_attn(host(o), host(lse), o_ref.reshape(-1, d), lse_ref.reshape(-1), "f32" if dtype == "f32" else "bf16")
    return state


@pytest.mark.parametrize("B,Hq,Hkv,d,dtype,chunks", [
    (2, 8, 2, 128, "bf16", [100, 1, 300, 64, 700]),
    (1, 4, 4, 64, "f32", [1, 1, 2, 511, 129]),
    (3, 8, 1, 128, "f32", [64, 64, 1000]),
    (2, 16, 2, 64, "bf16", [333, 4096]),
])
def test_stream_equals_attention(orc, B, Hq, Hkv, d, dtype, chunks):
    announce(f"extend B{B} Hq{Hq} Hkv{Hkv} d{d} {dtype} chunks {chunks}")
    stream(orc, B, Hq, Hkv, d, dtype, chunks, 5000 + sum(chunks))


def test_empty_chunk_keeps_state(orc):
    announce("extend with no new keys leaves the state unchanged")
    torch = torch_mod()
    state = stream(orc, 1, 4, 2, 128, "bf16", [200], 5100)
    before = [host_bits(t).copy() for t in state]
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    osm.attn_extend(q, kv, kv, state)
    torch.cuda.synchronize()
    for a, t in zip(before, state):
        assert np.array_equal(a, host_bits(t))


def test_fresh_state_equals_split_decode(orc):
    """One chunk into a fresh state, finalized, is the split decode of that
    chunk bit for bit (same pieces, same merge)."""
    announce("extend from the empty set equals osm_attn_decode_splitkv")
    inp = inputs.attention_inputs(2, 8, 2, 1, 777, 128, 5200, dtype="bf16")
    q = dev_input(inp.q[:, :, 0, :], "bf16")
    k = dev_input(inp.k, "bf16")
    v = dev_input(inp.v, "bf16")
    state = osm.attn_state(2, 8, 128)
    osm.attn_extend(q, k, v, state, scale=inp.scale, split_size=128)
    o_s, lse_s = osm.attn_state_finalize(state, out_dtype=q.dtype)
    o_d, lse_d = osm.attn_decode_splitkv(q, k, v, dev_i32(np.full(2, 777, np.int32)), scale=inp.scale,
                                         split_size=128)
    assert np.array_equal(host_bits(o_s.reshape(o_d.shape)), host_bits(o_d))
    assert np.array_equal(host_bits(lse_s.reshape(lse_d.shape)), host_bits(lse_d))


def test_bench_shape_sampled(orc):
    """The measured shape and launch configuration: B16 Hq32 Hkv8 d128 bf16,
    four chunks of 4096 keys, 512-key pieces."""
    announce("extend B16 Hq32 Hkv8 d128 bf16, 4 x 4096 keys, split 512")
    stream(orc, 16, 32, 8, 128, "bf16", [4096] * 4, 5300, split=512, check_every=False)


def test_random_sweep(orc):
    """Seeded random streams: element type, head dim, group, chunk sizes
    (1 key to several pieces), piece size; the finalized state checked after
    the last chunk of each stream."""
    g = inputs.rng(4747)
    for case in range(16):
        dtype = str(g.choice(["bf16", "f32"]))
        d = int(g.choice([64, 128]))
        group = int(g.choice([1, 2, 4, 8]))
        Hkv = int(g.choice([1, 2]))
        B = int(g.integers(1, 4))
        chunks = [int(g.integers(1, 900)) for _ in range(int(g.integers(1, 6)))]
        split = 64 * int(g.integers(1, 1 + min(16, 16384 // (64 * group))))
        announce(f"extend sweep {case}: {dtype} d={d} B={B} Hq={Hkv * group} Hkv={Hkv} chunks={chunks} split={split}")
        stream(orc, B, Hkv * group, Hkv, d, dtype, chunks, 9500 + case, split=split, check_every=False)
