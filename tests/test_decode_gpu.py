"""osm_attn_decode_splitkv and osm_merge_partials on the GPU against the oracle."""
import numpy as np
import pytest

import exact_attention_online_softmax_amd as osm
from exact_attention_online_softmax_amd import inputs
from gpu_util import announce, check_attn, dev_f32, dev_i32, dev_input, host, host_bits

pytestmark = pytest.mark.gpu


def run_decode(inp, split):
    q = dev_input(inp.q[:, :, 0, :], inp.dtype)
    kc = dev_input(inp.k, inp.dtype)
    vc = dev_input(inp.v, inp.dtype)
    o, lse = osm.attn_decode_splitkv(q, kc, vc, dev_i32(inp.seqlens_k), scale=inp.scale,
                                     split_size=split)
    return o, lse


def oracle_decode(orc, inp):
    q, k, v = inp.widened()
    o, lse = orc.attention(q, k, v, scale=inp.scale, seqlens_k=inp.seqlens_k)
    return o[:, :, 0, :], lse[:, :, 0]


def test_config1_fp32(orc):
    """Single query, q (64,), K, V (4096, 64) fp32, no scale, 64-key pieces."""
    announce("decode config1 fp32 split 64")
    inp = inputs.config1()
    o, lse = run_decode(inp, 64)
    o_ref, lse_ref = oracle_decode(orc, inp)
    check_attn(host(o), host(lse), o_ref, lse_ref, "f32")


def test_config5_full(orc):
    announce("decode config5 bf16 B16 Hq32 Hkv8 L<=32768 split 256")
    inp = inputs.config5()
    o, lse = run_decode(inp, 256)
    o_ref, lse_ref = oracle_decode(orc, inp)
    check_attn(host(o), host(lse), o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("dtype,d,hq,hkv,lmax,lo,hi,split", [
    ("bf16", 128, 8, 2, 1000, 1, 1000, 256),
    ("bf16", 64, 4, 4, 777, 0, 777, 64),
    ("f32", 128, 16, 2, 3000, 100, 3000, 512),
    ("f32", 64, 2, 1, 513, 1, 513, 128),
    ("bf16", 128, 8, 8, 4096, 4096, 4096, 2048),
    ("bf16", 128, 8, 1, 300, 1, 300, 64),
])
def test_shapes(orc, dtype, d, hq, hkv, lmax, lo, hi, split):
    announce(f"decode {dtype} d={d} hq={hq} hkv={hkv} lmax={lmax} split={split}")
    lens = inputs.uniform_lengths(inputs.rng(lmax), 3, lo, hi)
    lens[0], lens[-1] = lo, hi
    inp = inputs.attention_inputs(3, hq, hkv, 1, lmax, d, seed=lmax + d + hq, dtype=dtype,
                                  seqlens_k=lens, poison=True)
    o, lse = run_decode(inp, split)
    o_ref, lse_ref = oracle_decode(orc, inp)
    check_attn(host(o), host(lse), o_ref, lse_ref, dtype)


def test_empty_and_poison_bit_invariance(orc):
    """L_b = 0 gives 0 / -inf; NaN in the cache past L_b gives outputs
    bit-identical to zeros there."""
    announce("decode poison invariance and L=0")
    lens = np.array([0, 1, 700, 1500], np.int32)
    inp = inputs.attention_inputs(4, 8, 2, 1, 1500, 128, seed=77, seqlens_k=lens, poison=True)
    o1, l1 = run_decode(inp, 256)
    zk, zv = inp.k.copy(), inp.v.copy()
    for b, L in enumerate(inp.seqlens_k):
        zk[b, :, L:] = 0
        zv[b, :, L:] = 0
    inp2 = inputs.AttnInputs(inp.q, zk, zv, inp.dtype, None, inp.seqlens_k, inp.scale, False)
    o2, l2 = run_decode(inp2, 256)
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert np.array_equal(host_bits(l1), host_bits(l2))
    oh, lh = host(o1), host(l1)
    assert np.all(oh[0] == 0.0) and np.all(np.isneginf(lh[0]))
    o_ref, lse_ref = oracle_decode(orc, inp)
    check_attn(oh, lh, o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("rows,C,d", [(7, 1, 64), (64, 33, 128), (5, 700, 200), (3, 1, 1),
                                    (16, 128, 128), (9, 129, 64)])
def test_merge_standalone(orc, rows, C, d):
    announce(f"merge rows={rows} C={C} d={d}")
    pm, pl, po = inputs.random_partials(rows, C, d, seed=rows + C + d)
    # empty pieces hold garbage that must never be read
    po[np.isneginf(pm)] = np.nan
    pl[np.isneginf(pm)] = np.nan
    pm[0, :] = -np.inf                       # a row of empty pieces only
    o, lse = osm.merge_partials(dev_f32(pm), dev_f32(pl), dev_f32(po))
    o_ref, lse_ref = orc.merge(pm, pl, po)
    oh, lh = host(o), host(lse)
    assert np.all(oh[0] == 0.0) and np.isneginf(lh[0])
    live = np.isfinite(lse_ref)
    rowmax = np.abs(o_ref[live]).max(1)
    assert np.all(np.abs(oh[live] - o_ref[live]).max(1) <= 1e-5 * rowmax)
    assert np.all(np.abs(lh[live] - lse_ref[live]) <= 1e-5 * np.abs(lse_ref[live]) + 1e-6)


def test_merge_bf16_out(orc):
    announce("merge bf16 out")
    import torch
    pm, pl, po = inputs.random_partials(32, 16, 128, seed=5)
    o, lse = osm.merge_partials(dev_f32(pm), dev_f32(pl), dev_f32(po), out_dtype=torch.bfloat16)
    o_ref, lse_ref = orc.merge(pm, pl, po)
    assert np.abs(host(o) - o_ref).max() <= 2e-2
    assert np.abs(host(lse) - lse_ref).max() <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_every_split_instantiation(orc, dtype, d, group):
    """Each (element type, head_dim, heads per KV head) instantiation of the
    piece kernel, through decode (ragged lengths, NaN past them, an empty
    sequence, 192-key pieces so the last piece of a row is partial) and
    through extend (two chunks into a fresh state, 128-key pieces)."""
    announce(f"decode/extend instantiation {dtype} d={d} group={group}")
    hkv = 2
    hq = hkv * group
    lens = np.array([0, 1, 333, 700], np.int32)
    inp = inputs.attention_inputs(4, hq, hkv, 1, 700, d, seed=900 + 10 * d + group + (dtype == "f32"),
                                  dtype=dtype, seqlens_k=lens, poison=True)
    o, lse = run_decode(inp, 192)
    o_ref, lse_ref = oracle_decode(orc, inp)
    check_attn(host(o), host(lse), o_ref, lse_ref, dtype)

    torch = __import__("torch")
    e_inp = inputs.attention_inputs(2, hq, hkv, 1, 450, d, seed=950 + 10 * d + group, dtype=dtype)
    q = dev_input(e_inp.q[:, :, 0, :], dtype)
    k = dev_input(e_inp.k, dtype)
    v = dev_input(e_inp.v, dtype)
    state = osm.attn_state(2, hq, d)
    osm.attn_extend(q, k[:, :, :130].contiguous(), v[:, :, :130].contiguous(), state, scale=e_inp.scale,
                    split_size=128)
    osm.attn_extend(q, k[:, :, 130:].contiguous(), v[:, :, 130:].contiguous(), state, scale=e_inp.scale,
                    split_size=128)
    oe, le = osm.attn_state_finalize(state)
    torch.cuda.synchronize()
    qw, kw, vw = e_inp.widened()
    oe_ref, le_ref = orc.attention(qw, kw, vw, scale=e_inp.scale)
    check_attn(host(oe), host(le), oe_ref.reshape(-1, d), le_ref.reshape(-1), dtype)


def test_random_sweep(orc):
    """Seeded random decode configurations against the oracle: element type,
    head dim, GQA group, cache length, per-sequence lengths (0 included),
    piece size, NaN poison past the lengths."""
    g = inputs.rng(4343)
    for case in range(40):
        dtype = str(g.choice(["bf16", "f32"]))
        d = int(g.choice([64, 128]))
        group = int(g.choice([1, 2, 4, 8]))
        hkv = int(g.choice([1, 2, 4]))
        B = int(g.integers(1, 5))
        lmax = int(g.integers(1, 3000))
        split = 64 * int(g.integers(1, 1 + min(128, 16384 // (64 * group))))
        lens = g.integers(0, lmax + 1, size=B).astype(np.int32)
        announce(f"decode sweep {case}: {dtype} d={d} B={B} hq={hkv * group} hkv={hkv} lmax={lmax} "
                 f"split={split} lens={lens.tolist()}")
        inp = inputs.attention_inputs(B, hkv * group, hkv, 1, lmax, d, seed=6000 + case, dtype=dtype,
                                      seqlens_k=lens, poison=True)
        o, lse = run_decode(inp, split)
        o_ref, lse_ref = oracle_decode(orc, inp)
        check_attn(host(o), host(lse), o_ref, lse_ref, dtype)
