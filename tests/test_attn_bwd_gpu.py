"""osm_attn_bwd on the GPU against the oracle's gradients: element by
element on small ragged shapes (several tiles, ragged tails, grouped
heads, padding with NaN poison, empty lengths), whole heads at the full
benchmark sizes, the longest key sequences the ABI accepts, and the
bit-exact causal and padding properties; head dims 128 and 64.

The forward that feeds the backward is the GPU forward (its O and LSE), as
in use; the oracle differentiates the exact forward of the same bf16 inputs.

Tolerance (bf16, per gradient tensor): normwise ||g - g_ref||_F /
||g_ref||_F <= 1e-2 and max |g - g_ref| <= 2e-2 max |g_ref|.  An fp32
emulation of this arithmetic (P and dS rounded to bf16 as matrix operands,
O and the gradients rounded to bf16) measured normwise 2.4e-3 and at most
9e-3 max |g_ref| on such inputs."""
import numpy as np
import pytest

import exact_attention_online_softmax_amd as osm
from exact_attention_online_softmax_amd import inputs
from gpu_util import announce, dev_bf16, dev_i32, host, host_bits

pytestmark = pytest.mark.gpu


def run(inp, do_bits):
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    sq = None if inp.seqlens_q is None else dev_i32(inp.seqlens_q)
    sk = None if inp.seqlens_k is None else dev_i32(inp.seqlens_k)
    o, lse = osm.attn_fwd(q, k, v, scale=inp.scale, causal=inp.causal, seqlens_q=sq, seqlens_k=sk)
    return osm.attn_bwd(q, k, v, o, lse, dev_bf16(do_bits), scale=inp.scale, causal=inp.causal,
                        seqlens_q=sq, seqlens_k=sk)


def oracle(orc, inp, do_bits):
    q, k, v = inp.widened()
    return orc.attention_bwd(q, k, v, inputs.bf16_bits_to_f32(do_bits), scale=inp.scale,
                             causal=inp.causal, seqlens_q=inp.seqlens_q, seqlens_k=inp.seqlens_k)


def check_grad(g, ref, what):
    assert not np.isnan(g).any(), f"{what}: NaN"
    if not np.any(ref):
        # zero by cancellation, not by masking (one visible key: dS = dP - D
        # = 0): D = dO . O is summed in another order than dP, so fp32
        # rounding residue remains.  Masked and padded rows are checked to be
        # exactly zero by the tests that make them.
        assert np.abs(g).max() <= 1e-4, f"{what}: {np.abs(g).max()} where the gradient is 0"
        return
    err = np.abs(g - ref)
    top = np.abs(ref).max()
    assert err.max() <= 2e-2 * top, f"{what}: max err {err.max()} vs max |ref| {top}"
    nw = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    assert nw <= 1e-2, f"{what}: normwise err {nw}"


def check_all(got, ref, tag):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        check_grad(host(g), r, f"{tag} {name}")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,causal", [
    (1, 2, 1, 300, 300, False),
    (1, 2, 1, 300, 300, True),
    (2, 4, 2, 129, 517, False),
    (1, 2, 2, 517, 129, True),
    (1, 8, 1, 257, 257, False),
    (1, 1, 1, 1, 1, False),
    (1, 1, 1, 1, 64, True),
    (1, 2, 2, 640, 640, True),
])
def test_small(orc, B, Hq, Hkv, Nq, Nk, causal, d):
    announce(f"bwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    seed = 7000 + B * 1000 + Nq + Nk + (d == 64)
    inp = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, d, seed=seed, causal=causal)
    do = inputs.output_grad(B, Hq, Nq, d, seed + 1)
    check_all(run(inp, do), oracle(orc, inp, do), "small")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_poisoned(orc, causal, d):
    """Right padding with NaN in q, k, v and dO past the lengths: gradients
    match, padded rows are exactly 0, and the result is bit-identical to
    zero padding."""
    announce(f"bwd varlen poisoned d={d} causal={causal}")
    B, H, N = 4, 2, 400
    lens = np.array([1, 130, 257, 400], np.int32)
    inp = inputs.attention_inputs(B, H, H, N, N, d, seed=61, causal=causal, seqlens_q=lens,
                                  seqlens_k=lens, poison=True)
    do = inputs.output_grad(B, H, N, d, 62, seqlens_q=lens, poison=True)
    got = run(inp, do)
    check_all(got, oracle(orc, inp, do), "varlen")
    for g in got:
        gh = host(g)
        for b, L in enumerate(lens):
            assert np.all(gh[b, :, L:] == 0.0)
    clean = []
    for a in (inp.q, inp.k, inp.v, do):
        f = inputs.bf16_bits_to_f32(a).copy()
        f[np.isnan(f)] = 0.0
        clean.append(inputs.to_bf16_bits(f))
    inp0 = inputs.AttnInputs(clean[0], clean[1], clean[2], "bf16", lens, lens, inp.scale, causal)
    for g, g0 in zip(got, run(inp0, clean[3])):
        assert np.array_equal(host_bits(g), host_bits(g0))


@pytest.mark.parametrize("d", [128, 64])
def test_empty_lengths(orc, d):
    """A batch with no valid query and one with no valid key: their
    gradients are exactly zero; the others match."""
    announce(f"bwd empty lengths d={d}")
    sq = np.array([0, 150, 90], np.int32)
    sk = np.array([200, 0, 37], np.int32)
    inp = inputs.attention_inputs(3, 4, 2, 150, 200, d, seed=63, seqlens_q=sq, seqlens_k=sk,
                                  poison=True)
    do = inputs.output_grad(3, 4, 150, d, 64, seqlens_q=sq, poison=True)
    got = run(inp, do)
    check_all(got, oracle(orc, inp, do), "empty")
    dq, dk, dv = (host(g) for g in got)
    assert not dq[0].any() and not dk[1].any() and not dv[1].any() and not dq[1].any()


@pytest.mark.parametrize("d", [128, 64])
def test_causal_locality(d):
    """Causal: dQ of rows before 200 does not depend on keys from 200 on, and
    dK, dV of keys from 200 on do not depend on queries before 200 (bit for
    bit)."""
    announce(f"bwd causal locality d={d}")
    inp = inputs.attention_inputs(1, 2, 2, 512, 512, d, seed=65, causal=True)
    do = inputs.output_grad(1, 2, 512, d, 66)
    dq1, dk1, dv1 = run(inp, do)
    k2, v2 = inp.k.copy(), inp.v.copy()
    k2[:, :, 200:] = inputs.to_bf16_bits(np.full(k2[:, :, 200:].shape, 0.5, np.float32))
    v2[:, :, 200:] = inputs.to_bf16_bits(np.full(v2[:, :, 200:].shape, -3.0, np.float32))
    dq2, _, _ = run(inputs.AttnInputs(inp.q, k2, v2, "bf16", None, None, inp.scale, True), do)
    assert np.array_equal(host_bits(dq1)[:, :, :200], host_bits(dq2)[:, :, :200])
    assert not np.array_equal(host_bits(dq1)[:, :, 200:], host_bits(dq2)[:, :, 200:])
    q3, do3 = inp.q.copy(), do.copy()
    q3[:, :, :200] = inputs.to_bf16_bits(np.full(q3[:, :, :200].shape, 0.25, np.float32))
    do3[:, :, :200] = inputs.to_bf16_bits(np.full(do3[:, :, :200].shape, 2.0, np.float32))
    _, dk3, dv3 = run(inputs.AttnInputs(q3, inp.k, inp.v, "bf16", None, None, inp.scale, True), do3)
    assert np.array_equal(host_bits(dk1)[:, :, 200:], host_bits(dk3)[:, :, 200:])
    assert np.array_equal(host_bits(dv1)[:, :, 200:], host_bits(dv3)[:, :, 200:])


@pytest.mark.parametrize("d", [128, 64])
def test_deterministic(d):
    announce(f"bwd deterministic d={d}")
    inp = inputs.attention_inputs(2, 4, 1, 333, 333, d, seed=67, causal=True)
    do = inputs.output_grad(2, 4, 333, d, 68)
    a, b = run(inp, do), run(inp, do)
    for x, y in zip(a, b):
        assert np.array_equal(host_bits(x), host_bits(y))


def _head_slice(inp, do, b, heads):
    """The inputs of query heads `heads` of batch b (one kv head each)."""
    sl = (slice(b, b + 1), heads)
    sq = None if inp.seqlens_q is None else inp.seqlens_q[b:b + 1]
    sk = None if inp.seqlens_k is None else inp.seqlens_k[b:b + 1]
    sub = inputs.AttnInputs(inp.q[sl], inp.k[sl], inp.v[sl], "bf16", sq, sk, inp.scale, inp.causal)
    return sub, do[sl]


def test_full_size_heads(orc):
    """B4 H32 N4096 d128 non-causal (the forward's benchmark shape): two
    whole heads of every gradient against the oracle."""
    announce("bwd B4 H32 N4096 full size, two heads")
    inp = inputs.config3()
    do = inputs.output_grad(4, 32, 4096, 128, inputs.SEED_BASE + 8)
    dq, dk, dv = run(inp, do)
    heads = [5, 30]
    sub, dsub = _head_slice(inp, do, 2, heads)
    ref = oracle(orc, sub, dsub)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(host(g[2:3, heads]), r, f"full {name}")
    for g in (dq, dk, dv):
        assert not np.isnan(host(g)).any()


def test_full_size_causal_varlen_heads(orc):
    """B8 H16 N8192 causal with right padding and NaN poison: two whole heads
    (of the two shortest sequences) against the oracle; padded rows zero."""
    announce("bwd B8 H16 N8192 causal varlen full size, two heads")
    inp = inputs.config4()
    lens = inp.seqlens_q
    do = inputs.output_grad(8, 16, 8192, 128, inputs.SEED_BASE + 9, seqlens_q=lens, poison=True)
    dq, dk, dv = run(inp, do)
    for b in np.argsort(lens)[:2]:
        sub, dsub = _head_slice(inp, do, int(b), [3])
        ref = oracle(orc, sub, dsub)
        for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            check_grad(host(g[b:b + 1, [3]]), r, f"causal full b={b} {name}")
    for g in (dq, dk, dv):
        gh = host(g)
        assert not np.isnan(gh).any()
        for b, L in enumerate(lens):
            assert np.all(gh[b, :, L:] == 0.0)


def test_full_size_heads_d64(orc):
    """B4 H64 N4096 d64 non-causal (the head-dim-64 forward's benchmark
    shape): two whole heads of every gradient against the oracle."""
    announce("bwd B4 H64 N4096 d64 full size, two heads")
    inp = inputs.attention_inputs(4, 64, 64, 4096, 4096, 64, seed=inputs.SEED_BASE + 11)
    do = inputs.output_grad(4, 64, 4096, 64, inputs.SEED_BASE + 12)
    dq, dk, dv = run(inp, do)
    heads = [0, 63]
    sub, dsub = _head_slice(inp, do, 3, heads)
    ref = oracle(orc, sub, dsub)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(host(g[3:4, heads]), r, f"full d64 {name}")
    for g in (dq, dk, dv):
        assert not np.isnan(host(g)).any()


@pytest.mark.parametrize("d,seed0,cases", [(128, 4545, 20), (64, 4546, 12)])
def test_random_sweep(orc, d, seed0, cases):
    """Seeded random configurations against the oracle's gradients: GQA
    group, ragged lengths, masks, scale, NaN-poisoned padding."""
    g = inputs.rng(seed0)
    for case in range(cases):
        B = int(g.integers(1, 3))
        Hkv = int(g.choice([1, 2]))
        Hq = Hkv * int(g.choice([1, 2, 4]))
        Nq = int(g.integers(1, 400))
        Nk = int(g.integers(1, 400))
        causal = bool(g.random() < 0.5)
        mode = int(g.integers(0, 3))
        sq = sk = None
        if mode >= 1:
            sk = g.integers(1, Nk + 1, size=B).astype(np.int32)
        if mode == 2:
            sq = g.integers(1, Nq + 1, size=B).astype(np.int32)
        scale = float(g.uniform(0.03, 0.12))
        announce(f"bwd sweep d={d} {case}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} "
                 f"seqlens_q={None if sq is None else sq.tolist()} seqlens_k={None if sk is None else sk.tolist()}")
        seed = 9000 + case + (100 if d == 64 else 0)
        inp = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, d, seed=seed, causal=causal, scale=scale,
                                      seqlens_q=sq, seqlens_k=sk, poison=sk is not None)
        do = inputs.output_grad(B, Hq, Nq, d, seed + 1, seqlens_q=sq, poison=sq is not None)
        check_all(run(inp, do), oracle(orc, inp, do), f"sweep d={d} {case}")


@pytest.mark.parametrize("d,Nk", [(128, (1 << 23) - 1), (64, (1 << 24) - 1)])
def test_max_key_length_and_head_offsets(orc, d, Nk):
    """The longest key sequence the backward accepts at each head dim (one
    head's K just under 2 GiB, a ragged last key block), on three KV heads,
    so that the last head starts 4 GiB into K, V, dK and dV; GQA 2:1, four
    queries.  dQ of the last query head and sampled dK, dV rows of the last
    KV head (both of its query heads summed) against the oracle; every
    gradient finite."""
    import torch
    B, Hq, Hkv, Nq = 1, 6, 3, 4
    announce(f"bwd max key length B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d}")
    ktab, kidx = inputs.tiled_rows(Hkv * Nk, d, seed=inputs.SEED_BASE + 71 + d)
    vtab, vidx = inputs.tiled_rows(Hkv * Nk, d, seed=inputs.SEED_BASE + 72 + d)
    qbits = inputs.to_bf16_bits(inputs.normal_f32(inputs.rng(inputs.SEED_BASE + 73 + d), (B, Hq, Nq, d)))
    dobits = inputs.output_grad(B, Hq, Nq, d, inputs.SEED_BASE + 74 + d)
    k = dev_bf16(ktab)[torch.from_numpy(kidx).to("cuda")].view(B, Hkv, Nk, d)
    v = dev_bf16(vtab)[torch.from_numpy(vidx).to("cuda")].view(B, Hkv, Nk, d)
    q, do = dev_bf16(qbits), dev_bf16(dobits)
    scale = 1.0 / np.sqrt(d)
    o, lse = osm.attn_fwd(q, k, v, scale=scale)
    dq, dk, dv = osm.attn_bwd(q, k, v, o, lse, do, scale=scale)
    g = Hkv - 1                          # the last KV head and its query heads
    heads = [2 * g, 2 * g + 1]
    keys = np.array([0, 1, 31, 256, 1 << 20, Nk // 2 + 5, Nk - 2, Nk - 1])
    dqh = host(dq[0, heads])
    dkh = host(dk[0, g, torch.from_numpy(keys).to("cuda")])
    dvh = host(dv[0, g, torch.from_numpy(keys).to("cuda")])
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all().item()
    del k, v, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    sel = slice(g * Nk, (g + 1) * Nk)
    kh = inputs.bf16_bits_to_f32(ktab)[kidx[sel]][None, None]
    vh = inputs.bf16_bits_to_f32(vtab)[vidx[sel]][None, None]
    qh = inputs.bf16_bits_to_f32(qbits[:, heads])
    doh = inputs.bf16_bits_to_f32(dobits[:, heads])
    dq_ref, dk_ref, dv_ref = orc.attention_bwd(qh, kh, vh, doh, scale=scale)
    del kh, vh
    check_grad(dqh, dq_ref[0], f"max keys d={d} dq")
    check_grad(dkh, dk_ref[0, 0, keys], f"max keys d={d} dk")
    check_grad(dvh, dv_ref[0, 0, keys], f"max keys d={d} dv")


@pytest.mark.parametrize("d,Nq", [(128, (1 << 23) - 1), (64, (1 << 24) - 1)])
def test_max_query_length_and_head_offsets(orc, d, Nq):
    """The longest query sequence the ABI accepts at each head dim, on three
    query heads (the last starts 4 GiB into Q, O, dO and dQ), five keys, no
    GQA.  The forward runs on its persistent grid (more blocks than compute
    units); sampled O, LSE and dQ rows of the last head and all of its dK and
    dV rows (sums over every query) against the oracle; every output finite."""
    import torch
    B, Hq, Hkv, Nk = 1, 3, 3, 5
    announce(f"fwd+bwd max query length B={B} Hq={Hq} Nq={Nq} Nk={Nk} d={d}")
    qtab, qidx = inputs.tiled_rows(Hq * Nq, d, seed=inputs.SEED_BASE + 81 + d)
    gtab, gidx = inputs.tiled_rows(Hq * Nq, d, seed=inputs.SEED_BASE + 82 + d)
    kbits = inputs.to_bf16_bits(inputs.normal_f32(inputs.rng(inputs.SEED_BASE + 83 + d), (B, Hkv, Nk, d)))
    vbits = inputs.to_bf16_bits(inputs.normal_f32(inputs.rng(inputs.SEED_BASE + 84 + d), (B, Hkv, Nk, d)))
    q = dev_bf16(qtab)[torch.from_numpy(qidx).to("cuda")].view(B, Hq, Nq, d)
    do = dev_bf16(gtab)[torch.from_numpy(gidx).to("cuda")].view(B, Hq, Nq, d)
    k, v = dev_bf16(kbits), dev_bf16(vbits)
    scale = 1.0 / np.sqrt(d)
    o, lse = osm.attn_fwd(q, k, v, scale=scale)
    dq, dk, dv = osm.attn_bwd(q, k, v, o, lse, do, scale=scale)
    h = Hq - 1
    rows = np.array([0, 1, 255, 256, 1 << 20, Nq // 2 + 3, Nq - 2, Nq - 1])
    ridx = torch.from_numpy(rows).to("cuda")
    oh, lh, dqh = host(o[0, h, ridx]), host(lse[0, h, ridx]), host(dq[0, h, ridx])
    dkh, dvh = host(dk[0, h]), host(dv[0, h])
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t.float()).all().item()
    del q, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    sel = slice(h * Nq, (h + 1) * Nq)
    qh = inputs.bf16_bits_to_f32(qtab)[qidx[sel]][None, None]
    doh = inputs.bf16_bits_to_f32(gtab)[gidx[sel]][None, None]
    kh = inputs.bf16_bits_to_f32(kbits[:, h:h + 1])
    vh = inputs.bf16_bits_to_f32(vbits[:, h:h + 1])
    o_ref, lse_ref = orc.attention(np.ascontiguousarray(qh[:, :, rows]), kh, vh, scale=scale)
    assert np.abs(oh - o_ref[0, 0]).max() <= 2e-2
    assert np.abs(lh - lse_ref[0, 0]).max() <= 1e-3
    dq_ref, dk_ref, dv_ref = orc.attention_bwd(qh, kh, vh, doh, scale=scale)
    del qh, doh
    check_grad(dqh, dq_ref[0, 0, rows], f"max queries d={d} dq")
    check_grad(dkh, dk_ref[0, 0], f"max queries d={d} dk")
    check_grad(dvh, dv_ref[0, 0], f"max queries d={d} dv")
