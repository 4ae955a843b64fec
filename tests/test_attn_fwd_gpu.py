"""osm_attn_fwd on the GPU against the oracle: element by element on small
ragged shapes, sampled rows at the full benchmark sizes, and the bit-exact
mask properties."""
import numpy as np
import pytest

import exact_attention_online_softmax_amd as osm
from exact_attention_online_softmax_amd import inputs
from gpu_util import announce, check_attn, dev_bf16, dev_i32, host, host_bits, torch_mod

pytestmark = pytest.mark.gpu


def run(inp):
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    sq = None if inp.seqlens_q is None else dev_i32(inp.seqlens_q)
    sk = None if inp.seqlens_k is None else dev_i32(inp.seqlens_k)
    return osm.attn_fwd(q, k, v, scale=inp.scale, causal=inp.causal, seqlens_q=sq, seqlens_k=sk)


def oracle(orc, inp, rows=None):
    q, k, v = inp.widened()
    return orc.attention(q, k, v, scale=inp.scale, causal=inp.causal, seqlens_q=inp.seqlens_q,
                         seqlens_k=inp.seqlens_k, rows=rows)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,causal", [
    (2, 4, 2, 300, 300, False),
    (2, 4, 2, 300, 300, True),
    (1, 2, 1, 129, 517, False),
    (1, 2, 2, 1, 1, False),
    (1, 1, 1, 1, 64, True),
    (3, 8, 1, 64, 200, False),
    (1, 2, 2, 640, 640, True),
])
def test_small(orc, B, Hq, Hkv, Nq, Nk, causal):
    announce(f"fwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal}")
    inp = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, 128, seed=B * 1000 + Nq + Nk, causal=causal)
    o, lse = run(inp)
    o_ref, lse_ref = oracle(orc, inp)
    check_attn(host(o), host(lse), o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_poisoned(orc, causal):
    announce(f"fwd varlen poisoned causal={causal}")
    B, H, N = 4, 2, 400
    lens = np.array([1, 130, 257, 400], np.int32)
    inp = inputs.attention_inputs(B, H, H, N, N, 128, seed=31, causal=causal, seqlens_q=lens,
                                  seqlens_k=lens, poison=True)
    o, lse = run(inp)
    o_ref, lse_ref = oracle(orc, inp)
    oh, lh = host(o), host(lse)
    check_attn(oh, lh, o_ref, lse_ref, "bf16")
    for b, L in enumerate(lens):       # padded query rows: exactly 0 / -inf
        assert np.all(oh[b, :, L:] == 0.0) and np.all(np.isneginf(lh[b, :, L:]))
    # zero padding instead of NaN: bit-identical outputs
    zq, zk, zv = (inputs.bf16_bits_to_f32(a).copy() for a in (inp.q, inp.k, inp.v))
    for a in (zq, zk, zv):
        a[np.isnan(a)] = 0.0
    inp0 = inputs.AttnInputs(inputs.to_bf16_bits(zq), inputs.to_bf16_bits(zk), inputs.to_bf16_bits(zv),
                             "bf16", lens, lens, inp.scale, causal)
    o0, l0 = run(inp0)
    assert np.array_equal(host_bits(o), host_bits(o0))
    assert np.array_equal(host_bits(lse), host_bits(l0))


def test_seqlens_q_null_keys_padded(orc):
    """Only keys padded (seqlens_q NULL): every query row attends to the
    valid keys; Lk = 0 gives 0 / -inf."""
    announce("fwd key padding only, Lk=0 batch")
    lens = np.array([0, 77, 300], np.int32)
    inp = inputs.attention_inputs(3, 2, 2, 150, 300, 128, seed=41, seqlens_k=lens, poison=True)
    o, lse = run(inp)
    o_ref, lse_ref = oracle(orc, inp)
    check_attn(host(o), host(lse), o_ref, lse_ref, "bf16")


def test_causal_future_keys_do_not_matter(orc):
    announce("fwd causal future-key perturbation")
    inp = inputs.attention_inputs(1, 2, 2, 512, 512, 128, seed=51, causal=True)
    o1, l1 = run(inp)
    k2, v2 = inp.k.copy(), inp.v.copy()
    k2[:, :, 200:] = inputs.to_bf16_bits(np.full(k2[:, :, 200:].shape, 3.0, np.float32))
    v2[:, :, 200:] = inputs.to_bf16_bits(np.full(v2[:, :, 200:].shape, -5.0, np.float32))
    inp2 = inputs.AttnInputs(inp.q, k2, v2, "bf16", None, None, inp.scale, True)
    o2, l2 = run(inp2)
    b1, b2 = host_bits(o1), host_bits(o2)
    assert np.array_equal(b1[:, :, :200], b2[:, :, :200])
    assert np.array_equal(host_bits(l1)[:, :, :200], host_bits(l2)[:, :, :200])
    assert not np.array_equal(b1[:, :, 200:], b2[:, :, 200:])


def _sample_rows(rng, B, H, N, n, lens=None):
    rows = []
    for _ in range(n):
        b = int(rng.integers(0, B))
        h = int(rng.integers(0, H))
        top = N if lens is None else int(lens[b])
        i = int(rng.integers(0, top))
        rows.append((b * H + h) * N + i)
    # the first and last rows of a few heads and tiles
    for b in range(min(B, 2)):
        top = N if lens is None else int(lens[b])
        for i in (0, 63, 64, 127, 128, top - 1):
            if 0 <= i < top:
                rows.append((b * H) * N + i)
    return np.array(sorted(set(rows)), np.int64)


def test_config3_full_sampled(orc):
    """B4 H32 N4096 d128 non-causal at full size: 600 sampled query rows
    compared with the oracle one by one."""
    announce("fwd config3 full size, sampled rows")
    inp = inputs.config3()
    o, lse = run(inp)
    rows = _sample_rows(np.random.default_rng(3), 4, 32, 4096, 600)
    o_ref, lse_ref = oracle(orc, inp, rows=rows)
    oh = host(o).reshape(-1, 128)[rows]
    lh = host(lse).reshape(-1)[rows]
    check_attn(oh, lh, o_ref, lse_ref, "bf16")
    assert np.isfinite(host(lse)).all()


def test_config4_full_sampled(orc):
    """B8 H16 N8192 causal with key padding, NaN-poisoned padding, at full
    size: sampled rows vs the oracle, every padded row exactly 0 / -inf,
    no NaN anywhere."""
    announce("fwd config4 full size, sampled rows")
    inp = inputs.config4()
    o, lse = run(inp)
    lens = inp.seqlens_q
    rows = _sample_rows(np.random.default_rng(4), 8, 16, 8192, 400, lens)
    o_ref, lse_ref = oracle(orc, inp, rows=rows)
    oh_all = host(o)
    lh_all = host(lse)
    check_attn(oh_all.reshape(-1, 128)[rows], lh_all.reshape(-1)[rows], o_ref, lse_ref, "bf16")
    assert not np.isnan(oh_all).any()
    for b, L in enumerate(lens):
        assert np.all(oh_all[b, :, L:] == 0.0) and np.all(np.isneginf(lh_all[b, :, L:]))
        assert np.all(np.isfinite(lh_all[b, :, :L]))


def test_max_key_length_and_head_offsets(orc):
    """The longest supported key sequence, 2^23 - 1 keys (one head's K just
    under 2 GiB, with a ragged last tile), on three KV heads, so that the
    last head starts 4 GiB into K and V.  GQA 2:1, 100 queries (one partial
    block).  Sampled rows of the last query head against the oracle; every
    head finite."""
    torch = torch_mod()
    B, Hq, Hkv, Nq, Nk, d = 1, 6, 3, 100, (1 << 23) - 1, 128
    announce(f"fwd max key length B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk}")
    ktab, kidx = inputs.tiled_rows(Hkv * Nk, d, seed=inputs.SEED_BASE + 61)
    vtab, vidx = inputs.tiled_rows(Hkv * Nk, d, seed=inputs.SEED_BASE + 62)
    qbits = inputs.to_bf16_bits(inputs.normal_f32(inputs.rng(inputs.SEED_BASE + 63), (B, Hq, Nq, d)))
    k = dev_bf16(ktab)[torch.from_numpy(kidx).to("cuda")].view(B, Hkv, Nk, d)
    v = dev_bf16(vtab)[torch.from_numpy(vidx).to("cuda")].view(B, Hkv, Nk, d)
    scale = 1.0 / np.sqrt(d)
    o, lse = osm.attn_fwd(dev_bf16(qbits), k, v, scale=scale)
    oh, lh = host(o), host(lse)
    del k, v, o, lse
    torch.cuda.empty_cache()
    assert np.isfinite(oh).all() and np.isfinite(lh).all()
    h = Hq - 1
    g = h // (Hq // Hkv)               # its KV head: the last one
    rows = np.array([0, 57, Nq - 1])
    sel = slice(g * Nk, (g + 1) * Nk)
    kh = inputs.bf16_bits_to_f32(ktab)[kidx[sel]][None, None]
    vh = inputs.bf16_bits_to_f32(vtab)[vidx[sel]][None, None]
    qh = inputs.bf16_bits_to_f32(qbits[0, h, rows])[None, None]
    o_ref, lse_ref = orc.attention(qh, kh, vh, scale=scale)
    del kh, vh
    check_attn(oh[0, h, rows], lh[0, h, rows], o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk", [
    (1, 8, 8, 9000, 1),        # one key: the shortest blocks (one tile, zero fills up to four)
    (2, 16, 4, 2100, 300),     # GQA 4:1, ragged last query block and last key tile
    (1, 9, 3, 7500, 70),       # 9 heads: no per-XCD head grouping
    (4, 32, 32, 4096, 4096),   # the full-size non-causal workload
])
def test_persistent_grid(orc, B, Hq, Hkv, Nq, Nk):
    """Full-length non-causal inputs with more query blocks than compute
    units run on a persistent grid (each workgroup walks several blocks,
    prefetching the next block's Q and first key tiles).  The same inputs
    with explicit full lengths take the scheduled persistent grid (head
    counts divisible by 8) or the one-block-per-workgroup kernel (9 heads);
    the per-block arithmetic is the same, so the outputs must agree bit for
    bit.  Sampled rows are also checked against the oracle."""
    announce(f"fwd persistent grid B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk}")
    torch = torch_mod()
    assert B * Hq * ((Nq + 255) // 256) > torch.cuda.get_device_properties(0).multi_processor_count
    inp = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, 128, seed=B * 7 + Hq + Nq + Nk, causal=False)
    q, k, v = (dev_bf16(t) for t in (inp.q, inp.k, inp.v))
    o1, l1 = osm.attn_fwd(q, k, v, scale=inp.scale)
    full_q = dev_i32(np.full(B, Nq, np.int32))
    full_k = dev_i32(np.full(B, Nk, np.int32))
    o2, l2 = osm.attn_fwd(q, k, v, scale=inp.scale, seqlens_q=full_q, seqlens_k=full_k)
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert np.array_equal(host_bits(l1), host_bits(l2))
    rows = _sample_rows(np.random.default_rng(Nq + Nk), B, Hq, Nq, 300)
    o_ref, lse_ref = oracle(orc, inp, rows=rows)
    check_attn(host(o1).reshape(-1, 128)[rows], host(l1).reshape(-1)[rows], o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("persistent", [True, False])
def test_lse_null(persistent):
    """The C ABI lets lse be NULL: O is the same, bit for bit, as with an
    lse buffer, for the bf16 and the FP8 forward, on the persistent grid
    (full-length non-causal, 264 query blocks) and on one block per
    workgroup (causal, ragged lengths)."""
    announce(f"fwd lse NULL persistent={persistent}")
    torch = torch_mod()
    lib = osm.load_library()
    if persistent:
        B, Hq, Hkv, Nq, Nk, causal, lens = 1, 8, 4, 8448, 70, False, None
    else:
        B, Hq, Hkv, Nq, Nk, causal, lens = 2, 4, 2, 300, 300, True, np.array([300, 131], np.int32)
    sl = None if lens is None else dev_i32(lens)
    for dtype in ("bf16", "fp8"):
        inp = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, 128, seed=91 + Nq, causal=causal, dtype=dtype,
                                      seqlens_q=lens, seqlens_k=lens)
        if dtype == "bf16":
            q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
            o1, _ = osm.attn_fwd(q, k, v, scale=inp.scale, causal=causal, seqlens_q=sl, seqlens_k=sl)
        else:
            q, k, v = (torch.from_numpy(np.ascontiguousarray(t)).to("cuda") for t in (inp.q, inp.k, inp.v))
            o1, _ = osm.attn_fwd_fp8(q, k, v, scale=inp.scale, causal=causal, seqlens_q=sl, seqlens_k=sl)
        o2 = torch.full_like(o1, float("nan"))
        if dtype == "bf16":
            st = lib.osm_attn_fwd(osm._ptr(q), osm._ptr(k), osm._ptr(v), osm._ptr(o2), None, 1, B, Hq, Hkv, Nq,
                                  Nk, 128, osm._ptr(sl), osm._ptr(sl), float(inp.scale), int(causal),
                                  osm._stream())
        else:
            st = lib.osm_attn_fwd_fp8(osm._ptr(q), osm._ptr(k), osm._ptr(v), osm._ptr(o2), None, B, Hq, Hkv, Nq,
                                      Nk, 128, osm._ptr(sl), osm._ptr(sl), float(inp.scale), 1.0, int(causal),
                                      osm._stream())
        assert st == 0, lib.osm_status_str(st)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(o1), host_bits(o2)), dtype


def test_no_keys_through_abi():
    """seqlen_k == 0 with k = v = NULL: every query row sees no key, so
    O = +0 and LSE = -inf, for the bf16 and the FP8 forward (300 query
    blocks, causal and not)."""
    torch = torch_mod()
    lib = osm.load_library()
    B, Hq, Hkv, Nq = 2, 6, 3, 12800
    q8 = torch.zeros((B, Hq, Nq, 128), dtype=torch.uint8, device="cuda")
    qb = torch.randn((B, Hq, Nq, 128), device="cuda").to(torch.bfloat16)
    for causal in (0, 1):
        announce(f"fwd no keys causal={causal}")
        for fp8 in (False, True):
            o = torch.full((B, Hq, Nq, 128), float("nan"), device="cuda").to(torch.bfloat16)
            lse = torch.zeros((B, Hq, Nq), dtype=torch.float32, device="cuda")
            if fp8:
                st = lib.osm_attn_fwd_fp8(osm._ptr(q8), None, None, osm._ptr(o), osm._ptr(lse), B, Hq, Hkv, Nq, 0,
                                          128, None, None, 0.1, 1.0, causal, osm._stream())
            else:
                st = lib.osm_attn_fwd(osm._ptr(qb), None, None, osm._ptr(o), osm._ptr(lse), 1, B, Hq, Hkv, Nq, 0,
                                      128, None, None, 0.1, causal, osm._stream())
            assert st == 0, lib.osm_status_str(st)
            torch.cuda.synchronize()
            assert np.all(host_bits(o) == 0), f"fp8={fp8}"
            assert np.all(np.isneginf(host(lse))), f"fp8={fp8}"


def _run_in_groups(inp):
    """The same attention, one call per (batch, group of 8 query heads): at
    most 256 query blocks per call (N <= 8192), so every call runs one block
    per workgroup."""
    torch = torch_mod()
    B, Hq, Nq, d = inp.q.shape
    Hkv = inp.k.shape[1]
    g = Hq // Hkv
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    for b in range(B):
        for h0 in range(0, Hq, 8):
            kv0, kv1 = h0 // g, (h0 + 8 + g - 1) // g
            sq = None if inp.seqlens_q is None else dev_i32(inp.seqlens_q[b:b + 1])
            sk = None if inp.seqlens_k is None else dev_i32(inp.seqlens_k[b:b + 1])
            ob, lb = osm.attn_fwd(q[b:b + 1, h0:h0 + 8].contiguous(), k[b:b + 1, kv0:kv1].contiguous(),
                                  v[b:b + 1, kv0:kv1].contiguous(), scale=inp.scale, causal=inp.causal,
                                  seqlens_q=sq, seqlens_k=sk)
            o[b:b + 1, h0:h0 + 8] = ob
            lse[b:b + 1, h0:h0 + 8] = lb
    return o, lse


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,causal,lq,lk", [
    (4, 16, 16, 4096, 4096, True, [1, 1000, 2049, 4096], None),       # causal, ragged, one 1-row sequence
    (4, 16, 8, 3000, 2000, False, [3000, 17, 2999, 0], [0, 2000, 1234, 5]),   # no keys / no queries
    (2, 32, 8, 5000, 5000, True, [5000, 3333], None),                  # GQA 4:1, causal
    (2, 8, 8, 8192, 8192, True, [8192, 7777], None),                   # 1 head per XCD, 32-block heads
])
def test_scheduled_grid(orc, B, Hq, Hkv, Nq, Nk, causal, lq, lk):
    """Causal or varlen inputs with more query blocks than compute units run
    on the scheduled persistent grid (each workgroup walks a list of blocks
    built in-kernel from the lengths, prefetching the next block's Q and
    first tiles).  One call per group of 8 query heads of one sequence runs
    the same blocks one per workgroup; the per-block arithmetic is the same,
    so the outputs must agree bit for bit.  NaN past the lengths; padded
    rows exactly 0 / -inf; sampled rows against the oracle."""
    announce(f"fwd scheduled grid B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} lq={lq} lk={lk}")
    torch = torch_mod()
    assert B * Hq * ((Nq + 255) // 256) > torch.cuda.get_device_properties(0).multi_processor_count
    lq = np.array(lq, np.int32)
    lk = lq.copy() if lk is None else np.array(lk, np.int32)
    inp = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, 128, seed=B * 11 + Hq + Nq + Nk, causal=causal,
                                  seqlens_q=lq, seqlens_k=lk, poison=True)
    o1, l1 = run(inp)
    o2, l2 = _run_in_groups(inp)
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert np.array_equal(host_bits(l1), host_bits(l2))
    oh, lh = host(o1), host(l1)
    assert not np.isnan(oh).any()
    for b in range(B):
        dead_from = int(lq[b]) if lk[b] > 0 else 0
        assert np.all(oh[b, :, dead_from:] == 0.0) and np.all(np.isneginf(lh[b, :, dead_from:]))
    rows = _sample_rows(np.random.default_rng(Nq + B), B, Hq, Nq, 300, np.maximum(lq, 1))
    o_ref, lse_ref = oracle(orc, inp, rows=rows)
    check_attn(oh.reshape(-1, 128)[rows], lh.reshape(-1)[rows], o_ref, lse_ref, "bf16")


# Workgroups the forward keeps resident per compute unit: one at head dim 128,
# two at 64.  At head dim 128, inputs with more query blocks than compute units
# run on the persistent or scheduled grid; head dim 64 runs one block per
# workgroup on every input, many blocks per compute unit in these cases.
WG_PER_CU = {128: 1, 64: 2}


def _sweep_config(g, many_heads, d=128):
    """One random configuration: GQA group, ragged lengths, masks, scale.
    With many_heads, more query blocks than resident workgroups (persistent
    and scheduled grids); otherwise one block per workgroup."""
    if many_heads:
        B = int(g.integers(1, 4))
        Hkv = int(g.choice([8, 16]))
        Hq = Hkv * int(g.choice([1, 2, 4]))
        # query blocks per head: more blocks than 256 CUs' resident workgroups
        nqb = 256 * WG_PER_CU[d] // (B * Hq) + 1
        Nq = int(g.integers((nqb - 1) * 256 + 1, nqb * 256 + 1))
        Nk = int(g.integers(1, 450))
    else:
        B = int(g.integers(1, 4))
        Hkv = int(g.choice([1, 2]))
        Hq = Hkv * int(g.choice([1, 2, 4]))
        Nq = int(g.integers(1, 520))
        Nk = int(g.integers(1, 600))
    causal = bool(g.random() < 0.5)
    mode = int(g.integers(0, 3))          # 0: full lengths, 1: key lengths, 2: both
    sq = sk = None
    if mode >= 1:
        sk = g.integers(0, Nk + 1, size=B).astype(np.int32)
    if mode == 2:
        sq = g.integers(0, Nq + 1, size=B).astype(np.int32)
    scale = float(g.uniform(0.03, 0.25))
    return B, Hq, Hkv, Nq, Nk, causal, sq, sk, scale


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("many_heads", [False, True])
def test_random_sweep(orc, many_heads, d):
    """Seeded random configurations against the oracle: every row for the
    small ones, 200 sampled rows plus every padded row for the many-head
    ones (which run on the persistent or scheduled grids).  Padding is
    NaN-poisoned wherever a length array marks it."""
    g = inputs.rng(4242 + many_heads + 2 * (d == 64))
    n = 16 if many_heads else 60
    for case in range(n):
        B, Hq, Hkv, Nq, Nk, causal, sq, sk, scale = _sweep_config(g, many_heads, d)
        announce(f"fwd sweep {case}: d={d} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} "
                 f"seqlens_q={None if sq is None else sq.tolist()} seqlens_k={None if sk is None else sk.tolist()} "
                 f"scale={scale:.4f}")
        inp = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, d, seed=5000 + 100 * many_heads + 1000 * (d == 64) + case,
                                      causal=causal,
                                      scale=scale, seqlens_q=sq, seqlens_k=sk, poison=sk is not None)
        if many_heads:
            assert B * Hq * ((Nq + 255) // 256) > (torch_mod().cuda.get_device_properties(0).multi_processor_count
                                                   * WG_PER_CU[d])
        o, lse = run(inp)
        oh, lh = host(o), host(lse)
        assert not np.isnan(oh).any() and not np.isnan(lh).any()
        if many_heads:
            rows = _sample_rows(np.random.default_rng(case), B, Hq, Nq, 200)
            o_ref, lse_ref = oracle(orc, inp, rows=rows)
            check_attn(oh.reshape(-1, d)[rows], lh.reshape(-1)[rows], o_ref, lse_ref, "bf16")
        else:
            o_ref, lse_ref = oracle(orc, inp)
            check_attn(oh, lh, o_ref, lse_ref, "bf16")
        if sq is not None:
            for b, L in enumerate(sq):       # padded query rows: exactly 0 / -inf
                assert np.all(oh[b, :, L:] == 0.0) and np.all(np.isneginf(lh[b, :, L:]))


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,causal", [
    (2, 4, 2, 300, 300, False),
    (2, 4, 2, 300, 300, True),
    (1, 2, 1, 129, 517, False),
    (1, 2, 2, 1, 1, False),
    (1, 2, 2, 640, 640, True),
])
def test_small_d64(orc, B, Hq, Hkv, Nq, Nk, causal):
    """Head dim 64, element by element against the oracle."""
    announce(f"fwd d64 B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal}")
    inp = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, 64, seed=B * 1000 + Nq + Nk + 64, causal=causal)
    o, lse = run(inp)
    o_ref, lse_ref = oracle(orc, inp)
    check_attn(host(o), host(lse), o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_poisoned_d64(orc, causal):
    """Head dim 64 with NaN past the lengths: against the oracle, padded
    rows exactly 0 / -inf, and bit-identical to zero padding."""
    announce(f"fwd d64 varlen poisoned causal={causal}")
    B, H, N = 4, 2, 400
    lens = np.array([1, 130, 257, 400], np.int32)
    inp = inputs.attention_inputs(B, H, H, N, N, 64, seed=33, causal=causal, seqlens_q=lens,
                                  seqlens_k=lens, poison=True)
    o, lse = run(inp)
    o_ref, lse_ref = oracle(orc, inp)
    oh, lh = host(o), host(lse)
    check_attn(oh, lh, o_ref, lse_ref, "bf16")
    for b, L in enumerate(lens):
        assert np.all(oh[b, :, L:] == 0.0) and np.all(np.isneginf(lh[b, :, L:]))
    zq, zk, zv = (inputs.bf16_bits_to_f32(a).copy() for a in (inp.q, inp.k, inp.v))
    for a in (zq, zk, zv):
        a[np.isnan(a)] = 0.0
    inp0 = inputs.AttnInputs(inputs.to_bf16_bits(zq), inputs.to_bf16_bits(zk), inputs.to_bf16_bits(zv),
                             "bf16", lens, lens, inp.scale, causal)
    o0, l0 = run(inp0)
    assert np.array_equal(host_bits(o), host_bits(o0))
    assert np.array_equal(host_bits(lse), host_bits(l0))


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,causal,lq,lk", [
    (4, 32, 8, 4096, 4096, False, None, None),                       # full length, GQA 4:1
    (1, 16, 16, 8300, 1, False, None, None),                         # one key
    (4, 16, 16, 4096, 4096, True, [1, 1000, 2049, 4096], None),      # causal, ragged
    (4, 16, 8, 3000, 2000, False, [3000, 17, 2999, 0], [0, 2000, 1234, 5]),   # no keys / no queries
])
def test_grids_d64(orc, B, Hq, Hkv, Nq, Nk, causal, lq, lk):
    """Head dim 64 with more query blocks than resident workgroups (several
    blocks per workgroup slot, XCD-grouped heads) against the same attention
    computed one call per (batch, group of 8 heads), bit for bit; sampled rows
    against the oracle; padded rows exactly 0 / -inf."""
    announce(f"fwd d64 grids B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} lq={lq} lk={lk}")
    torch = torch_mod()
    assert B * Hq * ((Nq + 255) // 256) > torch.cuda.get_device_properties(0).multi_processor_count * WG_PER_CU[64]
    if lq is not None:
        lq = np.array(lq, np.int32)
        lk = lq.copy() if lk is None else np.array(lk, np.int32)
    inp = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, 64, seed=B * 13 + Hq + Nq + Nk, causal=causal,
                                  seqlens_q=lq, seqlens_k=lk, poison=lq is not None)
    o1, l1 = run(inp)
    o2, l2 = _run_in_groups(inp)
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert np.array_equal(host_bits(l1), host_bits(l2))
    oh, lh = host(o1), host(l1)
    assert not np.isnan(oh).any()
    if lq is not None:
        for b in range(B):
            dead_from = int(lq[b]) if lk[b] > 0 else 0
            assert np.all(oh[b, :, dead_from:] == 0.0) and np.all(np.isneginf(lh[b, :, dead_from:]))
    rows = _sample_rows(np.random.default_rng(Nq + B + 64), B, Hq, Nq, 300,
                        None if lq is None else np.maximum(lq, 1))
    o_ref, lse_ref = oracle(orc, inp, rows=rows)
    check_attn(oh.reshape(-1, 64)[rows], lh.reshape(-1)[rows], o_ref, lse_ref, "bf16")
