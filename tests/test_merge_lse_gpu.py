"""osm_merge_lse on the GPU against the oracle: the fold of the oracle's
two-way log-sum-exp merge, and, end to end, attention over chunks of the
keys merged on the GPU against the oracle's attention over all keys."""
import numpy as np
import pytest

import exact_attention_online_softmax_amd as osm
from exact_attention_online_softmax_amd import inputs
from gpu_util import announce, check_attn, dev_f32, dev_input, host, host_bits, torch_mod

pytestmark = pytest.mark.gpu


def oracle_fold(orc, o_parts, lse_parts):
    """Left fold of the oracle's two-way merge over the pieces (the merge is
    associative, [P3] "Merging partial results")."""
    o, lse = o_parts[0], lse_parts[0]
    for s in range(1, len(o_parts)):
        o, lse = orc.merge_lse(o, lse, o_parts[s], lse_parts[s])
    return o, lse


def widen(o, dtype):
    return inputs.bf16_bits_to_f32(o).astype(np.float64) if dtype == "bf16" else o.astype(np.float64)


def run(o_parts, lse_parts, in_dtype, out_dtype):
    torch = torch_mod()
    op = dev_input(o_parts, in_dtype)
    lp = dev_f32(lse_parts)
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    return osm.merge_lse(op, lp, out_dtype=odt)


@pytest.mark.parametrize("S,rows,d,it,ot", [
    (1, 7, 128, "f32", "f32"), (3, 100, 64, "f32", "f32"), (8, 513, 128, "bf16", "bf16"),
    (70, 33, 96, "f32", "f32"), (5, 40, 37, "f32", "bf16"), (4, 10, 1024, "bf16", "f32"),
    (2, 9, 511, "f32", "f32"), (6, 300, 128, "bf16", "f32"), (11, 77, 128, "bf16", "bf16"),
    (19, 5, 64, "f32", "f32")])
def test_fold(orc, S, rows, d, it, ot):
    announce(f"merge_lse S{S} rows{rows} d{d} {it}->{ot}")
    o_parts, lse_parts = inputs.lse_parts(S, rows, d, 4000 + S * 7 + d, dtype=it, empty_frac=0.2,
                                          poison=True)
    o, lse = run(o_parts, lse_parts, it, ot)
    # empty pieces (lse = -inf) drop out of the merge whatever their o holds;
    # the oracle multiplies them by a zero weight, so it is given zeros there
    o_ref, lse_ref = oracle_fold(orc, np.nan_to_num(widen(o_parts, it)), lse_parts.astype(np.float64))
    check_attn(host(o), host(lse), o_ref, lse_ref, ot)


def test_single_piece_is_identity(orc):
    """One piece: the merge returns it bit for bit (weight e^0 = 1)."""
    announce("merge_lse single piece identity")
    for dt in ("f32", "bf16"):
        o_parts, lse_parts = inputs.lse_parts(1, 64, 128, 4100, dtype=dt)
        o, lse = run(o_parts, lse_parts, dt, dt)
        ref = o_parts[0].view(np.int16) if dt == "bf16" else o_parts[0].view(np.int32)
        assert np.array_equal(host_bits(o), ref)
        assert np.array_equal(host(lse), lse_parts[0].astype(np.float64))


def test_all_empty_rows_and_poison(orc):
    """Rows whose pieces are all empty give exactly 0 / -inf; NaN in empty
    pieces' outputs never reaches the result."""
    announce("merge_lse empty rows and NaN poison")
    o_parts, lse_parts = inputs.lse_parts(4, 50, 128, 4200, empty_frac=0.5, poison=True)
    lse_parts[:, :5] = -np.inf                       # rows 0..4: every piece empty
    o_parts[:, :5] = np.nan
    o, lse = run(o_parts, lse_parts, "f32", "f32")
    oh, lh = host(o), host(lse)
    assert np.all(oh[:5] == 0.0) and np.all(np.isneginf(lh[:5]))
    assert not np.isnan(oh).any()
    o_ref, lse_ref = oracle_fold(orc, np.nan_to_num(o_parts.astype(np.float64)), lse_parts.astype(np.float64))
    check_attn(oh, lh, o_ref, lse_ref, "f32")


@pytest.mark.parametrize("chunks", [[130, 300, 517], [517], [1, 2, 3, 200, 517]])
def test_attention_over_key_chunks(orc, chunks):
    """Attention of all queries over each chunk of the keys (separate
    osm_attn_fwd calls), merged by osm_merge_lse, equals the oracle's
    attention over all the keys ([P3] "The same merge, in log-sum-exp form")."""
    announce(f"merge_lse of attention over key chunks {chunks}")
    torch = torch_mod()
    inp = inputs.attention_inputs(2, 4, 2, 300, 517, 128, 4300 + len(chunks))
    q = dev_input(inp.q, "bf16")
    k = dev_input(inp.k, "bf16")
    v = dev_input(inp.v, "bf16")
    starts = [0] + chunks[:-1]
    outs, lses = [], []
    for a, b in zip(starts, chunks):
        o_c, l_c = osm.attn_fwd(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), scale=inp.scale)
        outs.append(o_c.reshape(-1, 128))
        lses.append(l_c.reshape(-1))
    o, lse = osm.merge_lse(torch.stack(outs), torch.stack(lses), out_dtype=torch.float32)
    qw, kw, vw = inp.widened()
    o_ref, lse_ref = orc.attention(qw, kw, vw, scale=inp.scale)
    check_attn(host(o), host(lse), o_ref.reshape(-1, 128), lse_ref.reshape(-1), "bf16")


def test_bench_shape_sampled(orc):
    """The measured shape (8 pieces of the B4 H32 N4096 d128 output, bf16):
    sampled rows against the oracle fold."""
    announce("merge_lse bench shape S8 rows 524288 d128 bf16, sampled")
    S, rows, d = 8, 4 * 32 * 4096, 128
    o_parts, lse_parts = inputs.lse_parts(S, rows, d, 4400, dtype="bf16")
    o, lse = run(o_parts, lse_parts, "bf16", "bf16")
    idx = np.sort(inputs.rng(4401).choice(rows, 4096, replace=False))
    oh, lh = host(o)[idx], host(lse)[idx]
    o_ref, lse_ref = oracle_fold(orc, widen(o_parts[:, idx], "bf16"), lse_parts[:, idx].astype(np.float64))
    check_attn(oh, lh, o_ref, lse_ref, "bf16")
