"""osm_softmax_rows on the GPU against the oracle."""
import numpy as np
import pytest

import exact_attention_online_softmax_amd as osm
from exact_attention_online_softmax_amd import inputs
from gpu_util import announce, check_softmax, dev_f32, host
import pins

pytestmark = pytest.mark.gpu


def run(x, two_pass=False):
    y, m, l = osm.softmax_rows(dev_f32(x), return_stats=True, two_pass=two_pass)
    return host(y), host(m), host(l)


def test_worked_rows(orc):
    announce("softmax worked rows [1,3,2,0], [2,5,1,7]")
    x = np.array(inputs.WORKED_ROWS, np.float32)
    y, m, l = run(x)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    check_softmax(y, m, l, y_ref, m_ref, l_ref)
    g = pins.golden("p2_walkthrough_softmax.txt")
    assert [round(float(t), 6) for t in y[0]] == pins.floats(g["softmax_6dp"])
    g = pins.golden("p3_running_sum_2517.txt")
    assert m[1] == float(g["step4_m"]) and round(l[1], 4) == float(g["final_l_4dp"])


def test_config2_full(orc):
    announce("softmax 4096 x 32000, N(0,9) + spike U[20,90)")
    x = inputs.config2()
    y, m, l = run(x)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    check_softmax(y, m, l, y_ref, m_ref, l_ref)
    # rows whose spike passes the fp32 exp overflow point are finite too
    assert (m_ref > 88.7228).any() and np.isfinite(y).all()


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 4), (5, 7), (17, 129), (33, 4001), (8, 16384),
                                       (4, 65536), (3, 65537), (2, 100003), (1100000, 2)])
def test_shapes(orc, rows, cols):
    announce(f"softmax rows={rows} cols={cols}")
    x = inputs.softmax_rows_input(rows, cols, seed=rows * 7 + cols)
    y, m, l = run(x)
    if rows > 4096:
        sel = np.unique(np.concatenate([np.arange(64), np.arange(rows - 64, rows),
                                        np.random.default_rng(0).integers(0, rows, 512)]))
        y_ref, m_ref, l_ref = orc.softmax_rows(x, rows=sel)
        check_softmax(y[sel], m[sel], l[sel], y_ref, m_ref, l_ref)
    else:
        y_ref, m_ref, l_ref = orc.softmax_rows(x)
        check_softmax(y, m, l, y_ref, m_ref, l_ref)


def test_masked_entries(orc):
    announce("softmax with -inf entries and all -inf rows")
    x = inputs.softmax_rows_input(6, 3000, seed=5)
    x[0, :] = -np.inf
    x[1, ::3] = -np.inf
    x[2, 1:] = -np.inf
    x[3, :2999] = -np.inf
    y, m, l = run(x)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    assert np.all(y[0] == 0.0) and m[0] == -np.inf and l[0] == 0.0
    assert np.all(y[1, ::3] == 0.0)
    assert y[2, 0] == 1.0 and y[3, 2999] == 1.0
    check_softmax(y, m, l, y_ref, m_ref, l_ref)


def test_in_place(orc):
    announce("softmax in place")
    import torch
    x = inputs.softmax_rows_input(64, 5000, seed=9)
    t = dev_f32(x)
    osm.softmax_rows(t, out=t)
    torch.cuda.synchronize()
    y_ref, _, _ = orc.softmax_rows(x)
    err = np.abs(host(t) - y_ref)
    assert np.all(err <= 1e-5 * np.abs(y_ref) + 2.0 ** -126)


def test_invariance_to_shift(orc):
    """Adding an exact constant to a row leaves the GPU result unchanged
    (within tolerance): the maximum is subtracted."""
    announce("softmax shift")
    x = (np.round(inputs.softmax_rows_input(8, 2048, seed=3, spikes=False) * 64) / 64).astype(np.float32)
    y1, _, _ = run(x)
    y2, _, _ = run(x + np.float32(64.0))
    assert np.all(np.abs(y1 - y2) <= 2e-5 * np.abs(y1) + 2.0 ** -126)


@pytest.mark.parametrize("cols,ld_x,ld_y", [(32000, 32004, 32008), (3000, 3004, 3000),
                                            (2048, 2051, 2053), (129, 132, 136)])
def test_row_stride(orc, cols, ld_x, ld_y):
    """Rows ld_x / ld_y elements apart, through the C ABI (the binding passes
    contiguous rows): whole-vector rows on 16-byte strides, odd strides, and
    a ragged width; the gap between rows of y is never written."""
    announce(f"softmax strided rows cols={cols} ld_x={ld_x} ld_y={ld_y}")
    torch = __import__("torch")
    rows = 37
    x = inputs.softmax_rows_input(rows, cols, seed=cols + ld_x)
    xb = np.full((rows, ld_x), np.nan, np.float32)
    xb[:, :cols] = x
    xd = dev_f32(xb)
    sentinel = np.float32(-7.25)
    yd = torch.full((rows, ld_y), float(sentinel), dtype=torch.float32, device="cuda")
    md = torch.empty(rows, dtype=torch.float32, device="cuda")
    sd = torch.empty(rows, dtype=torch.float32, device="cuda")
    lib = osm.load_library()
    st = lib.osm_softmax_rows(osm._ptr(xd), osm._ptr(yd), rows, cols, ld_x, ld_y, osm._ptr(md),
                              osm._ptr(sd), osm._stream())
    assert st == 0, lib.osm_status_str(st)
    torch.cuda.synchronize()
    yb = host(yd)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    check_softmax(yb[:, :cols], host(md), host(sd), y_ref, m_ref, l_ref)
    assert np.all(yb[:, cols:] == sentinel)


def test_zero_columns_through_abi():
    """cols == 0 with x = y = NULL: each empty row's statistics are the
    empty set's, m = -inf and l = 0 (nothing is read or written through
    the NULL pointers)."""
    announce("softmax cols=0, x = y = NULL")
    torch = __import__("torch")
    rows = 37
    md = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    sd = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    lib = osm.load_library()
    st = lib.osm_softmax_rows(None, None, rows, 0, 0, 0, osm._ptr(md), osm._ptr(sd), osm._stream())
    assert st == 0, lib.osm_status_str(st)
    torch.cuda.synchronize()
    assert np.all(np.isneginf(host(md))) and np.all(host(sd) == 0.0)


# ---- the streaming two-pass kernels (rows past 65536 columns, and every row
# through osm_softmax_rows_twopass) ------------------------------------------
def run_abi(x, cols, ld_x, ld_y, *, two_pass, stats=True, rows=None):
    """Rows of x (ld_x apart, NaN in the gaps) through the C ABI; y is
    ld_y apart with a sentinel in its gaps.  Returns y (gaps included), m, l."""
    torch = __import__("torch")
    rows = x.shape[0] if rows is None else rows
    xb = np.full((rows, ld_x), np.nan, np.float32)
    xb[:, :cols] = x
    xd = dev_f32(xb)
    yd = torch.full((rows, ld_y), -7.25, dtype=torch.float32, device="cuda")
    md = torch.full((rows,), np.nan, dtype=torch.float32, device="cuda") if stats else None
    sd = torch.full((rows,), np.nan, dtype=torch.float32, device="cuda") if stats else None
    lib = osm.load_library()
    fn = lib.osm_softmax_rows_twopass if two_pass else lib.osm_softmax_rows
    st = fn(osm._ptr(xd), osm._ptr(yd), rows, cols, ld_x, ld_y, osm._ptr(md), osm._ptr(sd), osm._stream())
    assert st == 0, lib.osm_status_str(st)
    torch.cuda.synchronize()
    return host(yd), (host(md) if stats else None), (host(sd) if stats else None)


@pytest.mark.parametrize("rows,cols", [(4, 65540), (2, 131072), (3, 65537), (2, 100003)])
def test_streaming_wide_rows(orc, rows, cols):
    """Automatic choice past 65536 columns: whole-vector rows (65540, 131072)
    take the buffer-resource streaming kernel, odd widths the generic one."""
    announce(f"softmax streaming rows={rows} cols={cols}")
    x = inputs.softmax_rows_input(rows, cols, seed=rows * 13 + cols)
    y, m, l = run(x)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    check_softmax(y, m, l, y_ref, m_ref, l_ref)


@pytest.mark.parametrize("two_pass", [False, True])
def test_streaming_masked(orc, two_pass):
    """-inf entries in rows wider than 65536 columns: a whole row, every
    third entry, all but the first, all but the last, and a row whose first
    65536 entries are -inf (a lane's early vectors are all empty)."""
    announce(f"softmax streaming -inf rows two_pass={two_pass}")
    cols = 70000
    x = inputs.softmax_rows_input(6, cols, seed=21)
    x[0, :] = -np.inf
    x[1, ::3] = -np.inf
    x[2, 1:] = -np.inf
    x[3, :cols - 1] = -np.inf
    x[4, :65536] = -np.inf
    y, m, l = run(x, two_pass=two_pass)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    assert np.all(y[0] == 0.0) and m[0] == -np.inf and l[0] == 0.0
    assert np.all(y[1, ::3] == 0.0) and np.all(y[4, :65536] == 0.0)
    assert y[2, 0] == 1.0 and y[3, cols - 1] == 1.0
    check_softmax(y, m, l, y_ref, m_ref, l_ref)


@pytest.mark.parametrize("cols,ld_x,ld_y", [(65537, 65540, 65544), (70000, 70004, 70008),
                                            (70000, 70001, 70003), (66001, 66004, 66001)])
def test_streaming_row_stride(orc, cols, ld_x, ld_y):
    """Strided rows through the C ABI past 65536 columns: 16-byte strides with
    a ragged width (the aligned generic kernel), whole vectors (the buffer
    kernel), odd strides (unaligned); the gaps of y are never written."""
    announce(f"softmax streaming strided cols={cols} ld_x={ld_x} ld_y={ld_y}")
    rows = 5
    x = inputs.softmax_rows_input(rows, cols, seed=cols + ld_y)
    y, m, l = run_abi(x, cols, ld_x, ld_y, two_pass=False)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    check_softmax(y[:, :cols], m, l, y_ref, m_ref, l_ref)
    assert np.all(y[:, cols:] == np.float32(-7.25))


@pytest.mark.parametrize("two_pass", [False, True])
def test_streaming_stats_null(two_pass):
    """row_max / row_sum NULL leave y bit-identical to the call that writes them."""
    announce(f"softmax streaming stats NULL two_pass={two_pass}")
    x = inputs.softmax_rows_input(3, 70004, seed=31)
    y1, _, _ = run_abi(x, 70004, 70004, 70004, two_pass=two_pass, stats=True)
    y2, _, _ = run_abi(x, 70004, 70004, 70004, two_pass=two_pass, stats=False)
    assert np.array_equal(y1.view(np.uint64), y2.view(np.uint64))


@pytest.mark.parametrize("two_pass", [False, True])
def test_spike_near_exp_limit(orc, two_pass):
    """A spike of 89.9 (past fp32's e^x overflow at 88.72) in rows wider than
    the on-chip limit and in the 32000-column width: m exact, l within 2e-6
    relative, y within the usual gate."""
    announce(f"softmax spike 89.9 two_pass={two_pass}")
    for cols in (32000, 70004, 131071):
        x = inputs.softmax_rows_input(4, cols, seed=cols + 7, spikes=False)
        x[np.arange(4), [0, cols // 3, cols - 1, 12345]] = np.float32(89.9)
        y, m, l = run(x, two_pass=two_pass)
        y_ref, m_ref, l_ref = orc.softmax_rows(x)
        assert np.all(m == m_ref)
        assert np.all(np.abs(l - l_ref) <= 2e-6 * l_ref), np.max(np.abs(l - l_ref) / l_ref)
        check_softmax(y, m, l, y_ref, m_ref, l_ref)


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 4), (5, 7), (17, 129), (33, 4001), (8, 16384),
                                       (4, 65536), (2, 100003)])
def test_twopass_shapes(orc, rows, cols):
    announce(f"softmax two-pass rows={rows} cols={cols}")
    x = inputs.softmax_rows_input(rows, cols, seed=rows * 11 + cols)
    y, m, l = run(x, two_pass=True)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    check_softmax(y, m, l, y_ref, m_ref, l_ref)


def test_twopass_config2_full(orc):
    """The measured two-pass configuration: 4096 x 32000, N(0, 9) + one spike
    per row in [20, 90), every row read twice from memory."""
    announce("softmax two-pass 4096 x 32000")
    x = inputs.config2()
    y, m, l = run(x, two_pass=True)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    check_softmax(y, m, l, y_ref, m_ref, l_ref)


@pytest.mark.parametrize("cols,ld_x,ld_y", [(32000, 32004, 32008), (2048, 2051, 2053), (129, 132, 136)])
def test_twopass_row_stride(orc, cols, ld_x, ld_y):
    announce(f"softmax two-pass strided cols={cols} ld_x={ld_x} ld_y={ld_y}")
    x = inputs.softmax_rows_input(9, cols, seed=cols * 3 + ld_x)
    y, m, l = run_abi(x, cols, ld_x, ld_y, two_pass=True)
    y_ref, m_ref, l_ref = orc.softmax_rows(x)
    check_softmax(y[:, :cols], m, l, y_ref, m_ref, l_ref)
    assert np.all(y[:, cols:] == np.float32(-7.25))


def test_random_sweep(orc):
    """Seeded random rows against the oracle through both the one-read and
    the two-pass kernels: widths on both sides of the resident limit,
    spikes, -inf entries and whole -inf rows, large offsets."""
    g = inputs.rng(4646)
    for case in range(30):
        rows = int(g.integers(1, 40))
        cols = int(g.choice([int(g.integers(1, 300)), int(g.integers(300, 20000)), int(g.integers(60000, 140000))]))
        x = inputs.softmax_rows_input(rows, cols, seed=7000 + case)
        x += np.float32(g.uniform(-50, 50))
        if g.random() < 0.5:
            x[g.integers(0, rows), :] = -np.inf
        if g.random() < 0.5:
            x[:, g.integers(0, cols, size=max(1, cols // 5))] = -np.inf
        for two_pass in (False, True):
            announce(f"softmax sweep {case}: rows={rows} cols={cols} two_pass={two_pass}")
            y, m, l = run(x, two_pass)
            y_ref, m_ref, l_ref = orc.softmax_rows(x)
            check_softmax(y, m, l, y_ref, m_ref, l_ref)
