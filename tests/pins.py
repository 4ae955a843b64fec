"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a printed value, a closed form, an invariant
or a brute-force evaluation.  ``test_oracle_pins.py`` runs them against the
real oracle; ``test_oracle_mutants.py`` runs them against oracles compiled
from deliberately broken source and requires that every break is caught.

None of these re-types the oracle's own formula: the references are the
pages' printed numbers (fixtures under ``tests/golden/``, each citing its
page and section), closed forms, invariants and brute force in pure Python
(unsafe exponentials on small values, explicit index loops).
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    """Parse a ``key: values`` fixture (``#`` lines are citations)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.strip()
    return out


def floats(s: str):
    return [float(t) for t in s.replace("|", " ").split()]


def close(a, b, rtol, atol=0.0, what=""):
    a = np.atleast_1d(np.asarray(a, np.float64))
    b = np.atleast_1d(np.asarray(b, np.float64))
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    with np.errstate(invalid="ignore"):
        err = np.abs(a - b)
    err[same_inf] = 0.0
    bad = ~(err <= atol + rtol * np.abs(b))
    assert not bad.any(), f"{what}: max err {np.nanmax(err)} (first bad {np.argwhere(bad)[:3].tolist()})"


# ---------------------------------------------------------------------------
# brute-force helpers (pure Python, tiny inputs, no max subtraction)
# ---------------------------------------------------------------------------
def brute_softmax(row):
    e = [math.exp(x) for x in row]
    z = math.fsum(e)
    return [t / z for t in e]


def brute_attention(q, k, v, scale, causal, lq, lk, group):
    """q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] nested float arrays; explicit loops."""
    B, Hq, Nq, d = q.shape
    o = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), -math.inf)
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            for i in range(Nq):
                if i >= lq[b]:
                    continue
                keys = [j for j in range(lk[b]) if (not causal or j <= i)]
                if not keys:
                    continue
                w = {}
                for j in keys:
                    dot = math.fsum(float(q[b, h, i, c]) * float(k[b, kvh, j, c]) for c in range(d))
                    w[j] = math.exp(scale * dot)
                z = math.fsum(w.values())
                for c in range(d):
                    o[b, h, i, c] = math.fsum(w[j] * float(v[b, kvh, j, c]) for j in keys) / z
                lse[b, h, i] = math.log(z)
    return o, lse


def blocked_recurrence_single_query(qv, K, V, block):
    """An fp64 block-at-a-time online attention for one query, written here
    independently of the oracle (running max, running sum, running output,
    one division at the end)."""
    m, l = -math.inf, 0.0
    acc = np.zeros(K.shape[1])
    for start in range(0, K.shape[0], block):
        s = K[start:start + block] @ qv
        m_new = max(m, float(s.max()))
        a = 0.0 if m == -math.inf else math.exp(m - m_new)
        p = np.exp(s - m_new)
        l = a * l + float(p.sum())
        acc = a * acc + p @ V[start:start + block]
        m = m_new
    return acc / l, m + math.log(l)


# ---------------------------------------------------------------------------
# softmax
# ---------------------------------------------------------------------------
def pin_softmax_worked_example(orc):
    g = golden("p2_walkthrough_softmax.txt")
    row = floats(g["row"])
    y, m, l = orc.softmax_rows(np.array([row], np.float32))
    printed = floats(g["softmax_6dp"])
    assert [round(float(t), 6) for t in y[0]] == printed, (y[0], printed)
    assert m[0] == max(row)
    # the two tiles of the page give the same 6-digit result as the whole row
    tiles = [floats(t) for t in g["tiles"].split("|")]
    assert sum(tiles, []) == row


def pin_softmax_brute_force(orc):
    gen = np.random.default_rng(11)
    for n in (1, 2, 3, 7, 16, 33):
        row = (gen.standard_normal(n) * 6).astype(np.float32)
        y, m, l = orc.softmax_rows(row[None, :])
        ref = brute_softmax([float(t) for t in row])
        close(y[0], ref, 1e-13, what=f"softmax n={n}")
        mx = max(float(t) for t in row)
        assert m[0] == mx
        close(l[0], math.fsum(math.exp(float(t) - mx) for t in row), 1e-14, what="l")


def pin_softmax_invariants(orc):
    gen = np.random.default_rng(12)
    # multiples of 2^-10, so that adding 16 below is exact in fp32
    row = (np.round(gen.standard_normal(50) * 3 * 1024) / 1024).astype(np.float32)
    y, _, _ = orc.softmax_rows(row[None, :])
    close(y.sum(), 1.0, 1e-14, what="sum to 1")
    y2, _, _ = orc.softmax_rows((row + np.float32(16.0))[None, :])
    close(y2, y, 1e-12, what="shift invariance")
    perm = gen.permutation(50)
    y3, _, _ = orc.softmax_rows(row[perm][None, :])
    close(y3[0], y[0][perm], 1e-14, what="permutation equivariance")
    yu, mu, lu = orc.softmax_rows(np.full((1, 40), 2.5, np.float32))
    close(yu, np.full((1, 40), 1 / 40), 1e-15, what="uniform row")
    close(lu, [40.0], 1e-15, what="uniform l")
    # a spike past the fp32 overflow point: the unsafe formula overflows,
    # the safe softmax stays finite, sums to 1 and puts nearly all mass there
    spike = row.copy()
    spike[7] = np.float32(89.5)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(spike)                      # fp32, no max subtraction
        unsafe = e / e.sum()
    assert not np.all(np.isfinite(unsafe))
    ys, ms, ls = orc.softmax_rows(spike[None, :])
    assert np.all(np.isfinite(ys)) and abs(ys.sum() - 1) < 1e-14
    assert ms[0] == np.float64(np.float32(89.5)) and 1.0 <= ls[0] <= 50.0
    assert ys[0, 7] > 0.999


def pin_softmax_masked_rows(orc):
    x = np.full((2, 6), -np.inf, np.float32)
    x[1, [1, 4]] = [0.5, -1.25]
    y, m, l = orc.softmax_rows(x)
    assert np.all(y[0] == 0.0) and m[0] == -np.inf and l[0] == 0.0
    assert np.all(y[1][[0, 2, 3, 5]] == 0.0)
    close(y[1][[1, 4]], brute_softmax([0.5, -1.25]), 1e-15, what="partially masked row")


def pin_softmax_rows_selection(orc):
    gen = np.random.default_rng(13)
    x = (gen.standard_normal((9, 21)) * 3).astype(np.float32)
    y_all, m_all, l_all = orc.softmax_rows(x)
    sel = [8, 0, 3]
    y_s, m_s, l_s = orc.softmax_rows(x, rows=sel)
    assert np.array_equal(y_s, y_all[sel]) and np.array_equal(m_s, m_all[sel])
    for r in range(9):
        close(y_all[r], brute_softmax([float(t) for t in x[r]]), 1e-13, what=f"row {r}")


# ---------------------------------------------------------------------------
# the recurrence
# ---------------------------------------------------------------------------
def pin_recurrence_worked_example(orc):
    g = golden("p3_running_sum_2517.txt")
    row = floats(g["row"])
    m, l = orc.online_normalizer(np.array(row))
    assert list(m) == [float(g["step1_m"]), float(g["step2_m"]), float(g["step3_m"]),
                       float(g["step4_m"])]
    assert l[0] == float(g["step1_l"])
    assert round(l[1], 4) == float(g["step2_l_4dp"])
    assert round(math.exp(row[0] - row[1]), 4) == float(g["rescale_e^-3_4dp"])
    assert round(l[2] - l[1], 4) == float(g["added_e^-4_4dp"])
    assert round(l[3], 4) == float(g["final_l_4dp"])


def pin_recurrence_theorem(orc):
    gen = np.random.default_rng(21)
    for n in (1, 5, 40):
        s = gen.standard_normal(n) * 5
        m, l = orc.online_normalizer(s)
        for j in range(n):
            pref = [float(t) for t in s[:j + 1]]
            mj = max(pref)
            assert m[j] == mj
            close(l[j], math.fsum(math.exp(t - mj) for t in pref), 1e-13, what=f"l_{j + 1}")
            assert 1.0 <= l[j] <= j + 1 + 1e-12        # the bounds 1 <= l_j <= j
    # the final state is the definition's (m, l)
    s = (gen.standard_normal(64) * 4).astype(np.float32)
    m, l = orc.online_normalizer(s.astype(np.float64))
    _, m2, l2 = orc.softmax_rows(s[None, :])
    assert m[-1] == m2[0]
    close(l[-1], l2[0], 1e-13, what="recurrence end vs definition")
    # a masked (-inf) score at the start and in the middle changes nothing
    m3, l3 = orc.online_normalizer(np.array([-np.inf, 1.0, -np.inf, 2.0]))
    assert m3[0] == -np.inf and l3[0] == 0.0
    close(l3[-1], 1.0 + math.exp(-1.0), 1e-15, what="masked scores")


# ---------------------------------------------------------------------------
# summary triples and the merge
# ---------------------------------------------------------------------------
def _merged_l(orc, parts):
    """(m, l) after merging scalar summaries (d = 1, v = 0)."""
    pm = np.array([[p[0] for p in parts]], np.float32)
    pl = np.array([[p[1] for p in parts]], np.float32)
    po = np.zeros((1, len(parts), 1), np.float32)
    _, lse = orc.merge(pm, pl, po)
    m = max(p[0] for p in parts)
    return m, math.exp(lse[0] - m)


def pin_merge_worked_example(orc):
    g = golden("p3_merge_halves_2517.txt")
    a = floats(g["first_half"])
    b = floats(g["second_half"])
    ma, la, _ = orc.summary(np.array(a), np.zeros((2, 1)))
    mb, lb, _ = orc.summary(np.array(b), np.zeros((2, 1)))
    assert ma == float(g["first_m"]) and round(la, 4) == float(g["first_l_4dp"])
    assert mb == float(g["second_m"]) and round(lb, 4) == float(g["second_l_4dp"])
    assert round(la * math.exp(ma - mb), 4) == float(g["first_rescaled_4dp"])
    m, l = _merged_l(orc, [(ma, la), (mb, lb)])
    assert m == float(g["merged_m"]) and round(l, 4) == float(g["merged_l_4dp"])
    m, l = _merged_l(orc, [(mb, lb), (ma, la)])          # order makes no difference
    assert round(l, 4) == float(g["merged_l_4dp"])


def pin_summary_definition(orc):
    gen = np.random.default_rng(31)
    s = gen.standard_normal(12) * 3
    v = gen.standard_normal((12, 5))
    m, l, o = orc.summary(s, v)
    mx = max(float(t) for t in s)
    assert m == mx
    w = [math.exp(float(t) - mx) for t in s]
    close(l, math.fsum(w), 1e-14, what="summary l")
    close(o, [math.fsum(w[i] * float(v[i, c]) for i in range(12)) for c in range(5)], 1e-13,
          what="summary o~")
    m0, l0, o0 = orc.summary(np.array([]), np.zeros((0, 5)))
    assert m0 == -np.inf and l0 == 0.0 and np.all(o0 == 0.0)


def pin_merge_union(orc):
    """Merging the summaries of any split equals the union's result."""
    gen = np.random.default_rng(32)
    n, d = 37, 6
    s = gen.standard_normal(n) * 4
    v = gen.standard_normal((n, d))
    # brute force on the union, pure Python
    w = [math.exp(float(t)) for t in s]
    z = math.fsum(w)
    o_ref = [math.fsum(w[i] * float(v[i, c]) for i in range(n)) / z for c in range(d)]
    for k in (1, 2, 5, 9):
        idx = gen.permutation(n)
        cuts = np.sort(gen.choice(np.arange(1, n), size=k - 1, replace=False)) if k > 1 else []
        pieces = np.split(idx, cuts)
        pm, pl, po = [], [], []
        for piece in pieces:
            m, l, o = orc.summary(s[piece], v[piece])
            pm.append(m)
            pl.append(l)
            po.append(o)
        o, lse = orc.merge(np.array([pm], np.float32), np.array([pl], np.float32),
                           np.array([po], np.float32))
        close(o[0], o_ref, 2e-6, 1e-7, what=f"merge of {k} pieces")   # fp32 partials
        close(lse[0], math.log(z), 2e-7, what=f"merged lse, {k} pieces")
        # any order of the pieces gives the same result
        order = gen.permutation(len(pieces))
        o2, lse2 = orc.merge(np.array([pm], np.float32)[:, order],
                             np.array([pl], np.float32)[:, order],
                             np.array([po], np.float32)[:, order])
        close(o2, o, 1e-13, what="merge order")
        close(lse2, lse, 1e-14, what="merge order lse")


def pin_merge_identity(orc):
    """The empty set's summary (-inf, 0, anything) changes nothing; a row of
    empty pieces only gives o = 0, lse = -inf."""
    pm = np.array([[1.5, -np.inf, 0.25, -np.inf]], np.float32)
    pl = np.array([[2.0, 0.0, 3.0, 0.0]], np.float32)
    po = np.array([[[1.0, -2.0], [np.nan, np.inf], [0.5, 4.0], [np.nan, np.nan]]], np.float32)
    o, lse = orc.merge(pm, pl, po)
    ea, eb = 1.0, math.exp(0.25 - 1.5)
    lt = 2.0 * ea + 3.0 * eb
    close(o[0], [(1.0 * ea + 0.5 * eb) / lt, (-2.0 * ea + 4.0 * eb) / lt], 1e-15, what="identity")
    close(lse[0], 1.5 + math.log(lt), 1e-15, what="identity lse")
    o, lse = orc.merge(np.full((1, 3), -np.inf, np.float32), np.zeros((1, 3), np.float32),
                       np.full((1, 3, 2), np.nan, np.float32))
    assert np.all(o == 0.0) and lse[0] == -np.inf


def pin_merge_far_maxima(orc):
    """Pieces whose maxima are far apart still merge without overflow: every
    exponent is taken relative to the larger maximum, so none is positive."""
    pm = np.array([[0.0, 1000.0, -900.0]], np.float32)
    pl = np.array([[1.0, 2.0, 3.0]], np.float32)
    po = np.array([[[1.0], [4.0], [-6.0]]], np.float32)
    o, lse = orc.merge(pm, pl, po)
    assert np.all(np.isfinite(o)) and np.isfinite(lse[0])
    close(o[0], [2.0], 1e-15, what="far maxima")
    close(lse[0], 1000.0 + math.log(2.0), 1e-15, what="far maxima lse")


def pin_merge_lse(orc):
    """The log-sum-exp form: two disjoint halves' (o, lse) merge into the
    union's, and the two weights sum to 1."""
    gen = np.random.default_rng(33)
    n, d = 20, 4
    s = gen.standard_normal(n) * 3
    v = gen.standard_normal((n, d))
    halves = (np.arange(0, 8), np.arange(8, n))
    res = []
    for hv in halves:
        w = [math.exp(float(t)) for t in s[hv]]
        z = math.fsum(w)
        res.append(([math.fsum(w[i] * float(v[hv][i, c]) for i in range(len(hv))) / z
                     for c in range(d)], math.log(z)))
    (oa, la), (ob, lb) = res
    o, lse = orc.merge_lse(np.array([oa]), np.array([la]), np.array([ob]), np.array([lb]))
    w = [math.exp(float(t)) for t in s]
    z = math.fsum(w)
    close(lse[0], math.log(z), 1e-14, what="lse merge")
    close(o[0], [math.fsum(w[i] * float(v[i, c]) for i in range(n)) / z for c in range(d)],
          1e-13, what="o merge")
    close(math.exp(la - lse[0]) + math.exp(lb - lse[0]), 1.0, 1e-14, what="weights sum to 1")
    o, lse = orc.merge_lse(np.array([oa]), np.array([la]), np.zeros((1, d)),
                           np.array([-np.inf]))
    close(o[0], oa, 1e-15, what="empty piece")
    assert lse[0] == la


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def pin_attention_page_experiment(orc):
    """The single-query experiment: blocked recurrence vs naive, fp64."""
    g = golden("p1_online_vs_naive.txt")
    d, n, block = int(g["d"]), int(g["keys"]), int(g["block"])
    gen = np.random.default_rng(41)
    qv = gen.standard_normal(d).astype(np.float32)
    K = gen.standard_normal((n, d)).astype(np.float32)
    V = gen.standard_normal((n, d)).astype(np.float32)
    o, lse = orc.attention(qv.reshape(1, 1, 1, d), K.reshape(1, 1, n, d), V.reshape(1, 1, n, d),
                           scale=1.0)
    o_rec, lse_rec = blocked_recurrence_single_query(qv.astype(np.float64), K.astype(np.float64),
                                                     V.astype(np.float64), block)
    diff = float(np.max(np.abs(o[0, 0, 0] - o_rec)))
    assert diff <= 10 * float(g["max_abs_diff_order"]), diff
    assert abs(lse[0, 0, 0] - lse_rec) <= 1e-12


def _tiny(seed, B=2, Hq=4, Hkv=2, Nq=5, Nk=7, d=3, sigma=1.0):
    gen = np.random.default_rng(seed)
    q = (gen.standard_normal((B, Hq, Nq, d)) * sigma).astype(np.float32)
    k = (gen.standard_normal((B, Hkv, Nk, d)) * sigma).astype(np.float32)
    v = gen.standard_normal((B, Hkv, Nk, d)).astype(np.float32)
    return q, k, v


def pin_attention_brute_force(orc):
    q, k, v = _tiny(42)
    B, Hq, Nq, d = q.shape
    Nk = k.shape[2]
    for causal in (False, True):
        for lq, lk in (([Nq, Nq], [Nk, Nk]), ([3, 5], [6, 2]), ([0, 4], [7, 0])):
            o, lse = orc.attention(q, k, v, scale=0.37, causal=causal,
                                   seqlens_q=np.array(lq), seqlens_k=np.array(lk))
            o_ref, lse_ref = brute_attention(q, k, v, 0.37, causal, lq, lk, Hq // k.shape[1])
            close(o, o_ref, 1e-12, 1e-14, what=f"attention causal={causal} lq={lq} lk={lk}")
            close(lse, lse_ref, 1e-13, 1e-14, what="lse")
    # Hq == Hkv and NULL lengths
    o, lse = orc.attention(q, np.concatenate([k, k], 1), np.concatenate([v, v], 1), scale=1.0)
    o_ref, lse_ref = brute_attention(q, np.concatenate([k, k], 1), np.concatenate([v, v], 1),
                                     1.0, False, [Nq] * B, [Nk] * B, 1)
    close(o, o_ref, 1e-12, 1e-14, what="attention, no lengths")


def pin_attention_closed_forms(orc):
    gen = np.random.default_rng(43)
    d = 8
    # one key: o = v_0, lse = s_0
    q = gen.standard_normal((1, 1, 3, d)).astype(np.float32)
    k = gen.standard_normal((1, 1, 1, d)).astype(np.float32)
    v = gen.standard_normal((1, 1, 1, d)).astype(np.float32)
    o, lse = orc.attention(q, k, v, scale=0.5)
    close(o[0, 0], np.repeat(v[0, 0], 3, 0), 1e-15, what="one key")
    close(lse[0, 0], [0.5 * math.fsum(float(q[0, 0, i, c]) * float(k[0, 0, 0, c])
                                      for c in range(d)) for i in range(3)], 1e-14, 1e-15, "s_0")
    # all scores equal (K = 0): o = mean of the visible values, lse = ln n
    n = 11
    v = gen.standard_normal((1, 1, n, d)).astype(np.float32)
    o, lse = orc.attention(gen.standard_normal((1, 1, 2, d)).astype(np.float32),
                           np.zeros((1, 1, n, d), np.float32), v, scale=1.0,
                           seqlens_k=np.array([9]))
    close(o[0, 0], np.repeat(v[0, 0, :9].astype(np.float64).mean(0, keepdims=True), 2, 0), 1e-14,
          1e-15, what="mean of values")
    close(lse[0, 0], [math.log(9)] * 2, 1e-15, what="ln n")
    # V = identity: rows of O are the softmax weights
    q = gen.standard_normal((1, 1, 4, d)).astype(np.float32)
    k = gen.standard_normal((1, 1, d, d)).astype(np.float32)
    o, _ = orc.attention(q, k, np.eye(d, dtype=np.float32).reshape(1, 1, d, d), scale=1.0)
    for i in range(4):
        s = [math.fsum(float(q[0, 0, i, c]) * float(k[0, 0, j, c]) for c in range(d))
             for j in range(d)]
        close(o[0, 0, i], brute_softmax(s), 1e-13, what="V = I")
    # causal: query 0 sees key 0 only
    q, k, v = _tiny(44, B=1, Hq=1, Hkv=1, Nq=6, Nk=6, d=4)
    o, lse = orc.attention(q, k, v, scale=1.0, causal=True)
    close(o[0, 0, 0], v[0, 0, 0], 1e-15, what="causal row 0")
    # non-causal: permuting keys and values together changes nothing
    perm = gen.permutation(6)
    o1, l1 = orc.attention(q, k, v, scale=0.7)
    o2, l2 = orc.attention(q, k[:, :, perm], v[:, :, perm], scale=0.7)
    close(o2, o1, 1e-13, 1e-15, what="key permutation")
    close(l2, l1, 1e-14, what="key permutation lse")


def pin_attention_masks(orc):
    """NaN poison at padded positions is never read; padded query rows are
    exactly 0 / -inf; future keys do not affect a causal row."""
    q, k, v = _tiny(45, B=2, Hq=2, Hkv=1, Nq=6, Nk=6, d=4)
    lens = np.array([4, 6])
    qp, kp, vp = q.copy(), k.copy(), v.copy()
    qp[0, :, 4:] = np.nan
    kp[0, :, 4:] = np.nan
    vp[0, :, 4:] = np.inf
    qz, kz, vz = q.copy(), k.copy(), v.copy()
    qz[0, :, 4:] = 0
    kz[0, :, 4:] = 0
    vz[0, :, 4:] = 0
    for causal in (False, True):
        o1, l1 = orc.attention(qp, kp, vp, scale=0.5, causal=causal, seqlens_q=lens,
                               seqlens_k=lens)
        o2, l2 = orc.attention(qz, kz, vz, scale=0.5, causal=causal, seqlens_q=lens,
                               seqlens_k=lens)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        assert np.all(o1[0, :, 4:] == 0.0) and np.all(l1[0, :, 4:] == -np.inf)
        assert np.all(np.isfinite(o1))
    o1, l1 = orc.attention(q, k, v, scale=0.5, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 4:] = 100.0
    v2[:, :, 4:] = -7.0
    o2, l2 = orc.attention(q, k2, v2, scale=0.5, causal=True)
    assert np.array_equal(o1[:, :, :4], o2[:, :, :4]) and np.array_equal(l1[:, :, :4],
                                                                          l2[:, :, :4])
    assert not np.array_equal(o1[:, :, 5], o2[:, :, 5])


def pin_attention_lse_rebuilds_weights(orc):
    """y_j = exp(s_j - lse) are the weights: they sum to 1 and rebuild o."""
    q, k, v = _tiny(46, B=1, Hq=2, Hkv=2, Nq=3, Nk=9, d=5, sigma=2.0)
    o, lse = orc.attention(q, k, v, scale=0.3)
    for h in range(2):
        for i in range(3):
            s = [0.3 * math.fsum(float(q[0, h, i, c]) * float(k[0, h, j, c]) for c in range(5))
                 for j in range(9)]
            y = [math.exp(t - lse[0, h, i]) for t in s]
            close(math.fsum(y), 1.0, 1e-14, what="weights sum")
            close(o[0, h, i], [math.fsum(y[j] * float(v[0, h, j, c]) for j in range(9))
                               for c in range(5)], 1e-13, 1e-15, what="rebuilt o")


def pin_attention_row_selection(orc):
    q, k, v = _tiny(47, B=2, Hq=4, Hkv=2, Nq=5, Nk=7, d=3)
    o, lse = orc.attention(q, k, v, scale=0.5, causal=True, seqlens_q=np.array([5, 3]),
                           seqlens_k=np.array([7, 4]))
    rows = np.array([0, 13, 39, 22, 5])
    o_s, lse_s = orc.attention(q, k, v, scale=0.5, causal=True, seqlens_q=np.array([5, 3]),
                               seqlens_k=np.array([7, 4]), rows=rows)
    assert np.array_equal(o_s, o.reshape(-1, 3)[rows])
    assert np.array_equal(lse_s, lse.reshape(-1)[rows])


def pin_merge_of_attention_pieces(orc):
    """Decode by pieces: summaries of 64-key pieces of one query's keys,
    merged, equal the oracle's unsplit attention (the split the GPU decode
    path takes)."""
    gen = np.random.default_rng(48)
    d, n, piece = 16, 300, 64
    qv = gen.standard_normal(d).astype(np.float32)
    K = gen.standard_normal((n, d)).astype(np.float32)
    V = gen.standard_normal((n, d)).astype(np.float32)
    o_ref, lse_ref = orc.attention(qv.reshape(1, 1, 1, d), K.reshape(1, 1, n, d),
                                   V.reshape(1, 1, n, d), scale=0.25)
    pm, pl, po = [], [], []
    for start in range(0, 384, piece):
        sl = slice(start, min(start + piece, n))
        s = (K[sl].astype(np.float64) @ qv.astype(np.float64)) * 0.25
        m, l, o = orc.summary(s, V[sl].astype(np.float64))
        pm.append(m)
        pl.append(l)
        po.append(o)
    o, lse = orc.merge(np.array([pm], np.float32), np.array([pl], np.float32),
                       np.array([po], np.float32))
    close(o[0], o_ref[0, 0, 0], 2e-6, 1e-7, what="pieces merged")
    close(lse[0], lse_ref[0, 0, 0], 2e-7, what="pieces lse")


# ---------------------------------------------------------------------------
# backward: the derivative of the forward definition (the pages print none)
# ---------------------------------------------------------------------------
_BWD_MASKS = [  # (causal, seqlens_q, seqlens_k) for B = 2
    (False, None, None),
    (True, None, None),
    (True, [5, 3], [7, 4]),
    (False, [0, 4], [6, 0]),
]


def _dyadic(gen, shape, step=2.0 ** -6, bound=2.0):
    """Values that are multiples of ``step`` in [-bound, bound): a nudge by a
    power of two no larger than ``step`` stays exact in fp32."""
    return (np.round(gen.uniform(-bound, bound, shape) / step) * step).astype(np.float32)


def pin_attention_bwd_finite_differences(orc):
    """Each gradient entry against central differences of the loss
    L = sum(dO * O) computed by the forward oracle, Richardson-extrapolated
    (error O(h^4)); inputs are dyadic so every nudged input is exact."""
    gen = np.random.default_rng(50)
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 5, 7, 3
    q = _dyadic(gen, (B, Hq, Nq, d))
    k = _dyadic(gen, (B, Hkv, Nk, d))
    v = _dyadic(gen, (B, Hkv, Nk, d))
    do = _dyadic(gen, (B, Hq, Nq, d))
    scale = 0.625
    h = 2.0 ** -9
    for causal, lq, lk in _BWD_MASKS:
        sq = None if lq is None else np.array(lq)
        sk = None if lk is None else np.array(lk)

        def loss(qq, kk, vv):
            o, _ = orc.attention(qq, kk, vv, scale=scale, causal=causal, seqlens_q=sq,
                                 seqlens_k=sk)
            return math.fsum((o * do.astype(np.float64)).ravel())

        dq, dk, dv = orc.attention_bwd(q, k, v, do, scale=scale, causal=causal,
                                       seqlens_q=sq, seqlens_k=sk)
        for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            fd = np.empty(x.shape)
            for idx in np.ndindex(x.shape):
                def central(step):
                    xp, xm = x.copy(), x.copy()
                    xp[idx] += step
                    xm[idx] -= step
                    args_p = [xp if name == n else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
                    args_m = [xm if name == n else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
                    return (loss(*args_p) - loss(*args_m)) / (2 * step)
                fd[idx] = (4 * central(h / 2) - central(h)) / 3
            close(g, fd, 1e-7, 1e-9, what=f"{name} causal={causal} lq={lq} lk={lk}")


def pin_attention_bwd_autograd(orc):
    """Against fp64 reverse-mode autodiff (torch, CPU) of a forward written
    here row by row over the visible keys only."""
    import torch
    gen = np.random.default_rng(51)
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 9, 11, 5
    group = Hq // Hkv
    q, k, v = (gen.standard_normal(s).astype(np.float32)
               for s in ((B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)))
    do = gen.standard_normal((B, Hq, Nq, d)).astype(np.float32)
    scale = 0.41
    for causal, lq, lk in ((False, [9, 9], [11, 11]), (True, [9, 9], [11, 11]),
                           (True, [7, 2], [9, 5]), (False, [9, 0], [3, 11])):
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        tdo = torch.tensor(do, dtype=torch.float64)
        loss = torch.zeros((), dtype=torch.float64)
        for b in range(B):
            for hh in range(Hq):
                g = hh // group
                for i in range(min(lq[b], Nq)):
                    n = min(lk[b], i + 1) if causal else lk[b]
                    if n == 0:
                        continue
                    w = torch.softmax(scale * (tk[b, g, :n] @ tq[b, hh, i]), 0)
                    loss = loss + torch.dot(w @ tv[b, g, :n], tdo[b, hh, i])
        loss.backward()
        dq, dk, dv = orc.attention_bwd(q, k, v, do, scale=scale, causal=causal,
                                       seqlens_q=np.array(lq), seqlens_k=np.array(lk))
        for name, got, ref in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
            close(got, ref.numpy(), 1e-12, 1e-14, what=f"{name} causal={causal} lq={lq} lk={lk}")


def pin_attention_bwd_invariants(orc):
    """Each visible row's score gradients sum to zero (softmax is shift
    invariant), so the key gradients of a head sum to zero; each visible row's
    weights sum to one, so the value gradients of a head sum to the output
    gradients of the rows that see any key; padded rows get exact zeros."""
    gen = np.random.default_rng(52)
    B, Hq, Hkv, Nq, Nk, d = 2, 6, 2, 13, 10, 4
    q, k, v = (gen.standard_normal(s).astype(np.float32)
               for s in ((B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)))
    do = gen.standard_normal((B, Hq, Nq, d)).astype(np.float32)
    lq, lk = np.array([11, 13]), np.array([10, 6])
    for causal in (False, True):
        dq, dk, dv = orc.attention_bwd(q, k, v, do, scale=0.5, causal=causal, seqlens_q=lq,
                                       seqlens_k=lk)
        for b in range(B):
            for g in range(Hkv):
                close(dk[b, g].sum(0), np.zeros(d), 0, 1e-13, what="sum of dk")
                seen = [(hh, i) for hh in range(3 * g, 3 * g + 3) for i in range(lq[b])
                        if (min(lk[b], i + 1) if causal else lk[b]) > 0]
                want = np.sum([do[b, hh, i].astype(np.float64) for hh, i in seen], 0)
                close(dv[b, g].sum(0), want, 1e-13, 1e-13, what="sum of dv")
            assert np.all(dq[b, :, lq[b]:] == 0.0)
            assert np.all(dk[b, :, lk[b]:] == 0.0) and np.all(dv[b, :, lk[b]:] == 0.0)


def pin_attention_bwd_one_key(orc):
    """One visible key: the weight is 1 whatever the scores, so dq = dk = 0
    and dv_0 is the sum of the output gradients of every row of the group."""
    gen = np.random.default_rng(53)
    q = gen.standard_normal((1, 2, 4, 6)).astype(np.float32)
    k = gen.standard_normal((1, 1, 1, 6)).astype(np.float32)
    v = gen.standard_normal((1, 1, 1, 6)).astype(np.float32)
    do = gen.standard_normal((1, 2, 4, 6)).astype(np.float32)
    dq, dk, dv = orc.attention_bwd(q, k, v, do, scale=0.9)
    close(dq, np.zeros_like(dq), 0, 1e-15, what="dq")
    close(dk, np.zeros_like(dk), 0, 1e-15, what="dk")
    close(dv[0, 0, 0], do[0].reshape(-1, 6).astype(np.float64).sum(0), 1e-14, 1e-15, what="dv")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
