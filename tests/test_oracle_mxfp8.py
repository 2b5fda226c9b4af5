"""Pins of the MXFP8 oracle (CPU): each check ties it to something other than
itself -- the E4M3 field definition and known values, brute force over every finite
E4M3 value, the scale rule's defining inequality, exact reduction to the dense
oracle when P is exactly representable, invariance under integer score shifts, and
the quantization error bound against the dense oracle.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import mxfp8 as mx


def _finite_table():
    vals = {}
    for c in range(256):
        v = mx.e4m3_value(c)
        if not math.isnan(v):
            vals[c] = v
    return vals


def test_e4m3_table_known_values():
    t = _finite_table()
    assert len(t) == 254                                     # two NaN codes, no infinities
    assert math.isnan(mx.e4m3_value(0x7F)) and math.isnan(mx.e4m3_value(0xFF))
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in known.items():
        assert t[c] == v, hex(c)
    pos = [t[c] for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))          # monotone in the code
    # the positive finite set in closed form: subnormals k 2^-9 and normals (8+m) 2^(E-3)
    closed = {k * 2.0 ** -9 for k in range(8)}
    closed |= {(8 + m) * 2.0 ** (E - 3) for E in range(-6, 9) for m in range(8)}
    closed.discard(15 * 2.0 ** 5)                            # S.1111.111 is NaN, not 480
    assert set(pos) == closed


def _brute_round(y, table):
    best = min(table.values(), key=lambda v: abs(v - y))
    ties = [c for c, v in table.items() if abs(v - y) == abs(best - y)]
    if len({table[c] for c in ties}) > 1:                    # a true tie: even mantissa
        ties = [c for c in ties if c % 2 == 0]
    return table[ties[0]]


def test_e4m3_round_against_brute_force():
    t = _finite_table()
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-12, np.log2(448.0), 3000))
    ys = list(mags * rng.choice([-1.0, 1.0], 3000))
    vals = sorted(v for v in t.values() if v >= 0)
    ys += [(a + b) / 2 for a, b in zip(vals, vals[1:])]      # every tie
    ys += [-(a + b) / 2 for a, b in zip(vals, vals[1:])]
    ys += [0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -11, 440.0, 447.9]
    got = mx.e4m3_round(np.array(ys))
    for y, g in zip(ys, got):
        assert g == _brute_round(y, t), y
    with pytest.raises(ValueError):
        mx.e4m3_round(np.array([449.0]))


def test_scale_rule_is_the_smallest_non_saturating_power_of_two():
    rng = np.random.default_rng(1)
    a = np.exp2(rng.uniform(-100, 100, 5000)) * rng.uniform(1, 2, 5000)
    a = np.concatenate([a, [448.0, 448.0 * 2.0 ** -20, 224.0, 1.75, 1.0, 0.875]])
    e = mx.scale_exponent(a)
    assert np.all(a <= 448.0 * np.ldexp(1.0, e))
    assert np.all(a > 448.0 * np.ldexp(1.0, e - 1))
    assert mx.scale_exponent(np.array([0.0]))[0] == -127
    assert mx.scale_exponent(np.array([1e-45]))[0] == -127   # clamped to the E8M0 range
    assert mx.scale_exponent(np.array([448.0]))[0] == 0


def test_quantize_rows_by_explicit_blocks():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 2, 64)) * np.exp2(rng.integers(-6, 6, (5, 2, 64)))
    deq, codes = mx.quantize_rows(x)
    assert codes.shape == (5, 2, 2)
    for r in range(5):
        for h in range(2):
            for blk in range(2):
                xs = x[r, h, 32 * blk:32 * blk + 32]
                e = codes[r, h, blk] - 127
                assert np.abs(xs).max() <= 448 * 2.0 ** e and np.abs(xs).max() > 224 * 2.0 ** e
                want = [_brute_round(v / 2.0 ** e, _finite_table()) * 2.0 ** e for v in xs[:6]]
                assert np.array_equal(deq[r, h, 32 * blk:32 * blk + 6], want)
    # relative error of the rounding: half an E4M3 step
    s = np.repeat(np.ldexp(1.0, codes - 127), 32, axis=-1)
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) + 1e-300)
    # quantizing the quantized values changes no value (a block maximum that rounded
    # down onto 224 * 2^e may take the next smaller scale)
    deq2, codes2 = mx.quantize_rows(deq)
    assert np.array_equal(deq2, deq)
    assert np.all((codes2 == codes) | (codes2 == codes - 1))
    with pytest.raises(ValueError):
        mx.quantize_rows(np.zeros((2, 1, 48)))


def test_quantize_v_blocks_follow_sequences():
    rng = np.random.default_rng(3)
    lengths = [1, 31, 32, 33, 70, 0, 5]
    off = np.concatenate([[0], np.cumsum(lengths)])
    v = rng.standard_normal((off[-1], 2, 32))
    # one sequence with values 2^20 larger: its scales must not leak into neighbours
    v[off[4]:off[5]] *= 2.0 ** 20
    deq, scales = mx.quantize_v(v, off)
    for b, n in enumerate(lengths):
        a = off[b]
        assert scales[b].shape == ((n + 31) // 32, 2, 32)
        sub_deq, sub_scales = mx.quantize_v(v[a:a + n], np.array([0, n]))
        assert np.array_equal(deq[a:a + n], sub_deq) and np.array_equal(scales[b], sub_scales[0])
        for j in range((n + 31) // 32):
            blk = v[a + 32 * j:a + min(n, 32 * j + 32)]                # [keys, H, D]
            e = scales[b][j] - 127
            amax = np.abs(blk).max(axis=0)
            assert np.all(amax <= 448 * np.ldexp(1.0, e)) and np.all(amax > 224 * np.ldexp(1.0, e))
    assert np.all(scales[3] < scales[4].min())


def _integer_case(rng, n, r, d=32):
    """Q rows a_i * e_{c_i}, K entries in [-2, 2]: integer scores in [-6, 6], so with
    c = ln 2 every p is an exact power of two within 2^-12 of its block maximum."""
    q = np.zeros((r, d))
    q[np.arange(r), rng.integers(0, d, r)] = rng.integers(0, 4, r)
    k = rng.integers(-2, 3, (n, d)).astype(np.float64)
    return q, k


@pytest.mark.parametrize("causal", [False, True])
def test_exact_powers_of_two_reduce_to_the_dense_oracle(causal):
    rng = np.random.default_rng(4)
    n = 150
    q, k = _integer_case(rng, n, n)
    v = rng.standard_normal((n, 1, 32))
    vd, _ = mx.quantize_v(v, np.array([0, n]))
    qd, _ = mx.quantize_rows(q[:, None, :])
    kd, _ = mx.quantize_rows(k[:, None, :])
    assert np.array_equal(qd[:, 0], q) and np.array_equal(kd[:, 0], k)
    o, lse, slack = mx.sequence_forward_mx(q, k, vd[:, 0], math.log(2.0), causal)
    o_ref, lse_ref = oracle.sequence_forward(q, k, vd[:, 0], math.log(2.0), causal)
    assert np.abs(o - o_ref).max() <= 1e-12
    assert np.abs(lse - lse_ref).max() <= 1e-12


@pytest.mark.parametrize("broadcast_q,causal", [(True, False), (False, False), (False, True)])
def test_batch_assembly_reduces_to_the_dense_oracle(broadcast_q, causal):
    rng = np.random.default_rng(5)
    lengths = [3, 0, 40, 97]
    off = np.concatenate([[0], np.cumsum(lengths)])
    heads, d, lq = 2, 64, 20
    q = np.zeros((lq if broadcast_q else off[-1], heads, d))
    idx = rng.integers(0, d, q.shape[:2])
    q[np.arange(q.shape[0])[:, None], np.arange(heads)[None, :], idx] = rng.integers(0, 4, q.shape[:2])
    k = rng.integers(-2, 3, (off[-1], heads, d)).astype(np.float64)
    v = rng.standard_normal((off[-1], heads, d))
    o, lse, _ = mx.forward_mx(q, k, v, off, broadcast_q=broadcast_q, causal=causal, scale=math.log(2.0))
    vd, _ = mx.quantize_v(v, off)
    o_ref, lse_ref = oracle.forward(q, k, vd, off, broadcast_q=broadcast_q, causal=causal,
                                    scale=math.log(2.0))
    assert np.abs(o - o_ref).max() <= 1e-12
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= 1e-12


def test_integer_score_shift_changes_nothing():
    rng = np.random.default_rng(6)
    x = (rng.integers(-3000, 3000, (40, 130)) / 256.0).astype(np.float32)   # exact in fp32
    x[:, 100:] = -np.inf                                    # masked keys
    v = rng.standard_normal((130, 16))
    o0, l0, _ = mx.attend_base2(x, v)
    for t in (1.0, -7.0, 13.0):
        o1, l1, _ = mx.attend_base2(x + np.float32(t), v)
        assert np.array_equal(o1, o0)
        assert np.allclose(l1, l0 + t, rtol=0, atol=1e-12)
    # a non-integer shift moves the quantization grid: results differ
    o2, _, _ = mx.attend_base2(x + np.float32(0.375), v)
    assert not np.array_equal(o2, o0)


def test_p_quantization_error_bound_against_dense():
    rng = np.random.default_rng(7)
    n, r, d = 300, 64, 128
    q = rng.standard_normal((r, 1, d))
    k = rng.standard_normal((n, 1, d))
    v = rng.standard_normal((n, 1, d))
    c = 1 / math.sqrt(d)
    qd, _ = mx.quantize_rows(q)
    kd, _ = mx.quantize_rows(k)
    vd, _ = mx.quantize_v(v, np.array([0, n]))
    o, lse, _ = mx.sequence_forward_mx(qd[:, 0], kd[:, 0], vd[:, 0], c)
    o_d, lse_d = oracle.sequence_forward(qd[:, 0], kd[:, 0], vd[:, 0], c)
    # |q(p) - p| <= 2^-4 p (normal range) or 2^-10 2^e (subnormal range), per key
    x = mx.base2_scores(qd[:, 0], kd[:, 0], c)
    m = np.ceil(x.max(axis=1).astype(np.float64))
    p = np.exp2(x.astype(np.float64) - m[:, None])
    _, e, _ = mx.quantize_p(p.astype(np.float32))
    s = np.repeat(np.ldexp(1.0, e), 32, axis=1)[:, :n]
    vmax = np.abs(vd[:, 0]).max(axis=1)
    bound = ((2.0 ** -4 * p + 2.0 ** -10 * s) * vmax[None, :]).sum(axis=1) / p.sum(axis=1)
    err = np.abs(o - o_d).max(axis=1)
    assert np.all(err <= bound * (1 + 1e-3) + 1e-6)
    assert np.abs(lse - lse_d).max() <= 1e-5                 # fp32 scores only
    assert err.max() > 0                                       # P is really quantized


def test_empty_and_slack():
    o, lse, slack = mx.sequence_forward_mx(np.ones((3, 32)), np.zeros((0, 32)), np.zeros((0, 32)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse)) and np.all(slack == 0)
    # a value placed exactly on a rounding tie is reported with a positive slack
    x = np.zeros((1, 2), dtype=np.float32)
    x[0, 1] = np.float32(np.log2(1.0625))                     # p = 1.0625 / 2: y on a tie
    _, _, slack = mx.attend_base2(x, np.ones((2, 4)))
    assert slack[0] > 0


def test_worked_example_by_hand():
    """One row, two keys, base-2 scores x = (0.5, -0.25), worked by hand:
    m = ceil(0.5) = 1, p = (2^-0.5, 2^-1.25) = (0.7071068, 0.4204482);
    block max 0.7071 -> e = -9 (448 * 2^-9 = 0.875 >= 0.7071 > 0.4375);
    y = 512 p = (362.04, 215.27) -> nearest E4M3 (352, 208) (steps 32 and 16);
    deq P = (0.6875, 0.40625); l = 1.1275550 (unquantized);
    O = deq P . V / l with V = I: (0.6097264, 0.3602928); LSE2 = 1 + log2 l.
    (With m = max x = 0.5 instead the quantized weights would be (1, 0.59375).)"""
    x = np.array([[0.5, -0.25]], dtype=np.float32)
    o, lse2, _ = mx.attend_base2(x, np.eye(2))
    l = 2 ** -0.5 + 2 ** -1.25
    assert np.allclose(o[0], [0.6875 / l, 0.40625 / l], rtol=1e-7, atol=0)
    assert np.allclose(o[0], [0.6097264, 0.3602928], rtol=0, atol=1e-6)
    assert abs(lse2[0] - (1 + math.log2(l))) <= 1e-7


# ---- the slack (sensitivity of P's rounding decisions) ----------------------------

def _e4m3_positive_values():
    """Finite non-negative E4M3 values from the field definition: subnormals k 2^-9
    (k = 0..7) and normals (1 + m / 8) 2^(e - 7), e = 1..15, except e = 15, m = 7."""
    vals = [k * 2.0 ** -9 for k in range(8)]
    vals += [(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8) if not (e == 15 and m == 7)]
    return np.array(sorted(vals))


def _decisions(x, rel=2.0 ** -12):
    """Brute-force rounding decisions of P for one row of fp32 base-2 scores x: p in
    fp32, block exponents e by search, y = p / 2^e, and for every element its two
    E4M3 neighbours; flags near a rounding midpoint, and blocks whose maximum is near
    a scale boundary (448 2^e or 448 2^(e - 1))."""
    table = _e4m3_positive_values()
    x = np.asarray(x, dtype=np.float32)
    m = np.float32(np.ceil(np.float64(x.max())))
    p = np.exp2((x - m).astype(np.float32)).astype(np.float32).astype(np.float64)
    n = len(p)
    e = np.zeros(n, dtype=np.int64)
    edge = np.zeros(n, dtype=bool)
    for j0 in range(0, n, 32):
        blk = p[j0:j0 + 32]
        amax = blk.max()
        ee = -127
        while amax > 448.0 * 2.0 ** ee:
            ee += 1
        e[j0:j0 + 32] = ee
        near = lambda a, b: abs(a - b) <= rel * max(abs(a), abs(b))   # noqa: E731
        edge[j0:j0 + 32] = (near(amax, 448.0 * 2.0 ** ee) or near(amax, 448.0 * 2.0 ** (ee - 1))) and amax > 0
    y = p / np.ldexp(1.0, e)
    hi_i = np.searchsorted(table, y, side="left")
    lo = table[np.maximum(hi_i - 1, 0)]
    hi = table[np.minimum(hi_i, len(table) - 1)]
    lo = np.where(table[np.minimum(hi_i, len(table) - 1)] == y, y, lo)   # exactly representable
    mid = 0.5 * (lo + hi)
    tie = (np.abs(y - mid) <= rel * np.maximum(np.abs(y), np.abs(mid))) & (p > 0) & (lo != hi)
    return p, e, y, lo, hi, tie, edge & (p > 0)


def _o_from(pd, v, l):
    return (pd @ v) / l


def test_slack_is_zero_exactly_when_no_decision_is_near_a_tie():
    """Random rows: the slack is exactly 0 on every row whose rounding decisions are
    all clear of a tie and of a scale boundary (found by brute force over the E4M3
    values), and positive on every row with such a decision."""
    rng = np.random.default_rng(11)
    n, d = 70, 8
    v = rng.standard_normal((n, d))
    rows = [rng.standard_normal(n).astype(np.float32) * 3 for _ in range(40)]
    # rows with a planted near-tie: p = 2^(x - m) lands within fp32 rounding of 1.0625 / 2
    for k in range(6):
        x = rng.standard_normal(n).astype(np.float32) - 4.0
        x[k] = np.float32(np.log2(1.0625))
        rows.append(x)
    zero_rows = flagged_rows = 0
    for x in rows:
        _, _, slack = mx.attend_base2(x[None, :], v)
        _, _, _, _, _, tie, edge = _decisions(x)
        if tie.any() or edge.any():
            assert slack[0] > 0
            flagged_rows += 1
        else:
            assert slack[0] == 0.0
            zero_rows += 1
    assert zero_rows >= 30 and flagged_rows >= 6


def test_slack_bounds_every_flipped_decision():
    """Every flagged decision taken the other way (the other E4M3 neighbour for a
    near-tie, the neighbouring block exponent for a near-boundary scale), one at a
    time and all together, moves O by no more than the slack, and a flip of a
    near-tie does move O."""
    rng = np.random.default_rng(12)
    n, d = 90, 6
    v = rng.standard_normal((n, d))
    x = (rng.standard_normal(n) - 3.0).astype(np.float32)
    x[3] = np.float32(np.log2(1.0625))          # near-tie in block 0 (p close to 0.53125)
    x[40] = np.float32(np.log2(1.0625))         # near-tie in block 1
    x[70] = np.float32(np.log2(1.8125))         # another binade's midpoint (y near 464 / 2 ...)
    o, _, slack = mx.attend_base2(x[None, :], v)
    p, e, y, lo, hi, tie, edge = _decisions(x)
    assert tie.sum() >= 2
    scale = np.ldexp(1.0, e)
    q = np.where(np.abs(y - lo) < np.abs(y - hi), lo, hi)
    q = np.where(np.abs(y - lo) == np.abs(y - hi), mx.e4m3_round(y), q)
    pd = q * scale
    l = p.sum()
    np.testing.assert_allclose(_o_from(pd, v, l), o[0], rtol=0, atol=1e-12)   # the same decisions
    flips = []
    for j in np.nonzero(tie)[0]:
        alt = pd.copy()
        alt[j] = (lo[j] if q[j] == hi[j] else hi[j]) * scale[j]
        flips.append(alt)
    for j0 in sorted({int(j) // 32 * 32 for j in np.nonzero(edge)[0]}):
        for de in (-1, 1):
            alt = pd.copy()
            s2 = np.ldexp(1.0, e[j0] + de)
            yy = np.minimum(p[j0:j0 + 32] / s2, 448.0)
            alt[j0:j0 + 32] = mx.e4m3_round(yy) * s2
            flips.append(alt)
    assert flips
    moved = 0.0
    for alt in flips:
        delta = np.abs(_o_from(alt, v, l) - o[0]).max()
        assert delta <= slack[0] * (1 + 1e-9)
        moved = max(moved, delta)
    assert moved > 0
    all_flipped = pd.copy()
    for j in np.nonzero(tie)[0]:
        all_flipped[j] = (lo[j] if q[j] == hi[j] else hi[j]) * scale[j]
    assert np.abs(_o_from(all_flipped, v, l) - o[0]).max() <= slack[0] * (1 + 1e-9)


def test_slack_of_a_single_tie_is_that_flip_exactly():
    """With one near-tie and no near-boundary scale in a row, flipping that one
    decision moves O by exactly the slack (so the slack is not loose)."""
    rng = np.random.default_rng(13)
    n, d = 50, 5
    v = rng.standard_normal((n, d))
    x = (rng.standard_normal(n) - 5.0).astype(np.float32)
    x[7] = np.float32(np.log2(1.0625))
    _, _, slack = mx.attend_base2(x[None, :], v)
    p, e, y, lo, hi, tie, edge = _decisions(x)
    assert tie.sum() == 1 and not edge.any()
    j = int(np.nonzero(tie)[0][0])
    step = (hi[j] - lo[j]) * np.ldexp(1.0, e[j])
    delta = step * np.abs(v[j]).max() / p.sum()
    assert abs(slack[0] - delta) <= 1e-12 * delta
