"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a padded
dense library reference (torch's scaled_dot_product_attention in fp64 with
autograd), central finite differences, closed forms, a hand-derived worked
example, and exact identities of softmax attention.  A plausible slip in the
oracle (dropped scale, wrong sign, transposed operand, wrong causal direction,
wrong LSE base, missing batch sum of the shared dQ, off-by-one offsets) fails
at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, lengths, h, d, broadcast_q, lq):
    t = int(sum(lengths))
    q = rng.standard_normal((lq if broadcast_q else t, h, d))
    k = rng.standard_normal((t, h, d))
    v = rng.standard_normal((t, h, d))
    rows = len(lengths) * lq if broadcast_q else t
    g = rng.standard_normal((rows, h, d))
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, v, g, off


def _padded_reference(q, k, v, g, off, broadcast_q, causal, scale):
    """Padded dense masked attention via torch SDPA (fp64, CPU) + autograd."""
    b = len(off) - 1
    h, d = k.shape[1], k.shape[2]
    lens = np.diff(off)
    lmax = int(lens.max())
    lq = q.shape[0] if broadcast_q else lmax
    kp = torch.zeros(b, h, lmax, d, dtype=torch.float64)
    vp = torch.zeros(b, h, lmax, d, dtype=torch.float64)
    gp = torch.zeros(b, h, lq, d, dtype=torch.float64)
    mask = torch.zeros(b, 1, lq, lmax, dtype=torch.bool)
    if broadcast_q:
        qsh = torch.tensor(q, dtype=torch.float64).permute(1, 0, 2).contiguous().requires_grad_(True)
        qp = qsh.unsqueeze(0).expand(b, h, lq, d)
    else:
        qp0 = torch.zeros(b, h, lq, d, dtype=torch.float64)
    for i in range(b):
        a, e = int(off[i]), int(off[i + 1])
        n = e - a
        kp[i, :, :n] = torch.tensor(k[a:e]).permute(1, 0, 2)
        vp[i, :, :n] = torch.tensor(v[a:e]).permute(1, 0, 2)
        if broadcast_q:
            gp[i] = torch.tensor(g[i * lq:(i + 1) * lq]).permute(1, 0, 2)
            mask[i, 0, :, :n] = True
        else:
            qp0[i, :, :n] = torch.tensor(q[a:e]).permute(1, 0, 2)
            gp[i, :, :n] = torch.tensor(g[a:e]).permute(1, 0, 2)
            vis = torch.ones(lq, lmax, dtype=torch.bool)
            vis[:, n:] = False
            if causal:
                vis &= torch.tril(torch.ones(lq, lmax, dtype=torch.bool))
            mask[i, 0] = vis
            mask[i, 0, n:, :] = False
            mask[i, 0, n:, 0] = True  # padded query rows: keep finite, discarded below
    if not broadcast_q:
        qp = qp0.requires_grad_(True)
    kp.requires_grad_(True)
    vp.requires_grad_(True)
    o = F.scaled_dot_product_attention(qp, kp, vp, attn_mask=mask, scale=scale)
    scores = (qp @ kp.transpose(-1, -2)) * scale
    lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
    (o * gp).sum().backward()
    rows = b * lq if broadcast_q else int(off[-1])
    o_ref = np.zeros((rows, h, d))
    lse_ref = np.zeros((h, rows))
    dk_ref = np.zeros_like(k)
    dv_ref = np.zeros_like(v)
    dq_ref = np.zeros_like(q)
    for i in range(b):
        a, e = int(off[i]), int(off[i + 1])
        n = e - a
        r0, r1 = (i * lq, (i + 1) * lq) if broadcast_q else (a, e)
        nr = lq if broadcast_q else n
        o_ref[r0:r1] = o[i, :, :nr].permute(1, 0, 2).detach().numpy()
        lse_ref[:, r0:r1] = lse[i, :, :nr].detach().numpy()
        dk_ref[a:e] = kp.grad[i, :, :n].permute(1, 0, 2).numpy()
        dv_ref[a:e] = vp.grad[i, :, :n].permute(1, 0, 2).numpy()
        if not broadcast_q:
            dq_ref[a:e] = qp.grad[i, :, :n].permute(1, 0, 2).numpy()
    if broadcast_q:
        dq_ref = qsh.grad.permute(1, 0, 2).numpy()
    return o_ref, lse_ref, dq_ref, dk_ref, dv_ref


MODES = [(True, False), (False, False), (False, True)]  # (broadcast_q, causal)


@pytest.mark.parametrize("broadcast_q,causal", MODES)
@pytest.mark.parametrize("seed", [0, 1])
def test_matches_padded_dense_sdpa(broadcast_q, causal, seed):
    rng = np.random.default_rng(100 + seed)
    lengths = [5, 1, 17, 9] if seed == 0 else [33, 2, 64, 7, 1]
    h, d, lq = 3, 8, (6 if seed == 0 else 19)
    scale = 0.37
    q, k, v, g, off = _rand_case(rng, lengths, h, d, broadcast_q, lq)
    o, lse = oracle.forward(q, k, v, off, broadcast_q=broadcast_q, causal=causal, scale=scale)
    dq, dk, dv = oracle.backward(q, k, v, off, g, broadcast_q=broadcast_q, causal=causal, scale=scale)
    ro, rlse, rdq, rdk, rdv = _padded_reference(q, k, v, g, off, broadcast_q, causal, scale)
    for name, a, r in [("O", o, ro), ("LSE", lse, rlse), ("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)]:
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("broadcast_q,causal", MODES)
def test_finite_differences(broadcast_q, causal):
    """Central differences of L = sum(O * G) for every element of Q, K and V."""
    rng = np.random.default_rng(7)
    lengths, h, d, lq, scale = [1, 2, 5], 2, 4, 3, 0.8
    q, k, v, g, off = _rand_case(rng, lengths, h, d, broadcast_q, lq)
    kw = dict(broadcast_q=broadcast_q, causal=causal, scale=scale)
    dq, dk, dv = oracle.backward(q, k, v, off, g, **kw)

    def loss(q_, k_, v_):
        return float((oracle.forward(q_, k_, v_, off, **kw)[0] * g).sum())

    eps = 1e-6
    for name, x, grad in [("q", q, dq), ("k", k, dk), ("v", v, dv)]:
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{n + "_": a for n, a in args_p.items()})
                        - loss(**{n + "_": a for n, a in args_m.items()})) / (2 * eps)
        err = np.abs(num - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err <= 1e-6, (name, err)


@pytest.mark.parametrize("broadcast_q,causal", MODES)
def test_rows_sum_to_one(broadcast_q, causal):
    """With V = 1 everywhere the output is exactly the softmax row sum, i.e. 1."""
    rng = np.random.default_rng(3)
    q, k, v, g, off = _rand_case(rng, [4, 1, 30], 2, 16, broadcast_q, 9)
    o, _ = oracle.forward(q * 3, k * 3, np.ones_like(v), off, broadcast_q=broadcast_q,
                          causal=causal, scale=1.0)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("broadcast_q", [True, False])
def test_single_key_closed_form(broadcast_q):
    """n_b = 1: O_i = V_0, LSE_i = c q_i.k_0, dK_0 = 0, dQ contribution 0, dV_0 = sum_i G_i."""
    rng = np.random.default_rng(11)
    lq, h, d, c = 5, 2, 8, 0.3
    q, k, v, g, off = _rand_case(rng, [1], h, d, broadcast_q, lq)
    o, lse = oracle.forward(q, k, v, off, broadcast_q=broadcast_q, scale=c)
    dq, dk, dv = oracle.backward(q, k, v, off, g, broadcast_q=broadcast_q, scale=c)
    rows = o.shape[0]
    for hh in range(h):
        np.testing.assert_array_equal(o[:, hh, :], np.broadcast_to(v[0, hh], (rows, d)))
        np.testing.assert_allclose(lse[hh], c * (q[:, hh, :] @ k[0, hh]), atol=1e-14)
        np.testing.assert_allclose(dv[0, hh], g[:, hh, :].sum(axis=0), atol=1e-13)
    assert np.abs(dk).max() < 1e-14
    assert np.abs(dq).max() < 1e-14


def test_broadcast_dq_is_sum_over_sequences():
    rng = np.random.default_rng(5)
    lengths, h, d, lq, c = [7, 3, 12, 1], 2, 8, 6, 0.5
    q, k, v, g, off = _rand_case(rng, lengths, h, d, True, lq)
    dq, dk, dv = oracle.backward(q, k, v, off, g, broadcast_q=True, scale=c)
    acc = np.zeros_like(q)
    for b in range(len(lengths)):
        a, e = off[b], off[b + 1]
        dq_b, dk_b, dv_b = oracle.backward(q, k[a:e], v[a:e], np.array([0, e - a]),
                                           g[b * lq:(b + 1) * lq], broadcast_q=True, scale=c)
        acc += dq_b
        np.testing.assert_allclose(dk[a:e], dk_b, atol=1e-13)
        np.testing.assert_allclose(dv[a:e], dv_b, atol=1e-13)
    np.testing.assert_allclose(dq, acc, atol=1e-12)


@pytest.mark.parametrize("broadcast_q,causal", MODES)
def test_exact_identities(broadcast_q, causal):
    rng = np.random.default_rng(9)
    lengths, h, d, lq, c = [6, 1, 20, 3], 2, 8, 5, 0.45
    q, k, v, g, off = _rand_case(rng, lengths, h, d, broadcast_q, lq)
    kw = dict(broadcast_q=broadcast_q, causal=causal, scale=c)
    o, _ = oracle.forward(q, k, v, off, **kw)
    dq, dk, dv = oracle.backward(q, k, v, off, g, **kw)
    for b in range(len(lengths)):
        a, e = off[b], off[b + 1]
        r0, r1 = (b * lq, (b + 1) * lq) if broadcast_q else (a, e)
        # softmax shift invariance: the key gradients of one sequence sum to zero
        np.testing.assert_allclose(dk[a:e].sum(axis=0), 0.0, atol=1e-12)
        # rows of P sum to one: the value gradients sum to the upstream gradient sum
        np.testing.assert_allclose(dv[a:e].sum(axis=0), g[r0:r1].sum(axis=0), atol=1e-12)
    for hh in range(h):
        # scores depend on Q K^T only: scaling Q by t and K by 1/t changes nothing
        np.testing.assert_allclose((q[:, hh] * dq[:, hh]).sum(), (k[:, hh] * dk[:, hh]).sum(), atol=1e-11)
    # O is linear in V
    np.testing.assert_allclose((v * dv).sum(), (o * g).sum(), atol=1e-11)
    if causal:
        for b in range(len(lengths)):
            a = off[b]
            np.testing.assert_array_equal(o[a], v[a])


def test_permuting_sequences():
    rng = np.random.default_rng(12)
    lengths, h, d, lq, c = [4, 9, 1, 6], 2, 8, 5, 0.6
    q, k, v, g, off = _rand_case(rng, lengths, h, d, True, lq)
    perm = [2, 0, 3, 1]
    ks = [k[off[b]:off[b + 1]] for b in range(4)]
    vs = [v[off[b]:off[b + 1]] for b in range(4)]
    gs = [g[b * lq:(b + 1) * lq] for b in range(4)]
    k2 = np.concatenate([ks[p] for p in perm])
    v2 = np.concatenate([vs[p] for p in perm])
    g2 = np.concatenate([gs[p] for p in perm])
    off2 = np.concatenate([[0], np.cumsum([lengths[p] for p in perm])])
    o, lse = oracle.forward(q, k, v, off, broadcast_q=True, scale=c)
    o2, lse2 = oracle.forward(q, k2, v2, off2, broadcast_q=True, scale=c)
    dq, dk, dv = oracle.backward(q, k, v, off, g, broadcast_q=True, scale=c)
    dq2, dk2, dv2 = oracle.backward(q, k2, v2, off2, g2, broadcast_q=True, scale=c)
    for j, p in enumerate(perm):
        np.testing.assert_array_equal(o2[j * lq:(j + 1) * lq], o[p * lq:(p + 1) * lq])
        np.testing.assert_array_equal(lse2[:, j * lq:(j + 1) * lq], lse[:, p * lq:(p + 1) * lq])
        np.testing.assert_array_equal(dk2[off2[j]:off2[j + 1]], dk[off[p]:off[p + 1]])
        np.testing.assert_array_equal(dv2[off2[j]:off2[j + 1]], dv[off[p]:off[p + 1]])
    np.testing.assert_allclose(dq2, dq, atol=1e-12)


def test_duplicating_a_broadcast_sequence_doubles_its_dq():
    rng = np.random.default_rng(13)
    h, d, lq, c = 2, 8, 4, 0.7
    q, k, v, g, off = _rand_case(rng, [5], h, d, True, lq)
    dq1, _, _ = oracle.backward(q, k, v, off, g, broadcast_q=True, scale=c)
    k2, v2, g2 = np.concatenate([k, k]), np.concatenate([v, v]), np.concatenate([g, g])
    o2, _ = oracle.forward(q, k2, v2, [0, 5, 10], broadcast_q=True, scale=c)
    o1, _ = oracle.forward(q, k, v, off, broadcast_q=True, scale=c)
    dq2, _, _ = oracle.backward(q, k2, v2, [0, 5, 10], g2, broadcast_q=True, scale=c)
    np.testing.assert_array_equal(o2[:lq], o1)
    np.testing.assert_array_equal(o2[lq:], o1)
    np.testing.assert_allclose(dq2, 2 * dq1, atol=1e-13)


@pytest.mark.parametrize("block", [4, 64])
def test_fixed_length_self_attention_is_block_diagonal(block):
    """All n_b equal: jagged self-attention == dense attention with a block-diagonal mask."""
    rng = np.random.default_rng(21)
    nblk, h, d, c = 3, 2, 8, 0.35
    t = nblk * block
    q, k, v, g, off = _rand_case(rng, [block] * nblk, h, d, False, 0)
    o, lse = oracle.forward(q, k, v, off, broadcast_q=False, scale=c)
    blk = np.arange(t) // block
    for hh in range(h):
        s = c * q[:, hh] @ k[:, hh].T
        s = np.where(blk[:, None] == blk[None, :], s, -np.inf)
        ref_lse = np.log(np.exp(s).sum(axis=1))
        ref_o = (np.exp(s - ref_lse[:, None])) @ v[:, hh]
        np.testing.assert_allclose(o[:, hh], ref_o, atol=1e-12)
        np.testing.assert_allclose(lse[hh], ref_lse, atol=1e-12)


def test_golden_two_key_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "two_key_worked_example.json")))
    q = np.array(ex["q"])[:, None, :]
    k = np.array(ex["k"])[:, None, :]
    v = np.array(ex["v"])[:, None, :]
    g = np.array(ex["g"])[:, None, :]
    off = [0, 2]
    o, lse = oracle.forward(q, k, v, off, broadcast_q=True, scale=ex["scale"])
    dq, dk, dv = oracle.backward(q, k, v, off, g, broadcast_q=True, scale=ex["scale"])
    np.testing.assert_allclose(o[:, 0], ex["o"], atol=1e-15)
    np.testing.assert_allclose(lse[0], ex["lse"], atol=1e-15)
    np.testing.assert_allclose(dq[:, 0], ex["dq"], atol=1e-15)
    np.testing.assert_allclose(dk[:, 0], ex["dk"], atol=1e-15)
    np.testing.assert_allclose(dv[:, 0], ex["dv"], atol=1e-15)


def test_golden_causal_two_token_example():
    ex = json.load(open(os.path.join(GOLDEN, "causal_two_token_example.json")))
    q = np.array(ex["q"])[:, None, :]
    k = np.array(ex["k"])[:, None, :]
    v = np.array(ex["v"])[:, None, :]
    o, lse = oracle.forward(q, k, v, [0, 2], broadcast_q=False, causal=True, scale=ex["scale"])
    np.testing.assert_allclose(o[:, 0], ex["o"], atol=1e-15)
    np.testing.assert_allclose(lse[0], ex["lse"], atol=1e-15)


def test_empty_sequence_reading():
    """n_b = 0: its O rows are 0, LSE is -inf, and it adds nothing to dQ."""
    rng = np.random.default_rng(4)
    lq, h, d = 3, 2, 4
    q, k, v, g, off = _rand_case(rng, [2, 0, 3], h, d, True, lq)
    o, lse = oracle.forward(q, k, v, off, broadcast_q=True, scale=0.5)
    assert np.all(o[lq:2 * lq] == 0) and np.all(np.isneginf(lse[:, lq:2 * lq]))
    dq, _, _ = oracle.backward(q, k, v, off, g, broadcast_q=True, scale=0.5)
    keep = [0, 1, 2, 5, 6, 7, 8]
    off2 = [0, 2, 5]
    g2 = np.concatenate([g[:lq], g[2 * lq:]])
    dq2, _, _ = oracle.backward(q, k, v, off2, g2, broadcast_q=True, scale=0.5)
    np.testing.assert_allclose(dq, dq2, atol=1e-14)
    assert keep  # rows of the empty sequence were checked above


def test_rejects_broadcast_causal_and_bad_offsets():
    rng = np.random.default_rng(1)
    q, k, v, g, off = _rand_case(rng, [3], 1, 4, True, 2)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, off, broadcast_q=True, causal=True, scale=1.0)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, [0, 2], broadcast_q=True, scale=1.0)


def test_workload_recipes_seed0():
    """The length recipes reproduce the seed-0 statistics recorded for the workloads."""
    c = workloads.make_workload("tiny_broadcast")
    assert list(c["lengths"]) == [218, 164, 131, 70]
    assert c["offsets"].dtype == torch.int64
    rng = np.random.default_rng(0)
    assert int(workloads.draw_lengths(workloads.WORKLOADS["gem_broadcast"], rng).sum()) == 1017228
    rng = np.random.default_rng(0)
    assert int(workloads.draw_lengths(workloads.WORKLOADS["dq_stress"], rng).sum()) == 1121466
    rng = np.random.default_rng(0)
    ln = workloads.draw_lengths(workloads.WORKLOADS["self_causal"], rng)
    assert int(ln.sum()) == 528065 and ln.min() == 64 and ln.max() == 4096
    rng = np.random.default_rng(0)
    assert int(workloads.draw_lengths(workloads.WORKLOADS["block64"], rng).sum()) == 1152 * 2048


def test_bf16_inputs_round_to_nearest_even():
    x = workloads.normal_bf16(np.random.default_rng(0), (1000,))
    ref = torch.from_numpy(np.random.default_rng(0).standard_normal(1000, dtype=np.float32))
    assert torch.equal(x, ref.to(torch.bfloat16))


@pytest.mark.parametrize("causal", [False, True])
def test_dq_rows_match_full_backward(causal):
    """The row-restricted dQ equals the matching rows of the full backward."""
    rng = np.random.default_rng(31)
    n, d, c = 23, 8, 0.4
    qb, kb, vb, gb = (rng.standard_normal((n, d)) for _ in range(4))
    dq, _, _ = oracle.sequence_backward(qb, kb, vb, gb, c, causal)
    rows = [0, 3, 22, 11]
    np.testing.assert_allclose(oracle.sequence_dq_rows(qb, kb, vb, gb, rows, c, causal), dq[rows],
                               atol=1e-13)


# ---- rotary-embedding conjugate (oracle/rope.py) ---------------------------------

def _angle_tables(rng, max_pos, d):
    ang = rng.uniform(-np.pi, np.pi, (max_pos, d // 2))
    return np.cos(ang), np.sin(ang)


def test_rope_conjugate_is_the_transpose_of_the_rotation():
    """<R x, y> = <x, R^T y> for random angles and positions, and with
    cos^2 + sin^2 = 1 the conjugate undoes the rotation."""
    rng = np.random.default_rng(21)
    d, rows, h, max_pos = 8, 7, 2, 5
    cos, sin = _angle_tables(rng, max_pos, d)
    pos = rng.integers(0, max_pos, rows)
    x = rng.standard_normal((rows, h, d))
    y = rng.standard_normal((rows, h, d))
    lhs = float((oracle.rope_rotate(x, cos, sin, pos) * y).sum())
    rhs = float((x * oracle.rope_conjugate(y, cos, sin, pos)).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    back = oracle.rope_conjugate(oracle.rope_rotate(x, cos, sin, pos), cos, sin, pos)
    np.testing.assert_allclose(back, x, atol=1e-12)


def test_rope_quarter_turn_closed_form():
    """At a quarter turn (cos 0, sin 1) each pair (a, b) = (x[d], x[d + D/2])
    becomes (-b, a), and the conjugate turns it back: (a, b) -> (b, -a)."""
    d = 4
    x = np.arange(1.0, 1.0 + 2 * d).reshape(2, 1, d)
    cos, sin, pos = np.zeros((1, d // 2)), np.ones((1, d // 2)), np.zeros(2, dtype=np.int64)
    a, b = x[..., : d // 2], x[..., d // 2:]
    np.testing.assert_array_equal(oracle.rope_rotate(x, cos, sin, pos), np.concatenate([-b, a], axis=2))
    np.testing.assert_array_equal(oracle.rope_conjugate(x, cos, sin, pos), np.concatenate([b, -a], axis=2))


def test_rope_zero_angle_is_the_plain_backward():
    rng = np.random.default_rng(4)
    lengths, h, d = [2, 5], 2, 8
    q, k, v, g, off = _rand_case(rng, lengths, h, d, False, 0)
    cos, sin = np.ones((6, d // 2)), np.zeros((6, d // 2))
    pos = np.concatenate([np.arange(n) for n in lengths])
    kw = dict(broadcast_q=False, causal=True, scale=0.5)
    got = oracle.backward_rope(q, k, v, off, g, cos, sin, pos, pos, **kw)
    ref = oracle.backward(q, k, v, off, g, **kw)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("broadcast_q,causal", MODES)
def test_rope_backward_finite_differences(broadcast_q, causal):
    """Central differences of L(q0, k0) = sum(O(R q0, R k0, V) * G), where attention
    runs on the rotated vectors, for every element of q0 and k0."""
    rng = np.random.default_rng(9)
    lengths, h, d, lq, scale = [1, 3, 4], 2, 4, 3, 0.7
    q0, k0, v, g, off = _rand_case(rng, lengths, h, d, broadcast_q, lq)
    cos, sin = _angle_tables(rng, 5, d)
    pos_k = np.concatenate([np.arange(n) for n in lengths])
    pos_q = np.arange(lq) if broadcast_q else pos_k
    kw = dict(broadcast_q=broadcast_q, causal=causal, scale=scale)

    def rot(x, pos):
        return oracle.rope_rotate(x, cos, sin, pos)

    dq, dk, dv = oracle.backward_rope(rot(q0, pos_q), rot(k0, pos_k), v, off, g, cos, sin, pos_q, pos_k, **kw)
    np.testing.assert_array_equal(dv, oracle.backward(rot(q0, pos_q), rot(k0, pos_k), v, off, g, **kw)[2])

    def loss(q_, k_):
        return float((oracle.forward(rot(q_, pos_q), rot(k_, pos_k), v, off, **kw)[0] * g).sum())

    eps = 1e-6
    for name, x, grad in [("q0", q0, dq), ("k0", k0, dk)]:
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            if name == "q0":
                num[idx] = (loss(xp, k0) - loss(xm, k0)) / (2 * eps)
            else:
                num[idx] = (loss(q0, xp) - loss(q0, xm)) / (2 * eps)
        err = np.abs(num - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err <= 1e-6, (name, err)


def test_rope_inputs_recipe():
    """The generated tables hold cos / sin of p * 10000^(-2d/D) rounded to fp32, and
    positions count from each sequence's start (broadcast queries: 0 .. Lq - 1)."""
    case = workloads.make_case([3, 1, 4], heads=1, head_dim=8, broadcast_q=True, q_len=5, seed=0)
    r = workloads.rope_inputs(case)
    assert r["cos"].shape == (5, 4) and r["cos"].dtype == torch.float32
    assert r["pos_k"].tolist() == [0, 1, 2, 0, 0, 1, 2, 3]
    assert r["pos_q"].tolist() == [0, 1, 2, 3, 4]
    ang = 3 * 10000.0 ** (-2 * 2 / 8)
    assert r["cos"][3, 2].item() == np.float32(math.cos(ang))
    assert r["sin"][3, 2].item() == np.float32(math.sin(ang))


# ---- block-sparse top-k forward (oracle/sparse.py) ---------------------------------

def _block_mask_reference(q, k, v, off, selection, broadcast_q, scale):
    """Padded dense torch SDPA (fp64, CPU) with a key mask that keeps, for every query
    block, the keys of its selected blocks."""
    from oracle.sparse import KV_BLOCK, q_block
    Q_BLOCK = q_block(broadcast_q)
    b, h, d = len(off) - 1, k.shape[1], k.shape[2]
    lens = np.diff(off)
    lmax = max(int(lens.max()), 1)
    nq = q.shape[0] if broadcast_q else lmax
    qp = torch.zeros(b, h, nq, d, dtype=torch.float64)
    kp = torch.zeros(b, h, lmax, d, dtype=torch.float64)
    vp = torch.zeros(b, h, lmax, d, dtype=torch.float64)
    mask = torch.zeros(b, h, nq, lmax, dtype=torch.bool)
    for i in range(b):
        a, e = int(off[i]), int(off[i + 1])
        qp[i, :, :, :] = torch.from_numpy(q.transpose(1, 0, 2) if broadcast_q else
                                          np.pad(q[a:e], ((0, nq - (e - a)), (0, 0), (0, 0))).transpose(1, 0, 2))
        kp[i, :, :e - a] = torch.from_numpy(k[a:e].transpose(1, 0, 2))
        vp[i, :, :e - a] = torch.from_numpy(v[a:e].transpose(1, 0, 2))
        rows = nq if broadcast_q else e - a
        for hh in range(h):
            for m, blocks in enumerate(selection[hh][i]):
                r0, r1 = m * Q_BLOCK, min((m + 1) * Q_BLOCK, rows)
                for j in blocks:
                    mask[i, hh, r0:r1, j * KV_BLOCK:min((j + 1) * KV_BLOCK, e - a)] = True
    o = F.scaled_dot_product_attention(qp, kp, vp, attn_mask=mask, scale=scale)
    return o, mask


@pytest.mark.parametrize("broadcast_q", [True, False])
def test_sparse_forward_matches_block_masked_sdpa(broadcast_q):
    """A fixed selection equals dense attention with the matching block mask."""
    rng = np.random.default_rng(41)
    lengths, h, d, lq, scale = [70, 200, 129], 2, 8, 300, 0.3
    q, k, v, g, off = _rand_case(rng, lengths, h, d, broadcast_q, lq)
    sel = oracle.sparse.select_all(q, k, off, 2, broadcast_q=broadcast_q, scale=scale)
    o, lse = oracle.sparse.sparse_forward(q, k, v, off, sel, broadcast_q=broadcast_q, scale=scale)
    ref, mask = _block_mask_reference(q, k, v, off, sel, broadcast_q, scale)
    for i in range(len(lengths)):
        a, e = int(off[i]), int(off[i + 1])
        r0, r1 = (i * lq, (i + 1) * lq) if broadcast_q else (a, e)
        got = o[r0:r1].transpose(1, 0, 2)
        np.testing.assert_allclose(got, ref[i, :, :r1 - r0].numpy(), atol=1e-12)


def test_sparse_with_every_block_is_dense():
    rng = np.random.default_rng(42)
    lengths, h, d, scale = [1, 64, 65, 300], 2, 8, 0.5
    for bq, lq in ((True, 130), (False, 0)):
        q, k, v, g, off = _rand_case(rng, lengths, h, d, bq, lq)
        sel = oracle.sparse.select_all(q, k, off, 99, broadcast_q=bq, scale=scale)
        o, lse = oracle.sparse.sparse_forward(q, k, v, off, sel, broadcast_q=bq, scale=scale)
        o_ref, lse_ref = oracle.forward(q, k, v, off, broadcast_q=bq, scale=scale)
        np.testing.assert_allclose(o, o_ref, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_block_scores_by_explicit_loops():
    rng = np.random.default_rng(43)
    qb, kb, scale = rng.standard_normal((200, 4)), rng.standard_normal((130, 4)), 0.7
    got = oracle.sparse.block_scores(qb, kb, scale, 128)
    assert got.shape == (2, 3)
    for m, (q0, q1) in enumerate(((0, 128), (128, 200))):
        for j, (k0, k1) in enumerate(((0, 64), (64, 128), (128, 130))):
            qm = [sum(qb[r, c] for r in range(q0, q1)) / (q1 - q0) for c in range(4)]
            km = [sum(kb[r, c] for r in range(k0, k1)) / (k1 - k0) for c in range(4)]
            assert abs(got[m, j] - scale * sum(a * b for a, b in zip(qm, km))) <= 1e-12


@pytest.mark.parametrize("nq,nk,qblk", [(200, 130, 128), (256, 64, 256), (300, 1, 256), (17, 200, 128)])
def test_block_scores_are_means_of_exact_scores(nq, nk, qblk):
    """By linearity, c * mean(q rows) . mean(k rows) equals the mean over the block of
    the exact scores c * q_i . k_j.  The exact scores come from the full score matrix
    (one product of all rows), so a wrong divisor for a partial block, a sum in place
    of a mean, a dropped scale or a shifted block boundary fails here."""
    rng = np.random.default_rng(nq * 1000 + nk)
    d, scale = 16, 0.37
    qb, kb = rng.standard_normal((nq, d)), rng.standard_normal((nk, d))
    got = oracle.sparse.block_scores(qb, kb, scale, qblk)
    s = scale * (qb @ kb.T)                      # every exact score
    kv = oracle.sparse.KV_BLOCK
    nqb, nkb = -(-nq // qblk), -(-nk // kv)
    assert got.shape == (nqb, nkb)
    for m in range(nqb):
        for j in range(nkb):
            blk = s[m * qblk:min((m + 1) * qblk, nq), j * kv:min((j + 1) * kv, nk)]
            assert abs(got[m, j] - blk.mean()) <= 1e-12 * max(1.0, np.abs(blk).max())


def test_sparse_block_sizes_match_the_library_header():
    """The oracle's block sizes are the ones the C ABI documents as the method's."""
    import re
    with open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "jfa.h")) as f:
        text = f.read()
    val = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (JFA_SPARSE_\w+) (\d+)", text)}
    assert val == {"JFA_SPARSE_KEY_BLOCK": oracle.sparse.KV_BLOCK,
                   "JFA_SPARSE_QUERY_BLOCK_BROADCAST": oracle.sparse.Q_BLOCK_BROADCAST,
                   "JFA_SPARSE_QUERY_BLOCK_SELF": oracle.sparse.Q_BLOCK_SELF}


def test_top_k_selection_by_brute_force():
    scores = np.array([[0.5, 2.0, -1.0, 2.0, 0.1],
                       [3.0, 3.0, 3.0, 0.0, -2.0],
                       [1.0, 0.0, 0.0, 0.0, 0.0]])
    assert oracle.sparse.select_top_k(scores, 2) == [[1, 3], [0, 1], [0, 1]]   # ties to the lower index
    assert oracle.sparse.select_top_k(scores, 9) == [[0, 1, 2, 3, 4]] * 3
    rng = np.random.default_rng(44)
    s = rng.standard_normal((6, 11))
    for row, sel in zip(s, oracle.sparse.select_top_k(s, 4)):
        assert len(sel) == 4 and sel == sorted(sel)
        assert min(row[sel]) >= max(np.delete(row, sel))
