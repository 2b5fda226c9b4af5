"""GPU parity of the MXFP8 path (quantizers and forward) against the oracle.

Quantizers: byte work whose every decision is exact (bf16 inputs, power-of-two
scales, round to nearest even), so they must match the oracle bit for bit: equal
E8M0 codes, and equal E4M3 values (+0 and -0 count as equal).

Forward: max |O - O_ref| <= 1e-2 + slack + half a bf16 ulp of O, where O_ref and
slack come from oracle.mxfp8.forward_mx on the same bf16 inputs: slack bounds the
effect of P rounding decisions that sit within 2^-12 of a tie (the fp32 scores of
the kernel and the oracle differ in the last bits, so such a decision may go either
way), and the half ulp is the rounding of O to bf16.  max |LSE - LSE_ref| <= 1e-3.
"""
import zlib

import numpy as np
import pytest
import torch

import workloads
from oracle import mxfp8 as mx
import test_gpu_parity as tp   # the growing-score key ramp

pytestmark = pytest.mark.gpu

TOL_O = 1e-2
TOL_LSE = 1e-3
LUT = np.array([mx.e4m3_value(c) for c in range(256)])


def _jfa():
    import variable_length_flash_jfa_amd as jfa
    return jfa


def _f64(t):
    return t.to(torch.float64).cpu().numpy()


def _decode(b):
    return LUT[b.cpu().numpy().astype(np.int64)]


def _v_pos(k):
    return 16 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3)


def test_quantize_rows_bit_exact():
    jfa = _jfa()
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 3, 128)) * np.exp2(rng.integers(-20, 20, (300, 3, 1)))
    x[5] = 0.0                                     # all-zero blocks: code 0, values 0
    x[6, :, 7] = 3.0e4                             # one large element per block
    xb = torch.from_numpy(x).to(torch.bfloat16)
    vals, scl = jfa.mxfp8_quantize_rows(xb.cuda())
    torch.cuda.synchronize()
    deq, codes = mx.quantize_rows(xb.to(torch.float64).numpy())
    assert np.array_equal(scl.cpu().numpy().astype(np.int64), codes)
    got = _decode(vals) * np.repeat(np.ldexp(1.0, codes - 127), 32, axis=-1)
    assert np.array_equal(got, deq)


@pytest.mark.parametrize("offsets_dtype", [torch.int64, torch.int32])
def test_quantize_v_bit_exact(offsets_dtype):
    jfa = _jfa()
    rng = np.random.default_rng(12)
    lengths = [1, 31, 32, 33, 70, 0, 5, 64, 200]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    v = rng.standard_normal((off[-1], 2, 64)) * np.exp2(rng.integers(-8, 8, (off[-1], 2, 1)))
    vb = torch.from_numpy(v).to(torch.bfloat16)
    vals, scl = jfa.mxfp8_quantize_v(vb.cuda(), torch.from_numpy(off).to(offsets_dtype).cuda())
    torch.cuda.synchronize()
    assert vals.shape == (len(lengths) + (off[-1] + 31) // 32, 2, 64, 32)
    deq, scales = mx.quantize_v(vb.to(torch.float64).numpy(), off)
    vals, scl = vals.cpu(), scl.cpu().numpy().astype(np.int64)
    for b, n in enumerate(lengths):
        for j in range((n + 31) // 32):
            g = b + off[b] // 32 + j
            assert np.array_equal(scl[g], scales[b][j]), (b, j)
            s = np.ldexp(1.0, scales[b][j] - 127)                  # [H, D]
            blk = _decode(vals[g])                                  # [H, D, 32] in operand order
            for k in range(32):
                want = deq[off[b] + 32 * j + k] if 32 * j + k < n else np.zeros((2, 64))
                assert np.array_equal(blk[:, :, _v_pos(k)] * s, want), (b, j, k)


CASES = {
    # name: (lengths, heads, head_dim, broadcast_q, causal, q_len)
    "bcast_d128_lq256": ([1, 63, 300, 700, 1000], 2, 128, True, False, 256),
    "bcast_d64_lq100": ([17, 64, 129, 0, 2], 2, 64, True, False, 100),
    "bcast_d128_lq33": ([5, 31, 32, 33, 95], 2, 128, True, False, 33),
    "self_d128": ([1, 17, 64, 65, 200, 513], 2, 128, False, False, 0),
    "self_d128_causal": ([1, 5, 64, 127, 128, 129, 300], 2, 128, False, True, 0),
    "self_d64_causal": ([2, 33, 190, 257], 3, 64, False, True, 0),
    "self_d64": ([3, 96, 160], 2, 64, False, False, 0),
    "self_empty_seq": ([20, 0, 45], 2, 128, False, False, 0),
    # mean length >= 384: eight-wave workgroups in self mode (two waves at <= 96)
    "self_d128_causal_long": ([400, 700, 513, 1], 2, 128, False, True, 0),
    "self_d64_long": ([900, 385, 64], 2, 64, False, False, 0),
}


def _mx_run(jfa, q, k, v, off, bq, causal, scale):
    q8, qs = jfa.mxfp8_quantize_rows(q)
    k8, ks = jfa.mxfp8_quantize_rows(k)
    v8, vs = jfa.mxfp8_quantize_v(v, off)
    return jfa.fwd_mxfp8(q8, qs, k8, ks, v8, vs, off, broadcast_q=bq, causal=causal, scale=scale)


def _check_o(got, ref, slack):
    """got [rows, H, D] bf16 tensor; ref fp64 [rows, H, D]; slack [H, rows]."""
    got = _f64(got)
    nz = slack[slack > 0]
    print(f"slack: largest {slack.max() if slack.size else 0.0:.3e}, rows with slack > 0: {nz.size} of "
          f"{slack.size}", flush=True)
    _, e = np.frexp(np.maximum(np.abs(got), np.abs(ref)))
    half_ulp = np.ldexp(1.0, e - 9)
    excess = np.abs(got - ref) - half_ulp - slack.T[:, :, None]
    assert excess.max() <= TOL_O, f"O: max error beyond rounding and slack {excess.max():.3e}"


def _check_lse(got, ref):
    got = got.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = ~np.isneginf(ref)
    if fin.any():
        assert np.abs(got[fin] - ref[fin]).max() <= TOL_LSE


@pytest.mark.parametrize("name", list(CASES))
def test_mxfp8_forward_matches_oracle(name):
    lengths, h, d, bq, causal, lq = CASES[name]
    case = workloads.make_case(lengths, heads=h, head_dim=d, broadcast_q=bq, causal=causal, q_len=lq,
                               seed=zlib.crc32(name.encode()) % 1000)
    jfa = _jfa()
    q, k, v = (case[x].cuda() for x in ("q", "k", "v"))
    off = case["offsets"].cuda()
    if name == "self_d64":
        off = off.to(torch.int32)
    o, lse = _mx_run(jfa, q, k, v, off, bq, causal, case["scale"])
    torch.cuda.synchronize()
    o_ref, lse_ref, slack = mx.forward_mx(*(_f64(case[x]) for x in ("q", "k", "v")), case["offsets"].numpy(),
                                          broadcast_q=bq, causal=causal, scale=case["scale"])
    _check_o(o, o_ref, slack)
    _check_lse(lse, lse_ref)


RAMP_CASES = {
    # name: (lengths, heads, head_dim, broadcast_q, causal, q_len, growth of the largest
    # score along a sequence, base 2)
    "bcast_ramp_within_lazy_bound": ([300, 700, 1000], 2, 128, True, False, 256, 4.0),
    "bcast_ramp_rescales": ([300, 700, 1000], 2, 128, True, False, 256, 24.0),
    "self_causal_ramp_rescales": ([400, 700, 513, 64], 2, 128, False, True, 0, 24.0),
}


@pytest.mark.parametrize("name", list(RAMP_CASES))
def test_mxfp8_forward_growing_scores(name):
    """Scores that climb along each sequence (keys ramped along the mean query
    direction): the running maximum either stays stale, within 2^8 of the scores, or
    is rescaled several times per row; O and LSE match the oracle either way."""
    lengths, h, d, bq, causal, lq, growth = RAMP_CASES[name]
    case = workloads.make_case(lengths, heads=h, head_dim=d, broadcast_q=bq, causal=causal, q_len=lq,
                               seed=zlib.crc32(name.encode()) % 1000)
    case = tp._ramp_keys(case, growth)
    jfa = _jfa()
    q, k, v = (case[x].cuda() for x in ("q", "k", "v"))
    off = case["offsets"].cuda()
    o, lse = _mx_run(jfa, q, k, v, off, bq, causal, case["scale"])
    torch.cuda.synchronize()
    o_ref, lse_ref, slack = mx.forward_mx(*(_f64(case[x]) for x in ("q", "k", "v")), case["offsets"].numpy(),
                                          broadcast_q=bq, causal=causal, scale=case["scale"])
    _check_o(o, o_ref, slack)
    _check_lse(lse, lse_ref)


@pytest.mark.parametrize("bq", [True, False])
def test_mxfp8_forward_many_tiles_per_workgroup(bq):
    # Many more tiles than workgroups (about 12 to 20 each, 4-wave workgroups): each
    # workgroup loads its next tile's first block (and, in self mode, its Q fragment)
    # during the current tile, and broadcast tiles keep their Q fragment; the
    # broadcast batch has an empty sequence every 37, so empty tiles sit between
    # others.  Every row against the oracle.
    rng = np.random.default_rng(41 if bq else 47)
    if bq:
        lengths = [int(x) for x in rng.integers(0, 150, size=2500)]
        for i in range(0, len(lengths), 37):
            lengths[i] = 0
        case = workloads.make_case(lengths, heads=2, head_dim=64, broadcast_q=True, causal=False, q_len=100,
                                   seed=43)
    else:
        lengths = [int(x) for x in rng.integers(100, 300, size=800)]
        case = workloads.make_case(lengths, heads=2, head_dim=64, broadcast_q=False, causal=True, q_len=0,
                                   seed=49)
    jfa = _jfa()
    q, k, v = (case[x].cuda() for x in ("q", "k", "v"))
    o, lse = _mx_run(jfa, q, k, v, case["offsets"].cuda(), bq, not bq, case["scale"])
    torch.cuda.synchronize()
    o_ref, lse_ref, slack = mx.forward_mx(*(_f64(case[x]) for x in ("q", "k", "v")), case["offsets"].numpy(),
                                          broadcast_q=bq, causal=not bq, scale=case["scale"])
    _check_o(o, o_ref, slack)
    _check_lse(lse, lse_ref)


def test_mxfp8_forward_close_to_bf16_forward():
    """The 8-bit forward stays near the bf16 forward on the same inputs: a coarse
    check of the whole path (quantization of Q, K, V and P shifts O by a few
    percent of its scale)."""
    jfa = _jfa()
    case = workloads.make_case([100, 700, 1000], heads=2, head_dim=128, broadcast_q=True, q_len=256, seed=9)
    q, k, v = (case[x].cuda() for x in ("q", "k", "v"))
    off = case["offsets"].cuda()
    o8, lse8 = _mx_run(jfa, q, k, v, off, True, False, case["scale"])
    o16, lse16 = jfa.fwd(q, k, v, off, broadcast_q=True, scale=case["scale"])
    torch.cuda.synchronize()
    assert (o8.float() - o16.float()).abs().max().item() <= 0.1
    assert (lse8 - lse16).abs().max().item() <= 0.05


@pytest.mark.parametrize("name", ["gem_broadcast", "self_causal", "block64"])
def test_mxfp8_full_size_sampled(name):
    """Full-size workloads through the MXFP8 path, checked on sampled sequences
    (the shortest, the longest up to 2048 keys, the median and random ones) and on
    the first and last head."""
    jfa = _jfa()
    w = workloads.WORKLOADS[name]
    case = workloads.make_workload(name, device="cuda", with_grad=False)
    q, k, v, off = case["q"], case["k"], case["v"], case["offsets"]
    o, lse = _mx_run(jfa, q, k, v, off, w.broadcast_q, w.causal, case["scale"])
    torch.cuda.synchronize()
    lengths = case["lengths"]
    rng = np.random.default_rng(8)
    order = [int(i) for i in np.argsort(lengths, kind="stable") if lengths[i] <= 2048]
    seqs = sorted({order[0], order[-1], order[len(order) // 2],
                   *rng.choice(order, 3, replace=False).tolist()})
    heads = sorted({0, w.heads - 1})
    offn = off.cpu().numpy().astype(np.int64)
    qf = _f64(q[:, heads]) if w.broadcast_q else None
    for b in seqs:
        a, e = int(offn[b]), int(offn[b + 1])
        qb = qf if w.broadcast_q else _f64(q[a:e, heads])
        o_ref, lse_ref, slack = mx.forward_mx(qb, _f64(k[a:e, heads]), _f64(v[a:e, heads]), np.array([0, e - a]),
                                              broadcast_q=w.broadcast_q, causal=w.causal, scale=case["scale"])
        rows = slice(b * w.q_len, (b + 1) * w.q_len) if w.broadcast_q else slice(a, e)
        _check_o(o[rows][:, heads], o_ref, slack)
        _check_lse(lse[heads][:, rows], lse_ref)
