"""GPU parity of the fused rotary backward (jfa_bwd_rope) against the fp64 oracle.

The forward attends with the rotated vectors; any bf16 q and k serve as those.  The
oracle's ``backward_rope`` is the plain attention backward with respect to them
followed by the conjugate rotation; the HIP path applies that rotation in fp32 in
its dK epilogue and dQ finalize.  Tolerances as for the plain backward:
max abs error <= 2e-2 * max |ref| for dQ, dK, dV.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2

CASES = {
    # name: (lengths, heads, head_dim, broadcast_q, causal, q_len)
    "bcast_d128_lq256": ([1, 63, 300, 700], 2, 128, True, False, 256),
    "bcast_d64_lq100": ([17, 64, 129], 2, 64, True, False, 100),
    "self_d128_causal": ([1, 5, 64, 127, 300], 2, 128, False, True, 0),
    "self_d64": ([2, 33, 190, 257], 3, 64, False, False, 0),
    # every sequence within one 64-key tile: the single-tile kernel rotates and stores dQ
    "self_d128_single_tile_lengths": ([64, 17, 64, 40], 2, 128, False, False, 0),
    # split between the single-tile kernel and the reduce-adding one, whose rows the
    # finalize rotates
    "self_d128_causal_short": ([3, 64, 100, 128, 1], 2, 128, False, True, 0),
    "self_d128_split": ([64, 17, 150, 10, 5, 64, 30, 20], 2, 128, False, False, 0),
    # mean length above one 128-key tile: with and without the conjugate every tile
    # reduce-adds its dQ, so the two calls run the same kernels
    "self_d128_causal_long_mean": ([1, 5, 64, 700, 300], 2, 128, False, True, 0),
}


def _jfa():
    import variable_length_flash_jfa_amd as jfa
    return jfa


def _case(name):
    lengths, h, d, bq, causal, lq = CASES[name]
    return workloads.make_case(lengths, heads=h, head_dim=d, broadcast_q=bq, causal=causal, q_len=lq,
                               seed=zlib.crc32(name.encode()) % 1000)


def _run(case, rope):
    jfa = _jfa()
    q, k, v, g = (case[x].cuda() for x in ("q", "k", "v", "g"))
    off = case["offsets"].cuda()
    kw = dict(broadcast_q=case["broadcast_q"], causal=case["causal"], scale=case["scale"])
    o, lse = jfa.fwd(q, k, v, off, **kw)
    rope_dev = None if rope is None else tuple(rope[x].cuda() for x in ("cos", "sin", "pos_q", "pos_k"))
    dq, dk, dv = jfa.bwd(q, k, v, off, o, lse, g, rope=rope_dev, **kw)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _f64(t):
    return t.to(torch.float64).numpy()


def _reference(case, rope):
    q, k, v, g = (_f64(case[x]) for x in ("q", "k", "v", "g"))
    return oracle.backward_rope(q, k, v, case["offsets"].numpy(), g, rope["cos"].numpy(),
                                rope["sin"].numpy(), rope["pos_q"].numpy(), rope["pos_k"].numpy(),
                                broadcast_q=case["broadcast_q"], causal=case["causal"], scale=case["scale"])


@pytest.mark.parametrize("name", list(CASES))
def test_rope_backward_matches_oracle(name):
    case = _case(name)
    rope = workloads.rope_inputs(case)
    got = _run(case, rope)
    ref = _reference(case, rope)
    for what, a, b in zip(("dQ", "dK", "dV"), got, ref):
        err = np.abs(_f64(a) - b).max()
        tol = TOL_GRAD * max(np.abs(b).max(), 1e-30)
        assert err <= tol, f"{name} {what}: max abs err {err:.3e} > {tol:.3e}"


def test_rope_at_zero_angle_equals_plain_backward():
    """cos = 1, sin = 0: the conjugate is the identity (self mode: bitwise, on a batch
    whose calls with and without the conjugate take the same kernels).  In a batch
    of short sequences the plain call gives most of them to the single-tile kernel,
    which forms delta as sum_j P dP instead of dO . O: equal up to rounding only."""
    case = _case("self_d128_causal_long_mean")
    rope = workloads.rope_inputs(case)
    rope["cos"] = torch.ones_like(rope["cos"])
    rope["sin"] = torch.zeros_like(rope["sin"])
    got = _run(case, rope)
    ref = _run(case, None)
    for what, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), what


def test_fused_rotation_beats_rotating_bf16_gradients():
    """The pages' accuracy point: rotating in fp32 before the bf16 rounding gives a
    smaller dQ / dK error than rotating the bf16 gradients of the plain backward."""
    case = _case("bcast_d128_lq256")
    rope = workloads.rope_inputs(case)
    fused = _run(case, rope)
    plain = _run(case, None)
    ref = _reference(case, rope)
    cos, sin = rope["cos"].numpy(), rope["sin"].numpy()
    for i, (what, pos) in enumerate((("dQ", rope["pos_q"].numpy()), ("dK", rope["pos_k"].numpy()))):
        unfused = oracle.rope_conjugate(_f64(plain[i]), cos, sin, pos)
        unfused = torch.from_numpy(unfused).to(torch.bfloat16).to(torch.float64).numpy()
        err_fused = np.abs(_f64(fused[i]) - ref[i]).max()
        err_unfused = np.abs(unfused - ref[i]).max()
        print(f"{what}: fused max err {err_fused:.3e}, unfused {err_unfused:.3e}")
        assert err_fused < err_unfused, (what, err_fused, err_unfused)
