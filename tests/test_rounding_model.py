"""CPU pins of the fp64 rounding model (tests/rounding_model.py) that sets the gradient
bar of the growing-score GPU cases.

The model must be the oracle's backward exactly when its roundings are taken out; on
ordinary N(0, 1) inputs its gradient error must stay well inside the 2e-2 target (so
the target and the model agree where the target is met); and on the growing-score
inputs it shows the error those roundings alone cause, which is what the wider bar of
those cases rests on.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import rounding_model
import workloads


def _f64(t):
    return t.to(torch.float64).numpy()


def _rel_errors(case):
    kw = dict(broadcast_q=case["broadcast_q"], causal=case["causal"], scale=case["scale"])
    q, k, v, g = (_f64(case[x]) for x in ("q", "k", "v", "g"))
    off = case["offsets"].numpy()
    ref = oracle.backward(q, k, v, off, g, **kw)
    mod = rounding_model.backward_rounded(q, k, v, off, g, **kw)
    return [np.abs(a - b).max() / np.abs(b).max() for a, b in zip(mod, ref)]


@pytest.mark.parametrize("bq,causal", [(True, False), (False, True), (False, False)])
def test_model_without_rounding_is_the_oracle(bq, causal, monkeypatch):
    case = workloads.make_case([1, 17, 64, 90], heads=2, head_dim=32, broadcast_q=bq, causal=causal,
                               q_len=40 if bq else 0, seed=5)
    monkeypatch.setattr(rounding_model, "_bf16", lambda x: np.asarray(x, dtype=np.float64))
    assert max(_rel_errors(case)) <= 1e-12


def test_model_error_on_unit_normal_inputs_is_inside_the_target():
    case = workloads.make_case([1, 63, 64, 65, 130, 1000], heads=2, head_dim=128, broadcast_q=True,
                               q_len=256, seed=1)
    errs = _rel_errors(case)
    assert 0 < max(errs) <= 5e-3, errs


def test_model_error_on_growing_scores_approaches_the_target():
    """The D = 64 broadcast ramp case: bf16 dS and delta from the stored O alone give
    more than 1% of max |dQ|, near the 2e-2 target."""
    import test_gpu_parity as tp
    name = "bcast_d64_growing"
    lengths, h, d, bq, causal, lq, growth = tp.RESCALE_CASES[name]
    case = workloads.make_case(lengths, heads=h, head_dim=d, broadcast_q=bq, causal=causal, q_len=lq,
                               seed=zlib.crc32(name.encode()) % 1000)
    errs = _rel_errors(tp._ramp_keys(case, growth))
    assert 1e-2 < errs[0] < 2e-2, errs
