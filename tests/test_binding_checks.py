"""The Python binding rejects every shape, dtype and device mismatch before it calls
the library (CPU tests: the checks run before any launch).

The C ABI receives raw pointers and indexes q, v, o and the gradients with k's row
stride, so a tensor of the wrong shape would be read or written out of bounds on the
device; the binding is the only layer that can catch it.
"""
import os

import pytest
import torch

from variable_length_flash_jfa_amd import _binding as jb

pytestmark = pytest.mark.skipif(not os.path.exists(jb.library_path()), reason="libjfa.so not built")

T, H, D, LQ = 40, 2, 64, 16


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def inputs(broadcast_q=True):
    q = bf16(LQ, H, D) if broadcast_q else bf16(T, H, D)
    k, v = bf16(T, H, D), bf16(T, H, D)
    off = torch.tensor([0, 10, 40], dtype=torch.int32)
    return q, k, v, off


ROWS_B = 2 * LQ


def expect(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_valid_cpu_tensors_fail_only_on_the_device_check():
    q, k, v, off = inputs()
    expect("on the GPU", jb.fwd, q, k, v, off, broadcast_q=True)
    o, lse = bf16(ROWS_B, H, D), torch.zeros(H, ROWS_B)
    expect("on the GPU", jb.bwd, q, k, v, off, o, lse, bf16(ROWS_B, H, D), broadcast_q=True)
    expect("on the GPU", jb.fwd_sparse, q, k, v, off, broadcast_q=True, topk=2)


@pytest.mark.parametrize("fn", ["fwd", "fwd_sparse"])
def test_forward_input_mismatches(fn):
    f = getattr(jb, fn)
    kw = {"topk": 2} if fn == "fwd_sparse" else {}
    q, k, v, off = inputs()
    expect("v must have k's shape", f, q, k, bf16(T, H, D // 2), off, broadcast_q=True, **kw)
    expect("v must have k's shape", f, q, k, bf16(T - 1, H, D), off, broadcast_q=True, **kw)
    expect("broadcast q must be", f, bf16(LQ, H + 1, D), k, v, off, broadcast_q=True, **kw)
    expect("broadcast q must be", f, bf16(LQ, H, 2 * D), k, v, off, broadcast_q=True, **kw)
    qs, ks, vs, off = inputs(broadcast_q=False)
    expect("self-mode q must have", f, bf16(T + 1, H, D), ks, vs, off, broadcast_q=False, **kw)
    expect("q must be bfloat16", f, q.float(), k, v, off, broadcast_q=True, **kw)
    expect("must be a \\[rows, heads, head_dim\\]", f, q[0], k, v, off, broadcast_q=True, **kw)
    expect("offsets must be", f, q, k, v, off.float(), broadcast_q=True, **kw)
    expect("offsets must be", f, q, k, v, off[None], broadcast_q=True, **kw)
    expect("k must be contiguous", f, q, bf16(H, T, D).transpose(0, 1), v, off, broadcast_q=True, **kw)
    expect("out must have shape", f, q, k, v, off, broadcast_q=True, out=bf16(ROWS_B - 1, H, D), **kw)
    expect("out must be torch.bfloat16", f, q, k, v, off, broadcast_q=True,
           out=torch.zeros(ROWS_B, H, D), **kw)
    expect("lse must have shape", f, q, k, v, off, broadcast_q=True, lse=torch.zeros(ROWS_B, H), **kw)
    expect("lse must be torch.float32", f, q, k, v, off, broadcast_q=True,
           lse=torch.zeros(H, ROWS_B, dtype=torch.float64), **kw)
    expect("workspace must be", f, q, k, v, off, broadcast_q=True,
           workspace=torch.zeros(64, 2)[:, 0], **kw)


def test_backward_mismatches():
    q, k, v, off = inputs()
    o, g, lse = bf16(ROWS_B, H, D), bf16(ROWS_B, H, D), torch.zeros(H, ROWS_B)
    kw = dict(broadcast_q=True)
    expect("o must have shape", jb.bwd, q, k, v, off, bf16(ROWS_B, H, D // 2), lse, g, **kw)
    expect("d_o must have shape", jb.bwd, q, k, v, off, o, lse, bf16(ROWS_B + 1, H, D), **kw)
    expect("d_o must be torch.bfloat16", jb.bwd, q, k, v, off, o, lse, g.float(), **kw)
    expect("lse must have shape", jb.bwd, q, k, v, off, o, torch.zeros(H, ROWS_B - 1), g, **kw)
    expect("dq must have shape", jb.bwd, q, k, v, off, o, lse, g, dq=bf16(T, H, D), **kw)
    expect("dk must have shape", jb.bwd, q, k, v, off, o, lse, g, dk=bf16(T, H, D // 2), **kw)
    expect("dv must be torch.bfloat16", jb.bwd, q, k, v, off, o, lse, g, dv=torch.zeros(T, H, D), **kw)
    expect("v must have k's shape", jb.bwd, q, k, bf16(T, H + 1, D), off, o, lse, g, **kw)
    cos, sin = torch.zeros(50, D // 2), torch.zeros(50, D // 2)
    pq, pk = torch.zeros(LQ, dtype=torch.int32), torch.zeros(T, dtype=torch.int32)
    expect("rope cos must have shape", jb.bwd, q, k, v, off, o, lse, g, rope=(torch.zeros(50, D), sin, pq, pk), **kw)
    expect("rope sin must have shape", jb.bwd, q, k, v, off, o, lse, g, rope=(cos, torch.zeros(49, D // 2), pq, pk),
           **kw)
    expect("rope pos_k must have shape", jb.bwd, q, k, v, off, o, lse, g,
           rope=(cos, sin, pq, torch.zeros(T - 1, dtype=torch.int32)), **kw)
    expect("rope pos_q must be torch.int32", jb.bwd, q, k, v, off, o, lse, g,
           rope=(cos, sin, pq.long(), pk), **kw)
    # self mode: rows are the packed sequences
    qs, ks, vs, off = inputs(broadcast_q=False)
    expect("o must have shape", jb.bwd, qs, ks, vs, off, o, torch.zeros(H, T), bf16(T, H, D), broadcast_q=False)
