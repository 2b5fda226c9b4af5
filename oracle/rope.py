"""fp64 CPU oracle for the rotary-embedding conjugate in the attention backward.

TEST INFRASTRUCTURE, like the rest of this package: the plain definition of what
the fused HIP path computes, never on the product path.

Source: "Meta's TLX Block Attention Beats Flash Attention v2 by 2.3x on Blackwell
GPUs", section "The Rotary Fusion Bonus".  Rotary position embeddings rotate the
query and key vectors by a position-dependent angle before attention; the
backward pass applies the conjugate (inverse) rotation to the query and key
gradients.  The pages fuse that conjugate into the attention backward, in fp32,
before the gradients are rounded to bf16.

Readings where the pages are silent (each also listed in the design notes):

* Pairing: element d is rotated together with element d + D/2 (the two halves
  of the head dimension), for d < D/2.
* The angles come from the caller as tables ``cos[p, d]`` and ``sin[p, d]``
  (shape [max_pos, D/2]) and per-row positions; the rotation of a row at
  position p is

      x'[d]       = x[d] cos[p, d] - x[d + D/2] sin[p, d]
      x'[d + D/2] = x[d + D/2] cos[p, d] + x[d] sin[p, d].

* The attention inputs are the rotated vectors q' = R q0 and k' = R k0; the
  gradients returned are those with respect to q0 and k0.

Parity status: pinned by CPU tests (tests/test_oracle.py): the adjoint identity
<R x, y> = <x, R^T y>, the quarter-turn closed form, the zero-angle reduction to
the plain backward, and central finite differences of
L(q0, k0, v) = sum(O(R q0, R k0, v) * G) for every element of q0 and k0.
"""
from __future__ import annotations

import numpy as np

from .attention import backward


def _tables(cos, sin, pos, d):
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    if cos.shape != sin.shape or cos.ndim != 2 or cos.shape[1] * 2 != d:
        raise ValueError("cos / sin must both be [max_pos, D/2]")
    if pos.size and (pos.min() < 0 or pos.max() >= cos.shape[0]):
        raise ValueError("positions must lie in [0, max_pos)")
    # [rows, 1 (heads), D/2]
    return cos[pos][:, None, :], sin[pos][:, None, :]


def rope_rotate(x, cos, sin, pos):
    """x' = R(pos) x for x of shape [rows, H, D]: the pair (d, d + D/2) of row r
    is rotated by the angle with cosine cos[pos[r], d] and sine sin[pos[r], d]."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[2] // 2
    c, s = _tables(cos, sin, pos, x.shape[2])
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=2)


def rope_conjugate(g, cos, sin, pos):
    """R(pos)^T g: the gradient with respect to x of a loss whose gradient with
    respect to x' = R(pos) x is g (the rotation by the opposite angle)."""
    g = np.asarray(g, dtype=np.float64)
    half = g.shape[2] // 2
    c, s = _tables(cos, sin, pos, g.shape[2])
    a, b = g[..., :half], g[..., half:]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=2)


def backward_rope(q_rot, k_rot, v, offsets, g, cos, sin, pos_q, pos_k, *, broadcast_q: bool,
                  causal: bool = False, scale: float):
    """Gradients with respect to (q0, k0, v) where attention ran on q_rot = R(pos_q) q0
    and k_rot = R(pos_k) k0: the plain attention backward with respect to q_rot and
    k_rot, then the conjugate rotation of those two gradients."""
    dq_rot, dk_rot, dv = backward(q_rot, k_rot, v, offsets, g, broadcast_q=broadcast_q,
                                  causal=causal, scale=scale)
    return (rope_conjugate(dq_rot, cos, sin, pos_q), rope_conjugate(dk_rot, cos, sin, pos_k), dv)
