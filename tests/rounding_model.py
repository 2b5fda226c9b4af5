"""An fp64 model of the two roundings the HIP backward makes before its gradient
products (test infrastructure).

The backward rounds dS = P (dP - delta) to bf16 for its matrix products, rounds P to
bf16 for dV, and takes delta = sum_d dO O from the O the forward stored (where the exact
delta is sum_j P dP); that O carries the forward's own roundings, P to bf16 in its P V
product and the result to bf16.  Everything else here is exact: the model shows how large
the gradient error of those roundings alone is for a given input, which is what a
parity bar wider than the method's target must rest on.  It shares nothing with the
HIP path; P, O and the products are the oracle's definition in fp64.
"""
from __future__ import annotations

import numpy as np
import torch


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def sequence_backward_rounded(qb, kb, vb, gb, scale, causal=False):
    """(dq, dk, dv) of one sequence and head with the backward's roundings modelled."""
    s = scale * (qb @ kb.T)
    if causal:
        r, n = s.shape
        s = np.where(np.arange(n)[None, :] <= np.arange(r)[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    # the forward's stored output: its P V product takes P in bf16 (the row sum l does
    # not), and O is stored in bf16
    o_bf16 = _bf16((_bf16(e) @ vb) / l)
    dp = gb @ vb.T
    delta = (gb * o_bf16).sum(axis=1, keepdims=True)
    ds = _bf16(p * (dp - delta))
    return scale * ds @ kb, scale * ds.T @ qb, _bf16(p).T @ gb


def backward_rounded(q, k, v, offsets, g, *, broadcast_q, causal, scale):
    offsets = np.asarray(offsets, dtype=np.int64)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    lq = q.shape[0] if broadcast_q else 0
    for b in range(len(offsets) - 1):
        a, e = int(offsets[b]), int(offsets[b + 1])
        if e == a:
            continue
        r0, r1 = (b * lq, (b + 1) * lq) if broadcast_q else (a, e)
        for h in range(k.shape[1]):
            qb = q[:, h] if broadcast_q else q[a:e, h]
            dqb, dkb, dvb = sequence_backward_rounded(qb, k[a:e, h], v[a:e, h], g[r0:r1, h], scale, causal)
            if broadcast_q:
                dq[:, h] += dqb
            else:
                dq[a:e, h] = dqb
            dk[a:e, h], dv[a:e, h] = dkb, dvb
    return dq, dk, dv
