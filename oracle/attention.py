"""fp64 CPU oracle for Jagged Flash Attention (JFA).

TEST INFRASTRUCTURE.  This module is the plain definition of what the HIP path
computes, written for a reader to check by eye.  It shares no code with the HIP
library and is never on the product path: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg use it.

What is computed (sources: the web pages on the method):

* "Meta's TLX attention kernel outpaces FlashAttention-4 on B200",
  section "GEM's sequences do not fit a fixed grid": sequences are packed
  back to back without padding and addressed through an offsets tensor; JFA is
  exact attention run directly on the packed tensors.  One dense query sequence
  may be broadcast to every batch element, and then every sequence adds into
  the same query gradient.
* "Optimizing Jagged Flash Attention with TLX" (reading note), section
  "Why variable lengths change the problem": the same two modes, and the
  batch-wide accumulation of the shared query gradient.
* "Meta's TLX Block Attention Beats Flash Attention v2 by 2.3x on Blackwell
  GPUs", section "The Pattern That Changes Everything": block-diagonal
  attention, where a token sees only the tokens of its own fixed-size group;
  here that is self-attention with every sequence of length 64.
  Section "One Constraint, Five Eliminations": the saved per-row
  log-sum-exp and the row-wise sum that the backward pass needs.

Readings where the pages are silent (each also listed in the design notes):

* The log-sum-exp is the natural logarithm of sum_j exp(c * q_i . k_j), taken
  over the scaled scores.  A row with no visible key (an empty sequence) has
  LSE = -inf and output 0.
* Causal masking is defined for self-attention only: key j is visible to
  query i (both counted from the start of the sequence) iff j <= i.
* The softmax scale c multiplies Q K^T before the softmax; gradients carry it.

Parity status: every function here is pinned by CPU tests against a padded
dense library reference, central finite differences, closed forms, a
hand-derived worked example and exact identities (tests/test_oracle.py).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def sequence_forward(qb, kb, vb, scale: float, causal: bool = False):
    """Exact softmax attention for one sequence and one head.

    qb: [Lq, D] queries, kb/vb: [n, D] keys/values.  Returns
    (O [Lq, D], lse [Lq]) in fp64.  Follows the plain definition
    O = softmax(c Q K^T) V, with the row log-sum-exp kept for the backward
    ("Meta's TLX Block Attention Beats Flash Attention v2 by 2.3x on Blackwell
    GPUs", section "One Constraint, Five Eliminations").
    """
    qb, kb, vb = _f64(qb), _f64(kb), _f64(vb)
    lq, n = qb.shape[0], kb.shape[0]
    if n == 0:
        return np.zeros((lq, vb.shape[1])), np.full(lq, -np.inf)
    s = scale * (qb @ kb.T)                                    # [Lq, n] scores
    if causal:
        i = np.arange(lq)[:, None]
        j = np.arange(n)[None, :]
        s = np.where(j <= i, s, -np.inf)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])                               # rows sum to 1
    return p @ vb, lse


def sequence_backward(qb, kb, vb, gb, scale: float, causal: bool = False):
    """Analytic gradients of L = sum(O * G) for one sequence and one head.

    Returns (dQ [Lq, D], dK [n, D], dV [n, D]).  Standard softmax-attention
    calculus: dV = P^T G; dP = G V^T; delta_i = sum_j P_ij dP_ij (the row-wise
    sum that "Meta's TLX Block Attention Beats Flash Attention v2 by 2.3x on
    Blackwell GPUs", section "One Constraint, Five Eliminations", calls the Di
    preprocessing); dS = P * (dP - delta);
    dK = c dS^T Q; dQ = c dS K.
    """
    qb, kb, vb, gb = _f64(qb), _f64(kb), _f64(vb), _f64(gb)
    lq, n, d = qb.shape[0], kb.shape[0], qb.shape[1]
    if n == 0:
        return np.zeros((lq, d)), np.zeros((0, d)), np.zeros((0, d))
    s = scale * (qb @ kb.T)
    if causal:
        i = np.arange(lq)[:, None]
        j = np.arange(n)[None, :]
        s = np.where(j <= i, s, -np.inf)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])
    dv = p.T @ gb
    dp = gb @ vb.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dk = scale * (ds.T @ qb)
    dq = scale * (ds @ kb)
    return dq, dk, dv


def sequence_dq_rows(qb, kb, vb, gb, rows, scale: float, causal: bool = False):
    """dQ of selected query rows only, for one sequence and one head.

    Each row of dQ depends only on that row's scores: dQ_i = c sum_j dS_ij k_j with
    dS_ij = P_ij (dP_ij - delta_i).  Same definition as sequence_backward, restricted
    to the listed rows so that a batch-summed dQ row can be checked at full size.
    Returns [len(rows), D].
    """
    qb, kb, vb, gb = _f64(qb), _f64(kb), _f64(vb), _f64(gb)
    rows = np.asarray(rows, dtype=np.int64)
    n, d = kb.shape[0], kb.shape[1]
    if n == 0:
        return np.zeros((len(rows), d))
    s = scale * (qb[rows] @ kb.T)
    if causal:
        j = np.arange(n)[None, :]
        s = np.where(j <= rows[:, None], s, -np.inf)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])
    dp = gb[rows] @ vb.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    return scale * (ds @ kb)


def row_count(offsets, broadcast_q: bool, q_len: int) -> int:
    """Number of output rows: B * Lq for broadcast-Q, T = offsets[B] otherwise."""
    offsets = np.asarray(offsets, dtype=np.int64)
    b = len(offsets) - 1
    return b * q_len if broadcast_q else int(offsets[-1])


def _check(q, k, offsets, broadcast_q, causal):
    if broadcast_q and causal:
        raise ValueError("causal masking is defined for self-attention only")
    offsets = np.asarray(offsets, dtype=np.int64)
    if offsets[0] != 0 or np.any(np.diff(offsets) < 0) or offsets[-1] != k.shape[0]:
        raise ValueError("offsets must start at 0, be non-decreasing and end at T")
    return offsets


def forward(q, k, v, offsets, *, broadcast_q: bool, causal: bool = False, scale: float):
    """Jagged attention forward over a packed batch.

    q: [Lq, H, D] (broadcast-Q) or [T, H, D] (self); k, v: [T, H, D];
    offsets: [B + 1].  Returns O [rows, H, D] and LSE [H, rows] in fp64 where
    rows = B * Lq (broadcast, row b * Lq + i belongs to sequence b) or T.
    Plain per-sequence, per-head loop ("Meta's TLX attention kernel outpaces
    FlashAttention-4 on B200", section "GEM's sequences do not fit a fixed grid").
    """
    offsets = _check(q, k, offsets, broadcast_q, causal)
    b_count = len(offsets) - 1
    h_count, d = k.shape[1], k.shape[2]
    lq = q.shape[0] if broadcast_q else 0
    rows = row_count(offsets, broadcast_q, lq)
    out = np.zeros((rows, h_count, d))
    lse = np.full((h_count, rows), -np.inf)
    for b in range(b_count):
        a, e = int(offsets[b]), int(offsets[b + 1])
        r0, r1 = (b * lq, (b + 1) * lq) if broadcast_q else (a, e)
        for h in range(h_count):
            qb = q[:, h, :] if broadcast_q else q[a:e, h, :]
            o_b, lse_b = sequence_forward(qb, k[a:e, h, :], v[a:e, h, :], scale, causal)
            out[r0:r1, h, :] = o_b
            lse[h, r0:r1] = lse_b
    return out, lse


def backward(q, k, v, offsets, g, *, broadcast_q: bool, causal: bool = False, scale: float):
    """Gradients of L = sum(O * G) for the packed batch.

    Returns dQ (shape of q), dK, dV (shape of k).  In broadcast-Q mode every
    sequence adds its query gradient into the one shared dQ ("Meta's TLX attention
    kernel outpaces FlashAttention-4 on B200", section "GEM's sequences do not fit a
    fixed grid").
    """
    offsets = _check(q, k, offsets, broadcast_q, causal)
    b_count = len(offsets) - 1
    h_count, d = k.shape[1], k.shape[2]
    lq = q.shape[0] if broadcast_q else 0
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(b_count):
        a, e = int(offsets[b]), int(offsets[b + 1])
        r0, r1 = (b * lq, (b + 1) * lq) if broadcast_q else (a, e)
        for h in range(h_count):
            qb = q[:, h, :] if broadcast_q else q[a:e, h, :]
            dq_b, dk_b, dv_b = sequence_backward(qb, k[a:e, h, :], v[a:e, h, :],
                                                 g[r0:r1, h, :], scale, causal)
            if broadcast_q:
                dq[:, h, :] += dq_b
            else:
                dq[a:e, h, :] = dq_b
            dk[a:e, h, :] = dk_b
            dv[a:e, h, :] = dv_b
    return dq, dk, dv
