"""fp64 CPU oracle for block-sparse top-k attention (forward).

TEST INFRASTRUCTURE, like the rest of this package: the plain definition of what
the block-sparse HIP path computes, never on the product path.

Source: "Optimizing Jagged Flash Attention with TLX" (reading note), and "Meta's
TLX attention kernel outpaces FlashAttention-4 on B200", section on the kernel's
variants: a scoring step picks the top k key/value blocks for every query block,
and attention then runs only over the keys of the selected blocks.

Readings where the pages are silent (each also listed in the design notes):

* Key/value blocks are 64 consecutive keys of a sequence (the last one may be
  partial); query blocks are 256 consecutive rows of the broadcast query sequence,
  or 128 consecutive rows of the sequence itself in self-attention (the last one
  may be partial).  These sizes are fixed constants of the method as read here;
  the pages give none.
* The score of (query block m, key block j) for a head is
  c * mean(Q rows of m) . mean(K rows of j): the dot product of the mean query row
  and the mean key row, times the softmax scale c.
* The k highest scores are selected, ties going to the lower block index; a
  sequence with k or fewer key blocks keeps all of them.  Selections are listed in
  ascending block order.
* Attention over the selection is exact softmax attention restricted to the keys
  of the selected blocks (no causal mask: the sparse variant is defined for the
  non-causal modes).

Where floating point decides the selection, the HIP path decides in fp32; the
tests therefore compare the attention over the selection the HIP path returns,
and check that selection against these fp64 scores up to near-ties.

Parity status: pinned by CPU tests (tests/test_oracle.py): k at least the number
of blocks reduces to the dense oracle; a fixed selection equals a padded dense
torch reference with the matching block mask; every block score equals the mean
of the exact scores c q_i . k_j over the block's rows and keys (linearity),
computed from the full score matrix, partial last blocks included; the selection
against a brute-force sort.
"""
from __future__ import annotations

import numpy as np

from .attention import sequence_forward

KV_BLOCK = 64
Q_BLOCK_BROADCAST = 256
Q_BLOCK_SELF = 128


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def q_block(broadcast_q: bool) -> int:
    return Q_BLOCK_BROADCAST if broadcast_q else Q_BLOCK_SELF


def query_blocks(n_rows: int, qblk: int) -> int:
    return (n_rows + qblk - 1) // qblk


def kv_blocks(n_keys: int) -> int:
    return (n_keys + KV_BLOCK - 1) // KV_BLOCK


def block_scores(qb, kb, scale: float, qblk: int):
    """Scores [query blocks, key blocks] for one sequence and head, query blocks of
    qblk rows: c * mean(query block rows) . mean(key block rows)."""
    qb, kb = _f64(qb), _f64(kb)
    nq, nk = query_blocks(len(qb), qblk), kv_blocks(len(kb))
    qm = np.stack([qb[m * qblk:(m + 1) * qblk].mean(axis=0) for m in range(nq)]) if nq else \
        np.zeros((0, qb.shape[1]))
    km = np.stack([kb[j * KV_BLOCK:(j + 1) * KV_BLOCK].mean(axis=0) for j in range(nk)]) if nk else \
        np.zeros((0, kb.shape[1]))
    return scale * qm @ km.T


def select_top_k(scores, topk: int):
    """Per row of scores: the indices of the topk highest, ties to the lower index,
    in ascending order (all indices when there are at most topk)."""
    out = []
    for row in np.asarray(scores, dtype=np.float64):
        order = sorted(range(len(row)), key=lambda j: (-row[j], j))
        out.append(sorted(order[:topk]))
    return out


def sequence_sparse_forward(qb, kb, vb, selection, scale: float, qblk: int):
    """Exact attention of each query block (qblk rows) over the keys of its selected
    blocks.  selection[m] lists the key blocks of query block m.  Returns (o, lse)."""
    qb, kb, vb = _f64(qb), _f64(kb), _f64(vb)
    o = np.zeros((len(qb), vb.shape[1]))
    lse = np.full(len(qb), -np.inf)
    for m in range(query_blocks(len(qb), qblk)):
        rows = slice(m * qblk, min((m + 1) * qblk, len(qb)))
        keys = np.concatenate([np.arange(j * KV_BLOCK, min((j + 1) * KV_BLOCK, len(kb)))
                               for j in selection[m]]) if len(selection[m]) else np.zeros(0, dtype=np.int64)
        o[rows], lse[rows] = sequence_forward(qb[rows], kb[keys], vb[keys], scale)
    return o, lse


def sparse_forward(q, k, v, offsets, selection, *, broadcast_q: bool, scale: float):
    """Block-sparse forward for the packed batch.  selection[h][b][m] lists the key
    blocks of query block m of sequence b for head h.  Returns (O, LSE) laid out as
    the dense forward's."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    offsets = np.asarray(offsets, dtype=np.int64)
    b_count, h_count = len(offsets) - 1, k.shape[1]
    lq = q.shape[0] if broadcast_q else 0
    rows = b_count * lq if broadcast_q else k.shape[0]
    out = np.zeros((rows, h_count, v.shape[2]))
    lse = np.full((h_count, rows), -np.inf)
    for b in range(b_count):
        a, e = int(offsets[b]), int(offsets[b + 1])
        r0, r1 = (b * lq, (b + 1) * lq) if broadcast_q else (a, e)
        for h in range(h_count):
            qb = q[:, h, :] if broadcast_q else q[a:e, h, :]
            o_b, l_b = sequence_sparse_forward(qb, k[a:e, h, :], v[a:e, h, :], selection[h][b], scale,
                                               q_block(broadcast_q))
            out[r0:r1, h, :] = o_b
            lse[h, r0:r1] = l_b
    return out, lse


def select_all(q, k, offsets, topk: int, *, broadcast_q: bool, scale: float):
    """The oracle's own selection for the whole batch, selection[h][b][m]."""
    q, k = _f64(q), _f64(k)
    offsets = np.asarray(offsets, dtype=np.int64)
    sel = []
    for h in range(k.shape[1]):
        per_b = []
        for b in range(len(offsets) - 1):
            a, e = int(offsets[b]), int(offsets[b + 1])
            qb = q[:, h, :] if broadcast_q else q[a:e, h, :]
            per_b.append(select_top_k(block_scores(qb, k[a:e, h, :], scale, q_block(broadcast_q)), topk))
        sel.append(per_b)
    return sel
