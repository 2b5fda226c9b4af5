"""GPU parity of the block-sparse top-k forward (jfa_fwd_sparse) against the fp64 oracle.

The selection is decided in fp32 on the GPU, so a near-tie may be broken
differently than in fp64.  The tests therefore check the selection the GPU returns
for validity (size min(k, blocks), ascending, distinct, in range, and no unselected
block scoring clearly above a selected one by the fp64 scores), and compare O and
LSE with the oracle's attention over exactly that selection
(max |O - O_ref| <= 1e-2, max |LSE - LSE_ref| <= 1e-3).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.sparse import KV_BLOCK, q_block

pytestmark = pytest.mark.gpu

TOL_O = 1e-2
TOL_LSE = 1e-3

CASES = {
    # name: (lengths, heads, head_dim, broadcast_q, q_len, topk)
    "bcast_d128_lq256": ([1, 63, 300, 700, 1000], 2, 128, True, 256, 4),
    "bcast_d128_lq512": ([5, 300, 700], 2, 128, True, 512, 3),
    "bcast_d64_lq200": ([3, 77, 256, 513], 2, 64, True, 200, 2),
    "bcast_empty_seq": ([10, 0, 70], 2, 64, True, 64, 2),
    "self_d128": ([1, 17, 64, 65, 200, 513, 1000], 2, 128, False, 0, 3),
    "self_d64": ([2, 33, 190, 257], 3, 64, False, 0, 1),
    "self_topk_covers_all": ([100, 64, 300], 2, 128, False, 0, 64),
}


def _jfa():
    import variable_length_flash_jfa_amd as jfa
    return jfa


def _f64(t):
    return t.to(torch.float64).numpy()


def _selection_from_gpu(sel, lengths, heads, broadcast_q, q_len):
    """GPU output [H, query blocks, k] -> selection[h][b][m] lists (natural order)."""
    sel = sel.cpu().numpy()
    qb = q_block(broadcast_q)
    nqb_b = [(q_len + qb - 1) // qb if broadcast_q else (n + qb - 1) // qb for n in lengths]
    out = []
    for h in range(heads):
        per_b, base = [], 0
        for b, nq in enumerate(nqb_b):
            per_b.append([[int(x) for x in sel[h, base + m] if x >= 0] for m in range(nq)])
            base += nq
        out.append(per_b)
    return out


def _check_selection(q, k, off, selection, topk, broadcast_q, scale, seqs=None):
    for h in range(k.shape[1]):
        for b in (range(len(off) - 1) if seqs is None else seqs):
            a, e = int(off[b]), int(off[b + 1])
            qb = q[:, h, :] if broadcast_q else q[a:e, h, :]
            scores = oracle.sparse.block_scores(qb, k[a:e, h, :], scale, q_block(broadcast_q))
            nkv = (e - a + KV_BLOCK - 1) // KV_BLOCK
            for m, got in enumerate(selection[h][b]):
                assert len(got) == min(topk, nkv), (h, b, m, got)
                assert got == sorted(set(got)) and all(0 <= j < nkv for j in got), (h, b, m, got)
                if len(got) < nkv:
                    rest = [j for j in range(nkv) if j not in got]
                    tol = 1e-4 * max(1.0, np.abs(scores[m]).max())
                    assert scores[m, got].min() >= scores[m, rest].max() - tol, (h, b, m)


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_forward_matches_oracle(name):
    lengths, h, d, bq, lq, topk = CASES[name]
    case = workloads.make_case(lengths, heads=h, head_dim=d, broadcast_q=bq, q_len=lq,
                               seed=zlib.crc32(name.encode()) % 1000)
    jfa = _jfa()
    q, k, v = (case[x].cuda() for x in ("q", "k", "v"))
    off = case["offsets"].cuda()
    o, lse, sel = jfa.fwd_sparse(q, k, v, off, broadcast_q=bq, topk=topk, scale=case["scale"], blocks=True)
    torch.cuda.synchronize()
    qf, kf, vf = (_f64(case[x]) for x in ("q", "k", "v"))
    offn = case["offsets"].numpy()
    selection = _selection_from_gpu(sel, lengths, h, bq, lq)
    _check_selection(qf, kf, offn, selection, topk, bq, case["scale"])
    o_ref, lse_ref = oracle.sparse.sparse_forward(qf, kf, vf, offn, selection, broadcast_q=bq,
                                                  scale=case["scale"])
    err = np.abs(_f64(o.cpu()) - o_ref).max()
    assert err <= TOL_O, f"O: {err:.3e}"
    got_lse = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(lse_ref))
    fin = ~np.isneginf(lse_ref)
    if fin.any():
        assert np.abs(got_lse[fin] - lse_ref[fin]).max() <= TOL_LSE


def test_sparse_with_every_block_matches_dense_forward():
    """topk at least the number of blocks: the dense attention (same tolerance)."""
    jfa = _jfa()
    case = workloads.make_case([1, 130, 400], heads=2, head_dim=128, broadcast_q=True, q_len=256, seed=3)
    q, k, v = (case[x].cuda() for x in ("q", "k", "v"))
    off = case["offsets"].cuda()
    o_s, lse_s = jfa.fwd_sparse(q, k, v, off, broadcast_q=True, topk=64, scale=case["scale"])
    o_d, lse_d = jfa.fwd(q, k, v, off, broadcast_q=True, scale=case["scale"])
    torch.cuda.synchronize()
    assert (o_s.float() - o_d.float()).abs().max().item() <= 2 * TOL_O
    assert (lse_s - lse_d).abs().max().item() <= 2 * TOL_LSE


def test_sparse_full_size_gem_sampled():
    """The GEM-shaped workload with half of a median sequence's blocks kept (k = 8):
    selection validity and O / LSE on sampled sequences."""
    jfa = _jfa()
    name, topk = "gem_broadcast", 8
    w = workloads.WORKLOADS[name]
    case = workloads.make_workload(name, device="cuda")
    q, k, v, off = case["q"], case["k"], case["v"], case["offsets"]
    o, lse, sel = jfa.fwd_sparse(q, k, v, off, broadcast_q=True, topk=topk, scale=case["scale"], blocks=True)
    torch.cuda.synchronize()
    lengths = case["lengths"]
    rng = np.random.default_rng(5)
    seqs = sorted(set(rng.choice(len(lengths), 6, replace=False).tolist()) | {int(np.argmax(lengths))})
    offn = case["offsets"].cpu().numpy().astype(np.int64)
    selection = _selection_from_gpu(sel, lengths, w.heads, True, w.q_len)
    qf = _f64(q.cpu())
    for b in seqs:
        a, e = int(offn[b]), int(offn[b + 1])
        kb = _f64(k[a:e].cpu())
        vb = _f64(v[a:e].cpu())
        sub_off = np.array([0, e - a])
        sub_sel = [[selection[h][b]] for h in range(w.heads)]
        _check_selection(qf, kb, sub_off, sub_sel, topk, True, case["scale"])
        o_ref, lse_ref = oracle.sparse.sparse_forward(qf, kb, vb, sub_off, sub_sel, broadcast_q=True,
                                                      scale=case["scale"])
        rows = slice(b * w.q_len, (b + 1) * w.q_len)
        assert np.abs(_f64(o[rows].cpu()) - o_ref).max() <= TOL_O, b
        assert np.abs(lse[:, rows].cpu().numpy() - lse_ref).max() <= TOL_LSE, b
