"""Every-row GPU parity of the four large workloads at full size, in the launch
configuration the benchmark times (default schedule, int32 offsets).

Every output row -- O, LSE, dK, dV, and dQ (per row in self mode; the batch-summed
[Lq, H, D] in broadcast mode) -- is compared with a plain fp32 PyTorch reference run
on the GPU.  The reference is the definition written out with library products, one
chunk of length-sorted sequences at a time, padded to the chunk's longest sequence:
S = c Q K^T (masked), P = softmax(S), O = P V, LSE = m + log l; dV = P^T G, dP = G V^T,
delta = rowsum(P dP), dS = P (dP - delta), dK = c dS^T Q, dQ = c dS K.  It is independent
of the HIP path; the fp64 oracle itself is checked against the HIP path on sampled
sequences of the same workloads in test_gpu_parity.py (at this size the oracle would
take hours on the host).

Tolerances (the method's accuracy target): max |O - O_ref| <= 1e-2 plus half a bf16 ulp
of O (the output's rounding, see test_gpu_many_sequences.py), max |LSE - LSE_ref| <= 1e-3,
and for dQ, dK, dV max abs error <= 2e-2 * max |ref| over the whole tensor.
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
CHUNK_ELEMS = 1 << 26   # score elements per head and reference chunk (256 MiB in fp32)


def _jfa():
    import variable_length_flash_jfa_amd as jfa
    return jfa


class _Err:
    """Running max abs error and max |ref| of one output tensor."""

    def __init__(self):
        self.err = 0.0
        self.ref = 0.0

    def add(self, got, ref):
        if ref.numel():
            self.err = max(self.err, (got.float() - ref).abs().max().item())
            self.ref = max(self.ref, ref.abs().max().item())


def _o_excess(got, ref):
    """max over elements of |got - ref| minus half a bf16 ulp of the larger magnitude."""
    if not ref.numel():
        return 0.0
    got = got.float()
    _, e = torch.frexp(torch.maximum(got.abs(), ref.abs()))
    return ((got - ref).abs() - torch.ldexp(torch.ones_like(ref), e - 9)).max().item()


def _chunks(lengths, rows_per_seq):
    """Sequences sorted by length, grouped so that a chunk's padded score tensor holds at
    most CHUNK_ELEMS elements per head."""
    order = np.argsort(lengths, kind="stable")
    i = 0
    while i < len(order):
        j = i
        while j < len(order):
            lmax = max(int(lengths[order[j]]), 1)
            r = rows_per_seq if rows_per_seq else lmax
            if j > i and (j - i + 1) * r * lmax > CHUNK_ELEMS:
                break
            j += 1
        yield order[i:j]
        i = j


def reference_compare(case, out, rope=None):
    """Compares the HIP outputs `out` (dict of GPU tensors) with the fp32 reference,
    chunk by chunk; returns the error summary.  rope: optional (cos, sin, pos_q, pos_k)
    GPU tensors, applied to the reference dQ and dK as the conjugate rotation."""
    w = case["workload"]
    bq, causal, c = w.broadcast_q, w.causal, case["scale"]
    q, k, v, g = case["q"], case["k"], case["v"], case["g"]
    dev = k.device
    off = case["offsets"].cpu().numpy().astype(np.int64)
    lengths = np.diff(off)
    heads, d = k.shape[1], k.shape[2]
    lq = w.q_len
    err = {x: _Err() for x in ("lse", "dq", "dk", "dv")}
    o_excess = 0.0
    dq_sum = torch.zeros(lq, heads, d, device=dev, dtype=torch.float32) if bq else None

    def conj(x, pos):   # x [..., D] fp32 with a position per row, R(pos)^T x
        cs, sn = rope[0][pos], rope[1][pos]
        a, b = x[..., :d // 2], x[..., d // 2:]
        return torch.cat([a * cs + b * sn, b * cs - a * sn], dim=-1)

    qt = q.float().permute(1, 0, 2)[None] if bq else None            # [1, H, Lq, D]
    for seqs in _chunks(lengths, lq if bq else 0):
        n = torch.from_numpy(lengths[seqs]).to(dev)
        start = torch.from_numpy(off[seqs]).to(dev)
        lc = max(int(n.max().item()), 1)
        j = torch.arange(lc, device=dev)
        kv_ok = j[None, :] < n[:, None]                                # [Bc, Lc]
        idx = torch.where(kv_ok, start[:, None] + j[None, :], torch.zeros_like(j)[None, :])
        kc = k[idx].float().permute(0, 2, 1, 3).contiguous()           # [Bc, H, Lc, D]
        vc = v[idx].float().permute(0, 2, 1, 3).contiguous()
        if bq:
            qc = qt
            rows = torch.from_numpy(seqs).to(dev)[:, None] * lq + torch.arange(lq, device=dev)[None, :]
            row_ok = torch.ones(len(seqs), lq, dtype=torch.bool, device=dev)
        else:
            qc = q[idx].float().permute(0, 2, 1, 3).contiguous()
            rows = idx
            row_ok = kv_ok
        gc = g[rows].float().permute(0, 2, 1, 3).contiguous() * row_ok[:, None, :, None]
        s = torch.matmul(qc, kc.transpose(-1, -2).contiguous()) * c     # [Bc, H, R, Lc]
        keep = kv_ok[:, None, None, :]
        if causal:
            r_idx = torch.arange(s.shape[2], device=dev)
            keep = keep & (j[None, None, None, :] <= r_idx[None, None, :, None])
        s = s.masked_fill(~keep, float("-inf"))
        m = s.amax(dim=-1, keepdim=True)
        m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
        p = torch.exp(s - m)
        del s
        l = p.sum(dim=-1, keepdim=True)
        p = p / l.clamp_min(1e-30)
        o_ref = torch.matmul(p, vc)                                      # [Bc, H, R, D]
        lse_ref = torch.where(l > 0, m + torch.log(l.clamp_min(1e-30)), torch.full_like(l, float("-inf")))[..., 0]
        dv_ref = torch.matmul(p.transpose(-1, -2).contiguous(), gc)     # [Bc, H, Lc, D]
        dp = torch.matmul(gc, vc.transpose(-1, -2).contiguous())
        delta = (p * dp).sum(dim=-1, keepdim=True)
        ds = p * (dp - delta)
        del dp, p
        dk_ref = c * torch.matmul(ds.transpose(-1, -2).contiguous(), qc)   # qc broadcasts over Bc
        dq_ref = c * torch.matmul(ds, kc)                                # [Bc, H, R, D]
        del ds
        # HIP rows of this chunk, in the reference layout
        sel_rows = rows[row_ok]
        o_got = out["o"][sel_rows]                                       # [nrows, H, D]
        o_r = o_ref.permute(0, 2, 1, 3)[row_ok]
        o_excess = max(o_excess, _o_excess(o_got, o_r))
        lse_got = out["lse"][:, sel_rows]                                # [H, nrows]
        lse_r = lse_ref.permute(1, 0, 2)[:, row_ok]
        inf_r = torch.isneginf(lse_r)
        assert torch.equal(torch.isneginf(lse_got), inf_r), "LSE: -inf pattern differs"
        err["lse"].add(lse_got[~inf_r], lse_r[~inf_r])
        keys = idx[kv_ok]
        dk_r = dk_ref.permute(0, 2, 1, 3)[kv_ok]
        if rope is not None:
            dk_r = conj(dk_r, rope[3][keys].long()[:, None])
        err["dk"].add(out["dk"][keys], dk_r)
        err["dv"].add(out["dv"][keys], dv_ref.permute(0, 2, 1, 3)[kv_ok])
        if bq:
            dq_sum += dq_ref.sum(dim=0).permute(1, 0, 2)
        else:
            dq_r = dq_ref.permute(0, 2, 1, 3)[row_ok]
            if rope is not None:
                dq_r = conj(dq_r, rope[2][sel_rows].long()[:, None])
            err["dq"].add(out["dq"][sel_rows], dq_r)
    if bq:
        if rope is not None:
            dq_sum = conj(dq_sum, rope[2].long()[:, None])
        err["dq"].add(out["dq"], dq_sum)
    summary = {"o_excess": o_excess, **{x: (e.err, e.ref) for x, e in err.items()}}
    print(f"{w.name}: " + ", ".join(f"{x} {v_[0]:.3e} (max|ref| {v_[1]:.3e})" if isinstance(v_, tuple)
                                     else f"{x} {v_:.3e}" for x, v_ in summary.items()), flush=True)
    assert o_excess <= TOL_O, f"O: max abs err beyond bf16 rounding {o_excess:.3e} > {TOL_O}"
    assert err["lse"].err <= TOL_LSE, f"LSE: max abs err {err['lse'].err:.3e}"
    for x in ("dq", "dk", "dv"):
        tol = TOL_GRAD * max(err[x].ref, 1e-30)
        assert err[x].err <= tol, f"{x}: max abs err {err[x].err:.3e} > {tol:.3e}"
    return summary


def _run(case, rope=None):
    jfa = _jfa()
    w = case["workload"]
    q, k, v, g, off = case["q"], case["k"], case["v"], case["g"], case["offsets"]
    kw = dict(broadcast_q=w.broadcast_q, causal=w.causal, scale=case["scale"])
    o, lse = jfa.fwd(q, k, v, off, **kw)
    dq, dk, dv = jfa.bwd(q, k, v, off, o, lse, g, rope=rope, **kw)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("name", ["gem_broadcast", "dq_stress", "self_causal", "block64"])
def test_full_size_every_row(name):
    torch.backends.cuda.matmul.allow_tf32 = False
    print(f"{name}: running the HIP forward and backward", flush=True)
    case = workloads.make_workload(name, seed=0, device="cuda")
    out = _run(case)
    print(f"{name}: fp32 reference, every row", flush=True)
    reference_compare(case, out)


def test_full_size_block64_rope_every_row():
    """The fused rotary backward (jfa_bwd_rope) on the block-diagonal workload: dQ and
    dK against the reference gradients rotated back in fp32, dV as the plain one."""
    torch.backends.cuda.matmul.allow_tf32 = False
    case = workloads.make_workload("block64", seed=0, device="cuda")
    r = workloads.rope_inputs(case)
    rope = tuple(r[x].cuda() for x in ("cos", "sin", "pos_q", "pos_k"))
    print("block64 rope: running the HIP forward and fused rotary backward", flush=True)
    out = _run(case, rope=rope)
    reference_compare(case, out, rope=rope)
