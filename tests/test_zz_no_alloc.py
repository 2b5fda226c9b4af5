"""jfa_fwd_noalloc (the forward that allocates nothing; its plan lives in a device array
inside the library) against jfa_fwd with a workspace, both called through the C ABI.

The two run the same plan and attention kernels, and a tile's result does not depend
on which workgroup runs it, so O and LSE must agree bit for bit.  Two calls in a row,
the second on a smaller problem, check that a call does not read the plan the previous
call left in the array.
"""
import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

WS_TOO_SMALL = 3


def _lib():
    from variable_length_flash_jfa_amd import _binding
    lib = _binding.library()
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    lib.jfa_fwd_noalloc.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, i32, f32, vp, vp, vp]
    lib.jfa_fwd_noalloc.restype = i32
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _sizes(case):
    lengths = case["lengths"]
    q, k = case["q"], case["k"]
    bq = case["broadcast_q"]
    batch, total_kv = len(lengths), int(k.shape[0])
    q_len = q.shape[0] if bq else 0
    rows = batch * q_len if bq else total_kv
    return batch, k.shape[1], k.shape[2], q_len, total_kv, rows


def _with_workspace(lib, case, off, q, k, v):
    batch, heads, d, q_len, total_kv, rows = _sizes(case)
    o = torch.full((rows, heads, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((heads, rows), float("nan"), dtype=torch.float32, device="cuda")
    need = lib.jfa_fwd_workspace_size(batch, heads, d, q_len, total_kv, int(case["broadcast_q"]),
                                      int(case["causal"]))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = lib.jfa_fwd(_p(q), _p(k), _p(v), _p(off), int(off.dtype == torch.int64), batch, heads, d, q_len,
                     total_kv, int(case["broadcast_q"]), int(case["causal"]), case["scale"], _p(o), _p(lse),
                     _p(ws), need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.jfa_last_error()
    return o, lse


def _noalloc(lib, case, off, q, k, v):
    batch, heads, d, q_len, total_kv, rows = _sizes(case)
    o = torch.full((rows, heads, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((heads, rows), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.jfa_fwd_noalloc(_p(q), _p(k), _p(v), _p(off), int(off.dtype == torch.int64), batch, heads, d,
                             q_len, total_kv, int(case["broadcast_q"]), int(case["causal"]), case["scale"],
                             _p(o), _p(lse), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.jfa_last_error()
    return o, lse


CASES = [
    # the larger problem first: long causal self-mode sequences (many plan items)
    ([900, 1200, 64, 700, 1, 333, 0, 2048], 2, 128, False, True, 0),
    # then a smaller broadcast problem: a stale plan from the first call would misplace tiles
    ([17, 64, 129], 3, 128, True, False, 100),
    # and a tiny self-mode problem of short sequences
    ([5, 64, 3], 2, 64, False, False, 0),
]


@pytest.mark.parametrize("sched", [2, 0])
def test_noalloc_forward_equals_workspace_forward_on_consecutive_calls(sched):
    import variable_length_flash_jfa_amd as jfa
    lib = _lib()
    old = jfa.get_schedule()
    jfa.set_schedule(sched)
    try:
        for i, (lengths, h, d, bq, causal, lq) in enumerate(CASES):
            print(f"case {i}: lengths {lengths}, H={h}, D={d}, broadcast={bq}, causal={causal}, Lq={lq}",
                  flush=True)
            case = workloads.make_case(lengths, heads=h, head_dim=d, broadcast_q=bq, causal=causal, q_len=lq,
                                       seed=100 + i)
            q, k, v = (case[x].cuda() for x in ("q", "k", "v"))
            off = case["offsets"].cuda()
            got_o, got_lse = _noalloc(lib, case, off, q, k, v)
            ref_o, ref_lse = _with_workspace(lib, case, off, q, k, v)
            torch.cuda.synchronize()
            assert torch.equal(got_o, ref_o), f"O differs in case {i}"
            assert torch.equal(got_lse, ref_lse), f"LSE differs in case {i}"
    finally:
        jfa.set_schedule(old)


def test_noalloc_rejects_a_plan_larger_than_its_scratch():
    """A self-mode batch of 200,000 one-token sequences needs more than 2 MiB of plan;
    the call is rejected before anything is launched."""
    lib = _lib()
    fake = ctypes.c_void_p(1 << 20)
    st = lib.jfa_fwd_noalloc(fake, fake, fake, fake, 0, 200000, 2, 128, 0, 200000, 0, 0, 0.1, fake, fake, None)
    assert st == WS_TOO_SMALL
    assert b"plan scratch" in lib.jfa_last_error()
