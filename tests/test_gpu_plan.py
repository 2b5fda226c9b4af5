"""The tile plans the device builds (white-box: read from the workspace).

The plan is a stable descending counting sort of the work items by their cost, the
number of 64-key blocks a tile visits ("Meta's TLX attention kernel outpaces
FlashAttention-4 on B200", section "Five changes unlocked the gains", item 1): costs
must not increase along the list, items of equal cost keep (sequence, query block)
order, every item appears exactly once, and two calls give the same list.  The
backward plan lists the tiles of each sequence in order, split in self mode between
the sequences of one tile and the longer ones.

Workspace layout (api.cpp): the buffer is aligned up to 256 bytes, then the meta words
(item count first) take 256 bytes and the items follow, 16 bytes each:
(sequence, query block, first row, length).
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def _jfa():
    import variable_length_flash_jfa_amd as jfa
    return jfa


def _plan(case, sched):
    jfa = _jfa()
    q, k, v = (case[x].cuda() for x in ("q", "k", "v"))
    off = case["offsets"].cuda()
    bq, causal = case["broadcast_q"], case["causal"]
    lengths = case["lengths"]
    need = jfa.fwd_workspace_size(len(lengths), k.shape[1], k.shape[2], q.shape[0] if bq else 0,
                                  k.shape[0], bq, causal)
    ws = torch.zeros(need + 256, dtype=torch.uint8, device="cuda")
    old = jfa.get_schedule()
    jfa.set_schedule(sched)
    try:
        jfa.fwd(q, k, v, off, broadcast_q=bq, causal=causal, scale=case["scale"], workspace=ws)
        torch.cuda.synchronize()
    finally:
        jfa.set_schedule(old)
    base = (-ws.data_ptr()) % 256
    raw = ws.cpu().numpy()[base:].view(np.int32)
    count = int(raw[0])
    items = raw[64:64 + 4 * count].reshape(count, 4).astype(np.int64)
    return items


def _cost(n, m, bm, causal):
    kv = min(n, (m + 1) * bm) if causal else n
    return min((kv + 63) // 64, 1023)


CASES = {
    # name: (lengths, broadcast_q, causal, q_len, rows per tile)
    "bcast": ([700, 3, 64, 129, 1000, 65, 2000, 31, 64, 64, 700, 0, 5000], True, False, 256, 256),
    "self_causal_long": ([700, 3, 640, 1290, 1000, 65, 2000, 31, 1290, 700], False, True, 0, 256),
    "self_short": ([100, 5, 300, 129, 128, 127, 300, 1, 64, 100], False, False, 0, 128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_plan_is_a_stable_descending_sort(name):
    lengths, bq, causal, lq, bm = CASES[name]
    case = workloads.make_case(lengths, heads=2, head_dim=128, broadcast_q=bq, causal=causal, q_len=lq,
                               seed=3, with_grad=False)
    off = np.concatenate([[0], np.cumsum(lengths)])
    items = _plan(case, 0)
    # every item exactly once, with its sequence's first row and length
    expect = sorted((b, m) for b, n in enumerate(lengths)
                    for m in range(1 if bq else (n + bm - 1) // bm))
    assert sorted(map(tuple, items[:, :2].tolist())) == expect
    assert np.array_equal(items[:, 2], off[items[:, 0]])
    assert np.array_equal(items[:, 3], np.asarray(lengths)[items[:, 0]])
    costs = np.array([_cost(int(n), int(m), bm, causal) for _, m, _, n in items])
    assert np.all(np.diff(costs) <= 0), "costs must not increase"
    for c in np.unique(costs):
        sel = items[costs == c][:, :2]
        keys = sel[:, 0] * 100000 + sel[:, 1]
        assert np.all(np.diff(keys) > 0), f"ties of cost {c} out of (sequence, block) order"
    # the same list on every call and under the dynamic schedule (which claims from it)
    assert np.array_equal(items, _plan(case, 0))
    assert np.array_equal(items, _plan(case, 2))


def test_forward_plan_of_many_segments_is_stable():
    """More than one planner segment (8192 sequences): the cursors carry over."""
    rng = np.random.default_rng(9)
    lengths = [int(x) for x in rng.integers(1, 700, size=9000)]
    case = workloads.make_case(lengths, heads=1, head_dim=64, broadcast_q=True, q_len=16, seed=4,
                               with_grad=False)
    items = _plan(case, 0)
    assert len(items) == 9000
    costs = (np.asarray(lengths)[items[:, 0]] + 63) // 64
    assert np.all(np.diff(costs) <= 0)
    for c in np.unique(costs):
        assert np.all(np.diff(items[costs == c][:, 0]) > 0)
    assert sorted(items[:, 0].tolist()) == list(range(9000))


def _bwd_plan(case):
    """meta words and items of the backward plan (same workspace layout as above)."""
    jfa = _jfa()
    q, k, v, g = (case[x].cuda() for x in ("q", "k", "v", "g"))
    off = case["offsets"].cuda()
    lengths = case["lengths"]
    kw = dict(broadcast_q=False, causal=case["causal"], scale=case["scale"])
    o, lse = jfa.fwd(q, k, v, off, **kw)
    need = jfa.bwd_workspace_size(len(lengths), k.shape[1], k.shape[2], 0, k.shape[0], False, case["causal"])
    ws = torch.zeros(need + 256, dtype=torch.uint8, device="cuda")
    jfa.bwd(q, k, v, off, o, lse, g, workspace=ws, **kw)
    torch.cuda.synchronize()
    base = (-ws.data_ptr()) % 256
    raw = ws.cpu().numpy()[base:].view(np.int32)
    meta = raw[:8].astype(np.int64)
    items = raw[64:64 + 4 * int(meta[0])].reshape(-1, 4).astype(np.int64)
    return meta, items


BWD_PLAN_CASES = {
    # name: (lengths, causal, keys per backward tile, split)
    # mean 49: 64-key tiles, and every sequence may fit one: the plan splits
    "split": ([64, 17, 150, 0, 10, 5, 64, 130, 30, 20], True, 64, True),
    # mean 224: 128-key tiles, too long on average for the single-tile kernel
    "no_split": ([700, 3, 64, 129, 0, 448], False, 128, False),
}


@pytest.mark.parametrize("name", list(BWD_PLAN_CASES))
def test_backward_plan_lists(name):
    """Self mode: the tiles of sequences longer than one tile come first, in (sequence,
    key block) order; with split the sequences of 1..bn keys follow, one item each, in
    sequence order, and the meta words give both lists' tile counts and the second's
    first item."""
    lengths, causal, bn, split = BWD_PLAN_CASES[name]
    heads = 2
    case = workloads.make_case(lengths, heads=heads, head_dim=128, broadcast_q=False, causal=causal,
                               q_len=0, seed=5)
    meta, items = _bwd_plan(case)
    off = np.concatenate([[0], np.cumsum(lengths)])
    first = [(b, j) for b, n in enumerate(lengths) if not (split and n <= bn)
             for j in range((n + bn - 1) // bn)]
    second = [(b, 0) for b, n in enumerate(lengths) if split and 1 <= n <= bn]
    assert int(meta[0]) == len(first) + len(second)
    assert int(meta[2]) == len(first) * heads
    assert int(meta[3]) == len(second) * heads
    if split:
        assert int(meta[5]) == len(first)
    assert [tuple(x) for x in items[:, :2].tolist()] == first + second
    assert np.array_equal(items[:, 2], off[items[:, 0]])
    assert np.array_equal(items[:, 3], np.asarray(lengths)[items[:, 0]])
