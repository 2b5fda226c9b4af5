"""fp64 CPU oracle for the MXFP8 forward (block-scaled 8-bit attention).

TEST INFRASTRUCTURE, like the rest of this package: the plain definition of what
the MXFP8 HIP path computes, never on the product path.

Source: "Meta's TLX attention kernel outpaces FlashAttention-4 on B200", section on
the kernel's variants (an MXFP8 fork: E4M3 values with an E8M0 scale for each
block, the forward ahead of FA4's FP8 path); "Optimizing Jagged Flash Attention
with TLX" reading note (the same kernel structure reused for the low-precision
variant).

Readings where the pages are silent (each also listed in the design notes):

* E4M3 is the OCP 8-bit float: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits, subnormals, no infinities, S.1111.111 is NaN, largest finite value 448.
  E8M0 is an 8-bit power of two, code c standing for 2^(c - 127).
* An MX block is 32 consecutive elements along a product's contraction axis:
  Q and K rows in blocks of 32 columns of the head dimension; V in blocks of 32
  consecutive keys of one sequence and one column (the first block starts at the
  sequence's first key, the last may be partial); P in blocks of 32 consecutive
  keys of a row, aligned the same way.
* A block's scale is the smallest power of two 2^e with max|x| <= 448 * 2^e, so
  that no element saturates (code clamped to [0, 254]; an all-zero block gets
  code 0).  Each element becomes x / 2^e rounded to the nearest E4M3 value, ties
  to the even mantissa.
* Softmax in base 2: x = fp32(S) * fp32(c log2 e); the row maximum is rounded up to
  an integer m, so every rescale of the running sums is an exact power of two and
  the quantized P does not depend on the order in which the key blocks are visited;
  p = 2^(x - m) in fp32; l = sum of the unquantized p; O = (deq P)(deq V) / l and
  LSE = ln 2 * (m + log2 l).  The quantization decisions for P are taken on these
  fp32 values (the precision of the HIP path); the sums are fp64.

Parity status: pinned by CPU tests (tests/test_oracle_mxfp8.py): the E4M3 table
against its field definition and known values; rounding against brute force over
all finite values; the scale rule's minimality; scores that are integers in base 2
reduce the forward to the dense oracle exactly; the P quantization error bound
against the dense oracle on the dequantized inputs; integer shifts of the scores
leave the result unchanged.  The slack is pinned by brute force over the E4M3
values: exactly 0 on rows with no decision near a tie or a scale boundary; every
flagged decision taken the other way (singly and all together) moves O by no more
than it; and a row with a single near-tie gets exactly that flip's effect.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
MX_BLOCK = 32
E8M0_MAX_CODE = 254
LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code (the field definition)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_ulp(y):
    """Spacing of E4M3 values at |y| (|y| <= 448)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    out = np.full(a.shape, 2.0 ** -9)
    big = a >= 2.0 ** -6
    out[big] = 2.0 ** (np.floor(np.log2(a[big])) - 3)
    return out


def e4m3_round(y):
    """Nearest E4M3 value to each y (|y| <= 448), ties to the even mantissa."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("e4m3_round: |y| above 448")
    step = e4m3_ulp(y)
    # within a binade the values are k * step with k = 8 .. 16, and an even k is an
    # even mantissa; below 2^-6 they are k * 2^-9, k = 0 .. 8.  np.round ties to even.
    return np.round(y / step) * step


def scale_exponent(amax) -> np.ndarray:
    """Smallest e with amax <= 448 * 2^e, clamped to the E8M0 range [-127, 127];
    -127 (code 0) for an all-zero block."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(a)                        # a = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 10               # 448 * 2^(ex - 10) < 0.5 * 2^ex <= a: below the answer
    for _ in range(4):                         # step up while the bound fails
        e = np.where(a > E4M3_MAX * np.ldexp(1.0, e), e + 1, e)
    e = np.where(a == 0.0, -127, e)
    return np.clip(e, -127, E8M0_MAX_CODE - 127)


def _quantize_last_axis(x):
    """Blocks of 32 along the last axis (zero-padded): (dequantized values, scale
    codes [..., blocks])."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    nb = (n + MX_BLOCK - 1) // MX_BLOCK
    pad = np.zeros(x.shape[:-1] + (nb * MX_BLOCK,))
    pad[..., :n] = x
    blocks = pad.reshape(x.shape[:-1] + (nb, MX_BLOCK))
    e = scale_exponent(np.abs(blocks).max(axis=-1))
    s = np.ldexp(1.0, e)[..., None]
    deq = e4m3_round(blocks / s) * s
    return deq.reshape(pad.shape)[..., :n], (e + 127).astype(np.int64)


def quantize_rows(x):
    """Q or K [rows, H, D] (D a multiple of 32): blocks of 32 head-dimension columns.
    Returns (dequantized [rows, H, D] fp64, scale codes [rows, H, D / 32])."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % MX_BLOCK:
        raise ValueError("head_dim must be a multiple of 32")
    return _quantize_last_axis(x)


def quantize_v(v, offsets):
    """V [total_kv, H, D]: blocks of 32 consecutive keys of one sequence and column.
    Returns (dequantized [total_kv, H, D] fp64, per-sequence scale codes: a list of
    [blocks_b, H, D] arrays, block j covering keys 32 j .. 32 j + 31 of sequence b)."""
    v = np.asarray(v, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    deq = np.zeros_like(v)
    scales = []
    for b in range(len(offsets) - 1):
        a, e = int(offsets[b]), int(offsets[b + 1])
        vt = np.moveaxis(v[a:e], 0, -1)                      # [H, D, n]
        d, s = _quantize_last_axis(vt)
        deq[a:e] = np.moveaxis(d, -1, 0)
        scales.append(np.moveaxis(s, -1, 0))                 # [blocks, H, D]
    return deq, scales


def quantize_p(p):
    """P [rows, n] (fp32 values, as computed by the forward): blocks of 32 keys.
    Returns (dequantized P fp64, the block exponents [rows, blocks], y = p / 2^e)."""
    p = np.asarray(p, dtype=np.float64)
    deq, codes = _quantize_last_axis(p)
    e = codes - 127
    n = p.shape[-1]
    y = p / np.repeat(np.ldexp(1.0, e), MX_BLOCK, axis=-1)[..., :n]
    return deq, e, y


def _near(a, b, rel):
    return np.abs(a - b) <= rel * np.maximum(np.abs(a), np.abs(b))


def attend_base2(x, vd, rel_tie: float = 2.0 ** -12):
    """Softmax attention from fp32 base-2 scores x [rows, n] (-inf for masked keys,
    every row with at least one key) over dequantized V [n, D], with P quantized in
    blocks of 32 keys.  Returns (o, lse2, slack): lse2 = m + log2 l in base 2, and
    slack[i] bounds how far O[i] may move when a rounding decision for P that lies
    within rel_tie of a tie (or of a block-scale boundary) is taken the other way
    by a computation of the same values in another order."""
    x = np.asarray(x, dtype=np.float32)
    vd = np.asarray(vd, dtype=np.float64)
    n = x.shape[1]
    m = np.ceil(x.max(axis=1).astype(np.float64))
    p = np.exp2((x - m[:, None].astype(np.float32)).astype(np.float32)).astype(np.float32)
    l = p.astype(np.float64).sum(axis=1)
    pd, e, y = quantize_p(p)
    o = (pd @ vd) / l[:, None]
    lse2 = m + np.log2(l)
    # sensitivity of the rounding decisions
    ulp = e4m3_ulp(y)
    mid = (np.floor(y / ulp) + 0.5) * ulp
    tie = _near(y, mid, rel_tie) & (p > 0)
    nb = e.shape[1]
    amax = np.stack([p[:, j * MX_BLOCK:(j + 1) * MX_BLOCK].astype(np.float64).max(axis=1)
                     for j in range(nb)], axis=1)
    # a scale decision near one of its boundaries
    edge = (_near(amax, E4M3_MAX * np.ldexp(1.0, e - 1), rel_tie)
            | _near(amax, E4M3_MAX * np.ldexp(1.0, e), rel_tie))
    edge_el = np.repeat(edge, MX_BLOCK, axis=1)[:, :n] & (p > 0)
    sens = (np.where(tie, ulp, 0.0)
            + np.where(edge_el, 2.0 * ulp + 2.0 * e4m3_ulp(np.minimum(2 * y, E4M3_MAX)), 0.0))
    sens = sens * np.repeat(np.ldexp(1.0, e), MX_BLOCK, axis=1)[:, :n]
    slack = (sens * np.abs(vd).max(axis=1)[None, :]).sum(axis=1) / l
    return o, lse2, slack


def base2_scores(qd, kd, scale: float, causal: bool = False):
    """x = fp32(Q K^T) * fp32(c log2 e), -inf above the diagonal when causal."""
    s = np.asarray(qd, dtype=np.float64) @ np.asarray(kd, dtype=np.float64).T
    x = s.astype(np.float32) * np.float32(scale * LOG2E)
    if causal:
        r, n = x.shape
        x = np.where(np.arange(n)[None, :] <= np.arange(r)[:, None], x, np.float32(-np.inf))
    return x


def sequence_forward_mx(qd, kd, vd, scale: float, causal: bool = False):
    """One sequence and head on dequantized (exactly representable) Q, K, V.
    Returns (o, lse, slack) with LSE in natural log units."""
    qd, kd, vd = (np.asarray(t, dtype=np.float64) for t in (qd, kd, vd))
    r, n = len(qd), len(kd)
    if n == 0 or r == 0:
        return np.zeros((r, vd.shape[1])), np.full(r, -np.inf), np.zeros(r)
    o, lse2, slack = attend_base2(base2_scores(qd, kd, scale, causal), vd)
    return o, LN2 * lse2, slack


def forward_mx(q, k, v, offsets, *, broadcast_q: bool, causal: bool = False, scale: float):
    """MXFP8 forward for the packed batch from bf16-valued Q, K, V: quantize Q and K
    by rows, V by key blocks, then attend.  Returns (O, LSE, slack) laid out as the
    dense forward's outputs (slack per output row and head, [H, rows])."""
    offsets = np.asarray(offsets, dtype=np.int64)
    qd, _ = quantize_rows(q)
    kd, _ = quantize_rows(k)
    vd, _ = quantize_v(v, offsets)
    b_count, h_count = len(offsets) - 1, kd.shape[1]
    lq = qd.shape[0] if broadcast_q else 0
    rows = b_count * lq if broadcast_q else kd.shape[0]
    out = np.zeros((rows, h_count, vd.shape[2]))
    lse = np.full((h_count, rows), -np.inf)
    slack = np.zeros((h_count, rows))
    for b in range(b_count):
        a, e = int(offsets[b]), int(offsets[b + 1])
        r0, r1 = (b * lq, (b + 1) * lq) if broadcast_q else (a, e)
        for h in range(h_count):
            qb = qd[:, h, :] if broadcast_q else qd[a:e, h, :]
            o_b, l_b, s_b = sequence_forward_mx(qb, kd[a:e, h, :], vd[a:e, h, :], scale, causal)
            out[r0:r1, h, :] = o_b
            lse[h, r0:r1] = l_b
            slack[h, r0:r1] = s_b
    return out, lse, slack
