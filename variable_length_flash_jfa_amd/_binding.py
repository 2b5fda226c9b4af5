"""ctypes binding of libjfa.so: argument marshalling only.

Names follow the C ABI (``jfa_fwd`` -> ``fwd``, ``jfa_bwd`` -> ``bwd``).  Tensors
must live on the current HIP device; work is enqueued on torch's current stream.
The library must have been built (``__graft_entry__.build()``); there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_lib", "libjfa.so")

SCHED_SORTED_ZIGZAG = 0
SCHED_IDENTITY = 1
SCHED_DYNAMIC = 2

_STATUS = {
    0: "JFA_OK",
    1: "JFA_ERR_INVALID_ARGUMENT",
    2: "JFA_ERR_UNSUPPORTED",
    3: "JFA_ERR_WORKSPACE_TOO_SMALL",
    4: "JFA_ERR_HIP",
}

_lock = threading.Lock()
_lib = None


class JfaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """Loads libjfa.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is missing: build the HIP library first "
                    "(python -c 'import __graft_entry__ as g; g.build()')")
            lib = ctypes.CDLL(_LIB_PATH)
            i64, i32, vp, f32, sz = (ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_float, ctypes.c_size_t)
            lib.jfa_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32]
            lib.jfa_fwd_workspace_size.restype = sz
            lib.jfa_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32]
            lib.jfa_bwd_workspace_size.restype = sz
            lib.jfa_fwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, i32, f32,
                                    vp, vp, vp, sz, vp]
            lib.jfa_fwd.restype = i32
            lib.jfa_bwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, i32, f32,
                                    vp, vp, vp, vp, vp, vp, vp, sz, vp]
            lib.jfa_bwd.restype = i32
            lib.jfa_bwd_rope.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, i32, f32,
                                         vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
            lib.jfa_bwd_rope.restype = i32
            lib.jfa_fwd_sparse_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32]
            lib.jfa_fwd_sparse_workspace_size.restype = sz
            lib.jfa_fwd_sparse_query_blocks.argtypes = [i64, i64, i64, i32]
            lib.jfa_fwd_sparse_query_blocks.restype = i64
            lib.jfa_fwd_sparse.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, f32, i32,
                                           vp, vp, vp, vp, sz, vp]
            lib.jfa_fwd_sparse.restype = i32
            lib.jfa_mxfp8_v_blocks.argtypes = [i64, i64]
            lib.jfa_mxfp8_v_blocks.restype = i64
            lib.jfa_mxfp8_quantize_rows.argtypes = [vp, i64, i64, i64, vp, vp, vp]
            lib.jfa_mxfp8_quantize_rows.restype = i32
            lib.jfa_mxfp8_quantize_v.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, vp]
            lib.jfa_mxfp8_quantize_v.restype = i32
            lib.jfa_fwd_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i64,
                                          i32, i32, f32, vp, vp, vp, sz, vp]
            lib.jfa_fwd_mxfp8.restype = i32
            lib.jfa_last_error.argtypes = []
            lib.jfa_last_error.restype = ctypes.c_char_p
            lib.jfa_version.argtypes = []
            lib.jfa_version.restype = ctypes.c_char_p
            lib.jfa_set_schedule.argtypes = [i32]
            lib.jfa_set_schedule.restype = i32
            lib.jfa_get_schedule.argtypes = []
            lib.jfa_get_schedule.restype = i32
            lib.jfa_profile_enable.argtypes = [i32]
            lib.jfa_profile_enable.restype = i32
            lib.jfa_profile_read.argtypes = [ctypes.c_char_p, i32, ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(ctypes.c_int64), i32,
                                             ctypes.POINTER(ctypes.c_int)]
            lib.jfa_profile_read.restype = i32
            _lib = lib
        return _lib


def _check(status: int) -> None:
    if status != 0:
        msg = library().jfa_last_error().decode(errors="replace")
        raise JfaError(status, msg)


def version() -> str:
    return library().jfa_version().decode()


def set_schedule(schedule: int) -> None:
    _check(library().jfa_set_schedule(int(schedule)))


def get_schedule() -> int:
    return int(library().jfa_get_schedule())


def profile_enable(enable: bool = True) -> None:
    """Brackets every kernel launch of this thread with HIP events on its stream."""
    _check(library().jfa_profile_enable(int(bool(enable))))


def profile_read(max_entries: int = 16) -> dict:
    """Waits for the recorded launches; returns {kernel: (total_ms, launches)} and clears."""
    name_len = 32
    names = ctypes.create_string_buffer(name_len * max_entries)
    ms = (ctypes.c_double * max_entries)()
    cnt = (ctypes.c_int64 * max_entries)()
    count = ctypes.c_int(0)
    _check(library().jfa_profile_read(names, name_len, ms, cnt, max_entries, ctypes.byref(count)))
    out = {}
    for i in range(min(count.value, max_entries)):
        raw = names.raw[i * name_len:(i + 1) * name_len]
        out[raw.split(b"\0", 1)[0].decode()] = (ms[i], int(cnt[i]))
    return out


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensor(name, t, dtype, shape, dev):
    """Raises ValueError unless t is a contiguous `dtype` tensor of `shape` on `dev`."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _problem(q, k, v, offsets, broadcast_q):
    """Checks q, k, v and offsets against each other; returns (device, batch, heads,
    head_dim, q_len, total_kv, rows).  The library indexes q, v, o, dq with k's row
    stride, so every tensor's shape is checked here: the C ABI sees raw pointers."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3:
            raise ValueError(f"{name} must be a [rows, heads, head_dim] tensor")
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    total_kv, heads, head_dim = k.shape
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v must have k's shape {tuple(k.shape)}, got {tuple(v.shape)}")
    if broadcast_q:
        if tuple(q.shape[1:]) != (heads, head_dim):
            raise ValueError(f"broadcast q must be [q_len, {heads}, {head_dim}], got {tuple(q.shape)}")
    elif tuple(q.shape) != tuple(k.shape):
        raise ValueError(f"self-mode q must have k's shape {tuple(k.shape)}, got {tuple(q.shape)}")
    if not isinstance(offsets, torch.Tensor) or offsets.dtype not in (torch.int32, torch.int64) or \
            offsets.dim() != 1 or offsets.numel() < 1:
        raise ValueError("offsets must be a 1-D int32 / int64 tensor of batch + 1 entries")
    for name, t in (("q", q), ("k", k), ("v", v), ("offsets", offsets)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dev = k.device
    for name, t in (("q", q), ("v", v), ("offsets", offsets)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    batch = offsets.numel() - 1
    q_len = q.shape[0] if broadcast_q else 0
    rows = batch * q_len if broadcast_q else total_kv
    return dev, batch, heads, head_dim, q_len, total_kv, rows


def _require_gpu(dev):
    """Checked last, so that every shape, dtype and device mismatch is reported first."""
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on the GPU, got {dev}")


def _workspace(ws, need, dev):
    """A caller-supplied workspace (any dtype, contiguous, on dev) or a new one; returns
    (tensor, bytes)."""
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif not isinstance(ws, torch.Tensor) or not ws.is_contiguous() or ws.device != dev:
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    return ws, ws.numel() * ws.element_size()


def fwd_workspace_size(batch, heads, head_dim, q_len, total_kv, broadcast_q, causal) -> int:
    return int(library().jfa_fwd_workspace_size(batch, heads, head_dim, q_len, total_kv,
                                                 int(broadcast_q), int(causal)))


def bwd_workspace_size(batch, heads, head_dim, q_len, total_kv, broadcast_q, causal) -> int:
    return int(library().jfa_bwd_workspace_size(batch, heads, head_dim, q_len, total_kv,
                                                int(broadcast_q), int(causal)))


def fwd(q, k, v, offsets, *, broadcast_q: bool, causal: bool = False, scale=None,
        out=None, lse=None, workspace=None):
    """O, LSE = jfa_fwd(...).  O: [rows, H, D] bf16; LSE: [H, rows] fp32."""
    dev, batch, heads, head_dim, q_len, total_kv, rows = _problem(q, k, v, offsets, broadcast_q)
    scale = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    if out is None:
        out = torch.empty((rows, heads, head_dim), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((heads, rows), dtype=torch.float32, device=dev)
    _check_tensor("out", out, torch.bfloat16, (rows, heads, head_dim), dev)
    _check_tensor("lse", lse, torch.float32, (heads, rows), dev)
    need = fwd_workspace_size(batch, heads, head_dim, q_len, total_kv, broadcast_q, causal)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    _require_gpu(dev)
    with torch.cuda.device(dev):
        st = library().jfa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                               int(offsets.dtype == torch.int64), batch, heads, head_dim, q_len,
                               total_kv, int(broadcast_q), int(causal), scale, _ptr(out), _ptr(lse),
                               _ptr(workspace), ws_bytes, _stream(dev))
    _check(st)
    return out, lse


def fwd_sparse(q, k, v, offsets, *, broadcast_q: bool, topk: int, scale=None, out=None, lse=None,
               blocks=False, workspace=None):
    """O, LSE (, blocks) = jfa_fwd_sparse(...): attention of every query block (256
    rows of the broadcast query, or 128 rows of a sequence in self mode) over its topk
    best-scoring 64-key blocks.  With blocks=True also returns the selection, int32
    [H, query blocks, topk] (ascending, -1 padded)."""
    dev, batch, heads, head_dim, q_len, total_kv, rows = _problem(q, k, v, offsets, broadcast_q)
    scale = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    if out is None:
        out = torch.empty((rows, heads, head_dim), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((heads, rows), dtype=torch.float32, device=dev)
    _check_tensor("out", out, torch.bfloat16, (rows, heads, head_dim), dev)
    _check_tensor("lse", lse, torch.float32, (heads, rows), dev)
    sel = None
    if blocks:
        nqb = int(library().jfa_fwd_sparse_query_blocks(batch, q_len, total_kv, int(broadcast_q)))
        sel = torch.empty((heads, nqb, int(topk)), dtype=torch.int32, device=dev)
    need = int(library().jfa_fwd_sparse_workspace_size(batch, heads, head_dim, q_len, total_kv,
                                                       int(broadcast_q), int(topk)))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    _require_gpu(dev)
    with torch.cuda.device(dev):
        st = library().jfa_fwd_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                                      int(offsets.dtype == torch.int64), batch, heads, head_dim, q_len,
                                      total_kv, int(broadcast_q), scale, int(topk), _ptr(out), _ptr(lse),
                                      _ptr(sel), _ptr(workspace), ws_bytes, _stream(dev))
    _check(st)
    return (out, lse, sel) if blocks else (out, lse)


def _check_bf16(name, t):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_contiguous() or \
            not t.is_cuda or t.dim() != 3:
        raise ValueError(f"{name} must be a contiguous bf16 GPU tensor [rows, heads, head_dim]")


def _check_offsets(offsets, dev):
    if not isinstance(offsets, torch.Tensor) or offsets.dtype not in (torch.int32, torch.int64) or \
            offsets.dim() != 1 or offsets.numel() < 1 or not offsets.is_contiguous() or offsets.device != dev:
        raise ValueError(f"offsets must be a contiguous 1-D int32 / int64 tensor on {dev}")


def mxfp8_quantize_rows(x, values=None, scales=None):
    """Q or K rows -> (E4M3 values uint8 [rows, H, D], E8M0 scales uint8 [rows, H, D / 32])."""
    _check_bf16("x", x)
    rows, heads, head_dim = x.shape
    if values is None:
        values = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, heads, head_dim // 32), dtype=torch.uint8, device=x.device)
    _check_tensor("values", values, torch.uint8, x.shape, x.device)
    _check_tensor("scales", scales, torch.uint8, (rows, heads, head_dim // 32), x.device)
    _require_gpu(x.device)
    with torch.cuda.device(x.device):
        _check(library().jfa_mxfp8_quantize_rows(_ptr(x), rows, heads, head_dim, _ptr(values), _ptr(scales),
                                                 _stream(x.device)))
    return values, scales


def mxfp8_v_blocks(batch: int, total_kv: int) -> int:
    return int(library().jfa_mxfp8_v_blocks(batch, total_kv))


def mxfp8_quantize_v(v, offsets, values=None, scales=None):
    """V -> (E4M3 values uint8 [G, H, D, 32], E8M0 scales uint8 [G, H, D]) in 32-key
    blocks of each sequence, G = mxfp8_v_blocks(batch, total_kv)."""
    _check_bf16("v", v)
    _check_offsets(offsets, v.device)
    total_kv, heads, head_dim = v.shape
    batch = offsets.numel() - 1
    g = mxfp8_v_blocks(batch, total_kv)
    if values is None:
        values = torch.zeros((g, heads, head_dim, 32), dtype=torch.uint8, device=v.device)
    if scales is None:
        scales = torch.zeros((g, heads, head_dim), dtype=torch.uint8, device=v.device)
    _check_tensor("values", values, torch.uint8, (g, heads, head_dim, 32), v.device)
    _check_tensor("scales", scales, torch.uint8, (g, heads, head_dim), v.device)
    _require_gpu(v.device)
    with torch.cuda.device(v.device):
        _check(library().jfa_mxfp8_quantize_v(_ptr(v), _ptr(offsets), int(offsets.dtype == torch.int64), batch,
                                              heads, head_dim, total_kv, _ptr(values), _ptr(scales),
                                              _stream(v.device)))
    return values, scales


def fwd_mxfp8(q8, q_scales, k8, k_scales, v8, v_scales, offsets, *, broadcast_q: bool,
              causal: bool = False, scale=None, out=None, lse=None, workspace=None):
    """O, LSE = jfa_fwd_mxfp8(...) on the outputs of mxfp8_quantize_rows (Q, K) and
    mxfp8_quantize_v (V).  O: [rows, H, D] bf16; LSE: [H, rows] fp32."""
    if not isinstance(k8, torch.Tensor) or k8.dim() != 3 or not isinstance(q8, torch.Tensor) or q8.dim() != 3:
        raise ValueError("q8 and k8 must be [rows, heads, head_dim] tensors")
    dev = k8.device
    total_kv, heads, head_dim = k8.shape
    _check_offsets(offsets, dev)
    batch = offsets.numel() - 1
    q_len = q8.shape[0] if broadcast_q else 0
    rows = batch * q_len if broadcast_q else total_kv
    g = mxfp8_v_blocks(batch, total_kv)
    _check_tensor("q8", q8, torch.uint8, (q8.shape[0] if broadcast_q else total_kv, heads, head_dim), dev)
    _check_tensor("q_scales", q_scales, torch.uint8, (q8.shape[0], heads, head_dim // 32), dev)
    _check_tensor("k8", k8, torch.uint8, (total_kv, heads, head_dim), dev)
    _check_tensor("k_scales", k_scales, torch.uint8, (total_kv, heads, head_dim // 32), dev)
    _check_tensor("v8", v8, torch.uint8, (g, heads, head_dim, 32), dev)
    _check_tensor("v_scales", v_scales, torch.uint8, (g, heads, head_dim), dev)
    scale = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    if out is None:
        out = torch.empty((rows, heads, head_dim), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((heads, rows), dtype=torch.float32, device=dev)
    _check_tensor("out", out, torch.bfloat16, (rows, heads, head_dim), dev)
    _check_tensor("lse", lse, torch.float32, (heads, rows), dev)
    need = fwd_workspace_size(batch, heads, head_dim, q_len, total_kv, broadcast_q, causal)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    _require_gpu(dev)
    with torch.cuda.device(dev):
        st = library().jfa_fwd_mxfp8(_ptr(q8), _ptr(q_scales), _ptr(k8), _ptr(k_scales), _ptr(v8),
                                     _ptr(v_scales), _ptr(offsets), int(offsets.dtype == torch.int64), batch,
                                     heads, head_dim, q_len, total_kv, int(broadcast_q), int(causal), scale,
                                     _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(dev))
    _check(st)
    return out, lse


def bwd(q, k, v, offsets, o, lse, d_o, *, broadcast_q: bool, causal: bool = False, scale=None,
        dq=None, dk=None, dv=None, workspace=None, rope=None):
    """dQ, dK, dV = jfa_bwd(...) (bf16, shapes of q, k, v).

    rope: optional (cos, sin, pos_q, pos_k) for jfa_bwd_rope: fp32 tables
    [max_pos, D/2] and int32 positions of the query rows and key rows, all on the
    GPU; q and k are then the rotated inputs and dQ, dK are returned with respect
    to the unrotated ones."""
    dev, batch, heads, head_dim, q_len, total_kv, rows = _problem(q, k, v, offsets, broadcast_q)
    _check_tensor("o", o, torch.bfloat16, (rows, heads, head_dim), dev)
    _check_tensor("d_o", d_o, torch.bfloat16, (rows, heads, head_dim), dev)
    _check_tensor("lse", lse, torch.float32, (heads, rows), dev)
    scale = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor("dq", dq, torch.bfloat16, q.shape, dev)
    _check_tensor("dk", dk, torch.bfloat16, k.shape, dev)
    _check_tensor("dv", dv, torch.bfloat16, v.shape, dev)
    need = bwd_workspace_size(batch, heads, head_dim, q_len, total_kv, broadcast_q, causal)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    if rope is not None:
        cos, sin, pos_q, pos_k = rope
        if not isinstance(cos, torch.Tensor) or cos.dim() != 2:
            raise ValueError("rope cos / sin must both be [max_pos, head_dim / 2]")
        max_pos = cos.shape[0]
        _check_tensor("rope cos", cos, torch.float32, (max_pos, head_dim // 2), dev)
        _check_tensor("rope sin", sin, torch.float32, (max_pos, head_dim // 2), dev)
        _check_tensor("rope pos_q", pos_q, torch.int32, (q.shape[0],), dev)
        _check_tensor("rope pos_k", pos_k, torch.int32, (k.shape[0],), dev)
    _require_gpu(dev)
    with torch.cuda.device(dev):
        if rope is None:
            st = library().jfa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                                   int(offsets.dtype == torch.int64), batch, heads, head_dim, q_len,
                                   total_kv, int(broadcast_q), int(causal), scale, _ptr(o), _ptr(lse),
                                   _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                   ws_bytes, _stream(dev))
        else:
            st = library().jfa_bwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                                        int(offsets.dtype == torch.int64), batch, heads, head_dim, q_len,
                                        total_kv, int(broadcast_q), int(causal), scale, _ptr(o), _ptr(lse),
                                        _ptr(d_o), _ptr(cos), _ptr(sin), _ptr(pos_q), _ptr(pos_k),
                                        max_pos, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                        ws_bytes, _stream(dev))
    _check(st)
    return dq, dk, dv
