"""Python binding of liblcsa (LCSA select + block-sparse attention on MI355X).

Argument marshalling only: every step runs in the HIP kernels of liblcsa.so.
torch supplies device memory and the current stream.  If the library is not
built the import fails; there is no other code path.

    import block_sparse_attention_lcsa_amd as lcsa
    plan = lcsa.Plan(batch=1, heads=12, head_dim=128, grid_h=48, grid_w=80,
                     q_frames=6, kv_ratio=3.0, local_range=11, topk_ratio=2.0)
    row_ptr, col_idx = lcsa.select(plan, q, k)
    o = lcsa.attend(plan, q, k, v, row_ptr, col_idx)

q, k, v are bf16 CUDA(HIP) tensors of shape [batch, tokens, heads, 128] in
raster token order; any strides with a contiguous last dimension.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["Plan", "LcsaError", "select", "select_noalloc", "attend", "select_ring", "attend_ring", "select_rope",
           "select_ring_rope", "rope", "select_steady", "select_reuse", "attend_varlen", "lib_path", "abi_version", "EXPORTS", "MAX_KV_FRAMES"]

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "liblcsa.so")


if not os.path.exists(lib_path()):
    raise ImportError(
        "liblcsa.so is not built; run `python block_sparse_attention_lcsa_amd/build_lib.py` "
        "(hipcc, gfx950). There is no fallback implementation.")

# torch first: its HIP runtime must be the one in the process before
# liblcsa.so is loaded.  liblcsa.so asks for libamdhip64.so.7, which the loader
# then resolves to torch's copy (same soname); loaded the other way round,
# torch would bring a second HIP runtime, and device pointers and streams from
# torch would not belong to the runtime liblcsa.so calls.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(lib_path())

# Every symbol include/lcsa.h declares.
EXPORTS = [
    "lcsa_plan_create", "lcsa_plan_destroy", "lcsa_plan_get_info", "lcsa_plan_row_ptr",
    "lcsa_plan_window", "lcsa_select", "lcsa_attend", "lcsa_select_rope",
    "lcsa_select_ring_rope", "lcsa_select_ring", "lcsa_attend_ring", "lcsa_select_steady",
    "lcsa_select_reuse", "lcsa_select_noalloc", "lcsa_attend_varlen",
    "lcsa_status_string", "lcsa_last_error", "lcsa_abi_version",
]
SELECT_NOALLOC_MAX_BYTES = 48 << 20
MAX_KV_FRAMES = 64

LCSA_DTYPE_BF16 = 1
STATUS = {0: "LCSA_OK", 1: "LCSA_ERR_NULL", 2: "LCSA_ERR_INVALID", 3: "LCSA_ERR_SHAPE",
          4: "LCSA_ERR_ALIGN", 5: "LCSA_ERR_WORKSPACE", 6: "LCSA_ERR_DEVICE",
          7: "LCSA_ERR_LAUNCH", 8: "LCSA_ERR_INTERNAL"}


class LcsaDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("q_frames", ctypes.c_int32),
                ("cached_frames", ctypes.c_int32), ("block_t", ctypes.c_int32),
                ("block_h", ctypes.c_int32), ("block_w", ctypes.c_int32),
                ("local_range", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("topk_ratio", ctypes.c_double), ("kv_ratio", ctypes.c_float),
                ("scale", ctypes.c_float)]


class LcsaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("batch", ctypes.c_int64), ("tokens", ctypes.c_int64),
                ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64)]


class LcsaKvRing(ctypes.Structure):
    _fields_ = [("slots", ctypes.c_int32), ("frame_slot", ctypes.c_int32 * 64)]


class LcsaRope(ctypes.Structure):
    _fields_ = [("pairs_t", ctypes.c_int32), ("pairs_h", ctypes.c_int32),
                ("pairs_w", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("table_t", ctypes.c_void_p), ("table_h", ctypes.c_void_p),
                ("table_w", ctypes.c_void_p)]


class LcsaPlanInfo(ctypes.Structure):
    _fields_ = [("kv_frames", ctypes.c_int32), ("blocks_per_frame", ctypes.c_int32),
                ("nbh", ctypes.c_int32), ("nbw", ctypes.c_int32), ("nqb", ctypes.c_int32),
                ("nkb", ctypes.c_int32), ("k", ctypes.c_int32), ("block_h", ctypes.c_int32),
                ("block_w", ctypes.c_int32), ("block_tokens", ctypes.c_int32),
                ("half_window", ctypes.c_int32), ("max_row_nnz", ctypes.c_int32),
                ("min_window", ctypes.c_int32), ("max_window", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("q_tokens", ctypes.c_int64), ("kv_tokens", ctypes.c_int64),
                ("select_workspace_bytes", ctypes.c_uint64),
                ("attend_workspace_bytes", ctypes.c_uint64),
                ("kcache_slot_bytes", ctypes.c_uint64), ("scale", ctypes.c_double),
                ("useful_flops", ctypes.c_double)]


_P = ctypes.c_void_p
_lib.lcsa_plan_create.argtypes = [ctypes.POINTER(LcsaDesc), ctypes.POINTER(_P)]
_lib.lcsa_plan_create.restype = ctypes.c_int32
_lib.lcsa_plan_destroy.argtypes = [_P]
_lib.lcsa_plan_destroy.restype = None
_lib.lcsa_plan_get_info.argtypes = [_P, ctypes.POINTER(LcsaPlanInfo)]
_lib.lcsa_plan_get_info.restype = ctypes.c_int32
_lib.lcsa_plan_row_ptr.argtypes = [_P, ctypes.POINTER(ctypes.c_int32), ctypes.c_int64]
_lib.lcsa_plan_row_ptr.restype = ctypes.c_int32
_lib.lcsa_plan_window.argtypes = [_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                  ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
_lib.lcsa_plan_window.restype = ctypes.c_int32
_lib.lcsa_select.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                             _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.lcsa_select.restype = ctypes.c_int32
_lib.lcsa_select_noalloc.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                                     _P, _P, _P, _P]
_lib.lcsa_select_noalloc.restype = ctypes.c_int32
_lib.lcsa_attend.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                             ctypes.POINTER(LcsaTensor), _P, _P, ctypes.c_int64,
                             ctypes.POINTER(LcsaTensor), _P, _P, ctypes.c_size_t, _P]
_lib.lcsa_attend.restype = ctypes.c_int32
_lib.lcsa_select_ring.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                                  ctypes.POINTER(LcsaKvRing), ctypes.c_int32, _P,
                                  _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.lcsa_select_ring.restype = ctypes.c_int32
_lib.lcsa_select_rope.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                                  ctypes.POINTER(LcsaRope), ctypes.POINTER(LcsaTensor),
                                  ctypes.POINTER(LcsaTensor), _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.lcsa_select_rope.restype = ctypes.c_int32
_lib.lcsa_select_ring_rope.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                                       ctypes.POINTER(LcsaKvRing), ctypes.c_int32, _P,
                                       ctypes.POINTER(LcsaRope), ctypes.POINTER(LcsaTensor),
                                       ctypes.POINTER(LcsaTensor), _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]
_lib.lcsa_select_ring_rope.restype = ctypes.c_int32
_lib.lcsa_attend_ring.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                                  ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaKvRing), _P, _P,
                                  ctypes.c_int64, ctypes.POINTER(LcsaTensor), _P, _P,
                                  ctypes.c_size_t, _P]
_lib.lcsa_attend_ring.restype = ctypes.c_int32
_lib.lcsa_attend_varlen.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                                    ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaKvRing), _P, _P,
                                    ctypes.c_int64, ctypes.POINTER(LcsaTensor), _P, _P,
                                    ctypes.c_size_t, _P]
_lib.lcsa_attend_varlen.restype = ctypes.c_int32
_lib.lcsa_select_steady.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                                    ctypes.POINTER(LcsaKvRing), ctypes.c_int32, _P,
                                    ctypes.POINTER(LcsaRope), ctypes.POINTER(LcsaTensor),
                                    ctypes.POINTER(LcsaTensor), _P, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]
_lib.lcsa_select_steady.restype = ctypes.c_int32
_lib.lcsa_select_reuse.argtypes = [_P, ctypes.POINTER(LcsaTensor), ctypes.POINTER(LcsaTensor),
                                   ctypes.POINTER(LcsaKvRing), ctypes.c_int32, _P,
                                   ctypes.POINTER(LcsaRope), ctypes.POINTER(LcsaTensor),
                                   ctypes.POINTER(LcsaTensor), _P, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]
_lib.lcsa_select_reuse.restype = ctypes.c_int32
_lib.lcsa_status_string.argtypes = [ctypes.c_int32]
_lib.lcsa_status_string.restype = ctypes.c_char_p
_lib.lcsa_last_error.argtypes = []
_lib.lcsa_last_error.restype = ctypes.c_char_p
_lib.lcsa_abi_version.argtypes = []
_lib.lcsa_abi_version.restype = ctypes.c_int32


class LcsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        detail = _lib.lcsa_last_error().decode()
        super().__init__(f"{where}: {self.name}: {detail}")


def _check(st: int, where: str):
    if st != 0:
        raise LcsaError(st, where)


def abi_version() -> int:
    return _lib.lcsa_abi_version()


class Plan:
    """Host-side plan of one LCSA layer shape (no GPU needed)."""

    def __init__(self, batch, heads, grid_h, grid_w, q_frames, head_dim=128, cached_frames=0,
                 kv_ratio=3.0, block_t=0, block_h=0, block_w=0, local_range=11,
                 topk_ratio=0.0, topk=0, scale=0.0):
        d = LcsaDesc(batch=batch, heads=heads, head_dim=head_dim, grid_h=grid_h, grid_w=grid_w,
                     q_frames=q_frames, cached_frames=cached_frames, block_t=block_t,
                     block_h=block_h, block_w=block_w, local_range=local_range, topk=topk,
                     topk_ratio=topk_ratio, kv_ratio=kv_ratio, scale=scale)
        h = _P()
        _check(_lib.lcsa_plan_create(ctypes.byref(d), ctypes.byref(h)), "lcsa_plan_create")
        self._h = h
        # held on the instance: module globals may already be gone when a plan
        # is collected at interpreter exit
        self._destroy = _lib.lcsa_plan_destroy
        self.desc = {f: getattr(d, f) for f, _ in LcsaDesc._fields_}
        inf = LcsaPlanInfo()
        _check(_lib.lcsa_plan_get_info(h, ctypes.byref(inf)), "lcsa_plan_get_info")
        self.info = {f: getattr(inf, f) for f, _ in LcsaPlanInfo._fields_}

    @classmethod
    def from_desc(cls, desc: dict) -> "Plan":
        return cls(**{k: v for k, v in desc.items()})

    def __del__(self):
        h = getattr(self, "_h", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def row_ptr(self):
        import numpy as np
        n = self.info["rows"] + 1
        out = np.zeros(n, dtype=np.int32)
        _check(_lib.lcsa_plan_row_ptr(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n),
               "lcsa_plan_row_ptr")
        return out

    def window(self, qb: int):
        import numpy as np
        cap = self.info["max_window"]
        out = np.zeros(max(cap, 1), dtype=np.int32)
        cnt = ctypes.c_int32()
        _check(_lib.lcsa_plan_window(self._h, qb, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     len(out), ctypes.byref(cnt)), "lcsa_plan_window")
        return out[:cnt.value]


def tensor_view(t) -> LcsaTensor:
    """lcsa_tensor of a [B, S, H, D] bf16 torch tensor (contiguous last dim)."""
    import torch
    if t.dtype != torch.bfloat16:
        raise TypeError(f"expected bfloat16, got {t.dtype}")
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [batch, tokens, heads, head_dim] view with contiguous last dim")
    sb, ss, sh, _ = t.stride()
    nb, ns, nh, nd = t.shape
    return LcsaTensor(data=t.data_ptr(), dtype=LCSA_DTYPE_BF16, reserved=0,
                      stride_b=sb, stride_s=ss, stride_h=sh, batch=nb, tokens=ns, heads=nh,
                      head_dim=nd)


def _check_shape(t, plan: Plan, tokens_key: str, name: str):
    inf, d = plan.info, plan.desc
    want = (d["batch"], inf[tokens_key], d["heads"], d["head_dim"])
    if tuple(t.shape) != want:
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {want}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")


def _stream_ptr(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream


def select(plan: Plan, q, k, return_scores: bool = False, workspace=None, stream=None):
    """Top-k block selection.  Returns (row_ptr int32 [rows+1], col_idx int32
    [nnz]) and, with return_scores, the float64 pooled scores
    [B, H, NQB, NKB] (-inf outside the window)."""
    import torch
    _check_shape(q, plan, "q_tokens", "q")
    _check_shape(k, plan, "kv_tokens", "k")
    inf = plan.info
    dev = q.device
    row_ptr = torch.empty(inf["rows"] + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(inf["nnz"], 1), dtype=torch.int32, device=dev)[: inf["nnz"]]
    ws_bytes = int(inf["select_workspace_bytes"])
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    scores = None
    if return_scores:
        d = plan.desc
        scores = torch.empty((d["batch"], d["heads"], inf["nqb"], inf["nkb"]),
                             dtype=torch.float64, device=dev)
    qv, kv = tensor_view(q), tensor_view(k)
    st = _lib.lcsa_select(plan.handle, ctypes.byref(qv), ctypes.byref(kv),
                          row_ptr.data_ptr(), col_idx.data_ptr() if inf["nnz"] else None,
                          scores.data_ptr() if scores is not None else None,
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream_ptr(q, stream))
    _check(st, "lcsa_select")
    if return_scores:
        return row_ptr, col_idx, scores
    return row_ptr, col_idx


def select_noalloc(plan: Plan, q, k, row_ptr=None, col_idx=None, return_scores: bool = False,
                   stream=None):
    """select without a workspace (lcsa_select_noalloc): the library's own
    per-device scratch array holds the pooled vectors, so the C call
    allocates nothing.  row_ptr / col_idx may be passed in (int32, rows + 1
    and nnz entries) so that nothing is allocated here either.  Calls that
    overlap on one device race on the scratch array."""
    import torch
    _check_shape(q, plan, "q_tokens", "q")
    _check_shape(k, plan, "kv_tokens", "k")
    inf = plan.info
    dev = q.device
    if row_ptr is None:
        row_ptr = torch.empty(inf["rows"] + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(inf["nnz"], 1), dtype=torch.int32, device=dev)[: inf["nnz"]]
    if row_ptr.dtype != torch.int32 or row_ptr.numel() != inf["rows"] + 1:
        raise ValueError("row_ptr must be int32 [rows + 1]")
    if col_idx.dtype != torch.int32 or col_idx.numel() != inf["nnz"]:
        raise ValueError("col_idx must be int32 [nnz]")
    scores = None
    if return_scores:
        d = plan.desc
        scores = torch.empty((d["batch"], d["heads"], inf["nqb"], inf["nkb"]),
                             dtype=torch.float64, device=dev)
    qv, kv = tensor_view(q), tensor_view(k)
    st = _lib.lcsa_select_noalloc(plan.handle, ctypes.byref(qv), ctypes.byref(kv),
                                  row_ptr.data_ptr(), col_idx.data_ptr() if inf["nnz"] else None,
                                  scores.data_ptr() if scores is not None else None,
                                  _stream_ptr(q, stream))
    _check(st, "lcsa_select_noalloc")
    if return_scores:
        return row_ptr, col_idx, scores
    return row_ptr, col_idx


def attend(plan: Plan, q, k, v, row_ptr, col_idx, out=None, return_lse: bool = False,
           workspace=None, split_tail: bool = True, stream=None):
    """Block-sparse attention forward over the CSR (row_ptr, col_idx).

    With split_tail (default) a workspace of attend_workspace_bytes is used
    (allocated here if not given) so that rows of a last, partly filled round
    of workgroups are split and merged; split_tail=False runs every row as
    one workgroup."""
    import torch
    _check_shape(q, plan, "q_tokens", "q")
    _check_shape(k, plan, "kv_tokens", "k")
    _check_shape(v, plan, "kv_tokens", "v")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise TypeError("row_ptr and col_idx must be int32")
    if row_ptr.numel() != plan.info["rows"] + 1 or not row_ptr.is_contiguous():
        raise ValueError("row_ptr must hold rows + 1 contiguous int32")
    if not col_idx.is_contiguous():
        raise ValueError("col_idx must be contiguous")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    else:
        _check_shape(out, plan, "q_tokens", "out")
    lse = None
    if return_lse:
        d = plan.desc
        lse = torch.empty((d["batch"], d["heads"], plan.info["q_tokens"]), dtype=torch.float32,
                          device=q.device)
    ws_ptr, ws_bytes = None, 0
    if split_tail:
        if workspace is None:
            workspace = torch.empty(int(plan.info["attend_workspace_bytes"]), dtype=torch.uint8,
                                    device=q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    qv, kv, vv, ov = tensor_view(q), tensor_view(k), tensor_view(v), tensor_view(out)
    st = _lib.lcsa_attend(plan.handle, ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv),
                          row_ptr.data_ptr(), col_idx.data_ptr() if col_idx.numel() else None,
                          col_idx.numel(), ctypes.byref(ov),
                          lse.data_ptr() if lse is not None else None, ws_ptr, ws_bytes,
                          _stream_ptr(q, stream))
    _check(st, "lcsa_attend")
    if return_lse:
        return out, lse
    return out


def kv_ring(slots: int, frame_slot) -> LcsaKvRing:
    """Frame-ring descriptor: window frame t (oldest first) lives in ring slot
    frame_slot[t] of K/V ring buffers that hold `slots` frames."""
    r = LcsaKvRing()
    r.slots = int(slots)
    fs = [int(x) for x in frame_slot]
    if len(fs) > MAX_KV_FRAMES:
        raise ValueError(f"at most {MAX_KV_FRAMES} window frames")
    for i, x in enumerate(fs):
        r.frame_slot[i] = x
    return r


def _check_ring_tensor(t, plan: Plan, slots: int, name: str):
    d = plan.desc
    want = (d["batch"], slots * d["grid_h"] * d["grid_w"], d["heads"], d["head_dim"])
    if tuple(t.shape) != want:
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {want}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")


def kcache_bytes(plan: Plan, slots: int) -> int:
    """Bytes of the pooled-K cache of a ring with `slots` frames."""
    return int(plan.info["kcache_slot_bytes"]) * int(slots)


def select_ring(plan: Plan, q, k_ring, ring: LcsaKvRing, new_frames: int, kcache,
                return_scores: bool = False, workspace=None, stream=None):
    """Top-k block selection with K read from a frame ring and the pooled K of
    older frames taken from `kcache` (float64 device tensor of
    kcache_bytes(plan, ring.slots) bytes); the newest `new_frames` window
    frames are pooled and stored there."""
    import torch
    _check_shape(q, plan, "q_tokens", "q")
    _check_ring_tensor(k_ring, plan, ring.slots, "k_ring")
    if kcache.dtype != torch.float64 or kcache.numel() * 8 < kcache_bytes(plan, ring.slots):
        raise ValueError("kcache must be float64 with kcache_bytes(plan, slots) bytes")
    inf = plan.info
    dev = q.device
    row_ptr = torch.empty(inf["rows"] + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(inf["nnz"], 1), dtype=torch.int32, device=dev)[: inf["nnz"]]
    if workspace is None:
        workspace = torch.empty(max(int(inf["select_workspace_bytes"]), 256), dtype=torch.uint8,
                                device=dev)
    scores = None
    if return_scores:
        d = plan.desc
        scores = torch.empty((d["batch"], d["heads"], inf["nqb"], inf["nkb"]),
                             dtype=torch.float64, device=dev)
    qv, kv = tensor_view(q), tensor_view(k_ring)
    st = _lib.lcsa_select_ring(plan.handle, ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(ring),
                               int(new_frames), kcache.data_ptr(), row_ptr.data_ptr(),
                               col_idx.data_ptr() if inf["nnz"] else None,
                               scores.data_ptr() if scores is not None else None,
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream_ptr(q, stream))
    _check(st, "lcsa_select_ring")
    if return_scores:
        return row_ptr, col_idx, scores
    return row_ptr, col_idx


def attend_ring(plan: Plan, q, k_ring, v_ring, ring: LcsaKvRing, row_ptr, col_idx, out=None,
                return_lse: bool = False, workspace=None, split_tail: bool = True, stream=None):
    """Block-sparse attention with K and V read from a frame ring."""
    import torch
    _check_shape(q, plan, "q_tokens", "q")
    _check_ring_tensor(k_ring, plan, ring.slots, "k_ring")
    _check_ring_tensor(v_ring, plan, ring.slots, "v_ring")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise TypeError("row_ptr and col_idx must be int32")
    if row_ptr.numel() != plan.info["rows"] + 1 or not row_ptr.is_contiguous():
        raise ValueError("row_ptr must hold rows + 1 contiguous int32")
    if not col_idx.is_contiguous():
        raise ValueError("col_idx must be contiguous")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    else:
        _check_shape(out, plan, "q_tokens", "out")
    lse = None
    if return_lse:
        d = plan.desc
        lse = torch.empty((d["batch"], d["heads"], plan.info["q_tokens"]), dtype=torch.float32,
                          device=q.device)
    ws_ptr, ws_bytes = None, 0
    if split_tail:
        if workspace is None:
            workspace = torch.empty(int(plan.info["attend_workspace_bytes"]), dtype=torch.uint8,
                                    device=q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    qv, kv, vv, ov = tensor_view(q), tensor_view(k_ring), tensor_view(v_ring), tensor_view(out)
    st = _lib.lcsa_attend_ring(plan.handle, ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv),
                               ctypes.byref(ring), row_ptr.data_ptr(),
                               col_idx.data_ptr() if col_idx.numel() else None, col_idx.numel(),
                               ctypes.byref(ov), lse.data_ptr() if lse is not None else None,
                               ws_ptr, ws_bytes, _stream_ptr(q, stream))
    _check(st, "lcsa_attend_ring")
    if return_lse:
        return out, lse
    return out


def attend_varlen(plan: Plan, q, k, v, row_ptr, col_idx, out=None, return_lse: bool = False,
                  workspace=None, ring: LcsaKvRing = None, stream=None):
    """lcsa_attend_varlen: attention over a CSR whose rows differ in length
    (a threshold selection), rows taken longest first.  k, v are the
    contiguous KV window, or the rings when `ring` is given.  Same result as
    attend / attend_ring to rounding."""
    import torch
    _check_shape(q, plan, "q_tokens", "q")
    if ring is None:
        _check_shape(k, plan, "kv_tokens", "k")
        _check_shape(v, plan, "kv_tokens", "v")
    else:
        _check_ring_tensor(k, plan, ring.slots, "k_ring")
        _check_ring_tensor(v, plan, ring.slots, "v_ring")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise TypeError("row_ptr and col_idx must be int32")
    if row_ptr.numel() != plan.info["rows"] + 1 or not row_ptr.is_contiguous():
        raise ValueError("row_ptr must hold rows + 1 contiguous int32")
    if not col_idx.is_contiguous():
        raise ValueError("col_idx must be contiguous")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    else:
        _check_shape(out, plan, "q_tokens", "out")
    lse = None
    if return_lse:
        d = plan.desc
        lse = torch.empty((d["batch"], d["heads"], plan.info["q_tokens"]), dtype=torch.float32,
                          device=q.device)
    if workspace is None:
        workspace = torch.empty(int(plan.info["attend_workspace_bytes"]), dtype=torch.uint8,
                                device=q.device)
    qv, kv, vv, ov = tensor_view(q), tensor_view(k), tensor_view(v), tensor_view(out)
    st = _lib.lcsa_attend_varlen(plan.handle, ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv),
                                 ctypes.byref(ring) if ring is not None else None,
                                 row_ptr.data_ptr(),
                                 col_idx.data_ptr() if col_idx.numel() else None, col_idx.numel(),
                                 ctypes.byref(ov), lse.data_ptr() if lse is not None else None,
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _stream_ptr(q, stream))
    _check(st, "lcsa_attend_varlen")
    if return_lse:
        return out, lse
    return out


def rope(table_t, table_h, table_w) -> "RopeTables":
    """Rotary tables for select_rope / select_ring_rope: float32 device
    tensors [kv_frames, pairs_t, 2], [grid_h, pairs_h, 2], [grid_w, pairs_w, 2]
    of (cos, sin); pairs_t + pairs_h + pairs_w = 64."""
    return RopeTables(table_t, table_h, table_w)


class RopeTables:
    def __init__(self, table_t, table_h, table_w):
        import torch
        tabs = (table_t, table_h, table_w)
        for t in tabs:
            if t.dtype != torch.float32 or t.dim() != 3 or t.shape[2] != 2 or not t.is_contiguous():
                raise ValueError("rotary tables must be contiguous float32 [positions, pairs, 2]")
            if not t.is_cuda:
                raise ValueError("rotary tables must be device tensors")
        self.tables = tabs
        self.desc = LcsaRope(pairs_t=table_t.shape[1], pairs_h=table_h.shape[1],
                             pairs_w=table_w.shape[1], reserved=0,
                             table_t=table_t.data_ptr() if table_t.numel() else None,
                             table_h=table_h.data_ptr() if table_h.numel() else None,
                             table_w=table_w.data_ptr() if table_w.numel() else None)

    def check(self, plan: Plan):
        d, inf = plan.desc, plan.info
        want = ((inf["kv_frames"],), (d["grid_h"],), (d["grid_w"],))
        for t, w in zip(self.tables, want):
            if t.numel() and t.shape[0] != w[0]:
                raise ValueError(f"rotary table of {t.shape[0]} positions, plan needs {w[0]}")


def select_rope(plan: Plan, q, k, tables: "RopeTables", q_rot=None, k_rot=None,
                return_scores: bool = False, workspace=None, stream=None):
    """Rotary embedding fused into selection: returns (q_rot, k_rot, row_ptr,
    col_idx[, scores]) where q_rot / k_rot are the turned bf16 Q and K
    (written into the given tensors if passed, which may be q and k) and the
    CSR is selected on them.  Pass q_rot, k_rot to attend."""
    import torch
    _check_shape(q, plan, "q_tokens", "q")
    _check_shape(k, plan, "kv_tokens", "k")
    tables.check(plan)
    q_rot = torch.empty_like(q, memory_format=torch.contiguous_format) if q_rot is None else q_rot
    k_rot = torch.empty_like(k, memory_format=torch.contiguous_format) if k_rot is None else k_rot
    _check_shape(q_rot, plan, "q_tokens", "q_rot")
    _check_shape(k_rot, plan, "kv_tokens", "k_rot")
    inf = plan.info
    dev = q.device
    row_ptr = torch.empty(inf["rows"] + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(inf["nnz"], 1), dtype=torch.int32, device=dev)[: inf["nnz"]]
    if workspace is None:
        workspace = torch.empty(max(int(inf["select_workspace_bytes"]), 256), dtype=torch.uint8,
                                device=dev)
    scores = None
    if return_scores:
        d = plan.desc
        scores = torch.empty((d["batch"], d["heads"], inf["nqb"], inf["nkb"]),
                             dtype=torch.float64, device=dev)
    qv, kv, qr, kr = tensor_view(q), tensor_view(k), tensor_view(q_rot), tensor_view(k_rot)
    st = _lib.lcsa_select_rope(plan.handle, ctypes.byref(qv), ctypes.byref(kv),
                               ctypes.byref(tables.desc), ctypes.byref(qr), ctypes.byref(kr),
                               row_ptr.data_ptr(), col_idx.data_ptr() if inf["nnz"] else None,
                               scores.data_ptr() if scores is not None else None,
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream_ptr(q, stream))
    _check(st, "lcsa_select_rope")
    out = (q_rot, k_rot, row_ptr, col_idx)
    return out + (scores,) if return_scores else out


def select_ring_rope(plan: Plan, q, k_ring, ring: LcsaKvRing, new_frames: int, kcache,
                     tables: "RopeTables", k_rot_ring, q_rot=None, workspace=None, stream=None):
    """select_ring with the rotary embedding: the newest new_frames window
    frames of k_ring are turned into the same slots of k_rot_ring and pooled
    into kcache; Q is turned into q_rot.  Returns (q_rot, row_ptr, col_idx)."""
    import torch
    _check_shape(q, plan, "q_tokens", "q")
    _check_ring_tensor(k_ring, plan, ring.slots, "k_ring")
    _check_ring_tensor(k_rot_ring, plan, ring.slots, "k_rot_ring")
    tables.check(plan)
    if kcache.dtype != torch.float64 or kcache.numel() * 8 < kcache_bytes(plan, ring.slots):
        raise ValueError("kcache must be float64 with kcache_bytes(plan, slots) bytes")
    q_rot = torch.empty_like(q, memory_format=torch.contiguous_format) if q_rot is None else q_rot
    _check_shape(q_rot, plan, "q_tokens", "q_rot")
    inf = plan.info
    dev = q.device
    row_ptr = torch.empty(inf["rows"] + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(inf["nnz"], 1), dtype=torch.int32, device=dev)[: inf["nnz"]]
    if workspace is None:
        workspace = torch.empty(max(int(inf["select_workspace_bytes"]), 256), dtype=torch.uint8,
                                device=dev)
    qv, kv, qr, kr = tensor_view(q), tensor_view(k_ring), tensor_view(q_rot), tensor_view(k_rot_ring)
    st = _lib.lcsa_select_ring_rope(plan.handle, ctypes.byref(qv), ctypes.byref(kv),
                                    ctypes.byref(ring), int(new_frames), kcache.data_ptr(),
                                    ctypes.byref(tables.desc), ctypes.byref(qr), ctypes.byref(kr),
                                    row_ptr.data_ptr(), col_idx.data_ptr() if inf["nnz"] else None,
                                    None, workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(),
                                    _stream_ptr(q, stream))
    _check(st, "lcsa_select_ring_rope")
    return q_rot, row_ptr, col_idx


def _threshold_select(fn, plan: Plan, q, k, tau, ring, new_frames, kcache, tables, q_rot, k_rot,
                      return_scores, workspace, stream):
    import torch
    _check_shape(q, plan, "q_tokens", "q")
    if ring is not None:
        _check_ring_tensor(k, plan, ring.slots, "k")
        if kcache is None or kcache.dtype != torch.float64 or \
                kcache.numel() * 8 < kcache_bytes(plan, ring.slots):
            raise ValueError("kcache must be float64 with kcache_bytes(plan, slots) bytes")
    else:
        _check_shape(k, plan, "kv_tokens", "k")
    if tables is not None:
        tables.check(plan)
        if q_rot is None or k_rot is None:
            raise ValueError("with rotary tables pass q_rot and k_rot (they may be q and k)")
        _check_shape(q_rot, plan, "q_tokens", "q_rot")
        if ring is not None:
            _check_ring_tensor(k_rot, plan, ring.slots, "k_rot")
        else:
            _check_shape(k_rot, plan, "kv_tokens", "k_rot")
    inf = plan.info
    dev = q.device
    rows = int(inf["rows"])
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if tau is None:
        n_idx = int(inf["nnz"])
        kth = torch.empty(rows, dtype=torch.float64, device=dev)
    else:
        if tau.dtype != torch.float64 or tau.numel() != rows or not tau.is_contiguous():
            raise ValueError(f"tau must be contiguous float64 [{rows}]")
        n_idx = rows * int(inf["max_window"])
        kth = None
    col_idx = torch.empty(max(n_idx, 1), dtype=torch.int32, device=dev)[:n_idx]
    if workspace is None:
        workspace = torch.empty(max(int(inf["select_workspace_bytes"]), 256), dtype=torch.uint8,
                                device=dev)
    scores = None
    if return_scores:
        d = plan.desc
        scores = torch.empty((d["batch"], d["heads"], inf["nqb"], inf["nkb"]),
                             dtype=torch.float64, device=dev)
    qv, kv = tensor_view(q), tensor_view(k)
    rope_p = ctypes.byref(tables.desc) if tables is not None else None
    qr = ctypes.byref(tensor_view(q_rot)) if tables is not None else None
    kr = ctypes.byref(tensor_view(k_rot)) if tables is not None else None
    ring_p = ctypes.byref(ring) if ring is not None else None
    kc = kcache.data_ptr() if ring is not None else None
    common = (plan.handle, ctypes.byref(qv), ctypes.byref(kv), ring_p,
              int(new_frames) if ring is not None else 0, kc, rope_p, qr, kr)
    tail = (scores.data_ptr() if scores is not None else None, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_ptr(q, stream))
    ci = col_idx.data_ptr() if n_idx else None
    if tau is None:
        st = _lib.lcsa_select_steady(*common, row_ptr.data_ptr(), ci, kth.data_ptr(), *tail)
    else:
        st = _lib.lcsa_select_reuse(*common, tau.data_ptr(), row_ptr.data_ptr(), ci, *tail)
    _check(st, fn)
    out = (row_ptr, col_idx) if tau is not None else (row_ptr, col_idx, kth)
    return out + (scores,) if return_scores else out


def select_steady(plan: Plan, q, k, ring: LcsaKvRing = None, new_frames: int = 0, kcache=None,
                  tables: "RopeTables" = None, q_rot=None, k_rot=None,
                  return_scores: bool = False, workspace=None, stream=None):
    """Top-k selection that also returns each CSR row's threshold (its
    keep-th largest window score, float64 [rows]) for select_reuse.  With
    ring, k is the K ring and kcache the pooled-K cache as in select_ring;
    with tables, q and k are turned into q_rot and k_rot (which may be q and
    k) as in select_rope.  Returns (row_ptr, col_idx, kth[, scores])."""
    return _threshold_select("lcsa_select_steady", plan, q, k, None, ring, new_frames, kcache,
                             tables, q_rot, k_rot, return_scores, workspace, stream)


def select_reuse(plan: Plan, q, k, tau, ring: LcsaKvRing = None, new_frames: int = 0,
                 kcache=None, tables: "RopeTables" = None, q_rot=None, k_rot=None,
                 return_scores: bool = False, workspace=None, stream=None):
    """Selection by per-row thresholds tau (float64 [rows], e.g. the kth of
    an earlier select_steady): row r keeps its window blocks scored >= tau[r].
    Returns the padded CSR (row_ptr = r * max_window, col_idx int32
    [rows * max_window] with -1 after each row's blocks[, scores]); attend
    accepts it as it is."""
    return _threshold_select("lcsa_select_reuse", plan, q, k, tau, ring, new_frames, kcache,
                             tables, q_rot, k_rot, return_scores, workspace, stream)
