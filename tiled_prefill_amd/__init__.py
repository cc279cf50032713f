"""Python binding of libattn.so, the MI355X tiled flash-attention library
(forward pass, split-KV combine, and backward pass).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C-ABI declared in include/attn.h. PyTorch provides
device memory and the current stream. There is no fallback path: if the
library is not built, or a tensor is not on a GPU, the call raises.

Layouts: q, o [B, Sq, Hq, d]; k, v [B, Sk, Hkv, d]; lse [B, Hq, Sq] fp32.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIB may name another build of the same library (same ABI), e.g. one
# compiled with different flags, to compare two builds in one process tree.
LIB_PATH = os.environ.get("ATTN_LIB") or os.path.join(_PKG, "libattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "attn.h")

FP32, BF16 = 0, 1
MAX_SPLITS = 256
ERRORS = {-1: "EINVAL", -2: "EUNSUPPORTED", -3: "EHIP", -4: "ENOMEM"}


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"attn error {code} ({ERRORS.get(code, '?')}): {msg}")
        self.code = code


class Plan(ctypes.Structure):
    _fields_ = [
        ("pack_gqa", ctypes.c_int), ("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
        ("waves_m", ctypes.c_int), ("waves_n", ctypes.c_int), ("num_m_blocks", ctypes.c_int),
        ("grid_heads", ctypes.c_int), ("num_splits", ctypes.c_int), ("chunk_blocks", ctypes.c_int),
        ("grid_x", ctypes.c_int), ("grid_y", ctypes.c_int), ("grid_z", ctypes.c_int),
        ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int), ("num_cus", ctypes.c_int),
        ("lpt", ctypes.c_int), ("work_units", ctypes.c_int), ("visited_blocks", ctypes.c_longlong),
        ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class BwdPlan(ctypes.Structure):
    _fields_ = [
        ("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("num_n_blocks", ctypes.c_int),
        ("grid_x", ctypes.c_int), ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int),
        ("dq_block_m", ctypes.c_int), ("visited_blocks", ctypes.c_longlong),
        ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def load():
    """Load libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run tiled_prefill_amd/_build.py "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    ll = ctypes.c_longlong
    ip = ctypes.POINTER(ctypes.c_int)
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd_noalloc.restype = i
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, i, vp, ll, vp]
    lib.attn_fwd_varlen.restype = i
    lib.attn_plan_fwd.argtypes = [i, i, i, i, i, i, i, i, i, i, i, ll, i, ctypes.POINTER(Plan)]
    lib.attn_plan_fwd.restype = i
    lib.attn_plan.argtypes = lib.attn_plan_fwd.argtypes
    lib.attn_plan.restype = i
    lib.attn_fwd_dv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd_dv.restype = i
    lib.attn_plan_fwd_dv.argtypes = [i, i, i, i, i, i, i, i, i, i, i, i, ctypes.POINTER(Plan)]
    lib.attn_plan_fwd_dv.restype = i
    lib.attn_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_lse_combine.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.attn_lse_combine.restype = i
    lib.attn_n_block_range.argtypes = [i, i, i, i, i, i, i, i, i, i, i, ip, ip]
    lib.attn_n_block_range.restype = i
    lib.attn_should_pack_gqa.argtypes = [i, i, i, i]
    lib.attn_should_pack_gqa.restype = i
    lib.attn_num_splits_fa3.argtypes = [i, i, i, i, ll, i, i]
    lib.attn_num_splits_fa3.restype = i
    lib.attn_num_splits_occupancy.argtypes = [i, i, i, i, i, i]
    lib.attn_num_splits_occupancy.restype = i
    lib.attn_profile_begin.argtypes = [i]
    lib.attn_profile_begin.restype = i
    dp = ctypes.POINTER(ctypes.c_double)
    lib.attn_profile_end.argtypes = [dp, ip, dp, ip, dp, ip]
    lib.attn_profile_end.restype = i
    lib.attn_profile_end_kinds.argtypes = [dp, ip, i]
    lib.attn_profile_end_kinds.restype = i
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp]
    lib.attn_bwd.restype = i
    lib.attn_plan_bwd.argtypes = [i, i, i, i, i, i, i, i, i, ctypes.POINTER(BwdPlan)]
    lib.attn_plan_bwd.restype = i
    lib.attn_m_block_range.argtypes = [i, i, i, i, i, i, i, ip, ip]
    lib.attn_m_block_range.restype = i
    lib.attn_stream_read.argtypes = [vp, ctypes.c_size_t, i, vp, vp]
    lib.attn_stream_read.restype = i
    lib.attn_set_workspace.argtypes = [vp, ctypes.c_size_t]
    lib.attn_set_workspace.restype = i
    lib.attn_set_option.argtypes = [ctypes.c_char_p, i]
    lib.attn_set_option.restype = i
    lib.attn_get_option.argtypes = [ctypes.c_char_p, ip]
    lib.attn_get_option.restype = i
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise AttnError(rc, load().attn_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (fp32 or bf16)")


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _check_tensors(q, k, v, same_width=True):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if (k.shape != v.shape) if same_width else (k.shape[:3] != v.shape[:3]):
        raise ValueError("k and v must have the same shape" if same_width else
                         "k and v must agree in batch, keys and heads")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError("batch and head dim of q and k must match")


def fwd(q, k, v, causal: bool = False, window_left: int = -1, scale: Optional[float] = None,
        num_splits: int = 0, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, return_lse: bool = True, stream=None):
    """Attention forward on the GPU. Returns (o, lse) (lse None if not requested)."""
    _check_tensors(q, k, v)
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    rc = load().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr() if lse is not None else None,
                           B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), int(window_left),
                           float(scale), int(num_splits), _dtype_code(q), _stream_ptr(stream))
    _check(rc)
    return out, lse


def fwd_noalloc(q, k, v, out: torch.Tensor, lse: Optional[torch.Tensor], causal: bool = False,
                window_left: int = -1, scale: Optional[float] = None, num_splits: int = 0,
                stream=None):
    """attn_fwd_noalloc: attn_fwd with its scratch in the library's static device array
    (nothing allocated; the caller passes the outputs)."""
    _check_tensors(q, k, v)
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rc = load().attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None,
                                 B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), int(window_left),
                                 float(scale), int(num_splits), _dtype_code(q), _stream_ptr(stream))
    _check(rc)
    return out, lse


def fwd_dv(q, k, v, causal: bool = False, window_left: int = -1, scale: Optional[float] = None,
           num_splits: int = 0, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, return_lse: bool = True, stream=None):
    """Forward with values of their own width (attn_fwd_dv): q, k [.., d], v [.., d_v].
    Returns (o [B, Sq, Hq, d_v], lse)."""
    _check_tensors(q, k, v, same_width=False)
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, dv = v.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Sq, Hq, dv), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    rc = load().attn_fwd_dv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr() if lse is not None else None,
                              B, Hq, Hkv, Sq, Sk, d, dv, int(bool(causal)), int(window_left),
                              float(scale), int(num_splits), _dtype_code(q), _stream_ptr(stream))
    _check(rc)
    return out, lse


def fwd_varlen(q, k, v, seqlens_k: torch.Tensor, causal: bool = False, window_left: int = -1,
               scale: Optional[float] = None, num_splits: int = 0, sum_seqlens_k: int = -1,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               return_lse: bool = True, stream=None):
    """Attention forward with per-sequence key lengths (device int32 seqlens_k [B])."""
    _check_tensors(q, k, v)
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    if not (seqlens_k.is_cuda and seqlens_k.dtype == torch.int32 and seqlens_k.shape == (B,)
            and seqlens_k.is_contiguous()):
        raise ValueError("seqlens_k must be a contiguous int32 GPU tensor of shape [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    rc = load().attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr() if lse is not None else None,
                                  B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), int(window_left),
                                  float(scale), int(num_splits), _dtype_code(q),
                                  seqlens_k.data_ptr(), int(sum_seqlens_k), _stream_ptr(stream))
    _check(rc)
    return out, lse


def bwd(q, k, v, o, dout, lse, causal: bool = False, window_left: int = -1,
        scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
        dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None, stream=None):
    """Attention backward on the GPU (attn_bwd). o and lse are the forward's outputs
    for (q, k, v); dout the gradient of o. Returns (dq, dk, dv) in the dtype of q."""
    _check_tensors(q, k, v)
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    for name, t in (("o", o), ("dout", dout)):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must have the shape and dtype of q")
    if not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32
            and lse.shape == (B, Hq, Sq)):
        raise ValueError("lse must be a contiguous fp32 GPU tensor of shape [B, Hq, Sq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype or not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor like {name[1:]}")
    rc = load().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                           lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                           B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), int(window_left),
                           float(scale), _dtype_code(q), _stream_ptr(stream))
    _check(rc)
    return dq, dk, dv


def plan_bwd(B, Hq, Hkv, Sq, Sk, d, causal=False, window_left=-1, dtype="bf16") -> dict:
    """The backward plan (host only)."""
    p = BwdPlan()
    code = FP32 if dtype in ("fp32", FP32, torch.float32) else BF16
    _check(load().attn_plan_bwd(B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), int(window_left),
                                  code, ctypes.byref(p)))
    return p.as_dict()


def m_block_range(Sq, Sk, causal, window_left, block_m, block_n, n_block):
    """get_m_block_min_max: query-block range of key block n_block (host mirror)."""
    lo, hi = ctypes.c_int(), ctypes.c_int()
    _check(load().attn_m_block_range(Sq, Sk, int(bool(causal)), window_left, block_m, block_n,
                                       n_block, ctypes.byref(lo), ctypes.byref(hi)))
    return lo.value, hi.value


def lse_combine(o_part: torch.Tensor, lse_part: torch.Tensor, out: torch.Tensor,
                lse: Optional[torch.Tensor], B: int, Sq: int, Hq: int, stream=None):
    """Merge split partials o_part [S, B*Sq*Hq, d] fp32, lse_part [S, B*Sq*Hq] into out/lse."""
    S, rows, d = o_part.shape
    if rows != B * Sq * Hq or lse_part.shape != (S, rows):
        raise ValueError("partial shapes do not match B*Sq*Hq rows")
    for t in (o_part, lse_part, out):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("tensors must be contiguous GPU tensors")
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise ValueError("partials must be fp32")
    rc = load().attn_lse_combine(o_part.data_ptr(), lse_part.data_ptr(), out.data_ptr(),
                                   lse.data_ptr() if lse is not None else None,
                                   B, Sq, Hq, d, S, _dtype_code(out), _stream_ptr(stream))
    _check(rc)
    return out, lse


def plan(B, Hq, Hkv, Sq, Sk, d, causal=False, window_left=-1, num_splits=0, dtype="bf16",
         varlen=False, sum_seqlens_k=-1, num_cus=0) -> dict:
    """The planner's choices for a problem (host only)."""
    p = Plan()
    code = FP32 if dtype in ("fp32", FP32, torch.float32) else BF16
    rc = load().attn_plan_fwd(B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), int(window_left),
                                int(num_splits), code, int(bool(varlen)), int(sum_seqlens_k),
                                int(num_cus), ctypes.byref(p))
    _check(rc)
    return p.as_dict()


def plan_dv(B, Hq, Hkv, Sq, Sk, d, d_v, causal=False, window_left=-1, num_splits=0, dtype="bf16",
            num_cus=0) -> dict:
    """The plan of attn_fwd_dv (host only)."""
    p = Plan()
    code = FP32 if dtype in ("fp32", FP32, torch.float32) else BF16
    _check(load().attn_plan_fwd_dv(B, Hq, Hkv, Sq, Sk, d, d_v, int(bool(causal)), int(window_left),
                                     int(num_splits), code, int(num_cus), ctypes.byref(p)))
    return p.as_dict()


def workspace_bytes(B, Hq, Sq, d, num_splits) -> int:
    return int(load().attn_workspace_bytes(B, Hq, Sq, d, num_splits))


def n_block_range(Sq, Skb, G, pack, causal, window_left, block_m, block_n, m_block,
                  split=0, num_splits=1):
    lo, hi = ctypes.c_int(), ctypes.c_int()
    rc = load().attn_n_block_range(Sq, Skb, G, int(bool(pack)), int(bool(causal)),
                                     window_left, block_m, block_n, m_block, split, num_splits,
                                     ctypes.byref(lo), ctypes.byref(hi))
    _check(rc)
    return lo.value, hi.value


def should_pack_gqa(varlen, seqlen_q, qhead_per_khead, block_m) -> bool:
    return bool(load().attn_should_pack_gqa(int(bool(varlen)), seqlen_q, qhead_per_khead, block_m))


def num_splits_fa3(total_mblocks, num_sms, num_n_blocks, num_m_blocks, size_one_kv_head,
                   is_causal_or_local, max_splits) -> int:
    return int(load().attn_num_splits_fa3(total_mblocks, num_sms, num_n_blocks, num_m_blocks,
                                            size_one_kv_head, int(bool(is_causal_or_local)),
                                            max_splits))


def num_splits_occupancy(tiles, num_cus, n_blocks, block_n, min_chunk_rows=256, wg_per_cu=2):
    return int(load().attn_num_splits_occupancy(tiles, num_cus, n_blocks, block_n,
                                                  min_chunk_rows, wg_per_cu))


def stream_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 0, stream=None):
    """attn_stream_read: read a GPU buffer once (the streaming-read reference)."""
    if not (buf.is_cuda and buf.is_contiguous() and sink.is_cuda):
        raise ValueError("buf and sink must be GPU tensors")
    _check(load().attn_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                   int(workgroups), sink.data_ptr(), _stream_ptr(stream)))


def set_workspace(buf: Optional[torch.Tensor]):
    """Bind a caller-owned GPU workspace (any dtype, 256-byte aligned) to this host
    thread (attn_set_workspace); None unbinds. The caller keeps `buf` alive while
    calls that use it may run."""
    if buf is None:
        _check(load().attn_set_workspace(None, 0))
        return
    if not (isinstance(buf, torch.Tensor) and buf.is_cuda and buf.is_contiguous()):
        raise ValueError("the workspace must be a contiguous GPU tensor")
    _check(load().attn_set_workspace(buf.data_ptr(), buf.numel() * buf.element_size()))


def set_option(name: str, value: int):
    """Set a process-wide planner switch (attn_set_option), e.g. "PREFILL_WAVES"."""
    _check(load().attn_set_option(name.encode(), int(value)))


def get_option(name: str) -> int:
    out = ctypes.c_int()
    _check(load().attn_get_option(name.encode(), ctypes.byref(out)))
    return out.value


class options:
    """Context manager: set switches for a block, restore them afterwards."""

    def __init__(self, **kw):
        self.kw = kw
        self.old = {}

    def __enter__(self):
        for k, v in self.kw.items():
            self.old[k] = get_option(k)
            set_option(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.old.items():
            set_option(k, v)
        return False


def profile_begin(max_launches: int = 4096):
    _check(load().attn_profile_begin(int(max_launches)))


KINDS = ("fwd", "combine", "prep", "bwd", "bwd_prepost", "bwd_dq")


def profile_end_kinds() -> dict:
    """Summed event time (ms) and launch count of every kernel kind since profile_begin."""
    ms = (ctypes.c_double * len(KINDS))()
    n = (ctypes.c_int * len(KINDS))()
    _check(load().attn_profile_end_kinds(ms, n, len(KINDS)))
    out = {}
    for i, name in enumerate(KINDS):
        out[name + "_ms"] = ms[i]
        out[name + "_launches"] = n[i]
    return out


def profile_end() -> dict:
    f_ms, c_ms, p_ms = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    f_n, c_n, p_n = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(load().attn_profile_end(ctypes.byref(f_ms), ctypes.byref(f_n), ctypes.byref(c_ms),
                                     ctypes.byref(c_n), ctypes.byref(p_ms), ctypes.byref(p_n)))
    return {"fwd_ms": f_ms.value, "fwd_launches": f_n.value,
            "combine_ms": c_ms.value, "combine_launches": c_n.value,
            "prep_ms": p_ms.value, "prep_launches": p_n.value}
