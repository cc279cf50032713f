"""fp64 CPU oracle for the attention forward and backward passes (ctypes wrapper).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package. The product library
(``tiled_prefill_amd``) never imports it and shares no code with it.

The arithmetic lives in ``attn_ref.c`` (plain C, fp64, OpenMP over query
rows); this module only builds it with gcc and marshals numpy arrays.

Parity status of each oracle function (what pins it, in tests/test_oracle.py):
  attn_ref          pinned: closed forms (constant keys, one-hot dominant
                    key, single visible key), invariants (key shift, key/value
                    permutation, GQA = repeated-head MHA), a library routine
                    (torch fp64 scaled_dot_product_attention with masks built
                    by torch.tril/triu), and the printed causal block count.
  attn_ref_partial  pinned: the merge of partials over any key partition
                    equals attn_ref; one split covering all keys equals it.
  lse_combine_ref   pinned: closed forms (equal lse, single split, all empty)
                    and the partition identity above.
  needed_block_range
                    pinned: the printed causal block count (528 of 1024); with a
                    left window, a count derived by hand for square blocks
                    (min(m, ceil(wl / B)) + 1 key blocks per query block m) and
                    the per-block ranges it implies; with GQA packing, the hull
                    of the one-row-per-block ranges of the packed rows'
                    positions.
  attn_bwd_ref      pinned: central finite differences of attn_ref (tiny
                    shapes with causal, window, GQA and fully masked rows), a
                    library routine (torch fp64 autograd through an explicitly
                    masked softmax), invariants (the key gradients of a head
                    sum to zero; the value gradients sum to the output
                    gradients of rows that see a key; a constant added to
                    every value row leaves dq and dk unchanged) and a closed
                    form (identical keys give dq = 0).
  needed_m_block_range
                    pinned: over all key blocks it visits as many (query
                    block, key block) pairs as needed_block_range (the printed
                    528 of 1024 for the causal example).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_ref.c")
_LIB_PATH = os.environ.get("ATTNREF_LIB") or os.path.join(_HERE, "libattnref.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile attn_ref.c into oracle/libattnref.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out_dir: str) -> str:
    """The same library with host AddressSanitizer + UndefinedBehaviorSanitizer
    (clang, so that one sanitizer runtime serves it and the HIP library; no
    OpenMP: the loops run serially), loaded through ATTNREF_LIB."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cc = os.path.join(rocm, "llvm", "bin", "clang")
    out = os.path.join(out_dir, "libattnref_asan.so")
    subprocess.check_call([cc if os.path.exists(cc) else "clang", "-O1", "-g", "-fPIC", "-shared", "-std=c99",
                           "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-o", out, _SRC, "-lm"])
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    i = ctypes.c_int
    lib.attn_ref_f64.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, ip, i, i, i,
                                 ctypes.c_double, i]
    lib.attn_ref_f64.restype = i
    lib.attn_ref_dv_f64.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, ip, i, i, i, i,
                                    ctypes.c_double, i]
    lib.attn_ref_dv_f64.restype = i
    lib.attn_ref_partial_f64.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, ip, i, i, i,
                                         ctypes.c_double, i, i, i]
    lib.attn_ref_partial_f64.restype = i
    lib.lse_combine_ref_f64.argtypes = [dp, dp, i, ctypes.c_long, i, dp, dp]
    lib.lse_combine_ref_f64.restype = i
    lib.attn_bwd_ref_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, i, i,
                                     ctypes.c_double, i]
    lib.attn_bwd_ref_f64.restype = i
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    """Exact upcast to a contiguous fp64 numpy array (torch or numpy input)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _seqlens(seqlens_k, B):
    if seqlens_k is None:
        return None, None
    try:
        import torch
        if isinstance(seqlens_k, torch.Tensor):
            seqlens_k = seqlens_k.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    arr = np.ascontiguousarray(np.asarray(seqlens_k, dtype=np.int32))
    assert arr.shape == (B,)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def attn_ref(q, k, v, causal: bool, window_left: int, scale: float, seqlens_k=None,
             n_threads: int = 0, key_range=None):
    """Exact attention in fp64. q [B,Sq,Hq,d], k [B,Sk,Hkv,d], v [B,Sk,Hkv,dv].

    Returns (o [B,Sq,Hq,dv] fp64, lse [B,Hq,Sq] fp64). ``key_range=(j0, j1)``
    gives the partial result of one key split instead (attn_ref_partial_f64,
    dv == d only). With dv != d the values have a width of their own
    (attn_ref_dv_f64: the latent-attention verify shape, 576-wide keys and
    512-wide values).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, d = q.shape
    Bk, Sk, Hkv, dk = k.shape
    dv = v.shape[-1]
    assert Bk == B and dk == d and v.shape[:3] == k.shape[:3]
    o = np.zeros((B, Sq, Hq, dv), dtype=np.float64)
    lse = np.zeros((B, Hq, Sq), dtype=np.float64)
    keep, sp = _seqlens(seqlens_k, B)
    lib = _load()
    if dv != d:
        assert key_range is None, "split partials are for dv == d"
        rc = lib.attn_ref_dv_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq,
                                 Sk, sp, d, dv, int(bool(causal)), int(window_left), float(scale),
                                 int(n_threads))
    elif key_range is None:
        rc = lib.attn_ref_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Sk,
                              sp, d, int(bool(causal)), int(window_left), float(scale),
                              int(n_threads))
    else:
        j0, j1 = key_range
        rc = lib.attn_ref_partial_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                      Sq, Sk, sp, d, int(bool(causal)), int(window_left),
                                      float(scale), int(j0), int(j1), int(n_threads))
    del keep
    if rc != 0:
        raise ValueError("attn_ref_f64 rejected its arguments")
    return o, lse


def lse_combine_ref(o_part, lse_part):
    """Merge split partials. o_part [S, rows, d], lse_part [S, rows] -> (o [rows, d], lse [rows])."""
    o_part, lse_part = _f64(o_part), _f64(lse_part)
    S, rows, d = o_part.shape
    assert lse_part.shape == (S, rows)
    o = np.zeros((rows, d), dtype=np.float64)
    lse = np.zeros((rows,), dtype=np.float64)
    rc = _load().lse_combine_ref_f64(_ptr(o_part), _ptr(lse_part), S, rows, d, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("lse_combine_ref_f64 rejected its arguments")
    return o, lse


def visible_mask(Sq: int, Skb: int, causal: bool, window_left: int) -> np.ndarray:
    """Boolean [Sq, Skb] visibility of key j to query row i (bottom-right aligned).

    Per element, the causal bound keeps j <= i + (Skb - Sq) and the window keeps
    j >= i + (Skb - Sq) - window_left, the element-level reading of the block
    bounds in "分块策略与调度" §3.1.
    """
    i = np.arange(Sq)[:, None]
    j = np.arange(Skb)[None, :]
    delta = Skb - Sq
    m = np.ones((Sq, Skb), dtype=bool)
    if causal:
        m &= j <= i + delta
    if window_left >= 0:
        m &= j >= i + delta - window_left
    return m


def needed_block_range(Sq: int, Skb: int, causal: bool, window_left: int, BM: int, BN: int,
                       G: int = 1, pack: bool = False):
    """Brute-force key-block range each query block must visit.

    Rows of query block m are rows [m*BM, (m+1)*BM) of the (optionally
    GQA-packed, row r -> position r // G) query rows. Returns a list, one entry
    per query block, of (first, last+1) key-block indices that hold at least one
    visible (row, key) pair, or None if the block sees no key at all.
    """
    vis = visible_mask(Sq, Skb, causal, window_left)
    nrows = Sq * (G if pack else 1)
    out = []
    for m in range((nrows + BM - 1) // BM):
        r0, r1 = m * BM, min((m + 1) * BM, nrows)
        pos = np.arange(r0, r1) // (G if pack else 1)
        cols = np.nonzero(vis[pos].any(axis=0))[0]
        if cols.size == 0:
            out.append(None)
        else:
            out.append((int(cols[0]) // BN, int(cols[-1]) // BN + 1))
    return out


def attn_bwd_ref(q, k, v, dout, causal: bool, window_left: int, scale: float, n_threads: int = 0):
    """Gradients of L = <dout, attn(q, k, v)> in fp64 (attn_bwd_ref_f64).

    q, dout [B,Sq,Hq,d], k, v [B,Sk,Hkv,d]. Returns (dq, dk, dv) with the shapes
    of q, k, v.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Hq, d = q.shape
    Bk, Sk, Hkv, dk_ = k.shape
    assert Bk == B and dk_ == d and v.shape == k.shape and dout.shape == q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rc = _load().attn_bwd_ref_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                  _ptr(dv), B, Hq, Hkv, Sq, Sk, d, int(bool(causal)),
                                  int(window_left), float(scale), int(n_threads))
    if rc != 0:
        raise ValueError("attn_bwd_ref_f64 rejected its arguments")
    return dq, dk, dv


def needed_m_block_range(Sq: int, Sk: int, causal: bool, window_left: int, BM: int, BN: int):
    """Brute-force query-block range each key block must visit (backward loop order).

    The backward pass of "分块策略与调度" §3.4 runs over key blocks outside and
    the query blocks that see them inside. Returns, per key block n, (first,
    last+1) query-block indices holding at least one (row, key) pair visible
    under the mask of visible_mask, or None if no row sees any key of block n.
    """
    vis = visible_mask(Sq, Sk, causal, window_left)
    out = []
    for n in range((Sk + BN - 1) // BN):
        rows = np.nonzero(vis[:, n * BN:min((n + 1) * BN, Sk)].any(axis=1))[0]
        if rows.size == 0:
            out.append(None)
        else:
            out.append((int(rows[0]) // BM, int(rows[-1]) // BM + 1))
    return out
