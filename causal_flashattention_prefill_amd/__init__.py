"""Causal prefill attention for MI355X (gfx950): Python binding of libzyfa.so.

A thin ctypes layer over the C ABI in include/zyfa.h, with the same names.
It only marshals arguments: torch tensors supply device memory and the
current stream, and every step of the computation runs in the library's HIP
kernels. There is no fallback: if libzyfa.so is missing or cannot be loaded,
importing the binding succeeds but every call raises.

    out, lse = zyfa_fwd(q, k, v, return_lse=True)             # bf16
    q8, qs = zyfa_fp8_quantize(q)                               # fp8 + device descale
    out = zyfa_fwd(q8, k8, v8, q_descale=qs, k_descale=ks, v_descale=vs)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

# ZYFA_LIB selects another build of the same library (e.g. to compare two
# builds on one machine); by default the in-tree libzyfa.so is loaded.
LIB_PATH = os.environ.get("ZYFA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzyfa.so")

LAYOUTS = {"bshd": 0, "bhsd": 1}
DTYPE_BF16, DTYPE_FP8, DTYPE_FP32 = 0, 1, 2

ZYFA_OK = 0
STATUS = {
    "ZYFA_ERR_NULL": -1, "ZYFA_ERR_SHAPE": -2, "ZYFA_ERR_HEADDIM": -3, "ZYFA_ERR_GQA": -4,
    "ZYFA_ERR_DTYPE": -5, "ZYFA_ERR_LAYOUT": -6, "ZYFA_ERR_DESCALE": -7, "ZYFA_ERR_CAPTURE": -8,
    "ZYFA_ERR_HIP": -9, "ZYFA_ERR_RANGE": -10, "ZYFA_ERR_ALIGN": -11, "ZYFA_ERR_PMODE": -12, "ZYFA_ERR_SIGNS": -13,
    "ZYFA_ERR_SCRATCH": -14,
}
# FP8 probability modes (zyfa_p_mode): default = lean P below the diagonal at
# d_qk 128, exact P at d_qk 192; precise = bf16-MFMA scores and P split into
# hi + lo e4m3 parts.
P_MODES = {"default": 0, "exact": 1, "lean": 2, "precise": 3}

_lib = None
_lib_err: Optional[str] = None


class ZyfaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: status {status} ({zyfa_status_string(status)})")


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it is not built or cannot load)."""
    global _lib, _lib_err
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libzyfa.so not built ({LIB_PATH}); run causal_flashattention_prefill_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, ll = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong
    fwd_args = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, vp]
    L.zyfa_fwd.argtypes = fwd_args + [vp]
    L.zyfa_fwd.restype = i
    L.zyfa_fwd_ex.argtypes = fwd_args + [f, i, vp]
    L.zyfa_fwd_ex.restype = i
    L.zyfa_fwd_noalloc.argtypes = fwd_args + [f, i, vp]
    L.zyfa_fwd_noalloc.restype = i
    L.zyfa_fwd_range.argtypes = [vp, vp, vp, vp, vp, i, i, i, ll, ll, i, i, i, i, i, i, vp, vp, vp, f, i, vp]
    L.zyfa_fwd_range.restype = i
    L.zyfa_lse_merge.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    L.zyfa_lse_merge.restype = i
    L.zyfa_prepare.argtypes = [i, i, i, i, i, i, i, i, i, vp]
    L.zyfa_prepare.restype = i
    L.zyfa_set_tile_q.argtypes = [i, i, i, i, i, i, i]
    L.zyfa_set_tile_q.restype = i
    L.zyfa_fp8_quantize.argtypes = [vp, i, ll, vp, vp, vp]
    L.zyfa_fp8_quantize_rotated.argtypes = [vp, i, ll, i, vp, vp, vp, vp]
    L.zyfa_fp8_quantize_rotated.restype = i
    L.zyfa_fp8_quantize_rotated_shifted.argtypes = [vp, i, i, i, i, i, i, vp, vp, vp, vp, vp]
    L.zyfa_fp8_quantize_rotated_shifted.restype = i
    L.zyfa_key_mean.argtypes = [vp, i, i, i, i, i, i, vp, vp]
    L.zyfa_key_mean.restype = i
    L.zyfa_fp8_quantize.restype = i
    L.zyfa_status_string.argtypes = [i]
    L.zyfa_status_string.restype = ctypes.c_char_p
    L.zyfa_release.argtypes = []
    L.zyfa_release.restype = None
    ip = ctypes.POINTER(ctypes.c_int)
    L.zyfa_plan_jobs.argtypes = [i, i, i, i, i, i, i, ip, ip, ip, vp, ll]
    L.zyfa_plan_jobs.restype = i
    _lib = L
    return L


def zyfa_status_string(status: int) -> str:
    return lib().zyfa_status_string(int(status)).decode()


def _check(rc: int, what: str) -> None:
    if rc != ZYFA_OK:
        raise ZyfaError(rc, what)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, ref=None) -> Optional[int]:
    """The HIP stream handle: `stream`, or the current stream of ref's device."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(ref.device if ref is not None and ref.is_cuda else None)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on_device(ref):
    """Makes ref's GPU the current device for a library call: the library
    keeps its plans per current device and launches on the given stream."""
    import contextlib
    import torch
    return torch.cuda.device(ref.device) if ref is not None and ref.is_cuda else contextlib.nullcontext()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DTYPE_FP8
    raise TypeError(f"unsupported input dtype {t.dtype}")


# The C ABI takes plain pointers and cannot see buffer sizes, so the binding
# checks every tensor it passes: shape, dtype and contiguity first, then that
# all of them live on the same GPU (a host pointer or a short buffer would
# otherwise reach the kernels).

def _require(t, name: str, shape, dtypes) -> None:
    if t.dim() != len(shape) or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_gpu(ref, named) -> None:
    if not ref.is_cuda:
        raise ValueError("tensors must be on a GPU (cuda) device")
    for name, t in named:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _check_descales(named) -> None:
    import torch
    for name, t in named:
        if t is not None and (t.dtype != torch.float32 or t.numel() < 1 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 tensor with at least one element")


def _attn_checks(q, k, v, out, lse, layout: str, descales, seqlen_k: Optional[int] = None):
    """Shapes of q, k, v (k and v with seqlen_k positions when given, else
    q's), out and lse; one input dtype; descales; one GPU. Returns the dims
    (B, Sq, Sk, H, Hk, d_qk, d_v)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D ({layout})")
    in_dtypes = (torch.bfloat16, torch.float8_e4m3fn, torch.uint8)
    if q.dtype not in in_dtypes:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    bshd = layout == "bshd"
    B, Sq, H, dqk = (q.shape[0], q.shape[1], q.shape[2], q.shape[3]) if bshd else \
        (q.shape[0], q.shape[2], q.shape[1], q.shape[3])
    Sk = Sq if seqlen_k is None else seqlen_k          # whole-sequence calls: k and v have q's length
    Hk = k.shape[2] if bshd else k.shape[1]
    dv = v.shape[3]
    shp = (lambda s, h, d: (B, s, h, d)) if bshd else (lambda s, h, d: (B, h, s, d))
    same = (q.dtype,) if q.dtype == torch.bfloat16 else (torch.float8_e4m3fn, torch.uint8)
    _require(q, "q", shp(Sq, H, dqk), in_dtypes)
    _require(k, "k", shp(Sk, Hk, dqk), same)
    _require(v, "v", shp(Sk, Hk, dv), same)
    if out is not None:
        _require(out, "out", shp(Sq, H, dv), (torch.bfloat16,))
    if lse is not None:
        _require(lse, "lse", (B, H, Sq), (torch.float32,))
    _check_descales(descales)
    _same_gpu(q, [("k", k), ("v", v), ("out", out), ("lse", lse)] + list(descales))
    return B, Sq, Sk, H, Hk, dqk, dv


def zyfa_fwd(q, k, v, out=None, lse=None, *, layout: str = "bshd", return_lse: bool = False,
             q_descale=None, k_descale=None, v_descale=None, softmax_scale: Optional[float] = None,
             p_mode: str = "default", stream=None):
    """Causal forward attention. q, k, v: contiguous CUDA tensors (bf16, or
    float8_e4m3fn / uint8 codes with fp32 device descales). p_mode selects
    the FP8 probability rounding ("default", "exact", "lean", "precise"; see
    zyfa_p_mode in zyfa.h). Returns out, or (out, lse) when return_lse (or
    an lse tensor is passed)."""
    import torch
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    desc = [("q_descale", q_descale), ("k_descale", k_descale), ("v_descale", v_descale)]
    B, S, _, H, Hk, dqk, dv = _attn_checks(q, k, v, out, lse, layout, desc, None)
    dt = _dtype_code(q)
    if out is None:
        shape = (B, S, H, dv) if layout == "bshd" else (B, H, S, dv)
        out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    L = lib()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, S, H, Hk, dqk, dv, LAYOUTS[layout], dt,
            _ptr(q_descale), _ptr(k_descale), _ptr(v_descale))
    if p_mode not in P_MODES:
        raise ValueError(f"p_mode must be one of {list(P_MODES)}")
    with _on_device(q):
        if softmax_scale is None and p_mode == "default":
            rc = L.zyfa_fwd(*args, _stream(stream, q))
        else:
            rc = L.zyfa_fwd_ex(*args, 0.0 if softmax_scale is None else float(softmax_scale), P_MODES[p_mode],
                               _stream(stream, q))
    _check(rc, "zyfa_fwd")
    return (out, lse) if lse is not None else out


def zyfa_fwd_noalloc(q, k, v, out, lse=None, *, layout: str = "bshd", q_descale=None, k_descale=None,
                     v_descale=None, softmax_scale: Optional[float] = None, p_mode: str = "default", stream=None):
    """zyfa_fwd into caller-given out (and lse) with no device allocation by
    the library: the job table goes into its static buffer (see
    zyfa_fwd_noalloc in zyfa.h; overlapping calls on one GPU race). Returns
    out, or (out, lse)."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    if p_mode not in P_MODES:
        raise ValueError(f"p_mode must be one of {list(P_MODES)}")
    if out is None:
        raise ValueError("zyfa_fwd_noalloc writes into a caller-given out")
    desc = [("q_descale", q_descale), ("k_descale", k_descale), ("v_descale", v_descale)]
    B, S, _, H, Hk, dqk, dv = _attn_checks(q, k, v, out, lse, layout, desc, None)
    with _on_device(q):
        rc = lib().zyfa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, S, H, Hk, dqk, dv,
                                    LAYOUTS[layout], _dtype_code(q), _ptr(q_descale), _ptr(k_descale),
                                    _ptr(v_descale), 0.0 if softmax_scale is None else float(softmax_scale),
                                    P_MODES[p_mode], _stream(stream, q))
    _check(rc, "zyfa_fwd_noalloc")
    return (out, lse) if lse is not None else out


def zyfa_fwd_range(q, k, v, q_pos0: int, k_pos0: int, out=None, lse=None, *, layout: str = "bshd",
                   return_lse: bool = True, q_descale=None, k_descale=None, v_descale=None,
                   softmax_scale: Optional[float] = None, p_mode: str = "default", stream=None):
    """Causal attention of queries at positions q_pos0 + r over keys at
    positions k_pos0 + c (key visible when its position <= the query's).
    k and v may have another seqlen than q. Rows that see no key get out = 0
    and lse = -inf. Returns (out, lse) (lse allocated unless return_lse is
    False and none is passed)."""
    import torch
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    if p_mode not in P_MODES:
        raise ValueError(f"p_mode must be one of {list(P_MODES)}")
    desc = [("q_descale", q_descale), ("k_descale", k_descale), ("v_descale", v_descale)]
    if k.dim() != 4:
        raise ValueError(f"k must be 4-D ({layout})")
    Sk = k.shape[1] if layout == "bshd" else k.shape[2]
    B, Sq, Sk, H, Hk, dqk, dv = _attn_checks(q, k, v, out, lse, layout, desc, Sk)
    if out is None:
        shape = (B, Sq, H, dv) if layout == "bshd" else (B, H, Sq, dv)
        out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    with _on_device(q):
        rc = lib().zyfa_fwd_range(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Sk, int(q_pos0),
                                  int(k_pos0), H, Hk, dqk, dv, LAYOUTS[layout], _dtype_code(q), _ptr(q_descale),
                                  _ptr(k_descale), _ptr(v_descale),
                                  0.0 if softmax_scale is None else float(softmax_scale), P_MODES[p_mode],
                                  _stream(stream, q))
    _check(rc, "zyfa_fwd_range")
    return (out, lse) if lse is not None else out


def zyfa_lse_merge(out_a, lse_a, out_b, lse_b, out=None, lse=None, *, layout: str = "bshd", stream=None):
    """Merge two partial results (bf16 out, fp32 lse) of the same query rows
    over disjoint key sets. out/lse may be out_a/lse_a (in place). Returns
    (out, lse)."""
    import torch
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    for t in (out_a, out_b, lse_a, lse_b):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    if out_a.shape != out_b.shape or lse_a.shape != lse_b.shape:
        raise ValueError("the two partial results must have the same shapes")
    if out_a.dtype != torch.bfloat16 or lse_a.dtype != torch.float32 or lse_b.dtype != torch.float32:
        raise TypeError("out must be bf16 and lse fp32")
    if lse_a.dim() != 3 or out_a.dim() != 4:
        raise ValueError("lse must be (batch, heads, seqlen) and out 4-D")
    B, H, S = lse_a.shape
    dv = out_a.shape[-1]
    want = (B, S, H, dv) if layout == "bshd" else (B, H, S, dv)
    _require(out_a, "out_a", want, (torch.bfloat16,))
    if out is not None:
        _require(out, "out", want, (torch.bfloat16,))
    if lse is not None:
        _require(lse, "lse", (B, H, S), (torch.float32,))
    _same_gpu(out_a, [("out_b", out_b), ("lse_a", lse_a), ("lse_b", lse_b), ("out", out), ("lse", lse)])
    if out is None:
        out = torch.empty_like(out_a)
    if lse is None:
        lse = torch.empty_like(lse_a)
    with _on_device(out_a):
        rc = lib().zyfa_lse_merge(_ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), _ptr(out), _ptr(lse), B, S, H,
                                  dv, LAYOUTS[layout], _stream(stream, out_a))
    _check(rc, "zyfa_lse_merge")
    return out, lse


def zyfa_prepare(batch, seqlen, nheads, nheads_k, d_qk, d_v, layout="bshd", dtype=DTYPE_BF16, with_lse=False,
                 stream=None) -> None:
    _check(lib().zyfa_prepare(batch, seqlen, nheads, nheads_k, d_qk, d_v, LAYOUTS[layout], dtype, int(with_lse),
                              _stream(stream)), "zyfa_prepare")


def zyfa_set_tile_q(batch, seqlen, nheads, nheads_k, d_qk=128, dtype=DTYPE_BF16, tile_q=0) -> None:
    """Query-tile height (128 or 256; 0 = automatic) that calls of this shape
    use on the current device from now on."""
    _check(lib().zyfa_set_tile_q(batch, seqlen, nheads, nheads_k, d_qk, dtype, tile_q), "zyfa_set_tile_q")


def zyfa_fp8_quantize(x, x8=None, descale=None, stream=None):
    """Per-tensor power-of-two e4m3fn quantization of a bf16 or fp32 CUDA
    tensor. Returns (codes as torch.float8_e4m3fn, descale as a 1-element fp32
    CUDA tensor)."""
    import torch
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    xd = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_FP32}.get(x.dtype)
    if xd is None:
        raise TypeError(f"unsupported dtype {x.dtype}")
    if x8 is not None:
        _require(x8, "x8", tuple(x.shape), (torch.float8_e4m3fn, torch.uint8))
    _check_descales([("descale", descale)])
    _same_gpu(x, [("x8", x8), ("descale", descale)])
    if x8 is None:
        x8 = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    if descale is None:
        descale = torch.empty(1, dtype=torch.float32, device=x.device)
    with _on_device(x):
        rc = lib().zyfa_fp8_quantize(_ptr(x), xd, x.numel(), _ptr(x8), _ptr(descale), _stream(stream, x))
    _check(rc, "zyfa_fp8_quantize")
    return x8, descale


def zyfa_fp8_quantize_rotated(x, signs=None, x8=None, descale=None, *, shift=None, layout: str = "bshd",
                              stream=None):
    """Rotate the last axis of x (d = 128; other d raise) by the orthogonal
    matrix of zyfa.h's zyfa_fp8_quantize_rotated, then quantize per tensor. signs:
    d values of +1 / -1 (a sequence or array on the host), or None for all
    +1. shift: optional (batch, heads, d) fp32 CUDA tensor subtracted from
    every position of its head before the rotation (K smoothing; x is then
    a 4-D tensor in `layout`). Returns (codes as torch.float8_e4m3fn,
    descale as a 1-element fp32 CUDA tensor)."""
    import numpy as np
    import torch
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    xd = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_FP32}.get(x.dtype)
    if xd is None:
        raise TypeError(f"unsupported dtype {x.dtype}")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    sg = None
    if signs is not None:
        sg = np.ascontiguousarray(np.asarray(signs.cpu() if hasattr(signs, "cpu") else signs).astype(np.int8))
        if sg.shape != (d,):
            raise ValueError(f"signs must hold {d} values")
    if x8 is not None:
        _require(x8, "x8", tuple(x.shape), (torch.float8_e4m3fn, torch.uint8))
    _check_descales([("descale", descale)])
    _same_gpu(x, [("x8", x8), ("descale", descale), ("shift", shift)])
    if x8 is None:
        x8 = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    if descale is None:
        descale = torch.empty(1, dtype=torch.float32, device=x.device)
    sp = None if sg is None else sg.ctypes.data
    if shift is None:
        with _on_device(x):
            rc = lib().zyfa_fp8_quantize_rotated(_ptr(x), xd, rows, d, sp, _ptr(x8), _ptr(descale),
                                                 _stream(stream, x))
    else:
        if x.dim() != 4 or layout not in LAYOUTS:
            raise ValueError("a shift needs a 4-D x in bshd or bhsd")
        B, S, H = (x.shape[0], x.shape[1], x.shape[2]) if layout == "bshd" else (x.shape[0], x.shape[2], x.shape[1])
        if shift.dtype != torch.float32 or tuple(shift.shape) != (B, H, d) or not shift.is_contiguous():
            raise ValueError(f"shift must be a contiguous fp32 tensor of shape {(B, H, d)}")
        with _on_device(x):
            rc = lib().zyfa_fp8_quantize_rotated_shifted(_ptr(x), xd, B, S, H, d, LAYOUTS[layout], sp, _ptr(shift),
                                                         _ptr(x8), _ptr(descale), _stream(stream, x))
    _check(rc, "zyfa_fp8_quantize_rotated")
    return x8, descale


def zyfa_key_mean(k, *, layout: str = "bshd", mean=None, stream=None):
    """Mean key of each (batch, head) over the sequence: (batch, heads, d)
    fp32 CUDA tensor (K smoothing, see zyfa.h)."""
    import torch
    if not k.is_contiguous() or k.dim() != 4:
        raise ValueError("k must be a contiguous 4-D tensor")
    kd = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_FP32}.get(k.dtype)
    if kd is None:
        raise TypeError(f"unsupported dtype {k.dtype}")
    B, S, H = (k.shape[0], k.shape[1], k.shape[2]) if layout == "bshd" else (k.shape[0], k.shape[2], k.shape[1])
    d = k.shape[3]
    if mean is not None:
        _require(mean, "mean", (B, H, d), (torch.float32,))
    _same_gpu(k, [("mean", mean)])
    if mean is None:
        mean = torch.empty((B, H, d), dtype=torch.float32, device=k.device)
    with _on_device(k):
        rc = lib().zyfa_key_mean(_ptr(k), kd, B, S, H, d, LAYOUTS[layout], _ptr(mean), _stream(stream, k))
    _check(rc, "zyfa_key_mean")
    return mean


def zyfa_release() -> None:
    lib().zyfa_release()


def zyfa_plan_jobs(batch, seqlen, nheads, nheads_k, d_qk=128, dtype=DTYPE_BF16, num_cus=256):
    """Host-only job table: returns (tile_q, num_wgs, jobs_per_wg, table) with
    table an int array of shape (jobs_per_wg, num_wgs, 2)."""
    import numpy as np
    L = lib()
    tq, nw, jp = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(L.zyfa_plan_jobs(batch, seqlen, nheads, nheads_k, d_qk, dtype, num_cus, ctypes.byref(tq),
                            ctypes.byref(nw), ctypes.byref(jp), None, 0), "zyfa_plan_jobs")
    table = np.empty((jp.value, nw.value, 2), dtype=np.int32)
    _check(L.zyfa_plan_jobs(batch, seqlen, nheads, nheads_k, d_qk, dtype, num_cus, ctypes.byref(tq),
                            ctypes.byref(nw), ctypes.byref(jp), table.ctypes.data, table.size), "zyfa_plan_jobs")
    return tq.value, nw.value, jp.value, table
