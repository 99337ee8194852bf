"""Python binding of the gfx950 MuonClip library (libmuonclip.so).

Argument marshalling only: torch tensors supply device pointers, shapes and
the current HIP stream; every step of the optimizer runs in the library's HIP
kernels. There is no fallback: if the library is not built, load() raises.

Names follow the C ABI in include/muonclip.h: muonclip_step,
max_logits_per_head, qk_clip_apply, plus workspace sizing and kernel timing.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuonclip.so")

MC_OK, MC_ERR_NULL, MC_ERR_SHAPE, MC_ERR_DTYPE, MC_ERR_WORKSPACE, MC_ERR_HPARAM, MC_ERR_HIP, MC_ERR_ALIGN = range(8)
MC_F32, MC_BF16 = 0, 1

EXPORTS = ("mc_default_hparams", "mc_workspace_size", "mc_workspace_min_size", "muonclip_step",
           "muonclip_step_overlapped", "muonclip_step_noalloc",
           "max_logits_per_head", "qk_clip_apply", "mc_last_error", "mc_version",
           "mc_profile_enable", "mc_profile_read", "mc_default_adamw_hparams", "adamw_step",
           "attention_forward")


class MuonClipError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class Segment(ctypes.Structure):
    _fields_ = [("offset", c_int32), ("length", c_int32), ("expo", c_float)]


class Matrix(ctypes.Structure):
    _fields_ = [("w", c_void_p), ("g", c_void_p), ("m", c_void_p), ("o_out", c_void_p),
                ("rows", c_int64), ("cols", c_int64), ("ld", c_int64),
                ("w_dtype", c_int32), ("g_dtype", c_int32),
                ("clip_slot", c_int32), ("period", c_int32), ("nseg", c_int32),
                ("seg", Segment * 2)]


class HParams(ctypes.Structure):
    _fields_ = [("lr", c_float), ("mu", c_float), ("weight_decay", c_float), ("rms_scale", c_float),
                ("tau", c_float), ("ns_a", c_float), ("ns_b", c_float), ("ns_c", c_float),
                ("ns_eps", c_float), ("ns_steps", c_int32), ("nesterov", c_int32), ("clip_global", c_int32)]


class Vector(ctypes.Structure):
    _fields_ = [("p", c_void_p), ("g", c_void_p), ("m", c_void_p), ("v", c_void_p), ("n", c_int64),
                ("p_dtype", c_int32), ("g_dtype", c_int32)]


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("weight_decay", c_float), ("step", c_int32)]


class ProfileEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", c_int32), ("ms", c_double),
                ("flops", c_double), ("bytes", c_double)]


_lib = None


def load():
    """Load libmuonclip.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m muonclip_step_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    MP = POINTER(Matrix)
    HP = POINTER(HParams)
    lib.mc_default_hparams.argtypes = [HP]
    lib.mc_default_hparams.restype = None
    lib.mc_workspace_size.argtypes = [MP, c_int32, HP]
    lib.mc_workspace_size.restype = c_size_t
    lib.mc_workspace_min_size.argtypes = [MP, c_int32, HP]
    lib.mc_workspace_min_size.restype = c_size_t
    lib.muonclip_step.argtypes = [MP, c_int32, HP, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.muonclip_step.restype = c_int32
    lib.muonclip_step_overlapped.argtypes = lib.muonclip_step.argtypes + [c_void_p]
    lib.muonclip_step_overlapped.restype = c_int32
    lib.muonclip_step_noalloc.argtypes = [MP, c_int32, HP, c_void_p, c_int32, c_int32, c_void_p, c_void_p]
    lib.muonclip_step_noalloc.restype = c_int32
    lib.max_logits_per_head.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                        c_int32, c_int32, c_int32, POINTER(c_int64), POINTER(c_int64),
                                        POINTER(c_int64), c_int32, c_float, c_void_p, c_void_p]
    lib.max_logits_per_head.restype = c_int32
    lib.qk_clip_apply.argtypes = [MP, c_int32, c_void_p, c_int32, c_int32, c_float, c_void_p, c_void_p]
    lib.qk_clip_apply.restype = c_int32
    lib.mc_last_error.argtypes = []
    lib.mc_last_error.restype = c_char_p
    lib.mc_version.argtypes = []
    lib.mc_version.restype = c_char_p
    lib.mc_profile_enable.argtypes = [c_int32]
    lib.mc_profile_enable.restype = c_int32
    lib.mc_profile_read.argtypes = [POINTER(ProfileEntry), c_int32]
    lib.mc_profile_read.restype = c_int32
    lib.mc_default_adamw_hparams.argtypes = [POINTER(AdamWHParams)]
    lib.mc_default_adamw_hparams.restype = None
    lib.adamw_step.argtypes = [POINTER(Vector), c_int32, POINTER(AdamWHParams), c_void_p]
    lib.adamw_step.restype = c_int32
    lib.attention_forward.argtypes = [c_void_p] * 7 + [c_int32] * 7 + [c_void_p] * 5 + [c_int32, c_float, c_void_p]
    lib.attention_forward.restype = c_int32
    _lib = lib
    return lib


def _check(status: int):
    if status != MC_OK:
        raise MuonClipError(status, load().mc_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MC_F32
    if t.dtype == torch.bfloat16:
        return MC_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def hparams(**kw) -> HParams:
    """Default hyper-parameters with keyword overrides."""
    hp = HParams()
    load().mc_default_hparams(ctypes.byref(hp))
    for k, v in kw.items():
        setattr(hp, k, v)
    return hp


def matrix(w, g, m, o_out=None, clip_slot: int = -1, period: int = 0, segments=()) -> Matrix:
    """Describe one parameter. w/g/m: 2-D tensors with unit column stride and
    a common row stride; segments: ((offset, length, expo), ...)."""
    if w.dim() != 2 or w.shape != g.shape or w.shape != m.shape:
        raise ValueError("w, g, m must be 2-D tensors of one shape")
    for t in (w, g, m):
        if t.stride(1) != 1:
            raise ValueError("columns must be contiguous")
    if not (w.stride(0) == g.stride(0) == m.stride(0)):
        raise ValueError("w, g, m must share the row stride")
    mat = Matrix()
    mat.w, mat.g, mat.m = w.data_ptr(), g.data_ptr(), m.data_ptr()
    mat.o_out = o_out.data_ptr() if o_out is not None else None
    mat.rows, mat.cols, mat.ld = w.shape[0], w.shape[1], w.stride(0)
    mat.w_dtype, mat.g_dtype = _dtype_code(w), _dtype_code(g)
    mat.clip_slot, mat.period, mat.nseg = clip_slot, period, len(segments)
    for i, (off, ln, ex) in enumerate(segments):
        mat.seg[i] = Segment(off, ln, ex)
    return mat


def _array(mats):
    arr = (Matrix * max(1, len(mats)))(*mats)
    return arr, len(mats)


def workspace_size(mats, hp: HParams | None = None, minimal: bool = False) -> int:
    lib = load()
    hp = hp or hparams()
    arr, n = _array(mats)
    fn = lib.mc_workspace_min_size if minimal else lib.mc_workspace_size
    size = fn(arr, n, ctypes.byref(hp))
    if size == 0 and n > 0:
        raise MuonClipError(-1, lib.mc_last_error().decode())
    return size


def muonclip_step(mats, hp: HParams | None = None, s_max=None, slots: int = 0, heads: int = 0,
                  gamma_out=None, workspace=None, stream=None, s_max_ready=None):
    """One MuonClip step over `mats` (list of Matrix) on the current stream.
    workspace: a uint8 device tensor (allocated here when None).
    s_max_ready: a torch.cuda.Event recorded after the launch that writes
    s_max on another stream; only the launches that read s_max wait on it
    (muonclip_step_overlapped)."""
    lib = load()
    hp = hp or hparams()
    arr, n = _array(mats)
    if workspace is None:
        import torch
        workspace = torch.empty(max(workspace_size(mats, hp), 256), dtype=torch.uint8, device="cuda")
    args = (arr, n, ctypes.byref(hp), _ptr(s_max), slots, heads, _ptr(gamma_out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if s_max_ready is None:
        _check(lib.muonclip_step(*args))
    else:
        ev = s_max_ready if isinstance(s_max_ready, int) else s_max_ready.cuda_event
        if not ev:
            raise ValueError("s_max_ready has not been recorded")
        _check(lib.muonclip_step_overlapped(*args, ctypes.c_void_p(ev)))
    return workspace


NOALLOC_SCRATCH_BYTES = 256 << 20   # MC_NOALLOC_SCRATCH_BYTES of include/muonclip.h


def muonclip_step_noalloc(mats, hp: HParams | None = None, s_max=None, slots: int = 0, heads: int = 0,
                          gamma_out=None, stream=None):
    """muonclip_step with the library's static per-device scratch as the
    workspace: allocates nothing (calls on one device must not overlap)."""
    lib = load()
    hp = hp or hparams()
    arr, n = _array(mats)
    _check(lib.muonclip_step_noalloc(arr, n, ctypes.byref(hp), _ptr(s_max), slots, heads, _ptr(gamma_out),
                                     _stream(stream)))


def max_logits_per_head(q, k, k_shared=None, causal: bool = True, scale: float | None = None, out=None,
                        stream=None):
    """Per-head max logit; q [B,T,H,d_q], k [B,T,H,d_k], k_shared [B,T,d_s]."""
    import torch
    B, T, H, d_q = q.shape
    d_k = k.shape[3]
    d_s = k_shared.shape[2] if k_shared is not None else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d_q)
    if out is None:
        out = torch.empty(H, dtype=torch.float32, device=q.device)
    qs = (c_int64 * 3)(q.stride(0), q.stride(1), q.stride(2))
    ks = (c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
    kss = (c_int64 * 2)(k_shared.stride(0), k_shared.stride(1)) if k_shared is not None else None
    for t in (q, k) + ((k_shared,) if k_shared is not None else ()):
        if t.stride(-1) != 1:
            raise ValueError("last dimension must be contiguous")
    _check(load().max_logits_per_head(_ptr(q), _ptr(k), _ptr(k_shared), _dtype_code(q), B, T, H, d_q, d_k, d_s,
                                      qs, ks, kss, int(bool(causal)), scale, _ptr(out), _stream(stream)))
    return out


def attention_forward(q, k, k_shared, v, causal: bool = True, scale: float | None = None, out=None, lse=None,
                      s_max=None, stream=None):
    """Softmax attention forward (bf16) with the per-head max logit taken on
    the way: q [B,T,H,d_q], k [B,T,H,d_k], k_shared [B,T,d_s] or None,
    v [B,T,H,d_v]. Returns out [B,T,H,d_v] (allocated when None). lse
    (fp32 [B,H,T], contiguous) and s_max (fp32 [H]) are filled when given."""
    import torch
    B, T, H, d_q = q.shape
    d_k = k.shape[3]
    d_s = k_shared.shape[2] if k_shared is not None else 0
    d_v = v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d_q)
    if out is None:
        out = torch.empty(B, T, H, d_v, dtype=v.dtype, device=v.device)
    for t in (q, k, v, out) + ((k_shared,) if k_shared is not None else ()):
        if t.stride(-1) != 1:
            raise ValueError("last dimension must be contiguous")
    if lse is not None and not lse.is_contiguous():
        raise ValueError("lse must be contiguous [B, H, T]")
    st3 = lambda t: (c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))
    kss = (c_int64 * 2)(k_shared.stride(0), k_shared.stride(1)) if k_shared is not None else None
    _check(load().attention_forward(_ptr(q), _ptr(k), _ptr(k_shared), _ptr(v), _ptr(out), _ptr(lse), _ptr(s_max),
                                    B, T, H, d_q, d_k, d_s, d_v, st3(q), st3(k), kss, st3(v), st3(out),
                                    int(bool(causal)), scale, _stream(stream)))
    return out


def qk_clip_apply(mats, s_max, slots: int, heads: int, tau: float, gamma_out=None, stream=None):
    arr, n = _array(mats)
    _check(load().qk_clip_apply(arr, n, _ptr(s_max), slots, heads, tau, _ptr(gamma_out), _stream(stream)))


def adamw_hparams(**kw) -> AdamWHParams:
    """Default AdamW hyper-parameters with keyword overrides."""
    hp = AdamWHParams()
    load().mc_default_adamw_hparams(ctypes.byref(hp))
    for k, v in kw.items():
        setattr(hp, k, v)
    return hp


def vector(p, g, m, v) -> Vector:
    """Describe one non-matrix parameter: contiguous tensors of one size."""
    for t in (p, g, m, v):
        if not t.is_contiguous():
            raise ValueError("AdamW tensors must be contiguous")
    if not (p.numel() == g.numel() == m.numel() == v.numel()):
        raise ValueError("p, g, m, v must have the same number of elements")
    d = Vector()
    d.p, d.g, d.m, d.v = p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr()
    d.n = p.numel()
    d.p_dtype, d.g_dtype = _dtype_code(p), _dtype_code(g)
    return d


def adamw_step(vecs, hp: AdamWHParams | None = None, stream=None):
    """One AdamW step over `vecs` (list of Vector) on the current stream."""
    hp = hp or adamw_hparams()
    arr = (Vector * max(1, len(vecs)))(*vecs)
    _check(load().adamw_step(arr, len(vecs), ctypes.byref(hp), _stream(stream)))


def profile_enable(on: bool = True):
    _check(load().mc_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{family: {"launches", "ms", "flops", "bytes"}} of the recorded launches."""
    lib = load()
    buf = (ProfileEntry * 32)()
    k = lib.mc_profile_read(buf, 32)
    if k < 0:
        raise MuonClipError(MC_ERR_HIP, lib.mc_last_error().decode())
    return {buf[i].name.decode(): dict(launches=buf[i].launches, ms=buf[i].ms, flops=buf[i].flops,
                                       bytes=buf[i].bytes) for i in range(min(k, 32))}


def version() -> str:
    return load().mc_version().decode()
