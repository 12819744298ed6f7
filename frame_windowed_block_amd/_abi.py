"""ctypes binding of libfsa.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module only
turns torch tensors into device pointers and streams, allocates outputs with
torch when the caller passes none, and raises ``FsaError`` on a non-zero
status. If libfsa.so is missing it raises at first use: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfsa.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fsa.h")

FSA_OK = 0
FSA_ERR_INVALID_ARG = 1
FSA_ERR_UNALIGNED = 2
FSA_ERR_UNSUPPORTED = 3
FSA_ERR_BUFFER_TOO_SMALL = 4
FSA_ERR_HIP = 5


class FsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fsa status {status}: {message}")
        self.status = status
        self.message = message


class PlanInfo(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "frames", "tokens_per_frame", "window", "ref_frame", "seq_len",
        "block_q", "block_k", "n_qblocks", "n_kblocks", "nnz")]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}

    def __repr__(self) -> str:
        return f"PlanInfo({self.as_dict()})"


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_I32P = ctypes.POINTER(ctypes.c_int32)


def lib() -> ctypes.CDLL:
    """Load libfsa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with "
                               "`python -m frame_windowed_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.fsa_version.restype = _I32
        L.fsa_version.argtypes = []
        L.fsa_status_string.restype = ctypes.c_char_p
        L.fsa_status_string.argtypes = [ctypes.c_int]
        L.fsa_last_error.restype = ctypes.c_char_p
        L.fsa_last_error.argtypes = []
        L.fsa_plan.restype = ctypes.c_int
        L.fsa_plan.argtypes = [_I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(PlanInfo),
                               _I32P, _I64, _I32P, _I64]
        L.fsa_bounds.restype = ctypes.c_int
        L.fsa_bounds.argtypes = [ctypes.POINTER(PlanInfo), _P, _P, _P, _P, _I32, _I32, _I32,
                                 _I32, _I32, _F32, _F32, _P, _P, _P, _P, _P, _P]
        L.fsa_attention.restype = ctypes.c_int
        L.fsa_attention.argtypes = [ctypes.POINTER(PlanInfo), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _I32, _I32, _I32, _F32, _I32, _I32, _P]
        L.fsa_pre_attention.restype = ctypes.c_int
        L.fsa_pre_attention.argtypes = [_P, _P, _I32, _I32, _I32, _I32, _I32, _F32, _F32,
                                        _P, _P, _P, _P]
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Names of the functions include/fsa.h declares."""
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsa_[a-z_]+)\s*\(", text)))


def _check(status: int):
    if status != FSA_OK:
        L = lib()
        raise FsaError(status, L.fsa_last_error().decode() or L.fsa_status_string(status).decode())


def version() -> int:
    return int(lib().fsa_version())


def plan(frames: int, tokens_per_frame: int, window: int, ref_frame: int,
         block_q: int = 0, block_k: int = 0):
    """Frame-aligned active-block list (host). Returns (PlanInfo, row_ptr, col_idx)
    with numpy int32 arrays."""
    L = lib()
    info = PlanInfo()
    _check(L.fsa_plan(frames, tokens_per_frame, window, ref_frame, block_q, block_k,
                      ctypes.byref(info), None, 0, None, 0))
    row_ptr = np.zeros(info.n_qblocks + 1, dtype=np.int32)
    col_idx = np.zeros(max(info.nnz, 1), dtype=np.int32)
    _check(L.fsa_plan(frames, tokens_per_frame, window, ref_frame, block_q, block_k,
                      ctypes.byref(info), row_ptr.ctypes.data_as(_I32P), row_ptr.size,
                      col_idx.ctypes.data_as(_I32P), col_idx.size))
    return info, row_ptr, col_idx[:info.nnz]


# ----------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_qkv(name, t, shape=None):
    torch = _torch()
    if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor [B, H, N, D]")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_buf(name, t, dtype, shape, device):
    """A caller-supplied device buffer must be contiguous, of the dtype and
    shape the library indexes it with, and on the tensors' device: the C ABI
    takes plain pointers and cannot tell an undersized buffer."""
    if (t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous()
            or t.device != device):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on "
                         f"{device}; got {t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def _check_plan(dplan, q):
    """The plan must describe q's sequence, and its CSR must sit on q's device."""
    torch = _torch()
    info = dplan.info
    n = q.shape[2]
    if n != info.seq_len:
        raise ValueError(f"q has {n} tokens per head but the plan covers {info.seq_len}")
    _check_buf("plan row_ptr", dplan.row_ptr, torch.int32, (info.n_qblocks + 1,), q.device)
    _check_buf("plan col_idx", dplan.col_idx, torch.int32, (info.nnz,), q.device)


class DevicePlan:
    """A plan plus device copies of its CSR arrays (allocated by torch)."""

    def __init__(self, frames, tokens_per_frame, window, ref_frame, block_q=0, block_k=0,
                 device="cuda"):
        torch = _torch()
        self.info, self.row_ptr_host, self.col_idx_host = plan(
            frames, tokens_per_frame, window, ref_frame, block_q, block_k)
        self.row_ptr = torch.from_numpy(self.row_ptr_host).to(device)
        self.col_idx = torch.from_numpy(np.ascontiguousarray(self.col_idx_host)).to(device)


def bounds(dplan: DevicePlan, q, k, scale: float, bound_limit: float = 0.0,
           head_offset: int = 0, head_count: int = 0,
           qnorm=None, kmax=None, eligible=None, bmax=None, stream=None,
           kmean=None, center: bool = False):
    """fsa_bounds. Returns (qnorm fp32 [B,H,N], kmax fp32 [B,H,n_kb],
    eligible int32 [B,H], bmax fp32 [B,H], kmean fp32 [B,H,D] or None).
    Keys are mean-centred when ``center`` is set or a ``kmean`` buffer is given."""
    torch = _torch()
    _check_qkv("q", q)
    _check_qkv("k", k, q.shape)
    _check_plan(dplan, q)
    bsz, heads, n, d = q.shape
    info = dplan.info
    dev = q.device
    if k.device != dev:
        raise ValueError(f"k is on {k.device}, q on {dev}")
    if qnorm is None:
        qnorm = torch.empty((bsz, heads, n), dtype=torch.float32, device=dev)
    if kmax is None:
        kmax = torch.empty((bsz, heads, info.n_kblocks), dtype=torch.float32, device=dev)
    if eligible is None:
        eligible = torch.empty((bsz, heads), dtype=torch.int32, device=dev)
    if bmax is None:
        bmax = torch.empty((bsz, heads), dtype=torch.float32, device=dev)
    if center and kmean is None:
        kmean = torch.empty((bsz, heads, d), dtype=torch.float32, device=dev)
    _check_buf("qnorm", qnorm, torch.float32, (bsz, heads, n), dev)
    _check_buf("kmax", kmax, torch.float32, (bsz, heads, info.n_kblocks), dev)
    _check_buf("eligible", eligible, torch.int32, (bsz, heads), dev)
    _check_buf("bmax", bmax, torch.float32, (bsz, heads), dev)
    if kmean is not None:
        _check_buf("kmean", kmean, torch.float32, (bsz, heads, d), dev)
    _check(lib().fsa_bounds(ctypes.byref(info), _ptr(dplan.row_ptr), _ptr(dplan.col_idx),
                            _ptr(q), _ptr(k), bsz, heads, d, head_offset, head_count,
                            float(scale), float(bound_limit), _ptr(qnorm), _ptr(kmax),
                            _ptr(eligible), _ptr(bmax), _ptr(kmean), _stream_handle(stream)))
    return qnorm, kmax, eligible, bmax, kmean


def attention(dplan: DevicePlan, q, k, v, qnorm, kmax, eligible, scale: float,
              head_offset: int = 0, head_count: int = 0, out=None, stream=None, kmean=None):
    """fsa_attention. Returns o (bf16 [B,H,N,D]). ``kmean`` is the key mean of a
    centred fsa_bounds call, or None."""
    torch = _torch()
    _check_qkv("q", q)
    _check_qkv("k", k, q.shape)
    _check_qkv("v", v, q.shape)
    _check_plan(dplan, q)
    bsz, heads, n, d = q.shape
    info = dplan.info
    dev = q.device
    for name, t in (("k", k), ("v", v)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
    _check_buf("qnorm", qnorm, torch.float32, (bsz, heads, n), dev)
    _check_buf("kmax", kmax, torch.float32, (bsz, heads, info.n_kblocks), dev)
    _check_buf("eligible", eligible, torch.int32, (bsz, heads), dev)
    if kmean is not None:
        _check_buf("kmean", kmean, torch.float32, (bsz, heads, d), dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_qkv("out", out, q.shape)
        if out.device != dev:
            raise ValueError(f"out is on {out.device}, q on {dev}")
    _check(lib().fsa_attention(ctypes.byref(info), _ptr(dplan.row_ptr), _ptr(dplan.col_idx),
                               _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(qnorm), _ptr(kmax),
                               _ptr(eligible), _ptr(kmean), bsz, heads, d, float(scale), head_offset,
                               head_count, _stream_handle(stream)))
    return out


def forward(dplan: DevicePlan, q, k, v, scale: float, bound_limit: float = 0.0,
            head_offset: int = 0, head_count: int = 0, out=None, stream=None,
            center: bool = False):
    """fsa_bounds then fsa_attention on the same stream. Returns (o, bounds tuple)."""
    b = bounds(dplan, q, k, scale, bound_limit, head_offset, head_count, stream=stream,
               center=center)
    o = attention(dplan, q, k, v, b[0], b[1], b[2], scale, head_offset, head_count,
                  out=out, stream=stream, kmean=b[4])
    return o, b


def pre_attention(x, w_qkv, heads: int, head_dim: int, eps: float = 1e-6,
                  rope_base: float = 10000.0, q=None, k=None, v=None, stream=None):
    """fsa_pre_attention: x bf16 [B, N, C], w_qkv bf16 [3 H D, C] (a norm gain
    already folded in) -> (q, k, v), each bf16 [B, H, N, D]."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 3 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous bf16 CUDA tensor [B, N, C]")
    bsz, n, c = x.shape
    if (w_qkv.dtype != torch.bfloat16 or tuple(w_qkv.shape) != (3 * heads * head_dim, c)
            or not w_qkv.is_contiguous()):
        raise ValueError("w_qkv must be a contiguous bf16 tensor [3 H D, C]")
    if w_qkv.device != x.device:
        raise ValueError(f"w_qkv is on {w_qkv.device}, x on {x.device}")
    outs = []
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            t = torch.empty((bsz, heads, n, head_dim), dtype=torch.bfloat16, device=x.device)
        else:
            _check_qkv(name, t, (bsz, heads, n, head_dim))
            if t.device != x.device:
                raise ValueError(f"{name} is on {t.device}, x on {x.device}")
        outs.append(t)
    _check(lib().fsa_pre_attention(_ptr(x), _ptr(w_qkv), bsz, n, c, heads, head_dim,
                                   float(eps), float(rope_base), _ptr(outs[0]), _ptr(outs[1]),
                                   _ptr(outs[2]), _stream_handle(stream)))
    return tuple(outs)
