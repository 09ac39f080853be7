"""Exact tiled attention for AMD MI355X (gfx950): Python binding of libfa.so.

The functions fa_fwd, fa_fwd_window, fa_fwd_splitkv,
fa_fwd_splitkv_workspace_bytes, fa_fwd_alibi, fa_bwd, fa_bwd_window,
fa_bwd_alibi, fa_bwd_noalloc, fa_bwd_workspace_bytes and fa_status_string
mirror the C ABI in include/fa.h one for one; this module only marshals
arguments (device pointers, sizes, the current HIP stream).  Every step of the computation runs in the library's HIP
kernels; there is no fallback path, and importing this package fails if
libfa.so has not been built.

Convenience wrappers attention_fwd / attention_bwd allocate the outputs with
torch on the inputs' device and call the same entry points.
"""
import ctypes
import math
import os

__all__ = ["fa_fwd", "fa_fwd_window", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_bytes",
           "fa_fwd_alibi", "fa_bwd_alibi", "fa_bwd", "fa_bwd_window", "fa_bwd_noalloc",
           "fa_bwd_workspace_bytes", "fa_status_string", "FAError",
           "attention_fwd", "attention_bwd", "LIB_PATH", "STATUS", "MAX_SPLITS",
           "NOALLOC_MAX_WORKSPACE", "BWD_ATOMIC", "BWD_SEPARATE", "BWD_ORDERED",
           "BWD_ATOMIC_PAIRED"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

MAX_SPLITS = 64  # FA_MAX_SPLITS
NOALLOC_MAX_WORKSPACE = 32 << 20  # FA_NOALLOC_MAX_WORKSPACE (bytes)

# dQ modes of fa_bwd's `deterministic` argument (FA_BWD_ATOMIC, FA_BWD_SEPARATE,
# FA_BWD_ORDERED, FA_BWD_ATOMIC_PAIRED); False and True select the first two.
BWD_ATOMIC, BWD_SEPARATE, BWD_ORDERED, BWD_ATOMIC_PAIRED = 0, 1, 2, 3

STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED",
          4: "FA_ERR_ALIGN", 5: "FA_ERR_WORKSPACE", 6: "FA_ERR_HIP"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950) first")

# torch ships its own HIP runtime (libamdhip64.so.7).  Loading torch first makes
# libfa.so's dependency on that soname resolve to the same runtime, so the
# library launches on torch's streams and sees torch's allocations; loading
# libfa.so first would bring a second HIP runtime into the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_vp, _fp = ctypes.c_void_p, ctypes.c_void_p
_i, _f, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_lib.fa_fwd.argtypes = [_vp, _vp, _vp, _fp, _fp, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.fa_fwd.restype = _i
_lib.fa_fwd_window.argtypes = [_vp, _vp, _vp, _fp, _fp, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.fa_fwd_window.restype = _i
_lib.fa_bwd_window.argtypes = [_vp, _vp, _vp, _fp, _fp, _vp, _fp, _fp, _fp, _i, _i, _i, _i, _i,
                               _f, _i, _i, _vp, _sz, _vp]
_lib.fa_bwd_window.restype = _i
_lib.fa_fwd_splitkv.argtypes = [_vp, _vp, _vp, _fp, _fp, _i, _i, _i, _i, _i, _f, _i, _i, _vp,
                                _sz, _vp]
_lib.fa_fwd_splitkv.restype = _i
_lib.fa_fwd_splitkv_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.fa_fwd_splitkv_workspace_bytes.restype = _sz
_lib.fa_bwd.argtypes = [_vp, _vp, _vp, _fp, _fp, _vp, _fp, _fp, _fp, _i, _i, _i, _i, _i, _f,
                        _i, _i, _vp, _sz, _vp]
_lib.fa_bwd.restype = _i
_lib.fa_bwd_noalloc.argtypes = [_vp, _vp, _vp, _fp, _fp, _vp, _fp, _fp, _fp, _i, _i, _i, _i, _i,
                                _f, _i, _i, _vp]
_lib.fa_bwd_noalloc.restype = _i
_lib.fa_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.fa_bwd_workspace_bytes.restype = _sz
_lib.fa_fwd_alibi.argtypes = [_vp, _vp, _vp, _fp, _fp, _fp, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.fa_fwd_alibi.restype = _i
_lib.fa_bwd_alibi.argtypes = [_vp, _vp, _vp, _fp, _fp, _vp, _fp, _fp, _fp, _fp, _i, _i, _i, _i,
                              _i, _f, _i, _i, _vp, _sz, _vp]
_lib.fa_bwd_alibi.restype = _i
_lib.fa_status_string.argtypes = [_i]
_lib.fa_status_string.restype = ctypes.c_char_p


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)}")


def _addr(x):
    """Device (or host) address of a tensor, or an integer address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(int(status)).decode()


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, stream=None) -> int:
    """C ABI fa_fwd.  Tensors (or integer device addresses) in, status out."""
    return _lib.fa_fwd(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), B, Hq, Hkv, N, d,
                       float(scale), int(bool(causal)), _stream(stream, q, o))


def fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, window, stream=None) -> int:
    """C ABI fa_fwd_window (causal sliding window).  Status out."""
    return _lib.fa_fwd_window(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), B, Hq, Hkv, N,
                              d, float(scale), int(window), _stream(stream, q, o))


def fa_bwd_window(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, window,
                  deterministic, workspace, workspace_bytes, stream=None) -> int:
    """C ABI fa_bwd_window (causal sliding window).  Status out."""
    return _lib.fa_bwd_window(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), _addr(dout),
                              _addr(dq), _addr(dk), _addr(dv), B, Hq, Hkv, N, d, float(scale),
                              int(window), int(deterministic), _addr(workspace),
                              int(workspace_bytes), _stream(stream, q, dq))


def fa_fwd_alibi(q, k, v, o, lse, slopes, B, Hq, Hkv, N, d, scale, causal, stream=None) -> int:
    """C ABI fa_fwd_alibi (linear position bias; slopes fp32 [Hq] on the device).  Status out."""
    return _lib.fa_fwd_alibi(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), _addr(slopes),
                             B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
                             _stream(stream, q, o))


def fa_bwd_alibi(q, k, v, o, lse, dout, dq, dk, dv, slopes, B, Hq, Hkv, N, d, scale, causal,
                 deterministic, workspace, workspace_bytes, stream=None) -> int:
    """C ABI fa_bwd_alibi.  Status out."""
    return _lib.fa_bwd_alibi(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), _addr(dout),
                             _addr(dq), _addr(dk), _addr(dv), _addr(slopes), B, Hq, Hkv, N, d,
                             float(scale), int(bool(causal)), int(deterministic),
                             _addr(workspace), int(workspace_bytes), _stream(stream, q, dq))


def fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, num_splits, workspace,
                   workspace_bytes, stream=None) -> int:
    """C ABI fa_fwd_splitkv.  Tensors (or integer device addresses) in, status out."""
    return _lib.fa_fwd_splitkv(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), B, Hq, Hkv,
                               N, d, float(scale), int(bool(causal)), int(num_splits),
                               _addr(workspace), int(workspace_bytes), _stream(stream, q, o))


def fa_fwd_splitkv_workspace_bytes(B, Hq, Hkv, N, d, num_splits) -> int:
    return int(_lib.fa_fwd_splitkv_workspace_bytes(B, Hq, Hkv, N, d, int(num_splits)))


def fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, deterministic) -> int:
    return int(_lib.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, int(deterministic)))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, deterministic,
           workspace, workspace_bytes, stream=None) -> int:
    """C ABI fa_bwd.  Tensors (or integer device addresses) in, status out."""
    return _lib.fa_bwd(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), _addr(dout),
                       _addr(dq), _addr(dk), _addr(dv), B, Hq, Hkv, N, d, float(scale),
                       int(bool(causal)), int(deterministic), _addr(workspace),
                       int(workspace_bytes), _stream(stream, q, dq))


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal,
                   deterministic, stream=None) -> int:
    """C ABI fa_bwd_noalloc (workspace in the library's static device array).
    Status out."""
    return _lib.fa_bwd_noalloc(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), _addr(dout),
                               _addr(dq), _addr(dk), _addr(dv), B, Hq, Hkv, N, d, float(scale),
                               int(bool(causal)), int(deterministic), _stream(stream, q, dq))


def _dims(q, k):
    B, Hq, N, d = q.shape
    return B, Hq, k.shape[1], N, d


def _check_inputs(*ts):
    import torch
    for t in ts:
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("q/k/v/dout must be contiguous bfloat16 [B, H, N, d] tensors")


def attention_fwd(q, k, v, scale=None, causal=False, o=None, lse=None, stream=None,
                  num_splits=1, workspace=None):
    """Forward attention on device tensors.  Returns (o fp32, lse fp32).
    num_splits > 1 runs the split-KV forward (fa_fwd_splitkv)."""
    import torch
    _check_inputs(q, k, v)
    B, Hq, Hkv, N, d = _dims(q, k)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if o is None:
        o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if num_splits == 1:
        st = fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, stream)
        if st:
            raise FAError(st, "fa_fwd")
        return o, lse
    need = fa_fwd_splitkv_workspace_bytes(B, Hq, Hkv, N, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, num_splits, workspace,
                        workspace.numel() * workspace.element_size(), stream)
    if st:
        raise FAError(st, "fa_fwd_splitkv")
    return o, lse


def attention_bwd(q, k, v, o, lse, dout, scale=None, causal=False, deterministic=False,
                  dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward attention on device tensors.  Returns (dq, dk, dv) fp32.
    deterministic: BWD_ATOMIC (False), BWD_SEPARATE (True), BWD_ORDERED or
    BWD_ATOMIC_PAIRED."""
    import torch
    _check_inputs(q, k, v, dout)
    B, Hq, Hkv, N, d = _dims(q, k)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dev = q.device
    dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev) if dv is None else dv
    need = fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, deterministic)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal,
                deterministic, workspace, workspace.numel() * workspace.element_size(), stream)
    if st:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv
