"""Python binding of libfa.so, the gfx950 exact IO-aware attention library.

Argument marshalling only: every step of the forward and backward runs in
the HIP kernels behind the C ABI declared in include/fa.h. torch supplies
device memory and streams. There is no fallback: if libfa.so is missing or
fails to load, importing this package raises.

Functions carry the C names:
    fa_fwd(Q, K, V, O, LSE, scale, causal=False, blockmask=None, stream=None)
    fa_bwd(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, causal=False,
           blockmask=None, workspace=None, stream=None)
    fa_fwd_f32(...), fa_bwd_f32(...)  -- the fp32 debug path, same arguments
    fa_bwd_workspace_bytes(B, H, N, d)
    fa_bwd_noalloc(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, causal=False,
                   blockmask=None, stream=None)  -- scratch in the library's static
                   device array (FA_NOALLOC_SCRATCH_BYTES per GPU), no workspace
    fa_fwd_dropout(Q, K, V, O, LSE, scale, p_drop, seed, causal=False, blockmask=None,
                   stream=None)
    fa_bwd_dropout(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, p_drop, seed, causal=False,
                   blockmask=None, workspace=None, stream=None)
    fa_fwd_fp8(Q8, K8, V8, O, LSE, scale, q_descale, k_descale, v_descale,
               causal=False, workspace=None, stream=None)
    fa_fwd_fp8_workspace_bytes(B, H, N, d)
    fa_decode(Q, K, V, O, LSE, scale, causal=False, workspace=None, stream=None)
    fa_decode_workspace_bytes(B, H, Nq, Nk, d)
Tensors are contiguous CUDA (HIP) tensors of shape [B, H, N, d]: bfloat16 for
fa_fwd / fa_bwd, float32 for the _f32 entry points; LSE is float32 [B, H, N];
blockmask is uint8 [ceil(N/128), ceil(N/128)] on the same device, or None.
Every tensor (LSE, blockmask and workspaces included) must be a contiguous
device tensor on Q's device; a workspace must hold at least the bytes its
*_workspace_bytes function returns. These checks raise ValueError before any
launch.
fa_decode takes Q, O of shape [B, H, Nq, d] and K, V of shape [B, H, Nk, d]
(bfloat16), LSE float32 [B, H, Nq].
"""
import ctypes
import os

# torch first: it loads its own HIP runtime, and libfa.so must bind to that
# same runtime (two HIP runtimes in one process do not share the device).
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python exact_io_aware_attention_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

FA_OK = 0
FA_MASK_BLOCK = 128
FA_NOALLOC_SCRATCH_BYTES = 16 << 20  # include/fa.h
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADDIM",
                4: "FA_ERR_ALIGN", 5: "FA_ERR_SCALE", 6: "FA_ERR_WORKSPACE", 7: "FA_ERR_HIP",
                8: "FA_ERR_SCRATCH"}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_lib.fa_fwd.restype = _i
_lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp]
_lib.fa_fwd_f32.restype = _i
_lib.fa_fwd_f32.argtypes = _lib.fa_fwd.argtypes
_lib.fa_bwd.restype = _i
_lib.fa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                        _i, _i, _i, _i, _f, _i, _vp, _vp, _sz, _vp]
_lib.fa_bwd_f32.restype = _i
_lib.fa_bwd_f32.argtypes = _lib.fa_bwd.argtypes
_lib.fa_bwd_noalloc.restype = _i
_lib.fa_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _i, _i, _i, _i, _f, _i, _vp, _vp]
_lib.fa_bwd_prep.restype = _i
_lib.fa_bwd_prep.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]
_lib.fa_bwd_dq.restype = _i
_lib.fa_bwd_dq.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _sz, _vp]
_lib.fa_bwd_dkdv.restype = _i
_lib.fa_bwd_dkdv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp,
                             _sz, _vp]
_lib.fa_bwd_workspace_bytes.restype = _sz
_lib.fa_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i]
_lib.fa_fwd_dropout.restype = _i
_lib.fa_fwd_dropout.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _f,
                                ctypes.c_ulonglong, _vp]
_lib.fa_bwd_dropout.restype = _i
_lib.fa_bwd_dropout.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f,
                                _i, _vp, _f, ctypes.c_ulonglong, _vp, _sz, _vp]
_lib.fa_fwd_fp8.restype = _i
_lib.fa_fwd_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _f, _f, _f, _i, _vp,
                            _sz, _vp]
_lib.fa_fwd_fp8_workspace_bytes.restype = _sz
_lib.fa_fwd_fp8_workspace_bytes.argtypes = [_i, _i, _i, _i]
_lib.fa_decode.restype = _i
_lib.fa_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]
_lib.fa_decode_workspace_bytes.restype = _sz
_lib.fa_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
_lib.fa_status_str.restype = ctypes.c_char_p
_lib.fa_status_str.argtypes = [_i]
_lib.fa_last_hip_error.restype = ctypes.c_char_p
_lib.fa_last_hip_error.argtypes = []
_lib.fa_version.restype = ctypes.c_char_p
_lib.fa_version.argtypes = []

# Symbols declared in include/fa.h (checked by the ABI test).
EXPORTED = ("fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_prep", "fa_bwd_dq", "fa_bwd_dkdv",
            "fa_fwd_f32", "fa_bwd_f32", "fa_bwd_workspace_bytes", "fa_fwd_dropout", "fa_bwd_dropout",
            "fa_fwd_fp8", "fa_fwd_fp8_workspace_bytes", "fa_decode", "fa_decode_workspace_bytes",
            "fa_status_str", "fa_last_hip_error", "fa_version")


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = f"{STATUS_NAMES.get(status, status)}: {_lib.fa_status_str(status).decode()}"
        if status == 7:
            msg += f" ({_lib.fa_last_hip_error().decode()})"
        super().__init__(msg)


def lib():
    """The loaded ctypes library (raw pointer-level access)."""
    return _lib


def version() -> str:
    return _lib.fa_version().decode()


def _check(status: int):
    if status != FA_OK:
        raise FaError(status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _shape(q):
    if q.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    return tuple(int(x) for x in q.shape)


def _require(ts, dtype, shape):
    dev0 = ts[0].device
    for t in ts:
        if (t.dtype != dtype or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda
                or t.device != dev0):
            raise ValueError(f"expected contiguous {dtype} tensors of shape {shape} on one device")


def _on(t, device):
    """Whether t lives on `device` (the device of the main tensors)."""
    return t.is_cuda and t.device == device


def _require_lse(lse, shape, device):
    import torch
    B, H, N, _ = shape
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous()
            or not _on(lse, device)):
        raise ValueError(f"LSE must be a contiguous float32 tensor of shape {(B, H, N)} on {device}")


def _require_mask(mask, N, device):
    import torch
    if mask is None:
        return
    nb = (N + FA_MASK_BLOCK - 1) // FA_MASK_BLOCK
    if (mask.dtype != torch.uint8 or tuple(mask.shape) != (nb, nb) or not mask.is_contiguous()
            or not _on(mask, device)):
        raise ValueError(f"blockmask must be a contiguous uint8 tensor of shape {(nb, nb)} on {device}")


def _require_ws(ws, need, device):
    """A caller's workspace: contiguous, on `device`, at least `need` bytes.
    Returns its size in bytes."""
    nbytes = ws.numel() * ws.element_size()
    if not ws.is_contiguous() or not _on(ws, device) or nbytes < need:
        raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes on {device}")
    return nbytes


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.fa_bwd_workspace_bytes(B, H, N, d))


def _fwd(fn, dtype, Q, K, V, O, LSE, scale, causal, blockmask, stream):
    shape = _shape(Q)
    _require((Q, K, V, O), dtype, shape)
    _require_lse(LSE, shape, Q.device)
    _require_mask(blockmask, shape[2], Q.device)
    B, H, N, d = shape
    _check(fn(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, H, N, d, float(scale),
              int(bool(causal)), _ptr(blockmask), _stream_ptr(stream)))


def _workspace(need, workspace, device):
    """The caller's workspace after its checks, or a new one of `need` bytes;
    returns (tensor, bytes)."""
    import torch
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, _require_ws(workspace, need, device)


def _bwd(fn, dtype, dO, Q, K, V, O, LSE, dQ, dK, dV, scale, causal, blockmask, workspace,
         stream):
    shape = _shape(Q)
    _require((dO, Q, K, V, O, dQ, dK, dV), dtype, shape)
    _require_lse(LSE, shape, Q.device)
    _require_mask(blockmask, shape[2], Q.device)
    ws, nbytes = _workspace(fa_bwd_workspace_bytes(*shape), workspace, Q.device)
    B, H, N, d = shape
    _check(fn(_ptr(dO), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), _ptr(dQ), _ptr(dK),
              _ptr(dV), B, H, N, d, float(scale), int(bool(causal)), _ptr(blockmask),
              _ptr(ws), nbytes, _stream_ptr(stream)))


def fa_fwd(Q, K, V, O, LSE, scale, causal=False, blockmask=None, stream=None):
    """Forward, bf16: writes O and LSE in place."""
    import torch
    _fwd(_lib.fa_fwd, torch.bfloat16, Q, K, V, O, LSE, scale, causal, blockmask, stream)


def fa_fwd_f32(Q, K, V, O, LSE, scale, causal=False, blockmask=None, stream=None):
    """Forward, fp32 debug path: writes O and LSE in place."""
    import torch
    _fwd(_lib.fa_fwd_f32, torch.float32, Q, K, V, O, LSE, scale, causal, blockmask, stream)


def fa_bwd(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, causal=False, blockmask=None,
           workspace=None, stream=None):
    """Backward, bf16: writes dQ, dK, dV in place."""
    import torch
    _bwd(_lib.fa_bwd, torch.bfloat16, dO, Q, K, V, O, LSE, dQ, dK, dV, scale, causal,
         blockmask, workspace, stream)


def fa_bwd_f32(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, causal=False, blockmask=None,
               workspace=None, stream=None):
    """Backward, fp32 debug path: writes dQ, dK, dV in place."""
    import torch
    _bwd(_lib.fa_bwd_f32, torch.float32, dO, Q, K, V, O, LSE, dQ, dK, dV, scale, causal,
         blockmask, workspace, stream)


def fa_bwd_noalloc(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, causal=False, blockmask=None,
                   stream=None):
    """Backward, bf16, with its scratch in the library's static device array
    instead of a workspace (allocates nothing): writes dQ, dK, dV in place.
    Calls on one GPU must not overlap in time (they share that array)."""
    shape = _shape(Q)
    _require((dO, Q, K, V, O, dQ, dK, dV), torch.bfloat16, shape)
    _require_lse(LSE, shape, Q.device)
    _require_mask(blockmask, shape[2], Q.device)
    B, H, N, d = shape
    _check(_lib.fa_bwd_noalloc(_ptr(dO), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), _ptr(dQ),
                               _ptr(dK), _ptr(dV), B, H, N, d, float(scale), int(bool(causal)),
                               _ptr(blockmask), _stream_ptr(stream)))


def fa_bwd_prep(dO, O, LSE, workspace, stream=None):
    """Backward phase 1: D and LSE*log2(e) into the workspace."""
    shape = _shape(dO)
    _require((dO, O), torch.bfloat16, shape)
    _require_lse(LSE, shape, dO.device)
    nbytes = _require_ws(workspace, fa_bwd_workspace_bytes(*shape), dO.device)
    B, H, N, d = shape
    _check(_lib.fa_bwd_prep(_ptr(dO), _ptr(O), _ptr(LSE), B, H, N, d, _ptr(workspace),
                            nbytes, _stream_ptr(stream)))


def fa_bwd_dq(dO, Q, K, V, dQ, scale, workspace, causal=False, blockmask=None, stream=None):
    """Backward phase 2: dQ (needs fa_bwd_prep's workspace)."""
    shape = _shape(Q)
    _require((dO, Q, K, V, dQ), torch.bfloat16, shape)
    _require_mask(blockmask, shape[2], Q.device)
    nbytes = _require_ws(workspace, fa_bwd_workspace_bytes(*shape), Q.device)
    B, H, N, d = shape
    _check(_lib.fa_bwd_dq(_ptr(dO), _ptr(Q), _ptr(K), _ptr(V), _ptr(dQ), B, H, N, d,
                          float(scale), int(bool(causal)), _ptr(blockmask), _ptr(workspace),
                          nbytes, _stream_ptr(stream)))


def fa_bwd_dkdv(dO, Q, K, V, dK, dV, scale, workspace, causal=False, blockmask=None,
                stream=None):
    """Backward phase 3: dK and dV (needs fa_bwd_prep's workspace)."""
    shape = _shape(Q)
    _require((dO, Q, K, V, dK, dV), torch.bfloat16, shape)
    _require_mask(blockmask, shape[2], Q.device)
    nbytes = _require_ws(workspace, fa_bwd_workspace_bytes(*shape), Q.device)
    B, H, N, d = shape
    _check(_lib.fa_bwd_dkdv(_ptr(dO), _ptr(Q), _ptr(K), _ptr(V), _ptr(dK), _ptr(dV), B, H, N,
                            d, float(scale), int(bool(causal)), _ptr(blockmask),
                            _ptr(workspace), nbytes, _stream_ptr(stream)))


def new_workspace(B, H, N, d, device="cuda"):
    """A device buffer of fa_bwd_workspace_bytes (torch allocates it)."""
    return torch.empty(max(fa_bwd_workspace_bytes(B, H, N, d), 1), dtype=torch.uint8,
                       device=device)


def fa_decode_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(_lib.fa_decode_workspace_bytes(B, H, Nq, Nk, d))


def fa_decode(Q, K, V, O, LSE, scale, causal=False, workspace=None, stream=None):
    """Decode-shaped forward, bf16: Q, O [B, H, Nq, d]; K, V [B, H, Nk, d];
    writes O and LSE [B, H, Nq] in place."""
    import torch
    qs, ks = _shape(Q), _shape(K)
    if qs[:2] != ks[:2] or qs[3] != ks[3]:
        raise ValueError("Q [B, H, Nq, d] and K, V [B, H, Nk, d] must agree on B, H, d")
    _require((Q, O), torch.bfloat16, qs)
    _require((K, V), torch.bfloat16, ks)
    if K.device != Q.device or V.device != Q.device:
        raise ValueError("Q, K, V, O must be on one device")
    _require_lse(LSE, qs, Q.device)
    B, H, Nq, d = qs
    Nk = ks[2]
    workspace, nbytes = _workspace(fa_decode_workspace_bytes(B, H, Nq, Nk, d), workspace, Q.device)
    _check(_lib.fa_decode(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, H, Nq, Nk, d,
                          float(scale), int(bool(causal)), _ptr(workspace), nbytes,
                          _stream_ptr(stream)))


def fa_fwd_dropout(Q, K, V, O, LSE, scale, p_drop, seed, causal=False, blockmask=None,
                   stream=None):
    """Forward with dropout on P, bf16: writes O and LSE in place."""
    import torch
    shape = _shape(Q)
    _require((Q, K, V, O), torch.bfloat16, shape)
    _require_lse(LSE, shape, Q.device)
    _require_mask(blockmask, shape[2], Q.device)
    B, H, N, d = shape
    _check(_lib.fa_fwd_dropout(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, H, N, d,
                               float(scale), int(bool(causal)), _ptr(blockmask), float(p_drop),
                               int(seed), _stream_ptr(stream)))


def fa_bwd_dropout(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, p_drop, seed, causal=False,
                   blockmask=None, workspace=None, stream=None):
    """Backward of fa_fwd_dropout, bf16: writes dQ, dK, dV in place."""
    import torch
    shape = _shape(Q)
    _require((dO, Q, K, V, O, dQ, dK, dV), torch.bfloat16, shape)
    _require_lse(LSE, shape, Q.device)
    _require_mask(blockmask, shape[2], Q.device)
    ws, nbytes = _workspace(fa_bwd_workspace_bytes(*shape), workspace, Q.device)
    B, H, N, d = shape
    _check(_lib.fa_bwd_dropout(_ptr(dO), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), _ptr(dQ),
                               _ptr(dK), _ptr(dV), B, H, N, d, float(scale), int(bool(causal)),
                               _ptr(blockmask), float(p_drop), int(seed), _ptr(ws), nbytes,
                               _stream_ptr(stream)))


def fa_fwd_fp8_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.fa_fwd_fp8_workspace_bytes(B, H, N, d))


def fa_fwd_fp8(Q8, K8, V8, O, LSE, scale, q_descale, k_descale, v_descale, causal=False,
               workspace=None, stream=None):
    """FP8 forward: Q8, K8, V8 contiguous uint8 E4M3 codes [B, H, N, d] (value =
    code * descale); writes O (bfloat16) and LSE in place."""
    import torch
    shape = _shape(Q8)
    _require((Q8, K8, V8), torch.uint8, shape)
    _require((O,), torch.bfloat16, shape)
    if any(t.device != Q8.device for t in (K8, V8, O)):
        raise ValueError("Q8, K8, V8, O must be on one device")
    _require_lse(LSE, shape, Q8.device)
    B, H, N, d = shape
    workspace, nbytes = _workspace(fa_fwd_fp8_workspace_bytes(B, H, N, d), workspace, Q8.device)
    _check(_lib.fa_fwd_fp8(_ptr(Q8), _ptr(K8), _ptr(V8), _ptr(O), _ptr(LSE), B, H, N, d,
                           float(scale), float(q_descale), float(k_descale), float(v_descale),
                           int(bool(causal)), _ptr(workspace), nbytes, _stream_ptr(stream)))
