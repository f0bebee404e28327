"""ctypes view of ``libstreamkl.so`` (the C ABI in ``include/streamkl.h``).

Argument marshalling only.  The library must have been built (see
``build_lib.py``); loading fails loudly otherwise -- there is no fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstreamkl.so")
# The same sources built with -DSTREAMKL_DEBUG (bounds-checked accesses,
# plus streamkl_debug_take); tests load it with load(DEBUG_LIB_PATH).
DEBUG_LIB_PATH = os.path.join(HERE, "libstreamkl_debug.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, BF16 = 0, 1
GRAD_Q1K1, GRAD_Q2K2, GRAD_ALL = 1, 2, 3

NOALLOC_SCRATCH_BYTES = 16 << 20   # STREAMKL_NOALLOC_SCRATCH_BYTES

EXPORTS = ("streamkl_fwd", "streamkl_fwd_splits", "streamkl_fwd_workspace_size", "streamkl_fwd_splitk",
           "streamkl_fwd_splitk_noalloc",
           "streamkl_bwd", "streamkl_bwd_dq", "streamkl_bwd_dq_ws", "streamkl_bwd_dk", "streamkl_bwd_dk_ws",
           "streamkl_bwd_workspace_size", "streamkl_bwd_fused", "streamkl_bwd_fused_workspace_size",
           "streamkl_bwd_fused_selected", "streamkl_status_str", "streamkl_abi_version")


class StreamKLError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where} failed: {status_str(status)} ({status})")


_lib = None
_vp, _fp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def load(path: str = None):
    """Open the library (once) and declare the exported signatures.  ``path``
    defaults to LIB_PATH, read at the call (so a test can point the binding
    at another build of the same sources)."""
    global _lib
    if path is None:
        path = LIB_PATH
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    lib.streamkl_fwd.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i,
                                 _fp, _fp, _fp, _vp]
    lib.streamkl_fwd.restype = _i
    lib.streamkl_fwd_splits.argtypes = [_i, _i, _i, _i, _i, _i, _i]
    lib.streamkl_fwd_splits.restype = _i
    lib.streamkl_fwd_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
    lib.streamkl_fwd_workspace_size.restype = _sz
    lib.streamkl_fwd_splitk.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i,
                                        _fp, _fp, _fp, _vp, _sz, _vp]
    lib.streamkl_fwd_splitk.restype = _i
    lib.streamkl_fwd_splitk_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i,
                                                _fp, _fp, _fp, _vp]
    lib.streamkl_fwd_splitk_noalloc.restype = _i
    lib.streamkl_bwd.argtypes = [_vp, _vp, _vp, _vp, _fp, _fp, _fp, _fp, _i, _i, _i, _i, _i,
                                 _f, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.streamkl_bwd.restype = _i
    for name in ("streamkl_bwd_dq", "streamkl_bwd_dk"):
        fn = getattr(lib, name)
        fn.argtypes = [_vp, _vp, _vp, _vp, _fp, _fp, _fp, _fp, _i, _i, _i, _i, _i,
                       _f, _i, _i, _i, _vp, _vp, _vp]
        fn.restype = _i
    lib.streamkl_bwd_dq_ws.argtypes = [_vp, _vp, _vp, _vp, _fp, _fp, _fp, _fp, _i, _i, _i, _i, _i,
                                       _f, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]
    lib.streamkl_bwd_dq_ws.restype = _i
    lib.streamkl_bwd_dk_ws.argtypes = lib.streamkl_bwd_dq_ws.argtypes
    lib.streamkl_bwd_dk_ws.restype = _i
    lib.streamkl_bwd_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
    lib.streamkl_bwd_workspace_size.restype = _sz
    lib.streamkl_bwd_fused.argtypes = lib.streamkl_bwd.argtypes
    lib.streamkl_bwd_fused.restype = _i
    lib.streamkl_bwd_fused_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
    lib.streamkl_bwd_fused_workspace_size.restype = _sz
    lib.streamkl_bwd_fused_selected.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
    lib.streamkl_bwd_fused_selected.restype = _i
    lib.streamkl_status_str.argtypes = [_i]
    lib.streamkl_status_str.restype = ctypes.c_char_p
    lib.streamkl_abi_version.argtypes = []
    lib.streamkl_abi_version.restype = _i
    if hasattr(lib, "streamkl_debug_take"):  # debug builds only
        lib.streamkl_debug_take.argtypes = []
        lib.streamkl_debug_take.restype = ctypes.c_uint
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().streamkl_status_str(int(status)).decode()


def abi_version() -> int:
    return load().streamkl_abi_version()


def debug_take(lib) -> int:
    """streamkl_debug_take of a debug build ``lib`` (from load(DEBUG_LIB_PATH)):
    the first out-of-range access its kernels met since the last call, as
    (file << 16) | line, or 0; synchronises the device."""
    return int(lib.streamkl_debug_take())


def debug_site(code: int) -> str:
    """Readable form of a streamkl_debug_take code."""
    files = {1: "streamkl_fwd.hip", 2: "streamkl_bwd.h", 3: "streamkl_bwd_fused.hip"}
    if code == 0:
        return "none"
    if code == 0xFFFFFFFF:
        return "device not readable"
    return f"{files.get(code >> 16, f'file {code >> 16}')}:{code & 0xFFFF}"


def fwd(q1, k1, q2, k2, B, H, NQ, NK, d, scale, causal, dtype, kl, lse1, lse2, stream):
    """Raw call with integer addresses; returns the status code."""
    return load().streamkl_fwd(q1, k1, q2, k2, B, H, NQ, NK, d, scale, causal, dtype,
                               kl, lse1, lse2, stream)


def fwd_splits(B, H, NQ, NK, d, causal, dtype):
    """The library's choice of key partitions for the split-K forward (1 = none)."""
    return load().streamkl_fwd_splits(B, H, NQ, NK, d, causal, dtype)


def fwd_workspace_size(B, H, NQ, NK, d, causal, dtype, splits):
    return load().streamkl_fwd_workspace_size(B, H, NQ, NK, d, causal, dtype, splits)


def fwd_splitk(q1, k1, q2, k2, B, H, NQ, NK, d, scale, causal, dtype, splits, kl, lse1, lse2,
               workspace, workspace_bytes, stream):
    return load().streamkl_fwd_splitk(q1, k1, q2, k2, B, H, NQ, NK, d, scale, causal, dtype, splits,
                                      kl, lse1, lse2, workspace, workspace_bytes, stream)


def fwd_splitk_noalloc(q1, k1, q2, k2, B, H, NQ, NK, d, scale, causal, dtype, splits, kl, lse1, lse2, stream):
    """streamkl_fwd_splitk_noalloc: the split-K forward with the library's
    fixed device scratch array instead of a caller's workspace."""
    return load().streamkl_fwd_splitk_noalloc(q1, k1, q2, k2, B, H, NQ, NK, d, scale, causal, dtype, splits,
                                              kl, lse1, lse2, stream)


def bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale, causal, dtype, grad_mask,
        dq1, dk1, dq2, dk2, workspace, workspace_bytes, stream):
    return load().streamkl_bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale,
                               causal, dtype, grad_mask, dq1, dk1, dq2, dk2, workspace,
                               workspace_bytes, stream)


def bwd_half(which, q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale, causal, dtype,
             grad_mask, out1, out2, stream):
    """streamkl_bwd_dq (which='dq') or streamkl_bwd_dk (which='dk')."""
    fn = getattr(load(), f"streamkl_bwd_{which}")
    return fn(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale, causal, dtype, grad_mask,
              out1, out2, stream)


def bwd_dq_ws(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale, causal, dtype, grad_mask,
              dq1, dq2, workspace, workspace_bytes, stream):
    """streamkl_bwd_dq_ws: the query-gradient half with the backward's workspace."""
    return load().streamkl_bwd_dq_ws(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale, causal,
                                     dtype, grad_mask, dq1, dq2, workspace, workspace_bytes, stream)


def bwd_dk_ws(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale, causal, dtype, grad_mask,
              dk1, dk2, workspace, workspace_bytes, stream):
    """streamkl_bwd_dk_ws: the key-gradient half with the backward's workspace."""
    return load().streamkl_bwd_dk_ws(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale, causal,
                                     dtype, grad_mask, dk1, dk2, workspace, workspace_bytes, stream)


def bwd_workspace_size(B, H, NQ, NK, d, causal, dtype, grad_mask):
    return load().streamkl_bwd_workspace_size(B, H, NQ, NK, d, causal, dtype, grad_mask)


def bwd_fused(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale, causal, dtype, grad_mask,
              dq1, dk1, dq2, dk2, workspace, workspace_bytes, stream):
    """streamkl_bwd_fused: the single-pass backward with atomic query gradients."""
    return load().streamkl_bwd_fused(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, NQ, NK, d, scale, causal, dtype,
                                     grad_mask, dq1, dk1, dq2, dk2, workspace, workspace_bytes, stream)


def bwd_fused_workspace_size(B, H, NQ, NK, d, causal, dtype, grad_mask):
    return load().streamkl_bwd_fused_workspace_size(B, H, NQ, NK, d, causal, dtype, grad_mask)


def bwd_fused_selected(B, H, NQ, NK, d, causal, dtype, grad_mask):
    """1 where streamkl_bwd runs the single-pass (fused) backward."""
    return load().streamkl_bwd_fused_selected(B, H, NQ, NK, d, causal, dtype, grad_mask)
